// The general 8-bit blockwise codec: quantize_blockwise / dequantize_blockwise
// ("Feat/mps gemm 4bit bf16", table "What runs natively now"; "Known
// failures": the exact float64 nearest-code search is the reference, a
// lookup of the normalised value on a fixed grid is not).
//
// quantize:   absmax[b] = max |x| over block b; q = index of the table value
//             nearest to x / absmax[b], ties toward the smaller magnitude.
// dequantize: out = fp32(code[q] * absmax[b]), rounded to the output type.
//
// Exactness.  With mid_j the midpoint of table values j and j + 1 (exact in
// float64 for midpoints of at most 29 significant bits, checked on the host),
// the code of x is the number of j with x above absmax * mid_j ("above": >
// for mid_j > 0, >= for mid_j < 0, so ties go toward zero).  The predicate
// falls as j grows, so the code is the unique c with x above threshold c - 1
// and not above threshold c: any first guess, moved up or down one threshold
// at a time, reaches it.
//
// One comparison per threshold: d = fma(-absmax, mid_j, x) is x - absmax *
// mid_j rounded once, so its sign (and whether it is zero) is exact.  x,
// absmax and mid_j are multiples of 2^-149, 2^-149 and 2^-150, so a nonzero
// d is at least 2^-299 in magnitude, and "above" is d > e_j with e_j = 0 for
// mid_j > 0 and e_j = -2^-900 for mid_j < 0 (d >= 0 there, -0 included).
#include <algorithm>
#include <type_traits>

#include "qmv_launch.hpp"

#pragma clang fp contract(off)

namespace qmv {

// ---------------------------------------------------------------------------
// quantize_blockwise
//
// A workgroup takes tiles of 4096 consecutive elements (every supported
// block size divides it).  Each thread holds 16 of them as R 16-byte loads of
// VE elements; load r of thread t covers elements r * 256 VE + t VE .. + VE - 1
// of the tile, so each load instruction reads one contiguous range.  A block
// spans G = blocksize / VE neighbouring lanes of one load (reduced with DPP
// and shuffles), or several waves (through LDS), or several of the loads.
//
// First guess of the code, from the fp32 approximation n ~ x / absmax:
//   linear table (k - 127) / 127: rint(127 n) + 127;
//   any other table: a 4224-entry byte table indexed by the sign, the binade
//   (2^-32 .. 2^0, clamped) and the top six fraction bits of n, holding the
//   number of midpoints below the lower edge of that range.
// Linear table: the guess is the code unless 127 n + 127 is within a small
// guard of a half-integer (bound below); then the guess k is within one of
// the code, and the code is k - 1 + [x above threshold k - 1] + [x above
// threshold k].  Other tables: three independent comparisons around the
// guess g settle every code in {g, g + 1} (a range of n holds at most one
// midpoint for most tables); otherwise the guess is moved one threshold at a
// time.
// ---------------------------------------------------------------------------
constexpr int kQbTile = 4096;

// Linear table: the fp32 y = fma(x up, fp32(127 / (absmax up)), 127) differs
// from the exact 127 n + 127 by at most 127 2^-24 (the reciprocal) plus
// 255 2^-24 (the fma), under 2.3e-5; each threshold 127 mid_j + 127 lies
// within 127 2^-25 < 3.9e-6 of j + 1/2 (table values are (j - 127) / 127
// rounded to fp32).  When y is more than 2^-13 (> 2.7e-5) inside the
// half-integers around rint(y), every threshold is strictly on its side of
// the exact value, and rint(y) is the code.
constexpr float kLinGuard = 0x1p-13f;
constexpr int kQbSub = 6;          // fraction bits of n in the key
constexpr int kQbHalf = 33 << kQbSub;  // keys per sign: 33 binades x 64 sub-ranges
constexpr int kQbKeys = 2 * kQbHalf;
constexpr int kQbBin0 = 95 << kQbSub;  // (fp32 bits >> (23 - kQbSub)) of 2^-32

// Key of n: increasing in n; keys kQbHalf.. for n >= +0, below for n <= -0.
__device__ __forceinline__ int qb_key(float n) {
  const uint32_t u = __float_as_uint(n);
  int i = (int)((u & 0x7fffffffu) >> (23 - kQbSub)) - kQbBin0;
  i = i < 0 ? 0 : (i > kQbHalf - 1 ? kQbHalf - 1 : i);
  return (u >> 31) ? kQbHalf - 1 - i : kQbHalf + i;
}

// Lower edge of the range of n that maps to key k.
__device__ __forceinline__ double qb_key_low(int k) {
  if (k >= kQbHalf) {
    const int i = k - kQbHalf;
    return i == 0 ? 0.0 : (double)__uint_as_float((uint32_t)(i + kQbBin0) << (23 - kQbSub));
  }
  const int i = kQbHalf - 1 - k;
  return -(double)__uint_as_float((uint32_t)(i + 1 + kQbBin0) << (23 - kQbSub));
}

// One threshold of the search: the midpoint and its tie bias (see above).
struct alignas(16) QbThr {
  double mid;
  double eps;
};

__device__ __forceinline__ bool qb_above(const QbThr &t, double x, double sd) {
  return __builtin_fma(-sd, t.mid, x) > t.eps;
}

// The code of x from any start k (0 .. 255), one threshold at a time.  th
// points at the entry of threshold 0 (thresholds 0 .. 254 are read).
__device__ __attribute__((noinline)) int qb_search(const QbThr *th, double x, double sd, int k) {
  while (k < 255 && qb_above(th[k], x, sd)) ++k;
  while (k > 0 && !qb_above(th[k - 1], x, sd)) --k;
  return k;
}

template <int DT>
__global__ __launch_bounds__(256) void quantize_blockwise_kernel(const void *__restrict__ Av,
                                                                 int64_t n, int log2bs,
                                                                 Code2Table code, int linear,
                                                                 uint8_t *__restrict__ q,
                                                                 float *__restrict__ absmax) {
  using T = typename Storage<DT>::type;
  constexpr int VE = DT == kF32 ? 4 : 8;  // elements per 16-byte load
  constexpr int R = 16 / VE;              // loads per thread and tile
  const T *A = static_cast<const T *>(Av);
  // thresholds 0 .. 254 at th_s[1 ..]; th_s[0] (-inf: every x with absmax > 0
  // is above it) and th_s[256], th_s[257] (+inf: none is) bound the search
  __shared__ QbThr th_s[258];
  __shared__ uint8_t guess[kQbKeys];
  // two sets, used by alternate tiles: a set is rewritten only after every
  // thread has passed the next tile's barrier
  __shared__ float wave_max[2][R][4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const QbThr *th = th_s + 1;
  {
    const double md = tid < 255 ? ((double)code.v[tid] + (double)code.v[tid + 1]) * 0.5 : INFINITY;
    th_s[tid + 1] = QbThr{md, md > 0.0 ? 0.0 : -0x1p-900};  // md exact
    if (tid == 0) th_s[0] = QbThr{-INFINITY, 0.0};
    if (tid == 1) th_s[257] = QbThr{INFINITY, 0.0};
  }
  __syncthreads();
  if (!linear) {
    for (int k = tid; k < kQbKeys; k += 256) {
      const double lo = qb_key_low(k);
      int a = 0, b = 255;  // number of midpoints below lo, by bisection
      while (a < b) {
        const int md = (a + b) >> 1;
        if (th[md].mid < lo) a = md + 1;
        else b = md;
      }
      guess[k] = (uint8_t)a;
    }
    __syncthreads();
  }

  const int bs = 1 << log2bs;
  const int G = bs / VE;  // lanes per block within one load: 4 .. 1024
  const int64_t ntiles = (n + kQbTile - 1) / kQbTile;
  const int64_t nfull = n / kQbTile;

  auto load_full = [&](int64_t t, uint4 (&raw)[R]) {
    const uint4 *src = reinterpret_cast<const uint4 *>(A + t * kQbTile) + tid;
#pragma unroll
    for (int r = 0; r < R; ++r) raw[r] = src[r * 256];
  };
  auto convert = [&](const uint4 (&raw)[R], float (&v)[R][VE]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t w[4] = {raw[r].x, raw[r].y, raw[r].z, raw[r].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (DT == kF32) {
          v[r][j] = __uint_as_float(w[j]);
        } else {
          v[r][2 * j] = bits16_to_f32<DT>(w[j] & 0xffffu);
          v[r][2 * j + 1] = bits16_to_f32<DT>(w[j] >> 16);
        }
      }
    }
  };

  auto process = [&](int64_t t, const float (&v)[R][VE], int par, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int64_t base = t * kQbTile;
    float m[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float mm = 0.f;
#pragma unroll
      for (int j = 0; j < VE; ++j) mm = fmaxf(mm, fabsf(v[r][j]));
      m[r] = group_max(mm, G < 64 ? G : 64);
    }
    if (G > 64) {  // uniform across the launch
      if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) wave_max[par][r][wave] = m[r];
      }
      __syncthreads();
      const int wpb = G >= 256 ? 4 : G >> 6;  // waves of a block within one load
      const int w0 = (wave / wpb) * wpb;
      const int lpb = G > 256 ? G >> 8 : 1;   // loads a block spans
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int r0 = (r / lpb) * lpb;
        float mm = 0.f;
        for (int rr = r0; rr < r0 + lpb; ++rr)
          for (int w = w0; w < w0 + wpb; ++w) mm = fmaxf(mm, wave_max[par][rr][w]);
        m[r] = mm;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t e0 = base + r * 256 * VE + tid * VE;
      if ((e0 & (bs - 1)) == 0 && (FULL || e0 < n)) absmax[e0 >> log2bs] = m[r];
      const double sd = (double)m[r];
      int c[VE];
      // n ~ x / absmax is formed as (x up) / (absmax up): tiny maxima are
      // scaled up by an exact 2^64 so the reciprocal stays finite
      const float up = m[r] < 0x1p-60f ? 0x1p64f : 1.f;
      if (linear) {
        // y = fp32(127 n + 127) and k = rint(y), saturated to 0 .. 255 by the
        // conversion (|n| <= 1, so k <= 254).  k is the code unless y lies
        // within kLinGuard of a half-integer; such elements take the exact
        // two-threshold check (the code is k - 1, k or k + 1)
        const float inv = m[r] > 0.f ? 127.f / (m[r] * up) : 0.f;
        uint32_t unsure = 0;
#pragma unroll
        for (int j = 0; j < VE; ++j) {
          const float y = fmaf(v[r][j] * up, inv, 127.f);
          c[j] = (int)__builtin_amdgcn_cvt_pk_u8_f32(y, 0, 0u);
          unsure |= fabsf(y - (float)c[j]) < 0.5f - kLinGuard ? 0u : (1u << j);
        }
        if (__builtin_amdgcn_ballot_w64(unsure != 0) != 0) {
#pragma unroll
          for (int j = 0; j < VE; ++j) {
            if (unsure & (1u << j)) {
              const int k = c[j];
              const double x = (double)v[r][j];
              c[j] = k - 1 + (qb_above(th[k - 1], x, sd) ? 1 : 0) + (qb_above(th[k], x, sd) ? 1 : 0);
            }
          }
        }
      } else {
        const float inv = m[r] > 0.f ? __builtin_amdgcn_rcpf(m[r] * up) : 0.f;
        uint32_t slow = 0;
#pragma unroll
        for (int j = 0; j < VE; ++j) {
          const int k = guess[qb_key((v[r][j] * up) * inv)];
          const double x = (double)v[r][j];
          const bool lo = qb_above(th[k - 1], x, sd);
          const bool at = qb_above(th[k], x, sd);
          const bool hi = qb_above(th[k + 1], x, sd);  // th[255], th[256]: +inf
          c[j] = k + (at ? 1 : 0);
          slow |= (lo && !hi) ? 0u : (1u << j);  // the code is not k or k + 1
        }
        if (__builtin_amdgcn_ballot_w64(slow != 0) != 0) {
#pragma unroll
          for (int j = 0; j < VE; ++j)
            if (slow & (1u << j)) c[j] = qb_search(th, (double)v[r][j], sd, c[j]);
        }
      }
      uint32_t word[VE / 4];
#pragma unroll
      for (int w = 0; w < VE / 4; ++w)
        word[w] = (uint32_t)c[4 * w] | ((uint32_t)c[4 * w + 1] << 8) |
                  ((uint32_t)c[4 * w + 2] << 16) | ((uint32_t)c[4 * w + 3] << 24);
      if (FULL || e0 + VE <= n) {
        if constexpr (VE == 8) *reinterpret_cast<uint2 *>(q + e0) = make_uint2(word[0], word[1]);
        else *reinterpret_cast<uint32_t *>(q + e0) = word[0];
      } else {
#pragma unroll
        for (int j = 0; j < VE; ++j)
          if (e0 + j < n) q[e0 + j] = (uint8_t)c[j];
      }
    }
  };

  // full tiles: the next tile's loads are issued before this one is processed
  // (clamped to the last full tile, so every lane issues the same loads)
  int64_t t = blockIdx.x;
  int par = 0;
  if (nfull > 0) {
    uint4 nx[R];
    load_full(t < nfull ? t : nfull - 1, nx);
    for (; t < nfull; t += gridDim.x) {
      float v[R][VE];
      convert(nx, v);
      const int64_t tn = t + gridDim.x;
      load_full(tn < nfull ? tn : nfull - 1, nx);
      process(t, v, par, std::true_type{});
      par ^= 1;
    }
  }
  // the ragged last tile, if any (same workgroup stride, so exactly one takes it)
  if (t < ntiles) {
    const int64_t base = t * kQbTile;
    float v[R][VE];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < VE; ++j) {
        const int64_t e = base + r * 256 * VE + tid * VE + j;
        v[r][j] = e < n ? load_elem<DT>(A, e) : 0.f;
      }
    process(t, v, par, std::false_type{});
  }
}

hipError_t launch_quantize_blockwise(const void *A, int a_dtype, int64_t n, int log2bs,
                                     const Code2Table &code, bool linear, uint8_t *q,
                                     float *absmax, hipStream_t st) {
  const int64_t ntiles = (n + kQbTile - 1) / kQbTile;
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(ntiles, 8 * device_cu_count()));
  const int lin = linear ? 1 : 0;
  if (a_dtype == kF32)
    hipLaunchKernelGGL(quantize_blockwise_kernel<kF32>, dim3(grid), dim3(256), 0, st, A, n, log2bs,
                       code, lin, q, absmax);
  else if (a_dtype == kF16)
    hipLaunchKernelGGL(quantize_blockwise_kernel<kF16>, dim3(grid), dim3(256), 0, st, A, n, log2bs,
                       code, lin, q, absmax);
  else
    hipLaunchKernelGGL(quantize_blockwise_kernel<kBF16>, dim3(grid), dim3(256), 0, st, A, n, log2bs,
                       code, lin, q, absmax);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dequantize_blockwise
//
// A wave takes chunks of 2048 codes: four 8-byte loads per lane, the lanes of
// each load adjacent; the eight values of a load share one block (blocks are
// 32 or more) and are written with one 16-byte store (two for fp32).  kBwU
// chunks are loaded before any is converted.
// ---------------------------------------------------------------------------
constexpr int kBwU = 2;

template <int ODT>
__global__ __launch_bounds__(256) void dequantize_blockwise_kernel(const uint8_t *__restrict__ q,
                                                                   const float *__restrict__ absmax,
                                                                   int64_t n, int log2bs,
                                                                   Code2Table code, void *out_v) {
  using OT = typename Storage<ODT>::type;
  OT *out = static_cast<OT *>(out_v);
  __shared__ float tab[256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  tab[tid] = code.v[tid];
  __syncthreads();

  auto emit = [&](int64_t e, uint2 w, float a) {
    const uint32_t ws[2] = {w.x, w.y};
    float v[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) v[b] = tab[(ws[b >> 2] >> (8 * (b & 3))) & 0xffu] * a;
    if constexpr (ODT == kF32) {
      float4 *dst = reinterpret_cast<float4 *>(out + e);
      dst[0] = make_float4(v[0], v[1], v[2], v[3]);
      dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      *reinterpret_cast<uint4 *>(out + e) =
          make_uint4(cvt_pair<ODT>(v[0], v[1]), cvt_pair<ODT>(v[2], v[3]),
                     cvt_pair<ODT>(v[4], v[5]), cvt_pair<ODT>(v[6], v[7]));
    }
  };

  const int64_t nchunk = n >> 11;
  const int64_t wave = ((int64_t)blockIdx.x * 256 + tid) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * 256) >> 6;
  const uint2 *qw = reinterpret_cast<const uint2 *>(q);
  for (int64_t c0 = wave; c0 < nchunk; c0 += nwaves * kBwU) {
    uint2 w[kBwU][4];
    float a[kBwU][4];
#pragma unroll
    for (int u = 0; u < kBwU; ++u) {
      const int64_t cu = c0 + u * nwaves;
      const int64_t c = cu < nchunk ? cu : nchunk - 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[u][i] = qw[c * 256 + 64 * i + lane];
        a[u][i] = absmax[((c << 11) + 512 * i + 8 * lane) >> log2bs];
      }
    }
#pragma unroll
    for (int u = 0; u < kBwU; ++u) {
      const int64_t c = c0 + u * nwaves;
      if (c >= nchunk) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) emit((c << 11) + 512 * i + 8 * lane, w[u][i], a[u][i]);
    }
  }
  // tail: the last n % 2048 elements, one per thread
  for (int64_t e = (nchunk << 11) + (int64_t)blockIdx.x * 256 + tid; e < n;
       e += (int64_t)gridDim.x * 256)
    store_elem<ODT>(out, e, materialize(tab[q[e]] * absmax[e >> log2bs]));
}

hipError_t launch_dequantize_blockwise(const uint8_t *q, const float *absmax, int64_t n, int log2bs,
                                       const Code2Table &code, void *out, int out_dtype,
                                       hipStream_t st) {
  const int64_t nchunk = n >> 11;
  const int64_t want = (nchunk + 4 * kBwU - 1) / (4 * kBwU);  // 4 waves per workgroup
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(want, 8 * device_cu_count()));
  if (out_dtype == kF32)
    hipLaunchKernelGGL(dequantize_blockwise_kernel<kF32>, dim3(grid), dim3(256), 0, st, q, absmax, n,
                       log2bs, code, out);
  else if (out_dtype == kF16)
    hipLaunchKernelGGL(dequantize_blockwise_kernel<kF16>, dim3(grid), dim3(256), 0, st, q, absmax, n,
                       log2bs, code, out);
  else
    hipLaunchKernelGGL(dequantize_blockwise_kernel<kBF16>, dim3(grid), dim3(256), 0, st, q, absmax, n,
                       log2bs, code, out);
  return hipGetLastError();
}

}  // namespace qmv
