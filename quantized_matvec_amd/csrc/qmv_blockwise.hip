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

// A 16-byte store marked non-temporal (streamed out: the output is not read
// back by the kernel, and the hint measured faster for large outputs).
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_nt(void *p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  __builtin_nontemporal_store(u32x4_nt{a, b, c, d}, static_cast<u32x4_nt *>(p));
}

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
//   any other table: n is placed in one of 4224 ranges by its sign, binade
//   (2^-32 .. 2^0, clamped) and top six fraction bits (qb_key).  Widened by
//   the error of n, a range holds g midpoints below it and, for nearly every
//   range of nearly every table, at most one inside it (QbRange).
// Linear table: the guess is the code unless 127 n + 127 is within a small
// guard of a half-integer (bound below); then the guess k is within one of
// the code, and the code is k - 1 + [x above threshold k - 1] + [x above
// threshold k].  Other tables: the code is g, or g + [n > the range's
// midpoint] when n is clearly away from it; elements near a midpoint, and
// ranges holding several, take the exact search.
// ---------------------------------------------------------------------------
constexpr int kQbTile = 4096;
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// Linear table: y = fma(x, fp32(127 rcp(absmax)), 127) in fp32 differs from
// the exact 127 n + 127 by at most 127 (2^-23 + 2^-24) (the reciprocal, 1 ulp,
// and the product) plus 2^-17 (the fma), under 3.1e-5; each threshold
// 127 mid_j + 127 lies within 127 2^-25 < 3.9e-6 of j + 1/2 (table values are
// (j - 127) / 127 rounded to fp32).  When y is more than 2^-13 (1.2e-4)
// inside the half-integers around rint(y), every threshold is strictly on its
// side of the exact value, and rint(y) is the code.
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
  return kQbHalf + (i ^ ((int)u >> 31));  // negative: kQbHalf - 1 - i
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

// One range of n for tables other than the linear one (n' = x * rcp(absmax)
// in fp32 is within 2^-22 of n, relative): g = number of midpoints under the
// range widened by 2^-20 of its edges; hi = the top of an interval of doubt
// [hi - 2^-19 |hi|, hi] that covers mf -+ 2^-20 |mf| (each bound rounded
// once: still beyond mf -+ 2^-21 |mf|), mf the one midpoint inside the
// widened range rounded to fp32 (n' outside it is on the same side of mf as
// n is of the exact midpoint: both errors together are under 2^-21 |mf|);
// hi = FLT_MAX when the range holds no midpoint (n' is always below), NaN
// when it holds several (and for the range around zero when it holds any:
// there n' may be subnormal, without a relative bound).  An element in
// doubt in a range with one midpoint has code g or g + 1: its exact n lies
// inside the widened range, above the g midpoints below it and below the
// ones above it, so one exact test against midpoint g decides.
struct alignas(8) QbRange {
  float hi;
  int g;
};

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

template <int DT, bool LIN>
__global__ __launch_bounds__(256) void quantize_blockwise_kernel(const void *__restrict__ Av,
                                                                 int64_t n, int log2bs,
                                                                 Code2Table code,
                                                                 uint8_t *__restrict__ q,
                                                                 float *__restrict__ absmax) {
  using T = typename Storage<DT>::type;
  constexpr int VE = DT == kF32 ? 4 : 8;  // elements per 16-byte load
  constexpr int R = 16 / VE;              // loads per thread and tile
  const T *A = static_cast<const T *>(Av);
  // thresholds 0 .. 254 at th_s[1 ..]; th_s[0] (-inf: every x with absmax > 0
  // is above it) and th_s[256], th_s[257] (+inf: none is) bound the search
  __shared__ QbThr th_s[258];
  __shared__ QbRange ranges[LIN ? 1 : kQbKeys];
  // two sets, used by alternate tiles: a set is rewritten only after every
  // thread has passed the next tile's barrier
  __shared__ uint32_t wave_max[2][R][4];
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
  if constexpr (!LIN) {
    // thread t fills ranges [17 t, 17 t + 17): one bisection for the first
    // range's counts, then both counts only move up (the widened edges grow
    // with the key); th[255].mid = +inf stops the walks
    constexpr int kPer = (kQbKeys + 255) / 256;
    const int k0 = tid * kPer;
    const int k1 = k0 + kPer < kQbKeys ? k0 + kPer : kQbKeys;
    int g = 0, h = 0;
    for (int k = k0; k < k1; ++k) {
      const bool pos = k >= kQbHalf;
      const int i = pos ? k - kQbHalf : kQbHalf - 1 - k;  // |n| sub-range
      const double a0 = i == 0 ? 0.0 : (double)__uint_as_float((uint32_t)(i + kQbBin0) << (23 - kQbSub));
      const double a1 = (double)__uint_as_float((uint32_t)(i + 1 + kQbBin0) << (23 - kQbSub));
      const double lo = pos ? a0 * (1.0 - 0x1p-20) : -a1 * (1.0 + 0x1p-20);
      const double hi = pos ? a1 * (1.0 + 0x1p-20) : -a0 * (1.0 - 0x1p-20);
      if (k == k0) {
        int a = 0, b = 255;
        while (a < b) {  // midpoints < lo
          const int md = (a + b) >> 1;
          if (th[md].mid < lo) a = md + 1;
          else b = md;
        }
        g = a;
        a = g, b = 255;
        while (a < b) {  // midpoints <= hi
          const int md = (a + b) >> 1;
          if (th[md].mid <= hi) a = md + 1;
          else b = md;
        }
        h = a;
      } else {
        while (th[g].mid < lo) ++g;
        if (h < g) h = g;
        while (th[h].mid <= hi) ++h;
      }
      const int inside = h - g;
      float hi_d;
      if (inside == 0) {
        hi_d = 3.4028234663852886e38f;  // n' is always below the interval
      } else if (inside == 1 && i != 0) {
        const float mf = (float)th[g].mid;
        hi_d = mf + fabsf(mf) * 0x1p-20f;  // the interval covers mf -+ 2^-20 |mf|
      } else {
        hi_d = __builtin_nanf("");  // never decided
      }
      ranges[k] = QbRange{hi_d, g};
    }
    __syncthreads();
  }

  const int bs = 1 << log2bs;
  const int G = bs / VE;  // lanes per block within one load: 4 .. 1024
  const int64_t ntiles = (n + kQbTile - 1) / kQbTile;
  const int64_t nfull = n / kQbTile;

  auto load_full = [&](int64_t t, uint4 (&raw)[R]) {
    typedef uint32_t u32x4_ld __attribute__((ext_vector_type(4)));
    const u32x4_ld *src = reinterpret_cast<const u32x4_ld *>(A + t * kQbTile) + tid;
#pragma unroll
    for (int r = 0; r < R; ++r) {  // read once: non-temporal
      const u32x4_ld v = __builtin_nontemporal_load(src + r * 256);
      raw[r] = make_uint4(v.x, v.y, v.z, v.w);
    }
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

  // per-load max |x| as fp32 bits (non-negative floats order as their bits;
  // integer maxima also skip the NaN quieting a float max needs)
  auto local_max_raw = [&](const uint4 (&raw)[R], uint32_t (&mb)[R]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t w[4] = {raw[r].x, raw[r].y, raw[r].z, raw[r].w};
      if constexpr (DT == kF32) {
        mb[r] = max(max(w[0] & 0x7fffffffu, w[1] & 0x7fffffffu),
                    max(w[2] & 0x7fffffffu, w[3] & 0x7fffffffu));
      } else {
        u16x2_t acc = __builtin_bit_cast(u16x2_t, w[0] & 0x7fff7fffu);
#pragma unroll
        for (int i = 1; i < 4; ++i)
          acc = __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2_t, w[i] & 0x7fff7fffu));
        mb[r] = __float_as_uint(bits16_to_f32<DT>(max((uint32_t)acc.x, (uint32_t)acc.y)));
      }
    }
  };

  auto process = [&](int64_t t, const float (&v)[R][VE], const uint32_t (&mb)[R], int par,
                     auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int64_t base = t * kQbTile;
    float m[R];
#pragma unroll
    for (int r = 0; r < R; ++r) m[r] = group_max(__uint_as_float(mb[r]), G < 64 ? G : 64);
    if (G > 64) {  // uniform across the launch
      if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) wave_max[par][r][wave] = __float_as_uint(m[r]);
      }
      __syncthreads();
      if (G >= 256) {  // a block covers whole loads: all four waves, lpb loads
        uint32_t wm[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
          wm[r] = max(max(wave_max[par][r][0], wave_max[par][r][1]),
                      max(wave_max[par][r][2], wave_max[par][r][3]));
        const int lpb = G >> 8;  // 1, 2 or 4 (4 only when R == 4)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint32_t mm = wm[r];
          if (lpb >= 2) mm = max(mm, wm[r ^ 1]);
          if constexpr (R == 4) {
            if (lpb == 4) mm = max(mm, max(wm[r ^ 2], wm[r ^ 3]));
          }
          m[r] = __uint_as_float(mm);
        }
      } else {  // two waves per block
#pragma unroll
        for (int r = 0; r < R; ++r)
          m[r] = __uint_as_float(max(wave_max[par][r][wave], wave_max[par][r][wave ^ 1]));
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t e0 = base + r * 256 * VE + tid * VE;
      if ((e0 & (bs - 1)) == 0 && (FULL || e0 < n)) absmax[e0 >> log2bs] = m[r];
      const float mr = m[r];
      const double sd = (double)mr;
      int c[VE];
      // the fast guess uses an fp32 reciprocal of absmax (absmax >= 2^-120;
      // NaN below, which sends the group to the exact path; 0 for a zero block)
      const float rc = mr == 0.f ? 0.f : (mr >= 0x1p-120f ? __builtin_amdgcn_rcpf(mr) : __builtin_nanf(""));
      // exact path: n from (x up) / (absmax up), tiny maxima scaled up by an
      // exact 2^64 so that the reciprocal stays finite
      const float up = mr < 0x1p-60f ? 0x1p64f : 1.f;
      if constexpr (LIN) {
        // y = fp32(127 n + 127) and k = rint(y), saturated to 0 .. 255 by the
        // conversion (|n| <= 1, so k <= 254).  k is the code unless y lies
        // within kLinGuard of a half-integer: then only the threshold between
        // floor(y) and floor(y) + 1 is near, and one exact comparison settles
        // the code.  A NaN y (absmax below 2^-120) takes the scaled path.
        const float inv = 127.f * rc;
        float y[VE];
        bool any = false;
#pragma unroll
        for (int j = 0; j < VE; ++j) {
          y[j] = fmaf(v[r][j], inv, 127.f);
          c[j] = (int)__builtin_amdgcn_cvt_pk_u8_f32(y[j], 0, 0u);
          any |= !(fabsf(y[j] - (float)c[j]) < 0.5f - kLinGuard);
        }
        if (__builtin_amdgcn_ballot_w64(any) != 0) {
#pragma unroll
          for (int j = 0; j < VE; ++j) {
            const float d = y[j] - (float)c[j];
            const bool u = !(fabsf(d) < 0.5f - kLinGuard);
            if (__builtin_amdgcn_ballot_w64(u) != 0 && u) {
              const double x = (double)v[r][j];
              if (mr >= 0x1p-120f) {
                const int kf = c[j] - (d < 0.f ? 1 : 0);  // th[-1] is -inf
                c[j] = kf + (qb_above(th[kf], x, sd) ? 1 : 0);
              } else {  // tiny absmax: k from a correctly rounded 127 / (absmax up)
                const int k = (int)__builtin_amdgcn_cvt_pk_u8_f32(
                    fmaf(v[r][j] * up, 127.f / (mr * up), 127.f), 0, 0u);
                c[j] = k - 1 + (qb_above(th[k - 1], x, sd) ? 1 : 0) + (qb_above(th[k], x, sd) ? 1 : 0);
              }
            }
          }
        }
      } else {
        // the code is g, or g + 1 when n' is above the range's interval of
        // doubt [hi - 2^-19 |hi|, hi]; n' inside it takes one exact test
        // against midpoint g, a NaN range (or a rescaled block) the search
        // per element: in doubt (u) and whether its range has a single
        // midpoint (one): kept as lane masks, so the exact path below needs
        // no second range read (an element in doubt is not above the
        // interval, so its guess c is the range's g)
        bool any = false;
        bool u[VE], one[VE];
#pragma unroll
        for (int j = 0; j < VE; ++j) {
          const float nn = v[r][j] * rc;
          const QbRange e = ranges[qb_key(nn)];
          c[j] = e.g + (nn > e.hi ? 1 : 0);
          u[j] = !(nn > e.hi || nn < fmaf(-0x1p-19f, fabsf(e.hi), e.hi));
          one[j] = e.hi == e.hi;
          any |= u[j];
        }
        if (__builtin_amdgcn_ballot_w64(any) != 0) {
          const float rc2 = mr > 0.f ? __builtin_amdgcn_rcpf(mr * up) : 0.f;
#pragma unroll
          for (int j = 0; j < VE; ++j) {
            if (__builtin_amdgcn_ballot_w64(u[j]) != 0 && u[j]) {
              if (up == 1.f && one[j])  // one midpoint inside, unscaled key
                c[j] = c[j] + (qb_above(th[c[j]], (double)v[r][j], sd) ? 1 : 0);
              else
                c[j] = qb_search(th, (double)v[r][j], sd, ranges[qb_key((v[r][j] * up) * rc2)].g);
            }
          }
        }
      }
      uint32_t word[VE / 4];
#pragma unroll
      for (int w = 0; w < VE / 4; ++w)
        word[w] = (uint32_t)c[4 * w] | ((uint32_t)c[4 * w + 1] << 8) |
                  ((uint32_t)c[4 * w + 2] << 16) | ((uint32_t)c[4 * w + 3] << 24);
      if (FULL || e0 + VE <= n) {
        if constexpr (VE == 8) {
          typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
          __builtin_nontemporal_store(u32x2_nt{word[0], word[1]}, reinterpret_cast<u32x2_nt *>(q + e0));
        }
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
      uint32_t mb[R];
      convert(nx, v);
      local_max_raw(nx, mb);
      const int64_t tn = t + gridDim.x;
      load_full(tn < nfull ? tn : nfull - 1, nx);
      process(t, v, mb, par, std::true_type{});
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
    uint32_t mb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t mm = 0;
#pragma unroll
      for (int j = 0; j < VE; ++j) mm = max(mm, __float_as_uint(v[r][j]) & 0x7fffffffu);
      mb[r] = mm;
    }
    process(t, v, mb, par, std::false_type{});
  }
}

template <int DT>
static void launch_qb_t(int64_t ntiles, const void *A, int64_t n, int log2bs, const Code2Table &code,
                        bool linear, uint8_t *q, float *absmax, hipStream_t st) {
  // one resident generation of workgroups, each striding over the tiles
  static const int occ_lin = resident_wgs_per_cu(
      reinterpret_cast<const void *>(&quantize_blockwise_kernel<DT, true>), 256);
  static const int occ_gen = resident_wgs_per_cu(
      reinterpret_cast<const void *>(&quantize_blockwise_kernel<DT, false>), 256);
  const int64_t slots = (int64_t)device_cu_count() * (linear ? occ_lin : occ_gen);
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(ntiles, slots));
  if (linear)
    hipLaunchKernelGGL((quantize_blockwise_kernel<DT, true>), dim3(grid), dim3(256), 0, st, A, n,
                       log2bs, code, q, absmax);
  else
    hipLaunchKernelGGL((quantize_blockwise_kernel<DT, false>), dim3(grid), dim3(256), 0, st, A, n,
                       log2bs, code, q, absmax);
}

hipError_t launch_quantize_blockwise(const void *A, int a_dtype, int64_t n, int log2bs,
                                     const Code2Table &code, bool linear, uint8_t *q,
                                     float *absmax, hipStream_t st) {
  const int64_t ntiles = (n + kQbTile - 1) / kQbTile;
  if (a_dtype == kF32) launch_qb_t<kF32>(ntiles, A, n, log2bs, code, linear, q, absmax, st);
  else if (a_dtype == kF16) launch_qb_t<kF16>(ntiles, A, n, log2bs, code, linear, q, absmax, st);
  else launch_qb_t<kBF16>(ntiles, A, n, log2bs, code, linear, q, absmax, st);
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
      store16_nt(out + e, __float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                 __float_as_uint(v[3]));
      store16_nt(out + e + 4, __float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                 __float_as_uint(v[7]));
    } else {
      store16_nt(out + e, cvt_pair<ODT>(v[0], v[1]), cvt_pair<ODT>(v[2], v[3]),
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
