// Codec kernels: quantize_4bit, double quantization of the scales, scale
// reconstruction and dequantize_4bit.
//
// Operation set: "Feat/mps gemm 4bit bf16", table "What runs natively now"
// (quantize_4bit / dequantize_4bit); block size and double quantization:
// "mps-bitsandbytes 0.4.7", section "Functional API".  Every result here is
// bit-exact: the nearest-code decision is made against exact thresholds, and
// every float operation is an explicitly rounded one.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
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


int log2_exact(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}

// Rank among the midpoints (0..15 for NF4, 0..14 for FP4) -> code.
template <int QT>
__device__ __forceinline__ uint32_t rank_to_code(int r) {
  if constexpr (QT == kNF4) {
    return (uint32_t)r;  // NF4 codes are ascending ranks
  } else {
    // FP4 ascending values: codes 15..9 (negatives), 0 (zero), 1..7 (positives),
    // as nibble r of one 64-bit constant
    return (uint32_t)(0x0765432109ABCDEFull >> (4 * r)) & 15u;
  }
}

// ---------------------------------------------------------------------------
// quantize_4bit
//
// A workgroup of 256 threads takes a tile of 256 * E consecutive elements
// (E = 16: a 32-byte load for 16-bit inputs); G = blocksize / E neighbouring
// threads share a block.  The block absmax is reduced across those G threads
// (DPP moves within rows of 16 lanes, shuffles beyond, LDS when a block spans
// waves).
//
// Nearest code, exactly.  Let m_0 < m_1 < ... be the midpoints of adjacent
// distinct code values.  The code of x in a block with absmax a is its rank:
// the number of midpoints it lies above, where "above" a positive midpoint
// means x > a m_j (a tie stays with the smaller magnitude) and above a
// negative one x >= a m_j.
//
// The rank is read off a bin position.  u = S x / a + O; bin = floor(u).  The
// host picks S and O so that every bin holds at most one midpoint, none
// within 0.02 of a bin edge, and tabulates per bin J(b) = the midpoints below
// it and pos(b) = S m_J + O - 1/2 for the midpoint inside it (+inf when there
// is none).  The kernel computes t = u - 1/2 in fp32 as fma(x, S rcp(a),
// O - 1/2), takes the bin as t rounded to the nearest integer (one
// conversion, saturated), and
//   rank = J(b) + [t > pos(b)].
// The fp32 t is within 1e-5 of the exact u - 1/2 (rcp is within an ulp, the
// rest one rounding each; |t| < 64) and pos(b) within 2e-6 of the exact
// S m_J + O - 1/2, so whenever |t - pos(b)| >= 2^-15 the comparison has the
// exact answer; an element whose approximate t falls in a neighbouring bin
// sits within 1e-5 of a bin edge, where no midpoint is, so the count is the
// same.
// The few elements inside the 2^-15 band (exact ties among them) are decided
// exactly in float64: a m_J is exact there (24 x 29 significant bits), as is
// the comparison with x.
// ---------------------------------------------------------------------------
constexpr int kQBins = 64;
constexpr float kQBand = 0x1p-15f;  // certificate band around a midpoint, in bins
struct QuantArgs {
  Midpoints4 mids;
  uint8_t cand[256];     // J(b); bins 64 .. 255 count every midpoint
  float pos[256];        // pos(b) (less 1/2), +inf for a bin without a midpoint
  float bin_scale;       // S
  float bin_offset;      // O - 1/2
};

template <int DT, int QT, int E>
__global__ __launch_bounds__(256) void quantize_4bit_kernel(const void *__restrict__ Wv,
                                                            int64_t numel, int log2bs,
                                                            QuantArgs qa,
                                                            uint8_t *__restrict__ packed,
                                                            float *__restrict__ absmax) {
  using T = typename Storage<DT>::type;
  const T *W = static_cast<const T *>(Wv);
  __shared__ float wave_max[2][4];  // blocks spanning waves, alternate tiles
  __shared__ uint8_t cand[256];     // bytes: the bin is the address
  __shared__ float pos[256];
  __shared__ double mids[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int G = (1 << log2bs) / E;  // threads per block: 2 .. 256
  const int64_t tile = 256 * E;
  const int64_t ntiles = (numel + tile - 1) / tile;
  cand[tid] = qa.cand[tid];
  pos[tid] = qa.pos[tid];
  if (tid < 15) mids[tid] = qa.mids.mid[tid];
  __syncthreads();

  // full tiles' loads: E elements per thread as raw 16-byte words (E / 4
  // for fp32, E / 8 for 16-bit types); they are converted only when the tile
  // is processed, so a prefetched tile is not waited for at its load
  constexpr int NW = DT == kF32 ? E / 4 : E / 8;
  auto load_full = [&](int64_t tt, uint4 (&raw)[NW]) {
    const int64_t e0 = tt * tile + (int64_t)tid * E;
    const uint4 *src = reinterpret_cast<const uint4 *>(W + e0);
#pragma unroll
    for (int i = 0; i < NW; ++i) raw[i] = src[i];
  };
  auto convert = [&](const uint4 (&raw)[NW], float (&v)[E]) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
      if constexpr (DT == kF32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * i + j] = __uint_as_float(w[j]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = bits16_to_f32<DT>(w[j] & 0xffffu);
          v[8 * i + 2 * j + 1] = bits16_to_f32<DT>(w[j] >> 16);
        }
      }
    }
  };

  // FULL: a whole tile, whose stores are all unconditional (every lane of a
  // block writes the same absmax), so the load waits can be counted exactly
  auto process = [&](int64_t t, const float (&v)[E], int par, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int64_t e0 = t * tile + (int64_t)tid * E;
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) m = fmaxf(m, fabsf(v[i]));
    m = group_max(m, G);
    if (G > 64) {  // uniform across the launch
      if (lane == 0) wave_max[par][wave] = m;
      __syncthreads();
      const int wpb = G >> 6;
      const int w0 = (wave / wpb) * wpb;
      float mm = wave_max[par][w0];
      for (int i = 1; i < wpb; ++i) mm = fmaxf(mm, wave_max[par][w0 + i]);
      m = mm;
    }
    if (FULL || ((tid & (G - 1)) == 0 && e0 < numel)) absmax[e0 >> log2bs] = m;

    // t = S x / a + O: tiny blocks are scaled up by 2^100 (exact) so the
    // reciprocal stays finite, huge ones down by 2^100 so it stays normal;
    // an all-zero block has t = O - 1/2, the position of 0
    const float sc = m < 0x1p-100f ? 0x1p100f : (m > 0x1p100f ? 0x1p-100f : 1.f);
    const float inv = m > 0.f ? qa.bin_scale * __builtin_amdgcn_rcpf(m * sc) : 0.f;
    const float O = qa.bin_offset;
    float tq[E];
    if (__builtin_amdgcn_ballot_w64(sc != 1.f) == 0) {  // wave-uniform: no rescaled block
#pragma unroll
      for (int i = 0; i < E; ++i) tq[i] = fmaf(v[i], inv, O);
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) tq[i] = fmaf(v[i] * sc, inv, O);
    }
    int J[E];
    float pb[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
      // the bin: t carries the offset O - 1/2, so rounding to the nearest
      // integer (saturated to 0 .. 255, NaN to 0) is the floor of S x / a + O;
      // where the rounding and the floor can differ, t is within an ulp of a
      // bin edge, and either neighbouring bin gives the same rank
      const uint32_t b = __builtin_amdgcn_cvt_pk_u8_f32(tq[i], 0, 0u);
      J[i] = (int)cand[b];
      pb[i] = pos[b];
    }
    uint32_t rank[E];
    bool amb = false;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      rank[i] = (uint32_t)J[i] + (tq[i] > pb[i] ? 1u : 0u);
      amb |= fabsf(tq[i] - pb[i]) < kQBand;
    }
    if (__builtin_amdgcn_ballot_w64(amb) != 0) {  // rare: decide the band exactly
      const double ad = (double)m;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        if (fabsf(tq[i] - pb[i]) < kQBand) {
          const double mid = mids[J[i]];
          const double p = ad * mid;  // exact
          const double xd = (double)v[i];
          rank[i] = (uint32_t)J[i] + ((mid > 0.0 ? xd > p : xd >= p) ? 1u : 0u);
        }
      }
    }
    uint32_t code[E];
#pragma unroll
    for (int i = 0; i < E; ++i) code[i] = (FULL || e0 + i < numel) ? rank_to_code<QT>((int)rank[i]) : 0u;

    uint32_t word[E / 8];
#pragma unroll
    for (int w = 0; w < E / 8; ++w) {
      uint32_t x = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        x |= ((code[8 * w + 2 * b] << 4) | code[8 * w + 2 * b + 1]) << (8 * b);
      word[w] = x;
    }
    uint8_t *dst = packed + (e0 >> 1);
    if (FULL || e0 + E <= numel) {
      if constexpr (E == 8) {
        *reinterpret_cast<uint32_t *>(dst) = word[0];
      } else {
        typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(u32x2_nt{word[0], word[1]}, reinterpret_cast<u32x2_nt *>(dst));
      }
    } else {
#pragma unroll
      for (int b = 0; b < E / 2; ++b)
        if (e0 + 2 * b < numel) dst[b] = (uint8_t)(word[b >> 2] >> (8 * (b & 3)));
    }
  };

  // full tiles: the next tile's loads are issued before this one is processed
  // (unconditionally, clamped to the last full tile, so the waits are exact)
  const int64_t nfull = numel / tile;
  int64_t t = blockIdx.x;
  int par = 0;
  if (nfull > 0) {
    uint4 nx[NW];
    load_full(t < nfull ? t : nfull - 1, nx);
    for (; t < nfull; t += gridDim.x) {
      float v[E];
      convert(nx, v);
      const int64_t tn = t + gridDim.x;
      load_full(tn < nfull ? tn : nfull - 1, nx);
      process(t, v, par, std::true_type{});
      par ^= 1;
    }
  }
  // the ragged last tile, if any (same workgroup stride, so exactly one takes it)
  if (t < ntiles) {
    const int64_t e0 = t * tile + (int64_t)tid * E;
    float v[E];
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = (e0 + i < numel) ? load_elem<DT>(W, e0 + i) : 0.f;
    process(t, v, par, std::false_type{});
  }
}

template <int DT, int QT>
static hipError_t launch_quantize_t(const void *W, int64_t numel, int log2bs, const QuantArgs &qa,
                                    uint8_t *packed, float *absmax, hipStream_t st) {
  // 16 elements per thread: a tile (4096) holds whole blocks of every size
  constexpr int E = 16;
  const int64_t tile = 256 * E;
  const int64_t ntiles = (numel + tile - 1) / tile;
  // one resident generation of workgroups, each striding over the tiles
  static const int occ = resident_wgs_per_cu(
      reinterpret_cast<const void *>(&quantize_4bit_kernel<DT, QT, E>), 256);
  const int64_t slots = (int64_t)device_cu_count() * occ;
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(ntiles, slots));
  hipLaunchKernelGGL((quantize_4bit_kernel<DT, QT, E>), dim3(grid), dim3(256), 0, st, W, numel,
                     log2bs, qa, packed, absmax);
  return hipGetLastError();
}

// Bin geometry of the rank search (see above): S in 14..30 bins per unit of
// n and offset O = S + 1 + k / 64 + 1 / 128, chosen so that no two midpoints
// share a bin and the midpoint nearest to a bin edge is as far from it as
// possible (at least 0.02 bin); J(b) counts the midpoints below bin b.
// Bins of n in [-1, 1] are 1 .. 2 S + 2 < kQBins.
static_assert(2 * 30 + 2 < kQBins, "the bins of n in [-1, 1] lie below kQBins for every S tried");
static bool bin_geometry(const Midpoints4 &m, int nt, QuantArgs &qa) {
  double best = 0.0;
  for (int S = 14; S <= 30; ++S) {
    for (int k = 0; k < 64; ++k) {
      const double o = S + 1 + k / 64.0 + 1.0 / 128.0;
      double worst = 1.0;
      long prev = -1;
      bool distinct = true;
      for (int j = 0; j < nt; ++j) {
        const double v = S * m.mid[j] + o;
        const double b = std::floor(v);
        worst = std::min(worst, std::min(v - b, b + 1.0 - v));
        distinct = distinct && (long)b != prev;
        prev = (long)b;
      }
      if (distinct && worst > best) {
        best = worst;
        qa.bin_scale = (float)S;
        qa.bin_offset = (float)o;
      }
    }
  }
  if (best < 0.02) return false;
  for (int b = 0; b < 256; ++b) {
    int c = 0;
    for (int j = 0; j < nt; ++j)
      c += std::floor((double)qa.bin_scale * m.mid[j] + (double)qa.bin_offset) < b ? 1 : 0;
    qa.cand[b] = (uint8_t)c;
    // the midpoint inside bin b, if any, is midpoint c; its position is kept
    // less 1/2, like t (below)
    const double pj = c < nt ? (double)qa.bin_scale * m.mid[c] + (double)qa.bin_offset : 0.0;
    qa.pos[b] = (c < nt && std::floor(pj) == (double)b) ? (float)(pj - 0.5) : INFINITY;
  }
  // the kernels compute t = S x / a + O - 1/2 and take the bin as t rounded
  // to the nearest integer (O - 1/2 has 8 fraction bits: exact in fp32)
  qa.bin_offset -= 0.5f;
  return true;
}

hipError_t launch_quantize_4bit(const void *W, int w_dtype, int64_t numel, int log2bs, int qt,
                                const Midpoints4 &m, uint8_t *packed, float *absmax,
                                hipStream_t st) {
  // candidate rank at each bin centre, from the exact midpoints
  // the geometry depends only on the table: found once per table
  static std::mutex mu;
  static Midpoints4 cached_m[2];
  static QuantArgs cached_qa[2];
  static bool cached_ok[2] = {false, false};
  const int nt = qt == kNF4 ? 15 : 14;
  QuantArgs qa{};
  {
    std::lock_guard<std::mutex> lock(mu);
    const int i = qt == kNF4 ? 0 : 1;
    if (!cached_ok[i] || memcmp(&cached_m[i], &m, sizeof(m)) != 0) {
      QuantArgs g{};
      g.mids = m;
      if (!bin_geometry(m, nt, g)) return hipErrorInvalidValue;
      cached_m[i] = m;
      cached_qa[i] = g;
      cached_ok[i] = true;
    }
    qa = cached_qa[i];
  }
#define QMV_Q(DT, QT) return launch_quantize_t<DT, QT>(W, numel, log2bs, qa, packed, absmax, st)
  if (qt == kNF4) {
    if (w_dtype == kF32) QMV_Q(kF32, kNF4);
    if (w_dtype == kF16) QMV_Q(kF16, kNF4);
    QMV_Q(kBF16, kNF4);
  } else {
    if (w_dtype == kF32) QMV_Q(kF32, kFP4);
    if (w_dtype == kF16) QMV_Q(kF16, kFP4);
    QMV_Q(kBF16, kFP4);
  }
#undef QMV_Q
}

// ---------------------------------------------------------------------------
// Double quantization.
//
// 1. The mean of the scales: float64 sums over consecutive runs of 256 in a
//    fixed order, level after level, until one value S is left; offset =
//    fp32(S / nblocks).  The order is part of the contract, but a float64
//    sum of fp32 values is exact, and then independent of the order, when
//    all its partial sums are integer multiples of the smallest ulp u among
//    the values and below 2^53 u: for k values below 2^h with ulp >= 2^l
//    that holds when log2(k) + h - l <= 53.  So every workgroup of the first
//    launch takes 16 runs of the first level and, when its values pass that
//    test for k = 256, sums each run as a wave reduction, otherwise as the
//    plain sequential loop; it also records h and l.  The encode launch then
//    combines the first-level sums: if all n values pass the test (log2 n in
//    place of log2 256) any order gives the tree's exact sum, else it runs
//    the remaining levels in tree order.  Beyond 4096 first-level runs one
//    workgroup of a third launch sums the remaining levels in tree order.
// 2. Per group of blocksize2 scales: c = fp32(a - offset), s = max |c|, and
//    the code of c / s is the rank of c among the exact float64 thresholds
//    s * mid[j] of the (strictly increasing) 256-entry table; ties go toward
//    zero as in quantize_4bit.  For the default linear table the rank is
//    within one of round(127 c / s) + 127 and two threshold compares settle
//    it; any other table takes a binary search.
// ---------------------------------------------------------------------------
constexpr int kFanIn = 256;
constexpr int kSumRuns = 16;              // runs per workgroup pass

// Sums runs [16 g, 16 g + 16) of `in` (n values): the runs are staged in LDS
// (rows padded to 257 doubles so that the 16 summing threads hit different
// banks) with all loads in flight together; thread r then adds run r in
// order.  Values past n load as zero, and adding +0 leaves the (non-negative)
// sum unchanged, so a short last run needs no length test.
template <typename In>
__device__ __forceinline__ void sum_runs16(const In *__restrict__ in, int64_t n, int64_t g,
                                           double *__restrict__ out, double *stage) {
  const int tid = threadIdx.x;
  const int64_t nout = (n + kFanIn - 1) / kFanIn;
  const int64_t run0 = g * kSumRuns;
  const int64_t base = run0 * kFanIn;
  const int64_t rem = n - base;
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(in + base, (uint32_t)((rem < kSumRuns * kFanIn ? rem : kSumRuns * kFanIn) * sizeof(In)));
  In v[kSumRuns];
#pragma unroll
  for (int i = 0; i < kSumRuns; ++i) {  // element base + i * 256 + tid
    const uint32_t off = (uint32_t)((i * kFanIn + tid) * sizeof(In));
    if constexpr (sizeof(In) == 4)
      v[i] = __builtin_bit_cast(In, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
    else
      v[i] = __builtin_bit_cast(In, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
  }
#pragma unroll
  for (int i = 0; i < kSumRuns; ++i) stage[i * (kFanIn + 1) + tid] = (double)v[i];
  __syncthreads();
  if (tid < kSumRuns && run0 + tid < nout) {
    const double *row = stage + tid * (kFanIn + 1);
    double s = 0.0;
    // 32 values at a time: the reads of a chunk are independent of the
    // additions, so they are in flight together
    for (int k0 = 0; k0 < kFanIn; k0 += 32) {
      double w[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) w[k] = row[k0 + k];
#pragma unroll
      for (int k = 0; k < 32; ++k) s = __dadd_rn(s, w[k]);
    }
    out[run0 + tid] = s;
  }
  __syncthreads();  // stage is reused
}

// Exponent bounds of an fp32 value for the exactness test: |v| < 2^h and
// ulp(v) >= 2^l.  Zero contributes nothing (h = -1000, l = +1000); inf and
// NaN fail the test (h = +1000).
__device__ __forceinline__ void exp_bounds(float v, int &h, int &l) {
  const uint32_t e = (__builtin_bit_cast(uint32_t, v) >> 23) & 255u;
  const bool zero = (__builtin_bit_cast(uint32_t, v) & 0x7fffffffu) == 0u;
  h = zero ? -1000 : (e == 255u ? 1000 : (e == 0u ? -126 : (int)e - 126));
  l = zero ? 1000 : (e == 0u ? -149 : (int)e - 150);
}

// First level: workgroup g sums runs [16 g, 16 g + 16) of the scales and
// stores (max h, min l) of its values in stats[g].  When that level is
// already a single run it also writes the offset.
__global__ __launch_bounds__(256) void dq_sum_kernel(const float *__restrict__ absmax, int64_t n,
                                                     double *__restrict__ levels,
                                                     int2 *__restrict__ stats,
                                                     float *__restrict__ offset) {
  __shared__ double stage[kSumRuns * (kFanIn + 1)];
  __shared__ int wh[4], wl[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t g = blockIdx.x;
  const int64_t nout = (n + kFanIn - 1) / kFanIn;
  const int64_t run0 = g * kSumRuns;
  const int64_t base = run0 * kFanIn;
  const int64_t rem = n - base;
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(absmax + base, (uint32_t)((rem < kSumRuns * kFanIn ? rem : kSumRuns * kFanIn) * 4));
  float v[kSumRuns];
#pragma unroll
  for (int i = 0; i < kSumRuns; ++i)  // element base + i * 256 + tid (zero past n)
    v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         rs, (uint32_t)((i * kFanIn + tid) * 4), 0, 0));
  int h = -1000, l = 1000;
#pragma unroll
  for (int i = 0; i < kSumRuns; ++i) {
    int hi, li;
    exp_bounds(v[i], hi, li);
    h = max(h, hi);
    l = min(l, li);
    stage[i * (kFanIn + 1) + tid] = (double)v[i];
  }
  h = wave_max_i32(h);
  l = wave_min_i32(l);
  if (lane == 0) {
    wh[wave] = h;
    wl[wave] = l;
  }
  __syncthreads();
  h = max(max(wh[0], wh[1]), max(wh[2], wh[3]));
  l = min(min(wl[0], wl[1]), min(wl[2], wl[3]));
  if (tid == 0) stats[g] = make_int2(h, l);
  if (8 + h - l <= 53) {
    // exact: wave w sums runs 4 w .. 4 w + 3, lane l adds values 4 l .. 4 l + 3
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int run = 4 * wave + r;
      const double *row = stage + run * (kFanIn + 1) + 4 * lane;
      const double t = wave_sum_f64((row[0] + row[1]) + (row[2] + row[3]));
      if (lane == 0 && run0 + run < nout) levels[run0 + run] = t;
    }
  } else if (tid < kSumRuns && run0 + tid < nout) {
    const double *row = stage + tid * (kFanIn + 1);
    double t = 0.0;
    for (int k0 = 0; k0 < kFanIn; k0 += 32) {
      double w[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) w[k] = row[k0 + k];
#pragma unroll
      for (int k = 0; k < 32; ++k) t = __dadd_rn(t, w[k]);  // + 0 past n: unchanged
    }
    levels[run0 + tid] = t;
  }
  if (n <= kFanIn) {  // one run: its sum is S
    __syncthreads();
    if (tid == 0) offset[0] = (float)__ddiv_rn(levels[0], (double)n);
  }
}

// The remaining levels, in one workgroup (a kernel boundary separates it from
// the first level, so no cross-workgroup hand-off is needed), then the offset.
__global__ __launch_bounds__(256) void dq_top_kernel(double *__restrict__ levels, int64_t nl,
                                                     int64_t n, float *__restrict__ offset) {
  __shared__ double stage[kSumRuns * (kFanIn + 1)];
  double *level = levels;
  while (nl > 1) {
    double *next = level + nl;
    const int64_t nn = (nl + kFanIn - 1) / kFanIn;
    for (int64_t g = 0; g * kSumRuns < nn; ++g) sum_runs16<double>(level, nl, g, next, stage);
    level = next;
    nl = nn;
  }
  if (threadIdx.x == 0) offset[0] = (float)__ddiv_rn(level[0], (double)n);  // written by thread 0
}

// Encode: a workgroup takes a tile of 256 * E consecutive scales, E per
// thread (E = 8, or 16 when a group of 4096 would span more than 256
// threads); the G = blocksize2 / E threads of a group reduce max |c|.
//
// With 1 < nl <= kTopFused first-level sums every workgroup first derives
// the offset from them (the same bits in every workgroup; workgroup 0 writes
// them); otherwise an earlier launch wrote it.
constexpr int kTopFused = 4096;

__device__ __forceinline__ float fused_offset(const double *__restrict__ levels, int64_t nl,
                                              const int2 *__restrict__ stats, int64_t n, double *red) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // the first-level sums this thread may need (levels tid + 256 k), all in flight
  constexpr int kPer = kTopFused / 256;
  double v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int64_t i = tid + 256 * k;
    v[k] = i < nl ? levels[i] : 0.0;
  }
  // exactness over all n values: combine the first launch's per-workgroup bounds
  const int64_t nst = (nl + kSumRuns - 1) / kSumRuns;  // <= 256
  int h = -1000, l = 1000;
  for (int64_t i = tid; i < nst; i += 256) {
    const int2 st = stats[i];
    h = max(h, st.x);
    l = min(l, st.y);
  }
  h = wave_max_i32(h);
  l = wave_min_i32(l);
  int *ri = reinterpret_cast<int *>(red);
  if (lane == 0) {
    ri[2 * wave] = h;
    ri[2 * wave + 1] = l;
  }
  __syncthreads();
  h = max(max(ri[0], ri[2]), max(ri[4], ri[6]));
  l = min(min(ri[1], ri[3]), min(ri[5], ri[7]));
  int log2n = 0;
  while (((int64_t)1 << log2n) < n) ++log2n;
  __syncthreads();
  double total;
  if (log2n + h - l <= 53) {
    // exact: any order
    double t = 0.0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) t += v[k];
    t = wave_sum_f64(t);
    if (lane == 0) red[wave] = t;
    __syncthreads();
    total = (red[0] + red[1]) + (red[2] + red[3]);
  } else {
    // the remaining levels in tree order: <= 16 runs, then one; thread r
    // reads run r 32 values at a time (all in flight), adding +0 past nl
    const int64_t nn = (nl + kFanIn - 1) / kFanIn;
    if (tid < nn) {
      const double *row = levels + (int64_t)tid * kFanIn;
      const int64_t len = nl - (int64_t)tid * kFanIn < kFanIn ? nl - (int64_t)tid * kFanIn : kFanIn;
      double t = 0.0;
      for (int64_t k0 = 0; k0 < len; k0 += 32) {
        double w[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) w[k] = k0 + k < len ? row[k0 + k] : 0.0;
#pragma unroll
        for (int k = 0; k < 32; ++k) t = __dadd_rn(t, w[k]);
      }
      red[tid] = t;
    }
    __syncthreads();
    total = red[0];
    if (nn > 1) {
      total = 0.0;
      for (int64_t r = 0; r < nn; ++r) total = __dadd_rn(total, red[r]);
    }
  }
  return (float)__ddiv_rn(total, (double)n);
}

template <int E>
__global__ __launch_bounds__(256) void dq_encode_kernel(const float *__restrict__ absmax,
                                                        int64_t n, int log2bs2, Code2Table code2,
                                                        int linear, const double *__restrict__ levels,
                                                        const int2 *__restrict__ stats, int64_t nl,
                                                        float *__restrict__ offset,
                                                        uint8_t *__restrict__ q,
                                                        float *__restrict__ absmax2,
                                                        float *__restrict__ code2_out) {
  __shared__ double mid[256];
  __shared__ float wave_max[4];
  __shared__ double red[kTopFused / kFanIn];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (tid < 255) mid[tid] = ((double)code2.v[tid] + (double)code2.v[tid + 1]) * 0.5;  // exact
  if (code2_out && blockIdx.x == 0) code2_out[tid] = code2.v[tid];

  const int G = (1 << log2bs2) / E;  // threads per group: 2 .. 256
  const int64_t tile = (int64_t)256 * E;
  const int64_t ntiles = (n + tile - 1) / tile;
  // a tile's scales through a range-limited buffer: no branch per load.  The
  // first tile is loaded before the offset is formed, so the two memory round
  // trips overlap.
  float a[E];
  auto load_tile = [&](int64_t tt) {
    const int64_t rem = n - tt * tile;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(absmax + tt * tile, (uint32_t)((rem < tile ? rem : tile) * sizeof(float)));
#pragma unroll
    for (int e = 0; e < E; ++e)
      a[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           rs, (uint32_t)((tid * E + e) * 4), 0, 0));
  };
  if (blockIdx.x < ntiles) load_tile(blockIdx.x);

  float off;
  if (nl > 1 && nl <= kTopFused) {
    off = fused_offset(levels, nl, stats, n, red);
    if (blockIdx.x == 0 && tid == 0) offset[0] = off;
  } else {
    off = offset[0];  // written by an earlier launch
  }
  __syncthreads();

  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t i0 = t * tile + (int64_t)tid * E;
    if (t != (int64_t)blockIdx.x) load_tile(t);
    float c[E];
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      c[e] = (i0 + e < n) ? __fsub_rn(a[e], off) : 0.f;
      m = fmaxf(m, fabsf(c[e]));
    }
    const int gw = G < 64 ? G : 64;
    for (int o = 1; o < gw; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (G > 64) {
      if (lane == 0) wave_max[wave] = m;
      __syncthreads();
      const int wpg = G >> 6;
      const int w0 = (wave / wpg) * wpg;
      float mm = wave_max[w0];
      for (int i = 1; i < wpg; ++i) mm = fmaxf(mm, wave_max[w0 + i]);
      m = mm;
      __syncthreads();
    }
    if ((tid & (G - 1)) == 0 && i0 < n) absmax2[i0 >> log2bs2] = m;
    const double sd = (double)m;
    // c above the threshold of midpoint j (ties toward zero)
    auto above = [&](double x, int j) {
      const double mj = mid[j];
      const double thr = sd * mj;  // exact
      return mj > 0.0 ? (x > thr) : (x >= thr);
    };
    int code[E];
    if (linear) {
      // y = fp32(127 n + 127), n = c / m, and k = rint(y) saturated to
      // 0 .. 255 (|n| <= 1, so k <= 254; a group with a tiny max is scaled up
      // by an exact 2^64 so that 127 / m stays finite).  y is within 2.3e-5
      // of the exact 127 n + 127 (the reciprocal's and the fma's roundings)
      // and each threshold 127 mid_j + 127 within 3.9e-6 of j + 1/2, so when
      // y is more than 2^-13 inside the half-integers around k, k is the
      // code; otherwise k is within one of it and two exact comparisons
      // settle it.
      const float up = m < 0x1p-60f ? 0x1p64f : 1.f;
      const float inv = m > 0.f ? 127.f / (m * up) : 0.f;
      uint32_t unsure = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float y = fmaf(c[e] * up, inv, 127.f);
        code[e] = (int)__builtin_amdgcn_cvt_pk_u8_f32(y, 0, 0u);
        unsure |= fabsf(y - (float)code[e]) < 0.5f - 0x1p-13f ? 0u : (1u << e);
      }
      if (__builtin_amdgcn_ballot_w64(unsure != 0) != 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (unsure & (1u << e)) {
            int k = code[e];
            const double x = (double)c[e];
            k += (k < 255 && above(x, k)) ? 1 : 0;
            k -= (k > 0 && !above(x, k - 1)) ? 1 : 0;
            code[e] = k;
          }
        }
      }
    } else {
      int lo[E], hi[E];
#pragma unroll
      for (int e = 0; e < E; ++e) { lo[e] = 0; hi[e] = 255; }
#pragma unroll
      for (int step = 0; step < 8; ++step) {  // 255 thresholds: 8 halvings
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int md = (lo[e] + hi[e]) >> 1;
          const bool up = above((double)c[e], md);
          lo[e] = up ? md + 1 : lo[e];
          hi[e] = up ? hi[e] : md;
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) code[e] = lo[e];
    }
    if (i0 + E <= n) {  // whole: E codes in E / 4 word stores (q + i0 is E-byte aligned)
#pragma unroll
      for (int w = 0; w < E / 4; ++w)
        reinterpret_cast<uint32_t *>(q + i0)[w] =
            (uint32_t)code[4 * w] | ((uint32_t)code[4 * w + 1] << 8) |
            ((uint32_t)code[4 * w + 2] << 16) | ((uint32_t)code[4 * w + 3] << 24);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (i0 + e < n) q[i0 + e] = (uint8_t)code[e];
    }
  }
}

static constexpr size_t dq_workspace_bytes(int64_t nblocks) {
  size_t total = 0;
  int64_t n = nblocks;
  do {
    n = (n + kFanIn - 1) / kFanIn;
    total += (size_t)n * sizeof(double);
  } while (n > 1);
  const int64_t runs = (nblocks + kFanIn - 1) / kFanIn;
  return total + (size_t)((runs + kSumRuns - 1) / kSumRuns) * sizeof(int2);  // + exponent bounds
}

size_t double_quant_workspace_bytes(int64_t nblocks) { return dq_workspace_bytes(nblocks); }

// The fixed scratch of the allocation-free double quantization: the mean tree
// and exponent bounds for up to kNoAllocMaxBlocks scales.  One copy per GPU,
// held until the process ends; every call on that GPU reuses it (the kernels
// overwrite it before reading it, so it needs no clearing), so calls that
// overlap on one GPU race.  In host code `scratch` is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = 576 * 1024;
static_assert(dq_workspace_bytes(kNoAllocMaxBlocks) <= kNoAllocScratchBytes,
              "scratch too small for kNoAllocMaxBlocks scales");
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void *scratch_ptr[kMaxDevices];
hipError_t scratch_status[kMaxDevices];
}  // namespace

hipError_t double_quant_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(scratch_once[dev], [dev] {
    void *p = nullptr;  // the current device is `dev`: this resolves its own copy
    scratch_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    scratch_ptr[dev] = scratch_status[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = scratch_ptr[dev];
  return scratch_status[dev];
}

hipError_t launch_double_quant(const float *absmax, int64_t nblocks, int log2bs2,
                               const Code2Table &code2, bool linear, uint8_t *q, float *absmax2,
                               float *offset, float *code2_out, void *ws, hipStream_t st) {
  double *levels = static_cast<double *>(ws);
  const int64_t runs = (nblocks + kFanIn - 1) / kFanIn;
  size_t lv = 0;  // doubles in all levels
  for (int64_t m = nblocks; m > 1 || lv == 0;) {
    m = (m + kFanIn - 1) / kFanIn;
    lv += (size_t)m;
    if (m <= 1) break;
  }
  int2 *stats = reinterpret_cast<int2 *>(levels + lv);
  hipLaunchKernelGGL(dq_sum_kernel, dim3((unsigned)((runs + kSumRuns - 1) / kSumRuns)), dim3(256), 0,
                     st, absmax, nblocks, levels, stats, offset);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (runs > kTopFused) {  // else the encode launch combines the first level itself
    hipLaunchKernelGGL(dq_top_kernel, dim3(1), dim3(256), 0, st, levels, runs, nblocks, offset);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int bs2 = 1 << log2bs2;
  const int E = bs2 > 2048 ? 16 : 8;
  const int64_t tile = 256 * (int64_t)E;
  const int64_t ntiles = (nblocks + tile - 1) / tile;
  const unsigned grid = (unsigned)std::min<int64_t>(ntiles, 1 << 16);
#define QMV_E(EV)                                                                          \
  hipLaunchKernelGGL((dq_encode_kernel<EV>), dim3(grid), dim3(256), 0, st, absmax, nblocks, log2bs2, \
                     code2, linear ? 1 : 0, levels, stats, runs > kTopFused ? (int64_t)1 : runs, \
                     offset, q, absmax2, code2_out)
  if (E == 8) QMV_E(8); else QMV_E(16);
#undef QMV_E
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scale reconstruction ("Functional API": dequant_absmax).
// ---------------------------------------------------------------------------
template <bool DQ>
__global__ __launch_bounds__(256) void dequantize_absmax_kernel(Scales sc, int64_t n,
                                                                float *__restrict__ out) {
  const float offset = DQ ? sc.offset[0] : 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out[i] = block_scale<DQ>(sc, i, offset);
}

hipError_t launch_dequantize_absmax(const Scales &sc, bool dq, int64_t n, float *out,
                                    hipStream_t st) {
  const unsigned grid = (unsigned)std::min<int64_t>((n + 255) / 256, 1 << 16);
  if (dq)
    hipLaunchKernelGGL(dequantize_absmax_kernel<true>, dim3(grid), dim3(256), 0, st, sc, n, out);
  else
    hipLaunchKernelGGL(dequantize_absmax_kernel<false>, dim3(grid), dim3(256), 0, st, sc, n, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dequantize_4bit
//
// A wave handles chunks of 2048 elements (1 KB packed).  Lane l reads the
// 4-byte words at byte 256 w + 4 l of the chunk (w = 0..3), i.e. elements
// 512 w + 8 l .. + 7, so that each of its output stores (8 elements) lands
// next to its neighbours' and one store instruction writes a contiguous
// range (16 B per lane for bf16 / fp16; lane-strided stores measured at half
// the bandwidth).  U chunks per wave have all their loads issued before the
// first is used; loads past the last full chunk are clamped to it (never
// stored), so the compiler counts them.  Each packed byte indexes a 256-entry
// LDS table of fp32 code pairs; the products with the block scale are rounded
// once to fp32 and then converted (bf16: v_cvt_pk_bf16_f32, round to nearest
// even).  Elements past the last full chunk are written by the tail loop.
// ---------------------------------------------------------------------------
constexpr int kDeqThreads = 256;
constexpr int kDeqU = 2;  // chunks in flight per wave

template <int QT, int ODT, bool DQ>
__global__ __launch_bounds__(kDeqThreads) void dequantize_4bit_kernel(
    const uint8_t *__restrict__ packed, Scales sc, int64_t numel, int log2bs, void *__restrict__ outv) {
  using OT = typename Storage<ODT>::type;
  OT *out = static_cast<OT *>(outv);
  __shared__ float2 lut2[256];  // byte -> (T[byte >> 4], T[byte & 15])
  __shared__ float code2[256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  {
    const uint32_t *tb = table_bits(QT);
    lut2[tid] = make_float2(__uint_as_float(tb[tid >> 4]), __uint_as_float(tb[tid & 15]));
    if constexpr (DQ) code2[tid] = sc.code2[tid];
  }
  const float offset = DQ ? sc.offset[0] : 0.f;
  __syncthreads();

  // 8 elements (one packed word) -> output
  auto emit = [&](int64_t e, uint32_t word, float a) {
    if constexpr (ODT == kF32) {
      float o[8];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const float2 t = lut2[(word >> (8 * bb)) & 0xffu];
        o[2 * bb] = t.x * a;
        o[2 * bb + 1] = t.y * a;
      }
      store16_nt(out + e, __float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                 __float_as_uint(o[3]));
      store16_nt(out + e + 4, __float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]),
                 __float_as_uint(o[7]));
    } else {
      uint32_t o[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const float2 t = lut2[(word >> (8 * bb)) & 0xffu];
        o[bb] = cvt_pair<ODT>(t.x * a, t.y * a);
      }
      store16_nt(out + e, o[0], o[1], o[2], o[3]);
    }
  };

  const int64_t nchunk = numel >> 11;
  const int64_t wave = ((int64_t)blockIdx.x * kDeqThreads + tid) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kDeqThreads) >> 6;
  const uint32_t *pk = reinterpret_cast<const uint32_t *>(packed);
  for (int64_t c0 = wave; c0 < nchunk; c0 += nwaves * kDeqU) {
    uint32_t pw[kDeqU][4], sq[kDeqU][4];
    float sa[kDeqU][4];
#pragma unroll
    for (int u = 0; u < kDeqU; ++u) {
      const int64_t cu = c0 + u * nwaves;
      const int64_t c = cu < nchunk ? cu : nchunk - 1;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pw[u][w] = __builtin_nontemporal_load(pk + c * 256 + 64 * w + lane);  // read once
        const int64_t b = ((c << 11) + 512 * w + 8 * lane) >> log2bs;
        if constexpr (DQ) {
          sq[u][w] = sc.q[b];
          sa[u][w] = sc.absmax2[b >> sc.log2bs2];
        } else {
          sa[u][w] = sc.absmax[b];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kDeqU; ++u) {
      const int64_t c = c0 + u * nwaves;
      if (c >= nchunk) break;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = DQ ? code2[sq[u][w]] * sa[u][w] + offset : sa[u][w];
        emit((c << 11) + 512 * w + 8 * lane, pw[u][w], a);
      }
    }
  }
  // tail: elements [2048 nchunk, numel); whole 8-element words by any thread,
  // the last (numel % 8) elements by one
  const int64_t t0 = nchunk << 11;
  const int64_t nword = (numel - t0) >> 3;
  for (int64_t i = (int64_t)blockIdx.x * kDeqThreads + tid; i < nword;
       i += (int64_t)gridDim.x * kDeqThreads) {
    const int64_t e = t0 + 8 * i;
    emit(e, pk[e >> 3], block_scale<DQ>(sc, e >> log2bs, offset));
  }
  if (blockIdx.x == 0 && tid == 0 && (numel & 7)) {
    const int64_t e0 = numel & ~int64_t(7);
    const float a = block_scale<DQ>(sc, e0 >> log2bs, offset);
    for (int64_t e = e0; e < numel; ++e) {
      const uint32_t byte = packed[e >> 1];
      const uint32_t code = (e & 1) ? (byte & 15u) : (byte >> 4);
      const float2 t = lut2[code << 4];  // (T[code], T[0])
      store_elem<ODT>(out, e, t.x * a);
    }
  }
}


template <int QT, int ODT>
static hipError_t launch_dequant_t(const uint8_t *packed, const Scales &sc, bool dq, int64_t numel,
                                   int log2bs, void *out, hipStream_t st) {
  const int64_t nchunk = numel >> 11;
  const int64_t waves_per_wg = kDeqThreads / 64;
  const int64_t want = std::max<int64_t>(1, (nchunk + waves_per_wg * kDeqU - 1) / (waves_per_wg * kDeqU));
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(want, 8 * device_cu_count()));
  if (dq)
    hipLaunchKernelGGL((dequantize_4bit_kernel<QT, ODT, true>), dim3(grid), dim3(kDeqThreads), 0, st,
                       packed, sc, numel, log2bs, out);
  else
    hipLaunchKernelGGL((dequantize_4bit_kernel<QT, ODT, false>), dim3(grid), dim3(kDeqThreads), 0,
                       st, packed, sc, numel, log2bs, out);
  return hipGetLastError();
}

hipError_t launch_dequantize_4bit(const uint8_t *packed, const Scales &sc, bool dq, int64_t numel,
                                  int log2bs, int qt, void *out, int out_dtype, hipStream_t st) {
#define QMV_D(QT, ODT) return launch_dequant_t<QT, ODT>(packed, sc, dq, numel, log2bs, out, st)
  if (qt == kNF4) {
    if (out_dtype == kF32) QMV_D(kNF4, kF32);
    if (out_dtype == kF16) QMV_D(kNF4, kF16);
    QMV_D(kNF4, kBF16);
  } else {
    if (out_dtype == kF32) QMV_D(kFP4, kF32);
    if (out_dtype == kF16) QMV_D(kFP4, kF16);
    QMV_D(kFP4, kBF16);
  }
#undef QMV_D
}

}  // namespace qmv
