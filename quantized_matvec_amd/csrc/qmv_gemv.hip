// gemv_4bit: y[m, n] = sum_k x[m, k] * W_hat[n, k] for 1 <= M <= 8 rows of
// activations, with the 4-bit dequantization fused into the dot product
// ("Feat/mps gemm 4bit bf16", table "What runs natively now": gemv_4bit is a
// fused dequant + dot for the decode step).
//
// 16-bit activations (the decode case) take gemv_4bit_lut_kernel:
//  * A persistent grid of 16 waves per CU (one 1024-thread workgroup for
//    M = 1, two of 512 threads otherwise, each with its own 64 KB table);
//    wave w owns the
//    contiguous output rows [w N / W, (w + 1) N / W), so every wave streams a
//    contiguous run of the packed weight.
//  * A row is cut into slices of 64 lanes x 16 bytes (2048 weights); a lane's
//    16 bytes are 32 weights inside one block, so one scale per lane-piece.
//  * Decode: a 64 KB LDS table maps every packed byte to the two code values
//    as a bf16 (or fp16) pair.  It is replicated 64 times, one copy per lane,
//    so the lookups of a wave never share a bank; one v_perm_b32 turns a
//    packed byte and the lane number into the LDS address.
//  * Multiply: v_dot2_f32_bf16 (v_dot2_f32_f16) multiplies a looked-up pair
//    with two activations and accumulates in fp32; the block scale is applied
//    once per 32-weight piece.
//  * The loads of the next (row group, slice) -- weights, scales and, for
//    M = 1, the activations -- are issued before the current one is decoded,
//    and the first ones before the table is built, so HBM latency overlaps
//    the table setup and the arithmetic.  The table is written as
//    consecutive 16-byte chunks from kernel-argument values: no global load
//    and no bank conflict on the way to the barrier.
//  * Rows finish with a DPP wave reduction.
// fp32 activations take gemv_4bit_f32x_kernel, a plain fp32 path.
#include <algorithm>

#include "qmv_launch.hpp"

namespace qmv {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t uint4v;

constexpr int kLutReplicas = 64;  // one table copy per lane of a wave

// The 16 code values already rounded to the activation type (bf16 or fp16
// bits), computed on the host.
struct Table16 {
  uint32_t h[16];
};

// Builds the 64 KB code-pair table: entry e = (T[e >> 4], T[e & 15]) as two
// 16-bit values, 64 copies.  Written as consecutive 16-byte chunks (lane i ->
// chunk i, so no two lanes of a wave share a bank); the high half of a
// thread's entries is fixed, the low half is wave-uniform per chunk row and
// read from the kernel arguments with a scalar index.
template <int THREADS>
__device__ __forceinline__ void build_pair_table(uint32_t *lut, const Table16 &table, int tid) {
  const uint32_t hi_idx = (tid >> 4) & 15;
  uint32_t hi = 0;
#pragma unroll
  for (int c = 0; c < 16; ++c) hi = (hi_idx == (uint32_t)c) ? table.h[c] : hi;
  hi <<= 16;
  uint4 *dst = reinterpret_cast<uint4 *>(lut);
  constexpr int kChunks = 256 * kLutReplicas * 4 / 16;
#pragma unroll
  for (int it = 0; it < kChunks / THREADS; ++it) {
    const int c = it * THREADS + tid;
    const uint32_t e_hi = __builtin_amdgcn_readfirstlane((uint32_t)c >> 8);  // wave-uniform
    const uint32_t v = table.h[e_hi] | hi;
    dst[c] = make_uint4(v, v, v, v);
  }
}

template <int XDT>
__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
  if constexpr (XDT == kBF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                           __builtin_bit_cast(bf16x2_t, x), acc, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), __builtin_bit_cast(f16x2_t, x),
                                  acc, false);
}

// y[i] = v (+ bias[n], in the output type, added in fp32), rounded once to
// the output type.
__device__ __forceinline__ void store_y(void *y, int ydt, int64_t i, float v, const void *bias,
                                        int64_t n) {
  if (bias) {
    if (ydt == kF32) v = v + static_cast<const float *>(bias)[n];
    else if (ydt == kBF16) v = v + bits16_to_f32<kBF16>(static_cast<const uint16_t *>(bias)[n]);
    else v = v + bits16_to_f32<kF16>(static_cast<const uint16_t *>(bias)[n]);
  }
  if (ydt == kF32) static_cast<float *>(y)[i] = v;
  else if (ydt == kBF16) static_cast<uint16_t *>(y)[i] = (uint16_t)f32_to_bf16_rne(v);
  else static_cast<uint16_t *>(y)[i] = (uint16_t)f32_to_f16_rne(v);
}

__device__ __forceinline__ float bias_value(const void *bias, int ydt, int64_t n) {
  if (ydt == kF32) return static_cast<const float *>(bias)[n];
  if (ydt == kBF16) return bits16_to_f32<kBF16>(static_cast<const uint16_t *>(bias)[n]);
  return bits16_to_f32<kF16>(static_cast<const uint16_t *>(bias)[n]);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float x) {  // rows outside ROW_MASK read 0
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, false));
}

// Sum over the 64 lanes of a wave with DPP moves; the total ends in lane 63
// and is broadcast from there.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
  v += dpp_move<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
  v += dpp_move<0x141, 0xf>(v);  // row_half_mirror
  v += dpp_move<0x140, 0xf>(v);  // row_mirror: every lane holds its row's sum
  v += dpp_move<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_move<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Rows decoded together per step: more rows give more loads in flight, more
// activation rows more registers per row.
// M = 1 runs one 1024-thread workgroup per CU (16 waves, <= 128 VGPRs);
// larger M needs more registers and runs two 512-thread workgroups per CU.
template <int M>
struct LutShape {
  static constexpr int RG = M <= 2 ? 4 : (M <= 4 ? 2 : 1);
  static constexpr int kThreads = M == 1 ? 1024 : 512;
  static constexpr int kWgPerCu = M == 1 ? 1 : 2;
  static constexpr int kMinWavesPerSimd = kThreads / 256;
  static constexpr bool kPrefetchX = M == 1;  // x pieces travel with the weight loads
};

template <int M, int XDT, bool DQ>
__global__ __launch_bounds__(LutShape<M>::kThreads, LutShape<M>::kMinWavesPerSimd) void gemv_4bit_lut_kernel(
    const uint16_t *__restrict__ x, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    Scales sc, int log2bs, Table16 table, void *__restrict__ y, int ydt, int rows_per_wave,
    int rows_rem, const void *__restrict__ bias) {
  constexpr int RG = LutShape<M>::RG;
  constexpr int kGemvThreads = LutShape<M>::kThreads;
  constexpr bool PX = LutShape<M>::kPrefetchX;
  constexpr int XW = PX ? 16 : 1;
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * kLutReplicas];
  __shared__ float code2[256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform: keeps the per-wave bookkeeping in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * (kGemvThreads / 64) + (tid >> 6));
  const int64_t r_begin = (int64_t)wave * rows_per_wave + (wave < rows_rem ? wave : rows_rem);
  const int64_t r_end = r_begin + rows_per_wave + (wave < rows_rem ? 1 : 0);
  const int64_t pieces = K >> 5;
  const int S = (int)((pieces + 63) >> 6);
  const int64_t ngroups = (r_end - r_begin + RG - 1) / RG;
  const int64_t half_k = K >> 1;

  struct Buf {
    uint4 w[RG];
    float sa[RG];
    uint32_t sq[RG];
    uint32_t xs[XW];
  };
  auto load_x = [&](int s, uint32_t *xs, int m) {
    const int64_t pc = (int64_t)s * 64 + lane;
    uint4 xv[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                   make_uint4(0, 0, 0, 0)};
    if (pc < pieces) {
      const uint4 *xp = reinterpret_cast<const uint4 *>(x + m * K + (pc << 5));
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[q] = xp[q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xs[4 * q] = xv[q].x;
      xs[4 * q + 1] = xv[q].y;
      xs[4 * q + 2] = xv[q].z;
      xs[4 * q + 3] = xv[q].w;
    }
  };
  // issue the loads of (row group g, slice s)
  auto load = [&](int64_t g, int s, Buf &buf) {
    const int64_t pc = (int64_t)s * 64 + lane;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int64_t row = r_begin + g * RG + r;
      buf.w[r] = make_uint4(0, 0, 0, 0);
      buf.sa[r] = 0.f;
      buf.sq[r] = 0;
      if (row < r_end && pc < pieces) {
        buf.w[r] = *reinterpret_cast<const uint4 *>(packed + row * half_k + (pc << 4));
        const int64_t b = (row * K + (pc << 5)) >> log2bs;
        if constexpr (DQ) {
          buf.sq[r] = sc.q[b];
          buf.sa[r] = sc.absmax2[b >> sc.log2bs2];
        } else {
          buf.sa[r] = sc.absmax[b];
        }
      }
    }
    if constexpr (PX) load_x(s, buf.xs, 0);
  };

  Buf b0, b1;
  if (ngroups > 0) load(0, 0, b0);
  float offset = 0.f, c2v = 0.f;
  if constexpr (DQ) {
    c2v = sc.code2[tid & 255];
    offset = sc.offset[0];
  }
  // the table first: it waits on no load
  build_pair_table<kGemvThreads>(lut, table, tid);
  if constexpr (DQ) {
    if (tid < 256) code2[tid] = c2v;
  }
  __syncthreads();
  const uint32_t lane_sel = (uint32_t)lane << 2;
  const char *lut_bytes = reinterpret_cast<const char *>(lut);

  float acc[RG][M];
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

  auto compute = [&](int64_t g, int s, const Buf &buf) {
    uint32_t xl[PX ? 1 : M][16];
    if constexpr (!PX) {
#pragma unroll
      for (int m = 0; m < M; ++m) load_x(s, xl[m], m);
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const uint32_t w[4] = {buf.w[r].x, buf.w[r].y, buf.w[r].z, buf.w[r].w};
      uint32_t t[16];
#pragma unroll
      for (int bb = 0; bb < 16; ++bb) {
        const uint32_t addr =
            __builtin_amdgcn_perm(w[bb >> 2], lane_sel, 0x0c0c0000u | ((4u + (bb & 3)) << 8));
        t[bb] = *reinterpret_cast<const uint32_t *>(lut_bytes + addr);
      }
      const float ahat = DQ ? code2[buf.sq[r]] * buf.sa[r] + offset : buf.sa[r];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint32_t *xs = PX ? buf.xs : xl[m];
        float part = 0.f;
#pragma unroll
        for (int bb = 0; bb < 16; ++bb) part = dot2<XDT>(t[bb], xs[bb], part);
        acc[r][m] = fmaf(ahat, part, acc[r][m]);
      }
    }
    if (s == S - 1) {  // the rows of group g are complete
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const int64_t row = r_begin + g * RG + r;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float v = wave_sum(acc[r][m]);
          acc[r][m] = 0.f;
          if (lane == r * M + m && row < r_end) store_y(y, ydt, m * N + row, v, bias, row);
        }
      }
    }
  };

  // steps (g, s) in order; the loads of the next step go out before the
  // current one is decoded (two buffers, alternating)
  int64_t g = 0;
  int s = 0;
  while (g < ngroups) {
    int64_t g1 = g, g2;
    int s1 = s + 1, s2;
    if (s1 == S) { s1 = 0; ++g1; }
    if (g1 < ngroups) load(g1, s1, b1);
    compute(g, s, b0);
    if (g1 >= ngroups) break;
    g2 = g1;
    s2 = s1 + 1;
    if (s2 == S) { s2 = 0; ++g2; }
    if (g2 < ngroups) load(g2, s2, b0);
    compute(g1, s1, b1);
    g = g2;
    s = s2;
  }
}

// ---------------------------------------------------------------------------
// M = 1 (the decode step): gemv_4bit_m1_kernel
//
// Same table as above, one 1024-thread workgroup per CU, organised for the
// smallest vector-instruction count per 16-byte piece and an even load:
//  * The unit of work is an item: one slice (64 lanes x 16 bytes, 2048
//    weights) of one output row.  A wave owns a contiguous run of rows and
//    walks its items row by row, slice by slice.  The loads of the next item
//    are issued before the current one is decoded, so one item per wave is
//    in flight while it decodes (measured faster than 2-4 items in flight:
//    deeper queues leave loaded data waiting behind the decode).
//  * Runs are dealt so that the ones holding an extra row (when the rows do
//    not divide evenly) are spread over all workgroups: wave slot i of
//    workgroup b takes run i * gridDim.x + b.  Each wave stops after its own
//    last item.
//  * Every load is a buffer load whose range covers exactly the item's live
//    bytes (weights, block codes, group scales); a lane past the row's last
//    piece, or an item past the run's end, reads zeros and moves no data.
//    The weights, read once, carry the non-temporal hint.
//  * The activation vector is staged once in LDS (when it fits), transposed
//    so that a slice's 64 lanes read consecutive 16-byte chunks.  With 1 to 4
//    slices per row every lane then keeps its chunks of all slices in
//    registers; otherwise it reads the current slice's chunks per item.
// ---------------------------------------------------------------------------
constexpr int kM1Threads = 1024;
constexpr int kM1XLdsBytes = 90112;  // activations staged in LDS up to K = 45056 (whole slices)

// XC: x chunks staged per thread (0: no staging); SX: slices per row held in
// registers (0: none); UG: every item's blocks share one double-quant group
// (rows a multiple of 2048 weights and a slice's blocks no more than a
// group), so the group scale has a wave-uniform address
// MR: rows of activations (1 to 4): one table lookup per packed byte serves
// all of them.
template <int XDT, bool DQ, int XC, int SX, bool UG, int MR>
__global__ __launch_bounds__(kM1Threads) void gemv_4bit_m1_kernel(
    const uint16_t *__restrict__ x, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    Scales sc, int log2bs, Table16 table, void *__restrict__ y, int ydt, int rows_per_wave,
    int rows_rem, const void *__restrict__ bias) {
  constexpr bool XLDS = XC > 0;
  static_assert(SX == 0 || XLDS, "register-held activations are read from the staged copy");
  // one LDS block with the code-pair table at address 0, so a lookup address
  // needs no base added; then the DQ table and the staged activations
  __shared__ __attribute__((aligned(16))) uint32_t lds[256 * kLutReplicas + 256 +
                                                       (XLDS ? kM1XLdsBytes / 4 : 4)];
  uint32_t *lut = lds;
  float *code2 = reinterpret_cast<float *>(lds + 256 * kLutReplicas);
  uint16_t *xl = reinterpret_cast<uint16_t *>(lds + 256 * kLutReplicas + 256);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // run of this wave (wave-uniform, so the bookkeeping stays in scalar registers)
  const int run = __builtin_amdgcn_readfirstlane((tid >> 6) * (int)gridDim.x + (int)blockIdx.x);
  const int64_t r_begin = (int64_t)run * rows_per_wave + (run < rows_rem ? run : rows_rem);
  const int64_t nrows = rows_per_wave + (run < rows_rem ? 1 : 0);
  const int64_t pieces = K >> 5;
  const int S = SX > 0 ? SX : (int)((pieces + 63) >> 6);  // slices per row
  const int64_t T = nrows * S;                             // items of this wave
  const int bs_shift = log2bs - 5;                         // blocks per piece: lane >> bs_shift
  const uint32_t lane_w = (uint32_t)lane << 4;             // byte offset of the lane's piece
  const uint32_t lane_b = (uint32_t)lane >> bs_shift;      // block offset of the lane's piece

  // Prologue loads, oldest first: staged activations, the DQ table, then the
  // first item.  Loads return in order, so the staging waits only for its own.
  // staged chunk c: activation row c / (S * 256), chunk c % (S * 256) of it
  const int nch = (int)(K >> 3);  // 16-byte chunks of an activation row
  const int rch = S * 256;        // staged chunks per activation row (whole slices)
  uint4 xch[XC > 0 ? XC : 1];
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int c = i * kM1Threads + tid;
    const int m = c / rch, cr = c - m * rch;
    xch[i] = make_uint4(0, 0, 0, 0);
    if (m < MR && cr < nch) xch[i] = reinterpret_cast<const uint4 *>(x + (int64_t)m * K)[cr];
  }
  float c2v = 0.f, offset = 0.f;
  if constexpr (DQ) {
    c2v = sc.code2[tid & 255];
    offset = sc.offset[0];
  }

  uint4v w[2];
  float sa[2];
  uint8_t sq[2];
  // issue the loads of item (row rr of the run, slice s) into slot j
  auto issue = [&](int64_t rr, int s, bool live, int j) {
    const int64_t row = r_begin + (live ? rr : 0);
    const int64_t e0 = row * K + (int64_t)s * 2048;  // first weight of the item
    const int64_t left = K - (int64_t)s * 2048;
    const int64_t ne = left < 2048 ? left : 2048;   // live weights of the item
    // the weights are read once: non-temporal hint (cache policy 2)
    w[j] = __builtin_amdgcn_raw_buffer_load_b128(
        make_rsrc(packed + (e0 >> 1), live ? (uint32_t)(ne >> 1) : 0u), lane_w, 0, 2);
    const int64_t ub = e0 >> log2bs;             // block of the first weight
    const int64_t ue = (e0 + ne - 1) >> log2bs;  // block of the last weight
    const uint32_t nbl = live ? (uint32_t)(ue - ub + 1) : 0u;
    if constexpr (DQ && UG) {
      sq[j] = __builtin_amdgcn_raw_buffer_load_b8(make_rsrc(sc.q + ub, nbl), lane_b, 0, 0);
      sa[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           make_rsrc(sc.absmax2 + (ub >> sc.log2bs2), live ? 4u : 0u),
                                           0, 0, 0));
    } else if constexpr (DQ) {
      sq[j] = __builtin_amdgcn_raw_buffer_load_b8(make_rsrc(sc.q + ub, nbl), lane_b, 0, 0);
      const int64_t g0 = ub >> sc.log2bs2;
      const uint32_t ng = live ? (uint32_t)((ue >> sc.log2bs2) - g0 + 1) : 0u;
      const uint32_t gl = ((uint32_t)(ub & ((1 << sc.log2bs2) - 1)) + lane_b) >> sc.log2bs2;
      sa[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           make_rsrc(sc.absmax2 + g0, ng << 2), gl << 2, 0, 0));
    } else {
      sa[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           make_rsrc(sc.absmax + ub, nbl << 2), lane_b << 2, 0, 0));
    }
  };
  issue(0, 0, T > 0, 0);
  // the bias of the run's first 64 rows, lane i holding row i's, read ahead
  // of every item so that finishing a row never waits on a new load
  // (raw bits, through a bounded buffer load: no branch, so no wait here)
  uint32_t bias_run = 0;
  {
    const int64_t nb = bias ? (nrows < 64 ? nrows : 64) : 0;
    if (ydt == kF32)
      bias_run = __builtin_amdgcn_raw_buffer_load_b32(
          make_rsrc(static_cast<const float *>(bias) + r_begin, (uint32_t)(nb * 4)), lane * 4, 0, 0);
    else
      bias_run = __builtin_amdgcn_raw_buffer_load_b16(
          make_rsrc(static_cast<const uint16_t *>(bias) + r_begin, (uint32_t)(nb * 2)), lane * 2, 0,
          0);
  }

  // the table first: it waits on no load, so it is built while the
  // activations and the DQ table are still on their way
  build_pair_table<kM1Threads>(lut, table, tid);
  if constexpr (XLDS) {
    // x as 16-byte chunks, transposed: chunk q (8 values) of piece pc goes to
    // ((pc / 64) * 4 + q) * 64 + pc % 64
    // chunks past the end of x, up to whole slices, are zero: a lane past the
    // row's last piece then multiplies its (zero) codes by zero activations
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const int c = i * kM1Threads + tid;
      const int m = c / rch, cr = c - m * rch;
      const int pc = cr >> 2, q = cr & 3;
      if (m < MR) reinterpret_cast<uint4 *>(xl)[m * rch + (((pc >> 6) << 2) + q) * 64 + (pc & 63)] = xch[i];
    }
  }
  if constexpr (DQ) {
    if (tid < 256) code2[tid] = c2v;
  }
  __syncthreads();
  const uint32_t lane_sel = (uint32_t)lane << 2;
  const char *lut_bytes = reinterpret_cast<const char *>(lut);
  const uint4v *xlv = reinterpret_cast<const uint4v *>(xl);

  // activations of every slice, when they stay in registers
  uint4v xr[SX > 0 ? MR : 1][SX > 0 ? SX : 1][4];
#pragma unroll
  for (int m = 0; m < (SX > 0 ? MR : 0); ++m)
#pragma unroll
    for (int s = 0; s < SX; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q) xr[m][s][q] = xlv[m * rch + s * 256 + q * 64 + lane];

  // sums over the item of T[code] * x, before the block scale, into part[m]
  auto decode = [&](const uint4v &wd, const uint4v (*xq)[4], float *part) {
#pragma unroll
    for (int m = 0; m < MR; ++m) part[m] = 0.f;
#pragma unroll
    for (int bb = 0; bb < 16; ++bb) {
      const uint32_t addr =
          __builtin_amdgcn_perm(wd[bb >> 2], lane_sel, 0x0c0c0000u | ((4u + (bb & 3)) << 8));
      const uint32_t tv = *reinterpret_cast<const uint32_t *>(lut_bytes + addr);
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const uint32_t xv = xq[m][bb >> 2][bb & 3];
        part[m] = dot2<XDT>(tv, xv, part[m]);
      }
    }
  };
  auto finish_row = [&](int64_t rr, const float *acc) {
    const int64_t n = r_begin + rr;
    float b = 0.f;
    if (bias) {
      if (rr < 64) {
        const uint32_t bits = (uint32_t)__builtin_amdgcn_readlane((int)bias_run, (int)rr);
        b = ydt == kF32 ? __builtin_bit_cast(float, bits)
                        : (ydt == kBF16 ? bits16_to_f32<kBF16>(bits) : bits16_to_f32<kF16>(bits));
      } else {
        b = bias_value(bias, ydt, n);
      }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float v = wave_sum(acc[m]);
      if (bias) v = v + b;
      if (lane == m) {
        if (ydt == kF32) {
          static_cast<float *>(y)[m * N + n] = v;
        } else {  // both roundings computed, one selected: no branch
          const uint32_t h = ydt == kBF16 ? f32_to_bf16_rne(v) : f32_to_f16_rne(v);
          static_cast<uint16_t *>(y)[m * N + n] = (uint16_t)h;
        }
      }
    }
  };

  // block scale of an item's piece.  The code byte stays 8 bits wide until
  // here: widened where it is loaded, the widening would be hoisted ahead of
  // the loop and wait for the first item's loads before the second is issued.
  auto item_scale = [&](uint8_t q8, float a) {
    if constexpr (DQ) {
      return code2[q8] * a + offset;
    } else {
      return a;
    }
  };

  float acc[MR], part[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.f;
  if constexpr (SX > 0) {
    // slot and slice of every step known at compile time: unroll lcm(2, SX)
    constexpr int U = SX == 3 ? 6 : (SX == 1 ? 2 : SX);
    for (int64_t t0 = 0; t0 < T; t0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t t = t0 + u;
        if (t >= T) break;
        const int j = u & 1, s = u % SX;
        issue((t + 1) / SX, (u + 1) % SX, t + 1 < T, j ^ 1);
        // keep the item's loads together, ahead of the decode
        __builtin_amdgcn_sched_barrier(0);
        const float ahat = item_scale(sq[j], sa[j]);
        uint4v xq[MR][4];
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q) xq[m][q] = xr[m][s][q];
        decode(w[j], xq, part);
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[m] = fmaf(ahat, part[m], acc[m]);
        if (s == SX - 1) {
          finish_row(t / SX, acc);
#pragma unroll
          for (int m = 0; m < MR; ++m) acc[m] = 0.f;
        }
      }
    }
  } else if (MR <= 2 && XLDS && nrows >= 2) {
    // one or two activation rows too long for registers: weight rows in
    // pairs, slice by slice, so that each slice's activations are read from
    // LDS once for two items; item (2 p + r, s) decodes from slot r.  An odd
    // last row is paired with a dead one (its loads move nothing, its sums
    // are dropped).
    const int64_t np = (nrows + 1) >> 1;
    float acc2[2][MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc2[0][m] = acc2[1][m] = 0.f;
    for (int64_t p = 0; p < np; ++p) {
      const bool two = 2 * p + 1 < nrows;
      for (int s = 0; s < S; ++s) {
        uint4v xq[MR][4];
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q) xq[m][q] = xlv[m * rch + s * 256 + q * 64 + lane];
        issue(2 * p + 1, s, two, 1);
        __builtin_amdgcn_sched_barrier(0);
        float a = item_scale(sq[0], sa[0]);
        decode(w[0], xq, part);
#pragma unroll
        for (int m = 0; m < MR; ++m) acc2[0][m] = fmaf(a, part[m], acc2[0][m]);
        const bool more = s + 1 < S;
        issue(more ? 2 * p : 2 * p + 2, more ? s + 1 : 0, more || p + 1 < np, 0);
        __builtin_amdgcn_sched_barrier(0);
        a = item_scale(sq[1], sa[1]);
        decode(w[1], xq, part);
#pragma unroll
        for (int m = 0; m < MR; ++m) acc2[1][m] = fmaf(a, part[m], acc2[1][m]);
      }
      finish_row(2 * p, acc2[0]);
      if (two) finish_row(2 * p + 1, acc2[1]);
#pragma unroll
      for (int m = 0; m < MR; ++m) acc2[0][m] = acc2[1][m] = 0.f;
    }
  } else {
    int64_t rd = 0, rn = 0;  // row (within the run) of the item decoded / issued next
    int sd = 0, sn = 1;      // and its slice
    if (sn == S) {
      sn = 0;
      ++rn;
    }
    for (int64_t t0 = 0; t0 < T; t0 += 2) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t t = t0 + j;
        if (t >= T) break;
        issue(rn, sn, t + 1 < T, j ^ 1);
        __builtin_amdgcn_sched_barrier(0);
        if (++sn == S) {
          sn = 0;
          ++rn;
        }
        uint4v xq[MR][4];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          if constexpr (XLDS) {
#pragma unroll
            for (int q = 0; q < 4; ++q) xq[m][q] = xlv[m * rch + sd * 256 + q * 64 + lane];
          } else {
            // a lane past the row's last piece multiplies its (zero) codes by
            // zero activations, so it adds nothing
            const int64_t pc = (int64_t)sd * 64 + lane;
            const uint4v *xp =
                reinterpret_cast<const uint4v *>(x + m * K + ((pc < pieces ? pc : 0) << 5));
#pragma unroll
            for (int q = 0; q < 4; ++q) xq[m][q] = pc < pieces ? xp[q] : uint4v{0, 0, 0, 0};
          }
        }
        const float ahat = item_scale(sq[j], sa[j]);
        decode(w[j], xq, part);
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[m] = fmaf(ahat, part[m], acc[m]);
        if (sd == S - 1) {
          finish_row(rd, acc);
#pragma unroll
          for (int m = 0; m < MR; ++m) acc[m] = 0.f;
        }
        if (++sd == S) {
          sd = 0;
          ++rd;
        }
      }
    }
  }
}

// Plain fp32 path (fp32 activations): a wave per row, fp32 table values and
// fp32 multiply-adds.
constexpr int kF32Rows = 4;    // rows a wave of the fp32 kernel works on together
constexpr int kF32Pieces = 2;  // 16-byte pieces per lane and row in flight

template <int M, int XDT, int YDT, bool DQ, int QT>
__global__ __launch_bounds__(256) void gemv_4bit_f32x_kernel(const void *__restrict__ xv, int64_t N,
                                                        int64_t K, const uint8_t *__restrict__ packed,
                                                        Scales sc, int log2bs, void *__restrict__ yv,
                                                        const void *__restrict__ biasv) {
  using XT = typename Storage<XDT>::type;
  using YT = typename Storage<YDT>::type;
  const YT *bias = static_cast<const YT *>(biasv);
  const XT *x = static_cast<const XT *>(xv);
  YT *y = static_cast<YT *>(yv);
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = __uint_as_float(table_bits(QT)[threadIdx.x]);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int64_t pieces = K >> 5;  // 16-byte pieces per row
  const float offset = DQ ? sc.offset[0] : 0.f;

  // a wave takes RW rows at a time and issues the packed words and scales of
  // PL pieces per lane of every row before decoding any (addresses clamped,
  // so the loads are unconditional; a dead slot gets a zero scale).  Each
  // lane adds its pieces in ascending order, then the wave's lanes are summed.
  for (int64_t n0 = wave * kF32Rows; n0 < N; n0 += nwaves * kF32Rows) {
    float acc[kF32Rows][M];
#pragma unroll
    for (int r = 0; r < kF32Rows; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
    for (int64_t pb = 0; pb < pieces; pb += 64 * kF32Pieces) {
      uint4 pk[kF32Rows][kF32Pieces];
      float a[kF32Rows][kF32Pieces];
#pragma unroll
      for (int r = 0; r < kF32Rows; ++r) {
        const int64_t row = n0 + r < N ? n0 + r : N - 1;
#pragma unroll
        for (int p = 0; p < kF32Pieces; ++p) {
          const int64_t pc = pb + p * 64 + lane;
          const int64_t e0 = row * K + ((pc < pieces ? pc : pieces - 1) << 5);
          pk[r][p] = *reinterpret_cast<const uint4 *>(packed + (e0 >> 1));
          const float sv = block_scale<DQ>(sc, e0 >> log2bs, offset);
          a[r][p] = (n0 + r < N && pc < pieces) ? sv : 0.f;
        }
      }
#pragma unroll
      for (int p = 0; p < kF32Pieces; ++p) {
        const int64_t pc = pb + p * 64 + lane;
        const int64_t pcc = pc < pieces ? pc : pieces - 1;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          // the piece's 32 activations of row m as eight 16-byte loads
          float xv[32];
          const float4 *xr = reinterpret_cast<const float4 *>(x + m * K + (pcc << 5));
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float4 f = xr[q];
            xv[4 * q] = f.x;
            xv[4 * q + 1] = f.y;
            xv[4 * q + 2] = f.z;
            xv[4 * q + 3] = f.w;
          }
#pragma unroll
          for (int r = 0; r < kF32Rows; ++r) {
            const uint32_t pw[4] = {pk[r][p].x, pk[r][p].y, pk[r][p].z, pk[r][p].w};
            float sum = 0.f;
#pragma unroll
            for (int b = 0; b < 16; ++b) {
              const uint32_t byte = (pw[b >> 2] >> (8 * (b & 3))) & 0xffu;
              sum = fmaf(lut[byte >> 4], xv[2 * b], sum);
              sum = fmaf(lut[byte & 15u], xv[2 * b + 1], sum);
            }
            acc[r][m] = fmaf(a[r][p], sum, acc[r][m]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kF32Rows; ++r) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float v = acc[r][m];
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        acc[r][m] = v;
      }
      if (lane == 0 && n0 + r < N) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float v = acc[r][m];
          if (bias) v = v + load_elem<YDT>(bias, n0 + r);  // one fp32 add, then one rounding
          store_elem<YDT>(y, m * N + n0 + r, v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int M, int YDT>
static hipError_t launch_f32x_m(const void *x, int64_t N, int64_t K, const uint8_t *packed,
                                const Scales &sc, bool dq, int log2bs, int qt, void *y,
                                const void *bias, hipStream_t st) {
  const unsigned grid = (unsigned)std::min<int64_t>((N + 4 * kF32Rows - 1) / (4 * kF32Rows), 1 << 16);
#define QMV_G(DQV, QTV)                                                                       \
  hipLaunchKernelGGL((gemv_4bit_f32x_kernel<M, kF32, YDT, DQV, QTV>), dim3(grid), dim3(256), 0, \
                     st, x, N, K, packed, sc, log2bs, y, bias)
  if (dq) {
    if (qt == kNF4) QMV_G(true, kNF4); else QMV_G(true, kFP4);
  } else {
    if (qt == kNF4) QMV_G(false, kNF4); else QMV_G(false, kFP4);
  }
#undef QMV_G
  return hipGetLastError();
}

template <int YDT>
static hipError_t launch_f32x(const void *x, int M, int64_t N, int64_t K, const uint8_t *packed,
                              const Scales &sc, bool dq, int log2bs, int qt, void *y,
                              const void *bias, hipStream_t st) {
  switch (M) {
#define QMV_C(MV) case MV: return launch_f32x_m<MV, YDT>(x, N, K, packed, sc, dq, log2bs, qt, y, bias, st);
    QMV_C(1) QMV_C(2) QMV_C(3) QMV_C(4) QMV_C(5) QMV_C(6) QMV_C(7)
#undef QMV_C
    default: return launch_f32x_m<8, YDT>(x, N, K, packed, sc, dq, log2bs, qt, y, bias, st);
  }
}

// fp32 -> bf16 / fp16 bits, round to nearest even, on the host.
static uint32_t host_bits16(float f, int dt) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (dt == kBF16) return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

static Table16 host_table16(int qt, int dt) {
  Table16 t;
  const uint32_t *bits = table_bits(qt);
  for (int c = 0; c < 16; ++c) t.h[c] = host_bits16(__builtin_bit_cast(float, bits[c]), dt);
  return t;
}

// Compute units of the current device (cached per device).
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int resident_wgs_per_cu(const void *kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1)
    n = 1;
  return n;
}

template <int M, int XDT>
static hipError_t launch_lut_m(const void *x, int64_t N, int64_t K, const uint8_t *packed,
                               const Scales &sc, bool dq, int log2bs, int qt, void *y, int ydt,
                               const void *bias, hipStream_t st) {
  constexpr int kGemvThreads = LutShape<M>::kThreads;
  const int64_t waves_per_wg = kGemvThreads / 64;
  int64_t grid = (int64_t)device_cu_count() * LutShape<M>::kWgPerCu;
  grid = std::min<int64_t>(grid, (N + waves_per_wg - 1) / waves_per_wg);
  const int64_t total_waves = grid * waves_per_wg;
  const int rpw = (int)(N / total_waves), rem = (int)(N % total_waves);
  const uint16_t *xh = static_cast<const uint16_t *>(x);
  const Table16 table = host_table16(qt, XDT);
  if (dq)
    hipLaunchKernelGGL((gemv_4bit_lut_kernel<M, XDT, true>), dim3((unsigned)grid),
                       dim3(kGemvThreads), 0, st, xh, N, K, packed, sc, log2bs, table, y, ydt,
                       rpw, rem, bias);
  else
    hipLaunchKernelGGL((gemv_4bit_lut_kernel<M, XDT, false>), dim3((unsigned)grid),
                       dim3(kGemvThreads), 0, st, xh, N, K, packed, sc, log2bs, table, y, ydt,
                       rpw, rem, bias);
  return hipGetLastError();
}

template <int XDT, int MR>
static hipError_t launch_m1(const void *x, int64_t N, int64_t K, const uint8_t *packed,
                            const Scales &sc, bool dq, int log2bs, int qt, void *y, int ydt,
                            const void *bias, hipStream_t st) {
  const int64_t waves_per_wg = kM1Threads / 64;
  int64_t grid = (int64_t)device_cu_count();
  grid = std::min<int64_t>(grid, (N + waves_per_wg - 1) / waves_per_wg);
  const int64_t total_waves = grid * waves_per_wg;
  const int rpw = (int)(N / total_waves), rem = (int)(N % total_waves);
  const uint16_t *xh = static_cast<const uint16_t *>(x);
  const Table16 table = host_table16(qt, XDT);
  // the MR activation rows staged in LDS as whole slices of 16-byte chunks
  // (the tail of the last one zero-filled), XC chunks per thread
  const int64_t slices = (K + 2047) / 2048;
  const int64_t need = (MR * slices * 256 + kM1Threads - 1) / kM1Threads;
  const int xc = MR * slices * 4096 > kM1XLdsBytes
                     ? 0
                     : (need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 6);
  // slices per row held in registers: all of them, up to 4 slice-rows
  const int sx = (xc > 0 && MR * slices <= 4) ? (int)slices : 0;
  // one double-quant group per item: whole slices, and a slice's blocks
  // (2048 / blocksize, at least one) within a group
  const int64_t slice_blocks = log2bs >= 11 ? 1 : (int64_t)1 << (11 - log2bs);
  const bool ug = dq && K % 2048 == 0 && slice_blocks <= ((int64_t)1 << sc.log2bs2);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kM1Threads), 0, st, xh, N, K, packed, sc,
                       log2bs, table, y, ydt, rpw, rem, bias);
  };
#define QMV_M1(DQV, XCV, SV)                                               \
  if (DQV && ug) go(gemv_4bit_m1_kernel<XDT, DQV, XCV, SV, DQV, MR>);      \
  else go(gemv_4bit_m1_kernel<XDT, DQV, XCV, SV, false, MR>)
#define QMV_M1X(DQV)                                                       \
  if (sx == 1) { QMV_M1(DQV, 1, 1); }                                      \
  else if constexpr (MR <= 2) {                                            \
    if (sx == 2) { QMV_M1(DQV, 1, 2); }                                    \
    else if constexpr (MR == 1) {                                          \
      if (sx == 3) { QMV_M1(DQV, 1, 3); }                                  \
      else if (sx == 4) { QMV_M1(DQV, 1, 4); }                             \
      else QMV_M1XC(DQV);                                                  \
    } else QMV_M1XC(DQV);                                                  \
  } else QMV_M1XC(DQV)
#define QMV_M1XC(DQV)                                                      \
  switch (xc) {                                                            \
    case 0: QMV_M1(DQV, 0, 0); break;                                      \
    case 1: QMV_M1(DQV, 1, 0); break;                                      \
    case 2: QMV_M1(DQV, 2, 0); break;                                      \
    case 4: QMV_M1(DQV, 4, 0); break;                                      \
    default: QMV_M1(DQV, 6, 0); break;                                     \
  }
  if (dq) {
    QMV_M1X(true);
  } else {
    QMV_M1X(false);
  }
#undef QMV_M1XC
#undef QMV_M1X
#undef QMV_M1
  return hipGetLastError();
}

template <int XDT>
static hipError_t launch_lut(const void *x, int M, int64_t N, int64_t K, const uint8_t *packed,
                             const Scales &sc, bool dq, int log2bs, int qt, void *y, int ydt,
                             const void *bias, hipStream_t st) {
  // 1 to 4 rows: the item-pipelined kernel, while the activation rows fit
  // in its LDS copy (longer rows of 2 to 4 activation rows take the table
  // kernel below, which re-reads them per slice from the cache)
  const int64_t slices = (K + 2047) / 2048;
  if (M == 1) return launch_m1<XDT, 1>(x, N, K, packed, sc, dq, log2bs, qt, y, ydt, bias, st);
  if (M <= 4 && M * slices * 4096 <= kM1XLdsBytes) {
    if (M == 2) return launch_m1<XDT, 2>(x, N, K, packed, sc, dq, log2bs, qt, y, ydt, bias, st);
    if (M == 3) return launch_m1<XDT, 3>(x, N, K, packed, sc, dq, log2bs, qt, y, ydt, bias, st);
    return launch_m1<XDT, 4>(x, N, K, packed, sc, dq, log2bs, qt, y, ydt, bias, st);
  }
  switch (M) {
#define QMV_C(MV) case MV: return launch_lut_m<MV, XDT>(x, N, K, packed, sc, dq, log2bs, qt, y, ydt, bias, st);
    QMV_C(1) QMV_C(2) QMV_C(3) QMV_C(4) QMV_C(5) QMV_C(6) QMV_C(7)
#undef QMV_C
    default: return launch_lut_m<8, XDT>(x, N, K, packed, sc, dq, log2bs, qt, y, ydt, bias, st);
  }
}

hipError_t launch_gemv_4bit(const void *x, int x_dtype, int M, int64_t N, int64_t K,
                            const uint8_t *packed, const Scales &sc, bool dq, int log2bs, int qt,
                            void *y, int y_dtype, const void *bias, hipStream_t st) {
  // 4 to 8 rows of 16-bit activations, or 2 to 3 rows too long for the
  // item-pipelined kernel's LDS copy: the MFMA kernel of gemm_4bit (the
  // table kernel's dot products grow with M, the MFMA's do not)
  const bool rows_fit = (int64_t)M * ((K + 2047) / 2048) * 4096 <= kM1XLdsBytes;
  if (x_dtype != kF32 && (M >= 4 || (M >= 2 && !rows_fit)) && gemm_narrow_eligible(M, K, log2bs))
    return launch_gemm_4bit(x, x_dtype, M, N, K, packed, sc, dq, log2bs, qt, y, y_dtype, bias, st);
  if (x_dtype == kBF16) return launch_lut<kBF16>(x, M, N, K, packed, sc, dq, log2bs, qt, y, y_dtype, bias, st);
  if (x_dtype == kF16) return launch_lut<kF16>(x, M, N, K, packed, sc, dq, log2bs, qt, y, y_dtype, bias, st);
  if (y_dtype == kF32) return launch_f32x<kF32>(x, M, N, K, packed, sc, dq, log2bs, qt, y, bias, st);
  if (y_dtype == kF16) return launch_f32x<kF16>(x, M, N, K, packed, sc, dq, log2bs, qt, y, bias, st);
  return launch_f32x<kBF16>(x, M, N, K, packed, sc, dq, log2bs, qt, y, bias, st);
}

}  // namespace qmv
