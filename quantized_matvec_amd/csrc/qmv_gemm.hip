// gemm_4bit: C[M, N] = A[M, K] @ W_hat[N, K]^T for general M
// ("Feat/mps gemm 4bit bf16", table "What runs natively now": gemm_4bit).
//
// The pages' design dequantizes into a scratch buffer and then runs a GEMM.
// Here the weight never leaves the chip in bf16: it is read packed, decoded
// on the fly and consumed by bf16 matrix-core instructions
// (v_mfma_f32_32x32x16_bf16) with fp32 accumulation.  Three kernels, by the
// number of rows M (launch_gemm_4bit picks one):
//  * gemm_4bit_narrow_kernel (M <= 16): split-K over 32-column workgroups,
//    operands staged through LDS-direct loads, block scale applied per step;
//  * gemm_4bit_skinny_kernel (M <= 64): split-K over 32-column workgroups,
//    operands loaded straight into registers;
//  * gemm_4bit_kernel (the rest): BM x BN C tiles, weight tiles dequantized
//    by VALU into double-buffered LDS tiles.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "qmv_launch.hpp"

namespace qmv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;

// One 32 x 32 x 16 matrix-core step on 16-bit inputs of type ADT (bf16 or
// fp16; operands carried as raw 16-bit patterns, 8 k-values per lane), fp32
// accumulation: v_mfma_f32_32x32x16_bf16 or v_mfma_f32_32x32x16_f16.
template <int ADT>
__device__ __forceinline__ f32x16_t mfma16(const bf16x8_t &a, const bf16x8_t &b, const f32x16_t &c) {
  if constexpr (ADT == kBF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                   __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Output element with the optional bias: fp32 accumulator + fp32(bias[n]),
// one fp32 addition, then one rounding to the output type.
template <int CDT>
__device__ __forceinline__ void store_out(typename Storage<CDT>::type *C, int64_t idx, float v,
                                          const typename Storage<CDT>::type *bias, int64_t n) {
  if (bias) v = v + load_elem<CDT>(bias, n);
  store_elem<CDT>(C, idx, v);
}

// Tile: BM (M, 128 or 256) x BN (N, 128 or 64) x 64 (K) for NT = 2 BM
// threads; the waves form (BM / 64) x WN, each computing 64 x BN / WN as
// 2 x NJ accumulators of v_mfma_f32_32x32x16_bf16.  LDS rows are padded to
// 72 bf16 (144 bytes) so that the 32 rows an operand read touches fall in
// different banks.  Two LDS stages: while the matrix cores consume stage k,
// the global loads of tile k + 1 are in flight, and they are dequantized
// into the other stage afterwards (one barrier per k-tile).  BN = 64 doubles
// the workgroups for row counts whose 128-wide tiles would leave compute
// units idle; BM = 256 halves how often a weight tile is dequantized.
constexpr int kBK = 64;
constexpr int kLd = kBK + 8;  // padded row, bf16 elements

struct Table16f {
  float v[16];
};

template <int ADT, int CDT, bool DQ, int BM, int BN>
__global__ __launch_bounds__(2 * BM, BM == 128 ? 2 : 1) void gemm_4bit_kernel(const uint16_t *__restrict__ A, int64_t M,
                                                           int64_t N, int64_t K,
                                                           const uint8_t *__restrict__ packed,
                                                           Scales sc, int log2bs, Table16f table,
                                                           void *__restrict__ Cv,
                                                           const void *__restrict__ biasv) {
  constexpr int NT = 2 * BM;                // threads
  constexpr int kStage = (BM + BN) * kLd;   // bf16 elements per stage
  constexpr int WN = NT / 64 / (BM / 64);   // waves along N (2)
  constexpr int NJ = BN / WN / 32;          // 32-column accumulators per wave
  constexpr int BPT = BN * kBK / NT;        // weights per thread and tile: 32 or 16
  constexpr int TPR = kBK / BPT;            // threads per weight row: 2 or 4
  static_assert(NJ >= 1 && (BPT == 32 || BPT == 16), "tile shape");
  using CT = typename Storage<CDT>::type;
  using PW = typename std::conditional<BPT == 32, uint4, uint2>::type;  // packed bytes per thread
  CT *C = static_cast<CT *>(Cv);
  const CT *bias = static_cast<const CT *>(biasv);
  const float dq_offset = DQ ? sc.offset[0] : 0.f;  // read once, not per tile
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStage];
  __shared__ float2 lut2[256];  // packed byte -> (T[byte >> 4], T[byte & 15])
  __shared__ float code2[256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t KT = (K + kBK - 1) / kBK;
  const bool k_tail = (K % kBK) != 0;  // last tile has 32 of 64 columns

  // loader roles: thread t moves row t / 2, columns [32 (t % 2), +32) of the
  // A tile, and row t / TPR, columns [BPT (t % TPR), +BPT) of the weight tile
  const int lr = tid >> 1, lh = tid & 1;
  const int br = tid / TPR, bq = tid % TPR;
  const int64_t arow = m0 + lr < M ? m0 + lr : M - 1;  // rows past M are never stored
  const int64_t brow = n0 + br < N ? n0 + br : N - 1;  // columns past N likewise
  // two register sets: tile k + 2 is loaded while tile k is multiplied and
  // tile k + 1 (loaded an iteration earlier) is staged
  uint4 ra_[2][4];
  PW rb_[2];
  float rsa_[2];
  uint32_t rsq_[2];
  auto load_tile = [&](int64_t kt, auto slot_tag) {
    constexpr int SL = decltype(slot_tag)::value;
    uint4(&ra)[4] = ra_[SL];
    int64_t k = kt * kBK + 32 * lh;
    if (k >= K) k = K - 32;  // the missing half of a tail tile (zeroed when staged)
    const uint4 *ap = reinterpret_cast<const uint4 *>(A + arow * K + k);
#pragma unroll
    for (int q = 0; q < 4; ++q) ra[q] = ap[q];
    int64_t kb = kt * kBK + BPT * bq;
    if (kb >= K) kb = K - BPT;  // likewise
    const int64_t e0 = brow * K + kb;
    rb_[SL] = *reinterpret_cast<const PW *>(packed + (e0 >> 1));
    const int64_t b = e0 >> log2bs;
    if constexpr (DQ) {
      rsq_[SL] = sc.q[b];
      rsa_[SL] = sc.absmax2[b >> sc.log2bs2];
    } else {
      rsa_[SL] = sc.absmax[b];
    }
  };
  auto stage_tile = [&](int64_t kt, int buf, auto slot_tag) {
    constexpr int SL = decltype(slot_tag)::value;
    const uint4(&ra)[4] = ra_[SL];
    const float rsa = rsa_[SL];
    const uint32_t rsq = rsq_[SL];
    (void)rsq;
    uint16_t *As = smem + buf * kStage;
    uint16_t *Bs = As + BM * kLd;
    const bool last = k_tail && kt == KT - 1;
    const bool zero_a = last && lh == 1;
    uint4 *ad = reinterpret_cast<uint4 *>(As + lr * kLd + 32 * lh);
#pragma unroll
    for (int q = 0; q < 4; ++q) ad[q] = zero_a ? make_uint4(0, 0, 0, 0) : ra[q];
    const bool zero_b = last && BPT * bq >= 32;
    const float a = zero_b ? 0.f : (DQ ? code2[rsq] * rsa + dq_offset : rsa);
    uint32_t pw[BPT / 8];
    __builtin_memcpy(pw, &rb_[SL], sizeof(pw));
    uint32_t o[BPT / 2];
#pragma unroll
    for (int bb = 0; bb < BPT / 2; ++bb) {
      const float2 t = lut2[(pw[bb >> 2] >> (8 * (bb & 3))) & 0xffu];
      // dequantized weights: fp32(T * a_hat) rounded to the input's 16-bit
      // type (nearest even), as dequantize_4bit returns them
      o[bb] = cvt_pair<ADT>(t.x * a, t.y * a);
    }
    uint4 *bd = reinterpret_cast<uint4 *>(Bs + br * kLd + BPT * bq);
#pragma unroll
    for (int q = 0; q < BPT / 8; ++q) bd[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  load_tile(0, S0{});
  load_tile(KT > 1 ? 1 : 0, S1{});
  if (tid < 256) {
    lut2[tid] = make_float2(table.v[tid >> 4], table.v[tid & 15]);
    if constexpr (DQ) code2[tid] = sc.code2[tid];
  }
  __syncthreads();
  stage_tile(0, 0, S0{});
  __syncthreads();

  f32x16_t acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto mma_tile = [&](int buf) {
    const uint16_t *As = smem + buf * kStage;
    const uint16_t *Bs = As + BM * kLd;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8_t af[2], bfr[NJ];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8_t *>(As + row * kLd + ks * 16 + (lane >> 5) * 8);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = wn * (BN / WN) + j * 32 + (lane & 31);
        bfr[j] = *reinterpret_cast<const bf16x8_t *>(Bs + col * kLd + ks * 16 + (lane >> 5) * 8);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = mfma16<ADT>(af[i], bfr[j], acc[i][j]);
    }
  };

  // tile kt sits in LDS stage kt % 2 and tile kt + 1 in register set (kt + 1) % 2;
  // each step loads tile kt + 2 into the register set tile kt used
  // (loads past the end re-read the last tile, so they are unconditional)
  auto clampk = [&](int64_t k) { return k < KT ? k : KT - 1; };
  int64_t kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    load_tile(clampk(kt + 2), S0{});
    mma_tile(0);
    stage_tile(kt + 1, 1, S1{});
    __syncthreads();
    load_tile(clampk(kt + 3), S1{});
    mma_tile(1);
    if (kt + 2 < KT) stage_tile(kt + 2, 0, S0{});
    __syncthreads();
  }
  if (kt < KT) mma_tile(0);  // odd tile count: the last tile is in stage 0

  // 32 x 32 accumulator layout: column = lane % 32,
  // row = 8 * (r / 4) + 4 * (lane / 32) + r % 4 for accumulator register r.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t col = n0 + wn * (BN / WN) + j * 32 + (lane & 31);
      if (col >= N) continue;
      // one bias value per column: the fp32 result + fp32(bias[col]), then
      // one rounding (no addition at all without a bias, so -0 stays -0)
      const float b = bias ? load_elem<CDT>(bias, col) : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) store_elem<CDT>(C, row * N + col, bias ? acc[i][j][r] + b : acc[i][j][r]);
      }
    }
}

// ---------------------------------------------------------------------------
// Skinny M (M <= 32 MT <= 64): gemm_4bit_skinny_kernel
//
// A workgroup of KW waves owns 32 output columns (weight rows n0 .. n0 + 31)
// and all M rows (MT tiles of 32); its waves split K (wave w takes the 64-wide
// k-steps w, w + KW, ...) and their partial tiles are summed through LDS at
// the end, in wave order.  With N / 32 workgroups the grid fills the GPU even
// for a handful of rows.
//
// No LDS staging: each lane loads exactly its operands of
// v_mfma_f32_32x32x16_bf16.  In k-step s lane l covers column n0 + l % 32 and
// the 32 k-values 64 s + 32 (l / 32) .. + 31 (one 16-byte packed load, one
// block scale); the order of k inside the four MFMAs of the step is chosen so
// that MFMA j takes that lane's k-values 8 j .. 8 j + 7 (a sum does not depend
// on the order of its terms, and A is read in the same order), so every
// operand is a contiguous 16 bytes.  The weights are dequantized in registers
// exactly as in the tile kernel (fp32(T * a_hat) rounded to bf16).  The next
// two steps' loads are issued before the current step is computed.
// ---------------------------------------------------------------------------
template <int ADT, int CDT, bool DQ, int MT, int KW>
__global__ __launch_bounds__(64 * KW) void gemm_4bit_skinny_kernel(
    const uint16_t *__restrict__ A, int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    Scales sc, int log2bs, Table16f table, void *__restrict__ Cv, const void *__restrict__ biasv) {
  using CT = typename Storage<CDT>::type;
  CT *C = static_cast<CT *>(Cv);
  const CT *bias = static_cast<const CT *>(biasv);
  __shared__ float2 lut2[256];  // packed byte -> (T[byte >> 4], T[byte & 15])
  __shared__ float code2[256];
  __shared__ float red[(KW - 1) * MT * 16 * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < 256; i += 64 * KW) {
    lut2[i] = make_float2(table.v[i >> 4], table.v[i & 15]);
    if constexpr (DQ) code2[i] = sc.code2[i];
  }
  const float offset = DQ ? sc.offset[0] : 0.f;
  __syncthreads();

  const int kh = lane >> 5;
  const int col = lane & 31;
  const int64_t n0 = (int64_t)blockIdx.x * 32;
  const int64_t n = n0 + col;
  const int64_t nc = n < N ? n : N - 1;  // columns past N are computed, never stored
  const int64_t nsteps = (K + 63) >> 6;
  // Workgroup-uniform bounded buffers (the host keeps every offset below 2^31
  // and K a multiple of 64): rows of A past M and weight rows past N read as
  // zeros.  The prefetch past a wave's last step reads whatever lies there (or
  // zeros) and is never used.
  const uint32_t rowb = (uint32_t)(K >> 1);
  const __amdgpu_buffer_rsrc_t prs =
      make_rsrc(packed + n0 * (int64_t)rowb, (uint32_t)((N - n0 < 32 ? N - n0 : 32) * rowb));
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(A, (uint32_t)(M * K * 2));
  const uint32_t poff = (uint32_t)col * rowb + 16u * kh;
  const uint32_t aoff = (uint32_t)(col * K * 2) + 64u * kh;
  const uint32_t atile = (uint32_t)(32 * K * 2);

  struct Regs {
    uint4 p;
    uint4 a[MT][4];
    uint32_t q;
    float s;
  };
  auto load = [&](int64_t st, Regs &r) {
    r.p = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(prs, poff + (uint32_t)(32 * st), 0, 0));
    const uint32_t ao = aoff + (uint32_t)(128 * st);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        r.a[t][j] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(ars, ao + t * atile, 16 * j, 0));
    const int64_t sl = st < nsteps ? st : nsteps - 1;
    const int64_t b = (nc * K + 64 * sl + 32 * kh) >> log2bs;
    if constexpr (DQ) {
      r.q = sc.q[b];
      r.s = sc.absmax2[b >> sc.log2bs2];
    } else {
      r.s = sc.absmax[b];
    }
  };

  f32x16_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;

  auto compute = [&](const Regs &r) {
    const float a = DQ ? code2[r.q] * r.s + offset : r.s;
    const uint32_t pw[4] = {r.p.x, r.p.y, r.p.z, r.p.w};
    float2 tv[16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) tv[4 * j + q] = lut2[(pw[j] >> (8 * q)) & 0xffu];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t bw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // dequantized weights: fp32(T * a_hat) rounded to the input's type
        bw[q] = cvt_pair<ADT>(tv[4 * j + q].x * a, tv[4 * j + q].y * a);
      }
      const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, make_uint4(bw[0], bw[1], bw[2], bw[3]));
#pragma unroll
      for (int t = 0; t < MT; ++t)
        acc[t] = mfma16<ADT>(__builtin_bit_cast(bf16x8_t, r.a[t][j]), bop, acc[t]);
    }
  };

  // three register sets: the wave's steps i + 1 and i + 2 are in flight
  // while step i is computed.  No branch separates a load from the
  // computation it feeds (a load that could be moved past the computation
  // before it would be issued late).
  const int64_t nw = nsteps > wave ? (nsteps - wave + KW - 1) / KW : 0;  // this wave's steps
  Regs r0, r1, r2;
  load(wave, r0);
  load(wave + KW, r1);
  int64_t i = 0;
  for (; i + 2 < nw; i += 3) {
    load(wave + (i + 2) * KW, r2);
    compute(r0);
    load(wave + (i + 3) * KW, r0);
    compute(r1);
    load(wave + (i + 4) * KW, r1);
    compute(r2);
  }
  if (i < nw) compute(r0);
  if (i + 1 < nw) compute(r1);

  // sum the waves' partial tiles (wave order) and store
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[(((wave - 1) * MT + t) * 16 + i) * 64 + lane] = acc[t][i];
  }
  __syncthreads();
  if (wave == 0 && n < N) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = acc[t][i];
        for (int w = 1; w < KW; ++w) v += red[(((w - 1) * MT + t) * 16 + i) * 64 + lane];
        // accumulator layout: column = lane % 32, row = 8 (i / 4) + 4 (lane / 32) + i % 4
        const int64_t m = 32 * t + 8 * (i >> 2) + 4 * kh + (i & 3);
        if (m < M) store_out<CDT>(C, m * N + n, v, bias, n);
      }
  }
}

// ---------------------------------------------------------------------------
// Narrow M (M <= MP <= 16, blocks of 64 or more): gemm_4bit_narrow_kernel
//
// A workgroup of KW waves owns 32 output columns (weight rows n0 .. n0 + 31);
// wave w takes a contiguous share of K, in groups of two 64-wide k-steps, and
// the waves' partial tiles are summed through LDS at the end, in wave order.
// With N / 32 workgroups the grid fills the GPU even for a handful of rows.
//
//  * A group's weights (32 rows x 64 bytes) and activations (MP rows x 128
//    k-values) go to a private LDS slot of the wave through LDS-direct buffer
//    loads: the weight loads read 64 contiguous bytes of each of 16 rows per
//    instruction, and nothing in flight holds registers.  NB slots form a
//    ring, NB - 1 groups are in flight, and as loads complete in issue order
//    a wave waits for exactly the oldest group it has in flight.
//  * One v_mfma_f32_32x32x16_bf16 takes, per lane, 8 k-values of one column;
//    lane (column c, half h) holds the 32 k-values 32 h .. 32 h + 31 of a
//    step, and MFMA j takes values 8 j .. 8 j + 7 of them, with the
//    activations read in the same order (the sum is unchanged).  A packed
//    byte is decoded by one LDS lookup into the bf16 pair of its two code
//    values.
//  * A 64-wide step lies inside one block (block size >= 64), so the four
//    MFMAs of a step sum code value x activation into a fresh tile, and the
//    block scale is applied once per step and column, in fp32, as that tile
//    is added to the accumulator.  Only accumulator registers that can hold a
//    row below MP are scaled, reduced and stored.
//
// Slot layout, in 16-byte chunks: 128 weight chunks, chunk 4 r + (p ^ f(r))
// holding 16-byte piece p of row r, f(r) = (r / 4) % 4 (the xor spreads the
// reads of one MFMA operand over the LDS banks); then 16 MP activation
// chunks, chunk ((t * 4 + j) * 2 + h) * MP + m holding the 8 k-values of row
// m that lane (m, h) feeds MFMA j of step t; then one zero chunk, read by
// the lanes of rows MP .. 31.
// ---------------------------------------------------------------------------
template <int N_, class F, int... Us>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Us...>) {
  (f(std::integral_constant<int, Us>{}), ...);
}
template <int N_, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl<N_>(f, std::make_integer_sequence<int, N_>{});
}

// LDS-direct load of 16 bytes per lane: lane i's bytes land at dst + 16 i
// (dst is wave-uniform); out-of-range lanes write zeros.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, uint4 *dst, uint32_t voff) {
  typedef __attribute__((address_space(3))) void lds_void_t;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)dst, 16, voff, 0, 0, 0);
}

template <int ADT, int CDT, bool DQ, int MP, int NB, int KW>
__global__ __launch_bounds__(64 * KW) void gemm_4bit_narrow_kernel(
    const uint16_t *__restrict__ A, int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    Scales sc, int log2bs, Table16f table, void *__restrict__ Cv, const void *__restrict__ biasv) {
  constexpr int WCH = 128;              // weight chunks per group (32 rows x 64 bytes)
  constexpr int ACH = 16 * MP;          // activation chunks per group (MP rows x 128 k-values)
  constexpr int WND = WCH / 64, AND = ACH / 64;  // LDS-direct loads per group
  constexpr int SLOT = WCH + ACH + 1;   // + the zero chunk
  constexpr int RR = MP < 8 ? 4 : MP / 2;  // accumulator registers holding rows < MP (lanes 0..31 hold rows 0..3)
  constexpr int PER = WND + AND + (DQ ? 4 : 2);  // loads per group
  static_assert(MP % 4 == 0 && MP <= 16 && NB >= 2 && NB <= 8 && (NB - 1) * PER < 64 && KW >= 4,
                "narrow gemm shape");
  using CT = typename Storage<CDT>::type;
  CT *C = static_cast<CT *>(Cv);
  __shared__ uint32_t lut[256];  // packed byte -> (T[byte >> 4], T[byte & 15]) as the input type
  __shared__ float code2[256];
  __shared__ float red[(KW - 1) * RR * 64];
  // one array per ring slot, so that the compiler can tell an LDS-direct load
  // into one slot from reads of another
  __shared__ uint4 ring0[KW * SLOT], ring1[KW * SLOT];
  __shared__ uint4 ring2[NB > 2 ? KW * SLOT : 1], ring3[NB > 3 ? KW * SLOT : 1];
  __shared__ uint4 ring4[NB > 4 ? KW * SLOT : 1], ring5[NB > 5 ? KW * SLOT : 1];
  __shared__ uint4 ring6[NB > 6 ? KW * SLOT : 1], ring7[NB > 7 ? KW * SLOT : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto slot = [&](auto U) -> uint4 * {
    constexpr int u = decltype(U)::value;
    uint4 *r = u == 0 ? ring0 : u == 1 ? ring1 : u == 2 ? ring2 : u == 3 ? ring3
             : u == 4 ? ring4 : u == 5 ? ring5 : u == 6 ? ring6 : ring7;
    return r + wave * SLOT;
  };

  const int kh = lane >> 5;
  const int col = lane & 31;
  const int64_t n0 = (int64_t)blockIdx.x * 32;
  const int64_t n = n0 + col;
  const int64_t nc = n < N ? n : N - 1;  // columns past N are computed, never stored
  const int64_t nsteps = K >> 6;         // K % 64 == 0 (host)
  const int64_t ngroups = (nsteps + 1) >> 1;
  const int64_t qg = ngroups / KW, rg = ngroups % KW;
  const int64_t g0 = wave * qg + (wave < rg ? wave : rg);  // this wave's groups: g0 .. g0 + nw - 1
  const int64_t nw = qg + (wave < rg ? 1 : 0);
  // Bounded buffers, uniform per workgroup (the host keeps offsets below
  // 2^31): activation rows past M and weight rows past N read as zeros.
  // Loads past the wave's last group (or past the end of a row) read
  // whatever lies in range, or zeros, and are never used.
  const uint32_t rowb = (uint32_t)(K >> 1);
  const __amdgpu_buffer_rsrc_t prs =
      make_rsrc(packed + n0 * (int64_t)rowb, (uint32_t)((N - n0 < 32 ? N - n0 : 32) * rowb));
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(A, (uint32_t)(M * K * 2));
  uint32_t woff[WND];  // weight piece this lane moves in LDS-direct load d (group 0)
#pragma unroll
  for (int d = 0; d < WND; ++d) {
    const int r = 16 * d + (lane >> 2);
    woff[d] = (uint32_t)r * rowb + 16u * ((lane & 3) ^ ((r >> 2) & 3));
  }
  uint32_t aoff[AND];  // activation chunk this lane moves in LDS-direct load d (group 0)
#pragma unroll
  for (int d = 0; d < AND; ++d) {
    const int c = 64 * d + lane, m = c % MP, q = c / MP;
    aoff[d] = (uint32_t)(m * K * 2) + 128u * (q >> 3) + 64u * (q & 1) + 16u * ((q >> 1) & 3);
  }
  int wrd[2];     // weight chunk this lane reads in step t
  int ard[2][4];  // activation chunk this lane reads for MFMA j of step t
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    wrd[t] = 4 * col + ((2 * t + kh) ^ ((col >> 2) & 3));
#pragma unroll
    for (int j = 0; j < 4; ++j) ard[t][j] = WCH + (col < MP ? ((t * 4 + j) * 2 + kh) * MP + col : ACH);
  }

  float c2v = 0.f, offset = 0.f;
  if constexpr (DQ) {
    if (tid < 256) c2v = sc.code2[tid];
    offset = sc.offset[0];
  }

  struct SR {
    uint32_t q[2];
    float s[2];
  };
  SR sr[NB];
  auto issue = [&](int64_t i, auto U) {  // group i of this wave into ring slot U
    constexpr int u = decltype(U)::value;
    const int64_t g = g0 + i;
    uint4 *dst = slot(U);
#pragma unroll
    for (int d = 0; d < WND; ++d) load_lds16(prs, dst + 64 * d, woff[d] + (uint32_t)(64 * g));
#pragma unroll
    for (int d = 0; d < AND; ++d) load_lds16(ars, dst + WCH + 64 * d, aoff[d] + (uint32_t)(256 * g));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t st = 2 * g + t;
      const int64_t sl = st < nsteps ? st : nsteps - 1;
      const int64_t b = (nc * K + 64 * sl) >> log2bs;  // one block per (column, step)
      if constexpr (DQ) {
        sr[u].q[t] = sc.q[b];
        sr[u].s[t] = sc.absmax2[b >> sc.log2bs2];
      } else {
        sr[u].s[t] = sc.absmax[b];
      }
    }
  };

  // prologue: groups 0 .. NB - 2 in flight while the tables are built
  static_for<NB - 1>([&](auto U) { issue(decltype(U)::value, U); });
  if (tid < 256) {
    lut[tid] = f32_to_bits16<ADT>(table.v[tid >> 4]) | (f32_to_bits16<ADT>(table.v[tid & 15]) << 16);
    if constexpr (DQ) code2[tid] = c2v;
  }
  if (lane < NB) {
    static_for<NB>([&](auto U) {
      if (lane == decltype(U)::value) slot(U)[WCH + ACH] = make_uint4(0, 0, 0, 0);
    });
  }
  __syncthreads();

  float acc[RR];
#pragma unroll
  for (int i = 0; i < RR; ++i) acc[i] = 0.f;

  auto compute = [&](int64_t i, auto U) {
    constexpr int u = decltype(U)::value;
    const uint4 *sl = slot(U);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (2 * (g0 + i) + t < nsteps) {  // wave-uniform
        const uint4 w = sl[wrd[t]];
        const uint32_t pw[4] = {w.x, w.y, w.z, w.w};
        f32x16_t tile;
#pragma unroll
        for (int e = 0; e < 16; ++e) tile[e] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t bw[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) bw[q] = lut[(pw[j] >> (8 * q)) & 0xffu];
          tile = mfma16<ADT>(__builtin_bit_cast(bf16x8_t, sl[ard[t][j]]),
                             __builtin_bit_cast(bf16x8_t, make_uint4(bw[0], bw[1], bw[2], bw[3])), tile);
        }
        const float a = DQ ? code2[sr[u].q[t]] * sr[u].s[t] + offset : sr[u].s[t];  // block scale
#pragma unroll
        for (int e = 0; e < RR; ++e) acc[e] = fmaf(a, tile[e], acc[e]);
      }
    }
  };

  // steady state: issue group i + NB - 1, wait for group i (the oldest in
  // flight: (NB - 1) * PER younger loads may stay outstanding), compute it
  constexpr int kWait = (NB - 1) * PER;
  const int64_t npad = (nw + NB - 1) / NB * NB;
  for (int64_t i0 = 0; i0 < npad; i0 += NB) {
    static_for<NB>([&](auto U) {
      constexpr int u = decltype(U)::value;
      const int64_t i = i0 + u;
      issue(i + NB - 1, std::integral_constant<int, (u + NB - 1) % NB>{});
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt((kWait & 15) | ((kWait >> 4) << 14) | (7 << 4) | (15 << 8));
      asm volatile("" ::: "memory");
      if (i < nw) compute(i, U);
    });
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): no LDS-direct load outlives the loop

  // sum the waves' partial tiles (wave order) and store
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < RR; ++e) red[((wave - 1) * RR + e) * 64 + lane] = acc[e];
  }
  __syncthreads();
  if (wave == 0 && n < N) {
#pragma unroll
    for (int e = 0; e < RR; ++e) {
      float v = acc[e];
      for (int w = 1; w < KW; ++w) v += red[((w - 1) * RR + e) * 64 + lane];
      // accumulator layout: column = lane % 32, row = 8 (e / 4) + 4 (lane / 32) + e % 4
      const int64_t m = 8 * (e >> 2) + 4 * kh + (e & 3);
      if (m < M) store_out<CDT>(C, m * N + n, v, static_cast<const CT *>(biasv), n);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 activations with M > 8: gemm_4bit_f32_kernel
//
// C = A @ W_hat^T with fp32 A, the fp32 dequantized weights fp32(T * a_hat)
// (exactly as dequantize_4bit returns them in fp32), and fp32 products and
// sums on the fp32 matrix cores: v_mfma_f32_32x32x2_f32, where lane l holds
// A[l % 32][l / 32] and B[l / 32][l % 32] of a 32 x 2 x 32 step.  A 128 x 128
// tile of C per workgroup of 4 waves (2 x 2, 64 x 64 each); k-tiles of 32 are
// staged in LDS as fp32 rows of 33 floats, so the 32 rows x 2 columns an
// operand read touches fall in 64 different banks.  Two LDS stages: the
// next tiles' global loads are in flight while the current one is multiplied.
constexpr int kF32BK = 32;
constexpr int kF32Ld = kF32BK + 1;

template <int CDT, bool DQ>
__global__ __launch_bounds__(256, 2) void gemm_4bit_f32_kernel(const float *__restrict__ A, int64_t M,
                                                               int64_t N, int64_t K,
                                                               const uint8_t *__restrict__ packed,
                                                               Scales sc, int log2bs, Table16f table,
                                                               void *__restrict__ Cv,
                                                               const void *__restrict__ biasv) {
  constexpr int BM = 128, BN = 128;
  constexpr int kStage = (BM + BN) * kF32Ld;  // floats per stage
  using CT = typename Storage<CDT>::type;
  CT *C = static_cast<CT *>(Cv);
  const CT *bias = static_cast<const CT *>(biasv);
  const float dq_offset = DQ ? sc.offset[0] : 0.f;
  __shared__ float smem[2 * kStage];
  __shared__ float lut[16];
  __shared__ float code2[256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t KT = K / kF32BK;  // K % 32 == 0

  // loader roles: thread t moves row t / 2, columns [16 (t % 2), +16) of the
  // A tile (four 16-byte loads) and decodes the same span of weight row t / 2
  // (one 8-byte load; 16 weights lie in one block: blocks are 32 or more)
  const int lr = tid >> 1, lh = tid & 1;
  const int64_t arow = m0 + lr < M ? m0 + lr : M - 1;  // rows past M are never stored
  const int64_t brow = n0 + lr < N ? n0 + lr : N - 1;  // columns past N likewise
  float4 ra_[2][4];
  uint2 rb_[2];
  float rsa_[2];
  uint32_t rsq_[2];
  auto load_tile = [&](int64_t kt, auto slot_tag) {
    constexpr int SL = decltype(slot_tag)::value;
    const int64_t k = kt * kF32BK + 16 * lh;
    const float4 *ap = reinterpret_cast<const float4 *>(A + arow * K + k);
#pragma unroll
    for (int q = 0; q < 4; ++q) ra_[SL][q] = ap[q];
    const int64_t e0 = brow * K + k;
    rb_[SL] = *reinterpret_cast<const uint2 *>(packed + (e0 >> 1));
    const int64_t b = e0 >> log2bs;
    if constexpr (DQ) {
      rsq_[SL] = sc.q[b];
      rsa_[SL] = sc.absmax2[b >> sc.log2bs2];
    } else {
      rsa_[SL] = sc.absmax[b];
    }
  };
  auto stage_tile = [&](int buf, auto slot_tag) {
    constexpr int SL = decltype(slot_tag)::value;
    float *As = smem + buf * kStage;
    float *Bs = As + BM * kF32Ld;
    float *ad = As + lr * kF32Ld + 16 * lh;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ad[4 * q] = ra_[SL][q].x;
      ad[4 * q + 1] = ra_[SL][q].y;
      ad[4 * q + 2] = ra_[SL][q].z;
      ad[4 * q + 3] = ra_[SL][q].w;
    }
    const float a = DQ ? code2[rsq_[SL]] * rsa_[SL] + dq_offset : rsa_[SL];
    const uint32_t pw[2] = {rb_[SL].x, rb_[SL].y};
    float *bd = Bs + lr * kF32Ld + 16 * lh;
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      const uint32_t byte = (pw[bb >> 2] >> (8 * (bb & 3))) & 0xffu;  // even element: high nibble
      bd[2 * bb] = lut[byte >> 4] * a;
      bd[2 * bb + 1] = lut[byte & 15u] * a;
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  load_tile(0, S0{});
  load_tile(KT > 1 ? 1 : 0, S1{});
  if (tid < 16) lut[tid] = table.v[tid];
  if constexpr (DQ) code2[tid] = sc.code2[tid];
  __syncthreads();
  stage_tile(0, S0{});
  __syncthreads();

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto mma_tile = [&](int buf) {
    const float *As = smem + buf * kStage;
    const float *Bs = As + BM * kF32Ld;
    const int kl = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < kF32BK / 2; ++ks) {
      float af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = As[(wm * 64 + i * 32 + (lane & 31)) * kF32Ld + 2 * ks + kl];
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = Bs[(wn * 64 + j * 32 + (lane & 31)) * kF32Ld + 2 * ks + kl];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  // tile kt sits in LDS stage kt % 2 and tile kt + 1 in register set (kt + 1) % 2;
  // each step loads tile kt + 2 into the register set tile kt used
  // (loads past the end re-read the last tile, so they are unconditional)
  auto clampk = [&](int64_t k) { return k < KT ? k : KT - 1; };
  int64_t kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    load_tile(clampk(kt + 2), S0{});
    mma_tile(0);
    stage_tile(1, S1{});
    __syncthreads();
    load_tile(clampk(kt + 3), S1{});
    mma_tile(1);
    if (kt + 2 < KT) stage_tile(0, S0{});
    __syncthreads();
  }
  if (kt < KT) mma_tile(0);  // odd tile count: the last tile is in stage 0

  // 32 x 32 accumulator layout: column = lane % 32,
  // row = 8 * (r / 4) + 4 * (lane / 32) + r % 4 for accumulator register r.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= N) continue;
      const float b = bias ? load_elem<CDT>(bias, col) : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) store_elem<CDT>(C, row * N + col, bias ? acc[i][j][r] + b : acc[i][j][r]);
      }
    }
}

// ---------------------------------------------------------------------------
// Large M (M >= 448): gemm_4bit_rb_kernel
//
// A workgroup of 4 waves owns a 128 (M) x 256 (N) tile of C; wave w computes
// all 128 rows x columns [64 w, 64 w + 64) as 4 x 2 accumulators of
// v_mfma_f32_32x32x16_bf16 (f16), one wave per SIMD.  Per k-tile of 64:
//  * the activations go global -> LDS with 16-byte LDS-direct loads into a
//    3-stage ring (128 rows x 128 B per stage; a row's 16-byte chunks are
//    XOR-swizzled by (row / 2) % 8: two 128-byte rows share one 256-byte
//    sweep of the banks, so 16 consecutive rows read at one chunk position
//    land on 16 different 16-byte bank groups), issued two k-tiles ahead;
//  * each wave decodes its own weights straight into MFMA operand registers
//    (no LDS tile for the weights): lane l covers column 32 j + l % 32 and the
//    32 k-values 32 (l / 32) .. + 31 (one 16-byte packed load), so MFMA t
//    takes its k-values 8 t .. 8 t + 7 (the activations are read in the same
//    order).  A packed byte is one v_perm_b32 (its LDS address) and one
//    ds_read_b64 of a 64 KB table of fp32 pairs (T[hi], T[lo]) with 32
//    copies, one per lane of a half-wave (no bank conflicts); the weights
//    are fp32(T * a_hat) rounded to the input type, exactly the
//    dequantize_4bit values;
//  * the packed weights and scales are loaded two k-tiles ahead, into three
//    register sets.
// Workgroups are ordered so that the row tiles of one column tile run on one
// XCD (dispatch is round-robin over the 8 XCDs): its packed weights are read
// from HBM once and then from that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kRbM = 128, kRbN = 256, kRbK = 64;

// Tile (row, column origin) of workgroup `id` of the large-M kernel.
__host__ __device__ inline void rb_tile(int id, int ncol, int nrow, int64_t &m0, int64_t &n0) {
  int cb, rb;
  if (ncol % 8 == 0) {  // XCD k = id % 8 takes column tiles k, k + 8, ..., each for every row tile
    const int xcd = id & 7, s = id >> 3;
    cb = xcd + 8 * (s / nrow);
    rb = s % nrow;
  } else {
    cb = id % ncol;
    rb = id / ncol;
  }
  m0 = (int64_t)rb * kRbM;
  n0 = (int64_t)cb * kRbN;
}

// A buffer resource with its base and size made wave-uniform explicitly (they
// are uniform already; this keeps the descriptor in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_u(const void *base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  return make_rsrc(reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo),
                   __builtin_amdgcn_readfirstlane(bytes));
}

template <int ADT, int CDT, bool DQ>
__global__ __launch_bounds__(256, 1) void gemm_4bit_rb_kernel(
    const uint16_t *__restrict__ A, int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    Scales sc, int log2bs, Table16f table, void *__restrict__ Cv, const void *__restrict__ biasv,
    int ncol, int nrow) {
  using CT = typename Storage<CDT>::type;
  CT *C = static_cast<CT *>(Cv);
  const CT *bias = static_cast<const CT *>(biasv);
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * 32 * 2];  // byte -> (T[hi], T[lo]), 32 copies
  __shared__ float code2[256];
  // one array per ring stage, so that the compiler can tell an LDS-direct
  // load into one stage from reads of another
  __shared__ uint4 st0[kRbM * 8], st1[kRbM * 8], st2[kRbM * 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int64_t m0, n0;
  rb_tile((int)blockIdx.x, ncol, nrow, m0, n0);
  const int KT = (int)(K / kRbK);
  {  // table: 16-byte chunk c holds copies 2 (c % 16) and + 1 of entry c / 16
    const uint32_t lo = __float_as_uint(table.v[(tid >> 4) & 15]);
    uint4 *dst = reinterpret_cast<uint4 *>(lut);
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const uint32_t hi = __float_as_uint(table.v[it]);
      dst[it * 256 + tid] = make_uint4(hi, lo, hi, lo);
    }
  }
  float offset = 0.f;
  if constexpr (DQ) {
    code2[tid] = sc.code2[tid];
    offset = sc.offset[0];
  }
  // activations: wave w moves rows (4 w + d) * 8 + l / 8 of a stage, lane l
  // into position l % 8 of its row, from chunk (l % 8) ^ ((row / 2) % 8); rows
  // past M read zeros (bounded resource)
  const int64_t mrows = M - m0 < kRbM ? M - m0 : kRbM;
  const uint16_t *a_base = A + m0 * K;
  const uint32_t a_bytes = (uint32_t)(mrows * K * 2);
  uint32_t aoff[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int r = (4 * wave + d) * 8 + (lane >> 3);
    aoff[d] = (uint32_t)(r * K * 2) + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
  }
  auto issue_a = [&](int kt, uint4 *stage) {  // k-tiles past the end re-read the last one
    const uint32_t ko = (uint32_t)(kt < KT ? kt : KT - 1) * (kRbK * 2);
    const __amdgpu_buffer_rsrc_t ars = make_rsrc_u(a_base, a_bytes);
#pragma unroll
    for (int d = 0; d < 4; ++d) load_lds16(ars, stage + (4 * wave + d) * 64, aoff[d] + ko);
  };
  // weights: lane -> columns n0 + 64 w + 32 j + l % 32 (j = 0, 1), k half h = l / 32;
  // columns past N read zeros, and their scales are the last column's
  const int h = lane >> 5, colw = lane & 31;
  const int64_t ncols = N - n0 < kRbN ? N - n0 : kRbN;
  const uint32_t rowb = (uint32_t)(K >> 1);
  const uint8_t *p_base = packed + n0 * (int64_t)rowb;
  const uint32_t p_bytes = (uint32_t)(ncols * rowb);
  const int64_t bpr = K >> log2bs;  // blocks per weight row
  uint32_t boff[2];
  int64_t scol[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = 64 * wave + 32 * j + colw;
    boff[j] = (uint32_t)c * rowb + 16u * h;
    scol[j] = n0 + c < N ? n0 + c : N - 1;
  }
  struct BR {
    uint4 w[2];
    uint32_t q[2];
    float s[2];
  };
  auto issue_b = [&](int kt, BR &b) {
    const int kc = kt < KT ? kt : KT - 1;
    const __amdgpu_buffer_rsrc_t prs = make_rsrc_u(p_base, p_bytes);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      b.w[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(prs, boff[j] + (uint32_t)kc * 32u, 0, 0));
      const int64_t blk = scol[j] * bpr + (((int64_t)kc * kRbK + 32 * h) >> log2bs);
      if constexpr (DQ) {
        b.q[j] = sc.q[blk];
        b.s[j] = sc.absmax2[blk >> sc.log2bs2];
      } else {
        b.s[j] = sc.absmax[blk];
      }
    }
  };
  issue_a(0, st0);
  issue_a(1, st1);
  BR br0, br1, br2;
  issue_b(0, br0);
  issue_b(1, br1);
  __syncthreads();  // table and code2

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const uint32_t lane_sel = (uint32_t)colw << 3;
  const char *lut_b = reinterpret_cast<const char *>(lut);
  auto scale_of = [&](const BR &b, int j) __attribute__((always_inline)) {
    return DQ ? code2[b.q[j] & 255u] * b.s[j] + offset : b.s[j];
  };
  // table reads of decode chunk c = 4 j + t (weights (j, t): bytes 4 t .. 4 t + 3
  // of column j, k 32 h + 8 t .. + 7)
  auto tread = [&](const BR &b, int c, float2 (&tv)[4]) __attribute__((always_inline)) {
    const uint4 wv = b.w[c >> 2];
    const int t = c & 3;
    const uint32_t w = t == 0 ? wv.x : t == 1 ? wv.y : t == 2 ? wv.z : wv.w;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const uint32_t addr = __builtin_amdgcn_perm(w, lane_sel, 0x0c0c0000u | ((4u + bb) << 8));
      tv[bb] = *reinterpret_cast<const float2 *>(lut_b + addr);
    }
  };
  auto cvt4 = [&](const float2 (&tv)[4], float a) __attribute__((always_inline)) {
    uint32_t o[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) o[bb] = cvt_pair<ADT>(tv[bb].x * a, tv[bb].y * a);
    return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
  };
  bf16x8_t bfc[2][4], bfn[2][4];  // decoded weights of k-tiles kt and kt + 1
  {  // k-tile 0, before the loop
    const float a[2] = {scale_of(br0, 0), scale_of(br0, 1)};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float2 tv[4];
      tread(br0, c, tv);
      bfc[c >> 2][c & 3] = cvt4(tv, a[c >> 2]);
    }
  }
  // iteration kt: A(kt) in stage kt % 3, the weights of k-tile kt decoded by
  // the previous iteration; B(kt + 1) in register set (kt + 1) % 3 is decoded
  // here, cut into 8 chunks, each placed between 4 of the 32 MFMAs of k-tile
  // kt (a chunk's 4 table reads are issued two chunks ahead) so that the
  // decode arithmetic and table reads overlap the matrix cores; A and B are
  // loaded two k-tiles ahead (loads complete in order, so the wait for one
  // k-tile also waits for everything issued before it)
  auto step = [&](int kt, uint4 *sa_cur, uint4 *sa_next2, const BR &bnext1, BR &bnext2) __attribute__((always_inline)) {
    // A(kt) must have landed for every wave: this wave's loads issued since
    // are B(kt), A(kt + 1) and B(kt + 1) (4 + 2 x (2 + 4), or 2 + 2 per B
    // without double quantization)
    constexpr int after = 4 + 2 * (DQ ? 6 : 4);
    __builtin_amdgcn_s_waitcnt((after & 15) | (7 << 4) | (15 << 8) | ((after >> 4) << 14));
    __syncthreads();  // and every wave is done with stage (kt + 2) % 3
    issue_a(kt + 2, sa_next2);
    issue_b(kt + 2, bnext2);
    const float a[2] = {scale_of(bnext1, 0), scale_of(bnext1, 1)};
    float2 tv[8][4];
    tread(bnext1, 0, tv[0]);
    tread(bnext1, 1, tv[1]);
    bf16x8_t af[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = 4 * h + t;  // this lane's 16-byte chunk of the row for MFMA t
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 32 * i + colw;
        af[t][i] = __builtin_bit_cast(bf16x8_t, sa_cur[r * 8 + (c ^ ((r >> 1) & 7))]);
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      // scheduling fence: keeps each chunk's decode beside its 4 MFMAs
      __builtin_amdgcn_sched_barrier(0);
      if (c + 2 < 8) tread(bnext1, c + 2, tv[c + 2]);
      const int t = c >> 1;
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int i = 2 * (c & 1) + ii;
          acc[i][j] = mfma16<ADT>(af[t][i], bfc[j][t], acc[i][j]);
        }
      bfn[c >> 2][c & 3] = cvt4(tv[c], a[c >> 2]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) bfc[j][t] = bfn[j][t];
  };
  int kt = 0;
  for (; kt + 3 <= KT; kt += 3) {
    step(kt, st0, st2, br1, br2);
    step(kt + 1, st1, st0, br2, br0);
    step(kt + 2, st2, st1, br0, br1);
  }
  {  // the remaining 0..2 k-tiles (kt is a multiple of 3 here)
    const int rem = KT - kt;
    if (rem > 0) step(kt, st0, st2, br1, br2);
    if (rem > 1) step(kt + 1, st1, st0, br2, br0);
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): no LDS-direct load outlives the kernel

  // 32 x 32 accumulator layout: column = lane % 32, row = 8 (r / 4) + 4 (lane / 32) + r % 4
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + 64 * wave + 32 * j + colw;
      if (col >= N) continue;
      const float bv = bias ? load_elem<CDT>(bias, col) : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < M) store_elem<CDT>(C, row * N + col, bias ? acc[i][j][r] + bv : acc[i][j][r]);
      }
    }
}

// Which kernel gemm_4bit runs for 16-bit activations, and its grid.
// kind 0: narrow, 1: skinny (both: N / 32 workgroups, each all M rows of 32
// columns); 2: tile kernel (grid x over N tiles of bn, y over M tiles of bm);
// 3: large-M kernel (gx workgroups mapped by rb_tile).
struct GemmChoice {
  int kind;
  int bm, bn;
  int64_t gx, gy;
};

GemmChoice gemm_choice(int64_t M, int64_t N, int64_t K, int log2bs) {
  if (gemm_narrow_eligible(M, K, log2bs)) return {0, (int)M, 32, (N + 31) / 32, 1};
  if (M <= 64 && K % 64 == 0 && K < (1 << 23)) return {1, (int)M, 32, (N + 31) / 32, 1};
  if (gemm_rb_eligible(M, N, K)) {
    const int64_t ncol = (N + kRbN - 1) / kRbN, nrow = (M + kRbM - 1) / kRbM;
    return {3, kRbM, kRbN, ncol * nrow, 1};
  }
  // 256 x 128 tiles when they still give a workgroup to most compute units,
  // else 128 x 128, else 128 x 64 (narrower tiles, more workgroups)
  const int64_t cus = device_cu_count();
  const int64_t nt128 = (N + 127) / 128;
  const int shape = nt128 * ((M + 255) / 256) >= cus * 3 / 4 ? 2 : (nt128 * ((M + 127) / 128) >= cus ? 1 : 0);
  const int bm = shape == 2 ? 256 : 128, bn = shape ? 128 : 64;
  return {2, bm, bn, (N + bn - 1) / bn, (M + bm - 1) / bm};
}

// Host-side: the C tile [row0, row0 + rows) x [col0, col0 + cols) each
// workgroup of gemm_4bit's launch writes (it reads the same rows of A),
// computed with the kernels' own tile mapping.  Returns the number of
// workgroups; tiles gets 4 values per workgroup, up to cap of them.
int64_t gemm_plan(int64_t M, int64_t N, int64_t K, int log2bs, int64_t *tiles, int64_t cap, int *kind) {
  const GemmChoice g = gemm_choice(M, N, K, log2bs);
  *kind = g.kind;
  const int64_t nwg = g.gx * g.gy;
  for (int64_t w = 0; w < nwg && w < cap; ++w) {
    int64_t m0, n0;
    if (g.kind == 3) {
      rb_tile((int)w, (int)((N + kRbN - 1) / kRbN), (int)((M + kRbM - 1) / kRbM), m0, n0);
    } else {
      m0 = (w / g.gx) * g.bm;
      n0 = (w % g.gx) * g.bn;
    }
    int64_t *t = tiles + 4 * w;
    t[0] = m0;
    t[1] = n0;
    t[2] = M - m0 < g.bm ? M - m0 : g.bm;
    t[3] = N - n0 < g.bn ? N - n0 : g.bn;
  }
  return nwg;
}

template <int ADT>
static hipError_t launch_gemm_t(const void *A, int64_t M, int64_t N, int64_t K,
                                const uint8_t *packed, const Scales &sc, bool dq, int log2bs,
                                int qt, void *C, int c_dtype, const void *bias, hipStream_t st) {
  const uint16_t *a = static_cast<const uint16_t *>(A);
  Table16f table;
  const uint32_t *bits = table_bits(qt);
  for (int c = 0; c < 16; ++c) table.v[c] = __builtin_bit_cast(float, bits[c]);
  const GemmChoice g = gemm_choice(M, N, K, log2bs);
  if (g.kind == 0) {  // narrow M
    const dim3 sgrid((unsigned)g.gx);
#define QMV_N(CDT, DQV, MPV, NBV, KWV)                                                          \
  hipLaunchKernelGGL((gemm_4bit_narrow_kernel<ADT, CDT, DQV, MPV, NBV, KWV>), sgrid, dim3(64 * KWV), \
                     0, st, a, M, N, K, packed, sc, log2bs, table, C, bias)
    // waves per workgroup splitting K: more when the N / 32 workgroups leave
    // compute units without a second workgroup (8192 columns: one per CU),
    // as long as every wave still gets a few 128-k groups; with more
    // workgroups than CUs, 4 waves (14336 x 4096: 14.3 us at M = 8 against
    // 15.2 with 8 waves, 18.1 against 21.6 at M = 16)
    const int64_t cus = device_cu_count(), groups = (K / 64 + 1) / 2;
    const int kw = g.gx > cus ? 4 : (groups >= 32 ? 16 : (groups >= 16 ? 8 : 4));
#define QMV_NM(CDT, DQV)                                                        \
  if (M <= 8) {                                                                 \
    if (kw == 16) { QMV_N(CDT, DQV, 8, 2, 16); }                                \
    else if (kw == 8) { QMV_N(CDT, DQV, 8, 2, 8); }                             \
    else { QMV_N(CDT, DQV, 8, 2, 4); }                                          \
  } else {                                                                      \
    if (kw >= 8) { QMV_N(CDT, DQV, 16, 2, 8); }                                 \
    else { QMV_N(CDT, DQV, 16, 2, 4); }                                         \
  }
#define QMV_ND(CDT) \
  if (dq) { QMV_NM(CDT, true); } else { QMV_NM(CDT, false); }
    if (c_dtype == kF32) { QMV_ND(kF32); }
    else if (c_dtype == kF16) { QMV_ND(kF16); }
    else { QMV_ND(kBF16); }
#undef QMV_ND
#undef QMV_NM
#undef QMV_N
    return hipGetLastError();
  }
  if (g.kind == 1) {  // skinny M: N / 32 workgroups of 8 waves splitting K
    const dim3 sgrid((unsigned)g.gx);
#define QMV_S(CDT, DQV, MTV)                                                                   \
  hipLaunchKernelGGL((gemm_4bit_skinny_kernel<ADT, CDT, DQV, MTV, 8>), sgrid, dim3(512), 0, st, a, \
                     M, N, K, packed, sc, log2bs, table, C, bias)
#define QMV_SM(CDT, DQV) \
  if (M <= 32) { QMV_S(CDT, DQV, 1); } else { QMV_S(CDT, DQV, 2); }
#define QMV_SD(CDT) \
  if (dq) { QMV_SM(CDT, true); } else { QMV_SM(CDT, false); }
    if (c_dtype == kF32) { QMV_SD(kF32); }
    else if (c_dtype == kF16) { QMV_SD(kF16); }
    else { QMV_SD(kBF16); }
#undef QMV_SD
#undef QMV_SM
#undef QMV_S
    return hipGetLastError();
  }
  if (g.kind == 3) {  // large M: 128 x 256 tiles, weights decoded in registers
    const int ncol = (int)((N + kRbN - 1) / kRbN), nrow = (int)((M + kRbM - 1) / kRbM);
    const dim3 rgrid((unsigned)g.gx);
#define QMV_R(CDT, DQV)                                                                            \
  hipLaunchKernelGGL((gemm_4bit_rb_kernel<ADT, CDT, DQV>), rgrid, dim3(256), 0, st, a, M, N, K, packed, \
                     sc, log2bs, table, C, bias, ncol, nrow)
#define QMV_RD(CDT) \
  if (dq) { QMV_R(CDT, true); } else { QMV_R(CDT, false); }
    if (c_dtype == kF32) { QMV_RD(kF32); }
    else if (c_dtype == kF16) { QMV_RD(kF16); }
    else { QMV_RD(kBF16); }
#undef QMV_RD
#undef QMV_R
    return hipGetLastError();
  }
  const int shape = g.bm == 256 ? 2 : (g.bn == 128 ? 1 : 0);
  const dim3 grid((unsigned)g.gx, (unsigned)g.gy);
#define QMV_M(CDT, DQV, BMV, BNV)                                                                    \
  hipLaunchKernelGGL((gemm_4bit_kernel<ADT, CDT, DQV, BMV, BNV>), grid, dim3(2 * BMV), 0, st, a, M, N, \
                     K, packed, sc, log2bs, table, C, bias)
#define QMV_MB(CDT, DQV)                                     \
  if (shape == 2) { QMV_M(CDT, DQV, 256, 128); }             \
  else if (shape == 1) { QMV_M(CDT, DQV, 128, 128); }        \
  else { QMV_M(CDT, DQV, 128, 64); }
#define QMV_MD(CDT) \
  if (dq) { QMV_MB(CDT, true); } else { QMV_MB(CDT, false); }
  if (c_dtype == kF32) { QMV_MD(kF32); }
  else if (c_dtype == kF16) { QMV_MD(kF16); }
  else { QMV_MD(kBF16); }
#undef QMV_MD
#undef QMV_MB
#undef QMV_M
  return hipGetLastError();
}

hipError_t launch_gemm_4bit(const void *A, int a_dtype, int64_t M, int64_t N, int64_t K,
                            const uint8_t *packed, const Scales &sc, bool dq, int log2bs, int qt,
                            void *C, int c_dtype, const void *bias, hipStream_t st) {
  if (a_dtype == kF32) {
    // fp32 activations: up to 8 rows take the fp32 kernel of gemv_4bit, more
    // the fp32 matrix cores
    if (M <= 8)
      return launch_gemv_4bit(A, kF32, (int)M, N, K, packed, sc, dq, log2bs, qt, C, c_dtype, bias, st);
    Table16f table;
    const uint32_t *bits = table_bits(qt);
    for (int c = 0; c < 16; ++c) table.v[c] = __builtin_bit_cast(float, bits[c]);
    const dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128));
    const float *a = static_cast<const float *>(A);
#define QMV_F(CDT, DQV)                                                                       \
  hipLaunchKernelGGL((gemm_4bit_f32_kernel<CDT, DQV>), grid, dim3(256), 0, st, a, M, N, K, packed, \
                     sc, log2bs, table, C, bias)
#define QMV_FD(CDT) \
  if (dq) { QMV_F(CDT, true); } else { QMV_F(CDT, false); }
    if (c_dtype == kF32) { QMV_FD(kF32); }
    else if (c_dtype == kF16) { QMV_FD(kF16); }
    else { QMV_FD(kBF16); }
#undef QMV_FD
#undef QMV_F
    return hipGetLastError();
  }
  if (a_dtype == kF16) return launch_gemm_t<kF16>(A, M, N, K, packed, sc, dq, log2bs, qt, C, c_dtype, bias, st);
  return launch_gemm_t<kBF16>(A, M, N, K, packed, sc, dq, log2bs, qt, C, c_dtype, bias, st);
}

// ---------------------------------------------------------------------------
// gemm_4bit_backward, register-free transpose: gemm_4bit_dxt_kernel
//
// dX[M, K] = dY[M, N] @ W_hat[N, K] with the reduction over N, whose packed
// rows run along K: the weight tile has to be turned around before the
// matrix cores can take it as their B operand (8 consecutive reduction
// values n per lane).  A workgroup of 8 waves owns a 128 (M) x 256 (K) tile
// of dX and a contiguous range of reduction steps of 64 rows of W; wave
// (h, g) computes rows [64 h, 64 h + 64) x columns [64 g, 64 g + 64) as 2 x 2
// accumulators of v_mfma_f32_32x32x16_bf16 (f16), two waves per SIMD.  Per
// step:
//  * dY's 128 x 64 tile goes global -> LDS through 16-byte LDS-direct loads
//    into a 3-stage ring issued two steps ahead (the forward large-M
//    kernel's activation ring, with n in place of k);
//  * the two waves of column group g decode its 64 rows of the step, columns
//    [64 g, + 64): lane l of wave (h, g) takes row 32 h + l / 2, 32 columns
//    (one 16-byte packed load, one block scale: blocks >= 64 columns), 16
//    lookups of the fp32 pair table, fp32(T * a_hat) rounded to dY's type --
//    exactly the dequantize_4bit values -- and writes its 64 bytes into the
//    group's 64 x 64 LDS block; a barrier then makes the block whole;
//  * the B operand comes back out of that block with ds_read_b64_tr_b16:
//    within each 16 lanes the instruction returns, to lane i, element i % 4
//    of what lanes 4 e + i / 4 (e = 0..3) addressed, so lanes that address 4
//    consecutive rows x 4 consecutive columns hand every lane one column's 4
//    rows.  Two such reads give a lane the 8 reduction values of its column.
//    The block's 16-byte chunks are XOR-swizzled by g(n) = ((j & 1) << 2) |
//    (j >> 1), j = (n / 2) % 8, which keeps both the row writes (16 rows,
//    one chunk position) and the transposed reads (4 rows x 8 eight-byte
//    units) on distinct banks.
// When 128 x 256 tiles would leave compute units idle, the reduction is split
// over S workgroups per tile: each writes its fp32 partial tile to the
// workspace and bumps the tile's counter; the workgroup that finds the count
// complete adds the S partials in split order (the same sum whichever
// finishes last) and stores dX.  A one-block launch zeroes the counters
// first (a workspace that served another shape may hold partials where the
// counters are now).  The workgroups of a
// tile run on different XCDs, whose L2 caches are not coherent with each
// other for ordinary accesses: the partials are written and read with the
// SC1 cache policy and the counter with an agent-scope atomic, which bypass
// the non-coherent caches.
// ---------------------------------------------------------------------------
constexpr int kDxM = 128, kDxK = 256, kDxN = 64;

__device__ __forceinline__ int dxt_swz(int n) {  // 16-byte chunk swizzle of weight row n
  const int j = (n >> 1) & 7;
  return ((j & 1) << 2) | (j >> 1);
}

template <int ADT, int CDT, bool DQ>
__global__ __launch_bounds__(512, 1) void gemm_4bit_dxt_kernel(
    const uint16_t *__restrict__ dY, int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    Scales sc, int log2bs, Table16f table, void *__restrict__ dXv, int ktiles, int splits, int steps_per_split,
    float *__restrict__ part, uint32_t *__restrict__ counters) {
  using CT = typename Storage<CDT>::type;
  CT *dX = static_cast<CT *>(dXv);
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * 32 * 2];  // byte -> (T[hi], T[lo]), 32 copies
  __shared__ float code2[256];
  __shared__ uint4 st0[kDxM * 8], st1[kDxM * 8], st2[kDxM * 8];       // dY ring
  __shared__ __attribute__((aligned(16))) uint4 wbuf[4 * kDxN * 8];  // decoded weights, 8 KB per column group
  __shared__ int last_flag;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg = wave & 3;   // column group: dX columns [64 cg, 64 cg + 64) of the tile
  const int mh = wave >> 2;  // row half: dX rows [64 mh, 64 mh + 64) of the tile
  const int s = (int)blockIdx.x % splits;
  const int tile = (int)blockIdx.x / splits;
  const int64_t m0 = (int64_t)(tile / ktiles) * kDxM;
  const int64_t k0 = (int64_t)(tile % ktiles) * kDxK;
  const int NT = (int)(N / kDxN);
  const int nt0 = s * steps_per_split;
  const int nsteps = NT - nt0 < steps_per_split ? NT - nt0 : steps_per_split;  // >= 1
  {  // table: 16-byte chunk c holds copies 2 (c % 16) and + 1 of entry c / 16
    const uint32_t lo = __float_as_uint(table.v[(tid >> 4) & 15]);
    uint4 *dst = reinterpret_cast<uint4 *>(lut);
#pragma unroll
    for (int it = 0; it < 8; ++it) {  // chunk it * 512 + tid: entry hi nibble 2 it + tid / 256
      const uint32_t hi = __float_as_uint((tid >> 8) ? table.v[2 * it + 1] : table.v[2 * it]);
      dst[it * 512 + tid] = make_uint4(hi, lo, hi, lo);
    }
  }
  float offset = 0.f;
  if constexpr (DQ) {
    if (tid < 256) code2[tid] = sc.code2[tid];
    offset = sc.offset[0];
  }
  // dY: wave w moves rows (2 w + d) * 8 + l / 8 of a stage, lane l into
  // position l % 8 of its row, from chunk (l % 8) ^ ((row / 2) % 8); rows past
  // M read zeros (bounded resource)
  const int64_t mrows = M - m0 < kDxM ? M - m0 : kDxM;
  const uint16_t *a_base = dY + m0 * N;
  const uint32_t a_bytes = (uint32_t)(mrows * N * 2);
  uint32_t aoff[2];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const int r = (2 * wave + d) * 8 + (lane >> 3);
    aoff[d] = (uint32_t)(r * N * 2) + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
  }
  auto issue_a = [&](int l, uint4 *stage) __attribute__((always_inline)) {
    // step l of this split; steps past the end re-read the last
    const uint32_t no = (uint32_t)(nt0 + (l < nsteps ? l : nsteps - 1)) * (kDxN * 2);
    const __amdgpu_buffer_rsrc_t ars = make_rsrc_u(a_base, a_bytes);
#pragma unroll
    for (int d = 0; d < 2; ++d) load_lds16(ars, stage + (2 * wave + d) * 64, aoff[d] + no);
  };
  // weights: the two waves of a column group decode its 64 rows of the step,
  // wave (mh, cg) rows 32 mh .. 32 mh + 31: lane l takes row 32 mh + l / 2,
  // columns k0 + 64 cg + 32 (l % 2) .. + 31 (one 16-byte load, one block)
  const uint32_t rowb = (uint32_t)(K >> 1);
  const int64_t kcol = k0 + 64 * cg;
  const int64_t bpr = K >> log2bs;  // blocks per weight row
  const int wrow = 32 * mh + (lane >> 1);
  struct BR {
    uint4 w;
    uint32_t q;
    float s;
  };
  auto issue_b = [&](int l, BR &b) __attribute__((always_inline)) {
    const int64_t row0 = (int64_t)(nt0 + (l < nsteps ? l : nsteps - 1)) * kDxN;
    const __amdgpu_buffer_rsrc_t prs = make_rsrc_u(packed + row0 * rowb, kDxN * rowb);
    const uint32_t off = (uint32_t)wrow * rowb + (uint32_t)(kcol >> 1) + 16u * (uint32_t)(lane & 1);
    b.w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(prs, off, 0, 0));
    const int64_t blk = (row0 + wrow) * bpr + (kcol >> log2bs);
    if constexpr (DQ) {
      b.q = sc.q[blk];
      b.s = sc.absmax2[blk >> sc.log2bs2];
    } else {
      b.s = sc.absmax[blk];
    }
  };
  issue_a(0, st0);
  issue_a(1, st1);
  BR br0, br1, br2;
  issue_b(0, br0);
  issue_b(1, br1);
  __syncthreads();  // table and code2

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const uint32_t lane_sel = (uint32_t)(lane & 31) << 3;
  const char *lut_b = reinterpret_cast<const char *>(lut);
  uint4 *wblk = wbuf + cg * (kDxN * 8);  // the column group's decoded 64 x 64 block
  const int wsw = dxt_swz(wrow);
  // decode this lane's 32 columns of row wrow: chunk p (columns 8 p .. 8 p + 7
  // of the block) at position p ^ swizzle
  auto decode = [&](const BR &b) __attribute__((always_inline)) {
    const float a = DQ ? code2[b.q & 255u] * b.s + offset : b.s;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const uint32_t w = pp == 0 ? b.w.x : pp == 1 ? b.w.y : pp == 2 ? b.w.z : b.w.w;
      float2 tv[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const uint32_t addr = __builtin_amdgcn_perm(w, lane_sel, 0x0c0c0000u | ((4u + bb) << 8));
        tv[bb] = *reinterpret_cast<const float2 *>(lut_b + addr);
      }
      uint32_t o[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) o[bb] = cvt_pair<ADT>(tv[bb].x * a, tv[bb].y * a);
      const int p = 4 * (lane & 1) + pp;
      wblk[wrow * 8 + (p ^ wsw)] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  };
  // transposed B operand of MFMA step t (reduction rows 16 t + 8 h .. + 7)
  // for column block j (columns 32 j + lane % 32): lane l addresses row
  // 16 t + 8 h + 4 r + (l % 16) / 4 and the 4 columns starting at
  // 32 j + 16 ((l / 16) % 2) + 4 (l % 4)
  typedef short v4s_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;
  const int h = lane >> 5, colw = lane & 31;
  auto bfrag = [&](int t, int j) __attribute__((always_inline)) {
    uint32_t v[4];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int n = 16 * t + 8 * h + 4 * r + ((lane & 15) >> 2);
      const int u = 8 * j + 4 * ((lane >> 4) & 1) + (lane & 3);  // 8-byte unit of the row
      const int phys = ((((u >> 1) ^ dxt_swz(n)) << 1) | (u & 1));
      const v4s_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4s_t *)(reinterpret_cast<char *>(wblk) + n * 128 + phys * 8));
      const uint2 xx = __builtin_bit_cast(uint2, x);
      v[2 * r] = xx.x;
      v[2 * r + 1] = xx.y;
    }
    return __builtin_bit_cast(bf16x8_t, make_uint4(v[0], v[1], v[2], v[3]));
  };
  auto mma = [&](const uint4 *stage) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8_t b0 = bfrag(t, 0), b1 = bfrag(t, 1);
      const int c = 2 * t + h;  // this lane's 16-byte chunk of the dY row for MFMA t
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 64 * mh + 32 * i + colw;
        const bf16x8_t af = __builtin_bit_cast(bf16x8_t, stage[r * 8 + (c ^ ((r >> 1) & 7))]);
        acc[i][0] = mfma16<ADT>(af, b0, acc[i][0]);
        acc[i][1] = mfma16<ADT>(af, b1, acc[i][1]);
      }
    }
  };
  // step l: dY(l) in stage l % 3, weights(l) in register set l % 3, both
  // loaded two steps ahead (loads complete in order, so the wait for a
  // step's weights also waits for everything issued before them: with two
  // steps between issue and use neither the activations nor the weights and
  // their scattered block scales stall the step)
  auto step = [&](int l, uint4 *sa_cur, uint4 *sa_next2, BR &bcur, BR &bnext2) __attribute__((always_inline)) {
    // dY(l) must have landed for every wave: this wave's loads issued since
    // are W(l) and dY(l + 1), W(l + 1) (2 + 2 x (1 + 2), or 1 + 1 per W
    // without double quantization)
    constexpr int after = 2 + 2 * (DQ ? 3 : 2);
    __builtin_amdgcn_s_waitcnt((after & 15) | (7 << 4) | (15 << 8) | ((after >> 4) << 14));
    __syncthreads();  // and every wave is done with stage (l + 2) % 3 and with the weight blocks
    issue_a(l + 2, sa_next2);
    issue_b(l + 2, bnext2);
    decode(bcur);
    __syncthreads();  // both halves of every column group's block are written
    mma(sa_cur);
  };
  int l = 0;
  for (; l + 3 <= nsteps; l += 3) {
    step(l, st0, st2, br0, br2);
    step(l + 1, st1, st0, br1, br0);
    step(l + 2, st2, st1, br2, br1);
  }
  {  // the remaining 0..2 steps (l is a multiple of 3 here)
    const int rem = nsteps - l;
    if (rem > 0) step(l, st0, st2, br0, br2);
    if (rem > 1) step(l + 1, st1, st0, br1, br0);
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): no LDS-direct load outlives the loop

  if (splits > 1) {
    // this split's partial tile, per wave 16-byte pieces: elements 4 c ..
    // 4 c + 3 of lane l at piece c * 64 + l.  Stored and later read with the
    // SC1 cache policy (coherent at agent scope: the non-coherent caches are
    // bypassed), 16 bytes per lane per instruction.
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    constexpr int kSC1 = 16;  // cache-policy bit SC1
    constexpr int kPer = 64 * 64;  // floats per wave
    float *mine = part + ((int64_t)(tile * splits + s) * 8 + wave) * kPer;
    {
      const __amdgpu_buffer_rsrc_t mrs = make_rsrc(mine, kPer * 4);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const int i = c >> 3, j = (c >> 2) & 1, r0 = 4 * (c & 3);
        const u32x4_t v = {__float_as_uint(acc[i][j][r0]), __float_as_uint(acc[i][j][r0 + 1]),
                           __float_as_uint(acc[i][j][r0 + 2]), __float_as_uint(acc[i][j][r0 + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(v, mrs, (uint32_t)((c * 64 + lane) * 16), 0, kSC1);
      }
    }
    // the partial's SC1 stores write through to the point of coherence;
    // waiting for their completion (vmcnt(0)) in every wave before the count
    // is bumped publishes them.  No release or acquire fence: at agent scope
    // those write back and invalidate the whole L2 of the XCD (measured: +33
    // us on 512 x 14336 x 4096), and nothing else this kernel writes needs
    // publishing.
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
    __syncthreads();
    if (tid == 0)
      last_flag = __hip_atomic_fetch_add(counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  (uint32_t)(splits - 1);
    __syncthreads();
    if (!last_flag) return;  // the partials are read below with SC1 (coherent) loads
    // the S partials added in split order, all of a split's loads in flight
    // together
    float sum[64];
    for (int s2 = 0; s2 < splits; ++s2) {
      float v[64];
      if (s2 == s) {
#pragma unroll
        for (int e = 0; e < 64; ++e) v[e] = acc[e >> 5][(e >> 4) & 1][e & 15];
      } else {
        const __amdgpu_buffer_rsrc_t prs = make_rsrc(part + ((int64_t)(tile * splits + s2) * 8 + wave) * kPer, kPer * 4);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(prs, (uint32_t)((c * 64 + lane) * 16), 0, kSC1);
          v[4 * c] = __uint_as_float(x.x);
          v[4 * c + 1] = __uint_as_float(x.y);
          v[4 * c + 2] = __uint_as_float(x.z);
          v[4 * c + 3] = __uint_as_float(x.w);
        }
      }
#pragma unroll
      for (int e = 0; e < 64; ++e) sum[e] = s2 == 0 ? v[e] : sum[e] + v[e];
    }
#pragma unroll
    for (int e = 0; e < 64; ++e) acc[e >> 5][(e >> 4) & 1][e & 15] = sum[e];
  }

  // 32 x 32 accumulator layout: column = lane % 32, row = 8 (r / 4) + 4 (lane / 32) + r % 4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = kcol + 32 * j + colw;  // < K: K % 256 == 0
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + 64 * mh + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < M) store_elem<CDT>(dX, row * K + col, acc[i][j][r]);
      }
    }
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t *__restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += 256) p[i] = 0u;
}

// Launch shape of gemm_4bit_dxt_kernel: column tiles, splits of the
// reduction and steps per split, and the workspace it needs (tile counters,
// then fp32 partial tiles).  Eligible: N % 64 == 0, K % 256 == 0, blocks of
// at least 64 columns (so a wave's 64 columns of a row lie in one block).
struct DxtPlan {
  bool ok;
  int ktiles, mtiles, splits, steps;
  size_t counter_bytes, bytes;
};

DxtPlan dxt_plan(int64_t M, int64_t N, int64_t K, int log2bs) {
  DxtPlan p{};
  if (N % kDxN != 0 || K % kDxK != 0 || log2bs < 6 || N >= ((int64_t)1 << 24) ||
      (int64_t)kDxN * (K / 2) >= ((int64_t)1 << 32))
    return p;
  p.ok = true;
  p.ktiles = (int)(K / kDxK);
  p.mtiles = (int)((M + kDxM - 1) / kDxM);
  const int64_t tiles = (int64_t)p.ktiles * p.mtiles;
  const int NT = (int)(N / kDxN);
  const int64_t cus = device_cu_count();
  int S = (int)std::min<int64_t>(NT, std::max<int64_t>(1, (cus + tiles - 1) / tiles));
  p.steps = (NT + S - 1) / S;
  p.splits = (NT + p.steps - 1) / p.steps;  // every split has at least one step
  if (tiles * p.splits > 0x7fffffff) {
    p.ok = false;
    return p;
  }
  p.counter_bytes = p.splits > 1 ? (size_t)((tiles * 4 + 255) / 256 * 256) : 0;
  p.bytes = p.splits > 1 ? p.counter_bytes + (size_t)tiles * p.splits * 4 * 128 * 64 * sizeof(float) : 0;
  return p;
}

// ---------------------------------------------------------------------------
// gemm_4bit_backward: dX[M, K] = dY[M, N] @ W_hat[N, K] ("Feat/mps gemm 4bit
// bf16", table "What runs natively now": gemm_4bit_backward, the fused form
// of grad_output @ dequantize_4bit(B)).
//
// The tile kernel's structure with the weight tile transposed on its way into
// LDS: a workgroup computes a 128 x BN tile of dX (BN = 128 or 64 columns of
// K) and walks the reduction over N in steps of 64.  Thread t decodes RN rows
// (n) x 8 columns (k) of the step's weight tile -- RN 4-byte loads, 64
// contiguous bytes per row across 16 (or 8) neighbouring threads -- and writes
// each column's RN bf16 values as one 8- (or 4-) byte store into the LDS
// tile kept [k][n], which is the layout the MFMA B operand reads, exactly as
// in the forward kernel.  Dequantization is the forward's: fp32(T * a_hat)
// rounded to bf16, so the matrix cores see the dequantize_4bit weights.
// Requires N % 32 == 0 (a step past N is half zero) and K % 32 == 0.
// ---------------------------------------------------------------------------
template <int ADT, int CDT, bool DQ, int BN, int G>
__global__ __launch_bounds__(256 * G, 2 / G) void gemm_4bit_dx_kernel(const uint16_t *__restrict__ dY,
                                                                      int64_t M, int64_t N, int64_t K,
                                                                      const uint8_t *__restrict__ packed,
                                                                      Scales sc, int log2bs, Table16f table,
                                                                      void *__restrict__ dXv) {
  constexpr int BM = 128;
  constexpr int kStage = (BM + BN) * kLd;
  constexpr int NJ = BN / 64;     // 32-column accumulators per wave (2 x 2 waves per group)
  constexpr int OCT = BN / 8;     // 8-column groups of the weight tile
  constexpr int RN = 64 / (256 / OCT);  // weight rows per thread: 4 or 2
  using CT = typename Storage<CDT>::type;
  CT *dX = static_cast<CT *>(dXv);
  const float dq_offset = DQ ? sc.offset[0] : 0.f;  // read once, not per tile
  __shared__ __attribute__((aligned(16))) uint16_t smem_all[G * 2 * kStage];
  __shared__ float2 lut2[256];
  __shared__ float code2[256];
  const int tid = threadIdx.x;
  const int grp = tid >> 8;       // group: takes reduction steps grp, grp + G, ...
  const int t = tid & 255;        // thread within the group
  const int lane = tid & 63;
  const int wave = t >> 6;        // wave within the group
  const int wm = wave >> 1, wn = wave & 1;
  uint16_t *smem = smem_all + grp * 2 * kStage;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t k0 = (int64_t)blockIdx.x * BN;
  const int64_t NT_ = (N + 63) / 64;  // reduction steps
  const int64_t NL = (NT_ + G - 1) / G;  // steps per group (the last may be past the end)
  const bool n_tail = (N % 64) != 0;  // last step has 32 of 64 rows

  // loaders: dY row t / 2, 32 values of the step from 32 (t % 2); weight rows
  // RN q .. RN q + RN - 1 of the step, columns 8 o .. 8 o + 7
  const int lr = t >> 1, lh = t & 1;
  const int o = t % OCT, q = t / OCT;
  const int64_t arow = m0 + lr < M ? m0 + lr : M - 1;  // rows past M are never stored
  const int64_t kc = k0 + 8 * o < K ? k0 + 8 * o : K - 8;  // columns past K likewise
  uint4 ra_[2][4];
  uint32_t rb_[2][RN];
  float rsa_[2][RN];
  uint32_t rsq_[2][RN];
  auto gstep = [&](int64_t l) {  // the group's l-th step, clamped to the last one
    const int64_t s2 = grp + (int64_t)G * l;
    return s2 < NT_ ? s2 : NT_ - 1;
  };
  auto load_step = [&](int64_t st, auto slot_tag) {
    constexpr int SL = decltype(slot_tag)::value;
    int64_t n = st * 64 + 32 * lh;
    if (n >= N) n = N - 32;  // the missing half of a tail step (zeroed when staged)
    const uint4 *ap = reinterpret_cast<const uint4 *>(dY + arow * N + n);
#pragma unroll
    for (int i = 0; i < 4; ++i) ra_[SL][i] = ap[i];
#pragma unroll
    for (int r = 0; r < RN; ++r) {
      int64_t row = st * 64 + RN * q + r;
      if (row >= N) row = N - 1;  // zeroed when staged
      const int64_t e0 = row * K + kc;
      rb_[SL][r] = *reinterpret_cast<const uint32_t *>(packed + (e0 >> 1));
      const int64_t b = e0 >> log2bs;
      if constexpr (DQ) {
        rsq_[SL][r] = sc.q[b];
        rsa_[SL][r] = sc.absmax2[b >> sc.log2bs2];
      } else {
        rsa_[SL][r] = sc.absmax[b];
      }
    }
  };
  auto stage_step = [&](int64_t st, int buf, auto slot_tag) {
    constexpr int SL = decltype(slot_tag)::value;
    uint16_t *As = smem + buf * kStage;
    uint16_t *Bs = As + BM * kLd;
    const bool last = n_tail && st == NT_ - 1;
    uint4 *ad = reinterpret_cast<uint4 *>(As + lr * kLd + 32 * lh);
#pragma unroll
    for (int i = 0; i < 4; ++i) ad[i] = (last && lh == 1) ? make_uint4(0, 0, 0, 0) : ra_[SL][i];
    // w[r][i]: bf16 pair (column 8 o + 2 i, 8 o + 2 i + 1) of weight row r
    uint32_t w[RN][4];
#pragma unroll
    for (int r = 0; r < RN; ++r) {
      const bool zero = last && RN * q + r >= 32;
      const float a = zero ? 0.f : (DQ ? code2[rsq_[SL][r]] * rsa_[SL][r] + dq_offset : rsa_[SL][r]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 tv = lut2[(rb_[SL][r] >> (8 * i)) & 0xffu];
        w[r][i] = cvt_pair<ADT>(tv.x * a, tv.y * a);
      }
    }
    // column c = 8 o + 2 i (+1): its RN values, rows in order, in one store
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const uint32_t sel = hi ? 0x07060302u : 0x05040100u;  // high or low bf16 of each pair
        uint16_t *dst = Bs + (8 * o + 2 * i + hi) * kLd + RN * q;
        if constexpr (RN == 4) {
          const uint32_t x0 = __builtin_amdgcn_perm(w[1][i], w[0][i], sel);
          const uint32_t x1 = __builtin_amdgcn_perm(w[3][i], w[2][i], sel);
          *reinterpret_cast<uint2 *>(dst) = make_uint2(x0, x1);
        } else {
          *reinterpret_cast<uint32_t *>(dst) = __builtin_amdgcn_perm(w[1][i], w[0][i], sel);
        }
      }
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  load_step(gstep(0), S0{});
  load_step(gstep(1), S1{});
  if (tid < 256) {
    lut2[tid] = make_float2(table.v[tid >> 4], table.v[tid & 15]);
    if constexpr (DQ) code2[tid] = sc.code2[tid];
  }
  __syncthreads();
  stage_step(gstep(0), 0, S0{});
  __syncthreads();

  f32x16_t acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  auto mma_step = [&](int64_t l, int buf) {
    if (grp + (int64_t)G * l >= NT_) return;  // past this group's last step (wave-uniform)
    const uint16_t *As = smem + buf * kStage;
    const uint16_t *Bs = As + BM * kLd;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t af[2], bfr[NJ];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8_t *>(As + row * kLd + ks * 16 + (lane >> 5) * 8);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = wn * (BN / 2) + j * 32 + (lane & 31);
        bfr[j] = *reinterpret_cast<const bf16x8_t *>(Bs + col * kLd + ks * 16 + (lane >> 5) * 8);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = mfma16<ADT>(af[i], bfr[j], acc[i][j]);
    }
  };

  // the group's step l sits in LDS stage l % 2 and step l + 1 in register set
  // (l + 1) % 2; loads past the end re-read the last step, so every group
  // runs the same loop (and the same barriers)
  int64_t l = 0;
  for (; l + 1 < NL; l += 2) {
    load_step(gstep(l + 2), S0{});
    mma_step(l, 0);
    stage_step(gstep(l + 1), 1, S1{});
    __syncthreads();
    load_step(gstep(l + 3), S1{});
    mma_step(l + 1, 1);
    if (l + 2 < NL) stage_step(gstep(l + 2), 0, S0{});
    __syncthreads();
  }
  if (l < NL) mma_step(l, 0);

  if constexpr (G > 1) {  // add the other groups' tiles, in group order
    float *part = reinterpret_cast<float *>(smem_all);
    constexpr int PER = 2 * NJ * 16;  // floats per lane
    __syncthreads();
    if (grp > 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            part[(((grp - 1) * 4 + wave) * PER + (i * NJ + j) * 16 + r) * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int g2 = 1; g2 < G; ++g2)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[i][j][r] += part[(((g2 - 1) * 4 + wave) * PER + (i * NJ + j) * 16 + r) * 64 + lane];
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t col = k0 + wn * (BN / 2) + j * 32 + (lane & 31);
      if (col >= K) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) store_elem<CDT>(dX, row * K + col, acc[i][j][r]);
      }
    }
}

template <int ADT>
static hipError_t launch_backward_t(const void *dY, int64_t M, int64_t N, int64_t K,
                                    const uint8_t *packed, const Scales &sc, bool dq, int log2bs,
                                    int qt, void *dX, int dx_dtype, void *ws, hipStream_t st) {
  const uint16_t *g = static_cast<const uint16_t *>(dY);
  Table16f table;
  const uint32_t *bits = table_bits(qt);
  for (int c = 0; c < 16; ++c) table.v[c] = __builtin_bit_cast(float, bits[c]);
  const DxtPlan p = dxt_plan(M, N, K, log2bs);
  if (p.ok) {  // the transposed-read kernel (the caller supplied p.bytes of workspace)
    uint32_t *counters = static_cast<uint32_t *>(ws);
    float *part = p.splits > 1 ? reinterpret_cast<float *>(static_cast<char *>(ws) + p.counter_bytes) : nullptr;
    const dim3 grid((unsigned)((int64_t)p.ktiles * p.mtiles * p.splits));
    if (p.splits > 1) {
      hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(256), 0, st, counters, p.ktiles * p.mtiles);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
#define QMV_T(CDT, DQV)                                                                              \
  hipLaunchKernelGGL((gemm_4bit_dxt_kernel<ADT, CDT, DQV>), grid, dim3(512), 0, st, g, M, N, K, packed, sc, \
                     log2bs, table, dX, p.ktiles, p.splits, p.steps, part, counters)
#define QMV_TD(CDT) \
  if (dq) { QMV_T(CDT, true); } else { QMV_T(CDT, false); }
    if (dx_dtype == kF32) { QMV_TD(kF32); }
    else if (dx_dtype == kF16) { QMV_TD(kF16); }
    else { QMV_TD(kBF16); }
#undef QMV_TD
#undef QMV_T
    return hipGetLastError();
  }
  const int64_t mt = (M + 127) / 128;
  const bool wide = ((K + 127) / 128) * mt >= (int64_t)device_cu_count();
  const dim3 grid((unsigned)(wide ? (K + 127) / 128 : (K + 63) / 64), (unsigned)mt);
#define QMV_B(CDT, DQV, BNV)                                                                    \
  hipLaunchKernelGGL((gemm_4bit_dx_kernel<ADT, CDT, DQV, BNV, 2>), grid, dim3(512), 0, st, g, M, N, K, \
                     packed, sc, log2bs, table, dX)
#define QMV_BB(CDT, DQV) \
  if (wide) { QMV_B(CDT, DQV, 128); } else { QMV_B(CDT, DQV, 64); }
#define QMV_BD(CDT) \
  if (dq) { QMV_BB(CDT, true); } else { QMV_BB(CDT, false); }
  if (dx_dtype == kF32) { QMV_BD(kF32); }
  else if (dx_dtype == kF16) { QMV_BD(kF16); }
  else { QMV_BD(kBF16); }
#undef QMV_BD
#undef QMV_BB
#undef QMV_B
  return hipGetLastError();
}

size_t gemm_backward_workspace_bytes(int64_t M, int64_t N, int64_t K, int log2bs) {
  const DxtPlan p = dxt_plan(M, N, K, log2bs);
  return p.ok ? p.bytes : 0;
}

hipError_t launch_gemm_4bit_backward(const void *dY, int dy_dtype, int64_t M, int64_t N, int64_t K,
                                     const uint8_t *packed, const Scales &sc, bool dq, int log2bs,
                                     int qt, void *dX, int dx_dtype, void *ws, hipStream_t st) {
  if (dy_dtype == kF16) return launch_backward_t<kF16>(dY, M, N, K, packed, sc, dq, log2bs, qt, dX, dx_dtype, ws, st);
  return launch_backward_t<kBF16>(dY, M, N, K, packed, sc, dq, log2bs, qt, dX, dx_dtype, ws, st);
}

}  // namespace qmv
