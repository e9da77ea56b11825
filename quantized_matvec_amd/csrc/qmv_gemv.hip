// gemv_4bit: y[m, n] = sum_k x[m, k] * W_hat[n, k] for 1 <= M <= 8 rows of
// activations, with the 4-bit dequantization fused into the dot product
// ("Feat/mps gemm 4bit bf16", table "What runs natively now": gemv_4bit is a
// fused dequant + dot for the decode step).
//
// Data flow: a wave owns one weight row at a time; each lane streams 16-byte
// pieces of the packed row (32 weights, always inside one block), looks the
// codes up in a 16-entry table in LDS, multiplies with x in fp32, folds the
// block scale into the piece's partial sum, and the row is finished with a
// wave-level shuffle reduction.
#include <algorithm>

#include "qmv_launch.hpp"

namespace qmv {

template <int M, int XDT, int YDT, bool DQ, int QT>
__global__ __launch_bounds__(256) void gemv_4bit_kernel(const void *__restrict__ xv, int64_t N,
                                                        int64_t K, const uint8_t *__restrict__ packed,
                                                        Scales sc, int log2bs, void *__restrict__ yv) {
  using XT = typename Storage<XDT>::type;
  using YT = typename Storage<YDT>::type;
  const XT *x = static_cast<const XT *>(xv);
  YT *y = static_cast<YT *>(yv);
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = __uint_as_float(table_bits(QT)[threadIdx.x]);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int64_t pieces = K >> 5;  // 16-byte pieces per row

  for (int64_t n = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6; n < N; n += nwaves) {
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;
    for (int64_t pc = lane; pc < pieces; pc += 64) {
      const int64_t e0 = n * K + (pc << 5);
      const float a = block_scale<DQ>(sc, e0 >> log2bs);
      const uint4 p = *reinterpret_cast<const uint4 *>(packed + (e0 >> 1));
      const uint32_t pw[4] = {p.x, p.y, p.z, p.w};
      float part[M];
#pragma unroll
      for (int m = 0; m < M; ++m) part[m] = 0.f;
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        const uint32_t byte = (pw[b >> 2] >> (8 * (b & 3))) & 0xffu;
        const float t0 = lut[byte >> 4];
        const float t1 = lut[byte & 15u];
        const int64_t k = (pc << 5) + 2 * b;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          part[m] = fmaf(t0, load_elem<XDT>(x, m * K + k), part[m]);
          part[m] = fmaf(t1, load_elem<XDT>(x, m * K + k + 1), part[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = fmaf(a, part[m], acc[m]);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = acc[m];
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      acc[m] = v;
    }
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < M; ++m) store_elem<YDT>(y, m * N + n, acc[m]);
    }
  }
}

template <int M, int XDT, int YDT>
static hipError_t launch_gemv_m(const void *x, int64_t N, int64_t K, const uint8_t *packed,
                                const Scales &sc, bool dq, int log2bs, int qt, void *y,
                                hipStream_t st) {
  const unsigned grid = (unsigned)std::min<int64_t>((N + 3) / 4, 1 << 16);
#define QMV_G(DQV, QTV)                                                                         \
  hipLaunchKernelGGL((gemv_4bit_kernel<M, XDT, YDT, DQV, QTV>), dim3(grid), dim3(256), 0, st, x, \
                     N, K, packed, sc, log2bs, y)
  if (dq) {
    if (qt == kNF4) QMV_G(true, kNF4); else QMV_G(true, kFP4);
  } else {
    if (qt == kNF4) QMV_G(false, kNF4); else QMV_G(false, kFP4);
  }
#undef QMV_G
  return hipGetLastError();
}

template <int XDT, int YDT>
static hipError_t launch_gemv_xy(const void *x, int M, int64_t N, int64_t K, const uint8_t *packed,
                                 const Scales &sc, bool dq, int log2bs, int qt, void *y,
                                 hipStream_t st) {
  switch (M) {
    case 1: return launch_gemv_m<1, XDT, YDT>(x, N, K, packed, sc, dq, log2bs, qt, y, st);
    case 2: return launch_gemv_m<2, XDT, YDT>(x, N, K, packed, sc, dq, log2bs, qt, y, st);
    case 3: return launch_gemv_m<3, XDT, YDT>(x, N, K, packed, sc, dq, log2bs, qt, y, st);
    case 4: return launch_gemv_m<4, XDT, YDT>(x, N, K, packed, sc, dq, log2bs, qt, y, st);
    case 5: return launch_gemv_m<5, XDT, YDT>(x, N, K, packed, sc, dq, log2bs, qt, y, st);
    case 6: return launch_gemv_m<6, XDT, YDT>(x, N, K, packed, sc, dq, log2bs, qt, y, st);
    case 7: return launch_gemv_m<7, XDT, YDT>(x, N, K, packed, sc, dq, log2bs, qt, y, st);
    default: return launch_gemv_m<8, XDT, YDT>(x, N, K, packed, sc, dq, log2bs, qt, y, st);
  }
}

template <int XDT>
static hipError_t launch_gemv_x(const void *x, int M, int64_t N, int64_t K, const uint8_t *packed,
                                const Scales &sc, bool dq, int log2bs, int qt, void *y, int y_dtype,
                                hipStream_t st) {
  if (y_dtype == kF32) return launch_gemv_xy<XDT, kF32>(x, M, N, K, packed, sc, dq, log2bs, qt, y, st);
  if (y_dtype == kF16) return launch_gemv_xy<XDT, kF16>(x, M, N, K, packed, sc, dq, log2bs, qt, y, st);
  return launch_gemv_xy<XDT, kBF16>(x, M, N, K, packed, sc, dq, log2bs, qt, y, st);
}

hipError_t launch_gemv_4bit(const void *x, int x_dtype, int M, int64_t N, int64_t K,
                            const uint8_t *packed, const Scales &sc, bool dq, int log2bs, int qt,
                            void *y, int y_dtype, hipStream_t st) {
  if (x_dtype == kF32) return launch_gemv_x<kF32>(x, M, N, K, packed, sc, dq, log2bs, qt, y, y_dtype, st);
  if (x_dtype == kF16) return launch_gemv_x<kF16>(x, M, N, K, packed, sc, dq, log2bs, qt, y, y_dtype, st);
  return launch_gemv_x<kBF16>(x, M, N, K, packed, sc, dq, log2bs, qt, y, y_dtype, st);
}

}  // namespace qmv
