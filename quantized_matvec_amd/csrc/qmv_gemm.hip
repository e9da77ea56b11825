// gemm_4bit: C[M, N] = A[M, K] @ W_hat[N, K]^T for general M
// ("Feat/mps gemm 4bit bf16", table "What runs natively now": gemm_4bit).
//
// The pages' design dequantizes into a scratch buffer and then runs a GEMM.
// Here the weight never leaves the chip in bf16: each 128 x 32 weight tile is
// read packed (16 bytes per row), dequantized by VALU into an LDS tile, and
// consumed by bf16 matrix-core instructions (v_mfma_f32_32x32x16_bf16) with
// fp32 accumulation.  A 256-thread workgroup computes a 128 x 128 C tile as
// 2 x 2 waves of 64 x 64.
#include <algorithm>

#include "qmv_launch.hpp"

namespace qmv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kLds = kBK + 8;  // padded LDS row, in bf16 elements (80 bytes)

template <int CDT, bool DQ, int QT>
__global__ __launch_bounds__(256) void gemm_4bit_kernel(const uint16_t *__restrict__ A, int64_t M,
                                                        int64_t N, int64_t K,
                                                        const uint8_t *__restrict__ packed,
                                                        Scales sc, int log2bs,
                                                        void *__restrict__ Cv) {
  using CT = typename Storage<CDT>::type;
  CT *C = static_cast<CT *>(Cv);
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLds];
  __shared__ float lut[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  if (tid < 16) lut[tid] = __uint_as_float(table_bits(QT)[tid]);

  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int64_t n0 = (int64_t)blockIdx.x * kBN;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  __syncthreads();

  for (int64_t k0 = 0; k0 < K; k0 += kBK) {
    {  // A tile: 128 rows x 64 bytes, two 16-byte pieces per thread
      const int r = tid >> 1, h = tid & 1;
      const int64_t gm = m0 + r;
      uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
      if (gm < M) {
        const uint4 *src = reinterpret_cast<const uint4 *>(A + gm * K + k0 + h * 16);
        v0 = src[0];
        v1 = src[1];
      }
      *reinterpret_cast<uint4 *>(&As[r * kLds + h * 16]) = v0;
      *reinterpret_cast<uint4 *>(&As[r * kLds + h * 16 + 8]) = v1;
    }
    if (tid < kBN) {  // B tile: one packed 16-byte row piece per thread -> 32 bf16
      const int64_t gn = n0 + tid;
      uint32_t o[16];
#pragma unroll
      for (int b = 0; b < 16; ++b) o[b] = 0;
      if (gn < N) {
        const int64_t e0 = gn * K + k0;
        const float a = block_scale<DQ>(sc, e0 >> log2bs);
        const uint4 p = *reinterpret_cast<const uint4 *>(packed + (e0 >> 1));
        const uint32_t pw[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int b = 0; b < 16; ++b) {
          const uint32_t byte = (pw[b >> 2] >> (8 * (b & 3))) & 0xffu;
          const uint32_t h0 = f32_to_bf16_rne(lut[byte >> 4] * a);
          const uint32_t h1 = f32_to_bf16_rne(lut[byte & 15u] * a);
          o[b] = h0 | (h1 << 16);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint4 *>(&Bs[tid * kLds + 8 * q]) =
            make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + (lane & 31);
        a[i] = *reinterpret_cast<const bf16x8_t *>(&As[row * kLds + ks * 16 + (lane >> 5) * 8]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wn * 64 + j * 32 + (lane & 31);
        b[j] = *reinterpret_cast<const bf16x8_t *>(&Bs[col * kLds + ks * 16 + (lane >> 5) * 8]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // 32 x 32 accumulator layout: column = lane % 32,
  // row = 8 * (r / 4) + 4 * (lane / 32) + r % 4 for accumulator register r.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) store_elem<CDT>(C, row * N + col, acc[i][j][r]);
      }
    }
}

hipError_t launch_gemm_4bit(const void *A, int64_t M, int64_t N, int64_t K, const uint8_t *packed,
                            const Scales &sc, bool dq, int log2bs, int qt, void *C, int c_dtype,
                            hipStream_t st) {
  const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
  const uint16_t *a = static_cast<const uint16_t *>(A);
#define QMV_M(CDT, DQV, QTV)                                                                    \
  hipLaunchKernelGGL((gemm_4bit_kernel<CDT, DQV, QTV>), grid, dim3(256), 0, st, a, M, N, K, \
                     packed, sc, log2bs, C)
#define QMV_MQ(CDT, DQV) \
  if (qt == kNF4) QMV_M(CDT, DQV, kNF4); else QMV_M(CDT, DQV, kFP4)
#define QMV_MD(CDT) \
  if (dq) { QMV_MQ(CDT, true); } else { QMV_MQ(CDT, false); }
  if (c_dtype == kF32) { QMV_MD(kF32); }
  else if (c_dtype == kF16) { QMV_MD(kF16); }
  else { QMV_MD(kBF16); }
#undef QMV_MD
#undef QMV_MQ
#undef QMV_M
  return hipGetLastError();
}

}  // namespace qmv
