// Host-side launchers of the HIP kernels (internal to libqmv.so).  Each
// launcher assumes its arguments were validated by the C ABI layer and only
// maps them onto a grid; it returns the status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv_device.hpp"

namespace qmv {

// Midpoints of adjacent distinct values of a sorted code table, exact in
// float64; the encoder compares x against absmax * mid[j].  NF4 uses all 15,
// FP4 (whose +0 and -0 are one value) the first 14.
struct Midpoints4 {
  double mid[15];
};

struct Code2Table {
  float v[256];
};

int log2_exact(int64_t v);  // log2 of a power of two

hipError_t launch_quantize_4bit(const void *W, int w_dtype, int64_t numel, int log2bs, int qt,
                                const Midpoints4 &mids, uint8_t *packed, float *absmax,
                                hipStream_t st);

size_t double_quant_workspace_bytes(int64_t nblocks);

// The allocation-free double quantization: most scales it takes, and its
// per-device scratch (at least double_quant_workspace_bytes of that many).
constexpr int64_t kNoAllocMaxBlocks = int64_t(1) << 24;
hipError_t double_quant_scratch(void **ptr);

// ws: double_quant_workspace_bytes(nblocks) bytes for the partial sums.
// linear: code2 is the default table (k - 127) / 127.
hipError_t launch_double_quant(const float *absmax, int64_t nblocks, int log2bs2,
                               const Code2Table &code2, bool linear, uint8_t *q, float *absmax2,
                               float *offset, float *code2_out, void *ws, hipStream_t st);

hipError_t launch_dequantize_absmax(const Scales &sc, bool dq, int64_t nblocks, float *out,
                                    hipStream_t st);

hipError_t launch_dequantize_4bit(const uint8_t *packed, const Scales &sc, bool dq, int64_t numel,
                                  int log2bs, int qt, void *out, int out_dtype, hipStream_t st);

// bias: NULL or [N] in the output type, added to the fp32 result before the
// one rounding to the output type.
hipError_t launch_gemv_4bit(const void *x, int x_dtype, int M, int64_t N, int64_t K,
                            const uint8_t *packed, const Scales &sc, bool dq, int log2bs, int qt,
                            void *y, int y_dtype, const void *bias, hipStream_t st);

// Compute units of the current device (cached per device).
int device_cu_count();

// Workgroups of `threads` threads of `kernel` resident on one compute unit at
// once (at least 1).  A grid-stride kernel launched with this many per unit
// runs in one generation, with no partly filled second one.
int resident_wgs_per_cu(const void *kernel, int threads);

// True when gemm_4bit takes its narrow kernel: M <= 16 rows, blocks of 64 or
// more, K a multiple of 64 (below 2^23).
inline bool gemm_narrow_eligible(int64_t M, int64_t K, int log2bs) {
  return M <= 16 && log2bs >= 6 && K % 64 == 0 && K < (1 << 23);
}
// True when gemm_4bit takes its large-M kernel (128 x 256 tiles): at least
// 448 rows (four row tiles: the grid covers most compute units), K a
// multiple of 64 and its offsets within 32 bits.
inline bool gemm_rb_eligible(int64_t M, int64_t N, int64_t K) {
  return M >= 448 && K % 64 == 0 && K < (1 << 22) &&
         ((N + 255) / 256) * ((M + 127) / 128) < ((int64_t)1 << 31);
}
// Host-side launch plan of gemm_4bit (16-bit activations): see qmv_gemm.hip.
int64_t gemm_plan(int64_t M, int64_t N, int64_t K, int log2bs, int64_t *tiles, int64_t cap, int *kind);
// a_dtype: kBF16 or kF16 (the matrix cores' input type); bias as for gemv.
hipError_t launch_gemm_4bit(const void *A, int a_dtype, int64_t M, int64_t N, int64_t K,
                            const uint8_t *packed, const Scales &sc, bool dq, int log2bs, int qt,
                            void *C, int c_dtype, const void *bias, hipStream_t st);

hipError_t launch_quantize_blockwise(const void *A, int a_dtype, int64_t n, int log2bs,
                                     const Code2Table &code, bool linear, uint8_t *q,
                                     float *absmax, hipStream_t st);

hipError_t launch_dequantize_blockwise(const uint8_t *q, const float *absmax, int64_t n, int log2bs,
                                       const Code2Table &code, void *out, int out_dtype,
                                       hipStream_t st);

// idx: T int64 row indices (device); out [T, D] of out_dtype.
hipError_t launch_embedding_4bit(const int64_t *idx, int64_t T, int64_t V, int64_t D,
                                 const uint8_t *packed, const Scales &sc, bool dq, int log2bs,
                                 int qt, void *out, int out_dtype, hipStream_t st);

// Bytes of workspace launch_gemm_4bit_backward needs (0: none).
size_t gemm_backward_workspace_bytes(int64_t M, int64_t N, int64_t K, int log2bs);
hipError_t launch_gemm_4bit_backward(const void *dY, int dy_dtype, int64_t M, int64_t N, int64_t K,
                                     const uint8_t *packed, const Scales &sc, bool dq, int log2bs,
                                     int qt, void *dX, int dx_dtype, void *ws, hipStream_t st);

}  // namespace qmv
