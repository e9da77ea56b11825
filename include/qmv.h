/*
 * qmv.h -- C ABI of libqmv.so: 4-bit blockwise weight quantization (NF4 / FP4,
 * optional double-quantized scales) and the fused dequantize-and-multiply, as
 * hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * The op set follows the pull-request page "Feat/mps gemm 4bit bf16", table
 * "What runs natively now": quantize_4bit / dequantize_4bit (with .out forms),
 * gemv_4bit (a fused dequant + dot for the decode step) and gemm_4bit (general
 * M).  Block size and double quantization follow "mps-bitsandbytes 0.4.7",
 * section "Functional API" (quantize_nf4(tensor, block_size=64),
 * double_quant(absmax, double_quant_block=256), dequant_absmax).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Ownership: every array argument is caller-owned.  Device arrays are plain
 *   device pointers (for example torch tensor data pointers); the library never
 *   allocates, frees or keeps a pointer after the call returns.
 * - Streams: ``stream`` is a hipStream_t (NULL = the null stream).  Work is
 *   enqueued asynchronously on it; no call synchronizes the host.
 * - Errors: every call returns a qmv_status.  All argument checks run on the
 *   host before anything is enqueued, so a non-zero status means nothing was
 *   launched and no output was touched.  There is no fallback path.  Faults
 *   inside a kernel surface at the caller's next synchronization.
 * - Alignment: device pointers must be 16-byte aligned (QMV_ERR_ALIGNMENT).
 * - Layout: a weight W is [N, K] row-major (out_features, in_features) and is
 *   handled as its row-major flattening of numel elements.  Blocks are runs of
 *   ``blocksize`` consecutive elements; the last block may be partial.
 *   packed[j] holds element 2j in its high nibble and element 2j+1 in its low
 *   nibble; an odd tail leaves the last low nibble 0.
 * - Codes: NF4 code c is the c-th smallest NF4 value (c = 7 is 0, c = 0 is -1,
 *   c = 15 is +1).  FP4 code bits are s e1 e0 m of an E2M1 number, scaled by
 *   1/6 so the largest magnitude is 1.  The nearest code is found exactly; an
 *   exact tie goes to the smaller magnitude, and a value that rounds to zero
 *   gets the lowest zero code.
 * - Numbers: inputs must be finite; NaN / Inf behaviour is unspecified.
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QMV_OK = 0,
  QMV_ERR_INVALID_ARG = -1, /* null pointer, negative or inconsistent size, bad enum */
  QMV_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels cover (blocksize, K % 32, M range, table) */
  QMV_ERR_ALIGNMENT = -3,   /* a device pointer is not 16-byte aligned */
  QMV_ERR_LAUNCH = -4,      /* the HIP runtime refused a kernel launch */
  QMV_ERR_HIP = -5,         /* another HIP runtime call failed */
  QMV_ERR_WORKSPACE = -6,   /* workspace missing, misaligned or smaller than its size query */
  QMV_ERR_TOO_LARGE = -7    /* more scales than qmv_double_quant_noalloc's fixed scratch holds */
} qmv_status;

typedef enum { QMV_NF4 = 0, QMV_FP4 = 1 } qmv_quant_type;
typedef enum { QMV_F32 = 0, QMV_F16 = 1, QMV_BF16 = 2 } qmv_dtype;

/*
 * Per-block scales, either plain fp32 (absmax != NULL, the DQ fields NULL) or
 * double-quantized (absmax == NULL, every DQ field set).  Double quantization
 * ("mps-bitsandbytes 0.4.7", "Features": double quantization of the scales)
 * stores 8-bit codes of (absmax - offset) per group of blocksize2 scales:
 *   a_hat[b] = fp32( fp32(code2[absmax_q[b]] * absmax2[b / blocksize2]) + offset[0] )
 * with two separate roundings (no fused multiply-add).
 */
typedef struct {
  const float *absmax;     /* [nblocks] fp32 (device), or NULL when double-quantized */
  const uint8_t *absmax_q; /* [nblocks] 8-bit codes (device) */
  const float *absmax2;    /* [ceil(nblocks / blocksize2)] fp32 group scales (device) */
  const float *code2;      /* [256] fp32 second-level table (device) */
  const float *offset;     /* [1] fp32 mean that was subtracted (device) */
  int32_t blocksize2;      /* group size of the second level: power of two in [32, 4096] */
} qmv_absmax;

/*
 * quantize_4bit ("Feat/mps gemm 4bit bf16", "What runs natively now";
 * "mps-bitsandbytes 0.4.7", "Functional API": quantize_nf4 / quantize_fp4).
 *   W       [numel] device, element type w_dtype (F32, F16 or BF16)
 *   numel   > 0
 *   blocksize  power of two in [32, 4096]
 *   packed  [ceil(numel / 2)] device out
 *   absmax  [ceil(numel / blocksize)] device out: per-block max |W| (exact)
 * Codes are the exact nearest code of W / absmax (bit-exact, deterministic).
 */
int qmv_quantize_4bit(const void *W, qmv_dtype w_dtype, int64_t numel, int32_t blocksize,
                      qmv_quant_type quant_type, uint8_t *packed, float *absmax, void *stream);

/* Bytes of device workspace qmv_double_quant needs for ``nblocks`` scales in
 * groups of ``blocksize2`` (the partial sums of the mean and the exponent
 * bounds of their inputs; the mean's tree does not depend on blocksize2).
 * Returns 0 when nblocks <= 0 or blocksize2 is not a power of two in
 * [32, 4096]. */
size_t qmv_double_quant_workspace(int64_t nblocks, int32_t blocksize2);

/*
 * double_quant ("mps-bitsandbytes 0.4.7", "Functional API", Double
 * Quantization: double_quant(absmax, double_quant_block=256)).
 * The second-level table comes in on the host and goes out on the device:
 * the host checks that its midpoints are exact before anything is launched
 * (the encoder's exactness depends on it), and the device copy is what every
 * decoding call (qmv_absmax.code2) reads.
 *   absmax      [nblocks] device fp32 scales (non-negative)
 *   blocksize2  power of two in [32, 4096] (256 in the reference usage)
 *   code2_host  [256] HOST fp32 table, strictly increasing, or NULL for the
 *               default (k - 127) / 127.  Tables whose adjacent midpoints are
 *               not exactly representable with at most 29 significant bits
 *               are refused (QMV_ERR_UNSUPPORTED): the encoder's decisions are
 *               exact only for those.
 *   absmax_q    [nblocks] device out: nearest code of (absmax - offset) / absmax2
 *   absmax2     [ceil(nblocks / blocksize2)] device out: max |absmax - offset| per group
 *   offset      [1] device out: fp32(S / nblocks), S the float64 sum of the
 *               scales taken in a fixed tree (sequential runs of 256, repeated)
 *   code2_out   [256] device out: the table used, for the decode side
 *   workspace   device scratch of at least
 *               qmv_double_quant_workspace(nblocks, blocksize2) bytes (any
 *               contents); calls that share a workspace must not overlap.
 *               QMV_ERR_WORKSPACE when it is NULL or smaller.
 */
int qmv_double_quant(const float *absmax, int64_t nblocks, int32_t blocksize2,
                     const float *code2_host, uint8_t *absmax_q, float *absmax2, float *offset,
                     float *code2_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * double_quant without a workspace and without any allocation: for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The same operation,
 * kernels and results as qmv_double_quant; the mean's partial sums go to a
 * scratch array of 576 KiB that the library holds in each GPU's memory until
 * the process ends (its address is looked up once per device on the first
 * call there).  Arguments as for qmv_double_quant, without the workspace.
 *   nblocks  at most 2^24 (16,777,216 scales), else QMV_ERR_TOO_LARGE
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (on different streams or from different threads) race.
 */
int qmv_double_quant_noalloc(const float *absmax, int64_t nblocks, int32_t blocksize2,
                             const float *code2_host, uint8_t *absmax_q, float *absmax2,
                             float *offset, float *code2_out, void *stream);

/* dequant_absmax ("Functional API": dequant_absmax).  absmax_out [nblocks]
 * device fp32; with plain scales it is a copy. */
int qmv_dequantize_absmax(const qmv_absmax *scales, int64_t nblocks, float *absmax_out, void *stream);

/*
 * dequantize_4bit and its .out form ("What runs natively now").
 *   out[i] = fp32(T[code_i] * a_hat[i / blocksize]) converted to out_dtype by
 *   round-to-nearest-even; bit-exact.
 *   out  [numel] device, element type out_dtype
 */
int qmv_dequantize_4bit(const uint8_t *packed, const qmv_absmax *scales, int64_t numel,
                        int32_t blocksize, qmv_quant_type quant_type, void *out,
                        qmv_dtype out_dtype, void *stream);

/*
 * gemv_4bit: the decode step ("What runs natively now": gemv_4bit as a fused
 * dequant + dot), widened to 1 <= M <= 8 rows of activations.
 *   y[m, n] = sum_k x[m, k] * W_hat[n, k], fp32 accumulation.
 *   x  [M, K] device row-major, x_dtype;  y [M, N] device row-major, y_dtype
 *   W_hat is [N, K]: packed [N * K / 2], scales for N * K / blocksize blocks.
 *   bias  NULL, or [N] device in y_dtype ("mps-bitsandbytes 0.4.7",
 *         "Functional API": matmul_nf4's bias argument): y[m, n] = the fp32
 *         sum + fp32(bias[n]), one fp32 addition, then one rounding to y_dtype.
 *         Aligned to its element size (QMV_ERR_ALIGNMENT).
 * x_dtype fp32 computes in fp32 (fp32 weights and products); bf16 / fp16 x
 * multiply the weights rounded to x's type ("Feat/mps gemm 4bit bf16",
 * "Performance": gemv over fp16 / bf16 / fp32).
 * Requires K % blocksize == 0 and K % 32 == 0 ("unsupported blocksize" and
 * "K % 32 != 0" are the guards the PR page lists), else QMV_ERR_UNSUPPORTED.
 */
int qmv_gemv_4bit(const void *x, qmv_dtype x_dtype, int32_t M, int64_t N, int64_t K,
                  const uint8_t *packed, const qmv_absmax *scales, int32_t blocksize,
                  qmv_quant_type quant_type, void *y, qmv_dtype y_dtype, const void *bias,
                  void *stream);

/*
 * gemm_4bit: general M ("What runs natively now": gemm_4bit).
 *   A [M, K] device row-major, a_dtype;  C [M, N] device row-major, c_dtype
 *   bias  NULL or [N] in c_dtype, as for gemv_4bit ("Functional API":
 *         matmul_nf4(..., bias)).
 * a_dtype bf16 / fp16: the weight is dequantized tile by tile into LDS exactly
 * as dequantize_4bit returns it in a_dtype and multiplied on the matrix cores
 * in that type (v_mfma_f32_32x32x16_bf16 / _f16), fp32 accumulation.
 * a_dtype fp32: fp32 weights, products and sums on the vector units, 8 rows
 * per pass (slow for large M).
 * Requires K % blocksize == 0 and K % 32 == 0.
 */
int qmv_gemm_4bit(const void *A, qmv_dtype a_dtype, int64_t M, int64_t N, int64_t K,
                  const uint8_t *packed, const qmv_absmax *scales, int32_t blocksize,
                  qmv_quant_type quant_type, void *C, qmv_dtype c_dtype, const void *bias,
                  void *stream);

/*
 * quantize_blockwise / dequantize_blockwise: the general 8-bit blockwise codec
 * ("Feat/mps gemm 4bit bf16", table "What runs natively now": quantize_blockwise
 * / dequantize_blockwise; "Known failures": the exact float64 nearest-code
 * search is the reference, a normalised-value lookup table is not).
 *   quantize:   absmax[b] = max |A_i| over block b (fp32, exact);
 *               q[i] = code index nearest to A_i / absmax[b], exactly (ties
 *               toward zero; a zero block gives the code of 0, whose index
 *               is the table's).
 *   dequantize: out[i] = fp32(code[q[i]] * absmax[i / blocksize]), rounded to
 *               out_dtype (round to nearest even).
 *   A          [n] device, a_dtype (fp32 / fp16 / bf16)
 *   q          [n] device uint8;  absmax [ceil(n / blocksize)] device fp32
 *   blocksize  power of two in [32, 4096]
 *   code_host  [256] HOST fp32 table (as for qmv_double_quant: strictly
 *              increasing, midpoints exact with <= 29 significant bits, else
 *              QMV_ERR_UNSUPPORTED), or NULL for (k - 127) / 127.
 * Buffers are the caller's, 16-byte aligned (QMV_ERR_ALIGNMENT).
 */
int qmv_quantize_blockwise(const void *A, qmv_dtype a_dtype, int64_t n, int32_t blocksize,
                           const float *code_host, uint8_t *q, float *absmax, void *stream);
int qmv_dequantize_blockwise(const uint8_t *q, const float *absmax, int64_t n, int32_t blocksize,
                             const float *code_host, void *out, qmv_dtype out_dtype, void *stream);

/*
 * gemm_4bit_backward: the input gradient of a 4-bit linear layer ("Feat/mps
 * gemm 4bit bf16", table "What runs natively now": gemm_4bit_backward, the
 * fused form of grad_output @ dequantize_4bit(B)).
 *   dX[m, k] = sum_n dY[m, n] * W_hat[n, k], fp32 accumulation.
 *   dY [M, N] device row-major bf16 or fp16;  dX [M, K] device row-major, dx_dtype
 *   W_hat [N, K] as for gemm_4bit (the same packed codes and scales).
 * The weight is dequantized tile by tile exactly as by dequantize_4bit to
 * dY's type and multiplied on the matrix cores in that type.  No bias: the
 * backward has no epilogue.
 *   workspace  device scratch of at least qmv_gemm_4bit_backward_workspace(M,
 *              N, K, blocksize) bytes, 16-byte aligned, any contents (NULL
 *              when that is 0; QMV_ERR_WORKSPACE when missing or smaller).
 *              When the reduction over N is split across workgroups it holds
 *              one counter per output tile, which the call zeroes on its
 *              stream first, and the fp32 partial tiles.  Calls that share a
 *              workspace must not overlap.
 * Requires dy_dtype bf16 or fp16, N % 32 == 0, K % blocksize == 0 and
 * K % 32 == 0, else QMV_ERR_UNSUPPORTED.  Buffers are the caller's; dX is
 * fully overwritten.
 */
size_t qmv_gemm_4bit_backward_workspace(int64_t M, int64_t N, int64_t K, int32_t blocksize);
int qmv_gemm_4bit_backward(const void *dY, qmv_dtype dy_dtype, int64_t M, int64_t N, int64_t K,
                           const uint8_t *packed, const qmv_absmax *scales, int32_t blocksize,
                           qmv_quant_type quant_type, void *dX, qmv_dtype dx_dtype, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * embedding_4bit: rows of a 4-bit quantized embedding table
 * ("mps-bitsandbytes 0.4.7", "Quantized Embeddings": Embedding4bit,
 * EmbeddingNF4, EmbeddingFP4).
 *   W [V, D] quantized as one flat tensor by qmv_quantize_4bit (packed
 *   [ceil(V * D / 2)], scales for ceil(V * D / blocksize) blocks, plain or
 *   double-quantized).
 *   out[t, d] = dequantize_4bit(W)[idx[t], d], bit for bit (fp32(T * a_hat)
 *   rounded to out_dtype); a row whose index is outside [0, V) is zeros
 *   (the kernel checks each index; nothing faults).
 *   idx  [T] device int64, 8-byte aligned;  out [T, D] device row-major, out_dtype
 * Buffers are the caller's; packed and out 16-byte aligned (QMV_ERR_ALIGNMENT).
 */
int qmv_embedding_4bit(const int64_t *idx, int64_t T, int64_t V, int64_t D, const uint8_t *packed,
                       const qmv_absmax *scales, int32_t blocksize, qmv_quant_type quant_type,
                       void *out, qmv_dtype out_dtype, void *stream);

/* Host-side: the 16 fp32 code values the kernels use, by code. */
int qmv_code_table(qmv_quant_type quant_type, float out16[16]);

/* Host-side: the default 256-entry second-level table, (k - 127) / 127 in fp32. */
int qmv_default_code2(float out256[256]);

/* Host-side: the signed dynamic-tree 8-bit table, ascending, for
 * qmv_quantize_blockwise / qmv_dequantize_blockwise and double quantization
 * ("Feat/mps gemm 4bit bf16", "What runs natively now": the 8-bit blockwise
 * codec; the pages name no table, so this is the reading taken): after the
 * sign bit, a run of e zero bits (e = 0..6) is a decimal exponent, then a one
 * bit, then 6 - e fraction bits j picking the centre of bin j of [0.1, 1] cut
 * into 2^(6-e) bins.  Each value 10^-e (0.1 + 0.9 (j + 1/2) / 2^(6-e)) is
 * rounded once, exactly, to fp32; with their negatives, 0 and 1 that is 256
 * strictly increasing values. */
int qmv_dynamic_code2(float out256[256]);

/* Host-side: a static, human-readable name of a qmv_status value. */
const char *qmv_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* QMV_H */
