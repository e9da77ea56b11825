// The C ABI of libqmv.so (declared in include/qmv.h): argument validation on
// the host, then a launch on the caller's stream.  Nothing here allocates,
// synchronizes or falls back to another path.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <set>
#include <vector>

#include "qmv.h"
#include "qmv_probe.h"
#include "qmv_launch.hpp"

namespace qmv {
// the streaming-read probe (qmv_probe.hip)
hipError_t launch_stream_read(const void *p, int64_t bytes, uint32_t *sink, hipStream_t st);
}  // namespace qmv

using namespace qmv;

namespace {

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_dtype(int d) { return d == QMV_F32 || d == QMV_F16 || d == QMV_BF16; }
bool valid_qt(int q) { return q == QMV_NF4 || q == QMV_FP4; }
bool valid_blocksize(int64_t bs) { return is_pow2(bs) && bs >= 32 && bs <= 4096; }

float bits_to_float(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// Significant bits of a finite nonzero double.
int sig_bits(double d) {
  int e;
  double m = frexp(fabs(d), &e);  // m in [0.5, 1)
  int bits = 0;
  while (m != 0.0) {
    m = m * 2.0;
    const double ip = floor(m);
    m -= ip;
    ++bits;
  }
  return bits;
}

// Midpoint of two doubles if it is exact, else NaN.
double exact_midpoint(double lo, double hi) {
  const double s = lo + hi;
  const double bb = s - lo;
  const double err = (lo - (s - bb)) + (hi - bb);  // TwoSum error term
  if (err != 0.0) return NAN;
  return s * 0.5;  // halving is exact for these magnitudes
}

// Sorted distinct values of the 16-entry table and their midpoints.
Midpoints4 table_midpoints(int qt) {
  const uint32_t *bits = table_bits(qt);
  std::set<double> vals;
  for (int c = 0; c < 16; ++c) vals.insert((double)bits_to_float(bits[c]));  // +0 == -0
  std::vector<double> v(vals.begin(), vals.end());
  Midpoints4 m{};
  for (size_t j = 0; j + 1 < v.size() && j < 15; ++j) m.mid[j] = exact_midpoint(v[j], v[j + 1]);
  return m;
}

const Midpoints4 &midpoints(int qt) {
  static const Midpoints4 nf4 = table_midpoints(QMV_NF4);
  static const Midpoints4 fp4 = table_midpoints(QMV_FP4);
  return qt == QMV_NF4 ? nf4 : fp4;
}

int check_scales(const qmv_absmax *s, Scales *out, bool *dq) {
  if (!s) return QMV_ERR_INVALID_ARG;
  const bool plain = s->absmax != nullptr;
  const bool any_dq = s->absmax_q || s->absmax2 || s->code2 || s->offset;
  const bool all_dq = s->absmax_q && s->absmax2 && s->code2 && s->offset;
  if (plain == any_dq) return QMV_ERR_INVALID_ARG;  // exactly one form
  if (!plain && !all_dq) return QMV_ERR_INVALID_ARG;
  Scales sc{};
  if (plain) {
    if (!aligned16(s->absmax)) return QMV_ERR_ALIGNMENT;
    sc.absmax = s->absmax;
  } else {
    if (!valid_blocksize(s->blocksize2)) return QMV_ERR_UNSUPPORTED;
    if (!aligned16(s->absmax_q) || !aligned16(s->absmax2) || !aligned16(s->code2) ||
        !aligned16(s->offset))
      return QMV_ERR_ALIGNMENT;
    sc.q = s->absmax_q;
    sc.absmax2 = s->absmax2;
    sc.code2 = s->code2;
    sc.offset = s->offset;
    sc.log2bs2 = log2_exact(s->blocksize2);
  }
  *out = sc;
  *dq = !plain;
  return QMV_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? QMV_OK : QMV_ERR_LAUNCH; }

int check_matmul(int64_t M, int64_t N, int64_t K, int32_t blocksize, int qt) {
  if (M <= 0 || N <= 0 || K <= 0 || !valid_qt(qt)) return QMV_ERR_INVALID_ARG;
  if (!valid_blocksize(blocksize)) return QMV_ERR_UNSUPPORTED;
  if (K % blocksize != 0 || K % 32 != 0) return QMV_ERR_UNSUPPORTED;
  if (N > INT64_MAX / K || M > INT64_MAX / K || M > INT64_MAX / N) return QMV_ERR_INVALID_ARG;
  return QMV_OK;
}

}  // namespace

extern "C" {

int qmv_quantize_4bit(const void *W, qmv_dtype w_dtype, int64_t numel, int32_t blocksize,
                      qmv_quant_type quant_type, uint8_t *packed, float *absmax, void *stream) {
  if (!W || !packed || !absmax || numel <= 0 || !valid_dtype(w_dtype) || !valid_qt(quant_type))
    return QMV_ERR_INVALID_ARG;
  if (!valid_blocksize(blocksize)) return QMV_ERR_UNSUPPORTED;
  if (!aligned16(W) || !aligned16(packed) || !aligned16(absmax)) return QMV_ERR_ALIGNMENT;
  const int nt = quant_type == QMV_NF4 ? 15 : 14;  // thresholds between distinct values
  for (int j = 0; j < nt; ++j) {  // the exactness argument needs these
    const double m = midpoints(quant_type).mid[j];
    if (isnan(m) || m == 0.0 || sig_bits(m) > 29) return QMV_ERR_UNSUPPORTED;
  }
  return launch_status(launch_quantize_4bit(W, w_dtype, numel, log2_exact(blocksize), quant_type,
                                            midpoints(quant_type), packed, absmax,
                                            (hipStream_t)stream));
}

size_t qmv_double_quant_workspace(int64_t nblocks, int32_t blocksize2) {
  return nblocks > 0 && valid_blocksize(blocksize2) ? double_quant_workspace_bytes(nblocks) : 0;
}

// A second-level table is usable when it is finite and strictly increasing
// and every midpoint of neighbours is nonzero and exact with <= 29
// significant bits (so the encoder's float64 thresholds are exact).
static int check_code2(const Code2Table &t) {
  for (int k = 0; k < 256; ++k)
    if (!isfinite(t.v[k])) return QMV_ERR_INVALID_ARG;
  for (int k = 0; k + 1 < 256; ++k) {
    if (!(t.v[k] < t.v[k + 1])) return QMV_ERR_UNSUPPORTED;  // strictly increasing
    const double m = exact_midpoint((double)t.v[k], (double)t.v[k + 1]);
    if (isnan(m) || m == 0.0 || sig_bits(m) > 29) return QMV_ERR_UNSUPPORTED;
  }
  return QMV_OK;
}

// The caller's table (or the default), validated as for double_quant.
static int code_table8(const float *code_host, Code2Table &t, bool &linear) {
  static const Code2Table kDefault = [] {
    Code2Table d{};
    qmv_default_code2(d.v);
    return d;
  }();
  static const int kDefaultStatus = check_code2(kDefault);
  t = kDefault;
  linear = true;
  if (code_host) {
    memcpy(t.v, code_host, sizeof(t.v));
    linear = memcmp(t.v, kDefault.v, sizeof(t.v)) == 0;
  }
  return linear ? kDefaultStatus : check_code2(t);
}

int qmv_double_quant(const float *absmax, int64_t nblocks, int32_t blocksize2,
                     const float *code2_host, uint8_t *absmax_q, float *absmax2, float *offset,
                     float *code2_out, void *workspace, size_t workspace_bytes, void *stream) {
  if (!absmax || !absmax_q || !absmax2 || !offset || !code2_out || nblocks <= 0)
    return QMV_ERR_INVALID_ARG;
  if (!valid_blocksize(blocksize2)) return QMV_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < double_quant_workspace_bytes(nblocks))
    return QMV_ERR_WORKSPACE;
  if (!aligned16(absmax) || !aligned16(absmax_q) || !aligned16(absmax2) || !aligned16(offset) ||
      !aligned16(code2_out) || !aligned16(workspace))
    return QMV_ERR_ALIGNMENT;
  // the default table is checked once; a caller's table on every call
  Code2Table t;
  bool linear;
  const int rc = code_table8(code2_host, t, linear);
  if (rc != QMV_OK) return rc;
  return launch_status(launch_double_quant(absmax, nblocks, log2_exact(blocksize2), t, linear,
                                           absmax_q, absmax2, offset, code2_out, workspace,
                                           (hipStream_t)stream));
}

int qmv_double_quant_noalloc(const float *absmax, int64_t nblocks, int32_t blocksize2,
                             const float *code2_host, uint8_t *absmax_q, float *absmax2,
                             float *offset, float *code2_out, void *stream) {
  if (!absmax || !absmax_q || !absmax2 || !offset || !code2_out || nblocks <= 0)
    return QMV_ERR_INVALID_ARG;
  if (!valid_blocksize(blocksize2)) return QMV_ERR_UNSUPPORTED;
  if (nblocks > kNoAllocMaxBlocks) return QMV_ERR_TOO_LARGE;
  if (!aligned16(absmax) || !aligned16(absmax_q) || !aligned16(absmax2) || !aligned16(offset) ||
      !aligned16(code2_out))
    return QMV_ERR_ALIGNMENT;
  Code2Table t;
  bool linear;
  const int rc = code_table8(code2_host, t, linear);
  if (rc != QMV_OK) return rc;
  void *ws = nullptr;  // this device's copy of the library's scratch
  if (double_quant_scratch(&ws) != hipSuccess || ws == nullptr) return QMV_ERR_HIP;
  return launch_status(launch_double_quant(absmax, nblocks, log2_exact(blocksize2), t, linear,
                                           absmax_q, absmax2, offset, code2_out, ws,
                                           (hipStream_t)stream));
}

int qmv_quantize_blockwise(const void *A, qmv_dtype a_dtype, int64_t n, int32_t blocksize,
                           const float *code_host, uint8_t *q, float *absmax, void *stream) {
  if (!A || !q || !absmax || n <= 0 || !valid_dtype(a_dtype)) return QMV_ERR_INVALID_ARG;
  if (!valid_blocksize(blocksize)) return QMV_ERR_UNSUPPORTED;
  if (!aligned16(A) || !aligned16(q) || !aligned16(absmax)) return QMV_ERR_ALIGNMENT;
  Code2Table t;
  bool linear;
  const int rc = code_table8(code_host, t, linear);
  if (rc != QMV_OK) return rc;
  return launch_status(launch_quantize_blockwise(A, a_dtype, n, log2_exact(blocksize), t, linear, q,
                                                 absmax, (hipStream_t)stream));
}

int qmv_dequantize_blockwise(const uint8_t *q, const float *absmax, int64_t n, int32_t blocksize,
                             const float *code_host, void *out, qmv_dtype out_dtype, void *stream) {
  if (!q || !absmax || !out || n <= 0 || !valid_dtype(out_dtype)) return QMV_ERR_INVALID_ARG;
  if (!valid_blocksize(blocksize)) return QMV_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(absmax) || !aligned16(out)) return QMV_ERR_ALIGNMENT;
  Code2Table t;
  bool linear;
  const int rc = code_table8(code_host, t, linear);
  if (rc != QMV_OK) return rc;
  return launch_status(launch_dequantize_blockwise(q, absmax, n, log2_exact(blocksize), t, out,
                                                   out_dtype, (hipStream_t)stream));
}

int qmv_dequantize_absmax(const qmv_absmax *scales, int64_t nblocks, float *absmax_out,
                          void *stream) {
  if (!absmax_out || nblocks <= 0) return QMV_ERR_INVALID_ARG;
  Scales sc;
  bool dq;
  int rc = check_scales(scales, &sc, &dq);
  if (rc != QMV_OK) return rc;
  if (!aligned16(absmax_out)) return QMV_ERR_ALIGNMENT;
  return launch_status(launch_dequantize_absmax(sc, dq, nblocks, absmax_out, (hipStream_t)stream));
}

int qmv_dequantize_4bit(const uint8_t *packed, const qmv_absmax *scales, int64_t numel,
                        int32_t blocksize, qmv_quant_type quant_type, void *out,
                        qmv_dtype out_dtype, void *stream) {
  if (!packed || !out || numel <= 0 || !valid_qt(quant_type) || !valid_dtype(out_dtype))
    return QMV_ERR_INVALID_ARG;
  if (!valid_blocksize(blocksize)) return QMV_ERR_UNSUPPORTED;
  Scales sc;
  bool dq;
  int rc = check_scales(scales, &sc, &dq);
  if (rc != QMV_OK) return rc;
  if (!aligned16(packed) || !aligned16(out)) return QMV_ERR_ALIGNMENT;
  return launch_status(launch_dequantize_4bit(packed, sc, dq, numel, log2_exact(blocksize),
                                              quant_type, out, out_dtype, (hipStream_t)stream));
}

// bias: NULL, or [N] elements of the output type at their natural alignment.
static bool bias_aligned(const void *bias, qmv_dtype out_dtype) {
  const uintptr_t a = out_dtype == QMV_F32 ? 4 : 2;
  return bias == nullptr || (reinterpret_cast<uintptr_t>(bias) % a) == 0;
}

int qmv_gemv_4bit(const void *x, qmv_dtype x_dtype, int32_t M, int64_t N, int64_t K,
                  const uint8_t *packed, const qmv_absmax *scales, int32_t blocksize,
                  qmv_quant_type quant_type, void *y, qmv_dtype y_dtype, const void *bias,
                  void *stream) {
  if (!x || !packed || !y || !valid_dtype(x_dtype) || !valid_dtype(y_dtype))
    return QMV_ERR_INVALID_ARG;
  int rc = check_matmul(M, N, K, blocksize, quant_type);
  if (rc != QMV_OK) return rc;
  if (M > 8) return QMV_ERR_UNSUPPORTED;
  Scales sc;
  bool dq;
  rc = check_scales(scales, &sc, &dq);
  if (rc != QMV_OK) return rc;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(y) || !bias_aligned(bias, y_dtype))
    return QMV_ERR_ALIGNMENT;
  return launch_status(launch_gemv_4bit(x, x_dtype, M, N, K, packed, sc, dq, log2_exact(blocksize),
                                        quant_type, y, y_dtype, bias, (hipStream_t)stream));
}

int qmv_gemm_4bit(const void *A, qmv_dtype a_dtype, int64_t M, int64_t N, int64_t K,
                  const uint8_t *packed, const qmv_absmax *scales, int32_t blocksize,
                  qmv_quant_type quant_type, void *C, qmv_dtype c_dtype, const void *bias,
                  void *stream) {
  if (!A || !packed || !C || !valid_dtype(a_dtype) || !valid_dtype(c_dtype))
    return QMV_ERR_INVALID_ARG;
  int rc = check_matmul(M, N, K, blocksize, quant_type);
  if (rc != QMV_OK) return rc;
  if ((M + 127) / 128 > 65535) return QMV_ERR_UNSUPPORTED;
  Scales sc;
  bool dq;
  rc = check_scales(scales, &sc, &dq);
  if (rc != QMV_OK) return rc;
  if (!aligned16(A) || !aligned16(packed) || !aligned16(C) || !bias_aligned(bias, c_dtype))
    return QMV_ERR_ALIGNMENT;
  return launch_status(launch_gemm_4bit(A, a_dtype, M, N, K, packed, sc, dq, log2_exact(blocksize),
                                        quant_type, C, c_dtype, bias, (hipStream_t)stream));
}

size_t qmv_gemm_4bit_backward_workspace(int64_t M, int64_t N, int64_t K, int32_t blocksize) {
  if (check_matmul(M, N, K, blocksize, QMV_NF4) != QMV_OK) return 0;
  return gemm_backward_workspace_bytes(M, N, K, log2_exact(blocksize));
}

int qmv_gemm_4bit_backward(const void *dY, qmv_dtype dy_dtype, int64_t M, int64_t N, int64_t K,
                           const uint8_t *packed, const qmv_absmax *scales, int32_t blocksize,
                           qmv_quant_type quant_type, void *dX, qmv_dtype dx_dtype, void *workspace,
                           size_t workspace_bytes, void *stream) {
  if (!dY || !packed || !dX || !valid_dtype(dy_dtype) || !valid_dtype(dx_dtype))
    return QMV_ERR_INVALID_ARG;
  int rc = check_matmul(M, N, K, blocksize, quant_type);
  if (rc != QMV_OK) return rc;
  if (dy_dtype == QMV_F32 || N % 32 != 0) return QMV_ERR_UNSUPPORTED;
  if ((M + 127) / 128 > 65535) return QMV_ERR_UNSUPPORTED;
  Scales sc;
  bool dq;
  rc = check_scales(scales, &sc, &dq);
  if (rc != QMV_OK) return rc;
  if (!aligned16(dY) || !aligned16(packed) || !aligned16(dX)) return QMV_ERR_ALIGNMENT;
  const size_t need = gemm_backward_workspace_bytes(M, N, K, log2_exact(blocksize));
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return QMV_ERR_WORKSPACE;
  return launch_status(launch_gemm_4bit_backward(dY, dy_dtype, M, N, K, packed, sc, dq, log2_exact(blocksize),
                                                 quant_type, dX, dx_dtype, workspace, (hipStream_t)stream));
}

int qmv_embedding_4bit(const int64_t *idx, int64_t T, int64_t V, int64_t D, const uint8_t *packed,
                       const qmv_absmax *scales, int32_t blocksize, qmv_quant_type quant_type,
                       void *out, qmv_dtype out_dtype, void *stream) {
  if (!idx || !packed || !out || T <= 0 || V <= 0 || D <= 0 || !valid_qt(quant_type) ||
      !valid_dtype(out_dtype))
    return QMV_ERR_INVALID_ARG;
  if (V > ((int64_t)1 << 62) / D) return QMV_ERR_INVALID_ARG;  // V * D must fit
  if (!valid_blocksize(blocksize)) return QMV_ERR_UNSUPPORTED;
  Scales sc;
  bool dq;
  const int rc = check_scales(scales, &sc, &dq);
  if (rc != QMV_OK) return rc;
  if (reinterpret_cast<uintptr_t>(idx) % 8 != 0 || !aligned16(packed) || !aligned16(out))
    return QMV_ERR_ALIGNMENT;
  return launch_status(launch_embedding_4bit(idx, T, V, D, packed, sc, dq, log2_exact(blocksize),
                                             quant_type, out, out_dtype, (hipStream_t)stream));
}

int qmv_stream_read(const void *p, int64_t bytes, uint32_t *sink, void *stream) {
  if (!p || !sink || bytes <= 0 || bytes % 16 != 0) return QMV_ERR_INVALID_ARG;
  if (!aligned16(p) || reinterpret_cast<uintptr_t>(sink) % 4 != 0) return QMV_ERR_ALIGNMENT;
  return launch_status(launch_stream_read(p, bytes, sink, (hipStream_t)stream));
}

int64_t qmv_gemm_4bit_plan(int64_t M, int64_t N, int64_t K, int32_t blocksize, int64_t *tiles,
                           int64_t cap, int32_t *kernel) {
  const int rc = check_matmul(M, N, K, blocksize, QMV_NF4);
  if (rc != QMV_OK) return rc;
  if (!kernel || cap < 0 || (cap > 0 && !tiles)) return QMV_ERR_INVALID_ARG;
  int kind = 0;
  const int64_t n = gemm_plan(M, N, K, log2_exact(blocksize), tiles, cap, &kind);
  *kernel = kind;
  return n;
}

int qmv_code_table(qmv_quant_type quant_type, float out16[16]) {
  if (!out16 || !valid_qt(quant_type)) return QMV_ERR_INVALID_ARG;
  const uint32_t *bits = table_bits(quant_type);
  for (int c = 0; c < 16; ++c) out16[c] = bits_to_float(bits[c]);
  return QMV_OK;
}

int qmv_default_code2(float out256[256]) {
  if (!out256) return QMV_ERR_INVALID_ARG;
  for (int k = 0; k < 256; ++k) out256[k] = (float)(k - 127) / 127.0f;  // correctly rounded
  return QMV_OK;
}

// Exact round-to-nearest-even of p / q (p, q > 0 integers, p / q in the
// normal fp32 range) to fp32, in integer arithmetic.
static float rational_to_f32(uint64_t p, uint64_t q) {
  int k = 0;  // p / q = m * 2^k with m in [2^23, 2^24)
  unsigned __int128 num = p, den = q;
  while (num < (den << 23)) { num <<= 1; --k; }
  while (num >= (den << 24)) { den <<= 1; ++k; }
  uint64_t m = (uint64_t)(num / den);
  const unsigned __int128 rem2 = (num - (unsigned __int128)m * den) * 2;
  if (rem2 > den || (rem2 == den && (m & 1))) ++m;  // nearest, ties to even
  return ldexpf((float)m, k);                         // m <= 2^24: exact
}

int qmv_dynamic_code2(float out256[256]) {
  if (!out256) return QMV_ERR_INVALID_ARG;
  // 10^-e (0.1 + 0.9 (j + 1/2) / 2^(6-e)) = (2^(7-e) + 18 j + 9) / (10^(e+1) 2^(7-e))
  std::vector<float> v = {0.0f, 1.0f};
  for (int e = 0; e <= 6; ++e) {
    uint64_t pow10 = 10;
    for (int i = 0; i < e; ++i) pow10 *= 10;
    const uint64_t bins = 1ull << (6 - e);
    for (uint64_t j = 0; j < bins; ++j) {
      const float f = rational_to_f32(2 * bins + 18 * j + 9, pow10 * 2 * bins);
      v.push_back(f);
      v.push_back(-f);
    }
  }
  std::sort(v.begin(), v.end());
  if (v.size() != 256) return QMV_ERR_INVALID_ARG;
  for (int k = 0; k < 256; ++k) out256[k] = v[k];
  return QMV_OK;
}

const char *qmv_status_string(int status) {
  switch (status) {
    case QMV_OK: return "ok";
    case QMV_ERR_INVALID_ARG: return "invalid argument";
    case QMV_ERR_UNSUPPORTED: return "unsupported configuration";
    case QMV_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
    case QMV_ERR_LAUNCH: return "kernel launch failed";
    case QMV_ERR_HIP: return "HIP runtime error";
    case QMV_ERR_WORKSPACE: return "workspace missing or too small";
    case QMV_ERR_TOO_LARGE: return "more than 2^24 scales for the fixed scratch of qmv_double_quant_noalloc";
    default: return "unknown status";
  }
}

}  // extern "C"
