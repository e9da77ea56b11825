// Codec kernels: quantize_4bit, double quantization of the scales, scale
// reconstruction and dequantize_4bit.
//
// Operation set: "Feat/mps gemm 4bit bf16", table "What runs natively now"
// (quantize_4bit / dequantize_4bit); block size and double quantization:
// "mps-bitsandbytes 0.4.7", section "Functional API".  Every result here is
// bit-exact: the nearest-code decision is made against exact thresholds, and
// every float operation is an explicitly rounded one.
#include <algorithm>

#include "qmv_launch.hpp"

#pragma clang fp contract(off)

namespace qmv {

int log2_exact(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}

// ---------------------------------------------------------------------------
// Directed conversions used to turn an exact float64 threshold into an fp32
// one that makes a single fp32 comparison exact.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_step_down_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if (f > 0.f) return u - 1u;
  if (f == 0.f) return 0x80000001u;  // -denorm_min
  return u + 1u;
}

// Largest fp32 <= d.
__device__ __forceinline__ float f64_to_f32_rd(double d) {
  const float f = (float)d;  // round to nearest even
  return ((double)f > d) ? __uint_as_float(f32_step_down_bits(f)) : f;
}

// Smallest fp32 >= d.
__device__ __forceinline__ float f64_to_f32_ru(double d) {
  const float f = (float)d;
  if ((double)f < d) {
    const uint32_t u = __float_as_uint(f);
    if (f > 0.f) return __uint_as_float(u + 1u);
    if (f == 0.f) return __uint_as_float(0x00000001u);
    return __uint_as_float(u - 1u);
  }
  return f;
}

// Rank among the thresholds (0..15 for NF4, 0..14 for FP4) -> code.
template <int QT>
__device__ __forceinline__ uint32_t rank_to_code(int r) {
  if constexpr (QT == kNF4) {
    return (uint32_t)r;  // NF4 codes are ascending ranks
  } else {
    // FP4 ascending values: codes 15..9 (negatives), 0 (zero), 1..7 (positives)
    return (uint32_t)(r < 7 ? 15 - r : (r == 7 ? 0 : r - 7));
  }
}

// ---------------------------------------------------------------------------
// quantize_4bit
//
// A workgroup of 256 threads takes a tile of 256 * E consecutive elements;
// each thread owns E of them (one 16- or 32-byte load), so G = blocksize / E
// neighbouring threads share a block.  The block absmax is reduced across
// those G threads (wave shuffles, then LDS when a block spans waves).  For
// each block the fp32 thresholds are derived from the exact float64 products
// absmax * mid[j]:
//   mid > 0: x moves up past the threshold only when x > absmax * mid
//            (a tie stays with the smaller magnitude), and for fp32 x that is
//            x > RD(absmax * mid);
//   mid < 0: x moves up when x >= absmax * mid, i.e. x > pred(RU(absmax * mid)).
// The code is the number of thresholds x exceeds, mapped to the table's code.
// ---------------------------------------------------------------------------
template <int DT, int QT, int E>
__global__ __launch_bounds__(256) void quantize_4bit_kernel(const void *__restrict__ Wv,
                                                            int64_t numel, int log2bs,
                                                            Midpoints4 mids,
                                                            uint8_t *__restrict__ packed,
                                                            float *__restrict__ absmax) {
  using T = typename Storage<DT>::type;
  const T *W = static_cast<const T *>(Wv);
  __shared__ float wave_max[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int G = (1 << log2bs) / E;  // threads per block: 4 .. 256
  const int64_t tile = 256 * E;
  const int64_t ntiles = (numel + tile - 1) / tile;

  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t e0 = t * tile + (int64_t)tid * E;
    float v[E];
    if (e0 + E <= numel) {
      if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < E; i += 4) {
          const float4 q = *reinterpret_cast<const float4 *>(W + e0 + i);
          v[i] = q.x; v[i + 1] = q.y; v[i + 2] = q.z; v[i + 3] = q.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < E; i += 8) {
          const uint4 q = *reinterpret_cast<const uint4 *>(W + e0 + i);
          const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[i + 2 * j] = bits16_to_f32<DT>(w[j] & 0xffffu);
            v[i + 2 * j + 1] = bits16_to_f32<DT>(w[j] >> 16);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = (e0 + i < numel) ? load_elem<DT>(W, e0 + i) : 0.f;
    }

    float m = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) m = fmaxf(m, fabsf(v[i]));
    const int gw = G < 64 ? G : 64;
    for (int off = 1; off < gw; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (G > 64) {  // uniform across the launch
      if (lane == 0) wave_max[wave] = m;
      __syncthreads();
      const int wpb = G >> 6;
      const int w0 = (wave / wpb) * wpb;
      float mm = wave_max[w0];
      for (int i = 1; i < wpb; ++i) mm = fmaxf(mm, wave_max[w0 + i]);
      m = mm;
      __syncthreads();
    }
    if ((tid & (G - 1)) == 0 && e0 < numel) absmax[e0 >> log2bs] = m;

    // NF4 has 16 distinct values (15 thresholds); FP4's +0 and -0 coincide (14)
    constexpr int NT = QT == kNF4 ? 15 : 14;
    float th[NT];
    const double ad = (double)m;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const double p = ad * mids.mid[j];  // exact
      th[j] = mids.mid[j] > 0.0 ? f64_to_f32_rd(p)
                                : __uint_as_float(f32_step_down_bits(f64_to_f32_ru(p)));
    }

    uint32_t code[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
      int r = 0;
#pragma unroll
      for (int j = 0; j < NT; ++j) r += (v[i] > th[j]) ? 1 : 0;
      code[i] = (e0 + i < numel) ? rank_to_code<QT>(r) : 0u;
    }

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
    if (e0 + E <= numel) {
      if constexpr (E == 8) {
        *reinterpret_cast<uint32_t *>(dst) = word[0];
      } else {
        *reinterpret_cast<uint2 *>(dst) = make_uint2(word[0], word[1]);
      }
    } else {
#pragma unroll
      for (int b = 0; b < E / 2; ++b)
        if (e0 + 2 * b < numel) dst[b] = (uint8_t)(word[b >> 2] >> (8 * (b & 3)));
    }
  }
}

template <int DT, int QT>
static hipError_t launch_quantize_t(const void *W, int64_t numel, int log2bs, const Midpoints4 &m,
                                    uint8_t *packed, float *absmax, hipStream_t st) {
  const int E = log2bs > 11 ? 16 : 8;  // a tile always holds whole blocks
  const int64_t tile = 256 * E;
  const int64_t ntiles = (numel + tile - 1) / tile;
  const unsigned grid = (unsigned)std::min<int64_t>(ntiles, 1 << 20);
  if (E == 8)
    hipLaunchKernelGGL((quantize_4bit_kernel<DT, QT, 8>), dim3(grid), dim3(256), 0, st, W, numel,
                       log2bs, m, packed, absmax);
  else
    hipLaunchKernelGGL((quantize_4bit_kernel<DT, QT, 16>), dim3(grid), dim3(256), 0, st, W, numel,
                       log2bs, m, packed, absmax);
  return hipGetLastError();
}

hipError_t launch_quantize_4bit(const void *W, int w_dtype, int64_t numel, int log2bs, int qt,
                                const Midpoints4 &m, uint8_t *packed, float *absmax,
                                hipStream_t st) {
#define QMV_Q(DT, QT) return launch_quantize_t<DT, QT>(W, numel, log2bs, m, packed, absmax, st)
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
//    fp32(S / nblocks).  The order is part of the contract, so every run is a
//    plain sequential loop in one thread.
// 2. Per group of blocksize2 scales: c = fp32(a - offset), s = max |c|, and
//    the code of c / s is the rank of c among the exact float64 thresholds
//    s * mid[j] of the (strictly increasing) 256-entry table, found by binary
//    search; ties go toward zero as in quantize_4bit.
// ---------------------------------------------------------------------------
constexpr int kFanIn = 256;

template <typename In>
__global__ __launch_bounds__(256) void dq_sum_kernel(const In *__restrict__ in, int64_t n,
                                                     double *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nout = (n + kFanIn - 1) / kFanIn;
  if (i >= nout) return;
  const int64_t s0 = i * kFanIn;
  const int64_t s1 = s0 + kFanIn < n ? s0 + kFanIn : n;
  double s = 0.0;
  for (int64_t k = s0; k < s1; ++k) s = __dadd_rn(s, (double)in[k]);
  out[i] = s;
}

__global__ void dq_offset_kernel(const double *__restrict__ S, int64_t n, float *__restrict__ offset) {
  if (threadIdx.x == 0 && blockIdx.x == 0) offset[0] = (float)__ddiv_rn(S[0], (double)n);
}

template <int E>  // scales per thread: blocksize2 / min(blocksize2, 256)
__global__ __launch_bounds__(256) void dq_encode_kernel(const float *__restrict__ absmax,
                                                        int64_t n, int log2bs2, Code2Table code2,
                                                        const float *__restrict__ offset,
                                                        uint8_t *__restrict__ q,
                                                        float *__restrict__ absmax2,
                                                        float *__restrict__ code2_out) {
  __shared__ double mid[255];
  __shared__ float wave_max[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (tid < 255) mid[tid] = ((double)code2.v[tid] + (double)code2.v[tid + 1]) * 0.5;  // exact
  if (blockIdx.x == 0) code2_out[tid] = code2.v[tid];
  __syncthreads();

  const int bs2 = 1 << log2bs2;
  const int G = bs2 / E;  // threads per group: 32 .. 256
  const int64_t tile = (int64_t)256 * E;
  const int64_t ntiles = (n + tile - 1) / tile;
  const float off = offset[0];

  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    // thread tid owns scales i0, i0 + G, ... of its group (strided, coalesced)
    const int g_in_tile = tid / G;
    const int j = tid % G;
    const int64_t gbase = t * tile + (int64_t)g_in_tile * bs2;
    float c[E];
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t i = gbase + j + (int64_t)e * G;
      c[e] = (i < n) ? __fsub_rn(absmax[i], off) : 0.f;
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
    if (j == 0 && gbase < n) absmax2[gbase >> log2bs2] = m;
    const double sd = (double)m;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t i = gbase + j + (int64_t)e * G;
      if (i >= n) continue;
      const double x = (double)c[e];
      int lo = 0, hi = 255;
      while (lo < hi) {
        const int md = (lo + hi) >> 1;
        const double mj = mid[md];
        const double thr = sd * mj;  // exact
        const bool up = mj > 0.0 ? (x > thr) : (x >= thr);
        if (up) lo = md + 1; else hi = md;
      }
      q[i] = (uint8_t)lo;
    }
  }
}

size_t double_quant_workspace_bytes(int64_t nblocks) {
  size_t total = 0;
  int64_t n = nblocks;
  do {
    n = (n + kFanIn - 1) / kFanIn;
    total += (size_t)n * sizeof(double);
  } while (n > 1);
  return total;
}

hipError_t launch_double_quant(const float *absmax, int64_t nblocks, int log2bs2,
                               const Code2Table &code2, uint8_t *q, float *absmax2, float *offset,
                               float *code2_out, double *ws, hipStream_t st) {
  // summation tree
  int64_t n = nblocks;
  double *level = ws;
  int64_t nout = (n + kFanIn - 1) / kFanIn;
  hipLaunchKernelGGL(dq_sum_kernel<float>, dim3((unsigned)((nout + 255) / 256)), dim3(256), 0, st,
                     absmax, n, level);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  while (nout > 1) {
    double *next = level + nout;
    const int64_t n2 = (nout + kFanIn - 1) / kFanIn;
    hipLaunchKernelGGL(dq_sum_kernel<double>, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, st,
                       level, nout, next);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    level = next;
    nout = n2;
  }
  hipLaunchKernelGGL(dq_offset_kernel, dim3(1), dim3(64), 0, st, level, nblocks, offset);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int bs2 = 1 << log2bs2;
  const int64_t tile = bs2 > 256 ? bs2 : 256;
  const int64_t ntiles = (nblocks + tile - 1) / tile;
  const unsigned grid = (unsigned)std::min<int64_t>(ntiles, 1 << 16);
#define QMV_E(EV)                                                                          \
  hipLaunchKernelGGL(dq_encode_kernel<EV>, dim3(grid), dim3(256), 0, st, absmax, nblocks, log2bs2, \
                     code2, offset, q, absmax2, code2_out)
  switch (bs2 <= 256 ? 1 : bs2 / 256) {
    case 1: QMV_E(1); break;
    case 2: QMV_E(2); break;
    case 4: QMV_E(4); break;
    case 8: QMV_E(8); break;
    default: QMV_E(16); break;
  }
#undef QMV_E
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scale reconstruction ("Functional API": dequant_absmax).
// ---------------------------------------------------------------------------
template <bool DQ>
__global__ __launch_bounds__(256) void dequantize_absmax_kernel(Scales sc, int64_t n,
                                                                float *__restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out[i] = block_scale<DQ>(sc, i);
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
// One thread per 16 packed bytes (32 elements, always inside one block since
// blocksize >= 32 and chunks are 32-aligned): one 16-byte load, the block
// scale, 32 explicitly rounded fp32 products from a 16-entry table in LDS,
// then RNE to the output type and 16-byte stores.  A ragged tail is handled
// element by element by the thread that owns the last chunk.
// ---------------------------------------------------------------------------
template <int QT, int ODT, bool DQ>
__global__ __launch_bounds__(256) void dequantize_4bit_kernel(const uint8_t *__restrict__ packed,
                                                              Scales sc, int64_t numel,
                                                              int log2bs, void *__restrict__ outv) {
  using OT = typename Storage<ODT>::type;
  OT *out = static_cast<OT *>(outv);
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = __uint_as_float(table_bits(QT)[threadIdx.x]);
  __syncthreads();
  const int64_t nfull = numel >> 5;
  const int64_t nchunks = (numel + 31) >> 5;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nchunks;
       c += (int64_t)gridDim.x * 256) {
    const float a = block_scale<DQ>(sc, (c << 5) >> log2bs);
    if (c < nfull) {
      const uint4 p = *reinterpret_cast<const uint4 *>(packed + (c << 4));
      const uint32_t pw[4] = {p.x, p.y, p.z, p.w};
      if constexpr (ODT == kF32) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float o[8];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const uint32_t byte = (pw[w] >> (8 * b)) & 0xffu;
            o[2 * b] = lut[byte >> 4] * a;
            o[2 * b + 1] = lut[byte & 15u] * a;
          }
          float4 *dst = reinterpret_cast<float4 *>(out + (c << 5) + 8 * w);
          dst[0] = make_float4(o[0], o[1], o[2], o[3]);
          dst[1] = make_float4(o[4], o[5], o[6], o[7]);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t o[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const uint32_t byte = (pw[w] >> (8 * b)) & 0xffu;
            const uint32_t h0 = f32_to_bits16<ODT>(lut[byte >> 4] * a);
            const uint32_t h1 = f32_to_bits16<ODT>(lut[byte & 15u] * a);
            o[b] = h0 | (h1 << 16);
          }
          *reinterpret_cast<uint4 *>(out + (c << 5) + 8 * w) = make_uint4(o[0], o[1], o[2], o[3]);
        }
      }
    } else {
      for (int64_t e = c << 5; e < numel; ++e) {
        const uint32_t byte = packed[e >> 1];
        const uint32_t code = (e & 1) ? (byte & 15u) : (byte >> 4);
        store_elem<ODT>(out, e, lut[code] * a);
      }
    }
  }
}

template <int QT, int ODT>
static hipError_t launch_dequant_t(const uint8_t *packed, const Scales &sc, bool dq, int64_t numel,
                                   int log2bs, void *out, hipStream_t st) {
  const int64_t nchunks = (numel + 31) >> 5;
  const unsigned grid = (unsigned)std::min<int64_t>((nchunks + 255) / 256, 1 << 16);
  if (dq)
    hipLaunchKernelGGL((dequantize_4bit_kernel<QT, ODT, true>), dim3(grid), dim3(256), 0, st,
                       packed, sc, numel, log2bs, out);
  else
    hipLaunchKernelGGL((dequantize_4bit_kernel<QT, ODT, false>), dim3(grid), dim3(256), 0, st,
                       packed, sc, numel, log2bs, out);
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
