// embedding_4bit: rows of a 4-bit quantized embedding table
// ("mps-bitsandbytes 0.4.7", sections "Features" and "Quantized Embeddings":
// Embedding4bit / EmbeddingNF4 / EmbeddingFP4).
//
// The table W [V, D] is quantized as one flat tensor by quantize_4bit
// (blocks of `blocksize` consecutive elements, two codes per byte, plain or
// double-quantized scales).  out[t, :] = the dequantized row idx[t], exactly
// as dequantize_4bit returns those elements: fp32(T[code] * a_hat) rounded to
// the output type.  An index outside [0, V) yields a row of zeros.
//
// A workgroup of 256 threads writes a 2048-element segment of output rows
// (grid: row segments x groups of rows).  When D is a multiple of 8, thread t
// of the segment decodes 8 elements from one 4-byte load (one block: blocks
// are at least 32 and aligned) and writes them with one 16-byte (or two,
// fp32) store, for 4 rows at a time whose loads are all issued first;
// otherwise each thread decodes single elements of one row at a time.
#include <algorithm>

#include "qmv_launch.hpp"

#pragma clang fp contract(off)

namespace qmv {

// A 16-byte store marked non-temporal (streamed out: the output is not read
// back by the kernel, and the hint measured faster for large outputs).
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_nt(void *p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  __builtin_nontemporal_store(u32x4_nt{a, b, c, d}, static_cast<u32x4_nt *>(p));
}

constexpr int kEmbSeg = 2048;  // elements of a row per workgroup
constexpr int kEmbTok = 4;     // tokens per pass of a workgroup (D a multiple of 8)

template <int QT, int ODT, bool DQ, bool VEC>
__global__ __launch_bounds__(256) void embedding_4bit_kernel(const int64_t *__restrict__ idx,
                                                             int64_t T, int64_t V, int64_t D,
                                                             const uint8_t *__restrict__ packed,
                                                             Scales sc, int log2bs,
                                                             void *__restrict__ outv) {
  using OT = typename Storage<ODT>::type;
  OT *out = static_cast<OT *>(outv);
  __shared__ float2 lut2[256];  // packed byte -> (T[byte >> 4], T[byte & 15])
  const int tid = threadIdx.x;
  {
    const uint32_t *tb = table_bits(QT);
    lut2[tid] = make_float2(__uint_as_float(tb[tid >> 4]), __uint_as_float(tb[tid & 15]));
  }
  __syncthreads();
  const int64_t d0 = (int64_t)blockIdx.x * kEmbSeg;
  const float offset = DQ ? sc.offset[0] : 0.f;

  if constexpr (VEC) {
    // kEmbTok tokens per pass: their indices, then all their codes and
    // scales are requested before any is used, so the dependent loads
    // (index -> code and scale code -> table entry) of the tokens overlap
    const int64_t d = d0 + 8 * (int64_t)tid;
    for (int64_t t0 = (int64_t)blockIdx.y * kEmbTok; t0 < T; t0 += (int64_t)gridDim.y * kEmbTok) {
      int64_t row[kEmbTok];
      bool valid[kEmbTok];
#pragma unroll
      for (int k = 0; k < kEmbTok; ++k) {
        row[k] = t0 + k < T ? idx[t0 + k] : -1;     // the same for the whole workgroup
        valid[k] = row[k] >= 0 && row[k] < V && d < D;
      }
      uint32_t w[kEmbTok];
      float a[kEmbTok];
#pragma unroll
      for (int k = 0; k < kEmbTok; ++k) {
        w[k] = 0u;
        a[k] = 0.f;
        if (valid[k]) {
          const int64_t e = row[k] * D + d;        // a multiple of 8: one block, 4 aligned bytes
          w[k] = *reinterpret_cast<const uint32_t *>(packed + (e >> 1));
          a[k] = block_scale<DQ>(sc, e >> log2bs, offset);
        }
      }
#pragma unroll
      for (int k = 0; k < kEmbTok; ++k) {
        if (t0 + k >= T || d >= D) continue;
        float v[8];
        if (valid[k]) {
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const float2 tv = lut2[(w[k] >> (8 * b)) & 0xffu];
            v[2 * b] = tv.x * a[k];
            v[2 * b + 1] = tv.y * a[k];
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = 0.f;
        }
        OT *dst = out + (t0 + k) * D;
        if constexpr (ODT == kF32) {
          store16_nt(dst + d, __float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                     __float_as_uint(v[3]));
          store16_nt(dst + d + 4, __float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                     __float_as_uint(v[7]));
        } else {
          store16_nt(dst + d, cvt_pair<ODT>(v[0], v[1]), cvt_pair<ODT>(v[2], v[3]),
                     cvt_pair<ODT>(v[4], v[5]), cvt_pair<ODT>(v[6], v[7]));
        }
      }
    }
    return;
  }
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
    const int64_t row = idx[t];                       // the same for the whole workgroup
    const bool valid = row >= 0 && row < V;
    OT *dst = out + t * D;
    {
      const int64_t d_end = std::min<int64_t>(D, d0 + kEmbSeg);
      for (int64_t d = d0 + tid; d < d_end; d += 256) {
        float v = 0.f;
        if (valid) {
          const int64_t e = row * D + d;
          const uint32_t byte = packed[e >> 1];
          const uint32_t code = (e & 1) ? (byte & 15u) : (byte >> 4);  // even element: high nibble
          v = lut2[code * 17u].x * block_scale<DQ>(sc, e >> log2bs, offset);      // entry 17 c = (T[c], T[c])
        }
        store_elem<ODT>(dst, d, materialize(v));
      }
    }
  }
}

template <int QT, int ODT, bool DQ>
static void launch_emb_t(bool vec, dim3 grid, const int64_t *idx, int64_t T, int64_t V, int64_t D,
                         const uint8_t *packed, const Scales &sc, int log2bs, void *out,
                         hipStream_t st) {
  if (vec)
    hipLaunchKernelGGL((embedding_4bit_kernel<QT, ODT, DQ, true>), grid, dim3(256), 0, st, idx, T, V,
                       D, packed, sc, log2bs, out);
  else
    hipLaunchKernelGGL((embedding_4bit_kernel<QT, ODT, DQ, false>), grid, dim3(256), 0, st, idx, T,
                       V, D, packed, sc, log2bs, out);
}

hipError_t launch_embedding_4bit(const int64_t *idx, int64_t T, int64_t V, int64_t D,
                                 const uint8_t *packed, const Scales &sc, bool dq, int log2bs,
                                 int qt, void *out, int out_dtype, hipStream_t st) {
  const bool vec = D % 8 == 0;
  const int64_t passes = vec ? (T + kEmbTok - 1) / kEmbTok : T;
  const dim3 grid((unsigned)((D + kEmbSeg - 1) / kEmbSeg), (unsigned)std::min<int64_t>(passes, 65535));
#define QMV_E(QTV, ODTV)                                                                     \
  if (dq) launch_emb_t<QTV, ODTV, true>(vec, grid, idx, T, V, D, packed, sc, log2bs, out, st); \
  else launch_emb_t<QTV, ODTV, false>(vec, grid, idx, T, V, D, packed, sc, log2bs, out, st)
#define QMV_EO(QTV)                                  \
  if (out_dtype == kF32) { QMV_E(QTV, kF32); }       \
  else if (out_dtype == kF16) { QMV_E(QTV, kF16); }  \
  else { QMV_E(QTV, kBF16); }
  if (qt == kNF4) { QMV_EO(kNF4); } else { QMV_EO(kFP4); }
#undef QMV_EO
#undef QMV_E
  return hipGetLastError();
}

}  // namespace qmv
