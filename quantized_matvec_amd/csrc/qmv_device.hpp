// Device-side building blocks shared by the codec, gemv and gemm kernels.
//
// Code tables, scale decoding and number-format conversions for gfx950.  All
// arithmetic that the codec's bit-exact contract depends on is compiled with
// floating-point contraction off, so no multiply-add fusion can change a
// result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {

enum : int { kNF4 = 0, kFP4 = 1 };
enum : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// NF4 values in fp32, by code (ascending).  The 16 numbers are the QLoRA
// normal-quantile construction: 8 positive and 7 negative quantiles of N(0,1)
// at evenly spaced probabilities between 1/2 and 0.9677083, plus 0, divided by
// the largest and rounded once to fp32.
constexpr uint32_t kNF4Bits[16] = {
    0xbf800000u, 0xbf3239b3u, 0xbf066b30u, 0xbeca32a0u, 0xbe91a24cu, 0xbe3d353fu,
    0xbdba786bu, 0x00000000u, 0x3da2fb03u, 0x3e24cae1u, 0x3e7c04dcu, 0x3ead0338u,
    0x3ee1a4b7u, 0x3f1007aau, 0x3f3913b1u, 0x3f800000u};

// FP4 values in fp32, by code: E2M1 (bits s e1 e0 m) divided by 6, so the
// magnitudes are 0, 1/12, 1/6, 1/4, 1/3, 1/2, 2/3, 1; code 8 is -0.
constexpr uint32_t kFP4Bits[16] = {
    0x00000000u, 0x3daaaaabu, 0x3e2aaaabu, 0x3e800000u, 0x3eaaaaabu, 0x3f000000u,
    0x3f2aaaabu, 0x3f800000u, 0x80000000u, 0xbdaaaaabu, 0xbe2aaaabu, 0xbe800000u,
    0xbeaaaaabu, 0xbf000000u, 0xbf2aaaabu, 0xbf800000u};

__host__ __device__ inline const uint32_t *table_bits(int qt) {
  return qt == kNF4 ? kNF4Bits : kFP4Bits;
}

// Kernel-argument form of the per-block scales (plain or double-quantized).
struct Scales {
  const float *absmax;    // plain fp32 scales
  const uint8_t *q;       // DQ: 8-bit codes
  const float *absmax2;   // DQ: group scales
  const float *code2;     // DQ: 256-entry table
  const float *offset;    // DQ: subtracted mean
  int log2bs2;            // DQ: log2(group size)
};

// Scale of block b.  With double quantization:
// fp32(fp32(code2[q[b]] * absmax2[b / bs2]) + offset), two roundings; the
// caller reads the offset (s.offset[0]) once, outside its loops.
template <bool DQ>
__device__ __forceinline__ float block_scale(const Scales &s, int64_t b, float offset) {
  if constexpr (!DQ) {
    return s.absmax[b];
  } else {
#pragma clang fp contract(off)
    const float c = s.code2[s.q[b]];
    const float g = s.absmax2[b >> s.log2bs2];
    const float p = c * g;   // rounded to fp32 on its own: never fused with the add
    return p + offset;
  }
}


// A raw buffer resource over [base, base + bytes): loads past the end return
// zero and move no data, so range checks need no branch (a branch around a
// load makes the compiler wait for it right there).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Pins an fp32 value in a register so the backend cannot merge the
// instruction that produced it with the one that consumes it (for instance a
// multiply followed by an fp16 conversion becoming one mixed-precision FMA
// with a single rounding, which also turns -0 into +0).
__device__ __forceinline__ float materialize(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 on an fp32 input).
__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)materialize(f));
}

template <int DT>
__device__ __forceinline__ uint32_t f32_to_bits16(float f) {
  if constexpr (DT == kBF16) return f32_to_bf16_rne(f);
  else return f32_to_f16_rne(f);
}

template <int DT>
__device__ __forceinline__ float bits16_to_f32(uint32_t h) {
  if constexpr (DT == kBF16) return bf16_bits_to_f32(h);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Element storage type per dtype tag.
template <int DT> struct Storage;
template <> struct Storage<kF32> { using type = float; };
template <> struct Storage<kF16> { using type = uint16_t; };
template <> struct Storage<kBF16> { using type = uint16_t; };

template <int DT>
__device__ __forceinline__ float load_elem(const typename Storage<DT>::type *p, int64_t i) {
  if constexpr (DT == kF32) return p[i];
  else return bits16_to_f32<DT>(p[i]);
}

template <int DT>
__device__ __forceinline__ void store_elem(typename Storage<DT>::type *p, int64_t i, float v) {
  if constexpr (DT == kF32) p[i] = v;
  else p[i] = (uint16_t)f32_to_bits16<DT>(v);
}

// Lane moves and lane-group reductions.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}

// Max over aligned groups of G lanes (G a power of two, uniform) of a
// non-negative float, compared as unsigned bits (same order, and no NaN
// canonicalisation around each step): DPP moves inside rows of 16 lanes,
// lane shuffles beyond.
__device__ __forceinline__ float group_max(float m, int G) {
  uint32_t u = __float_as_uint(m);
  if (G >= 2) u = max(u, dpp_u32<0xb1>(u));   // quad_perm [1,0,3,2]
  if (G >= 4) u = max(u, dpp_u32<0x4e>(u));   // quad_perm [2,3,0,1]
  if (G >= 8) u = max(u, dpp_u32<0x141>(u));  // row_half_mirror
  if (G >= 16) u = max(u, dpp_u32<0x140>(u)); // row_mirror
  if (G >= 32) u = max(u, (uint32_t)__shfl_xor((int)u, 16));
  if (G >= 64) u = max(u, (uint32_t)__shfl_xor((int)u, 32));
  return __uint_as_float(u);
}

// Whole-wave reductions with DPP: row moves inside rows of 16 lanes, then
// row broadcasts (lane 15 into row 1 and 3, lane 31 into rows 2 and 3), so
// lane 63 ends with the total, which is read back as a uniform value.  Lanes
// a move does not write keep `fill` (the operation's identity).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_fill(int x, int fill) {
  return __builtin_amdgcn_update_dpp(fill, x, CTRL, ROW_MASK, 0xf, false);
}

__device__ __forceinline__ int wave_max_i32(int v) {
  constexpr int lo = -2147483647 - 1;
  v = max(v, dpp_fill<0xb1, 0xf>(v, lo));   // quad_perm [1,0,3,2]
  v = max(v, dpp_fill<0x4e, 0xf>(v, lo));   // quad_perm [2,3,0,1]
  v = max(v, dpp_fill<0x141, 0xf>(v, lo));  // row_half_mirror
  v = max(v, dpp_fill<0x140, 0xf>(v, lo));  // row_mirror
  v = max(v, dpp_fill<0x142, 0xa>(v, lo));  // row_bcast:15
  v = max(v, dpp_fill<0x143, 0xc>(v, lo));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ int wave_min_i32(int v) { return -wave_max_i32(-v); }

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double x) {  // lanes not written read +0
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)dpp_fill<CTRL, ROW_MASK>((int)(uint32_t)u, 0);
  const uint32_t hi = (uint32_t)dpp_fill<CTRL, ROW_MASK>((int)(uint32_t)(u >> 32), 0);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum of a double over the wave.  The additions happen in a fixed tree, so
// it is the exact sum only when every partial sum is exact (the callers
// check that first).
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xb1, 0xf>(v);
  v += dpp_f64<0x4e, 0xf>(v);
  v += dpp_f64<0x141, 0xf>(v);
  v += dpp_f64<0x140, 0xf>(v);
  v += dpp_f64<0x142, 0xa>(v);
  v += dpp_f64<0x143, 0xc>(v);
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2v_t;

template <int ODT>
__device__ __forceinline__ uint32_t cvt_pair(float lo, float hi) {
  if constexpr (ODT == kBF16) {
    const f32x2_t v = {materialize(lo), materialize(hi)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));
  } else {
    return f32_to_f16_rne(lo) | (f32_to_f16_rne(hi) << 16);
  }
}

}  // namespace qmv
