// Device helpers shared by the gfx950 kernels: bfloat16 conversion, streaming
// (non-temporal) 16-byte loads and stores, the LDS bank swizzle, and the
// per-stage descriptors the host passes by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace harp {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Per-stage descriptor in processing order (already reversed for inverses).
struct StageDesc {
  int b;          // radix
  int s;          // digit stride
  int blk_off;    // first coefficient of the stage in the block array
  int grp_off;    // first group of the stage (int8 scale index)
};

constexpr int kMaxStagesDev = 16;

// bfloat16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bfloat16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}
// Same rounding (nearest, ties to even) through gfx950's packed conversion
// instruction, one VALU op for two values.
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
  const bf16x2_t h = __builtin_convertvector(f32x2{lo, hi}, bf16x2_t);
  uint32_t w;
  __builtin_memcpy(&w, &h, 4);
  return w;
}

// fp64 -> bfloat16 bits, round to nearest, ties to even, directly from the
// binary64 pattern (normal range; zero and binary32-subnormal range -> 0).
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  uint32_t sign = (uint32_t)(u >> 63);
  int e = (int)((u >> 52) & 0x7ff);
  uint64_t mant = u & ((1ull << 52) - 1);
  int be = e - 1023 + 127;
  if (e == 0 || be <= 0) return (uint16_t)(sign << 15);
  uint64_t keep = mant >> 45;
  uint64_t rest = mant & ((1ull << 45) - 1);
  const uint64_t half = 1ull << 44;
  if (rest > half || (rest == half && (keep & 1))) ++keep;
  if (keep == 128) { keep = 0; ++be; }
  return (uint16_t)((sign << 15) | ((uint32_t)be << 7) | (uint32_t)keep);
}

__device__ __forceinline__ u32x4 ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// LDS row swizzle: XOR bits 3..5 of a column index with bits 6..8.  It is a
// bijection inside every 64-column block, keeps 8-column chunks contiguous,
// and spreads digit-strided accesses with strides 8, 64 and 512 over all
// banks.  Rows in LDS are padded to a multiple of 64 columns.
__device__ __forceinline__ int swz(int col) { return col ^ (((col >> 6) & 7) << 3); }

// Coefficient read with on-the-fly dequantisation.
template <typename TB>
__device__ __forceinline__ float coef(const TB* blk, int64_t i, float scale);
template <>
__device__ __forceinline__ float coef<float>(const float* blk, int64_t i, float) { return blk[i]; }
template <>
__device__ __forceinline__ float coef<uint16_t>(const uint16_t* blk, int64_t i, float) { return bf16_to_f32(blk[i]); }
template <>
__device__ __forceinline__ float coef<int8_t>(const int8_t* blk, int64_t i, float scale) {
  return (float)blk[i] * scale;
}

}  // namespace harp
