// Row-tile plumbing shared by the row kernels: launch parameters, 16-byte
// streaming loads/stores between HBM and an fp32 LDS tile (bf16 widened
// exactly on load, rounded to nearest even on store), optional sign flip.
#pragma once

#include "common.h"

namespace harp {

struct TileParams {
  int d;             // row length
  int ldsrow;        // LDS row stride in floats (multiple of 64, >= d)
  int m;             // stages in processing order
  int R;             // rows per tile
  int transpose;     // 1: blocks act transposed (inverse)
  int sign_mode;     // 0 none, 1 on load, 2 on store
  int vec_in;        // 16-byte vector loads are legal
  int vec_out;       // 16-byte vector stores are legal
  StageDesc st[kMaxStagesDev];
  const void* blocks;
  const float* scales;
  const int8_t* signs;
  const void* x;
  int64_t ldx;
  void* y;
  int64_t ldy;
  int64_t rows;
  int64_t ntiles;
  float out_scale;   // multiplies every stored value (1 = none)
};

template <typename T> struct IoTraits;
template <> struct IoTraits<float> { static constexpr int V = 4; };
template <> struct IoTraits<uint16_t> { static constexpr int V = 8; };

__device__ __forceinline__ float apply_sign(float v, int8_t s) {
  return __uint_as_float(__float_as_uint(v) ^ (s < 0 ? 0x80000000u : 0u));
}

template <typename TIN>
__device__ __forceinline__ void unpack16(u32x4 w, float* v);
template <>
__device__ __forceinline__ void unpack16<uint16_t>(u32x4 w, float* v) {
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}
template <>
__device__ __forceinline__ void unpack16<float>(u32x4 w, float* v) {
  v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
  v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
}
template <typename TOUT>
__device__ __forceinline__ u32x4 pack16(const float* v);
template <>
__device__ __forceinline__ u32x4 pack16<uint16_t>(const float* v) {
  u32x4 w;
  w.x = pack_bf16x2_hw(v[0], v[1]); w.y = pack_bf16x2_hw(v[2], v[3]);
  w.z = pack_bf16x2_hw(v[4], v[5]); w.w = pack_bf16x2_hw(v[6], v[7]);
  return w;
}
template <>
__device__ __forceinline__ u32x4 pack16<float>(const float* v) {
  u32x4 w;
  w.x = __float_as_uint(v[0]); w.y = __float_as_uint(v[1]);
  w.z = __float_as_uint(v[2]); w.w = __float_as_uint(v[3]);
  return w;
}
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
__device__ __forceinline__ void from_f32(float v, float* o) { *o = v; }
__device__ __forceinline__ void from_f32(float v, uint16_t* o) { *o = (uint16_t)f32_to_bf16_rne(v); }

template <typename TIN>
__device__ void load_tile(const TileParams& p, float* tile, int64_t row0, int nr) {
  const TIN* x = static_cast<const TIN*>(p.x);
  const bool sgn = p.signs != nullptr && p.sign_mode == 1;
  if (p.vec_in) {
    constexpr int V = IoTraits<TIN>::V;
    const int cpr = p.d / V;
    const int total = nr * cpr;
    for (int i = threadIdx.x; i < total; i += blockDim.x) {
      const int r = i / cpr;
      const int c = i - r * cpr;
      float v[V];
      unpack16<TIN>(ld_stream(x + (row0 + r) * p.ldx + (int64_t)c * V), v);
      if (sgn) {
#pragma unroll
        for (int j = 0; j < V; ++j) v[j] = apply_sign(v[j], p.signs[c * V + j]);
      }
      float* dst = tile + r * p.ldsrow + swz(c * V);
#pragma unroll
      for (int j = 0; j < V; ++j) dst[j] = v[j];
    }
  } else {
    const int total = nr * p.d;
    for (int i = threadIdx.x; i < total; i += blockDim.x) {
      const int r = i / p.d;
      const int c = i - r * p.d;
      float v = to_f32(x[(row0 + r) * p.ldx + c]);
      if (sgn) v = apply_sign(v, p.signs[c]);
      tile[r * p.ldsrow + swz(c)] = v;
    }
  }
}

template <typename TOUT>
__device__ void store_tile(const TileParams& p, const float* tile, int64_t row0, int nr) {
  TOUT* y = static_cast<TOUT*>(p.y);
  const bool sgn = p.signs != nullptr && p.sign_mode == 2;
  if (p.vec_out) {
    constexpr int V = IoTraits<TOUT>::V;
    const int cpr = p.d / V;
    const int total = nr * cpr;
    for (int i = threadIdx.x; i < total; i += blockDim.x) {
      const int r = i / cpr;
      const int c = i - r * cpr;
      const float* src = tile + r * p.ldsrow + swz(c * V);
      float v[V];
#pragma unroll
      for (int j = 0; j < V; ++j) v[j] = src[j];
      if (sgn) {
#pragma unroll
        for (int j = 0; j < V; ++j) v[j] = apply_sign(v[j], p.signs[c * V + j]);
      }
      if (p.out_scale != 1.0f) {
#pragma unroll
        for (int j = 0; j < V; ++j) v[j] *= p.out_scale;
      }
      st_stream(y + (row0 + r) * p.ldy + (int64_t)c * V, pack16<TOUT>(v));
    }
  } else {
    const int total = nr * p.d;
    for (int i = threadIdx.x; i < total; i += blockDim.x) {
      const int r = i / p.d;
      const int c = i - r * p.d;
      float v = tile[r * p.ldsrow + swz(c)];
      if (sgn) v = apply_sign(v, p.signs[c]);
      v *= p.out_scale;
      from_f32(v, &y[(row0 + r) * p.ldy + c]);
    }
  }
}

}  // namespace harp
