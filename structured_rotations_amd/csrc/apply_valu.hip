// Vector-ALU row kernel for the HARP transform (radices 2, 4, 5, 8; d <= 5120).
//
// HARP technical summary (gist.science 2605.29843), §2.1/§2.2: stage t
// applies, to every group of coordinates that agree on all digits but digit
// t, its own b_t x b_t orthogonal block.  Over a tile of 8 rows each group is
// a tiny product Y(b x 8) = C(b x b) X(b x 8) with C = B_{t,c} (or its
// transpose for the inverse).  Here one compute thread owns one group per
// round: it holds all b^2 coefficients of the group in registers (loaded one
// round ahead, also across stage and tile boundaries), reads the group's b
// input columns as 16-byte units (one column of one row quad), runs b^2 fp32
// FMAs per row, and writes its b output columns back in place.  Every
// coefficient is fetched once per tile and used for all 8 rows.
//
// The LDS tile layout and the data waves (HBM <-> LDS streaming, sign
// application) are shared with the matrix-core kernel; when the last stage
// is contiguous (digit stride 1, radix 8) the compute threads store their 8
// consecutive outputs per row straight to HBM.
#include <type_traits>

#include "row_io.h"

namespace harp {

namespace {

using namespace rowk;

// CT compute threads, IOW data waves, each data thread prefetching up to MIO
// 16-byte chunks per row quad of the next tile into registers.
template <int CT, int IOW, int MIO>
struct ValuRoles {
  static constexpr int kCompThreads = CT;
  static constexpr int kThreads = CT + 64 * IOW;
  static constexpr int kIoThreads = 64 * IOW;
  static constexpr int kMaxIo = MIO;
};

// Raw coefficient registers of one group (radix <= 8): packed storage words,
// or for radix 5 (whose blocks are not 16-byte aligned) one element per word;
// for int8 blocks the last word holds the group's fp32 scale.
template <typename TB> struct Raw;
template <> struct Raw<float> { static constexpr int N = 64; };
template <> struct Raw<uint16_t> { static constexpr int N = 32; };
template <> struct Raw<int8_t> { static constexpr int N = 26; };

template <int B, typename TB>
__device__ __forceinline__ void load_raw(const RowParams& p, const StageFast& sd, int g, uint32_t (&raw)[Raw<TB>::N]) {
  const TB* blk = static_cast<const TB*>(p.blocks) + sd.blk_off + (int64_t)g * B * B;
  if constexpr (B == 5) {
#pragma unroll
    for (int e = 0; e < 25; ++e) {
      if constexpr (std::is_same<TB, float>::value) raw[e] = __float_as_uint(blk[e]);
      else if constexpr (std::is_same<TB, uint16_t>::value) raw[e] = blk[e];
      else raw[e] = (uint32_t)(int32_t)blk[e];
    }
  } else {
    constexpr int NB = B * B * (int)sizeof(TB);
    if constexpr (NB >= 16) {
#pragma unroll
      for (int i = 0; i < NB / 16; ++i) {
        const u32x4 v = reinterpret_cast<const u32x4*>(blk)[i];
        raw[4 * i] = v.x; raw[4 * i + 1] = v.y; raw[4 * i + 2] = v.z; raw[4 * i + 3] = v.w;
      }
    } else if constexpr (NB == 8) {
      const uint2 v = *reinterpret_cast<const uint2*>(blk);
      raw[0] = v.x; raw[1] = v.y;
    } else {
      raw[0] = *reinterpret_cast<const uint32_t*>(blk);
    }
  }
  if constexpr (std::is_same<TB, int8_t>::value) raw[Raw<TB>::N - 1] = __float_as_uint(p.scales[sd.grp_off + g]);
}

template <typename TB>
__device__ __forceinline__ void load_raw_any(const RowParams& p, const StageFast& sd, int g,
                                             uint32_t (&raw)[Raw<TB>::N]) {
  switch (sd.b) {
    case 2: load_raw<2, TB>(p, sd, g, raw); break;
    case 4: load_raw<4, TB>(p, sd, g, raw); break;
    case 5: load_raw<5, TB>(p, sd, g, raw); break;
    default: load_raw<8, TB>(p, sd, g, raw); break;
  }
}

// Element e (row-major index into the b x b block) of the raw registers.
template <int B, typename TB>
__device__ __forceinline__ float raw_val(const uint32_t (&raw)[Raw<TB>::N], int e) {
  if constexpr (std::is_same<TB, float>::value) {
    return __uint_as_float(raw[e]);
  } else if constexpr (std::is_same<TB, uint16_t>::value) {
    if constexpr (B == 5) return __uint_as_float(raw[e] << 16);
    else return (e & 1) ? bf16_hi(raw[e >> 1]) : bf16_lo(raw[e >> 1]);
  } else {
    const float scale = __uint_as_float(raw[Raw<TB>::N - 1]);
    if constexpr (B == 5) return (float)(int32_t)raw[e] * scale;
    else return (float)(int8_t)(raw[e >> 2] >> (8 * (e & 3))) * scale;
  }
}

// One stage over the tile.  raw holds round 0's coefficients on entry and the
// next stage's (or, after the last stage, the next tile's first) on exit.
// Within a stage every group's columns are read and written only by the
// thread that owns the group.
template <int B, typename T, typename TB, bool TR, bool DIRECT, int CT>
__device__ void valu_stage(const RowParams& p, int t, float* tile, uint32_t (&raw)[Raw<TB>::N], int64_t row0,
                           int nr, int tid) {
  const StageFast sd = p.st[t];
  const int ngroups = sd.G;
  const int s = sd.s;
  const int plane = 4 * p.d;
  for (int base = 0; base < ngroups; base += CT) {
    const int g = base + tid;
    // C[o][k] = B[o][k] (forward) or B[k][o] (inverse)
    float cf[B][B];
#pragma unroll
    for (int o = 0; o < B; ++o)
#pragma unroll
      for (int k = 0; k < B; ++k) cf[o][k] = raw_val<B, TB>(raw, TR ? k * B + o : o * B + k);
    if (base + CT < ngroups) {
      const int gn = base + CT + tid;
      load_raw<B, TB>(p, sd, gn < ngroups ? gn : 0, raw);
    } else {
      const StageFast& sn = p.st[t + 1 < p.m ? t + 1 : 0];
      load_raw_any<TB>(p, sn, tid < sn.G ? tid : 0, raw);
    }
    // group counts are multiples of 64 and CT is a whole number of waves, so
    // this test is uniform per wave: idle waves only prefetch
    if (g >= ngroups) continue;
    const int hi = s == 1 ? g : (int)__umulhi((uint32_t)g, sd.mag_s);
    const int col0 = hi * (B - 1) * s + g;      // = hi * B * s + (g - hi * s)
    int a[B];
#pragma unroll
    for (int k = 0; k < B; ++k) a[k] = 4 * pcol(col0 + k * s);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      f32x4 xv[B];
#pragma unroll
      for (int k = 0; k < B; ++k) xv[k] = *reinterpret_cast<const f32x4*>(tile + a[k] + q * plane);
      if constexpr (!DIRECT) {
#pragma unroll
        for (int o = 0; o < B; ++o) {
          f32x4 acc = cf[o][0] * xv[0];
#pragma unroll
          for (int k = 1; k < B; ++k) acc += cf[o][k] * xv[k];
          *reinterpret_cast<f32x4*>(tile + a[o] + q * plane) = acc;
        }
      } else {
        // digit stride 1, radix 8: outputs o = 0..7 of row 4q+i are columns col0..col0+7
        f32x4 yv[8];
#pragma unroll
        for (int o = 0; o < 8; ++o) {
          f32x4 acc = cf[o][0] * xv[0];
#pragma unroll
          for (int k = 1; k < 8; ++k) acc += cf[o][k] * xv[k];
          yv[o] = acc;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * q + i;
          if (r < nr) {
            float v[8];
#pragma unroll
            for (int o = 0; o < 8; ++o) v[o] = yv[o][i];
            T* y = static_cast<T*>(p.y) + (row0 + r) * p.ldy + col0;
            st_stream(y, pack_row<T>(v));
            if constexpr (std::is_same<T, float>::value) st_stream(y + 4, pack_row<T>(v + 4));
          }
        }
      }
    }
  }
}

template <typename T, typename TB, bool TR, int CT>
__device__ void run_valu_stage(const RowParams& p, int t, float* tile, uint32_t (&raw)[Raw<TB>::N], int64_t row0,
                               int nr, int tid) {
  if (p.direct_out && t == p.m - 1) {
    valu_stage<8, T, TB, TR, true, CT>(p, t, tile, raw, row0, nr, tid);
    return;
  }
  switch (p.st[t].b) {
    case 2: valu_stage<2, T, TB, TR, false, CT>(p, t, tile, raw, row0, nr, tid); break;
    case 4: valu_stage<4, T, TB, TR, false, CT>(p, t, tile, raw, row0, nr, tid); break;
    case 5: valu_stage<5, T, TB, TR, false, CT>(p, t, tile, raw, row0, nr, tid); break;
    case 8: valu_stage<8, T, TB, TR, false, CT>(p, t, tile, raw, row0, nr, tid); break;
    default: break;
  }
}

template <typename T, typename TB, bool TR, typename RL>
__global__ void __launch_bounds__(RL::kThreads) apply_valu_kernel(RowParams p) {
  constexpr int CT = RL::kCompThreads;
  extern __shared__ float tile[];
  int64_t tix = blockIdx.x;
  if (tix >= p.ntiles) return;   // uniform per workgroup
  if (threadIdx.x >= CT) {
    data_waves<T, RL::kIoThreads, RL::kMaxIo>(p, tile, threadIdx.x - CT);
    return;
  }
  const int tid = threadIdx.x;
  uint32_t raw[Raw<TB>::N];
  load_raw_any<TB>(p, p.st[0], tid < p.st[0].G ? tid : 0, raw);
  __syncthreads();
  for (; tix < p.ntiles; tix += gridDim.x) {
    const int64_t row0 = tix * kRows;
    const int nr = tile_rows(p, tix);
    for (int t = 0; t < p.m; ++t) {
      run_valu_stage<T, TB, TR, CT>(p, t, tile, raw, row0, nr, tid);
      __syncthreads();
    }
    if (!p.direct_out) __syncthreads();
    __syncthreads();
  }
}

template <typename T, typename TB, typename RL>
hipError_t launch_valu_roles(const RowParams& p, int grid, size_t lds, hipStream_t st) {
  auto kern = p.transpose ? apply_valu_kernel<T, TB, true, RL> : apply_valu_kernel<T, TB, false, RL>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(RL::kThreads), lds, st, p);
  return hipGetLastError();
}

template <typename T, typename TB>
hipError_t launch_valu_typed(const RowParams& p, int, int grid, size_t lds, hipStream_t st) {
  // 4 compute waves (one per SIMD, 256 VGPRs for the 64 coefficients, their
  // prefetch and the inputs) + 4 data waves
  return launch_valu_roles<T, TB, ValuRoles<256, 4, 2>>(p, grid, lds, st);
}

template <typename T>
hipError_t launch_valu_blk(DT bdt, const RowParams& p, int roles, int grid, size_t lds, hipStream_t st) {
  switch (bdt) {
    case DT::F32: return launch_valu_typed<T, float>(p, roles, grid, lds, st);
    case DT::BF16: return launch_valu_typed<T, uint16_t>(p, roles, grid, lds, st);
    case DT::I8: return launch_valu_typed<T, int8_t>(p, roles, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_apply_valu(const Plan& pl, bool inverse, const void* blocks, DT bdt, const float* scales,
                             const int8_t* signs, const void* x, int64_t ldx, DT io, void* y, int64_t ldy,
                             int64_t rows, int roles, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  RowParams p = make_row_params(pl, inverse, blocks, scales, signs, x, ldx, io, y, ldy, rows);
  const size_t lds = (size_t)kRows * pl.d * sizeof(float);
  int64_t grid = cu_count();
  if (grid > p.ntiles) grid = p.ntiles;
  if (io == DT::BF16) return launch_valu_blk<uint16_t>(bdt, p, roles, (int)grid, lds, stream);
  return launch_valu_blk<float>(bdt, p, roles, (int)grid, lds, stream);
}

}  // namespace harp
