// Matrix-core row kernel for the HARP transform (radices 2, 4, 5, 8; d <= 5120).
//
// HARP technical summary (gist.science 2605.29843), §2.1/§2.2: stage t
// applies, to every group of coordinates that agree on all digits but digit
// t, its own b_t x b_t orthogonal block.  Across a tile of 8 rows that is a
// batch of tiny dense products, one per group, all with different blocks.
// gfx950's v_mfma_f32_4x4x1f32 runs 16 independent 4x4 fp32 outer products
// per instruction, so it carries these products with no padding and no
// precision loss: a block of 4 lanes owns one group, lane i supplies row i's
// input x[i][k] and the coefficient C[4h+i][k] (C = B, or B^T for the
// inverse); after b instructions (k = 0..b-1) lane j holds output 4h+j of the
// group for the 4 rows of a row quad.  Each lane keeps 2b coefficients of its
// group in registers, loaded one round ahead, also across stage and tile
// boundaries.
//
// Layout.  No permutation is ever materialised: the 8-row tile sits in LDS
// as two row-quad planes of 16-byte units (one column's 4 rows), columns
// XOR-swizzled so that the 4-byte input gathers of every digit stride spread
// over all banks; each stage reads its groups' columns at digit stride s_t and
// writes the results back in place.
//
// Roles.  Waves 0..7 compute.  Waves 8..15 move data: while the compute waves
// run the stages of tile n they stream tile n+1 (and its sign bytes) from
// HBM into registers -- their outstanding loads never stall the compute
// waves, whose wait counters only see coefficient loads -- and between tiles
// they write it into LDS.  When the last stage is contiguous (digit stride 1,
// radix 8) the compute waves store its result straight to HBM, with the MFMA
// operands swapped for that stage so each lane ends with 8 consecutive
// outputs of one row; otherwise the data waves copy the finished tile out.
#include <type_traits>

#include "row_io.h"

namespace harp {

namespace {

using namespace rowk;


// Wave roles: CW compute waves, IOW data waves, each data thread prefetching
// up to MIO 16-byte chunks per row quad of the next tile into registers.
template <int CW, int IOW, int MIO>
struct Roles {
  static constexpr int kCompWaves = CW;
  static constexpr int kThreads = 64 * (CW + IOW);
  static constexpr int kIoThreads = 64 * IOW;
  static constexpr int kMaxIo = MIO;
  static constexpr int kGroupsPerRound = 16 * CW;
};

// ---------------------------------------------------------------- coefficients
// cf[h][k] = C[4h + j][k] of group g (C = B forward, B^T inverse); zero
// outside the radix or for an idle lane.
template <int B, typename TB, bool TR>
__device__ __forceinline__ void load_coef(const RowParams& p, const StageFast& sd, int g, int j, bool valid,
                                          float (&cf)[2][8]) {
  const TB* blk = static_cast<const TB*>(p.blocks) + sd.blk_off + (int64_t)g * B * B;
  float scale = 1.0f;
  if constexpr (std::is_same<TB, int8_t>::value) scale = valid ? p.scales[sd.grp_off + g] : 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) cf[h][k] = 0.0f;
  if (!valid) return;
  constexpr bool kVec = (B == 8 || B == 4);
  if constexpr (kVec && !TR) {
#pragma unroll
    for (int h = 0; h < (B == 8 ? 2 : 1); ++h) {
      const TB* row = blk + (4 * h + j) * B;
      if constexpr (std::is_same<TB, float>::value) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(row);
        cf[h][0] = __uint_as_float(a.x); cf[h][1] = __uint_as_float(a.y);
        cf[h][2] = __uint_as_float(a.z); cf[h][3] = __uint_as_float(a.w);
        if constexpr (B == 8) {
          const u32x4 b = *reinterpret_cast<const u32x4*>(row + 4);
          cf[h][4] = __uint_as_float(b.x); cf[h][5] = __uint_as_float(b.y);
          cf[h][6] = __uint_as_float(b.z); cf[h][7] = __uint_as_float(b.w);
        }
      } else if constexpr (std::is_same<TB, uint16_t>::value) {
        if constexpr (B == 8) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(row);
          cf[h][0] = bf16_lo(a.x); cf[h][1] = bf16_hi(a.x); cf[h][2] = bf16_lo(a.y); cf[h][3] = bf16_hi(a.y);
          cf[h][4] = bf16_lo(a.z); cf[h][5] = bf16_hi(a.z); cf[h][6] = bf16_lo(a.w); cf[h][7] = bf16_hi(a.w);
        } else {
          const uint2 a = *reinterpret_cast<const uint2*>(row);
          cf[h][0] = bf16_lo(a.x); cf[h][1] = bf16_hi(a.x); cf[h][2] = bf16_lo(a.y); cf[h][3] = bf16_hi(a.y);
        }
      } else {
        uint32_t wd[2];
        if constexpr (B == 8) {
          const uint2 a = *reinterpret_cast<const uint2*>(row);
          wd[0] = a.x; wd[1] = a.y;
        } else {
          wd[0] = *reinterpret_cast<const uint32_t*>(row);
          wd[1] = 0;
        }
#pragma unroll
        for (int k = 0; k < B; ++k) cf[h][k] = (float)(int8_t)(wd[k >> 2] >> (8 * (k & 3))) * scale;
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int o = 4 * h + j;
#pragma unroll
      for (int k = 0; k < B; ++k)
        if (o < B) cf[h][k] = coef<TB>(blk, TR ? k * B + o : o * B + k, scale);
    }
  }
}

template <typename TB, bool TR>
__device__ __forceinline__ void load_coef_any(const RowParams& p, const StageFast& sd, int g, int j, bool valid,
                                              float (&cf)[2][8]) {
  switch (sd.b) {
    case 2: load_coef<2, TB, TR>(p, sd, g, j, valid, cf); break;
    case 4: load_coef<4, TB, TR>(p, sd, g, j, valid, cf); break;
    case 5: load_coef<5, TB, TR>(p, sd, g, j, valid, cf); break;
    default: load_coef<8, TB, TR>(p, sd, g, j, valid, cf); break;
  }
}

// ---------------------------------------------------------------- compute waves
// One stage over the tile.  cf holds round 0's coefficients on entry and the
// next stage's (or, after the last stage, the next tile's first) on exit.
template <int B, typename T, typename TB, bool TR, bool DIRECT, int GPR>
__device__ void mfma_stage(const RowParams& p, int t, float* tile, float (&cf)[2][8], int64_t row0, int nr) {
  constexpr int NH = B > 4 ? 2 : 1;
  const StageFast& sd = p.st[t];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int bk = lane >> 2;
  const int j = lane & 3;
  const int ngroups = sd.G;
  const int s = sd.s;
  const int plane = 4 * p.d;                  // floats between the two row quads
  float nx[2][8];
  for (int base_g = 0; base_g < ngroups; base_g += GPR) {
    const int g = base_g + wave * 16 + bk;
    const bool valid = g < ngroups;
    // prefetch the next round (or the next stage's / next tile's first round)
    {
      const int nb = base_g + GPR;
      if (nb < ngroups) {
        const int gn = nb + wave * 16 + bk;
        load_coef<B, TB, TR>(p, sd, gn < ngroups ? gn : 0, j, gn < ngroups, nx);
      } else {
        const StageFast& sn = p.st[t + 1 < p.m ? t + 1 : 0];
        const int gn = wave * 16 + bk;
        load_coef_any<TB, TR>(p, sn, gn < sn.G ? gn : 0, j, gn < sn.G, nx);
      }
    }
    const int gg = valid ? g : 0;
    const int hi = fdiv(gg, sd.div_s);
    const int col0 = hi * (B - 1) * s + gg;     // = hi * B * s + (gg - hi * s)
    const float* src = tile + j;
    float xv[2][B];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int a = 4 * pcol(col0 + k * s);
      xv[0][k] = src[a];
      xv[1][k] = src[a + plane];
    }
    f32x4 acc[2][2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int h = 0; h < NH; ++h) acc[q][h] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (!DIRECT) {
      // D[i][j] = sum_k x[row i][k] C[4h+j][k]: lane j gets output 4h+j of the
      // quad's rows; four accumulation chains (2 quads x 2 halves) interleaved
#pragma unroll
      for (int k = 0; k < B; ++k)
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int q = 0; q < 2; ++q)
            acc[q][h] = __builtin_amdgcn_mfma_f32_4x4x1f32(xv[q][k], cf[h][k], acc[q][h], 0, 0, 0);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int o = 4 * h + j;
        if (valid && o < B) {
          float* dst = tile + 4 * pcol(col0 + o * s);
          *reinterpret_cast<f32x4*>(dst) = acc[0][h];
          *reinterpret_cast<f32x4*>(dst + plane) = acc[1][h];
        }
      }
    } else {
      // D[i][j] = sum_k C[4h+i][k] x[row j][k]: lane j gets outputs 4h..4h+3 of row 4q+j
#pragma unroll
      for (int k = 0; k < B; ++k)
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int q = 0; q < 2; ++q)
            acc[q][h] = __builtin_amdgcn_mfma_f32_4x4x1f32(cf[h][k], xv[q][k], acc[q][h], 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int r = 4 * q + j;
        if (valid && r < nr) {
          float v[8] = {acc[q][0].x, acc[q][0].y, acc[q][0].z, acc[q][0].w,
                        acc[q][1].x, acc[q][1].y, acc[q][1].z, acc[q][1].w};
          T* y = static_cast<T*>(p.y) + (row0 + r) * p.ldy + col0;
          if constexpr (std::is_same<T, uint16_t>::value) {
            st_stream(y, pack_row<T>(v));
          } else {
            st_stream(y, pack_row<T>(v));
            st_stream(y + 4, pack_row<T>(v + 4));
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int k = 0; k < 8; ++k) cf[h][k] = nx[h][k];
  }
}

template <typename T, typename TB, bool TR, int GPR>
__device__ void run_stage(const RowParams& p, int t, float* tile, float (&cf)[2][8], int64_t row0, int nr) {
  if (p.direct_out && t == p.m - 1) {
    mfma_stage<8, T, TB, TR, true, GPR>(p, t, tile, cf, row0, nr);
    return;
  }
  switch (p.st[t].b) {
    case 2: mfma_stage<2, T, TB, TR, false, GPR>(p, t, tile, cf, row0, nr); break;
    case 4: mfma_stage<4, T, TB, TR, false, GPR>(p, t, tile, cf, row0, nr); break;
    case 5: mfma_stage<5, T, TB, TR, false, GPR>(p, t, tile, cf, row0, nr); break;
    case 8: mfma_stage<8, T, TB, TR, false, GPR>(p, t, tile, cf, row0, nr); break;
    default: break;
  }
}


template <typename T, typename TB, bool TR, typename RL>
__global__ void __launch_bounds__(RL::kThreads) apply_mfma_kernel(RowParams p) {
  constexpr int kCompWaves = RL::kCompWaves;
  constexpr int kIoThreads = RL::kIoThreads;
  constexpr int kMaxIo = RL::kMaxIo;
  extern __shared__ float tile[];
  const bool io_wave = threadIdx.x >= 64 * kCompWaves;
  int64_t tix = blockIdx.x;
  if (tix >= p.ntiles) return;   // uniform per workgroup
  if (io_wave) {
    data_waves<T, kIoThreads, kMaxIo>(p, tile, threadIdx.x - 64 * kCompWaves);
    return;
  }
  {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float cf[2][8];
    {
      const int g0 = wave * 16 + (lane >> 2);
      load_coef_any<TB, TR>(p, p.st[0], g0 < p.st[0].G ? g0 : 0, lane & 3, g0 < p.st[0].G, cf);
    }
    __syncthreads();
    for (; tix < p.ntiles; tix += gridDim.x) {
      const int64_t row0 = tix * kRows;
      const int nr = tile_rows(p, tix);
      for (int t = 0; t < p.m; ++t) {
        run_stage<T, TB, TR, RL::kGroupsPerRound>(p, t, tile, cf, row0, nr);
        __syncthreads();
      }
      if (!p.direct_out) __syncthreads();
      __syncthreads();
    }
  }
}

template <typename T, typename TB, typename RL>
hipError_t launch_mfma_roles(const RowParams& p, int grid, size_t lds, hipStream_t st) {
  auto kern = p.transpose ? apply_mfma_kernel<T, TB, true, RL> : apply_mfma_kernel<T, TB, false, RL>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(RL::kThreads), lds, st, p);
  return hipGetLastError();
}

template <typename T, typename TB>
hipError_t launch_mfma_typed(const RowParams& p, int roles, int grid, size_t lds, hipStream_t st) {
  if (roles == 1) return launch_mfma_roles<T, TB, Roles<8, 4, 2>>(p, grid, lds, st);
  return launch_mfma_roles<T, TB, Roles<8, 8, 1>>(p, grid, lds, st);
}

template <typename T>
hipError_t launch_mfma_blk(DT bdt, const RowParams& p, int roles, int grid, size_t lds, hipStream_t st) {
  switch (bdt) {
    case DT::F32: return launch_mfma_typed<T, float>(p, roles, grid, lds, st);
    case DT::BF16: return launch_mfma_typed<T, uint16_t>(p, roles, grid, lds, st);
    case DT::I8: return launch_mfma_typed<T, int8_t>(p, roles, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool row_path_supported(const Plan& pl, DT io, const void* blocks, const int8_t* signs, const void* x, int64_t ldx,
                         const void* y, int64_t ldy) {
  if (io != DT::F32 && io != DT::BF16) return false;
  if (reinterpret_cast<uintptr_t>(blocks) % 16 != 0) return false;
  if (pl.d % 64 != 0 || pl.d > 5120) return false;
  for (int t = 0; t < pl.m; ++t) {
    const int b = pl.radix[t];
    if (b != 2 && b != 4 && b != 5 && b != 8) return false;
    if ((pl.d / b) % 64 != 0) return false;
  }
  const int eb = io_bytes(io);
  if ((ldx * eb) % 16 || (ldy * eb) % 16) return false;
  if (reinterpret_cast<uintptr_t>(signs) % 8 != 0) return false;
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(y) % 16) return false;
  return true;
}

hipError_t launch_apply_mfma(const Plan& pl, bool inverse, const void* blocks, DT bdt, const float* scales,
                             const int8_t* signs, const void* x, int64_t ldx, DT io, void* y, int64_t ldy,
                             int64_t rows, int roles, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  RowParams p = make_row_params(pl, inverse, blocks, scales, signs, x, ldx, io, y, ldy, rows);
  const size_t lds = (size_t)kRows * pl.d * sizeof(float);
  int64_t grid = cu_count();
  if (grid > p.ntiles) grid = p.ntiles;
  if (io == DT::BF16) return launch_mfma_blk<uint16_t>(bdt, p, roles, (int)grid, lds, stream);
  return launch_mfma_blk<float>(bdt, p, roles, (int)grid, lds, stream);
}

}  // namespace harp