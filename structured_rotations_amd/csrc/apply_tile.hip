// Generic row-tile kernel for the HARP transform and its inverse.
//
// HARP technical summary (gist.science 2605.29843), §2.1: the rotation is a
// product of stages; stage t applies a block-diagonal orthogonal matrix to
// groups of coordinates separated by stride permutations.  Here no
// permutation is materialised: a row tile sits in LDS (fp32, bank-swizzled)
// and stage t reads each group's b_t coordinates directly at digit stride s_t,
// multiplies by the group's block (held in registers and reused over every
// row of the tile) and writes the result back in place.  §2.2 defines the
// blocks; §2.4 notes the deployment path fuses the stride stages.
//
// Any schedule (radices 2..16, d <= 32768), fp32 or bf16 rows, fp32 / bf16 /
// int8+scale blocks.  The inverse runs the stages in reverse order with
// transposed blocks and applies the sign on the output side.
#include <cstdlib>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tile_io.h"

namespace harp {

// One stage on the whole tile.  Work item = (group g, row slice); a slice is
// every `slices`-th row, so small-d stages still occupy every thread.
template <int B, typename TB>
__device__ void stage_impl(const TileParams& p, const StageDesc& sd, float* tile, int nr) {
  const int ngroups = p.d / B;
  const int s = sd.s;
  int slices = (int)blockDim.x / ngroups;
  if (slices < 1) slices = 1;
  const int items = ngroups * slices;
  const TB* blk = static_cast<const TB*>(p.blocks) + sd.blk_off;
  const bool contiguous = (s == 1) && (B == 4 || B == 8);
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int g = it % ngroups;
    const int slice = it / ngroups;
    const int lo = g % s;
    const int hi = g / s;
    const int base = hi * B * s + lo;
    float scale = 1.0f;
    if constexpr (std::is_same<TB, int8_t>::value) scale = p.scales[sd.grp_off + g];
    const int64_t gb = (int64_t)g * B * B;
    if constexpr (B <= 8) {
      float c[B][B];
#pragma unroll
      for (int o = 0; o < B; ++o)
#pragma unroll
        for (int k = 0; k < B; ++k)
          c[o][k] = coef<TB>(blk, gb + (p.transpose ? k * B + o : o * B + k), scale);
      for (int r = slice; r < nr; r += slices) {
        float* row = tile + r * p.ldsrow;
        float v[B];
        if (contiguous) {
          const float* q = row + swz(base);
#pragma unroll
          for (int k = 0; k < B; ++k) v[k] = q[k];
        } else {
#pragma unroll
          for (int k = 0; k < B; ++k) v[k] = row[swz(base + k * s)];
        }
        float out[B];
#pragma unroll
        for (int o = 0; o < B; ++o) {
          float acc = 0.0f;
#pragma unroll
          for (int k = 0; k < B; ++k) acc = fmaf(c[o][k], v[k], acc);
          out[o] = acc;
        }
        if (contiguous) {
          float* q = row + swz(base);
#pragma unroll
          for (int o = 0; o < B; ++o) q[o] = out[o];
        } else {
#pragma unroll
          for (int o = 0; o < B; ++o) row[swz(base + o * s)] = out[o];
        }
      }
    } else {
      for (int r = slice; r < nr; r += slices) {
        float* row = tile + r * p.ldsrow;
        float v[B];
#pragma unroll
        for (int k = 0; k < B; ++k) v[k] = row[swz(base + k * s)];
        float out[B];
        for (int o = 0; o < B; ++o) {
          float acc = 0.0f;
#pragma unroll
          for (int k = 0; k < B; ++k)
            acc = fmaf(coef<TB>(blk, gb + (p.transpose ? k * B + o : o * B + k), scale), v[k], acc);
          out[o] = acc;
        }
#pragma unroll
        for (int o = 0; o < B; ++o) row[swz(base + o * s)] = out[o];
      }
    }
  }
}

// BIG: radices 9..16 compiled in.  Their b x b register blocks set the
// register count (and spills) of the whole kernel, so schedules whose radices
// are all at most 8 run a variant without them.
template <typename TB, bool BIG>
__device__ void run_stage(const TileParams& p, int t, float* tile, int nr) {
  const StageDesc& sd = p.st[t];
  switch (sd.b) {
    case 2: stage_impl<2, TB>(p, sd, tile, nr); break;
    case 3: stage_impl<3, TB>(p, sd, tile, nr); break;
    case 4: stage_impl<4, TB>(p, sd, tile, nr); break;
    case 5: stage_impl<5, TB>(p, sd, tile, nr); break;
    case 6: stage_impl<6, TB>(p, sd, tile, nr); break;
    case 7: stage_impl<7, TB>(p, sd, tile, nr); break;
    case 8: stage_impl<8, TB>(p, sd, tile, nr); break;
    default:
      if constexpr (BIG) {
        switch (sd.b) {
          case 9: stage_impl<9, TB>(p, sd, tile, nr); break;
          case 10: stage_impl<10, TB>(p, sd, tile, nr); break;
          case 11: stage_impl<11, TB>(p, sd, tile, nr); break;
          case 12: stage_impl<12, TB>(p, sd, tile, nr); break;
          case 13: stage_impl<13, TB>(p, sd, tile, nr); break;
          case 14: stage_impl<14, TB>(p, sd, tile, nr); break;
          case 15: stage_impl<15, TB>(p, sd, tile, nr); break;
          case 16: stage_impl<16, TB>(p, sd, tile, nr); break;
          default: break;
        }
      }
      break;
  }
}

template <typename TIN, typename TOUT, typename TB, bool BIG>
__global__ void __launch_bounds__(512) apply_tile_kernel(TileParams p) {
  extern __shared__ float tile[];
  for (int64_t tix = blockIdx.x; tix < p.ntiles; tix += gridDim.x) {
    const int64_t row0 = tix * p.R;
    const int64_t left = p.rows - row0;
    const int nr = left < p.R ? (int)left : p.R;
    load_tile<TIN>(p, tile, row0, nr);
    __syncthreads();
    for (int t = 0; t < p.m; ++t) {
      run_stage<TB, BIG>(p, t, tile, nr);
      __syncthreads();
    }
    store_tile<TOUT>(p, tile, row0, nr);
    __syncthreads();
  }
}

namespace {

bool env_flag(const char* name) {
  const char* v = std::getenv(name);
  return v != nullptr && v[0] != '\0' && v[0] != '0';
}

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  return (v != nullptr && v[0] != '\0') ? std::atoi(v) : dflt;
}

int device_cu_count() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus = v;
  }
  return cus;
}

template <typename TIN, typename TOUT, typename TB, bool BIG>
hipError_t launch_typed(const TileParams& p, int threads, int grid, size_t lds, hipStream_t stream) {
  auto kern = apply_tile_kernel<TIN, TOUT, TB, BIG>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, stream, p);
  return hipGetLastError();
}

template <typename TIN, typename TOUT, bool BIG>
hipError_t launch_blk_b(DT bdt, const TileParams& p, int threads, int grid, size_t lds, hipStream_t st) {
  switch (bdt) {
    case DT::F32: return launch_typed<TIN, TOUT, float, BIG>(p, threads, grid, lds, st);
    case DT::BF16: return launch_typed<TIN, TOUT, uint16_t, BIG>(p, threads, grid, lds, st);
    case DT::I8: return launch_typed<TIN, TOUT, int8_t, BIG>(p, threads, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename TIN, typename TOUT>
hipError_t launch_blk(DT bdt, const TileParams& p, int threads, int grid, size_t lds, hipStream_t st) {
  bool big = false;
  for (int i = 0; i < p.m; ++i) big = big || p.st[i].b > 8;
  return big ? launch_blk_b<TIN, TOUT, true>(bdt, p, threads, grid, lds, st)
             : launch_blk_b<TIN, TOUT, false>(bdt, p, threads, grid, lds, st);
}

}  // namespace

hipError_t launch_apply_rows(const Plan& pl, bool inverse, const void* blocks, DT bdt,
                             const float* scales, const int8_t* signs, const void* x,
                             int64_t ldx, DT in_dt, void* y, int64_t ldy, DT out_dt,
                             int64_t rows, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  // Row-tile kernels: the schedule-specialised matrix-core kernel where the
  // schedule has one, else the matrix-core kernel for fp32 and bf16 blocks
  // and the vector-ALU kernel for int8 blocks (whose coefficient traffic is
  // small enough that the plain FMA path wins).  HARP_ROW_KERNEL overrides
  // the choice (1 generic matrix-core, 2 vector-ALU, 3 generic tile kernel,
  // 4 schedule-specialised kernels where they apply);
  // HARP_ROW_ROLES picks the matrix-core kernel's wave split.
  static const int row_kernel = env_int("HARP_ROW_KERNEL", 0);
  if (in_dt == out_dt && row_kernel != 3 && row_path_supported(pl, in_dt, blocks, signs, x, ldx, y, ldy)) {
    static const int roles = env_int("HARP_ROW_ROLES", 0);
    if ((row_kernel == 0 || row_kernel == 4) && fast_path_supported(pl, bdt))
      return launch_apply_fast(pl, inverse, blocks, bdt, scales, signs, x, ldx, in_dt, y, ldy, rows, stream);
    const bool valu = row_kernel == 2 || (row_kernel == 0 && bdt == DT::I8);
    if (valu)
      return launch_apply_valu(pl, inverse, blocks, bdt, scales, signs, x, ldx, in_dt, y, ldy, rows, roles, stream);
    return launch_apply_mfma(pl, inverse, blocks, bdt, scales, signs, x, ldx, in_dt, y, ldy, rows, roles, stream);
  }
  TileParams p{};
  p.d = (int)pl.d;
  p.ldsrow = (int)((pl.d + 63) / 64 * 64);
  p.m = pl.m;
  p.transpose = inverse ? 1 : 0;
  p.sign_mode = signs ? (inverse ? 2 : 1) : 0;
  for (int i = 0; i < pl.m; ++i) {
    const int t = inverse ? pl.m - 1 - i : i;
    p.st[i].b = pl.radix[t];
    p.st[i].s = (int)pl.stride[t];
    p.st[i].blk_off = (int)pl.blk_off[t];
    p.st[i].grp_off = (int)pl.grp_off[t];
  }
  const int ib = io_bytes(in_dt), ob = io_bytes(out_dt);
  p.vec_in = (pl.d * ib % 16 == 0) && (ldx * ib % 16 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  p.vec_out = (pl.d * ob % 16 == 0) && (ldy * ob % 16 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0);
  p.blocks = blocks;
  p.scales = scales;
  p.signs = signs;
  p.x = x;
  p.ldx = ldx;
  p.y = y;
  p.ldy = ldy;
  p.rows = rows;
  p.out_scale = 1.0f;
  // Tile: as many rows as fit the LDS budget; large rows take the whole LDS
  // (one workgroup per CU), small rows leave room for several workgroups.
  const size_t row_bytes = (size_t)p.ldsrow * sizeof(float);
  const size_t budget = pl.d >= 2048 ? (size_t)160 * 1024 : (size_t)64 * 1024;
  const int threads = pl.d >= 2048 ? 512 : 256;
  const int wg_per_cu = pl.d >= 2048 ? 1 : 2;
  const int64_t slots = (int64_t)device_cu_count() * wg_per_cu;
  int64_t R = (int64_t)(budget / row_bytes);
  if (R < 1) R = 1;
  // a small batch is spread over every workgroup slot rather than packed
  // into as few tiles as the LDS allows
  const int64_t spread = (rows + slots - 1) / slots;
  if (R > spread) R = spread;
  if (R > rows) R = rows;
  p.R = (int)R;
  p.ntiles = (rows + R - 1) / R;
  const size_t lds = (size_t)R * row_bytes;
  int64_t grid = slots;
  if (grid > p.ntiles) grid = p.ntiles;
  if (in_dt == DT::F32 && out_dt == DT::F32) return launch_blk<float, float>(bdt, p, threads, (int)grid, lds, stream);
  if (in_dt == DT::BF16 && out_dt == DT::BF16) return launch_blk<uint16_t, uint16_t>(bdt, p, threads, (int)grid, lds, stream);
  if (in_dt == DT::BF16 && out_dt == DT::F32) return launch_blk<uint16_t, float>(bdt, p, threads, (int)grid, lds, stream);
  if (in_dt == DT::F32 && out_dt == DT::BF16) return launch_blk<float, uint16_t>(bdt, p, threads, (int)grid, lds, stream);
  return hipErrorInvalidValue;
}

}  // namespace harp
