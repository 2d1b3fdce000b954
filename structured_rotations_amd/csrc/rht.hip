// Composition of k randomized Hadamard transforms over rows.
//
// "Quantizing With Randomized Hadamard Transforms: Efficient Heuristic Now
// Proven" (arXiv 2605.06014, abstract): composing two RHTs brings every
// coordinate's marginal close to Gaussian, three give decaying coordinate
// covariance.  One RHT is a sign flip D_j followed by the normalised Hadamard
// H_d.  H_d (natural Sylvester order) factors as the Kronecker product of
// Sylvester blocks along the schedule's digits, so each stage is an
// in-register butterfly network over a group's b_t coordinates, with no
// coefficients.  The row tile stays in LDS for all k passes; signs are
// applied as the first stage of a pass reads (forward) or the last stage of a
// pass writes (inverse); the k normalisations are one scale at the store.
#include <cmath>

#include "common.h"
#include "kernels.h"
#include "tile_io.h"

namespace harp {

struct RhtExtra {
  int k;
  int inverse;
};

template <int B>
__device__ __forceinline__ void fwht_inreg(float* v) {
#pragma unroll
  for (int h = 1; h < B; h *= 2) {
#pragma unroll
    for (int i = 0; i < B; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

__device__ __forceinline__ float sgn_mul(float v, int8_t s) {
  return __uint_as_float(__float_as_uint(v) ^ (s < 0 ? 0x80000000u : 0u));
}

// One Sylvester stage on the tile.  pre / post: sign vector applied to the
// group's coordinates before / after the butterflies (or NULL).
template <int B>
__device__ void hstage(const TileParams& p, const StageDesc& sd, float* tile, int nr,
                       const int8_t* pre, const int8_t* post) {
  const int ngroups = p.d / B;
  const int s = sd.s;
  int slices = (int)blockDim.x / ngroups;
  if (slices < 1) slices = 1;
  const int items = ngroups * slices;
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int g = it % ngroups;
    const int slice = it / ngroups;
    const int base = (g / s) * B * s + (g % s);
    for (int r = slice; r < nr; r += slices) {
      float* row = tile + r * p.ldsrow;
      float v[B];
#pragma unroll
      for (int k = 0; k < B; ++k) v[k] = row[swz(base + k * s)];
      if (pre) {
#pragma unroll
        for (int k = 0; k < B; ++k) v[k] = sgn_mul(v[k], pre[base + k * s]);
      }
      fwht_inreg<B>(v);
      if (post) {
#pragma unroll
        for (int k = 0; k < B; ++k) v[k] = sgn_mul(v[k], post[base + k * s]);
      }
#pragma unroll
      for (int k = 0; k < B; ++k) row[swz(base + k * s)] = v[k];
    }
  }
}

__device__ void run_hstage(const TileParams& p, int t, float* tile, int nr, const int8_t* pre,
                           const int8_t* post) {
  const StageDesc& sd = p.st[t];
  switch (sd.b) {
    case 2: hstage<2>(p, sd, tile, nr, pre, post); break;
    case 4: hstage<4>(p, sd, tile, nr, pre, post); break;
    case 8: hstage<8>(p, sd, tile, nr, pre, post); break;
    case 16: hstage<16>(p, sd, tile, nr, pre, post); break;
    default: break;
  }
}

template <typename TIN, typename TOUT>
__global__ void __launch_bounds__(512) rht_tile_kernel(TileParams p, RhtExtra ex) {
  extern __shared__ float tile[];
  for (int64_t tix = blockIdx.x; tix < p.ntiles; tix += gridDim.x) {
    const int64_t row0 = tix * p.R;
    const int64_t left = p.rows - row0;
    const int nr = left < p.R ? (int)left : p.R;
    load_tile<TIN>(p, tile, row0, nr);
    __syncthreads();
    for (int pass = 0; pass < ex.k; ++pass) {
      // forward pass j = pass uses D_{j+1} before H; inverse pass uses
      // D_{k-pass} after H.
      const int8_t* sg = p.signs + (int64_t)(ex.inverse ? ex.k - 1 - pass : pass) * p.d;
      for (int t = 0; t < p.m; ++t) {
        const int8_t* pre = (!ex.inverse && t == 0) ? sg : nullptr;
        const int8_t* post = (ex.inverse && t == p.m - 1) ? sg : nullptr;
        run_hstage(p, t, tile, nr, pre, post);
        __syncthreads();
      }
    }
    store_tile<TOUT>(p, tile, row0, nr);
    __syncthreads();
  }
}

namespace {
int cu_count() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
    else
      return 256;
  }
  return cus;
}

template <typename TIN, typename TOUT>
hipError_t launch_rht_typed(const TileParams& p, const RhtExtra& ex, int threads, int grid, size_t lds,
                            hipStream_t stream) {
  auto kern = rht_tile_kernel<TIN, TOUT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, stream, p, ex);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_rht(const Plan& pl, const int8_t* signs, int k, bool inverse, const void* x,
                      int64_t ldx, DT in_dt, void* y, int64_t ldy, DT out_dt, int64_t rows,
                      hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  TileParams p{};
  p.d = (int)pl.d;
  p.ldsrow = (int)((pl.d + 63) / 64 * 64);
  p.m = pl.m;
  p.sign_mode = 0;
  for (int t = 0; t < pl.m; ++t) {
    p.st[t].b = pl.radix[t];
    p.st[t].s = (int)pl.stride[t];
  }
  const int ib = io_bytes(in_dt), ob = io_bytes(out_dt);
  p.vec_in = (pl.d * ib % 16 == 0) && (ldx * ib % 16 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  p.vec_out = (pl.d * ob % 16 == 0) && (ldy * ob % 16 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0);
  p.signs = signs;
  p.x = x;
  p.ldx = ldx;
  p.y = y;
  p.ldy = ldy;
  p.rows = rows;
  p.out_scale = (float)std::pow((double)pl.d, -0.5 * (double)k);
  const size_t row_bytes = (size_t)p.ldsrow * sizeof(float);
  const size_t budget = pl.d >= 2048 ? (size_t)160 * 1024 : (size_t)64 * 1024;
  int64_t R = (int64_t)(budget / row_bytes);
  if (R < 1) R = 1;
  if (R > rows) R = rows;
  p.R = (int)R;
  p.ntiles = (rows + R - 1) / R;
  const size_t lds = (size_t)R * row_bytes;
  const int threads = pl.d >= 2048 ? 512 : 256;
  int64_t grid = (int64_t)cu_count() * (pl.d >= 2048 ? 1 : 2);
  if (grid > p.ntiles) grid = p.ntiles;
  RhtExtra ex{k, inverse ? 1 : 0};
  if (in_dt == DT::F32 && out_dt == DT::F32) return launch_rht_typed<float, float>(p, ex, threads, (int)grid, lds, stream);
  if (in_dt == DT::BF16 && out_dt == DT::BF16) return launch_rht_typed<uint16_t, uint16_t>(p, ex, threads, (int)grid, lds, stream);
  return hipErrorInvalidValue;
}

}  // namespace harp
