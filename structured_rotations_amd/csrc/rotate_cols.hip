// Column passes of the two-sided weight rotation  W~ = M_U W M_V^T.
//
// HARP technical summary (gist.science 2605.29843), §2 and §3, and the arXiv
// abstract: HARP is a two-sided processor, an output-side rotation U and an
// input-side rotation V, acting as an exact change of basis.  M_V acts along
// every row (the row kernels); M_U acts along every column, i.e. on the row
// index of W.  A pass applies a run of consecutive U stages [t0, t1): it
// stages, for one fixed value of the digits outside the run and one panel of
// columns, the prod_{t0<=t<t1} b_t rows that the run mixes, into an LDS tile
// (the tile transpose that turns column work into contiguous panel loads),
// applies the run's stages with columns as the batch dimension (every block
// is reused across the panel), and writes the tile back.  Each tile is owned
// by one workgroup, so a pass may run in place.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace harp {

struct ColStage {
  int b;         // radix
  int ls;        // stride of the digit inside the run's sub-index
  int blk_off;   // first coefficient of the stage
  int grp_off;   // first group of the stage
};

struct ColParams {
  int nsub;          // rows per tile: product of the run's radices
  int nstage;        // stages in the run (processing order in st[])
  int pw;            // panel width (columns per tile)
  int transpose;     // inverse: transposed blocks
  int sign_mode;     // 0 none, 1 on load, 2 on store (indexed by row)
  int64_t suf;       // product of the radices after the run
  int64_t npanels;
  int64_t ntiles;    // (d / nsub) * npanels
  int64_t ncols;
  ColStage st[kMaxStagesDev];
  const void* blocks;
  const float* scales;
  const int8_t* signs;
  const void* x;
  int64_t ldx;
  void* y;
  int64_t ldy;
};

__device__ __forceinline__ float ld_el(const float* p) { return *p; }
__device__ __forceinline__ float ld_el(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void st_el(float* p, float v) { *p = v; }
__device__ __forceinline__ void st_el(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16_rne(v); }

template <int B, typename TB>
__device__ void col_stage(const ColParams& p, const ColStage& cs, float* tile, int64_t pre, int64_t q) {
  const int ngl = p.nsub / B;             // local groups in the tile
  const int items = ngl * p.pw;
  const TB* blk = static_cast<const TB*>(p.blocks) + cs.blk_off;
  const int ls = cs.ls;
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int j = it % p.pw;
    const int gl = it / p.pw;
    const int u_lo = gl % ls;
    const int u_hi = gl / ls;
    const int ubase = u_hi * B * ls + u_lo;
    // global group: C-order index of every digit of the row index except this one
    const int64_t c = pre * (int64_t)ngl * p.suf + (int64_t)gl * p.suf + q;
    float scale = 1.0f;
    if constexpr (std::is_same<TB, int8_t>::value) scale = p.scales[cs.grp_off + c];
    const int64_t gb = c * B * B;
    float v[B];
#pragma unroll
    for (int k = 0; k < B; ++k) v[k] = tile[(ubase + k * ls) * p.pw + j];
    float out[B];
#pragma unroll
    for (int o = 0; o < B; ++o) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < B; ++k)
        acc = fmaf(coef<TB>(blk, gb + (p.transpose ? k * B + o : o * B + k), scale), v[k], acc);
      out[o] = acc;
    }
#pragma unroll
    for (int o = 0; o < B; ++o) tile[(ubase + o * ls) * p.pw + j] = out[o];
  }
}

template <typename TB>
__device__ void run_col_stage(const ColParams& p, int i, float* tile, int64_t pre, int64_t q) {
  const ColStage& cs = p.st[i];
  switch (cs.b) {
    case 2: col_stage<2, TB>(p, cs, tile, pre, q); break;
    case 3: col_stage<3, TB>(p, cs, tile, pre, q); break;
    case 4: col_stage<4, TB>(p, cs, tile, pre, q); break;
    case 5: col_stage<5, TB>(p, cs, tile, pre, q); break;
    case 6: col_stage<6, TB>(p, cs, tile, pre, q); break;
    case 7: col_stage<7, TB>(p, cs, tile, pre, q); break;
    case 8: col_stage<8, TB>(p, cs, tile, pre, q); break;
    case 9: col_stage<9, TB>(p, cs, tile, pre, q); break;
    case 10: col_stage<10, TB>(p, cs, tile, pre, q); break;
    case 11: col_stage<11, TB>(p, cs, tile, pre, q); break;
    case 12: col_stage<12, TB>(p, cs, tile, pre, q); break;
    case 13: col_stage<13, TB>(p, cs, tile, pre, q); break;
    case 14: col_stage<14, TB>(p, cs, tile, pre, q); break;
    case 15: col_stage<15, TB>(p, cs, tile, pre, q); break;
    case 16: col_stage<16, TB>(p, cs, tile, pre, q); break;
    default: break;
  }
}

template <typename TIN, typename TOUT, typename TB>
__global__ void __launch_bounds__(512) col_pass_kernel(ColParams p) {
  extern __shared__ float tile[];
  const TIN* x = static_cast<const TIN*>(p.x);
  TOUT* y = static_cast<TOUT*>(p.y);
  for (int64_t tix = blockIdx.x; tix < p.ntiles; tix += gridDim.x) {
    const int64_t rt = tix / p.npanels;
    const int64_t pn = tix - rt * p.npanels;
    const int64_t pre = rt / p.suf;
    const int64_t q = rt - pre * p.suf;
    const int64_t col0 = pn * p.pw;
    const int64_t left = p.ncols - col0;
    const int w = left < p.pw ? (int)left : p.pw;
    const int64_t row_base = pre * (int64_t)p.nsub * p.suf + q;
    for (int i = threadIdx.x; i < p.nsub * p.pw; i += blockDim.x) {
      const int u = i / p.pw;
      const int j = i - u * p.pw;
      float v = 0.0f;
      if (j < w) {
        const int64_t row = row_base + (int64_t)u * p.suf;
        v = ld_el(x + row * p.ldx + col0 + j);
        if (p.sign_mode == 1 && p.signs[row] < 0) v = -v;
      }
      tile[i] = v;
    }
    __syncthreads();
    for (int s = 0; s < p.nstage; ++s) {
      run_col_stage<TB>(p, s, tile, pre, q);
      __syncthreads();
    }
    for (int i = threadIdx.x; i < p.nsub * p.pw; i += blockDim.x) {
      const int u = i / p.pw;
      const int j = i - u * p.pw;
      if (j < w) {
        const int64_t row = row_base + (int64_t)u * p.suf;
        float v = tile[i];
        if (p.sign_mode == 2 && p.signs[row] < 0) v = -v;
        st_el(y + row * p.ldy + col0 + j, v);
      }
    }
    __syncthreads();
  }
}

namespace {
int cus_for_cols() {
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

template <typename TIN, typename TOUT, typename TB>
hipError_t launch_cols_typed(const ColParams& p, int grid, size_t lds, hipStream_t st) {
  auto kern = col_pass_kernel<TIN, TOUT, TB>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(512), lds, st, p);
  return hipGetLastError();
}

template <typename TIN, typename TOUT>
hipError_t launch_cols_blk(DT bdt, const ColParams& p, int grid, size_t lds, hipStream_t st) {
  switch (bdt) {
    case DT::F32: return launch_cols_typed<TIN, TOUT, float>(p, grid, lds, st);
    case DT::BF16: return launch_cols_typed<TIN, TOUT, uint16_t>(p, grid, lds, st);
    case DT::I8: return launch_cols_typed<TIN, TOUT, int8_t>(p, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_apply_cols(const Plan& pl, int t0, int t1, bool inverse, const void* blocks,
                             DT bdt, const float* scales, const int8_t* signs, int sign_mode,
                             const void* x, int64_t ldx, DT in_dt, void* y, int64_t ldy,
                             DT out_dt, int64_t ncols, hipStream_t stream) {
  if (ncols <= 0) return hipSuccess;
  ColParams p{};
  int nsub = 1;
  for (int t = t0; t < t1; ++t) nsub *= pl.radix[t];
  p.nsub = nsub;
  p.nstage = t1 - t0;
  p.suf = pl.stride[t1 - 1];
  p.transpose = inverse ? 1 : 0;
  p.sign_mode = signs ? sign_mode : 0;
  for (int i = 0; i < p.nstage; ++i) {
    const int t = inverse ? t1 - 1 - i : t0 + i;
    p.st[i].b = pl.radix[t];
    p.st[i].ls = (int)(pl.stride[t] / p.suf);
    p.st[i].blk_off = (int)pl.blk_off[t];
    p.st[i].grp_off = (int)pl.grp_off[t];
  }
  // Panel width: the widest multiple of 64 columns (at most 512) whose fp32
  // tile fits in 160 KiB.
  int pw = 512;
  while (pw > 64 && (size_t)nsub * pw * sizeof(float) > (size_t)160 * 1024) pw -= 64;
  while (pw > 1 && (size_t)nsub * pw * sizeof(float) > (size_t)160 * 1024) pw /= 2;
  p.pw = pw;
  p.ncols = ncols;
  p.npanels = (ncols + pw - 1) / pw;
  p.ntiles = (pl.d / nsub) * p.npanels;
  p.blocks = blocks;
  p.scales = scales;
  p.signs = signs;
  p.x = x;
  p.ldx = ldx;
  p.y = y;
  p.ldy = ldy;
  const size_t lds = (size_t)nsub * pw * sizeof(float);
  int64_t grid = (int64_t)cus_for_cols() * (lds > 80 * 1024 ? 1 : 2);
  if (grid > p.ntiles) grid = p.ntiles;
  if (in_dt == DT::F32 && out_dt == DT::F32) return launch_cols_blk<float, float>(bdt, p, (int)grid, lds, stream);
  if (in_dt == DT::BF16 && out_dt == DT::BF16) return launch_cols_blk<uint16_t, uint16_t>(bdt, p, (int)grid, lds, stream);
  if (in_dt == DT::BF16 && out_dt == DT::F32) return launch_cols_blk<uint16_t, float>(bdt, p, (int)grid, lds, stream);
  if (in_dt == DT::F32 && out_dt == DT::BF16) return launch_cols_blk<float, uint16_t>(bdt, p, (int)grid, lds, stream);
  return hipErrorInvalidValue;
}

}  // namespace harp
