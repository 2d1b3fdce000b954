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
  int vec_in;        // 16-byte row segments: aligned base, ld and panel starts
  int vec_out;
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

// Row stride of a staged block in LDS: each output row of C starts on a
// 16-byte boundary so a task reads it with 128-bit broadcast loads.
template <int B>
constexpr int coef_row_stride() { return (B + 3) & ~3; }

// Stage the coefficients of the tile's groups for one stage into LDS as
// fp32 C[o][k] (C = B forward, B^T inverse; int8 blocks dequantised), rows
// padded to coef_row_stride<B>() floats, so the stage's tasks read them with
// broadcast LDS loads.
template <int B, typename TB>
__device__ void stage_coefs(const ColParams& p, const ColStage& cs, float* cbuf, int64_t pre, int64_t q) {
  constexpr int Bp = coef_row_stride<B>();
  const int ngl = p.nsub / B;
  const TB* blocks = static_cast<const TB*>(p.blocks) + cs.blk_off;
  for (int e = threadIdx.x; e < ngl * B * B; e += blockDim.x) {
    const int gl = e / (B * B);
    const int i = e - gl * (B * B);
    const int o = i / B, k = i - o * B;
    const int64_t c = pre * (int64_t)ngl * p.suf + (int64_t)gl * p.suf + q;
    float scale = 1.0f;
    if constexpr (std::is_same<TB, int8_t>::value) scale = p.scales[cs.grp_off + c];
    cbuf[gl * (B * Bp) + o * Bp + k] = coef<TB>(blocks, c * B * B + (p.transpose ? k * B + o : i), scale);
  }
}

// One stage of the run on the tile.  The tile is [nsub][pw] fp32; a task is
// one group of the stage and a block of 64 columns, one column per lane, so
// every lane of a wave uses the same coefficients (read from cbuf).  All
// reads of a task come before its stores (the tile and the coefficients
// never overlap), so they are issued back to back.
template <int B>
__device__ void col_stage(const ColParams& p, const ColStage& cs, float* __restrict__ tile,
                          const float* __restrict__ cbuf, int wave, int nwaves, int lane) {
  constexpr int Bp = coef_row_stride<B>();
  const int ngl = p.nsub / B;             // local groups in the tile
  const int ncb = p.pw / 64;              // 64-column blocks
  const int ntask = ngl * ncb;
  const int ls = cs.ls;
  for (int task = wave; task < ntask; task += nwaves) {
    const int gl = task / ncb;
    const int cb = task - gl * ncb;
    const int u_lo = gl % ls;
    const int u_hi = gl / ls;
    const int ubase = u_hi * B * ls + u_lo;
    const f32x4* cf = reinterpret_cast<const f32x4*>(cbuf + gl * (B * Bp));
    float* col = tile + ubase * p.pw + cb * 64 + lane;
    float v[B];
#pragma unroll
    for (int k = 0; k < B; ++k) v[k] = col[k * ls * p.pw];
    float acc[B];
#pragma unroll
    for (int o = 0; o < B; ++o) {
      f32x4 c4[Bp / 4];
#pragma unroll
      for (int j = 0; j < Bp / 4; ++j) c4[j] = cf[o * (Bp / 4) + j];
      float a = 0.0f;
#pragma unroll
      for (int k = 0; k < B; ++k) a = fmaf(c4[k >> 2][k & 3], v[k], a);
      acc[o] = a;
    }
#pragma unroll
    for (int o = 0; o < B; ++o) col[o * ls * p.pw] = acc[o];
  }
}

// BIG: radices 9..16 compiled in (their b^2 coefficients raise the
// register count of the whole kernel, so runs of radices <= 8 use a kernel
// without them).
template <typename TB, bool BIG>
__device__ void run_col_stage(const ColParams& p, int i, float* tile, float* cbuf, int64_t pre, int64_t q, int wave,
                              int nwaves, int lane) {
  const ColStage& cs = p.st[i];
  switch (cs.b) {
    case 2:
      stage_coefs<2, TB>(p, cs, cbuf, pre, q);
      __syncthreads();
      col_stage<2>(p, cs, tile, cbuf, wave, nwaves, lane);
      break;
    case 3:
      stage_coefs<3, TB>(p, cs, cbuf, pre, q);
      __syncthreads();
      col_stage<3>(p, cs, tile, cbuf, wave, nwaves, lane);
      break;
    case 4:
      stage_coefs<4, TB>(p, cs, cbuf, pre, q);
      __syncthreads();
      col_stage<4>(p, cs, tile, cbuf, wave, nwaves, lane);
      break;
    case 5:
      stage_coefs<5, TB>(p, cs, cbuf, pre, q);
      __syncthreads();
      col_stage<5>(p, cs, tile, cbuf, wave, nwaves, lane);
      break;
    case 6:
      stage_coefs<6, TB>(p, cs, cbuf, pre, q);
      __syncthreads();
      col_stage<6>(p, cs, tile, cbuf, wave, nwaves, lane);
      break;
    case 7:
      stage_coefs<7, TB>(p, cs, cbuf, pre, q);
      __syncthreads();
      col_stage<7>(p, cs, tile, cbuf, wave, nwaves, lane);
      break;
    case 8:
      stage_coefs<8, TB>(p, cs, cbuf, pre, q);
      __syncthreads();
      col_stage<8>(p, cs, tile, cbuf, wave, nwaves, lane);
      break;
    case 9:
      if constexpr (BIG) {
        stage_coefs<9, TB>(p, cs, cbuf, pre, q);
        __syncthreads();
        col_stage<9>(p, cs, tile, cbuf, wave, nwaves, lane);
      }
      break;
    case 10:
      if constexpr (BIG) {
        stage_coefs<10, TB>(p, cs, cbuf, pre, q);
        __syncthreads();
        col_stage<10>(p, cs, tile, cbuf, wave, nwaves, lane);
      }
      break;
    case 11:
      if constexpr (BIG) {
        stage_coefs<11, TB>(p, cs, cbuf, pre, q);
        __syncthreads();
        col_stage<11>(p, cs, tile, cbuf, wave, nwaves, lane);
      }
      break;
    case 12:
      if constexpr (BIG) {
        stage_coefs<12, TB>(p, cs, cbuf, pre, q);
        __syncthreads();
        col_stage<12>(p, cs, tile, cbuf, wave, nwaves, lane);
      }
      break;
    case 13:
      if constexpr (BIG) {
        stage_coefs<13, TB>(p, cs, cbuf, pre, q);
        __syncthreads();
        col_stage<13>(p, cs, tile, cbuf, wave, nwaves, lane);
      }
      break;
    case 14:
      if constexpr (BIG) {
        stage_coefs<14, TB>(p, cs, cbuf, pre, q);
        __syncthreads();
        col_stage<14>(p, cs, tile, cbuf, wave, nwaves, lane);
      }
      break;
    case 15:
      if constexpr (BIG) {
        stage_coefs<15, TB>(p, cs, cbuf, pre, q);
        __syncthreads();
        col_stage<15>(p, cs, tile, cbuf, wave, nwaves, lane);
      }
      break;
    case 16:
      if constexpr (BIG) {
        stage_coefs<16, TB>(p, cs, cbuf, pre, q);
        __syncthreads();
        col_stage<16>(p, cs, tile, cbuf, wave, nwaves, lane);
      }
      break;
    default: break;
  }
}

template <typename T> struct ColIo;
template <> struct ColIo<uint16_t> { static constexpr int V = 8; };
template <> struct ColIo<float> { static constexpr int V = 4; };

// 16-byte chunk <-> V consecutive fp32 tile entries
__device__ __forceinline__ void unpack_chunk(const u32x4& w, float* v, const uint16_t*) {
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void unpack_chunk(const u32x4& w, float* v, const float*) {
  v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y); v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
}
__device__ __forceinline__ u32x4 pack_chunk(const float* v, uint16_t*) {
  return u32x4{pack_bf16x2_hw(v[0], v[1]), pack_bf16x2_hw(v[2], v[3]), pack_bf16x2_hw(v[4], v[5]),
               pack_bf16x2_hw(v[6], v[7])};
}
__device__ __forceinline__ u32x4 pack_chunk(const float* v, float*) {
  return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
}

// Tile geometry of one persistent-loop iteration.
struct ColTile {
  int64_t row_base;   // first row; tile row u is row_base + u * suf
  int64_t col0;
  int64_t pre, q;
  int w;              // valid columns
};

__device__ __forceinline__ ColTile col_tile(const ColParams& p, int64_t tix) {
  ColTile t;
  const int64_t rt = tix / p.npanels;
  const int64_t pn = tix - rt * p.npanels;
  t.pre = rt / p.suf;
  t.q = rt - t.pre * p.suf;
  t.col0 = pn * p.pw;
  const int64_t left = p.ncols - t.col0;
  t.w = left < p.pw ? (int)left : p.pw;
  t.row_base = t.pre * (int64_t)p.nsub * p.suf + t.q;
  return t;
}

// The tile's 16-byte input chunks owned by this thread (chunk i = threadIdx.x
// + j * blockDim.x), loaded into registers ahead of use.
template <typename TIN, int MAXC>
__device__ __forceinline__ void col_prefetch(const ColParams& p, const ColTile& t, u32x4 (&r)[MAXC]) {
  constexpr int VI = ColIo<TIN>::V;
  const TIN* x = static_cast<const TIN*>(p.x);
  const int cpr = p.pw / VI;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int i = threadIdx.x + j * blockDim.x;
    if (i < p.nsub * cpr) {
      const int u = i / cpr;
      const int ch = i - u * cpr;
      r[j] = ld_stream(x + (t.row_base + (int64_t)u * p.suf) * p.ldx + t.col0 + ch * VI);
    }
  }
}

template <typename TIN, int MAXC>
__device__ __forceinline__ void col_to_lds(const ColParams& p, const ColTile& t, const u32x4 (&r)[MAXC], float* tile) {
  constexpr int VI = ColIo<TIN>::V;
  const int cpr = p.pw / VI;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int i = threadIdx.x + j * blockDim.x;
    if (i < p.nsub * cpr) {
      const int u = i / cpr;
      const int ch = i - u * cpr;
      float v[VI];
      unpack_chunk(r[j], v, static_cast<const TIN*>(nullptr));
      if (p.sign_mode == 1 && p.signs[t.row_base + (int64_t)u * p.suf] < 0) {
#pragma unroll
        for (int e = 0; e < VI; ++e) v[e] = -v[e];
      }
      float* dst = tile + u * p.pw + ch * VI;
#pragma unroll
      for (int e = 0; e < VI; e += 4) *reinterpret_cast<f32x4*>(dst + e) = f32x4{v[e], v[e + 1], v[e + 2], v[e + 3]};
    }
  }
}

// MAXC: 16-byte input chunks per thread of a full tile (128 KiB of fp32 at
// most: 8 for bf16 input, 16 for fp32 input, with 512 threads).
template <typename TIN, typename TOUT, typename TB, bool BIG>
__global__ void __launch_bounds__(512) col_pass_kernel(ColParams p) {
  extern __shared__ float tile[];
  float* cbuf = tile + p.nsub * p.pw;     // one stage's coefficients (nsub * padded row floats)
  constexpr int VI = ColIo<TIN>::V, VO = ColIo<TOUT>::V;
  constexpr int MAXC = VI == 8 ? 8 : 16;
  const TIN* x = static_cast<const TIN*>(p.x);
  TOUT* y = static_cast<TOUT*>(p.y);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  // full tiles of a 16-byte aligned matrix stream through registers: the next
  // tile's loads are in flight while this one is transformed and stored
  const bool vec = p.vec_in && p.vec_out && p.ncols % p.pw == 0;
  u32x4 pf[MAXC];
  int64_t tix = blockIdx.x;
  if (vec && tix < p.ntiles) col_prefetch<TIN, MAXC>(p, col_tile(p, tix), pf);
  for (; tix < p.ntiles; tix += gridDim.x) {
    const ColTile t = col_tile(p, tix);
    if (vec) {
      col_to_lds<TIN, MAXC>(p, t, pf, tile);
      const int64_t nxt = tix + gridDim.x;
      if (nxt < p.ntiles) col_prefetch<TIN, MAXC>(p, col_tile(p, nxt), pf);
    } else {
      for (int i = threadIdx.x; i < p.nsub * p.pw; i += blockDim.x) {
        const int u = i / p.pw;
        const int j = i - u * p.pw;
        float v = 0.0f;
        if (j < t.w) {
          const int64_t row = t.row_base + (int64_t)u * p.suf;
          v = ld_el(x + row * p.ldx + t.col0 + j);
          if (p.sign_mode == 1 && p.signs[row] < 0) v = -v;
        }
        tile[i] = v;
      }
    }
    __syncthreads();
    for (int s = 0; s < p.nstage; ++s) {
      run_col_stage<TB, BIG>(p, s, tile, cbuf, t.pre, t.q, wave, nwaves, lane);
      __syncthreads();
    }
    if (vec) {
      const int cpr = p.pw / VO;
      for (int i = threadIdx.x; i < p.nsub * cpr; i += blockDim.x) {
        const int u = i / cpr;
        const int ch = i - u * cpr;
        const int64_t row = t.row_base + (int64_t)u * p.suf;
        const float* src = tile + u * p.pw + ch * VO;
        float v[VO];
#pragma unroll
        for (int e = 0; e < VO; e += 4) {
          const f32x4 q4 = *reinterpret_cast<const f32x4*>(src + e);
          v[e] = q4.x; v[e + 1] = q4.y; v[e + 2] = q4.z; v[e + 3] = q4.w;
        }
        if (p.sign_mode == 2 && p.signs[row] < 0) {
#pragma unroll
          for (int e = 0; e < VO; ++e) v[e] = -v[e];
        }
        st_stream(y + row * p.ldy + t.col0 + ch * VO, pack_chunk(v, y));
      }
    } else {
      for (int i = threadIdx.x; i < p.nsub * p.pw; i += blockDim.x) {
        const int u = i / p.pw;
        const int j = i - u * p.pw;
        if (j < t.w) {
          const int64_t row = t.row_base + (int64_t)u * p.suf;
          float v = tile[i];
          if (p.sign_mode == 2 && p.signs[row] < 0) v = -v;
          st_el(y + row * p.ldy + t.col0 + j, v);
        }
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
hipError_t launch_cols_typed(const ColParams& p, bool big, int grid, size_t lds, hipStream_t st) {
  auto kern = big ? col_pass_kernel<TIN, TOUT, TB, true> : col_pass_kernel<TIN, TOUT, TB, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(512), lds, st, p);
  return hipGetLastError();
}

template <typename TIN, typename TOUT>
hipError_t launch_cols_blk(DT bdt, const ColParams& p, bool big, int grid, size_t lds, hipStream_t st) {
  switch (bdt) {
    case DT::F32: return launch_cols_typed<TIN, TOUT, float>(p, big, grid, lds, st);
    case DT::BF16: return launch_cols_typed<TIN, TOUT, uint16_t>(p, big, grid, lds, st);
    case DT::I8: return launch_cols_typed<TIN, TOUT, int8_t>(p, big, grid, lds, st);
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
  // tile fits in 128 KiB; stage tasks are 64-column blocks, so a run wider
  // than 512 rows is not supported here (the host splits runs at 512).
  int pw = 512;
  while (pw > 64 && (size_t)nsub * pw * sizeof(float) > (size_t)128 * 1024) pw -= 64;
  if ((size_t)nsub * (pw + 16) * sizeof(float) > (size_t)160 * 1024) return hipErrorInvalidValue;
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
  const int ib = io_bytes(in_dt), ob = io_bytes(out_dt);
  p.vec_in = reinterpret_cast<uintptr_t>(x) % 16 == 0 && (ldx * ib) % 16 == 0;
  p.vec_out = reinterpret_cast<uintptr_t>(y) % 16 == 0 && (ldy * ob) % 16 == 0;
  int bmax = 2, cw = 4;   // largest radix; widest padded coefficient row (a stage stages nsub * row floats)
  for (int t = t0; t < t1; ++t) {
    bmax = pl.radix[t] > bmax ? pl.radix[t] : bmax;
    cw = ((pl.radix[t] + 3) & ~3) > cw ? ((pl.radix[t] + 3) & ~3) : cw;
  }
  const size_t lds = ((size_t)nsub * pw + (size_t)nsub * cw) * sizeof(float);
  int64_t grid = (int64_t)cus_for_cols() * (lds > 80 * 1024 ? 1 : 2);
  if (grid > p.ntiles) grid = p.ntiles;
  if (in_dt == DT::F32 && out_dt == DT::F32) return launch_cols_blk<float, float>(bdt, p, bmax > 8, (int)grid, lds, stream);
  if (in_dt == DT::BF16 && out_dt == DT::BF16) return launch_cols_blk<uint16_t, uint16_t>(bdt, p, bmax > 8, (int)grid, lds, stream);
  if (in_dt == DT::BF16 && out_dt == DT::F32) return launch_cols_blk<uint16_t, float>(bdt, p, bmax > 8, (int)grid, lds, stream);
  if (in_dt == DT::F32 && out_dt == DT::BF16) return launch_cols_blk<float, uint16_t>(bdt, p, bmax > 8, (int)grid, lds, stream);
  return hipErrorInvalidValue;
}

}  // namespace harp
