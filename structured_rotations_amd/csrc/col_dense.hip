// Column runs of at most 32 rows as one dense product per row group (the
// second pass over the row index in "Technical Summary: HARP", §3, the
// two-sided processor, for runs of small radices such as (3, 3, 3)).
//
// A run of stages acting on the row sub-index u < nsub of the groups of rows
// r = row_base + u * suf is, for each group, one nsub x nsub orthogonal matrix
// M (the product of the run's stages, with the row signs of the pass folded
// in).  For nsub <= 32 the workgroup composes M once in LDS (a few thousand
// FMAs) and then streams its columns through the matrix cores: every lane
// owns one column, loads its nsub values, and 4 x 4 x 1 fp32 products with
// A = four rows of M and B = the lane's column value accumulate all nsub
// outputs in registers.  No tile, no per-stage barrier, no swap: the pass is a
// load -> products -> store stream, at the price of nsub products per element
// instead of the sum of the radices (27 against 9 for (3, 3, 3), cheap on the
// matrix cores).
#include "common.h"
#include "kernels.h"

namespace harp {
namespace {

constexpr int kDenseMaxRows = 32;    // nsub <= 32: at most 8 row quads
constexpr int kDenseStride = 36;     // LDS row stride of M (floats): 16-byte aligned, 4-row reads conflict-free
constexpr int kDenseWaves = 4;
constexpr int kDenseThreads = 64 * kDenseWaves;

struct DenseStage {
  int b;         // radix
  int ls;        // stride of the digit inside the run's sub-index
  int blk_off;   // first coefficient of the stage
  int grp_off;   // first group of the stage (int8 scales)
};

struct DenseParams {
  int nsub;
  int nstage;       // processing order in st[]
  int transpose;    // inverse: transposed blocks
  int sign_mode;    // 0 none, 1 on the rows entering the run, 2 on the rows leaving it
  int bdt;          // DT of the blocks
  int splits;       // workgroups per row group
  int64_t suf;      // product of the radices after the run
  int64_t ngroups;  // d / nsub
  int64_t ncols;
  int64_t nchunks;  // ceil(ncols / 64)
  DenseStage st[kMaxStagesDev];
  const void* blocks;
  const float* scales;
  const int8_t* signs;
  const void* x;
  int64_t ldx;
  void* y;
  int64_t ldy;
};

__device__ __forceinline__ float block_coef(const DenseParams& p, int64_t idx, int64_t grp) {
  if (p.bdt == (int)DT::F32) return static_cast<const float*>(p.blocks)[idx];
  if (p.bdt == (int)DT::BF16) return bf16_to_f32(static_cast<const uint16_t*>(p.blocks)[idx]);
  return (float)static_cast<const int8_t*>(p.blocks)[idx] * p.scales[grp];
}

// M of row group rt into Mf[i * kDenseStride + j] (output row i, input row j),
// zero outside nsub x nsub.  The run's coefficients go into LDS first (one
// load per thread and element, all in flight together), then each stage maps
// the columns of the current product to the next one: element (u, j) of the
// result is the radix-b inner product of the coefficient row of u's digit
// with the b entries of column j in u's group.  Two buffers, one barrier per
// stage.
__device__ void compose(const DenseParams& p, int64_t rt, float* Mf, float* Mt, float* cf) {
  const int n = p.nsub;
  const int64_t pre = rt / p.suf, q = rt - pre * p.suf;
  const int64_t row_base = pre * n * p.suf + q;
  // coefficients C_s[gl][d][k] (transposed blocks for the inverse), stage by stage
  int off = 0;
  for (int s = 0; s < p.nstage; ++s) {
    const DenseStage& ds = p.st[s];
    const int B = ds.b, BB = B * B, ngl = n / B;
    for (int e = threadIdx.x; e < ngl * BB; e += kDenseThreads) {
      const int gl = e / BB, i = e - gl * BB, d = i / B, k = i - d * B;
      const int64_t grp = (pre * ngl + gl) * p.suf + q;
      cf[off + e] = block_coef(p, ds.blk_off + grp * BB + (p.transpose ? k * B + d : i), ds.grp_off + grp);
    }
    off += ngl * BB;
  }
  // start: the identity, or the input signs on its diagonal
  for (int e = threadIdx.x; e < kDenseMaxRows * kDenseStride; e += kDenseThreads) {
    const int i = e / kDenseStride, j = e - i * kDenseStride;
    float v = 0.f;
    if (i == j && i < n) v = (p.sign_mode == 1 && p.signs[row_base + (int64_t)i * p.suf] < 0) ? -1.f : 1.f;
    Mf[e] = v;
    Mt[e] = 0.f;
  }
  __syncthreads();
  float* src = Mf;
  float* dst = Mt;
  off = 0;
  for (int s = 0; s < p.nstage; ++s) {
    const DenseStage& ds = p.st[s];
    const int B = ds.b, ls = ds.ls;
    const bool last = s + 1 == p.nstage;
    for (int e = threadIdx.x; e < n * n; e += kDenseThreads) {
      const int u = e / n, j = e - u * n;
      const int uh = u / (B * ls), rem = u - uh * B * ls, d = rem / ls, ul = rem - d * ls;
      const int gl = uh * ls + ul, base = uh * B * ls + ul;
      const float* c = cf + off + gl * B * B + d * B;
      float acc = 0.f;
      for (int k = 0; k < B; ++k) acc = fmaf(c[k], src[(base + k * ls) * kDenseStride + j], acc);
      if (last && p.sign_mode == 2 && p.signs[row_base + (int64_t)u * p.suf] < 0) acc = -acc;
      dst[u * kDenseStride + j] = acc;
    }
    off += (n / B) * B * B;
    __syncthreads();
    float* t = src; src = dst; dst = t;
  }
  // the result is in src; make Mf hold it
  if (src != Mf) {
    for (int e = threadIdx.x; e < n * kDenseStride; e += kDenseThreads) {
      const int i = e / kDenseStride, j = e - i * kDenseStride;
      if (j < n) Mf[e] = src[e];
    }
    __syncthreads();
  }
}

// CPL adjacent columns per lane (1, or 2 for bf16 input when rows, pointers
// and the column count are even: 4-byte loads instead of 2-byte ones, and
// 4- or 8-byte stores).  The loaded words stay as loaded until their product.
template <typename T, int CPL> struct ColWord;
template <> struct ColWord<uint16_t, 1> { using W = uint16_t; };
template <> struct ColWord<uint16_t, 2> { using W = uint32_t; };
template <> struct ColWord<float, 1> { using W = float; };
template <> struct ColWord<float, 2> { using W = f32x2; };

template <typename T, int CPL>
__device__ __forceinline__ float col_val(const typename ColWord<T, CPL>::W& w, int e) {
  if constexpr (std::is_same<T, float>::value) {
    if constexpr (CPL == 1) return w;
    else return e ? w.y : w.x;
  } else {
    if constexpr (CPL == 1) return bf16_to_f32(w);
    else return e ? bf16_hi(w) : bf16_lo(w);
  }
}

// Buffer loads and stores: the row group's first row is the resource base
// (uniform), the lane's column the 32-bit vector offset and the row within
// the group the scalar offset, so no per-row 64-bit addresses are kept.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dense_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
template <typename W> __device__ __forceinline__ W buf_ld(__amdgpu_buffer_rsrc_t r, int vo, int so);
template <> __device__ __forceinline__ uint16_t buf_ld<uint16_t>(__amdgpu_buffer_rsrc_t r, int vo, int so) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0);
}
template <> __device__ __forceinline__ uint32_t buf_ld<uint32_t>(__amdgpu_buffer_rsrc_t r, int vo, int so) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0);
}
template <> __device__ __forceinline__ float buf_ld<float>(__amdgpu_buffer_rsrc_t r, int vo, int so) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0));
}
template <> __device__ __forceinline__ f32x2 buf_ld<f32x2>(__amdgpu_buffer_rsrc_t r, int vo, int so) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0);
  return f32x2{__uint_as_float(v.x), __uint_as_float(v.y)};
}

template <typename T, int CPL>
__device__ __forceinline__ void col_store(__amdgpu_buffer_rsrc_t r, int vo, int so, const float (&v)[CPL]) {
  if constexpr (std::is_same<T, float>::value) {
    if constexpr (CPL == 1) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), r, vo, so, 0);
    else __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(v[0]), __float_as_uint(v[CPL - 1])}, r, vo, so, 0);
  } else {
    const uint32_t w = pack_bf16x2_hw(v[0], CPL == 2 ? v[CPL - 1] : 0.f);
    if constexpr (CPL == 1) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w & 0xffffu), r, vo, so, 0);
    else __builtin_amdgcn_raw_buffer_store_b32(w, r, vo, so, 0);
  }
}

// NQ row quads (nsub <= 4 NQ).  Workgroup blockIdx.x: row group
// blockIdx.x / splits, its share of the 64 CPL-column chunks; each wave takes
// every kDenseWaves-th chunk of the share.  Columns past ncols re-read the
// last column (pair) and are not stored.
template <int NQ, int CPL, typename TIN, typename TOUT>
__global__ void __launch_bounds__(kDenseThreads) __attribute__((amdgpu_waves_per_eu(NQ == 8 || (CPL == 2 && NQ == 7) ? 3 : 4)))
col_dense_kernel(DenseParams p) {
  __shared__ __align__(16) float Mf[kDenseMaxRows * kDenseStride];
  __shared__ __align__(16) float Mt[kDenseMaxRows * kDenseStride];
  __shared__ float cf[kDenseMaxRows * kDenseMaxRows];   // the run's coefficients: sum over stages of nsub * b <= 32 * 32
  using W = typename ColWord<TIN, CPL>::W;
  constexpr int KP = 4 * NQ;
  const int64_t rt = blockIdx.x / p.splits;
  const int split = blockIdx.x - (int)rt * p.splits;
  const int n = p.nsub;
  const int64_t pre = rt / p.suf, q = rt - pre * p.suf;
  const int64_t row_base = pre * n * p.suf + q;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r4 = lane & 3;
  const int64_t per = (p.nchunks + p.splits - 1) / p.splits;
  const int64_t c_lo = split * per;
  const int64_t c_hi = c_lo + per < p.nchunks ? c_lo + per : p.nchunks;
  const __amdgpu_buffer_rsrc_t rx = dense_rsrc(static_cast<const TIN*>(p.x) + row_base * p.ldx);
  const __amdgpu_buffer_rsrc_t ry = dense_rsrc(static_cast<TOUT*>(p.y) + row_base * p.ldy);
  // bytes from one row of the group to the next (the host keeps nsub of them below 2^31)
  const int sx = (int)(p.suf * p.ldx * (int64_t)sizeof(TIN));
  const int sy = (int)(p.suf * p.ldy * (int64_t)sizeof(TOUT));
  // The chunk's column words: the next chunk's loads go out as soon as this
  // chunk's products are issued (before its stores), the first chunk's before
  // M is composed, so each wave has one chunk's loads in flight while it
  // computes, stores or composes.
  W xw[KP];
  auto load = [&](int64_t cc) {
    const int64_t col = (cc * 64 + lane) * CPL;
    const int vx = (int)((col < p.ncols ? col : p.ncols - CPL) * (int64_t)sizeof(TIN));
#pragma unroll
    for (int k = 0; k < KP; ++k) xw[k] = k < n ? buf_ld<W>(rx, vx, k * sx) : W{};
  };
  int64_t c = c_lo + wave;
  if (c < c_hi) load(c);
  compose(p, rt, Mf, Mt, cf);
  for (; c < c_hi; c += kDenseWaves) {
    const int64_t col = (c * 64 + lane) * CPL;
    const bool valid = col < p.ncols;
    f32x4 acc[CPL][NQ];
#pragma unroll
    for (int e = 0; e < CPL; ++e)
#pragma unroll
      for (int i = 0; i < NQ; ++i) acc[e][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // M is re-read from LDS for every chunk: kept in registers across the
    // loop it would take 4 NQ^2 of them and most of the occupancy
    int moff = r4 * kDenseStride;
    asm volatile("" : "+v"(moff));
    // one k quad at a time: its NQ reads of M, then its products (reading
    // every quad up front would hold 4 NQ^2 registers)
#pragma unroll
    for (int kq = 0; kq < NQ; ++kq) {
      f32x4 a[NQ];
#pragma unroll
      for (int i = 0; i < NQ; ++i)   // M[4i + r4][4kq .. 4kq + 3]: four distinct 16-byte reads per wave
        a[i] = *reinterpret_cast<const f32x4*>(Mf + moff + 4 * i * kDenseStride + 4 * kq);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < NQ; ++i)
#pragma unroll
          for (int e = 0; e < CPL; ++e)
            acc[e][i] = __builtin_amdgcn_mfma_f32_4x4x1f32(a[i][kk], col_val<TIN, CPL>(xw[4 * kq + kk], e), acc[e][i],
                                                           0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c + kDenseWaves < c_hi) load(c + kDenseWaves);
    __builtin_amdgcn_sched_barrier(0);
    if (valid) {
      const int vy = (int)(col * (int64_t)sizeof(TOUT));
#pragma unroll
      for (int i = 0; i < NQ; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * i + r < n) {
            float v[CPL];
#pragma unroll
            for (int e = 0; e < CPL; ++e) v[e] = acc[e][i][r];
            col_store<TOUT, CPL>(ry, vy, (4 * i + r) * sy, v);
          }
    }
  }
}

template <int NQ, typename TIN, typename TOUT>
hipError_t launch_nq(const DenseParams& p, int cpl, int64_t grid, hipStream_t st) {
  // two columns per lane: bf16 input and up to 28 rows (beyond that, or with
  // fp32 words, the doubled registers spill)
  if constexpr (std::is_same<TIN, uint16_t>::value && NQ < 8) {
    if (cpl == 2) {
      hipLaunchKernelGGL((col_dense_kernel<NQ, 2, TIN, TOUT>), dim3((unsigned)grid), dim3(kDenseThreads), 0, st, p);
      return hipGetLastError();
    }
  }
  if (cpl != 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL((col_dense_kernel<NQ, 1, TIN, TOUT>), dim3((unsigned)grid), dim3(kDenseThreads), 0, st, p);
  return hipGetLastError();
}

template <typename TIN, typename TOUT>
hipError_t launch_io(const DenseParams& p, int cpl, int64_t grid, hipStream_t st) {
  switch ((p.nsub + 3) / 4) {
    case 1: return launch_nq<1, TIN, TOUT>(p, cpl, grid, st);
    case 2: return launch_nq<2, TIN, TOUT>(p, cpl, grid, st);
    case 3: return launch_nq<3, TIN, TOUT>(p, cpl, grid, st);
    case 4: return launch_nq<4, TIN, TOUT>(p, cpl, grid, st);
    case 5: return launch_nq<5, TIN, TOUT>(p, cpl, grid, st);
    case 6: return launch_nq<6, TIN, TOUT>(p, cpl, grid, st);
    case 7: return launch_nq<7, TIN, TOUT>(p, cpl, grid, st);
    case 8: return launch_nq<8, TIN, TOUT>(p, cpl, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool cols_dense_supported(const Plan& pl, int t0, int t1) {
  int64_t nsub = 1;
  for (int t = t0; t < t1; ++t) nsub *= pl.radix[t];
  return t1 > t0 && nsub <= kDenseMaxRows;
}

hipError_t launch_apply_cols_dense(const Plan& pl, int t0, int t1, bool inverse, const void* blocks, DT bdt,
                                   const float* scales, const int8_t* signs, int sign_mode, const void* x,
                                   int64_t ldx, DT in_dt, void* y, int64_t ldy, DT out_dt, int64_t ncols,
                                   hipStream_t stream) {
  if (ncols <= 0) return hipSuccess;
  if (!cols_dense_supported(pl, t0, t1)) return hipErrorInvalidValue;
  DenseParams p{};
  int nsub = 1;
  for (int t = t0; t < t1; ++t) nsub *= pl.radix[t];
  p.nsub = nsub;
  p.nstage = t1 - t0;
  p.transpose = inverse ? 1 : 0;
  p.sign_mode = signs ? sign_mode : 0;
  p.bdt = (int)bdt;
  p.suf = pl.stride[t1 - 1];
  p.ngroups = pl.d / nsub;
  p.ncols = ncols;
  // two columns per lane where every access of a pair is aligned
  const int ei = io_bytes(in_dt), eo = io_bytes(out_dt);
  const int cpl = (in_dt == DT::BF16 && nsub <= 28 && ncols % 2 == 0 && ldx % 2 == 0 && ldy % 2 == 0 &&
                   reinterpret_cast<uintptr_t>(x) % (2 * ei) == 0 && reinterpret_cast<uintptr_t>(y) % (2 * eo) == 0)
                      ? 2 : 1;
  p.nchunks = (ncols + 64 * cpl - 1) / (64 * cpl);
  for (int i = 0; i < p.nstage; ++i) {
    const int t = inverse ? t1 - 1 - i : t0 + i;
    p.st[i].b = pl.radix[t];
    p.st[i].ls = (int)(pl.stride[t] / p.suf);
    p.st[i].blk_off = (int)pl.blk_off[t];
    p.st[i].grp_off = (int)pl.grp_off[t];
  }
  p.blocks = blocks;
  p.scales = scales;
  p.signs = signs;
  p.x = x;
  p.ldx = ldx;
  p.y = y;
  p.ldy = ldy;
  // about 1024 workgroups in all (four waves per SIMD), at least four chunks
  // (one per wave) per workgroup
  int64_t splits = (1024 + p.ngroups - 1) / p.ngroups;
  const int64_t most = p.nchunks / kDenseWaves > 0 ? p.nchunks / kDenseWaves : 1;
  if (splits > most) splits = most;
  p.splits = (int)splits;
  const int64_t grid = p.ngroups * splits;
  // 32-bit buffer offsets: the group's rows and columns, in bytes
  const int64_t span_x = ((int64_t)(nsub - 1) * p.suf * ldx + ncols) * ei;
  const int64_t span_y = ((int64_t)(nsub - 1) * p.suf * ldy + ncols) * eo;
  if (span_x >= ((int64_t)1 << 31) || span_y >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (in_dt == DT::BF16 && out_dt == DT::BF16) return launch_io<uint16_t, uint16_t>(p, cpl, grid, stream);
  if (in_dt == DT::BF16 && out_dt == DT::F32) return launch_io<uint16_t, float>(p, cpl, grid, stream);
  if (in_dt == DT::F32 && out_dt == DT::BF16) return launch_io<float, uint16_t>(p, cpl, grid, stream);
  if (in_dt == DT::F32 && out_dt == DT::F32) return launch_io<float, float>(p, cpl, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace harp
