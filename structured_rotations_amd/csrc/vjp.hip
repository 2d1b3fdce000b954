// Reverse-mode derivative of the row transform, for fitting the parameters on
// calibration data.
//
// HARP technical summary (gist.science 2605.29843), §2.3: the parameters are
// fitted per layer by minimising a calibration loss; §2.1-§2.2: the transform
// is y = S_{m-1} ... S_0 D_s x with block-diagonal stages.  For an upstream
// gradient dy per row:
//   x_0 = D_s x, x_{t+1} = S_t x_t;   g_m = dy, g_t = S_t^T g_{t+1};
//   dL/dB_{t,c}[r][k] = sum over rows of g_{t+1}[c, r] * x_t[c, k];
//   dL/dx = D_s g_0.
// The forward launches store x_1 .. x_{m-1} (fp32) in the workspace; x_0 is
// re-read from x.  Each backward launch handles one stage: a thread owns one
// group (half a group for radices 6..8) and a chunk of rows, keeps its part
// of the group's block and of its b x b gradient in registers, and writes the
// gradient of its chunk to a slot of its own;
// a last launch sums the slots in a fixed order (no atomics, so the result
// does not depend on scheduling).  Radices up to 8.
#include "common.h"
#include "kernels.h"

namespace harp {

namespace {

constexpr int kVjpThreads = 256;
constexpr int64_t kVjpTargetThreads = 262144;   // threads per stage launch (group x row chunk)

struct VjpStage {
  int b, s;           // radix, digit stride
  int ngroups;        // d / b
  int64_t blk_off;    // first coefficient of the stage
  int64_t grp_off;    // first group of the stage
};

struct VjpArgs {
  VjpStage st;
  int64_t d, rows, rpc;      // rows per chunk
  int nchunk;
  const void* blocks;
  const float* scales;
  const int8_t* signs;       // applied where the input is x (or the output is dx)
  const void* xin;           // x_t (or x for t = 0)
  int64_t ldx;
  int x_bf16;                // x_t stored as bf16 (only x itself can be)
  int x_sign;                // x_t = D_s x (t = 0)
  const void* gin;           // g_{t+1}
  int64_t ldg;
  int g_bf16;
  void* out;                 // forward: x_{t+1}; backward: g_t (or dx)
  int64_t ldo;
  int o_bf16;
  int o_sign;
  float* partial;            // backward: [nchunk][n_blk]
  int64_t n_blk;
};

template <typename TB>
__device__ __forceinline__ float coef_at(const TB* b, int64_t i);
template <>
__device__ __forceinline__ float coef_at<float>(const float* b, int64_t i) { return b[i]; }
template <>
__device__ __forceinline__ float coef_at<uint16_t>(const uint16_t* b, int64_t i) { return bf16_to_f32(b[i]); }
template <>
__device__ __forceinline__ float coef_at<int8_t>(const int8_t* b, int64_t i) { return (float)b[i]; }

template <int B, typename TB>
__device__ __forceinline__ void load_block(const VjpArgs& a, int c, float (&blk)[B][B]) {
  const TB* bp = static_cast<const TB*>(a.blocks) + a.st.blk_off + (int64_t)c * B * B;
  const float sc = sizeof(TB) == 1 ? a.scales[a.st.grp_off + c] : 1.0f;
#pragma unroll
  for (int r = 0; r < B; ++r)
#pragma unroll
    for (int k = 0; k < B; ++k) blk[r][k] = coef_at<TB>(bp, r * B + k) * sc;
}

// x_{t+1} = S_t x_t for the rows of one chunk and one group (TX: bf16 only
// when the input is the caller's x, t = 0).
template <typename T>
__device__ __forceinline__ float ld_t(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld_t<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_t<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <int B, typename TB, typename TX>
__global__ void __launch_bounds__(kVjpThreads) vjp_fwd_kernel(VjpArgs a) {
  const int64_t id = (int64_t)blockIdx.x * kVjpThreads + threadIdx.x;
  if (id >= (int64_t)a.st.ngroups * a.nchunk) return;
  const int c = (int)(id % a.st.ngroups);
  const int chunk = (int)(id / a.st.ngroups);
  const int s = a.st.s;
  const int64_t base = (int64_t)(c / s) * B * s + c % s;
  float blk[B][B];
  load_block<B, TB>(a, c, blk);
  float sg[B];
#pragma unroll
  for (int j = 0; j < B; ++j) sg[j] = a.x_sign ? (float)a.signs[base + j * s] : 1.0f;
  const int64_t r0 = (int64_t)chunk * a.rpc;
  const int64_t r1 = r0 + a.rpc < a.rows ? r0 + a.rpc : a.rows;
  const TX* xin = static_cast<const TX*>(a.xin) + base;
  float* out = static_cast<float*>(a.out) + base;
  for (int64_t row = r0; row < r1; ++row) {
    const TX* xr = xin + row * a.ldx;
    float* orow = out + row * a.ldo;
    float v[B];
#pragma unroll
    for (int j = 0; j < B; ++j) v[j] = ld_t<TX>(xr, j * s) * sg[j];
#pragma unroll
    for (int r = 0; r < B; ++r) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < B; ++k) acc = fmaf(blk[r][k], v[k], acc);
      orow[r * s] = acc;
    }
  }
}

// Threads per group in the backward launch: radices 6..8 split a group over
// two threads (thread h owns gradient rows and block columns [h*RH, h*RH+RH)),
// which halves the registers a thread keeps and doubles the waves per SIMD.
template <int B>
constexpr int bwd_split() {
  return B >= 6 ? 2 : 1;
}

template <typename T>
__device__ __forceinline__ void st_t(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void st_t<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void st_t<uint16_t>(uint16_t* p, int64_t i, float v) {
  p[i] = (uint16_t)f32_to_bf16_rne(v);
}

// g_t = S_t^T g_{t+1} and the chunk's sum of g_{t+1}[c] x_t[c]^T.  TX, TG, TO:
// element types of x_t, g_{t+1} and the output (bf16 only where they are the
// caller's rows: x and dx for t = 0, dy for t = m - 1).
template <int B, typename TB, typename TX, typename TG, typename TO>
__global__ void __launch_bounds__(kVjpThreads) vjp_bwd_kernel(VjpArgs a) {
  constexpr int H = bwd_split<B>();
  constexpr int RH = (B + H - 1) / H;            // rows (and columns) per thread
  const int64_t id = (int64_t)blockIdx.x * kVjpThreads + threadIdx.x;
  if (id >= (int64_t)a.st.ngroups * a.nchunk * H) return;
  const int h = (int)(id % H);
  const int64_t gid = id / H;
  const int c = (int)(gid % a.st.ngroups);
  const int chunk = (int)(gid / a.st.ngroups);
  const int s = a.st.s;
  const int64_t base = (int64_t)(c / s) * B * s + c % s;
  // blk[r][kk] = B[r][h * RH + kk]: the block columns this thread's outputs need
  float blk[B][RH];
  {
    const TB* bp = static_cast<const TB*>(a.blocks) + a.st.blk_off + (int64_t)c * B * B;
    const float sc = sizeof(TB) == 1 ? a.scales[a.st.grp_off + c] : 1.0f;
#pragma unroll
    for (int r = 0; r < B; ++r)
#pragma unroll
      for (int kk = 0; kk < RH; ++kk) {
        const int k = h * RH + kk;
        blk[r][kk] = k < B ? coef_at<TB>(bp, r * B + k) * sc : 0.0f;
      }
  }
  float xs[B], os[RH];
#pragma unroll
  for (int j = 0; j < B; ++j) xs[j] = a.x_sign ? (float)a.signs[base + j * s] : 1.0f;
#pragma unroll
  for (int kk = 0; kk < RH; ++kk) {
    const int k = h * RH + kk;
    os[kk] = (a.o_sign && k < B) ? (float)a.signs[base + k * s] : 1.0f;
  }
  float acc[RH][B];
#pragma unroll
  for (int rr = 0; rr < RH; ++rr)
#pragma unroll
    for (int k = 0; k < B; ++k) acc[rr][k] = 0.0f;
  const int64_t r0 = (int64_t)chunk * a.rpc;
  const int64_t r1 = r0 + a.rpc < a.rows ? r0 + a.rpc : a.rows;
  const TG* gin = static_cast<const TG*>(a.gin) + base;
  const TX* xin = static_cast<const TX*>(a.xin) + base;
  TO* out = static_cast<TO*>(a.out) + base;
  for (int64_t row = r0; row < r1; ++row) {
    const TG* gr = gin + row * a.ldg;
    const TX* xr = xin + row * a.ldx;
    float g[B], v[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      g[j] = ld_t<TG>(gr, j * s);
      v[j] = ld_t<TX>(xr, j * s) * xs[j];
    }
#pragma unroll
    for (int rr = 0; rr < RH; ++rr) {
      const int r = h * RH + rr;
      const float gv = r < B ? g[r < B ? r : 0] : 0.0f;
#pragma unroll
      for (int k = 0; k < B; ++k) acc[rr][k] = fmaf(gv, v[k], acc[rr][k]);
    }
    if (a.out != nullptr) {
      TO* orow = out + row * a.ldo;
#pragma unroll
      for (int kk = 0; kk < RH; ++kk) {
        const int k = h * RH + kk;
        if (k < B) {
          float o = 0.0f;
#pragma unroll
          for (int r = 0; r < B; ++r) o = fmaf(blk[r][kk], g[r], o);
          st_t<TO>(orow, k * s, o * os[kk]);
        }
      }
    }
  }
  float* pp = a.partial + (int64_t)chunk * a.n_blk + a.st.blk_off + (int64_t)c * B * B;
#pragma unroll
  for (int rr = 0; rr < RH; ++rr) {
    const int r = h * RH + rr;
    if (r < B) {
#pragma unroll
      for (int k = 0; k < B; ++k) pp[r * B + k] = acc[rr][k];
    }
  }
}

__global__ void __launch_bounds__(kVjpThreads) vjp_reduce_kernel(const float* partial, int nchunk, int64_t n_blk,
                                                                 float* dblocks) {
  const int64_t i = (int64_t)blockIdx.x * kVjpThreads + threadIdx.x;
  if (i >= n_blk) return;
  float acc = 0.0f;
  for (int ch = 0; ch < nchunk; ++ch) acc += partial[(int64_t)ch * n_blk + i];
  dblocks[i] = acc;
}

int vjp_chunks(const Plan& pl, int64_t rows) {
  int64_t ng = pl.d;
  for (int t = 0; t < pl.m; ++t)
    if (pl.d / pl.radix[t] < ng) ng = pl.d / pl.radix[t];
  int64_t n = (kVjpTargetThreads + ng - 1) / ng;
  if (n > rows) n = rows;
  if (n < 1) n = 1;
  return (int)n;
}

template <int B, typename TB>
hipError_t launch_stage(bool fwd, const VjpArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.st.ngroups * a.nchunk * (fwd ? 1 : bwd_split<B>());
  const int64_t grid = (n + kVjpThreads - 1) / kVjpThreads;
  if (fwd) {
    if (a.x_bf16)
      hipLaunchKernelGGL((vjp_fwd_kernel<B, TB, uint16_t>), dim3((unsigned)grid), dim3(kVjpThreads), 0, st, a);
    else
      hipLaunchKernelGGL((vjp_fwd_kernel<B, TB, float>), dim3((unsigned)grid), dim3(kVjpThreads), 0, st, a);
  } else {
    using F = float;
    using H16 = uint16_t;
    const int code = (a.x_bf16 ? 4 : 0) | (a.g_bf16 ? 2 : 0) | (a.o_bf16 ? 1 : 0);
    switch (code) {
      case 0: hipLaunchKernelGGL((vjp_bwd_kernel<B, TB, F, F, F>), dim3((unsigned)grid), dim3(kVjpThreads), 0, st, a); break;
      case 5: hipLaunchKernelGGL((vjp_bwd_kernel<B, TB, H16, F, H16>), dim3((unsigned)grid), dim3(kVjpThreads), 0, st, a); break;
      case 4: hipLaunchKernelGGL((vjp_bwd_kernel<B, TB, H16, F, F>), dim3((unsigned)grid), dim3(kVjpThreads), 0, st, a); break;
      case 2: hipLaunchKernelGGL((vjp_bwd_kernel<B, TB, F, H16, F>), dim3((unsigned)grid), dim3(kVjpThreads), 0, st, a); break;
      case 7: hipLaunchKernelGGL((vjp_bwd_kernel<B, TB, H16, H16, H16>), dim3((unsigned)grid), dim3(kVjpThreads), 0, st, a); break;
      case 6: hipLaunchKernelGGL((vjp_bwd_kernel<B, TB, H16, H16, F>), dim3((unsigned)grid), dim3(kVjpThreads), 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <typename TB>
hipError_t launch_stage_b(bool fwd, const VjpArgs& a, hipStream_t st) {
  switch (a.st.b) {
    case 2: return launch_stage<2, TB>(fwd, a, st);
    case 3: return launch_stage<3, TB>(fwd, a, st);
    case 4: return launch_stage<4, TB>(fwd, a, st);
    case 5: return launch_stage<5, TB>(fwd, a, st);
    case 6: return launch_stage<6, TB>(fwd, a, st);
    case 7: return launch_stage<7, TB>(fwd, a, st);
    case 8: return launch_stage<8, TB>(fwd, a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stage_any(bool fwd, DT bdt, const VjpArgs& a, hipStream_t st) {
  if (bdt == DT::F32) return launch_stage_b<float>(fwd, a, st);
  if (bdt == DT::BF16) return launch_stage_b<uint16_t>(fwd, a, st);
  return launch_stage_b<int8_t>(fwd, a, st);
}

}  // namespace

int64_t vjp_workspace_bytes(const Plan& pl, int64_t rows) {
  for (int t = 0; t < pl.m; ++t)
    if (pl.radix[t] > 8) return -1;
  // at most (m + 1) + 16 fp32 values per row element: keep 4x that in int64
  if (rows > (INT64_MAX / 256) / pl.d) return -1;
  const int64_t acts = (int64_t)(pl.m - 1) * rows * pl.d;
  const int64_t gbuf = (pl.m > 1 ? 2 : 0) * rows * pl.d;
  const int64_t part = (int64_t)vjp_chunks(pl, rows) * pl.n_blk;
  return 4 * (acts + gbuf + part);
}

hipError_t launch_apply_vjp(const Plan& pl, const void* blocks, DT bdt, const float* scales, const int8_t* signs,
                            const void* x, int64_t ldx, const void* dy, int64_t lddy, void* dx, int64_t lddx,
                            DT io, int64_t rows, float* dblocks, void* ws, hipStream_t stream) {
  const int64_t rd = rows * pl.d;
  float* acts = static_cast<float*>(ws);                    // x_1 .. x_{m-1}
  float* gbuf = acts + (int64_t)(pl.m - 1) * rd;            // two g buffers
  float* part = gbuf + (pl.m > 1 ? 2 : 0) * rd;
  const int nchunk = vjp_chunks(pl, rows);
  const int bf = io == DT::BF16 ? 1 : 0;

  auto stage_of = [&](int t) {
    VjpStage s;
    s.b = pl.radix[t];
    s.s = (int)pl.stride[t];
    s.ngroups = (int)(pl.d / s.b);
    s.blk_off = pl.blk_off[t];
    s.grp_off = pl.grp_off[t];
    return s;
  };
  VjpArgs base{};
  base.d = pl.d;
  base.rows = rows;
  base.nchunk = nchunk;
  base.rpc = (rows + nchunk - 1) / nchunk;
  base.blocks = blocks;
  base.scales = scales;
  base.signs = signs;
  base.n_blk = pl.n_blk;
  base.partial = part;

  // forward: x_{t+1} = S_t x_t for t = 0 .. m-2
  for (int t = 0; t + 1 < pl.m; ++t) {
    VjpArgs a = base;
    a.st = stage_of(t);
    a.xin = t == 0 ? x : static_cast<const void*>(acts + (int64_t)(t - 1) * rd);
    a.ldx = t == 0 ? ldx : pl.d;
    a.x_bf16 = t == 0 ? bf : 0;
    a.x_sign = (t == 0 && signs != nullptr) ? 1 : 0;
    a.out = acts + (int64_t)t * rd;
    a.ldo = pl.d;
    hipError_t e = launch_stage_any(true, bdt, a, stream);
    if (e != hipSuccess) return e;
  }
  // backward: t = m-1 .. 0
  for (int t = pl.m - 1; t >= 0; --t) {
    VjpArgs a = base;
    a.st = stage_of(t);
    const int k = pl.m - 1 - t;   // backward step
    a.gin = t == pl.m - 1 ? dy : static_cast<const void*>(gbuf + (int64_t)((k + 1) & 1) * rd);
    a.ldg = t == pl.m - 1 ? lddy : pl.d;
    a.g_bf16 = t == pl.m - 1 ? bf : 0;
    a.xin = t == 0 ? x : static_cast<const void*>(acts + (int64_t)(t - 1) * rd);
    a.ldx = t == 0 ? ldx : pl.d;
    a.x_bf16 = t == 0 ? bf : 0;
    a.x_sign = (t == 0 && signs != nullptr) ? 1 : 0;
    if (t == 0) {
      a.out = dx;
      a.ldo = lddx;
      a.o_bf16 = bf;
      a.o_sign = signs != nullptr ? 1 : 0;
    } else {
      a.out = gbuf + (int64_t)(k & 1) * rd;
      a.ldo = pl.d;
    }
    hipError_t e = launch_stage_any(false, bdt, a, stream);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = (pl.n_blk + kVjpThreads - 1) / kVjpThreads;
  hipLaunchKernelGGL(vjp_reduce_kernel, dim3((unsigned)grid), dim3(kVjpThreads), 0, stream, part, nchunk, pl.n_blk,
                     dblocks);
  return hipGetLastError();
}

}  // namespace harp
