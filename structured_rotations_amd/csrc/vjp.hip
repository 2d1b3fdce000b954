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
// group (half a group for radices 6..8) and a chunk of rows, and keeps its
// part of the group's block and of its b x b gradient in registers.  The
// four waves of a workgroup own the same 64 groups over four consecutive
// row chunks; they add their gradients through LDS in wave order and write
// one slot per workgroup (at ~160 registers a thread, three such workgroups
// fit on a CU).  A last launch sums the slots in slot order.  No atomics
// anywhere, so the result does not depend on scheduling.  Radices up to 8.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace harp {

namespace {

constexpr int kVjpThreads = 256;
constexpr int kBwdWaves = 4;                    // row chunks per backward workgroup
constexpr int kBwdThreads = 64 * kBwdWaves;
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
  float* partial;            // backward: [nchunk / kBwdWaves][n_blk]
  int64_t n_blk;
  int vec1;                  // backward: stride-1 stage whose rows of x_t, g_{t+1} and the output
                             // allow 16-byte (8-byte for 4 bf16) accesses of a group's coordinates
  VjpStage st2;              // fused last pair: the last stage (st is the one before it)
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

// The b consecutive values of a group in a stride-1 stage, as 16-byte (or,
// for 4 bf16, 8-byte) loads.
template <int B, typename T>
__device__ __forceinline__ void ld_vec(const T* p, float (&v)[B]) {
  if constexpr (B != 4 && B != 8) {
    (void)p;   // never reached: only radices 4 and 8 take the vector path
    (void)v;
  } else if constexpr (std::is_same<T, float>::value) {
#pragma unroll
    for (int q = 0; q < B / 4; ++q) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(p + 4 * q);
      v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
    }
  } else if constexpr (B == 8) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  } else {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  }
}

// 4 consecutive outputs (16 bytes of fp32 or 8 of bf16).
template <typename T>
__device__ __forceinline__ void st_vec4(T* p, const float (&o)[4]) {
  if constexpr (std::is_same<T, float>::value)
    *reinterpret_cast<f32x4*>(p) = f32x4{o[0], o[1], o[2], o[3]};
  else
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2_hw(o[0], o[1]), pack_bf16x2_hw(o[2], o[3])};
}

template <int B>
constexpr bool vec1_ok() {
  return B == 8 || B == 4;
}

// g_t = S_t^T g_{t+1} and the sum over the rows of g_{t+1}[c] x_t[c]^T.  TX,
// TG, TO: element types of x_t, g_{t+1} and the output (bf16 only where they
// are the caller's rows: x and dx for t = 0, dy for t = m - 1).  Workgroup
// (chunk block cb, group block gs): lane l of wave w owns the l-th
// (group, half) pair of block gs over row chunk kBwdWaves * cb + w.
template <int B, typename TB, typename TX, typename TG, typename TO>
__global__ void __launch_bounds__(kBwdThreads) vjp_bwd_kernel(VjpArgs a) {
  constexpr int H = bwd_split<B>();
  constexpr int RH = (B + H - 1) / H;            // rows (and columns) per thread
  constexpr int NA = RH * B;                     // gradient entries per thread
  __shared__ float red[kBwdWaves - 1][NA][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t npair = (int64_t)a.st.ngroups * H;
  const int nsb = (int)((npair + 63) / 64);
  const int gs = (int)(blockIdx.x % nsb);
  const int cb = (int)(blockIdx.x / nsb);
  const int64_t pid = (int64_t)gs * 64 + lane;
  const bool valid = pid < npair;                // uniform per wave except in the last group block
  const int h = (int)(pid % H);
  const int c = valid ? (int)(pid / H) : 0;
  const int chunk = cb * kBwdWaves + wave;
  const int s = a.st.s;
  const int64_t base = (int64_t)(c / s) * B * s + c % s;
  float acc[RH][B];
#pragma unroll
  for (int rr = 0; rr < RH; ++rr)
#pragma unroll
    for (int k = 0; k < B; ++k) acc[rr][k] = 0.0f;
  if (valid) {
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
    const int64_t r0 = (int64_t)chunk * a.rpc;
    const int64_t r1 = r0 + a.rpc < a.rows ? r0 + a.rpc : a.rows;
    const TG* gin = static_cast<const TG*>(a.gin) + base;
    const TX* xin = static_cast<const TX*>(a.xin) + base;
    TO* out = static_cast<TO*>(a.out) + base;
    const bool v1 = vec1_ok<B>() && a.vec1;
    for (int64_t row = r0; row < r1; ++row) {
      const TG* gr = gin + row * a.ldg;
      const TX* xr = xin + row * a.ldx;
      float g[B], v[B];
      if (v1) {
        ld_vec<B, TG>(gr, g);
        ld_vec<B, TX>(xr, v);
#pragma unroll
        for (int j = 0; j < B; ++j) v[j] *= xs[j];
      } else {
#pragma unroll
        for (int j = 0; j < B; ++j) {
          g[j] = ld_t<TG>(gr, j * s);
          v[j] = ld_t<TX>(xr, j * s) * xs[j];
        }
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
        float o4[RH];
#pragma unroll
        for (int kk = 0; kk < RH; ++kk) {
          const int k = h * RH + kk;
          float o = 0.0f;
#pragma unroll
          for (int r = 0; r < B; ++r) o = fmaf(blk[r][kk], g[r], o);
          o4[kk] = k < B ? o * os[kk] : 0.0f;
        }
        if constexpr (RH == 4) {
          if (v1) {
            st_vec4<TO>(orow + h * RH, o4);
            continue;
          }
        }
#pragma unroll
        for (int kk = 0; kk < RH; ++kk) {
          const int k = h * RH + kk;
          if (k < B) st_t<TO>(orow, k * s, o4[kk]);
        }
      }
    }
  }
  // fixed-order sum over the workgroup's row chunks: wave 0 adds waves 1, 2, ... in order
  if (wave > 0) {
#pragma unroll
    for (int rr = 0; rr < RH; ++rr)
#pragma unroll
      for (int k = 0; k < B; ++k) red[wave - 1][rr * B + k][lane] = acc[rr][k];
  }
  __syncthreads();
  if (wave == 0 && valid) {
#pragma unroll
    for (int w = 0; w < kBwdWaves - 1; ++w)
#pragma unroll
      for (int rr = 0; rr < RH; ++rr)
#pragma unroll
        for (int k = 0; k < B; ++k) acc[rr][k] += red[w][rr * B + k][lane];
    float* pp = a.partial + (int64_t)cb * a.n_blk + a.st.blk_off + (int64_t)c * B * B;
#pragma unroll
    for (int rr = 0; rr < RH; ++rr) {
      const int r = h * RH + rr;
      if (r < B) {
#pragma unroll
        for (int k = 0; k < B; ++k) pp[r * B + k] = acc[rr][k];
      }
    }
  }
}

// The last two stages in one backward launch.  With radices BA (stage m-2,
// digit stride BB) and BB (stage m-1, stride 1), their groups live in units
// of BA * BB consecutive coordinates c = U u + BB a + b (U = BA * BB): stage
// m-2 mixes a (group BB u + b), stage m-1 mixes b (group BA u + a).  A wave
// owns 64 / U units over a chunk of rows, lane U v + BB a + b owning
// coordinate c of its v-th unit, and per row:
//   x_{m-1}[a,b] = sum_k B_{m-2}[a][k] x_{m-2}[k,b]     (recomputed: the
//                                                        forward never stores it)
//   g_{m-1}[a,b] = sum_r B_{m-1}[r][b] dy[a,r]
//   g_{m-2}[a,b] = sum_r B_{m-2}[r][a] g_{m-1}[r,b]
// with the gradient rows dB_{m-1}[BA u+a][b][.] += dy[a,b] x_{m-1}[a,.] and
// dB_{m-2}[BB u+b][a][.] += g_{m-1}[a,b] x_{m-2}[.,b] in registers.  The
// values of a column (same b) or a row (same a) of a unit reach the lane
// through the wave's own LDS slots (two 16-byte words for radix-8 rows and
// columns).  Against two stage launches it reads x_{m-2} and dy once and
// writes g_{m-2} once, and the forward saves writing x_{m-1}.  Rows are
// taken kPairRows at a time so that their loads are in flight together.
constexpr int kPairRows = 4;

template <int N>
__device__ __forceinline__ void read_n(const float* p, float (&v)[N]) {
  if constexpr (N == 8) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = p[k];
  }
}

template <int BA, int BB, typename TB, typename TX, typename TG, typename TO>
__global__ void __launch_bounds__(kBwdThreads, 3) vjp_bwd_pair_kernel(VjpArgs a) {
  constexpr int U = BA * BB;
  constexpr int UPW = 64 / U;    // units per wave
  __shared__ float red[kBwdWaves - 1][BA + BB][64];
  // per wave and row in flight: x_{m-2} by column (b-major), x_{m-1} and dy
  // by row (a-major), g_{m-1} by column
  __shared__ __align__(16) float xch[kBwdWaves][kPairRows][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nunit = a.d / U;
  const int64_t nset = (nunit + UPW - 1) / UPW;   // unit sets (one per wave and chunk)
  const int64_t set = (int64_t)blockIdx.x % nset;
  const int cb = (int)((int64_t)blockIdx.x / nset);
  const int chunk = cb * kBwdWaves + wave;
  const int v = lane / U, li = lane - v * U;
  const int64_t unit = set * UPW + v;
  // lanes past the last unit only pass values along (with one unit per
  // wave, every lane has one)
  const bool valid = UPW == 1 || (v < UPW && unit < nunit);
  // lanes without a unit read unit 0's slots and write only to their own
  // lane's slot, which no unit uses (every index below stays under 64)
  const int ia = valid ? li / BB : 0, ib = valid ? li - (li / BB) * BB : 0;
  const int ubase = valid ? v * U : 0;
  const int tl = valid ? ubase + ib * BA + ia : lane;   // the lane's slot in a b-major unit
  const int64_t c = valid ? unit * U + li : 0;
  const int64_t g0 = valid ? unit * BB + ib : 0;  // stage m-2 group
  const int64_t g1 = valid ? unit * BA + ia : 0;  // stage m-1 group
  float brow[BA], bcol[BA], b1col[BB];
  {
    const TB* p0 = static_cast<const TB*>(a.blocks) + a.st.blk_off + g0 * BA * BA;
    const TB* p1 = static_cast<const TB*>(a.blocks) + a.st2.blk_off + g1 * BB * BB;
    const float s0 = sizeof(TB) == 1 ? a.scales[a.st.grp_off + g0] : 1.0f;
    const float s1 = sizeof(TB) == 1 ? a.scales[a.st2.grp_off + g1] : 1.0f;
#pragma unroll
    for (int k = 0; k < BA; ++k) {
      brow[k] = coef_at<TB>(p0, ia * BA + k) * s0;
      bcol[k] = coef_at<TB>(p0, k * BA + ia) * s0;
    }
#pragma unroll
    for (int k = 0; k < BB; ++k) b1col[k] = coef_at<TB>(p1, k * BB + ib) * s1;
  }
  const float xs = a.x_sign ? (float)a.signs[c] : 1.0f;
  const float os = a.o_sign ? (float)a.signs[c] : 1.0f;
  float acc1[BB], acc0[BA];
#pragma unroll
  for (int k = 0; k < BB; ++k) acc1[k] = 0.0f;
#pragma unroll
  for (int k = 0; k < BA; ++k) acc0[k] = 0.0f;
  const int64_t r0 = (int64_t)chunk * a.rpc;
  const int64_t r1 = r0 + a.rpc < a.rows ? r0 + a.rpc : a.rows;
  const TX* xin = static_cast<const TX*>(a.xin) + c;
  const TG* gin = static_cast<const TG*>(a.gin) + c;
  TO* out = static_cast<TO*>(a.out);
  float(*buf)[4][64] = xch[wave];
  // the wave's own LDS writes before its cross-lane reads of them
  auto lds_wait = [] {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
  };
  for (int64_t row0 = r0; row0 < r1; row0 += kPairRows) {
    float xv[kPairRows], gv[kPairRows];
#pragma unroll
    for (int i = 0; i < kPairRows; ++i) {
      // rows past the chunk re-read its last row; their results are dropped
      const int64_t row = row0 + i < r1 ? row0 + i : r1 - 1;
      xv[i] = valid ? ld_t<TX>(xin + row * a.ldx, 0) * xs : 0.0f;
      gv[i] = valid ? ld_t<TG>(gin + row * a.ldg, 0) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kPairRows; ++i) {
      buf[i][0][tl] = xv[i];
      buf[i][2][lane] = gv[i];
    }
    lds_wait();
    float xcol[kPairRows][BA];
#pragma unroll
    for (int i = 0; i < kPairRows; ++i) {
      read_n<BA>(&buf[i][0][ubase + ib * BA], xcol[i]);
      float s1 = 0.0f;
#pragma unroll
      for (int k = 0; k < BA; ++k) s1 = fmaf(brow[k], xcol[i][k], s1);
      buf[i][1][lane] = s1;
    }
    lds_wait();
    float g1v[kPairRows];
#pragma unroll
    for (int i = 0; i < kPairRows; ++i) {
      const bool live = valid && row0 + i < r1;
      float x1row[BB], g2row[BB];
      read_n<BB>(&buf[i][1][ubase + ia * BB], x1row);
      read_n<BB>(&buf[i][2][ubase + ia * BB], g2row);
      float g = 0.0f;
#pragma unroll
      for (int k = 0; k < BB; ++k) {
        if (live) acc1[k] = fmaf(gv[i], x1row[k], acc1[k]);
        g = fmaf(b1col[k], g2row[k], g);
      }
      g1v[i] = g;
      buf[i][3][tl] = g;
    }
    lds_wait();
#pragma unroll
    for (int i = 0; i < kPairRows; ++i) {
      const bool live = valid && row0 + i < r1;
      float g1col[BA];
      read_n<BA>(&buf[i][3][ubase + ib * BA], g1col);
      float o = 0.0f;
#pragma unroll
      for (int k = 0; k < BA; ++k) {
        if (live) acc0[k] = fmaf(g1v[i], xcol[i][k], acc0[k]);
        o = fmaf(bcol[k], g1col[k], o);
      }
      if (live && out != nullptr) st_t<TO>(out + (row0 + i) * a.ldo, c, o * os);
    }
    // the next rows overwrite this wave's slots only after these reads
    lds_wait();
  }
  // fixed-order sum over the workgroup's row chunks, as in vjp_bwd_kernel
  if (wave > 0) {
#pragma unroll
    for (int k = 0; k < BB; ++k) red[wave - 1][k][lane] = acc1[k];
#pragma unroll
    for (int k = 0; k < BA; ++k) red[wave - 1][BB + k][lane] = acc0[k];
  }
  __syncthreads();
  if (wave == 0 && valid) {
#pragma unroll
    for (int w = 0; w < kBwdWaves - 1; ++w) {
#pragma unroll
      for (int k = 0; k < BB; ++k) acc1[k] += red[w][k][lane];
#pragma unroll
      for (int k = 0; k < BA; ++k) acc0[k] += red[w][BB + k][lane];
    }
    float* pp = a.partial + (int64_t)cb * a.n_blk;
#pragma unroll
    for (int k = 0; k < BB; ++k) pp[a.st2.blk_off + g1 * BB * BB + ib * BB + k] = acc1[k];
#pragma unroll
    for (int k = 0; k < BA; ++k) pp[a.st.blk_off + g0 * BA * BA + ia * BA + k] = acc0[k];
  }
}

// Last-stage pairs compiled in (radices of stages m-2, m-1).
__host__ __device__ constexpr bool pair_compiled(int ba, int bb) {
  return (ba == 8 && bb == 8) || (ba == 5 && bb == 2) || (ba == 3 && bb == 3);
}

__global__ void __launch_bounds__(kVjpThreads) vjp_reduce_kernel(const float* partial, int nslot, int64_t n_blk,
                                                                 float* dblocks) {
  const int64_t i = (int64_t)blockIdx.x * kVjpThreads + threadIdx.x;
  if (i >= n_blk) return;
  float acc = 0.0f;
  for (int sl = 0; sl < nslot; ++sl) acc += partial[(int64_t)sl * n_blk + i];
  dblocks[i] = acc;
}

int vjp_chunks(const Plan& pl, int64_t rows) {
  int64_t ng = pl.d;
  for (int t = 0; t < pl.m; ++t)
    if (pl.d / pl.radix[t] < ng) ng = pl.d / pl.radix[t];
  int64_t n = (kVjpTargetThreads + ng - 1) / ng;
  if (n > rows) n = rows;
  if (n < 1) n = 1;
  // whole backward workgroups (chunks past the last row are empty)
  return (int)((n + kBwdWaves - 1) / kBwdWaves * kBwdWaves);
}

template <int B, typename TB>
hipError_t launch_stage(bool fwd, const VjpArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.st.ngroups * a.nchunk;
  const int64_t grid = fwd ? (n + kVjpThreads - 1) / kVjpThreads
                           : ((int64_t)a.st.ngroups * bwd_split<B>() + 63) / 64 * (a.nchunk / kBwdWaves);
  const dim3 blk(fwd ? kVjpThreads : kBwdThreads);
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
      case 0: hipLaunchKernelGGL((vjp_bwd_kernel<B, TB, F, F, F>), dim3((unsigned)grid), blk, 0, st, a); break;
      case 5: hipLaunchKernelGGL((vjp_bwd_kernel<B, TB, H16, F, H16>), dim3((unsigned)grid), blk, 0, st, a); break;
      case 4: hipLaunchKernelGGL((vjp_bwd_kernel<B, TB, H16, F, F>), dim3((unsigned)grid), blk, 0, st, a); break;
      case 2: hipLaunchKernelGGL((vjp_bwd_kernel<B, TB, F, H16, F>), dim3((unsigned)grid), blk, 0, st, a); break;
      case 7: hipLaunchKernelGGL((vjp_bwd_kernel<B, TB, H16, H16, H16>), dim3((unsigned)grid), blk, 0, st, a); break;
      case 6: hipLaunchKernelGGL((vjp_bwd_kernel<B, TB, H16, H16, F>), dim3((unsigned)grid), blk, 0, st, a); break;
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

template <int BA, int BB, typename TB>
hipError_t launch_pair_ab(const VjpArgs& a, hipStream_t st) {
  constexpr int U = BA * BB, UPW = 64 / U;
  const int64_t nset = (a.d / U + UPW - 1) / UPW;
  const dim3 grid((unsigned)(nset * (a.nchunk / kBwdWaves)));
  using F = float;
  using H16 = uint16_t;
  // x_{m-2} and the output are the caller's rows only when m = 2
  if (!a.x_bf16 && !a.g_bf16 && !a.o_bf16)
    hipLaunchKernelGGL((vjp_bwd_pair_kernel<BA, BB, TB, F, F, F>), grid, dim3(kBwdThreads), 0, st, a);
  else if (!a.x_bf16 && a.g_bf16 && !a.o_bf16)
    hipLaunchKernelGGL((vjp_bwd_pair_kernel<BA, BB, TB, F, H16, F>), grid, dim3(kBwdThreads), 0, st, a);
  else if (a.x_bf16 && a.g_bf16 && a.o_bf16)
    hipLaunchKernelGGL((vjp_bwd_pair_kernel<BA, BB, TB, H16, H16, H16>), grid, dim3(kBwdThreads), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename TB>
hipError_t launch_pair(const VjpArgs& a, hipStream_t st) {
  if (a.st.b == 8 && a.st2.b == 8) return launch_pair_ab<8, 8, TB>(a, st);
  if (a.st.b == 5 && a.st2.b == 2) return launch_pair_ab<5, 2, TB>(a, st);
  if (a.st.b == 3 && a.st2.b == 3) return launch_pair_ab<3, 3, TB>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_pair_any(DT bdt, const VjpArgs& a, hipStream_t st) {
  if (bdt == DT::F32) return launch_pair<float>(a, st);
  if (bdt == DT::BF16) return launch_pair<uint16_t>(a, st);
  return launch_pair<int8_t>(a, st);
}

}  // namespace

int64_t vjp_workspace_bytes(const Plan& pl, int64_t rows) {
  for (int t = 0; t < pl.m; ++t)
    if (pl.radix[t] > 8) return -1;
  // at most (m + 1) + 16 fp32 values per row element: keep 4x that in int64
  if (rows > (INT64_MAX / 256) / pl.d) return -1;
  const int64_t acts = (int64_t)(pl.m - 1) * rows * pl.d;
  const int64_t gbuf = (pl.m > 1 ? 2 : 0) * rows * pl.d;
  const int64_t part = (int64_t)(vjp_chunks(pl, rows) / kBwdWaves) * pl.n_blk;
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

  // last two stages of a compiled-in pair: one fused backward launch, which
  // recomputes x_{m-1} itself
  const bool pair = pl.m >= 2 && pair_compiled(pl.radix[pl.m - 2], pl.radix[pl.m - 1]);
  // forward: x_{t+1} = S_t x_t for t = 0 .. m-2 (m-3 with the fused pair)
  for (int t = 0; t + 1 < pl.m - (pair ? 1 : 0); ++t) {
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
  int t_top = pl.m - 1;
  if (pair) {
    VjpArgs a = base;
    const int t = pl.m - 2;
    a.st = stage_of(t);
    a.st2 = stage_of(t + 1);
    a.gin = dy;
    a.ldg = lddy;
    a.g_bf16 = bf;
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
      a.out = gbuf + rd;   // the buffer the step for stage m-2 writes (step 1: gbuf[1])
      a.ldo = pl.d;
    }
    hipError_t e = launch_pair_any(bdt, a, stream);
    if (e != hipSuccess) return e;
    t_top = pl.m - 3;
  }
  for (int t = t_top; t >= 0; --t) {
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
    if (a.st.s == 1) {
      // stride 1: a group's coordinates are contiguous; vector accesses need
      // every row of the three arrays to start on their alignment
      const int xb = a.x_bf16 ? 2 : 4, gb = a.g_bf16 ? 2 : 4, ob = a.o_bf16 ? 2 : 4;
      auto al = [](const void* ptr, int64_t ld, int eb, int bytes) {
        return reinterpret_cast<uintptr_t>(ptr) % 16 == 0 && (ld * eb) % bytes == 0;
      };
      const int gbytes = a.st.b * 4;   // a group's fp32 bytes: 32 or 16
      a.vec1 = al(a.xin, a.ldx, xb, a.st.b * xb < 16 ? a.st.b * xb : 16) &&
               al(a.gin, a.ldg, gb, a.st.b * gb < 16 ? a.st.b * gb : 16) &&
               al(a.out, a.ldo, ob, 4 * ob) && gbytes >= 16;
    }
    hipError_t e = launch_stage_any(false, bdt, a, stream);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = (pl.n_blk + kVjpThreads - 1) / kVjpThreads;
  hipLaunchKernelGGL(vjp_reduce_kernel, dim3((unsigned)grid), dim3(kVjpThreads), 0, stream, part, nchunk / kBwdWaves,
                     pl.n_blk, dblocks);
  return hipGetLastError();
}

}  // namespace harp
