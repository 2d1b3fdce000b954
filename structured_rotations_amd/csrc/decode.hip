// Small-batch (per-token decode) apply: y = S_{m-1} ... S_0 D_s x for 1 to a
// few hundred rows, latency first.
//
// HARP technical summary (gist.science 2605.29843), §2.1: the transform is a
// product of block-diagonal stages, stage t mixing digit t of the mixed-radix
// row index; §4 quotes its cost per generated token.  At one row the
// throughput kernels leave all but one or a few CUs idle and walk the stages
// through a chain of dependent coefficient fetches.  Here the digits are cut
// into two runs, [0, k) and [k, m): within a run the row splits into
// independent sub-problems (the elements that share the digits outside the
// run), so each run is one launch of many small workgroups.  A workgroup
// issues every load it needs (its rows' elements and the blocks of every stage
// of the run) at once, then runs the stages out of LDS and writes its result:
// one memory round trip per launch.  The first launch leaves fp32 rows in a
// caller-provided workspace for the second; a schedule small enough for one
// workgroup per row block runs as a single launch.
//
// Element h of sub-problem n (0 <= h < P, P = prod of the run's radices) sits
// at row position (n / inner) * (P * inner) + h * inner + n % inner, where
// inner is the product of the radices after the run.  Digit t of the run has
// stride s_t = prod of the run's radices after t inside the sub-problem and
// s_t * inner inside the row.
#include "common.h"
#include "kernels.h"

namespace harp {

namespace {

struct DecStage {
  int b;        // radix
  int s;        // digit stride inside the sub-problem
  int S;        // digit stride inside the row
  int cof;      // first staged coefficient of the stage (LDS, elements)
  int sof;      // first staged int8 scale of the stage (LDS, floats)
  int blk_off;  // first coefficient of the stage in the block array
  int grp_off;  // first group of the stage
};

struct DecParams {
  int P;          // elements per sub-problem
  int inner;      // product of the radices after the run
  int nsub;       // sub-problems per row (d / P)
  int ns;         // consecutive sub-problems per workgroup
  int R;          // rows per workgroup
  int nchunks;    // ceil(nsub / ns)
  int nst;        // stages in the run
  int transpose;  // inverse: transposed blocks (stages already in reverse order)
  int sign_in;    // multiply the input by the sign
  int sign_out;   // multiply the output by the sign
  int ncoef;      // staged coefficients (all stages)
  int nscale;     // staged int8 scales (all stages)
  DecStage st[kMaxStagesDev];
  const void* blocks;
  const float* scales;
  const int8_t* signs;
  const void* x;
  int64_t ldx;
  void* y;
  int64_t ldy;
  int64_t rows;
};

constexpr int kDecThreads = 256;
constexpr int64_t kDecodeRowsMax = 128;   // more rows go to the throughput row kernels
constexpr int kDecBatch = 16;    // loads in flight per thread

__device__ __forceinline__ int sub_pos(const DecParams& p, int n, int h) {
  return (n / p.inner) * (p.P * p.inner) + h * p.inner + n % p.inner;
}

// Flat index over (r, jj, h) in the order that makes neighbouring threads touch
// neighbouring row positions: jj fastest when sub-problems interleave
// (inner > 1), h fastest when each sub-problem is contiguous.
struct RJH {
  int r, jj, h;
};
__device__ __forceinline__ RJH split_rjh(const DecParams& p, int f) {
  const int per_row = p.ns * p.P;
  RJH o;
  o.r = f / per_row;
  const int rem = f - o.r * per_row;
  if (p.inner > 1) {
    o.h = rem / p.ns;
    o.jj = rem - o.h * p.ns;
  } else {
    o.jj = rem / p.P;
    o.h = rem - o.jj * p.P;
  }
  return o;
}

template <typename T>
__device__ __forceinline__ float load_elem(const T* ptr);
template <>
__device__ __forceinline__ float load_elem<float>(const float* ptr) { return *ptr; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* ptr) { return bf16_to_f32(*ptr); }

template <typename T>
__device__ __forceinline__ void store_elem(T* ptr, float v);
template <>
__device__ __forceinline__ void store_elem<float>(float* ptr, float v) { *ptr = v; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t* ptr, float v) { *ptr = (uint16_t)f32_to_bf16_rne(v); }

template <typename TB>
__device__ __forceinline__ float coef_val(TB c);
template <>
__device__ __forceinline__ float coef_val<float>(float c) { return c; }
template <>
__device__ __forceinline__ float coef_val<uint16_t>(uint16_t c) { return bf16_to_f32(c); }
template <>
__device__ __forceinline__ float coef_val<int8_t>(int8_t c) { return (float)c; }

// Block index of group q (0 <= q < P / b) of a stage inside sub-problem n.
__device__ __forceinline__ int group_of(const DecParams& p, int b, int s, int S, int n, int q) {
  const int hb = (q / s) * (b * s) + q % s;
  const int pos = sub_pos(p, n, hb);
  return (pos / (b * S)) * S + pos % S;
}

// Raw bits of a stored coefficient, and back.
__device__ __forceinline__ uint32_t coef_bits(const float* b, int64_t i) { return __float_as_uint(b[i]); }
__device__ __forceinline__ uint32_t coef_bits(const uint16_t* b, int64_t i) { return b[i]; }
__device__ __forceinline__ uint32_t coef_bits(const int8_t* b, int64_t i) { return (uint8_t)b[i]; }
__device__ __forceinline__ void coef_put(float* c, int i, uint32_t v) { c[i] = __uint_as_float(v); }
__device__ __forceinline__ void coef_put(uint16_t* c, int i, uint32_t v) { c[i] = (uint16_t)v; }
__device__ __forceinline__ void coef_put(int8_t* c, int i, uint32_t v) { c[i] = (int8_t)(uint8_t)v; }

// The stage (in run order) whose staged range holds idx: a uniform loop over
// the stages with per-lane selects, so the descriptors stay in scalar loads.
struct StSel {
  int b, s, S, off, blk_off, grp_off;
};
__device__ __forceinline__ StSel stage_at(const DecParams& p, int idx, bool scales) {
  StSel r{1, 1, 1, 0, 0, 0};
  for (int i = 0; i < p.nst; ++i) {
    const DecStage& q = p.st[i];
    if (idx >= (scales ? q.sof : q.cof)) r = StSel{q.b, q.s, q.S, scales ? q.sof : q.cof, q.blk_off, q.grp_off};
  }
  return r;
}

template <typename TIN, typename TOUT, typename TB>
__global__ void __launch_bounds__(kDecThreads) decode_kernel(DecParams p) {
  extern __shared__ __align__(16) char lds[];
  const int tile = p.R * p.ns * p.P;
  float* buf0 = reinterpret_cast<float*>(lds);
  float* buf1 = buf0 + tile;
  float* bscale = buf1 + tile;
  TB* coef = reinterpret_cast<TB*>(bscale + p.nscale);

  const int chunk = blockIdx.x % p.nchunks;
  const int64_t row0 = (int64_t)(blockIdx.x / p.nchunks) * p.R;
  const int n0 = chunk * p.ns;
  const int tid = threadIdx.x;
  const TIN* x = static_cast<const TIN*>(p.x);
  const TB* blocks = static_cast<const TB*>(p.blocks);

  // Every load of the workgroup, kDecBatch per thread in flight at a time:
  // [0, tile) rows, [tile, tile + ncoef) blocks, then the int8 scales.
  const int c_end = tile + p.ncoef;
  const int total = c_end + p.nscale;
  for (int base = 0; base < total; base += kDecThreads * kDecBatch) {
    uint32_t v[kDecBatch];
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      const int f = base + u * kDecThreads + tid;
      v[u] = 0u;
      if (f < tile) {
        const RJH q = split_rjh(p, f);
        const int n = n0 + q.jj;
        if (row0 + q.r < p.rows && n < p.nsub) {
          const int pos = sub_pos(p, n, q.h);
          float e = load_elem<TIN>(x + (row0 + q.r) * p.ldx + pos);
          if (p.sign_in) e *= (float)p.signs[pos];
          v[u] = __float_as_uint(e);
        }
      } else if (f < c_end) {
        const int idx = f - tile;
        const StSel st = stage_at(p, idx, false);
        const int bb = st.b * st.b;
        const int slot = (idx - st.off) / bb;
        const int w = (idx - st.off) - slot * bb;
        const int per = p.P / st.b;
        const int jj = slot / per;
        const int n = n0 + jj;
        if (n < p.nsub) {
          const int c = group_of(p, st.b, st.s, st.S, n, slot - jj * per);
          v[u] = coef_bits(blocks, st.blk_off + (int64_t)c * bb + w);
        }
      } else if (f < total) {
        const int idx = f - c_end;
        const StSel st = stage_at(p, idx, true);
        const int per = p.P / st.b;
        const int slot = idx - st.off;
        const int jj = slot / per;
        const int n = n0 + jj;
        if (n < p.nsub) v[u] = __float_as_uint(p.scales[st.grp_off + group_of(p, st.b, st.s, st.S, n, slot - jj * per)]);
      }
    }
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      const int f = base + u * kDecThreads + tid;
      if (f < tile) {
        const RJH q = split_rjh(p, f);
        buf0[(q.r * p.ns + q.jj) * p.P + q.h] = __uint_as_float(v[u]);
      } else if (f < c_end) {
        coef_put(coef, f - tile, v[u]);
      } else if (f < total) {
        bscale[f - c_end] = __uint_as_float(v[u]);
      }
    }
  }
  __syncthreads();

  float* src = buf0;
  float* dst = buf1;
  for (int i = 0; i < p.nst; ++i) {
    const DecStage st = p.st[i];
    const int b = st.b, s = st.s, per = p.P / b;
    for (int e = tid; e < tile; e += kDecThreads) {
      const int rj = e / p.P;            // r * ns + jj
      const int h = e - rj * p.P;
      const int jj = rj % p.ns;
      const int dig = (h / s) % b;
      const int hb = h - dig * s;
      const int slot = jj * per + (h / (b * s)) * s + h % s;
      const TB* cb = coef + st.cof + slot * b * b;
      const float* xs = src + rj * p.P + hb;
      float acc = 0.0f;
      if (p.transpose) {
        for (int k = 0; k < b; ++k) acc = fmaf(coef_val<TB>(cb[k * b + dig]), xs[k * s], acc);
      } else {
        for (int k = 0; k < b; ++k) acc = fmaf(coef_val<TB>(cb[dig * b + k]), xs[k * s], acc);
      }
      if (sizeof(TB) == 1) acc *= bscale[st.sof + slot];
      dst[e] = acc;
    }
    __syncthreads();
    float* t = src;
    src = dst;
    dst = t;
  }

  TOUT* y = static_cast<TOUT*>(p.y);
  for (int f = tid; f < tile; f += kDecThreads) {
    const RJH q = split_rjh(p, f);
    const int n = n0 + q.jj;
    if (row0 + q.r >= p.rows || n >= p.nsub) continue;
    const int pos = sub_pos(p, n, q.h);
    float v = src[(q.r * p.ns + q.jj) * p.P + q.h];
    if (p.sign_out) v *= (float)p.signs[pos];
    store_elem<TOUT>(y + (row0 + q.r) * p.ldy + pos, v);
  }
}

int esize(DT t) { return t == DT::F32 ? 4 : (t == DT::BF16 ? 2 : 1); }

// LDS bytes of a run with R rows and ns sub-problems per workgroup.
int64_t run_lds(const Plan& pl, int t0, int t1, int64_t P, int R, int ns, DT bdt) {
  int64_t sum_b = 0, ngroups = 0;
  for (int t = t0; t < t1; ++t) {
    sum_b += pl.radix[t];
    ngroups += P / pl.radix[t];
  }
  int64_t bytes = 2 * (int64_t)R * ns * P * 4;
  if (bdt == DT::I8) bytes += (int64_t)ns * ngroups * 4;
  bytes += (int64_t)ns * P * sum_b * esize(bdt);
  return bytes;
}

constexpr int64_t kDecLds = 64 * 1024;

struct Run {
  int t0, t1;
  int64_t P, inner;
};

template <typename TIN, typename TOUT, typename TB>
hipError_t launch_run(const DecParams& p, int grid, int lds, hipStream_t st) {
  auto kern = decode_kernel<TIN, TOUT, TB>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kDecThreads), lds, st, p);
  return hipGetLastError();
}

template <typename TIN, typename TOUT>
hipError_t launch_run_b(DT bdt, const DecParams& p, int grid, int lds, hipStream_t st) {
  if (bdt == DT::F32) return launch_run<TIN, TOUT, float>(p, grid, lds, st);
  if (bdt == DT::BF16) return launch_run<TIN, TOUT, uint16_t>(p, grid, lds, st);
  return launch_run<TIN, TOUT, int8_t>(p, grid, lds, st);
}

// ---------------------------------------------------------------------------
// The same run with its radices fixed at compile time: every index is a
// multiply or shift, each stage's blocks arrive as 16-byte loads (a run that
// starts at digit 0 needs group q * inner + n of each stage, one contiguous
// block each; a run that ends at the last digit needs groups n * P / b + q,
// one contiguous slab), and a workgroup handles one sub-problem.

struct DecFixed {
  int inner;      // product of the radices after the run (1 for the last run)
  int nsub;       // sub-problems per row
  int R;          // rows per workgroup
  int first;      // the run starts at digit 0
  int inverse;    // transposed blocks, stages in reverse order
  int sign_in, sign_out;
  int blk_off[kMaxStagesDev];   // per digit of the run (run order, not application order)
  int grp_off[kMaxStagesDev];
  const void* blocks;
  const float* scales;
  const int8_t* signs;
  const void* x;
  int64_t ldx;
  void* y;
  int64_t ldy;
  int64_t rows;
};

template <int... Bs>
struct RunT {
  static constexpr int n = sizeof...(Bs);
  static constexpr int b[n] = {Bs...};
  static constexpr int P = (Bs * ...);
  static constexpr int sum_b = (Bs + ...);
  static constexpr int stride(int i) {
    int v = 1;
    for (int u = i + 1; u < n; ++u) v *= b[u];
    return v;
  }
  static constexpr int coef_off(int i) {   // staged coefficients before digit i
    int v = 0;
    for (int u = 0; u < i; ++u) v += P * b[u];
    return v;
  }
  static constexpr int scale_off(int i) {
    int v = 0;
    for (int u = 0; u < i; ++u) v += P / b[u];
    return v;
  }
};

constexpr int kFixRows = 8;

template <typename TB, int B, int S, int P>
__device__ __forceinline__ void fixed_stage(const float* src, float* dst, const TB* cb, const float* bsc, int tile,
                                            bool inv) {
  for (int e = threadIdx.x; e < tile; e += kDecThreads) {
    const int r = e / P;
    const int h = e - r * P;
    const int dig = (h / S) % B;
    const int hb = h - dig * S;
    const int q = (h / (B * S)) * S + h % S;
    const TB* c = cb + q * B * B;
    const float* xs = src + r * P + hb;
    float acc = 0.0f;
    if (inv) {
#pragma unroll
      for (int k = 0; k < B; ++k) acc = fmaf(coef_val<TB>(c[k * B + dig]), xs[k * S], acc);
    } else {
#pragma unroll
      for (int k = 0; k < B; ++k) acc = fmaf(coef_val<TB>(c[dig * B + k]), xs[k * S], acc);
    }
    if (sizeof(TB) == 1) acc *= bsc[q];
    dst[e] = acc;
  }
}

template <typename TB, typename Rn, int I>
__device__ __forceinline__ void fixed_stage_at(const float* src, float* dst, const TB* coef, const float* bsc,
                                               int tile, bool inv) {
  fixed_stage<TB, Rn::b[I], Rn::stride(I), Rn::P>(src, dst, coef + Rn::coef_off(I), bsc + Rn::scale_off(I), tile,
                                                 inv);
}

// Applies digit I of the run (forward: I = 0, 1, ...; inverse: I = n-1, ...),
// one LDS buffer to the other, with a barrier after each stage.
template <typename TB, typename Rn, int I>
__device__ __forceinline__ float* fixed_stages(float* src, float* dst, const TB* coef, const float* bsc, int tile,
                                               bool inv) {
  if constexpr (I == Rn::n) {
    return src;
  } else {
    fixed_stage_at<TB, Rn, I>(src, dst, coef, bsc, tile, false);
    __syncthreads();
    return fixed_stages<TB, Rn, I + 1>(dst, src, coef, bsc, tile, inv);
  }
}
template <typename TB, typename Rn, int I>
__device__ __forceinline__ float* fixed_stages_inv(float* src, float* dst, const TB* coef, const float* bsc, int tile) {
  if constexpr (I < 0) {
    return src;
  } else {
    fixed_stage_at<TB, Rn, I>(src, dst, coef, bsc, tile, true);
    __syncthreads();
    return fixed_stages_inv<TB, Rn, I - 1>(dst, src, coef, bsc, tile);
  }
}

// Byte offset, in the block array, of 16-byte chunk k of digit I's staged
// blocks, and in LDS; false if k is past digit I's range.
template <typename TB, typename Rn, int I>
__device__ __forceinline__ void chunk_src(const DecFixed& p, int n, int k, int64_t* src_byte) {
  constexpr int b = Rn::b[I];
  constexpr int esz = (int)sizeof(TB);
  constexpr int begin = Rn::coef_off(I) * esz / 16;
  const int kk = k - begin;
  if (p.first) {
    // chunks per block: the host takes this kernel for a run that starts at
    // digit 0 only when each block is whole 16-byte chunks; the guard only
    // keeps the constant nonzero in instantiations that never get here
    constexpr int cpb = b * b * esz / 16 > 0 ? b * b * esz / 16 : 1;
    const int q = kk / cpb;
    const int w = kk - q * cpb;
    *src_byte = ((int64_t)p.blk_off[I] + (int64_t)(q * p.inner + n) * (b * b)) * esz + w * 16;
  } else {
    *src_byte = ((int64_t)p.blk_off[I] + (int64_t)n * (Rn::P * b)) * esz + (int64_t)kk * 16;
  }
}
template <typename TB, typename Rn, int I>
__device__ __forceinline__ int64_t chunk_byte(const DecFixed& p, int n, int k) {
  if constexpr (I + 1 < Rn::n) {
    constexpr int next = Rn::coef_off(I + 1) * (int)sizeof(TB) / 16;
    if (k >= next) return chunk_byte<TB, Rn, I + 1>(p, n, k);
  }
  int64_t off;
  chunk_src<TB, Rn, I>(p, n, k, &off);
  return off;
}
template <typename Rn, int I>
__device__ __forceinline__ int scale_index(const DecFixed& p, int n, int j) {
  if constexpr (I + 1 < Rn::n) {
    if (j >= Rn::scale_off(I + 1)) return scale_index<Rn, I + 1>(p, n, j);
  }
  constexpr int per = Rn::P / Rn::b[I];
  const int q = j - Rn::scale_off(I);
  return p.grp_off[I] + (p.first ? q * p.inner + n : n * per + q);
}

template <typename TIN, typename TOUT, typename TB, typename Rn>
__global__ void __launch_bounds__(kDecThreads) decode_fixed_kernel(DecFixed p) {
  constexpr int P = Rn::P;
  constexpr int esz = (int)sizeof(TB);
  constexpr int NCH = Rn::coef_off(Rn::n) * esz / 16;   // 16-byte coefficient chunks
  constexpr int NSC = sizeof(TB) == 1 ? Rn::scale_off(Rn::n) : 0;
  constexpr int KC = (NCH + kDecThreads - 1) / kDecThreads;
  constexpr int KS = (NSC + kDecThreads - 1) / kDecThreads;
  constexpr int KD = (kFixRows * P + kDecThreads - 1) / kDecThreads;
  __shared__ __align__(16) float buf[2][kFixRows * P];
  __shared__ __align__(16) unsigned char coef_raw[NCH * 16];
  __shared__ float bsc[NSC > 0 ? NSC : 1];

  const int n = blockIdx.x % p.nsub;
  const int64_t row0 = (int64_t)(blockIdx.x / p.nsub) * p.R;
  const int tile = p.R * P;
  const int tid = threadIdx.x;
  const TIN* x = static_cast<const TIN*>(p.x);
  const unsigned char* braw = static_cast<const unsigned char*>(p.blocks);

  // all loads first (coefficients, scales, rows), then the LDS stores
  u32x4 cv[KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    const int k = j * kDecThreads + tid;
    if (k < NCH) cv[j] = *reinterpret_cast<const u32x4*>(braw + chunk_byte<TB, Rn, 0>(p, n, k));
  }
  float sv[KS > 0 ? KS : 1];
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const int k = j * kDecThreads + tid;
    if (k < NSC) sv[j] = p.scales[scale_index<Rn, 0>(p, n, k)];
  }
  float dv[KD];
#pragma unroll
  for (int j = 0; j < KD; ++j) {
    const int e = j * kDecThreads + tid;
    dv[j] = 0.0f;
    const int r = e / P;
    const int h = e - r * P;
    if (e < tile && row0 + r < p.rows) {
      const int pos = p.first ? h * p.inner + n : n * P + h;
      float v = load_elem<TIN>(x + (row0 + r) * p.ldx + pos);
      if (p.sign_in) v *= (float)p.signs[pos];
      dv[j] = v;
    }
  }
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    const int k = j * kDecThreads + tid;
    if (k < NCH) *reinterpret_cast<u32x4*>(coef_raw + k * 16) = cv[j];
  }
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const int k = j * kDecThreads + tid;
    if (k < NSC) bsc[k] = sv[j];
  }
#pragma unroll
  for (int j = 0; j < KD; ++j) {
    const int e = j * kDecThreads + tid;
    if (e < tile) buf[0][e] = dv[j];
  }
  __syncthreads();

  const TB* coef = reinterpret_cast<const TB*>(coef_raw);
  const float* res = p.inverse ? fixed_stages_inv<TB, Rn, Rn::n - 1>(buf[0], buf[1], coef, bsc, tile)
                               : fixed_stages<TB, Rn, 0>(buf[0], buf[1], coef, bsc, tile, false);

  TOUT* y = static_cast<TOUT*>(p.y);
  for (int e = tid; e < tile; e += kDecThreads) {
    const int r = e / P;
    const int h = e - r * P;
    if (row0 + r >= p.rows) continue;
    const int pos = p.first ? h * p.inner + n : n * P + h;
    float v = res[e];
    if (p.sign_out) v *= (float)p.signs[pos];
    store_elem<TOUT>(y + (row0 + r) * p.ldy + pos, v);
  }
}

template <typename TIN, typename TOUT, typename Rn>
hipError_t launch_fixed_t(DT bdt, const DecFixed& p, int grid, hipStream_t st) {
  if (bdt == DT::F32) hipLaunchKernelGGL((decode_fixed_kernel<TIN, TOUT, float, Rn>), dim3(grid), dim3(kDecThreads), 0, st, p);
  else if (bdt == DT::BF16)
    hipLaunchKernelGGL((decode_fixed_kernel<TIN, TOUT, uint16_t, Rn>), dim3(grid), dim3(kDecThreads), 0, st, p);
  else hipLaunchKernelGGL((decode_fixed_kernel<TIN, TOUT, int8_t, Rn>), dim3(grid), dim3(kDecThreads), 0, st, p);
  return hipGetLastError();
}

template <typename Rn>
hipError_t launch_fixed_io(DT in_dt, DT out_dt, DT bdt, const DecFixed& p, int grid, hipStream_t st) {
  const bool in_f = in_dt == DT::F32, out_f = out_dt == DT::F32;
  if (in_f && out_f) return launch_fixed_t<float, float, Rn>(bdt, p, grid, st);
  if (in_f) return launch_fixed_t<float, uint16_t, Rn>(bdt, p, grid, st);
  if (out_f) return launch_fixed_t<uint16_t, float, Rn>(bdt, p, grid, st);
  return launch_fixed_t<uint16_t, uint16_t, Rn>(bdt, p, grid, st);
}

template <int... Bs>
bool run_is(const Plan& pl, const Run& run) {
  constexpr int want[] = {Bs...};
  if (run.t1 - run.t0 != (int)sizeof...(Bs)) return false;
  for (int i = 0; i < (int)sizeof...(Bs); ++i)
    if (pl.radix[run.t0 + i] != want[i]) return false;
  return true;
}

// Launches the fixed-radix kernel if the run's radices have one and the
// blocks meet its 16-byte layout; *done says whether it did.
hipError_t launch_fixed(const Plan& pl, const Run& run, bool inverse, bool first_launch, bool last_launch,
                        const void* blocks, DT bdt, const float* scales, const int8_t* signs, const void* x,
                        int64_t ldx, DT in_dt, void* y, int64_t ldy, DT out_dt, int64_t rows, hipStream_t stream,
                        bool* done) {
  *done = false;
  const int esz = esize(bdt);
  const bool first = run.t0 == 0;
  if (reinterpret_cast<uintptr_t>(blocks) % 16 != 0) return hipSuccess;
  for (int t = run.t0; t < run.t1; ++t) {
    const int b = pl.radix[t];
    if ((pl.blk_off[t] * esz) % 16 != 0) return hipSuccess;
    if (first ? (b * b * esz) % 16 != 0 : (run.P * b * esz) % 16 != 0) return hipSuccess;
  }
  DecFixed p{};
  p.inner = (int)run.inner;
  p.nsub = (int)(pl.d / run.P);
  p.R = (int)(rows < kFixRows ? rows : kFixRows);
  p.first = first ? 1 : 0;
  p.inverse = inverse ? 1 : 0;
  p.sign_in = (!inverse && first_launch && signs != nullptr) ? 1 : 0;
  p.sign_out = (inverse && last_launch && signs != nullptr) ? 1 : 0;
  for (int i = 0; i < run.t1 - run.t0; ++i) {
    p.blk_off[i] = (int)pl.blk_off[run.t0 + i];
    p.grp_off[i] = (int)pl.grp_off[run.t0 + i];
  }
  p.blocks = blocks;
  p.scales = scales;
  p.signs = signs;
  p.x = x;
  p.ldx = ldx;
  p.y = y;
  p.ldy = ldy;
  p.rows = rows;
  const int64_t grid = (int64_t)p.nsub * ((rows + p.R - 1) / p.R);
  if (grid > 0x7fffffff) return hipSuccess;
  hipError_t e;
  if (run_is<8, 8>(pl, run)) e = launch_fixed_io<RunT<8, 8>>(in_dt, out_dt, bdt, p, (int)grid, stream);
  else if (run_is<8, 5, 2>(pl, run)) e = launch_fixed_io<RunT<8, 5, 2>>(in_dt, out_dt, bdt, p, (int)grid, stream);
  else if (run_is<8, 3, 3, 3>(pl, run)) e = launch_fixed_io<RunT<8, 3, 3, 3>>(in_dt, out_dt, bdt, p, (int)grid, stream);
  else if (run_is<8, 16>(pl, run)) e = launch_fixed_io<RunT<8, 16>>(in_dt, out_dt, bdt, p, (int)grid, stream);
  else return hipSuccess;
  *done = true;
  return e;
}

hipError_t launch_one(const Plan& pl, const Run& run, bool inverse, bool first, bool last,
                      const void* blocks, DT bdt, const float* scales, const int8_t* signs,
                      const void* x, int64_t ldx, DT in_dt, void* y, int64_t ldy, DT out_dt,
                      int64_t rows, hipStream_t stream) {
  if (run.t0 == 0 || run.t1 == pl.m) {
    bool done = false;
    hipError_t e = launch_fixed(pl, run, inverse, first, last, blocks, bdt, scales, signs, x, ldx, in_dt, y, ldy,
                                out_dt, rows, stream, &done);
    if (done || e != hipSuccess) return e;
  }
  DecParams p{};
  p.P = (int)run.P;
  p.inner = (int)run.inner;
  p.nsub = (int)(pl.d / run.P);
  p.R = (int)(rows < 8 ? rows : 8);
  while (p.R > 1 && run_lds(pl, run.t0, run.t1, run.P, p.R, 1, bdt) > kDecLds) p.R >>= 1;
  const int64_t rblocks = (rows + p.R - 1) / p.R;
  p.ns = 1;
  while (p.ns * 2 <= p.nsub && ((p.nsub + p.ns - 1) / p.ns) * rblocks > 512 &&
         run_lds(pl, run.t0, run.t1, run.P, p.R, p.ns * 2, bdt) <= kDecLds)
    p.ns *= 2;
  p.nchunks = (p.nsub + p.ns - 1) / p.ns;
  p.nst = run.t1 - run.t0;
  p.transpose = inverse ? 1 : 0;
  p.sign_in = (!inverse && first && signs != nullptr) ? 1 : 0;
  p.sign_out = (inverse && last && signs != nullptr) ? 1 : 0;
  int cof = 0, sof = 0;
  for (int i = 0; i < p.nst; ++i) {
    const int t = inverse ? run.t1 - 1 - i : run.t0 + i;
    DecStage& s = p.st[i];
    s.b = pl.radix[t];
    int64_t sub = 1;
    for (int u = t + 1; u < run.t1; ++u) sub *= pl.radix[u];
    s.s = (int)sub;
    s.S = (int)(sub * run.inner);
    s.cof = cof;
    s.sof = sof;
    s.blk_off = (int)pl.blk_off[t];
    s.grp_off = (int)pl.grp_off[t];
    cof += p.ns * p.P * s.b;
    sof += bdt == DT::I8 ? p.ns * (p.P / s.b) : 0;
  }
  p.ncoef = cof;
  p.nscale = sof;
  p.blocks = blocks;
  p.scales = scales;
  p.signs = signs;
  p.x = x;
  p.ldx = ldx;
  p.y = y;
  p.ldy = ldy;
  p.rows = rows;
  const int64_t lds = run_lds(pl, run.t0, run.t1, run.P, p.R, p.ns, bdt);
  const int64_t grid = (int64_t)p.nchunks * rblocks;
  if (lds > kDecLds || grid > 0x7fffffff) return hipErrorInvalidValue;
  const bool in_f = in_dt == DT::F32, out_f = out_dt == DT::F32;
  if (in_f && out_f) return launch_run_b<float, float>(bdt, p, (int)grid, (int)lds, stream);
  if (in_f) return launch_run_b<float, uint16_t>(bdt, p, (int)grid, (int)lds, stream);
  if (out_f) return launch_run_b<uint16_t, float>(bdt, p, (int)grid, (int)lds, stream);
  return launch_run_b<uint16_t, uint16_t>(bdt, p, (int)grid, (int)lds, stream);
}

// The digit runs: one run over every stage if a single row fits a workgroup,
// else the split point k that balances the two runs' sub-problem sizes.
// Returns 0 if no split fits.
int plan_runs(const Plan& pl, DT bdt, Run runs[2]) {
  if (run_lds(pl, 0, pl.m, pl.d, 1, 1, bdt) <= kDecLds) {
    runs[0] = Run{0, pl.m, pl.d, 1};
    return 1;
  }
  int best = -1;
  int64_t best_max = 0;
  int64_t pa = 1;
  for (int k = 1; k < pl.m; ++k) {
    pa *= pl.radix[k - 1];
    const int64_t pb = pl.d / pa;
    if (run_lds(pl, 0, k, pa, 1, 1, bdt) > kDecLds || run_lds(pl, k, pl.m, pb, 1, 1, bdt) > kDecLds) continue;
    const int64_t mx = pa > pb ? pa : pb;
    if (best < 0 || mx < best_max) {
      best = k;
      best_max = mx;
    }
  }
  if (best < 0) return 0;
  int64_t p0 = 1;
  for (int t = 0; t < best; ++t) p0 *= pl.radix[t];
  runs[0] = Run{0, best, p0, pl.d / p0};
  runs[1] = Run{best, pl.m, pl.d / p0, 1};
  return 2;
}

}  // namespace

int64_t decode_workspace_bytes(const Plan& pl, DT bdt, int64_t rows) {
  Run runs[2];
  const int n = plan_runs(pl, bdt, runs);
  if (n == 0) return -1;
  if (rows > (INT64_MAX / 4) / pl.d) return -1;   // size not representable
  // one launch, or a call handed to the throughput row kernels: no hand-off
  if (n == 1 || rows > kDecodeRowsMax) return 0;
  return rows * pl.d * 4;
}

hipError_t launch_apply_decode(const Plan& pl, bool inverse, const void* blocks, DT bdt, const float* scales,
                               const int8_t* signs, const void* x, int64_t ldx, DT io, void* y, int64_t ldy,
                               int64_t rows, float* ws, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  // Above this many rows the 8-row tiles of the throughput kernels, which
  // fetch every block once per tile rather than once per row block and run,
  // are faster (measured crossover between 64 and 256 rows at d = 4096/5120).
  if (rows > kDecodeRowsMax)
    return launch_apply_rows(pl, inverse, blocks, bdt, scales, signs, x, ldx, io, y, ldy, io, rows, stream);
  Run runs[2];
  const int n = plan_runs(pl, bdt, runs);
  if (n == 0) return hipErrorInvalidValue;
  if (n == 1)
    return launch_one(pl, runs[0], inverse, true, true, blocks, bdt, scales, signs, x, ldx, io, y, ldy, io, rows,
                      stream);
  const Run& a = inverse ? runs[1] : runs[0];
  const Run& b = inverse ? runs[0] : runs[1];
  hipError_t e = launch_one(pl, a, inverse, true, false, blocks, bdt, scales, signs, x, ldx, io, ws, pl.d,
                            DT::F32, rows, stream);
  if (e != hipSuccess) return e;
  return launch_one(pl, b, inverse, false, true, blocks, bdt, scales, signs, ws, pl.d, DT::F32, y, ldy, io, rows,
                    stream);
}

}  // namespace harp
