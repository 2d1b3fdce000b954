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

// ------------------------------------------------------------------------
// Wave-per-row kernel for d = 4096 and 8192.  Because the normalised
// Sylvester H_d is the n-fold Kronecker power of H_2 (n = log2 d), every
// factoring of its n butterfly levels gives the same matrix, so the kernel
// orders the levels to suit the hardware rather than the schedule.  One wave
// owns one row; lane l holds E = d/64 coordinates in registers.  Three
// register layouts (bit maps from the coordinate index e to register bits
// and lane bits) are used:
//   A  (HBM I/O):  e bits 0-2 and 9.. in registers, 3-8 in lanes, so each lane
//                  moves 16 contiguous bytes per access;
//   A' :           A with lane bits 4 and 5 exchanged against the top two
//                  register bits (v_permlane16_swap / v_permlane32_swap);
//   B  :           the remaining lane bits of A' in registers.
// Butterflies over register bits are plain add/sub pairs; A' <-> B is one
// transpose through a 16 KB per-wave LDS buffer (in two halves of the
// coordinates for d = 8192), with 16-byte accesses and an XOR swizzle that
// keeps both directions free of bank conflicts.  A pass starting in A ends in
// B and vice versa.  Signs come from a per-workgroup LDS table of packed bits
// built once, one bit per (pass, lane, register) in the layout where that
// pass applies them.
namespace rhtw {

template <int N> struct Lay;
template <> struct Lay<13> {
  static constexpr int EB = 7;
  static constexpr int A_reg[7] = {0, 1, 2, 9, 10, 11, 12};
  static constexpr int A_lane[6] = {3, 4, 5, 6, 7, 8};
  static constexpr int P_reg[7] = {0, 1, 2, 9, 10, 7, 8};     // A'
  static constexpr int P_lane[6] = {3, 4, 5, 6, 11, 12};
  static constexpr int B_reg[7] = {0, 1, 2, 3, 4, 5, 6};
  static constexpr int B_lane[6] = {7, 8, 9, 10, 11, 12};
  static constexpr int SPLIT = 2;               // e bit in register bit 2 of A' and B: transpose halves
  static constexpr unsigned B_AFTER_A = 0x78u;  // B register bits left after a pass's A / A' levels
  static constexpr unsigned P_AFTER_B = 0x78u;  // A' register bits left after a pass's B levels
};
template <> struct Lay<12> {
  static constexpr int EB = 6;
  static constexpr int A_reg[6] = {0, 1, 2, 9, 10, 11};
  static constexpr int A_lane[6] = {3, 4, 5, 6, 7, 8};
  static constexpr int P_reg[6] = {0, 1, 2, 9, 7, 8};
  static constexpr int P_lane[6] = {3, 4, 5, 6, 10, 11};
  static constexpr int B_reg[6] = {0, 1, 3, 4, 5, 6};
  static constexpr int B_lane[6] = {2, 7, 8, 9, 10, 11};
  static constexpr int SPLIT = -1;
  static constexpr unsigned B_AFTER_A = 0x3cu;
  static constexpr unsigned P_AFTER_B = 0x3cu;
};

enum Which { kA = 0, kP = 1, kB = 2 };

template <int N, int W>
__device__ __forceinline__ int reg_part(int r) {
  using L = Lay<N>;
  int e = 0;
#pragma unroll
  for (int i = 0; i < L::EB; ++i) {
    const int b = W == kA ? L::A_reg[i] : (W == kP ? L::P_reg[i] : L::B_reg[i]);
    e |= ((r >> i) & 1) << b;
  }
  return e;
}
template <int N, int W>
__device__ __forceinline__ int lane_part(int lane) {
  using L = Lay<N>;
  int e = 0;
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const int b = W == kA ? L::A_lane[i] : (W == kP ? L::P_lane[i] : L::B_lane[i]);
    e |= ((lane >> i) & 1) << b;
  }
  return e;
}

// Float offset of coordinate e in the per-wave transpose buffer (within its
// half when the transpose is split).  XOR-linear in e, so the offset of
// reg_part | lane_part is off(reg_part) ^ off(lane_part).
template <int N>
__device__ __forceinline__ int buf_off(int e) {
  constexpr int S = Lay<N>::SPLIT;
  const int ep = S < 0 ? e : ((e & ((1 << S) - 1)) | ((e >> (S + 1)) << S));
  const int u = ep >> 2;
  return 4 * (u ^ ((u >> 4) & 15)) + (ep & 3);
}

// Butterflies over the register bits in MASK.
template <int E, unsigned MASK>
__device__ __forceinline__ void levels(float (&v)[E]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if ((MASK >> i) & 1u) {
      const int m = 1 << i;
#pragma unroll
      for (int r = 0; r < E; ++r) {
        if ((r & m) == 0) {
          const float a = v[r], b = v[r + m];
          v[r] = a + b;
          v[r + m] = a - b;
        }
      }
      // level by level: interleaving levels only lengthens live ranges
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// A <-> A': exchange lane bit 5 with register bit EB-1 and lane bit 4 with
// register bit EB-2 (each swap is its own inverse).
template <int N>
__device__ __forceinline__ void swap_lanes(float (&v)[1 << Lay<N>::EB]) {
  constexpr int EB = Lay<N>::EB;
  constexpr int E = 1 << EB;
  constexpr int m5 = 1 << (EB - 1), m4 = 1 << (EB - 2);
#pragma unroll
  for (int r = 0; r < E; ++r) {
    if ((r & m5) == 0) {
      auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[r]), __float_as_uint(v[r + m5]), false, false);
      v[r] = __uint_as_float(t[0]);
      v[r + m5] = __uint_as_float(t[1]);
    }
  }
#pragma unroll
  for (int r = 0; r < E; ++r) {
    if ((r & m4) == 0) {
      auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[r]), __float_as_uint(v[r + m4]), false, false);
      v[r] = __uint_as_float(t[0]);
      v[r + m4] = __uint_as_float(t[1]);
    }
  }
}

// Layout FROM -> TO (A' <-> B) through the wave's LDS buffer.
template <int N, int FROM, int TO>
__device__ __forceinline__ void transpose(float (&v)[1 << Lay<N>::EB], float* buf, int lane) {
  constexpr int EB = Lay<N>::EB;
  constexpr int E = 1 << EB;
  constexpr int S = Lay<N>::SPLIT;
  int lw = buf_off<N>(lane_part<N, FROM>(lane));
  int lr = buf_off<N>(lane_part<N, TO>(lane));
  // keep the 2 * E / 4 per-access addresses (lane base ^ constant) out of
  // loop-invariant hoisting: they are one XOR each, live registers are not
  __asm__ volatile("" : "+v"(lw), "+v"(lr));
#pragma unroll
  for (int h = 0; h < (S < 0 ? 1 : 2); ++h) {
#pragma unroll
    for (int r = 0; r < E; r += 4) {
      if (S < 0 || ((r >> 2) & 1) == h) {   // register bit 2 holds e bit SPLIT in both layouts
        f32x4 w = {v[r], v[r + 1], v[r + 2], v[r + 3]};
        *reinterpret_cast<f32x4*>(buf + (lw ^ buf_off<N>(reg_part<N, FROM>(r)))) = w;
        // a few accesses at a time: hoisting all addresses costs registers
        if ((r & 31) == 28) __builtin_amdgcn_sched_barrier(0);
      }
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int r = 0; r < E; r += 4) {
      if (S < 0 || ((r >> 2) & 1) == h) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(buf + (lr ^ buf_off<N>(reg_part<N, TO>(r))));
        v[r] = w.x; v[r + 1] = w.y; v[r + 2] = w.z; v[r + 3] = w.w;
        if ((r & 31) == 28) __builtin_amdgcn_sched_barrier(0);
      }
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

template <int E>
__device__ __forceinline__ void apply_sign(float (&v)[E], const uint32_t* bits) {
#pragma unroll
  for (int w = 0; w < E / 32; ++w) {
    const uint32_t word = bits[w];
#pragma unroll
    for (int j = 0; j < 32; ++j)
      v[32 * w + j] = __uint_as_float(__float_as_uint(v[32 * w + j]) ^ ((word << (31 - j)) & 0x80000000u));
  }
}

struct WaveParams {
  const int8_t* signs;
  const void* x;
  int64_t ldx;
  void* y;
  int64_t ldy;
  int64_t rows;
  int k;
  float out_scale;
};

template <typename T> struct IoV;
template <> struct IoV<uint16_t> { static constexpr int V = 8; };
template <> struct IoV<float> { static constexpr int V = 4; };

// WPB waves per workgroup (8: two waves per SIMD).  For d = 8192 (128
// coordinates per lane) the 256-register budget spills a few dozen values;
// one wave per SIMD avoids the spills but measured slower (the second wave
// hides the LDS and memory latencies).
template <int N, typename T, bool INV, int WPB>
__global__ void __launch_bounds__(64 * WPB) rht_wave_kernel(WaveParams p) {
  constexpr int EB = Lay<N>::EB;
  constexpr int E = 1 << EB;
  constexpr int NW = E / 32;                 // sign words per lane per pass
  constexpr int d = 1 << N;
  constexpr int V = IoV<T>::V;
  extern __shared__ float lds[];
  uint32_t* tbl = reinterpret_cast<uint32_t*>(lds);          // [k][64][NW]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float* buf = lds + 8 * 64 * NW + wave * 4096;   // 16 KB per wave
  // sign bits: pass q starts in A when q is even; forward passes use sign
  // vector q before their levels, inverse passes sign vector k-1-q after them
  for (int idx = threadIdx.x; idx < p.k * 64 * NW; idx += blockDim.x) {
    const int q = idx / (64 * NW);
    const int l = (idx / NW) % 64;
    const int w = idx % NW;
    const bool in_a = INV ? (q & 1) : !(q & 1);
    const int8_t* sg = p.signs + (int64_t)(INV ? p.k - 1 - q : q) * d;
    uint32_t word = 0;
    for (int j = 0; j < 32; ++j) {
      const int r = 32 * w + j;
      const int e = in_a ? (reg_part<N, kA>(r) | lane_part<N, kA>(l)) : (reg_part<N, kB>(r) | lane_part<N, kB>(l));
      word |= (sg[e] < 0 ? 1u : 0u) << j;
    }
    tbl[idx] = word;
  }
  __syncthreads();
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int la = lane << 3;                  // lane part of A: e bits 3..8
  for (int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave; row < p.rows; row += nwaves) {
    float v[E];
    const T* x = static_cast<const T*>(p.x) + row * p.ldx;
#pragma unroll
    for (int c = 0; c < E / 8; ++c) {
#pragma unroll
      for (int h = 0; h < 8 / V; ++h) {
        const u32x4 w = ld_stream(x + (c << 9) + la + h * V);
        if constexpr (V == 8) {
          v[8 * c + 0] = bf16_lo(w.x); v[8 * c + 1] = bf16_hi(w.x);
          v[8 * c + 2] = bf16_lo(w.y); v[8 * c + 3] = bf16_hi(w.y);
          v[8 * c + 4] = bf16_lo(w.z); v[8 * c + 5] = bf16_hi(w.z);
          v[8 * c + 6] = bf16_lo(w.w); v[8 * c + 7] = bf16_hi(w.w);
        } else {
          v[8 * c + 4 * h + 0] = __uint_as_float(w.x); v[8 * c + 4 * h + 1] = __uint_as_float(w.y);
          v[8 * c + 4 * h + 2] = __uint_as_float(w.z); v[8 * c + 4 * h + 3] = __uint_as_float(w.w);
        }
      }
    }
    for (int q = 0; q < p.k; ++q) {
      const uint32_t* bits = tbl + (q * 64 + lane) * NW;
      if ((q & 1) == 0) {
        // A -> A' -> B
        if (!INV) apply_sign<E>(v, bits);
        levels<E, (1u << EB) - 1>(v);
        swap_lanes<N>(v);
        levels<E, (3u << (EB - 2))>(v);
        transpose<N, kP, kB>(v, buf, lane);
        levels<E, Lay<N>::B_AFTER_A>(v);
        if (INV) apply_sign<E>(v, bits);
      } else {
        // B -> A' -> A
        if (!INV) apply_sign<E>(v, bits);
        levels<E, (1u << EB) - 1>(v);
        transpose<N, kB, kP>(v, buf, lane);
        levels<E, Lay<N>::P_AFTER_B>(v);
        swap_lanes<N>(v);
        levels<E, (3u << (EB - 2))>(v);
        if (INV) apply_sign<E>(v, bits);
      }
    }
    if (p.k & 1) {
      transpose<N, kB, kP>(v, buf, lane);
      swap_lanes<N>(v);
    }
    T* y = static_cast<T*>(p.y) + row * p.ldy;
#pragma unroll
    for (int c = 0; c < E / 8; ++c) {
#pragma unroll
      for (int h = 0; h < 8 / V; ++h) {
        u32x4 w;
        if constexpr (V == 8) {
          w.x = pack_bf16x2_hw(v[8 * c + 0] * p.out_scale, v[8 * c + 1] * p.out_scale);
          w.y = pack_bf16x2_hw(v[8 * c + 2] * p.out_scale, v[8 * c + 3] * p.out_scale);
          w.z = pack_bf16x2_hw(v[8 * c + 4] * p.out_scale, v[8 * c + 5] * p.out_scale);
          w.w = pack_bf16x2_hw(v[8 * c + 6] * p.out_scale, v[8 * c + 7] * p.out_scale);
        } else {
          w.x = __float_as_uint(v[8 * c + 4 * h + 0] * p.out_scale);
          w.y = __float_as_uint(v[8 * c + 4 * h + 1] * p.out_scale);
          w.z = __float_as_uint(v[8 * c + 4 * h + 2] * p.out_scale);
          w.w = __float_as_uint(v[8 * c + 4 * h + 3] * p.out_scale);
        }
        st_stream(y + (c << 9) + la + h * V, w);
      }
    }
  }
}

}  // namespace rhtw

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
template <int N, typename T, bool INV>
hipError_t launch_wave_typed(const rhtw::WaveParams& wp, hipStream_t stream) {
  constexpr int WPB = 8;
  auto kern = rhtw::rht_wave_kernel<N, T, INV, WPB>;
  const size_t lds = (size_t)8 * 64 * ((1 << (N - 6)) / 32) * 4 + (size_t)WPB * 4096 * 4;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  int64_t grid = cu_count();
  const int64_t need = (wp.rows + WPB - 1) / WPB;
  if (grid > need) grid = need;
  hipLaunchKernelGGL(kern, dim3((int)grid), dim3(64 * WPB), lds, stream, wp);
  return hipGetLastError();
}

template <int N>
hipError_t launch_wave_n(DT io, bool inverse, const rhtw::WaveParams& wp, hipStream_t stream) {
  if (io == DT::BF16)
    return inverse ? launch_wave_typed<N, uint16_t, true>(wp, stream) : launch_wave_typed<N, uint16_t, false>(wp, stream);
  return inverse ? launch_wave_typed<N, float, true>(wp, stream) : launch_wave_typed<N, float, false>(wp, stream);
}

// Wave-per-row path: d = 2^n with n in {12, 13}, k <= 8, 16-byte aligned rows.
hipError_t launch_rht_wave(int n, DT io, bool inverse, const int8_t* signs, int k, const void* x, int64_t ldx,
                           void* y, int64_t ldy, int64_t rows, float out_scale, hipStream_t stream) {
  rhtw::WaveParams wp{signs, x, ldx, y, ldy, rows, k, out_scale};
  return n == 13 ? launch_wave_n<13>(io, inverse, wp, stream) : launch_wave_n<12>(io, inverse, wp, stream);
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
  const bool aligned = reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0 &&
                       (ldx * ib) % 16 == 0 && (ldy * ob) % 16 == 0;
  if ((pl.d == 4096 || pl.d == 8192) && in_dt == out_dt && k <= 8 && aligned)
    return launch_rht_wave(pl.d == 8192 ? 13 : 12, in_dt, inverse, signs, k, x, ldx, y, ldy, rows,
                           p.out_scale, stream);
  RhtExtra ex{k, inverse ? 1 : 0};
  if (in_dt == DT::F32 && out_dt == DT::F32) return launch_rht_typed<float, float>(p, ex, threads, (int)grid, lds, stream);
  if (in_dt == DT::BF16 && out_dt == DT::BF16) return launch_rht_typed<uint16_t, uint16_t>(p, ex, threads, (int)grid, lds, stream);
  return hipErrorInvalidValue;
}

}  // namespace harp
