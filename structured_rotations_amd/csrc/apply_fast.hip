// Schedule-specialised matrix-core row kernels for the HARP transform.
//
// HARP technical summary (gist.science 2605.29843), §2.1/§2.2: stage t
// applies, to every group of coordinates that agree on all digits but digit
// t, its own b_t x b_t orthogonal block.  These kernels compute what the
// generic matrix-core kernel computes (8-row tiles in LDS, data waves that
// stream tiles in and out, v_mfma_f32_4x4x1f32 with a block of 4 lanes per
// group and lane j carrying row j of a row quad), for two schedules known at
// compile time:
//   * d = 4096, (8,8,8,8): 16 rounds of 16 groups per compute wave; the
//     padded LDS layout makes every gather an immediate offset; coefficients
//     come through a buffer resource three rounds ahead into four rotating
//     register buffers; rounds are ordered so no LDS latency lands on the
//     matrix cores; wave-local group sets leave one exchange barrier per
//     tile; the last stage stores straight to HBM.
//   * d = 5120, (8,8,8,5,2): three radix-8 stages and one fused stage for the
//     radix-5 / radix-2 pair, whose digits both lie inside 10 consecutive
//     columns (4 rounds instead of 28).
#include <type_traits>

#include "row_io.h"

namespace harp {

namespace {

using namespace rowk;

constexpr int kCW = 8;                    // compute waves
constexpr int kGPR = 16 * kCW;            // groups per round (16 per compute wave)

template <int B_, int S_>
struct St {
  static constexpr int B = B_;
  static constexpr int S = S_;
};

template <class... Ss>
struct List {
  static constexpr int size = sizeof...(Ss);
};
template <int I, class L>
struct At;
template <class H, class... T>
struct At<0, List<H, T...>> {
  using type = H;
};
template <int I, class H, class... T>
struct At<I, List<H, T...>> {
  using type = typename At<I - 1, List<T...>>::type;
};

// D: row length; Lay: LDS unit layout; L: stages in processing order.
template <int D_, class Lay_, class L_>
struct Sched {
  static constexpr int D = D_;
  using Lay = Lay_;
  using L = L_;
  static constexpr int M = L::size;
};

template <int B, int S>
__host__ __device__ constexpr int col0_of(int g) {
  return (g / S) * (B - 1) * S + g;
}

// True when, for every group of the stage, the units of its B columns are
// unit(col0) + (unit(k S) - unit(0)): then one address per group suffices.
template <class Lay, int D, int B, int S>
constexpr bool linear_stage() {
  for (int g = 0; g < D / B; ++g) {
    const int c0 = col0_of<B, S>(g);
    for (int k = 0; k < B; ++k)
      if (Lay::unit(c0 + k * S) - Lay::unit(c0) != Lay::unit(k * S) - Lay::unit(0)) return false;
  }
  return true;
}

template <class Sch, int I = 0>
constexpr int rounds_before_rt(int t) {
  if constexpr (I >= Sch::M) {
    return 0;
  } else {
    using Si = typename At<I, typename Sch::L>::type;
    return I < t ? Sch::D / Si::B / kGPR + rounds_before_rt<Sch, I + 1>(t) : 0;
  }
}

// Coefficients are read through a buffer resource: the part of the byte
// offset that is the same for the whole wave (stage, round) goes in an SGPR,
// the lane's part (its group within the round and its coefficient row) is
// one 32-bit VGPR that never changes, so a round costs no 64-bit address
// arithmetic and keeps no per-round pointers live.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coef_rsrc(const RowParams& p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.blocks), (short)0, -1, 0x00020000);
}

// cf[h][k] = C[4h + j][k] of group g0 + gb (C = B forward, B^T inverse; g0
// uniform); lanes whose row 4h + j is past the radix re-read row B - 1 (their
// outputs are dropped).
template <int B, typename TB, bool TR>
__device__ __forceinline__ void load_coef(__amdgpu_buffer_rsrc_t rs, const StageFast& sd, int g0, int gb, int j,
                                          float (&cf)[2][8]) {
  constexpr int NH = B > 4 ? 2 : 1;
  constexpr int SZ = (int)sizeof(TB);
  const int soff = __builtin_amdgcn_readfirstlane((sd.blk_off + g0 * B * B) * SZ);
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int o = 4 * h + j < B ? 4 * h + j : B - 1;
    if constexpr (!TR && (B == 8 || B == 4)) {
      const int voff = (gb * B * B + o * B) * SZ;
      if constexpr (std::is_same<TB, float>::value) {
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
        cf[h][0] = __uint_as_float(a.x); cf[h][1] = __uint_as_float(a.y);
        cf[h][2] = __uint_as_float(a.z); cf[h][3] = __uint_as_float(a.w);
        if constexpr (B == 8) {
          const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, soff, 0);
          cf[h][4] = __uint_as_float(b.x); cf[h][5] = __uint_as_float(b.y);
          cf[h][6] = __uint_as_float(b.z); cf[h][7] = __uint_as_float(b.w);
        }
      } else if constexpr (B == 8) {
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
        cf[h][0] = bf16_lo(a.x); cf[h][1] = bf16_hi(a.x); cf[h][2] = bf16_lo(a.y); cf[h][3] = bf16_hi(a.y);
        cf[h][4] = bf16_lo(a.z); cf[h][5] = bf16_hi(a.z); cf[h][6] = bf16_lo(a.w); cf[h][7] = bf16_hi(a.w);
      } else {
        const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
        cf[h][0] = bf16_lo(a.x); cf[h][1] = bf16_hi(a.x); cf[h][2] = bf16_lo(a.y); cf[h][3] = bf16_hi(a.y);
      }
    } else {
      // element (o, k) of C sits at k * B + o (transposed) or o * B + k
      const int voff = (gb * B * B + (TR ? o : o * B)) * SZ;
#pragma unroll
      for (int k = 0; k < B; ++k) {
        const int imm = (TR ? k * B : k) * SZ;
        if constexpr (std::is_same<TB, float>::value)
          cf[h][k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voff + imm, soff, 0));
        else
          cf[h][k] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, voff + imm, soff, 0) << 16);
      }
    }
  }
}

// One round: 16 groups per compute wave, both row quads.
template <class Sch, int B, int S, bool TR, bool DIRECT, typename T>
__device__ __forceinline__ void round_compute(const RowParams& p, float* tile, int g, const float (&cf)[2][8],
                                              int64_t row0, int nr, int j) {
  using Lay = typename Sch::Lay;
  constexpr int D = Sch::D;
  constexpr int NH = B > 4 ? 2 : 1;
  constexpr int PLANE = 4 * Lay::units(D);
  constexpr bool LIN = linear_stage<Lay, D, B, S>();
  const int col0 = col0_of<B, S>(g);
  float xv[2][B];
  const float* src = tile + 4 * Lay::unit(col0) + j;
#pragma unroll
  for (int k = 0; k < B; ++k) {
    const int a = LIN ? 4 * (Lay::unit(k * S) - Lay::unit(0)) : 4 * Lay::unit(col0 + k * S) - 4 * Lay::unit(col0);
    xv[0][k] = src[a];
    xv[1][k] = src[a + PLANE];
  }
  // D[i][j] = sum_k C[4h+i][k] x[row 4q+j][k]: lane j ends with outputs
  // 4h..4h+3 of row 4q+j.  Written back as 4-byte stores (output 4h+i of the
  // four rows of a quad lands in one 16-byte unit, filled by the block's four
  // lanes), which keeps every store free of bank conflicts; for a contiguous
  // radix-8 last stage the 8 outputs are 8 consecutive columns of one row and
  // go straight to HBM.
  f32x4 acc[2][2];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int q = 0; q < 2; ++q)
      acc[q][h] = __builtin_amdgcn_mfma_f32_4x4x1f32(cf[h][0], xv[q][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
  for (int k = 1; k < B; ++k)
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        acc[q][h] = __builtin_amdgcn_mfma_f32_4x4x1f32(cf[h][k], xv[q][k], acc[q][h], 0, 0, 0);
  if constexpr (!DIRECT) {
    float* dst = tile + 4 * Lay::unit(col0) + j;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = 4 * h + i;
        if (o < B) {
          const int a = LIN ? 4 * (Lay::unit(o * S) - Lay::unit(0)) : 4 * Lay::unit(col0 + o * S) - 4 * Lay::unit(col0);
          dst[a] = acc[0][h][i];
          dst[a + PLANE] = acc[1][h][i];
        }
      }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = 4 * q + j;
      if (r < nr) {
        float v[8] = {acc[q][0].x, acc[q][0].y, acc[q][0].z, acc[q][0].w,
                      acc[q][1].x, acc[q][1].y, acc[q][1].z, acc[q][1].w};
        T* y = static_cast<T*>(p.y) + (row0 + r) * p.ldy + col0;
        if constexpr (std::is_same<T, uint16_t>::value) {
          st_stream(y, u32x4{pack_bf16x2_hw(v[0], v[1]), pack_bf16x2_hw(v[2], v[3]), pack_bf16x2_hw(v[4], v[5]),
                             pack_bf16x2_hw(v[6], v[7])});
        } else {
          st_stream(y, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
          st_stream(y + 4, u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
        }
      }
    }
  }
}

// ------------------------------------------------------------------------
// Pipelined variant for schedules whose tile takes a number of rounds
// divisible by 4 (d = 4096, (8,8,8,8): 16 rounds).  Every round of a tile is
// unrolled, so the coefficient buffers rotate at compile time: round n uses
// buffer n % 4 and prefetches round n + 3 (possibly of the next tile) into
// buffer (n + 3) % 4, three rounds of latency instead of one.  Inside a
// stage the next round's LDS inputs are read while this round's products
// run.  8 compute waves + 4 data waves (three waves per SIMD) leave room for
// the extra buffers.
constexpr int kPCW = 8;
constexpr int kPIOW = 4;
constexpr int kPThreads = 64 * (kPCW + kPIOW);
static_assert(kPCW == kCW, "the round size kGPR assumes 8 compute waves");

template <class Sch, int N>
constexpr int stage_of() {
  int t = 0;
  while (t + 1 < Sch::M && N >= rounds_before_rt<Sch>(t + 1)) ++t;
  return t;
}

template <class Sch, int B, int S>
__device__ __forceinline__ void read_inputs(const float* tile, int g, int j, float (&xv)[2][8]) {
  using Lay = typename Sch::Lay;
  constexpr int PLANE = 4 * Lay::units(Sch::D);
  constexpr bool LIN = linear_stage<Lay, Sch::D, B, S>();
  const int col0 = col0_of<B, S>(g);
  const float* src = tile + 4 * Lay::unit(col0) + j;
#pragma unroll
  for (int k = 0; k < B; ++k) {
    const int a = LIN ? 4 * (Lay::unit(k * S) - Lay::unit(0)) : 4 * Lay::unit(col0 + k * S) - 4 * Lay::unit(col0);
    xv[0][k] = src[a];
    xv[1][k] = src[a + PLANE];
  }
}

// One round of products, ordered so that no LDS latency lands on the matrix
// cores: the h = 0 outputs are written while the h = 1 chain runs, the next
// round's inputs are read after those writes (so the next round waits only
// for its own reads and the writes before them, never for the last writes),
// and the h = 1 outputs go last.  Radix 8 only (two output halves).
template <class Sch, int B, int S, bool DIRECT, bool NEXT, typename T>
__device__ __forceinline__ void products_write(const RowParams& p, float* tile, int g, int gn, const float (&cf)[2][8],
                                               const float (&xv)[2][8], float (&xn)[2][8], int64_t row0, int nr,
                                               int j) {
  static_assert(B == 8, "the pipelined round is written for radix 8");
  using Lay = typename Sch::Lay;
  constexpr int PLANE = 4 * Lay::units(Sch::D);
  constexpr bool LIN = linear_stage<Lay, Sch::D, B, S>();
  const int col0 = col0_of<B, S>(g);
  float* dst = tile + 4 * Lay::unit(col0) + j;
  auto out_addr = [&](int o) {
    return LIN ? 4 * (Lay::unit(o * S) - Lay::unit(0)) : 4 * Lay::unit(col0 + o * S) - 4 * Lay::unit(col0);
  };
  f32x4 acc[2][2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
    acc[q][0] = __builtin_amdgcn_mfma_f32_4x4x1f32(cf[0][0], xv[q][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
  for (int k = 1; k < B; ++k)
#pragma unroll
    for (int q = 0; q < 2; ++q)
      acc[q][0] = __builtin_amdgcn_mfma_f32_4x4x1f32(cf[0][k], xv[q][k], acc[q][0], 0, 0, 0);
#pragma unroll
  for (int q = 0; q < 2; ++q)
    acc[q][1] = __builtin_amdgcn_mfma_f32_4x4x1f32(cf[1][0], xv[q][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
  for (int q = 0; q < 2; ++q)
    acc[q][1] = __builtin_amdgcn_mfma_f32_4x4x1f32(cf[1][1], xv[q][1], acc[q][1], 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!DIRECT) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dst[out_addr(i)] = acc[0][0][i];
      dst[out_addr(i) + PLANE] = acc[1][0][i];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NEXT) read_inputs<Sch, B, S>(tile, gn, j, xn);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 2; k < B; ++k) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
      acc[q][1] = __builtin_amdgcn_mfma_f32_4x4x1f32(cf[1][k], xv[q][k], acc[q][1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!DIRECT) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dst[out_addr(4 + i)] = acc[0][1][i];
      dst[out_addr(4 + i) + PLANE] = acc[1][1][i];
    }
  } else {
    // rows past a ragged last tile hold the last row's result again (their
    // inputs re-read the last row), so they store the same bytes over it:
    // the stores stay unconditional and the wait counts static
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r0 = 4 * q + j;
      const int r = r0 < nr ? r0 : nr - 1;
      float v[8] = {acc[q][0].x, acc[q][0].y, acc[q][0].z, acc[q][0].w,
                    acc[q][1].x, acc[q][1].y, acc[q][1].z, acc[q][1].w};
      T* y = static_cast<T*>(p.y) + (row0 + r) * p.ldy + col0;
      if constexpr (std::is_same<T, uint16_t>::value) {
        st_stream(y, u32x4{pack_bf16x2_hw(v[0], v[1]), pack_bf16x2_hw(v[2], v[3]), pack_bf16x2_hw(v[4], v[5]),
                           pack_bf16x2_hw(v[6], v[7])});
      } else {
        st_stream(y, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
        st_stream(y + 4, u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
      }
    }
  }
}

// Wave-local group sets.  For d = 4096 = 64 x 64 (column c = 64 hi + lo), in
// the two stages on the digits of hi (strides 512 and 64) wave w takes the
// groups whose lo lies in [8w, 8w + 8), and in the two stages on the digits
// of lo (strides 8 and 1) those whose hi lies in [8w, 8w + 8).  Inside each
// pair of stages a wave therefore reads only columns it wrote itself, so the
// pair needs no workgroup barrier in between (LDS accesses of one wave are
// performed in order); only the change of pair is an all-to-all exchange.
// Round rr of a stage covers, per wave, 16 groups: the uniform part of the
// group index is grp_round(rr), the lane's part lane_grp(gA, gB).
template <int S>
constexpr bool hi_pair() {
  return S >= 64;
}
template <int S>
__device__ __forceinline__ int grp_round(int rr) {
  return hi_pair<S>() ? rr * 128 : rr * 16;
}
template <int S>
__device__ __forceinline__ int lane_grp(int gA, int gB) {
  return hi_pair<S>() ? gA : gB;
}

template <class Sch, int N, bool TR, bool DOUT, typename T, typename TB>
__device__ __forceinline__ void pipe_round(const RowParams& p, float* tile, float (&cf)[4][2][8],
                                           float (&xv)[2][2][8], int gA, int gB, int rot, int j, int64_t row0,
                                           int nr) {
  constexpr int M = Sch::M;
  constexpr int RT = rounds_before_rt<Sch>(M);
  constexpr int t = stage_of<Sch, N>();
  constexpr int r = N - rounds_before_rt<Sch>(t);
  using Sg = typename At<t, typename Sch::L>::type;
  constexpr int B = Sg::B, S = Sg::S, R = Sch::D / B / kGPR;
  constexpr bool DIRECT = DOUT && t == M - 1;
  constexpr int NP = (N + 3) % RT;
  constexpr int tp = stage_of<Sch, NP>();
  constexpr int rp = NP - rounds_before_rt<Sch>(tp);
  using Sp = typename At<tp, typename Sch::L>::type;
  constexpr int Rp = Sch::D / Sp::B / kGPR;
  const __amdgpu_buffer_rsrc_t rs = coef_rsrc(p);
  const int gl = lane_grp<S>(gA, gB);
  __builtin_amdgcn_sched_barrier(0);
  load_coef<Sp::B, TB, TR>(rs, p.st[tp], grp_round<Sp::S>((rp + rot) % Rp), lane_grp<Sp::S>(gA, gB), j,
                           cf[(N + 3) % 4]);
  __builtin_amdgcn_sched_barrier(0);
  products_write<Sch, B, S, DIRECT, (r + 1 < R), T>(p, tile, grp_round<S>((r + rot) % R) + gl,
                                                   grp_round<S>((r + 1 + rot) % R) + gl, cf[N % 4], xv[N % 2],
                                                   xv[(N + 1) % 2], row0, nr, j);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (r + 1 == R) {
    if constexpr (t + 1 < M) {
      using Sn = typename At<t + 1, typename Sch::L>::type;
      constexpr int Rn = Sch::D / Sn::B / kGPR;
      if constexpr (hi_pair<S>() != hi_pair<Sn::S>()) {
        __syncthreads();
      } else {
        // the next stage reads what this wave has just written
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
      }
      read_inputs<Sch, Sn::B, Sn::S>(tile, grp_round<Sn::S>(rot % Rn) + lane_grp<Sn::S>(gA, gB), j,
                                     xv[(N + 1) % 2]);
    } else {
      __syncthreads();   // the tile is finished
    }
  }
  if constexpr (N + 1 < RT) pipe_round<Sch, N + 1, TR, DOUT, T, TB>(p, tile, cf, xv, gA, gB, rot, j, row0, nr);
}

template <class Sch, bool TR, bool DOUT, typename T, typename TB>
__global__ void __launch_bounds__(kPThreads) apply_pipe_kernel(RowParams p) {
  constexpr int RT = rounds_before_rt<Sch>(Sch::M);
  static_assert(RT % 4 == 0, "the coefficient buffers rotate with period 4");
  static_assert(Sch::D == 4096 && kGPR == 128, "wave-local group sets are laid out for d = 4096");
  extern __shared__ float tile[];
  int64_t tix = blockIdx.x;
  if (tix >= p.ntiles) return;   // uniform per workgroup
  if (threadIdx.x >= 64 * kPCW) {
    // 2 x 512 (bf16) or 2 x 1024 (fp32) micro-blocks over 256 data threads
    constexpr bool F = std::is_same<T, float>::value;
    data_waves_exact<T, typename Sch::Lay, 64 * kPIOW, F ? 8 : 4, 4, 2, DOUT, false>(p, tile,
                                                                                   threadIdx.x - 64 * kPCW);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int blk = lane >> 2;
  const int gA = (blk >> 3) * 64 + 8 * wave + (blk & 7);
  const int gB = 64 * wave + blk;
  const int j = lane & 3;
  // Rounds inside a stage are independent, so each workgroup starts the
  // round sequence at its own offset: at any moment the CUs of an XCD (which
  // receives every eighth workgroup) then fetch different parts of the
  // coefficient array instead of all hitting the same L2 lines.
  const int rot = (int)((blockIdx.x >> 3) & 0xffff);
  using S0 = typename At<0, typename Sch::L>::type;
  constexpr int R0 = Sch::D / S0::B / kGPR;
  float cf[4][2][8];
  float xv[2][2][8];
#pragma unroll
  for (int n = 0; n < 3; ++n) {
    // rounds 0..2 all lie in stage 0 (it has at least 4 rounds)
    load_coef<S0::B, TB, TR>(coef_rsrc(p), p.st[0], grp_round<S0::S>((n + rot) % R0), lane_grp<S0::S>(gA, gB), j,
                             cf[n]);
  }
  __syncthreads();
  for (; tix < p.ntiles; tix += gridDim.x) {
    const int64_t row0 = tix * kRows;
    const int nr = tile_rows(p, tix);
    read_inputs<Sch, S0::B, S0::S>(tile, grp_round<S0::S>(rot % R0) + lane_grp<S0::S>(gA, gB), j, xv[0]);
    pipe_round<Sch, 0, TR, DOUT, T, TB>(p, tile, cf, xv, gA, gB, rot, j, row0, nr);
    __syncthreads();   // data waves have swapped the tile
  }
}

// ------------------------------------------------------------------------
// d = 5120, (8,8,8,5,2).  The radix-5 stage (stride 2) and the radix-2 stage
// (stride 1) both act inside the 10 consecutive columns 10 hi .. 10 hi + 9
// of one value hi of the first three digits, so one round does both for 16
// such chunks per compute wave: the radix-5 products on the matrix cores and
// the 2 x 2 blocks on the vector ALU, in registers, with one LDS round trip
// for the pair instead of two and 4 rounds instead of 28.  Operands are
// swapped against the radix-8 rounds (the data is the A operand): lane j then
// ends with output 4h + j of the radix-5 block for the four rows of its quad,
// so both halves d4 = 0, 1 of a radix-2 pair sit in the same lane, and each
// result is one 16-byte unit (4 rows of one column) of the tile.
// Coefficient buffer of a round: radix-8 rounds use the first 16 floats as
// cf[h][k]; tail rounds use [0, 20) for the radix-5 operands c5[d4][h][k]
// and [20, 40) for 2 x 2 blocks.
struct Cbuf {
  float v[40];
};
__device__ __forceinline__ float (&as8(Cbuf& c))[2][8] { return *reinterpret_cast<float(*)[2][8]>(&c.v[0]); }
__device__ __forceinline__ const float (&as8(const Cbuf& c))[2][8] {
  return *reinterpret_cast<const float(*)[2][8]>(&c.v[0]);
}

template <typename TB>
__device__ __forceinline__ float ld_coef1(__amdgpu_buffer_rsrc_t rs, int voff_el, int soff_bytes) {
  if constexpr (std::is_same<TB, float>::value)
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voff_el * 4, soff_bytes, 0));
  else
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, voff_el * 2, soff_bytes, 0) << 16);
}
// four consecutive coefficients starting at a 4-aligned element
template <typename TB>
__device__ __forceinline__ void ld_coef4(__amdgpu_buffer_rsrc_t rs, int voff_el, int soff_bytes, float* d) {
  if constexpr (std::is_same<TB, float>::value) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, voff_el * 4, soff_bytes, 0);
    d[0] = __uint_as_float(a.x); d[1] = __uint_as_float(a.y); d[2] = __uint_as_float(a.z); d[3] = __uint_as_float(a.w);
  } else {
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(rs, voff_el * 2, soff_bytes, 0);
    d[0] = bf16_lo(a.x); d[1] = bf16_hi(a.x); d[2] = bf16_lo(a.y); d[3] = bf16_hi(a.y);
  }
}

// Tail coefficients for chunk g = g0 + gb (g0 uniform).  s5: the radix-5
// stage, s2: the radix-2 stage.  Forward: c5[d4][h][k] = C5_{2g+d4}[o][k],
// o = min(4h + j, 4), and the two 2 x 2 blocks of columns o (h = 0, 1).
// Inverse: c5[d4][h][k] = C5_{2g+d4}[k][o] and all five 2 x 2 blocks.
template <typename TB, bool TR>
__device__ __forceinline__ void load_tail(__amdgpu_buffer_rsrc_t rs, const StageFast& s5, const StageFast& s2, int g0,
                                          int gb, int j, Cbuf& c) {
  constexpr int SZ = (int)sizeof(TB);
  const int soff5 = __builtin_amdgcn_readfirstlane((s5.blk_off + g0 * 2 * 25) * SZ);
  const int soff2 = __builtin_amdgcn_readfirstlane((s2.blk_off + g0 * 5 * 4) * SZ);
#pragma unroll
  for (int d4 = 0; d4 < 2; ++d4)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int o = 4 * h + j < 5 ? 4 * h + j : 4;
      const int base = (2 * gb + d4) * 25;
      float* d = &c.v[(d4 * 2 + h) * 5];
      if constexpr (!TR && std::is_same<TB, float>::value) {
        // row o of the block: 5 consecutive floats, 4-byte aligned (a
        // 16-byte load needs only dword alignment here)
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, (base + o * 5) * 4, soff5, 0);
        d[0] = __uint_as_float(a.x); d[1] = __uint_as_float(a.y); d[2] = __uint_as_float(a.z); d[3] = __uint_as_float(a.w);
        d[4] = ld_coef1<TB>(rs, base + o * 5 + 4, soff5);
      } else {
#pragma unroll
        for (int k = 0; k < 5; ++k) d[k] = ld_coef1<TB>(rs, base + (TR ? k * 5 + o : o * 5 + k), soff5);
      }
    }
  if constexpr (!TR) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int o = 4 * h + j < 5 ? 4 * h + j : 4;
      ld_coef4<TB>(rs, (5 * gb + o) * 4, soff2, &c.v[20 + 4 * h]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 5; ++k) ld_coef4<TB>(rs, (5 * gb + k) * 4, soff2, &c.v[20 + 4 * k]);
  }
}

template <class Lay, bool TR>
__device__ __forceinline__ void tail_round(float* tile, int g, const Cbuf& c, int j) {
  constexpr int PLANE = 4 * Lay::units(5120);
  const int col0 = 10 * g;
  float x[2][2][5];   // [q][d4][d3]: row 4q + j, column col0 + 2 d3 + d4
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int k = 0; k < 5; ++k)
#pragma unroll
      for (int d4 = 0; d4 < 2; ++d4) x[q][d4][k] = tile[4 * Lay::unit(col0 + 2 * k + d4) + j + PLANE * q];
  if constexpr (TR) {
    // inverse: transposed 2 x 2 blocks first, z[e] = sum_d G[d][e] x[d]
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int k = 0; k < 5; ++k) {
        const float* G = &c.v[20 + 4 * k];
        const float a = x[q][0][k], b = x[q][1][k];
        x[q][0][k] = G[0] * a + G[2] * b;
        x[q][1][k] = G[1] * a + G[3] * b;
      }
  }
  // D[i][jj] = x[row 4q + i][(k, d4)] * C5[4h + jj][k]
  f32x4 acc[2][2][2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int d4 = 0; d4 < 2; ++d4)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        acc[q][d4][h] = __builtin_amdgcn_mfma_f32_4x4x1f32(x[q][d4][0], c.v[(d4 * 2 + h) * 5], f32x4{0.f, 0.f, 0.f, 0.f},
                                                           0, 0, 0);
#pragma unroll
  for (int k = 1; k < 5; ++k)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int d4 = 0; d4 < 2; ++d4)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc[q][d4][h] = __builtin_amdgcn_mfma_f32_4x4x1f32(x[q][d4][k], c.v[(d4 * 2 + h) * 5 + k], acc[q][d4][h], 0, 0, 0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int o = 4 * h + j;   // this lane's radix-5 output
    if (o < 5) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        f32x4 z0 = acc[q][0][h], z1 = acc[q][1][h];
        if constexpr (!TR) {
          // forward: 2 x 2 block of column o on the pair (d4 = 0, 1)
          const float* G = &c.v[20 + 4 * h];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a = acc[q][0][h][i], b = acc[q][1][h][i];
            z0[i] = G[0] * a + G[1] * b;
            z1[i] = G[2] * a + G[3] * b;
          }
        }
        *reinterpret_cast<f32x4*>(tile + 4 * Lay::unit(col0 + 2 * o) + PLANE * q) = z0;
        *reinterpret_cast<f32x4*>(tile + 4 * Lay::unit(col0 + 2 * o + 1) + PLANE * q) = z1;
      }
    }
  }
}

constexpr int k5CW = 8;                       // compute waves
constexpr int k5IOW = 4;                      // data waves
constexpr int k5Threads = 64 * (k5CW + k5IOW);

// One radix-8 stage of the 5120 kernel (5 rounds, stride S, stage params sd),
// coefficient buffers alternating; on exit the next stage's first round is in
// the buffer given by the round parity.
template <class Lay, int S, bool TR, typename TB, typename NextLoad>
__device__ __forceinline__ void stage8_5120(const RowParams& p, float* tile, const StageFast& sd, Cbuf& X, Cbuf& Y,
                                            int gb, int j, NextLoad next) {
  using Sch = Sched<5120, Lay, List<St<8, S>>>;
  const __amdgpu_buffer_rsrc_t rs = coef_rsrc(p);
  // rounds 0..4: X holds round 0
  load_coef<8, TB, TR>(rs, sd, 1 * kGPR, gb, j, as8(Y));
  round_compute<Sch, 8, S, TR, false, uint16_t>(p, tile, 0 * kGPR + gb, as8(X), 0, 0, j);
  load_coef<8, TB, TR>(rs, sd, 2 * kGPR, gb, j, as8(X));
  round_compute<Sch, 8, S, TR, false, uint16_t>(p, tile, 1 * kGPR + gb, as8(Y), 0, 0, j);
  load_coef<8, TB, TR>(rs, sd, 3 * kGPR, gb, j, as8(Y));
  round_compute<Sch, 8, S, TR, false, uint16_t>(p, tile, 2 * kGPR + gb, as8(X), 0, 0, j);
  load_coef<8, TB, TR>(rs, sd, 4 * kGPR, gb, j, as8(X));
  round_compute<Sch, 8, S, TR, false, uint16_t>(p, tile, 3 * kGPR + gb, as8(Y), 0, 0, j);
  next(Y);   // the next stage's round 0 goes to Y
  round_compute<Sch, 8, S, TR, false, uint16_t>(p, tile, 4 * kGPR + gb, as8(X), 0, 0, j);
  __syncthreads();
}

template <class Lay, bool TR, typename TB, typename NextLoad>
__device__ __forceinline__ void stage_tail_5120(const RowParams& p, float* tile, const StageFast& s5,
                                                const StageFast& s2, Cbuf& X, Cbuf& Y, int gb, int j,
                                                NextLoad next) {
  const __amdgpu_buffer_rsrc_t rs = coef_rsrc(p);
  // rounds 0..3: X holds round 0
  load_tail<TB, TR>(rs, s5, s2, 1 * kGPR, gb, j, Y);
  tail_round<Lay, TR>(tile, 0 * kGPR + gb, X, j);
  load_tail<TB, TR>(rs, s5, s2, 2 * kGPR, gb, j, X);
  tail_round<Lay, TR>(tile, 1 * kGPR + gb, Y, j);
  load_tail<TB, TR>(rs, s5, s2, 3 * kGPR, gb, j, Y);
  tail_round<Lay, TR>(tile, 2 * kGPR + gb, X, j);
  next(X);   // the next stage's round 0 goes to X
  tail_round<Lay, TR>(tile, 3 * kGPR + gb, Y, j);
  __syncthreads();
}

// Stage parameters p.st[] are in processing order: forward 640, 80, 10,
// radix 5, radix 2; inverse radix 2, radix 5, 10, 80, 640.
template <bool TR, typename T, typename TB>
__global__ void __launch_bounds__(k5Threads) apply_5120_kernel(RowParams p) {
  using Lay = LayXor;
  extern __shared__ float tile[];
  int64_t tix = blockIdx.x;
  if (tix >= p.ntiles) return;   // uniform per workgroup
  if (threadIdx.x >= 64 * k5CW) {
    // 2 x 640 (bf16) or 2 x 1280 (fp32) micro-blocks over 256 data threads
    constexpr bool F = std::is_same<T, float>::value;
    data_waves_exact<T, Lay, 64 * k5IOW, F ? 10 : 5, F ? 4 : 5, 4, false, true>(p, tile, threadIdx.x - 64 * k5CW);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int gb = wave * 16 + (lane >> 2);
  int j = lane & 3;
  const __amdgpu_buffer_rsrc_t rs = coef_rsrc(p);
  Cbuf ca, cb;
  if constexpr (!TR) load_coef<8, TB, TR>(rs, p.st[0], 0, gb, j, as8(ca));
  else load_tail<TB, TR>(rs, p.st[1], p.st[0], 0, gb, j, ca);
  __syncthreads();
  // The loop body covers two tiles: the first starts from ca, the second from
  // cb (where the first tile's last stage leaves the next tile's first round).
  // Every tile ends with the barrier after which the data waves have written
  // the next tile, also the last one, so both roles pass the same barriers.
  while (true) {
    // keep per-round addresses inside the loop (hoisting them all out of it
    // would exhaust the registers)
    asm volatile("" : "+v"(gb), "+v"(j));
    if constexpr (!TR) {
      stage8_5120<Lay, 640, TR, TB>(p, tile, p.st[0], ca, cb, gb, j,
                                    [&](Cbuf& d) { load_coef<8, TB, TR>(rs, p.st[1], 0, gb, j, as8(d)); });
      stage8_5120<Lay, 80, TR, TB>(p, tile, p.st[1], cb, ca, gb, j,
                                   [&](Cbuf& d) { load_coef<8, TB, TR>(rs, p.st[2], 0, gb, j, as8(d)); });
      stage8_5120<Lay, 10, TR, TB>(p, tile, p.st[2], ca, cb, gb, j,
                                   [&](Cbuf& d) { load_tail<TB, TR>(rs, p.st[3], p.st[4], 0, gb, j, d); });
      stage_tail_5120<Lay, TR, TB>(p, tile, p.st[3], p.st[4], cb, ca, gb, j,
                                   [&](Cbuf& d) { load_coef<8, TB, TR>(rs, p.st[0], 0, gb, j, as8(d)); });
    } else {
      stage_tail_5120<Lay, TR, TB>(p, tile, p.st[1], p.st[0], ca, cb, gb, j,
                                   [&](Cbuf& d) { load_coef<8, TB, TR>(rs, p.st[2], 0, gb, j, as8(d)); });
      stage8_5120<Lay, 10, TR, TB>(p, tile, p.st[2], ca, cb, gb, j,
                                   [&](Cbuf& d) { load_coef<8, TB, TR>(rs, p.st[3], 0, gb, j, as8(d)); });
      stage8_5120<Lay, 80, TR, TB>(p, tile, p.st[3], cb, ca, gb, j,
                                   [&](Cbuf& d) { load_coef<8, TB, TR>(rs, p.st[4], 0, gb, j, as8(d)); });
      stage8_5120<Lay, 640, TR, TB>(p, tile, p.st[4], ca, cb, gb, j,
                                    [&](Cbuf& d) { load_tail<TB, TR>(rs, p.st[1], p.st[0], 0, gb, j, d); });
    }
    __syncthreads();   // data waves have swapped the tile
    tix += gridDim.x;
    if (tix >= p.ntiles) break;
    asm volatile("" : "+v"(gb), "+v"(j));
    if constexpr (!TR) {
      stage8_5120<Lay, 640, TR, TB>(p, tile, p.st[0], cb, ca, gb, j,
                                    [&](Cbuf& d) { load_coef<8, TB, TR>(rs, p.st[1], 0, gb, j, as8(d)); });
      stage8_5120<Lay, 80, TR, TB>(p, tile, p.st[1], ca, cb, gb, j,
                                   [&](Cbuf& d) { load_coef<8, TB, TR>(rs, p.st[2], 0, gb, j, as8(d)); });
      stage8_5120<Lay, 10, TR, TB>(p, tile, p.st[2], cb, ca, gb, j,
                                   [&](Cbuf& d) { load_tail<TB, TR>(rs, p.st[3], p.st[4], 0, gb, j, d); });
      stage_tail_5120<Lay, TR, TB>(p, tile, p.st[3], p.st[4], ca, cb, gb, j,
                                   [&](Cbuf& d) { load_coef<8, TB, TR>(rs, p.st[0], 0, gb, j, as8(d)); });
    } else {
      stage_tail_5120<Lay, TR, TB>(p, tile, p.st[1], p.st[0], cb, ca, gb, j,
                                   [&](Cbuf& d) { load_coef<8, TB, TR>(rs, p.st[2], 0, gb, j, as8(d)); });
      stage8_5120<Lay, 10, TR, TB>(p, tile, p.st[2], cb, ca, gb, j,
                                   [&](Cbuf& d) { load_coef<8, TB, TR>(rs, p.st[3], 0, gb, j, as8(d)); });
      stage8_5120<Lay, 80, TR, TB>(p, tile, p.st[3], ca, cb, gb, j,
                                   [&](Cbuf& d) { load_coef<8, TB, TR>(rs, p.st[4], 0, gb, j, as8(d)); });
      stage8_5120<Lay, 640, TR, TB>(p, tile, p.st[4], cb, ca, gb, j,
                                    [&](Cbuf& d) { load_tail<TB, TR>(rs, p.st[1], p.st[0], 0, gb, j, d); });
    }
    __syncthreads();   // data waves have swapped the tile
    tix += gridDim.x;
    if (tix >= p.ntiles) break;
  }
}

// Compile-time schedules (processing order; the inverse runs the stages in
// reverse).  d = 4096 uses the padded layout (147 KiB of LDS); d = 5120 fills
// the 160 KiB LDS exactly and keeps the unpadded XOR layout.
using F4096 = Sched<4096, LayPad8, List<St<8, 512>, St<8, 64>, St<8, 8>, St<8, 1>>>;
using I4096 = Sched<4096, LayPad8, List<St<8, 1>, St<8, 8>, St<8, 64>, St<8, 512>>>;

static_assert(linear_stage<LayPad8, 4096, 8, 512>() && linear_stage<LayPad8, 4096, 8, 64>() &&
                  linear_stage<LayPad8, 4096, 8, 8>() && linear_stage<LayPad8, 4096, 8, 1>(),
              "padded layout must give constant column offsets for d = 4096, (8,8,8,8)");

template <class Sch, bool TR, bool DOUT, typename T, typename TB>
hipError_t launch_sched(const RowParams& p, int grid, hipStream_t st) {
  void (*kern)(RowParams) = apply_pipe_kernel<Sch, TR, DOUT, T, TB>;
  const size_t lds = (size_t)kRows * 4 * Sch::Lay::units(Sch::D);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kPThreads), lds, st, p);
  return hipGetLastError();
}

template <class F, class I, typename T, typename TB>
hipError_t launch_pair(const RowParams& p, int grid, hipStream_t st) {
  using Last = typename At<F::M - 1, typename F::L>::type;
  if (p.transpose) return launch_sched<I, true, false, T, TB>(p, grid, st);
  if constexpr (Last::B == 8 && Last::S == 1) {
    if (p.direct_out) return launch_sched<F, false, true, T, TB>(p, grid, st);
  }
  return launch_sched<F, false, false, T, TB>(p, grid, st);
}

template <typename T, typename TB>
hipError_t launch_5120(const RowParams& p, int grid, hipStream_t st) {
  void (*kern)(RowParams) = p.transpose ? apply_5120_kernel<true, T, TB> : apply_5120_kernel<false, T, TB>;
  const size_t lds = (size_t)kRows * 4 * LayXor::units(5120);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(k5Threads), lds, st, p);
  return hipGetLastError();
}

template <typename T, typename TB>
hipError_t launch_d(int d, const RowParams& p, int grid, hipStream_t st) {
  return d == 4096 ? launch_pair<F4096, I4096, T, TB>(p, grid, st) : launch_5120<T, TB>(p, grid, st);
}

}  // namespace

bool fast_path_supported(const Plan& pl, DT bdt) {
  if (bdt != DT::F32 && bdt != DT::BF16) return false;
  static const int r4096[] = {8, 8, 8, 8};
  static const int r5120[] = {8, 8, 8, 5, 2};
  const int* want = pl.d == 4096 ? r4096 : (pl.d == 5120 ? r5120 : nullptr);
  const int m = pl.d == 4096 ? 4 : 5;
  if (want == nullptr || pl.m != m) return false;
  for (int t = 0; t < m; ++t)
    if (pl.radix[t] != want[t]) return false;
  return true;
}

hipError_t launch_apply_fast(const Plan& pl, bool inverse, const void* blocks, DT bdt, const int8_t* signs,
                             const void* x, int64_t ldx, DT io, void* y, int64_t ldy, int64_t rows,
                             hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  RowParams p = make_row_params(pl, inverse, blocks, nullptr, signs, x, ldx, io, y, ldy, rows);
  int64_t grid = cu_count();
  if (grid > p.ntiles) grid = p.ntiles;
  const int d = (int)pl.d;
  if (io == DT::BF16)
    return bdt == DT::F32 ? launch_d<uint16_t, float>(d, p, (int)grid, stream)
                          : launch_d<uint16_t, uint16_t>(d, p, (int)grid, stream);
  return bdt == DT::F32 ? launch_d<float, float>(d, p, (int)grid, stream)
                        : launch_d<float, uint16_t>(d, p, (int)grid, stream);
}

}  // namespace harp
