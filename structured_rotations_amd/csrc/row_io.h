// Row-tile plumbing shared by the gfx950 row kernels (matrix-core and
// vector-ALU variants): the per-stage descriptors, the swizzled LDS tile
// layout, and the data waves that stream rows between HBM and LDS.
#pragma once

#include "common.h"
#include "kernels.h"

namespace harp {
namespace rowk {

constexpr int kRows = 8;   // rows per tile (two row quads)


struct StageFast {
  int b;
  int s;
  int G;            // groups = d / b
  int blk_off;
  int grp_off;
  uint64_t div_s;   // floor(2^32 / s) + 1: n / s == (n * div_s) >> 32 for n, s < 2^16
  uint64_t div_b;
  uint32_t mag_s;   // low 32 bits of div_s: n / s == umulhi(n, mag_s) for s >= 2 and n, s < 2^16
};

struct RowParams {
  int d;
  int m;
  int transpose;
  int sign_mode;     // 0 none, 1 on input, 2 on output
  int chunks;        // 16-byte chunks per row
  int direct_out;    // last stage stores straight to HBM
  StageFast st[kMaxStagesDev];
  const void* blocks;
  const float* scales;
  const int8_t* signs;
  const void* x;
  int64_t ldx;
  void* y;
  int64_t ldy;
  int64_t rows;
  int64_t ntiles;
};

__device__ __forceinline__ int fdiv(int n, uint64_t magic) { return (int)(((uint64_t)(uint32_t)n * magic) >> 32); }
// LDS layout (one order for every stage, so each stage updates the tile in
// place): two row-quad planes, plane q (rows 4q..4q+3) at q * 4d floats; in
// a plane, column c's 4 rows form one 16-byte unit at unit index pcol(c).
// pcol XORs bits 0..3 of c with bits 3..6 (bijective inside every 16
// columns); for digit strides 512, 64, 8 and 1 the 4-byte gathers of a wave
// hit every bank once.
__device__ __forceinline__ int pcol(int c) { return c ^ ((c >> 3) & 15); }

// Unit layouts of a row-quad plane: unit(c) is the 16-byte unit of column c,
// units(d) the plane size in units.
struct LayXor {   // the swizzle above, no padding (fits 8 rows of d = 5120)
  __host__ __device__ static constexpr int unit(int c) { return c ^ ((c >> 3) & 15); }
  __host__ __device__ static constexpr int units(int d) { return d; }
};
struct LayPad8 {  // one padding unit after every 8 columns
  __host__ __device__ static constexpr int unit(int c) { return c + (c >> 3); }
  __host__ __device__ static constexpr int units(int d) { return d + d / 8; }
};

template <typename T> struct Io;
template <> struct Io<uint16_t> { static constexpr int V = 8; };
template <> struct Io<float> { static constexpr int V = 4; };

__device__ __forceinline__ float sgnf(float v, uint32_t negbit) { return __uint_as_float(__float_as_uint(v) ^ negbit); }

template <typename T>
__device__ __forceinline__ float elem(const u32x4& w, int u);
template <>
__device__ __forceinline__ float elem<uint16_t>(const u32x4& w, int u) {
  const uint32_t word = u < 2 ? w.x : (u < 4 ? w.y : (u < 6 ? w.z : w.w));
  return (u & 1) ? bf16_hi(word) : bf16_lo(word);
}
template <>
__device__ __forceinline__ float elem<float>(const u32x4& w, int u) {
  return __uint_as_float(u == 0 ? w.x : (u == 1 ? w.y : (u == 2 ? w.z : w.w)));
}

template <typename T>
__device__ __forceinline__ u32x4 pack_row(const float* v);
template <>
__device__ __forceinline__ u32x4 pack_row<uint16_t>(const float* v) {
  return u32x4{pack_bf16x2_hw(v[0], v[1]), pack_bf16x2_hw(v[2], v[3]), pack_bf16x2_hw(v[4], v[5]),
               pack_bf16x2_hw(v[6], v[7])};
}
template <>
__device__ __forceinline__ u32x4 pack_row<float>(const float* v) {
  return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
}

// ---------------------------------------------------------------- data waves
// Micro-block mb = (row quad q, 16-byte chunk c): rows 4q..4q+3 x V columns,
// plus the V sign bytes of those columns (zero = no flip).
struct IoBlock {
  u32x4 w[4];
  uint2 sg;
};

template <typename T>
__device__ __forceinline__ void io_load(const RowParams& p, int64_t row0, int nr, int q, int c, IoBlock& blk) {
  constexpr int V = Io<T>::V;
  const T* x = static_cast<const T*>(p.x);
  // rows past the end of a ragged last tile re-read the last row: they are
  // transformed like the others but never stored
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * q + i < nr ? 4 * q + i : nr - 1;
    blk.w[i] = ld_stream(x + (row0 + r) * p.ldx + (int64_t)c * V);
  }
  blk.sg = uint2{0u, 0u};
  if (p.sign_mode == 1) {
    const int8_t* sp = p.signs + c * V;
    if constexpr (V == 8) blk.sg = *reinterpret_cast<const uint2*>(sp);
    else blk.sg.x = *reinterpret_cast<const uint32_t*>(sp);
  }
}

template <typename T>
__device__ __forceinline__ f32x4 io_column(const IoBlock& blk, int u) {
  // sign byte u (0x01 or 0xff): bit 7 set for -1
  const uint32_t neg = (((u < 4 ? blk.sg.x : blk.sg.y) >> (8 * (u & 3))) & 0x80u) << 24;
  f32x4 v;
  v.x = sgnf(elem<T>(blk.w[0], u), neg); v.y = sgnf(elem<T>(blk.w[1], u), neg);
  v.z = sgnf(elem<T>(blk.w[2], u), neg); v.w = sgnf(elem<T>(blk.w[3], u), neg);
  return v;
}

// Writes a micro-block (rows 4q..4q+3 of the V columns of chunk c).  The
// chunk's columns c*V + u share bits 3..6 (V <= 8 and chunks are aligned), so
// their units are (c*V ^ m) ^ u with one mask m.
template <typename T, class Lay = LayXor>
__device__ __forceinline__ void io_to_lds(const RowParams& p, float* tile, int q, int c, const IoBlock& blk) {
  constexpr int V = Io<T>::V;
  float* plane = tile + q * 4 * Lay::units(p.d);
#pragma unroll
  for (int u = 0; u < V; ++u)
    *reinterpret_cast<f32x4*>(plane + 4 * Lay::unit(c * V + u)) = io_column<T>(blk, u);
}

template <typename T, class Lay = LayXor>
__device__ __forceinline__ void io_store(const RowParams& p, const float* tile, int64_t row0, int nr, int q, int c) {
  constexpr int V = Io<T>::V;
  T* y = static_cast<T*>(p.y);
  const float* plane = tile + q * 4 * Lay::units(p.d);
  float v[4][V];
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int col = c * V + u;
    f32x4 t = *reinterpret_cast<const f32x4*>(plane + 4 * Lay::unit(col));
    if (p.sign_mode == 2 && p.signs[col] < 0) {
      t.x = -t.x; t.y = -t.y; t.z = -t.z; t.w = -t.w;
    }
    v[0][u] = t.x; v[1][u] = t.y; v[2][u] = t.z; v[3][u] = t.w;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * q + i;
    if (r < nr) st_stream(y + (row0 + r) * p.ldy + (int64_t)c * V, pack_row<T>(v[i]));
  }
}

__device__ __forceinline__ int tile_rows(const RowParams& p, int64_t tix) {
  const int64_t left = p.rows - tix * kRows;
  return left < kRows ? (int)left : kRows;
}

// Data waves (threads it = 0 .. kIoThreads-1 of the data role).  They load the
// workgroup's first tile into LDS; then, for every tile, they stream the next
// tile into registers while the compute waves run the m stages, copy the
// finished tile out (unless the compute waves stored the last stage straight
// to HBM), and write the prefetched tile into LDS.  Barriers per tile:
// m + (direct_out ? 0 : 1) + 1, after one initial barrier; the compute waves
// pass the same sequence.
template <typename T, int kIoThreads, int kMaxIo, class Lay = LayXor>
__device__ __forceinline__ void data_waves(const RowParams& p, float* tile, int it) {
  int64_t tix = blockIdx.x;
  IoBlock pf[2][kMaxIo];
  {
    const int nr = tile_rows(p, tix);
    for (int q = 0; q < 2; ++q)
      for (int c = it; c < p.chunks; c += kIoThreads) {
        IoBlock one;
        io_load<T>(p, tix * kRows, nr, q, c, one);
        io_to_lds<T, Lay>(p, tile, q, c, one);
      }
  }
  __syncthreads();
  for (; tix < p.ntiles; tix += gridDim.x) {
    const int64_t row0 = tix * kRows;
    const int nr = tile_rows(p, tix);
    const int64_t nxt = tix + gridDim.x;
    const bool has_next = nxt < p.ntiles;
    const int nr_next = has_next ? tile_rows(p, nxt) : 0;
    if (has_next) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int u = 0; u < kMaxIo; ++u) {
          const int c = it + u * kIoThreads;
          if (c < p.chunks) io_load<T>(p, nxt * kRows, nr_next, q, c, pf[q][u]);
        }
    }
    for (int t = 0; t < p.m; ++t) __syncthreads();
    if (!p.direct_out) {
      for (int q = 0; q < 2; ++q)
        for (int c = it; c < p.chunks; c += kIoThreads) io_store<T, Lay>(p, tile, row0, nr, q, c);
      __syncthreads();
    }
    if (has_next) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int u = 0; u < kMaxIo; ++u) {
          const int c = it + u * kIoThreads;
          if (c < p.chunks) io_to_lds<T, Lay>(p, tile, q, c, pf[q][u]);
        }
      for (int q = 0; q < 2; ++q)
        for (int c = it + kMaxIo * kIoThreads; c < p.chunks; c += kIoThreads) {
          IoBlock one;
          io_load<T>(p, nxt * kRows, nr_next, q, c, one);
          io_to_lds<T, Lay>(p, tile, q, c, one);
        }
    }
    __syncthreads();
  }
}

// Data waves with a fixed amount of memory work per tile.  The 2 x chunks
// micro-blocks of a tile (row quad q, chunk c) are split evenly: data thread
// it owns slots s = 0 .. NS-1, micro-block it + s * kIoT (the caller makes
// 2 * chunks == NS * kIoT).  Slots 0 .. NP-1 of the next tile are prefetched
// into registers while the compute waves run; the rest are loaded at the
// swap, two at a time.  Rows past a ragged tile are clamped to its last row
// (they hold that row's values), so every load and store is unconditional and
// the waits count exactly.  Per tile the compute waves pass NB barriers (the
// last one after their last stage); then each data thread, slot by slot,
// stores its finished micro-block row by row (unless DOUT: the compute waves
// stored the result) and writes the next tile's micro-block over it; the
// stores are issued after every load the swap waits for except the later
// slots' prefetches, so each wait counts them exactly.  One more barrier
// releases the compute waves.
template <typename T, class Lay, int kIoT, int NS, int NP, int NB, bool DOUT, bool SPREAD>
__device__ __forceinline__ void data_waves_exact(const RowParams& p, float* tile, int it) {
  constexpr int V = Io<T>::V;
  static_assert(NP <= NS && (NS - NP) % 2 == 0, "synchronous slots go in pairs");
  int64_t tix = blockIdx.x;
  int qs[NS], cs[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int i = it + u * kIoT;
    qs[u] = i >= p.chunks ? 1 : 0;
    cs[u] = i - qs[u] * p.chunks;
  }
  {
    const int nr = tile_rows(p, tix);
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      IoBlock one;
      io_load<T>(p, tix * kRows, nr, qs[u], cs[u], one);
      io_to_lds<T, Lay>(p, tile, qs[u], cs[u], one);
    }
  }
  __syncthreads();
  IoBlock pf[NP > 0 ? NP : 1];
  for (; tix < p.ntiles; tix += gridDim.x) {
    // recompute the slot addresses every tile instead of keeping them all
    // live across the loop
#pragma unroll
    for (int u = 0; u < NS; ++u) asm volatile("" : "+v"(qs[u]), "+v"(cs[u]));
    const int64_t row0 = tix * kRows;
    const int nr = tile_rows(p, tix);
    const int64_t nxt = tix + gridDim.x;
    const bool has_next = nxt < p.ntiles;
    const int nr_next = has_next ? tile_rows(p, nxt) : 1;
    uint2 osg[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      osg[u] = uint2{0u, 0u};
      if (!DOUT && p.sign_mode == 2) {
        const int8_t* sp = p.signs + cs[u] * V;
        if constexpr (V == 8) osg[u] = *reinterpret_cast<const uint2*>(sp);
        else osg[u].x = *reinterpret_cast<const uint32_t*>(sp);
      }
    }
    // SPREAD: the prefetch is spread over the stages (slot u goes out after
    // barrier u * NB / NP), so that not a whole tile of loads sits in the
    // vector cache's miss queue at once, in front of the compute waves'
    // coefficient reads; otherwise it all goes out at the tile start.
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int u = 0; u < NP; ++u)
        if ((SPREAD ? u * NB / NP : 0) == b && has_next) io_load<T>(p, nxt * kRows, nr_next, qs[u], cs[u], pf[u]);
      __syncthreads();
    }
    // one slot: read the finished micro-block, write the next one in its
    // place, store the finished one
    auto swap = [&](int u, const IoBlock& nb) {
      if constexpr (!DOUT) {
        T* y = static_cast<T*>(p.y);
        const float* plane = tile + qs[u] * 4 * Lay::units(p.d);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v[V];
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const uint32_t neg = (((e < 4 ? osg[u].x : osg[u].y) >> (8 * (e & 3))) & 0x80u) << 24;
            v[e] = sgnf(plane[4 * Lay::unit(cs[u] * V + e) + i], neg);
          }
          const int r = 4 * qs[u] + i < nr ? 4 * qs[u] + i : nr - 1;
          st_stream(y + (row0 + r) * p.ldy + (int64_t)cs[u] * V, pack_row<T>(v));
        }
      }
      if (has_next) io_to_lds<T, Lay>(p, tile, qs[u], cs[u], nb);
    };
#pragma unroll
    for (int u = 0; u < NP; ++u) swap(u, pf[u]);
#pragma unroll
    for (int u = NP; u < NS; u += 2) {
      IoBlock a, b;
      if (has_next) {
        io_load<T>(p, nxt * kRows, nr_next, qs[u], cs[u], a);
        io_load<T>(p, nxt * kRows, nr_next, qs[u + 1], cs[u + 1], b);
      }
      swap(u, a);
      swap(u + 1, b);
    }
    __syncthreads();
  }
}

// Stores micro-block `blk` (row quad blk / chunks, chunk blk % chunks) of the
// finished tile to y, the inverse's row signs applied on the way.  Rows past a
// ragged tile are clamped to its last row (the same values to the same
// address).
template <typename T, class Lay>
__device__ __forceinline__ void io_copy_out(const RowParams& p, const float* tile, int64_t row0, int nr, int blk) {
  constexpr int V = Io<T>::V;
  const int q = blk >= p.chunks ? 1 : 0;
  const int c = blk - q * p.chunks;
  uint2 osg = uint2{0u, 0u};
  if (p.sign_mode == 2) {
    const int8_t* sp = p.signs + c * V;
    if constexpr (V == 8) osg = *reinterpret_cast<const uint2*>(sp);
    else osg.x = *reinterpret_cast<const uint32_t*>(sp);
  }
  T* y = static_cast<T*>(p.y);
  const float* plane = tile + q * 4 * Lay::units(p.d);
  f32x4 col[V];
#pragma unroll
  for (int e = 0; e < V; ++e) col[e] = *reinterpret_cast<const f32x4*>(plane + 4 * Lay::unit(c * V + e));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const uint32_t neg = (((e < 4 ? osg.x : osg.y) >> (8 * (e & 3))) & 0x80u) << 24;
      v[e] = sgnf(col[e][i], neg);
    }
    const int r = 4 * q + i < nr ? 4 * q + i : nr - 1;
    st_stream(y + (row0 + r) * p.ldy + (int64_t)c * V, pack_row<T>(v));
  }
}

// The compute waves' part of a shared copy-out (see data_waves_shared_out):
// compute thread t stores micro-blocks t + k * NCT, k < KC, then the barrier
// after which the data waves overwrite the tile.
template <typename T, class Lay, int NCT, int KC>
__device__ __forceinline__ void compute_copy_out(const RowParams& p, const float* tile, int64_t tix, int t) {
  const int nr = tile_rows(p, tix);
#pragma unroll
  for (int k = 0; k < KC; ++k) io_copy_out<T, Lay>(p, tile, tix * kRows, nr, t + k * NCT);
  __syncthreads();
}

// Data waves that share the copy-out of the finished tile with the compute
// waves, which would otherwise wait at the swap barrier: every slot of the
// next tile is prefetched into registers over the NB stage barriers (NS slots
// per thread, 2 * chunks == NS * kIoT); after the last stage the compute
// threads store micro-blocks 0 .. CB-1 (compute_copy_out) and data thread it
// stores CB + it + k * kIoT, refilling each at once; one barrier, then the
// rest of the prefetched tile goes into LDS and one more barrier releases
// the compute waves.  Barriers per tile:
// NB + 2, after one initial barrier.  SPREAD: slot u of the prefetch goes out
// after barrier u * NB / NS (spread over the stages), else all at the tile start.
template <typename T, class Lay, int kIoT, int NS, int NB, int CB, bool SPREAD>
__device__ __forceinline__ void data_waves_shared_out(const RowParams& p, float* tile, int it) {
  static_assert(CB % kIoT == 0 && CB <= NS * kIoT, "the data threads' share is whole rounds of micro-blocks");
  constexpr int ND = (NS * kIoT - CB) / kIoT;
  int64_t tix = blockIdx.x;
  int qs[NS], cs[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int i = it + u * kIoT;
    qs[u] = i >= p.chunks ? 1 : 0;
    cs[u] = i - qs[u] * p.chunks;
  }
  {
    const int nr = tile_rows(p, tix);
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      IoBlock one;
      io_load<T>(p, tix * kRows, nr, qs[u], cs[u], one);
      io_to_lds<T, Lay>(p, tile, qs[u], cs[u], one);
    }
  }
  __syncthreads();
  IoBlock pf[NS];
  for (; tix < p.ntiles; tix += gridDim.x) {
#pragma unroll
    for (int u = 0; u < NS; ++u) asm volatile("" : "+v"(qs[u]), "+v"(cs[u]));
    const int64_t row0 = tix * kRows;
    const int nr = tile_rows(p, tix);
    const int64_t nxt = tix + gridDim.x;
    const bool has_next = nxt < p.ntiles;
    const int nr_next = has_next ? tile_rows(p, nxt) : 1;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int u = 0; u < NS; ++u)
        if ((SPREAD ? u * NB / NS : 0) == b && has_next) io_load<T>(p, nxt * kRows, nr_next, qs[u], cs[u], pf[u]);
      __syncthreads();
    }
    // the data thread's own micro-blocks are its slots U0 .. NS-1: each is
    // refilled right after it is stored, the compute waves' ones after the
    // barrier that ends their copy-out
    constexpr int U0 = CB / kIoT;
#pragma unroll
    for (int k = 0; k < ND; ++k) {
      io_copy_out<T, Lay>(p, tile, row0, nr, CB + it + k * kIoT);
      if (has_next) io_to_lds<T, Lay>(p, tile, qs[U0 + k], cs[U0 + k], pf[U0 + k]);
    }
    __syncthreads();
    if (has_next) {
#pragma unroll
      for (int u = 0; u < U0; ++u) io_to_lds<T, Lay>(p, tile, qs[u], cs[u], pf[u]);
    }
    __syncthreads();
  }
}

// Host side: kernel parameters for rows of length pl.d (stages in processing
// order, reversed for the inverse).
inline RowParams make_row_params(const Plan& pl, bool inverse, const void* blocks, const float* scales,
                                 const int8_t* signs, const void* x, int64_t ldx, DT io, void* y, int64_t ldy,
                                 int64_t rows) {
  RowParams p{};
  p.d = (int)pl.d;
  p.m = pl.m;
  p.transpose = inverse ? 1 : 0;
  p.sign_mode = signs ? (inverse ? 2 : 1) : 0;
  for (int i = 0; i < pl.m; ++i) {
    const int t = inverse ? pl.m - 1 - i : i;
    StageFast& sf = p.st[i];
    sf.b = pl.radix[t];
    sf.s = (int)pl.stride[t];
    sf.G = (int)(pl.d / sf.b);
    sf.blk_off = (int)pl.blk_off[t];
    sf.grp_off = (int)pl.grp_off[t];
    sf.div_s = (uint64_t)((1ull << 32) / (uint64_t)sf.s) + 1ull;
    sf.div_b = (uint64_t)((1ull << 32) / (uint64_t)sf.b) + 1ull;
    sf.mag_s = (uint32_t)sf.div_s;
  }
  const StageFast& last = p.st[pl.m - 1];
  p.direct_out = (last.s == 1 && last.b == 8 && p.sign_mode != 2) ? 1 : 0;
  p.chunks = (int)(pl.d / (io == DT::BF16 ? 8 : 4));
  p.blocks = blocks;
  p.scales = scales;
  p.signs = signs;
  p.x = x;
  p.ldx = ldx;
  p.y = y;
  p.ldy = ldy;
  p.rows = rows;
  p.ntiles = (rows + kRows - 1) / kRows;
  return p;
}

inline int cu_count() {
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

}  // namespace rowk
}  // namespace harp
