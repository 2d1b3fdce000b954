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
  uint32_t mag_b, mag_bb;   // ceil(2^32 / b), ceil(2^32 / b^2) (see udiv)
  uint32_t mag_ls;          // same for ls (0 for ls = 1)
  int ncu;                  // coefficient slots per thread: ceil(nsub * b / 512)
  int nq;                   // quad path (b even, blk_off a multiple of 4; the kernels that
                            // compile it in): 4-element quads per thread,
                            // ceil(nsub * b / 2048); 0 for the one-element path
};

struct ColParams {
  int nsub;          // rows per tile: product of the run's radices
  int nstage;        // stages in the run (processing order in st[])
  int pw;            // panel width (columns per tile)
  int cslot;         // floats of one coefficient slot in LDS (nsub * widest padded row)
  int transpose;     // inverse: transposed blocks
  int sign_mode;     // 0 none, 1 on the input of the first stage, 2 on the output of the last
  int64_t suf;       // product of the radices after the run
  int64_t npanels;
  int64_t ntiles;    // (d / nsub) * npanels
  int64_t ncols;
  int vec;           // 16-byte row segments and whole panels: aligned bases, ld and widths
  int split_swap;    // store every finished chunk before any incoming one is written: chunk
                     // slots wrap around (some chunks have two owners), or an output chunk is
                     // made of two input chunks of different threads (fp32 in, bf16 out)
  uint32_t mag_ncb;  // ceil(2^32 / (pw / 64)) (0 for one block)
  uint32_t mag_cpr;  // same for the input chunks per tile row, pw / (16 / input element bytes)
  uint32_t mag_tot;  // same for the input chunks per tile, nsub * pw / (16 / input element bytes)
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

// e / d for 0 <= e < 2^16 with mag = ceil(2^32 / d) (d >= 2), or mag = 0 for d = 1
__device__ __forceinline__ int udiv(int e, uint32_t mag) { return mag ? (int)__umulhi((uint32_t)e, mag) : e; }

// Row stride of a staged block in LDS: each output row of C starts on a
// 16-byte boundary so a task reads it with 128-bit broadcast loads.
template <int B>
constexpr int coef_row_stride() { return (B + 3) & ~3; }

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

// Coefficients of one stage of one tile, C[o][k] (C = B forward, B^T
// inverse), fetched into registers a stage ahead as the stored words (fp32
// bits, bf16 bits, or int8 code and its fp32 scale); coef_put turns them into
// fp32.  Thread t fetches elements e = t + u * 512 of the ngl * b * b for
// u < ncu = ceil(ngl * b * b / 512) (at most NCU); slots past the stage's
// count repeat its last element.  Every thread issues the same ncu loads (2 ncu
// for int8) and nothing is computed from them before coef_put, so the wait in
// front of coef_put is for these loads and the ones before them, never for the
// tile prefetch issued after them.
template <typename TB, int NCU, bool QUAD>
__device__ __forceinline__ void coef_fetch(const ColParams& p, int s, const ColTile& t, uint32_t (&cw)[NCU],
                                           float (&csc)[NCU]) {
  const ColStage& cs = p.st[s];
  const int B = cs.b, BB = B * B, ngl = p.nsub / B;
  const int n = ngl * BB;
  // group c = (pre * ngl + gl) * suf + q: uniform base plus gl * suf
  const TB* blocks = static_cast<const TB*>(p.blocks) + cs.blk_off +
                     (t.pre * (int64_t)ngl * p.suf + t.q) * BB;
  const float* scales = p.scales + cs.grp_off + t.pre * (int64_t)ngl * p.suf + t.q;
  const int sufi = (int)p.suf;
  if (QUAD && cs.nq > 0) {
    // quads of 4 consecutive stored elements (never across a block: b^2 is a
    // multiple of 4), one 16-, 8- or 4-byte load each, in memory order
#pragma unroll
    for (int v = 0; v < NCU / 4; ++v) {
      if (v >= cs.nq) break;   // uniform
      int e = 4 * ((int)threadIdx.x + v * 512);
      e = e < n ? e : n - 4;
      const int gl = udiv(e, cs.mag_bb);
      const TB* src = blocks + gl * sufi * BB + (e - gl * BB);
      if constexpr (std::is_same<TB, float>::value) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(src);
        cw[4 * v] = a.x; cw[4 * v + 1] = a.y; cw[4 * v + 2] = a.z; cw[4 * v + 3] = a.w;
      } else if constexpr (std::is_same<TB, uint16_t>::value) {
        const uint2 a = *reinterpret_cast<const uint2*>(src);
        cw[4 * v] = a.x & 0xffffu; cw[4 * v + 1] = a.x >> 16; cw[4 * v + 2] = a.y & 0xffffu; cw[4 * v + 3] = a.y >> 16;
      } else {
        const uint32_t a = *reinterpret_cast<const uint32_t*>(src);
        const float sc = scales[gl * sufi];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          cw[4 * v + c] = (uint32_t)(int)(int8_t)(a >> (8 * c));
          csc[4 * v + c] = sc;
        }
      }
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < NCU; ++u) {
    if (u >= cs.ncu) break;   // uniform: slots past the stage's count are never put
    int e = threadIdx.x + u * 512;
    e = e < n ? e : n - 1;
    const int gl = udiv(e, cs.mag_bb);
    const int i = e - gl * BB;
    const int o = udiv(i, cs.mag_b);
    const int k = i - o * B;
    const TB* src = blocks + gl * sufi * BB + (p.transpose ? k * B + o : i);
    if constexpr (std::is_same<TB, float>::value) {
      cw[u] = __float_as_uint(*src);
    } else if constexpr (std::is_same<TB, uint16_t>::value) {
      cw[u] = *src;
    } else {
      cw[u] = (uint32_t)(int)*src;
      csc[u] = scales[gl * sufi];
    }
  }
}

// Writes the fetched coefficients into a slot as C[gl][o][k] in fp32 with
// rows padded to 4 floats (the layout the stage tasks read).
template <typename TB, int NCU, bool QUAD>
__device__ __forceinline__ void coef_put(const ColParams& p, int s, const uint32_t (&cw)[NCU], const float (&csc)[NCU],
                                         float* slot) {
  const ColStage& cs = p.st[s];
  const int B = cs.b, BB = B * B, Bp = (B + 3) & ~3;
  const int n = (p.nsub / B) * BB;
  auto decode = [&](int u) {
    if constexpr (std::is_same<TB, float>::value) return __uint_as_float(cw[u]);
    else if constexpr (std::is_same<TB, uint16_t>::value) return __uint_as_float(cw[u] << 16);
    else return (float)(int)cw[u] * csc[u];
  };
  if (QUAD && cs.nq > 0) {
    // stored element m of block gl is C[m / B][m % B] forward, C[m % B][m / B]
    // transposed
#pragma unroll
    for (int v = 0; v < NCU / 4; ++v) {
      const int e = 4 * ((int)threadIdx.x + v * 512);
      if (v < cs.nq && e < n) {
        const int gl = udiv(e, cs.mag_bb);
        const int m0 = e - gl * BB;
        float* g = slot + gl * (B * Bp);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int hi = udiv(m0 + c, cs.mag_b), lo = m0 + c - hi * B;
          g[p.transpose ? lo * Bp + hi : hi * Bp + lo] = decode(4 * v + c);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < NCU; ++u) {
    const int e = threadIdx.x + u * 512;
    if (u < cs.ncu && e < n) {
      const int gl = udiv(e, cs.mag_bb);
      const int i = e - gl * BB;
      const int o = udiv(i, cs.mag_b);
      slot[gl * (B * Bp) + o * Bp + (i - o * B)] = decode(u);
    }
  }
}

// One stage of the run on the tile.  The tile is [nsub][pw] fp32; a task is
// one group of the stage and a block of 64 columns, one column per lane, so
// every lane of a wave uses the same coefficients (read from the slot).  All
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
    const int gl = udiv(task, p.mag_ncb);
    const int cb = task - gl * ncb;
    const int u_hi = udiv(gl, cs.mag_ls);
    const int u_lo = gl - u_hi * ls;
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

// The same stage on the matrix cores (radix <= 8): per task and output quad
// h, v_mfma_f32_4x4x1f32 with A = C[4h + i][k] (i = lane & 3, read from the
// slot as padded rows) and B = the lane's column value x[k]; lane 4b + j then
// holds outputs 4h .. 4h+3 of its own column.  The coefficients reach the
// lanes as four distinct rows per read instead of a broadcast of every value
// to all 64 lanes, which is what bounds the vector-ALU form.
template <int B>
__device__ void col_stage_mfma(const ColParams& p, const ColStage& cs, float* __restrict__ tile,
                               const float* __restrict__ cbuf, int wave, int nwaves, int lane) {
  constexpr int Bp = coef_row_stride<B>();
  constexpr int NH = (B + 3) / 4;
  const int i = lane & 3;
  const int ngl = p.nsub / B;
  const int ncb = p.pw / 64;
  const int ntask = ngl * ncb;
  const int ls = cs.ls;
  for (int task = wave; task < ntask; task += nwaves) {
    const int gl = udiv(task, p.mag_ncb);
    const int cb = task - gl * ncb;
    const int u_hi = udiv(gl, cs.mag_ls);
    const int u_lo = gl - u_hi * ls;
    const int ubase = u_hi * B * ls + u_lo;
    float* col = tile + ubase * p.pw + cb * 64 + lane;
    float a[NH][Bp];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int o = 4 * h + i < B ? 4 * h + i : B - 1;   // rows past B: outputs dropped
      const f32x4* row = reinterpret_cast<const f32x4*>(cbuf + gl * (B * Bp) + o * Bp);
#pragma unroll
      for (int c = 0; c < Bp / 4; ++c) {
        const f32x4 q = row[c];
        a[h][4 * c] = q.x; a[h][4 * c + 1] = q.y; a[h][4 * c + 2] = q.z; a[h][4 * c + 3] = q.w;
      }
    }
    float v[B];
#pragma unroll
    for (int k = 0; k < B; ++k) v[k] = col[k * ls * p.pw];
    f32x4 acc[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) acc[h] = __builtin_amdgcn_mfma_f32_4x4x1f32(a[h][0], v[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
    for (int k = 1; k < B; ++k)
#pragma unroll
      for (int h = 0; h < NH; ++h) acc[h] = __builtin_amdgcn_mfma_f32_4x4x1f32(a[h][k], v[k], acc[h], 0, 0, 0);
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        if (4 * h + ii < B) col[(4 * h + ii) * ls * p.pw] = acc[h][ii];
  }
}

// BIG: radices 9..16 compiled in (their b^2 coefficients raise the
// register count of the whole kernel, so runs of radices <= 8 use a kernel
// without them).
template <bool BIG>
__device__ __forceinline__ void run_col_tasks(const ColParams& p, int s, float* tile, const float* slot, int wave,
                                              int lane) {
  const ColStage& cs = p.st[s];
  switch (cs.b) {
    case 2: col_stage_mfma<2>(p, cs, tile, slot, wave, 8, lane); break;
    case 3: col_stage_mfma<3>(p, cs, tile, slot, wave, 8, lane); break;
    case 4: col_stage_mfma<4>(p, cs, tile, slot, wave, 8, lane); break;
    case 5: col_stage_mfma<5>(p, cs, tile, slot, wave, 8, lane); break;
    case 6: col_stage_mfma<6>(p, cs, tile, slot, wave, 8, lane); break;
    case 7: col_stage_mfma<7>(p, cs, tile, slot, wave, 8, lane); break;
    case 8: col_stage_mfma<8>(p, cs, tile, slot, wave, 8, lane); break;
    default:
      if constexpr (BIG) {
        switch (cs.b) {
          case 9: col_stage<9>(p, cs, tile, slot, wave, 8, lane); break;
          case 10: col_stage<10>(p, cs, tile, slot, wave, 8, lane); break;
          case 11: col_stage<11>(p, cs, tile, slot, wave, 8, lane); break;
          case 12: col_stage<12>(p, cs, tile, slot, wave, 8, lane); break;
          case 13: col_stage<13>(p, cs, tile, slot, wave, 8, lane); break;
          case 14: col_stage<14>(p, cs, tile, slot, wave, 8, lane); break;
          case 15: col_stage<15>(p, cs, tile, slot, wave, 8, lane); break;
          case 16: col_stage<16>(p, cs, tile, slot, wave, 8, lane); break;
          default: break;
        }
      }
      break;
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

// Chunk slots of the 16-byte path: slot j of thread t is chunk t + 512 j of
// the tile's nsub * pw / V.  A slot past the end repeats the thread's own
// slot-0 chunk (it loads the same bytes, writes them to LDS again and stores
// slot 0's finished data again), so every thread issues exactly MAXC loads
// and stores per tile and the waits before a prefetched tile goes into LDS
// count them exactly.  With fewer than 512 chunks a thread may have no chunk
// of its own: then the slot wraps to another thread's chunk (p.split_swap).
__device__ __forceinline__ int chunk_of(int j, int total, uint32_t mag_tot) {
  const int i = (int)threadIdx.x + j * 512;
  return i < total ? i : (total >= 512 ? (int)threadIdx.x : i - udiv(i, mag_tot) * total);
}

// The D_s factor of the pass (sign_mode 1: on the rows as they enter the
// first stage; 2: on the rows as they leave the last one) is applied to the
// data chunks in the swap, from one sign byte per chunk slot loaded with the
// chunk (a byte of the blocks when there are no signs: always a valid
// address, never used).  Every thread issues the same 2 MAXC loads per tile.
template <typename TIN, int MAXC>
__device__ __forceinline__ void col_prefetch(const ColParams& p, const ColTile& t, u32x4 (&r)[MAXC], uint8_t (&sg)[MAXC]) {
  constexpr int VI = ColIo<TIN>::V;
  const TIN* x = static_cast<const TIN*>(p.x);
  const int cpr = p.pw / VI;
  const int total = p.nsub * cpr;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int i = chunk_of(j, total, p.mag_tot);
    const int u = udiv(i, p.mag_cpr);
    const int ch = i - u * cpr;
    const int64_t row = t.row_base + (int64_t)u * p.suf;
    r[j] = ld_stream(x + row * p.ldx + t.col0 + ch * VI);
    // the raw byte; its bit 7 is tested in the swap
    sg[j] = reinterpret_cast<const uint8_t*>(p.signs)[p.sign_mode ? row : 0];
  }
}

// Sign bit(s) of every value of a 16-byte chunk
template <typename T> struct ChunkSign;
template <> struct ChunkSign<uint16_t> { static constexpr uint32_t m = 0x80008000u; };
template <> struct ChunkSign<float> { static constexpr uint32_t m = 0x80000000u; };
__device__ __forceinline__ u32x4 flip_chunk(u32x4 w, uint32_t m) { return u32x4{w.x ^ m, w.y ^ m, w.z ^ m, w.w ^ m}; }

template <typename TIN, typename TOUT, int MAXC>
__device__ __forceinline__ void col_swap_part(const ColParams& p, const ColTile& done, bool has_done, bool has_next,
                                              const u32x4 (&r)[MAXC], const uint8_t (&sg)[MAXC], uint32_t& smask,
                                              float* tile) {
  constexpr int V = ColIo<TIN>::V;
  static_assert(ColIo<TIN>::V == ColIo<TOUT>::V || true, "");
  constexpr int VI = ColIo<TIN>::V, VO = ColIo<TOUT>::V;
  static_assert(VI == VO || VI == 8 || VI == 4, "chunk widths");
  (void)V;
  TOUT* y = static_cast<TOUT*>(p.y);
  const int cpr_i = p.pw / VI;
  const int total = p.nsub * cpr_i;
  constexpr int NO = VI / VO > 0 ? VI / VO : 1;
  u32x4 keep[NO];   // slot 0's finished data, stored again by repeated slots
  uint32_t nmask = 0;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int i = chunk_of(j, total, p.mag_tot);
    const bool rep = j > 0 && total >= 512 && (int)threadIdx.x + j * 512 >= total;
    const int u = udiv(i, p.mag_cpr);
    const int ch = i - u * cpr_i;
    float* loc = tile + u * p.pw + ch * VI;
    if (has_done) {
      // VI / VO output chunks cover the same columns
#pragma unroll
      for (int h = 0; h < VI / VO; ++h) {
        float v[VO];
#pragma unroll
        for (int e = 0; e < VO; e += 4) {
          const f32x4 q4 = *reinterpret_cast<const f32x4*>(loc + h * VO + e);
          v[e] = q4.x; v[e + 1] = q4.y; v[e + 2] = q4.z; v[e + 3] = q4.w;
        }
        u32x4 o = pack_chunk(v, static_cast<TOUT*>(nullptr));
        if (p.sign_mode == 2 && ((smask >> j) & 1u)) o = flip_chunk(o, ChunkSign<TOUT>::m);
        if (j == 0) keep[h] = o;
        else if (rep) o = keep[h];
        st_stream(y + (done.row_base + (int64_t)u * p.suf) * p.ldy + done.col0 + ch * VI + h * VO, o);
      }
      if constexpr (VO > VI) {
        // fp32 in, bf16 out: pairs of input chunks make one output chunk;
        // the even chunk of a pair stores both halves
        static_assert(VO == 2 * VI, "chunk widths");
        // (both chunks of a pair lie in one tile row, so the slot's sign bit
        // is the pair's)
        if ((ch & 1) == 0) {
          float v[VO];
#pragma unroll
          for (int e = 0; e < VO; e += 4) {
            const f32x4 q4 = *reinterpret_cast<const f32x4*>(loc + e);
            v[e] = q4.x; v[e + 1] = q4.y; v[e + 2] = q4.z; v[e + 3] = q4.w;
          }
          u32x4 o = pack_chunk(v, static_cast<TOUT*>(nullptr));
          if (p.sign_mode == 2 && ((smask >> j) & 1u)) o = flip_chunk(o, ChunkSign<TOUT>::m);
          st_stream(y + (done.row_base + (int64_t)u * p.suf) * p.ldy + done.col0 + ch * VI, o);
        }
      }
    }
    if (has_next) {
      const bool neg = (sg[j] & 0x80) != 0;
      nmask |= (neg ? 1u : 0u) << j;
      float v[VI];
      unpack_chunk(p.sign_mode == 1 && neg ? flip_chunk(r[j], ChunkSign<TIN>::m) : r[j], v,
                   static_cast<const TIN*>(nullptr));
#pragma unroll
      for (int e = 0; e < VI; e += 4) *reinterpret_cast<f32x4*>(loc + e) = f32x4{v[e], v[e + 1], v[e + 2], v[e + 3]};
    }
  }
  if (has_next) smask = nmask;
}

// Slot by slot: store the finished tile's chunk (unless there is none yet),
// then put the next tile's chunk in its place; the same thread owns both.
// smask holds, per slot, whether the row of the tile in LDS has a negative
// sign: it is the same row in every tile of the pass, and the swap replaces
// it with the incoming tile's.
// When slots wrap around to other threads' chunks, a chunk has two owners,
// and one of them could overwrite it before the other has stored it; with
// fp32 in and bf16 out, the thread of an even chunk stores its odd neighbour
// too, which another thread replaces.  In both cases (p.split_swap) every
// store is done first and a barrier separates them from the writes.
template <typename TIN, typename TOUT, int MAXC>
__device__ __forceinline__ void col_swap(const ColParams& p, const ColTile& done, bool has_done, bool has_next,
                                         const u32x4 (&r)[MAXC], const uint8_t (&sg)[MAXC], uint32_t& smask,
                                         float* tile) {
  if (p.split_swap) {
    if (has_done) col_swap_part<TIN, TOUT, MAXC>(p, done, true, false, r, sg, smask, tile);
    __syncthreads();
    if (has_next) col_swap_part<TIN, TOUT, MAXC>(p, done, false, true, r, sg, smask, tile);
  } else {
    col_swap_part<TIN, TOUT, MAXC>(p, done, has_done, has_next, r, sg, smask, tile);
  }
}

// Element path (unaligned matrices, ragged last panel): thread t owns
// elements t + 512 k of the tile, for both the store and the load.
template <typename TIN, typename TOUT>
__device__ __forceinline__ void col_swap_el(const ColParams& p, const ColTile& done, bool has_done,
                                            const ColTile& nt, bool has_next, float* tile) {
  const TIN* x = static_cast<const TIN*>(p.x);
  TOUT* y = static_cast<TOUT*>(p.y);
  for (int i = threadIdx.x; i < p.nsub * p.pw; i += 512) {
    const int u = i / p.pw;
    const int j = i - u * p.pw;
    if (has_done && j < done.w) {
      const int64_t row = done.row_base + (int64_t)u * p.suf;
      const float v = tile[i];
      st_el(y + row * p.ldy + done.col0 + j, p.sign_mode == 2 && p.signs[row] < 0 ? -v : v);
    }
    if (has_next) {
      float v = 0.0f;
      const int64_t row = nt.row_base + (int64_t)u * p.suf;
      if (j < nt.w) v = ld_el(x + row * p.ldx + nt.col0 + j);
      tile[i] = p.sign_mode == 1 && p.signs[row] < 0 ? -v : v;
    }
  }
}

// A pass over the tiles of one run.  Per tile: one barrier per stage; the
// coefficients of the stage after the current one go into the other of two
// LDS slots while the current stage runs (fetched into registers a stage
// earlier, crossing into the next tile), and the finished tile is swapped
// for the prefetched next one chunk by chunk after the last stage.  Every
// thread issues the same global loads whatever the position in the pass
// (past the last tile it re-reads the last one), so the waits count them
// exactly: the prefetch is issued in the first stage behind that stage's
// coefficient fetch, and only the last stage's coefficients (fetched behind
// it) and the swap wait for it.
template <typename TIN, typename TOUT, typename TB, bool BIG, bool VEC, int MAXC>
__global__ void __launch_bounds__(512) col_pass_kernel(ColParams p) {
  constexpr int NCU = BIG ? 16 : 8;
  // the quad coefficient path is compiled into the bf16-input kernels of more
  // than 4 chunks per thread: the 4-chunk ones must stay at 128 VGPRs (two
  // workgroups per CU), and in the fp32-input ones the second path slowed the
  // one-element path of the radix-3 pass by 15%
  constexpr bool kQuad = MAXC > 4 && std::is_same<TIN, uint16_t>::value;
  extern __shared__ float tile[];
  float* slots = tile + p.nsub * p.pw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t tix = blockIdx.x;
  if (tix >= p.ntiles) return;   // uniform per workgroup
  const int64_t last = p.ntiles - 1;
  auto clampt = [&](int64_t x) { return x < p.ntiles ? x : last; };
  ColTile t = col_tile(p, tix);
  uint32_t cw[NCU];
  float csc[NCU];
  // prologue: first tile and its first stage's coefficients in place
  coef_fetch<TB, NCU, kQuad>(p, 0, t, cw, csc);
  coef_put<TB, NCU, kQuad>(p, 0, cw, csc, slots);
  u32x4 pf[MAXC];
  uint8_t pfs[MAXC];
  uint32_t smask = 0;
  if constexpr (VEC) {
    col_prefetch<TIN, MAXC>(p, t, pf, pfs);
    col_swap<TIN, TOUT, MAXC>(p, t, false, true, pf, pfs, smask, tile);
  } else {
    col_swap_el<TIN, TOUT>(p, t, false, t, true, tile);
  }
  // the stage after the current one: (sn, tixn)
  int sn = 1;
  int64_t tixn = tix;
  if (sn == p.nstage) { sn = 0; tixn = tix + gridDim.x; }
  coef_fetch<TB, NCU, kQuad>(p, sn, col_tile(p, clampt(tixn)), cw, csc);
  __syncthreads();
  int slot = 0;
  while (true) {
    for (int s = 0; s < p.nstage; ++s) {
      // coefficients of the next stage into the other slot, then fetch the
      // one after; the next tile's prefetch goes out behind the first
      // stage's fetch, so the first two stages never wait for it
      if (tixn < p.ntiles) coef_put<TB, NCU, kQuad>(p, sn, cw, csc, slots + (slot ^ 1) * p.cslot);
      ++sn;
      if (sn == p.nstage) { sn = 0; tixn += gridDim.x; }
      coef_fetch<TB, NCU, kQuad>(p, sn, col_tile(p, clampt(tixn)), cw, csc);
      if constexpr (VEC) {
        if (s == 0) col_prefetch<TIN, MAXC>(p, col_tile(p, clampt(tix + gridDim.x)), pf, pfs);
      }
      run_col_tasks<BIG>(p, s, tile, slots + slot * p.cslot, wave, lane);
      __syncthreads();
      slot ^= 1;
    }
    const int64_t tnx = tix + gridDim.x;
    const bool has_next = tnx < p.ntiles;
    const ColTile nt = col_tile(p, clampt(tnx));
    if constexpr (VEC) col_swap<TIN, TOUT, MAXC>(p, t, true, has_next, pf, pfs, smask, tile);
    else col_swap_el<TIN, TOUT>(p, t, true, nt, has_next, tile);
    if (!has_next) break;
    tix = tnx;
    t = nt;
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

// MAXC: 16-byte chunks per thread and tile; two sizes per input type (the
// smaller one for short tiles), anything larger takes the element path.
template <typename TIN> struct ColMaxc;
template <> struct ColMaxc<uint16_t> { static constexpr int lo = 4, hi = 8; };
template <> struct ColMaxc<float> { static constexpr int lo = 8, hi = 16; };


template <typename TIN, typename TOUT, typename TB, bool BIG>
hipError_t launch_cols_k(const ColParams& p, int maxc, int grid, size_t lds, hipStream_t st) {
  void (*kern)(ColParams) = col_pass_kernel<TIN, TOUT, TB, BIG, false, 1>;
  if (p.vec)
    kern = maxc <= ColMaxc<TIN>::lo ? col_pass_kernel<TIN, TOUT, TB, BIG, true, ColMaxc<TIN>::lo>
                                    : col_pass_kernel<TIN, TOUT, TB, BIG, true, ColMaxc<TIN>::hi>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(512), lds, st, p);
  return hipGetLastError();
}

template <typename TIN, typename TOUT>
hipError_t launch_cols_blk(DT bdt, const ColParams& p, bool big, int maxc, int grid, size_t lds, hipStream_t st) {
  switch (bdt) {
    case DT::F32:
      return big ? launch_cols_k<TIN, TOUT, float, true>(p, maxc, grid, lds, st)
                 : launch_cols_k<TIN, TOUT, float, false>(p, maxc, grid, lds, st);
    case DT::BF16:
      return big ? launch_cols_k<TIN, TOUT, uint16_t, true>(p, maxc, grid, lds, st)
                 : launch_cols_k<TIN, TOUT, uint16_t, false>(p, maxc, grid, lds, st);
    case DT::I8:
      return big ? launch_cols_k<TIN, TOUT, int8_t, true>(p, maxc, grid, lds, st)
                 : launch_cols_k<TIN, TOUT, int8_t, false>(p, maxc, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_apply_cols(const Plan& pl, int t0, int t1, bool inverse, const void* blocks,
                             DT bdt, const float* scales, const int8_t* signs, int sign_mode,
                             const void* x, int64_t ldx, DT in_dt, void* y, int64_t ldy,
                             DT out_dt, int64_t ncols, hipStream_t stream) {
  if (ncols <= 0) return hipSuccess;
  if (cols_dense_supported(pl, t0, t1))
    return launch_apply_cols_dense(pl, t0, t1, inverse, blocks, bdt, scales, signs, sign_mode, x, ldx, in_dt, y, ldy,
                                   out_dt, ncols, stream);
  ColParams p{};
  int nsub = 1;
  for (int t = t0; t < t1; ++t) nsub *= pl.radix[t];
  p.nsub = nsub;
  p.nstage = t1 - t0;
  p.suf = pl.stride[t1 - 1];
  p.transpose = inverse ? 1 : 0;
  p.sign_mode = signs ? sign_mode : 0;
  auto mag = [](int d) { return d == 1 ? 0u : (uint32_t)(((1ull << 32) + (uint64_t)d - 1) / (uint64_t)d); };
  int bmax = 2, cw = 4;   // largest radix; widest padded coefficient row
  for (int i = 0; i < p.nstage; ++i) {
    const int t = inverse ? t1 - 1 - i : t0 + i;
    ColStage& cs = p.st[i];
    cs.b = pl.radix[t];
    cs.ls = (int)(pl.stride[t] / p.suf);
    cs.blk_off = (int)pl.blk_off[t];
    cs.grp_off = (int)pl.grp_off[t];
    cs.mag_b = mag(cs.b);
    cs.mag_bb = mag(cs.b * cs.b);
    cs.mag_ls = mag(cs.ls);
    cs.ncu = (nsub * cs.b + 511) / 512;
    cs.nq = (cs.b % 2 == 0 && cs.blk_off % 4 == 0) ? (nsub * cs.b + 2047) / 2048 : 0;
    bmax = cs.b > bmax ? cs.b : bmax;
    cw = ((cs.b + 3) & ~3) > cw ? ((cs.b + 3) & ~3) : cw;
  }
  // A stage stages nsub * b coefficients per thread block of 512 threads:
  // at most 8 (radix <= 8) or 16 per thread.
  const bool big = bmax > 8;
  if ((size_t)nsub * bmax > (size_t)512 * (big ? 16 : 8)) return hipErrorInvalidValue;
  p.cslot = nsub * cw;
  // Panel width: a multiple of 64 columns (stage tasks are 64-column blocks)
  // up to 1024, as wide as fits next to two coefficient slots in 80 KiB (two
  // workgroups per CU) or, failing that, in 160 KiB; among those the widest
  // that divides the column count (whole panels take the 16-byte path).
  //
  // Among the dividing widths, the 16-byte path gives every thread the same
  // number of chunk slots (4 or 8 for bf16 input, 8 or 16 for fp32), and a
  // slot past the tile's chunks loads and stores its thread's first chunk
  // again; a width whose chunk count fills its slots best is taken (ties go
  // to the wider), so the repeated streaming stores stay few.
  auto fits = [&](int w, size_t cap) { return (size_t)nsub * (w + 2 * cw) * sizeof(float) <= cap; };
  const size_t cap = fits(256, (size_t)80 * 1024) ? (size_t)80 * 1024 : (size_t)160 * 1024;
  const int vi_c = 16 / io_bytes(in_dt);
  const int lo_c = in_dt == DT::F32 ? 8 : 4;
  auto slot_waste = [&](int w) {   // slots per chunk of the 16-byte path
    const int64_t chunks = (int64_t)nsub * (w / vi_c);
    const int64_t need = (chunks + 511) / 512;
    if (need > 2 * lo_c) return 1e9;   // element path
    return (double)(512 * (need <= lo_c ? lo_c : 2 * lo_c)) / (double)chunks;
  };
  int pw = 0;
  for (int w = 64; w <= 1024; w += 64) {
    if (!fits(w, cap)) break;
    pw = w;
  }
  if (pw == 0) return hipErrorInvalidValue;
  int pw_div = 0;
  for (int w = 64; w <= pw; w += 64) {
    if (ncols % w != 0 || w < pw / 2) continue;
    if (pw_div == 0 || slot_waste(w) <= slot_waste(pw_div)) pw_div = w;
  }
  if (pw_div > 0) pw = pw_div;
  p.pw = pw;
  p.mag_ncb = mag(pw / 64);
  {
    // input chunks per tile row and per tile (below 2^16: the tile is at most 160 KiB of fp32)
    const int vin = 16 / io_bytes(in_dt);
    p.mag_cpr = mag(pw / vin);
    p.mag_tot = mag(nsub * (pw / vin));
  }
  p.ncols = ncols;
  p.npanels = (ncols + pw - 1) / pw;
  p.ntiles = (pl.d / nsub) * p.npanels;
  p.blocks = blocks;
  p.scales = scales;
  // without signs the kernel still reads a (discarded) byte: point at the blocks
  p.signs = signs ? signs : static_cast<const int8_t*>(blocks);
  p.x = x;
  p.ldx = ldx;
  p.y = y;
  p.ldy = ldy;
  const int ib = io_bytes(in_dt), ob = io_bytes(out_dt);
  const int vi = 16 / ib;
  const int maxc = (int)(((int64_t)nsub * (pw / vi) + 511) / 512);
  const int maxc_cap = in_dt == DT::F32 ? 16 : 8;
  p.vec = reinterpret_cast<uintptr_t>(x) % 16 == 0 && (ldx * ib) % 16 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0 &&
          (ldy * ob) % 16 == 0 && ncols % pw == 0 && maxc <= maxc_cap;
  p.split_swap = (int64_t)nsub * (pw / vi) < 512 || (in_dt == DT::F32 && out_dt == DT::BF16);
  const size_t lds = ((size_t)nsub * pw + (size_t)2 * p.cslot) * sizeof(float);
  int64_t grid = (int64_t)cus_for_cols() * (lds > 80 * 1024 ? 1 : 2);
  if (grid > p.ntiles) grid = p.ntiles;
  if (in_dt == DT::F32 && out_dt == DT::F32) return launch_cols_blk<float, float>(bdt, p, big, maxc, (int)grid, lds, stream);
  if (in_dt == DT::BF16 && out_dt == DT::BF16) return launch_cols_blk<uint16_t, uint16_t>(bdt, p, big, maxc, (int)grid, lds, stream);
  if (in_dt == DT::BF16 && out_dt == DT::F32) return launch_cols_blk<uint16_t, float>(bdt, p, big, maxc, (int)grid, lds, stream);
  if (in_dt == DT::F32 && out_dt == DT::BF16) return launch_cols_blk<float, uint16_t>(bdt, p, big, maxc, (int)grid, lds, stream);
  return hipErrorInvalidValue;
}

}  // namespace harp
