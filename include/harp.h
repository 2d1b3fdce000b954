/*
 * harp.h - C ABI of the HARP / randomized-Hadamard apply library (gfx950).
 *
 * The library computes batched structured orthogonal transforms over rows of
 * length d.  A mixed-radix schedule b = (b_0, ..., b_{m-1}) with prod b_t = d
 * splits a row index into digits; stage t applies, to every group of
 * coordinates that agree on all digits except digit t, a b_t x b_t orthogonal
 * block B_{t,c} = Q_{t,c} G_{b_t}.
 *
 *   Sources cited below:
 *   [TS]  "Technical Summary: HARP (Hadamard-Preconditioned Adaptive Rotation
 *         Processor)", gist.science paper 2605.29843: §2.1 Core Architecture,
 *         §2.2 Hadamard Preconditioning & Initialization, §2.4 Deployment
 *         Efficiency, §3 Key Contributions, §5 Significance and Claims.
 *   [ABS] arXiv 2605.29843v1 abstract (HARP).
 *   [RHT] arXiv 2605.06014 abstract, "Quantizing With Randomized Hadamard
 *         Transforms: Efficient Heuristic Now Proven".
 *
 * Conventions fixed by this library where the pages leave the choice open:
 *   - a row is viewed as a C-order array of shape (b_0, ..., b_{m-1}); digit t
 *     has stride s_t = prod_{u>t} b_u; the group index c of stage t is the
 *     C-order index of the remaining digits;
 *   - stage 0 acts first; the forward operator is M = S_{m-1} ... S_0 D_s,
 *     with the sign vector s acting on the input;
 *   - a block acts as y_r = sum_k B[r][k] x_k;
 *   - G_b is the natural-order Sylvester Hadamard scaled by 1/sqrt(b) for a
 *     power-of-two b, otherwise the Q factor (diag R > 0) of the QR
 *     factorisation of a caller-supplied Gaussian b x b matrix;
 *   - Q is a Givens rotation [[c,-s],[s,c]] for b = 2 and the Cayley map
 *     (I - A)(I + A)^-1 of a skew-symmetric A (strict upper triangle filled
 *     row-major from the group's parameters) for b > 2.
 *
 * Memory and streams.  Every array argument is a DEVICE pointer unless marked
 * (host).  The caller owns every buffer; the library never allocates or frees
 * device memory, never synchronises, and keeps no state apart from a cached
 * device-property query and a per-thread copy of the last error message.
 * Every call only enqueues work on `stream` (NULL = the default stream) and
 * returns; buffers must stay valid until that work has completed.
 *
 * Errors.  Every entry point returns a harp_status; nothing throws across the
 * ABI.  Argument checks run on the host before any HIP call, so a rejected
 * call enqueues nothing.  harp_last_error() returns a message for the most
 * recent non-OK status on the calling thread.
 *
 * Data layouts.
 *   rows:   row-major, `rows` rows of d elements, consecutive rows `ld`
 *           ELEMENTS apart (ld >= d).  x == y with ldx == ldy is allowed (in
 *           place); any other overlap is undefined.
 *   blocks: concatenation over stages t = 0..m-1 of arrays [d/b_t][b_t][b_t]
 *           (group, row r, column k), row-major, in the block dtype.
 *   block_scales: HARP_I8 storage only: concatenation over stages of one fp32
 *           scale per group; the coefficient is code * scale.
 *   signs:  d int8 values in {+1, -1}; NULL means all +1.
 */
#ifndef HARP_H_
#define HARP_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HARP_OK = 0,
  HARP_ERR_INVALID_ARG = -1, /* malformed schedule, size, pointer or stride */
  HARP_ERR_UNSUPPORTED = -2, /* well-formed but outside what the kernels do  */
  HARP_ERR_LAUNCH = -3       /* the HIP runtime reported an error            */
} harp_status;

typedef enum {
  HARP_F32 = 0,  /* IEEE binary32                                  */
  HARP_BF16 = 1, /* bfloat16 (upper half of a binary32)            */
  HARP_I8 = 2,   /* int8 code with one fp32 scale per block        */
  HARP_F64 = 3   /* IEEE binary64 (parameters only)                */
} harp_dtype;

#define HARP_MAX_STAGES 16
#define HARP_MAX_RADIX 16
/* Largest row length the single-pass kernels hold on chip. */
#define HARP_MAX_D 32768

/* (host) A mixed-radix schedule; read at call time, not retained. */
typedef struct {
  int32_t m;                       /* number of stages, 1..HARP_MAX_STAGES */
  int32_t radix[HARP_MAX_STAGES];  /* b_t in 2..HARP_MAX_RADIX            */
} harp_schedule;

/* ------------------------------------------------------------------------
 * Sizes (host only; -1 if the schedule is malformed or prod b_t != d).
 * ---------------------------------------------------------------------- */

/* Learnable parameters [TS §2.2]: d/2 Givens angles for each radix-2 stage,
 * (d/b_t) * b_t(b_t-1)/2 skew entries for each other stage; concatenated
 * over stages. */
int64_t harp_theta_count(const harp_schedule* s, int64_t d);
/* Gaussian entries for the QR base mixers [TS §2.1]: b_t*b_t for every stage
 * whose radix is not a power of two, in stage order. */
int64_t harp_gauss_count(const harp_schedule* s, int64_t d);
/* Block coefficients: sum_t d * b_t. */
int64_t harp_block_count(const harp_schedule* s, int64_t d);
/* Blocks (= int8 scales): sum_t d / b_t. */
int64_t harp_group_count(const harp_schedule* s, int64_t d);

/* ------------------------------------------------------------------------
 * Block materialisation  B_{t,c} = Q_{t,c}(theta) G_{b_t}   [TS §2.2]
 *
 * theta: harp_theta_count() fp64 values (layout above).
 * gauss: harp_gauss_count() fp64 values, one row-major b x b standard-normal
 *        matrix per non-power-of-two stage; NULL allowed if there is none.
 * blocks_out: harp_block_count() values of block_dtype (F32, BF16 or I8).
 *        F32 and BF16 round the fp64 block to nearest, ties to even.
 * scales_out: I8 only, harp_group_count() fp32 scales; scale =
 *        fp32(max|B| / 127), code = clamp(rint(B / scale), -127, 127) with the
 *        decision taken in fp64.  Must be NULL for the other dtypes.
 * The whole computation (QR of the Gaussian matrices, Cayley solves,
 * products, rounding) runs on the device in fp64.
 * ---------------------------------------------------------------------- */
harp_status harp_materialize_blocks(const harp_schedule* s, int64_t d,
                                    const double* theta, const double* gauss,
                                    harp_dtype block_dtype, void* blocks_out,
                                    float* scales_out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * int8 parameter storage   [TS §2.4: the learnable parameters may be kept in
 * int8 with little loss]
 *
 * Codes: harp_theta_count() int8 values, in theta's layout.  Scales: one fp32
 * per stage (s->m values), shared by all of that stage's parameters.  The
 * value of a parameter is code * scale.  (A scale per stage, not per group,
 * is what keeps the [TS §4] overhead of 2.00 -> 2.05 bits per weight.)
 *
 * harp_quantize_theta: scale = fp32(max|theta of the stage| / 127), code =
 *   clamp(rint(theta / scale), -127, 127), decided in fp64; a stage of zeros
 *   gets scale 0 and codes 0.  theta, theta_codes and theta_scales are device
 *   pointers; the caller owns all three.
 * harp_materialize_blocks_q8: as harp_materialize_blocks, with each parameter
 *   formed on the device as the exact fp64 product code * scale; gauss,
 *   blocks_out and scales_out as there.
 * Both return HARP_ERR_INVALID_ARG (nothing launched) for a NULL pointer
 * that is required or a schedule that does not factor d.
 * ---------------------------------------------------------------------- */
harp_status harp_quantize_theta(const harp_schedule* s, int64_t d,
                                const double* theta, int8_t* theta_codes,
                                float* theta_scales, hipStream_t stream);
harp_status harp_materialize_blocks_q8(const harp_schedule* s, int64_t d,
                                       const int8_t* theta_codes,
                                       const float* theta_scales,
                                       const double* gauss,
                                       harp_dtype block_dtype, void* blocks_out,
                                       float* scales_out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Forward apply   y = S_{m-1} ... S_0 D_s x    for each of `rows` rows
 * [TS §2.1, §2.2; the deployment-time stride stages of TS §2.4].
 *
 * blocks/block_dtype/block_scales: layout above; block_dtype F32, BF16 or I8
 *   (block_scales non-NULL exactly for I8).
 * io_dtype: F32 or BF16 for both x and y.  Arithmetic is fp32 throughout;
 *   BF16 input is widened exactly and the output rounded to nearest even.
 * Pointers must be 4-byte aligned (F32 rows) or 2-byte aligned (BF16 rows).
 * rows == 0 returns HARP_OK without a launch.
 * d must be at most HARP_MAX_D.
 * ---------------------------------------------------------------------- */
harp_status harp_apply(const harp_schedule* s, int64_t d, const void* blocks,
                       harp_dtype block_dtype, const float* block_scales,
                       const int8_t* signs, const void* x, int64_t ldx, void* y,
                       int64_t ldy, int64_t rows, harp_dtype io_dtype,
                       hipStream_t stream);

/* Inverse apply   x = D_s S_0^T ... S_{m-1}^T y   (transposed blocks in
 * reverse stage order, then the sign): the exact inverse, since every block
 * is orthogonal [TS §5, ABS].  Same arguments as harp_apply. */
harp_status harp_apply_inverse(const harp_schedule* s, int64_t d,
                               const void* blocks, harp_dtype block_dtype,
                               const float* block_scales, const int8_t* signs,
                               const void* y, int64_t ldy, void* x, int64_t ldx,
                               int64_t rows, harp_dtype io_dtype,
                               hipStream_t stream);

/* ------------------------------------------------------------------------
 * Small-batch (per-token decode) apply   [TS §2.1; TS §4 quotes the
 * transform's cost per generated token]
 *
 *   inverse == 0:  y = S_{m-1} ... S_0 D_s x       (as harp_apply)
 *   inverse != 0:  y = D_s S_0^T ... S_{m-1}^T x   (as harp_apply_inverse)
 *
 * For 1 <= rows <= HARP_DECODE_MAX_ROWS; built for latency at 1-64 rows.
 * The digits are split into two runs and each run is one launch of many
 * small workgroups; fp32 rows are handed from the first launch to the second
 * through `workspace`, so the arithmetic is fp32 throughout as in harp_apply.
 * Above 128 rows the call runs harp_apply's row kernels instead (faster at
 * those sizes); the workspace is then left untouched.
 * harp_apply_decode_workspace() gives the bytes needed: rows * d * 4; 0
 * when the whole row fits one workgroup and a single launch is made, or when
 * rows > 128 (the row kernels need no hand-off); -1 if no split of the
 * schedule fits (then harp_apply_decode returns HARP_ERR_UNSUPPORTED) or
 * rows * d * 4 does not fit in int64_t.  workspace: device memory owned by
 * the caller, 4-byte aligned, not overlapping x or y; its contents are
 * scratch; NULL is accepted whenever the size is 0.  Calls
 * that share one workspace must not overlap in time.  x and y may be the same
 * buffer (with ldx == ldy).  Other arguments, layouts and errors as
 * harp_apply; rows == 0 returns HARP_OK without a launch.
 * ---------------------------------------------------------------------- */
#define HARP_DECODE_MAX_ROWS 1024
int64_t harp_apply_decode_workspace(const harp_schedule* s, int64_t d,
                                    harp_dtype block_dtype, int64_t rows);
harp_status harp_apply_decode(const harp_schedule* s, int64_t d,
                              const void* blocks, harp_dtype block_dtype,
                              const float* block_scales, const int8_t* signs,
                              const void* x, int64_t ldx, void* y, int64_t ldy,
                              int64_t rows, harp_dtype io_dtype, int32_t inverse,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * Small-batch apply that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.
 *
 * Computes exactly what harp_apply_decode computes, with the same kernels,
 * arguments, layouts and errors, except that the fp32 hand-off between its
 * two launches lives in a buffer inside the library: a file-scope device
 * array of HARP_NOALLOC_SCRATCH_BYTES per GPU (each GPU the library runs on
 * holds its own copy until the process ends).  Its address is looked up once
 * per device, on the first call with that device current; the call uses the
 * calling thread's current device, which must be the device of `stream`.
 * No hipMalloc, hipFree or other allocating routine is called.
 * A call needing more than HARP_NOALLOC_SCRATCH_BYTES (rows * d * 4 bytes
 * for a two-launch schedule at up to 128 rows: e.g. 512 rows of d = 4096 is
 * handed to the row kernels and needs none, 128 rows of d = 16384 needs all
 * 8 MiB) returns HARP_ERR_INVALID_ARG without a launch.
 * Every call on one GPU shares that GPU's buffer and leaves the last call's
 * rows in it; nothing in it needs to start at zero (the first launch writes
 * every element the second one reads).  Calls that overlap in time on one
 * GPU (different streams, or host threads without ordering) race on it and
 * must not be issued.
 * ---------------------------------------------------------------------- */
#define HARP_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
harp_status harp_apply_decode_noalloc(const harp_schedule* s, int64_t d,
                                      const void* blocks, harp_dtype block_dtype,
                                      const float* block_scales, const int8_t* signs,
                                      const void* x, int64_t ldx, void* y, int64_t ldy,
                                      int64_t rows, harp_dtype io_dtype, int32_t inverse,
                                      hipStream_t stream);

/* ------------------------------------------------------------------------
 * Reverse mode, for fitting the parameters on calibration data   [TS §2.3:
 * the parameters are fitted per layer by minimising a calibration loss;
 * TS §2.1-§2.2 for the transform being differentiated]
 *
 * harp_apply_vjp: for y = S_{m-1} ... S_0 D_s x (as harp_apply) and an
 *   upstream gradient dy (rows x d, same dtype and layout rules as x):
 *     dx      = D_s S_0^T ... S_{m-1}^T dy          (skipped if dx is NULL)
 *     dblocks = dL/dB_{t,c}[r][k] = sum over rows of g_{t+1}[c, r] x_t[c, k],
 *               with x_0 = D_s x, x_{t+1} = S_t x_t, g_m = dy,
 *               g_t = S_t^T g_{t+1};  harp_block_count() fp32 values in the
 *               block layout, overwritten.  The derivative is taken with
 *               respect to the block values actually multiplied by (for I8
 *               blocks, code * scale).
 *   Arithmetic in fp32; the sum over rows runs in chunks whose partial sums
 *   are added in a fixed order, so the result is deterministic.
 *   workspace: at least harp_apply_vjp_workspace() bytes of device memory,
 *   4-byte aligned, owned by the caller (x_1 .. x_{m-1} and two gradient rows
 *   in fp32, plus the partial sums).  Every radix must be at most 8 (else
 *   HARP_ERR_UNSUPPORTED, and harp_apply_vjp_workspace() returns -1; it also
 *   returns -1 when the size would not fit in int64_t).
 *   rows must be at least 1.
 * harp_theta_vjp: dtheta (harp_theta_count() fp64, theta's layout) from
 *   dblocks through B = Q(theta) G: dL/dQ = dL/dB G^T; Givens
 *   dQ/dtheta = [[-sin, -cos], [cos, -sin]]; Cayley Q = (I - A)(I + A)^-1 gives
 *   dL/dA = -(I + Q)^T (dL/dQ) (I + A)^-T and
 *   dL/dtheta_(r,k) = dL/dA[r][k] - dL/dA[k][r].  fp64 on the device; theta
 *   and gauss as harp_materialize_blocks.
 * ---------------------------------------------------------------------- */
int64_t harp_apply_vjp_workspace(const harp_schedule* s, int64_t d,
                                 int64_t rows);
harp_status harp_apply_vjp(const harp_schedule* s, int64_t d,
                           const void* blocks, harp_dtype block_dtype,
                           const float* block_scales, const int8_t* signs,
                           const void* x, int64_t ldx, const void* dy,
                           int64_t lddy, void* dx, int64_t lddx, int64_t rows,
                           harp_dtype io_dtype, float* dblocks,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);
harp_status harp_theta_vjp(const harp_schedule* s, int64_t d,
                           const double* theta, const double* gauss,
                           const float* dblocks, double* dtheta,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * Two-sided weight rotation [TS §2, §3; ABS: a two-sided processor]
 *   inverse == 0:  W_out = M_U W M_V^T      (M_V on every row of W,
 *                                           M_U on every column)
 *   inverse != 0:  W_out = M_U^T W M_V
 * W is d_out x d_in with d_out = prod su, d_in = prod sv, row stride ldw;
 * W_out has row stride ldo.  io_dtype F32 or BF16 for both.  blocks_u /
 * blocks_v use the common block_dtype (scales non-NULL exactly for I8).
 * workspace: NULL, or at least harp_rotate_weight_workspace(d_out, d_in)
 *   bytes, 16-byte aligned (else HARP_ERR_INVALID_ARG).  With a workspace the
 *   intermediate passes are kept in fp32; with NULL they run in place in
 *   w_out and are rounded to io_dtype between passes.  w and w_out may be the same buffer (with ldw == ldo).
 * ---------------------------------------------------------------------- */
size_t harp_rotate_weight_workspace(int64_t d_out, int64_t d_in);
harp_status harp_rotate_weight(const harp_schedule* su, const void* blocks_u,
                               const float* scales_u, const int8_t* signs_u,
                               const harp_schedule* sv, const void* blocks_v,
                               const float* scales_v, const int8_t* signs_v,
                               harp_dtype block_dtype, const void* w,
                               int64_t ldw, void* w_out, int64_t ldo,
                               int64_t d_out, int64_t d_in, harp_dtype io_dtype,
                               int32_t inverse, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Composition of k randomized Hadamard transforms [RHT]
 *   inverse == 0:  y = (H D_k) ... (H D_1) x
 *   inverse != 0:  y = (D_1 H) ... (D_k H) x
 * H is the normalised Sylvester Hadamard of order d; every radix of s must be
 * a power of two (else HARP_ERR_UNSUPPORTED); the schedule only names a
 * factorisation of H.  signs: k x d int8 (row j is D_{j+1}).  1 <= k <= 8.
 * ---------------------------------------------------------------------- */
harp_status rht_compose(const harp_schedule* s, int64_t d, const int8_t* signs,
                        int32_t k, const void* x, int64_t ldx, void* y,
                        int64_t ldy, int64_t rows, harp_dtype io_dtype,
                        int32_t inverse, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Diagnostics (host).
 * ---------------------------------------------------------------------- */
const char* harp_status_str(harp_status st);
/* Message for the last non-OK status returned on this thread ("" if none). */
const char* harp_last_error(void);
/* Library version string. */
const char* harp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HARP_H_ */
