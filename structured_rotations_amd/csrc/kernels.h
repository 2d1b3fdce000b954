// Launchers for the gfx950 kernels (host side, called by the C ABI layer
// after every argument has been validated).
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace harp {

enum class DT : int { F32 = 0, BF16 = 1, I8 = 2, F64 = 3 };

// Element size in bytes of an I/O dtype (F32 or BF16).
inline int io_bytes(DT t) { return t == DT::F32 ? 4 : 2; }

// Rows of length pl.d:  y = M x  (inverse=false) or  y = M^T x  (inverse=true).
// sign_mode: 0 = no sign, 1 = sign on the input side (forward), 2 = sign on the
// output side (inverse).  stage_lo/stage_hi restrict the stages applied
// (all stages: 0, pl.m).
hipError_t launch_apply_rows(const Plan& pl, bool inverse, const void* blocks, DT bdt,
                             const float* scales, const int8_t* signs, const void* x,
                             int64_t ldx, DT in_dt, void* y, int64_t ldy, DT out_dt,
                             int64_t rows, hipStream_t stream);

// Row-tile kernels (radices 2, 4, 5, 8; d % 64 == 0, d <= 5120; 16-byte
// aligned rows and blocks; same I/O dtype on both sides): the vector-ALU
// kernel and the matrix-core kernel.  roles selects the wave split.
bool row_path_supported(const Plan& pl, DT io, const void* blocks, const int8_t* signs, const void* x, int64_t ldx,
                        const void* y, int64_t ldy);
hipError_t launch_apply_valu(const Plan& pl, bool inverse, const void* blocks, DT bdt, const float* scales,
                             const int8_t* signs, const void* x, int64_t ldx, DT io, void* y, int64_t ldy,
                             int64_t rows, int roles, hipStream_t stream);
// Schedule-specialised matrix-core kernel: d = 4096 (8,8,8,8) and d = 5120
// (8,8,8,5,2) with fp32, bf16 or int8 blocks (plus the row-path alignment
// rules); scales: the per-group scales of int8 blocks.
bool fast_path_supported(const Plan& pl, DT bdt);
hipError_t launch_apply_fast(const Plan& pl, bool inverse, const void* blocks, DT bdt, const float* scales,
                             const int8_t* signs, const void* x, int64_t ldx, DT io, void* y, int64_t ldy,
                             int64_t rows, hipStream_t stream);
hipError_t launch_apply_mfma(const Plan& pl, bool inverse, const void* blocks, DT bdt, const float* scales,
                             const int8_t* signs, const void* x, int64_t ldx, DT io, void* y, int64_t ldy,
                             int64_t rows, int roles, hipStream_t stream);

// Column passes of the two-sided rotation: apply stages [t0, t1) of the
// schedule `pl` (acting on the row index of a pl.d x ncols matrix) to every
// column.  Forward order (inverse=false) or transposed blocks in reverse
// order (inverse=true).  sign_mode as above (sign indexed by the row).
hipError_t launch_apply_cols(const Plan& pl, int t0, int t1, bool inverse, const void* blocks,
                             DT bdt, const float* scales, const int8_t* signs, int sign_mode,
                             const void* x, int64_t ldx, DT in_dt, void* y, int64_t ldy,
                             DT out_dt, int64_t ncols, hipStream_t stream);

// Column runs of at most 32 rows (the product of the radices of stages
// [t0, t1)): one dense nsub x nsub product per row group on the matrix cores;
// launch_apply_cols hands such runs over.  Any column count and row stride.
bool cols_dense_supported(const Plan& pl, int t0, int t1);
hipError_t launch_apply_cols_dense(const Plan& pl, int t0, int t1, bool inverse, const void* blocks, DT bdt,
                                   const float* scales, const int8_t* signs, int sign_mode, const void* x,
                                   int64_t ldx, DT in_dt, void* y, int64_t ldy, DT out_dt, int64_t ncols,
                                   hipStream_t stream);

// k composed randomized Hadamard transforms over rows (all radices powers of two).
hipError_t launch_rht(const Plan& pl, const int8_t* signs, int k, bool inverse, const void* x,
                      int64_t ldx, DT in_dt, void* y, int64_t ldy, DT out_dt, int64_t rows,
                      hipStream_t stream);

// B_{t,c} = Q_{t,c}(theta) G_{b_t} for all stages, in fp64, rounded to bdt.
// theta is fp64, or (theta NULL) int8 codes tcode with one fp32 scale per stage.
hipError_t launch_materialize(const Plan& pl, const double* theta, const int8_t* tcode,
                              const float* tscale, const double* gauss, DT bdt, void* blocks,
                              float* scales, hipStream_t stream);

// Small-batch apply: two launches over digit runs (fp32 rows in ws between
// them) or one.  decode_workspace_bytes: ws bytes needed (0 for one launch),
// -1 if no digit split fits a workgroup.
int64_t decode_workspace_bytes(const Plan& pl, DT bdt, int64_t rows);
hipError_t launch_apply_decode(const Plan& pl, bool inverse, const void* blocks, DT bdt, const float* scales,
                               const int8_t* signs, const void* x, int64_t ldx, DT io, void* y, int64_t ldy,
                               int64_t rows, float* ws, hipStream_t stream);

// Reverse mode of the row transform: dx (optional) and dL/dB for every block
// (fp32, overwritten).  ws: vjp_workspace_bytes(); -1 if a radix exceeds 8.
int64_t vjp_workspace_bytes(const Plan& pl, int64_t rows);
hipError_t launch_apply_vjp(const Plan& pl, const void* blocks, DT bdt, const float* scales, const int8_t* signs,
                            const void* x, int64_t ldx, const void* dy, int64_t lddy, void* dx, int64_t lddx,
                            DT io, int64_t rows, float* dblocks, void* ws, hipStream_t stream);
// dL/dtheta from dL/dB (fp64 per group).
hipError_t launch_theta_vjp(const Plan& pl, const double* theta, const double* gauss, const float* dblocks,
                            double* dtheta, hipStream_t stream);

// int8 codes + one fp32 scale per stage of fp64 theta.
hipError_t launch_quantize_theta(const Plan& pl, const double* theta, int8_t* codes, float* scales,
                                 hipStream_t stream);

}  // namespace harp
