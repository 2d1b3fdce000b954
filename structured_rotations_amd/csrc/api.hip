// extern "C" entry points declared in include/harp.h: argument validation on
// the host (before any HIP call), then the kernel launchers.
#include <cstdio>
#include <mutex>
#include <string>

#include "harp.h"
#include "kernels.h"
#include "plan.h"

using harp::DT;
using harp::Plan;

namespace {

harp_status fail(harp_status st, const std::string& msg) {
  harp::set_last_error(msg);
  return st;
}

harp_status launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return HARP_OK;
  std::string msg = std::string(what) + ": " + hipGetErrorString(e);
  return fail(HARP_ERR_LAUNCH, msg);
}

bool plan_of(const harp_schedule* s, int64_t d, Plan* p, std::string* err) {
  if (s == nullptr) {
    *err = "schedule is NULL";
    return false;
  }
  *err = harp::make_plan(s->m, s->radix, d, p);
  return err->empty();
}

bool io_ok(harp_dtype t) { return t == HARP_F32 || t == HARP_BF16; }
bool blk_ok(harp_dtype t) { return t == HARP_F32 || t == HARP_BF16 || t == HARP_I8; }

harp_status apply_impl(bool inverse, const harp_schedule* s, int64_t d, const void* blocks,
                       harp_dtype block_dtype, const float* block_scales, const int8_t* signs,
                       const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows,
                       harp_dtype io_dtype, hipStream_t stream) {
  Plan pl;
  std::string err;
  if (!plan_of(s, d, &pl, &err)) return fail(HARP_ERR_INVALID_ARG, err);
  if (!io_ok(io_dtype)) return fail(HARP_ERR_UNSUPPORTED, "io_dtype must be HARP_F32 or HARP_BF16");
  if (!blk_ok(block_dtype)) return fail(HARP_ERR_UNSUPPORTED, "block_dtype must be HARP_F32, HARP_BF16 or HARP_I8");
  if ((block_dtype == HARP_I8) != (block_scales != nullptr))
    return fail(HARP_ERR_INVALID_ARG, "block_scales must be given exactly for HARP_I8 blocks");
  const int eb = io_dtype == HARP_F32 ? 4 : 2;
  err = harp::check_rows(x, ldx, y, ldy, rows, d, eb);
  if (!err.empty()) return fail(HARP_ERR_INVALID_ARG, err);
  if (rows == 0) return HARP_OK;
  if (blocks == nullptr) return fail(HARP_ERR_INVALID_ARG, "blocks is NULL");
  const DT io = static_cast<DT>(io_dtype);
  return launch_status(harp::launch_apply_rows(pl, inverse, blocks, static_cast<DT>(block_dtype),
                                               block_scales, signs, x, ldx, io, y, ldy, io, rows,
                                               stream),
                       inverse ? "harp_apply_inverse" : "harp_apply");
}

}  // namespace

extern "C" {

int64_t harp_theta_count(const harp_schedule* s, int64_t d) {
  Plan p;
  std::string err;
  return plan_of(s, d, &p, &err) ? p.n_theta : -1;
}

int64_t harp_gauss_count(const harp_schedule* s, int64_t d) {
  Plan p;
  std::string err;
  return plan_of(s, d, &p, &err) ? p.n_gauss : -1;
}

int64_t harp_block_count(const harp_schedule* s, int64_t d) {
  Plan p;
  std::string err;
  return plan_of(s, d, &p, &err) ? p.n_blk : -1;
}

int64_t harp_group_count(const harp_schedule* s, int64_t d) {
  Plan p;
  std::string err;
  return plan_of(s, d, &p, &err) ? p.n_grp : -1;
}

harp_status harp_materialize_blocks(const harp_schedule* s, int64_t d, const double* theta,
                                    const double* gauss, harp_dtype block_dtype, void* blocks_out,
                                    float* scales_out, hipStream_t stream) {
  Plan pl;
  std::string err;
  if (!plan_of(s, d, &pl, &err)) return fail(HARP_ERR_INVALID_ARG, err);
  if (!blk_ok(block_dtype)) return fail(HARP_ERR_UNSUPPORTED, "block_dtype must be HARP_F32, HARP_BF16 or HARP_I8");
  if (theta == nullptr) return fail(HARP_ERR_INVALID_ARG, "theta is NULL");
  if (pl.n_gauss > 0 && gauss == nullptr)
    return fail(HARP_ERR_INVALID_ARG, "gauss is NULL but the schedule has a non-power-of-two radix");
  if (blocks_out == nullptr) return fail(HARP_ERR_INVALID_ARG, "blocks_out is NULL");
  if ((block_dtype == HARP_I8) != (scales_out != nullptr))
    return fail(HARP_ERR_INVALID_ARG, "scales_out must be given exactly for HARP_I8 blocks");
  return launch_status(harp::launch_materialize(pl, theta, nullptr, nullptr, gauss, static_cast<DT>(block_dtype),
                                                blocks_out, scales_out, stream),
                       "harp_materialize_blocks");
}

harp_status harp_quantize_theta(const harp_schedule* s, int64_t d, const double* theta, int8_t* theta_codes,
                                float* theta_scales, hipStream_t stream) {
  Plan pl;
  std::string err;
  if (!plan_of(s, d, &pl, &err)) return fail(HARP_ERR_INVALID_ARG, err);
  if (theta == nullptr) return fail(HARP_ERR_INVALID_ARG, "theta is NULL");
  if (theta_codes == nullptr) return fail(HARP_ERR_INVALID_ARG, "theta_codes is NULL");
  if (theta_scales == nullptr) return fail(HARP_ERR_INVALID_ARG, "theta_scales is NULL");
  return launch_status(harp::launch_quantize_theta(pl, theta, theta_codes, theta_scales, stream),
                       "harp_quantize_theta");
}

harp_status harp_materialize_blocks_q8(const harp_schedule* s, int64_t d, const int8_t* theta_codes,
                                       const float* theta_scales, const double* gauss, harp_dtype block_dtype,
                                       void* blocks_out, float* scales_out, hipStream_t stream) {
  Plan pl;
  std::string err;
  if (!plan_of(s, d, &pl, &err)) return fail(HARP_ERR_INVALID_ARG, err);
  if (!blk_ok(block_dtype)) return fail(HARP_ERR_UNSUPPORTED, "block_dtype must be HARP_F32, HARP_BF16 or HARP_I8");
  if (theta_codes == nullptr) return fail(HARP_ERR_INVALID_ARG, "theta_codes is NULL");
  if (theta_scales == nullptr) return fail(HARP_ERR_INVALID_ARG, "theta_scales is NULL");
  if (pl.n_gauss > 0 && gauss == nullptr)
    return fail(HARP_ERR_INVALID_ARG, "gauss is NULL but the schedule has a non-power-of-two radix");
  if (blocks_out == nullptr) return fail(HARP_ERR_INVALID_ARG, "blocks_out is NULL");
  if ((block_dtype == HARP_I8) != (scales_out != nullptr))
    return fail(HARP_ERR_INVALID_ARG, "scales_out must be given exactly for HARP_I8 blocks");
  return launch_status(harp::launch_materialize(pl, nullptr, theta_codes, theta_scales, gauss,
                                                static_cast<DT>(block_dtype), blocks_out, scales_out, stream),
                       "harp_materialize_blocks_q8");
}

int64_t harp_apply_decode_workspace(const harp_schedule* s, int64_t d, harp_dtype block_dtype, int64_t rows) {
  Plan pl;
  std::string err;
  if (!plan_of(s, d, &pl, &err) || !blk_ok(block_dtype) || rows < 0) return -1;
  return harp::decode_workspace_bytes(pl, static_cast<DT>(block_dtype), rows);
}

harp_status harp_apply_decode(const harp_schedule* s, int64_t d, const void* blocks, harp_dtype block_dtype,
                              const float* block_scales, const int8_t* signs, const void* x, int64_t ldx,
                              void* y, int64_t ldy, int64_t rows, harp_dtype io_dtype, int32_t inverse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Plan pl;
  std::string err;
  if (!plan_of(s, d, &pl, &err)) return fail(HARP_ERR_INVALID_ARG, err);
  if (!io_ok(io_dtype)) return fail(HARP_ERR_UNSUPPORTED, "io_dtype must be HARP_F32 or HARP_BF16");
  if (!blk_ok(block_dtype)) return fail(HARP_ERR_UNSUPPORTED, "block_dtype must be HARP_F32, HARP_BF16 or HARP_I8");
  if ((block_dtype == HARP_I8) != (block_scales != nullptr))
    return fail(HARP_ERR_INVALID_ARG, "block_scales must be given exactly for HARP_I8 blocks");
  if (rows > HARP_DECODE_MAX_ROWS)
    return fail(HARP_ERR_INVALID_ARG, "harp_apply_decode takes at most HARP_DECODE_MAX_ROWS rows; use harp_apply");
  const int eb = io_dtype == HARP_F32 ? 4 : 2;
  err = harp::check_rows(x, ldx, y, ldy, rows, d, eb);
  if (!err.empty()) return fail(HARP_ERR_INVALID_ARG, err);
  const int64_t need = harp::decode_workspace_bytes(pl, static_cast<DT>(block_dtype), rows);
  if (need < 0) return fail(HARP_ERR_UNSUPPORTED, "no split of this schedule into two digit runs fits a workgroup");
  if (rows == 0) return HARP_OK;
  if (blocks == nullptr) return fail(HARP_ERR_INVALID_ARG, "blocks is NULL");
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < (size_t)need)
      return fail(HARP_ERR_INVALID_ARG, "workspace missing or smaller than harp_apply_decode_workspace()");
    if (reinterpret_cast<uintptr_t>(workspace) % 4 != 0)
      return fail(HARP_ERR_INVALID_ARG, "workspace must be 4-byte aligned");
  }
  const DT io = static_cast<DT>(io_dtype);
  return launch_status(harp::launch_apply_decode(pl, inverse != 0, blocks, static_cast<DT>(block_dtype), block_scales,
                                                 signs, x, ldx, io, y, ldy, rows, static_cast<float*>(workspace),
                                                 stream),
                       "harp_apply_decode");
}

}  // extern "C"

// ------------------------------------------------------------------------
// Hand-off buffer of harp_apply_decode_noalloc: the fp32 rows passed from the
// first launch to the second.  Each GPU the library runs on holds its own
// copy until the process ends.  Host code never uses the array's name as an
// address (it is a host-side stand-in); it uses the device address obtained
// once per device with hipGetSymbolAddress, with that device current.
namespace {

static __device__ __align__(256) float scratch[HARP_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The calling thread's current device's copy of `scratch`.
harp_status device_scratch(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HARP_ERR_LAUNCH, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(HARP_ERR_UNSUPPORTED, "device index beyond the library's table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (es != hipSuccess || p == nullptr)
      return fail(HARP_ERR_LAUNCH, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(es));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HARP_OK;
}

}  // namespace

extern "C" {

harp_status harp_apply_decode_noalloc(const harp_schedule* s, int64_t d, const void* blocks, harp_dtype block_dtype,
                                      const float* block_scales, const int8_t* signs, const void* x, int64_t ldx,
                                      void* y, int64_t ldy, int64_t rows, harp_dtype io_dtype, int32_t inverse,
                                      hipStream_t stream) {
  Plan pl;
  std::string err;
  if (!plan_of(s, d, &pl, &err)) return fail(HARP_ERR_INVALID_ARG, err);
  if (!io_ok(io_dtype)) return fail(HARP_ERR_UNSUPPORTED, "io_dtype must be HARP_F32 or HARP_BF16");
  if (!blk_ok(block_dtype)) return fail(HARP_ERR_UNSUPPORTED, "block_dtype must be HARP_F32, HARP_BF16 or HARP_I8");
  if ((block_dtype == HARP_I8) != (block_scales != nullptr))
    return fail(HARP_ERR_INVALID_ARG, "block_scales must be given exactly for HARP_I8 blocks");
  if (rows > HARP_DECODE_MAX_ROWS)
    return fail(HARP_ERR_INVALID_ARG,
                "harp_apply_decode_noalloc takes at most HARP_DECODE_MAX_ROWS rows; use harp_apply");
  const int eb = io_dtype == HARP_F32 ? 4 : 2;
  err = harp::check_rows(x, ldx, y, ldy, rows, d, eb);
  if (!err.empty()) return fail(HARP_ERR_INVALID_ARG, err);
  const int64_t need = harp::decode_workspace_bytes(pl, static_cast<DT>(block_dtype), rows);
  if (need < 0) return fail(HARP_ERR_UNSUPPORTED, "no split of this schedule into two digit runs fits a workgroup");
  if (need > (int64_t)HARP_NOALLOC_SCRATCH_BYTES)
    return fail(HARP_ERR_INVALID_ARG,
                "rows * d * 4 exceeds HARP_NOALLOC_SCRATCH_BYTES; use harp_apply_decode with a workspace");
  if (rows == 0) return HARP_OK;
  if (blocks == nullptr) return fail(HARP_ERR_INVALID_ARG, "blocks is NULL");
  void* ws = nullptr;
  if (need > 0) {
    const harp_status st = device_scratch(&ws);
    if (st != HARP_OK) return st;
  }
  const DT io = static_cast<DT>(io_dtype);
  return launch_status(harp::launch_apply_decode(pl, inverse != 0, blocks, static_cast<DT>(block_dtype), block_scales,
                                                 signs, x, ldx, io, y, ldy, rows, static_cast<float*>(ws), stream),
                       "harp_apply_decode_noalloc");
}

int64_t harp_apply_vjp_workspace(const harp_schedule* s, int64_t d, int64_t rows) {
  Plan pl;
  std::string err;
  if (!plan_of(s, d, &pl, &err) || rows < 0) return -1;
  return harp::vjp_workspace_bytes(pl, rows);
}

harp_status harp_apply_vjp(const harp_schedule* s, int64_t d, const void* blocks, harp_dtype block_dtype,
                           const float* block_scales, const int8_t* signs, const void* x, int64_t ldx,
                           const void* dy, int64_t lddy, void* dx, int64_t lddx, int64_t rows,
                           harp_dtype io_dtype, float* dblocks, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  Plan pl;
  std::string err;
  if (!plan_of(s, d, &pl, &err)) return fail(HARP_ERR_INVALID_ARG, err);
  if (!io_ok(io_dtype)) return fail(HARP_ERR_UNSUPPORTED, "io_dtype must be HARP_F32 or HARP_BF16");
  if (!blk_ok(block_dtype)) return fail(HARP_ERR_UNSUPPORTED, "block_dtype must be HARP_F32, HARP_BF16 or HARP_I8");
  if ((block_dtype == HARP_I8) != (block_scales != nullptr))
    return fail(HARP_ERR_INVALID_ARG, "block_scales must be given exactly for HARP_I8 blocks");
  const int64_t need = harp::vjp_workspace_bytes(pl, rows < 0 ? 0 : rows);
  if (need < 0)
    return fail(HARP_ERR_UNSUPPORTED, "harp_apply_vjp needs every radix <= 8 and a workspace size that fits in int64");
  const int eb = io_dtype == HARP_F32 ? 4 : 2;
  err = harp::check_rows(x, ldx, dy, lddy, rows, d, eb);
  if (!err.empty()) return fail(HARP_ERR_INVALID_ARG, "x/dy: " + err);
  if (dx != nullptr) {
    err = harp::check_rows(dy, lddy, dx, lddx, rows, d, eb);
    if (!err.empty()) return fail(HARP_ERR_INVALID_ARG, "dx: " + err);
  }
  if (dblocks == nullptr) return fail(HARP_ERR_INVALID_ARG, "dblocks is NULL");
  if (blocks == nullptr) return fail(HARP_ERR_INVALID_ARG, "blocks is NULL");
  if (rows == 0) return fail(HARP_ERR_INVALID_ARG, "rows must be at least 1");
  if (workspace == nullptr || workspace_bytes < (size_t)need)
    return fail(HARP_ERR_INVALID_ARG, "workspace missing or smaller than harp_apply_vjp_workspace()");
  if (reinterpret_cast<uintptr_t>(workspace) % 4 != 0)
    return fail(HARP_ERR_INVALID_ARG, "workspace must be 4-byte aligned");
  return launch_status(harp::launch_apply_vjp(pl, blocks, static_cast<DT>(block_dtype), block_scales, signs, x, ldx,
                                              dy, lddy, dx, lddx, static_cast<DT>(io_dtype), rows, dblocks,
                                              workspace, stream),
                       "harp_apply_vjp");
}

harp_status harp_theta_vjp(const harp_schedule* s, int64_t d, const double* theta, const double* gauss,
                           const float* dblocks, double* dtheta, hipStream_t stream) {
  Plan pl;
  std::string err;
  if (!plan_of(s, d, &pl, &err)) return fail(HARP_ERR_INVALID_ARG, err);
  if (theta == nullptr) return fail(HARP_ERR_INVALID_ARG, "theta is NULL");
  if (pl.n_gauss > 0 && gauss == nullptr)
    return fail(HARP_ERR_INVALID_ARG, "gauss is NULL but the schedule has a non-power-of-two radix");
  if (dblocks == nullptr) return fail(HARP_ERR_INVALID_ARG, "dblocks is NULL");
  if (dtheta == nullptr) return fail(HARP_ERR_INVALID_ARG, "dtheta is NULL");
  return launch_status(harp::launch_theta_vjp(pl, theta, gauss, dblocks, dtheta, stream), "harp_theta_vjp");
}

harp_status harp_apply(const harp_schedule* s, int64_t d, const void* blocks, harp_dtype block_dtype,
                       const float* block_scales, const int8_t* signs, const void* x, int64_t ldx,
                       void* y, int64_t ldy, int64_t rows, harp_dtype io_dtype, hipStream_t stream) {
  return apply_impl(false, s, d, blocks, block_dtype, block_scales, signs, x, ldx, y, ldy, rows, io_dtype,
                    stream);
}

harp_status harp_apply_inverse(const harp_schedule* s, int64_t d, const void* blocks, harp_dtype block_dtype,
                               const float* block_scales, const int8_t* signs, const void* y, int64_t ldy,
                               void* x, int64_t ldx, int64_t rows, harp_dtype io_dtype,
                               hipStream_t stream) {
  return apply_impl(true, s, d, blocks, block_dtype, block_scales, signs, y, ldy, x, ldx, rows, io_dtype,
                    stream);
}

size_t harp_rotate_weight_workspace(int64_t d_out, int64_t d_in) {
  if (d_out <= 0 || d_in <= 0) return 0;
  return (size_t)d_out * (size_t)d_in * sizeof(float);
}

harp_status harp_rotate_weight(const harp_schedule* su, const void* blocks_u, const float* scales_u,
                               const int8_t* signs_u, const harp_schedule* sv, const void* blocks_v,
                               const float* scales_v, const int8_t* signs_v, harp_dtype block_dtype,
                               const void* w, int64_t ldw, void* w_out, int64_t ldo, int64_t d_out,
                               int64_t d_in, harp_dtype io_dtype, int32_t inverse, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  Plan pu, pv;
  std::string err;
  if (!plan_of(su, d_out, &pu, &err)) return fail(HARP_ERR_INVALID_ARG, "U schedule: " + err);
  if (!plan_of(sv, d_in, &pv, &err)) return fail(HARP_ERR_INVALID_ARG, "V schedule: " + err);
  if (!io_ok(io_dtype)) return fail(HARP_ERR_UNSUPPORTED, "io_dtype must be HARP_F32 or HARP_BF16");
  if (!blk_ok(block_dtype)) return fail(HARP_ERR_UNSUPPORTED, "block_dtype must be HARP_F32, HARP_BF16 or HARP_I8");
  if (blocks_u == nullptr || blocks_v == nullptr) return fail(HARP_ERR_INVALID_ARG, "blocks_u or blocks_v is NULL");
  const bool i8 = block_dtype == HARP_I8;
  if (i8 != (scales_u != nullptr) || i8 != (scales_v != nullptr))
    return fail(HARP_ERR_INVALID_ARG, "scales must be given exactly for HARP_I8 blocks");
  const int eb = io_dtype == HARP_F32 ? 4 : 2;
  err = harp::check_rows(w, ldw, w_out, ldo, d_out, d_in, eb);
  if (!err.empty()) return fail(HARP_ERR_INVALID_ARG, err);
  if (workspace != nullptr) {
    if (workspace_bytes < harp_rotate_weight_workspace(d_out, d_in))
      return fail(HARP_ERR_INVALID_ARG, "workspace smaller than harp_rotate_weight_workspace()");
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return fail(HARP_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  }
  const DT io = static_cast<DT>(io_dtype);
  const DT bdt = static_cast<DT>(block_dtype);
  const bool inv = inverse != 0;
  // Passes over the row index (U): runs of consecutive stages whose rows fit
  // one LDS tile of 64 columns next to two coefficient slots (nsub rows x
  // (64 + 2 x widest padded radix) floats in 160 KiB: 512 rows for radix 8).
  int cut[harp::kMaxStages + 1];
  int npass = 0;
  cut[0] = 0;
  auto pad4 = [](int b) { return (b + 3) & ~3; };
  for (int t = 0; t < pu.m;) {
    int64_t prod = pu.radix[t];
    int cw = pad4(pu.radix[t]) > 4 ? pad4(pu.radix[t]) : 4;
    int e = t + 1;
    while (e < pu.m) {
      const int64_t np = prod * pu.radix[e];
      const int cwn = pad4(pu.radix[e]) > cw ? pad4(pu.radix[e]) : cw;
      if (np * (64 + 2 * cwn) > 40960) break;
      prod = np;
      cw = cwn;
      ++e;
    }
    cut[++npass] = e;
    t = e;
  }
  // Buffer chain: the first pass reads w; every later pass reads what the
  // previous one wrote; the final pass writes w_out.
  float* ws = static_cast<float*>(workspace);
  const void* src = w;
  int64_t lds_ = ldw;
  DT sdt = io;
  void* mid = ws ? static_cast<void*>(ws) : w_out;
  const int64_t ldm = ws ? d_in : ldo;
  const DT mdt = ws ? DT::F32 : io;
  const int total = 1 + npass;
  int done = 0;
  auto dst_for = [&](int step, int64_t* ldd, DT* ddt) -> void* {
    if (step == total - 1) { *ldd = ldo; *ddt = io; return w_out; }
    *ldd = ldm; *ddt = mdt; return mid;
  };
  // U mixes the rows of W (it acts on every column) and V its columns (it
  // acts on every row), so the passes commute.  In place, V goes first.  With an fp32
  // workspace, the first and last passes convert between io_dtype and fp32
  // and the middle ones run fp32 to fp32: a column pass opens and closes the
  // chain (their 16-byte paths take either conversion) and V, whose fastest
  // kernels keep one element type, runs fp32 to fp32 in between.
  auto row_pass = [&]() -> harp_status {
    int64_t ldd; DT ddt;
    void* dst = dst_for(done, &ldd, &ddt);
    hipError_t e = harp::launch_apply_rows(pv, inv, blocks_v, bdt, scales_v, signs_v, src, lds_, sdt, dst, ldd,
                                           ddt, d_out, stream);
    if (e != hipSuccess) return launch_status(e, "harp_rotate_weight (row pass)");
    src = dst; lds_ = ldd; sdt = ddt; ++done;
    return HARP_OK;
  };
  // U on the columns: forward runs the passes in order with the sign read
  // with the first pass; the inverse runs them in reverse with the sign
  // written by the last pass.
  auto col_pass = [&](int i) -> harp_status {
    const int pi = inv ? npass - 1 - i : i;
    const int t0 = cut[pi], t1 = cut[pi + 1];
    int sign_mode = 0;
    if (!inv && t0 == 0) sign_mode = 1;
    if (inv && t0 == 0) sign_mode = 2;
    int64_t ldd; DT ddt;
    void* dst = dst_for(done, &ldd, &ddt);
    hipError_t e = harp::launch_apply_cols(pu, t0, t1, inv, blocks_u, bdt, scales_u, signs_u, sign_mode, src,
                                           lds_, sdt, dst, ldd, ddt, d_in, stream);
    if (e != hipSuccess) return launch_status(e, "harp_rotate_weight (column pass)");
    src = dst; lds_ = ldd; sdt = ddt; ++done;
    return HARP_OK;
  };
  const bool v_middle = ws != nullptr && npass >= 2;
  harp_status st = HARP_OK;
  if (v_middle) {
    st = col_pass(0);
    if (st == HARP_OK) st = row_pass();
    for (int i = 1; i < npass && st == HARP_OK; ++i) st = col_pass(i);
  } else {
    st = row_pass();
    for (int i = 0; i < npass && st == HARP_OK; ++i) st = col_pass(i);
  }
  return st;
}

harp_status rht_compose(const harp_schedule* s, int64_t d, const int8_t* signs, int32_t k, const void* x,
                        int64_t ldx, void* y, int64_t ldy, int64_t rows, harp_dtype io_dtype, int32_t inverse,
                        hipStream_t stream) {
  Plan pl;
  std::string err;
  if (!plan_of(s, d, &pl, &err)) return fail(HARP_ERR_INVALID_ARG, err);
  if (!pl.all_pow2) return fail(HARP_ERR_UNSUPPORTED, "rht_compose needs power-of-two radices");
  if (k < 1 || k > 8) return fail(HARP_ERR_INVALID_ARG, "k must be in 1..8");
  if (!io_ok(io_dtype)) return fail(HARP_ERR_UNSUPPORTED, "io_dtype must be HARP_F32 or HARP_BF16");
  const int eb = io_dtype == HARP_F32 ? 4 : 2;
  err = harp::check_rows(x, ldx, y, ldy, rows, d, eb);
  if (!err.empty()) return fail(HARP_ERR_INVALID_ARG, err);
  if (rows == 0) return HARP_OK;
  if (signs == nullptr) return fail(HARP_ERR_INVALID_ARG, "signs is NULL");
  const DT io = static_cast<DT>(io_dtype);
  return launch_status(harp::launch_rht(pl, signs, k, inverse != 0, x, ldx, io, y, ldy, io, rows, stream),
                       "rht_compose");
}

const char* harp_status_str(harp_status st) {
  switch (st) {
    case HARP_OK: return "HARP_OK";
    case HARP_ERR_INVALID_ARG: return "HARP_ERR_INVALID_ARG";
    case HARP_ERR_UNSUPPORTED: return "HARP_ERR_UNSUPPORTED";
    case HARP_ERR_LAUNCH: return "HARP_ERR_LAUNCH";
    default: return "HARP_STATUS_UNKNOWN";
  }
}

const char* harp_last_error(void) { return harp::last_error(); }

const char* harp_version(void) { return "harp-gfx950 0.1"; }

}  // extern "C"
