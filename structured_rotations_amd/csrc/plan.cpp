// Host-side schedule planning and argument validation (plain C++, no HIP).
#include "plan.h"

#include <cstdint>
#include <cstdio>

namespace harp {

namespace {
thread_local std::string g_last_error;
}

void set_last_error(const std::string& msg) { g_last_error = msg; }
const char* last_error() { return g_last_error.c_str(); }

std::string make_plan(int m, const int32_t* radix, int64_t d, Plan* p) {
  char buf[160];
  if (radix == nullptr) return "schedule is NULL";
  if (m < 1 || m > kMaxStages) {
    std::snprintf(buf, sizeof buf, "schedule has m=%d stages (allowed 1..%d)", m, kMaxStages);
    return buf;
  }
  if (d < 2 || d > kMaxD) {
    std::snprintf(buf, sizeof buf, "d=%lld outside 2..%lld", (long long)d, (long long)kMaxD);
    return buf;
  }
  int64_t prod = 1;
  for (int t = 0; t < m; ++t) {
    if (radix[t] < 2 || radix[t] > kMaxRadix) {
      std::snprintf(buf, sizeof buf, "radix[%d]=%d outside 2..%d", t, radix[t], kMaxRadix);
      return buf;
    }
    prod *= radix[t];
    if (prod > kMaxD) break;
  }
  if (prod != d) {
    std::snprintf(buf, sizeof buf, "product of the radices (%lld) != d (%lld)", (long long)prod, (long long)d);
    return buf;
  }
  Plan q;
  q.m = m;
  q.d = d;
  int64_t s = 1;
  for (int t = m - 1; t >= 0; --t) {
    q.radix[t] = radix[t];
    q.stride[t] = s;
    s *= radix[t];
  }
  for (int t = 0; t < m; ++t) {
    const int64_t b = radix[t];
    const int64_t ng = d / b;
    q.blk_off[t] = q.n_blk;
    q.grp_off[t] = q.n_grp;
    q.theta_off[t] = q.n_theta;
    q.n_blk += ng * b * b;
    q.n_grp += ng;
    q.n_theta += ng * (b == 2 ? 1 : b * (b - 1) / 2);
    if (is_pow2(b)) {
      q.gauss_off[t] = -1;
    } else {
      q.gauss_off[t] = q.n_gauss;
      q.n_gauss += b * b;
      q.all_pow2 = false;
    }
  }
  *p = q;
  return "";
}

std::string check_rows(const void* x, int64_t ldx, const void* y, int64_t ldy,
                       int64_t rows, int64_t d, int elem_bytes) {
  char buf[160];
  if (rows < 0) return "rows < 0";
  if (rows == 0) return "";
  if (x == nullptr || y == nullptr) return "x or y is NULL with rows > 0";
  if (d < 1) return "d < 1";
  if (ldx < d || ldy < d) {
    std::snprintf(buf, sizeof buf, "leading dimension smaller than d (ldx=%lld ldy=%lld d=%lld)",
                  (long long)ldx, (long long)ldy, (long long)d);
    return buf;
  }
  const auto ux = reinterpret_cast<uintptr_t>(x);
  const auto uy = reinterpret_cast<uintptr_t>(y);
  if (ux % elem_bytes != 0 || uy % elem_bytes != 0) return "x or y not aligned to its element size";
  if (x == y && ldx != ldy) return "in-place call (x == y) needs ldx == ldy";
  // byte extent (rows - 1) * ld + d elements of each buffer, which must fit
  // in the address space above its base
  auto extent = [&](uintptr_t base, int64_t ld, uint64_t* end) {
    if (rows - 1 > (INT64_MAX - d) / ld) return false;
    const int64_t el = (rows - 1) * ld + d;
    if (el > INT64_MAX / elem_bytes) return false;
    const uint64_t bytes = (uint64_t)el * (uint64_t)elem_bytes;
    if ((uint64_t)base > UINT64_MAX - bytes) return false;
    *end = (uint64_t)base + bytes;
    return true;
  };
  uint64_t ex = 0, ey = 0;
  if (!extent(ux, ldx, &ex) || !extent(uy, ldy, &ey)) return "rows x leading dimension exceeds the address space";
  // reject partial overlap: the byte ranges intersect but the bases differ
  if (x != y && ux < ey && uy < ex) return "x and y overlap without being the same buffer";
  return "";
}

}  // namespace harp
