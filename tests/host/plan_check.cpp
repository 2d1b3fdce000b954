// Host-side checks of the schedule planner and of the row-argument
// validation in structured_rotations_amd/csrc/plan.cpp, meant to be built
// with AddressSanitizer and UndefinedBehaviorSanitizer (g++, no HIP).
//
//   plan_check              randomized checks; prints "ok" or the first failure
//   plan_check print d b..  prints the plan of one schedule as key=value lines
//
// The schedule rules are those of the HARP technical summary, §2.1: radices
// b_t >= 2 whose product is d, digit t with stride prod_{u>t} b_u.
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "plan.h"

using harp::Plan;

namespace {

int fail(const char* what, long long it) {
  std::printf("FAIL at iteration %lld: %s\n", it, what);
  return 1;
}

void print_list(const char* key, const int64_t* v, int m) {
  std::printf("%s=", key);
  for (int t = 0; t < m; ++t) std::printf("%s%lld", t ? "," : "", (long long)v[t]);
  std::printf("\n");
}

int print_plan(int argc, char** argv) {
  const int64_t d = std::atoll(argv[2]);
  std::vector<int32_t> r;
  for (int i = 3; i < argc; ++i) r.push_back(std::atoi(argv[i]));
  Plan p;
  const std::string e = harp::make_plan((int)r.size(), r.data(), d, &p);
  if (!e.empty()) {
    std::printf("error=%s\n", e.c_str());
    return 0;
  }
  std::printf("n_blk=%lld\nn_grp=%lld\nn_theta=%lld\nn_gauss=%lld\n", (long long)p.n_blk, (long long)p.n_grp,
              (long long)p.n_theta, (long long)p.n_gauss);
  print_list("stride", p.stride, p.m);
  print_list("blk_off", p.blk_off, p.m);
  print_list("grp_off", p.grp_off, p.m);
  print_list("theta_off", p.theta_off, p.m);
  print_list("gauss_off", p.gauss_off, p.m);
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc >= 3 && std::strcmp(argv[1], "print") == 0) return print_plan(argc, argv);
  std::mt19937_64 rng(20261203);
  auto uni = [&](int64_t lo, int64_t hi) { return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1)); };

  // make_plan: valid schedules are accepted with consistent offsets, anything
  // else is rejected with a message
  for (long long it = 0; it < 200000; ++it) {
    int32_t radix[24];
    int m;
    int64_t d;
    if (it % 2 == 0) {
      m = (int)uni(1, 8);
      d = 1;
      for (int t = 0; t < m; ++t) {
        radix[t] = (int32_t)uni(2, 16);
        d *= radix[t];
      }
      if (it % 4 == 2) d += uni(-3, 3);   // sometimes off by a little
    } else {
      m = (int)uni(-2, 20);
      for (int t = 0; t < 24; ++t) radix[t] = (int32_t)uni(-3, 40);
      d = uni(-5, 70000);
    }
    bool valid = m >= 1 && m <= harp::kMaxStages && d >= 2 && d <= harp::kMaxD;
    int64_t prod = 1;
    for (int t = 0; valid && t < m; ++t) {
      if (radix[t] < 2 || radix[t] > harp::kMaxRadix) valid = false;
      else if ((prod *= radix[t]) > harp::kMaxD) valid = false;
    }
    valid = valid && prod == d;
    Plan p;
    const std::string e = harp::make_plan(m, radix, d, &p);
    if (valid != e.empty()) return fail(valid ? "valid schedule rejected" : "invalid schedule accepted", it);
    if (!valid) continue;
    int64_t s = 1, nb = 0, ng = 0, nt = 0, nga = 0;
    for (int t = m - 1; t >= 0; --t) {
      if (p.stride[t] != s) return fail("stride", it);
      s *= radix[t];
    }
    for (int t = 0; t < m; ++t) {
      const int64_t b = radix[t];
      if (p.blk_off[t] != nb || p.grp_off[t] != ng || p.theta_off[t] != nt) return fail("offsets", it);
      nb += d * b;
      ng += d / b;
      nt += (d / b) * (b == 2 ? 1 : b * (b - 1) / 2);
      if (harp::is_pow2(b) != (p.gauss_off[t] < 0)) return fail("gauss stage", it);
      if (!harp::is_pow2(b)) {
        if (p.gauss_off[t] != nga) return fail("gauss offset", it);
        nga += b * b;
      }
    }
    if (p.n_blk != nb || p.n_grp != ng || p.n_theta != nt || p.n_gauss != nga) return fail("totals", it);
  }
  if (harp::make_plan(2, nullptr, 4, nullptr).empty()) return fail("NULL schedule accepted", -1);

  // check_rows: any sizes, pointers and alignments, including extreme ones,
  // give an answer without overflow; the documented cases give the
  // documented answer
  const int64_t big[] = {INT64_MIN, -1, 0, 1, 2, 3, 4096, (int64_t)1 << 31, (int64_t)1 << 40, INT64_MAX / 2,
                         INT64_MAX};
  const int nbig = (int)(sizeof big / sizeof big[0]);
  for (long long it = 0; it < 200000; ++it) {
    const int64_t d = it % 3 == 0 ? big[uni(0, nbig - 1)] : uni(2, 40000);
    const int64_t rows = it % 5 == 0 ? big[uni(0, nbig - 1)] : uni(-2, 1 << 20);
    auto near_d = [&]() { return d > INT64_MAX - 64 || d < INT64_MIN + 2 ? d : d + uni(-2, 64); };
    const int64_t ldx = it % 7 == 0 ? big[uni(0, nbig - 1)] : near_d();
    const int64_t ldy = it % 11 == 0 ? big[uni(0, nbig - 1)] : (it % 2 ? ldx : near_d());
    const int eb = it % 2 ? 2 : 4;
    const uintptr_t bx = (uintptr_t)uni(0, (int64_t)1 << 44) * 16 + (uintptr_t)uni(0, 3);
    const uintptr_t by = it % 3 == 0 ? bx : (it % 3 == 1 ? bx + (uintptr_t)uni(-4096, 4096) * 2 : (uintptr_t)uni(0, (int64_t)1 << 44) * 16);
    const void* x = it % 13 == 0 ? nullptr : reinterpret_cast<const void*>(bx);
    const void* y = it % 17 == 0 ? nullptr : reinterpret_cast<const void*>(by);
    const std::string e = harp::check_rows(x, ldx, y, ldy, rows, d, eb);
    if (rows < 0 && e.empty()) return fail("rows < 0 accepted", it);
    if (rows == 0 && !e.empty()) return fail("rows == 0 rejected", it);
    if (rows > 0 && (x == nullptr || y == nullptr) && e.empty()) return fail("NULL accepted", it);
    if (rows > 0 && e.empty() && (ldx < d || ldy < d)) return fail("short leading dimension accepted", it);
    if (rows > 0 && e.empty() && x == y && ldx != ldy) return fail("in-place with different ld accepted", it);
  }
  // overlap cases with small, exact numbers
  {
    alignas(16) static float buf[4096];
    if (!harp::check_rows(buf, 16, buf + 8, 16, 4, 16, 4).size()) return fail("partial overlap accepted", -2);
    if (harp::check_rows(buf, 16, buf + 64, 16, 4, 16, 4).size()) return fail("adjacent buffers rejected", -2);
    if (harp::check_rows(buf, 16, buf, 16, 4, 16, 4).size()) return fail("in-place rejected", -2);
  }
  std::printf("ok\n");
  return 0;
}
