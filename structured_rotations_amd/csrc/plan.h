// Host-side schedule planning and argument validation (plain C++, no HIP).
//
// A schedule b = (b_0..b_{m-1}) with prod b_t = d splits a row index into
// C-order digits; digit t has stride s_t = prod_{u>t} b_u and stage t mixes
// digit t (HARP technical summary, §2.1 Core Architecture: block-diagonal
// stages separated by stride permutations, mixed-radix schedules).
#pragma once

#include <cstdint>
#include <string>

namespace harp {

constexpr int kMaxStages = 16;
constexpr int kMaxRadix = 16;
constexpr int64_t kMaxD = 32768;

struct Plan {
  int m = 0;
  int64_t d = 0;
  int radix[kMaxStages] = {};
  int64_t stride[kMaxStages] = {};     // s_t
  int64_t blk_off[kMaxStages] = {};    // coefficient offset of stage t
  int64_t grp_off[kMaxStages] = {};    // group (scale) offset of stage t
  int64_t theta_off[kMaxStages] = {};  // parameter offset of stage t
  int64_t gauss_off[kMaxStages] = {};  // Gaussian offset (-1: power of two)
  int64_t n_blk = 0, n_grp = 0, n_theta = 0, n_gauss = 0;
  bool all_pow2 = true;
};

inline bool is_pow2(int64_t b) { return b >= 1 && (b & (b - 1)) == 0; }

// Fills *p; returns "" on success, else a description of the problem.
std::string make_plan(int m, const int32_t* radix, int64_t d, Plan* p);

// Row-batch arguments shared by the apply-type entry points.
std::string check_rows(const void* x, int64_t ldx, const void* y, int64_t ldy,
                       int64_t rows, int64_t d, int elem_bytes);

// Thread-local last error message.
void set_last_error(const std::string& msg);
const char* last_error();

}  // namespace harp
