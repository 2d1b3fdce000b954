// Block materialisation  B_{t,c} = Q_{t,c}(theta) G_{b_t},  in fp64 on device.
//
// HARP technical summary (gist.science 2605.29843), §2.2: every learnable
// block is a learnable orthogonal factor Q (a Givens rotation for radix 2, a
// Cayley map for larger radices) times a fixed base mixer G (the normalised
// Sylvester Hadamard for power-of-two radices, otherwise the Q factor of the
// QR factorisation of a fixed Gaussian matrix, §2.1).  With all parameters
// zero, Q = I and the block is G.  §2.4: parameters may be stored in int8;
// the same idea is offered here for the blocks (one fp32 scale per block),
// and the parameters themselves may come in as int8 codes with one fp32 scale
// per stage: theta = code * scale, formed exactly in fp64 before the same
// solve.  quantize_theta_kernel produces that format from fp64 theta.
//
// One launch per stage.  Thread 0 of each workgroup builds G in LDS
// (Householder QR with the column signs fixed so that diag R > 0); every
// thread then forms one group's Q (Cayley: Gaussian elimination on
// (I + A) Q = (I - A); no pivoting is needed because I + A has the identity
// as its symmetric part), multiplies by G and rounds to the storage format.
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace harp {

struct MatParams {
  int64_t ngroups;
  const double* theta;   // the stage's parameters (fp64), or NULL when tcode is given
  const int8_t* tcode;   // the stage's int8 parameter codes, or NULL
  const float* tscale;   // the stage's fp32 scale (with tcode)
  const double* gauss;   // the stage's b x b Gaussian matrix, or NULL
  int out_dt;            // 0 F32, 1 BF16, 2 I8
  void* out;             // the stage's blocks
  float* scales;         // the stage's int8 scales
};

template <int B>
__device__ void base_mixer(const double* gauss, double* g) {
  if (gauss == nullptr) {
    const double inv = 1.0 / sqrt((double)B);
    for (int r = 0; r < B; ++r)
      for (int k = 0; k < B; ++k) g[r * B + k] = (__popc(r & k) & 1) ? -inv : inv;
    return;
  }
  double a[B][B], q[B][B];
  for (int r = 0; r < B; ++r)
    for (int k = 0; k < B; ++k) {
      a[r][k] = gauss[r * B + k];
      q[r][k] = (r == k) ? 1.0 : 0.0;
    }
  // Householder: a <- H_{B-2} ... H_0 a = R,  q <- q H_0 ... H_{B-2} = Q.
  for (int k = 0; k < B - 1; ++k) {
    double nrm = 0.0;
    for (int i = k; i < B; ++i) nrm += a[i][k] * a[i][k];
    nrm = sqrt(nrm);
    if (nrm == 0.0) continue;
    const double alpha = a[k][k] > 0 ? -nrm : nrm;
    double v[B];
    for (int i = 0; i < B; ++i) v[i] = (i < k) ? 0.0 : a[i][k];
    v[k] -= alpha;
    double vn = 0.0;
    for (int i = k; i < B; ++i) vn += v[i] * v[i];
    if (vn == 0.0) continue;
    for (int j = 0; j < B; ++j) {
      double dot = 0.0;
      for (int i = k; i < B; ++i) dot += v[i] * a[i][j];
      const double f = 2.0 * dot / vn;
      for (int i = k; i < B; ++i) a[i][j] -= f * v[i];
    }
    for (int r = 0; r < B; ++r) {
      double dot = 0.0;
      for (int i = k; i < B; ++i) dot += q[r][i] * v[i];
      const double f = 2.0 * dot / vn;
      for (int i = k; i < B; ++i) q[r][i] -= f * v[i];
    }
  }
  for (int k = 0; k < B; ++k) {
    const double sg = a[k][k] < 0 ? -1.0 : 1.0;
    for (int r = 0; r < B; ++r) g[r * B + k] = q[r][k] * sg;
  }
}

// Parameter i of group c (per parameters per group), dequantised if int8.
__device__ inline double param(const MatParams& p, int64_t c, int per, int i) {
  if (p.tcode != nullptr) return (double)p.tcode[c * per + i] * (double)p.tscale[0];
  return p.theta[c * per + i];
}

template <int B>
__global__ void __launch_bounds__(256) materialize_kernel(MatParams p) {
  __shared__ double g[B * B];
  if (threadIdx.x == 0) base_mixer<B>(p.gauss, g);
  __syncthreads();
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= p.ngroups) return;
  double q[B][B];
  if (B == 2) {
    const double th = param(p, c, 1, 0);
    const double cs = cos(th), sn = sin(th);
    q[0][0] = cs; q[0][1] = -sn;
    q[1][0] = sn; q[1][1] = cs;
  } else {
    constexpr int per = B * (B - 1) / 2;
    double mtx[B][B];
    for (int r = 0; r < B; ++r)
      for (int k = 0; k < B; ++k) { mtx[r][k] = (r == k) ? 1.0 : 0.0; q[r][k] = mtx[r][k]; }
    int idx = 0;
    for (int r = 0; r < B; ++r)
      for (int k = r + 1; k < B; ++k) {
        const double a = param(p, c, per, idx++);
        mtx[r][k] += a; mtx[k][r] -= a;   // I + A
        q[r][k] -= a;   q[k][r] += a;     // I - A
      }
    for (int k = 0; k < B; ++k) {
      const double inv = 1.0 / mtx[k][k];
      for (int i = k + 1; i < B; ++i) {
        const double f = mtx[i][k] * inv;
        if (f == 0.0) continue;
        for (int j = k; j < B; ++j) mtx[i][j] -= f * mtx[k][j];
        for (int j = 0; j < B; ++j) q[i][j] -= f * q[k][j];
      }
    }
    for (int k = B - 1; k >= 0; --k) {
      for (int j = 0; j < B; ++j) {
        double acc = q[k][j];
        for (int i = k + 1; i < B; ++i) acc -= mtx[k][i] * q[i][j];
        q[k][j] = acc / mtx[k][k];
      }
    }
  }
  double blk[B][B];
  double amax = 0.0;
  for (int r = 0; r < B; ++r)
    for (int k = 0; k < B; ++k) {
      double acc = 0.0;
      for (int i = 0; i < B; ++i) acc += q[r][i] * g[i * B + k];
      blk[r][k] = acc;
      amax = fmax(amax, fabs(acc));
    }
  const int64_t o = c * B * B;
  if (p.out_dt == 0) {
    float* out = static_cast<float*>(p.out) + o;
    for (int r = 0; r < B; ++r)
      for (int k = 0; k < B; ++k) out[r * B + k] = (float)blk[r][k];
  } else if (p.out_dt == 1) {
    uint16_t* out = static_cast<uint16_t*>(p.out) + o;
    for (int r = 0; r < B; ++r)
      for (int k = 0; k < B; ++k) out[r * B + k] = f64_to_bf16_rne(blk[r][k]);
  } else {
    int8_t* out = static_cast<int8_t*>(p.out) + o;
    const float sc = (float)(amax / 127.0);
    p.scales[c] = sc;
    for (int r = 0; r < B; ++r)
      for (int k = 0; k < B; ++k) {
        double code = 0.0;
        if (sc > 0.0f) code = fmin(127.0, fmax(-127.0, rint(blk[r][k] / (double)sc)));
        out[r * B + k] = (int8_t)code;
      }
  }
}

// Parameter gradient from block gradients, one thread per group, fp64:
// dL/dQ = dL/dB G^T; Givens: dQ/dtheta = [[-sin, -cos], [cos, -sin]];
// Cayley Q = (I - A) M with M = (I + A)^-1: dL/dA = -(I + Q)^T (dL/dQ) M^T and
// dL/dtheta_(r,k) = dL/dA[r][k] - dL/dA[k][r] (A = U - U^T, U row-major from
// the parameters).  M comes from the same elimination as the forward map,
// with the identity as right-hand side.
template <int B>
__global__ void __launch_bounds__(256) theta_vjp_kernel(int64_t ngroups, const double* theta, const double* gauss,
                                                        const float* dblocks, double* dtheta) {
  __shared__ double g[B * B];
  if (threadIdx.x == 0) base_mixer<B>(gauss, g);
  __syncthreads();
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= ngroups) return;
  const float* db = dblocks + c * B * B;
  double gq[B][B];
  for (int r = 0; r < B; ++r)
    for (int k = 0; k < B; ++k) {
      double acc = 0.0;
      for (int i = 0; i < B; ++i) acc += (double)db[r * B + i] * g[k * B + i];
      gq[r][k] = acc;
    }
  if (B == 2) {
    const double th = theta[c];
    const double cs = cos(th), sn = sin(th);
    dtheta[c] = -sn * gq[0][0] - cs * gq[0][1] + cs * gq[1][0] - sn * gq[1][1];
    return;
  }
  constexpr int per = B * (B - 1) / 2;
  const double* th = theta + c * per;
  double a[B][B], mtx[B][B], minv[B][B];
  for (int r = 0; r < B; ++r)
    for (int k = 0; k < B; ++k) {
      a[r][k] = 0.0;
      minv[r][k] = (r == k) ? 1.0 : 0.0;
    }
  int idx = 0;
  for (int r = 0; r < B; ++r)
    for (int k = r + 1; k < B; ++k) {
      a[r][k] = th[idx];
      a[k][r] = -th[idx];
      ++idx;
    }
  for (int r = 0; r < B; ++r)
    for (int k = 0; k < B; ++k) mtx[r][k] = (r == k ? 1.0 : 0.0) + a[r][k];
  for (int k = 0; k < B; ++k) {
    const double inv = 1.0 / mtx[k][k];
    for (int i = k + 1; i < B; ++i) {
      const double f = mtx[i][k] * inv;
      if (f == 0.0) continue;
      for (int j = k; j < B; ++j) mtx[i][j] -= f * mtx[k][j];
      for (int j = 0; j < B; ++j) minv[i][j] -= f * minv[k][j];
    }
  }
  for (int k = B - 1; k >= 0; --k)
    for (int j = 0; j < B; ++j) {
      double acc = minv[k][j];
      for (int i = k + 1; i < B; ++i) acc -= mtx[k][i] * minv[i][j];
      minv[k][j] = acc / mtx[k][k];
    }
  // P = (I + Q) = I + (I - A) M, reusing mtx
  for (int r = 0; r < B; ++r)
    for (int k = 0; k < B; ++k) {
      double acc = (r == k) ? 1.0 : 0.0;
      for (int i = 0; i < B; ++i) acc += ((r == i ? 1.0 : 0.0) - a[r][i]) * minv[i][k];
      mtx[r][k] = acc;
    }
  // T = gq M^T, reusing a
  for (int r = 0; r < B; ++r)
    for (int k = 0; k < B; ++k) {
      double acc = 0.0;
      for (int i = 0; i < B; ++i) acc += gq[r][i] * minv[k][i];
      a[r][k] = acc;
    }
  // dA = -P^T T, reusing gq
  for (int r = 0; r < B; ++r)
    for (int k = 0; k < B; ++k) {
      double acc = 0.0;
      for (int i = 0; i < B; ++i) acc += mtx[i][r] * a[i][k];
      gq[r][k] = -acc;
    }
  double* out = dtheta + c * per;
  idx = 0;
  for (int r = 0; r < B; ++r)
    for (int k = r + 1; k < B; ++k) out[idx++] = gq[r][k] - gq[k][r];
}

// One workgroup per stage: scale = fp32(max|theta of the stage| / 127), code =
// clamp(rint(theta / scale), -127, 127) decided in fp64; a zero stage -> 0, 0.
constexpr int kQThreads = 1024;
__global__ void __launch_bounds__(kQThreads) quantize_theta_kernel(int64_t n, const double* theta, int8_t* codes,
                                                                   float* scale_out) {
  __shared__ double red[kQThreads / 64];
  double amax = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += kQThreads) amax = fmax(amax, fabs(theta[i]));
  for (int off = 32; off > 0; off >>= 1) amax = fmax(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = red[0];
  for (int w = 1; w < kQThreads / 64; ++w) amax = fmax(amax, red[w]);
  const float sc = (float)(amax / 127.0);
  if (threadIdx.x == 0) scale_out[0] = sc;
  for (int64_t i = threadIdx.x; i < n; i += kQThreads) {
    double code = 0.0;
    if (sc > 0.0f) code = fmin(127.0, fmax(-127.0, rint(theta[i] / (double)sc)));
    codes[i] = (int8_t)code;
  }
}

namespace {
template <int B>
hipError_t launch_mat(const MatParams& p, hipStream_t st) {
  const int threads = 256;
  const int64_t grid = (p.ngroups + threads - 1) / threads;
  hipLaunchKernelGGL(materialize_kernel<B>, dim3((unsigned)grid), dim3(threads), 0, st, p);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_materialize(const Plan& pl, const double* theta, const int8_t* tcode,
                              const float* tscale, const double* gauss, DT bdt, void* blocks,
                              float* scales, hipStream_t stream) {
  const int esz = bdt == DT::F32 ? 4 : (bdt == DT::BF16 ? 2 : 1);
  for (int t = 0; t < pl.m; ++t) {
    MatParams p{};
    p.ngroups = pl.d / pl.radix[t];
    p.theta = theta ? theta + pl.theta_off[t] : nullptr;
    p.tcode = tcode ? tcode + pl.theta_off[t] : nullptr;
    p.tscale = tscale ? tscale + t : nullptr;
    p.gauss = pl.gauss_off[t] >= 0 ? gauss + pl.gauss_off[t] : nullptr;
    p.out_dt = (int)bdt;
    p.out = static_cast<char*>(blocks) + pl.blk_off[t] * esz;
    p.scales = scales ? scales + pl.grp_off[t] : nullptr;
    hipError_t e = hipSuccess;
    switch (pl.radix[t]) {
      case 2: e = launch_mat<2>(p, stream); break;
      case 3: e = launch_mat<3>(p, stream); break;
      case 4: e = launch_mat<4>(p, stream); break;
      case 5: e = launch_mat<5>(p, stream); break;
      case 6: e = launch_mat<6>(p, stream); break;
      case 7: e = launch_mat<7>(p, stream); break;
      case 8: e = launch_mat<8>(p, stream); break;
      case 9: e = launch_mat<9>(p, stream); break;
      case 10: e = launch_mat<10>(p, stream); break;
      case 11: e = launch_mat<11>(p, stream); break;
      case 12: e = launch_mat<12>(p, stream); break;
      case 13: e = launch_mat<13>(p, stream); break;
      case 14: e = launch_mat<14>(p, stream); break;
      case 15: e = launch_mat<15>(p, stream); break;
      case 16: e = launch_mat<16>(p, stream); break;
      default: e = hipErrorInvalidValue; break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

namespace {
template <int B>
hipError_t launch_tvjp(int64_t ng, const double* theta, const double* gauss, const float* db, double* dt,
                       hipStream_t st) {
  const int threads = 256;
  const int64_t grid = (ng + threads - 1) / threads;
  hipLaunchKernelGGL(theta_vjp_kernel<B>, dim3((unsigned)grid), dim3(threads), 0, st, ng, theta, gauss, db, dt);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_theta_vjp(const Plan& pl, const double* theta, const double* gauss, const float* dblocks,
                            double* dtheta, hipStream_t stream) {
  for (int t = 0; t < pl.m; ++t) {
    const int64_t ng = pl.d / pl.radix[t];
    const double* th = theta + pl.theta_off[t];
    const double* gs = pl.gauss_off[t] >= 0 ? gauss + pl.gauss_off[t] : nullptr;
    const float* db = dblocks + pl.blk_off[t];
    double* dt = dtheta + pl.theta_off[t];
    hipError_t e = hipSuccess;
    switch (pl.radix[t]) {
      case 2: e = launch_tvjp<2>(ng, th, gs, db, dt, stream); break;
      case 3: e = launch_tvjp<3>(ng, th, gs, db, dt, stream); break;
      case 4: e = launch_tvjp<4>(ng, th, gs, db, dt, stream); break;
      case 5: e = launch_tvjp<5>(ng, th, gs, db, dt, stream); break;
      case 6: e = launch_tvjp<6>(ng, th, gs, db, dt, stream); break;
      case 7: e = launch_tvjp<7>(ng, th, gs, db, dt, stream); break;
      case 8: e = launch_tvjp<8>(ng, th, gs, db, dt, stream); break;
      case 9: e = launch_tvjp<9>(ng, th, gs, db, dt, stream); break;
      case 10: e = launch_tvjp<10>(ng, th, gs, db, dt, stream); break;
      case 11: e = launch_tvjp<11>(ng, th, gs, db, dt, stream); break;
      case 12: e = launch_tvjp<12>(ng, th, gs, db, dt, stream); break;
      case 13: e = launch_tvjp<13>(ng, th, gs, db, dt, stream); break;
      case 14: e = launch_tvjp<14>(ng, th, gs, db, dt, stream); break;
      case 15: e = launch_tvjp<15>(ng, th, gs, db, dt, stream); break;
      case 16: e = launch_tvjp<16>(ng, th, gs, db, dt, stream); break;
      default: e = hipErrorInvalidValue; break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_quantize_theta(const Plan& pl, const double* theta, int8_t* codes, float* scales,
                                 hipStream_t stream) {
  for (int t = 0; t < pl.m; ++t) {
    const int b = pl.radix[t];
    const int64_t n = (pl.d / b) * (b == 2 ? 1 : b * (b - 1) / 2);
    hipLaunchKernelGGL(quantize_theta_kernel, dim3(1), dim3(kQThreads), 0, stream, n, theta + pl.theta_off[t],
                       codes + pl.theta_off[t], scales + t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace harp
