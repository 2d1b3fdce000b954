// Device-rate probe for one MI355X (gfx950): the ceilings the kernels of this
// package are measured against.  Prints one line per measurement:
//   * matrix-core issue rates (clocks per instruction per wave, from the
//     shader clock, and FMA/s from HIP events) for the shapes the kernels use
//     or could use, with 1 to 8 independent accumulation chains per wave and
//     one or two waves per SIMD;
//   * LDS read bandwidth for 4-, 8- and 16-byte accesses;
//   * vector-memory read bandwidth from L1/L2-resident regions, for a
//     contiguous pattern and the per-quad pattern of the row kernels'
//     coefficient reads;
//   * HBM: a 1 GiB device copy and a 1 GiB read.
//
//   python -m structured_rotations_amd.build --probe && structured_rotations_amd/hwprobe
//
// Every index below is masked into its buffer; the probe writes only its own
// allocations.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

#define CK(x)                                                                  \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                            \
    }                                                                          \
  } while (0)

// OP: 0 = 4x4x1 f32 (16 blocks), 1 = 4x4x4 bf16 (16 blocks), 2 = 16x16x32 bf16,
// 3 = 32x32x16 bf16, 4 = 16x16x4 f32, 5 = 16x16x16 bf16.
template <int OP, int NC>
__global__ void mfma_k(float* out, long long* cyc, int iters, float seed) {
  const float a = seed + threadIdx.x * 1e-3f, b = seed - threadIdx.x * 1e-3f;
  const s4 sa = {(short)threadIdx.x, 2, 3, 4};
  bf8 ba;
  for (int i = 0; i < 8; ++i) ba[i] = (__bf16)(a + i);
  float res = 0.f;
  long long t0, t1;
  if constexpr (OP == 3) {
    f16v acc[NC];
    for (int c = 0; c < NC; ++c) acc[c] = f16v{} + (float)c;
    t0 = clock64();
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ba, ba, acc[c], 0, 0, 0);
    t1 = clock64();
    for (int c = 0; c < NC; ++c) res += acc[c][0] + acc[c][15];
  } else {
    f4 acc[NC];
    for (int c = 0; c < NC; ++c) acc[c] = f4{(float)c, 0.f, 0.f, 0.f};
    t0 = clock64();
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if constexpr (OP == 0) acc[c] = __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, acc[c], 0, 0, 0);
        if constexpr (OP == 1) acc[c] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(sa, sa, acc[c], 0, 0, 0);
        if constexpr (OP == 2) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ba, ba, acc[c], 0, 0, 0);
        if constexpr (OP == 4) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[c], 0, 0, 0);
        if constexpr (OP == 5) acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(sa, sa, acc[c], 0, 0, 0);
      }
    t1 = clock64();
    for (int c = 0; c < NC; ++c) res += acc[c][0] + acc[c][3];
  }
  const int gt = blockIdx.x * blockDim.x + threadIdx.x;
  out[gt] = res;
  if ((threadIdx.x & 63) == 0) cyc[gt >> 6] = t1 - t0;
}

// LDS reads of W bytes per lane from a 64 KiB buffer, lane-contiguous.
template <int W>
__global__ void lds_k(float* out, long long* cyc, int iters) {
  __shared__ uint32_t buf[16384];
  for (int i = threadIdx.x; i < 16384; i += blockDim.x) buf[i] = i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int WW = W / 4;
  constexpr int ROW = 64 * WW;
  uint32_t acc = 0;
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int base = ((it * 8 + u + wave * 3) * ROW) & (16384 - 1);   // a multiple of ROW
      const uint32_t* p = buf + base + lane * WW;
      if constexpr (W == 4) acc ^= p[0];
      if constexpr (W == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        acc ^= v.x ^ v.y;
      }
      if constexpr (W == 16) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      }
    }
  }
  const long long t1 = clock64();
  const int gt = blockIdx.x * blockDim.x + threadIdx.x;
  out[gt] = (float)acc;
  if (lane == 0) cyc[gt >> 6] = t1 - t0;
}

// 16-byte vector-memory reads from a region of `words` uint32 (a power of
// two).  PAT 0: each wave access is 1 KiB contiguous; PAT 1: lane (b, i) =
// (lane / 4, lane % 4) reads 16 bytes at 256 b + 32 i (+16 every other access),
// the row kernels' coefficient pattern.
template <int PAT>
__global__ void vmem_k(const uint32_t* __restrict__ src, float* out, long long* cyc, int iters, int words) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = lane >> 2, i = lane & 3;
  const int mask = words - 1;
  uint32_t acc = 0;
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int base = ((it * 8 + u) * 1024 + (blockIdx.x * 16 + wave) * 4096) & mask;   // multiple of 1024 words
      const int off = PAT == 0 ? lane * 4 : b * 64 + i * 8 + (u & 1) * 4;               // < 1024 words
      const uint4 v = *reinterpret_cast<const uint4*>(src + ((base + off) & mask));
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  const long long t1 = clock64();
  const int gt = blockIdx.x * blockDim.x + threadIdx.x;
  out[gt] = (float)acc;
  if (lane == 0) cyc[gt >> 6] = t1 - t0;
}

__global__ void copy_k(const u4v* __restrict__ a, u4v* __restrict__ b, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    __builtin_nontemporal_store(__builtin_nontemporal_load(a + i), b + i);
}

__global__ void read_k(const u4v* __restrict__ a, size_t n, float* out) {
  uint32_t acc = 0;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const u4v v = __builtin_nontemporal_load(a + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x12345678u) out[0] = 1.f;
}

struct Res {
  double cyc_med;   // median per-wave clocks (shader clock)
  double ms;        // HIP event time of the launch
};

template <class K, class... A>
Res timed(K kern, int grid, int block, long long* cyc, A... args) {
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(block), 0, 0, args...);   // warm-up
  CK(hipDeviceSynchronize());
  CK(hipEventRecord(e0));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(block), 0, 0, args...);
  CK(hipEventRecord(e1));
  CK(hipDeviceSynchronize());
  float ms;
  CK(hipEventElapsedTime(&ms, e0, e1));
  const int nw = grid * block / 64;
  std::vector<long long> h(nw);
  CK(hipMemcpy(h.data(), cyc, nw * sizeof(long long), hipMemcpyDeviceToHost));
  std::sort(h.begin(), h.end());
  CK(hipEventDestroy(e0));
  CK(hipEventDestroy(e1));
  return {(double)h[nw / 2], ms};
}

template <int OP, int NC>
void mfma_line(const char* name, double fma_per_instr, int wps, float* out, long long* cyc) {
  const int iters = 2000;
  const Res r = timed(mfma_k<OP, NC>, 256, 256 * wps, cyc, out, cyc, iters, 1.0f);
  const double fmas = 256.0 * 4 * wps * iters * NC * fma_per_instr;
  std::printf("mfma %-13s waves/SIMD %d chains %d: %6.2f clk/instr per wave, %7.1f TFMA/s (%7.1f TFLOP/s)\n", name,
              wps, NC, r.cyc_med / (iters * (double)NC), fmas / (r.ms * 1e-3) / 1e12,
              2 * fmas / (r.ms * 1e-3) / 1e12);
}

int main() {
  hipDeviceProp_t prop;
  CK(hipGetDeviceProperties(&prop, 0));
  std::printf("device %s, %d CUs, max clock %d kHz\n", prop.gcnArchName, prop.multiProcessorCount, prop.clockRate);
  float* out;
  long long* cyc;
  uint32_t* src;
  CK(hipMalloc(&out, 256 * 1024 * sizeof(float)));
  CK(hipMalloc(&cyc, 256 * 16 * sizeof(long long)));
  const int maxw = 1 << 24;   // 64 MiB region
  CK(hipMalloc(&src, (size_t)maxw * sizeof(uint32_t)));
  CK(hipMemset(src, 1, (size_t)maxw * sizeof(uint32_t)));
  for (int wps = 1; wps <= 2; ++wps) {
    mfma_line<0, 1>("4x4x1 f32", 256, wps, out, cyc);
    mfma_line<0, 2>("4x4x1 f32", 256, wps, out, cyc);
    mfma_line<0, 4>("4x4x1 f32", 256, wps, out, cyc);
    mfma_line<0, 8>("4x4x1 f32", 256, wps, out, cyc);
    mfma_line<1, 4>("4x4x4 bf16", 1024, wps, out, cyc);
    mfma_line<1, 8>("4x4x4 bf16", 1024, wps, out, cyc);
    mfma_line<4, 4>("16x16x4 f32", 1024, wps, out, cyc);
    mfma_line<5, 4>("16x16x16 bf16", 4096, wps, out, cyc);
    mfma_line<2, 4>("16x16x32 bf16", 8192, wps, out, cyc);
    mfma_line<3, 4>("32x32x16 bf16", 16384, wps, out, cyc);
  }
  const int iters = 400;
  for (int wpc = 4; wpc <= 16; wpc *= 2) {
    const Res r4 = timed(lds_k<4>, 256, 64 * wpc, cyc, out, cyc, iters);
    const Res r8 = timed(lds_k<8>, 256, 64 * wpc, cyc, out, cyc, iters);
    const Res r16 = timed(lds_k<16>, 256, 64 * wpc, cyc, out, cyc, iters);
    auto bpc = [&](const Res& r, double bytes) { return wpc * iters * 8 * bytes / r.cyc_med; };
    auto tbs = [&](const Res& r, double bytes) { return 256.0 * wpc * iters * 8 * bytes / (r.ms * 1e-3) / 1e12; };
    std::printf("lds %2d waves/CU: b32 %6.1f B/clk/CU (%5.1f TB/s), b64 %6.1f (%5.1f), b128 %6.1f (%5.1f)\n", wpc,
                bpc(r4, 256), tbs(r4, 256), bpc(r8, 512), tbs(r8, 512), bpc(r16, 1024), tbs(r16, 1024));
  }
  for (int wpc = 8; wpc <= 16; wpc *= 2)
    for (int s : {4096, 131072, 1 << 20, 1 << 24}) {
      const int vi = 200;
      const Res r0 = timed(vmem_k<0>, 256, 64 * wpc, cyc, (const uint32_t*)src, out, cyc, vi, s);
      const Res r1 = timed(vmem_k<1>, 256, 64 * wpc, cyc, (const uint32_t*)src, out, cyc, vi, s);
      std::printf("vmem b128 region %6d KiB %2d waves/CU: contiguous %5.1f B/clk/CU (%5.1f TB/s), "
                  "coefficient pattern %5.1f B/clk/CU (%5.1f TB/s)\n",
                  s / 256, wpc, wpc * vi * 8 * 1024.0 / r0.cyc_med,
                  256.0 * wpc * vi * 8 * 1024 / (r0.ms * 1e-3) / 1e12, wpc * vi * 8 * 1024.0 / r1.cyc_med,
                  256.0 * wpc * vi * 8 * 1024 / (r1.ms * 1e-3) / 1e12);
    }
  {
    const size_t n4 = (size_t)1 << 26;   // 16-byte elements: 1 GiB
    u4v *a, *b;
    CK(hipMalloc(&a, n4 * 16));
    CK(hipMalloc(&b, n4 * 16));
    CK(hipMemset(a, 1, n4 * 16));
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    for (int rep = 0; rep < 3; ++rep) hipLaunchKernelGGL(copy_k, dim3(256 * 16), dim3(256), 0, 0, a, b, n4);
    CK(hipDeviceSynchronize());
    CK(hipEventRecord(e0));
    for (int rep = 0; rep < 5; ++rep) hipLaunchKernelGGL(copy_k, dim3(256 * 16), dim3(256), 0, 0, a, b, n4);
    CK(hipEventRecord(e1));
    CK(hipDeviceSynchronize());
    float ms;
    CK(hipEventElapsedTime(&ms, e0, e1));
    std::printf("hbm copy 1 GiB -> 1 GiB: %.3f ms, %.2f TB/s (read + write)\n", ms / 5,
                2.0 * n4 * 16 / (ms / 5 * 1e-3) / 1e12);
    CK(hipEventRecord(e0));
    for (int rep = 0; rep < 5; ++rep) hipLaunchKernelGGL(read_k, dim3(256 * 16), dim3(256), 0, 0, a, n4, out);
    CK(hipEventRecord(e1));
    CK(hipDeviceSynchronize());
    CK(hipEventElapsedTime(&ms, e0, e1));
    std::printf("hbm read 1 GiB: %.3f ms, %.2f TB/s\n", ms / 5, 1.0 * n4 * 16 / (ms / 5 * 1e-3) / 1e12);
    CK(hipFree(a));
    CK(hipFree(b));
  }
  std::printf("done\n");
  return 0;
}
