// Measured ceilings for the benchmark (not steps of the method): a streaming
// copy (HBM) and a loop of fp16 MFMAs (matrix cores).  The entry points are in
// abi.hip and declared in include/retention_calib.h.
#include "internal.h"

namespace ret {

namespace {

constexpr int CP_THREADS = 256, CP_INFLIGHT = 8;

// 16-byte words: each thread moves CP_INFLIGHT words per round, the words of
// one round 256 threads apart (coalesced), all loads issued before the stores
__global__ void __launch_bounds__(CP_THREADS) copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          size_t n) {
  const size_t stride = (size_t)gridDim.x * CP_THREADS * CP_INFLIGHT;
  for (size_t base = (size_t)blockIdx.x * CP_THREADS * CP_INFLIGHT + threadIdx.x; base < n; base += stride) {
    u32x4 v[CP_INFLIGHT];
#pragma unroll
    for (int i = 0; i < CP_INFLIGHT; ++i) {
      const size_t j = base + (size_t)i * CP_THREADS;
      if (j < n) v[i] = __builtin_nontemporal_load(src + j);
    }
#pragma unroll
    for (int i = 0; i < CP_INFLIGHT; ++i) {
      const size_t j = base + (size_t)i * CP_THREADS;
      if (j < n) __builtin_nontemporal_store(v[i], dst + j);
    }
  }
}

// four independent accumulator chains per wave, operands in registers
__global__ void __launch_bounds__(256) mfma_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (half)(0.001f * (float)(lane + e));
    b[e] = (half)(0.002f * (float)(63 - lane + e));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_calib_copy(const void* src, void* dst, size_t n16, hipStream_t st) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const size_t per_block = (size_t)CP_THREADS * CP_INFLIGHT;
  const size_t want = (n16 + per_block - 1) / per_block;
  const int grid = (int)(want < (size_t)cus * 8 ? want : (size_t)cus * 8);
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(CP_THREADS), 0, st, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_calib_mfma(float* out, int blocks, int iters, hipStream_t st) {
  hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(256), 0, st, out, iters);
  return hipGetLastError();
}

}  // namespace ret
