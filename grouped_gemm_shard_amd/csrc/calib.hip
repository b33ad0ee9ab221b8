// Calibration kernels: a streaming copy (the HBM bandwidth this GPU
// reaches) and a matrix-core loop (its bf16 MFMA throughput).  They are the
// measured ceilings the benchmark reports the layer's kernels against,
// beside the vendor's peak figures; they are not part of the layer.
#include <hip/hip_runtime.h>

#include "common.h"
#include "moe_calib.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// Nontemporal 16-byte accesses: the copy streams through the caches
// without displacing them (measured on MI355X: 5.2 TB/s for 1 GiB against
// 4.5 TB/s with ordinary accesses).
__global__ __launch_bounds__(256) void calib_copy_kernel(const v4i* __restrict__ src,
                                                         v4i* __restrict__ dst, long long n) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long stride = (long long)gridDim.x * blockDim.x;
  // four 16-byte loads in flight per lane, then their stores
  for (; i + 3 * stride < n; i += 4 * stride) {
    const v4i a = __builtin_nontemporal_load(src + i);
    const v4i b = __builtin_nontemporal_load(src + i + stride);
    const v4i c = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4i d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

constexpr int kCalibChains = 8;

__global__ __launch_bounds__(512) void calib_mfma_kernel(int iters, float* sink) {
  moe::floatx4 acc[kCalibChains];
#pragma unroll
  for (int c = 0; c < kCalibChains; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[c][q] = 0.0f;
  moe::bf16x8 a, b;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    a[q] = (__bf16)(0.001f * (float)(threadIdx.x & 7));
    b[q] = (__bf16)0.5f;
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kCalibChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kCalibChains; ++c) s += acc[c][0];
  if (blockIdx.x == 0) sink[threadIdx.x] = s;
}

}  // namespace

extern "C" {

int moe_calib_copy(const void* src, void* dst, int64_t bytes, int32_t blocks, void* stream) {
  if (src == nullptr || dst == nullptr || bytes <= 0 || bytes % 16 != 0 || blocks < 1)
    return MOE_EINVAL;
  if (((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return MOE_EINVAL;
  const char* s = (const char*)src;
  const char* d = (const char*)dst;
  if (s < d + bytes && d < s + bytes) return MOE_EINVAL;  // overlapping
  hipLaunchKernelGGL(calib_copy_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const v4i*)src, (v4i*)dst, (long long)(bytes / 16));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_calib_mfma(int32_t blocks, int32_t iters, float* sink, int64_t* flops, void* stream) {
  if (blocks < 1 || iters < 1 || sink == nullptr || flops == nullptr) return MOE_EINVAL;
  hipLaunchKernelGGL(calib_mfma_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters,
                     sink);
  *flops = (int64_t)blocks * 8 * iters * kCalibChains * (2LL * 16 * 16 * 32);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // extern "C"
