// Measurement aid of the benchmark, built into its own library
// (libcabf_probe.so), not part of the attention path or of libcabf's ABI: a
// dense bf16 matrix-core loop that reports the rate the chip sustains under
// load (its clock under a full MFMA load sits below the one the published
// peak assumes).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Every wave runs `iters` rounds of 8 independent 32x32x16 bf16 products
// (eight accumulators, so the matrix pipe never waits on a result) and
// stores one value per lane so that nothing is optimised away.
__global__ __launch_bounds__(256, 2) void mfma_peak(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(1.0f / (1 + lane + i));
    b[i] = static_cast<__bf16>(1.0f / (2 + lane + i));
  }
  f32x16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// Launches `workgroups` workgroups of 256 threads, each wave running iters x
// 8 products of v_mfma_f32_32x32x16_bf16; out: device float[workgroups * 256]
// (4-byte aligned). Returns 0, -1 for a bad argument (before any launch), -4
// if the launch failed.
extern "C" __attribute__((visibility("default"))) int probe_mfma_peak(int32_t workgroups,
                                                                       int32_t iters, float* out,
                                                                       hipStream_t stream) {
  if (workgroups < 1 || iters < 1 || out == nullptr || reinterpret_cast<uintptr_t>(out) % 4)
    return -1;
  hipLaunchKernelGGL(mfma_peak, dim3(static_cast<unsigned>(workgroups)), dim3(256), 0, stream,
                     iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
