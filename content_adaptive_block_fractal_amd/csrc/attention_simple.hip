// Block-sparse attention forward, plain VALU form (NABLA summary,
// Methodology item 2, expansion bullet: attention is computed on the kept
// block tiles only).
//
// One wave per query block, one lane per query row. Each kept key block is
// staged through LDS as fp32 and consumed 16 keys at a time with an fp32
// online softmax in base 2. This is the float32 path and the device-side
// cross-check of the matrix-core kernel; it is not the fast bf16 path.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attention_common.hpp"
#include "geometry.hpp"
#include "launch.hpp"

namespace cabf {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(64) void bsa_fwd_simple(AttnArgs a) {
  __shared__ float Ks[kBlock][D];
  __shared__ float Vs[kBlock][D];
  const int lane = threadIdx.x;
  const int64_t qblk = blockIdx.x;                 // over batch*heads*nb
  const int64_t bh = qblk / a.nb;
  const T* __restrict__ qp = static_cast<const T*>(a.qp);
  const T* __restrict__ kp = static_cast<const T*>(a.kp) + bh * a.N * D;
  const T* __restrict__ vp = static_cast<const T*>(a.vp) + bh * a.N * D;
  const int64_t qrow = qblk * kBlock + lane;
  float q[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = load_elem(qp + qrow * D + c) * a.scale_log2;
    acc[c] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  const int cnt = min(max(a.kv_count[qblk], 0), a.nb);
  const int32_t* __restrict__ list = a.kv_index + qblk * a.nb;
  for (int e = 0; e < cnt; ++e) {
    const int jb = list[e];
    if (static_cast<unsigned>(jb) >= static_cast<unsigned>(a.nb)) continue;   // not a block
    __syncthreads();
    const T* krow = kp + (static_cast<int64_t>(jb) * kBlock + lane) * D;
    const T* vrow = vp + (static_cast<int64_t>(jb) * kBlock + lane) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      Ks[lane][c] = load_elem(krow + c);
      Vs[lane][c] = load_elem(vrow + c);
    }
    __syncthreads();
    const BlockExtent ext = block_extent(jb, a);
    for (int k0 = 0; k0 < kBlock; k0 += 16) {
      float s[16];
      float mt = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const int k = k0 + kk;
        float dot = 0.0f;
#pragma unroll
        for (int c = 0; c < D; ++c) dot = fmaf(q[c], Ks[k][c], dot);
        s[kk] = ext.real(k) ? dot : -INFINITY;
        mt = fmaxf(mt, s[kk]);
      }
      const float mn = fmaxf(m, mt);
      if (mn == -INFINITY) continue;               // no real key yet
      const float alpha = exp2f(m - mn);           // m = -inf gives 0
      l *= alpha;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] *= alpha;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const float pk = exp2f(s[kk] - mn);
        l += pk;
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] = fmaf(pk, Vs[k0 + kk][c], acc[c]);
      }
      m = mn;
    }
  }
  T* __restrict__ op = static_cast<T*>(a.op);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
  for (int c = 0; c < D; ++c) store_elem(op + qrow * D + c, acc[c] * inv);
  if (a.lse != nullptr) a.lse[qrow] = l > 0.0f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

}  // namespace

void launch_bsa_forward_simple(const AttnArgs& a, bool bf16, int D, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(a.BH * a.nb);
  if (bf16) {
    if (D == 64)
      hipLaunchKernelGGL((bsa_fwd_simple<uint16_t, 64>), dim3(grid), dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((bsa_fwd_simple<uint16_t, 128>), dim3(grid), dim3(64), 0, stream, a);
  } else {
    if (D == 64)
      hipLaunchKernelGGL((bsa_fwd_simple<float, 64>), dim3(grid), dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((bsa_fwd_simple<float, 128>), dim3(grid), dim3(64), 0, stream, a);
  }
}

}  // namespace cabf
