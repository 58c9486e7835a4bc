// Non-temporal 16-byte loads and stores for the row-copy kernels (reorder,
// gather, scatter): every byte is read once and written once, and the
// tensors are far larger than the caches, so nothing is kept for reuse
// (720p: the fused reorder 0.92 -> 0.83 ms).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cabf {

typedef uint32_t stream_u32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint4 load_stream(const uint4* p) {
  const stream_u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const stream_u32x4*>(p));
  return make_uint4(q.x, q.y, q.z, q.w);
}

__device__ inline void store_stream(uint4* p, uint4 v) {
  const stream_u32x4 q = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(q, reinterpret_cast<stream_u32x4*>(p));
}

}  // namespace cabf
