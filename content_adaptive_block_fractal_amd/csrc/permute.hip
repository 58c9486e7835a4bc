// Fractal flattening and its inverse (NABLA summary, Methodology item 1;
// the inverse restores raster order as in the Sparse VideoGen2 summary,
// section 2A).
//
// Both directions are bitwise row copies, so they move 16-byte chunks and
// never look at the element type. One workgroup handles one 64-token block
// (one 8x8 patch of one frame): the reordered side is a contiguous 64-row run
// and the raster side is 8 runs of 8 consecutive tokens, so every wave reads
// and writes whole rows. Block coordinates are decoded once per workgroup in
// scalar registers. Loads and stores are non-temporal (nothing is reused).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "geometry.hpp"
#include "launch.hpp"
#include "streaming.hpp"

namespace cabf {
namespace {

constexpr int kThreads = 256;

struct CopySet {
  const uint4* src[3];
  uint4* dst[3];
};

struct BlockPos {
  int t, ty, tx;
};

__device__ inline BlockPos decode_block(int b, int Ty, int Tx) {
  const int per_frame = Ty * Tx;
  BlockPos p;
  p.t = b / per_frame;
  const int rem = b - p.t * per_frame;
  p.ty = rem / Tx;
  p.tx = rem - p.ty * Tx;
  return p;
}

// CH = 16-byte chunks per token row (head_dim * element bytes / 16).
// FORWARD: raster -> reordered (pad rows written as zeros).
// !FORWARD: reordered -> raster (pad rows skipped).
template <int CH, bool FORWARD>
__global__ __launch_bounds__(kThreads) void reorder_blocks(CopySet set, int64_t blocks_total,
                                                           int nb, int Ty, int Tx, int H, int W,
                                                           int64_t Nv) {
  const uint4* __restrict__ src = set.src[blockIdx.y];
  uint4* __restrict__ dst = set.dst[blockIdx.y];
  if (src == nullptr) return;
  constexpr int kChunks = kBlock * CH;
  constexpr int kIters = kChunks / kThreads;
  static_assert(kChunks % kThreads == 0, "block size must tile the workgroup");
  for (int64_t blk = blockIdx.x; blk < blocks_total; blk += gridDim.x) {
    const int64_t bh = blk / nb;
    const int b = static_cast<int>(blk - bh * nb);
    const BlockPos bp = decode_block(b, Ty, Tx);
    const int64_t raster_base = bh * Nv;
    const int64_t fractal_base = blk * kBlock;
    // raster row of reordered row `row` of this block, or -1 for a pad slot
    auto raster_of = [&](int row) -> int64_t {
      const int y = bp.ty * kP + (row >> 3);
      const int x = bp.tx * kP + (row & 7);
      if (y >= H || x >= W) return -1;
      return raster_base + (static_cast<int64_t>(bp.t) * H + y) * W + x;
    };
    if (FORWARD) {
      uint4 vals[kIters];
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int c = it * kThreads + static_cast<int>(threadIdx.x);
        const int row = c / CH;
        const int64_t r = raster_of(row);
        vals[it] = r >= 0 ? load_stream(src + r * CH + (c - row * CH)) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int c = it * kThreads + static_cast<int>(threadIdx.x);
        store_stream(dst + fractal_base * CH + c, vals[it]);
      }
    } else {
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int c = it * kThreads + static_cast<int>(threadIdx.x);
        const int row = c / CH;
        const int64_t r = raster_of(row);
        const uint4 val = load_stream(src + fractal_base * CH + c);
        if (r >= 0) store_stream(dst + r * CH + (c - row * CH), val);
      }
    }
  }
}

// Fractal flattening fused with the block pooling of the adaptive mask
// (NABLA summary, Methodology items 1 and 2, down-sampling bullet): while a
// block's rows are in registers, the fp32 mean of its real tokens is formed
// for the tensors that have a pooled output (Q and K). Each thread always
// holds the same 16-byte column chunk of rows group, group + G, ... (G
// threads share a chunk); the G partial sums are added through LDS in group
// order, so the means are deterministic. Pad rows are zero and add nothing.
struct PoolSet {
  float* dst[3];   // [B*h, nb, D] fp32 means, or null
};

template <int EB, int D>
__global__ __launch_bounds__(kThreads) void reorder_pool_blocks(CopySet set, PoolSet pool,
                                                                int64_t blocks_total, int nb,
                                                                int Ty, int Tx, int H, int W,
                                                                int64_t Nv) {
  constexpr int CH = D * EB / 16;            // 16-byte chunks per row
  constexpr int kEPC = 16 / EB;              // elements per chunk
  constexpr int kIters = kBlock * CH / kThreads;
  constexpr int kGroups = kThreads / CH;     // threads sharing one column chunk
  static_assert(kBlock * CH % kThreads == 0 && kThreads % CH == 0, "tiling");
  __shared__ float red[kGroups][D];
  const uint4* __restrict__ src = set.src[blockIdx.y];
  uint4* __restrict__ dst = set.dst[blockIdx.y];
  float* __restrict__ pdst = pool.dst[blockIdx.y];
  if (src == nullptr) return;
  const int tid = static_cast<int>(threadIdx.x);
  const int col = tid % CH, group = tid / CH;
  for (int64_t blk = blockIdx.x; blk < blocks_total; blk += gridDim.x) {
    const int64_t bh = blk / nb;
    const int b = static_cast<int>(blk - bh * nb);
    const BlockPos bp = decode_block(b, Ty, Tx);
    const int64_t raster_base = bh * Nv;
    const int64_t fractal_base = blk * kBlock;
    uint4 vals[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int row = group + it * kGroups;
      const int y = bp.ty * kP + (row >> 3);
      const int x = bp.tx * kP + (row & 7);
      const bool real = y < H && x < W;
      const int64_t r = raster_base + (static_cast<int64_t>(bp.t) * H + y) * W + x;
      vals[it] = real ? load_stream(src + r * CH + col) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int it = 0; it < kIters; ++it) store_stream(dst + fractal_base * CH + it * kThreads + tid, vals[it]);
    if (pdst != nullptr) {
      float acc[kEPC];
#pragma unroll
      for (int e = 0; e < kEPC; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const uint32_t w[4] = {vals[it].x, vals[it].y, vals[it].z, vals[it].w};
        if constexpr (EB == 2) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[e] += __uint_as_float((w[e >> 1] >> ((e & 1) * 16)) << 16);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(w[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < kEPC; ++e) red[group][col * kEPC + e] = acc[e];
      __syncthreads();
      if (tid < D) {
        float s = 0.0f;
#pragma unroll
        for (int gq = 0; gq < kGroups; ++gq) s += red[gq][tid];
        const int vy = min(kP, H - bp.ty * kP), vx = min(kP, W - bp.tx * kP);
        pdst[blk * D + tid] = s / static_cast<float>(vy * vx);
      }
      __syncthreads();              // red is reused by the next block
    }
  }
}

template <bool FORWARD>
void launch_reorder(const Geo& g, int elem_bytes, const CopySet& set, int tensors,
                    hipStream_t stream) {
  const int64_t blocks_total = g.BH * g.nb;
  const int64_t max_grid = int64_t{1} << 20;
  const dim3 grid(static_cast<unsigned>(blocks_total < max_grid ? blocks_total : max_grid),
                  static_cast<unsigned>(tensors));
  const int ch = g.D * elem_bytes / 16;
  switch (ch) {
    case 8:
      hipLaunchKernelGGL((reorder_blocks<8, FORWARD>), grid, dim3(kThreads), 0, stream, set,
                         blocks_total, g.nb, g.Ty, g.Tx, g.H, g.W, g.Nv);
      break;
    case 16:
      hipLaunchKernelGGL((reorder_blocks<16, FORWARD>), grid, dim3(kThreads), 0, stream, set,
                         blocks_total, g.nb, g.Ty, g.Tx, g.H, g.W, g.Nv);
      break;
    case 32:
      hipLaunchKernelGGL((reorder_blocks<32, FORWARD>), grid, dim3(kThreads), 0, stream, set,
                         blocks_total, g.nb, g.Ty, g.Tx, g.H, g.W, g.Nv);
      break;
    default:
      break;  // unreachable: head_dim and dtype are validated by the ABI layer
  }
}

}  // namespace

void launch_permute(const Geo& g, int elem_bytes, const void* const src[3], void* const dst[3],
                    hipStream_t stream) {
  // compact the non-null pairs so that blockIdx.y indexes only real work
  CopySet set{};
  int n = 0;
  for (int i = 0; i < 3; ++i) {
    if (src[i] == nullptr) continue;
    set.src[n] = static_cast<const uint4*>(src[i]);
    set.dst[n] = static_cast<uint4*>(dst[i]);
    ++n;
  }
  if (n == 0) return;
  launch_reorder<true>(g, elem_bytes, set, n, stream);
}

void launch_permute_pool(const Geo& g, int elem_bytes, const void* const src[3],
                        void* const dst[3], float* qb, float* kb, hipStream_t stream) {
  CopySet set{};
  PoolSet pool{};
  int n = 0;
  float* const pooled[3] = {qb, kb, nullptr};
  for (int i = 0; i < 3; ++i) {
    if (src[i] == nullptr) continue;
    set.src[n] = static_cast<const uint4*>(src[i]);
    set.dst[n] = static_cast<uint4*>(dst[i]);
    pool.dst[n] = pooled[i];
    ++n;
  }
  if (n == 0) return;
  const int64_t blocks_total = g.BH * g.nb;
  const int64_t max_grid = int64_t{1} << 20;
  const dim3 grid(static_cast<unsigned>(blocks_total < max_grid ? blocks_total : max_grid),
                  static_cast<unsigned>(n));
#define CABF_RP(EB, D)                                                                        \
  hipLaunchKernelGGL((reorder_pool_blocks<EB, D>), grid, dim3(kThreads), 0, stream, set, pool, \
                     blocks_total, g.nb, g.Ty, g.Tx, g.H, g.W, g.Nv)
  if (elem_bytes == 2) {
    if (g.D == 64) CABF_RP(2, 64); else CABF_RP(2, 128);
  } else {
    if (g.D == 64) CABF_RP(4, 64); else CABF_RP(4, 128);
  }
#undef CABF_RP
}

void launch_unpermute(const Geo& g, int elem_bytes, const void* src, void* dst,
                      hipStream_t stream) {
  CopySet set{};
  set.src[0] = static_cast<const uint4*>(src);
  set.dst[0] = static_cast<uint4*>(dst);
  launch_reorder<false>(g, elem_bytes, set, 1, stream);
}

}  // namespace cabf
