// Shared pieces of the block-sparse attention kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "geometry.hpp"

namespace cabf {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const void* qp;
  const void* kp;
  const void* vp;
  const int32_t* kv_count;
  const int32_t* kv_index;
  void* op;
  float* lse;
  float scale_log2;   // softmax scale times log2(e): logits are kept in base 2
  int nb, Ty, Tx, H, W;
  int64_t N;          // reordered tokens per (batch, head)
  int64_t BH;         // batch * heads
  // Device-clock ticks (100 MHz) a workgroup is expected to spend per kept
  // tile, or 0. Nonzero: a workgroup starts its pass over its (ascending) list
  // at the key block a clock-driven sweep of the key range has reached, and
  // wraps around, so that concurrent workgroups read the same K/V tiles
  // together and find them in L2. Only the summation order changes: results
  // agree to rounding but may differ bitwise between runs. 0 walks every list
  // from its first entry (bit-reproducible).
  uint32_t sweep_ticks;
  // First work item of this launch: a pass in list order runs as a series of
  // launches of as many workgroups as the device holds at once (see
  // resident_workgroups), each over the next items.
  int64_t item0;
  // XCDs that share a head in a pass over all BH * nb items in one launch
  // (xcd_head_order; xcd_group_for picks it), or 0: every XCD takes a
  // contiguous range of the items (xcd_order).
  int xcd_group;
};

// XCDs per head for a pass over all BH * nb items (nb per head, head-major)
// in one launch: the smallest group (1, 2, 4 or 8 of the 8 XCDs) whose heads
// in flight, 8 / group of them, keep their K and V (or Q and dO: 2 N D bf16
// values per head) within three quarters of the 256 MB last-level cache
// (MALL) beyond the L2s. With more heads in flight the tiles that miss L2
// come from HBM instead (720p, 40 heads of 41 MB: two XCDs per head, four
// heads in flight, gave the forward 1-4% over one head per XCD).
inline int xcd_group_for(int64_t BH, int nb, int64_t N, int D) {
  const int64_t head_bytes = 2 * N * D * 2;
  const int64_t budget = int64_t{192} << 20;
  for (int g = 1; g <= 8; g *= 2) {
    const int64_t in_flight = 8 / g;
    if (in_flight * head_bytes > budget || nb % g != 0 || BH % in_flight != 0) continue;
    return g;
  }
  return 1;
}

// Workgroups of `kernel` (launched with `threads` threads and no dynamic LDS)
// that the device of `stream` runs at once; 0 when the runtime cannot say.
int64_t resident_workgroups(const void* kernel, int threads, hipStream_t stream);

// Launches of a pass in list order: `launch(first, n)` for consecutive runs
// of `per` items (all of them in one launch when per <= 0).
template <typename F>
void launch_in_generations(int64_t items, int64_t per, F&& launch) {
  if (per <= 0) per = items;
  for (int64_t first = 0; first < items; first += per) launch(first, items - first < per ? items - first : per);
}

// Real rows / columns of block b's 8x8 patch (pads sit at the bottom/right
// edge of the padded frame).
struct BlockExtent {
  int vy, vx;
  __device__ bool real(int k) const { return (k >> 3) < vy && (k & 7) < vx; }
  __device__ bool full() const { return vy == kP && vx == kP; }
};

__device__ inline BlockExtent block_extent(int b, const AttnArgs& a) {
  const int per_frame = a.Ty * a.Tx;
  const int rem = b % per_frame;
  const int ty = rem / a.Tx;
  const int tx = rem - ty * a.Tx;
  BlockExtent e;
  e.vy = min(kP, a.H - ty * kP);
  e.vx = min(kP, a.W - tx * kP);
  return e;
}

// Bit r set when row 8 * (r / 4) + 4 * h + r % 4 of half `half` of a 64-token
// block (the rows or columns one lane holds in a 32x32 accumulator; block
// row k is patch cell (k / 8, k % 8)) is a real token of the patch.
__device__ inline uint32_t real_accumulator_bits(const BlockExtent& ext, int half, int h) {
  uint32_t bits = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int iy = 4 * half + (r >> 2), ix = 4 * h + (r & 3);
    bits |= (iy < ext.vy && ix < ext.vx) ? (1u << r) : 0u;
  }
  return bits;
}

// A block-list entry as the tile loops hold it: the block index in bits
// 0..23 and its real extent in bits 24..31 (vy << 4 | vx; 0 for an entry
// outside [0, nb)), so that a loop finds partial blocks without a division.
__device__ inline uint32_t pack_block_entry(const AttnArgs& a, int32_t e) {
  if (static_cast<unsigned>(e) >= static_cast<unsigned>(a.nb)) return 0u;
  const BlockExtent ext = block_extent(e, a);
  return static_cast<uint32_t>(e) | (static_cast<uint32_t>((ext.vy << 4) | ext.vx) << 24);
}
__device__ inline BlockExtent packed_extent(uint32_t p) {
  const int code = static_cast<int>(p >> 24);
  return BlockExtent{code >> 4, code & 15};
}
__device__ inline int packed_block(uint32_t p) { return static_cast<int>(p & 0xffffffu); }

__device__ inline float load_elem(const float* p) { return *p; }
__device__ inline float load_elem(const uint16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

// float -> bfloat16 bits, round to nearest even (finite inputs)
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ inline void store_elem(float* p, float v) { *p = v; }
__device__ inline void store_elem(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }

// Longest block row the paired forward (attention_pair.hip) merges in LDS.
constexpr int kPairMaxBlocks = 8192;
// Rows of at least this many blocks count as long (see launch_bsa_forward).
constexpr int kLongRowBlocks = 2048;
// Launches of a list-order pass hold this many device-fulls of workgroups.
constexpr int64_t kGenerationsPerLaunch = 1;

void launch_bsa_forward_simple(const AttnArgs& a, bool bf16, int D, hipStream_t stream);
// The bf16 forward over pairs of query blocks (frames 2t, 2t+1 of a patch) and
// the union of their lists, in list order; nb <= kPairMaxBlocks. T = frames.
void launch_bsa_forward_pair(const AttnArgs& a, int D, int T, hipStream_t stream);
int pairs_per_head(int T, int Ty, int Tx);
void launch_bsa_forward_mfma(const AttnArgs& a, int D, bool phased, hipStream_t stream);
// The bf16 forward over a list of n global query block ids only.
void launch_bsa_forward_subset_mfma(const AttnArgs& a, int D, bool phased,
                                    const int32_t* q_blocks, int64_t n, hipStream_t stream);
// Variable-size cluster attention on the same kernel: a.N = rows per head of
// the permuted (and padded) tensors; work items from the query-tile table.
void launch_cluster_attention_mfma(const AttnArgs& a, int D, const int32_t* tiles, int max_tiles,
                                   const int32_t* q_off, int cq, const int32_t* chunk_count,
                                   const int32_t* chunks, int cap, hipStream_t stream);

}  // namespace cabf
