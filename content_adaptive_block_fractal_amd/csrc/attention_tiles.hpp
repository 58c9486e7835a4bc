// Tile plumbing shared by the block-sparse attention kernels on bf16 matrix
// cores (forward and backward): 64-row K/V-like tiles streamed from global
// memory straight into swizzled LDS slots, row reads for the A/B operands of
// v_mfma_f32_32x32x16_bf16 and transposing reads for the transposed operand.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "geometry.hpp"

namespace cabf {
namespace tiles {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;

// Workgroup id -> query block: XCD x (which receives ids x, x+8, ...) gets
// the contiguous range [start_x, start_x + count_x).
__device__ inline int64_t xcd_order(int64_t wg, int64_t total) {
  const int64_t xcd = wg % kXcds, local = wg / kXcds;
  const int64_t per = total / kXcds, rem = total % kXcds;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// Workgroup id -> work item (h * per_head + i) of a pass over the items of
// all BH heads in one launch, with `group` XCDs sharing a head: XCD x =
// group * p + q works through heads p, p + 8 / group, p + 2 (8 / group), ...
// and takes the q-th share of each head's items, so the XCDs of a group are
// on the same head at about the same time and 8 / group heads are in flight.
// The share is the q-th of `group` contiguous parts, or with `interleaved`
// every group-th item from q (for items ordered by size, so that the XCDs of
// a group get the same mix). The caller guarantees per_head % group == 0 and
// BH % (8 / group) == 0 (xcd_group_for); group <= 1 is xcd_order.
__device__ inline int64_t xcd_head_order(int64_t wg, int64_t total, int64_t per_head, int group,
                                         bool interleaved = false) {
  if (group <= 1) return xcd_order(wg, total);
  const int64_t xcd = wg % kXcds, local = wg / kXcds;
  const int64_t groups = kXcds / group;
  const int64_t per = per_head / group;
  const int64_t j = local / per, i = local - j * per;
  const int64_t head = xcd / group + groups * j, q = xcd % group;
  return head * per_head + (interleaved ? i * group + q : q * per + i);
}

// K tile: 64 rows x D bf16 = 64 x (D/8) chunks of 16 bytes.
template <int D>
__device__ inline int k_chunk_slot(int key, int chunk) {
  constexpr int kChunks = D / 8;
  // D = 128: a row spans all 64 banks, rotate chunks by key % 16;
  // D = 64: two rows per bank sweep, rotate by (key / 2) % 8.
  const int swz = (D == 128) ? (key & 15) : ((key >> 1) & 7);
  return key * kChunks + (chunk ^ swz);
}

// V tile: 64 rows x D bf16, row-major like K. A transposing read fetches,
// per 16-lane group, 4 consecutive rows x 32 bytes; the two groups of a
// 32-lane half read the same rows at neighbouring 32-byte columns. XOR-ing
// the 16-byte chunk index with 4 * (row % 4) (D = 64: 4 * ((row / 2) % 2))
// keeps every 32-byte pair intact and gives the 8 (row, pair) reads of a
// half distinct banks.
template <int D>
__device__ inline int v_chunk_slot(int key, int chunk) {
  constexpr int kChunks = D / 8;
  const int swz = (D == 128) ? 4 * (key & 3) : 4 * ((key >> 1) & 1);
  return key * kChunks + (chunk ^ swz);
}

// A tile read both ways (the backward's Q, dO and K tiles): by rows, 16
// bytes per lane and 16 consecutive rows per 16-lane group, as K; and
// transposed, 4 consecutive rows x 64 bytes per 32-lane half, as V. The
// chunk index is XOR-ed with f(row), a permutation over 16 consecutive rows
// (D = 64: over the 8 rows of a bank half) whose bits 2-3 differ between
// the 4 rows of a transposing read (D = 64: between its two rows in a bank
// half), so both kinds of read hit 64 distinct banks. K's rotation by row
// leaves a transposing read four chunks in four banks' worth of space (a
// 4-way conflict); V's leaves row reads 4-way conflicted.
template <int D>
__device__ inline int b_chunk_slot(int row, int chunk) {
  constexpr int kChunks = D / 8;
  const int swz = (D == 128) ? 4 * (row & 3) + ((row >> 2) & 3)
                             : 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
  return row * kChunks + (chunk ^ swz);
}

// Which swizzle a tile copy lays out.
enum class Swz { K, V, B };

typedef short s16x4 __attribute__((ext_vector_type(4)));

// max of v over lanes l and l ^ 32 (v_permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second: with both set
// to v, the two results hold v of lane l and of lane l ^ 32 in every lane)
__device__ inline float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 4 consecutive keys of one head-dim column of the V tile (see above).
__device__ inline s16x4 read_v_transposed(const uint16_t* sv_row_chunk) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sv_row_chunk));
}

// The sweep period P in clock ticks (see clock_phased_start). Called by one
// whole wave; every lane returns the same value.
__device__ inline uint32_t sweep_period(const int32_t* head_counts, int nb, uint32_t ticks, int lane) {
  int total = min(max(head_counts[(lane * nb) >> 6], 1), nb);
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) total += __shfl_xor(total, sh);
  return static_cast<uint32_t>(max(total >> 6, 1)) * ticks;
}

// The block the sweep has reached now. 32 clock bits wrap every 43 s: one
// incoherent moment, harmless.
__device__ inline int swept_block(uint32_t period, int nb) {
  const uint32_t now = static_cast<uint32_t>(__builtin_amdgcn_s_memrealtime());
  return static_cast<int>(static_cast<uint64_t>(now % period) * nb / period);
}

// Where a pass over an ascending list of cnt block indices (in [0, nb))
// starts, for a clock-phased visit order: a sweep runs over the block range
// once every P ticks of the 100 MHz clock, and the pass starts at the first
// entry at or after the block the sweep has reached ((clock mod P) / P * nb),
// wrapping around. Workgroups that run at the same time then read about the
// same tiles (which stay in L2). P must be the same for every workgroup of a
// head, or clock mod P would not be coherent: P = ticks * the mean length of
// 64 lists spread evenly over the head (head_counts[0 .. nb)), which all of
// them sample alike; ticks approximates the time of one tile. Called by one
// whole wave; every lane returns the same value.
__device__ inline int clock_phased_start(const int32_t* head_counts, const int32_t* list, int nb,
                                         int cnt, uint32_t ticks, int lane) {
  if (ticks == 0 || cnt <= 1) return 0;
  const int swept = swept_block(sweep_period(head_counts, nb, ticks, lane), nb);
  int before = 0;   // entries below the swept block
  for (int i = lane; i < cnt; i += 64) before += list[i] < swept ? 1 : 0;
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) before += __shfl_xor(before, sh);
  return before >= cnt ? 0 : before;
}

// How a tile copy is issued. Both are direct-to-LDS copies (lane l's 4 or
// 16 bytes land at LDS byte address lds + 4 l or lds + 16 l; M0 holds the LDS
// base).
// - Builtin: the compiler's LDS-copy builtin. Its wait pass counts such a
//   copy against both the memory and the LDS counter, so while one is in
//   flight every wait it inserts for an LDS read is a full one (lgkmcnt(0)).
// - Asm: the same instruction as an asm statement (M0 write, one wait state,
//   the copy), which the compiler does not see: its waits for LDS reads then
//   count only the reads, and its waits for its own loads can only get
//   stricter by the copies it does not count. The caller waits for these
//   copies itself (the tile barrier's vmcnt) before their data is read.
// The backward passes use Asm (1.7-1.9% faster, bit-identical); the forward,
// held at the package power limit, measured 0.5% slower with it and keeps
// Builtin.
enum class Copy { Builtin, Asm };

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)p));
}
__device__ __forceinline__ void lds_copy_x4_asm(const void* sbase, uint32_t voff, const void* lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_address(lds)) : "memory", "m0");
}
__device__ __forceinline__ void lds_copy_x1_asm(const void* sbase, uint32_t voff, const void* lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_address(lds)) : "memory", "m0");
}

// Tile copies by a workgroup of NT threads (NT / 64 waves).
template <int D, int NT = kThreads>
struct Stage {
  static constexpr int kChunks = D / 8;                        // 16-byte chunks per row
  static constexpr int kIters = kBlock * kChunks / NT;         // chunks per thread per tensor
  static constexpr int kTile = kBlock * kChunks;               // 16-byte chunks per K (or V) tile
  static constexpr int kRowsPerIter = NT / kChunks;            // rows one pass of the workgroup fills
  static constexpr int kWavesPerGroup = NT / 64;
};

// Direct-to-LDS copy of one K or V tile into a ring slot: each wave
// instruction fills 64 consecutive 16-byte LDS chunks (lane l -> chunk base +
// l); the lane fetches the global chunk that the swizzle places there. Pass i
// covers the rows of pass 0 moved down by i * kRowsPerIter, a multiple of the
// swizzle's period in the row, so a lane's source offset in pass i is its
// offset in pass 0 plus a constant (added to the scalar base). The offsets are
// the same for every tile.
template <int D, Swz L, int NT = kThreads>
__device__ inline uint32_t tile_load_offset(int wave, int lane) {
  using S = Stage<D, NT>;
  static_assert(S::kRowsPerIter % 16 == 0, "swizzle period");
  const int phys = wave * 64 + lane;
  const int row = phys / S::kChunks;
  const int pc = phys % S::kChunks;
  // every swizzle is an XOR with a function of the row: its own inverse
  const int slot = L == Swz::V ? v_chunk_slot<D>(row, pc)
                               : (L == Swz::B ? b_chunk_slot<D>(row, pc) : k_chunk_slot<D>(row, pc));
  const int chunk = slot - row * S::kChunks;
  return static_cast<uint32_t>((row * D + chunk * 8) * 2);
}

// s_waitcnt immediate: vmcnt = the loads of one tile copy (Stage::kIters),
// expcnt and lgkmcnt not waited on (gfx9 encoding: vmcnt[3:0] and [15:14],
// expcnt[6:4], lgkmcnt[11:8])
template <int D, int NT = kThreads>
constexpr int kWaitAllButOneTile() {
  constexpr int n = Stage<D, NT>::kIters;
  static_assert(n < 64, "vmcnt range");
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// Rows of the tile at or past `real_rows`, or whose patch column (row % 8) is
// at or past `real_cols`, hold no token the kernel uses (pad rows and columns
// of a partial patch, keys past a chunk, or every row of an invalid entry): a
// wave's share of a pass that covers only such rows reloads its share of
// pass 0 instead (L1/L2-resident, finite data where masked rows read it),
// which keeps the number of loads per copy, and so the vmcnt bookkeeping,
// unchanged. A wave's share is 4 rows at d = 128 (half a patch row) and 8 at
// d = 64 (a whole patch row).
template <int D, int NT = kThreads, Copy C = Copy::Builtin>
__device__ __forceinline__ void issue_tile_load(const uint16_t* tile_src, u32x4* slot,
                                                uint32_t off, int wave, int real_rows = kBlock,
                                                int real_cols = kP) {
  using S = Stage<D, NT>;
  constexpr int kW = S::kWavesPerGroup;
  // An empty asm makes each load's scalar base (tile and pass) and lane
  // offset opaque, so the compiler cannot fold (base + lane offset) once and
  // rebuild every other address with 64-bit vector adds: the base stays in
  // SGPRs and the 32-bit offset in a VGPR (the saddr + voffset form).
  uint32_t o = off;
  asm volatile("" : "+v"(o));
#pragma unroll
  for (int i = 0; i < S::kIters; ++i) {
    // rows of this wave's instruction: first_row .. first_row + kRowsPerIter / kWaves - 1
    const int first_row = i * S::kRowsPerIter + wave * (S::kRowsPerIter / kW);
    const bool used = first_row < real_rows && (first_row & (kP - 1)) < real_cols;
    const uint16_t* src = used ? tile_src + i * S::kRowsPerIter * D : tile_src;
    if constexpr (C == Copy::Asm) {
      lds_copy_x4_asm(src, o, slot + (i * kW + wave) * 64);
    } else {
      const char* base = reinterpret_cast<const char*>(src);
      asm volatile("" : "+s"(base));
      __builtin_amdgcn_global_load_lds(base + o, slot + (i * kW + wave) * 64, 16, 0, 0);
    }
  }
}

}  // namespace tiles
}  // namespace cabf
