// Block-sparse attention forward for two query blocks at once, over the union
// of their kept lists (NABLA summary, Methodology item 2, expansion bullet:
// attention runs on the kept (query block, key block) tiles only).
//
// Why pairs: on long rows (2048 blocks or more; 241 frames at 768p has
// 4026) a head's key range no longer fits L2 and the tile fetches from
// beyond it set the pace. The same patch in consecutive frames keeps largely
// the same key blocks, so a workgroup serving both blocks streams each K/V
// tile of the union of their lists into LDS once where two workgroups would
// fetch it twice (1.38 kept tiles per union tile at 720p / 80% on the seeded
// smooth-field workload). Lists are walked in order, in launches of as many
// workgroups as the device holds (each launch's workgroups start together
// and walk the key range in step). On shorter rows the one-block kernel is
// faster: a tile kept by one block only leaves the other group idle.
//
// Work decomposition
//   One workgroup of 8 waves per pair (A, B): waves 0-3 serve block A and
//   waves 4-7 block B, each group split as in bsa_fwd_mfma (wave (wq, wk):
//   query rows 32 wq .. +31, key half 32 wk .. +31 of every tile, its own
//   running max, sum and output, the key halves merged once at the end).
//   Waves w and w + 4 share a SIMD, so on a tile only one block kept, the
//   other group's wave leaves the SIMD to it.
//   Pairs: frames 2t and 2t + 1 at the same patch; with an odd number of
//   frames the patches of the last frame pair with their right neighbours.
//   At the start the two lists are merged into their ascending union in
//   LDS (one bit per key block and list), each entry tagged with the blocks
//   that kept it. All eight waves copy every union tile into the LDS ring; a
//   group computes a tile only if its block kept it (a wave-uniform branch)
//   and otherwise waits at the tile barrier.
//
// Per tile and group the arithmetic is bsa_fwd_mfma's, tile by tile in the
// same order (in deterministic mode the result is bit-identical to it):
// S^T = K Q^T on v_mfma_f32_32x32x16_bf16, pad keys masked, base-2 online
// softmax with the lazily raised running max, P rounded to bf16, O^T += V^T
// P^T with V^T from transposing LDS reads.
//
// Pipeline: K tiles stream into a three-slot ring two union tiles ahead, V
// tiles into a two-slot ring one tile ahead (global_load_lds_dwordx4); one
// barrier per union tile waits for every copy but the newest K tile.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attention_common.hpp"
#include "attention_tiles.hpp"
#include "geometry.hpp"
#include "launch.hpp"

namespace cabf {
namespace {

using namespace tiles;

constexpr int kPairWaves = 8;
constexpr int kPairThreads = 64 * kPairWaves;
constexpr float kSlack = 8.0f;                 // base-2 headroom of the lazily raised max
constexpr uint32_t kInA = 1u << 22;            // union entry: block A kept it
constexpr uint32_t kInB = 1u << 23;            // union entry: block B kept it
constexpr uint32_t kBlockBits = (1u << 22) - 1;

// Query blocks of pair p of a head with T frames of F blocks.
__device__ inline void pair_blocks(int p, int T, int F, int& A, int& B) {
  const int tp = T / 2;
  if (p < tp * F) {
    const int t2 = p / F;
    A = 2 * t2 * F + (p - t2 * F);
    B = A + F;
  } else {
    A = (T - 1) * F + 2 * (p - tp * F);
    B = A + 1 < T * F ? A + 1 : -1;
  }
}

template <int D>
__global__ __launch_bounds__(kPairThreads, 1) void bsa_fwd_pair(AttnArgs a, int pairs_per_head,
                                                                 int64_t n_items) {
  using S = Stage<D, kPairThreads>;
  constexpr int kKS = D / 16;   // MFMA k-steps over d
  constexpr int kDT = D / 32;   // 32-row d subtiles of O^T
  __shared__ u32x4 k_slot0[S::kTile], k_slot1[S::kTile], k_slot2[S::kTile];
  __shared__ u32x4 v_slot0[S::kTile], v_slot1[S::kTile];
  __shared__ uint32_t ulist[kPairMaxBlocks];              // union entries, ascending
  __shared__ uint32_t bits[2 * (kPairMaxBlocks / 32)];    // kept bits of A, then of B
  __shared__ int scan[kPairWaves + 1];   // wave totals, union length

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;        // 0: block A, 1: block B
  const int wq = wave & 1;
  const int wk = (wave >> 1) & 1;
  const int li = lane & 31;
  const int h = lane >> 5;

  const int64_t item = a.item0 + xcd_order(blockIdx.x, n_items);
  const int64_t bh = item / pairs_per_head;
  const int F = a.Ty * a.Tx;
  int blk_a, blk_b;
  pair_blocks(static_cast<int>(item - bh * pairs_per_head), a.nb / F, F, blk_a, blk_b);
  const int nb = a.nb;
  const int32_t* __restrict__ counts = a.kv_count + bh * nb;
  const int cnt_a = min(max(counts[blk_a], 0), nb);
  const int cnt_b = blk_b >= 0 ? min(max(counts[blk_b], 0), nb) : 0;
  const int32_t* __restrict__ list_a = a.kv_index + (bh * nb + blk_a) * nb;
  const int32_t* __restrict__ list_b = a.kv_index + (bh * nb + (blk_b >= 0 ? blk_b : blk_a)) * nb;

  // ---- union of the two lists: bitmaps, word counts, scan, expansion -----
  const int words = (nb + 31) >> 5;
  for (int i = tid; i < 2 * words; i += kPairThreads) bits[i] = 0u;
  __syncthreads();
  for (int i = tid; i < cnt_a; i += kPairThreads) {
    const int e = list_a[i];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(nb)) atomicOr(&bits[e >> 5], 1u << (e & 31));
  }
  for (int i = tid; i < cnt_b; i += kPairThreads) {
    const int e = list_b[i];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(nb))
      atomicOr(&bits[words + (e >> 5)], 1u << (e & 31));
  }
  __syncthreads();
  const uint32_t wa = tid < words ? bits[tid] : 0u;
  const uint32_t wb = tid < words ? bits[words + tid] : 0u;
  const int c = __builtin_popcount(wa | wb);
  int incl = c;                       // inclusive scan over the wave
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) {
    const int o = __shfl_up(incl, sh);
    incl += lane >= sh ? o : 0;
  }
  if (lane == 63) scan[wave] = incl;
  __syncthreads();
  int before = incl - c;
  for (int w = 0; w < wave; ++w) before += scan[w];
  if (tid == kPairThreads - 1) {
    int total = 0;
    for (int w = 0; w < kPairWaves; ++w) total += scan[w];
    scan[kPairWaves] = total;
  }
  for (uint32_t u = wa | wb; u != 0u; u &= u - 1u) {
    const int b = __builtin_ctz(u);
    const uint32_t flags = ((wa >> b) & 1u ? kInA : 0u) | ((wb >> b) & 1u ? kInB : 0u);
    ulist[before++] = pack_block_entry(a, tid * 32 + b) | flags;
  }
  __syncthreads();
  const int cnt = __builtin_amdgcn_readfirstlane(scan[kPairWaves]);   // union length

  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.qp);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.kp) + bh * a.N * D;
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.vp) + bh * a.N * D;
  const int my_blk = grp == 0 ? blk_a : blk_b;      // -1: this group has no block
  const uint32_t my_flag = grp == 0 ? kInA : kInB;

  // first row of this wave's 32 query rows (uniform); the lane's row is li below it
  const int64_t qrow0 = (bh * nb + (my_blk >= 0 ? my_blk : blk_a)) * kBlock + wq * 32;
  bf16x8 qf[kKS];
  {
    const uint16_t* qsrc = Q + (qrow0 + li) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const uint4 u = *reinterpret_cast<const uint4*>(qsrc + 16 * ks);
      qf[ks] = __builtin_bit_cast(bf16x8, u);
    }
  }
  f32x16 o[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  float m = -INFINITY;
  float l = 0.0f;
  float msub = 0.0f;
  float raise_at = -INFINITY;
  const float cs = a.scale_log2;
  const float inv_c = 1.0f / cs;
  const int key0 = 32 * wk;

  // union entries of the pass, 64 at a time, one per lane (from LDS)
  auto load_batch = [&](int b) {
    return ulist[min(b * 64 + lane, cnt - 1)];
  };
  uint32_t batch_cur = 0, batch_nxt = 0;
  auto entry = [&](int t) {
    const int p = t < cnt ? t : cnt - 1;
    return __builtin_amdgcn_readlane(batch_cur, p & 63);
  };
  auto tile_off = [](uint32_t e) { return static_cast<int64_t>(e & kBlockBits) * kBlock * D; };
  auto tile_rows = [](uint32_t e) { return 8 * static_cast<int>(e >> 28); };
  auto tile_cols = [](uint32_t e) { return static_cast<int>((e >> 24) & 15u); };

  const int vgrp = lane >> 4, vsl = lane & 15;
  const int vcol = 16 * (vgrp & 1) + 4 * (vsl & 3);
  const int vrow = key0 + 4 * (vgrp >> 1) + (vsl >> 2);
  int vaddr[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    const int cc = 32 * dt + vcol;
    vaddr[dt] = v_chunk_slot<D>(vrow, cc >> 3) * 8 + (cc & 7);
  }

  // One union tile for this group: S^T, statistics (pad keys masked, the
  // running max raised when the tile's max exceeds it by more than kSlack),
  // numerators and P.V. A tile depends on the one before only through the
  // statistics, so S^T of the next tile cannot start before this tile's
  // numerators without knowing whether the group keeps it; on tiles both
  // blocks kept, the two groups' waves overlap on each SIMD instead.
  auto compute = [&](uint32_t e, const u32x4* kb, const u32x4* vb) {
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const u32x4 u = kb[k_chunk_slot<D>(key0 + li, 2 * ks + h)];
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), qf[ks], s, 0, 0,
                                                  0);
    }
    bf16x8 vf[kDT][2];
    const uint16_t* sv = reinterpret_cast<const uint16_t*>(vb);
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint16_t* p = sv + vaddr[dt] + 16 * st * D;
        const s16x4 both[2] = {read_v_transposed(p), read_v_transposed(p + 8 * D)};
        __builtin_memcpy(&vf[dt][st], both, sizeof(bf16x8));
      }
    const BlockExtent ext{static_cast<int>(e >> 28), static_cast<int>((e >> 24) & 15u)};
    if (!ext.full()) {
      const uint32_t keep = real_accumulator_bits(ext, wk, h);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = ((keep >> r) & 1u) ? s[r] : -INFINITY;
    }
    float mt = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
    mt = pair_max(mt);
    if (__any(mt > raise_at)) {
      const float mn = fmaxf(m, mt * cs);
      const float alpha = (mn == -INFINITY) ? 1.0f : exp2f(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      msub = (m == -INFINITY) ? 0.0f : m;
      raise_at = (m + kSlack) * inv_c;
    }
    bf16x8 pb[2];
    float ps[4];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], cs, -msub));
      ps[r & 3] = r < 4 ? pr : ps[r & 3] + pr;
      pb[r >> 3][r & 7] = static_cast<__bf16>(pr);
    }
    l += (ps[0] + ps[1]) + (ps[2] + ps[3]);
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int st = 0; st < 2; ++st)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt][st], pb[st], o[dt], 0, 0, 0);
  };

  if (cnt > 0) {
    const uint32_t koff = tile_load_offset<D, Swz::K, kPairThreads>(wave, lane);
    const uint32_t voff = tile_load_offset<D, Swz::V, kPairThreads>(wave, lane);
    batch_cur = load_batch(0);
    batch_nxt = load_batch(1);
    uint32_t e_cur = entry(0);
    uint32_t e_next = entry(1);
    uint32_t e_after = entry(2);
    issue_tile_load<D, kPairThreads>(K + tile_off(e_cur), k_slot0, koff, wave, tile_rows(e_cur),
                                     tile_cols(e_cur));
    issue_tile_load<D, kPairThreads>(V + tile_off(e_cur), v_slot0, voff, wave, tile_rows(e_cur),
                                     tile_cols(e_cur));
    issue_tile_load<D, kPairThreads>(K + tile_off(e_next), k_slot1, koff, wave,
                                     tile_rows(e_next), tile_cols(e_next));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // tile t: K of t in k_slot[t % 3], K of t + 1 in k_slot[(t + 1) % 3]
    // (landed), V of t in v_slot[t % 2]; V of t + 1 streams into
    // v_slot[(t + 1) % 2] and K of t + 2 into k_slot[(t + 2) % 3], whose
    // tiles were read in tile t - 1.
    auto body = [&](int t, auto parity, auto phase) {
      constexpr int kOdd = decltype(parity)::value;
      constexpr int kPh = decltype(phase)::value;
      u32x4* const k_here = kPh == 0 ? k_slot0 : (kPh == 1 ? k_slot1 : k_slot2);
      u32x4* const k_fill = kPh == 0 ? k_slot2 : (kPh == 1 ? k_slot0 : k_slot1);
      u32x4* const v_here = kOdd ? v_slot1 : v_slot0;
      u32x4* const v_fill = kOdd ? v_slot0 : v_slot1;
      if (((t + 3) & 63) == 0 && t + 3 < cnt) {   // entry t + 3 opens the next batch
        batch_cur = batch_nxt;
        batch_nxt = load_batch(((t + 3) >> 6) + 1);
      }
      const uint32_t e_t3 = entry(t + 3);
      issue_tile_load<D, kPairThreads>(V + tile_off(e_next), v_fill, voff, wave,
                                       tile_rows(e_next), tile_cols(e_next));
      issue_tile_load<D, kPairThreads>(K + tile_off(e_after), k_fill, koff, wave,
                                       tile_rows(e_after), tile_cols(e_after));
      __builtin_amdgcn_sched_barrier(0);
      if (e_cur & my_flag) compute(e_cur, k_here, v_here);
      e_cur = e_next;
      e_next = e_after;
      e_after = e_t3;
      // every copy but the newest (K of t + 2) has landed after the barrier
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitAllButOneTile<D, kPairThreads>());
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    // unrolled by six (three K slots, two V slots); each body is entered only
    // from the one before it
    for (int t = 0;;) {
      body(t, I0{}, I0{});
      if (++t >= cnt) break;
      body(t, I1{}, I1{});
      if (++t >= cnt) break;
      body(t, I0{}, I2{});
      if (++t >= cnt) break;
      body(t, I1{}, I0{});
      if (++t >= cnt) break;
      body(t, I0{}, I1{});
      if (++t >= cnt) break;
      body(t, I1{}, I2{});
      if (++t >= cnt) break;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- merge the two key halves of every query row, per group ------------
  l += __shfl_xor(l, 32);
  static_assert(S::kTile * 16 >= kDT * 16 * 64 * 4, "merge area");
  float* const part = reinterpret_cast<float*>(
      grp ? (wq ? v_slot0 : k_slot2) : (wq ? k_slot1 : k_slot0));
  float* const merge_ml = reinterpret_cast<float*>(ulist) + grp * 256;   // [2 * 2 * 64] per group
  if (wk == 1) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[(dt * 16 + r) * 64 + lane] = o[dt][r];
    merge_ml[wq * 64 + lane] = m;
    merge_ml[(2 + wq) * 64 + lane] = l;
  }
  __syncthreads();
  if (wk == 1 || my_blk < 0) return;
  const float m1 = merge_ml[wq * 64 + lane];
  const float l1 = merge_ml[(2 + wq) * 64 + lane];
  const float mm = fmaxf(m, m1);
  const float a0 = (m == -INFINITY) ? 0.0f : exp2f(m - mm);
  const float a1 = (m1 == -INFINITY) ? 0.0f : exp2f(m1 - mm);
  const float lt = l * a0 + l1 * a1;
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  const float w0 = a0 * inv, w1 = a1 * inv;
  uint16_t* __restrict__ O = static_cast<uint16_t*>(a.op);
  int lane_row = li;
  asm volatile("" : "+v"(lane_row));   // rebuilt here rather than held through the loop
  const int64_t qrow = qrow0 + lane_row;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * h;
      float v[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 4 * g + x;
        v[x] = o[dt][r] * w0 + part[(dt * 16 + r) * 64 + lane] * w1;
      }
      uint2 wv;
      wv.x = static_cast<uint32_t>(f32_to_bf16_rne(v[0])) |
             (static_cast<uint32_t>(f32_to_bf16_rne(v[1])) << 16);
      wv.y = static_cast<uint32_t>(f32_to_bf16_rne(v[2])) |
             (static_cast<uint32_t>(f32_to_bf16_rne(v[3])) << 16);
      *reinterpret_cast<uint2*>(O + qrow * D + d) = wv;
    }
  if (a.lse != nullptr && h == 0) a.lse[qrow] = lt > 0.0f ? (mm + log2f(lt)) * kLn2 : -INFINITY;
}

}  // namespace

int pairs_per_head(int T, int Ty, int Tx) {
  const int F = Ty * Tx;
  return (T / 2) * F + (T % 2 ? (F + 1) / 2 : 0);
}

void launch_bsa_forward_pair(const AttnArgs& args, int D, int T, hipStream_t stream) {
  const int pph = pairs_per_head(T, args.Ty, args.Tx);
  const int64_t n = args.BH * pph;
  AttnArgs a = args;
  a.sweep_ticks = 0u;
  const void* kernel = D == 64 ? reinterpret_cast<const void*>(&bsa_fwd_pair<64>)
                               : reinterpret_cast<const void*>(&bsa_fwd_pair<128>);
  const int64_t per = kGenerationsPerLaunch * resident_workgroups(kernel, kPairThreads, stream);
  launch_in_generations(n, per, [&](int64_t first, int64_t count) {
    a.item0 = first;
    const unsigned grid = static_cast<unsigned>(count);
    if (D == 64)
      hipLaunchKernelGGL((bsa_fwd_pair<64>), dim3(grid), dim3(kPairThreads), 0, stream, a, pph, count);
    else
      hipLaunchKernelGGL((bsa_fwd_pair<128>), dim3(grid), dim3(kPairThreads), 0, stream, a, pph, count);
  });
}

}  // namespace cabf
