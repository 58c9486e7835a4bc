// Block-sparse attention forward on bf16 matrix cores (NABLA summary,
// Methodology item 2, expansion bullet: attention runs on the kept
// (query block, key block) tiles only).
//
// Work decomposition
//   One workgroup = one 64-row query block, 4 waves. Wave w owns query rows
//   32*(w&1) .. +31 and the key half 32*(w>>1) .. +31 of every kept tile; it
//   keeps its own running max, sum and output for that half, and the two
//   halves of a query row are merged once at the end through LDS (the merge
//   of two partial softmax sums is exact). Workgroup ids are remapped so
//   that each XCD (its own L2) processes a contiguous run of query blocks of
//   the same head, and by default each workgroup starts its pass over its
//   ascending list where a clock-driven sweep of the key range stands, so
//   that the workgroups of a head sweep the key range together and read the
//   same K/V tiles at about the same time (in deterministic mode the list is
//   walked from its first entry, in launches of as many workgroups as the
//   device holds, which start together and walk the key range in step).
//
// Per kept tile, per wave, with v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T    A = K (LDS, row-major, 16-byte chunks XOR-swizzled by row)
//                  B = Q^T (registers, loaded once)
//                  -> each lane holds one query row and 16 of its 32 keys,
//                  the other 16 sit in lane ^ 32
//   online softmax in base 2 on the fp32 accumulators; the running max is
//   only raised (and the output rescaled) when a row's max grows by more than
//   2^8, so the numerators stay below 2^8 and most tiles skip the rescale
//   O^T += V^T P^T A = V^T, read from the row-major V tile in LDS with the
//                  transposing LDS read (ds_read_b64_tr_b16: within a
//                  16-lane group, lane i receives element i%4 of the
//                  8-byte rows read by lanes 4e + i/4, e = 0..3), so each
//                  lane gets 4 consecutive keys of one head-dim column
//                  B = P^T (the softmax numerators, rounded to bf16)
// The contraction index of each product only has to be spread over the
// lanes the same way in both operands; V^T is read with the key order the
// S^T accumulator layout gives P.
//
// Pipeline: K and V tiles stream straight from global memory into LDS rings
// (global_load_lds_dwordx4; three K slots, two V slots), one LDS object per
// slot so that reads of the current tile never wait for the tiles in
// flight. In tile e the products S^T of tile e+1 run on the matrix cores
// while the vector ALUs compute the softmax numerators of tile e (whose max
// was taken at the end of tile e-1), then P.V of tile e; the copies of V of
// e+1 and K of e+3 are issued at the top of the tile. One barrier per tile,
// which waits for every copy but the newest K tile.
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
constexpr float kRescaleSlack = 8.0f;   // base-2 headroom before the running max is raised

// A list entry decoded: element offset of its 64 K/V rows in the head, and
// what the layout needs to mask it (block index, or number of valid keys).
struct TileRef {
  int64_t off;
  int jb;
  int code;     // block list: the extent code of the entry (see BlockListLayout::prep)
  int rows;     // rows of the tile that can hold a used token (the rest need not be loaded)
  int cols;     // patch columns (row % 8) that can hold one
  bool real;
};

// What a workgroup computes: 64 consecutive rows of Q and O starting at the
// global row qrow0 (over all batch-heads), of which the first `rows` are
// stored, against the cnt key tiles of `list`, in head bh's K and V.
struct WorkItem {
  int64_t bh;
  int64_t qrow0;
  int rows;
  int cnt;
  const int32_t* list;
};

// Kept 64-token blocks of the reordered grid (NABLA path): one work item per
// query block, list entries are key block indices, pad keys of partially
// padded patches are masked.
struct BlockListLayout {
  static constexpr bool kPhased = true;   // clock-phased start (AttnArgs::sweep_ticks)
  // work items per head, and whether the XCDs sharing a head (xcd_head_order)
  // take contiguous parts of its items or interleave them
  static constexpr bool kInterleave = false;
  __device__ int64_t items_per_head(const AttnArgs& a) const { return a.nb; }
  __device__ bool work(const AttnArgs& a, int64_t item, WorkItem& w) const {
    w.bh = item / a.nb;
    w.qrow0 = item * kBlock;
    w.rows = kBlock;
    w.cnt = min(max(a.kv_count[item], 0), a.nb);
    w.list = a.kv_index + item * a.nb;
    return true;
  }
  // A list entry as the batch holds it (pack_block_entry), computed once per
  // batch of 64 entries, one per lane.
  __device__ uint32_t prep(const AttnArgs& a, int32_t e) const { return pack_block_entry(a, e); }
  // entries outside [0, nb) load block 0 and are masked out entirely
  template <int D>
  __device__ TileRef decode(const AttnArgs&, uint32_t p) const {
    TileRef r;
    r.code = static_cast<int>(p >> 24);
    r.real = r.code != 0;
    r.jb = packed_block(p);
    r.rows = 8 * (r.code >> 4);     // patch rows at or past vy are pads (0 for an invalid entry)
    r.cols = r.code & 15;           // and so are columns at or past vx
    r.off = static_cast<int64_t>(r.real ? r.jb : 0) * kBlock * D;
    return r;
  }
  // false when every key of the tile is real; else the lane's real-key bits
  __device__ bool partial(const AttnArgs&, const TileRef& t, int wk, int h, uint32_t& bits) const {
    const BlockExtent ext{t.code >> 4, t.code & 15};
    if (ext.full()) return false;
    bits = real_accumulator_bits(ext, wk, h);
    return true;
  }
};

// A caller-given subset of query blocks (active queries: HSA summary, KV-cache
// synchronisation, only the active tokens' queries attend, over the full K
// and V): work item = entry of a list of global query block ids; entries
// outside [0, B*h*nb) are skipped.
struct SubsetLayout : BlockListLayout {
  const int32_t* items;
  int64_t total;
  __device__ bool work(const AttnArgs& a, int64_t idx, WorkItem& w) const {
    const int32_t it = items[idx];
    if (it < 0 || it >= total) return false;
    return BlockListLayout::work(a, it, w);
  }
};

// Variable-size clusters (semantic-permutation path, Sparse VideoGen2
// summary, Methodology C: contiguous query tokens, the key tokens of the
// selected clusters): one work item per 64-row tile of a query cluster; list
// entries are key chunks (first key row << 6) | (keys - 1), 1 to 64 keys.
struct ClusterLayout {
  static constexpr bool kPhased = false;
  // the tiles of a head are ordered by cluster, unused entries last: XCDs
  // sharing a head interleave them, so each gets the same mix
  static constexpr bool kInterleave = true;
  const int32_t* tiles;         // [BH, max_tiles, 2]: query cluster (or -1), first row
  int max_tiles;
  const int32_t* q_off;         // [BH, cq + 1]
  int cq;
  const int32_t* chunk_count;   // [BH, cq]
  const int32_t* chunks;        // [BH, cq, cap]
  int cap;
  __device__ int64_t items_per_head(const AttnArgs&) const { return max_tiles; }
  __device__ bool work(const AttnArgs& a, int64_t item, WorkItem& w) const {
    const int qa = tiles[item * 2];
    if (qa < 0) return false;
    const int row0 = tiles[item * 2 + 1];
    w.bh = item / max_tiles;
    w.qrow0 = w.bh * a.N + row0;
    w.rows = min(kBlock, q_off[w.bh * (cq + 1) + qa + 1] - row0);
    const int64_t qc = w.bh * cq + qa;
    w.cnt = min(max(chunk_count[qc], 0), cap);
    w.list = chunks + qc * cap;
    return true;
  }
  __device__ uint32_t prep(const AttnArgs&, int32_t e) const { return static_cast<uint32_t>(e); }
  template <int D>
  __device__ TileRef decode(const AttnArgs&, uint32_t e) const {
    TileRef r;
    r.jb = static_cast<int>(e & 63u) + 1;      // keys of the chunk
    r.code = 0;
    r.rows = r.jb;
    r.cols = kP;
    r.real = true;
    r.off = static_cast<int64_t>(e >> 6) * D;
    return r;
  }
  __device__ bool partial(const AttnArgs&, const TileRef& t, int wk, int h, uint32_t& bits) const {
    if (t.jb == kBlock) return false;
    bits = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * wk + 8 * (r >> 2) + 4 * h + (r & 3);
      bits |= key < t.jb ? (1u << r) : 0u;
    }
    return true;
  }
};

template <int D, class L>
__global__ __launch_bounds__(kThreads, 2) void bsa_fwd_mfma(AttnArgs a, L lay, int64_t n_items) {
  using S = Stage<D>;
  constexpr int kKS = D / 16;   // MFMA k-steps over d
  constexpr int kDT = D / 32;   // 32-row d subtiles of O^T
  // Ring slots are separate LDS objects so that the compiler can tell the
  // tile being read from the tiles still streaming in (no wait on them).
  // K has three slots (K of e+3 streams in while S^T of e+1 is read), V two.
  // Five 16 KB slots (d = 128) leave room for two workgroups per CU; the
  // start position and the merge scalars borrow V slots when no tile is in
  // them.
  __shared__ u32x4 k_slot0[S::kTile], k_slot1[S::kTile], k_slot2[S::kTile];
  __shared__ u32x4 v_slot0[S::kTile], v_slot1[S::kTile];
  float* const merge_ml = reinterpret_cast<float*>(v_slot0);   // [2 * 2 * 64]
  int* const start_shared = reinterpret_cast<int*>(v_slot1);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
  const int wq = wave & 1;      // query half of the block
  const int wk = wave >> 1;     // key half of every tile
  const int li = lane & 31;
  const int h = lane >> 5;
  WorkItem w;
  if (!lay.work(a, a.item0 + xcd_head_order(blockIdx.x, n_items, lay.items_per_head(a), a.xcd_group,
                                             L::kInterleave),
                w))
    return;   // uniform per workgroup
  const int64_t bh = w.bh;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.qp);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.kp) + bh * a.N * D;
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.vp) + bh * a.N * D;

  // Q^T fragments: lane holds query row li of this wave's half, d = 16 ks + 8 h .. +7
  const int64_t qrow = w.qrow0 + wq * 32 + li;
  bf16x8 qf[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    const uint4 u = *reinterpret_cast<const uint4*>(Q + qrow * D + 16 * ks + 8 * h);
    qf[ks] = __builtin_bit_cast(bf16x8, u);
  }

  f32x16 o[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  float m = -INFINITY;   // running max of the row (this key half), base-2 scaled logits
  float l = 0.0f;        // this lane's part of the row sum
  const float c = a.scale_log2;

  const int cnt = w.cnt;
  const int32_t* __restrict__ list = w.list;
  const int key0 = 32 * wk;     // first key of this wave's half

  // Where the pass over the list starts (AttnArgs::sweep_ticks; see
  // clock_phased_start). Wave 0 computes it and shares it through LDS, so
  // that all waves agree on it.
  if (wave == 0) {
    const int start = L::kPhased ? clock_phased_start(a.kv_count + bh * a.nb, w.list, a.nb,
                                                      cnt, a.sweep_ticks, lane)
                                 : 0;
    if (lane == 0) *start_shared = start;
  }
  __syncthreads();
  const int start = __builtin_amdgcn_readfirstlane(*start_shared);
  // Entries of the pass are fetched 64 at a time, one per lane, a batch ahead
  // of use, and read out with readlane: no list load is waited on per tile.
  // Entry t of the pass is list entry start + t (wrapped); t is clamped to the
  // last one (loads past the end are redundant but in bounds, and their
  // results are never used).
  // The next batch is kept as loaded and prepared (lay.prep) only when it
  // comes into use: preparing it right after the load would wait for the
  // load, and with it for every tile copy issued before it.
  auto load_batch = [&](int b) {
    int pos = min(b * 64 + lane, cnt - 1) + start;
    pos -= pos >= cnt ? cnt : 0;
    return list[pos];
  };
  uint32_t batch_cur = 0;    // entries 64 B .. of the pass, prepared
  int32_t batch_nxt = 0;     // entries 64 (B + 1) .., as loaded
  auto tile = [&](int t) {
    const int p = t < cnt ? t : cnt - 1;
    return lay.template decode<D>(a, __builtin_amdgcn_readlane(batch_cur, p & 63));
  };
  // S^T of this wave's 32 keys from the K tile in `kb`
  auto scores = [&](const u32x4* kb) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const u32x4 u = kb[k_chunk_slot<D>(key0 + li, 2 * ks + h)];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), qf[ks], acc,
                                                    0, 0, 0);
    }
    return acc;
  };
  // V^T fragment addressing (see read_v_transposed): the lane reads rows
  // vrow + 16 st (+ 8), columns 32 dt + vcol. Rows 8 and 16 further down have
  // the same swizzle, so one element offset per dt serves all four reads
  // (the rest are constant offsets).
  const int vgrp = lane >> 4, vsl = lane & 15;
  const int vcol = 16 * (vgrp & 1) + 4 * (vsl & 3);
  const int vrow = key0 + 4 * (vgrp >> 1) + (vsl >> 2);
  int vaddr[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    const int cc = 32 * dt + vcol;
    vaddr[dt] = v_chunk_slot<D>(vrow, cc >> 3) * 8 + (cc & 7);
  }

  if (cnt > 0) {
    // Softmax statistics of a tile whose S^T is in `s`: pad keys masked, and
    // the running max raised (the output and the sum rescaled) when the
    // tile's max exceeds it by more than kRescaleSlack. They run one tile
    // ahead of the numerators, at the end of the previous tile, so that the
    // numerators and the products of a tile are one branch-free stretch of
    // code that the compiler can interleave.
    float msub = 0.0f;              // max the numerators are taken against (0 while m = -inf)
    const float inv_c = 1.0f / c;
    float raise_at = -INFINITY;     // raw tile max above which m is raised: (m + slack) / c
    auto stats = [&](f32x16& s, const TileRef& t) {
      uint32_t bits = 0;
      if (lay.partial(a, t, wk, h, bits)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = ((bits >> r) & 1u) ? s[r] : -INFINITY;
      }
      float mt = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
      mt = pair_max(mt);
      if (__any(mt > raise_at)) {
        const float mn = fmaxf(m, mt * c);
        const float alpha = (mn == -INFINITY) ? 1.0f : exp2f(m - mn);   // m = -inf gives 0
        m = mn;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        msub = (m == -INFINITY) ? 0.0f : m;
        raise_at = (m + kRescaleSlack) * inv_c;
      }
    };
    // Numerators of a tile (bf16, for the product) and their sum (fp32).
    auto numerators = [&](const f32x16& s, bf16x8 (&pb)[2]) {
      float ps[4];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // v_exp_f32 directly: arguments are <= 2^3 above the running max and
        // results below the fp32 normal range are flushed, which bf16 P and the
        // fp32 sums tolerate
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], c, -msub));
        ps[r & 3] = r < 4 ? pr : ps[r & 3] + pr;
        pb[r >> 3][r & 7] = static_cast<__bf16>(pr);
      }
      l += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    };

    // ---- prologue: K of tiles 0-2 and V of tile 0 in LDS, S^T of tile 0 ----
    const uint32_t koff = tile_load_offset<D, Swz::K>(wave, lane);
    const uint32_t voff = tile_load_offset<D, Swz::V>(wave, lane);
    batch_cur = lay.prep(a, load_batch(0));
    batch_nxt = load_batch(1);
    const TileRef t0 = tile(0);
    TileRef t_next = tile(1);
    TileRef t_after = tile(2);
    issue_tile_load<D>(K + t0.off, k_slot0, koff, wave, t0.rows, t0.cols);
    issue_tile_load<D>(V + t0.off, v_slot0, voff, wave, t0.rows, t0.cols);
    issue_tile_load<D>(K + t_next.off, k_slot1, koff, wave, t_next.rows, t_next.cols);
    issue_tile_load<D>(K + t_after.off, k_slot2, koff, wave, t_after.rows,
                       t_after.cols);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 s_cur = scores(k_slot0);
    stats(s_cur, t0);
    __syncthreads();            // tile 0's K slot is refilled next

    // tile e: K of e+1 is in k_slot[(e+1)%3], K of e+2 in k_slot[(e+2)%3] or
    // still arriving, V of e in v_slot[e%2]; V of e+1 streams into
    // v_slot[(e+1)%2] and K of e+3 into k_slot[e%3]. The statistics of tile
    // e are in m.
    auto body = [&](int e, auto parity, auto phase) {
      constexpr int kOdd = decltype(parity)::value;
      constexpr int kPh = decltype(phase)::value;
      u32x4* const k_fill = kPh == 0 ? k_slot0 : (kPh == 1 ? k_slot1 : k_slot2);   // e % 3
      u32x4* const k_next = kPh == 0 ? k_slot1 : (kPh == 1 ? k_slot2 : k_slot0);   // (e + 1) % 3
      u32x4* const v_here = kOdd ? v_slot1 : v_slot0;    // slot e % 2
      u32x4* const v_fill = kOdd ? v_slot0 : v_slot1;    // slot (e + 1) % 2
      if (((e + 3) & 63) == 0 && e + 3 < cnt) {   // entry e + 3 opens the next batch
        batch_cur = lay.prep(a, batch_nxt);
        batch_nxt = load_batch(((e + 3) >> 6) + 1);
      }
      const TileRef t3 = tile(e + 3);
      // V of e+1 first: the tile barrier waits for it but not for K of e+3.
      // Both slots were last read before the previous barrier. The copies
      // stay at the top of the tile, outside the interleaved stretch below.
      issue_tile_load<D>(V + t_next.off, v_fill, voff, wave, t_next.rows, t_next.cols);
      issue_tile_load<D>(K + t3.off, k_fill, koff, wave, t3.rows, t3.cols);
      __builtin_amdgcn_sched_barrier(0);

      // V^T fragments of tile e (16 transposing reads)
      bf16x8 vf[kDT][2];
      auto read_v = [&]() {
        const uint16_t* sv = reinterpret_cast<const uint16_t*>(v_here);
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const uint16_t* p = sv + vaddr[dt] + 16 * st * D;
            const s16x4 both[2] = {read_v_transposed(p), read_v_transposed(p + 8 * D)};
            __builtin_memcpy(&vf[dt][st], both, sizeof(bf16x8));
          }
      };
      // S^T of tile e+1 on the matrix cores, the V^T reads of tile e and the
      // numerators of tile e beside the products.
      f32x16 s_nxt = scores(k_next);
      read_v();
      bf16x8 pb[2];
      numerators(s_cur, pb);
      asm volatile("" : "+v"(l));   // the sum stays beside the products

      // ---- O^T += V^T P^T over this wave's 32 keys --------------------------
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int st = 0; st < 2; ++st)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt][st], pb[st], o[dt], 0, 0, 0);
      // Order for the scheduler: the S^T products interleaved with the K and
      // V reads and the exponentials, then the P.V products interleaved with
      // the conversions and sums (masks: 0x100 LDS read, 0x8 matrix, 0x402
      // vector incl. transcendental).
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < kKS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 32 / kKS, 0);
      }
#pragma unroll
      for (int i = 0; i < 2 * kDT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 24 / (2 * kDT), 0);
      }

      // statistics of tile e+1 (past the end of the list a repeat of tile e,
      // which changes nothing)
      stats(s_nxt, t_next);
      s_cur = s_nxt;
      t_next = t_after;
      t_after = t3;
      // Every load but the newest tile copy (K of e+3) has landed: K of e+2
      // and V of e+1 are in LDS for every wave after the barrier. The
      // scheduling barrier keeps the wait after this tile's work; the empty
      // asm statements keep the compiler from moving LDS accesses across it.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitAllButOneTile<D>());
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    // Unrolled by six (three K slots, two V slots); each body is entered only
    // from the one before it, so the compiler's wait bookkeeping follows the
    // ring exactly.
    for (int e = 0;;) {
      body(e, I0{}, I0{});
      if (++e >= cnt) break;
      body(e, I1{}, I1{});
      if (++e >= cnt) break;
      body(e, I0{}, I2{});
      if (++e >= cnt) break;
      body(e, I1{}, I0{});
      if (++e >= cnt) break;
      body(e, I0{}, I1{});
      if (++e >= cnt) break;
      body(e, I1{}, I2{});
      if (++e >= cnt) break;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);    // the last tile copies land before the slots are reused
  __syncthreads();

  // ---- merge the two key halves of every query row -----------------------
  l += __shfl_xor(l, 32);       // both lanes of a row hold the same m
  // lane-major partials of query half wq: element j of lane x at part[j * 64 + x]
  float* const part = reinterpret_cast<float*>(wq ? k_slot1 : k_slot0);
  static_assert(S::kTile * 16 >= kDT * 16 * 64 * 4, "merge area");
  if (wk == 1) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[(dt * 16 + r) * 64 + lane] = o[dt][r];
    merge_ml[wq * 64 + lane] = m;
    merge_ml[(2 + wq) * 64 + lane] = l;
  }
  __syncthreads();
  if (wk == 1) return;
  const float m1 = merge_ml[wq * 64 + lane];
  const float l1 = merge_ml[(2 + wq) * 64 + lane];
  const float mm = fmaxf(m, m1);
  const float a0 = (m == -INFINITY) ? 0.0f : exp2f(m - mm);
  const float a1 = (m1 == -INFINITY) ? 0.0f : exp2f(m1 - mm);
  const float lt = l * a0 + l1 * a1;
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  const float w0 = a0 * inv, w1 = a1 * inv;
  if (wq * 32 + li >= w.rows) return;      // rows past a query cluster are not stored
  uint16_t* __restrict__ O = static_cast<uint16_t*>(a.op);
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
      uint2 w;
      w.x = static_cast<uint32_t>(f32_to_bf16_rne(v[0])) |
            (static_cast<uint32_t>(f32_to_bf16_rne(v[1])) << 16);
      w.y = static_cast<uint32_t>(f32_to_bf16_rne(v[2])) |
            (static_cast<uint32_t>(f32_to_bf16_rne(v[3])) << 16);
      *reinterpret_cast<uint2*>(O + qrow * D + d) = w;
    }
  if (a.lse != nullptr && h == 0)
    a.lse[qrow] = lt > 0.0f ? (mm + log2f(lt)) * kLn2 : -INFINITY;
}

}  // namespace

// Period of the clock-phased order per tile, in ticks of the 100 MHz clock:
// about the time one workgroup spends on a kept tile at two workgroups per
// CU (1.24 us at head_dim 128, 720p / 80%). 110-135 ticks give 30.1-30.4 ms
// there; a much faster sweep leaves the workgroups behind it and loses the
// reuse, so the value sits on the slow side of the optimum.
static uint32_t sweep_ticks_for(int D) { return D == 64 ? 90u : 120u; }

void launch_bsa_forward_mfma(const AttnArgs& args, int D, bool phased, hipStream_t stream) {
  const int64_t n = args.BH * args.nb;
  AttnArgs a = args;
  a.sweep_ticks = phased ? sweep_ticks_for(D) : 0u;
  const void* kernel = D == 64 ? reinterpret_cast<const void*>(&bsa_fwd_mfma<64, BlockListLayout>)
                               : reinterpret_cast<const void*>(&bsa_fwd_mfma<128, BlockListLayout>);
  // In list order, workgroups that start together walk the key range
  // together; a launch as large as the device keeps them in step (see
  // launch_bsa_forward).
  const int64_t per = phased ? n : kGenerationsPerLaunch * resident_workgroups(kernel, kThreads, stream);
  // one launch over every head: XCDs share heads so that the heads in flight
  // fit the last-level cache
  a.xcd_group = phased ? xcd_group_for(a.BH, a.nb, a.N, D) : 0;
  launch_in_generations(n, per, [&](int64_t first, int64_t count) {
    a.item0 = first;
    const unsigned grid = static_cast<unsigned>(count);
    if (D == 64)
      hipLaunchKernelGGL((bsa_fwd_mfma<64, BlockListLayout>), dim3(grid), dim3(kThreads), 0, stream,
                         a, BlockListLayout{}, count);
    else
      hipLaunchKernelGGL((bsa_fwd_mfma<128, BlockListLayout>), dim3(grid), dim3(kThreads), 0,
                         stream, a, BlockListLayout{}, count);
  });
}

void launch_bsa_forward_subset_mfma(const AttnArgs& args, int D, bool phased,
                                    const int32_t* q_blocks, int64_t n, hipStream_t stream) {
  AttnArgs a = args;
  a.sweep_ticks = phased ? sweep_ticks_for(D) : 0u;
  SubsetLayout lay{};
  lay.items = q_blocks;
  lay.total = a.BH * a.nb;
  const unsigned grid = static_cast<unsigned>(n);
  if (D == 64)
    hipLaunchKernelGGL((bsa_fwd_mfma<64, SubsetLayout>), dim3(grid), dim3(kThreads), 0, stream, a,
                       lay, n);
  else
    hipLaunchKernelGGL((bsa_fwd_mfma<128, SubsetLayout>), dim3(grid), dim3(kThreads), 0, stream, a,
                       lay, n);
}

void launch_cluster_attention_mfma(const AttnArgs& args, int D, const int32_t* tiles, int max_tiles,
                                   const int32_t* q_off, int cq, const int32_t* chunk_count,
                                   const int32_t* chunks, int cap, hipStream_t stream) {
  ClusterLayout lay{tiles, max_tiles, q_off, cq, chunk_count, chunks, cap};
  AttnArgs a = args;
  const int64_t n = a.BH * max_tiles;
  // XCDs share heads so that the heads in flight keep their (gathered) K and
  // V in the last-level cache, as in the block-list forward
  a.xcd_group = xcd_group_for(a.BH, max_tiles, a.N, D);
  const unsigned grid = static_cast<unsigned>(n);
  if (D == 64)
    hipLaunchKernelGGL((bsa_fwd_mfma<64, ClusterLayout>), dim3(grid), dim3(kThreads), 0, stream, a,
                       lay, n);
  else
    hipLaunchKernelGGL((bsa_fwd_mfma<128, ClusterLayout>), dim3(grid), dim3(kThreads), 0, stream,
                       a, lay, n);
}

}  // namespace cabf
