// Block-sparse attention backward on bf16 matrix cores (gradients of the
// forward over the same kept tiles; NABLA summary, closing remarks: the
// sparse attention serves training as well as inference).
//
// For a real query row n of block i with kept key set K(i):
//   P_nm = exp(s q_n.k_m - lse_n), dP_nm = do_n.v_m, D_n = do_n.o_n,
//   dS_nm = P_nm (dP_nm - D_n), dq_n = s sum_m dS_nm k_m,
//   dk_m = s sum_n dS_nm q_n, dv_m = sum_n P_nm do_n.
// (D_n = sum_m P_nm dP_nm because o_n = sum_m P_nm v_m.)
//
//   bwd_rowdot     D = rowsum(dO * O), fp32
//   bwd_dq         one workgroup per query block over its kept key blocks, as
//                  the forward: S^T = K Q^T and dP^T = V dO^T on the matrix
//                  cores (K, V rows from LDS; Q^T, dO^T in registers), then
//                  dQ^T += K^T dS^T with K^T from transposing LDS reads
//   bwd_transpose  the kept lists turned around: for every key block, the
//                  query blocks that keep it, ascending (through a bitmap)
//   bwd_order      the key blocks of each head by the length of those lists,
//                  longest first (counting sort): the dK/dV pass runs them in
//                  that order, so workgroups side by side walk lists of about
//                  the same length
//   bwd_dkv        one workgroup of two four-wave groups per key block over
//                  those query blocks, both groups on the same Q and dO
//                  tiles: the dV group forms S = Q K^T and P, adds dV^T +=
//                  dO^T P and hands P to the dK group through LDS; the dK
//                  group forms dP = dO V^T, then dS = P (dP - D) and dK^T +=
//                  Q^T dS (Q, dO rows from LDS; K or V in registers; dO^T,
//                  Q^T from transposing LDS reads). Holding K, V and both
//                  accumulators in every lane would take over 256 registers;
//                  split over the groups, each wave stays within 256.
// Every gradient kernel splits the 64 x 64 tile over 4 waves (two halves of
// each side) and adds the two partial sums of a row once at the end, so with
// list-order walks (the deterministic flag) every result is reproducible.
// Pad query rows do not contribute and get dq = 0;
// pad key rows get dk = dv = 0.
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

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline float bf16_f(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

// D[row] = sum_d dO[row, d] O[row, d], and lse2[row] = lse[row] * log2(e)
// (+inf where lse is not finite: such a row gets P = 0); 16 threads per row
template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot(const uint16_t* __restrict__ o,
                                                  const uint16_t* __restrict__ dout,
                                                  const float* __restrict__ lse,
                                                  float* __restrict__ delta,
                                                  float* __restrict__ lse2, int64_t rows) {
  constexpr int kPer = D / 16;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  float s = 0.0f;
  if (row < rows) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int64_t e = row * D + sub * kPer + k;
      s = fmaf(bf16_f(o[e]), bf16_f(dout[e]), s);
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (sub == 0 && row < rows) {
    delta[row] = s;
    const float l = lse[row];
    lse2[row] = __builtin_isfinite(l) ? l * kLog2e : INFINITY;
  }
}

// Element offsets (within a 64-row tile in the two-way layout, b_chunk_slot)
// of the transposing reads that give a lane its fragments of X^T (d x rows)
// for rows rbase + 4 (vgrp / 2) + vsl / 4 + 16 st + 8 half and columns
// 32 dt + vcol: off[dt][half] for st = 0; the swizzle repeats every 16 rows,
// so st = 1 is 16 D elements further (kept out of the array, one register
// each less).
template <int D>
__device__ inline void transposed_offsets(int (&off)[D / 32][2], int rbase, int lane) {
  const int vgrp = lane >> 4, vsl = lane & 15;
  const int vcol = 16 * (vgrp & 1) + 4 * (vsl & 3);
  const int vrow = rbase + 4 * (vgrp >> 1) + (vsl >> 2);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int row = vrow + 8 * hf;
      const int col = 32 * dt + vcol;
      off[dt][hf] = b_chunk_slot<D>(row, col >> 3) * 8 + (col & 7);
    }
}

__device__ inline bf16x8 transposed_fragment(const uint16_t* tile, int off_lo, int off_hi) {
  const s16x4 both[2] = {read_v_transposed(tile + off_lo), read_v_transposed(tile + off_hi)};
  bf16x8 a;
  __builtin_memcpy(&a, both, sizeof(a));
  return a;
}

// Loads the D-wide rows of one 64-row tile of `a` and `b` (K/V, or Q/dO) into
// an LDS slot each, in the two-way layout (read by rows and transposed
// without bank conflicts).
template <int D>
__device__ __forceinline__ void load_pair(const uint16_t* a, const uint16_t* b, u32x4* sa, u32x4* sb,
                                          uint32_t off, int wave, int real_rows = kBlock,
                                          int real_cols = kP) {
  issue_tile_load<D, kThreads, Copy::Asm>(a, sa, off, wave, real_rows, real_cols);
  issue_tile_load<D, kThreads, Copy::Asm>(b, sb, off, wave, real_rows, real_cols);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per query block. Wave (wq, wk): query half wq, key half
// wk of every tile; lane holds query row li of its half (as in the forward).
// Software-pipelined by one tile: in tile e the matrix cores run S^T and dP^T
// of tile e + 1 and then dQ^T += K^T dS^T of tile e (dS of e formed in tile
// e - 1), and the vector units form dS of e + 1 while the dQ products run.
// K therefore stays in LDS for two tiles: three K slots, two V slots (80 KB
// at d = 128, two workgroups per CU); K and V of e + 2 stream in during tile
// e. Every product and dS value is the same as in a pass without the skew
// (bit-identical gradients); at 720p / 80% the backward took 99.2-99.5 ms
// against 100.5 ms without the skew in list order, and 100.0-100.4 against
// 100.1-100.6 ms clock-phased (one box, interleaved runs).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq(AttnArgs a, const uint16_t* __restrict__ dop,
                                                      const float* __restrict__ delta,
                                                      const float* __restrict__ lse2g,
                                                      uint16_t* __restrict__ dqp, int64_t n_items) {
  using S = Stage<D>;
  constexpr int kKS = D / 16;
  constexpr int kDT = D / 32;
  // One LDS array for the ring (K slots 0-2, V slots 3-4): a slot is a
  // constant offset from one base, which the reads take as their immediate
  // offset, so one address register per lane offset serves every slot (with
  // separate arrays the compiler kept an address per slot and spilled). The
  // copies are asm statements the compiler does not see, so it does not wait
  // for them where a read might alias a slot being filled.
  __shared__ u32x4 ring[5][S::kTile];
  u32x4* const k_slot0 = ring[0];
  u32x4* const k_slot1 = ring[1];
  u32x4* const k_slot2 = ring[2];
  u32x4* const v_slot0 = ring[3];
  u32x4* const v_slot1 = ring[4];
  // the start position borrows K slot 2, which the first copy into it
  // (tile 0) finds read
  int* const start_shared = reinterpret_cast<int*>(k_slot2);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave & 1, wk = wave >> 1;
  const int li = lane & 31, h = lane >> 5;
  const int64_t item = a.item0 + xcd_head_order(blockIdx.x, n_items, a.nb, a.xcd_group, true);
  const int64_t bh = item / a.nb;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.qp);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.kp) + bh * a.N * D;
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.vp) + bh * a.N * D;
  const int64_t qrow = item * kBlock + wq * 32 + li;

  bf16x8 qf[kKS], df[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Q + qrow * D + 16 * ks + 8 * h));
    df[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(dop + qrow * D + 16 * ks + 8 * h));
  }
  // +inf for a row without keys (lse = -inf): P = exp2(x - inf) = 0 everywhere
  const float lse2 = lse2g[qrow];
  const float dlt = delta[qrow];
  const float c = a.scale_log2;
  f32x16 acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;

  const int cnt = min(max(a.kv_count[item], 0), a.nb);
  const int32_t* __restrict__ list = a.kv_index + item * a.nb;
  const int key0 = 32 * wk;
  int toff[kDT][2];
  transposed_offsets<D>(toff, key0, lane);
  // first list entry of the pass (0, or clock-phased: see clock_phased_start)
  if (wave == 0) {
    const int st = clock_phased_start(a.kv_count + bh * a.nb, list, a.nb, cnt, a.sweep_ticks,
                                      lane);
    if (lane == 0) *start_shared = st;
  }
  __syncthreads();
  const int start = __builtin_amdgcn_readfirstlane(*start_shared);
  // List entries are fetched 64 at a time, one per lane, a batch ahead of
  // use, and read out with readlane (as in the forward): no list load is
  // waited on per tile. Entry t of the pass is list entry start + t
  // (wrapped); t is clamped to the last one.
  // Entries are packed with their extents (pack_block_entry) when their
  // batch comes into use, not right after the load (which would wait for
  // it, and with it for every tile copy issued before it).
  auto load_batch = [&](int b) {
    int pos = min(b * 64 + lane, cnt - 1) + start;
    pos -= pos >= cnt ? cnt : 0;
    return list[pos];
  };
  uint32_t batch_cur = 0;    // entries 64 B .. of the pass, packed
  int32_t batch_nxt = 0;     // entries 64 (B + 1) .., as loaded
  auto tile_of = [&](int t) {
    const int p = t < cnt ? t : cnt - 1;
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(batch_cur, p & 63));
  };
  // first element of key block `p` (block 0 for an invalid entry, which is masked) and
  // the rows of it that can hold real keys
  auto tile_off = [&](uint32_t p) {
    return static_cast<int64_t>(p != 0u ? packed_block(p) : 0) * kBlock * D;
  };
  auto tile_rows = [&](uint32_t p) { return 8 * packed_extent(p).vy; };
  auto tile_cols = [&](uint32_t p) { return packed_extent(p).vx; };
  // S^T or dP^T of this wave's 32 keys: rows of `tile` against fragments f
  auto rows_times = [&](const u32x4* tile, const bf16x8 (&f)[kKS]) {
    f32x16 r;
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const u32x4 u = tile[b_chunk_slot<D>(key0 + li, 2 * ks + h)];
      r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), f[ks], r, 0, 0, 0);
    }
    return r;
  };
  // dS^T = P (dP - D) in bf16 of a tile whose S^T and dP^T are in s, dp;
  // pad keys of a partial patch (a uniform branch) get S = -inf, hence P =
  // dS = 0
  auto form_ds = [&](f32x16 s, const f32x16& dp, uint32_t pe, bf16x8 (&dsb)[2]) {
    const BlockExtent ext = packed_extent(pe);
    if (!ext.full()) {
      const uint32_t bits = real_accumulator_bits(ext, wk, h);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = ((bits >> r) & 1u) ? s[r] : -INFINITY;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lse2));
      dsb[r >> 3][r & 7] = static_cast<__bf16>(pr * (dp[r] - dlt));
    }
  };
  // dQ^T += K^T dS^T with K^T from transposing reads of the K tile `ks_`
  auto dq_products = [&](const u32x4* ks_, const bf16x8 (&dsb)[2]) {
    const uint16_t* kt = reinterpret_cast<const uint16_t*>(ks_);
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int st = 0; st < 2; ++st)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            transposed_fragment(kt + 16 * st * D, toff[dt][0], toff[dt][1]), dsb[st], acc[dt], 0, 0, 0);
  };

  if (cnt > 0) {
    const uint32_t off = tile_load_offset<D, Swz::B>(wave, lane);
    batch_cur = pack_block_entry(a, load_batch(0));
    batch_nxt = load_batch(1);
    uint32_t jb_cur = tile_of(0);    // tile e
    uint32_t jb_n1 = tile_of(1);     // tile e + 1
    load_pair<D>(K + tile_off(jb_cur), V + tile_off(jb_cur), k_slot0, v_slot0, off, wave,
                 tile_rows(jb_cur), tile_cols(jb_cur));
    if (cnt > 1)
      load_pair<D>(K + tile_off(jb_n1), V + tile_off(jb_n1), k_slot1, v_slot1, off, wave,
                   tile_rows(jb_n1), tile_cols(jb_n1));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    bf16x8 dsb[2];   // dS^T of tile e
    form_ds(rows_times(k_slot0, qf), rows_times(v_slot0, df), jb_cur, dsb);
    __syncthreads();   // V slot 0 is refilled in tile 0
    // tile e: K of e in k_slot[e % 3], K and V of e + 1 in k_slot[(e + 1) % 3]
    // and v_slot[(e + 1) % 2]; K and V of e + 2 stream into k_slot[(e + 2) %
    // 3] and v_slot[e % 2], last read in tile e - 1.
    auto body = [&](int e, auto parity, auto phase) {
      constexpr int kOdd = decltype(parity)::value;
      constexpr int kPh = decltype(phase)::value;
      u32x4* const k_here = kPh == 0 ? k_slot0 : (kPh == 1 ? k_slot1 : k_slot2);   // e % 3
      u32x4* const k_next = kPh == 0 ? k_slot1 : (kPh == 1 ? k_slot2 : k_slot0);   // (e + 1) % 3
      u32x4* const k_fill = kPh == 0 ? k_slot2 : (kPh == 1 ? k_slot0 : k_slot1);   // (e + 2) % 3
      u32x4* const v_next = kOdd ? v_slot0 : v_slot1;    // (e + 1) % 2
      u32x4* const v_fill = kOdd ? v_slot1 : v_slot0;    // e % 2
      if (((e + 2) & 63) == 0 && e + 2 < cnt) {   // entry e + 2 opens the next batch
        batch_cur = pack_block_entry(a, batch_nxt);
        batch_nxt = load_batch(((e + 2) >> 6) + 1);
      }
      const uint32_t jb_n2 = tile_of(e + 2);
      if (e + 2 < cnt)
        load_pair<D>(K + tile_off(jb_n2), V + tile_off(jb_n2), k_fill, v_fill, off, wave,
                     tile_rows(jb_n2), tile_cols(jb_n2));
      __builtin_amdgcn_sched_barrier(0);
      // past the end of the list the products of tile e + 1 read a stale
      // slot; their results are not used
      const f32x16 s = rows_times(k_next, qf);
      const f32x16 dp = rows_times(v_next, df);
      dq_products(k_here, dsb);
      form_ds(s, dp, jb_n1, dsb);
      jb_n1 = jb_n2;
      // Every copy has landed: K and V of e + 2 are in LDS for every wave
      // after the barrier. The scheduling barrier keeps the wait after this
      // tile's work; the empty asm statements keep the compiler from moving
      // LDS accesses across the barrier.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    // unrolled by six (three K slots, two V slots) with a guard per body (a
    // chain of bodies joined by breaks moved the accumulators between
    // register sets and spilled)
    for (int e = 0; e < cnt; e += 6) {
      body(e, I0{}, I0{});
      if (e + 1 < cnt) body(e + 1, I1{}, I1{});
      if (e + 2 < cnt) body(e + 2, I0{}, I2{});
      if (e + 3 < cnt) body(e + 3, I1{}, I0{});
      if (e + 4 < cnt) body(e + 4, I0{}, I1{});
      if (e + 5 < cnt) body(e + 5, I1{}, I2{});
    }
  }

  // ---- add the two key halves, scale, store (pad query rows: 0) ------------
  float* const part = reinterpret_cast<float*>(wq ? k_slot1 : k_slot0);
  static_assert(S::kTile * 16 >= kDT * 16 * 64 * 4, "merge area");
  if (wk == 1) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[(dt * 16 + r) * 64 + lane] = acc[dt][r];
  }
  __syncthreads();
  if (wk == 1) return;
  const BlockExtent qext = block_extent(static_cast<int>(item % a.nb), a);
  const int rloc = wq * 32 + li;
  const bool real_row = qext.real(rloc);
  const float sc = real_row ? a.scale_log2 * kLn2 : 0.0f;   // the softmax scale s
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * h;
      float v[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 4 * g + x;
        v[x] = (acc[dt][r] + part[(dt * 16 + r) * 64 + lane]) * sc;
      }
      uint2 w;
      w.x = static_cast<uint32_t>(f32_to_bf16_rne(v[0])) |
            (static_cast<uint32_t>(f32_to_bf16_rne(v[1])) << 16);
      w.y = static_cast<uint32_t>(f32_to_bf16_rne(v[2])) |
            (static_cast<uint32_t>(f32_to_bf16_rne(v[3])) << 16);
      *reinterpret_cast<uint2*>(dqp + qrow * D + d) = w;
    }
}

// ---------------------------------------------------------------------------
// Transposed lists: bit (i, j) set when query block i keeps key block j.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_fill_zero(uint32_t* __restrict__ p, int64_t words) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e < words) p[e] = 0u;
}

// One wave per row (bh, query block i) over its list, 64 entries at a time.
// The list ascends, so entries in the same 32-bit word sit in consecutive
// lanes: an OR scan within each such run leaves the run's word in its last
// lane, which alone writes it (atomically: a word can span two batches).
__global__ __launch_bounds__(256) void bwd_bitmap(const int32_t* __restrict__ kv_count,
                                                  const int32_t* __restrict__ kv_index,
                                                  uint32_t* __restrict__ bitmap, int nb, int words,
                                                  int64_t rows /* BH * nb */) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int cnt = min(max(kv_count[row], 0), nb);
  const int32_t* lst = kv_index + row * nb;
  uint32_t* bm = bitmap + row * words;
  for (int t0 = 0; t0 < cnt; t0 += 64) {
    const int t = t0 + lane;
    const int j = t < cnt ? lst[t] : -1;
    const bool on = static_cast<unsigned>(j) < static_cast<unsigned>(nb);
    const int wd = on ? (j >> 5) : -1 - lane;     // lanes without an entry form runs of their own
    uint32_t bits = on ? 1u << (j & 31) : 0u;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const uint32_t b = __shfl_up(bits, sh);
      const int w = __shfl_up(wd, sh);
      bits |= (lane >= sh && w == wd) ? b : 0u;
    }
    const int next = __shfl_down(wd, 1);
    if (on && (lane == 63 || next != wd)) atomicOr(bm + wd, bits);
  }
}

// One wave per (bh, word column c): key blocks j = 32 c .. 32 c + 31. Each
// lane reads the word of query block i (64 at a time), which holds bits
// (i, j) for all 32 of them, so every word is read once; per key block a
// ballot over the lanes gives the kept query blocks of this batch in
// ascending order, appended to j's list. Lane b keeps the count of key
// block 32 c + b.
__global__ __launch_bounds__(256) void bwd_transpose(const uint32_t* __restrict__ bitmap,
                                                     int32_t* __restrict__ q_count,
                                                     int32_t* __restrict__ q_index, int nb,
                                                     int words, int64_t cols /* BH * words */) {
  const int lane = threadIdx.x & 63;
  const int64_t col = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (col >= cols) return;
  const int64_t bh = col / words;
  const int c = static_cast<int>(col - bh * words);
  const uint32_t* bm = bitmap + bh * nb * static_cast<int64_t>(words) + c;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int jn = min(32, nb - 32 * c);          // key blocks in this column
  int count = 0;                                // lane b < jn: count of key block 32 c + b
  for (int base = 0; base < nb; base += 64) {
    const int i = base + lane;
    const uint32_t wv = i < nb ? bm[static_cast<int64_t>(i) * words] : 0u;
    for (int b = 0; b < jn; ++b) {
      const bool keep = (wv >> b) & 1u;
      const uint64_t m = __ballot(keep);
      if (m == 0) continue;
      const int before = __shfl(count, b);      // key block 32 c + b's count so far
      const int64_t row = bh * nb + 32 * c + b;
      if (keep) q_index[row * nb + before + __popcll(m & lt)] = i;
      count += lane == b ? __popcll(m) : 0;
    }
  }
  if (lane < jn) q_count[bh * nb + 32 * c + lane] = count;
}

// Key blocks of each (batch, head) ordered by the length of their transposed
// lists, longest first, equal lengths by index: k_order[bh * nb + r] is the
// r-th. A stable counting sort in one workgroup per (batch, head), nb <=
// kMaxBlocks (the histogram lives in LDS).
__global__ __launch_bounds__(256) void bwd_order(const int32_t* __restrict__ q_count,
                                                 int32_t* __restrict__ k_order, int nb) {
  __shared__ int hist[kMaxBlocks + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * nb;
  auto key_of = [&](int j) { return nb - min(max(q_count[base + j], 0), nb); };   // 0: longest
  for (int i = tid; i <= nb; i += 256) hist[i] = 0;
  __syncthreads();
  for (int j = tid; j < nb; j += 256) atomicAdd(&hist[key_of(j)], 1);
  __syncthreads();
  if (tid < 64) {
    // exclusive scan of hist[0 .. nb]: each lane sums a run of bins, the
    // wave scans the run totals, each lane then writes its run's offsets
    const int per = (nb + 1 + 63) / 64;
    const int lo = min(lane * per, nb + 1), hi = min(lo + per, nb + 1);
    int run = 0;
    for (int i = lo; i < hi; ++i) run += hist[i];
    int incl = run;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int o = __shfl_up(incl, sh);
      incl += lane >= sh ? o : 0;
    }
    int off = incl - run;
    for (int i = lo; i < hi; ++i) {
      const int c = hist[i];
      hist[i] = off;
      off += c;
    }
    // stable scatter, 64 key blocks at a time in index order: a lane's place
    // is its key's next free slot plus the lanes before it with the same key
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int j0 = 0; j0 < nb; j0 += 64) {
      const int j = j0 + lane;
      const bool on = j < nb;
      const int key = on ? key_of(j) : -1;
      uint64_t same = __ballot(on);
      for (int bit = 0; (1 << bit) <= nb; ++bit) {
        const uint64_t b = __ballot(on && ((key >> bit) & 1));
        same &= ((key >> bit) & 1) ? b : ~b;
      }
      const int rank = __popcll(same & lt);
      const int pos = on ? hist[key] + rank : 0;
      if (on) k_order[base + pos] = j;
      if (on && rank == __popcll(same) - 1) hist[key] = pos + 1;
    }
  }
}

// ---------------------------------------------------------------------------
// dK and dV in one pass: one workgroup of eight waves per key block over the
// query blocks that keep it. Waves 0-3 form the dV group, waves 4-7 the dK
// group; in each group wave (wk, wq) takes key half wk and query half wq of
// every tile, lane li holding key li of its half, so waves w and w + 4 hold
// the same elements of a tile and share a SIMD. Both groups read the same Q
// and dO tiles, so a kept tile crosses the memory system once for both
// gradients (the dV group copies Q, the dK group dO).
// The softmax weights are formed once: per tile e the dV group forms S = Q
// K^T and P, adds dV^T += dO^T P, and leaves P (fp32) in LDS; the dK group
// forms dP = dO V^T and keeps dP - D, and in the next tile, once the barrier
// has made P visible, forms dS = P (dP - D) of tile e and adds dK^T += Q^T dS
// with tile e's Q, still in its ring. The products of dS therefore run one
// tile behind, and the dK group's dS work overlaps its own dP products of the
// next tile. Rings: Q in four slots, copied two tiles ahead (kept one tile
// after use); dO, P, lse and D in two, copied one tile ahead (dO two tiles
// ahead as well was slower: 77 against 67 ms at 720p / 80%). Computing P once
// instead of in both groups, and the deeper Q ring, took the pass from 74 to
// 67 ms there.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(2 * kThreads, 1) void bwd_dkv(AttnArgs a, const uint16_t* __restrict__ dop,
                                                           const float* __restrict__ delta,
                                                           const float* __restrict__ lse2,
                                                           const int32_t* __restrict__ q_count,
                                                           const int32_t* __restrict__ q_index,
                                                           const int32_t* __restrict__ k_order,
                                                           uint16_t* __restrict__ dkp,
                                                           uint16_t* __restrict__ dvp, int64_t n_items) {
  using S = Stage<D>;
  constexpr int kKS = D / 16;
  constexpr int kDT = D / 32;
  __shared__ u32x4 q_slot[4][S::kTile];
  __shared__ u32x4 d_slot[2][S::kTile];
  // lse2 and D of a query block, [lse2, D][4 rows], in two slots
  __shared__ f32x4 vec_slot0[2][kBlock / 4], vec_slot1[2][kBlock / 4];
  __shared__ f32x4 p_slot[2][4][4][64];          // [slot][wave of the group][r / 4][lane]: P, fp32
  __shared__ int start_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;                                // 0: dV group, 1: dK group
  const int w = wave & 3;                                   // wave within the group
  const int wk = w & 1, wq = w >> 1;
  const int li = lane & 31, h = lane >> 5;
  // bh * nb + key block j; with k_order, slot r of a head runs its r-th
  // longest transposed list
  const int64_t slot = a.item0 + xcd_head_order(blockIdx.x, n_items, a.nb, a.xcd_group, true);
  const int64_t bh = slot / a.nb;
  const int64_t item =
      k_order != nullptr ? bh * a.nb + min(max(k_order[slot], 0), a.nb - 1) : slot;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.qp) + bh * a.N * D;
  const uint16_t* __restrict__ dO = dop + bh * a.N * D;
  const float* __restrict__ lse_h = lse2 + bh * a.N;
  const float* __restrict__ dl_h = delta + bh * a.N;
  const int64_t krow = item * kBlock + wk * 32 + li;        // global key row of this lane
  const float c = a.scale_log2;
  f32x16 acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;

  const int cnt = min(max(q_count[item], 0), a.nb);
  const int32_t* __restrict__ list = q_index + item * a.nb;
  const int row0 = 32 * wq;                                 // first query row of this wave's half
  int toff[kDT][2];
  transposed_offsets<D>(toff, row0, lane);
  // first list entry of the pass (0, or clock-phased: see clock_phased_start)
  if (wave == 0) {
    const int st = clock_phased_start(q_count + bh * a.nb, list, a.nb, cnt, a.sweep_ticks, lane);
    if (lane == 0) start_sh = st;
  }
  __syncthreads();
  const int start = __builtin_amdgcn_readfirstlane(start_sh);
  // list entries, 64 at a time a batch ahead (as in the forward), packed
  // with their extents when their batch comes into use; entry t of the pass
  // is list entry start + t (wrapped), t clamped to the last one
  auto load_batch = [&](int b) {
    int pos = min(b * 64 + lane, cnt - 1) + start;
    pos -= pos >= cnt ? cnt : 0;
    return list[pos];
  };
  uint32_t batch_cur = 0;    // packed
  int32_t batch_nxt = 0;     // as loaded
  auto entry = [&](int t) {
    const int p = t < cnt ? t : cnt - 1;
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(batch_cur, p & 63));
  };
  // rows and patch columns that can hold real queries
  auto rows = [&](uint32_t p) { return 8 * packed_extent(p).vy; };
  auto cols = [&](uint32_t p) { return packed_extent(p).vx; };
  // S or dP of this wave's 32 queries x 32 keys: rows of `tile` against f
  auto rows_times = [&](const u32x4* tile, const bf16x8 (&f)[kKS]) {
    f32x16 r;
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const u32x4 u = tile[b_chunk_slot<D>(row0 + li, 2 * ks + h)];
      r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), f[ks], r, 0, 0, 0);
    }
    return r;
  };
  // acc^T += X^T W with X^T from transposing reads of the tile `xs` (dO for
  // the dV group, Q for the dK group)
  auto accumulate = [&](const u32x4* xs, const bf16x8 (&wb)[2]) {
    const uint16_t* xt = reinterpret_cast<const uint16_t*>(xs);
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int st = 0; st < 2; ++st)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            transposed_fragment(xt + 16 * st * D, toff[dt][0], toff[dt][1]), wb[st], acc[dt], 0, 0, 0);
  };
  // lse2 and D of query block pe -> vec slot, copied straight into LDS by
  // wave 0 (one dword per lane) ahead of its Q copy, so the tile's wait
  // covers them and no register waits on them.
  auto copy_vecs = [&](uint32_t pe, f32x4 (&vec)[2][kBlock / 4]) {
    if (wave == 0) {
      const int64_t r0 = static_cast<int64_t>(packed_block(pe)) * kBlock;
      lds_copy_x1_asm(lse_h + r0, 4 * lane, vec[0]);
      lds_copy_x1_asm(dl_h + r0, 4 * lane, vec[1]);
    }
  };
  const uint32_t off = tile_load_offset<D, Swz::B>(w, lane);
  // The two groups run the same tile loop, instantiated once per group, and
  // pass the same barriers.
  auto run = [&](auto group) {
    constexpr int kDk = decltype(group)::value;
    // this group's share of the copies of query block pe: Q (dV group) or
    // dO (dK group)
    auto copy_tile = [&](uint32_t pe, u32x4* qs, u32x4* ds) {
      const int64_t r0 = static_cast<int64_t>(packed_block(pe)) * kBlock * D;
      if constexpr (kDk)
        issue_tile_load<D, kThreads, Copy::Asm>(dO + r0, ds, off, w, rows(pe), cols(pe));
      else
        issue_tile_load<D, kThreads, Copy::Asm>(Q + r0, qs, off, w, rows(pe), cols(pe));
    };
    // K (dV group) or V (dK group) rows of this lane's key
    bf16x8 xf[kKS];
    {
      const uint16_t* src = static_cast<const uint16_t*>(kDk ? a.vp : a.kp) + krow * D + 8 * h;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        xf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(src + 16 * ks));
    }
    f32x16 dpm;   // dK group: dP - D of the tile before
    if (cnt == 0) return;
    batch_cur = pack_block_entry(a, load_batch(0));
    batch_nxt = load_batch(1);
    uint32_t ib_cur = entry(0), ib_n1 = entry(1);
    copy_vecs(ib_cur, vec_slot0);
    copy_tile(ib_cur, q_slot[0], d_slot[0]);
    if (!kDk && cnt > 1) copy_tile(ib_n1, q_slot[1], nullptr);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // dS = P (dP - D) of the tile before (P from the dV wave of the same
    // elements) in bf16, and dK^T += Q^T dS with that tile's Q
    auto dk_step = [&](const f32x4 (&pt)[4][64], const u32x4* qprev) {
      bf16x8 wb[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 pr = pt[g][lane];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 4 * g + x;
          wb[r >> 3][r & 7] = static_cast<__bf16>(pr[x] * dpm[r]);
        }
      }
      accumulate(qprev, wb);
    };
    // tile e: Q in slot e % 4, dO, P, lse and D in slot e % 2; the copies of
    // Q of e + 2 and of the rest of e + 1 go to the slots after
    auto body = [&](int e, auto pslot) {
      constexpr int PS = decltype(pslot)::value;
      constexpr int PN = PS ^ 1;
      f32x4 (&vec_here)[2][kBlock / 4] = PS ? vec_slot1 : vec_slot0;
      const int QS = e & 3, QB = (e - 1) & 3, Q2 = (e + 2) & 3;
      if (((e + 2) & 63) == 0 && e + 2 < cnt) {   // entry e + 2 opens the next batch
        batch_cur = pack_block_entry(a, batch_nxt);
        batch_nxt = load_batch(((e + 2) >> 6) + 1);
      }
      const uint32_t ib_next = ib_n1;
      const uint32_t ib_n2 = entry(e + 2);
      if (e + 1 < cnt) {
        copy_vecs(ib_next, PN ? vec_slot1 : vec_slot0);
        if constexpr (kDk) copy_tile(ib_next, nullptr, d_slot[PN]);
      }
      if constexpr (!kDk) {
        if (e + 2 < cnt) copy_tile(ib_n2, q_slot[Q2], nullptr);
      }
      ib_n1 = ib_n2;
      if constexpr (kDk) {
        const f32x16 dp = rows_times(d_slot[PS], xf);
        if (e > 0) dk_step(p_slot[PN][w], q_slot[QB]);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 dv4 = vec_here[1][(row0 >> 2) + 2 * g + h];   // rows row0 + 8 g + 4 h ..
#pragma unroll
          for (int x = 0; x < 4; ++x) dpm[4 * g + x] = dp[4 * g + x] - dv4[x];
        }
      } else {
        f32x16 s = rows_times(q_slot[QS], xf);
        f32x4 lv[4];   // lse2 of this wave's rows, read before the branch below
#pragma unroll
        for (int g = 0; g < 4; ++g) lv[g] = vec_here[0][(row0 >> 2) + 2 * g + h];   // rows row0 + 8 g + 4 h ..
        // pad query rows (partial patches only: a uniform branch) get S =
        // -inf, hence P = dS = 0
        const BlockExtent ext = packed_extent(ib_cur);
        if (!ext.full()) {
          const uint32_t bits = real_accumulator_bits(ext, wq, h);
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = ((bits >> r) & 1u) ? s[r] : -INFINITY;
        }
        bf16x8 wb[2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 pr;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            pr[x] = __builtin_amdgcn_exp2f(fmaf(s[4 * g + x], c, -lv[g][x]));
            wb[(4 * g + x) >> 3][(4 * g + x) & 7] = static_cast<__bf16>(pr[x]);
          }
          p_slot[PS][w][g][lane] = pr;
        }
        accumulate(d_slot[PS], wb);
      }
      ib_cur = ib_next;
      // Every copy and P store has landed, so Q, dO, lse and D of e + 1 and
      // P of e are in LDS for every wave after the barrier. The scheduling
      // barrier keeps the wait after this tile's work; the empty asm
      // statements keep the compiler from moving LDS accesses across the
      // barrier.
      __builtin_amdgcn_sched_barrier(0);
      if (!kDk && e + 2 < cnt)
        __builtin_amdgcn_s_waitcnt(kWaitAllButOneTile<D>());   // Q of e + 2 may stay in flight
      else
        __builtin_amdgcn_s_waitcnt(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    // unrolled by two (the slots other than Q's)
    for (int e = 0;;) {
      body(e, std::integral_constant<int, 0>{});
      if (++e >= cnt) break;
      body(e, std::integral_constant<int, 1>{});
      if (++e >= cnt) break;
    }
    // the dS products of the last tile (its P is visible after the last barrier)
    if constexpr (kDk) dk_step(p_slot[(cnt - 1) & 1][w], q_slot[(cnt - 1) & 3]);
  };
  if (grp == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});
  __syncthreads();   // the last dS products have read their Q slot

  // ---- add the two query halves of each group, store (pad keys: 0) --------
  float* const part = reinterpret_cast<float*>(grp == 0 ? q_slot[wk] : d_slot[wk]);
  static_assert(S::kTile * 16 >= kDT * 16 * 64 * 4, "merge area");
  if (wq == 1) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[(dt * 16 + r) * 64 + lane] = acc[dt][r];
  }
  __syncthreads();
  if (wq == 1) return;
  const BlockExtent kext = block_extent(static_cast<int>(item % a.nb), a);
  const bool real_key = kext.real(wk * 32 + li);
  // dK carries the softmax scale s; pad keys get 0
  const float sc = real_key ? (grp == 0 ? 1.0f : a.scale_log2 * kLn2) : 0.0f;
  uint16_t* const out = grp == 0 ? dvp : dkp;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * h;
      float x[4];
#pragma unroll
      for (int xx = 0; xx < 4; ++xx) {
        const int r = 4 * g + xx;
        x[xx] = (acc[dt][r] + part[(dt * 16 + r) * 64 + lane]) * sc;
      }
      uint2 o2;
      o2.x = static_cast<uint32_t>(f32_to_bf16_rne(x[0])) |
             (static_cast<uint32_t>(f32_to_bf16_rne(x[1])) << 16);
      o2.y = static_cast<uint32_t>(f32_to_bf16_rne(x[2])) |
             (static_cast<uint32_t>(f32_to_bf16_rne(x[3])) << 16);
      *reinterpret_cast<uint2*>(out + krow * D + d) = o2;
    }
}

dim3 grid_for(int64_t work, int per) { return dim3(static_cast<unsigned>((work + per - 1) / per)); }

size_t align256(size_t v) { return (v + 255) & ~size_t{255}; }

}  // namespace

BwdWorkspace bwd_workspace_layout(const Geo& g) {
  BwdWorkspace w{};
  w.words = (g.nb + 31) / 32;
  size_t o = 0;
  w.delta = o;    o += align256(static_cast<size_t>(g.BH) * g.N * sizeof(float));
  w.lse2 = o;     o += align256(static_cast<size_t>(g.BH) * g.N * sizeof(float));
  w.bitmap = o;   o += align256(static_cast<size_t>(g.BH) * g.nb * w.words * sizeof(uint32_t));
  w.q_count = o;  o += align256(static_cast<size_t>(g.BH) * g.nb * sizeof(int32_t));
  w.q_index = o;  o += align256(static_cast<size_t>(g.BH) * g.nb * g.nb * sizeof(int32_t));
  w.k_order = o;  o += align256(static_cast<size_t>(g.BH) * g.nb * sizeof(int32_t));
  w.total = o;
  return w;
}

void launch_bsa_backward(const Geo& g, const void* qp, const void* kp, const void* vp,
                         const void* op, const float* lse, const void* dop,
                         const int32_t* kv_count, const int32_t* kv_index, float scale, void* dqp,
                         void* dkp, void* dvp, void* workspace, bool phased, hipStream_t stream) {
  const BwdWorkspace w = bwd_workspace_layout(g);
  char* ws = static_cast<char*>(workspace);
  float* delta = reinterpret_cast<float*>(ws + w.delta);
  float* lse2 = reinterpret_cast<float*>(ws + w.lse2);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(ws + w.bitmap);
  int32_t* q_count = reinterpret_cast<int32_t*>(ws + w.q_count);
  int32_t* q_index = reinterpret_cast<int32_t*>(ws + w.q_index);
  const int64_t rows = g.BH * g.N;
  const uint16_t* o16 = static_cast<const uint16_t*>(op);
  const uint16_t* do16 = static_cast<const uint16_t*>(dop);
  if (g.D == 64)
    hipLaunchKernelGGL((bwd_rowdot<64>), grid_for(rows, 16), dim3(256), 0, stream, o16, do16, lse,
                       delta, lse2, rows);
  else
    hipLaunchKernelGGL((bwd_rowdot<128>), grid_for(rows, 16), dim3(256), 0, stream, o16, do16, lse,
                       delta, lse2, rows);
  const int64_t words = g.BH * g.nb * w.words;
  hipLaunchKernelGGL(bwd_fill_zero, grid_for(words, 256), dim3(256), 0, stream, bitmap, words);
  hipLaunchKernelGGL(bwd_bitmap, grid_for(g.BH * g.nb, 4), dim3(256), 0, stream, kv_count, kv_index,
                     bitmap, g.nb, w.words, g.BH * g.nb);
  hipLaunchKernelGGL(bwd_transpose, grid_for(g.BH * w.words, 4), dim3(256), 0, stream, bitmap,
                     q_count, q_index, g.nb, w.words, g.BH * w.words);
  // Key blocks by transposed-list length, longest first: the dK/dV pass
  // then runs lists of about the same length side by side (a key block is
  // kept by 57 to 427 query blocks at 720p / 80%), so concurrent workgroups
  // walk the query range at about the same rate, and the longest start first.
  int32_t* k_order = reinterpret_cast<int32_t*>(ws + w.k_order);
  const bool sorted = g.nb <= kMaxBlocks;
  if (sorted)
    hipLaunchKernelGGL(bwd_order, dim3(static_cast<unsigned>(g.BH)), dim3(256), 0, stream, q_count,
                       k_order, g.nb);

  AttnArgs a{};
  a.qp = qp;
  a.kp = kp;
  a.vp = vp;
  a.kv_count = kv_count;
  a.kv_index = kv_index;
  a.lse = nullptr;            // the kernels read lse2
  a.scale_log2 = scale * kLog2e;
  a.nb = g.nb;
  a.Ty = g.Ty;
  a.Tx = g.Tx;
  a.H = g.H;
  a.W = g.W;
  a.N = g.N;
  a.BH = g.BH;
  const int64_t items = g.BH * g.nb;
  uint16_t* dq16 = static_cast<uint16_t*>(dqp);
  uint16_t* dk16 = static_cast<uint16_t*>(dkp);
  uint16_t* dv16 = static_cast<uint16_t*>(dvp);
  // Clock-phased (default): both passes as one launch each, every list
  // started where a sweep of the 100 MHz clock stands (ticks per tile of each
  // pass at d = 128, 720p; d = 64 tiles take about half as long). In list
  // order (bit-reproducible): the dQ pass in launches of a device-full of
  // workgroups, which start together and walk the key range in step (as the
  // forward; uniform list lengths), the dK/dV pass in one launch in the
  // length-sorted order. 720p / 80%, one box: 100.2 ms clock-phased (103.3
  // unsorted), list order ~101 ms (106.9 with both passes as one unsorted
  // launch; generations of the dK/dV pass were slower, 111.7 ms).
  const uint32_t t_dq = phased ? (g.D == 64 ? 95u : 185u) : 0u;
  const uint32_t t_dkv = phased ? (g.D == 64 ? 110u : 220u) : 0u;
  AttnArgs a_dq = a, a_dkv = a;
  a_dq.sweep_ticks = t_dq;
  a_dkv.sweep_ticks = t_dkv;
  // Both passes in one launch share heads between XCDs as the forward does
  // (xcd_group_for), each XCD of a group taking every group-th item: in the
  // dK/dV pass (one launch in both orders) the key blocks of the
  // length-sorted order, so that both XCDs get the same mix of list lengths
  // (720p, whole backward 96.3 against 97.4 ms; contiguous halves, long lists
  // on one XCD and short ones on the other: 108 ms); in the clock-phased dQ
  // pass the query blocks (94.5 against 94.9-95.3 ms; contiguous halves: no
  // change).
  a_dkv.xcd_group = xcd_group_for(g.BH, g.nb, g.N, g.D);
  a_dq.xcd_group = phased ? xcd_group_for(g.BH, g.nb, g.N, g.D) : 0;
  const void* kdq = g.D == 64 ? reinterpret_cast<const void*>(&bwd_dq<64>)
                              : reinterpret_cast<const void*>(&bwd_dq<128>);
  const int64_t per_dq = phased ? items : kGenerationsPerLaunch * resident_workgroups(kdq, kThreads, stream);
  launch_in_generations(items, per_dq, [&](int64_t first, int64_t count) {
    a_dq.item0 = first;
    const unsigned gr = static_cast<unsigned>(count);
    if (g.D == 64)
      hipLaunchKernelGGL((bwd_dq<64>), dim3(gr), dim3(kThreads), 0, stream, a_dq, do16, delta, lse2,
                         dq16, count);
    else
      hipLaunchKernelGGL((bwd_dq<128>), dim3(gr), dim3(kThreads), 0, stream, a_dq, do16, delta, lse2,
                         dq16, count);
  });
  const int32_t* order = sorted ? k_order : nullptr;
  const unsigned grid = static_cast<unsigned>(items);
  if (g.D == 64)
    hipLaunchKernelGGL((bwd_dkv<64>), dim3(grid), dim3(2 * kThreads), 0, stream, a_dkv, do16, delta,
                       lse2, q_count, q_index, order, dk16, dv16, items);
  else
    hipLaunchKernelGGL((bwd_dkv<128>), dim3(grid), dim3(2 * kThreads), 0, stream, a_dkv, do16, delta,
                       lse2, q_count, q_index, order, dk16, dv16, items);
}

}  // namespace cabf
