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
//   bwd_dkv        one workgroup of two four-wave groups per key block over
//                  those query blocks, both groups on the same Q and dO
//                  tiles: the dV group forms S = Q K^T, then dV^T += dO^T P;
//                  the dK group S and dP = dO V^T, then dK^T += Q^T dS (Q, dO
//                  rows from LDS; K, V in registers; dO^T, Q^T from
//                  transposing LDS reads). Holding K, V and both accumulators
//                  in every lane would take over 256 registers; split over
//                  the groups, each wave stays within 256.
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

// Element offsets (within a 64-row K-swizzled tile) of the transposing reads
// that give a lane its fragments of X^T (d x rows) for rows
// rbase + 4 (vgrp / 2) + vsl / 4 + 16 st + 8 half and columns 32 dt + vcol:
// off[dt][half] for st = 0; the K swizzle repeats every 16 rows, so st = 1
// is 16 D elements further (kept out of the array, one register each less).
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
      off[dt][hf] = k_chunk_slot<D>(row, col >> 3) * 8 + (col & 7);
    }
}

__device__ inline bf16x8 transposed_fragment(const uint16_t* tile, int off_lo, int off_hi) {
  const s16x4 both[2] = {read_v_transposed(tile + off_lo), read_v_transposed(tile + off_hi)};
  bf16x8 a;
  __builtin_memcpy(&a, both, sizeof(a));
  return a;
}

// Loads the D-wide rows of one 64-row tile of `a` and `b` (K/V, or Q/dO) into
// a K-swizzled LDS slot each.
template <int D>
__device__ __forceinline__ void load_pair(const uint16_t* a, const uint16_t* b, u32x4* sa, u32x4* sb,
                                          uint32_t off, int wave, int real_rows = kBlock,
                                          int real_cols = kP) {
  issue_tile_load<D>(a, sa, off, wave, real_rows, real_cols);
  issue_tile_load<D>(b, sb, off, wave, real_rows, real_cols);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per query block. Wave (wq, wk): query half wq, key half
// wk of every tile; lane holds query row li of its half (as in the forward).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq(AttnArgs a, const uint16_t* __restrict__ dop,
                                                      const float* __restrict__ delta,
                                                      const float* __restrict__ lse2g,
                                                      uint16_t* __restrict__ dqp, int64_t n_items) {
  using S = Stage<D>;
  constexpr int kKS = D / 16;
  constexpr int kDT = D / 32;
  __shared__ u32x4 k_slot0[S::kTile], k_slot1[S::kTile];
  __shared__ u32x4 v_slot0[S::kTile], v_slot1[S::kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave & 1, wk = wave >> 1;
  const int li = lane & 31, h = lane >> 5;
  const int64_t item = xcd_order(blockIdx.x, n_items);
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
  __shared__ int start_sh;
  if (wave == 0) {
    const int st = clock_phased_start(a.kv_count + bh * a.nb, list, a.nb, cnt, a.sweep_ticks,
                                      lane);
    if (lane == 0) start_sh = st;
  }
  __syncthreads();
  const int start = __builtin_amdgcn_readfirstlane(start_sh);
  // List entries are fetched 64 at a time, one per lane, a batch ahead of
  // use, and read out with readlane (as in the forward): no list load is
  // waited on per tile. Entry t of the pass is list entry start + t
  // (wrapped); t is clamped to the last one.
  // Entries are packed with their extents (pack_block_entry).
  auto load_batch = [&](int b) {
    int pos = min(b * 64 + lane, cnt - 1) + start;
    pos -= pos >= cnt ? cnt : 0;
    return pack_block_entry(a, list[pos]);
  };
  uint32_t batch_cur = 0, batch_nxt = 0;   // entries 64 B .. and 64 (B + 1) .. of the pass
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
      const u32x4 u = tile[k_chunk_slot<D>(key0 + li, 2 * ks + h)];
      r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), f[ks], r, 0, 0, 0);
    }
    return r;
  };
  // pad keys of a partial patch (a uniform branch) get S = -inf, hence P = dS = 0
  auto step = [&](uint32_t pe, const u32x4* ks_, const u32x4* vs_) {
    f32x16 s = rows_times(ks_, qf);
    const f32x16 dp = rows_times(vs_, df);
    const BlockExtent ext = packed_extent(pe);
    if (!ext.full()) {
      const uint32_t bits = real_accumulator_bits(ext, wk, h);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = ((bits >> r) & 1u) ? s[r] : -INFINITY;
    }
    bf16x8 dsb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lse2));
      dsb[r >> 3][r & 7] = static_cast<__bf16>(pr * (dp[r] - dlt));
    }
    const uint16_t* kt = reinterpret_cast<const uint16_t*>(ks_);
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int st = 0; st < 2; ++st)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            transposed_fragment(kt + 16 * st * D, toff[dt][0], toff[dt][1]), dsb[st], acc[dt], 0, 0, 0);
  };

  if (cnt > 0) {
    const uint32_t off = tile_load_offset<D, false>(wave, lane);
    batch_cur = load_batch(0);
    batch_nxt = load_batch(1);
    uint32_t jb_cur = tile_of(0);
    load_pair<D>(K + tile_off(jb_cur), V + tile_off(jb_cur), k_slot0, v_slot0, off, wave,
                 tile_rows(jb_cur), tile_cols(jb_cur));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    auto body = [&](int e, auto parity) {
      constexpr int kOdd = decltype(parity)::value;
      u32x4* const kc = kOdd ? k_slot1 : k_slot0;
      u32x4* const vc = kOdd ? v_slot1 : v_slot0;
      u32x4* const kn = kOdd ? k_slot0 : k_slot1;
      u32x4* const vn = kOdd ? v_slot0 : v_slot1;
      if (((e + 1) & 63) == 0 && e + 1 < cnt) {   // entry e + 1 opens the next batch
        batch_cur = batch_nxt;
        batch_nxt = load_batch(((e + 1) >> 6) + 1);
      }
      const uint32_t jb_next = tile_of(e + 1);
      if (e + 1 < cnt)
        load_pair<D>(K + tile_off(jb_next), V + tile_off(jb_next), kn, vn, off, wave,
                     tile_rows(jb_next), tile_cols(jb_next));
      step(jb_cur, kc, vc);
      jb_cur = jb_next;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    for (int e = 0; e < cnt; e += 2) {
      body(e, std::integral_constant<int, 0>{});
      if (e + 1 < cnt) body(e + 1, std::integral_constant<int, 1>{});
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

__global__ __launch_bounds__(256) void bwd_bitmap(const int32_t* __restrict__ kv_count,
                                                  const int32_t* __restrict__ kv_index,
                                                  uint32_t* __restrict__ bitmap, int nb, int words,
                                                  int64_t total /* BH * nb * nb */) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int64_t row = e / nb;                     // bh * nb + i
  const int t = static_cast<int>(e - row * nb);
  if (t >= min(max(kv_count[row], 0), nb)) return;
  const int j = kv_index[e];
  if (static_cast<unsigned>(j) >= static_cast<unsigned>(nb)) return;
  atomicOr(bitmap + row * words + (j >> 5), 1u << (j & 31));
}

// one wave per (bh, key block j): the query blocks i with bit (i, j), ascending
__global__ __launch_bounds__(256) void bwd_transpose(const uint32_t* __restrict__ bitmap,
                                                     int32_t* __restrict__ q_count,
                                                     int32_t* __restrict__ q_index, int nb,
                                                     int words, int64_t rows /* BH * nb */) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t bh = row / nb;
  const int j = static_cast<int>(row - bh * nb);
  const uint32_t* bm = bitmap + bh * nb * static_cast<int64_t>(words) + (j >> 5);
  int32_t* out = q_index + row * nb;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int count = 0;
  for (int base = 0; base < nb; base += 64) {
    const int i = base + lane;
    const bool keep = i < nb && ((bm[static_cast<int64_t>(i) * words] >> (j & 31)) & 1u);
    const uint64_t b = __ballot(keep);
    if (keep) out[count + __popcll(b & lt)] = i;
    count += __popcll(b);
  }
  if (lane == 0) q_count[row] = count;
}

// ---------------------------------------------------------------------------
// dK and dV in one pass: one workgroup of eight waves per key block over the
// query blocks that keep it. Waves 0-3 form the dV group, waves 4-7 the dK
// group; in each group wave (wk, wq) takes key half wk and query half wq of
// every tile, lane li holding key li of its half. Both groups read the same
// Q and dO tiles, so a kept tile crosses the memory system once for both
// gradients: the dV group copies Q, the dK
// group dO. Per tile the dV group forms S and P and adds dV^T += dO^T P; the
// dK group forms S, dP = dO V^T and dS = P (dP - D) and adds dK^T += Q^T dS.
// A SIMD holds one wave of each group. Q, dO, lse and D of tile e+1 arrive
// during tile e (two-slot rings; a third slot, with copies two tiles ahead,
// was slower).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(2 * kThreads, 1) void bwd_dkv(AttnArgs a, const uint16_t* __restrict__ dop,
                                                           const float* __restrict__ delta,
                                                           const float* __restrict__ lse2,
                                                           const int32_t* __restrict__ q_count,
                                                           const int32_t* __restrict__ q_index,
                                                           uint16_t* __restrict__ dkp,
                                                           uint16_t* __restrict__ dvp, int64_t n_items) {
  using S = Stage<D>;
  constexpr int kKS = D / 16;
  constexpr int kDT = D / 32;
  __shared__ u32x4 q_slot0[S::kTile], q_slot1[S::kTile];
  __shared__ u32x4 d_slot0[S::kTile], d_slot1[S::kTile];
  __shared__ f32x4 vec_slot[2][2][kBlock / 4];   // [slot][lse2, D][4 rows]
  __shared__ int start_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;                                // 0: dV group, 1: dK group
  const int w = wave & 3;                                   // wave within the group
  const int wk = w & 1, wq = w >> 1;
  const int li = lane & 31, h = lane >> 5;
  const int64_t item = xcd_order(blockIdx.x, n_items);     // bh * nb + key block j
  const int64_t bh = item / a.nb;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.qp) + bh * a.N * D;
  const uint16_t* __restrict__ dO = dop + bh * a.N * D;
  const float* __restrict__ lse_h = lse2 + bh * a.N;
  const float* __restrict__ dl_h = delta + bh * a.N;
  const int64_t krow = item * kBlock + wk * 32 + li;        // global key row of this lane
  const uint16_t* __restrict__ Kg = static_cast<const uint16_t*>(a.kp);
  const uint16_t* __restrict__ Vg = static_cast<const uint16_t*>(a.vp);
  bf16x8 kf[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks)
    kf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Kg + krow * D + 16 * ks + 8 * h));
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
  // list entries, packed with their extents, 64 at a time a batch ahead (as
  // in the forward); entry t of the pass is list entry start + t (wrapped),
  // t clamped to the last one
  auto load_batch = [&](int b) {
    int pos = min(b * 64 + lane, cnt - 1) + start;
    pos -= pos >= cnt ? cnt : 0;
    return pack_block_entry(a, list[pos]);
  };
  uint32_t batch_cur = 0, batch_nxt = 0;
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
      const u32x4 u = tile[k_chunk_slot<D>(row0 + li, 2 * ks + h)];
      r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), f[ks], r, 0, 0, 0);
    }
    return r;
  };
  // pad query rows (partial patches only: a uniform branch) get S = -inf,
  // hence P = dS = 0
  auto mask = [&](uint32_t pe, f32x16& s) {
    const BlockExtent ext = packed_extent(pe);
    if (!ext.full()) {
      const uint32_t bits = real_accumulator_bits(ext, wq, h);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = ((bits >> r) & 1u) ? s[r] : -INFINITY;
    }
  };
  // P of the tile in bf16 (dV group)
  auto probs = [&](uint32_t pe, f32x16 s, const f32x4 (&vec)[2][kBlock / 4], bf16x8 (&wb)[2]) {
    mask(pe, s);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 lv = vec[0][(row0 >> 2) + 2 * g + h];     // rows row0 + 8 g + 4 h .. + 3
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 4 * g + x;
        wb[r >> 3][r & 7] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s[r], c, -lv[x])));
      }
    }
  };
  // dS of the tile in bf16, from S and dP (dK group)
  auto weights = [&](uint32_t pe, f32x16 s, const f32x16& dp, const f32x4 (&vec)[2][kBlock / 4],
                     bf16x8 (&wb)[2]) {
    mask(pe, s);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int m4 = (row0 >> 2) + 2 * g + h;              // rows row0 + 8 g + 4 h .. + 3
      const f32x4 lv = vec[0][m4];
      const f32x4 dv4 = vec[1][m4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 4 * g + x;
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lv[x]));
        wb[r >> 3][r & 7] = static_cast<__bf16>(pr * (dp[r] - dv4[x]));
      }
    }
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
  // covers them and no register waits on them. The LDS operand goes in as
  // float*: passed as a vector pointer, the compiler turned it into the null
  // LDS address.
  auto copy_vecs = [&](uint32_t pe, f32x4 (&vec)[2][kBlock / 4]) {
    if (wave == 0) {
      const int64_t r0 = static_cast<int64_t>(packed_block(pe)) * kBlock;
      __builtin_amdgcn_global_load_lds(lse_h + r0 + lane, reinterpret_cast<float*>(vec[0]), 4, 0, 0);
      __builtin_amdgcn_global_load_lds(dl_h + r0 + lane, reinterpret_cast<float*>(vec[1]), 4, 0, 0);
    }
  };
  const uint32_t off = tile_load_offset<D, false>(w, lane);
  // The two groups run the same tile loop, instantiated once per group so
  // that the dV group holds no V fragments; both pass the same barriers.
  auto run = [&](auto group) {
    constexpr int kDk = decltype(group)::value;
    // this group's share of the copies of query block pe: Q (dV group) or
    // dO (dK group)
    auto copy_tile = [&](uint32_t pe, u32x4* qs, u32x4* ds) {
      const int64_t r0 = static_cast<int64_t>(packed_block(pe)) * kBlock * D;
      if constexpr (kDk)
        issue_tile_load<D>(dO + r0, ds, off, w, rows(pe), cols(pe));
      else
        issue_tile_load<D>(Q + r0, qs, off, w, rows(pe), cols(pe));
    };
    bf16x8 vf[kKS];
    if constexpr (kDk) {
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        vf[ks] = __builtin_bit_cast(bf16x8,
                                    *reinterpret_cast<const uint4*>(Vg + krow * D + 16 * ks + 8 * h));
    }
    if (cnt == 0) return;
    batch_cur = load_batch(0);
    batch_nxt = load_batch(1);
    uint32_t ib_cur = entry(0);
    copy_vecs(ib_cur, vec_slot[0]);
    copy_tile(ib_cur, q_slot0, d_slot0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // tile e in slot e % 2; the copies of e+1 go to the other slot
    auto body = [&](int e, auto parity) {
      constexpr int kOdd = decltype(parity)::value;
      u32x4* const qc = kOdd ? q_slot1 : q_slot0;
      u32x4* const dc = kOdd ? d_slot1 : d_slot0;
      u32x4* const qn = kOdd ? q_slot0 : q_slot1;
      u32x4* const dn = kOdd ? d_slot0 : d_slot1;
      if (((e + 1) & 63) == 0 && e + 1 < cnt) {   // entry e + 1 opens the next batch
        batch_cur = batch_nxt;
        batch_nxt = load_batch(((e + 1) >> 6) + 1);
      }
      const uint32_t ib_next = entry(e + 1);
      if (e + 1 < cnt) {
        copy_vecs(ib_next, vec_slot[kOdd ^ 1]);
        copy_tile(ib_next, qn, dn);
      }
      const f32x16 sv = rows_times(qc, kf);
      bf16x8 wb[2];
      if constexpr (kDk) {
        const f32x16 dp = rows_times(dc, vf);
        weights(ib_cur, sv, dp, vec_slot[kOdd], wb);
        accumulate(qc, wb);
      } else {
        probs(ib_cur, sv, vec_slot[kOdd], wb);
        accumulate(dc, wb);
      }
      ib_cur = ib_next;
      // Every copy has landed, so Q, dO, lse and D of e+1 are in LDS for
      // every wave after the barrier. The scheduling barrier keeps the wait
      // after this tile's work; the empty asm statements keep the compiler
      // from moving LDS accesses across the barrier.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    for (int e = 0; e < cnt; e += 2) {
      body(e, std::integral_constant<int, 0>{});
      if (e + 1 < cnt) body(e + 1, std::integral_constant<int, 1>{});
    }
  };
  if (grp == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});

  // ---- add the two query halves of each group, store (pad keys: 0) --------
  float* const part = reinterpret_cast<float*>(grp == 0 ? (wk ? q_slot1 : q_slot0)
                                                        : (wk ? d_slot1 : d_slot0));
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
  const int64_t entries = g.BH * g.nb * g.nb;
  hipLaunchKernelGGL(bwd_bitmap, grid_for(entries, 256), dim3(256), 0, stream, kv_count, kv_index,
                     bitmap, g.nb, w.words, entries);
  hipLaunchKernelGGL(bwd_transpose, grid_for(g.BH * g.nb, 4), dim3(256), 0, stream, bitmap, q_count,
                     q_index, g.nb, w.words, g.BH * g.nb);

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
  const unsigned grid = static_cast<unsigned>(items);
  uint16_t* dq16 = static_cast<uint16_t*>(dqp);
  uint16_t* dk16 = static_cast<uint16_t*>(dkp);
  uint16_t* dv16 = static_cast<uint16_t*>(dvp);
  // clock-phased periods: ticks of the 100 MHz clock per tile of each pass
  // (d = 128 at 720p; d = 64 tiles take about half as long)
  const uint32_t t_dq = phased ? (g.D == 64 ? 95u : 185u) : 0u;
  const uint32_t t_dkv = phased ? (g.D == 64 ? 110u : 220u) : 0u;
  AttnArgs a_dq = a, a_dkv = a;
  a_dq.sweep_ticks = t_dq;
  a_dkv.sweep_ticks = t_dkv;
  if (g.D == 64) {
    hipLaunchKernelGGL((bwd_dq<64>), dim3(grid), dim3(kThreads), 0, stream, a_dq, do16, delta,
                       lse2, dq16, items);
    hipLaunchKernelGGL((bwd_dkv<64>), dim3(grid), dim3(2 * kThreads), 0, stream, a_dkv, do16,
                       delta, lse2, q_count, q_index, dk16, dv16, items);
  } else {
    hipLaunchKernelGGL((bwd_dq<128>), dim3(grid), dim3(kThreads), 0, stream, a_dq, do16, delta,
                       lse2, dq16, items);
    hipLaunchKernelGGL((bwd_dkv<128>), dim3(grid), dim3(2 * kThreads), 0, stream, a_dkv, do16,
                       delta, lse2, q_count, q_index, dk16, dv16, items);
  }
}

}  // namespace cabf
