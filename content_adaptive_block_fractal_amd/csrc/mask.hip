// Adaptive block mask (NABLA summary, Methodology items 2-3).
//
//  pool_blocks    Qb, Kb = fp32 means over the real tokens of each 64-token
//                 block (one wave per block; reads Qp/Kp once, HBM-bound).
//  block_logits   Z = scale * Qb Kb^T per (batch, head), fp32 register-tiled
//                 GEMM through LDS (nb x nb x head_dim).
//  select_rows    one wave per block row: softmax of the row, the CDF cut
//                 (or a fixed-budget top-k), the sliding-tile window and
//                 ascending compaction.
//  sta_rows       the sliding-tile window alone (no scores), one row per
//                 thread.
//
// The CDF cut keeps the shortest prefix of the row sorted by probability
// (descending, ties to the lower index) whose mass reaches 1 - thr. Instead
// of sorting, select_rows finds the probability p* of the last kept block
// directly: mass(u) = sum of p_j with bits(p_j) >= u is non-increasing in the
// bit pattern u of a non-negative float, so p* is the largest element value
// with mass(bits(p*)) >= 1 - thr, found by bisection over the bit patterns.
// Every block above p* is kept, and of the blocks equal to p* the lowest
// indices are kept until the mass reaches 1 - thr. In exact arithmetic this
// is the same set the sorted prefix gives; only the fp32 summation order
// differs. The top-k selection uses the same search with the count of blocks
// at or above u in place of their mass (exact integers).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "geometry.hpp"
#include "launch.hpp"
#include "svg.hpp"

namespace cabf {
namespace {

constexpr int kWave = 64;

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;  // identical in every lane: IEEE addition is commutative
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ inline uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off)));
  return v;
}

__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off)));
  return v;
}

__device__ inline uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

// ---------------------------------------------------------------------------
// pool_blocks: one wave per (tensor, batch*head, block)
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_blocks(const T* __restrict__ qp, const T* __restrict__ kp,
                                                   float* __restrict__ qb, float* __restrict__ kb,
                                                   int64_t blocks_total, int nb, int Ty, int Tx,
                                                   int H, int W) {
  constexpr int kEB = sizeof(T);
  constexpr int kCH = D * kEB / 16;        // 16-byte chunks per row
  constexpr int kEPC = 16 / kEB;           // elements per chunk
  constexpr int kRPP = kWave / kCH;        // rows per pass
  constexpr int kPasses = kBlock / kRPP;
  const T* __restrict__ src = blockIdx.y == 0 ? qp : kp;
  float* __restrict__ dst = blockIdx.y == 0 ? qb : kb;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (blk >= blocks_total) return;
  const int b = static_cast<int>(blk % nb);
  const int per_frame = Ty * Tx;
  const int rem = b % per_frame;
  const int ty = rem / Tx, tx = rem - (rem / Tx) * Tx;
  const int vy = min(kP, H - ty * kP);     // real rows of this patch
  const int vx = min(kP, W - tx * kP);     // real columns of this patch
  const int ch = lane % kCH;
  const int r0 = lane / kCH;
  const uint4* rows = reinterpret_cast<const uint4*>(src + blk * kBlock * D);
  float acc[kEPC];
#pragma unroll
  for (int e = 0; e < kEPC; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    const int row = r0 + ps * kRPP;
    if ((row >> 3) < vy && (row & 7) < vx) {
      const uint4 u = rows[row * kCH + ch];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      if constexpr (kEB == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[e] += bf16_to_f32(static_cast<uint16_t>(w[e >> 1] >> ((e & 1) * 16)));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(w[e]);
      }
    }
  }
#pragma unroll
  for (int off = kCH; off < kWave; off <<= 1) {
#pragma unroll
    for (int e = 0; e < kEPC; ++e) acc[e] += __shfl_xor(acc[e], off);
  }
  if (r0 == 0) {
    const float count = static_cast<float>(vy * vx);
    float* out = dst + blk * D + ch * kEPC;
#pragma unroll
    for (int e = 0; e < kEPC; ++e) out[e] = acc[e] / count;
  }
}

// ---------------------------------------------------------------------------
// block_logits: Z[bh] = scale * Qb[bh] Kb[bh]^T, 64x64 tiles, 4x4 per thread
// ---------------------------------------------------------------------------
constexpr int kTile = 64;
constexpr int kKC = 32;   // reduction chunk staged in LDS

template <int D>
__global__ __launch_bounds__(256) void block_logits(const float* __restrict__ qb,
                                                    const float* __restrict__ kb,
                                                    float* __restrict__ z, int nb, int ldz,
                                                    int tiles_per_side, float scale) {
  __shared__ float As[kKC][kTile + 4];
  __shared__ float Bs[kKC][kTile + 4];
  const int tiles = tiles_per_side * tiles_per_side;
  const int64_t bh = blockIdx.x / tiles;
  const int tile = static_cast<int>(blockIdx.x - bh * tiles);
  const int i0 = (tile / tiles_per_side) * kTile;
  const int j0 = (tile % tiles_per_side) * kTile;
  const float* __restrict__ A = qb + bh * static_cast<int64_t>(nb) * D;
  const float* __restrict__ Bm = kb + bh * static_cast<int64_t>(nb) * D;
  const int tid = threadIdx.x;
  const int tr = tid >> 4, tc = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.0f;
  // loader mapping: 64 rows x 32 columns = 512 float4 -> 2 per thread
  for (int k0 = 0; k0 < D; k0 += kKC) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int idx = tid + h * 256;
      const int row = idx >> 3;          // 0..63
      const int c4 = (idx & 7) * 4;      // 0..28
      float4 va = make_float4(0.f, 0.f, 0.f, 0.f), vb = va;
      if (i0 + row < nb) va = *reinterpret_cast<const float4*>(A + (int64_t)(i0 + row) * D + k0 + c4);
      if (j0 + row < nb) vb = *reinterpret_cast<const float4*>(Bm + (int64_t)(j0 + row) * D + k0 + c4);
      As[c4 + 0][row] = va.x; As[c4 + 1][row] = va.y; As[c4 + 2][row] = va.z; As[c4 + 3][row] = va.w;
      Bs[c4 + 0][row] = vb.x; Bs[c4 + 1][row] = vb.y; Bs[c4 + 2][row] = vb.z; Bs[c4 + 3][row] = vb.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < kKC; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(&As[k][tr * 4]);
      const float4 b = *reinterpret_cast<const float4*>(&Bs[k][tc * 4]);
      const float av[4] = {a.x, a.y, a.z, a.w};
      const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(av[x], bv[y], acc[x][y]);
    }
    __syncthreads();
  }
  float* __restrict__ Z = z + bh * static_cast<int64_t>(nb) * ldz;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int i = i0 + tr * 4 + x;
    if (i >= nb) continue;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int j = j0 + tc * 4 + y;
      if (j < nb) Z[(int64_t)i * ldz + j] = scale * acc[x][y];
    }
  }
}

// ---------------------------------------------------------------------------
// select_rows: one wave per block row
// ---------------------------------------------------------------------------
struct SelectArgs {
  const float* z;
  int ldz;
  int nb;
  int64_t rows_total;
  float thr;
  int topk;             // > 0: keep the topk most probable blocks instead of the CDF cut
  int sta_on, dt, dy, dx;
  int Ty, Tx;
  int32_t* kv_count;
  int32_t* kv_index;
  float* block_prob;
};

// floor(j / d) for 0 <= j < 2^24 with a float reciprocal and an exact fix-up
__device__ inline int div_small(int j, int d, float inv_d) {
  int q = static_cast<int>((static_cast<float>(j) + 0.5f) * inv_d);
  if (q * d > j) --q;
  if ((q + 1) * d <= j) ++q;
  return q;
}

template <int EPL>
__global__ __launch_bounds__(256) void select_rows(SelectArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= a.rows_total) return;
  const int nb = a.nb;
  const int nr = (nb + kWave - 1) / kWave;   // used register slots per lane
  const float* __restrict__ zr = a.z + row * a.ldz;
  float p[EPL];
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int j = r * kWave + lane;
    p[r] = (r < nr && j < nb) ? zr[j] : -INFINITY;
    m = fmaxf(m, p[r]);
  }
  m = wave_max(m);
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int j = r * kWave + lane;
    const float e = (r < nr && j < nb) ? expf(p[r] - m) : 0.0f;
    p[r] = e;
    s += e;
  }
  s = wave_sum(s);
#pragma unroll
  for (int r = 0; r < EPL; ++r) p[r] = p[r] / s;   // pads stay 0
  if (a.block_prob != nullptr) {
    float* __restrict__ out = a.block_prob + row * nb;
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      const int j = r * kWave + lane;
      if (r < nr && j < nb) out[j] = p[r];
    }
  }

  // --- the cut: ustar = bits of the last kept value, need = how many blocks
  // equal to it are kept (lowest indices first) ---------------------------
  bool keep_all = a.topk > 0 ? a.topk >= nb : !(a.thr > 0.0f);
  uint32_t ustar = 0;
  int need = 0;
  if (!keep_all && a.topk > 0) {
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      const int j = r * kWave + lane;
      if (r < nr && j < nb) {
        lo = min(lo, __float_as_uint(p[r]));
        hi = max(hi, __float_as_uint(p[r]));
      }
    }
    lo = uniform(wave_min_u32(lo));
    hi = uniform(wave_max_u32(hi));
    auto count_ge = [&](uint32_t u) {
      int acc = 0;
#pragma unroll
      for (int r = 0; r < EPL; ++r) {
        const int j = r * kWave + lane;
        acc += __popcll(__ballot(r < nr && j < nb && __float_as_uint(p[r]) >= u));
      }
      return acc;   // uniform
    };
    // largest u with at least topk blocks at or above it (count_ge(lo) = nb)
    while (lo < hi) {
      const uint32_t mid = lo + (hi - lo + 1u) / 2u;
      if (count_ge(mid) >= a.topk) lo = mid; else hi = mid - 1u;
      lo = uniform(lo);
      hi = uniform(hi);
    }
    ustar = lo;
    const int above = ustar == 0xffffffffu ? 0 : count_ge(ustar + 1u);
    need = uniform(static_cast<uint32_t>(a.topk - above));
  } else if (!keep_all) {
    const float target = 1.0f - a.thr;
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      const int j = r * kWave + lane;
      if (r < nr && j < nb) {
        lo = min(lo, __float_as_uint(p[r]));
        hi = max(hi, __float_as_uint(p[r]));
      }
    }
    lo = uniform(wave_min_u32(lo));
    hi = uniform(wave_max_u32(hi));
    auto mass_ge = [&](uint32_t u) {
      float acc = 0.0f;
#pragma unroll
      for (int r = 0; r < EPL; ++r) {
        const int j = r * kWave + lane;
        if (r < nr && j < nb && __float_as_uint(p[r]) >= u) acc += p[r];
      }
      return wave_sum(acc);
    };
    if (mass_ge(lo) < target) {
      keep_all = true;        // rounding kept the total below 1 - thr
    } else {
      while (lo < hi) {
        const uint32_t mid = lo + (hi - lo + 1u) / 2u;
        if (mass_ge(mid) >= target) lo = mid; else hi = mid - 1u;
        lo = uniform(lo);
        hi = uniform(hi);
      }
      ustar = lo;
      const float pstar = __uint_as_float(ustar);
      const float above = ustar == 0xffffffffu ? 0.0f : mass_ge(ustar + 1u);
      int ties = 0;
#pragma unroll
      for (int r = 0; r < EPL; ++r) {
        const int j = r * kWave + lane;
        ties += (r < nr && j < nb && __float_as_uint(p[r]) == ustar) ? 1 : 0;
      }
      ties = static_cast<int>(wave_sum(static_cast<float>(ties)) + 0.5f);
      // fewest equal-valued blocks that bring the mass to the target
      int k = 1;
      if (pstar > 0.0f) {
        const float need_f = ceilf((target - above) / pstar);
        k = need_f < 1.0f ? 1 : (need_f > static_cast<float>(ties) ? ties : static_cast<int>(need_f));
      } else {
        k = ties;
      }
      while (k > 1 && above + static_cast<float>(k - 1) * pstar >= target) --k;
      while (k < ties && above + static_cast<float>(k) * pstar < target) ++k;
      need = uniform(static_cast<uint32_t>(k));
    }
  }

  // --- window and ascending compaction --------------------------------------
  const int i = static_cast<int>(row % nb);
  const int per_frame = a.Ty * a.Tx;
  const float inv_pf = 1.0f / static_cast<float>(per_frame);
  const float inv_tx = 1.0f / static_cast<float>(a.Tx);
  int ti = 0, tyi = 0, txi = 0;
  if (a.sta_on) {
    ti = div_small(i, per_frame, inv_pf);
    const int rem = i - ti * per_frame;
    tyi = div_small(rem, a.Tx, inv_tx);
    txi = rem - tyi * a.Tx;
  }
  int32_t* __restrict__ out = a.kv_index + row * nb;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int count = 0, tie_seen = 0;
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    if (r >= nr) continue;    // uniform: keeps the loop fully unrolled
    const int j = r * kWave + lane;
    const bool real = j < nb;
    bool keep = real && keep_all;
    if (!keep_all) {
      const uint32_t u = __float_as_uint(p[r]);
      const bool tie = real && u == ustar;
      const uint64_t tb = __ballot(tie);
      const int rank = tie_seen + __popcll(tb & lt);
      keep = real && (u > ustar || (tie && rank < need));
      tie_seen += __popcll(tb);
    }
    if (a.sta_on && real && !keep) {
      const int tj = div_small(j, per_frame, inv_pf);
      const int rem = j - tj * per_frame;
      const int tyj = div_small(rem, a.Tx, inv_tx);
      const int txj = rem - tyj * a.Tx;
      keep = abs(tj - ti) <= a.dt && abs(tyj - tyi) <= a.dy && abs(txj - txi) <= a.dx;
    }
    const uint64_t kb = __ballot(keep);
    if (keep) out[count + __popcll(kb & lt)] = j;
    count += __popcll(kb);
  }
  if (lane == 0) a.kv_count[row] = count;
}

// Sliding-tile window alone: one thread per block row writes the ascending
// indices of its clipped box (frames, then patch rows, then patch columns).
__global__ __launch_bounds__(256) void sta_rows(int64_t rows_total, int nb, int T, int Ty, int Tx,
                                                int dt, int dy, int dx, int32_t* __restrict__ kv_count,
                                                int32_t* __restrict__ kv_index) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (row >= rows_total) return;
  const int i = static_cast<int>(row % nb);
  const int per_frame = Ty * Tx;
  const int ti = i / per_frame;
  const int tyi = (i - ti * per_frame) / Tx;
  const int txi = i - ti * per_frame - tyi * Tx;
  int32_t* __restrict__ out = kv_index + row * nb;
  int count = 0;
  for (int t = max(ti - dt, 0); t <= min(ti + dt, T - 1); ++t)
    for (int ty = max(tyi - dy, 0); ty <= min(tyi + dy, Ty - 1); ++ty)
      for (int tx = max(txi - dx, 0); tx <= min(txi + dx, Tx - 1); ++tx)
        out[count++] = (t * Ty + ty) * Tx + tx;
  kv_count[row] = count;
}

template <int EPL>
void launch_select(const SelectArgs& a, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>((a.rows_total + 3) / 4);
  hipLaunchKernelGGL((select_rows<EPL>), dim3(grid), dim3(256), 0, stream, a);
}

// register slots per lane of a row: the smallest instantiation that holds
// nb values (slots unused by the row still cost instructions in the search)
void dispatch_select(const SelectArgs& a, int slots, hipStream_t stream) {
  if (slots <= 1) launch_select<1>(a, stream);
  else if (slots <= 2) launch_select<2>(a, stream);
  else if (slots <= 4) launch_select<4>(a, stream);
  else if (slots <= 8) launch_select<8>(a, stream);
  else if (slots <= 12) launch_select<12>(a, stream);
  else if (slots <= 16) launch_select<16>(a, stream);
  else if (slots <= 20) launch_select<20>(a, stream);
  else if (slots <= 24) launch_select<24>(a, stream);
  else if (slots <= 32) launch_select<32>(a, stream);
  else if (slots <= 48) launch_select<48>(a, stream);
  else if (slots <= 64) launch_select<64>(a, stream);
  else if (slots <= 96) launch_select<96>(a, stream);
  else launch_select<128>(a, stream);
}

}  // namespace

MaskWorkspace mask_workspace_layout(const Geo& g) {
  auto align = [](size_t x) { return (x + 255) & ~size_t{255}; };
  MaskWorkspace w{};
  w.ldz = (g.nb + 63) / 64 * 64;
  const size_t pooled = static_cast<size_t>(g.BH) * g.nb * g.D * sizeof(float);
  w.qb_off = 0;
  w.kb_off = align(pooled);
  w.z_off = w.kb_off + align(pooled);
  w.total = w.z_off + align(static_cast<size_t>(g.BH) * g.nb * w.ldz * sizeof(float));
  return w;
}

void launch_select_matrix(const float* z, int ldz, int64_t rows, int cols, float thr,
                          int32_t* kv_count, int32_t* kv_index, float* probs, hipStream_t stream) {
  SelectArgs a{};
  a.z = z;
  a.ldz = ldz;
  a.nb = cols;
  a.rows_total = rows;
  a.thr = thr;
  a.kv_count = kv_count;
  a.kv_index = kv_index;
  a.block_prob = probs;
  a.Ty = 1;
  a.Tx = 1;
  const int slots = (cols + kWave - 1) / kWave;
  dispatch_select(a, slots, stream);
}

void launch_build_sta_mask(const Geo& g, int dt, int dy, int dx, int32_t* kv_count,
                           int32_t* kv_index, hipStream_t stream) {
  const int64_t rows = g.BH * g.nb;
  hipLaunchKernelGGL(sta_rows, dim3(static_cast<unsigned>((rows + 255) / 256)), dim3(256), 0,
                     stream, rows, g.nb, g.T, g.Ty, g.Tx, dt, dy, dx, kv_count, kv_index);
}

void launch_build_block_mask(const Geo& g, bool bf16, const void* qp, const void* kp, float scale,
                             float thr, int topk, bool sta_on, int dt, int dy, int dx,
                             int32_t* kv_count, int32_t* kv_index, float* block_prob,
                             void* workspace, hipStream_t stream) {
  const MaskWorkspace w = mask_workspace_layout(g);
  char* ws = static_cast<char*>(workspace);
  float* qb = reinterpret_cast<float*>(ws + w.qb_off);
  float* kb = reinterpret_cast<float*>(ws + w.kb_off);
  const int64_t blocks_total = g.BH * g.nb;

  const dim3 pool_grid(static_cast<unsigned>((blocks_total + 3) / 4), 2);
#define CABF_POOL(T, D)                                                                       \
  hipLaunchKernelGGL((pool_blocks<T, D>), pool_grid, dim3(256), 0, stream,                    \
                     static_cast<const T*>(qp), static_cast<const T*>(kp), qb, kb,            \
                     blocks_total, g.nb, g.Ty, g.Tx, g.H, g.W)
  if (bf16) {
    if (g.D == 64) CABF_POOL(uint16_t, 64); else CABF_POOL(uint16_t, 128);
  } else {
    if (g.D == 64) CABF_POOL(float, 64); else CABF_POOL(float, 128);
  }
#undef CABF_POOL
  launch_mask_from_pooled(g, scale, thr, topk, sta_on, dt, dy, dx, kv_count, kv_index, block_prob,
                          workspace, stream);
}

void launch_mask_from_pooled(const Geo& g, float scale, float thr, int topk, bool sta_on, int dt,
                             int dy, int dx, int32_t* kv_count, int32_t* kv_index,
                             float* block_prob, void* workspace, hipStream_t stream) {
  const MaskWorkspace w = mask_workspace_layout(g);
  char* ws = static_cast<char*>(workspace);
  const float* qb = reinterpret_cast<const float*>(ws + w.qb_off);
  const float* kb = reinterpret_cast<const float*>(ws + w.kb_off);
  float* z = reinterpret_cast<float*>(ws + w.z_off);
  const int64_t blocks_total = g.BH * g.nb;
  const int tps = (g.nb + kTile - 1) / kTile;
  const unsigned lg_grid = static_cast<unsigned>(g.BH * tps * tps);
  if (g.D == 64)
    hipLaunchKernelGGL((block_logits<64>), dim3(lg_grid), dim3(256), 0, stream, qb, kb, z, g.nb,
                       w.ldz, tps, scale);
  else
    hipLaunchKernelGGL((block_logits<128>), dim3(lg_grid), dim3(256), 0, stream, qb, kb, z, g.nb,
                       w.ldz, tps, scale);

  SelectArgs a{};
  a.z = z;
  a.ldz = w.ldz;
  a.nb = g.nb;
  a.rows_total = blocks_total;
  a.thr = thr;
  a.topk = topk;
  a.sta_on = sta_on ? 1 : 0;
  a.dt = dt;
  a.dy = dy;
  a.dx = dx;
  a.Ty = g.Ty;
  a.Tx = g.Tx;
  a.kv_count = kv_count;
  a.kv_index = kv_index;
  a.block_prob = block_prob;
  const int slots = (g.nb + kWave - 1) / kWave;
  dispatch_select(a, slots, stream);
}

}  // namespace cabf
