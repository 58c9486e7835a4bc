// Semantic-permutation path around the k-means (Sparse VideoGen2 summary,
// Methodology A-C):
//   gather_rows / scatter_rows   apply and undo a per-head token permutation
//   cluster_scores               z_ab = scale <cq_a, ck_b> + ln |K_b|, so that
//                                the row softmax of z is the attention share of
//                                key cluster b with every key token represented
//                                by its centroid (empty clusters: -inf)
//   (select_rows of mask.hip)    softmax, top-p cut (thr = 1 - p), compaction
//   cluster_chunks               kept key clusters -> 64-key chunks
//   query_tiles                  query clusters -> 64-row tiles
//   bsa_fwd_mfma<ClusterLayout>  the attention over those tables
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attention_common.hpp"
#include "streaming.hpp"
#include "svg.hpp"

namespace cabf {
namespace {

size_t align256(size_t v) { return (v + 255) & ~size_t{255}; }

// one thread per 16-byte chunk of an output row
__global__ __launch_bounds__(256) void gather_rows(const uint4* __restrict__ x,
                                                   const int32_t* __restrict__ perm,
                                                   uint4* __restrict__ xp, int n, int rows_out,
                                                   int chunks_per_row, int64_t total) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int64_t row = e / chunks_per_row;        // bh * rows_out + i
  const int ch = static_cast<int>(e - row * chunks_per_row);
  const int64_t bh = row / rows_out;
  const int i = static_cast<int>(row - bh * rows_out);
  uint4 v = make_uint4(0, 0, 0, 0);
  if (i < n) {
    const int src = min(max(perm[bh * n + i], 0), n - 1);
    v = load_stream(x + (bh * n + src) * chunks_per_row + ch);
  }
  store_stream(xp + e, v);
}

__global__ __launch_bounds__(256) void scatter_rows(const uint4* __restrict__ xp,
                                                    const int32_t* __restrict__ perm,
                                                    uint4* __restrict__ x, int n, int rows_in,
                                                    int chunks_per_row, int64_t total) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int64_t row = e / chunks_per_row;        // bh * n + i
  const int ch = static_cast<int>(e - row * chunks_per_row);
  const int64_t bh = row / n;
  const int i = static_cast<int>(row - bh * n);
  const int dst = min(max(perm[row], 0), n - 1);
  store_stream(x + (bh * n + dst) * chunks_per_row + ch,
               load_stream(xp + (bh * rows_in + i) * chunks_per_row + ch));
}

// one thread per (bh, a, b); padding columns b >= ck are never read
template <int D>
__global__ __launch_bounds__(256) void cluster_scores(const float* __restrict__ qc,
                                                      const float* __restrict__ kc,
                                                      const int32_t* __restrict__ k_counts,
                                                      float* __restrict__ z, int cq, int ck,
                                                      int ldz, float scale, int64_t total) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int64_t row = e / ck;                    // bh * cq + a
  const int b = static_cast<int>(e - row * ck);
  const int64_t bh = row / cq;
  const int cnt = k_counts[bh * ck + b];
  float out = -INFINITY;
  if (cnt > 0) {
    const float* q = qc + row * D;
    const float* k = kc + (bh * ck + b) * D;
    float s = 0.0f;
#pragma unroll 16
    for (int j = 0; j < D; ++j) s = fmaf(q[j], k[j], s);
    out = fmaf(scale, s, logf(static_cast<float>(cnt)));
  }
  z[row * ldz + b] = out;
}

// One wave per (bh, query cluster): the kept key clusters, ascending, become
// 64-key chunks (first key row << 6) | (keys - 1) of the permuted K/V.
// Offsets are clamped to [0, n]; at most cap chunks are written.
__global__ __launch_bounds__(256) void cluster_chunks(const int32_t* __restrict__ k_off,
                                                      const int32_t* __restrict__ kv_count,
                                                      const int32_t* __restrict__ kv_index,
                                                      int32_t* __restrict__ chunk_count,
                                                      int32_t* __restrict__ chunks, int n, int cq,
                                                      int ck, int cap, int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t bh = row / cq;
  const int32_t* off = k_off + bh * (ck + 1);
  const int cnt = min(max(kv_count[row], 0), ck);
  const int32_t* list = kv_index + row * ck;
  int32_t* out = chunks + row * cap;
  int written = 0;
  for (int base = 0; base < cnt; base += 64) {
    const int idx = base + lane;
    int start = 0, keys = 0;
    if (idx < cnt) {
      const int b = list[idx];
      if (b >= 0 && b < ck) {
        start = min(max(off[b], 0), n);
        keys = max(min(max(off[b + 1], 0), n) - start, 0);
      }
    }
    const int nch = (keys + 63) >> 6;
    // inclusive wave scan of the chunk counts
    int incl = nch;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int v = __shfl_up(incl, sh);
      if (lane >= sh) incl += v;
    }
    const int pos = written + incl - nch;
    for (int j = 0; j < nch; ++j) {
      if (pos + j < cap)
        out[pos + j] = ((start + 64 * j) << 6) | (min(64, keys - 64 * j) - 1);
    }
    written += __shfl(incl, 63);
  }
  if (lane == 0) chunk_count[row] = min(written, cap);
}

// One wave per bh: every query cluster's rows as 64-row tiles (query
// cluster, first row); unused entries up to max_tiles get cluster -1.
__global__ __launch_bounds__(64) void query_tiles(const int32_t* __restrict__ q_off,
                                                  int32_t* __restrict__ tiles, int n, int cq,
                                                  int max_tiles) {
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int32_t* off = q_off + bh * (cq + 1);
  int32_t* out = tiles + bh * max_tiles * 2;
  int written = 0;
  for (int base = 0; base < cq; base += 64) {
    const int a = base + lane;
    int start = 0, rows = 0;
    if (a < cq) {
      start = min(max(off[a], 0), n);
      rows = max(min(max(off[a + 1], 0), n) - start, 0);
    }
    const int nt = (rows + 63) >> 6;
    int incl = nt;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int v = __shfl_up(incl, sh);
      if (lane >= sh) incl += v;
    }
    const int pos = written + incl - nt;
    for (int t = 0; t < nt; ++t) {
      if (pos + t < max_tiles) {
        out[(pos + t) * 2] = a;
        out[(pos + t) * 2 + 1] = start + 64 * t;
      }
    }
    written += __shfl(incl, 63);
  }
  for (int i = min(written, max_tiles) + lane; i < max_tiles; i += 64) {
    out[i * 2] = -1;
    out[i * 2 + 1] = 0;
  }
}

dim3 grid_for(int64_t work, int per) { return dim3(static_cast<unsigned>((work + per - 1) / per)); }

}  // namespace

void launch_gather_rows(int64_t BH, int n, int rows_out, int row_bytes, const void* x,
                        const int32_t* perm, void* xp, hipStream_t stream) {
  const int cpr = row_bytes / 16;
  const int64_t total = BH * rows_out * cpr;
  hipLaunchKernelGGL(gather_rows, grid_for(total, 256), dim3(256), 0, stream,
                     static_cast<const uint4*>(x), perm, static_cast<uint4*>(xp), n, rows_out, cpr,
                     total);
}

void launch_scatter_rows(int64_t BH, int n, int rows_in, int row_bytes, const void* xp,
                         const int32_t* perm, void* x, hipStream_t stream) {
  const int cpr = row_bytes / 16;
  const int64_t total = BH * n * cpr;
  hipLaunchKernelGGL(scatter_rows, grid_for(total, 256), dim3(256), 0, stream,
                     static_cast<const uint4*>(xp), perm, static_cast<uint4*>(x), n, rows_in, cpr,
                     total);
}

SelectWorkspace cluster_select_workspace_layout(int64_t BH, int cq, int ck) {
  SelectWorkspace w{};
  w.ldz = (ck + 63) / 64 * 64;
  w.total = align256(static_cast<size_t>(BH) * cq * w.ldz * sizeof(float));
  return w;
}

void launch_cluster_select(int64_t BH, int cq, int ck, int D, const float* qc, const float* kc,
                           const int32_t* k_counts, float scale, float top_p, int32_t* kv_count,
                           int32_t* kv_index, float* probs, void* workspace, hipStream_t stream) {
  const SelectWorkspace w = cluster_select_workspace_layout(BH, cq, ck);
  float* z = static_cast<float*>(workspace);
  const int64_t total = BH * cq * ck;
  if (D == 64)
    hipLaunchKernelGGL((cluster_scores<64>), grid_for(total, 256), dim3(256), 0, stream, qc, kc,
                       k_counts, z, cq, ck, w.ldz, scale, total);
  else
    hipLaunchKernelGGL((cluster_scores<128>), grid_for(total, 256), dim3(256), 0, stream, qc, kc,
                       k_counts, z, cq, ck, w.ldz, scale, total);
  launch_select_matrix(z, w.ldz, BH * cq, ck, 1.0f - top_p, kv_count, kv_index, probs, stream);
}

ClusterAttnWorkspace cluster_attention_workspace_layout(int64_t BH, int n, int cq, int ck) {
  ClusterAttnWorkspace w{};
  w.cap = (n + 63) / 64 + ck;
  w.max_tiles = (n + 63) / 64 + cq;
  size_t o = 0;
  w.chunk_count = o;  o += align256(static_cast<size_t>(BH) * cq * sizeof(int32_t));
  w.chunks = o;       o += align256(static_cast<size_t>(BH) * cq * w.cap * sizeof(int32_t));
  w.tiles = o;        o += align256(static_cast<size_t>(BH) * w.max_tiles * 2 * sizeof(int32_t));
  w.total = o;
  return w;
}

void launch_cluster_attention(int64_t BH, int n, int D, int cq, int ck, const void* qp,
                              const void* kp, const void* vp, const int32_t* q_off,
                              const int32_t* k_off, const int32_t* kv_count,
                              const int32_t* kv_index, float scale, void* op, float* lse,
                              void* workspace, hipStream_t stream) {
  const ClusterAttnWorkspace w = cluster_attention_workspace_layout(BH, n, cq, ck);
  char* ws = static_cast<char*>(workspace);
  int32_t* chunk_count = reinterpret_cast<int32_t*>(ws + w.chunk_count);
  int32_t* chunks = reinterpret_cast<int32_t*>(ws + w.chunks);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + w.tiles);
  hipLaunchKernelGGL(cluster_chunks, grid_for(BH * cq, 4), dim3(256), 0, stream, k_off, kv_count,
                     kv_index, chunk_count, chunks, n, cq, ck, w.cap, BH * cq);
  hipLaunchKernelGGL(query_tiles, dim3(static_cast<unsigned>(BH)), dim3(64), 0, stream, q_off,
                     tiles, n, cq, w.max_tiles);
  AttnArgs a{};
  a.qp = qp;
  a.kp = kp;
  a.vp = vp;
  a.op = op;
  a.lse = lse;
  a.scale_log2 = scale * kLog2e;
  a.N = n + kBlock;          // rows per head of the permuted, padded tensors
  a.BH = BH;
  launch_cluster_attention_mfma(a, D, tiles, w.max_tiles, q_off, cq, chunk_count, chunks, w.cap,
                                stream);
}

}  // namespace cabf
