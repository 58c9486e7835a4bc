// Host-side launchers of the semantic-permutation path (Sparse VideoGen2
// summary, Methodology A-C): k-means and the cluster permutation, row
// gather/scatter, centroid scores with top-p selection, and the tables that
// drive the variable-size attention kernel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace cabf {

// Byte offsets inside the k-means workspace.
struct KmeansWorkspace {
  size_t terms, norm, hist, total;
};
KmeansWorkspace kmeans_workspace_layout(int64_t BH, int n, int C, int D);

// Always returns 0.
int launch_kmeans(int64_t BH, int n, int D, int C, int iters, const void* x, const int32_t* init,
                  float* cent, int32_t* counts, int32_t* label, int32_t* perm, int32_t* offsets,
                  void* workspace, hipStream_t stream);

// xp[bh, i] = x[bh, perm[bh, i]] for i < n, zero rows for n <= i < rows_out
void launch_gather_rows(int64_t BH, int n, int rows_out, int row_bytes, const void* x,
                        const int32_t* perm, void* xp, hipStream_t stream);
// x[bh, perm[bh, i]] = xp[bh, i] for i < n; xp has rows_in rows per head
void launch_scatter_rows(int64_t BH, int n, int rows_in, int row_bytes, const void* xp,
                         const int32_t* perm, void* x, hipStream_t stream);

// Cluster selection workspace: the score matrix [BH * cq, ldz].
struct SelectWorkspace {
  int ldz;
  size_t total;
};
SelectWorkspace cluster_select_workspace_layout(int64_t BH, int cq, int ck);
void launch_cluster_select(int64_t BH, int cq, int ck, int D, const float* qc, const float* kc,
                           const int32_t* k_counts, float scale, float top_p, int32_t* kv_count,
                           int32_t* kv_index, float* probs, void* workspace, hipStream_t stream);

// Row softmax + CDF cut (thr) + ascending compaction of an arbitrary
// row-major fp32 matrix (mask.hip's select_rows without a window).
void launch_select_matrix(const float* z, int ldz, int64_t rows, int cols, float thr,
                          int32_t* kv_count, int32_t* kv_index, float* probs, hipStream_t stream);

// Cluster attention workspace: chunk counts, chunk lists, query tiles.
struct ClusterAttnWorkspace {
  int cap, max_tiles;
  size_t chunk_count, chunks, tiles, total;
};
ClusterAttnWorkspace cluster_attention_workspace_layout(int64_t BH, int n, int cq, int ck);
void launch_cluster_attention(int64_t BH, int n, int D, int cq, int ck, const void* qp,
                              const void* kp, const void* vp, const int32_t* q_off,
                              const int32_t* k_off, const int32_t* kv_count,
                              const int32_t* kv_index, float scale, void* op, float* lse,
                              void* workspace, hipStream_t stream);

}  // namespace cabf
