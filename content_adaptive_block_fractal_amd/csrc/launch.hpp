// Internal launcher declarations (one per kernel family). Arguments are
// already validated by the C ABI layer when these run.
#pragma once

#include <hip/hip_runtime.h>

#include "geometry.hpp"

namespace cabf {

// Fractal reorder of up to three tensors (src[i] -> dst[i], null pairs skipped).
void launch_permute(const Geo& g, int elem_bytes, const void* const src[3], void* const dst[3],
                    hipStream_t stream);
// Inverse reorder of one tensor.
void launch_unpermute(const Geo& g, int elem_bytes, const void* src, void* dst, hipStream_t stream);
// permute that also writes the pooled means of src[0] (Q) and src[1] (K)
void launch_permute_pool(const Geo& g, int elem_bytes, const void* const src[3],
                         void* const dst[3], float* qb, float* kb, hipStream_t stream);

// Mask workspace layout (bytes from the workspace base).
struct MaskWorkspace {
  size_t qb_off, kb_off, z_off, total;
  int ldz;  // row stride of the block-logit matrix, in floats
};
MaskWorkspace mask_workspace_layout(const Geo& g);

// topk > 0 replaces the CDF cut (thr unused) by the topk most probable blocks
void launch_build_block_mask(const Geo& g, bool bf16, const void* qp, const void* kp, float scale,
                             float thr, int topk, bool sta_on, int dt, int dy, int dx,
                             int32_t* kv_count, int32_t* kv_index, float* block_prob,
                             void* workspace, hipStream_t stream);

// The CDF mask (no top-k) with the workspace in a fixed device array instead
// of a caller buffer (mask_noalloc.hip): noalloc_pairs_per_pass is the number
// of (batch, head) pairs one pass of the array holds (0: a single pair does
// not fit); the launcher returns a cabf_status.
int64_t noalloc_pairs_per_pass(const Geo& g);
int launch_build_block_mask_noalloc(const Geo& g, int elem_bytes, const void* qp, const void* kp,
                                    float scale, float thr, bool sta_on, int dt, int dy, int dx,
                                    int32_t* kv_count, int32_t* kv_index, float* block_prob,
                                    hipStream_t stream);

// logits, selection and compaction from pooled means already in the workspace
void launch_mask_from_pooled(const Geo& g, float scale, float thr, int topk, bool sta_on, int dt,
                             int dy, int dx, int32_t* kv_count, int32_t* kv_index,
                             float* block_prob, void* workspace, hipStream_t stream);

void launch_build_sta_mask(const Geo& g, int dt, int dy, int dx, int32_t* kv_count,
                           int32_t* kv_index, hipStream_t stream);

// Backward workspace: D = rowsum(dO * O), the kept-list bitmap and the
// transposed lists (query blocks of every key block), the key blocks of
// each head ordered by transposed-list length.
struct BwdWorkspace {
  int words;
  size_t delta, lse2, bitmap, q_count, q_index, k_order, total;
};
BwdWorkspace bwd_workspace_layout(const Geo& g);
void launch_bsa_backward(const Geo& g, const void* qp, const void* kp, const void* vp,
                         const void* op, const float* lse, const void* dop,
                         const int32_t* kv_count, const int32_t* kv_index, float scale, void* dqp,
                         void* dkp, void* dvp, void* workspace, bool phased,
                         hipStream_t stream);

void launch_bsa_forward(const Geo& g, bool bf16, const void* qp, const void* kp, const void* vp,
                        const int32_t* kv_count, const int32_t* kv_index, float scale, void* op,
                        float* lse, bool phased, hipStream_t stream);
// bf16 forward over the listed global query blocks (b*heads*nb + h*nb + block)
// only; entries outside that range are skipped
void launch_bsa_forward_subset(const Geo& g, const void* qp, const void* kp, const void* vp,
                               const int32_t* kv_count, const int32_t* kv_index,
                               const int32_t* q_blocks, int64_t n_blocks, float scale, void* op,
                               float* lse, bool phased, hipStream_t stream);

}  // namespace cabf
