/*
 * cabf.h - C ABI of the content-adaptive block-sparse video attention library
 * (libcabf.so, HIP for gfx950 / MI355X).
 *
 * The library runs one self-attention layer of a video diffusion transformer
 * the NABLA way (NABLA technical summary, gist.science paper 2507.13546,
 * "Methodology" items 1-3): reorder the (T, H, W) token grid so that every
 * P x P spatial patch of a frame is one contiguous 64-token block, build a
 * per-head block mask from mean-pooled Q and K (block softmax, descending
 * CDF cut at 1 - thr, optional union with a sliding-tile window), attend over
 * the kept (query block, key block) tiles only, and restore raster order.
 *
 * Conventions shared by every call
 *  - Pointers are device pointers unless a parameter says "host".
 *  - Token tensors are contiguous row-major [batch, heads, tokens, head_dim].
 *    "Raster" tensors have tokens = T*H*W in (t, y, x) order; "reordered"
 *    tensors have tokens = N = T*Hp*Wp with Hp = ceil(H/P)*P, Wp = ceil(W/P)*P.
 *  - The caller owns and allocates every buffer, including the workspace.
 *    The library never allocates, frees or synchronises; it keeps no state.
 *  - Work is enqueued on `stream` (NULL = the default stream) and is
 *    asynchronous: faults surface at the caller's next synchronisation.
 *  - Arguments are validated before anything is launched; on an error the
 *    call returns a negative cabf_status and has no side effects.
 *    CABF_EHIP reports a failed launch (hipGetLastError after the launch; an
 *    error left pending by earlier HIP calls of the same thread is reported
 *    the same way).
 *  - Thread-safe: calls share no mutable state.
 */
#ifndef CABF_H
#define CABF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden symbol visibility; these are its exports. */
#pragma GCC visibility push(default)

/* Same declaration as HIP's own; a compatible repeat of the typedef is legal. */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
  CABF_OK = 0,
  CABF_EINVAL = -1,        /* bad argument: null pointer, size, range           */
  CABF_EUNSUPPORTED = -2,  /* valid but not built: P != 8, head_dim, nb too big */
  CABF_EWORKSPACE = -3,    /* workspace smaller than cabf_mask_workspace_bytes  */
  CABF_EHIP = -4           /* the HIP runtime reported an error at launch       */
} cabf_status;

typedef enum {
  CABF_BF16 = 0,           /* bfloat16 tensors, fp32 accumulation and softmax   */
  CABF_F32 = 1,            /* float32 tensors                                   */
  /* Not dtypes: they make every 32-bit int a value of the type, so that any
   * int a caller passes can be read and rejected (CABF_EINVAL). */
  CABF_DTYPE_RANGE_LOW_ = -2147483647 - 1,
  CABF_DTYPE_RANGE_HIGH_ = 2147483647
} cabf_dtype;

/* Flags of cabf_bsa_forward. */
enum {
  CABF_BSA_DETERMINISTIC = 1u   /* visit each row's blocks in list order */
};

/* Layer geometry. The padded grid and block count are derived:
 *   Ty = ceil(H/P), Tx = ceil(W/P), Hp = Ty*P, Wp = Tx*P,
 *   nb = T*Ty*Tx blocks of P*P tokens, N = nb*P*P.
 * The library supports P = 8 (64-token blocks) and head_dim 64 or 128.
 * Block b = (t*Ty + ty)*Tx + tx is patch (ty, tx) of frame t. */
typedef struct {
  int32_t batch;
  int32_t heads;
  int32_t head_dim;
  int32_t T, H, W;   /* real latent grid: frames, rows, columns */
  int32_t P;         /* patch side */
} cabf_geom;

/* Sliding-tile window (NABLA summary, Methodology item 3: the final mask is
 * the adaptive mask OR a static sliding-tile-attention window). Query block
 * (t, ty, tx) also keeps every key block within +-dt frames, +-dy patch rows
 * and +-dx patch columns, clipped at the grid edges. enabled = 0 disables. */
typedef struct {
  int32_t enabled;
  int32_t dt, dy, dx;
} cabf_sta;

/* Derived sizes of a geometry (host call, no GPU needed). Any output pointer
 * (host) may be NULL. Returns CABF_OK, CABF_EINVAL or CABF_EUNSUPPORTED. */
int cabf_geom_sizes(const cabf_geom* g, int64_t* tokens_raster, int64_t* tokens_padded,
                    int32_t* n_blocks, int32_t* Hp, int32_t* Wp);

/* Fractal flattening (NABLA summary, Methodology item 1): reorders the input
 * sequence so the tokens of each P x P patch are contiguous while frames keep
 * their order. Token (t, y, x) moves to
 *   n' = ((t*Ty + y/P)*Tx + x/P)*P*P + (y%P)*P + x%P;
 * the N - T*H*W pad slots are written with zeros.
 * q, k, v: raster [B, heads, T*H*W, head_dim] of `dtype` (input);
 * qp, kp, vp: reordered [B, heads, N, head_dim] (output, no overlap with the
 * inputs). A (source, destination) pair may be skipped by passing NULL for
 * both; one NULL of a pair is CABF_EINVAL. Bitwise copy. */
int cabf_permute(const cabf_geom* g, cabf_dtype dtype,
                 const void* q, const void* k, const void* v,
                 void* qp, void* kp, void* vp, hipStream_t stream);

/* cabf_permute fused with step 1 of cabf_build_block_mask (NABLA summary,
 * Methodology items 1-2: the reordered Q and K are pooled per 64-token block;
 * doing both in one pass reads Q and K once instead of twice). Writes qp,
 * kp, vp exactly as cabf_permute does and, into `workspace`, the fp32 means
 * Qb, Kb of the real tokens of every block, for cabf_build_block_mask_pooled.
 * q, k, qp, kp are required; v and vp may both be NULL. workspace: at least
 * cabf_mask_workspace_bytes(g) bytes, 256-byte aligned, the same buffer then
 * handed to cabf_build_block_mask_pooled on the same stream, untouched in
 * between. Supports nb <= 8192 (else CABF_EUNSUPPORTED). The means are summed
 * in a fixed order, so they are bit-identical from run to run but may differ
 * in the last bits from the ones cabf_build_block_mask computes. */
int cabf_permute_pool(const cabf_geom* g, cabf_dtype dtype,
                      const void* q, const void* k, const void* v,
                      void* qp, void* kp, void* vp, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Inverse of cabf_permute for the attention output (Sparse VideoGen2
 * summary, section 2A: undoing the token permutation restores the original
 * order). op: reordered [B, heads, N, head_dim] (input); o: raster
 * [B, heads, T*H*W, head_dim] (output). Pad rows of op are ignored. */
int cabf_unpermute(const cabf_geom* g, cabf_dtype dtype, const void* op, void* o,
                   hipStream_t stream);

/* Bytes of device workspace cabf_build_block_mask needs for `g` (0 on an
 * invalid geometry). Holds the pooled Q and K blocks and the block logits. */
size_t cabf_mask_workspace_bytes(const cabf_geom* g);

/* Adaptive block mask (NABLA summary, Methodology items 2-3):
 *  1. Qb_i, Kb_i = mean of the real tokens of block i of qp, kp (fp32);
 *  2. z_ij = scale * <Qb_i, Kb_j>, p_i. = softmax_j(z_i.) (fp32);
 *  3. order row i by p descending (ties: lower block index first) and keep
 *     the shortest prefix whose mass reaches 1 - thr; thr <= 0 keeps every
 *     block, thr >= 1 keeps one;
 *  4. if sta is non-NULL and enabled, OR in the sliding-tile window;
 *  5. write the kept blocks of row i in ascending order.
 * qp, kp: reordered [B, heads, N, head_dim] (input; pad slots are ignored).
 * scale > 0 (usually 1/sqrt(head_dim)); 0 <= thr <= 1.
 * sta: host pointer, may be NULL.
 * kv_count: [B, heads, nb] int32 (output) number of kept blocks per row, >= 1.
 * kv_index: [B, heads, nb, nb] int32 (output) row i's kept block indices in
 *   its first kv_count entries, ascending; later entries are left untouched.
 * block_prob: NULL, or [B, heads, nb, nb] fp32 (output) the probabilities p.
 * workspace: device buffer of at least cabf_mask_workspace_bytes(g) bytes,
 *   256-byte aligned, not shared with a concurrent call.
 * Supports nb <= 8192. */
int cabf_build_block_mask(const cabf_geom* g, cabf_dtype dtype,
                          const void* qp, const void* kp, float scale, float thr,
                          const cabf_sta* sta, int32_t* kv_count, int32_t* kv_index,
                          float* block_prob, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Fixed-budget variant of cabf_build_block_mask (DynamicRad summary,
 * "Dual-Mode Strategy", Static-Ratio mode: a fixed ratio of blocks is kept
 * per row; the page gives no ranking, so the blocks are ranked by the same
 * pooled block probabilities). Steps 1, 2, 4 and 5 of cabf_build_block_mask;
 * step 3 keeps the k most probable blocks of the row (ties to the lower
 * index; k >= nb keeps every block). For a keep ratio r use k = ceil(r * nb).
 * k >= 1, else CABF_EINVAL. Other arguments, outputs, workspace and limits
 * as for cabf_build_block_mask. */
int cabf_build_block_mask_topk(const cabf_geom* g, cabf_dtype dtype,
                               const void* qp, const void* kp, float scale, int32_t k,
                               const cabf_sta* sta, int32_t* kv_count, int32_t* kv_index,
                               float* block_prob, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Device bytes cabf_build_block_mask_noalloc keeps in a static array on
 * every GPU it runs on, for the life of the process. */
#define CABF_NOALLOC_SCRATCH_BYTES ((size_t)96 * 1024 * 1024)

/* cabf_build_block_mask without a workspace argument, for callers that
 * cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): it allocates nothing. Its
 * workspace is a static device array of CABF_NOALLOC_SCRATCH_BYTES on the
 * stream's GPU, through which the (batch, head) pairs pass a few at a time;
 * the results are the same as cabf_build_block_mask's, bit for bit. All
 * calls on one GPU share that array: calls that overlap on a GPU (two
 * streams or two threads at once) race and must be serialised by the
 * caller. A geometry whose single (batch, head) pair needs more than the
 * array (2 nb head_dim + nb * ceil64(nb) floats; nb above about 4,600 at
 * head_dim 128) returns CABF_EWORKSPACE before any launch. Other arguments,
 * outputs, errors and limits as for cabf_build_block_mask. */
int cabf_build_block_mask_noalloc(const cabf_geom* g, cabf_dtype dtype,
                                  const void* qp, const void* kp, float scale, float thr,
                                  const cabf_sta* sta, int32_t* kv_count, int32_t* kv_index,
                                  float* block_prob, hipStream_t stream);

/* Steps 2-5 of cabf_build_block_mask (k = 0: the CDF cut at thr) or of
 * cabf_build_block_mask_topk (k >= 1), from the block means that
 * cabf_permute_pool left in `workspace` (the same buffer, same geometry).
 * k < 0 is CABF_EINVAL. Outputs and limits as for cabf_build_block_mask. */
int cabf_build_block_mask_pooled(const cabf_geom* g, float scale, float thr, int32_t k,
                                 const cabf_sta* sta, int32_t* kv_count, int32_t* kv_index,
                                 float* block_prob, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Pure sliding-tile block lists (NABLA summary, comparison with static
 * methods: the STA-only configuration), with no content scores: row i keeps
 * exactly the window of cabf_build_block_mask step 4, ascending.
 * sta: host pointer, required and enabled, dt, dy, dx >= 0 (else
 * CABF_EINVAL). kv_count [B, heads, nb] and kv_index [B, heads, nb, nb] int32
 * (outputs, 4-byte aligned). No workspace; any nb the geometry allows. */
int cabf_build_sta_mask(const cabf_geom* g, const cabf_sta* sta,
                        int32_t* kv_count, int32_t* kv_index, hipStream_t stream);

/* Block-sparse attention forward (NABLA summary, Methodology item 2,
 * expansion bullet: the block mask, expanded to token resolution, decides
 * which tiles of attention are computed). For every reordered query row n of
 * block i, over the real keys m of the blocks kv_index[i][0 .. kv_count[i]):
 *   o_n   = sum_m exp(scale q_n.k_m) v_m / sum_m exp(scale q_n.k_m)
 *   lse_n = ln sum_m exp(scale q_n.k_m)
 * computed with an fp32 online softmax. bf16: Q K^T and P V on bf16 matrix
 * cores with fp32 accumulation, P rounded to bf16, o rounded to bf16.
 * A row with kv_count = 0 gets o = 0, lse = -inf.
 * qp, kp, vp: reordered [B, heads, N, head_dim] (input). Pad slots never
 *   change a real row's result, but must hold finite values (cabf_permute
 *   writes zeros there): a pad key's weight is exactly 0, and 0 times an
 *   infinite or NaN V value is NaN.
 * kv_count [B, heads, nb], kv_index [B, heads, nb, nb] (input; entries must be
 *   valid block indices; duplicates would be attended twice).
 * op: reordered [B, heads, N, head_dim] (output, pad rows included).
 * lse: NULL, or [B, heads, N] fp32 (output). scale > 0.
 * flags: 0 or CABF_BSA_DETERMINISTIC (other bits give CABF_EINVAL). With 0, a
 *   bf16 row may start its pass anywhere in its list (chosen from the device
 *   clock so that concurrently running rows read the same K/V blocks, which
 *   then stay in L2) and wraps around; the result is the same softmax sum in
 *   another order, so it may differ from run to run in the last bits.
 *   CABF_BSA_DETERMINISTIC walks every list from its first entry and gives
 *   bit-identical results on every run. fp32, and bf16 rows of 2048 blocks
 *   or more (long lists, which run fastest in list order), are always
 *   deterministic. */
int cabf_bsa_forward(const cabf_geom* g, cabf_dtype dtype,
                     const void* qp, const void* kp, const void* vp,
                     const int32_t* kv_count, const int32_t* kv_index, float scale,
                     void* op, float* lse, unsigned flags, hipStream_t stream);

/* cabf_bsa_forward restricted to a set of query blocks (HSA summary,
 * section 2.2, KV-cache synchronisation: only the active tokens' queries are
 * computed, each attending over all of K and V; here the active set is given
 * at block granularity, and each active block attends over its kept list).
 * q_blocks: [n_blocks] int32 global block ids g = (b*heads + h)*nb + i
 * (device); the rows of those blocks of op (and lse) are written exactly as
 * cabf_bsa_forward writes them, with the same flags; every other row is left
 * untouched. Ids outside [0, B*heads*nb) are skipped; a repeated id writes
 * the same rows twice (identical values under CABF_BSA_DETERMINISTIC).
 * n_blocks = 0 is a no-op. dtype: CABF_BF16 only (else CABF_EUNSUPPORTED);
 * B*heads*nb must fit in int32 (else CABF_EUNSUPPORTED). Other arguments as
 * for cabf_bsa_forward. */
int cabf_bsa_forward_subset(const cabf_geom* g, cabf_dtype dtype,
                            const void* qp, const void* kp, const void* vp,
                            const int32_t* kv_count, const int32_t* kv_index,
                            const int32_t* q_blocks, int64_t n_blocks, float scale,
                            void* op, float* lse, unsigned flags, hipStream_t stream);

/* Bytes of workspace cabf_bsa_backward needs (0 if the geometry is
 * unsupported): fp32 D and base-2 lse per row, a kept-list bitmap, the
 * transposed lists (about B*heads*nb*nb*4 bytes) and the key blocks of each
 * head ordered by the length of their transposed lists. */
size_t cabf_bsa_backward_workspace_bytes(const cabf_geom* g);

/* Gradients of cabf_bsa_forward (NABLA summary, closing remarks: the sparse
 * attention serves training as well as inference). With a scalar loss of the
 * real output rows and dop = its gradient with respect to op: for a real
 * query row n of block i and the real keys m of i's kept blocks,
 *   P_nm = exp(scale q_n.k_m - lse_n), D_n = do_n . o_n,
 *   dS_nm = P_nm (do_n . v_m - D_n),
 *   dq_n = scale sum_m dS_nm k_m, dk_m = scale sum_n dS_nm q_n,
 *   dv_m = sum_n P_nm do_n.
 * Pad query rows do not contribute; pad rows of dq, dk, dv are zero. A row
 * whose lse is not finite (-inf: a row without kept keys) gets P = 0.
 * dtype: CABF_BF16 only (else CABF_EUNSUPPORTED). qp, kp, vp, op (the
 * forward's output) and dop: [B, heads, N, head_dim] bf16; lse: the
 * forward's [B, heads, N] fp32; kv_count / kv_index: the forward's lists
 * (inputs). Pad slots of the inputs must hold finite values, as for
 * cabf_bsa_forward (their weights are exactly 0). dqp, dkp, dvp:
 * [B, heads, N, head_dim] bf16 (outputs).
 * bf16 matrix products with fp32 accumulation.
 * flags: 0 or CABF_BSA_DETERMINISTIC (other bits give CABF_EINVAL), as for
 *   cabf_bsa_forward: with 0 each pass over a list starts at a clock-derived
 *   entry (the same sums in another order, so results may differ from run to
 *   run in the last bits); CABF_BSA_DETERMINISTIC walks the lists in order
 *   and gives bit-identical results on every run. */
int cabf_bsa_backward(const cabf_geom* g, cabf_dtype dtype, const void* qp, const void* kp,
                      const void* vp, const void* op, const float* lse, const void* dop,
                      const int32_t* kv_count, const int32_t* kv_index, float scale, void* dqp,
                      void* dkp, void* dvp, void* workspace, size_t workspace_bytes,
                      unsigned flags, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Semantic-permutation variant (Sparse VideoGen2 summary, Methodology A-C):
 * k-means clustering of Q and K, cluster-contiguous permutation, centroid
 * scores with top-p selection, attention over the selected cluster pairs.
 * ------------------------------------------------------------------------ */

/* batch x heads sequences of n tokens: tensors [batch, heads, n, head_dim]
 * row-major. head_dim 64 or 128; 1 <= n < 2^24 and batch*heads*n < 2^31. */
typedef struct {
  int32_t batch, heads, head_dim;
  int32_t n;
} cabf_seq;

/* Bytes of workspace cabf_kmeans needs for `clusters` clusters (0 if the
 * sizes are unsupported). */
size_t cabf_kmeans_workspace_bytes(const cabf_seq* s, int32_t clusters);

/* k-means of every (batch, head)'s tokens and the cluster permutation
 * (Methodology A). Lloyd's algorithm on the rows of x with squared Euclidean
 * distance: `iters` rounds of (assign every token to its nearest centroid,
 * ties to the lowest index; move every centroid to the mean of its members,
 * an empty cluster keeps its centroid), then a final assignment, so labels
 * are the nearest final centroids. Distances use the bf16 features exactly
 * and the centroids to about fp32 accuracy.
 * dtype: CABF_BF16 only (else CABF_EUNSUPPORTED).
 * x: [B, heads, n, d] bf16 (input).
 * init: [B, heads, clusters] int32 token indices of the initial centroids
 *   (input; the caller's random draw; values are clamped to [0, n)).
 * centroids: [B, heads, clusters, d] fp32 (output).
 * counts: [B, heads, clusters] int32 members per cluster (output).
 * labels: [B, heads, n] int32 cluster of every token (output).
 * perm: [B, heads, n] int32 (output): the tokens sorted by cluster, stable
 *   (a cluster's tokens keep their order); perm[i] = original index.
 * offsets: [B, heads, clusters + 1] int32 (output): cluster c occupies
 *   sorted positions offsets[c] .. offsets[c+1]-1.
 * 1 <= clusters <= min(n, 8192); iters >= 0. Results are deterministic. */
int cabf_kmeans(const cabf_seq* s, cabf_dtype dtype, const void* x, int32_t clusters,
                const int32_t* init, int32_t iters, float* centroids, int32_t* counts,
                int32_t* labels, int32_t* perm, int32_t* offsets, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/* Apply a per-(batch, head) permutation to token rows: xp[i] = x[perm[i]]
 * for i < n; rows n .. rows_out-1 of xp are set to zero (rows_out >= n).
 * x: [B, heads, n, d]; xp: [B, heads, rows_out, d]; bf16 or fp32; perm
 * entries are clamped to [0, n). */
int cabf_gather_rows(const cabf_seq* s, cabf_dtype dtype, const void* x, const int32_t* perm,
                     void* xp, int32_t rows_out, hipStream_t stream);

/* Undo it: x[perm[i]] = xp[i] for i < n (xp has rows_in >= n rows per
 * head). perm must be a permutation of 0 .. n-1 (repeated entries race). */
int cabf_scatter_rows(const cabf_seq* s, cabf_dtype dtype, const void* xp, int32_t rows_in,
                      const int32_t* perm, void* x, hipStream_t stream);

size_t cabf_cluster_select_workspace_bytes(const cabf_seq* s, int32_t cq, int32_t ck);

/* Centroid-based top-p selection (Methodology B). For query cluster a and
 * key cluster b: p_ab = |K_b| exp(scale <cq_a, ck_b>) / sum over b' (the
 * attention share of b's tokens when each is represented by its centroid;
 * empty clusters get 0); then the shortest prefix of row a sorted by p
 * (descending, ties to the lower index) whose mass reaches top_p is kept.
 * q_centroids [B, heads, cq, d], k_centroids [B, heads, ck, d] fp32 and
 * k_counts [B, heads, ck] int32 (inputs, e.g. from cabf_kmeans).
 * kv_count [B, heads, cq], kv_index [B, heads, cq, ck] int32 (outputs):
 * kept key clusters of each query cluster, ascending. probs: NULL or
 * [B, heads, cq, ck] fp32 (output). 0 < top_p <= 1, scale > 0,
 * 1 <= ck <= 8192. */
int cabf_cluster_select(const cabf_seq* s, int32_t cq, int32_t ck, const float* q_centroids,
                        const float* k_centroids, const int32_t* k_counts, float scale,
                        float top_p, int32_t* kv_count, int32_t* kv_index, float* probs,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t cabf_cluster_attention_workspace_bytes(const cabf_seq* s, int32_t cq, int32_t ck);

/* Attention over the selected cluster pairs (Methodology C): every query
 * row i of cluster a (permuted positions q_offsets[a] .. q_offsets[a+1]-1)
 * attends to the key rows of its kept key clusters b (positions
 * k_offsets[b] .. k_offsets[b+1]-1 of the permuted K and V):
 *   o_i = sum_m exp(scale q_i.k_m) v_m / sum_m exp(scale q_i.k_m),
 *   lse_i = ln sum_m exp(scale q_i.k_m),
 * with bf16 matrix products, fp32 softmax, o rounded to bf16.
 * dtype: CABF_BF16 only. qp, kp, vp: [B, heads, n + 64, d] permuted rows
 * (cabf_gather_rows with rows_out = n + 64: the 64 zero rows keep the
 * kernel's whole-tile loads in bounds). q_offsets [B, heads, cq + 1],
 * k_offsets [B, heads, ck + 1] (e.g. cabf_kmeans' offsets; clamped to
 * [0, n]), kv_count / kv_index as from cabf_cluster_select.
 * op: [B, heads, n + 64, d] bf16 (output, rows < n written); lse: NULL or
 * [B, heads, n + 64] fp32 (output, rows < n written). Rows of a query
 * cluster that keeps nothing get o = 0, lse = -inf. */
int cabf_cluster_attention(const cabf_seq* s, cabf_dtype dtype, int32_t cq, int32_t ck,
                           const void* qp, const void* kp, const void* vp,
                           const int32_t* q_offsets, const int32_t* k_offsets,
                           const int32_t* kv_count, const int32_t* kv_index, float scale,
                           void* op, float* lse, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* cabf_status_string(int status);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* CABF_H */
