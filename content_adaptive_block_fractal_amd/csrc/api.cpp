// C ABI of libcabf: argument validation and dispatch to the kernel launchers.
// Declared and documented in include/cabf.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>

#include "cabf.h"
#include "geometry.hpp"
#include "launch.hpp"
#include "svg.hpp"

namespace {

using cabf::Geo;

int make_geo(const cabf_geom* g, Geo* out) {
  if (g == nullptr) return CABF_EINVAL;
  if (g->batch < 1 || g->heads < 1 || g->head_dim < 1 || g->T < 1 || g->H < 1 || g->W < 1 ||
      g->P < 1)
    return CABF_EINVAL;
  if (g->P != cabf::kP) return CABF_EUNSUPPORTED;
  if (g->head_dim != 64 && g->head_dim != 128) return CABF_EUNSUPPORTED;
  Geo r{};
  r.B = g->batch;
  r.heads = g->heads;
  r.D = g->head_dim;
  r.T = g->T;
  r.H = g->H;
  r.W = g->W;
  const int64_t Ty = (static_cast<int64_t>(g->H) + cabf::kP - 1) / cabf::kP;
  const int64_t Tx = (static_cast<int64_t>(g->W) + cabf::kP - 1) / cabf::kP;
  const int64_t nb = static_cast<int64_t>(g->T) * Ty * Tx;
  if (nb > (int64_t{1} << 24)) return CABF_EUNSUPPORTED;
  r.Ty = static_cast<int>(Ty);
  r.Tx = static_cast<int>(Tx);
  r.nb = static_cast<int>(nb);
  r.BH = static_cast<int64_t>(g->batch) * g->heads;
  r.Nv = static_cast<int64_t>(g->T) * g->H * g->W;
  r.N = nb * cabf::kBlock;
  // every byte offset of a [B, heads, N, 128] fp32 tensor and of the
  // [B, heads, nb, nb] lists must fit comfortably in int64
  const double elems = static_cast<double>(r.BH) * static_cast<double>(r.N) * 128.0 * 4.0;
  const double lists = static_cast<double>(r.BH) * static_cast<double>(nb) * nb * 4.0;
  if (elems > 4.0e18 || lists > 4.0e18) return CABF_EINVAL;
  *out = r;
  return CABF_OK;
}

int elem_bytes(cabf_dtype dt) {
  if (dt == CABF_BF16) return 2;
  if (dt == CABF_F32) return 4;
  return 0;
}

int launched() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? CABF_OK : CABF_EHIP;
}

// Arguments of the mask entry points, validated (CABF_OK or the status).
struct MaskCall {
  Geo geo;
  bool sta_on = false;
  int dt = 0, dy = 0, dx = 0;
};

int check_mask(const cabf_geom* g, cabf_dtype dtype, const void* qp, const void* kp, bool pooled,
               float scale, float thr, const cabf_sta* sta, const int32_t* kv_count,
               const int32_t* kv_index, const float* block_prob, MaskCall* c) {
  const int st = make_geo(g, &c->geo);
  if (st != CABF_OK) return st;
  if (!pooled && (elem_bytes(dtype) == 0 || qp == nullptr || kp == nullptr)) return CABF_EINVAL;
  if (kv_count == nullptr || kv_index == nullptr) return CABF_EINVAL;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return CABF_EINVAL;
  if (!(thr >= 0.0f && thr <= 1.0f)) return CABF_EINVAL;
  if (reinterpret_cast<uintptr_t>(qp) % 16 || reinterpret_cast<uintptr_t>(kp) % 16 ||
      reinterpret_cast<uintptr_t>(kv_count) % 4 || reinterpret_cast<uintptr_t>(kv_index) % 4 ||
      reinterpret_cast<uintptr_t>(block_prob) % 4)
    return CABF_EINVAL;
  if (sta != nullptr && sta->enabled) {
    if (sta->dt < 0 || sta->dy < 0 || sta->dx < 0) return CABF_EINVAL;
    c->sta_on = true;
    c->dt = sta->dt;
    c->dy = sta->dy;
    c->dx = sta->dx;
  }
  if (c->geo.nb > cabf::kMaxBlocks) return CABF_EUNSUPPORTED;
  return CABF_OK;
}

// Shared by the CDF (topk = 0) and the top-k entry points.
// pooled: the block means are already in the workspace (cabf_permute_pool),
// qp, kp and dtype are unused
int build_mask(const cabf_geom* g, cabf_dtype dtype, const void* qp, const void* kp, bool pooled,
               float scale, float thr, int topk, const cabf_sta* sta, int32_t* kv_count,
               int32_t* kv_index, float* block_prob, void* workspace, size_t workspace_bytes,
               hipStream_t stream) {
  MaskCall c;
  const int st = check_mask(g, dtype, qp, kp, pooled, scale, thr, sta, kv_count, kv_index,
                            block_prob, &c);
  if (st != CABF_OK) return st;
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 256) return CABF_EINVAL;
  if (workspace_bytes < cabf::mask_workspace_layout(c.geo).total) return CABF_EWORKSPACE;
  if (pooled)
    cabf::launch_mask_from_pooled(c.geo, scale, thr, topk, c.sta_on, c.dt, c.dy, c.dx, kv_count,
                                  kv_index, block_prob, workspace, stream);
  else
    cabf::launch_build_block_mask(c.geo, dtype == CABF_BF16, qp, kp, scale, thr, topk, c.sta_on,
                                  c.dt, c.dy, c.dx, kv_count, kv_index, block_prob, workspace,
                                  stream);
  return launched();
}

// q, k, v, qp, kp, vp for the permute entries: CABF_OK or the status
int check_pairs(const void* const src[3], void* const dst[3], int* pairs) {
  *pairs = 0;
  for (int i = 0; i < 3; ++i) {
    if ((src[i] == nullptr) != (dst[i] == nullptr)) return CABF_EINVAL;
    if (src[i] != nullptr) {
      ++*pairs;
      if (reinterpret_cast<uintptr_t>(src[i]) % 16 || reinterpret_cast<uintptr_t>(dst[i]) % 16)
        return CABF_EINVAL;
    }
  }
  return CABF_OK;
}

// cabf_seq -> (BH, n, D); CABF_OK or the status to return
int check_seq(const cabf_seq* s, int64_t* BH) {
  if (s == nullptr) return CABF_EINVAL;
  if (s->batch < 1 || s->heads < 1 || s->n < 1 || s->head_dim < 1) return CABF_EINVAL;
  if (s->head_dim != 64 && s->head_dim != 128) return CABF_EUNSUPPORTED;
  if (s->n >= (1 << 24)) return CABF_EUNSUPPORTED;
  const int64_t bh = static_cast<int64_t>(s->batch) * s->heads;
  if (bh * s->n >= (int64_t{1} << 31)) return CABF_EUNSUPPORTED;
  *BH = bh;
  return CABF_OK;
}

bool misaligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a != 0; }

}  // namespace

extern "C" {

int cabf_geom_sizes(const cabf_geom* g, int64_t* tokens_raster, int64_t* tokens_padded,
                    int32_t* n_blocks, int32_t* Hp, int32_t* Wp) {
  Geo geo;
  const int st = make_geo(g, &geo);
  if (st != CABF_OK) return st;
  if (tokens_raster) *tokens_raster = geo.Nv;
  if (tokens_padded) *tokens_padded = geo.N;
  if (n_blocks) *n_blocks = geo.nb;
  if (Hp) *Hp = geo.Ty * cabf::kP;
  if (Wp) *Wp = geo.Tx * cabf::kP;
  return CABF_OK;
}

int cabf_permute(const cabf_geom* g, cabf_dtype dtype, const void* q, const void* k,
                 const void* v, void* qp, void* kp, void* vp, hipStream_t stream) {
  Geo geo;
  const int st = make_geo(g, &geo);
  if (st != CABF_OK) return st;
  const int eb = elem_bytes(dtype);
  if (eb == 0) return CABF_EINVAL;
  const void* src[3] = {q, k, v};
  void* dst[3] = {qp, kp, vp};
  int pairs = 0;
  if (check_pairs(src, dst, &pairs) != CABF_OK) return CABF_EINVAL;
  if (pairs == 0) return CABF_OK;
  cabf::launch_permute(geo, eb, src, dst, stream);
  return launched();
}

int cabf_permute_pool(const cabf_geom* g, cabf_dtype dtype, const void* q, const void* k,
                      const void* v, void* qp, void* kp, void* vp, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  Geo geo;
  const int st = make_geo(g, &geo);
  if (st != CABF_OK) return st;
  const int eb = elem_bytes(dtype);
  if (eb == 0 || q == nullptr || k == nullptr || workspace == nullptr) return CABF_EINVAL;
  const void* src[3] = {q, k, v};
  void* dst[3] = {qp, kp, vp};
  int pairs = 0;
  if (check_pairs(src, dst, &pairs) != CABF_OK) return CABF_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return CABF_EINVAL;
  if (geo.nb > cabf::kMaxBlocks) return CABF_EUNSUPPORTED;
  const cabf::MaskWorkspace lay = cabf::mask_workspace_layout(geo);
  if (workspace_bytes < lay.total) return CABF_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  cabf::launch_permute_pool(geo, eb, src, dst, reinterpret_cast<float*>(ws + lay.qb_off),
                            reinterpret_cast<float*>(ws + lay.kb_off), stream);
  return launched();
}

int cabf_unpermute(const cabf_geom* g, cabf_dtype dtype, const void* op, void* o,
                   hipStream_t stream) {
  Geo geo;
  const int st = make_geo(g, &geo);
  if (st != CABF_OK) return st;
  const int eb = elem_bytes(dtype);
  if (eb == 0 || op == nullptr || o == nullptr) return CABF_EINVAL;
  if (reinterpret_cast<uintptr_t>(op) % 16 || reinterpret_cast<uintptr_t>(o) % 16)
    return CABF_EINVAL;
  cabf::launch_unpermute(geo, eb, op, o, stream);
  return launched();
}

size_t cabf_mask_workspace_bytes(const cabf_geom* g) {
  Geo geo;
  if (make_geo(g, &geo) != CABF_OK) return 0;
  return cabf::mask_workspace_layout(geo).total;
}

int cabf_build_block_mask(const cabf_geom* g, cabf_dtype dtype, const void* qp, const void* kp,
                          float scale, float thr, const cabf_sta* sta, int32_t* kv_count,
                          int32_t* kv_index, float* block_prob, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return build_mask(g, dtype, qp, kp, false, scale, thr, 0, sta, kv_count, kv_index, block_prob,
                    workspace, workspace_bytes, stream);
}

int cabf_build_block_mask_noalloc(const cabf_geom* g, cabf_dtype dtype, const void* qp,
                                  const void* kp, float scale, float thr, const cabf_sta* sta,
                                  int32_t* kv_count, int32_t* kv_index, float* block_prob,
                                  hipStream_t stream) {
  MaskCall c;
  const int st = check_mask(g, dtype, qp, kp, false, scale, thr, sta, kv_count, kv_index,
                            block_prob, &c);
  if (st != CABF_OK) return st;
  if (cabf::noalloc_pairs_per_pass(c.geo) < 1) return CABF_EWORKSPACE;
  const int ls = cabf::launch_build_block_mask_noalloc(c.geo, elem_bytes(dtype), qp, kp, scale,
                                                       thr, c.sta_on, c.dt, c.dy, c.dx, kv_count,
                                                       kv_index, block_prob, stream);
  if (ls != CABF_OK) return ls;
  return launched();
}

int cabf_build_block_mask_topk(const cabf_geom* g, cabf_dtype dtype, const void* qp,
                               const void* kp, float scale, int32_t k, const cabf_sta* sta,
                               int32_t* kv_count, int32_t* kv_index, float* block_prob,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (k < 1) return CABF_EINVAL;
  return build_mask(g, dtype, qp, kp, false, scale, 0.0f, k, sta, kv_count, kv_index, block_prob,
                    workspace, workspace_bytes, stream);
}

int cabf_build_block_mask_pooled(const cabf_geom* g, float scale, float thr, int32_t k,
                                 const cabf_sta* sta, int32_t* kv_count, int32_t* kv_index,
                                 float* block_prob, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (k < 0) return CABF_EINVAL;
  return build_mask(g, CABF_BF16, nullptr, nullptr, true, scale, k > 0 ? 0.0f : thr, k, sta,
                    kv_count, kv_index, block_prob, workspace, workspace_bytes, stream);
}

int cabf_build_sta_mask(const cabf_geom* g, const cabf_sta* sta, int32_t* kv_count,
                        int32_t* kv_index, hipStream_t stream) {
  Geo geo;
  const int st = make_geo(g, &geo);
  if (st != CABF_OK) return st;
  if (sta == nullptr || !sta->enabled || sta->dt < 0 || sta->dy < 0 || sta->dx < 0 ||
      kv_count == nullptr || kv_index == nullptr)
    return CABF_EINVAL;
  if (reinterpret_cast<uintptr_t>(kv_count) % 4 || reinterpret_cast<uintptr_t>(kv_index) % 4)
    return CABF_EINVAL;
  cabf::launch_build_sta_mask(geo, sta->dt, sta->dy, sta->dx, kv_count, kv_index, stream);
  return launched();
}

int cabf_bsa_forward(const cabf_geom* g, cabf_dtype dtype, const void* qp, const void* kp,
                     const void* vp, const int32_t* kv_count, const int32_t* kv_index,
                     float scale, void* op, float* lse, unsigned flags, hipStream_t stream) {
  Geo geo;
  const int st = make_geo(g, &geo);
  if (st != CABF_OK) return st;
  if (elem_bytes(dtype) == 0) return CABF_EINVAL;
  if (qp == nullptr || kp == nullptr || vp == nullptr || kv_count == nullptr ||
      kv_index == nullptr || op == nullptr)
    return CABF_EINVAL;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return CABF_EINVAL;
  if ((flags & ~static_cast<unsigned>(CABF_BSA_DETERMINISTIC)) != 0) return CABF_EINVAL;
  if (reinterpret_cast<uintptr_t>(qp) % 16 || reinterpret_cast<uintptr_t>(kp) % 16 ||
      reinterpret_cast<uintptr_t>(vp) % 16 || reinterpret_cast<uintptr_t>(op) % 16 ||
      reinterpret_cast<uintptr_t>(kv_count) % 4 || reinterpret_cast<uintptr_t>(kv_index) % 4 ||
      reinterpret_cast<uintptr_t>(lse) % 4)
    return CABF_EINVAL;
  cabf::launch_bsa_forward(geo, dtype == CABF_BF16, qp, kp, vp, kv_count, kv_index, scale, op,
                           lse, (flags & CABF_BSA_DETERMINISTIC) == 0, stream);
  return launched();
}

int cabf_bsa_forward_subset(const cabf_geom* g, cabf_dtype dtype, const void* qp, const void* kp,
                            const void* vp, const int32_t* kv_count, const int32_t* kv_index,
                            const int32_t* q_blocks, int64_t n_blocks, float scale, void* op,
                            float* lse, unsigned flags, hipStream_t stream) {
  Geo geo;
  const int st = make_geo(g, &geo);
  if (st != CABF_OK) return st;
  if (dtype != CABF_BF16) return elem_bytes(dtype) == 0 ? CABF_EINVAL : CABF_EUNSUPPORTED;
  if (geo.BH * geo.nb > 0x7fffffff) return CABF_EUNSUPPORTED;   // int32 block ids
  if (n_blocks < 0 || n_blocks > 0x7fffffff) return CABF_EINVAL;
  if (qp == nullptr || kp == nullptr || vp == nullptr || kv_count == nullptr ||
      kv_index == nullptr || op == nullptr || (q_blocks == nullptr && n_blocks > 0))
    return CABF_EINVAL;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return CABF_EINVAL;
  if ((flags & ~static_cast<unsigned>(CABF_BSA_DETERMINISTIC)) != 0) return CABF_EINVAL;
  if (reinterpret_cast<uintptr_t>(qp) % 16 || reinterpret_cast<uintptr_t>(kp) % 16 ||
      reinterpret_cast<uintptr_t>(vp) % 16 || reinterpret_cast<uintptr_t>(op) % 16 ||
      reinterpret_cast<uintptr_t>(kv_count) % 4 || reinterpret_cast<uintptr_t>(kv_index) % 4 ||
      reinterpret_cast<uintptr_t>(lse) % 4 || reinterpret_cast<uintptr_t>(q_blocks) % 4)
    return CABF_EINVAL;
  if (n_blocks == 0) return CABF_OK;
  cabf::launch_bsa_forward_subset(geo, qp, kp, vp, kv_count, kv_index, q_blocks, n_blocks, scale,
                                  op, lse, (flags & CABF_BSA_DETERMINISTIC) == 0, stream);
  return launched();
}

size_t cabf_bsa_backward_workspace_bytes(const cabf_geom* g) {
  Geo geo;
  if (make_geo(g, &geo) != CABF_OK) return 0;
  return cabf::bwd_workspace_layout(geo).total;
}

int cabf_bsa_backward(const cabf_geom* g, cabf_dtype dtype, const void* qp, const void* kp,
                      const void* vp, const void* op, const float* lse, const void* dop,
                      const int32_t* kv_count, const int32_t* kv_index, float scale, void* dqp,
                      void* dkp, void* dvp, void* workspace, size_t workspace_bytes,
                      unsigned flags, hipStream_t stream) {
  Geo geo;
  const int st = make_geo(g, &geo);
  if (st != CABF_OK) return st;
  if (elem_bytes(dtype) == 0) return CABF_EINVAL;
  if (dtype != CABF_BF16) return CABF_EUNSUPPORTED;
  if ((flags & ~static_cast<unsigned>(CABF_BSA_DETERMINISTIC)) != 0) return CABF_EINVAL;
  if (qp == nullptr || kp == nullptr || vp == nullptr || op == nullptr || lse == nullptr ||
      dop == nullptr || kv_count == nullptr || kv_index == nullptr || dqp == nullptr ||
      dkp == nullptr || dvp == nullptr || workspace == nullptr)
    return CABF_EINVAL;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return CABF_EINVAL;
  if (misaligned(qp, 16) || misaligned(kp, 16) || misaligned(vp, 16) || misaligned(op, 16) ||
      misaligned(dop, 16) || misaligned(dqp, 16) || misaligned(dkp, 16) || misaligned(dvp, 16) ||
      misaligned(lse, 4) || misaligned(kv_count, 4) || misaligned(kv_index, 4) ||
      misaligned(workspace, 256))
    return CABF_EINVAL;
  if (workspace_bytes < cabf::bwd_workspace_layout(geo).total) return CABF_EWORKSPACE;
  cabf::launch_bsa_backward(geo, qp, kp, vp, op, lse, dop, kv_count, kv_index, scale, dqp, dkp,
                            dvp, workspace, (flags & CABF_BSA_DETERMINISTIC) == 0, stream);
  return launched();
}

size_t cabf_kmeans_workspace_bytes(const cabf_seq* s, int32_t clusters) {
  int64_t BH = 0;
  if (check_seq(s, &BH) != CABF_OK || clusters < 1 || clusters > s->n ||
      clusters > cabf::kMaxBlocks)
    return 0;
  return cabf::kmeans_workspace_layout(BH, s->n, clusters, s->head_dim).total;
}

int cabf_kmeans(const cabf_seq* s, cabf_dtype dtype, const void* x, int32_t clusters,
                const int32_t* init, int32_t iters, float* centroids, int32_t* counts,
                int32_t* labels, int32_t* perm, int32_t* offsets, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  int64_t BH = 0;
  const int st = check_seq(s, &BH);
  if (st != CABF_OK) return st;
  if (elem_bytes(dtype) == 0) return CABF_EINVAL;
  if (dtype != CABF_BF16) return CABF_EUNSUPPORTED;
  if (x == nullptr || init == nullptr || centroids == nullptr || counts == nullptr ||
      labels == nullptr || perm == nullptr || offsets == nullptr || workspace == nullptr)
    return CABF_EINVAL;
  if (clusters < 1 || clusters > s->n || iters < 0) return CABF_EINVAL;
  if (clusters > cabf::kMaxBlocks) return CABF_EUNSUPPORTED;
  if (misaligned(x, 16) || misaligned(init, 4) || misaligned(centroids, 16) ||
      misaligned(counts, 4) || misaligned(labels, 4) || misaligned(perm, 4) ||
      misaligned(offsets, 4) || misaligned(workspace, 256))
    return CABF_EINVAL;
  if (workspace_bytes < cabf::kmeans_workspace_layout(BH, s->n, clusters, s->head_dim).total)
    return CABF_EWORKSPACE;
  if (cabf::launch_kmeans(BH, s->n, s->head_dim, clusters, iters, x, init, centroids, counts,
                          labels, perm, offsets, workspace, stream) != 0)
    return CABF_EHIP;
  return launched();
}

int cabf_gather_rows(const cabf_seq* s, cabf_dtype dtype, const void* x, const int32_t* perm,
                     void* xp, int32_t rows_out, hipStream_t stream) {
  int64_t BH = 0;
  const int st = check_seq(s, &BH);
  if (st != CABF_OK) return st;
  const int eb = elem_bytes(dtype);
  if (eb == 0 || x == nullptr || perm == nullptr || xp == nullptr || rows_out < s->n)
    return CABF_EINVAL;
  if (BH * rows_out >= (int64_t{1} << 31)) return CABF_EUNSUPPORTED;
  if (misaligned(x, 16) || misaligned(xp, 16) || misaligned(perm, 4)) return CABF_EINVAL;
  cabf::launch_gather_rows(BH, s->n, rows_out, s->head_dim * eb, x, perm, xp, stream);
  return launched();
}

int cabf_scatter_rows(const cabf_seq* s, cabf_dtype dtype, const void* xp, int32_t rows_in,
                      const int32_t* perm, void* x, hipStream_t stream) {
  int64_t BH = 0;
  const int st = check_seq(s, &BH);
  if (st != CABF_OK) return st;
  const int eb = elem_bytes(dtype);
  if (eb == 0 || x == nullptr || perm == nullptr || xp == nullptr || rows_in < s->n)
    return CABF_EINVAL;
  if (BH * rows_in >= (int64_t{1} << 31)) return CABF_EUNSUPPORTED;
  if (misaligned(x, 16) || misaligned(xp, 16) || misaligned(perm, 4)) return CABF_EINVAL;
  cabf::launch_scatter_rows(BH, s->n, rows_in, s->head_dim * eb, xp, perm, x, stream);
  return launched();
}

size_t cabf_cluster_select_workspace_bytes(const cabf_seq* s, int32_t cq, int32_t ck) {
  int64_t BH = 0;
  if (check_seq(s, &BH) != CABF_OK || cq < 1 || ck < 1 || ck > cabf::kMaxBlocks) return 0;
  return cabf::cluster_select_workspace_layout(BH, cq, ck).total;
}

int cabf_cluster_select(const cabf_seq* s, int32_t cq, int32_t ck, const float* q_centroids,
                        const float* k_centroids, const int32_t* k_counts, float scale,
                        float top_p, int32_t* kv_count, int32_t* kv_index, float* probs,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int64_t BH = 0;
  const int st = check_seq(s, &BH);
  if (st != CABF_OK) return st;
  if (q_centroids == nullptr || k_centroids == nullptr || k_counts == nullptr ||
      kv_count == nullptr || kv_index == nullptr || workspace == nullptr)
    return CABF_EINVAL;
  if (cq < 1 || ck < 1) return CABF_EINVAL;
  if (ck > cabf::kMaxBlocks) return CABF_EUNSUPPORTED;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return CABF_EINVAL;
  if (!(top_p > 0.0f && top_p <= 1.0f)) return CABF_EINVAL;
  if (misaligned(q_centroids, 4) || misaligned(k_centroids, 4) || misaligned(k_counts, 4) ||
      misaligned(kv_count, 4) || misaligned(kv_index, 4) || misaligned(probs, 4) ||
      misaligned(workspace, 256))
    return CABF_EINVAL;
  if (workspace_bytes < cabf::cluster_select_workspace_layout(BH, cq, ck).total)
    return CABF_EWORKSPACE;
  cabf::launch_cluster_select(BH, cq, ck, s->head_dim, q_centroids, k_centroids, k_counts, scale,
                              top_p, kv_count, kv_index, probs, workspace, stream);
  return launched();
}

size_t cabf_cluster_attention_workspace_bytes(const cabf_seq* s, int32_t cq, int32_t ck) {
  int64_t BH = 0;
  if (check_seq(s, &BH) != CABF_OK || cq < 1 || ck < 1 || cq > s->n || ck > s->n) return 0;
  return cabf::cluster_attention_workspace_layout(BH, s->n, cq, ck).total;
}

int cabf_cluster_attention(const cabf_seq* s, cabf_dtype dtype, int32_t cq, int32_t ck,
                           const void* qp, const void* kp, const void* vp,
                           const int32_t* q_offsets, const int32_t* k_offsets,
                           const int32_t* kv_count, const int32_t* kv_index, float scale,
                           void* op, float* lse, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  int64_t BH = 0;
  const int st = check_seq(s, &BH);
  if (st != CABF_OK) return st;
  if (elem_bytes(dtype) == 0) return CABF_EINVAL;
  if (dtype != CABF_BF16) return CABF_EUNSUPPORTED;
  if (qp == nullptr || kp == nullptr || vp == nullptr || q_offsets == nullptr ||
      k_offsets == nullptr || kv_count == nullptr || kv_index == nullptr || op == nullptr ||
      workspace == nullptr)
    return CABF_EINVAL;
  if (cq < 1 || ck < 1 || cq > s->n || ck > s->n) return CABF_EINVAL;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return CABF_EINVAL;
  if (BH * (s->n + cabf::kBlock) >= (int64_t{1} << 31)) return CABF_EUNSUPPORTED;
  if (misaligned(qp, 16) || misaligned(kp, 16) || misaligned(vp, 16) || misaligned(op, 16) ||
      misaligned(q_offsets, 4) || misaligned(k_offsets, 4) || misaligned(kv_count, 4) ||
      misaligned(kv_index, 4) || misaligned(lse, 4) || misaligned(workspace, 256))
    return CABF_EINVAL;
  if (workspace_bytes < cabf::cluster_attention_workspace_layout(BH, s->n, cq, ck).total)
    return CABF_EWORKSPACE;
  cabf::launch_cluster_attention(BH, s->n, s->head_dim, cq, ck, qp, kp, vp, q_offsets, k_offsets,
                                 kv_count, kv_index, scale, op, lse, workspace, stream);
  return launched();
}

const char* cabf_status_string(int status) {
  switch (status) {
    case CABF_OK: return "ok";
    case CABF_EINVAL: return "invalid argument";
    case CABF_EUNSUPPORTED: return "unsupported configuration";
    case CABF_EWORKSPACE: return "workspace too small";
    case CABF_EHIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

}  // extern "C"
