// C ABI of libcabf: argument validation and dispatch to the kernel launchers.
// Declared and documented in include/cabf.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>

#include "cabf.h"
#include "geometry.hpp"
#include "launch.hpp"

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

// Shared by the CDF (topk = 0) and the top-k entry points.
int build_mask(const cabf_geom* g, cabf_dtype dtype, const void* qp, const void* kp, float scale,
               float thr, int topk, const cabf_sta* sta, int32_t* kv_count, int32_t* kv_index,
               float* block_prob, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Geo geo;
  const int st = make_geo(g, &geo);
  if (st != CABF_OK) return st;
  if (elem_bytes(dtype) == 0) return CABF_EINVAL;
  if (qp == nullptr || kp == nullptr || kv_count == nullptr || kv_index == nullptr ||
      workspace == nullptr)
    return CABF_EINVAL;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return CABF_EINVAL;
  if (!(thr >= 0.0f && thr <= 1.0f)) return CABF_EINVAL;
  if (reinterpret_cast<uintptr_t>(qp) % 16 || reinterpret_cast<uintptr_t>(kp) % 16 ||
      reinterpret_cast<uintptr_t>(workspace) % 256 || reinterpret_cast<uintptr_t>(kv_count) % 4 ||
      reinterpret_cast<uintptr_t>(kv_index) % 4 || reinterpret_cast<uintptr_t>(block_prob) % 4)
    return CABF_EINVAL;
  bool sta_on = false;
  int dt = 0, dy = 0, dx = 0;
  if (sta != nullptr && sta->enabled) {
    if (sta->dt < 0 || sta->dy < 0 || sta->dx < 0) return CABF_EINVAL;
    sta_on = true;
    dt = sta->dt;
    dy = sta->dy;
    dx = sta->dx;
  }
  if (geo.nb > cabf::kMaxBlocks) return CABF_EUNSUPPORTED;
  if (workspace_bytes < cabf::mask_workspace_layout(geo).total) return CABF_EWORKSPACE;
  cabf::launch_build_block_mask(geo, dtype == CABF_BF16, qp, kp, scale, thr, topk, sta_on, dt, dy,
                                dx, kv_count, kv_index, block_prob, workspace, stream);
  return launched();
}

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
  for (int i = 0; i < 3; ++i) {
    if ((src[i] == nullptr) != (dst[i] == nullptr)) return CABF_EINVAL;
    if (src[i] != nullptr) {
      ++pairs;
      if (reinterpret_cast<uintptr_t>(src[i]) % 16 || reinterpret_cast<uintptr_t>(dst[i]) % 16)
        return CABF_EINVAL;
    }
  }
  if (pairs == 0) return CABF_OK;
  cabf::launch_permute(geo, eb, src, dst, stream);
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
  return build_mask(g, dtype, qp, kp, scale, thr, 0, sta, kv_count, kv_index, block_prob,
                    workspace, workspace_bytes, stream);
}

int cabf_build_block_mask_topk(const cabf_geom* g, cabf_dtype dtype, const void* qp,
                               const void* kp, float scale, int32_t k, const cabf_sta* sta,
                               int32_t* kv_count, int32_t* kv_index, float* block_prob,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (k < 1) return CABF_EINVAL;
  return build_mask(g, dtype, qp, kp, scale, 0.0f, k, sta, kv_count, kv_index, block_prob,
                    workspace, workspace_bytes, stream);
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
