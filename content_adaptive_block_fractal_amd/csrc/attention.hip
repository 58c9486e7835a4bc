// Block-sparse attention forward: dispatch between the kernels.
#include <hip/hip_runtime.h>

#include "attention_common.hpp"
#include "geometry.hpp"
#include "launch.hpp"

namespace cabf {

namespace {
AttnArgs make_args(const Geo& g, const void* qp, const void* kp, const void* vp,
                   const int32_t* kv_count, const int32_t* kv_index, float scale, void* op,
                   float* lse) {
  AttnArgs a{};
  a.qp = qp;
  a.kp = kp;
  a.vp = vp;
  a.kv_count = kv_count;
  a.kv_index = kv_index;
  a.op = op;
  a.lse = lse;
  a.scale_log2 = scale * kLog2e;
  a.nb = g.nb;
  a.Ty = g.Ty;
  a.Tx = g.Tx;
  a.H = g.H;
  a.W = g.W;
  a.N = g.N;
  a.BH = g.BH;
  return a;
}
}  // namespace

void launch_bsa_forward(const Geo& g, bool bf16, const void* qp, const void* kp, const void* vp,
                        const int32_t* kv_count, const int32_t* kv_index, float scale, void* op,
                        float* lse, bool phased, hipStream_t stream) {
  const AttnArgs a = make_args(g, qp, kp, vp, kv_count, kv_index, scale, op, lse);
  // bf16 on matrix cores. Lists walked in order: the paired kernel, which
  // reads each K/V tile of two blocks' lists once (41.6 -> 33.9 ms at 720p /
  // 80%). Clock-phased: one block per workgroup, whose concurrent passes
  // share the tiles through L2 (29.2 ms; the paired kernel took 32.3 ms).
  if (bf16 && !phased && g.nb <= kPairMaxBlocks)
    launch_bsa_forward_pair(a, g.D, g.T, false, stream);
  else if (bf16)
    launch_bsa_forward_mfma(a, g.D, phased, stream);
  else
    launch_bsa_forward_simple(a, false, g.D, stream);  // always walks lists in order
}

void launch_bsa_forward_subset(const Geo& g, const void* qp, const void* kp, const void* vp,
                               const int32_t* kv_count, const int32_t* kv_index,
                               const int32_t* q_blocks, int64_t n_blocks, float scale, void* op,
                               float* lse, bool phased, hipStream_t stream) {
  const AttnArgs a = make_args(g, qp, kp, vp, kv_count, kv_index, scale, op, lse);
  launch_bsa_forward_subset_mfma(a, g.D, phased, q_blocks, n_blocks, stream);
}

}  // namespace cabf
