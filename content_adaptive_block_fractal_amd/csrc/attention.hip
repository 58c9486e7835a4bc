// Block-sparse attention forward: dispatch between the kernels.
#include <hip/hip_runtime.h>

#include "attention_common.hpp"
#include "geometry.hpp"
#include "launch.hpp"

namespace cabf {

void launch_bsa_forward(const Geo& g, bool bf16, const void* qp, const void* kp, const void* vp,
                        const int32_t* kv_count, const int32_t* kv_index, float scale, void* op,
                        float* lse, bool phased, hipStream_t stream) {
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
  if (bf16)
    launch_bsa_forward_mfma(a, g.D, phased, stream);   // bf16 matrix cores
  else
    launch_bsa_forward_simple(a, false, g.D, stream);  // always walks lists in order
}

}  // namespace cabf
