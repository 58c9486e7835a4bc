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

int64_t resident_workgroups(const void* kernel, int threads, hipStream_t stream) {
  int dev = 0;
  if (stream == nullptr) {
    if (hipGetDevice(&dev) != hipSuccess) return 0;
  } else {
    dev = hipGetStreamDeviceId(stream);
  }
  int cus = 0, per_cu = 0;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
    return 0;
  return static_cast<int64_t>(cus) * per_cu;
}

void launch_bsa_forward(const Geo& g, bool bf16, const void* qp, const void* kp, const void* vp,
                        const int32_t* kv_count, const int32_t* kv_index, float scale, void* op,
                        float* lse, bool phased, hipStream_t stream) {
  const AttnArgs a = make_args(g, qp, kp, vp, kv_count, kv_index, scale, op, lse);
  // bf16 on matrix cores. Rows of fewer than kLongRowBlocks blocks (lists
  // of a few hundred entries): by default the clock-phased one-block kernel
  // over the whole grid (720p / 80%: 29.5-30.2 ms); in list order the same
  // kernel in launches of a device-full of workgroups, which start together
  // and walk the key range in step (32.2 ms; one launch over the whole grid:
  // 43 ms, the paired kernel 34 ms). Longer rows, in both modes: the paired
  // kernel in device-full launches, in list order (241 frames at 768p / 85%,
  // 805 entries a row: 164.6 ms, against 196.7 ms clock-phased and 178.3 ms
  // for the one-block kernel in device-full launches); long passes drift
  // apart from a clock sweep, and a tile loaded once for two blocks matters
  // more when the key range no longer fits L2.
  const bool long_rows = g.nb >= kLongRowBlocks;
  if (bf16 && long_rows && g.nb <= kPairMaxBlocks)
    launch_bsa_forward_pair(a, g.D, g.T, stream);
  else if (bf16)
    launch_bsa_forward_mfma(a, g.D, phased && !long_rows, stream);
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
