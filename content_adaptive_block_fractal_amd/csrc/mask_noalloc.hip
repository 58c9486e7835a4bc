// Block mask without a caller workspace, for callers that cannot allocate
// device memory (code under graph capture, serving loops). The workspace of
// the mask kernels (pooled means and block logits) lives in a file-scope
// device array of fixed size; the (batch, head) pairs are processed in
// passes of as many pairs as the array holds, each pass the same three
// kernels as cabf_build_block_mask on a slice of the tensors.
//
// Each GPU the library runs on holds its own copy of the array for the life
// of the process. Every call on a GPU shares it and leaves its contents
// behind; no kernel reads a byte of it that the same pass has not written,
// so nothing needs clearing. Calls that overlap on one GPU (two streams,
// two threads) race on the array.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "cabf.h"
#include "geometry.hpp"
#include "launch.hpp"

namespace cabf {

static __device__ __align__(256) unsigned char scratch[CABF_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch`, per device

// The device address of `scratch` on device `dev`, resolved once per device
// with that device current. In host code `scratch` names a host-side stand-in;
// only this address may reach a kernel.
int scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return CABF_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return CABF_EHIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return CABF_EHIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return CABF_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CABF_OK;
}

Geo slice(const Geo& g, int64_t bh) {
  Geo s = g;
  s.B = 1;
  s.heads = static_cast<int>(bh);
  s.BH = bh;
  return s;
}

}  // namespace

int64_t noalloc_pairs_per_pass(const Geo& g) {
  const size_t one = mask_workspace_layout(slice(g, 1)).total;
  int64_t n = static_cast<int64_t>(CABF_NOALLOC_SCRATCH_BYTES / one);
  n = std::min<int64_t>(n, g.BH);
  // sections are 256-byte aligned as a whole, so n pairs never need more
  // than n times one pair's layout; checked all the same
  while (n > 0 && mask_workspace_layout(slice(g, n)).total > CABF_NOALLOC_SCRATCH_BYTES) --n;
  return n;
}

int launch_build_block_mask_noalloc(const Geo& g, int elem_bytes, const void* qp, const void* kp,
                                    float scale, float thr, bool sta_on, int dt, int dy, int dx,
                                    int32_t* kv_count, int32_t* kv_index, float* block_prob,
                                    hipStream_t stream) {
  const int64_t per = noalloc_pairs_per_pass(g);
  if (per < 1) return CABF_EWORKSPACE;
  int dev = -1;
  if (stream == nullptr) {
    if (hipGetDevice(&dev) != hipSuccess) return CABF_EHIP;
  } else {
    dev = hipGetStreamDeviceId(stream);
  }
  void* ws = nullptr;
  const int st = scratch_address(dev, &ws);
  if (st != CABF_OK) return st;
  const int64_t tensor = g.N * g.D * elem_bytes;        // bytes per (batch, head) of qp, kp
  const int64_t lists = static_cast<int64_t>(g.nb) * g.nb;
  for (int64_t b0 = 0; b0 < g.BH; b0 += per) {
    const Geo s = slice(g, std::min(per, g.BH - b0));
    launch_build_block_mask(s, elem_bytes == 2, static_cast<const char*>(qp) + b0 * tensor,
                            static_cast<const char*>(kp) + b0 * tensor, scale, thr, 0, sta_on, dt,
                            dy, dx, kv_count + b0 * g.nb, kv_index + b0 * lists,
                            block_prob == nullptr ? nullptr : block_prob + b0 * lists, ws, stream);
  }
  return CABF_OK;
}

}  // namespace cabf
