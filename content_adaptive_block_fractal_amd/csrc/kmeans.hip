// k-means clustering of token features and the stable cluster permutation
// (Sparse VideoGen2 summary, Methodology A: Q and K are clustered
// independently by k-means and each is reordered so that a cluster's tokens
// are contiguous).
//
// Per (batch, head) of x [BH, n, d] (bf16), Lloyd's algorithm:
//   km_prep     centroid c (fp32) -> three bf16 terms t0 + t1 + t2 (each the
//               bf16 rounding of what the previous terms leave) and |c|^2;
//               padded centroids get |c|^2 = +inf
//   km_assign   nearest centroid of every token: argmin_c |c|^2 - 2 x.c
//               (|x|^2 is common to all c). x.c = sum of three bf16 products
//               on the matrix cores (x is exact in bf16), fp32 accumulation,
//               so the dot product is close to fp32 accuracy. Ties go to the
//               lowest index.
//   sort        stable segmented radix sort of the labels (token index as
//               payload): the permutation, clusters contiguous, original
//               order inside a cluster
//   km_offsets  offsets[c] = first sorted position with label >= c
//   km_update   mean of the members, summed in sorted (token) order, so the
//               result is deterministic; an empty cluster keeps its centroid
// After the last update a final assignment and sort make labels, counts and
// the permutation consistent with the returned centroids.
#include <hip/hip_runtime.h>
#include <hipcub/hipcub.hpp>

#include <cmath>
#include <cstdint>

#include "svg.hpp"

namespace cabf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ inline float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bfloat16 bits, round to nearest even (finite inputs)
__device__ inline uint16_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// cent[bh, c, :] = x[bh, init[bh, c], :] (indices clamped to [0, n))
template <int D>
__global__ __launch_bounds__(256) void km_init(const uint16_t* __restrict__ x,
                                               const int32_t* __restrict__ init,
                                               float* __restrict__ cent, int n, int C,
                                               int64_t total) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= total * D) return;
  const int64_t row = e / D;            // bh * C + c
  const int j = static_cast<int>(e - row * D);
  const int64_t bh = row / C;
  const int t = min(max(init[row], 0), n - 1);
  cent[e] = bf16_bits_to_f32(x[(bh * n + t) * D + j]);
}

// one wave per padded centroid: the three bf16 terms and |c|^2
template <int D>
__global__ __launch_bounds__(256) void km_prep(const float* __restrict__ cent,
                                               uint16_t* __restrict__ terms,   // [3][BH, Cp, D]
                                               float* __restrict__ norm, int C, int Cp,
                                               int64_t rows_padded /* BH * Cp */) {
  constexpr int kPer = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows_padded) return;
  const int64_t bh = row / Cp;
  const int c = static_cast<int>(row - bh * Cp);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = lane * kPer + i;
    float v = c < C ? cent[(bh * C + c) * D + j] : 0.0f;
    s = fmaf(v, v, s);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const uint16_t b = f32_to_bf16_bits(v);
      terms[(k * rows_padded + row) * D + j] = b;
      v -= bf16_bits_to_f32(b);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) norm[row] = c < C ? s : INFINITY;
}

// Nearest centroid of 32 tokens per wave (128 per workgroup).
// S = C_chunk X^T with v_mfma_f32_32x32x16_bf16: A = 32 centroids x 16 d (one
// term), B = 16 d x 32 tokens; lane (token li, h) holds rows 8(r/4) + 4h + r%4
// of its token's column, increasing with r.
template <int D>
__global__ __launch_bounds__(256) void km_assign(const uint16_t* __restrict__ x,
                                                 const uint16_t* __restrict__ terms,
                                                 const float* __restrict__ norm,
                                                 int32_t* __restrict__ label, int n, int Cp,
                                                 int64_t rows_padded, int tiles_per_bh) {
  constexpr int kKS = D / 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int li = lane & 31, h = lane >> 5;
  const int64_t bh = blockIdx.x / tiles_per_bh;
  const int tile = static_cast<int>(blockIdx.x - bh * tiles_per_bh);
  const int t = tile * 128 + wave * 32 + li;
  const int tl = min(t, n - 1);                  // rows past n are computed, not stored
  bf16x8 xf[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    const uint4 u = *reinterpret_cast<const uint4*>(x + (bh * n + tl) * D + 16 * ks + 8 * h);
    xf[ks] = __builtin_bit_cast(bf16x8, u);
  }
  const uint16_t* t0 = terms + (bh * Cp) * D;
  const uint16_t* t1 = t0 + rows_padded * D;
  const uint16_t* t2 = t1 + rows_padded * D;
  const float* nb = norm + bh * Cp;
  float best = INFINITY;
  int best_c = 0;
  for (int c0 = 0; c0 < Cp; c0 += 32) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const int64_t crow = static_cast<int64_t>(c0 + li) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(t0 + crow + 16 * ks));
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(t1 + crow + 16 * ks));
      const bf16x8 a2 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(t2 + crow + 16 * ks));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, xf[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, xf[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, xf[ks], acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = c0 + 8 * (r >> 2) + 4 * h + (r & 3);
      const float dist = fmaf(-2.0f, acc[r], nb[c]);
      if (dist < best) {        // strict: the lower index wins ties
        best = dist;
        best_c = c;
      }
    }
  }
  // the other 16 rows of every group of 32 sit in lane ^ 32
  const float ob = __shfl_xor(best, 32);
  const int oc = __shfl_xor(best_c, 32);
  if (ob < best || (ob == best && oc < best_c)) {
    best = ob;
    best_c = oc;
  }
  if (h == 0 && t < n) label[bh * n + t] = best_c;
}

// offsets[bh, c] = first position of the sorted labels with label >= c, c <= C
__global__ __launch_bounds__(256) void km_offsets(const int32_t* __restrict__ sorted_label,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ counts, int n, int C,
                                                  int64_t total /* BH * (C + 1) */) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int64_t bh = e / (C + 1);
  const int c = static_cast<int>(e - bh * (C + 1));
  const int32_t* s = sorted_label + bh * n;
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s[mid] < c) lo = mid + 1; else hi = mid;
  }
  offsets[e] = lo;
  if (c > 0 && counts != nullptr) {
    // count of cluster c - 1 = offsets[c] - offsets[c - 1]
    int lo2 = 0, hi2 = n;
    while (lo2 < hi2) {
      const int mid = (lo2 + hi2) >> 1;
      if (s[mid] < c - 1) lo2 = mid + 1; else hi2 = mid;
    }
    counts[bh * C + c - 1] = lo - lo2;
  }
}

// one wave per cluster: mean of the members in sorted order
template <int D>
__global__ __launch_bounds__(256) void km_update(const uint16_t* __restrict__ x,
                                                 const int32_t* __restrict__ perm,
                                                 const int32_t* __restrict__ offsets,
                                                 float* __restrict__ cent, int n, int C,
                                                 int64_t rows /* BH * C */) {
  constexpr int kPer = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t bh = row / C;
  const int c = static_cast<int>(row - bh * C);
  const int32_t* off = offsets + bh * (C + 1);
  const int b = off[c], e = off[c + 1];
  if (e <= b) return;                       // empty: keep the centroid
  float acc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) acc[i] = 0.0f;
  const int32_t* p = perm + bh * n;
  const uint16_t* xb = x + bh * static_cast<int64_t>(n) * D + lane * kPer;
  // four rows in flight at a time, added in member order
  int i = b;
  for (; i + 4 <= e; i += 4) {
    uint16_t v[4][kPer];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint16_t* src = xb + static_cast<int64_t>(p[i + u]) * D;
#pragma unroll
      for (int k = 0; k < kPer; ++k) v[u][k] = src[k];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < kPer; ++k) acc[k] += bf16_bits_to_f32(v[u][k]);
  }
  for (; i < e; ++i) {
    const uint16_t* src = xb + static_cast<int64_t>(p[i]) * D;
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc[k] += bf16_bits_to_f32(src[k]);
  }
  const float inv = 1.0f / static_cast<float>(e - b);
#pragma unroll
  for (int k = 0; k < kPer; ++k) cent[row * D + lane * kPer + k] = acc[k] * inv;
}

__global__ __launch_bounds__(256) void km_iota(int32_t* __restrict__ v, int n, int64_t total) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e < total) v[e] = static_cast<int32_t>(e % n);
}

__global__ __launch_bounds__(256) void km_seg_offsets(int32_t* __restrict__ seg, int n, int BH) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e <= BH) seg[e] = e * n;
}

int key_bits(int C) {
  int b = 1;
  while ((1 << b) < C) ++b;
  return b;
}

// Labels are sorted as unsigned keys (they are non-negative) over their low
// key_bits(C) bits; radix sorting is stable, so a cluster's tokens keep their
// original order.
size_t sort_temp_bytes(int64_t BH, int n, int C) {
  size_t bytes = 0;
  const int items = static_cast<int>(BH * n);
  const int32_t* no_offsets = nullptr;
  const hipError_t e = hipcub::DeviceSegmentedRadixSort::SortPairs(nullptr, bytes, static_cast<const uint32_t*>(nullptr),
                                              static_cast<uint32_t*>(nullptr),
                                              static_cast<const int32_t*>(nullptr),
                                              static_cast<int32_t*>(nullptr), items,
                                              static_cast<int>(BH), no_offsets, no_offsets, 0,
                                              key_bits(C), nullptr);
  return e == hipSuccess ? bytes : 0;   // 0: the sort itself reports the failure at launch
}

size_t align256(size_t v) { return (v + 255) & ~size_t{255}; }

}  // namespace

KmeansWorkspace kmeans_workspace_layout(int64_t BH, int n, int C, int D) {
  KmeansWorkspace w{};
  const int Cp = (C + 31) / 32 * 32;
  size_t o = 0;
  w.terms = o;   o += align256(3 * static_cast<size_t>(BH) * Cp * D * sizeof(uint16_t));
  w.norm = o;    o += align256(static_cast<size_t>(BH) * Cp * sizeof(float));
  w.sorted = o;  o += align256(static_cast<size_t>(BH) * n * sizeof(int32_t));
  w.iota = o;    o += align256(static_cast<size_t>(BH) * n * sizeof(int32_t));
  w.seg = o;     o += align256((static_cast<size_t>(BH) + 1) * sizeof(int32_t));
  w.sort_tmp = o;
  w.sort_tmp_bytes = sort_temp_bytes(BH, n, C);
  o += align256(w.sort_tmp_bytes);
  w.total = o;
  return w;
}

int launch_kmeans(int64_t BH, int n, int D, int C, int iters, const void* x, const int32_t* init,
                  float* cent, int32_t* counts, int32_t* label, int32_t* perm, int32_t* offsets,
                  void* workspace, hipStream_t stream) {
  const KmeansWorkspace w = kmeans_workspace_layout(BH, n, C, D);
  char* ws = static_cast<char*>(workspace);
  uint16_t* terms = reinterpret_cast<uint16_t*>(ws + w.terms);
  float* norm = reinterpret_cast<float*>(ws + w.norm);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + w.sorted);
  int32_t* iota = reinterpret_cast<int32_t*>(ws + w.iota);
  int32_t* seg = reinterpret_cast<int32_t*>(ws + w.seg);
  void* tmp = ws + w.sort_tmp;
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  const int Cp = (C + 31) / 32 * 32;
  const int64_t rows_padded = BH * Cp;
  const int64_t items = BH * n;
  auto blocks = [](int64_t work, int per) { return dim3(static_cast<unsigned>((work + per - 1) / per)); };

  hipLaunchKernelGGL(km_iota, blocks(items, 256), dim3(256), 0, stream, iota, n, items);
  hipLaunchKernelGGL(km_seg_offsets, blocks(BH + 1, 256), dim3(256), 0, stream, seg, n,
                     static_cast<int>(BH));
  if (D == 64)
    hipLaunchKernelGGL((km_init<64>), blocks(BH * C * 64, 256), dim3(256), 0, stream, xs, init,
                       cent, n, C, BH * C);
  else
    hipLaunchKernelGGL((km_init<128>), blocks(BH * C * 128, 256), dim3(256), 0, stream, xs, init,
                       cent, n, C, BH * C);
  const int tiles = (n + 127) / 128;
  const int bits = key_bits(C);
  for (int it = 0; it <= iters; ++it) {
    if (D == 64) {
      hipLaunchKernelGGL((km_prep<64>), blocks(rows_padded, 4), dim3(256), 0, stream, cent, terms,
                         norm, C, Cp, rows_padded);
      hipLaunchKernelGGL((km_assign<64>), dim3(static_cast<unsigned>(BH * tiles)), dim3(256), 0,
                         stream, xs, terms, norm, label, n, Cp, rows_padded, tiles);
    } else {
      hipLaunchKernelGGL((km_prep<128>), blocks(rows_padded, 4), dim3(256), 0, stream, cent, terms,
                         norm, C, Cp, rows_padded);
      hipLaunchKernelGGL((km_assign<128>), dim3(static_cast<unsigned>(BH * tiles)), dim3(256), 0,
                         stream, xs, terms, norm, label, n, Cp, rows_padded, tiles);
    }
    size_t tmp_bytes = w.sort_tmp_bytes;
    const hipError_t e = hipcub::DeviceSegmentedRadixSort::SortPairs(
        tmp, tmp_bytes, reinterpret_cast<const uint32_t*>(label), reinterpret_cast<uint32_t*>(sorted),
        iota, perm, static_cast<int>(items), static_cast<int>(BH), seg, seg + 1, 0, bits, stream);
    if (e != hipSuccess) return -1;
    const bool last = it == iters;
    hipLaunchKernelGGL(km_offsets, blocks(BH * (C + 1), 256), dim3(256), 0, stream, sorted,
                       offsets, last ? counts : nullptr, n, C, BH * (C + 1));
    if (last) break;
    if (D == 64)
      hipLaunchKernelGGL((km_update<64>), blocks(BH * C, 4), dim3(256), 0, stream, xs, perm,
                         offsets, cent, n, C, BH * C);
    else
      hipLaunchKernelGGL((km_update<128>), blocks(BH * C, 4), dim3(256), 0, stream, xs, perm,
                         offsets, cent, n, C, BH * C);
  }
  return 0;
}

}  // namespace cabf
