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
//   counting sort of every head's labels, stable (original order inside a
//   cluster), in three passes over chunks of 1024 tokens:
//     km_hist     per-chunk label histogram (LDS)
//     km_scan     per head: cluster sizes and offsets (offsets[c] = first
//                 position of cluster c), and each chunk's first position
//                 inside every cluster
//     km_scatter  per chunk, in token order 64 at a time: a token's position
//                 is its chunk's next free position in its cluster plus the
//                 number of lanes before it with the same label (found with
//                 one ballot per label bit); perm[position] = token
//   km_update   mean of the members, summed in permutation (token) order, so
//               the result is deterministic; an empty cluster keeps its
//               centroid
// After the last update a final assignment and sort make labels, counts and
// the permutation consistent with the returned centroids.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "svg.hpp"

namespace cabf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// Nearest centroid of 64 tokens per wave (256 per workgroup).
// Distances against 32 centroids at a time: S = C_chunk X^T with
// v_mfma_f32_32x32x16_bf16, A = 32 centroids x 16 d (one bf16 term, from LDS),
// B = 16 d x 32 tokens (registers, two groups of 32 tokens per wave); lane
// (token li, h) holds rows 8(r/4) + 4h + r%4 of its token's column, which
// increase with r. The three terms of a chunk of 32 centroids (24 KB at
// d = 128) are staged in LDS by the whole workgroup, double-buffered; rows are
// padded by 16 bytes so that the 16 lanes of a read hit distinct banks.
template <int D>
__global__ __launch_bounds__(256) void km_assign(const uint16_t* __restrict__ x,
                                                 const uint16_t* __restrict__ terms,
                                                 const float* __restrict__ norm,
                                                 int32_t* __restrict__ label,
                                                 int n, int Cp, int64_t rows_padded,
                                                 int tiles_per_bh) {
  constexpr int kKS = D / 16;
  constexpr int kRow = D + 8;                       // padded LDS row (bf16 elements)
  constexpr int kChunkElems = 3 * 32 * kRow;        // three terms of 32 centroids
  constexpr int kLoads = 3 * 32 * (D / 8) / 256;    // 16-byte loads per thread per chunk
  static_assert(3 * 32 * (D / 8) % 256 == 0, "chunk load split");
  __shared__ uint16_t sc[2][kChunkElems];
  __shared__ float sn[2][32];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31, h = lane >> 5;
  const int64_t bh = blockIdx.x / tiles_per_bh;
  const int tile = static_cast<int>(blockIdx.x - bh * tiles_per_bh);
  bf16x8 xf[2][kKS];
  int tok[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    tok[g] = tile * 256 + wave * 64 + g * 32 + li;
    const int tl = min(tok[g], n - 1);             // rows past n are computed, not stored
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const uint4 u = *reinterpret_cast<const uint4*>(x + (bh * n + tl) * D + 16 * ks + 8 * h);
      xf[g][ks] = __builtin_bit_cast(bf16x8, u);
    }
  }
  const uint16_t* tb = terms + (bh * Cp) * D;
  const float* nb = norm + bh * Cp;
  // chunk c0 of the three terms: thread loads kLoads 16-byte pieces
  u32x4 stage[kLoads];
  float stage_n = 0.0f;
  auto fetch = [&](int c0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int piece = i * 256 + tid;             // (term, row, 16-byte column)
      const int term = piece / (32 * (D / 8));
      const int rem = piece - term * (32 * (D / 8));
      const int row = rem / (D / 8), col = rem - row * (D / 8);
      stage[i] = *reinterpret_cast<const u32x4*>(tb + term * rows_padded * D +
                                                  static_cast<int64_t>(c0 + row) * D + col * 8);
    }
    if (tid < 32) stage_n = nb[c0 + tid];
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int piece = i * 256 + tid;
      const int term = piece / (32 * (D / 8));
      const int rem = piece - term * (32 * (D / 8));
      const int row = rem / (D / 8), col = rem - row * (D / 8);
      *reinterpret_cast<u32x4*>(&sc[buf][(term * 32 + row) * kRow + col * 8]) = stage[i];
    }
    if (tid < 32) sn[buf][tid] = stage_n;
  };
  float best[2] = {INFINITY, INFINITY};
  int best_c[2] = {0, 0};
  fetch(0);
  store(0);
  __syncthreads();
  const int chunks = Cp / 32;
  for (int ci = 0; ci < chunks; ++ci) {
    const int buf = ci & 1;
    if (ci + 1 < chunks) fetch((ci + 1) * 32);     // next chunk in flight during the products
    f32x16 acc[2];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[g][r] = 0.0f;
    const uint16_t* base = &sc[buf][li * kRow + 8 * h];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
      for (int term = 2; term >= 0; --term) {      // smallest term first
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(base + term * 32 * kRow + 16 * ks));
#pragma unroll
        for (int g = 0; g < 2; ++g)
          acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xf[g][ks], acc[g], 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int cl = 8 * (r >> 2) + 4 * h + (r & 3);
      const float cn = sn[buf][cl];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const float dist = fmaf(-2.0f, acc[g][r], cn);
        if (dist < best[g]) {      // strict: the lower index wins ties
          best[g] = dist;
          best_c[g] = ci * 32 + cl;
        }
      }
    }
    if (ci + 1 < chunks) {
      __syncthreads();             // everyone is done with buffer buf ^ 1
      store(buf ^ 1);
      __syncthreads();
    }
  }
  // the other 16 rows of every group of 32 sit in lane ^ 32
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float ob = __shfl_xor(best[g], 32);
    const int oc = __shfl_xor(best_c[g], 32);
    if (ob < best[g] || (ob == best[g] && oc < best_c[g])) {
      best[g] = ob;
      best_c[g] = oc;
    }
    if (h == 0 && tok[g] < n) label[bh * n + tok[g]] = best_c[g];
  }
}

constexpr int kSortChunk = 1024;   // tokens per chunk of the counting sort (one wave each)

// hist[bh, chunk, c] = tokens of the chunk with label c (one wave per chunk;
// LDS histogram of C bins)
__global__ __launch_bounds__(64) void km_hist(const int32_t* __restrict__ label,
                                              int32_t* __restrict__ hist, int n, int C,
                                              int chunks) {
  extern __shared__ int32_t bins[];
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x / chunks;
  const int ch = static_cast<int>(blockIdx.x - bh * chunks);
  for (int c = lane; c < C; c += 64) bins[c] = 0;
  __syncthreads();
  const int t0 = ch * kSortChunk, t1 = min(t0 + kSortChunk, n);
  const int32_t* lb = label + bh * n;
  for (int t = t0 + lane; t < t1; t += 64) atomicAdd(&bins[lb[t]], 1);
  __syncthreads();
  int32_t* out = hist + (bh * chunks + ch) * static_cast<int64_t>(C);
  for (int c = lane; c < C; c += 64) out[c] = bins[c];
}

// Per head (one workgroup of 256): hist[bh, chunk, c] becomes the number of
// tokens of cluster c in the chunks before `chunk`; counts[c] (if requested)
// and offsets[c] = sum of the sizes of clusters below c, offsets[C] = n.
__global__ __launch_bounds__(256) void km_scan(int32_t* __restrict__ hist,
                                               int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ counts, int C, int chunks) {
  extern __shared__ int32_t size[];   // [C], then 256 partial sums
  int32_t* const part = size + C;
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  int32_t* hb = hist + bh * chunks * static_cast<int64_t>(C);
  for (int c = tid; c < C; c += 256) {
    int run = 0;
    for (int ch = 0; ch < chunks; ++ch) {
      const int v = hb[static_cast<int64_t>(ch) * C + c];
      hb[static_cast<int64_t>(ch) * C + c] = run;
      run += v;
    }
    size[c] = run;
    if (counts != nullptr) counts[bh * C + c] = run;
  }
  __syncthreads();
  // exclusive scan of size[0 .. C): thread tid takes a contiguous range
  const int per = (C + 255) / 256;
  const int c0 = min(tid * per, C), c1 = min(c0 + per, C);
  int sum = 0;
  for (int c = c0; c < c1; ++c) sum += size[c];
  part[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int v = part[i];
      part[i] = run;
      run += v;
    }
  }
  __syncthreads();
  int run = part[tid];
  int32_t* ob = offsets + bh * (C + 1);
  for (int c = c0; c < c1; ++c) {
    ob[c] = run;
    run += size[c];
  }
  if (tid == 255) ob[C] = run;
}

// perm[bh, position] = token, one wave per chunk walking its tokens in order,
// 64 at a time. next[c] (LDS) = the position the chunk's next token of
// cluster c takes; lanes with equal labels are found with one ballot per
// label bit, so a token's position is next[c] plus the number of lanes before
// it with the same label (the sort is stable).
__global__ __launch_bounds__(64) void km_scatter(const int32_t* __restrict__ label,
                                                 const int32_t* __restrict__ hist,
                                                 const int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ perm, int n, int C,
                                                 int chunks, int bits) {
  extern __shared__ int32_t next[];
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x / chunks;
  const int ch = static_cast<int>(blockIdx.x - bh * chunks);
  const int32_t* hrow = hist + (bh * chunks + ch) * static_cast<int64_t>(C);
  const int32_t* ob = offsets + bh * (C + 1);
  for (int c = lane; c < C; c += 64) next[c] = ob[c] + hrow[c];
  __syncthreads();
  const int t0 = ch * kSortChunk, t1 = min(t0 + kSortChunk, n);
  const int32_t* lb = label + bh * n;
  int32_t* pb = perm + bh * n;
  const uint64_t below = (uint64_t{1} << lane) - 1u;
  for (int base = t0; base < t1; base += 64) {
    const int t = base + lane;
    const bool in = t < t1;
    const int c = in ? lb[t] : 0;
    uint64_t same = __ballot(in);
    for (int b = 0; b < bits; ++b) {
      const bool bit = (c >> b) & 1;
      const uint64_t ones = __ballot(in && bit);
      same &= bit ? ones : ~ones;
    }
    const int before = __popcll(same & below);
    if (in) pb[next[c] + before] = t;
    __syncthreads();                       // every lane has read next[] for this batch
    if (in && before == 0) next[c] += __popcll(same);
    __syncthreads();
  }
}

// One workgroup per cluster: wave w sums members b + w*q .. (a contiguous
// quarter, in sorted order), the four partial sums are added in wave order,
// so the mean is deterministic. An empty cluster keeps its centroid. Rows are
// gathered through the permutation (256 bytes each at d = 128), so the loop
// keeps many of them in flight.
template <int D>
__global__ __launch_bounds__(256) void km_update(const uint16_t* __restrict__ x,
                                                 const int32_t* __restrict__ perm,
                                                 const int32_t* __restrict__ offsets,
                                                 float* __restrict__ cent, int n, int C) {
  constexpr int kPer = D / 64;
  __shared__ float part[4][D];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
  const int64_t row = blockIdx.x;                // bh * C + c
  const int64_t bh = row / C;
  const int c = static_cast<int>(row - bh * C);
  const int32_t* off = offsets + bh * (C + 1);
  const int b = off[c], e = off[c + 1];
  if (e <= b) return;                            // uniform: keep the centroid
  const int q = (e - b + 3) / 4;
  const int wb = min(b + wave * q, e), we = min(wb + q, e);
  float acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = 0.0f;
  const int32_t* p = perm + bh * n;
  // lane's kPer consecutive bf16 of a row, fetched as one load
  typedef uint16_t lane_vec __attribute__((ext_vector_type(kPer)));
  const uint16_t* xb = x + bh * static_cast<int64_t>(n) * D + lane * kPer;
  // kRows rows in flight at a time (the loop is latency-bound), added in
  // member order. The batch's member indices come in with one load (lane u
  // holds member i + u, clamped to the last one) and are read out with
  // readlane, so every row address is scalar and the row loads issue back
  // to back; rows past the end of the quarter are loaded (in bounds) but
  // contribute nothing.
  constexpr int kRows = 16;
  for (int i = wb; i < we; i += kRows) {
    const int mine = p[min(i + (lane & (kRows - 1)), we - 1)];
    lane_vec v[kRows];
#pragma unroll
    for (int u = 0; u < kRows; ++u)
      v[u] = *reinterpret_cast<const lane_vec*>(
          xb + static_cast<int64_t>(__builtin_amdgcn_readlane(mine, u)) * D);
    // rows past the end add -0 (x + -0 = x exactly), so every load is used
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const bool in = i + u < we;
#pragma unroll
      for (int k = 0; k < kPer; ++k) acc[k] += in ? bf16_bits_to_f32(v[u][k]) : -0.0f;
    }
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) part[wave][lane * kPer + k] = acc[k];
  __syncthreads();
  if (wave != 0) return;
  const float inv = 1.0f / static_cast<float>(e - b);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = lane * kPer + k;
    cent[row * D + j] = (((part[0][j] + part[1][j]) + part[2][j]) + part[3][j]) * inv;
  }
}

int bits_for(int64_t values) {
  int b = 1;
  while ((int64_t{1} << b) < values) ++b;
  return b;
}

int sort_chunks(int n) { return (n + kSortChunk - 1) / kSortChunk; }

size_t align256(size_t v) { return (v + 255) & ~size_t{255}; }

}  // namespace

KmeansWorkspace kmeans_workspace_layout(int64_t BH, int n, int C, int D) {
  KmeansWorkspace w{};
  const int Cp = (C + 31) / 32 * 32;
  size_t o = 0;
  w.terms = o;   o += align256(3 * static_cast<size_t>(BH) * Cp * D * sizeof(uint16_t));
  w.norm = o;    o += align256(static_cast<size_t>(BH) * Cp * sizeof(float));
  w.hist = o;    o += align256(static_cast<size_t>(BH) * sort_chunks(n) * C * sizeof(int32_t));
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
  int32_t* hist = reinterpret_cast<int32_t*>(ws + w.hist);
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  const int Cp = (C + 31) / 32 * 32;
  const int64_t rows_padded = BH * Cp;
  auto blocks = [](int64_t work, int per) { return dim3(static_cast<unsigned>((work + per - 1) / per)); };

  if (D == 64)
    hipLaunchKernelGGL((km_init<64>), blocks(BH * C * 64, 256), dim3(256), 0, stream, xs, init,
                       cent, n, C, BH * C);
  else
    hipLaunchKernelGGL((km_init<128>), blocks(BH * C * 128, 256), dim3(256), 0, stream, xs, init,
                       cent, n, C, BH * C);
  const int tiles = (n + 255) / 256;
  const int bits = bits_for(C);               // label bits
  const int chunks = sort_chunks(n);
  const unsigned sort_grid = static_cast<unsigned>(BH * chunks);
  const size_t bins_bytes = static_cast<size_t>(C) * sizeof(int32_t);
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
    const bool last = it == iters;
    hipLaunchKernelGGL(km_hist, dim3(sort_grid), dim3(64), bins_bytes, stream, label, hist, n, C,
                       chunks);
    hipLaunchKernelGGL(km_scan, dim3(static_cast<unsigned>(BH)), dim3(256),
                       bins_bytes + 256 * sizeof(int32_t), stream, hist, offsets,
                       last ? counts : nullptr, C, chunks);
    hipLaunchKernelGGL(km_scatter, dim3(sort_grid), dim3(64), bins_bytes, stream, label, hist,
                       offsets, perm, n, C, chunks, bits);
    if (last) break;
    if (D == 64)
      hipLaunchKernelGGL((km_update<64>), dim3(static_cast<unsigned>(BH * C)), dim3(256), 0, stream,
                         xs, perm, offsets, cent, n, C);
    else
      hipLaunchKernelGGL((km_update<128>), dim3(static_cast<unsigned>(BH * C)), dim3(256), 0,
                         stream, xs, perm, offsets, cent, n, C);
  }
  return 0;
}

}  // namespace cabf
