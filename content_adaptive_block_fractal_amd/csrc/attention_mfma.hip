// Block-sparse attention forward on bf16 matrix cores (NABLA summary,
// Methodology item 2, expansion bullet: attention runs on the kept
// (query block, key block) tiles only).
//
// Work decomposition
//   One workgroup = one 64-row query block, 4 waves. Wave w owns query rows
//   32*(w&1) .. +31 and the key half 32*(w>>1) .. +31 of every kept tile; it
//   keeps its own running max, sum and output for that half, and the two
//   halves of a query row are merged once at the end through LDS (the merge
//   of two partial softmax sums is exact). The workgroup walks its kept key
//   blocks in list order. Workgroup ids are remapped so that each XCD (its
//   own L2) processes a contiguous run of query blocks of the same head:
//   neighbouring blocks keep overlapping key blocks, so K/V tiles are shared
//   in that XCD's L2.
//
// Per kept tile, per wave, with v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T    A = K (LDS, row-major, 16-byte chunks XOR-swizzled by row)
//                  B = Q^T (registers, loaded once)
//                  -> each lane holds one query row and 16 of its 32 keys,
//                  the other 16 sit in lane ^ 32
//   online softmax in base 2 on the fp32 accumulators; the running max is
//   only raised (and the output rescaled) when a row's max grows by more than
//   2^8, so the numerators stay below 2^8 and most tiles skip the rescale
//   O^T += V^T P^T A = V^T, read from the row-major V tile in LDS with the
//                  transposing LDS read (ds_read_b64_tr_b16: within a
//                  16-lane group, lane i receives element i%4 of the
//                  8-byte rows read by lanes 4e + i/4, e = 0..3), so each
//                  lane gets 4 consecutive keys of one head-dim column
//                  B = P^T (the softmax numerators, rounded to bf16)
// The contraction index of each product only has to be spread over the
// lanes the same way in both operands; V^T is read with the key order the
// S^T accumulator layout gives P.
//
// Pipelining: while a tile is multiplied out of LDS, the next tile's K and V
// are already in flight from global memory into registers.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attention_common.hpp"
#include "geometry.hpp"
#include "launch.hpp"

namespace cabf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;
constexpr float kRescaleSlack = 8.0f;   // base-2 headroom before the running max is raised

// Workgroup id -> query block: XCD x (which receives ids x, x+8, ...) gets
// the contiguous range [start_x, start_x + count_x).
__device__ inline int64_t xcd_order(int64_t wg, int64_t total) {
#if defined(CABF_WG_ORDER) && CABF_WG_ORDER == 1
  return wg;   // plain dispatch order: all XCDs sweep the same head together
#endif
  const int64_t xcd = wg % kXcds, local = wg / kXcds;
  const int64_t per = total / kXcds, rem = total % kXcds;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// K tile: 64 rows x D bf16 = 64 x (D/8) chunks of 16 bytes.
template <int D>
__device__ inline int k_chunk_slot(int key, int chunk) {
  constexpr int kChunks = D / 8;
  // D = 128: a row spans all 64 banks, rotate chunks by key % 16;
  // D = 64: two rows per bank sweep, rotate by (key / 2) % 8.
  const int swz = (D == 128) ? (key & 15) : ((key >> 1) & 7);
  return key * kChunks + (chunk ^ swz);
}

// V tile: 64 rows x D bf16, row-major like K. The transposing read fetches
// 4 consecutive rows x 32 bytes per 16-lane group; XOR-ing the 16-byte chunk
// index with an even rotation keeps each 32-byte pair intact and puts the 4
// (D = 128: 8) rows of one read on distinct banks.
template <int D>
__device__ inline int v_chunk_slot(int key, int chunk) {
  constexpr int kChunks = D / 8;
  const int swz = (D == 128) ? 2 * (key & 7) : 2 * ((key >> 1) & 3);
  return key * kChunks + (chunk ^ swz);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// 4 consecutive keys of one head-dim column of the V tile (see above).
__device__ inline s16x4 read_v_transposed(const uint16_t* sv_row_chunk) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sv_row_chunk));
}

template <int D>
struct TileRegs {
  static constexpr int kChunks = D / 8;                        // 16-byte chunks per row
  static constexpr int kIters = kBlock * kChunks / kThreads;   // chunks per thread per tensor
  u32x4 k[kIters];
  u32x4 v[kIters];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& t, const uint16_t* __restrict__ kb,
                                          const uint16_t* __restrict__ vb, int tid) {
  using R = TileRegs<D>;
#pragma unroll
  for (int i = 0; i < R::kIters; ++i) {
    t.k[i] = *reinterpret_cast<const u32x4*>(kb + (tid + kThreads * i) * 8);
    t.v[i] = *reinterpret_cast<const u32x4*>(vb + (tid + kThreads * i) * 8);
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& t, u32x4* sk, u32x4* sv, int tid) {
  using R = TileRegs<D>;
#pragma unroll
  for (int i = 0; i < R::kIters; ++i) {
    const int cidx = tid + kThreads * i;
    const int row = cidx / R::kChunks, chunk = cidx % R::kChunks;
    sk[k_chunk_slot<D>(row, chunk)] = t.k[i];
    sv[v_chunk_slot<D>(row, chunk)] = t.v[i];
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void bsa_fwd_mfma(AttnArgs a, int64_t n_qblocks) {
  constexpr int kKS = D / 16;   // MFMA k-steps over d
  constexpr int kDT = D / 32;   // 32-row d subtiles of O^T
  constexpr int kTileBytes = kBlock * D * 2 * 2;                       // K + V
  constexpr int kMergeBytes = 2 * 64 * (kDT * 16 + 2) * 4;             // 2 waves' partials
  constexpr int kSmemBytes = kTileBytes > kMergeBytes ? kTileBytes : kMergeBytes;
  __shared__ uint4 smem[kSmemBytes / 16];
  u32x4* sk = reinterpret_cast<u32x4*>(smem);
  u32x4* sv = sk + kBlock * D / 8;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wq = wave & 1;      // query half of the block
  const int wk = wave >> 1;     // key half of every tile
  const int li = lane & 31;
  const int h = lane >> 5;
  const int64_t qblk = xcd_order(blockIdx.x, n_qblocks);
  const int64_t bh = qblk / a.nb;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.qp);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.kp) + bh * a.N * D;
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.vp) + bh * a.N * D;

  // Q^T fragments: lane holds query row li of this wave's half, d = 16 ks + 8 h .. +7
  const int64_t qrow = qblk * kBlock + wq * 32 + li;
  bf16x8 qf[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    const uint4 u = *reinterpret_cast<const uint4*>(Q + qrow * D + 16 * ks + 8 * h);
    qf[ks] = __builtin_bit_cast(bf16x8, u);
  }

  f32x16 o[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  float m = -INFINITY;   // running max of the row (this key half), base-2 scaled logits
  float l = 0.0f;        // this lane's part of the row sum
  const float c = a.scale_log2;

  const int cnt = min(max(a.kv_count[qblk], 0), a.nb);
  const int32_t* __restrict__ list = a.kv_index + qblk * a.nb;
  const unsigned nbu = static_cast<unsigned>(a.nb);
  const uint16_t* sv_elems = reinterpret_cast<const uint16_t*>(sv);
  const int key0 = 32 * wk;     // first key of this wave's half

  TileRegs<D> regs;
  int e = 0;
  while (e < cnt && static_cast<unsigned>(list[e]) >= nbu) ++e;
  if (e < cnt) {
    const int64_t off = static_cast<int64_t>(list[e]) * kBlock * D;
    load_tile<D>(regs, K + off, V + off, tid);
  }
  while (e < cnt) {
    const int jb = list[e];
    int en = e + 1;
    while (en < cnt && static_cast<unsigned>(list[en]) >= nbu) ++en;
    __syncthreads();            // every wave is done with the previous tile
    store_tile<D>(regs, sk, sv, tid);
    __syncthreads();
    if (en < cnt) {
      const int64_t off = static_cast<int64_t>(list[en]) * kBlock * D;
      load_tile<D>(regs, K + off, V + off, tid);
    }

    // ---- S^T = K Q^T for keys key0 .. key0+31 ---------------------------
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const u32x4 u = sk[k_chunk_slot<D>(key0 + li, 2 * ks + h)];
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), qf[ks], s, 0, 0, 0);
    }
    // ---- pad keys of a partial patch -----------------------------------
    const BlockExtent ext = block_extent(jb, a);
    if (!ext.full()) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (!ext.real(key)) s[r] = -INFINITY;
      }
    }
    // ---- online softmax (base 2, lazily rescaled) -----------------------
    float mt = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32)) * c;
    if (__any(mt > m + kRescaleSlack)) {
      const float mn = fmaxf(m, mt);
      const float alpha = (mn == -INFINITY) ? 1.0f : exp2f(m - mn);   // m = -inf gives 0
      m = mn;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    const float msub = (m == -INFINITY) ? 0.0f : m;
    bf16x8 pb[2];
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // v_exp_f32 directly: arguments are <= 2^3 above the running max and
      // results below the fp32 normal range are flushed, which bf16 P and the
      // fp32 sums tolerate
      p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -msub));
      pb[r >> 3][r & 7] = static_cast<__bf16>(p[r]);
    }
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int r = 0; r < w; ++r) p[r] += p[r + w];
    l += p[0];
    // ---- O^T += V^T P^T over this wave's 32 keys ------------------------
    // lane (d = 32 dt + li, h): A elements 0..3 = keys k0 .. k0+3 and 4..7 =
    // keys k0+8 .. k0+11 with k0 = key0 + 16 st + 4 h, the order in which the
    // S^T accumulator holds P. Source lane s of a 16-lane group reads row
    // k0 + s/4 at columns base + 4 (s % 4), base = 32 dt + 16 ((lane / 16) % 2).
    {
      const int grp = lane >> 4, sl = lane & 15;
      const int col = 16 * (grp & 1) + 4 * (sl & 3);     // + 32 dt
      const int rsub = 4 * (grp >> 1) + (sl >> 2);        // + key0 + 16 st (+ 8)
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int r0 = key0 + 16 * st + rsub;
          const int cc = 32 * dt + col;
          const uint16_t* a0 = sv_elems + v_chunk_slot<D>(r0, cc >> 3) * 8 + (cc & 7);
          const uint16_t* a1 = sv_elems + v_chunk_slot<D>(r0 + 8, cc >> 3) * 8 + (cc & 7);
          const s16x4 lo = read_v_transposed(a0);
          const s16x4 hi = read_v_transposed(a1);
          const s16x4 both[2] = {lo, hi};
          bf16x8 av;
          __builtin_memcpy(&av, both, sizeof(av));
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[st], o[dt], 0, 0, 0);
        }
      }
    }
    e = en;
  }

  // ---- merge the two key halves of every query row -----------------------
  l += __shfl_xor(l, 32);       // both lanes of a row hold the same m
  __syncthreads();              // tile buffers are free
  float* part = reinterpret_cast<float*>(smem) + wq * 64 * (kDT * 16 + 2);
  constexpr int kStride = 64;   // lane-major: element j of lane x at part[j * 64 + x]
  if (wk == 1) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[(dt * 16 + r) * kStride + lane] = o[dt][r];
    part[(kDT * 16) * kStride + lane] = m;
    part[(kDT * 16 + 1) * kStride + lane] = l;
  }
  __syncthreads();
  if (wk == 1) return;
  const float m1 = part[(kDT * 16) * kStride + lane];
  const float l1 = part[(kDT * 16 + 1) * kStride + lane];
  const float mm = fmaxf(m, m1);
  const float a0 = (m == -INFINITY) ? 0.0f : exp2f(m - mm);
  const float a1 = (m1 == -INFINITY) ? 0.0f : exp2f(m1 - mm);
  const float lt = l * a0 + l1 * a1;
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  const float w0 = a0 * inv, w1 = a1 * inv;
  uint16_t* __restrict__ O = static_cast<uint16_t*>(a.op);
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * h;
      float v[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 4 * g + x;
        v[x] = o[dt][r] * w0 + part[(dt * 16 + r) * kStride + lane] * w1;
      }
      uint2 w;
      w.x = static_cast<uint32_t>(f32_to_bf16_rne(v[0])) |
            (static_cast<uint32_t>(f32_to_bf16_rne(v[1])) << 16);
      w.y = static_cast<uint32_t>(f32_to_bf16_rne(v[2])) |
            (static_cast<uint32_t>(f32_to_bf16_rne(v[3])) << 16);
      *reinterpret_cast<uint2*>(O + qrow * D + d) = w;
    }
  if (a.lse != nullptr && h == 0)
    a.lse[qrow] = lt > 0.0f ? (mm + log2f(lt)) * kLn2 : -INFINITY;
}

}  // namespace

void launch_bsa_forward_mfma(const AttnArgs& a, int D, hipStream_t stream) {
  const int64_t n = a.BH * a.nb;
  const unsigned grid = static_cast<unsigned>(n);
  if (D == 64)
    hipLaunchKernelGGL((bsa_fwd_mfma<64>), dim3(grid), dim3(kThreads), 0, stream, a, n);
  else
    hipLaunchKernelGGL((bsa_fwd_mfma<128>), dim3(grid), dim3(kThreads), 0, stream, a, n);
}

}  // namespace cabf
