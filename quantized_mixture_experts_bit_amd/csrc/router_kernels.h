// Router GEMV/GEMM (8-bit affine, fp64 accumulation) fused with top-k + softmax.
//
// The router stays at 8 bits so that it picks the right experts (ai-heartland
// review "TurboFieldfareとは", system-design summary of quantisation). Every
// product w * x is exact in fp64 (w = s*q + b has <= 20 significant bits, x <= 24)
// and the sums are fp64, so the logits sit within ~1e-12 of exact and the
// top-k set matches an exact evaluation wherever the k-th/(k+1)-th gap exceeds
// that. The picks are ordered by (logit desc, expert id asc) and weighted by a
// softmax over the picked logits.
#pragma once

#include "common.h"

namespace qmoe {

__device__ __forceinline__ float x_as_f32(float v) { return v; }
__device__ __forceinline__ float x_as_f32(uint16_t v) { return bf16_to_f32(v); }

typedef double f64x4_t __attribute__((ext_vector_type(4)));

constexpr int kRouterSplits = 4;                  // workgroups along the reduction
constexpr int kRouterParts = 4 * kRouterSplits;   // wavefronts along the reduction
constexpr int kRouterMaxGPP = 6;                  // groups per part: d_model <= 6144

// a beats b: larger logit, ties to the lower expert id. A NaN logit ranks below
// every number (as -inf), so this is a strict total order on (logit, id) and the
// picks are always k distinct valid ids, whatever the activations hold.
__device__ __forceinline__ bool beats(double va, int ea, double vb, int eb) {
  va = va != va ? -INFINITY : va;
  vb = vb != vb ? -INFINITY : vb;
  return va > vb || (va == vb && ea < eb);
}

// Unsigned key with the order of beats() on the logit part: NaN as -inf, -0 as +0.
__device__ __forceinline__ uint64_t order_key(double v) {
  if (v != v) v = -INFINITY;
  v += 0.0;  // -0 -> +0
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// Top-k of E keys (E <= 256, a multiple of 64) by rank, all 256 threads of the
// workgroup: rank = the number of experts that beat this one under (key desc,
// id asc), a strict total order, so the ranks are a permutation. 256 / E threads
// per expert each count the competitors in their share, reading the keys 16 at a
// time (one LDS wait per batch). The count runs on the high 32 bits of the keys;
// a wavefront in which some expert meets another with equal high bits recounts on
// the whole keys and ids. Writes the ids of ranks 0..k-1 to sel_e[rank]. key,
// rank and sel_e are LDS; ends with a barrier.
__device__ __forceinline__ void rank_topk(const uint64_t* key, int E, int k, int (*rank)[256], int* sel_e) {
  const int tid = threadIdx.x;
  const int parts = 256 / E, h = tid / E, per = E / parts, me = tid % E;
  const uint64_t mine = key[me];
  const uint32_t mh = (uint32_t)(mine >> 32);
  const uint32_t* kw = reinterpret_cast<const uint32_t*>(key);
  int r = 0, eq = 0;
  for (int c0 = h * per; c0 < (h + 1) * per; c0 += 16) {
    uint32_t kh[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) kh[i] = kw[2 * (c0 + i) + 1];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      r += kh[i] > mh ? 1 : 0;
      eq += kh[i] == mh ? 1 : 0;
    }
  }
  if (me / per == h) --eq;  // itself
  if (__any(eq > 0)) {
    r = 0;
    for (int c0 = h * per; c0 < (h + 1) * per; c0 += 16) {
      uint64_t kk[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) kk[i] = key[c0 + i];
#pragma unroll
      for (int i = 0; i < 16; ++i) r += (kk[i] > mine || (kk[i] == mine && c0 + i < me)) ? 1 : 0;
    }
  }
  rank[h][me] = r;
  __syncthreads();
  if (tid < E) {
    int rk = 0;
    for (int j = 0; j < parts; ++j) rk += rank[j][tid];
    if (rk < k) sel_e[rk] = tid;
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t u4_at(const uint4& u, int c) {
  return c == 0 ? u.x : c == 1 ? u.y : c == 2 ? u.z : u.w;
}

// 16 consecutive activations of one row, loaded raw (32 bytes of bf16, 64 of fp32).
template <typename XT>
struct XRow16;
template <>
struct XRow16<uint16_t> {
  uint4 v[2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    v[0] = ldg16(reinterpret_cast<const uint8_t*>(p));
    v[1] = ldg16(reinterpret_cast<const uint8_t*>(p) + 16);
  }
  __device__ __forceinline__ double at(int t) const {
    const uint32_t w = u4_at(v[t >> 3], (t >> 1) & 3);
    return (double)((t & 1) ? bf16_hi(w) : bf16_lo(w));
  }
  // the 16 values added in order in fp32
  __device__ __forceinline__ float sum16() const {
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint32_t w = u4_at(v[t >> 3], (t >> 1) & 3);
      s += (t & 1) ? bf16_hi(w) : bf16_lo(w);
    }
    return s;
  }
};
template <>
struct XRow16<float> {
  uint4 v[4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = ldg16(reinterpret_cast<const uint8_t*>(p) + 16 * c);
  }
  __device__ __forceinline__ double at(int t) const { return (double)__uint_as_float(u4_at(v[t >> 2], t & 3)); }
  __device__ __forceinline__ float sum16() const {
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) s += __uint_as_float(u4_at(v[t >> 2], t & 3));
    return s;
  }
};

// Group sums X_g[row][g] = sum of the 64 activations of group g of the row, in fp32:
// the four lanes (i, j) holding 16 values each add theirs in order, then the quarter
// sums are added as (q0 + q1) + (q2 + q3). Used by the prefill gate/up kernel for the
// bias term of its affine epilogue. Wavefront `part` of the router mapping holds the
// groups part + kRouterParts n; lane i + 16 j holds row i, quarter j.
template <typename XT>
__device__ __forceinline__ void store_group_sums(const XRow16<XT>* xv, int part, int G, int row, bool row_ok,
                                                 float* __restrict__ xg) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int n = 0; n < kRouterMaxGPP; ++n) {
    const int g = part + n * kRouterParts;
    if (g < G) {  // wave-uniform
      float q = xv[n].sum16();
      q += __shfl_xor(q, 16, 64);
      q += __shfl_xor(q, 32, 64);
      if (lane < 16 && row_ok) xg[(size_t)row * ((G + 3) & ~3) + g] = q;  // rows padded to 4 groups
    }
  }
}

// Router logits over part of the reduction, on the fp64 matrix cores. Grid
// ceil(rows/16) * (n_experts/16) * kRouterSplits workgroups of 256 threads; workgroup
// (rt, et, split) computes the block rows [16 rt, +16) x experts [16 et, +16) over the
// groups g with g % kRouterParts in [4 split, +4), wavefront w taking g % kRouterParts ==
// 4 split + w. Each group is 16 steps of the 16x16x4 fp64 MFMA: lane l supplies the
// activation of row l%16 and the dequantised weight (s*q + b, exact in fp64) of expert
// l%16 at the same column, 16 (l/16) + t in step t, i.e. one quarter of the expert's
// packed 8-bit tile row and the matching 32 (bf16) or 64 (fp32) bytes of the activation
// row. All products are exact in fp64. The four wavefront sums are added in wave order
// and stored to partial[split][row][e]; rows past the end read the last row and are not
// stored.
template <typename XT>
__global__ __launch_bounds__(256) void k_router_logits(const uint8_t* __restrict__ router, const XT* __restrict__ x,
                                                       int rows, int d, int n_experts,
                                                       double* __restrict__ partial, float* __restrict__ xg) {
  __shared__ double red[4][256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_et = n_experts >> 4;
  int b = blockIdx.x;
  const int split = b % kRouterSplits;
  b /= kRouterSplits;
  const int et = b % n_et, rt = b / n_et;
  const int G = d / kGroup, part = split * 4 + wave;
  const int i = lane & 15, j = lane >> 4;
  const int e = et * 16 + i;
  const int row = min(rt * 16 + i, rows - 1);
  const uint8_t* wt = router + (size_t)(e >> 6) * G * kTile8 + j * 1024 + (e & 63) * 16;
  const uint8_t* st = router + (size_t)(e >> 6) * G * kTile8 + kTile8Codes + (e & 63) * 4;
  const XT* xr = x + (size_t)row * d + 16 * j;

  // every load of the part issued before any arithmetic
  uint4 q[kRouterMaxGPP];
  uint32_t sb[kRouterMaxGPP];
  XRow16<XT> xv[kRouterMaxGPP];
#pragma unroll
  for (int n = 0; n < kRouterMaxGPP; ++n) {
    const int g = part + n * kRouterParts;
    if (g < G) {
      q[n] = ldg16(wt + (size_t)g * kTile8);
      sb[n] = ldg4(st + (size_t)g * kTile8);
      xv[n].load(xr + g * kGroup);
    }
  }
  // the workgroups of the first 16 experts also leave the rows' group sums (if asked)
  if (xg && et == 0) store_group_sums<XT>(xv, part, G, rt * 16 + i, rt * 16 + i < rows, xg);
  f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int n = 0; n < kRouterMaxGPP; ++n) {
    if (part + n * kRouterParts < G) {
      const double s = (double)bf16_lo(sb[n]), bb = (double)bf16_hi(sb[n]);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const uint32_t code = (u4_at(q[n], t >> 2) >> (8 * (t & 3))) & 0xffu;
        const double wv = fma(s, (double)code, bb);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xv[n].at(t), wv, acc, 0, 0, 0);
      }
    }
  }
  // result layout of the 16x16 fp64 MFMA: element r of lane l is row l/16 + 4 r, column l%16
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][(j + 4 * r) * 16 + i] = acc[r];
  __syncthreads();
  const int orow = rt * 16 + (tid >> 4);
  if (orow < rows)
    partial[((size_t)split * rows + orow) * n_experts + et * 16 + (tid & 15)] =
        ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

// The group sums alone (the prefill calls that do not run the router): the router
// kernel's mapping without the experts, so the sums are the same bits. Grid
// ceil(rows/16) * kRouterSplits workgroups of 256 threads.
template <typename XT>
__global__ __launch_bounds__(256) void k_group_sums(const XT* __restrict__ x, int rows, int d,
                                                    float* __restrict__ xg) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x % kRouterSplits, rt = blockIdx.x / kRouterSplits;
  const int G = d / kGroup, part = split * 4 + wave;
  const int i = lane & 15, j = lane >> 4;
  const int row = min(rt * 16 + i, rows - 1);
  const XT* xr = x + (size_t)row * d + 16 * j;
  XRow16<XT> xv[kRouterMaxGPP];
#pragma unroll
  for (int n = 0; n < kRouterMaxGPP; ++n) {
    const int g = part + n * kRouterParts;
    if (g < G) xv[n].load(xr + g * kGroup);
  }
  store_group_sums<XT>(xv, part, G, rt * 16 + i, rt * 16 + i < rows, xg);
}

// One workgroup (256 threads) per row: the row's logits are the kRouterSplits partial
// sums added in split order, plus the offset; then the top-k by rank (rank_topk) and
// the softmax over the picks (fp64, in pick order).
__global__ __launch_bounds__(256) void k_router_select(const double* __restrict__ partial, int rows, int n_experts,
                                                       int top_k, const float* __restrict__ offset,
                                                       int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                       double* __restrict__ logits_out) {
  __shared__ double lgv[256];
  __shared__ uint64_t key[256];
  __shared__ int rank[4][256];
  __shared__ int sel_e[16];
  const int tid = threadIdx.x, row = blockIdx.x;
  if (tid < n_experts) {
    double pv[kRouterSplits];
#pragma unroll
    for (int sp = 0; sp < kRouterSplits; ++sp) pv[sp] = partial[((size_t)sp * rows + row) * n_experts + tid];
    double a = pv[0];
#pragma unroll
    for (int sp = 1; sp < kRouterSplits; ++sp) a += pv[sp];
    if (offset) a += (double)offset[tid];
    lgv[tid] = a;
    key[tid] = order_key(a);
    if (logits_out) logits_out[(size_t)row * n_experts + tid] = a;
  }
  __syncthreads();
  rank_topk(key, n_experts, top_k, rank, sel_e);
  if (tid < 64) {
    const int lane = tid;
    const int se = lane < top_k ? sel_e[lane] : 0;
    const double ex = lane < top_k ? exp(lgv[se] - lgv[sel_e[0]]) : 0.0;
    double sum = 0.0;
    for (int t = 0; t < top_k; ++t) sum += readlane_f64(ex, t);
    if (lane < top_k) {
      topk_idx[(size_t)row * top_k + lane] = se;
      topk_w[(size_t)row * top_k + lane] = (float)(ex / sum);
    }
  }
}

}  // namespace qmoe
