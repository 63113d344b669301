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

constexpr int kRouterGPW = 4;                   // groups per wavefront
constexpr int kRouterGPB = 4 * kRouterGPW;      // groups per workgroup (4 waves)
constexpr int kMaxRouterSplits = 6;             // d_model <= 6144: at most 96 groups / 16

__device__ __forceinline__ void st_agent_d(double* p, double v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_agent_d(const double* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// grid (n_experts/64, nsplit, ceil(rows/RPW)), block 256. Workgroup (nb, split, chunk):
// lane = expert nb*64 + lane, wave w = groups [split*16 + 4w, +4) of the reduction,
// rows [chunk*RPW, +RPW). Partial logits go to `partial` [nsplit][rows][E]; the
// last workgroup of a row chunk (arrival counter) sums them in split order, adds
// the offset and picks the top-k of each row of the chunk (rank_topk).
template <typename XT, int RPW>
__global__ __launch_bounds__(256) void k_router(const uint8_t* __restrict__ router, const XT* __restrict__ x,
                                                int rows, int d, int n_experts, int top_k, int nsplit,
                                                const float* __restrict__ offset, double* __restrict__ partial,
                                                uint32_t* __restrict__ counters, int32_t* __restrict__ topk_idx,
                                                float* __restrict__ topk_w, double* __restrict__ logits_out) {
  __shared__ double xs[RPW][kRouterGPB * kGroup];
  __shared__ double red[4][RPW][64];
  __shared__ int last;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = blockIdx.x, split = blockIdx.y, chunk = blockIdx.z;
  const int G = d / kGroup;
  const int gs0 = split * kRouterGPB;
  const int ngs = min(G - gs0, kRouterGPB);
  const int r0 = chunk * RPW;
  const int nr = min(rows - r0, RPW);

  // this wave's codes and scales, all loads issued before any arithmetic
  const int gw0 = gs0 + wave * kRouterGPW;
  const int ngw = max(0, min(kRouterGPW, gs0 + ngs - gw0));
  uint4 q[kRouterGPW][4];
  uint32_t sbw[kRouterGPW];
#pragma unroll
  for (int i = 0; i < kRouterGPW; ++i) {
    if (i < ngw) {
      const uint8_t* tile = router + ((size_t)nb * G + gw0 + i) * kTile8;
#pragma unroll
      for (int c = 0; c < 4; ++c) q[i][c] = ldg16(tile + c * 1024 + lane * 16);
      sbw[i] = ldg4(tile + kTile8Codes + lane * 4);
    }
  }
  for (int i = tid; i < RPW * kRouterGPB * kGroup; i += 256) {
    const int r = i / (kRouterGPB * kGroup), c = i % (kRouterGPB * kGroup);
    xs[r][c] = (r < nr && c < ngs * kGroup) ? (double)x_as_f32(x[(size_t)(r0 + r) * d + gs0 * kGroup + c]) : 0.0;
  }
  __syncthreads();

  double acc[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) acc[r] = 0.0;
#pragma unroll
  for (int i = 0; i < kRouterGPW; ++i) {
    if (i < ngw) {
      const double s = (double)bf16_lo(sbw[i]), b = (double)bf16_hi(sbw[i]);
      const int cbase = (wave * kRouterGPW + i) * kGroup;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t words[4] = {q[i][c].x, q[i][c].y, q[i][c].z, q[i][c].w};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const double wv = fma(s, (double)((words[j >> 2] >> (8 * (j & 3))) & 0xffu), b);
#pragma unroll
          for (int r = 0; r < RPW; ++r) acc[r] = fma(wv, xs[r][cbase + c * 16 + j], acc[r]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  if (wave == 0) {
    const int e = nb * 64 + lane;
#pragma unroll
    for (int r = 0; r < RPW; ++r)
      if (r < nr)
        st_agent_d(&partial[((size_t)split * rows + r0 + r) * n_experts + e],
                   ((red[0][r][lane] + red[1][r][lane]) + red[2][r][lane]) + red[3][r][lane]);
    wait_mem();
    if (lane == 0)
      last = (arrive(&counters[chunk]) == (uint32_t)((n_experts / 64) * nsplit - 1));
  }
  __syncthreads();
  if (!last) return;

  // ---- logits of the chunk's rows (partials summed in split order, + offset), then
  // per row: ranking by all 256 threads and the softmax over the picks
  __shared__ double lgv[RPW][256];
  __shared__ uint64_t key[256];
  __shared__ int rank[4][256];
  __shared__ int sel_e[16];
  for (int i = tid; i < nr * n_experts; i += 256) {
    const int r = i / n_experts, e = i % n_experts, row = r0 + r;
    double pv[kMaxRouterSplits];  // all loads in flight at once, summed in split order
#pragma unroll
    for (int sp = 0; sp < kMaxRouterSplits; ++sp)
      pv[sp] = sp < nsplit ? ld_agent_d(&partial[((size_t)sp * rows + row) * n_experts + e]) : 0.0;
    double a = 0.0;
#pragma unroll
    for (int sp = 0; sp < kMaxRouterSplits; ++sp) a += pv[sp];
    if (offset) a += (double)offset[e];
    lgv[r][e] = a;
    if (logits_out) logits_out[(size_t)row * n_experts + e] = a;
  }
  for (int r = 0; r < nr; ++r) {
    __syncthreads();  // lgv complete; the previous row's picks are read
    if (tid < n_experts) key[tid] = order_key(lgv[r][tid]);
    __syncthreads();
    rank_topk(key, n_experts, top_k, rank, sel_e);
    if (wave == 0) {
      // softmax over the picks in pick order (fp64), fixed summation order
      const int row = r0 + r;
      const int se = lane < top_k ? sel_e[lane] : 0;
      const double ex = lane < top_k ? exp(lgv[r][se] - lgv[r][sel_e[0]]) : 0.0;
      double sum = 0.0;
      for (int t = 0; t < top_k; ++t) sum += __shfl(ex, t, 64);
      if (lane < top_k) {
        topk_idx[(size_t)row * top_k + lane] = se;
        topk_w[(size_t)row * top_k + lane] = (float)(ex / sum);
      }
    }
  }
  if (tid == 0) counters[chunk] = 0u;
}

}  // namespace qmoe
