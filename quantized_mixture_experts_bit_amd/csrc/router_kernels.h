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

// grid (n_experts/64, nsplit, ceil(rows/RPW)), block 256. Workgroup (nb, split, chunk):
// lane = expert nb*64 + lane, wave w = groups [split*16 + 4w, +4) of the reduction,
// rows [chunk*RPW, +RPW). Partial logits go to `partial` [nsplit][rows][E]; the
// last workgroup of a row chunk (arrival counter) sums them in split order, adds
// the offset and picks the top-k of each row of the chunk (one wave per row).
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

  // ---- top-k + softmax for the chunk's rows, one wave per row
  if (wave < nr) {
    const int row = r0 + wave;
    double l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < n_experts) {
        double pv[kMaxRouterSplits];  // all loads in flight at once, summed in split order
#pragma unroll
        for (int sp = 0; sp < kMaxRouterSplits; ++sp)
          pv[sp] = sp < nsplit ? ld_agent_d(&partial[((size_t)sp * rows + row) * n_experts + e]) : 0.0;
        double a = 0.0;
#pragma unroll
        for (int sp = 0; sp < kMaxRouterSplits; ++sp) a += pv[sp];
        if (offset) a += (double)offset[e];
        l[j] = a;
        if (logits_out) logits_out[(size_t)row * n_experts + e] = a;
      } else {
        l[j] = -INFINITY;
      }
    }
    double sel_v = 0.0;  // lane t < top_k keeps pick t
    int sel_e = 0;
    unsigned taken = 0;
    double top = 0.0;
    for (int t = 0; t < top_k; ++t) {
      double bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        if (e < n_experts && !((taken >> j) & 1u) && beats(l[j], e, bv, be)) {
          bv = l[j];
          be = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const double ov = __shfl_xor(bv, off, 64);
        const int oe = __shfl_xor(be, off, 64);
        if (beats(ov, oe, bv, be)) {
          bv = ov;
          be = oe;
        }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      if (t == 0) top = bv;
      if (lane == t) {
        sel_v = bv;
        sel_e = be;
      }
    }
    // softmax over the picks in pick order (fp64), fixed summation order
    const double ex = lane < top_k ? exp(sel_v - top) : 0.0;
    double sum = 0.0;
    for (int t = 0; t < top_k; ++t) sum += __shfl(ex, t, 64);
    if (lane < top_k) {
      topk_idx[(size_t)row * top_k + lane] = sel_e;
      topk_w[(size_t)row * top_k + lane] = (float)(ex / sum);
    }
  }
  if (tid == 0) counters[chunk] = 0u;
}

}  // namespace qmoe
