// Router GEMV/GEMM (8-bit affine, fp64 accumulation) and top-k + softmax.
//
// The router stays at 8 bits so that it picks the right experts (ai-heartland
// review "TurboFieldfareとは", system-design summary of quantisation). Every
// product w * x is exact in fp64 (w = s*q + b has <= 20 significant bits, x <= 24)
// and the sums are fp64, so the logits sit within ~1e-12 of exact and the
// top-k set matches an exact evaluation wherever the k-th/(k+1)-th gap exceeds
// that.
#pragma once

#include "common.h"

namespace qmoe {

__device__ __forceinline__ float x_as_f32(float v) { return v; }
__device__ __forceinline__ float x_as_f32(uint16_t v) { return bf16_to_f32(v); }

// Partial logits of 64 experts (one per lane) over `gpw` groups for `RPW` rows.
// grid: (n_experts/64, nsplit, ceil(rows/RPW)); block 64.
// partial layout: [nsplit][rows][n_experts], fp64.
template <typename XT, int RPW, int GPW>
__global__ __launch_bounds__(64) void k_router_partial(const uint8_t* __restrict__ router, const XT* __restrict__ x,
                                                       int rows, int d, int n_experts,
                                                       double* __restrict__ partial) {
  const int lane = threadIdx.x;
  const int nb = blockIdx.x;
  const int split = blockIdx.y;
  const int r0 = blockIdx.z * RPW;
  const int G = d / kGroup;
  const int g0 = split * GPW;
  const int ng = min(G - g0, GPW);
  const int nr = min(rows - r0, RPW);
  __shared__ double xs[RPW][GPW * kGroup];
  for (int i = lane; i < RPW * GPW * kGroup; i += 64) {
    const int r = i / (GPW * kGroup), c = i % (GPW * kGroup);
    xs[r][c] = (r < nr && c < ng * kGroup) ? (double)x_as_f32(x[(size_t)(r0 + r) * d + g0 * kGroup + c]) : 0.0;
  }
  __syncthreads();
  double acc[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) acc[r] = 0.0;
  for (int gi = 0; gi < ng; ++gi) {
    const uint8_t* tile = router + ((size_t)nb * G + g0 + gi) * kTile8;
    uint4 q[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) q[c] = ldg16(tile + c * 1024 + lane * 16);
    const uint32_t sbw = ldg4(tile + kTile8Codes + lane * 4);
    const double s = (double)bf16_lo(sbw), b = (double)bf16_hi(sbw);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t words[4] = {q[c].x, q[c].y, q[c].z, q[c].w};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const double w = fma(s, (double)((words[i >> 2] >> (8 * (i & 3))) & 0xffu), b);
#pragma unroll
        for (int r = 0; r < RPW; ++r) acc[r] = fma(w, xs[r][gi * kGroup + c * 16 + i], acc[r]);
      }
    }
  }
  const int e = nb * 64 + lane;
#pragma unroll
  for (int r = 0; r < RPW; ++r)
    if (r < nr) partial[((size_t)split * rows + r0 + r) * n_experts + e] = acc[r];
}

// a beats b: larger logit, ties to the lower expert id
__device__ __forceinline__ bool beats(double va, int ea, double vb, int eb) {
  return va > vb || (va == vb && ea < eb);
}

// One wavefront per row: reduce the partials (fixed order), add the offset,
// pick top_k by (logit desc, id asc), softmax over the picks (fp64, then fp32).
__global__ __launch_bounds__(64) void k_topk(const double* __restrict__ partial, int nsplit, int rows,
                                             int n_experts, int top_k, const float* __restrict__ offset,
                                             int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                             double* __restrict__ logits_out) {
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  double l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < n_experts) {
      double acc = 0.0;
      for (int sp = 0; sp < nsplit; ++sp) acc += partial[((size_t)sp * rows + row) * n_experts + e];
      if (offset) acc += (double)offset[e];
      l[j] = acc;
      if (logits_out) logits_out[(size_t)row * n_experts + e] = acc;
    } else {
      l[j] = -INFINITY;
    }
  }
  __shared__ double sel_v[16];
  __shared__ int sel_e[16];
  unsigned taken = 0;
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
    if (lane == 0) {
      sel_v[t] = bv;
      sel_e[t] = be;
    }
  }
  __syncthreads();
  if (lane == 0) {
    double sum = 0.0;
    for (int t = 0; t < top_k; ++t) sum += exp(sel_v[t] - sel_v[0]);
    for (int t = 0; t < top_k; ++t) {
      topk_idx[(size_t)row * top_k + t] = sel_e[t];
      topk_w[(size_t)row * top_k + t] = (float)(exp(sel_v[t] - sel_v[0]) / sum);
    }
  }
}

}  // namespace qmoe
