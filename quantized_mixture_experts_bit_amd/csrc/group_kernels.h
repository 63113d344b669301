// Token-to-expert grouping (prefill) and the prefill combine.
//
// Prefill works on chunks of rows so that one fetched expert serves every row of
// the chunk routed to it (blog-mushroom article "TurboFieldfare: Gemma 4 26B on
// an 8 GB MacBook", section "Why 26B Fits in 2 GB"; paperfeed digest
// "drumih/turbo-fieldfare", "How it works"). The (row, slot) pairs are grouped
// by expert with a stable counting sort so each expert's rows form one
// contiguous range of a GEMM.
#pragma once

#include "common.h"

namespace qmoe {

// One wavefront. Thread t owns pairs [t*chunk, (t+1)*chunk) in order; cnt[e][t]
// counts them per expert, is turned into per-(expert, thread) start positions
// by an exclusive scan in (expert, thread) order, and every thread then places
// its own pairs in order: a stable counting sort, bit-exact.
__global__ __launch_bounds__(64) void k_group(const int32_t* __restrict__ topk_idx, int n_pairs, int n_experts,
                                              int32_t* __restrict__ count, int32_t* __restrict__ offset,
                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
  extern __shared__ uint16_t cnt[];  // [n_experts][64]
  __shared__ int32_t tot[257];
  const int t = threadIdx.x;
  const int chunk = (n_pairs + 63) / 64;
  for (int i = t; i < n_experts * 64; i += 64) cnt[i] = 0;
  __syncthreads();
  const int p0 = t * chunk, p1 = min(n_pairs, p0 + chunk);
  for (int p = p0; p < p1; ++p) {
    const int e = topk_idx[p];
    if (e < 0 || e >= n_experts) {  // not an expert id: reported, and the pair is dropped
      flag_device_error(2u);
      continue;
    }
    cnt[e * 64 + t] += 1;
  }
  __syncthreads();
  for (int e = t; e < n_experts; e += 64) {
    int s = 0;
    for (int j = 0; j < 64; ++j) s += cnt[e * 64 + j];
    tot[e] = s;
  }
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int e = 0; e < n_experts; ++e) {
      const int c = tot[e];
      count[e] = c;
      offset[e] = run;
      tot[e] = run;
      run += c;
    }
    offset[n_experts] = run;
  }
  __syncthreads();
  for (int e = t; e < n_experts; e += 64) {
    int run = tot[e];
    for (int j = 0; j < 64; ++j) {
      const int c = cnt[e * 64 + j];
      cnt[e * 64 + j] = (uint16_t)run;  // starts fit: n_pairs < 65536 is checked on the host
      run += c;
    }
  }
  __syncthreads();
  for (int p = p0; p < p1; ++p) {
    const int e = topk_idx[p];
    if (e < 0 || e >= n_experts) {
      inv_perm[p] = -1;
      continue;
    }
    const int pos = cnt[e * 64 + t];
    cnt[e * 64 + t] = (uint16_t)(pos + 1);
    perm[pos] = p;
    inv_perm[p] = pos;
  }
}

// y[r][n] = S[r][n] + sum_k w[r][k] * E[pos(r, k)][n], k in slot order; optional residual
// x' = bf16_rne(fp32(x) + y).
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ shared_out,
                                                 const float* __restrict__ expert_out,
                                                 const int32_t* __restrict__ inv_perm,
                                                 const float* __restrict__ topk_w, int rows, int d, int top_k,
                                                 float* __restrict__ y, uint16_t* __restrict__ residual) {
  const int r = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= d) return;
  float v = shared_out[(size_t)r * d + n];
  for (int k = 0; k < top_k; ++k) {
    const int pos = inv_perm ? inv_perm[r * top_k + k] : r * top_k + k;
    if (pos < 0) continue;  // a pair the grouping dropped (invalid id, already reported)
    v = fmaf(topk_w[r * top_k + k], expert_out[(size_t)pos * d + n], v);
  }
  y[(size_t)r * d + n] = v;
  if (residual) {
    const float t = bf16_to_f32(residual[(size_t)r * d + n]) + v;
    residual[(size_t)r * d + n] = (uint16_t)f32_to_bf16_bits(t);
  }
}

}  // namespace qmoe
