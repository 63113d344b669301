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

// Lanes of the wavefront holding the same expert id as this lane (ids < 256: one
// ballot per id bit); only lanes with `valid` set take part.
__device__ __forceinline__ uint64_t match_lanes(int e, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t on = __ballot(bit);
    m &= bit ? on : ~on;
  }
  return m;
}

constexpr int kGroupWaves = 16;  // one workgroup of 1024 threads
constexpr int kGroupRounds = 4;  // rounds of 64 pairs per wave kept in registers between the passes

// Stable counting sort of the (row, slot) pairs by expert, in one workgroup.
// Wave w owns the pairs [w*S, (w+1)*S) (S a multiple of 64) and walks them 64 at
// a time in order, so the pairs are visited in (wave, round, lane) = pair order.
// Pass 1 counts each wave's pairs per expert (lanes with the same id are matched
// with ballots; the lowest adds the group's size). Per expert, the wave counts are
// scanned in wave order, and the totals across experts. Pass 2 walks the pairs
// again: a pair's position is its expert's offset + the pairs of that expert in
// earlier waves + those in earlier rounds of its wave (the running count) + the
// matching lanes below it. The result is the order (expert, pair) exactly. The
// first kGroupRounds rounds of a wave keep their ids and lane matches in registers
// from pass 1 to pass 2.
__global__ __launch_bounds__(1024) void k_group(const int32_t* __restrict__ topk_idx, int n_pairs, int n_experts,
                                                int32_t* __restrict__ count, int32_t* __restrict__ offset,
                                                int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
  extern __shared__ int32_t cnt[];  // [kGroupWaves][n_experts]
  __shared__ int32_t off[256];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  const int S = ((n_pairs + kGroupWaves - 1) / kGroupWaves + 63) & ~63;
  const int p_end = min(n_pairs, (w + 1) * S);
  // ids of the first rounds: every load issued before the counters are cleared
  int ids[kGroupRounds];
#pragma unroll
  for (int r = 0; r < kGroupRounds; ++r) {
    const int p = w * S + 64 * r + lane;
    ids[r] = p < p_end ? topk_idx[p] : -1;
  }
  for (int i = t; i < kGroupWaves * n_experts; i += 1024) cnt[i] = 0;
  __syncthreads();
  int32_t* mine = cnt + w * n_experts;
  // pass 1; an id that is not an expert id is reported and its pair dropped
  auto count_round = [&](int p, int e) __attribute__((always_inline)) {
    if (p < p_end && (e < 0 || e >= n_experts)) {
      flag_device_error(2u);
      e = -1;
    }
    const uint64_t m = match_lanes(e, e >= 0);
    if (e >= 0 && (m & below) == 0) mine[e] += __popcll(m);
    return m;
  };
  uint64_t match[kGroupRounds];
#pragma unroll
  for (int r = 0; r < kGroupRounds; ++r) {
    if (w * S + 64 * r >= p_end) break;  // wave-uniform
    const int p = w * S + 64 * r + lane;
    match[r] = count_round(p, ids[r]);
    if (ids[r] >= n_experts) ids[r] = -1;
  }
  for (int p0 = w * S + 64 * kGroupRounds; p0 < p_end; p0 += 64) {
    const int p = p0 + lane;
    (void)count_round(p, p < p_end ? topk_idx[p] : -1);
  }
  __syncthreads();
  // per expert: wave counts -> starts within the expert, in wave order (all read first)
  for (int e = t; e < n_experts; e += 1024) {
    int c[kGroupWaves];
#pragma unroll
    for (int ww = 0; ww < kGroupWaves; ++ww) c[ww] = cnt[ww * n_experts + e];
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < kGroupWaves; ++ww) {
      cnt[ww * n_experts + e] = run;
      run += c[ww];
    }
    off[e] = run;  // total for now
  }
  __syncthreads();
  // exclusive scan of the totals over the experts (wave 0, four experts per lane)
  if (w == 0) {
    int v[4], local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      v[j] = e < n_experts ? off[e] : 0;
      local += v[j];
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    int run = incl - local;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      if (e < n_experts) {
        count[e] = v[j];
        offset[e] = run;
        off[e] = run;
      }
      run += v[j];
    }
    if (lane == 63) offset[n_experts] = incl;
  }
  __syncthreads();
  // pass 2; every lane reads the running count before the lowest lane of each group
  // advances it (one wavefront, LDS operations in order)
  auto place = [&](int p, int e, uint64_t m) __attribute__((always_inline)) {
    if (e >= 0) {
      const int pos = off[e] + mine[e] + __popcll(m & below);
      perm[pos] = p;
      inv_perm[p] = pos;
    } else if (p < p_end) {
      inv_perm[p] = -1;
    }
    if (e >= 0 && (m & below) == 0) mine[e] += __popcll(m);
  };
#pragma unroll
  for (int r = 0; r < kGroupRounds; ++r) {
    if (w * S + 64 * r >= p_end) break;  // wave-uniform
    place(w * S + 64 * r + lane, ids[r], match[r]);
  }
  for (int p0 = w * S + 64 * kGroupRounds; p0 < p_end; p0 += 64) {
    const int p = p0 + lane;
    int e = p < p_end ? topk_idx[p] : -1;
    if (e >= n_experts) e = -1;
    place(p, e, match_lanes(e, e >= 0));
  }
}

// y[r][n] = S[r][n] + sum_k w[r][k] * E[pos(r, k)][n], k in slot order; optional residual
// x' = bf16_rne(fp32(x) + y). Workgroup (column block, row r): four consecutive columns
// per thread; the row's positions and weights are uniform, and every routed output of
// the thread is loaded before the first one is added (top_k <= kMaxTopK).
constexpr int kMaxTopK = 16;
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ shared_out, int shared_parts,
                                                 const float* __restrict__ expert_out,
                                                 const int32_t* __restrict__ inv_perm,
                                                 const float* __restrict__ topk_w, int rows, int d, int top_k,
                                                 float* __restrict__ y, uint16_t* __restrict__ residual) {
  const int r = blockIdx.y;
  const int n = 4 * ((int)blockIdx.x * 256 + (int)threadIdx.x);
  if (n >= d) return;
  int pos[kMaxTopK];
  float4 e[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (k < top_k) {
      pos[k] = inv_perm ? inv_perm[r * top_k + k] : r * top_k + k;
      // a pair the grouping dropped (invalid id, already reported) has no output
      e[k] = *reinterpret_cast<const float4*>(expert_out + (size_t)max(pos[k], 0) * d + n);
    }
  }
  // the shared expert: its K parts (shared_out + p * rows * d) added in order
  float4 v = *reinterpret_cast<const float4*>(shared_out + (size_t)r * d + n);
  for (int p = 1; p < shared_parts; ++p) {
    const float4 u = *reinterpret_cast<const float4*>(shared_out + ((size_t)p * rows + r) * d + n);
    v.x += u.x;
    v.y += u.y;
    v.z += u.z;
    v.w += u.w;
  }
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (k < top_k && pos[k] >= 0) {
      const float w = topk_w[r * top_k + k];
      v.x = fmaf(w, e[k].x, v.x);
      v.y = fmaf(w, e[k].y, v.y);
      v.z = fmaf(w, e[k].z, v.z);
      v.w = fmaf(w, e[k].w, v.w);
    }
  }
  *reinterpret_cast<float4*>(y + (size_t)r * d + n) = v;
  if (residual) {
    const uint2 rb = *reinterpret_cast<const uint2*>(residual + (size_t)r * d + n);
    const float t0 = bf16_lo(rb.x) + v.x, t1 = bf16_hi(rb.x) + v.y;
    const float t2 = bf16_lo(rb.y) + v.z, t3 = bf16_hi(rb.y) + v.w;
    *reinterpret_cast<uint2*>(residual + (size_t)r * d + n) =
        make_uint2(f32_to_bf16_bits(t0) | (f32_to_bf16_bits(t1) << 16), f32_to_bf16_bits(t2) | (f32_to_bf16_bits(t3) << 16));
  }
}

}  // namespace qmoe
