// Decode (one activation row): fused 4-bit dequant + GEMV kernels.
//
// Lane r of a wavefront owns row r of a 64-row block and streams that row's
// codes with 16-byte loads (1 KiB contiguous per wavefront load). The affine
// dequantisation is factored out of the inner loop:
//   sum_i (s*q_i + b) v_i = s * sum_i q_i v_i + b * V_g,   V_g = sum_{i in g} v_i,
// and the inner sum runs on v_dot2_f32_bf16 with the code pair turned into the
// bf16 pair (128 + q) by masking and OR-ing an exponent (no conversions):
//   sum_i (128 + q_i) v_i = 128 V_g + sum_i q_i v_i,  so  out += s*acc + (b - 128 s) V_g.
// The vector operand (x, or the GeGLU output h) is wavefront-uniform, held as
// bf16 pairs: bf16 x is used as stored; an fp32 vector is split into
// hi + lo bf16 parts (two dot2 per pair; hi + lo carries 16 significant bits).
//
// Work split: gate/up/down rows are cut into 64-row blocks and the reduction
// dimension into P parts, so a decode call spreads over several hundred
// workgroups. Parts are reduced in fixed order by the last workgroup to arrive
// at a per-block counter (deterministic; no float atomics).
#pragma once

#include "common.h"

namespace qmoe {

// Wavefront-uniform view of the vector operand of a 4-bit GEMV.
struct VecBF16 {  // bf16 vector as stored
  const uint32_t* pairs;
  __device__ __forceinline__ uint32_t hi(int p) const { return pairs[p]; }
  __device__ __forceinline__ uint32_t lo(int) const { return 0; }
  static constexpr bool kLo = false;
};
struct VecF32 {  // fp32 vector, split into hi + lo bf16 on the fly
  const float* v;
  __device__ __forceinline__ uint32_t hi(int p) const {
    return f32_to_bf16_bits(v[2 * p]) | (f32_to_bf16_bits(v[2 * p + 1]) << 16);
  }
  __device__ __forceinline__ uint32_t lo(int p) const {
    const float a = v[2 * p], b = v[2 * p + 1];
    const float ra = a - bf16_to_f32((uint16_t)f32_to_bf16_bits(a));
    const float rb = b - bf16_to_f32((uint16_t)f32_to_bf16_bits(b));
    return f32_to_bf16_bits(ra) | (f32_to_bf16_bits(rb) << 16);
  }
  static constexpr bool kLo = true;
};
struct VecSplit {  // precomputed hi/lo bf16 arrays (the GeGLU output h)
  const uint32_t* h;
  const uint32_t* l;
  __device__ __forceinline__ uint32_t hi(int p) const { return h[p]; }
  __device__ __forceinline__ uint32_t lo(int p) const { return l[p]; }
  static constexpr bool kLo = true;
};

// sum over one group (64 columns) of one row: s * sum (128+q) v + (b - 128 s) * Vg
template <typename V>
__device__ __forceinline__ float group_dot(const V& v, int g, uint4 qa, uint4 qb, uint32_t sbw, float Vg) {
  const uint32_t words[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
  float acc4[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // four independent dot2 chains
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int pbase = g * 32 + (j >> 2) * 16 + (j & 3) * 4;  // pair index of column g*64 + h*32 + 8*jj
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t p = nib_pair(words[j], t);
      acc4[t] = dot2(p, v.hi(pbase + t), acc4[t]);
      if (V::kLo) acc4[t] = dot2(p, v.lo(pbase + t), acc4[t]);
    }
  }
  const float a = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
  const float s = bf16_lo(sbw), b = bf16_hi(sbw);
  return fmaf(s, a, fmaf(-128.0f, s, b) * Vg);
}

// Accumulate one 64-row block over the groups [g0, g1) of a 4-bit matrix with
// 4 wavefronts splitting the groups (wave w takes g0 + w, g0 + w + 4, ...).
// Returns the lane's row sum for this wavefront (to be reduced across waves).
template <int GW, typename V, typename VG>
__device__ __forceinline__ float block_rows_dot(const uint8_t* rowblock, int g0, int g1, int wave, int lane,
                                                const V& v, const VG& vg) {
  float acc = 0.0f;
  for (int gb = g0 + wave; gb < g1; gb += 4 * GW) {
    uint4 qa[GW], qb[GW];
    uint32_t sb[GW];
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int g = gb + 4 * i;
      if (g < g1) {
        const uint8_t* t = rowblock + (size_t)g * kTile4;
        qa[i] = ldg16(t + lane * 16);
        qb[i] = ldg16(t + 1024 + lane * 16);
        sb[i] = ldg4(t + kTile4Codes + lane * 4);
      }
    }
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int g = gb + 4 * i;
      if (g < g1) acc += group_dot(v, g, qa[i], qb[i], sb[i], vg(g, lane));
    }
  }
  return acc;
}

// group sums of a stored activation vector, computed by the wavefront
template <typename XT>
struct XGroupSum {
  const XT* x;
  __device__ __forceinline__ float operator()(int g, int lane) const {
    return wave_sum(x_as_f32_dev(x[g * kGroup + lane]));
  }
  __device__ __forceinline__ static float x_as_f32_dev(float v) { return v; }
  __device__ __forceinline__ static float x_as_f32_dev(uint16_t v) { return bf16_to_f32(v); }
};
struct PrecomputedGroupSum {
  const float* gs;
  __device__ __forceinline__ float operator()(int g, int) const { return gs[g]; }
};

// 4-wave reduction of a per-lane value; result valid in wave 0
__device__ __forceinline__ float reduce_waves4(float v, float (*red)[64], int wave, int lane) {
  red[wave][lane] = v;
  __syncthreads();
  float r = 0.0f;
  if (wave == 0) r = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
  return r;
}

struct DecodeArgs {
  const uint8_t* pool;
  uint64_t stride, n_blobs;
  const uint32_t* slot_table;
  const int32_t* topk_idx;
  const uint8_t* shared_blob;
  int d, f, fs, top_k, n_experts;
  int P;             // reduction parts of gate/up
  int Ps;            // reduction parts of the shared down
  int routed_units;  // workgroups for routed work (0 if none)
  int fmax, nbmax;   // per-slot capacity (max(f, fs), /64)
  float* gu_partial;  // [(top_k+1)][2][nbmax][P][64]
  uint32_t* gu_count; // [(top_k+1)][nbmax]
  uint16_t* h_hi;     // [(top_k+1)][fmax]
  uint16_t* h_lo;
  float* h_gsum;      // [(top_k+1)][nbmax]
  float* expert_out;  // [top_k][d]
  float* shared_part; // [Ps][d]
  uint32_t* dn_count; // [d/64]
  int combine_arrivals;  // 0: no combine
  int skip_ok;           // routed only, no combine: MOE_SLOT_SKIP entries leave their slots out
  const float* topk_w;
  float* y;
  uint16_t* residual;
};

// gate/up GEMVs + GeGLU. Workgroup = (slot, matrix, 64-row block, part).
template <typename XT, int GW>
__global__ __launch_bounds__(256) void k_decode_gateup(DecodeArgs A, const XT* __restrict__ x) {
  __shared__ float red[4][64];
  __shared__ int last;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int u = blockIdx.x;
  int slot, F;
  const uint8_t* blob;
  if (u < A.routed_units) {
    const int per = 2 * (A.f / 64) * A.P;
    slot = u / per;
    u -= slot * per;
    F = A.f;
    blob = expert_blob(A.pool, A.stride, A.n_blobs, A.slot_table, A.topk_idx[slot], A.n_experts, A.skip_ok != 0);
  } else {
    u -= A.routed_units;
    slot = A.top_k;
    F = A.fs;
    blob = A.shared_blob;
  }
  const int NB = F / 64;
  const int mat = u / (NB * A.P);
  const int nb = (u / A.P) % NB;
  const int part = u % A.P;
  const int G = A.d / kGroup;
  const int GP = (G + A.P - 1) / A.P;
  const int g0 = part * GP, g1 = min(G, g0 + GP);

  float acc = 0.0f;
  if (blob) {
    const uint8_t* rowblock = blob + (uint64_t)mat * m4_bytes(F, A.d) + (uint64_t)nb * G * kTile4;
    if constexpr (sizeof(XT) == 2) {
      acc = block_rows_dot<GW>(rowblock, g0, g1, wave, lane, VecBF16{reinterpret_cast<const uint32_t*>(x)},
                               XGroupSum<XT>{x});
    } else {
      acc = block_rows_dot<GW>(rowblock, g0, g1, wave, lane, VecF32{reinterpret_cast<const float*>(x)},
                               XGroupSum<XT>{x});
    }
  }
  const float r = reduce_waves4(acc, red, wave, lane);
  const size_t pbase = ((size_t)(slot * 2 + mat) * A.nbmax + nb) * A.P;
  if (wave == 0) {
    st_agent(&A.gu_partial[(pbase + part) * 64 + lane], r);
    wait_mem();
    if (lane == 0) last = (arrive(&A.gu_count[slot * A.nbmax + nb]) == (uint32_t)(2 * A.P - 1));
  }
  __syncthreads();
  if (!last) return;
  if (wave == 0) {
    const size_t gb = ((size_t)(slot * 2 + 0) * A.nbmax + nb) * A.P;
    const size_t ub = ((size_t)(slot * 2 + 1) * A.nbmax + nb) * A.P;
    float gv[8], uv[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      gv[p] = p < A.P ? ld_agent(&A.gu_partial[(gb + p) * 64 + lane]) : 0.0f;
      uv[p] = p < A.P ? ld_agent(&A.gu_partial[(ub + p) * 64 + lane]) : 0.0f;
    }
    float gs = 0.0f, us = 0.0f;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      gs += gv[p];
      us += uv[p];
    }
    const float h = gelu_tanh(gs) * us;
    const uint32_t hi = f32_to_bf16_bits(h);
    const float hif = bf16_to_f32((uint16_t)hi);
    const uint32_t lo = f32_to_bf16_bits(h - hif);
    const int j = nb * 64 + lane;
    A.h_hi[(size_t)slot * A.fmax + j] = (uint16_t)hi;
    A.h_lo[(size_t)slot * A.fmax + j] = (uint16_t)lo;
    const float hs = wave_sum(hif + bf16_to_f32((uint16_t)lo));
    if (lane == 0) {
      A.h_gsum[slot * A.nbmax + nb] = hs;
      A.gu_count[slot * A.nbmax + nb] = 0u;
    }
  }
}

// y[n] = the shared expert's parts summed in order, then + w_k E_k[n] in pick order;
// residual[n] <- bf16(residual[n] + y[n]) when there is a residual
__device__ __forceinline__ void combine_row(const DecodeArgs& A, int n) {
  float sp[8], ev[16];
#pragma unroll
  for (int p = 0; p < 8; ++p) sp[p] = p < A.Ps ? ld_agent(&A.shared_part[(size_t)p * A.d + n]) : 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) ev[k] = k < A.top_k ? ld_agent(&A.expert_out[(size_t)k * A.d + n]) : 0.0f;
  float yv = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) yv += sp[p];
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (k < A.top_k) yv = fmaf(A.topk_w[k], ev[k], yv);
  A.y[n] = yv;
  if (A.residual) {
    const float t = bf16_to_f32(A.residual[n]) + yv;
    A.residual[n] = (uint16_t)f32_to_bf16_bits(t);
  }
}

// down GEMVs (+ combine). Routed workgroup = (slot, 64-row block of d_model), all
// of d_ff; shared workgroup = (64-row block, part of d_ff_shared).
template <int GW>
__global__ __launch_bounds__(256) void k_decode_down(DecodeArgs A) {
  __shared__ float red[4][64];
  __shared__ int last;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NBd = A.d / 64;
  int u = blockIdx.x;
  int slot, F, g0, g1, part = 0, nb;
  const uint8_t* blob;
  bool skipped = false;  // a routed slot left out on purpose: its expert_out row is not written
  if (u < A.routed_units) {
    slot = u / NBd;
    nb = u % NBd;
    F = A.f;
    g0 = 0;
    g1 = F / kGroup;
    const int e = A.topk_idx[slot];
    blob = expert_blob(A.pool, A.stride, A.n_blobs, A.slot_table, e, A.n_experts, A.skip_ok != 0);
    skipped = A.skip_ok && !blob && e >= 0 && e < A.n_experts && A.slot_table[e] == kSlotSkip;
  } else {
    u -= A.routed_units;
    slot = A.top_k;
    nb = u / A.Ps;
    part = u % A.Ps;
    F = A.fs;
    const int G = F / kGroup, GP = (G + A.Ps - 1) / A.Ps;
    g0 = part * GP;
    g1 = min(G, g0 + GP);
    blob = A.shared_blob;
  }
  float acc = 0.0f;
  if (blob) {
    const uint8_t* rowblock = blob + 2 * m4_bytes(F, A.d) + (uint64_t)nb * (F / kGroup) * kTile4;
    VecSplit v{reinterpret_cast<const uint32_t*>(A.h_hi + (size_t)slot * A.fmax),
               reinterpret_cast<const uint32_t*>(A.h_lo + (size_t)slot * A.fmax)};
    acc = block_rows_dot<GW>(rowblock, g0, g1, wave, lane, v, PrecomputedGroupSum{A.h_gsum + slot * A.nbmax});
  }
  const float r = reduce_waves4(acc, red, wave, lane);
  const int n = nb * 64 + lane;
  if (wave == 0) {
    float* dst = slot < A.top_k ? &A.expert_out[(size_t)slot * A.d + n] : &A.shared_part[(size_t)part * A.d + n];
    if (A.combine_arrivals == 0) {
      if (!skipped) *dst = r;
    } else {
      st_agent(dst, r);
      wait_mem();
      if (lane == 0) last = (arrive(&A.dn_count[nb]) == (uint32_t)(A.combine_arrivals - 1));
    }
  }
  if (A.combine_arrivals == 0) return;
  __syncthreads();
  if (!last) return;
  if (wave == 0) {
    combine_row(A, n);
    if (lane == 0) A.dn_count[nb] = 0u;
  }
}

// The combine alone, after the shared expert's down parts (k_decode_down with the shared
// expert and no combine) and the routed outputs are in memory: one thread per output.
__global__ __launch_bounds__(256) void k_decode_combine(DecodeArgs A) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n < A.d) combine_row(A, n);
}

}  // namespace qmoe
