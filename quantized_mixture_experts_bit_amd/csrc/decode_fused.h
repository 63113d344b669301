// One decode row through the whole block in ONE persistent launch.
//
// The block's dependency chain for one token is router -> top-k -> routed gate/up
// -> GeGLU -> routed down -> combine, with the shared expert independent of the
// routing (the pages run the shared-expert branch while the routed experts are
// being fetched: blog-mushroom article "TurboFieldfare: Gemma 4 26B on an 8 GB
// MacBook", section "Why 26B Fits in 2 GB"). Separate launches serialise every
// step's latency; here the workgroups of one launch take work items in
// dependency order (workgroup index = item index):
//
//   [router partials | shared gate/up | routed gate/up | shared down | routed down]
//
// and a workgroup that needs earlier results waits on a flag (bounded spin; a
// timeout sets MOE_DEVERR_SYNC_TIMEOUT instead of hanging). Items wait only on
// items with smaller indices, and the launch is only used when the whole grid
// fits on the chip at once. Waiting items first issue every load that does not
// depend on the awaited data: a routed down item streams its weights as soon as
// the routing is known, before the GeGLU output exists.
//   - router: fp64 partial logits of 64 experts x 4 groups; the last arriving
//     router workgroup sums the partials, ranks all experts (logit desc, id asc),
//     and publishes a routing record (picks, softmax weights, blob offsets);
//   - gate/up: (slot, matrix, 64-row block, reduction part) -> fp32 partials;
//   - down: the item rebuilds h = gelu(gate) * up for its reduction range from the
//     partials (fixed order), then runs the 4-bit GEMV; the last of the
//     top_k + Ps items of each 64-row output block forms y (+ residual).
// Hand-offs use sc1 stores/loads (see common.h), never L2 flushes. Anything many
// workgroups poll or read is replicated 16 times, 4 KiB apart, so the readers
// spread over memory channels instead of queueing on one line, and arrival
// counters are two-level so no counter takes more than a few dozen atomics.
#pragma once

#include "common.h"
#include "decode_kernels.h"
#include "router_kernels.h"

namespace qmoe {

constexpr int kSpinLimit = 1 << 20;  // polls (~1 us each) before a wait gives up

__device__ __forceinline__ uint32_t ld_agent_u(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_u(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 spins until *p >= target; then the whole workgroup proceeds.
__device__ __forceinline__ void wait_counter(const uint32_t* p, uint32_t target) {
  if (threadIdx.x == 0) {
    int it = 0;
    while (ld_agent_u(p) < target) {
      if (++it > kSpinLimit) {
        flag_device_error(4u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  asm volatile("" ::: "memory");
}

// Sync words (uint32) in the workspace:
//   [0, 4096)       counters: router, shared, per-slot, per-output-block combine, done,
//                   and level-1 counters per (slot, 64-row block) from kL1
//   flags           (2 + 16) kinds x kCopies copies, kStride words apart
//   records         kCopies copies of the routing record, kStride words apart
struct FusedSync {
  static constexpr int kRouter = 0, kShared = 1, kSlot0 = 2, kL1 = 256;
  static constexpr int kCopies = 16, kStride = 1024;
  static constexpr int kFlagBase = 4096;
  static constexpr int kRecBase = kFlagBase + (2 + 16) * kCopies * kStride;
  static constexpr int kWords = kRecBase + kCopies * kStride;
  __device__ static int combine(int top_k, int nb) { return kSlot0 + top_k + nb; }
  __device__ static int done(int top_k, int nbd) { return kSlot0 + top_k + nbd; }
  // flags: 1 = shared gate/up done, 2 + slot = routed slot done (0 unused)
  __device__ static int flag(int f, int copy) { return kFlagBase + (f * kCopies + copy) * kStride; }
  // routing record copy: one 64-bit ticket per slot (16 slots), 0 until published:
  // low word = blob offset / 256 + 1 (all ones: no blob), high word = softmax weight bits
  __device__ static int rec(int copy) { return kRecBase + copy * kStride; }
};
constexpr int kFusedSyncWords = FusedSync::kWords;

__device__ __forceinline__ void raise_flag(uint32_t* sync, int f) {
  for (int c = 0; c < FusedSync::kCopies; ++c) st_agent_u(&sync[FusedSync::flag(f, c)], 1u);
}
__device__ __forceinline__ void wait_flag(const uint32_t* sync, int f) {
  wait_counter(&sync[FusedSync::flag(f, blockIdx.x % FusedSync::kCopies)], 1u);
}
__device__ __forceinline__ uint64_t* my_record(uint32_t* sync) {
  return reinterpret_cast<uint64_t*>(sync + FusedSync::rec(blockIdx.x % FusedSync::kCopies));
}
__device__ __forceinline__ uint64_t ld_agent_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Thread 0 polls the slot's ticket (one 64-bit load: readiness and payload arrive together);
// returns the expert blob (nullptr if the pick had no valid blob) to every thread.
__device__ __forceinline__ const uint8_t* wait_ticket(const uint8_t* pool, uint32_t* sync, int slot) {
  __shared__ uint64_t tk;
  if (threadIdx.x == 0) {
    const uint64_t* p = my_record(sync) + slot;
    uint64_t v = ld_agent_u64(p);
    int it = 0;
    while (v == 0) {
      if (++it > kSpinLimit) {
        flag_device_error(4u);
        v = 0xffffffffull;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      v = ld_agent_u64(p);
    }
    tk = v;
  }
  __syncthreads();
  const uint32_t lo = (uint32_t)tk;
  if (lo == 0xffffffffu) return nullptr;
  return pool + (uint64_t)(lo - 1) * 256;
}

struct FusedArgs {
  DecodeArgs A;              // weights, shapes, partial buffers, outputs
  const uint8_t* router_blob;
  const float* offset;       // [E] or null
  double* rt_partial;        // [nsplit_r][E]
  int32_t* idx_out;          // [top_k] caller's picks
  float* w_out;              // [top_k] caller's weights
  uint32_t* sync;            // kFusedSyncWords
  int n_experts, nsplit_r;
  int n_rt, n_sg, n_rg, n_sd, n_rd;
};

// group_dot with the vector operand in LDS as 32 hi and 32 lo pairs (hh, hl point at
// the group's pair 0): the pairs are read in two batches of 16, one LDS wait each,
// and accumulated in the same order as group_dot, so the result is the same
__device__ __forceinline__ float group_dot_lds(const uint32_t* hh, const uint32_t* hl, uint4 qa, uint4 qb,
                                               uint32_t sbw, float Vg) {
  const uint32_t words[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
  float acc4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint4 h4[4], l4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h4[i] = *reinterpret_cast<const uint4*>(hh + 16 * half + 4 * i);
      l4[i] = *reinterpret_cast<const uint4*>(hl + 16 * half + 4 * i);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t w = words[4 * half + jj];
      const uint32_t hv[4] = {h4[jj].x, h4[jj].y, h4[jj].z, h4[jj].w};
      const uint32_t lv[4] = {l4[jj].x, l4[jj].y, l4[jj].z, l4[jj].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t p = nib_pair(w, t);
        acc4[t] = dot2(p, hv[t], acc4[t]);
        acc4[t] = dot2(p, lv[t], acc4[t]);
      }
    }
  }
  const float a = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
  const float s = bf16_lo(sbw), b = bf16_hi(sbw);
  return fmaf(s, a, fmaf(-128.0f, s, b) * Vg);
}

// weights of one 64-row block for groups g0 + wave + 4i (i < GW), loaded ahead of use
template <int GW>
struct RowLoads {
  uint4 qa[GW], qb[GW];
  uint32_t sb[GW];
  __device__ __forceinline__ void load(const uint8_t* rowblock, int g0, int g1, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int g = g0 + wave + 4 * i;
      if (g < g1) {
        const uint8_t* t = rowblock + (size_t)g * kTile4;
        qa[i] = ldg16(t + lane * 16);
        qb[i] = ldg16(t + 1024 + lane * 16);
        sb[i] = ldg4(t + kTile4Codes + lane * 4);
      }
    }
  }
  // against h in LDS: pairs of group g at hh/hl + (g - g0) * 32, group sums at gs[g - g0]
  __device__ __forceinline__ float dot_lds(int g0, int g1, int wave, const uint32_t* hh, const uint32_t* hl,
                                           const float* gs) const {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int g = g0 + wave + 4 * i;
      if (g < g1) acc += group_dot_lds(hh + (g - g0) * 32, hl + (g - g0) * 32, qa[i], qb[i], sb[i], gs[g - g0]);
    }
    return acc;
  }
};

struct FusedSmem {
  double xs[256];
  double red[4][64];
  double lg[256];
  double sel_v[16];
  int sel_e[16];
  int rank[4][256];
  float redf[4][64];
  uint32_t slots[256];   // the layer's slot table (last router workgroup)
  __attribute__((aligned(16))) uint32_t hh[12 * 32];  // h hi pairs for up to 12 groups
  __attribute__((aligned(16))) uint32_t hl[12 * 32];
  float hsum[12];
  int last;
};

// ------------------------------------------------------------------ router item

template <typename XT>
__device__ __forceinline__ void fused_router(const FusedArgs& F, const XT* __restrict__ x, int item, FusedSmem& S) {
  const DecodeArgs& A = F.A;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = F.n_experts, nbe = E / 64;
  const int nb = item % nbe, split = item / nbe;
  const int G = A.d / kGroup;
  const int g = split * 4 + wave;
  uint4 q[4];
  uint32_t sbw = 0;
  if (g < G) {
    const uint8_t* tile = F.router_blob + ((size_t)nb * G + g) * kTile8;
#pragma unroll
    for (int c = 0; c < 4; ++c) q[c] = ldg16(tile + c * 1024 + lane * 16);
    sbw = ldg4(tile + kTile8Codes + lane * 4);
  }
  const int xi = split * 256 + tid;
  S.xs[tid] = xi < A.d ? (double)x_as_f32(x[xi]) : 0.0;
  __syncthreads();
  double acc = 0.0;
  if (g < G) {
    const double s = (double)bf16_lo(sbw), b = (double)bf16_hi(sbw);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t words[4] = {q[c].x, q[c].y, q[c].z, q[c].w};
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc = fma(fma(s, (double)((words[j >> 2] >> (8 * (j & 3))) & 0xffu), b), S.xs[wave * 64 + c * 16 + j], acc);
    }
  }
  S.red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    st_agent_d(&F.rt_partial[(size_t)split * E + nb * 64 + lane],
               ((S.red[0][lane] + S.red[1][lane]) + S.red[2][lane]) + S.red[3][lane]);
    wait_mem();
    if (lane == 0) S.last = (arrive(&F.sync[FusedSync::kRouter]) == (uint32_t)(F.n_rt - 1));
  }
  __syncthreads();
  if (!S.last) return;
  // last router workgroup: the slot table (read while the partials arrive), the full
  // logits (tpe threads per expert, loads in flight together), the ranking, the tickets
  const uint32_t slot_entry = tid < E ? A.slot_table[tid] : 0u;
  const int tpe = 256 / E;
  const int e = tid % E, sub = tid / E;
  double part = 0.0;
  for (int sp0 = sub; sp0 < F.nsplit_r; sp0 += 8 * tpe) {
    double pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int sp = sp0 + i * tpe;
      pv[i] = sp < F.nsplit_r ? ld_agent_d(&F.rt_partial[(size_t)sp * E + e]) : 0.0;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) part += pv[i];
  }
  S.xs[tid] = part;  // xs is free now: per-(sub, expert) partial sums
  __syncthreads();
  if (tid < E) {
    double l = 0.0;
    for (int s2 = 0; s2 < tpe; ++s2) l += S.xs[s2 * E + tid];
    if (F.offset) l += (double)F.offset[tid];
    S.lg[tid] = l;
  }
  __syncthreads();
  // the ranking (rank_topk: integer order keys, ties by id) and the picks' logits
  uint64_t* key = reinterpret_cast<uint64_t*>(S.xs);  // xs is free now
  if (tid < E) {
    key[tid] = order_key(S.lg[tid]);
    S.slots[tid] = slot_entry;
  }
  __syncthreads();
  rank_topk(key, E, A.top_k, S.rank, S.sel_e);
  if (tid < A.top_k) S.sel_v[tid] = S.lg[S.sel_e[tid]];
  __syncthreads();
  if (wave == 0) {
    const int k = A.top_k;
    const double ex = lane < k ? exp(S.sel_v[lane] - S.sel_v[0]) : 0.0;
    double sum = 0.0;
    for (int t = 0; t < k; ++t) sum += __shfl(ex, t, 64);
    // ticket of slot (lane & 15), stored by 4 lanes into 4 of the 16 record copies each
    const int t = lane & 15;
    const double ext = __shfl(ex, t, 64);
    uint64_t ticket = 0;
    if (t < k) {
      const int ei = S.sel_e[t];
      const float wv = (float)(ext / sum);
      const uint8_t* blob = nullptr;  // as expert_blob, from the table read above
      if (ei < 0 || ei >= E) {
        flag_device_error(2u);
      } else if ((uint64_t)S.slots[ei] >= A.n_blobs) {
        flag_device_error(1u);
      } else {
        blob = A.pool + (uint64_t)S.slots[ei] * A.stride;
      }
      const uint32_t lo = blob ? (uint32_t)((uint64_t)(blob - A.pool) / 256 + 1) : 0xffffffffu;
      ticket = ((uint64_t)__float_as_uint(wv) << 32) | lo;
      if (lane < 16) {
        F.idx_out[t] = ei;
        F.w_out[t] = wv;
      }
      for (int c = lane >> 4; c < FusedSync::kCopies; c += 4)
        __hip_atomic_store(reinterpret_cast<uint64_t*>(F.sync + FusedSync::rec(c)) + t, ticket, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------ gate/up item

template <typename XT>
__device__ __forceinline__ void fused_gateup(const FusedArgs& F, const XT* __restrict__ x, int u, bool routed,
                                             FusedSmem& S) {
  const DecodeArgs& A = F.A;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int slot, Fd;
  const uint8_t* blob;
  if (routed) {
    const int per = 2 * (A.f / 64) * A.P;
    slot = u / per;
    u -= slot * per;
    Fd = A.f;
    blob = wait_ticket(A.pool, F.sync, slot);
  } else {
    slot = A.top_k;
    Fd = A.fs;
    blob = A.shared_blob;
  }
  const int NB = Fd / 64;
  const int mat = u / (NB * A.P);
  const int nb = (u / A.P) % NB;
  const int part = u % A.P;
  const int G = A.d / kGroup;
  const int GP = (G + A.P - 1) / A.P;
  const int g0 = part * GP, g1 = min(G, g0 + GP);
  float acc = 0.0f;
  if (blob) {
    const uint8_t* rowblock = blob + (uint64_t)mat * m4_bytes(Fd, A.d) + (uint64_t)nb * G * kTile4;
    if constexpr (sizeof(XT) == 2)
      acc = block_rows_dot<3>(rowblock, g0, g1, wave, lane, VecBF16{reinterpret_cast<const uint32_t*>(x)},
                              XGroupSum<XT>{x});
    else
      acc = block_rows_dot<3>(rowblock, g0, g1, wave, lane, VecF32{reinterpret_cast<const float*>(x)},
                              XGroupSum<XT>{x});
  }
  const float r = reduce_waves4(acc, S.redf, wave, lane);
  if (wave == 0) {
    const size_t pbase = ((size_t)(slot * 2 + mat) * A.nbmax + nb) * A.P;
    st_agent(&A.gu_partial[(pbase + part) * 64 + lane], r);
    wait_mem();
    if (lane == 0) {
      // level 1: the 2P items of this (slot, block); level 2: the blocks of the slot
      uint32_t* l1 = &F.sync[FusedSync::kL1 + slot * A.nbmax + nb];
      if (arrive(l1) == (uint32_t)(2 * A.P - 1)) {
        st_agent_u(l1, 0u);
        const int c2 = routed ? FusedSync::kSlot0 + slot : FusedSync::kShared;
        if (arrive(&F.sync[c2]) == (uint32_t)(NB - 1)) raise_flag(F.sync, routed ? 2 + slot : 1);
      }
    }
  }
}

// ------------------------------------------------------------------ down item (+ combine)

// h = gelu(sum of gate parts) * (sum of up parts) for d_ff groups [g0, g1) of `slot`
// (at most 12 groups, P <= 4), into LDS as hi/lo bf16 pairs with per-group sums
__device__ __forceinline__ void build_h(const DecodeArgs& A, int slot, int g0, int g1, FusedSmem& S) {
  const int tid = threadIdx.x;
  const int n = (g1 - g0) * 64;
  float gv[3][4], uv[3][4];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int idx = tid + 256 * i;
    const int j = g0 * 64 + idx, nbj = j >> 6, r = j & 63;
    const size_t gb = ((size_t)(slot * 2 + 0) * A.nbmax + nbj) * A.P;
    const size_t ub = ((size_t)(slot * 2 + 1) * A.nbmax + nbj) * A.P;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const bool ok = idx < n && p < A.P;
      gv[i][p] = ok ? ld_agent(&A.gu_partial[(gb + p) * 64 + r]) : 0.0f;
      uv[i][p] = ok ? ld_agent(&A.gu_partial[(ub + p) * 64 + r]) : 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int idx = tid + 256 * i;
    if (idx < n) {
      const float gs = ((gv[i][0] + gv[i][1]) + gv[i][2]) + gv[i][3];
      const float us = ((uv[i][0] + uv[i][1]) + uv[i][2]) + uv[i][3];
      const float h = gelu_tanh(gs) * us;
      const uint32_t hi = f32_to_bf16_bits(h);
      const uint32_t lo = f32_to_bf16_bits(h - bf16_to_f32((uint16_t)hi));
      reinterpret_cast<uint16_t*>(S.hh)[idx] = (uint16_t)hi;
      reinterpret_cast<uint16_t*>(S.hl)[idx] = (uint16_t)lo;
    }
  }
  __syncthreads();
  // group sums of hi + lo, one wave per group
  const int lane = tid & 63, wave = tid >> 6;
  for (int gi = wave; gi < g1 - g0; gi += 4) {
    const int i = gi * 64 + lane;
    const float v = bf16_to_f32(reinterpret_cast<const uint16_t*>(S.hh)[i]) +
                    bf16_to_f32(reinterpret_cast<const uint16_t*>(S.hl)[i]);
    const float s = wave_sum(v);
    if (lane == 0) S.hsum[gi] = s;
  }
  __syncthreads();
}

__device__ __forceinline__ void fused_combine(const FusedArgs& F, int nb) {
  const DecodeArgs& A = F.A;
  const int lane = threadIdx.x & 63;
  if (threadIdx.x >= 64) return;
  const int n = nb * 64 + lane;
  const uint64_t* rec = my_record(F.sync);
  float sp[4], ev[16], wv[16];
#pragma unroll
  for (int p = 0; p < 4; ++p) sp[p] = p < A.Ps ? ld_agent(&A.shared_part[(size_t)p * A.d + n]) : 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    ev[k] = k < A.top_k ? ld_agent(&A.expert_out[(size_t)k * A.d + n]) : 0.0f;
    wv[k] = k < A.top_k ? __uint_as_float((uint32_t)(ld_agent_u64(&rec[k]) >> 32)) : 0.0f;
  }
  float yv = ((sp[0] + sp[1]) + sp[2]) + sp[3];
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (k < A.top_k) yv = fmaf(wv[k], ev[k], yv);
  A.y[n] = yv;
  if (A.residual) A.residual[n] = (uint16_t)f32_to_bf16_bits(bf16_to_f32(A.residual[n]) + yv);
  const int nbd = A.d / 64;
  bool final = false;
  if (lane == 0) {
    st_agent_u(&F.sync[FusedSync::combine(A.top_k, nb)], 0u);
    final = arrive(&F.sync[FusedSync::done(A.top_k, nbd)]) == (uint32_t)(nbd - 1);
  }
  if (__shfl(final ? 1 : 0, 0, 64)) {
    // every item has finished waiting: reset counters, flags and tickets for the next call,
    // spread over the wave's lanes
    if (lane < FusedSync::kSlot0 + A.top_k) st_agent_u(&F.sync[lane], 0u);
    if (lane == 0) st_agent_u(&F.sync[FusedSync::done(A.top_k, nbd)], 0u);
    for (int i = lane; i < (1 + A.top_k) * FusedSync::kCopies; i += 64)
      st_agent_u(&F.sync[FusedSync::flag(1 + i / FusedSync::kCopies, i % FusedSync::kCopies)], 0u);
    for (int i = lane; i < A.top_k * FusedSync::kCopies; i += 64)
      __hip_atomic_store(reinterpret_cast<uint64_t*>(F.sync + FusedSync::rec(i / A.top_k)) + i % A.top_k,
                         (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void fused_down(const FusedArgs& F, int u, bool routed, FusedSmem& S) {
  const DecodeArgs& A = F.A;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NBd = A.d / 64;
  int slot, Fd, g0, g1, part = 0, nb;
  const uint8_t* blob;
  if (routed) {
    slot = u / NBd;
    nb = u % NBd;
    Fd = A.f;
    g0 = 0;
    g1 = Fd / kGroup;
    blob = wait_ticket(A.pool, F.sync, slot);
  } else {
    slot = A.top_k;
    nb = u / A.Ps;
    part = u % A.Ps;
    Fd = A.fs;
    const int G = Fd / kGroup, GP = (G + A.Ps - 1) / A.Ps;
    g0 = part * GP;
    g1 = min(G, g0 + GP);
    blob = A.shared_blob;
  }
  const uint8_t* rowblock = blob ? blob + 2 * m4_bytes(Fd, A.d) + (uint64_t)nb * (Fd / kGroup) * kTile4 : nullptr;
  RowLoads<3> w;
  if (rowblock) w.load(rowblock, g0, g1, wave, lane);  // weights stream while h is produced
  wait_flag(F.sync, routed ? 2 + slot : 1);
  build_h(A, slot, g0, g1, S);
  float acc = 0.0f;
  if (rowblock)
    acc = w.dot_lds(g0, g1, wave, S.hh, S.hl, S.hsum);
  const float r = reduce_waves4(acc, S.redf, wave, lane);
  if (wave == 0) {
    const int n = nb * 64 + lane;
    st_agent(routed ? &A.expert_out[(size_t)slot * A.d + n] : &A.shared_part[(size_t)part * A.d + n], r);
    wait_mem();
    if (lane == 0)
      S.last = (arrive(&F.sync[FusedSync::combine(A.top_k, nb)]) == (uint32_t)(A.top_k + A.Ps - 1));
  }
  __syncthreads();
  if (S.last) fused_combine(F, nb);
}

// ------------------------------------------------------------------ the kernel

// Work item of a block. Blocks are dealt to the XCDs round robin (block b on XCD
// b % 8) and the XCDs start the launch one after another, the last several
// microseconds after the first; the router items head the dependency chain, so
// they take blocks 0, 8, 16, ... (the first XCD) and the
// other items the rest in order. Any placement is correct (all blocks are resident at once); this one is
// faster.
__device__ __forceinline__ int item_of_block(int b, int n_rt) {
  if ((int)gridDim.x < 8 * n_rt) return b;  // too few blocks to spread: identity
  if ((b & 7) == 0 && (b >> 3) < n_rt) return b >> 3;
  const int before = min(n_rt, (b + 7) >> 3);  // router blocks below b
  return n_rt + b - before;
}

template <typename XT>
__global__ __launch_bounds__(256, 6) void k_decode_fused(FusedArgs F, const XT* __restrict__ x) {
  __shared__ FusedSmem S;
  int b = item_of_block(blockIdx.x, F.n_rt);
  if (b < F.n_rt) return fused_router(F, x, b, S);
  b -= F.n_rt;
  // one call site per item kind, so each body is inlined once
  if (b < F.n_sg + F.n_rg) {
    const bool routed = b >= F.n_sg;
    return fused_gateup(F, x, routed ? b - F.n_sg : b, routed, S);
  }
  b -= F.n_sg + F.n_rg;
  if (b < F.n_sd + F.n_rd) {
    const bool routed = b >= F.n_sd;
    fused_down(F, routed ? b - F.n_sd : b, routed, S);
  }
}

}  // namespace qmoe
