// One decode row through the whole block in ONE launch.
//
// The dependency chain for one token is router -> top-k -> routed gate/up ->
// GeGLU -> routed down -> combine. The shared expert does not depend on the
// routing and streams while the routed experts are picked and fetched (the pages
// run the shared-expert branch while the routed experts are being read in:
// blog-mushroom article "TurboFieldfare: Gemma 4 26B on an 8 GB MacBook", section
// "Why 26B Fits in 2 GB"); its weight loads start once the router has published.
//
// Work items, one workgroup each, in dependency order (an item waits only for
// items before it; the launch is used only when the whole grid is resident),
// and a last workgroup that keeps the epoch (below):
//   router       2 experts over the whole reduction, fp64          -> 2 logits
//   shared g/u   16 rows of the shared gate and up matrices         -> 16 values of h
//   routed g/u   (slot, 16 rows) of the slot's expert               -> 16 values of h
//   routed down  (slot, 64 output rows) over the slot's whole h     -> 64 expert outputs
//   shared down  (64 output rows, second half of the shared h)      -> 64 partial outputs
//   combine      (64 output rows, first half of the shared h), then y for those rows
//
// A hand-off between workgroups goes through the coherence point the XCDs share
// and costs about a microsecond, so the chain is cut to the fewest hand-offs:
//   - there is no ranking workgroup: every routed item and every combine reads
//     the logits and ranks the experts itself (logit desc, id asc) on unique
//     31-bit keys with independent compares, checked exact around the picks;
//   - a gate/up item covers the whole reduction of its rows, so h needs no
//     partial sums and no separate GeGLU step;
//   - every hand-off is a set of 64-bit words (32-bit payload, 32-bit tag), each
//     written by one agent-scope store; a reader polls the words it needs until
//     all carry this call's tag. No arrival counters, flags or fences sit on
//     the path. Words that many readers need (logits, h) are written
//     in several copies some kilobytes apart, so the polling does not pile onto
//     a few channels.
// The tag is the call's epoch + 1. Every workgroup reads the epoch (one of
// several copies) when it starts and, once it has it, adds one to an arrival
// counter without waiting for the result. One extra workgroup, the last of the
// grid, waits until every other workgroup has arrived, then advances the epoch
// for the next call and clears the counters: nothing reads the epoch after that.
// Waits are bounded: a timeout sets MOE_DEVERR_SYNC_TIMEOUT instead of hanging
// (the workspace must then be re-initialised).
#pragma once

#include "common.h"
#include "decode_kernels.h"
#include "router_kernels.h"

namespace qmoe {

constexpr int kSpinLimit = 1 << 20;  // polling rounds (about a microsecond each) before a wait gives up
constexpr int kFusedRows = 16;       // gate/up rows per item
constexpr int kFusedRouterE = 2;     // experts per router item
constexpr int kLgCopies = 16;        // copies of the logits ...
constexpr int kLgStride = 1024;      // ... 8 KiB apart (words)
constexpr int kLgKeys = 512;         // word of a copy where the ranking keys start
constexpr int kHCopies = 4;          // copies of h
constexpr int kSyncLine = 32;        // words per 128-byte line: one sync word per line
constexpr int kEpochCopies = 64;     // epoch copy c at line c
constexpr int kArrivalCounters = 32; // arrival counter i at line kEpochCopies + i
constexpr int kFusedSyncWords = (kEpochCopies + kArrivalCounters) * kSyncLine;
constexpr int kFusedXWords = 3072;   // LDS words holding x, or h (fp32, then scaled fp16)
constexpr int kFusedMaxG = 48;       // d_model / 64
constexpr int kFusedGuI = 6;         // gate/up loads per lane and matrix: group pairs / 4 waves
constexpr int kFusedRoutedGW = 3;    // routed down: groups of d_ff per wave (d_ff <= 768)
constexpr int kFusedSharedGW = 5;    // shared down: groups of half of d_ff_shared per wave (<= 2560)
constexpr int kXCopies = 16;         // copies of the next layer's input in the stacked decode ...
constexpr int kXStride = 2048;       // ... 16 KiB apart (words; a copy holds d_model / 2 bf16 pairs)
constexpr int kMaxStackLayers = 32;  // layers of one stacked-decode launch

struct FusedArgs {
  const uint8_t* pool;
  uint64_t stride, n_blobs;
  const uint32_t* slot_table;
  const uint8_t* router_blob;
  const uint8_t* shared_blob;
  const float* offset;  // [E] or null
  int d, f, fs, E, top_k, fmax;
  int32_t* idx_out;     // [top_k]
  float* w_out;         // [top_k]
  float* expert_out;    // [top_k][d], unweighted
  float* y;             // [d]
  uint16_t* residual;   // [d] bf16 or null: residual <- bf16(residual + y)
  uint64_t* lg_tag;     // kLgCopies x kLgStride: fp64 logits as (low, high) 32-bit halves, then
                        // at kLgKeys one ranking key per expert (see rank_logits)
  uint64_t* h_tag;      // kHCopies x [(top_k + 1) * fmax] (h_stride apart): GeGLU outputs of the routed
                        // slots, then the shared expert
  uint64_t h_stride;
  uint64_t* eo_tag;     // [(top_k + 1) * d]: routed expert outputs, then the shared expert's second half
  uint32_t* sync;       // kFusedSyncWords
  int n_rt, n_sg, n_rg, n_rd, n_sd;  // n_sd = d / 64 second-half items, then as many combines
  // stacked decode (k_stack_decode) only; zero for one layer:
  uint64_t* x_tag;      // kXCopies x kXStride: the next layer's input as tagged bf16 pairs
  int x_in, x_out;      // this layer reads its input from / writes the next layer's to x_tag
  int arrive;           // this layer's items arrive at the epoch counters (the first layer)
  uint16_t* x_rec;      // [d] or null: receives this layer's input (bf16)
  int layer;            // index in the stack (timeline stamps only)
};

struct FusedSmem {
  __attribute__((aligned(16))) uint32_t xb[kFusedXWords];  // x pairs (or values), or h
  float xg[2 * kFusedMaxG];  // sums of x over 32-column halves of each group
  float hsum[48];            // sums of the scaled fp16 h per group
  float hmax[4];             // per-wave maxima of |h| (gather_h)
  float red[2][4][64];
  double rd[256];
  double rd2[32];            // router: first-level sums of the per-thread partials
  double lg[256];
  uint64_t key[256];
  uint32_t lgw[512];
  __attribute__((aligned(16))) uint32_t kp[256];
  int rank[4][256];
  uint32_t slots[256];
  float eo[17][64];
  double lgv[kFusedRouterE];
  int sel_e[17];
  float selw[16];
};

// Timeline build (QMOE_TIMELINE): thread 0 of each workgroup stamps the 100 MHz
// real-time counter at the phase boundaries of its item into g_timeline[block][slot],
// in a stacked decode g_timeline[layer][block][slot] (kStamps slots per block; the slot
// meanings per item kind are listed at each QMOE_STAMP, which names the item's
// FusedArgs F and the kStack of the function it is in). The default build compiles the
// stamps away.
constexpr int kStamps = 8;
#ifdef QMOE_TIMELINE
__device__ uint64_t* g_timeline = nullptr;
#define QMOE_STAMP(slot)                                                                       \
  do {                                                                                         \
    if (threadIdx.x == 0 && g_timeline) {                                                      \
      size_t row_ = blockIdx.x;                                                                \
      if constexpr (kStack) row_ += (size_t)F.layer * gridDim.x;                               \
      g_timeline[row_ * kStamps + (slot)] = __builtin_amdgcn_s_memrealtime();                  \
    }                                                                                          \
  } while (0)
#else
#define QMOE_STAMP(slot) \
  do {                   \
  } while (0)
#endif

__device__ __forceinline__ uint32_t ld_agent_u(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_u(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// threadIdx.x as a value the compiler must take as new where this is called: in the
// stacked decode's layer loop, values derived from the thread index are then computed in
// each layer instead of hoisted out of the loop and held (spilled) across it
template <bool kOpaque>
__device__ __forceinline__ int thread_index() {
  int t = threadIdx.x;
  if constexpr (kOpaque) asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ void put_tag(uint64_t* p, uint32_t payload, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_tag(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread of the workgroup calls this. Polls the n tagged words at addr(i)
// (thread t takes i = t + 256 j, j < N; words with skip(i) are not read) until all
// carry `tag`, then hands each payload to use(i, payload). The loads of one round
// are in flight together; a round reloads only the words not yet in. after_first()
// runs once the first round's loads are issued, before their results are waited
// for (stores issued there are not waited for by this poll).
// on_first_in(): if kWatch, runs once, after the first round in which some word came in.
template <int N, bool kWatch = false, typename Addr, typename Use, typename Skip, typename Hook, typename Hook2>
__device__ __forceinline__ void poll_tagged(Addr addr, int n, uint32_t tag, Use use, Skip skip, Hook after_first,
                                            Hook2 on_first_in) {
  const int tid = threadIdx.x;
  uint32_t todo = 0, pay[N];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    pay[j] = 0;
    if (tid + 256 * j < n && !skip(tid + 256 * j)) todo |= 1u << j;
  }
  const uint32_t want = todo;
  bool watching = kWatch;
  for (int it = 0;; ++it) {
    uint64_t v[N];
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = ((todo >> j) & 1u) ? get_tag(addr(tid + 256 * j)) : 0ull;
    if (it == 0) after_first();
#pragma unroll
    for (int j = 0; j < N; ++j)
      if (((todo >> j) & 1u) && (uint32_t)(v[j] >> 32) == tag) {
        pay[j] = (uint32_t)v[j];
        todo &= ~(1u << j);
      }
    if (kWatch && watching && __syncthreads_or(todo != want)) {
      on_first_in();
      watching = false;
    }
    if (!__syncthreads_or(todo != 0u)) break;
    if (it >= kSpinLimit) {
      if (tid == 0) flag_device_error(4u);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
#pragma unroll
  for (int j = 0; j < N; ++j)
    if ((want >> j) & 1u) use(tid + 256 * j, pay[j]);
}
template <int N, typename Addr, typename Use, typename Skip, typename Hook>
__device__ __forceinline__ void poll_tagged(Addr addr, int n, uint32_t tag, Use use, Skip skip, Hook after_first) {
  poll_tagged<N, false>(addr, n, tag, use, skip, after_first, [] {});
}
template <int N, typename Addr, typename Use>
__device__ __forceinline__ void poll_tagged(Addr addr, int n, uint32_t tag, Use use) {
  poll_tagged<N, false>(addr, n, tag, use, [](int) { return false; }, [] {}, [] {});
}

__device__ __forceinline__ uint32_t read_epoch(const FusedArgs& F) {
  return ld_agent_u(&F.sync[(blockIdx.x % kEpochCopies) * kSyncLine]);
}
// Thread 0: this workgroup has read the epoch (the inline asm makes the increment wait
// for the value read). No result is returned, so nothing waits for the atomic itself.
template <bool kStack>
__device__ __forceinline__ void arrive_epoch(const FusedArgs& F, uint32_t epoch) {
  if (kStack && !F.arrive) return;  // a later layer of a stacked decode: arrived with the first
  uint32_t one = 1u;
  asm volatile("" : "+v"(one) : "v"(epoch));
  __hip_atomic_fetch_add(&F.sync[(kEpochCopies + blockIdx.x % kArrivalCounters) * kSyncLine], one,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The last workgroup of the grid: waits for the arrivals of all others (blocks
// b < gridDim.x - 1 arrive at counter b % kArrivalCounters), then clears the counters
// and writes epoch + adv into every copy (adv = the tags the launch used: one per layer).
__device__ __forceinline__ void epoch_keeper(const FusedArgs& F, uint32_t epoch, uint32_t adv = 1u) {
  const int tid = threadIdx.x;
  const int n = (int)gridDim.x - 1;
  if (tid < kArrivalCounters) {
    const uint32_t expect = n > tid ? (uint32_t)((n - 1 - tid) / kArrivalCounters + 1) : 0u;
    const uint32_t* c = &F.sync[(kEpochCopies + tid) * kSyncLine];
    for (int it = 0; ld_agent_u(c) < expect; ++it) {
      if (it > kSpinLimit) {
        flag_device_error(4u);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
  __syncthreads();
  if (tid < kArrivalCounters) st_agent_u(&F.sync[(kEpochCopies + tid) * kSyncLine], 0u);
  if (tid < kEpochCopies) st_agent_u(&F.sync[tid * kSyncLine], epoch + adv);
}

// A later layer of a stacked decode: waits until the previous layer's combines have all
// begun to hand over this layer's input. One wave polls one word per combine (the first
// pair of its rows, in this block's copy), so that the many workgroups that wait through
// the previous layer's tail poll d / 64 words each, not the whole input or their own
// (later) inputs. Ends with a barrier.
__device__ __forceinline__ void wait_x_in(const FusedArgs& F, uint32_t tag) {
  const int tid = threadIdx.x;
  const uint64_t* xs = F.x_tag + (size_t)(blockIdx.x % kXCopies) * kXStride;
  if (tid < 64) {
    for (int it = 0;; ++it) {
      bool in = true;
      for (int j = tid; j < F.d / 64; j += 64) in &= (uint32_t)(get_tag(xs + 32 * j) >> 32) == tag;
      if (__all(in)) break;
      if (it >= kSpinLimit) {
        if (tid == 0) flag_device_error(4u);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// x into LDS. kRaw (router): bf16 x as stored pairs, fp32 x as values. Otherwise
// (gate/up): bf16 pairs, or for fp32 x hi pairs at xb[0, d/2) and lo pairs at
// xb[kFusedXWords/2, ...) with hi + lo the fp32 value to 16 significant bits;
// then xg = sums over the 32-column halves of each group. Ends with a barrier.
template <typename XT, bool kRaw, bool kStack>
__device__ __forceinline__ void stage_x(const XT* __restrict__ x, const FusedArgs& F, uint32_t tag, FusedSmem& S) {
  const int tid = threadIdx.x, d = F.d;
  if (kStack && sizeof(XT) == 2 && F.x_in) {
    // a later layer of a stacked decode: the previous layer's combines hand over the input
    // as tagged bf16 pairs (this block's copy)
    const uint64_t* xs = F.x_tag + (size_t)(blockIdx.x % kXCopies) * kXStride;
    wait_x_in(F, tag);
    poll_tagged<kFusedXWords / 2 / 256>([&](int i) { return xs + i; }, d / 2, tag,
                                        [&](int i, uint32_t p) { S.xb[i] = p; });
  } else if constexpr (sizeof(XT) == 2 || kRaw) {
    for (int i = tid; i < d * (int)sizeof(XT) / 16; i += 256)
      *reinterpret_cast<uint4*>(&S.xb[4 * i]) = ldg16(reinterpret_cast<const uint8_t*>(x) + 16 * i);
  } else {
    for (int i = tid; i < d / 4; i += 256) {
      const float4 v = *reinterpret_cast<const float4*>(x + 4 * i);
      const float xv[4] = {v.x, v.y, v.z, v.w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        hi[c] = f32_to_bf16_bits(xv[c]);
        lo[c] = f32_to_bf16_bits(xv[c] - bf16_to_f32((uint16_t)hi[c]));
      }
      S.xb[2 * i] = hi[0] | (hi[1] << 16);
      S.xb[2 * i + 1] = hi[2] | (hi[3] << 16);
      S.xb[kFusedXWords / 2 + 2 * i] = lo[0] | (lo[1] << 16);
      S.xb[kFusedXWords / 2 + 2 * i + 1] = lo[2] | (lo[3] << 16);
    }
  }
  __syncthreads();
  if constexpr (!kRaw) {
    if (tid < 2 * (d / kGroup)) {
      float sum = 0.0f;
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const uint32_t w = S.xb[16 * tid + p];
        sum += bf16_lo(w) + bf16_hi(w);
        if constexpr (sizeof(XT) == 4) {
          const uint32_t l = S.xb[kFusedXWords / 2 + 16 * tid + p];
          sum += bf16_lo(l) + bf16_hi(l);
        }
      }
      S.xg[tid] = sum;
    }
    __syncthreads();
  }
}

// The fp64 logits of this block's copy into S.lg and their order keys into S.key
// (every thread calls this; ends with a barrier).
__device__ __forceinline__ void load_logits(const FusedArgs& F, uint32_t tag, FusedSmem& S) {
  const int tid = threadIdx.x, E = F.E;
  const uint64_t* lg = F.lg_tag + (size_t)(blockIdx.x % kLgCopies) * kLgStride;
  poll_tagged<2>([&](int i) { return lg + i; }, 2 * E, tag, [&](int i, uint32_t p) { S.lgw[i] = p; });
  __syncthreads();
  if (tid < E) {
    const double v = __hiloint2double((int)S.lgw[2 * tid + 1], (int)S.lgw[2 * tid]);
    S.lg[tid] = v;
    S.key[tid] = order_key(v);
  }
  __syncthreads();
}

// Ranks the experts from the ranking keys the router items publish (this block's copy):
// S.sel_e[0, top_k) = the picks in rank order (logit desc, id asc; NaN as -inf). A key
// is a 31-bit value in one word: the top 31 - b bits of the order key above b bits of
// (E - 1 - id), b = 7 for E <= 128, else 8, so keys are unique and ties go to the lower
// id; a block reads one word per expert instead of the two of an fp64 logit. As keys
// are below 2^31, a key beats another when their difference is negative: a subtraction
// and a shift, independent of each other and summed in four chains. That is the true order wherever the truncated parts
// differ; when two neighbours among ranks 0..top_k share theirs, the logits are read
// in full and the ranking is redone on the whole keys (rank_topk). Ends with a barrier.
template <bool kStack>
__device__ __forceinline__ void rank_logits(const FusedArgs& F, uint32_t tag, FusedSmem& S) {
  const int tid = threadIdx.x, E = F.E, k = F.top_k;
  const uint64_t* lk = F.lg_tag + (size_t)(blockIdx.x % kLgCopies) * kLgStride + kLgKeys;
  poll_tagged<1>([&](int i) { return lk + i; }, E, tag, [&](int i, uint32_t p) { S.kp[i] = p; });
  __syncthreads();
  QMOE_STAMP(1);  // routed gate/up, down, combine: every key word held
  const int idbits = E <= 128 ? 7 : 8;
  // thread t: expert t % E against the competitors of share t / E (256 / E shares of
  // 64, 64 or 16 keys, all of a 32-key run read before the first comparison)
  const int lgE = E == 64 ? 6 : E == 128 ? 7 : 8;
  const int parts = 256 >> lgE, h = tid >> lgE, me = tid & (E - 1);
  const int mine = (int)S.kp[me];
  int r4[4] = {0, 0, 0, 0};
  auto count = [&](auto nc, int c0) __attribute__((always_inline)) {
    constexpr int N = decltype(nc)::value;
    u32x4_t kk[N / 4];
#pragma unroll
    for (int i = 0; i < N / 4; ++i) kk[i] = *reinterpret_cast<const u32x4_t*>(&S.kp[c0 + 4 * i]);
#pragma unroll
    for (int i = 0; i < N / 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) r4[c] += (int)((uint32_t)(mine - (int)kk[i][c]) >> 31);
  };
  if (parts == 4) {
    count(ic<16>{}, 16 * h);
  } else {
    for (int c0 = h * (E / parts); c0 < (h + 1) * (E / parts); c0 += 32) count(ic<32>{}, c0);
  }
  S.rank[h][me] = (r4[0] + r4[1]) + (r4[2] + r4[3]);
  __syncthreads();
  if (tid < E) {
    int rk = 0;
    for (int j = 0; j < parts; ++j) rk += S.rank[j][tid];
    if (rk <= k) S.sel_e[rk] = tid;  // ranks 0..top_k (sel_e holds 17)
  }
  __syncthreads();
  const bool clash = tid < min(k, E - 1) && (S.kp[S.sel_e[tid]] >> idbits) == (S.kp[S.sel_e[tid + 1]] >> idbits);
  if (__syncthreads_or(clash)) {
    load_logits(F, tag, S);
    rank_topk(S.key, E, k, S.rank, S.sel_e);
  }
  QMOE_STAMP(2);  // routed gate/up, down, combine: picks ranked
}

// The blob of the expert picked for `slot` (nullptr and the error flag if its table
// entry is outside the pool). slot_entry: thread t < E holds slot_table[t].
template <bool kStack>
__device__ __forceinline__ const uint8_t* routed_blob(const FusedArgs& F, int slot, uint32_t tag,
                                                      uint32_t slot_entry, FusedSmem& S) {
  if (threadIdx.x < F.E) S.slots[threadIdx.x] = slot_entry;
  rank_logits<kStack>(F, tag, S);
  const uint32_t b = S.slots[S.sel_e[slot]];  // ranks are a permutation: sel_e is a valid id
  if ((uint64_t)b >= F.n_blobs) {
    if (threadIdx.x == 0) flag_device_error(1u);
    return nullptr;
  }
  return F.pool + (uint64_t)b * F.stride;
}

// ------------------------------------------------------------------ router item

template <typename XT>
__device__ __forceinline__ float x_at(const FusedSmem& S, int col) {
  if constexpr (sizeof(XT) == 2) return bf16_to_f32((uint16_t)(S.xb[col >> 1] >> (16 * (col & 1))));
  else return __uint_as_float(S.xb[col]);
}

// experts [2 item, +2): thread t takes row (t & 1), column quarter (t >> 1) & 3 and the
// groups (t >> 3) + 32 j; products w * x are exact in fp64 (w = s q + b has at most
// 20 significant bits, x at most 24) and the sums are fp64.
template <typename XT, bool kStack>
__device__ __forceinline__ void fused_router(const FusedArgs& F, const XT* __restrict__ x, int item, uint32_t tag,
                                             uint32_t epoch, FusedSmem& S) {
  const int tid = thread_index<kStack>();
  const int G = F.d / kGroup;
  const int e0 = item * kFusedRouterE, nb = e0 / 64, row = e0 % 64 + (tid & 1);
  const int c = (tid >> 1) & 3, gs = tid >> 3;
  constexpr int J = kFusedMaxG / 32 + 1;
  u32x4_t q[J];
  uint32_t sb[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int g = min(gs + 32 * j, G - 1);
    const uint8_t* t = F.router_blob + ((uint64_t)nb * G + g) * kTile8;
    q[j] = *reinterpret_cast<const u32x4_t*>(t + c * 1024 + row * 16);
    sb[j] = ldg4(t + kTile8Codes + row * 4);
  }
  if (tid == 0) arrive_epoch<kStack>(F, epoch);  // before the first wait, which covers it
  stage_x<XT, true, kStack>(x, F, tag, S);
  QMOE_STAMP(1);  // router: weights and x in
  double acc = 0.0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int g = gs + 32 * j;
    if (g < G) {
      const double s = (double)bf16_lo(sb[j]), b = (double)bf16_hi(sb[j]);
      const int col = g * kGroup + 16 * c;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const double w = fma(s, (double)((q[j][m >> 2] >> (8 * (m & 3))) & 0xffu), b);
        acc = fma(w, (double)x_at<XT>(S, col + m), acc);
      }
    }
  }
  S.rd[tid] = acc;
  __syncthreads();
  // the 128 partials of expert e (entries of parity e) in two levels: 16 threads per
  // expert add 8 each, then one thread adds those 16
  if (tid < 32) {
    double a = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) a += S.rd[tid + 32 * i];
    S.rd2[tid] = a;
  }
  __syncthreads();
  if (tid < kFusedRouterE) {
    double l = 0.0;
#pragma unroll
    for (int k = 0; k < 16; ++k) l += S.rd2[tid + 2 * k];
    if (F.offset) l += (double)F.offset[e0 + tid];
    S.lgv[tid] = l;
  }
  __syncthreads();
  // into every copy: the 2 words of each logit, then each expert's ranking key
  const int idbits = F.E <= 128 ? 7 : 8;
  constexpr int kWords = 3 * kFusedRouterE;
  for (int i = tid; i < kWords * kLgCopies; i += 256) {
    const int wd = i % kWords, copy = i / kWords;
    uint64_t* dst = F.lg_tag + (size_t)copy * kLgStride;
    if (wd < 2 * kFusedRouterE) {
      const uint64_t bits = (uint64_t)__double_as_longlong(S.lgv[wd >> 1]);
      put_tag(dst + 2 * e0 + wd, (uint32_t)(bits >> (32 * (wd & 1))), tag);
    } else {
      const int j = wd - 2 * kFusedRouterE, e = e0 + j;
      const uint64_t key = order_key(S.lgv[j]);
      put_tag(dst + kLgKeys + e, ((uint32_t)(key >> (33 + idbits)) << idbits) | (uint32_t)(F.E - 1 - e), tag);
    }
  }
  QMOE_STAMP(2);  // router: logits and keys published
}

// ------------------------------------------------------------------ gate/up item

// sum over 32 columns of one row: codes q (4 words, see common.h) against 16 x pairs
// (and 16 lo pairs for fp32 x)
template <bool kLo>
__device__ __forceinline__ float half_dot(const u32x4_t& q, const uint32_t* xp, const uint32_t* xl) {
  u32x4_t xv[4], lv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xv[i] = *reinterpret_cast<const u32x4_t*>(xp + 4 * i);
    if constexpr (kLo) lv[i] = *reinterpret_cast<const u32x4_t*>(xl + 4 * i);
  }
  float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const NibK nk;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t p = nk.pair(q[jj], t);
      a4[t] = dot2(p, xv[jj][t], a4[t]);
      if constexpr (kLo) a4[t] = dot2(p, lv[jj][t], a4[t]);
    }
  return (a4[0] + a4[1]) + (a4[2] + a4[3]);
}

// Rows [16 q4, +16) of 64-row block nb of the gate and up matrices, whole reduction.
// Lane l of wave w: group pair (w + 4 i), group 2 (w + 4 i) + (l >> 5), column half
// (l >> 4) & 1, row l & 15: each wavefront load is 4 runs of 256 contiguous bytes.
template <typename XT, bool kStack>
__device__ __forceinline__ void fused_gateup(const FusedArgs& F, const XT* __restrict__ x, int u, bool routed,
                                             uint32_t tag, uint32_t epoch, FusedSmem& S) {
  const int tid = thread_index<kStack>(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = F.d / kGroup;
  int slot = F.top_k, Fd = F.fs;
  if (routed) {
    const int per = F.f / kFusedRows;
    slot = u / per;
    u -= slot * per;
    Fd = F.f;
  }
  const int nb = u >> 2, q4 = u & 3;
  const int tp = lane >> 5, half = (lane >> 4) & 1, row = q4 * kFusedRows + (lane & 15);
  u32x4_t q[2][kFusedGuI];
  uint32_t sb[2][kFusedGuI];
  auto load = [&](const uint8_t* blob) {
    const uint64_t mbytes = m4_bytes(Fd, F.d);
#pragma unroll
    for (int i = 0; i < kFusedGuI; ++i)
#pragma unroll
      for (int mat = 0; mat < 2; ++mat) {
        const int g = min(2 * (wave + 4 * i) + tp, G - 1);
        const uint8_t* t = blob + mat * mbytes + ((uint64_t)nb * G + g) * kTile4;
        q[mat][i] = *reinterpret_cast<const u32x4_t*>(t + half * 1024 + row * 16);
        sb[mat][i] = ldg4(t + kTile4Codes + row * 4);
      }
  };
  // the shared expert's weights stream from the start; a routed expert's once it is known
  const uint8_t* blob = F.shared_blob;
  if (!routed) {
    // the shared expert's weights start streaming once the router items have published
    // their keys: the router's own loads, which head the chain, then meet an idle
    // memory system instead of the shared expert's 10 MB. In a later layer of a stacked
    // decode they stream at once instead, while the previous layer finishes (its tail
    // leaves the memory system idle).
    if (!(kStack && F.x_in)) {
      const uint64_t* lk = F.lg_tag + (size_t)(blockIdx.x % kLgCopies) * kLgStride + kLgKeys;
      poll_tagged<1>([&](int i) { return lk + i; }, F.E, tag, [&](int i, uint32_t p) { S.kp[i] = p; });
    }
    QMOE_STAMP(1);  // shared gate/up: the router has published
    load(blob);
    if (tid == 0) arrive_epoch<kStack>(F, epoch);
  }
  const uint32_t slot_entry = (routed && tid < F.E) ? F.slot_table[tid] : 0u;
  stage_x<XT, false, kStack>(x, F, tag, S);
  if (routed) {
    // the arrival goes after the weight loads: no wait on the ticket's path covers it
    blob = routed_blob<kStack>(F, slot, tag, slot_entry, S);
    if (blob) load(blob);
    if (tid == 0) arrive_epoch<kStack>(F, epoch);
  }
  float acc[2] = {0.0f, 0.0f};
  if (blob) {
#pragma unroll
    for (int i = 0; i < kFusedGuI; ++i) {
      const int g = 2 * (wave + 4 * i) + tp;
      if (2 * (wave + 4 * i) < G) {  // wave-uniform; lanes of a missing odd group add nothing
        const int gc = min(g, G - 1);
        const uint32_t* xp = S.xb + gc * 32 + half * 16;
        const float xs = S.xg[2 * gc + half];
#pragma unroll
        for (int mat = 0; mat < 2; ++mat) {
          const float a = half_dot<sizeof(XT) == 4>(q[mat][i], xp, xp + kFusedXWords / 2);
          const float s = bf16_lo(sb[mat][i]), b = bf16_hi(sb[mat][i]);
          const float v = fmaf(s, a, fmaf(-128.0f, s, b) * xs);
          acc[mat] += g < G ? v : 0.0f;
        }
      }
    }
  }
  QMOE_STAMP(3);  // gate/up: dot products done
  S.red[0][wave][lane] = acc[0];
  S.red[1][wave][lane] = acc[1];
  __syncthreads();
  // the thread that stores copy c of row r adds that row's gate and up partials itself
  // (the same order in every copy), so no further barrier stands before the stores
  if (tid < kFusedRows * kHCopies) {
    const int r = tid % kFusedRows, copy = tid / kFusedRows;
    float v[2] = {0.0f, 0.0f};
#pragma unroll
    for (int mat = 0; mat < 2; ++mat)
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) v[mat] += S.red[mat][w][r + 16 * k4];
    put_tag(&F.h_tag[copy * F.h_stride + (size_t)slot * F.fmax + nb * 64 + q4 * kFusedRows + r],
            __float_as_uint(gelu_tanh(v[0]) * v[1]), tag);
  }
  QMOE_STAMP(4);  // gate/up: h stored
}

// ------------------------------------------------------------------ down item (+ combine)

// group sum of one row against h in LDS as 32 fp16 pairs (hh points at the group's
// pair 0; h scaled by the item's power of two), read in two batches of 16 pairs (one
// LDS wait each). The codes enter as fp16 pairs (1024 + q, 1024 + q'), one shift and
// one v_and_or_b32 each, and 1024 goes into the bias: s * sum (1024 + q) h + (b - 1024 s) V.
__device__ __forceinline__ float group_dot_lds(const uint32_t* hh, uint4 qa, uint4 qb, uint32_t sbw, float Vg) {
  const uint32_t words[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
  float acc4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const NibKT<0x64006400u> nk;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint4 h4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h4[i] = *reinterpret_cast<const uint4*>(hh + 16 * half + 4 * i);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t w = words[4 * half + jj];
      const uint32_t hv[4] = {h4[jj].x, h4[jj].y, h4[jj].z, h4[jj].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t p = nk.pair(w, t);
        acc4[t] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, p), __builtin_bit_cast(f16x2_t, hv[t]), acc4[t],
                                         false);
      }
    }
  }
  const float a = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
  const float s = bf16_lo(sbw), b = bf16_hi(sbw);
  return fmaf(s, a, fmaf(-1024.0f, s, b) * Vg);
}

// weights of one 64-row block for groups g0 + wave + 4i (i < GW) of [g0, g1), loaded ahead of use
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
  // against h in LDS: fp16 pairs of group g at hh + g * 32, group sums at gs[g]
  __device__ __forceinline__ float dot_lds(int g0, int g1, int wave, const uint32_t* hh, const float* gs) const {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int g = g0 + wave + 4 * i;
      if (g < g1) acc += group_dot_lds(hh + g * 32, qa[i], qb[i], sb[i], gs[g]);
    }
    return acc;
  }
};

// Values [j0, j1) of one slot's h (j0, j1 multiples of 64, j1 - j0 <= 256 kGatherPer)
// from their tagged words into LDS at the same positions as fp16 of h * sc, with sc the
// power of two that brings their largest |h| into [2^14, 2^15) (the prefill's H
// scaling), and the per-group sums of those fp16 values in S.hsum. Returns sc.
// on_first_in() (kWatch) runs once, as soon as the first values are in.
constexpr int kGatherPer = 5;
template <bool kWatch = false, typename Hook = void (*)()>
__device__ __forceinline__ float gather_h(const uint64_t* src, int j0, int j1, uint32_t tag, FusedSmem& S,
                                          Hook on_first_in = nullptr) {
  float* hf = reinterpret_cast<float*>(S.xb);
  for (int base = j0; base < j1; base += 1024)
    poll_tagged<4, kWatch>(
        [&](int i) { return src + base + i; }, min(1024, j1 - base), tag,
        [&](int i, uint32_t p) { hf[base + i] = __uint_as_float(p); }, [](int) { return false; }, [] {},
        [&] {
          if constexpr (kWatch) on_first_in();
        });
  __syncthreads();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // thread t holds values j0 + t + 256 k: wave w, value k is group j0/64 + 4 k + w
  float v[kGatherPer];
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < kGatherPer; ++k) {
    const int j = j0 + tid + 256 * k;
    v[k] = j < j1 ? hf[j] : 0.0f;
    m = fmaxf(m, fabsf(v[k]));  // a NaN is skipped, as fmaxf does
  }
  m = wave_fmax(m);
  if (lane == 0) S.hmax[wave] = m;
  __syncthreads();  // also: every fp32 value is read before the fp16 writes below
  const float sc = row_scale(fmaxf(fmaxf(S.hmax[0], S.hmax[1]), fmaxf(S.hmax[2], S.hmax[3])));
  uint16_t* hh = reinterpret_cast<uint16_t*>(S.xb);
#pragma unroll
  for (int k = 0; k < kGatherPer; ++k) {
    const int j = j0 + tid + 256 * k;
    if (j0 + 256 * k + 64 * wave < j1) {  // wave-uniform: j1 - j0 is a multiple of 64
      const _Float16 hv = (_Float16)(v[k] * sc);
      hh[j] = __builtin_bit_cast(uint16_t, hv);
      const float gsum = wave_sum((float)hv);
      if (lane == 0) S.hsum[j / kGroup] = gsum;
    }
  }
  __syncthreads();
  return sc;
}

// exp as a call: inlined into the layer loop of the stacked decode, its constants are
// hoisted out of the loop and held (spilled) across it
__device__ __attribute__((noinline)) double exp_call(double v) { return exp(v); }

// The picks and their softmax weights into S.sel_e, S.selw (fp64 softmax over the
// picked logits, fixed summation order).
template <bool kStack>
__device__ __forceinline__ void pick_weights(const FusedArgs& F, uint32_t tag, FusedSmem& S) {
  const int tid = thread_index<kStack>(), lane = tid & 63, k = F.top_k;
  rank_logits<kStack>(F, tag, S);
  load_logits(F, tag, S);  // the picked logits for the weights (long published by now)
  if (tid < 64) {
    double ex = 0.0;
    if (lane < k) {
      const double v = S.lg[S.sel_e[lane]] - S.lg[S.sel_e[0]];
      ex = kStack ? exp_call(v) : exp(v);
    }
    double sum = 0.0;
    for (int t = 0; t < k; ++t) sum += __shfl(ex, t, 64);
    if (lane < k) S.selw[lane] = (float)(ex / sum);
  }
}

// y for rows [64 ob, +64) once the picks are known (pick_weights): r (wave 0) is the
// shared expert's first half for the row; adds its second half, then the routed
// outputs weighted by the softmax over the picks, in pick order. old (wave 0): the
// residual's bf16 value for the row (when there is a residual).
template <bool kStack>
__device__ __forceinline__ void fused_combine(const FusedArgs& F, int ob, float r, uint16_t old, uint32_t tag,
                                              FusedSmem& S) {
  const int tid = thread_index<kStack>(), lane = tid & 63, k = F.top_k;
  poll_tagged<5>([&](int i) { return F.eo_tag + (size_t)(i >> 6) * F.d + ob * 64 + (i & 63); }, 64 * (k + 1), tag,
                 [&](int i, uint32_t p) { S.eo[i >> 6][i & 63] = __uint_as_float(p); });
  __syncthreads();
  QMOE_STAMP(6);  // combine: every expert output in
  if (tid < 64) {
    float yv = r + S.eo[k][lane];
    for (int s = 0; s < k; ++s) yv = fmaf(S.selw[s], S.eo[s][lane], yv);
    const int n = ob * 64 + lane;
    if (F.y) F.y[n] = yv;
    if (F.residual) {
      const uint32_t nv = f32_to_bf16_bits(bf16_to_f32(old) + yv);
      F.residual[n] = (uint16_t)nv;
      if (kStack && F.x_rec) F.x_rec[n] = old;
      if (kStack && F.x_out) {
        // the next layer's input as tagged pairs: lanes 2j and 2j + 1 hold the pair, each
        // writes half of the copies
        // both shuffles run in every lane (a shuffle reads lanes that take part in it)
        const uint32_t up = (uint32_t)__shfl_down((int)nv, 1, 64);
        const uint32_t dn = (uint32_t)__shfl_up((int)nv, 1, 64);
        const uint32_t pair = (lane & 1) ? (dn | (nv << 16)) : (nv | (up << 16));
#pragma unroll
        for (int c = lane & 1; c < kXCopies; c += 2)
          put_tag(&F.x_tag[(size_t)c * kXStride + (n >> 1)], pair, tag + 1u);
      }
    }
    if (ob == 0 && lane < k) {
      F.idx_out[lane] = S.sel_e[lane];
      F.w_out[lane] = S.selw[lane];
    }
  }
}

// Output rows [64 ob, +64) of the down matrix of `slot`, over groups [g0, g1) of its h.
// kind 0: routed slot u / (d/64) over its whole h -> expert_out and its tagged copy;
// kind 1: the shared expert's second half -> tagged partial; kind 2: the shared
// expert's first half, then the combine of the rows. The weights stream as soon as
// the expert is known, while h is still being produced.
template <int GW, bool kStack>
__device__ __forceinline__ void fused_down(const FusedArgs& F, int u, int kind, uint32_t tag, uint32_t epoch,
                                           FusedSmem& S) {
  const int tid = thread_index<kStack>(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NBd = F.d / 64;
  int slot = F.top_k, ob = u, Fd = F.fs;
  if (kind == 0) {
    slot = u / NBd;
    ob = u % NBd;
    Fd = F.f;
  }
  const int Gin = Fd / kGroup, Gh = (Gin + 1) / 2;
  const int g0 = kind == 1 ? Gh : 0, g1 = kind == 2 ? Gh : Gin;
  const uint32_t slot_entry = (kind == 0 && tid < F.E) ? F.slot_table[tid] : 0u;
  // the combine's residual rows, read now so that the read is not on the tail of the chain
  // (in a stacked decode this thread wrote them itself in the previous layer)
  const uint16_t old = (kind == 2 && F.residual && tid < 64) ? F.residual[ob * 64 + lane] : (uint16_t)0;
  // a later layer of a stacked decode: the waits for the keys and for h start once this
  // layer's input is in (they would otherwise poll through the previous layer's tail)
  if (kStack && kind == 0 && F.x_in) wait_x_in(F, tag);
  const uint8_t* blob = kind == 0 ? routed_blob<kStack>(F, slot, tag, slot_entry, S) : F.shared_blob;
  RowLoads<GW> w;
  const uint8_t* rowblock = blob ? blob + 2 * m4_bytes(Fd, F.d) + (uint64_t)ob * Gin * kTile4 : nullptr;
  const uint64_t* hsrc = F.h_tag + (blockIdx.x % kHCopies) * F.h_stride + (size_t)slot * F.fmax;
  float sc = 1.0f;
  if (kind == 0) {
    // a routed expert's down weights wait until its h starts to come in, so that they do
    // not take memory bandwidth from the gate/up loads h depends on; they arrive while
    // the rest of h is produced
    if (tid == 0) arrive_epoch<kStack>(F, epoch);
    sc = gather_h<true>(hsrc, g0 * kGroup, g1 * kGroup, tag, S, [&] {
      QMOE_STAMP(3);  // routed down: the first values of h in
      if (rowblock) w.load(rowblock, g0, g1, wave, lane);
    });
  } else {
    // in a stacked decode the combine ranks the picks before its weights stream: the
    // ranking's registers and the weights' then need not be held at once (the layer
    // loop leaves too few for both), and both are done long before the shared h is in
    const bool late = kStack && kind == 2;
    if (rowblock && !late) w.load(rowblock, g0, g1, wave, lane);
    if (tid == 0) arrive_epoch<kStack>(F, epoch);
    if (kStack && F.x_in) wait_x_in(F, tag);
    if (kind == 2) pick_weights<kStack>(F, tag, S);  // the logits are out long before the shared h
    if (rowblock && late) w.load(rowblock, g0, g1, wave, lane);
    sc = gather_h(hsrc, g0 * kGroup, g1 * kGroup, tag, S);
  }
  QMOE_STAMP(4);  // down, combine: all of h in
  const float acc = rowblock ? w.dot_lds(g0, g1, wave, S.xb, S.hsum) : 0.0f;
  const float r = reduce_waves4(acc, S.red[0], wave, lane) * (1.0f / sc);  // exact: sc is a power of two
  QMOE_STAMP(5);  // down, combine: dot products done
  if (kind == 2) {
    fused_combine<kStack>(F, ob, r, old, tag, S);
  } else if (wave == 0) {
    const int n = ob * 64 + lane;
    if (kind == 0 && F.expert_out) F.expert_out[(size_t)slot * F.d + n] = r;
    put_tag(&F.eo_tag[(size_t)slot * F.d + n], __float_as_uint(r), tag);
  }
  QMOE_STAMP(7);  // down: outputs stored; combine: y stored
}

// ------------------------------------------------------------------ the kernel

// Work item of block b is item b: the router items, which head the dependency chain,
// take the lowest blocks, so they are dispatched first and spread over all eight XCDs
// (blocks are dealt to the XCDs round robin). Any placement is correct (all blocks are
// resident at once); packing the router items onto two XCDs measured 0.66 us slower.
// the work item of this block for one layer
template <typename XT>
__device__ __forceinline__ void fused_item(const FusedArgs& F, const XT* __restrict__ x, uint32_t tag, uint32_t epoch,
                                           FusedSmem& S) {
  int b = blockIdx.x;
  if (b < F.n_rt) {
    fused_router<XT, false>(F, x, b, tag, epoch, S);
  } else if ((b -= F.n_rt) < F.n_sg + F.n_rg) {
    const bool routed = b >= F.n_sg;
    fused_gateup<XT, false>(F, x, routed ? b - F.n_sg : b, routed, tag, epoch, S);
  } else if ((b -= F.n_sg + F.n_rg) < F.n_rd) {
    fused_down<kFusedRoutedGW, false>(F, b, 0, tag, epoch, S);
  } else {
    b -= F.n_rd;
    fused_down<kFusedSharedGW, false>(F, b < F.n_sd ? b : b - F.n_sd, b < F.n_sd ? 1 : 2, tag, epoch, S);
  }
}

template <typename XT>
__global__ __launch_bounds__(256, 4) void k_decode_fused(FusedArgs F, const XT* __restrict__ x) {
  __shared__ FusedSmem S;
  constexpr bool kStack = false;
  QMOE_STAMP(0);  // every item: started
  const uint32_t epoch = read_epoch(F);
  if (blockIdx.x == gridDim.x - 1) return epoch_keeper(F, epoch);
  fused_item(F, x, epoch + 1u, epoch, S);
}

// ------------------------------------------------------------------ stacked decode

// One layer of a stack: its weights (every layer may have its own pool and table).
struct StackLayer {
  const uint8_t* pool;
  const uint32_t* slot_table;
  const uint8_t* router_blob;
  const uint8_t* shared_blob;
  const float* offset;  // [E] or null
  uint64_t stride, n_blobs;
};

struct StackArgs {
  FusedArgs F;  // the shape, the workspace words and the outputs of layer 0
  int n_layers;
  StackLayer layer[kMaxStackLayers];
};

// One decode row through n_layers blocks in ONE launch, x <- bf16(x + y) after each.
// Every workgroup keeps its work item from layer to layer, so an item starts the next
// layer as soon as it is done with this one: routing-independent weights (the router's,
// the shared expert's gate/up and down) stream while the previous layer finishes, and
// only the wait for the next layer's input remains. The combines hand the next input
// over as tagged bf16 pairs (kXCopies copies); layer l tags its words epoch + 1 + l and
// the keeper advances the epoch by n_layers. Every hand-off region is reused from layer
// to layer: a layer's words are written only after the next input is complete, which
// every reader of the previous layer's words precedes.
// a uniform pointer the compiler must treat as new in every layer: addresses derived
// from the workspace pointers are then computed where they are used instead of hoisted
// out of the layer loop and held in registers across it (which spills)
template <typename T>
__device__ __forceinline__ T* per_layer(T* p) {
#if __HIP_DEVICE_COMPILE__
  // laundered as a global pointer, so that accesses through it stay global (not flat)
  __attribute__((address_space(1))) T* g = (__attribute__((address_space(1))) T*)p;
  asm volatile("" : "+s"(g));
  return (T*)g;
#else
  return p;
#endif
}

__device__ __forceinline__ int per_layer_i(int v) {
  asm volatile("" : "+s"(v));
  return v;
}

// The arguments of layer l of a stacked decode, read through a pointer to the kernel's
// argument block (StackArgs is the kernel's first argument, so at offset 0 of the
// kernarg segment) that the compiler must treat as new in every layer: they are then
// loaded (scalar loads) in each layer instead of held in registers across the loop.
#if __HIP_DEVICE_COMPILE__
typedef const __attribute__((address_space(4))) StackArgs KernargStackArgs;
#else
typedef const StackArgs KernargStackArgs;
#endif
__device__ __forceinline__ FusedArgs stack_layer_args(int l) {
  KernargStackArgs* Ap = (KernargStackArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(Ap));
  KernargStackArgs& A = *Ap;
  const auto& L = A.layer[l];
  const int k = A.F.top_k, d = A.F.d;
  FusedArgs F = A.F;
  F.lg_tag = per_layer(F.lg_tag);
  F.h_tag = per_layer(F.h_tag);
  F.eo_tag = per_layer(F.eo_tag);
  F.x_tag = per_layer(F.x_tag);
  F.sync = per_layer(F.sync);
  F.pool = L.pool;
  F.slot_table = L.slot_table;
  F.router_blob = L.router_blob;
  F.shared_blob = L.shared_blob;
  F.offset = L.offset;
  F.stride = L.stride;
  F.n_blobs = L.n_blobs;
  F.arrive = l == 0;
  F.x_in = l > 0;
  F.x_out = l + 1 < A.n_layers;
  F.idx_out = A.F.idx_out + (size_t)l * k;
  F.w_out = A.F.w_out + (size_t)l * k;
  F.expert_out = A.F.expert_out ? A.F.expert_out + (size_t)l * k * d : nullptr;
  F.y = A.F.y ? A.F.y + (size_t)l * d : nullptr;
  F.x_rec = A.F.x_rec ? A.F.x_rec + (size_t)l * d : nullptr;
  F.layer = l;
  F.d = per_layer_i(F.d);
  F.f = per_layer_i(F.f);
  F.fs = per_layer_i(F.fs);
  F.E = per_layer_i(F.E);
  F.top_k = per_layer_i(F.top_k);
  F.fmax = per_layer_i(F.fmax);
  F.n_rt = per_layer_i(F.n_rt);
  F.n_sg = per_layer_i(F.n_sg);
  F.n_rg = per_layer_i(F.n_rg);
  F.n_rd = per_layer_i(F.n_rd);
  F.n_sd = per_layer_i(F.n_sd);
  return F;
}

template <typename XT>
__global__ __launch_bounds__(256, 4) void k_stack_decode(StackArgs A, const XT* __restrict__ x) {
  __shared__ FusedSmem S;
  const uint32_t epoch = read_epoch(A.F);
  if (blockIdx.x == gridDim.x - 1) return epoch_keeper(A.F, epoch, (uint32_t)A.n_layers);
  // one loop per item kind, so that a loop holds only its own kind's code
  auto layers = [&](auto item) __attribute__((always_inline)) {
    for (int l = 0; l < A.n_layers; ++l) {
      const FusedArgs F = stack_layer_args(l);
      constexpr bool kStack = true;
      QMOE_STAMP(0);  // every item: started (the layer)
      item(F, epoch + 1u + (uint32_t)l);
      __syncthreads();  // the next layer's item reuses the LDS
    }
  };
  const FusedArgs& F0 = A.F;
  int b = blockIdx.x;
  if (b < F0.n_rt) {
    layers([&](const FusedArgs& F, uint32_t tag) { fused_router<XT, true>(F, x, b, tag, epoch, S); });
  } else if ((b -= F0.n_rt) < F0.n_sg) {
    layers([&](const FusedArgs& F, uint32_t tag) { fused_gateup<XT, true>(F, x, b, false, tag, epoch, S); });
  } else if ((b -= F0.n_sg) < F0.n_rg) {
    layers([&](const FusedArgs& F, uint32_t tag) { fused_gateup<XT, true>(F, x, b, true, tag, epoch, S); });
  } else if ((b -= F0.n_rg) < F0.n_rd) {
    layers([&](const FusedArgs& F, uint32_t tag) { fused_down<kFusedRoutedGW, true>(F, b, 0, tag, epoch, S); });
  } else if ((b -= F0.n_rd) < F0.n_sd) {
    layers([&](const FusedArgs& F, uint32_t tag) { fused_down<kFusedSharedGW, true>(F, b, 1, tag, epoch, S); });
  } else {
    b -= F0.n_sd;
    layers([&](const FusedArgs& F, uint32_t tag) { fused_down<kFusedSharedGW, true>(F, b, 2, tag, epoch, S); });
  }
}

}  // namespace qmoe
