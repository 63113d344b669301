// C ABI of the quantized MoE FFN block (see include/moe.h): argument checks,
// workspace carve-up and kernel launches on the caller's stream. The whole
// device library is this one translation unit.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "cache_device.h"
#include "common.h"
#include "decode_fused.h"
#include "decode_kernels.h"
#include "moe.h"
#include "group_kernels.h"
#include "prefill_gemm.h"
#include "router_kernels.h"

using namespace qmoe;

// ------------------------------------------------------------------ expert cache, device policy

namespace qmoe {

namespace {
inline size_t cache_align(size_t v) { return (v + 255) & ~(size_t)255; }
}  // namespace

uint64_t cache_dev_state_bytes(int L, int E, int S) {
  size_t o = 0;
  o = cache_align(o + sizeof(uint32_t) * (size_t)L * E);          // freq
  o = cache_align(o + sizeof(int32_t) * (size_t)L * S);           // expert_in
  o = cache_align(o + sizeof(uint64_t) * (size_t)L * S);          // last_use
  o = cache_align(o + sizeof(uint64_t) * (size_t)L);              // clock
  o = cache_align(o + sizeof(uint32_t) * (1 + 2 * kCacheMaxPicks));  // miss list
  o = cache_align(o + sizeof(uint64_t) * 3);                      // stats
  return o;
}

CacheDevState cache_dev_state(void* base, uint32_t* tables, int L, int E, int S, uint64_t stride) {
  CacheDevState st;
  uint8_t* b = static_cast<uint8_t*>(base);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    uint8_t* p = b + o;
    o = cache_align(o + bytes);
    return p;
  };
  st.tables = tables;
  st.freq = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)L * E));
  st.expert_in = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)L * S));
  st.last_use = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * (size_t)L * S));
  st.clock = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * (size_t)L));
  st.miss = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (1 + 2 * kCacheMaxPicks)));
  st.stats = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * 3));
  st.L = L;
  st.E = E;
  st.S = S;
  st.stride = stride;
  return st;
}

__global__ __launch_bounds__(256) void k_cache_init(CacheDevState st) {
  const size_t LE = (size_t)st.L * st.E, LS = (size_t)st.L * st.S;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < LE + LS; i += (size_t)gridDim.x * 256) {
    if (i < LE) {
      st.tables[i] = (uint32_t)st.S;
      st.freq[i] = 0u;
    } else {
      st.expert_in[i - LE] = -1;
      st.last_use[i - LE] = 0u;
    }
  }
  if (blockIdx.x == 0) {
    for (int l = threadIdx.x; l < st.L; l += 256) st.clock[l] = 0u;
    if (threadIdx.x < 1 + 2 * kCacheMaxPicks) st.miss[threadIdx.x] = 0u;
    if (threadIdx.x < 3) st.stats[threadIdx.x] = 0u;
  }
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t w = ((uint64_t)(uint32_t)__shfl_xor((int)(v >> 32), o, 64) << 32) |
                       (uint32_t)__shfl_xor((int)(uint32_t)v, o, 64);
    v = min(v, w);
  }
  return v;
}

// The policy for one request, in request order (the host policy's rule). The layer's
// state is staged in LDS by the whole workgroup; one wave applies the requests, each
// lane holding slots lane, lane + 64, ... for the searches (the lowest never-used slot;
// else the smallest (frequency, last use, id) among the slots whose expert the request
// does not name, as three wave minima); lane 0 makes the updates; then the state goes
// back. E, S <= 256.
__global__ __launch_bounds__(256) void k_cache_plan(CacheDevState st, int layer, const int32_t* __restrict__ picks,
                                                    int n) {
  __shared__ uint32_t tab[256], fq[256];
  __shared__ int32_t ein[256];
  __shared__ uint64_t lu[256];
  __shared__ int32_t req[kCacheMaxPicks];
  const int E = st.E, S = st.S, t = threadIdx.x;
  uint32_t* table = st.tables + (size_t)layer * E;
  uint32_t* freq = st.freq + (size_t)layer * E;
  int32_t* expert_in = st.expert_in + (size_t)layer * S;
  uint64_t* last_use = st.last_use + (size_t)layer * S;
  for (int i = t; i < E; i += 256) {
    tab[i] = table[i];
    fq[i] = freq[i];
  }
  for (int i = t; i < S; i += 256) {
    ein[i] = expert_in[i];
    lu[i] = last_use[i];
  }
  if (t < n) req[t] = picks[t];
  __syncthreads();
  if (t < 64) {
    const int lane = t;
    const uint64_t now = st.clock[layer] + 1;
    uint32_t named[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int rq[kCacheMaxPicks];
    int m = 0;
    for (int i = 0; i < n; ++i) {
      const int e = req[i];
      if (e < 0 || e >= E) {  // not from the router; nothing to make resident for it
        if (lane == 0) flag_device_error(2u);
        continue;
      }
      rq[m++] = e;
      if (!((named[e >> 5] >> (e & 31)) & 1u) && lane == 0) fq[e] += 1u;
      named[e >> 5] |= 1u << (e & 31);
    }
    uint32_t misses = 0, hits = 0;
    for (int i = 0; i < m; ++i) {
      const int e = rq[i];
      int s = (int)tab[e];
      if (s < S) {
        ++hits;
      } else {
        uint32_t free_j = 0xffffffffu;
        for (int j = lane; j < S; j += 64)
          if (ein[j] < 0) free_j = min(free_j, (uint32_t)j);
        free_j = wave_min_u32(free_j);
        if (free_j != 0xffffffffu) {
          s = (int)free_j;
        } else {
          // every slot is in use: the victim among the experts the request does not name
          uint32_t f = 0xffffffffu;
          for (int j = lane; j < S; j += 64) {
            const int v = ein[j];
            if (!((named[v >> 5] >> (v & 31)) & 1u)) f = min(f, fq[v]);
          }
          f = wave_min_u32(f);
          uint64_t u = ~0ull;
          for (int j = lane; j < S; j += 64) {
            const int v = ein[j];
            if (!((named[v >> 5] >> (v & 31)) & 1u) && fq[v] == f) u = min(u, lu[j]);
          }
          u = wave_min_u64(u);
          uint32_t id = 0xffffffffu;
          for (int j = lane; j < S; j += 64) {
            const int v = ein[j];
            if (!((named[v >> 5] >> (v & 31)) & 1u) && fq[v] == f && lu[j] == u) id = min(id, (uint32_t)v);
          }
          id = wave_min_u32(id);
          if (id == 0xffffffffu) {  // unreachable while n <= S (checked on the host)
            if (lane == 0) flag_device_error(1u);
            continue;
          }
          s = (int)tab[id];
        }
        if (lane == 0) {
          if (ein[s] >= 0) tab[ein[s]] = (uint32_t)S;
          ein[s] = e;
          tab[e] = (uint32_t)s;
          st.miss[1 + 2 * misses] = (uint32_t)e;
          st.miss[2 + 2 * misses] = (uint32_t)s;
        }
        ++misses;
      }
      if (lane == 0) lu[s] = now;
    }
    if (lane == 0) {
      st.clock[layer] = now;
      st.miss[0] = misses;
      st.stats[0] += hits;
      st.stats[1] += misses;
      st.stats[2] += (uint64_t)misses * st.stride;
    }
  }
  __syncthreads();
  for (int i = t; i < E; i += 256) {
    table[i] = tab[i];
    freq[i] = fq[i];
  }
  for (int i = t; i < S; i += 256) {
    expert_in[i] = ein[i];
    last_use[i] = lu[i];
  }
}

// Workgroup b copies part b % kCacheCopyBlocks of miss b / kCacheCopyBlocks (16-byte
// words, four loads in flight per thread); workgroups past the plan's misses return.
__global__ __launch_bounds__(256) void k_cache_fill(CacheDevState st, int layer, const uint8_t* host_pool_dev,
                                                    uint8_t* dev_slots) {
  const uint32_t i = blockIdx.x / kCacheCopyBlocks, part = blockIdx.x % kCacheCopyBlocks;
  if (i >= st.miss[0]) return;
  const uint32_t e = st.miss[1 + 2 * i], s = st.miss[2 + 2 * i];
  const uint4* src = reinterpret_cast<const uint4*>(host_pool_dev + ((size_t)layer * st.E + e) * st.stride);
  uint4* dst = reinterpret_cast<uint4*>(dev_slots + ((size_t)layer * st.S + s) * st.stride);
  const uint64_t words = st.stride / 16, step = (uint64_t)kCacheCopyBlocks * 256;
  uint64_t j = (uint64_t)part * 256 + threadIdx.x;
  for (; j + 3 * step < words; j += 4 * step) {
    const uint4 v0 = src[j], v1 = src[j + step], v2 = src[j + 2 * step], v3 = src[j + 3 * step];
    dst[j] = v0;
    dst[j + step] = v1;
    dst[j + 2 * step] = v2;
    dst[j + 3 * step] = v3;
  }
  for (; j < words; j += step) dst[j] = src[j];
}

bool launch_cache_init(const CacheDevState& st, hipStream_t stream) {
  const size_t n = (size_t)st.L * st.E + (size_t)st.L * st.S;
  const int grid = (int)std::min<size_t>(1024, std::max<size_t>(1, (n + 255) / 256));
  k_cache_init<<<grid, 256, 0, stream>>>(st);
  return hipGetLastError() == hipSuccess;
}

bool launch_cache_plan(const CacheDevState& st, int layer, const int32_t* picks, int n, hipStream_t stream) {
  if (n < 1 || n > kCacheMaxPicks || n > st.S) return false;
  if (st.E > 256 || st.S > 256) return false;
  k_cache_plan<<<1, 256, 0, stream>>>(st, layer, picks, n);
  return hipGetLastError() == hipSuccess;
}

bool launch_cache_fill(const CacheDevState& st, int layer, const uint8_t* host_pool_dev, uint8_t* dev_slots,
                       int n_max, hipStream_t stream) {
  if (n_max < 1 || n_max > kCacheMaxPicks || st.stride % 16) return false;
  k_cache_fill<<<n_max * kCacheCopyBlocks, 256, 0, stream>>>(st, layer, host_pool_dev, dev_slots);
  return hipGetLastError() == hipSuccess;
}

}  // namespace qmoe

// Decode workspace of moe_layer_decode_noalloc (see "static scratch" below).
constexpr size_t kStaticScratchBytes = 5u << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
constexpr int kDecodeGW = 3;      // groups per wavefront per load batch in the decode GEMVs
constexpr int kGroupsPerPart = 12;  // reduction groups per decode workgroup

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
inline int cdiv(int a, int b) { return (a + b - 1) / b; }

bool shape_ok(const moe_shape* s) {
  if (!s) return false;
  if (s->group != 64) return false;
  if (s->d_model <= 0 || s->d_ff <= 0 || s->d_ff_shared <= 0) return false;
  if (s->d_model % 64 || s->d_ff % 64 || s->d_ff_shared % 64) return false;
  // reduction parts of the decode GEMVs: at most 8 of 12 groups each
  if (s->d_model > 8 * kGroupsPerPart * 64 || s->d_ff_shared > 8 * kGroupsPerPart * 64) return false;
  // the rankers split the 256 threads of a workgroup evenly over the experts: 64, 128 or 256
  if (s->n_experts != 64 && s->n_experts != 128 && s->n_experts != 256) return false;
  if (s->top_k < 1 || s->top_k > 16 || s->top_k > s->n_experts) return false;
  return true;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static_assert(kSlotSkip == MOE_SLOT_SKIP, "the kernels' skip entry is the one moe.h names");


struct DecodeCfg {
  int P, Ps, fmax, nbmax;
};
DecodeCfg decode_cfg(const moe_shape* s) {
  DecodeCfg c;
  c.P = cdiv(s->d_model / 64, kGroupsPerPart);
  c.Ps = cdiv(s->d_ff_shared / 64, kGroupsPerPart);
  c.fmax = std::max(s->d_ff, s->d_ff_shared);
  c.nbmax = c.fmax / 64;
  return c;
}

// words between the copies of the fused decode's h: one copy rounded up to 4 KiB, plus
// 4 KiB so the copies start on different channels
size_t fused_h_stride(const moe_shape* s) {
  const size_t words = (size_t)(s->top_k + 1) * std::max(s->d_ff, s->d_ff_shared);
  return (words + 511) / 512 * 512 + 512;
}

// Workspace layout. The counters come first in a region whose size depends on
// the shape only (zeroed once, left at zero by every call), so layouts for
// different row counts never place a counter where another call kept data.
struct Ws {
  size_t gu_count, dn_count, fused_sync, fused_lg, fused_h, fused_eo, fused_x, router_partial, gu_partial, h_hi,
      h_lo, h_gsum,
      shared_part, pf_shared_out, pf_hbs, pf_Hh, pf_xg, st_eo, st_y, total;
};
Ws ws_layout(const moe_shape* s, int rows) {
  const DecodeCfg dc = decode_cfg(s);
  const int k = s->top_k, d = s->d_model;
  const size_t R = (size_t)std::max(rows, 1);
  Ws w;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  w.gu_count = take(sizeof(uint32_t) * (k + 1) * dc.nbmax);
  w.dn_count = take(sizeof(uint32_t) * (d / 64));
  w.fused_sync = take(sizeof(uint32_t) * kFusedSyncWords);
  // tagged hand-off words of the fused decode: in the prefix whose layout depends on
  // the shape only, so no other call ever writes there (a stray tag would read as ready)
  w.fused_lg = take(sizeof(uint64_t) * kLgCopies * kLgStride);
  w.fused_h = take(sizeof(uint64_t) * kHCopies * fused_h_stride(s));
  w.fused_eo = take(sizeof(uint64_t) * (size_t)(k + 1) * d);
  w.fused_x = take(sizeof(uint64_t) * kXCopies * kXStride);
  w.router_partial = take(sizeof(double) * kRouterSplits * R * s->n_experts);
  w.gu_partial = take(sizeof(float) * (size_t)(k + 1) * 2 * dc.nbmax * dc.P * 64);
  w.h_hi = take(sizeof(uint16_t) * (size_t)(k + 1) * dc.fmax);
  w.h_lo = take(sizeof(uint16_t) * (size_t)(k + 1) * dc.fmax);
  w.h_gsum = take(sizeof(float) * (size_t)(k + 1) * dc.nbmax);
  w.shared_part = take(sizeof(float) * (size_t)dc.Ps * d);
  w.pf_shared_out = take(sizeof(float) * kSharedDownParts * R * d);
  w.pf_hbs = take(sizeof(float) * R * ((size_t)k * (s->d_ff / 64) + s->d_ff_shared / 64));
  w.pf_Hh = take(sizeof(uint16_t) * R * ((size_t)k * s->d_ff + s->d_ff_shared));
  w.pf_xg = take(sizeof(float) * R * ((d / 64 + 3) & ~3));  // rows padded to a multiple of 4 groups
  // the stacked decode's per-layer outputs the caller does not keep (layer-by-layer path)
  w.st_eo = take(sizeof(float) * (size_t)k * d);
  w.st_y = take(sizeof(float) * (size_t)d);
  w.total = o;
  return w;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<uint8_t*>(ws) + off);
}

moe_status check_layer(const moe_shape* s, const moe_layer* L, bool need_pool, bool need_router, bool need_shared) {
  if (!L) return MOE_ERR_INVALID_ARG;
  if (need_pool) {
    if (!L->pool || !L->slot_table || !aligned16(L->pool)) return MOE_ERR_INVALID_ARG;
    if (L->blob_stride < moe_expert_blob_bytes(s) || L->blob_stride % 256 || L->n_blobs == 0)
      return MOE_ERR_INVALID_ARG;
  }
  if (need_router && (!L->router_blob || !aligned16(L->router_blob))) return MOE_ERR_INVALID_ARG;
  if (need_shared && (!L->shared_blob || !aligned16(L->shared_blob))) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status check_common(const moe_shape* s, const void* x, moe_dtype dt, int rows, void* ws, size_t ws_bytes) {
  if (!shape_ok(s)) return s ? MOE_ERR_UNSUPPORTED_SHAPE : MOE_ERR_INVALID_ARG;
  if (rows < 0) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!x || !aligned16(x))) return MOE_ERR_INVALID_ARG;
  if ((int64_t)rows * s->top_k >= 65536) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (rows > 0) {
    if (!ws || ((uintptr_t)ws & 255u)) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < ws_layout(s, rows).total) return MOE_ERR_WORKSPACE;
  }
  return MOE_OK;
}

moe_status launched() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// ------------------------------------------------------------------ launches

template <typename XT>
void launch_router(const moe_shape* s, const moe_layer* L, const XT* x, int rows, const float* off, int32_t* idx,
                   float* w, double* logits, void* ws, const Ws& W, hipStream_t st, float* xg = nullptr) {
  double* part = at<double>(ws, W.router_partial);
  const int blocks = cdiv(rows, 16) * (s->n_experts / 16) * kRouterSplits;
  k_router_logits<XT><<<blocks, 256, 0, st>>>(L->router_blob, x, rows, s->d_model, s->n_experts, part, xg);
  k_router_select<<<rows, 256, 0, st>>>(part, rows, s->n_experts, s->top_k, off, idx, w, logits);
}

DecodeArgs decode_args(const moe_shape* s, const moe_layer* L, const int32_t* idx, void* ws, const Ws& W,
                       float* expert_out, const float* topk_w, float* y, uint16_t* residual) {
  const DecodeCfg dc = decode_cfg(s);
  DecodeArgs A;
  memset(&A, 0, sizeof A);
  if (L) {  // null for the combine alone
    A.pool = L->pool;
    A.stride = L->blob_stride;
    A.n_blobs = L->n_blobs;
    A.slot_table = L->slot_table;
    A.shared_blob = L->shared_blob;
  }
  A.topk_idx = idx;
  A.d = s->d_model;
  A.f = s->d_ff;
  A.fs = s->d_ff_shared;
  A.top_k = s->top_k;
  A.n_experts = s->n_experts;
  A.P = dc.P;
  A.Ps = dc.Ps;
  A.fmax = dc.fmax;
  A.nbmax = dc.nbmax;
  A.gu_partial = at<float>(ws, W.gu_partial);
  A.gu_count = at<uint32_t>(ws, W.gu_count);
  A.h_hi = at<uint16_t>(ws, W.h_hi);
  A.h_lo = at<uint16_t>(ws, W.h_lo);
  A.h_gsum = at<float>(ws, W.h_gsum);
  A.expert_out = expert_out;
  A.shared_part = at<float>(ws, W.shared_part);
  A.dn_count = at<uint32_t>(ws, W.dn_count);
  A.topk_w = topk_w;
  A.y = y;
  A.residual = residual;
  return A;
}

// gate/up (+GeGLU) for the routed slots and/or the shared expert
template <typename XT>
void launch_decode_gateup(DecodeArgs A, const XT* x, bool routed, bool shared, hipStream_t st) {
  A.routed_units = routed ? A.top_k * 2 * (A.f / 64) * A.P : 0;
  const int shared_units = shared ? 2 * (A.fs / 64) * A.P : 0;
  k_decode_gateup<XT, kDecodeGW><<<A.routed_units + shared_units, 256, 0, st>>>(A, x);
}

void launch_decode_down(DecodeArgs A, bool routed, bool shared, bool combine, hipStream_t st) {
  A.routed_units = routed ? A.top_k * (A.d / 64) : 0;
  const int shared_units = shared ? (A.d / 64) * A.Ps : 0;
  A.combine_arrivals = combine ? (shared ? A.Ps : 0) + (routed ? A.top_k : 0) : 0;
  k_decode_down<kDecodeGW><<<A.routed_units + shared_units, 256, 0, st>>>(A);
}

// Workgroups of the fused decode kernel the device can hold at once (per device, cached).
template <typename XT>
int fused_capacity() {
  static int cap[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cap[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode_fused<XT>, 256, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cap[dev] = std::max(1, per_cu * cus);
  }
  return cap[dev];
}

// whether the whole-block decode kernel's tiling takes the shape (see decode_fused.h)
bool fused_shape_ok(const moe_shape* s, bool f32_x) {
  const int d = s->d_model, f = s->d_ff, fs = s->d_ff_shared;
  if (d / 64 > kFusedMaxG || f > 64 * 4 * kFusedRoutedGW || fs > 2 * 64 * 4 * kFusedSharedGW) return false;
  return !(f32_x && d > kFusedXWords);
}

// arguments of the whole-block decode kernel for one layer (the grid is
// n_rt + n_sg + n_rg + n_rd + 2 n_sd + 1 workgroups)
FusedArgs fused_args(const moe_shape* s, const moe_layer* L, const float* off, int32_t* idx, float* w,
                     float* expert_out, float* y, uint16_t* residual, void* ws, const Ws& W) {
  const int d = s->d_model, f = s->d_ff, fs = s->d_ff_shared;
  FusedArgs F;
  memset(&F, 0, sizeof F);
  F.pool = L->pool;
  F.stride = L->blob_stride;
  F.n_blobs = L->n_blobs;
  F.slot_table = L->slot_table;
  F.router_blob = L->router_blob;
  F.shared_blob = L->shared_blob;
  F.offset = off;
  F.d = d;
  F.f = f;
  F.fs = fs;
  F.E = s->n_experts;
  F.top_k = s->top_k;
  F.fmax = std::max(f, fs);
  F.idx_out = idx;
  F.w_out = w;
  F.expert_out = expert_out;
  F.y = y;
  F.residual = residual;
  F.lg_tag = at<uint64_t>(ws, W.fused_lg);
  F.h_tag = at<uint64_t>(ws, W.fused_h);
  F.h_stride = fused_h_stride(s);
  F.eo_tag = at<uint64_t>(ws, W.fused_eo);
  F.sync = at<uint32_t>(ws, W.fused_sync);
  F.n_rt = s->n_experts / kFusedRouterE;
  F.n_sg = fs / kFusedRows;
  F.n_rg = s->top_k * (f / kFusedRows);
  F.n_rd = s->top_k * (d / 64);
  F.n_sd = d / 64;
  F.x_tag = at<uint64_t>(ws, W.fused_x);
  F.arrive = 1;
  return F;
}

int fused_grid(const FusedArgs& F) { return F.n_rt + F.n_sg + F.n_rg + F.n_rd + 2 * F.n_sd + 1; }  // + the keeper

// One persistent launch for the whole decode row, when the grid fits on the chip;
// returns false (nothing launched) otherwise.
template <typename XT>
bool launch_decode_fused(const moe_shape* s, const moe_layer* L, const XT* x, const float* off, int32_t* idx,
                         float* w, float* expert_out, float* y, uint16_t* residual, void* ws, const Ws& W,
                         hipStream_t st) {
  if (!fused_shape_ok(s, sizeof(XT) == 4)) return false;
  const FusedArgs F = fused_args(s, L, off, idx, w, expert_out, y, residual, ws, W);
  const int grid = fused_grid(F);
  if (grid > fused_capacity<XT>()) return false;
  k_decode_fused<XT><<<grid, 256, 0, st>>>(F, x);
  return true;
}

PrefillArgs prefill_args(const moe_shape* s, const moe_layer* L, int rows, const int32_t* offset, const int32_t* perm,
                         float* expert_out, void* ws) {
  const Ws W = ws_layout(s, rows);
  PrefillArgs A;
  memset(&A, 0, sizeof A);
  A.pool = L->pool;
  A.stride = L->blob_stride;
  A.n_blobs = L->n_blobs;
  A.slot_table = L->slot_table;
  A.shared_blob = L->shared_blob;
  A.offset = offset;
  A.perm = perm;
  A.d = s->d_model;
  A.f = s->d_ff;
  A.fs = s->d_ff_shared;
  A.n_experts = s->n_experts;
  A.top_k = s->top_k;
  A.rows = rows;
  const int P = rows * s->top_k;
  A.routed_mtiles = cdiv(P, 64) + std::min(s->n_experts, P);
  A.shared_mtiles = cdiv(rows, 64);
  A.expert_out = expert_out;
  A.shared_out = at<float>(ws, W.pf_shared_out);
  A.hbs = at<float>(ws, W.pf_hbs);
  A.Hh = at<uint16_t>(ws, W.pf_Hh);
  A.xg = at<float>(ws, W.pf_xg);
  return A;
}

// workgroups of `kernel` (256 threads, static LDS only) the device runs at once
template <typename K>
int resident_blocks(K kernel, int* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev] = std::max(1, per_cu * cus);
  }
  return cache[dev];
}

// The stacked decode in one launch, when the shape fits the fused kernel's tiling and
// the grid fits on the chip; returns false (nothing launched) otherwise.
bool launch_stack_decode(const moe_shape* s, const moe_layer* layers, int n_layers, uint16_t* x,
                         const float* const* offsets, int32_t* idx, float* w, float* expert_out, float* y,
                         uint16_t* x_layers, void* ws, const Ws& W, hipStream_t st) {
  static int cap[64];
  if (n_layers > kMaxStackLayers || !fused_shape_ok(s, false)) return false;
  StackArgs A;
  memset(&A, 0, sizeof A);
  A.F = fused_args(s, &layers[0], nullptr, idx, w, expert_out, y, x, ws, W);
  A.F.x_rec = x_layers;
  A.n_layers = n_layers;
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer& L = layers[l];
    A.layer[l] = StackLayer{L.pool, L.slot_table, L.router_blob, L.shared_blob, offsets ? offsets[l] : nullptr,
                            L.blob_stride, L.n_blobs};
  }
  const int grid = fused_grid(A.F);
  if (grid > resident_blocks(k_stack_decode<uint16_t>, cap)) return false;
  k_stack_decode<uint16_t><<<grid, 256, 0, st>>>(A, x);
  return true;
}

// grid of a persistent GEMM launch: what the chip holds at once (a multiple of the
// XCD count, so work item i always runs on XCD i % 8), at most the work items
int persistent_grid(int resident, int items) {
  int g = std::min(resident, items);
  if (g > kXcds) g -= g % kXcds;
  return std::max(g, 1);
}

// one gate/up launch and one down launch covering the routed
// tiles and/or the shared expert's tiles; with group_sums, first the activations'
// group sums (when the router kernel has not left them)
template <typename XT>
void launch_prefill(PrefillArgs A, const XT* x, bool routed, bool shared, bool group_sums, hipStream_t st) {
  static int cap_gu[64], cap_dn[64];
  if (!routed) A.routed_mtiles = 0;
  if (!shared) A.shared_mtiles = 0;
  if (group_sums)
    k_group_sums<XT><<<cdiv(A.rows, 16) * kRouterSplits, 256, 0, st>>>(x, A.rows, A.d, const_cast<float*>(A.xg));
  // items at most (routed tile count bounded by the pair count plus one per expert)
  const int gu_items = xcd_blocks(A.routed_mtiles, A.f / 64) + xcd_blocks(A.shared_mtiles, A.fs / 64);
  if (gu_items == 0) return;
  k_prefill_gateup<XT><<<persistent_grid(resident_blocks(k_prefill_gateup<XT>, cap_gu), gu_items), 256, 0, st>>>(A, x);
  const int dnc = (A.d / 64 + kDownBlocks - 1) / kDownBlocks;
  // (the shared expert's down runs in kSharedDownParts K parts per row tile)
  const int dn_items = xcd_blocks(A.routed_mtiles, dnc) + xcd_blocks(A.shared_mtiles * kSharedDownParts, dnc);
  k_prefill_down<<<persistent_grid(resident_blocks(k_prefill_down, cap_dn), dn_items), 256, 0, st>>>(A);
}

// The whole block for one decode row with the workspace at `ws` laid out as W: one
// launch when the grid fits the device at once, else three.
void layer_decode(const moe_shape* s, const moe_layer* L, const void* x, moe_dtype dt, const float* off, int32_t* idx,
                  float* w, float* expert_out, float* y, uint16_t* residual, void* ws, const Ws& W, hipStream_t hs) {
  const bool fused =
      dt == MOE_BF16 ? launch_decode_fused(s, L, (const uint16_t*)x, off, idx, w, expert_out, y, residual, ws, W, hs)
                     : launch_decode_fused(s, L, (const float*)x, off, idx, w, expert_out, y, residual, ws, W, hs);
  if (fused) return;
  // the grid does not fit on the device at once: three launches instead
  DecodeArgs A = decode_args(s, L, idx, ws, W, expert_out, w, y, residual);
  if (dt == MOE_BF16) {
    launch_router(s, L, (const uint16_t*)x, 1, off, idx, w, nullptr, ws, W, hs);
    launch_decode_gateup(A, (const uint16_t*)x, true, true, hs);
  } else {
    launch_router(s, L, (const float*)x, 1, off, idx, w, nullptr, ws, W, hs);
    launch_decode_gateup(A, (const float*)x, true, true, hs);
  }
  launch_decode_down(A, true, true, true, hs);
}

// ------------------------------------------------------------------ static scratch (moe_layer_decode_noalloc)

// The decode workspace of moe_layer_decode_noalloc, in the library's own device memory.
// Its layout is the one of the largest shape that entry point takes, so every region
// sits at the same offset for every shape: the counters (zero between calls) and the
// call counter of the fused decode keep their places, tagged hand-off words of any
// earlier call carry older tags, and scratch regions of one shape never overlap the
// tagged regions of another. Host code never passes `scratch` itself to a kernel: it
// passes the address hipGetSymbolAddress returns for the current device.
const moe_shape kStaticMaxShape = {3072, 768, 2560, 256, 16, 64};

const Ws& static_layout() {
  static const Ws W = ws_layout(&kStaticMaxShape, 1);
  return W;
}

bool static_shape_ok(const moe_shape* s) {
  return s->d_model <= kStaticMaxShape.d_model && s->d_ff <= kStaticMaxShape.d_ff &&
         s->d_ff_shared <= kStaticMaxShape.d_ff_shared && s->n_experts <= kStaticMaxShape.n_experts &&
         s->top_k <= kStaticMaxShape.top_k && static_layout().total <= kStaticScratchBytes;
}

__global__ __launch_bounds__(256) void k_zero16(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct ScratchState {
  void* ptr;     // device address of `scratch` on this device
  bool cleared;  // a clear has been enqueued outside graph capture
};
std::mutex g_scratch_mu;
ScratchState g_scratch[kMaxDevices];

// The current device's scratch address (looked up once per device, with that device
// current). The first call on a device enqueues a clear on `st`; so does every call
// made under graph capture until one outside capture has cleared it (a captured clear
// runs only when the graph is replayed). A clear covers the whole scratch, so a graph
// holding one starts every replay from a clean state.
moe_status static_scratch(hipStream_t st, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchState& S = g_scratch[dev];
  if (!S.ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    S.ptr = p;
  }
  if (!S.cleared) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cap) != hipSuccess) return MOE_ERR_HIP;
    k_zero16<<<256, 256, 0, st>>>((uint4*)S.ptr, kStaticScratchBytes / 16);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    if (cap == hipStreamCaptureStatusNone) S.cleared = true;
  }
  *out = S.ptr;
  return MOE_OK;
}

// After a fused-decode wait gave up, the current device's scratch is cleared again
// before its next use.
void static_scratch_invalidate() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  g_scratch[dev].cleared = false;
}

}  // namespace

extern "C" {

uint64_t moe_expert_blob_bytes(const moe_shape* s) {
  if (!shape_ok(s)) return 0;
  return 2 * moe_matrix4_bytes(s->d_ff, s->d_model) + moe_matrix4_bytes(s->d_model, s->d_ff);
}
uint64_t moe_shared_blob_bytes(const moe_shape* s) {
  if (!shape_ok(s)) return 0;
  return 2 * moe_matrix4_bytes(s->d_ff_shared, s->d_model) + moe_matrix4_bytes(s->d_model, s->d_ff_shared);
}
uint64_t moe_router_blob_bytes(const moe_shape* s) {
  if (!shape_ok(s)) return 0;
  return moe_matrix8_bytes(s->n_experts, s->d_model);
}

size_t moe_workspace_bytes(const moe_shape* s, int32_t rows) {
  if (!shape_ok(s) || rows < 0) return 0;
  return ws_layout(s, rows).total;
}

moe_status moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return MOE_ERR_INVALID_ARG;
  return hipMemsetAsync(ws, 0, ws_bytes, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_router_topk(const moe_shape* s, const moe_layer* L, const void* x, moe_dtype dt, int32_t rows,
                           const float* off, int32_t* idx, float* w, double* logits, void* ws, size_t ws_bytes,
                           void* stream) {
  moe_status st = check_common(s, x, dt, rows, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if ((st = check_layer(s, L, false, true, false)) != MOE_OK) return st;
  if (rows == 0) return MOE_OK;
  if (!idx || !w) return MOE_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  const Ws W = ws_layout(s, rows);
  if (dt == MOE_BF16)
    launch_router(s, L, (const uint16_t*)x, rows, off, idx, w, logits, ws, W, hs);
  else
    launch_router(s, L, (const float*)x, rows, off, idx, w, logits, ws, W, hs);
  return launched();
}

moe_status moe_group_by_expert(const moe_shape* s, const int32_t* idx, int32_t rows, int32_t* count,
                               int32_t* offset, int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes,
                               void* stream) {
  if (!shape_ok(s)) return s ? MOE_ERR_UNSUPPORTED_SHAPE : MOE_ERR_INVALID_ARG;
  if (rows < 0) return MOE_ERR_INVALID_ARG;
  if ((int64_t)rows * s->top_k >= 65536) return MOE_ERR_UNSUPPORTED_SHAPE;
  (void)ws;
  (void)ws_bytes;
  if (!count || !offset) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!idx || !perm || !inv_perm)) return MOE_ERR_INVALID_ARG;
  const size_t lds = sizeof(int32_t) * kGroupWaves * s->n_experts;
  k_group<<<1, 1024, lds, (hipStream_t)stream>>>(idx, rows * s->top_k, s->n_experts, count, offset, perm, inv_perm);
  return launched();
}

moe_status moe_expert_ffn_decode(const moe_shape* s, const moe_layer* L, const void* x, moe_dtype dt,
                                 const int32_t* idx, float* expert_out, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_common(s, x, dt, 1, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if ((st = check_layer(s, L, true, false, false)) != MOE_OK) return st;
  if (!idx || !expert_out) return MOE_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  DecodeArgs A = decode_args(s, L, idx, ws, ws_layout(s, 1), expert_out, nullptr, nullptr, nullptr);
  A.skip_ok = 1;
  if (dt == MOE_BF16)
    launch_decode_gateup(A, (const uint16_t*)x, true, false, hs);
  else
    launch_decode_gateup(A, (const float*)x, true, false, hs);
  launch_decode_down(A, true, false, false, hs);
  return launched();
}

moe_status moe_shared_expert_decode(const moe_shape* s, const moe_layer* L, const void* x, moe_dtype dt, void* ws,
                                    size_t ws_bytes, void* stream) {
  moe_status st = check_common(s, x, dt, 1, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if ((st = check_layer(s, L, false, false, true)) != MOE_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  DecodeArgs A = decode_args(s, L, nullptr, ws, ws_layout(s, 1), nullptr, nullptr, nullptr, nullptr);
  if (dt == MOE_BF16)
    launch_decode_gateup(A, (const uint16_t*)x, false, true, hs);
  else
    launch_decode_gateup(A, (const float*)x, false, true, hs);
  launch_decode_down(A, false, true, false, hs);  // the down parts stay in the workspace
  return launched();
}

moe_status moe_combine_decode(const moe_shape* s, const float* expert_out, const float* topk_w, float* y,
                              uint16_t* residual, void* ws, size_t ws_bytes, void* stream) {
  if (!shape_ok(s)) return s ? MOE_ERR_UNSUPPORTED_SHAPE : MOE_ERR_INVALID_ARG;
  if (!ws || ((uintptr_t)ws & 255u)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < ws_layout(s, 1).total) return MOE_ERR_WORKSPACE;
  if (!expert_out || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(expert_out) || !aligned16(y) || ((uintptr_t)residual & 7u)) return MOE_ERR_INVALID_ARG;
  DecodeArgs A = decode_args(s, nullptr, nullptr, ws, ws_layout(s, 1), const_cast<float*>(expert_out), topk_w, y,
                             residual);
  k_decode_combine<<<cdiv(s->d_model, 256), 256, 0, (hipStream_t)stream>>>(A);
  return launched();
}

moe_status moe_expert_ffn_prefill_chunk(const moe_shape* s, const moe_layer* L, const void* x, moe_dtype dt,
                                        int32_t rows, const int32_t* offset, const int32_t* perm,
                                        float* expert_out, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_common(s, x, dt, rows, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if ((st = check_layer(s, L, true, false, false)) != MOE_OK) return st;
  if (rows == 0) return MOE_OK;
  if (!offset || !perm || !expert_out) return MOE_ERR_INVALID_ARG;
  PrefillArgs A = prefill_args(s, L, rows, offset, perm, expert_out, ws);
  hipStream_t hs = (hipStream_t)stream;
  if (dt == MOE_BF16)
    launch_prefill(A, (const uint16_t*)x, true, false, true, hs);
  else
    launch_prefill(A, (const float*)x, true, false, true, hs);
  return launched();
}

moe_status moe_combine(const moe_shape* s, const moe_layer* L, const void* x, moe_dtype dt, int32_t rows,
                       const float* expert_out, const int32_t* inv_perm, const float* topk_w, float* y,
                       uint16_t* residual, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_common(s, x, dt, rows, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if ((st = check_layer(s, L, false, false, true)) != MOE_OK) return st;
  if (rows == 0) return MOE_OK;
  if (!expert_out || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(expert_out) || !aligned16(y) || ((uintptr_t)residual & 7u)) return MOE_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  if (rows == 1 && inv_perm == nullptr) {
    // decode: shared expert as GEMVs, the combine runs in the last workgroup of each output block
    DecodeArgs A = decode_args(s, L, nullptr, ws, ws_layout(s, 1), const_cast<float*>(expert_out), topk_w, y,
                               residual);
    if (dt == MOE_BF16)
      launch_decode_gateup(A, (const uint16_t*)x, false, true, hs);
    else
      launch_decode_gateup(A, (const float*)x, false, true, hs);
    launch_decode_down(A, false, true, true, hs);
    return launched();
  }
  PrefillArgs A = prefill_args(s, L, rows, nullptr, nullptr, nullptr, ws);
  if (dt == MOE_BF16)
    launch_prefill(A, (const uint16_t*)x, false, true, true, hs);
  else
    launch_prefill(A, (const float*)x, false, true, true, hs);
  k_combine<<<dim3(cdiv(s->d_model / 4, 256), rows), 256, 0, hs>>>(A.shared_out, kSharedDownParts, expert_out, inv_perm, topk_w, rows,
                                                                 s->d_model, s->top_k, y, residual);
  return launched();
}

moe_status moe_layer_decode(const moe_shape* s, const moe_layer* L, const void* x, moe_dtype dt, const float* off,
                            int32_t* idx, float* w, float* expert_out, float* y, uint16_t* residual, void* ws,
                            size_t ws_bytes, void* stream) {
  moe_status st = check_common(s, x, dt, 1, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if ((st = check_layer(s, L, true, true, true)) != MOE_OK) return st;
  if (!idx || !w || !expert_out || !y) return MOE_ERR_INVALID_ARG;
  layer_decode(s, L, x, dt, off, idx, w, expert_out, y, residual, ws, ws_layout(s, 1), (hipStream_t)stream);
  return launched();
}

moe_status moe_layer_decode_noalloc(const moe_shape* s, const moe_layer* L, const void* x, moe_dtype dt,
                                    const float* off, int32_t* idx, float* w, float* expert_out, float* y,
                                    uint16_t* residual, void* stream) {
  if (!shape_ok(s)) return s ? MOE_ERR_UNSUPPORTED_SHAPE : MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (!x || !aligned16(x)) return MOE_ERR_INVALID_ARG;
  if (!static_shape_ok(s)) return MOE_ERR_WORKSPACE;  // past what the static scratch holds
  moe_status st = check_layer(s, L, true, true, true);
  if (st != MOE_OK) return st;
  if (!idx || !w || !expert_out || !y) return MOE_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  void* scratch_ptr = nullptr;
  if ((st = static_scratch(hs, &scratch_ptr)) != MOE_OK) return st;
  layer_decode(s, L, x, dt, off, idx, w, expert_out, y, residual, scratch_ptr, static_layout(), hs);
  return launched();
}

moe_status moe_stack_decode(const moe_shape* s, const moe_layer* layers, int32_t n_layers, uint16_t* x,
                            const float* const* offsets, int32_t* idx, float* w, float* expert_out, float* y,
                            uint16_t* x_layers, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_common(s, x, MOE_BF16, 1, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (!layers || n_layers < 0) return MOE_ERR_INVALID_ARG;
  if (n_layers == 0) return MOE_OK;
  for (int l = 0; l < n_layers; ++l)
    if ((st = check_layer(s, &layers[l], true, true, true)) != MOE_OK) return st;
  if (!idx || !w) return MOE_ERR_INVALID_ARG;
  if (!aligned16(expert_out) || !aligned16(y) || !aligned16(x_layers)) return MOE_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  const Ws W = ws_layout(s, 1);
  if (launch_stack_decode(s, layers, n_layers, x, offsets, idx, w, expert_out, y, x_layers, ws, W, hs))
    return launched();
  // layer by layer (a shape or a layer count the one-launch kernel does not take)
  const int k = s->top_k, d = s->d_model;
  for (int l = 0; l < n_layers; ++l) {
    if (x_layers &&
        hipMemcpyAsync(x_layers + (size_t)l * d, x, sizeof(uint16_t) * d, hipMemcpyDeviceToDevice, hs) != hipSuccess)
      return MOE_ERR_HIP;
    float* eo = expert_out ? expert_out + (size_t)l * k * d : at<float>(ws, W.st_eo);
    float* yl = y ? y + (size_t)l * d : at<float>(ws, W.st_y);
    layer_decode(s, &layers[l], x, MOE_BF16, offsets ? offsets[l] : nullptr, idx + (size_t)l * k,
                 w + (size_t)l * k, eo, yl, x, ws, W, hs);
  }
  return launched();
}

moe_status moe_layer_prefill(const moe_shape* s, const moe_layer* L, const void* x, moe_dtype dt, int32_t rows,
                             const float* off, int32_t* idx, float* w, int32_t* count, int32_t* offset,
                             int32_t* perm, int32_t* inv_perm, float* expert_out, float* y, uint16_t* residual,
                             void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_common(s, x, dt, rows, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if ((st = check_layer(s, L, true, true, true)) != MOE_OK) return st;
  if (rows == 0) return MOE_OK;
  if (!idx || !w || !count || !offset || !perm || !inv_perm || !expert_out || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(expert_out) || !aligned16(y) || ((uintptr_t)residual & 7u)) return MOE_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  const Ws W = ws_layout(s, rows);
  float* xg = at<float>(ws, W.pf_xg);  // the router kernel leaves the group sums for gate/up
  if (dt == MOE_BF16)
    launch_router(s, L, (const uint16_t*)x, rows, off, idx, w, nullptr, ws, W, hs, xg);
  else
    launch_router(s, L, (const float*)x, rows, off, idx, w, nullptr, ws, W, hs, xg);
  const size_t lds = sizeof(int32_t) * kGroupWaves * s->n_experts;
  k_group<<<1, 1024, lds, hs>>>(idx, rows * s->top_k, s->n_experts, count, offset, perm, inv_perm);
  PrefillArgs A = prefill_args(s, L, rows, offset, perm, expert_out, ws);
  if (dt == MOE_BF16)
    launch_prefill(A, (const uint16_t*)x, true, true, false, hs);
  else
    launch_prefill(A, (const float*)x, true, true, false, hs);
  k_combine<<<dim3(cdiv(s->d_model / 4, 256), rows), 256, 0, hs>>>(A.shared_out, kSharedDownParts, expert_out, inv_perm, w, rows,
                                                                 s->d_model, s->top_k, y, residual);
  return launched();
}

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_DEVICE_CHECK: return "device error word set";
  }
  return "unknown status";
}

#ifdef QMOE_TIMELINE
// Timeline build only: device buffer of [grid][kStamps] uint64 that k_decode_fused fills
// with per-workgroup phase stamps (NULL switches the stamps off).
moe_status moe_debug_set_timeline(void* buf) {
  return hipMemcpyToSymbol(HIP_SYMBOL(g_timeline), &buf, sizeof buf, 0, hipMemcpyHostToDevice) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}
#endif

moe_status moe_check_device_error(void* stream, uint32_t* flags) {
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MOE_ERR_HIP;
  uint32_t v = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_moe_device_error), sizeof v, 0, hipMemcpyDeviceToHost) != hipSuccess)
    return MOE_ERR_HIP;
  if (flags) *flags = v;
  if (v == 0) return MOE_OK;
  if (v & MOE_DEVERR_SYNC_TIMEOUT) static_scratch_invalidate();
  const uint32_t zero = 0;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_moe_device_error), &zero, sizeof zero, 0, hipMemcpyHostToDevice) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_ERR_DEVICE_CHECK;
}

}  // extern "C"
