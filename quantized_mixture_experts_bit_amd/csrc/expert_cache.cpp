// Tiered expert residency (host side of the C ABI; no kernels).
//
// The pages keep every routed expert in the slow tier and, per layer, a 16-slot LFU
// cache of expert blobs in GPU-visible memory: for each token the router's 8 picks are
// looked up there, hits reuse the resident blob, misses are read in while the GPU runs
// the shared expert, then both paths merge (blog-mushroom article "TurboFieldfare:
// Gemma 4 26B on an 8 GB MacBook", section "Why 26B Fits in 2 GB", per-token flow;
// paperfeed digest "drumih/turbo-fieldfare", "How it works"). Here the slow tier is
// pinned host memory holding the blobs of every layer, the fast tier is `slots` HBM
// blobs per layer, and the kernels reach a resident expert through the layer's slot
// table (expert id -> slot), exactly as they reach the all-resident pool.
//
// Policy (per layer, deterministic): every request counts once toward its expert's
// frequency; a missing expert takes a never-used slot if one is left, else the slot of
// the resident expert with the smallest (frequency, last use, id) among those the
// current request does not name. Slot-table entries of experts that are not resident
// hold `slots` (outside the layer's pool), so a kernel that reached one would record a
// bad-slot error instead of reading another expert's weights.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "cache_device.h"
#include "moe.h"

struct moe_expert_cache {
  int32_t L = 0, E = 0, S = 0;
  uint64_t stride = 0;
  const uint8_t* host_pool = nullptr;  // [L][E] blobs, pinned host memory
  uint8_t* dev_slots = nullptr;        // [L][S] blobs, device memory
  uint32_t* dev_tables = nullptr;      // [L][E] device slot tables
  bool host_only = false;              // no device side: the policy alone (for tests)
  // the policy on the device instead (moe_cache_create_device): its state, and the
  // device address of the host tier the fills read
  bool device_policy = false;
  qmoe::CacheDevState dstate{};
  const uint8_t* host_pool_dev = nullptr;
  std::vector<uint32_t> freq;          // [L][E] requests so far
  std::vector<int32_t> slot_of;        // [L][E] slot or -1
  std::vector<int32_t> expert_in;      // [L][S] expert or -1
  std::vector<uint64_t> last_use;      // [L][S] request counter at the last use
  uint64_t clock = 0;
  uint32_t* table_stage = nullptr;     // [L][E] pinned host copy of the slot tables
  std::vector<hipEvent_t> staged;      // [L] the last table copy of each layer
  std::vector<bool> staged_live;
  // moe_cache_decode: the picks read back, the pass tables' staging, the stream joins
  int32_t* pick_stage = nullptr;       // [16] pinned
  uint32_t* pass_stage = nullptr;      // [L][2][E] pinned
  hipEvent_t ev_main = nullptr, ev_copy = nullptr;
  uint64_t hits = 0, misses = 0, bytes = 0;
};

namespace {

moe_status hip_ok(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

void release(moe_expert_cache* c) {
  if (!c) return;
  for (size_t l = 0; l < c->staged.size(); ++l)
    if (c->staged_live[l]) (void)hipEventDestroy(c->staged[l]);
  if (c->ev_main) (void)hipEventDestroy(c->ev_main);
  if (c->ev_copy) (void)hipEventDestroy(c->ev_copy);
  if (c->table_stage) (void)hipHostFree(c->table_stage);
  if (c->pick_stage) (void)hipHostFree(c->pick_stage);
  if (c->pass_stage) (void)hipHostFree(c->pass_stage);
  delete c;
}

}  // namespace

extern "C" {

moe_status moe_cache_create(int32_t n_layers, int32_t n_experts, int32_t slots, uint64_t blob_stride,
                            const uint8_t* host_pool, uint8_t* device_slots, uint32_t* slot_tables,
                            moe_expert_cache** cache) {
  if (!cache) return MOE_ERR_INVALID_ARG;
  *cache = nullptr;
  if (n_layers < 1 || n_experts < 1 || n_experts > 256 || slots < 1 || slots > n_experts) return MOE_ERR_INVALID_ARG;
  const bool host_only = device_slots == nullptr && slot_tables == nullptr;
  if (!host_only && (!device_slots || !slot_tables || !host_pool || blob_stride == 0 || blob_stride % 256))
    return MOE_ERR_INVALID_ARG;
  moe_expert_cache* c = new (std::nothrow) moe_expert_cache;
  if (!c) return MOE_ERR_INVALID_ARG;
  c->L = n_layers;
  c->E = n_experts;
  c->S = slots;
  c->stride = blob_stride;
  c->host_pool = host_pool;
  c->dev_slots = device_slots;
  c->dev_tables = slot_tables;
  c->host_only = host_only;
  const size_t LE = (size_t)n_layers * n_experts, LS = (size_t)n_layers * slots;
  c->freq.assign(LE, 0u);
  c->slot_of.assign(LE, -1);
  c->expert_in.assign(LS, -1);
  c->last_use.assign(LS, 0u);
  c->staged.resize(n_layers);
  c->staged_live.assign(n_layers, false);
  if (!host_only) {
    // nothing resident: every entry points past the layer's slots (synchronous)
    if (hipHostMalloc((void**)&c->table_stage, LE * sizeof(uint32_t), hipHostMallocDefault) != hipSuccess) {
      c->table_stage = nullptr;
      release(c);
      return MOE_ERR_HIP;
    }
    for (size_t i = 0; i < LE; ++i) c->table_stage[i] = (uint32_t)slots;
    if (hipHostMalloc((void**)&c->pick_stage, 16 * sizeof(int32_t), hipHostMallocDefault) != hipSuccess ||
        hipHostMalloc((void**)&c->pass_stage, 2 * LE * sizeof(uint32_t), hipHostMallocDefault) != hipSuccess ||
        hipEventCreateWithFlags(&c->ev_main, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c->ev_copy, hipEventDisableTiming) != hipSuccess) {
      release(c);
      return MOE_ERR_HIP;
    }
    for (int32_t l = 0; l < n_layers; ++l) {
      if (hipEventCreateWithFlags(&c->staged[l], hipEventDisableTiming) != hipSuccess) {
        release(c);
        return MOE_ERR_HIP;
      }
      c->staged_live[l] = true;
    }
    if (hipMemcpy(slot_tables, c->table_stage, LE * sizeof(uint32_t), hipMemcpyHostToDevice) != hipSuccess) {
      release(c);
      return MOE_ERR_HIP;
    }
  }
  *cache = c;
  return MOE_OK;
}

moe_status moe_cache_acquire(moe_expert_cache* c, int32_t layer, const int32_t* idx_host, int32_t n,
                             int32_t* slot_host, int32_t* n_misses, void* stream) {
  if (!c || c->device_policy || !idx_host || layer < 0 || layer >= c->L || n < 1 || n > c->S)
    return MOE_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (idx_host[i] < 0 || idx_host[i] >= c->E) return MOE_ERR_INVALID_ARG;
  const size_t le = (size_t)layer * c->E, ls = (size_t)layer * c->S;
  uint32_t* freq = c->freq.data() + le;
  int32_t* slot_of = c->slot_of.data() + le;
  int32_t* expert_in = c->expert_in.data() + ls;
  uint64_t* last_use = c->last_use.data() + ls;
  hipStream_t st = (hipStream_t)stream;

  // the staging copy of this layer's table is rewritten below: its previous upload must be done
  if (!c->host_only && hipEventSynchronize(c->staged[layer]) != hipSuccess) return MOE_ERR_HIP;

  const uint64_t now = ++c->clock;
  std::vector<bool> named(c->E, false);
  for (int32_t i = 0; i < n; ++i) {
    if (!named[idx_host[i]]) ++freq[idx_host[i]];
    named[idx_host[i]] = true;
  }
  int32_t miss = 0;
  bool table_changed = false;

  for (int32_t i = 0; i < n; ++i) {
    const int32_t e = idx_host[i];
    int32_t s = slot_of[e];
    if (s >= 0) {
      ++c->hits;
    } else {
      // a never-used slot, else the least-frequently used resident the request does not name
      s = -1;
      for (int32_t j = 0; j < c->S && s < 0; ++j)
        if (expert_in[j] < 0) s = j;
      if (s < 0) {
        for (int32_t j = 0; j < c->S; ++j) {
          const int32_t v = expert_in[j];
          if (named[v]) continue;
          if (s < 0) {
            s = j;
            continue;
          }
          const int32_t w = expert_in[s];
          if (freq[v] < freq[w] || (freq[v] == freq[w] && (last_use[j] < last_use[s] ||
                                                           (last_use[j] == last_use[s] && v < w))))
            s = j;
        }
      }
      if (s < 0) return MOE_ERR_INVALID_ARG;  // unreachable: n <= slots
      if (expert_in[s] >= 0) {
        slot_of[expert_in[s]] = -1;
        if (!c->host_only) c->table_stage[le + expert_in[s]] = (uint32_t)c->S;
      }
      expert_in[s] = e;
      slot_of[e] = s;
      if (!c->host_only) {
        c->table_stage[le + e] = (uint32_t)s;
        if (hipMemcpyAsync(c->dev_slots + (ls + s) * c->stride, c->host_pool + (le + e) * c->stride, c->stride,
                           hipMemcpyHostToDevice, st) != hipSuccess)
          return MOE_ERR_HIP;
        c->bytes += c->stride;
      }
      table_changed = true;
      ++c->misses;
      ++miss;
    }
    last_use[s] = now;
    if (slot_host) slot_host[i] = s;
  }
  if (!c->host_only && table_changed) {
    if (hipMemcpyAsync(c->dev_tables + le, c->table_stage + le, (size_t)c->E * sizeof(uint32_t),
                       hipMemcpyHostToDevice, st) != hipSuccess ||
        hipEventRecord(c->staged[layer], st) != hipSuccess)
      return MOE_ERR_HIP;
  }
  if (n_misses) *n_misses = miss;
  return MOE_OK;
}

moe_status moe_cache_decode(moe_expert_cache* c, int32_t layer, const moe_shape* shape, const uint8_t* router_blob,
                            const uint8_t* shared_blob, const void* x, moe_dtype x_dtype, const float* logit_offset,
                            int32_t* topk_idx, float* topk_w, float* expert_out, float* y, uint16_t* residual_bf16,
                            uint32_t* pass_tables, void* ws, size_t ws_bytes, void* stream, void* copy_stream) {
  if (!c || c->host_only || !shape || layer < 0 || layer >= c->L) return MOE_ERR_INVALID_ARG;
  if (shape->n_experts != c->E || shape->top_k > c->S || shape->top_k > 16 || shape->top_k < 1)
    return MOE_ERR_INVALID_ARG;
  if (c->stride < moe_expert_blob_bytes(shape)) return MOE_ERR_INVALID_ARG;
  if (copy_stream && !pass_tables && !c->device_policy) return MOE_ERR_INVALID_ARG;
  const int32_t E = c->E, S = c->S, k = shape->top_k;
  hipStream_t st = (hipStream_t)stream, cst = (hipStream_t)copy_stream;
  // the layer as the kernels see it: its slots as the pool, its slot table
  const moe_layer view{c->dev_slots + (size_t)layer * S * c->stride, c->stride, (uint64_t)S,
                       c->dev_tables + (size_t)layer * E, router_blob, shared_blob};
  moe_status r = moe_router_topk(shape, &view, x, x_dtype, 1, logit_offset, topk_idx, topk_w, nullptr, ws, ws_bytes,
                                 stream);
  if (r != MOE_OK) return r;
  if (c->device_policy) {
    // the policy and the copies on the device, in stream order: nothing comes back to the host
    if (!qmoe::launch_cache_plan(c->dstate, layer, topk_idx, k, st) ||
        !qmoe::launch_cache_fill(c->dstate, layer, c->host_pool_dev, c->dev_slots, k, st))
      return MOE_ERR_HIP;
    if ((r = moe_expert_ffn_decode(shape, &view, x, x_dtype, topk_idx, expert_out, ws, ws_bytes, stream)) != MOE_OK)
      return r;
    return moe_combine(shape, &view, x, x_dtype, 1, expert_out, nullptr, topk_w, y, residual_bf16, ws, ws_bytes,
                       stream);
  }
  // the host needs the picks
  if (hipMemcpyAsync(c->pick_stage, topk_idx, k * sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return MOE_ERR_HIP;
  const int32_t* picks = c->pick_stage;
  int32_t before[16], slots[16];
  if ((r = moe_cache_lookup(c, layer, picks, k, before)) != MOE_OK) return r;
  const bool all_hit = std::all_of(before, before + k, [](int32_t v) { return v >= 0; });
  if (!cst || all_hit) {
    // serial (or nothing to copy): the copies, then the routed experts, the shared expert
    // and the combine
    if ((r = moe_cache_acquire(c, layer, picks, k, nullptr, nullptr, stream)) != MOE_OK) return r;
    if ((r = moe_expert_ffn_decode(shape, &view, x, x_dtype, topk_idx, expert_out, ws, ws_bytes, stream)) != MOE_OK)
      return r;
    return moe_combine(shape, &view, x, x_dtype, 1, expert_out, nullptr, topk_w, y, residual_bf16, ws, ws_bytes,
                       stream);
  }
  // overlapped: the picks resident now (`before`) keep their slots through the acquire.
  // An evicted slot is overwritten only after the work already on the compute stream
  if (hipEventRecord(c->ev_main, st) != hipSuccess || hipStreamWaitEvent(cst, c->ev_main, 0) != hipSuccess)
    return MOE_ERR_HIP;
  if ((r = moe_cache_acquire(c, layer, picks, k, slots, nullptr, copy_stream)) != MOE_OK) return r;
  if (hipEventRecord(c->ev_copy, cst) != hipSuccess) return MOE_ERR_HIP;
  // the shared expert while the misses come in
  if ((r = moe_shared_expert_decode(shape, &view, x, x_dtype, ws, ws_bytes, stream)) != MOE_OK) return r;
  // tables of the two passes: the picks that hit, then those that missed; MOE_SLOT_SKIP elsewhere
  uint32_t* stage = c->pass_stage + (size_t)layer * 2 * E;
  bool any_hit = false, any_miss = false;
  for (int32_t i = 0; i < 2 * E; ++i) stage[i] = MOE_SLOT_SKIP;
  for (int32_t i = 0; i < k; ++i) {
    const bool hit = before[i] >= 0;
    stage[(hit ? 0 : E) + picks[i]] = (uint32_t)slots[i];
    any_hit |= hit;
    any_miss |= !hit;
  }
  if (hipMemcpyAsync(pass_tables, stage, 2 * (size_t)E * sizeof(uint32_t), hipMemcpyHostToDevice, st) != hipSuccess)
    return MOE_ERR_HIP;
  moe_layer pass = view;
  if (any_hit) {
    pass.slot_table = pass_tables;
    if ((r = moe_expert_ffn_decode(shape, &pass, x, x_dtype, topk_idx, expert_out, ws, ws_bytes, stream)) != MOE_OK)
      return r;
  }
  if (hipStreamWaitEvent(st, c->ev_copy, 0) != hipSuccess) return MOE_ERR_HIP;
  if (any_miss) {
    pass.slot_table = pass_tables + E;
    if ((r = moe_expert_ffn_decode(shape, &pass, x, x_dtype, topk_idx, expert_out, ws, ws_bytes, stream)) != MOE_OK)
      return r;
  }
  return moe_combine_decode(shape, expert_out, topk_w, y, residual_bf16, ws, ws_bytes, stream);
}

moe_status moe_cache_lookup(const moe_expert_cache* c, int32_t layer, const int32_t* idx_host, int32_t n,
                            int32_t* slot_host) {
  if (!c || c->device_policy || !idx_host || !slot_host || layer < 0 || layer >= c->L || n < 0) return MOE_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (idx_host[i] < 0 || idx_host[i] >= c->E) return MOE_ERR_INVALID_ARG;
  const int32_t* slot_of = c->slot_of.data() + (size_t)layer * c->E;
  for (int32_t i = 0; i < n; ++i) slot_host[i] = slot_of[idx_host[i]];
  return MOE_OK;
}

moe_status moe_cache_stats(const moe_expert_cache* c, uint64_t* hits, uint64_t* misses, uint64_t* bytes_copied) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->device_policy) {
    uint64_t v[3];
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(v, c->dstate.stats, sizeof v, hipMemcpyDeviceToHost) != hipSuccess)
      return MOE_ERR_HIP;
    if (hits) *hits = v[0];
    if (misses) *misses = v[1];
    if (bytes_copied) *bytes_copied = v[2];
    return MOE_OK;
  }
  if (hits) *hits = c->hits;
  if (misses) *misses = c->misses;
  if (bytes_copied) *bytes_copied = c->bytes;
  return MOE_OK;
}

uint64_t moe_cache_device_state_bytes(int32_t n_layers, int32_t n_experts, int32_t slots) {
  if (n_layers < 1 || n_experts < 1 || n_experts > 256 || slots < 1 || slots > n_experts) return 0;
  return qmoe::cache_dev_state_bytes(n_layers, n_experts, slots);
}

moe_status moe_cache_create_device(int32_t n_layers, int32_t n_experts, int32_t slots, uint64_t blob_stride,
                                   const uint8_t* host_pool, uint8_t* device_slots, uint32_t* slot_tables,
                                   void* device_state, uint64_t state_bytes, void* stream, moe_expert_cache** cache) {
  if (!cache) return MOE_ERR_INVALID_ARG;
  *cache = nullptr;
  if (n_layers < 1 || n_experts < 1 || n_experts > 256 || slots < 1 || slots > n_experts) return MOE_ERR_INVALID_ARG;
  if (!device_slots || !slot_tables || !host_pool || !device_state || blob_stride == 0 || blob_stride % 256 ||
      ((uintptr_t)device_state & 255u) || ((uintptr_t)slot_tables & 3u))
    return MOE_ERR_INVALID_ARG;
  if (state_bytes < qmoe::cache_dev_state_bytes(n_layers, n_experts, slots)) return MOE_ERR_WORKSPACE;
  // the fills read the host tier from the device: it must be mapped
  void* dev_view = nullptr;
  if (hipHostGetDevicePointer(&dev_view, const_cast<uint8_t*>(host_pool), 0) != hipSuccess || !dev_view) {
    (void)hipGetLastError();
    return MOE_ERR_INVALID_ARG;
  }
  moe_expert_cache* c = new (std::nothrow) moe_expert_cache;
  if (!c) return MOE_ERR_INVALID_ARG;
  c->L = n_layers;
  c->E = n_experts;
  c->S = slots;
  c->stride = blob_stride;
  c->host_pool = host_pool;
  c->host_pool_dev = static_cast<const uint8_t*>(dev_view);
  c->dev_slots = device_slots;
  c->dev_tables = slot_tables;
  c->device_policy = true;
  c->dstate = qmoe::cache_dev_state(device_state, slot_tables, n_layers, n_experts, slots, blob_stride);
  hipStream_t st = (hipStream_t)stream;
  if (!qmoe::launch_cache_init(c->dstate, st) || hipStreamSynchronize(st) != hipSuccess) {
    release(c);
    return MOE_ERR_HIP;
  }
  *cache = c;
  return MOE_OK;
}

moe_status moe_cache_destroy(moe_expert_cache* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (!c->host_only && !c->device_policy)
    for (int32_t l = 0; l < c->L; ++l)
      if (c->staged_live[l] && hipEventSynchronize(c->staged[l]) != hipSuccess) {
        release(c);
        return MOE_ERR_HIP;
      }
  release(c);
  return MOE_OK;
}

}  // extern "C"
