// The expert cache's replacement policy kept on the device (library-internal): the
// state views, and the launches the host side of the cache makes (defined with the
// kernels). The rule is the host policy's (expert_cache.cpp): every request counts
// once toward its expert's frequency; a miss takes a never-used slot, else the slot
// of the resident expert with the smallest (frequency, last use, id) that the request
// does not name. Here one thread applies it per request, so a decode row goes from its
// picks to its copies without a round trip to the host.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

constexpr int kCacheMaxPicks = 16;      // experts of one request (top_k <= 16)
constexpr int kCacheCopyBlocks = 64;    // workgroups per blob of a fill

struct CacheDevState {
  uint32_t* tables;     // [L][E] the slot tables: the slot of a resident expert, else S
  uint32_t* freq;       // [L][E] requests so far
  int32_t* expert_in;   // [L][S] expert in each slot, or -1
  uint64_t* last_use;   // [L][S] the layer's request counter at the slot's last use
  uint64_t* clock;      // [L] requests so far, per layer
  uint32_t* miss;       // [1 + 2 * kCacheMaxPicks]: the last plan's miss count, then (expert, slot)
  uint64_t* stats;      // [3]: requests that hit, that missed, bytes copied
  int L, E, S;
  uint64_t stride;
};

// bytes of the state buffer (without the slot tables, which the caller owns apart)
uint64_t cache_dev_state_bytes(int L, int E, int S);
CacheDevState cache_dev_state(void* base, uint32_t* tables, int L, int E, int S, uint64_t stride);

// everything empty: no expert resident, counters at zero
bool launch_cache_init(const CacheDevState& st, hipStream_t stream);
// the policy for the n experts picks[0..n) of `layer` (device memory): updates the state
// and the layer's slot table and leaves the misses in st.miss
bool launch_cache_plan(const CacheDevState& st, int layer, const int32_t* picks, int n, hipStream_t stream);
// copies the blobs of the last plan's misses (at most n_max) from the mapped host tier
// (host_pool_dev: the device address of blob (0, 0); blob (l, e) at (l * E + e) * stride)
// into the layer's slots (dev_slots: slot 0 of layer 0)
bool launch_cache_fill(const CacheDevState& st, int layer, const uint8_t* host_pool_dev, uint8_t* dev_slots,
                       int n_max, hipStream_t stream);

}  // namespace qmoe
