// C ABI of the quantized MoE FFN block (see include/moe.h): argument checks,
// workspace carve-up and kernel launches on the caller's stream. The whole
// device library is this one translation unit.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "common.h"
#include "decode_fused.h"
#include "decode_kernels.h"
#include "moe.h"
#include "group_kernels.h"
#include "prefill_gemm.h"
#include "router_kernels.h"

using namespace qmoe;

namespace {

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
  if (s->n_experts < 64 || s->n_experts > 256 || s->n_experts % 64) return false;
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
  size_t gu_count, dn_count, fused_sync, fused_lg, fused_h, fused_eo, router_partial, gu_partial, h_hi,
      h_lo, h_gsum,
      shared_part, pf_H, pf_Hs, pf_shared_out, pf_hmaxp, pf_Hh, pf_hsc, total;
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
  w.router_partial = take(sizeof(double) * kRouterSplits * R * s->n_experts);
  w.gu_partial = take(sizeof(float) * (size_t)(k + 1) * 2 * dc.nbmax * dc.P * 64);
  w.h_hi = take(sizeof(uint16_t) * (size_t)(k + 1) * dc.fmax);
  w.h_lo = take(sizeof(uint16_t) * (size_t)(k + 1) * dc.fmax);
  w.h_gsum = take(sizeof(float) * (size_t)(k + 1) * dc.nbmax);
  w.shared_part = take(sizeof(float) * (size_t)dc.Ps * d);
  w.pf_H = take(sizeof(float) * R * k * s->d_ff);
  w.pf_Hs = take(sizeof(float) * R * s->d_ff_shared);
  w.pf_shared_out = take(sizeof(float) * R * d);
  w.pf_hmaxp = take(sizeof(float) * R * ((size_t)k * (s->d_ff / 64) + s->d_ff_shared / 64));
  w.pf_Hh = take(sizeof(uint16_t) * R * ((size_t)k * s->d_ff + s->d_ff_shared));
  w.pf_hsc = take(sizeof(float) * R * (k + 1));
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
                   float* w, double* logits, void* ws, hipStream_t st) {
  const Ws W = ws_layout(s, rows);
  double* part = at<double>(ws, W.router_partial);
  const int blocks = cdiv(rows, 16) * (s->n_experts / 16) * kRouterSplits;
  k_router_logits<XT><<<blocks, 256, 0, st>>>(L->router_blob, x, rows, s->d_model, s->n_experts, part);
  k_router_select<<<rows, 256, 0, st>>>(part, rows, s->n_experts, s->top_k, off, idx, w, logits);
}

DecodeArgs decode_args(const moe_shape* s, const moe_layer* L, const int32_t* idx, void* ws, float* expert_out,
                       const float* topk_w, float* y, uint16_t* residual) {
  const DecodeCfg dc = decode_cfg(s);
  const Ws W = ws_layout(s, 1);
  DecodeArgs A;
  memset(&A, 0, sizeof A);
  A.pool = L->pool;
  A.stride = L->blob_stride;
  A.n_blobs = L->n_blobs;
  A.slot_table = L->slot_table;
  A.topk_idx = idx;
  A.shared_blob = L->shared_blob;
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

// One persistent launch for the whole decode row, when the grid fits on the chip;
// returns false (nothing launched) otherwise.
template <typename XT>
bool launch_decode_fused(const moe_shape* s, const moe_layer* L, const XT* x, const float* off, int32_t* idx,
                         float* w, float* expert_out, float* y, uint16_t* residual, void* ws, hipStream_t st) {
  // limits of the fused kernel's register and LDS tiling (see decode_fused.h)
  const int d = s->d_model, f = s->d_ff, fs = s->d_ff_shared;
  if (d / 64 > kFusedMaxG || f > 64 * 4 * kFusedRoutedGW || fs > 2 * 64 * 4 * kFusedSharedGW) return false;
  if (sizeof(XT) == 4 && d > kFusedXWords) return false;
  const Ws W = ws_layout(s, 1);
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
  const int grid = F.n_rt + F.n_sg + F.n_rg + F.n_rd + 2 * F.n_sd + 1;  // + the epoch keeper
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
  A.H = at<float>(ws, W.pf_H);
  A.Hs = at<float>(ws, W.pf_Hs);
  A.expert_out = expert_out;
  A.shared_out = at<float>(ws, W.pf_shared_out);
  A.hmaxp = at<float>(ws, W.pf_hmaxp);
  A.Hh = at<uint16_t>(ws, W.pf_Hh);
  A.hsc = at<float>(ws, W.pf_hsc);
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

// grid of a persistent GEMM launch: what the chip holds at once (a multiple of the
// XCD count, so work item i always runs on XCD i % 8), at most the work items
int persistent_grid(int resident, int items) {
  int g = std::min(resident, items);
  if (g > kXcds) g -= g % kXcds;
  return std::max(g, 1);
}

// one gate/up launch, the H conversion and one down launch covering the routed
// tiles and/or the shared expert's tiles
template <typename XT>
void launch_prefill(PrefillArgs A, const XT* x, bool routed, bool shared, hipStream_t st) {
  static int cap_gu[64], cap_dn[64];
  if (!routed) A.routed_mtiles = 0;
  if (!shared) A.shared_mtiles = 0;
  // items at most (routed tile count bounded by the pair count plus one per expert)
  const int gu_items = xcd_blocks(A.routed_mtiles, A.f / 64) + xcd_blocks(A.shared_mtiles, A.fs / 64);
  if (gu_items == 0) return;
  k_prefill_gateup<XT><<<persistent_grid(resident_blocks(k_prefill_gateup<XT>, cap_gu), gu_items), 256, 0, st>>>(A, x);
  const int P = A.rows * A.top_k;
  const int first = routed ? 0 : P;
  const int count = (routed ? P : 0) + (shared ? A.rows : 0);
  k_prefill_hconv<<<cdiv(count, 4), 256, 0, st>>>(A, first, count);
  const int dnc = (A.d / 64 + kDownBlocks - 1) / kDownBlocks;
  const int dn_items = xcd_blocks(A.routed_mtiles, dnc) + xcd_blocks(A.shared_mtiles, dnc);
  k_prefill_down<<<persistent_grid(resident_blocks(k_prefill_down, cap_dn), dn_items), 256, 0, st>>>(A);
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
  if (dt == MOE_BF16)
    launch_router(s, L, (const uint16_t*)x, rows, off, idx, w, logits, ws, hs);
  else
    launch_router(s, L, (const float*)x, rows, off, idx, w, logits, ws, hs);
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
  DecodeArgs A = decode_args(s, L, idx, ws, expert_out, nullptr, nullptr, nullptr);
  if (dt == MOE_BF16)
    launch_decode_gateup(A, (const uint16_t*)x, true, false, hs);
  else
    launch_decode_gateup(A, (const float*)x, true, false, hs);
  launch_decode_down(A, true, false, false, hs);
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
    launch_prefill(A, (const uint16_t*)x, true, false, hs);
  else
    launch_prefill(A, (const float*)x, true, false, hs);
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
    DecodeArgs A = decode_args(s, L, nullptr, ws, const_cast<float*>(expert_out), topk_w, y, residual);
    if (dt == MOE_BF16)
      launch_decode_gateup(A, (const uint16_t*)x, false, true, hs);
    else
      launch_decode_gateup(A, (const float*)x, false, true, hs);
    launch_decode_down(A, false, true, true, hs);
    return launched();
  }
  PrefillArgs A = prefill_args(s, L, rows, nullptr, nullptr, nullptr, ws);
  if (dt == MOE_BF16)
    launch_prefill(A, (const uint16_t*)x, false, true, hs);
  else
    launch_prefill(A, (const float*)x, false, true, hs);
  k_combine<<<dim3(cdiv(s->d_model / 4, 256), rows), 256, 0, hs>>>(A.shared_out, expert_out, inv_perm, topk_w, rows,
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
  hipStream_t hs = (hipStream_t)stream;
  const bool fused = dt == MOE_BF16
                         ? launch_decode_fused(s, L, (const uint16_t*)x, off, idx, w, expert_out, y, residual, ws, hs)
                         : launch_decode_fused(s, L, (const float*)x, off, idx, w, expert_out, y, residual, ws, hs);
  if (fused) return launched();
  // the grid does not fit on the device at once: three launches instead
  DecodeArgs A = decode_args(s, L, idx, ws, expert_out, w, y, residual);
  if (dt == MOE_BF16) {
    launch_router(s, L, (const uint16_t*)x, 1, off, idx, w, nullptr, ws, hs);
    launch_decode_gateup(A, (const uint16_t*)x, true, true, hs);
  } else {
    launch_router(s, L, (const float*)x, 1, off, idx, w, nullptr, ws, hs);
    launch_decode_gateup(A, (const float*)x, true, true, hs);
  }
  launch_decode_down(A, true, true, true, hs);
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
  if (dt == MOE_BF16)
    launch_router(s, L, (const uint16_t*)x, rows, off, idx, w, nullptr, ws, hs);
  else
    launch_router(s, L, (const float*)x, rows, off, idx, w, nullptr, ws, hs);
  const size_t lds = sizeof(int32_t) * kGroupWaves * s->n_experts;
  k_group<<<1, 1024, lds, hs>>>(idx, rows * s->top_k, s->n_experts, count, offset, perm, inv_perm);
  PrefillArgs A = prefill_args(s, L, rows, offset, perm, expert_out, ws);
  if (dt == MOE_BF16)
    launch_prefill(A, (const uint16_t*)x, true, true, hs);
  else
    launch_prefill(A, (const float*)x, true, true, hs);
  k_combine<<<dim3(cdiv(s->d_model / 4, 256), rows), 256, 0, hs>>>(A.shared_out, expert_out, inv_perm, w, rows,
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

moe_status moe_check_device_error(void* stream, uint32_t* flags) {
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MOE_ERR_HIP;
  uint32_t v = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_moe_device_error), sizeof v, 0, hipMemcpyDeviceToHost) != hipSuccess)
    return MOE_ERR_HIP;
  if (flags) *flags = v;
  if (v == 0) return MOE_OK;
  const uint32_t zero = 0;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_moe_device_error), &zero, sizeof zero, 0, hipMemcpyHostToDevice) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_ERR_DEVICE_CHECK;
}

}  // extern "C"
