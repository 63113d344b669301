"""Device-resident weights: the packed-expert pool, per-layer slot tables, router
and shared-expert blobs.

The pages keep every layer's 128 routed experts as fixed-size, page-aligned
blobs and bind sub-regions of them instead of building one buffer per expert
(blog-mushroom article "TurboFieldfare: Gemma 4 26B on an 8 GB MacBook",
model-file-layout section). Here all blobs of all layers live in one
HBM-resident torch uint8 tensor (the pool, 12.85 GB for 30 x 128 experts at the
Gemma-4 shape) and each layer has a device slot table (expert id -> blob
index) that the kernels read. Packing runs on the host through the library's
C packer; nothing here computes any part of the block.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import (MOE_SLOT_SKIP, as_shape, moe_cache_acquire, moe_cache_create, moe_cache_create_device,
               moe_cache_decode, moe_cache_destroy, moe_cache_device_state_bytes,
               moe_cache_stats, moe_combine, moe_expert_blob_bytes, moe_expert_ffn_prefill_chunk, moe_group_by_expert,
               moe_layer, moe_matrix4_bytes, moe_matrix8_bytes, moe_pack_matrix4, moe_pack_matrix8,
               moe_router_blob_bytes, moe_router_topk, moe_shared_blob_bytes)

BLOB_ALIGN = 4096  # blob stride granularity (a page)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def pack_expert_into(shape, expert, out: np.ndarray) -> None:
    """gate | up | down of one expert (objects with .q/.s/.b) into out[0:blob_bytes]."""
    d, f = shape.d_model, expert.gate.rows
    m_gu = moe_matrix4_bytes(f, d)
    moe_pack_matrix4(expert.gate.q, expert.gate.s, expert.gate.b, out[0:m_gu])
    moe_pack_matrix4(expert.up.q, expert.up.s, expert.up.b, out[m_gu:2 * m_gu])
    moe_pack_matrix4(expert.down.q, expert.down.s, expert.down.b, out[2 * m_gu:2 * m_gu + moe_matrix4_bytes(d, f)])


def pack_router(shape, router) -> np.ndarray:
    out = np.empty(moe_router_blob_bytes(as_shape(shape)), dtype=np.uint8)
    moe_pack_matrix8(router.q, router.s, router.b, out)
    return out


def pack_shared(shape, shared) -> np.ndarray:
    out = np.empty(moe_shared_blob_bytes(as_shape(shape)), dtype=np.uint8)
    pack_expert_into(shape, shared, out)
    return out


class DeviceLayer:
    """One layer's device handles; `c` is the moe_layer struct the C ABI takes."""

    def __init__(self, pool: "ExpertPool", router: torch.Tensor, shared: torch.Tensor, slot_table: torch.Tensor):
        self.pool = pool
        self.router = router
        self.shared = shared
        self.slot_table = slot_table
        self.c = moe_layer(pool.buf.data_ptr(), pool.stride, pool.n_blobs, slot_table.data_ptr(),
                           router.data_ptr(), shared.data_ptr())


class ExpertPool:
    """HBM pool of `n_blobs` expert blobs of `stride` bytes."""

    def __init__(self, shape, n_blobs: int, device="cuda", stride: Optional[int] = None):
        self.shape = shape
        blob = moe_expert_blob_bytes(as_shape(shape))
        self.blob_bytes = blob
        self.stride = stride or (blob + BLOB_ALIGN - 1) // BLOB_ALIGN * BLOB_ALIGN
        assert self.stride >= blob and self.stride % 256 == 0
        self.n_blobs = n_blobs
        self.device = torch.device(device)
        self.buf = torch.empty(n_blobs * self.stride, dtype=torch.uint8, device=self.device)

    def load_experts(self, shape, experts: Sequence, blob_index: Sequence[int]) -> None:
        """Pack `experts` on the host and copy expert i into blob blob_index[i]."""
        n = len(experts)
        staging = torch.empty(n * self.stride, dtype=torch.uint8, pin_memory=True)
        host = staging.numpy()
        with cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(lambda i: pack_expert_into(shape, experts[i], host[i * self.stride:(i + 1) * self.stride]),
                        range(n)))
        idx = list(blob_index)
        if idx == list(range(idx[0], idx[0] + n)):
            self.buf[idx[0] * self.stride:(idx[0] + n) * self.stride].copy_(staging)
        else:
            dev = staging.to(self.device)
            for i, b in enumerate(idx):
                self.buf[b * self.stride:(b + 1) * self.stride].copy_(dev[i * self.stride:(i + 1) * self.stride])
        torch.cuda.synchronize(self.device)

    def add_layer(self, layer, first_blob: int, placement: Optional[Sequence[int]] = None) -> DeviceLayer:
        """Upload one canonical layer (router, shared, experts). Expert e goes to blob
        first_blob + placement[e] (identity placement by default)."""
        shape = layer.shape
        E = shape.n_experts
        place = list(range(E)) if placement is None else list(placement)
        blobs = [first_blob + p for p in place]
        self.load_experts(shape, layer.experts, blobs)
        router = torch.from_numpy(pack_router(shape, layer.router)).to(self.device)
        shared = torch.from_numpy(pack_shared(shape, layer.shared)).to(self.device)
        table = torch.tensor(blobs, dtype=torch.int64).to(torch.int32).to(self.device)
        return DeviceLayer(self, router, shared, table)


def upload_layers(shape, layers: List, device="cuda") -> List[DeviceLayer]:
    """Pool with every expert of every layer, identity placement, layer-major."""
    E = shape.n_experts
    pool = ExpertPool(shape, len(layers) * E, device)
    return [pool.add_layer(L, i * E) for i, L in enumerate(layers)]


# ------------------------------------------------------------------ tiered residency

class HostExpertPool:
    """Slow tier: every expert blob of `n_layers` layers in pinned host memory,
    layer-major (blob (l, e) at (l * n_experts + e) * stride)."""

    def __init__(self, shape, n_layers: int, stride: Optional[int] = None):
        blob = moe_expert_blob_bytes(as_shape(shape))
        self.shape = shape
        self.n_layers = n_layers
        self.stride = stride or (blob + BLOB_ALIGN - 1) // BLOB_ALIGN * BLOB_ALIGN
        self.buf = torch.empty(n_layers * shape.n_experts * self.stride, dtype=torch.uint8, pin_memory=True)

    def load_layer(self, l: int, layer) -> None:
        E = self.shape.n_experts
        host = self.buf.numpy()
        base = l * E * self.stride
        with cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(lambda e: pack_expert_into(self.shape, layer.experts[e],
                                                   host[base + e * self.stride:base + (e + 1) * self.stride]),
                        range(E)))


class CachedLayer:
    """One layer of a TieredStore as the C ABI sees it (`c`): its HBM slots as the
    pool, its slot table, and the resident router and shared blobs."""

    def __init__(self, store: "TieredStore", l: int, router: torch.Tensor, shared: torch.Tensor):
        self.store, self.l, self.router, self.shared = store, l, router, shared
        S, st = store.slots, store.stride
        self.c = moe_layer(store.dev_slots.data_ptr() + l * S * st, st, S,
                           store.tables.data_ptr() + l * store.shape.n_experts * 4, router.data_ptr(),
                           shared.data_ptr())
        # the slots seen through a table of the prefill pass in flight (prefill())
        self.pass_table = torch.empty(store.shape.n_experts, dtype=torch.int32, device=store.tables.device)
        self.pass_view = moe_layer(store.dev_slots.data_ptr() + l * S * st, st, S, self.pass_table.data_ptr(),
                                   router.data_ptr(), shared.data_ptr())
        # decode: the tables of the passes over the picks that hit and those that missed
        self.dec_tables = torch.empty(2, store.shape.n_experts, dtype=torch.int32, device=store.tables.device)

    def acquire(self, idx, slots=None, stream=None) -> int:
        """Makes the experts idx (host int32 array) resident; returns the misses."""
        return moe_cache_acquire(self.store.handle, self.l, idx, slots, stream)

    def decode(self, x, logit_offset, topk_idx, topk_w, expert_out, y, residual, ws, copy_stream=None) -> None:
        """One decode row through the cache on the current stream (moe_cache_decode): the
        router, its picks to the host, the cache makes them resident; with copy_stream the
        misses are copied on it while the shared expert and the picks that hit run (the
        pages' per-token flow), without it the copies go first. y and the residual are
        bit-identical to the split calls on a resident pool."""
        moe_cache_decode(self.store.handle, self.l, self.store.shape, self.router, self.shared, x, logit_offset,
                         topk_idx, topk_w, expert_out, y, residual, self.dec_tables, ws, None, copy_stream)

    def prefill(self, x, rows: int, logit_offset, topk_idx, topk_w, count, offset, perm, inv_perm, expert_out,
                y, residual, ws):
        """A prefill chunk through the cache: router, grouping, then the routed experts
        in passes of at most `slots` experts (each pass makes its group resident and runs
        the routed GEMMs with a table that names that group and skips every other expert),
        then the shared expert and the combine. The same calls and outputs as the split
        prefill on an all-resident pool. Returns (passes, misses)."""
        shape, S, E = self.store.shape, self.store.slots, self.store.shape.n_experts
        moe_router_topk(shape, self.c, x, rows, logit_offset, topk_idx, topk_w, None, ws)
        moe_group_by_expert(shape, topk_idx, rows, count, offset, perm, inv_perm, ws)
        need = np.flatnonzero(count.cpu().numpy() > 0).astype(np.int32)  # the host plans the passes
        passes = misses = 0
        for i in range(0, need.size, S):
            group = need[i:i + S]
            slots = np.empty(group.size, dtype=np.int32)
            misses += self.acquire(group, slots)
            table = np.full(E, MOE_SLOT_SKIP, dtype=np.uint32)
            table[group] = slots
            self.pass_table.copy_(torch.from_numpy(table.view(np.int32)))  # ordered after the previous pass
            moe_expert_ffn_prefill_chunk(shape, self.pass_view, x, rows, offset, perm, expert_out, ws)
            passes += 1
        moe_combine(shape, self.c, x, rows, expert_out, inv_perm, topk_w, y, residual, ws)
        return passes, misses


class TieredStore:
    """Fast tier: `slots` HBM expert slots per layer in front of a HostExpertPool,
    managed by the library's cache (moe_cache_*). device_policy=True keeps the
    replacement policy on the device (moe_cache_create_device): decode rows then never
    wait for the host (and can be graph-captured); the prefill passes need the host
    policy."""

    def __init__(self, host: HostExpertPool, slots: int, device="cuda", device_policy: bool = False):
        self.shape, self.host, self.slots, self.stride = host.shape, host, slots, host.stride
        E, L = host.shape.n_experts, host.n_layers
        dev = torch.device(device)
        self.device_policy = device_policy
        self.dev_slots = torch.empty(L * slots * self.stride, dtype=torch.uint8, device=dev)
        self.tables = torch.empty(L * E, dtype=torch.int32, device=dev)
        if device_policy:
            self.state = torch.empty(moe_cache_device_state_bytes(L, E, slots), dtype=torch.uint8, device=dev)
            self.handle = moe_cache_create_device(L, E, slots, self.stride, host.buf, self.dev_slots, self.tables,
                                                  self.state)
        else:
            self.handle = moe_cache_create(L, E, slots, self.stride, host.buf, self.dev_slots, self.tables)

    def layer(self, l: int, router: torch.Tensor, shared: torch.Tensor) -> CachedLayer:
        return CachedLayer(self, l, router, shared)

    def stats(self):
        return moe_cache_stats(self.handle)

    def close(self) -> None:
        if self.handle:
            moe_cache_destroy(self.handle)
            self.handle = None
