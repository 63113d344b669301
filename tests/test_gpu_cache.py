"""Decode through the tiered expert store (HBM slots per layer in front of a pinned host
pool, moe_cache_*) gives the same bits as decode over the all-resident pool: the same
kernels run on the same bytes, reached through the cache's slot tables. Checked over a
stream of tokens that hits, misses and evicts."""
import numpy as np
import pytest
import torch

import synth
from _harness import device, empty_f32, empty_i32, to_dev_x, workspace

pytestmark = pytest.mark.gpu
q = pytest.importorskip("quantized_mixture_experts_bit_amd")
from quantized_mixture_experts_bit_amd.weights import HostExpertPool, TieredStore, upload_layers  # noqa: E402


def decode_split(shape, layer_c, x, off, ws, cached=None):
    """Router, (cache acquire), routed experts, shared + combine: the split calls."""
    k, d = shape.top_k, shape.d_model
    idx, w = empty_i32(k), empty_f32(k)
    eo, y = empty_f32(k, d), empty_f32(d)
    q.moe_router_topk(shape, layer_c, x, 1, off, idx, w, None, ws)
    miss = None
    if cached is not None:
        miss = cached.acquire(idx.cpu().numpy())  # the host needs the picks: a synchronising copy
    q.moe_expert_ffn_decode(shape, layer_c, x, idx, eo, ws)
    q.moe_combine(shape, layer_c, x, 1, eo, None, w, y, None, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), eo.cpu().numpy(), y.cpu().numpy(), miss


@pytest.mark.parametrize("shape,slots,zipf", [(synth.TINY, 16, True), (synth.GEMMA4, 16, True),
                                              (synth.GEMMA4, 8, False)], ids=["tiny-16", "gemma4-16-zipf",
                                                                             "gemma4-8-uniform"])
def test_cached_decode_matches_resident(shape, slots, zipf):
    n_layers, tokens = 2, 12
    layers = [synth.make_layer(shape, seed=5, layer=l) for l in range(n_layers)]
    resident = upload_layers(shape, layers, device())
    host = HostExpertPool(shape, n_layers)
    for l, L in enumerate(layers):
        host.load_layer(l, L)
    store = TieredStore(host, slots, device())
    try:
        cached = [store.layer(l, resident[l].router, resident[l].shared) for l in range(n_layers)]
        offs = [torch.from_numpy(synth.make_zipf_offset(shape, seed=0, layer=l)).to(device()) if zipf else None
                for l in range(n_layers)]
        ws = workspace(shape, 1)
        total_miss = 0
        for t in range(tokens):
            for l in range(n_layers):
                x = to_dev_x(synth.make_x(shape, 1, seed=100 + t, stream=l, dtype="bf16"))
                i0, e0, y0, _ = decode_split(shape, resident[l].c, x, offs[l], ws)
                i1, e1, y1, miss = decode_split(shape, cached[l].c, x, offs[l], ws, cached[l])
                np.testing.assert_array_equal(i1, i0)
                assert np.array_equal(e1.view(np.uint32), e0.view(np.uint32)), (t, l)
                assert np.array_equal(y1.view(np.uint32), y0.view(np.uint32)), (t, l)
                total_miss += miss
        assert q.moe_check_device_error() == 0
        hits, misses, nbytes = store.stats()
        assert hits + misses == tokens * n_layers * shape.top_k
        assert misses == total_miss and nbytes == misses * store.stride
        assert misses >= n_layers * min(slots, shape.top_k)  # cold start
        if zipf:
            assert hits > 0
        if slots < shape.n_experts and not zipf:
            assert misses > n_layers * slots  # evictions happened
    finally:
        store.close()


def split_prefill(shape, dl_c, x, rows, off, ws):
    """Router, grouping, routed experts, shared + combine on the resident pool."""
    k, d, E = shape.top_k, shape.d_model, shape.n_experts
    o = dict(idx=empty_i32(rows, k), w=empty_f32(rows, k), cnt=empty_i32(E), off=empty_i32(E + 1),
             perm=empty_i32(rows * k), inv=empty_i32(rows * k), eo=empty_f32(rows * k, d), y=empty_f32(rows, d))
    q.moe_router_topk(shape, dl_c, x, rows, off, o["idx"], o["w"], None, ws)
    q.moe_group_by_expert(shape, o["idx"], rows, o["cnt"], o["off"], o["perm"], o["inv"], ws)
    q.moe_expert_ffn_prefill_chunk(shape, dl_c, x, rows, o["off"], o["perm"], o["eo"], ws)
    q.moe_combine(shape, dl_c, x, rows, o["eo"], o["inv"], o["w"], o["y"], None, ws)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in o.items()}


@pytest.mark.parametrize("rows,zipf", [(48, False), (96, True)], ids=["48rows-uniform", "96rows-zipf"])
def test_cached_prefill_matches_resident(rows, zipf):
    """A chunk whose experts outnumber the 16 slots runs in passes (MOE_SLOT_SKIP for the
    experts of other passes) and gives the resident pool's bits."""
    shape, slots = synth.GEMMA4, 16
    k, d, E = shape.top_k, shape.d_model, shape.n_experts
    L = synth.make_layer(shape, seed=5, layer=0)
    (resident,) = upload_layers(shape, [L], device())
    host = HostExpertPool(shape, 1)
    host.load_layer(0, L)
    store = TieredStore(host, slots, device())
    try:
        cached = store.layer(0, resident.router, resident.shared)
        off = torch.from_numpy(synth.make_zipf_offset(shape, seed=0, layer=0)).to(device()) if zipf else None
        ws = workspace(shape, rows)
        for chunk in range(2):
            xd = to_dev_x(synth.make_x(shape, rows, seed=40 + chunk, dtype="bf16"))
            want = split_prefill(shape, resident.c, xd, rows, off, ws)
            o = dict(idx=empty_i32(rows, k), w=empty_f32(rows, k), cnt=empty_i32(E), off=empty_i32(E + 1),
                     perm=empty_i32(rows * k), inv=empty_i32(rows * k), eo=empty_f32(rows * k, d),
                     y=empty_f32(rows, d))
            passes, _ = cached.prefill(xd, rows, off, o["idx"], o["w"], o["cnt"], o["off"], o["perm"], o["inv"],
                                       o["eo"], o["y"], None, ws)
            torch.cuda.synchronize()
            got = {n: t.cpu().numpy() for n, t in o.items()}
            assert passes == -(-int((want["cnt"] > 0).sum()) // slots) and passes >= 2
            for n in ("idx", "cnt", "perm", "inv"):
                np.testing.assert_array_equal(got[n], want[n])
            assert np.array_equal(got["eo"].view(np.uint32), want["eo"].view(np.uint32)), chunk
            assert np.array_equal(got["y"].view(np.uint32), want["y"].view(np.uint32)), chunk
        assert q.moe_check_device_error() == 0
    finally:
        store.close()
