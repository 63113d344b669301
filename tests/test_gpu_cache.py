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
