"""moe_layer_decode_noalloc (the decode entry point for callers that cannot allocate:
its scratch is the library's static device array) against moe_layer_decode with a
caller workspace, through the C ABI: the same kernels, so the same bits. Two calls in
a row, the second on a smaller layer, then the first shape again; and shapes past the
static scratch's maximum are rejected before anything is launched."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle as O
import synth
from _harness import REL_TOL, check_topk, device, empty_f32, empty_i32, get_layer, rel_err, to_dev_x, workspace

q = pytest.importorskip("quantized_mixture_experts_bit_amd")


def _decode(shape, dl, x, off, noalloc, ws=None, residual=None):
    k, d = shape.top_k, shape.d_model
    o = dict(idx=empty_i32(k), w=empty_f32(k), eo=empty_f32(k, d), y=empty_f32(d))
    if noalloc:
        q.moe_layer_decode_noalloc(shape, dl.c, x, off, o["idx"], o["w"], o["eo"], o["y"], residual)
    else:
        q.moe_layer_decode(shape, dl.c, x, off, o["idx"], o["w"], o["eo"], o["y"], residual, ws)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in o.items()}


def _same_bits(a, b, what):
    for n in a:
        assert np.array_equal(a[n].view(np.uint32), b[n].view(np.uint32)), "%s: %s differs" % (what, n)


CALLS = [  # (shape, variant, x dtype, seed): the second call is on a smaller layer
    (synth.GEMMA4, synth.Variant(), "bf16", 3),
    (synth.TINY, synth.Variant(router_scale_log2=-6), "f32", 4),
    (synth.GEMMA4, synth.Variant(router_scale_log2=-6), "bf16", 5),
    (synth.TINY, synth.Variant(), "bf16", 6),
]


@pytest.mark.gpu
def test_noalloc_decode_matches_workspace_decode():
    print("noalloc decode: %d calls in a row" % len(CALLS), flush=True)
    for i, (shape, variant, dt, seed) in enumerate(CALLS):
        L, ol, dl = get_layer(shape, variant=variant)
        x_np = synth.make_x(shape, 1, seed=seed, dtype=dt)
        x = to_dev_x(x_np)
        ws = workspace(shape, 1)
        want = _decode(shape, dl, x, None, noalloc=False, ws=ws)
        got = _decode(shape, dl, x, None, noalloc=True)
        _same_bits(got, want, "call %d" % i)
        # and against the oracle
        ref = O.moe_rows(ol, x_np)
        if check_topk(got["idx"][None], ref, shape.top_k)[0]:
            ref = O.moe_rows(ol, x_np, idx=got["idx"][None])
        assert rel_err(got["y"], ref["y"][0]) <= REL_TOL, "call %d" % i
        print("  call %d (d_model %d, %s): same bits as the workspace call" % (i, shape.d_model, dt), flush=True)
    assert q.moe_check_device_error() == 0


@pytest.mark.gpu
def test_noalloc_decode_residual_in_place():
    """The residual add in place (x is the residual buffer) gives the workspace call's bits."""
    shape = synth.GEMMA4
    L, ol, dl = get_layer(shape)
    x_np = synth.make_x(shape, 1, seed=9, dtype="bf16")
    ha, hb = to_dev_x(x_np).clone(), to_dev_x(x_np).clone()
    ws = workspace(shape, 1)
    want = _decode(shape, dl, ha, None, noalloc=False, ws=ws, residual=ha)
    got = _decode(shape, dl, hb, None, noalloc=True, residual=hb)
    _same_bits(got, want, "residual")
    assert torch.equal(ha.view(torch.int16), hb.view(torch.int16))
    assert q.moe_check_device_error() == 0


def test_noalloc_rejects_shapes_past_the_scratch():
    """Checked before any launch (runs without a GPU)."""
    lib = q.lib()
    lay = q.moe_layer(0x100000, 4 << 20, 128, 0x200000, 0x300000, 0x400000)
    for shape in (q.MoeShape(2816, 704, 4096), q.MoeShape(4096, 704, 2112), q.MoeShape(2816, 1024, 2112)):
        st = lib.moe_layer_decode_noalloc(C.byref(shape), C.byref(lay), 0x50000, q.MOE_BF16, None, 0x60000, 0x70000,
                                          0x80000, 0x90000, None, None)
        assert st == q.MOE_ERR_WORKSPACE
    bad = q.MoeShape(2816, 704, 2112, n_experts=192)
    assert lib.moe_layer_decode_noalloc(C.byref(bad), C.byref(lay), 0x50000, q.MOE_BF16, None, 0x60000, 0x70000,
                                        0x80000, 0x90000, None, None) == q.MOE_ERR_UNSUPPORTED_SHAPE
    assert lib.moe_layer_decode_noalloc(C.byref(q.MoeShape(2816, 704, 2112)), C.byref(lay), 0x50008, q.MOE_BF16,
                                        None, 0x60000, 0x70000, 0x80000, 0x90000, None, None) == q.MOE_ERR_INVALID_ARG
