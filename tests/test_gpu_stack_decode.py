"""moe_stack_decode on small stacks against moe_layer_decode called once per layer
(the same bits), with per-layer logit offsets, on a shape the one-launch kernel takes
and on one it does not (layer by layer inside the call), and against the oracle
teacher-forced on the soft-router tiny stack."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _harness import BEYOND_FF, REL_TOL, check_topk, device, empty_f32, empty_i32, rel_err, to_dev_x, workspace

pytestmark = pytest.mark.gpu
q = pytest.importorskip("quantized_mixture_experts_bit_amd")


def bits16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_both(shape, n_layers, variant, zipf, dtype_seed=7):
    from quantized_mixture_experts_bit_amd.weights import upload_layers
    canon = [synth.make_layer(shape, seed=3, layer=l, variant=variant) for l in range(n_layers)]
    dls = upload_layers(shape, canon, device())
    k, d = shape.top_k, shape.d_model
    offs = None
    if zipf:
        sig = synth.router_logit_std(shape) * 2.0 ** variant.router_scale_log2
        offs = [torch.from_numpy(synth.make_zipf_offset(shape, seed=0, layer=l, sigma=sig)).to(device())
                for l in range(n_layers)]
    x0 = to_dev_x(synth.make_x(shape, 1, seed=dtype_seed, dtype="bf16"))
    ws = workspace(shape, 1)
    # reference: one moe_layer_decode per layer, residual in place
    h = x0.clone()
    ref = []
    for l in range(n_layers):
        idx, w, eo, y = empty_i32(k), empty_f32(k), empty_f32(k, d), empty_f32(d)
        xin = bits16(h)
        q.moe_layer_decode(shape, dls[l].c, h, offs[l] if offs else None, idx, w, eo, y, h, ws)
        torch.cuda.synchronize()
        ref.append(dict(x=xin, idx=idx.cpu().numpy(), w=w.cpu().numpy(), eo=eo.cpu().numpy(), y=y.cpu().numpy()))
    final = bits16(h)
    # the stack in one call
    x = x0.clone()
    idx, w = empty_i32(n_layers, k), empty_f32(n_layers, k)
    eo, y = empty_f32(n_layers, k, d), empty_f32(n_layers, d)
    xl = torch.empty(n_layers, d, dtype=torch.bfloat16, device=device())
    q.moe_stack_decode(shape, [dl.c for dl in dls], x, offs, idx, w, eo, y, xl, ws)
    torch.cuda.synchronize()
    assert q.moe_check_device_error() == 0
    got = dict(x=bits16(xl), idx=idx.cpu().numpy(), w=w.cpu().numpy(), eo=eo.cpu().numpy(), y=y.cpu().numpy())
    return canon, offs, ref, final, got, bits16(x)


@pytest.mark.parametrize("shape,n_layers,variant,zipf", [
    pytest.param(synth.TINY, 5, synth.LIVE_STACK, True, id="tiny-5layers-live-zipf"),
    pytest.param(synth.GEMMA4, 3, synth.Variant(router_scale_log2=-6), False, id="gemma4-3layers-soft"),
    pytest.param(BEYOND_FF, 3, synth.Variant(router_scale_log2=-6), True, id="dff832-3layers-layer-by-layer"),
    # the most layers one launch takes, on the tiny shape
    pytest.param(synth.TINY, 32, synth.LIVE_STACK, True, id="tiny-32layers-live-zipf"),
    # 256 experts, top-16 (the rankers' other share split), and 64 experts
    pytest.param(synth.MoeShape(512, 256, 512, n_experts=256, top_k=16), 3, synth.LIVE_STACK, True,
                 id="e256-k16-3layers"),
    pytest.param(synth.MoeShape(1024, 512, 1024, n_experts=64, top_k=4), 4, synth.LIVE_STACK, False,
                 id="e64-k4-4layers"),
    # more than one launch takes: layer by layer inside the call
    pytest.param(synth.TINY, 33, synth.LIVE_STACK, False, id="tiny-33layers-layer-by-layer"),
])
def test_stack_decode_matches_layer_calls(shape, n_layers, variant, zipf):
    canon, offs, ref, final, got, x_out = run_both(shape, n_layers, variant, zipf)
    for l in range(n_layers):
        assert np.array_equal(got["x"][l], ref[l]["x"][0]), "layer %d input" % l
        assert np.array_equal(got["idx"][l], ref[l]["idx"]), "layer %d picks" % l
        for n in ("w", "eo", "y"):
            assert np.array_equal(got[n][l].view(np.uint32), ref[l][n].view(np.uint32)), "layer %d %s" % (l, n)
    assert np.array_equal(x_out, final)


def test_stack_decode_teacher_forced_tiny():
    """Every layer of a 5-layer tiny live stack (per-layer Zipf offsets) against the oracle
    on the stack's own inputs: picks, weights, unweighted expert outputs, y."""
    shape, n_layers = synth.TINY, 5
    canon, offs, ref, final, got, x_out = run_both(shape, n_layers, synth.LIVE_STACK, True)
    k = shape.top_k
    for l in range(n_layers):
        ol = O.OracleLayer(canon[l])
        off_np = offs[l].cpu().numpy()
        xin = got["x"][l][None]
        r = O.moe_rows(ol, xin, offset=off_np)
        if check_topk(got["idx"][l][None], r, k)[0]:
            r = O.moe_rows(ol, xin, offset=off_np, idx=got["idx"][l][None])
        assert rel_err(got["y"][l], r["y"][0]) <= REL_TOL, "layer %d" % l
        for j in range(k):
            assert rel_err(got["eo"][l][j], r["expert_out"][0, j]) <= REL_TOL, "layer %d slot %d" % (l, j)
        np.testing.assert_allclose(got["w"][l], r["p"][0], rtol=0, atol=1e-6)
        assert np.abs(got["y"][l]).max() > 0.0


def test_stack_decode_rejects_bad_arguments():
    shape = synth.TINY
    ws = workspace(shape, 1)
    x = torch.zeros(1, shape.d_model, dtype=torch.bfloat16, device=device())
    k = shape.top_k
    with pytest.raises(q.MoeError):
        q.moe_stack_decode(shape, [q.moe_layer(0, 0, 0, 0, 0, 0)], x, None, empty_i32(1, k), empty_f32(1, k), None,
                           None, None, ws)
    # no layers: nothing to do
    q.moe_stack_decode(shape, [], x, None, empty_i32(1, k), empty_f32(1, k), None, None, None, ws)
