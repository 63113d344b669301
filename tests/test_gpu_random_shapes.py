"""A seeded sweep of shapes the library accepts, drawn at random (d_model, d_ff and
d_ff_shared multiples of 64 within the limits, 64/128/256 experts, top-k 1..16, bf16
and fp32 activations): the whole-block decode (moe_layer_decode, one launch where the
shape fits the fused tiling, three launches otherwise) and the whole-layer prefill
(moe_layer_prefill, a chunk of 1 to 80 rows, every row) against the fp64 oracle,
with the same bar as the fixed-shape tests."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _harness import REL_TOL, check_topk, device, empty_f32, empty_i32, get_layer, rel_err, to_dev_x, workspace

pytestmark = pytest.mark.gpu
q = pytest.importorskip("quantized_mixture_experts_bit_amd")

SOFT = synth.Variant(router_scale_log2=-6)


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.choice([64, 128, 256]))
    k = int(rng.integers(1, 17))
    d = 64 * int(rng.integers(2, 49))        # up to 3072
    f = 64 * int(rng.integers(1, 15))        # up to 896 (past the fused tiling's 768)
    fs = 64 * int(rng.integers(1, 45))       # up to 2816 (past 2560)
    dt = "bf16" if rng.random() < 0.6 else "f32"
    rows = int(rng.integers(1, 81))
    return synth.MoeShape(d, f, fs, n_experts=E, top_k=k), dt, rows


CASES = [pytest.param(*draw(s), id="s%d" % s) for s in range(12)]


@pytest.mark.parametrize("shape,dt,rows", CASES)
def test_random_shape_layer_decode(shape, dt, rows):
    L, ol, dl = get_layer(shape, seed=7, variant=SOFT)
    print("shape", shape, dt, flush=True)
    ws = workspace(shape, 1)
    k, d = shape.top_k, shape.d_model
    for stream in range(2):
        x = synth.make_x(shape, 1, seed=21, stream=stream, dtype=dt)
        ref = O.moe_rows(ol, x)
        idx, w, eo, y = empty_i32(k), empty_f32(k), empty_f32(k, d), empty_f32(d)
        q.moe_layer_decode(shape, dl.c, to_dev_x(x), None, idx, w, eo, y, None, ws)
        torch.cuda.synchronize()
        idx, eo, y = idx.cpu().numpy(), eo.cpu().numpy(), y.cpu().numpy()
        if check_topk(idx, ref, k)[0]:
            ref = O.moe_rows(ol, x, idx=idx.reshape(1, -1))
        assert rel_err(y, ref["y"][0]) <= REL_TOL
        for j in range(k):
            assert rel_err(eo[j], ref["expert_out"][0, j]) <= REL_TOL, j
    assert q.moe_check_device_error() == 0


@pytest.mark.parametrize("shape,dt,rows", CASES)
def test_random_shape_layer_prefill(shape, dt, rows):
    L, ol, dl = get_layer(shape, seed=7, variant=SOFT)
    print("shape", shape, dt, "rows", rows, flush=True)
    k, d, E = shape.top_k, shape.d_model, shape.n_experts
    x = synth.make_x(shape, rows, seed=22, dtype=dt)
    ws = workspace(shape, rows)
    o = dict(idx=empty_i32(rows, k), w=empty_f32(rows, k), cnt=empty_i32(E), off=empty_i32(E + 1),
             perm=empty_i32(rows * k), inv=empty_i32(rows * k), eo=empty_f32(rows * k, d), y=empty_f32(rows, d))
    q.moe_layer_prefill(shape, dl.c, to_dev_x(x), rows, None, o["idx"], o["w"], o["cnt"], o["off"], o["perm"],
                        o["inv"], o["eo"], o["y"], None, ws)
    torch.cuda.synchronize()
    got = {n: t.cpu().numpy() for n, t in o.items()}
    rc, ro, rp, ri = O.group_by_expert(got["idx"], E)
    np.testing.assert_array_equal(got["cnt"], rc)
    np.testing.assert_array_equal(got["perm"], rp)
    ref = O.moe_rows(ol, x)
    flagged = check_topk(got["idx"], ref, k)
    if flagged.any():
        ref = O.moe_rows(ol, x, idx=got["idx"])
    for r in range(rows):
        assert rel_err(got["y"][r], ref["y"][r]) <= REL_TOL, "row %d" % r
        for j in range(k):
            e = rel_err(got["eo"][got["inv"][r * k + j]], ref["expert_out"][r, j])
            assert e <= REL_TOL, "row %d slot %d: %g" % (r, j, e)
    assert q.moe_check_device_error() == 0
