"""GPU parity of the decode path (one activation row) against the fp64 oracle,
through the C ABI. Shapes: the tiny layer (d_model 512, fp32 x) and the
Gemma-4-like layer (d_model 2816, d_ff 704, shared 2112, bf16 x)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _harness import (BEYOND_D, BEYOND_FF, NARROW, REL_TOL, WIDE, check_topk, empty_f32, empty_i32, get_layer, rel_err, to_dev_x,
                      workspace, device)

pytestmark = pytest.mark.gpu
q = pytest.importorskip("quantized_mixture_experts_bit_amd")

SOFT = synth.Variant(router_scale_log2=-6)
CASES = [
    pytest.param(synth.TINY, "f32", synth.Variant(), id="tiny-f32"),
    pytest.param(synth.TINY, "f32", SOFT, id="tiny-f32-soft"),
    pytest.param(synth.TINY, "bf16", SOFT, id="tiny-bf16-soft"),
    pytest.param(synth.GEMMA4, "bf16", synth.Variant(), id="gemma4-bf16"),
    pytest.param(synth.GEMMA4, "bf16", SOFT, id="gemma4-bf16-soft"),
    pytest.param(WIDE, "bf16", SOFT, id="wide256x16-bf16-soft"),
    pytest.param(NARROW, "f32", SOFT, id="narrow64x4-f32-soft"),
    pytest.param(BEYOND_FF, "f32", SOFT, id="three-launch-dff832-f32-soft"),
    pytest.param(BEYOND_D, "bf16", SOFT, id="three-launch-d3200-bf16-soft"),
]


@pytest.mark.parametrize("shape,dt,variant", CASES)
def test_router_topk(shape, dt, variant):
    L, ol, dl = get_layer(shape, variant=variant)
    rows = 16
    x = synth.make_x(shape, rows, seed=1, dtype=dt)
    ref = O.moe_rows(ol, x, want=("logits", "idx", "p", "gap"))
    ws = workspace(shape, rows)
    k = shape.top_k
    idx, w = empty_i32(rows, k), empty_f32(rows, k)
    logits = torch.empty(rows, shape.n_experts, dtype=torch.float64, device=device())
    q.moe_router_topk(shape, dl.c, to_dev_x(x), rows, None, idx, w, logits, ws)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    assert np.abs(lg - ref["logits"]).max() <= 1e-9 * max(1.0, np.abs(ref["logits"]).max())
    flagged = check_topk(idx.cpu().numpy(), ref, k)
    wn = w.cpu().numpy()
    ok = ~flagged
    np.testing.assert_allclose(wn[ok], ref["p"][ok], rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("shape,dt,variant", CASES)
def test_expert_ffn_decode_per_expert(shape, dt, variant):
    """Unweighted E_k(x) of every pick, so experts 2..k are checked even when the softmax is one-hot."""
    L, ol, dl = get_layer(shape, variant=variant)
    x = synth.make_x(shape, 1, seed=2, dtype=dt)
    ref = O.moe_rows(ol, x)
    ws = workspace(shape, 1)
    k, d = shape.top_k, shape.d_model
    idx = torch.from_numpy(ref["idx"].astype(np.int32)).to(device())
    eo = empty_f32(k, d)
    q.moe_expert_ffn_decode(shape, dl.c, to_dev_x(x), idx, eo, ws)
    torch.cuda.synchronize()
    got = eo.cpu().numpy()
    for j in range(k):
        e = rel_err(got[j], ref["expert_out"][0, j])
        assert e <= REL_TOL, "slot %d expert %d: %g" % (j, ref["idx"][0, j], e)


@pytest.mark.parametrize("shape,dt,variant", CASES)
def test_combine_decode(shape, dt, variant):
    """Shared expert + weighted sum, fed with the oracle's expert outputs and weights."""
    L, ol, dl = get_layer(shape, variant=variant)
    x = synth.make_x(shape, 1, seed=3, dtype=dt)
    ref = O.moe_rows(ol, x)
    ws = workspace(shape, 1)
    k, d = shape.top_k, shape.d_model
    eo = torch.from_numpy(ref["expert_out"][0].astype(np.float32)).to(device())
    w = torch.from_numpy(ref["p"][0].astype(np.float32)).to(device())
    y = empty_f32(1, d)
    q.moe_combine(shape, dl.c, to_dev_x(x), 1, eo, None, w, y, None, ws)
    torch.cuda.synchronize()
    assert rel_err(y.cpu().numpy()[0], ref["y"][0]) <= REL_TOL


def run_layer_decode(shape, dl, x, ws, residual=None, offset=None):
    k, d = shape.top_k, shape.d_model
    idx, w, eo, y = empty_i32(k), empty_f32(k), empty_f32(k, d), empty_f32(d)
    q.moe_layer_decode(shape, dl.c, to_dev_x(x), offset, idx, w, eo, y, residual, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy(), eo.cpu().numpy(), y.cpu().numpy()


@pytest.mark.parametrize("shape,dt,variant", CASES)
def test_layer_decode(shape, dt, variant):
    L, ol, dl = get_layer(shape, variant=variant)
    ws = workspace(shape, 1)
    for stream in range(4):
        x = synth.make_x(shape, 1, seed=4, stream=stream, dtype=dt)
        ref = O.moe_rows(ol, x)
        idx, w, eo, y = run_layer_decode(shape, dl, x, ws)
        flagged = check_topk(idx, ref, shape.top_k)
        if flagged[0]:
            ref = O.moe_rows(ol, x, idx=idx.reshape(1, -1))  # conditional oracle on the GPU's picks
        assert rel_err(y, ref["y"][0]) <= REL_TOL
        for j in range(shape.top_k):
            assert rel_err(eo[j], ref["expert_out"][0, j]) <= REL_TOL
    assert q.moe_check_device_error() == 0


@pytest.mark.parametrize("log2_scale,dt", [(6, "f32"), (6, "bf16"), (-10, "f32")],
                         ids=["x-times-64-f32", "x-times-64-bf16", "x-over-1024-f32"])
def test_layer_decode_far_from_unit_scale(log2_scale, dt):
    """Activations scaled by a power of two: with x * 64 the GeGLU output h passes the
    fp16 range, with x / 1024 it sits far below 1; the down GEMV scales h by a power of
    two of its own, so y still meets the tolerance against the oracle."""
    shape = synth.GEMMA4
    L, ol, dl = get_layer(shape)
    ws = workspace(shape, 1)
    xf = synth.make_x(shape, 1, seed=9, dtype="f32") * np.float32(2.0 ** log2_scale)
    x = xf if dt == "f32" else synth.f32_to_bf16_bits(xf)
    ref = O.moe_rows(ol, x)
    # the premise, from the oracle: the first pick's h = gelu(gate x) * (up x)
    e0 = L.experts[int(ref["idx"][0, 0])]
    xr = O.x_to_f64(x)[0]
    h = np.array([O.gelu_tanh(g) for g in O.matvec(e0.gate, xr)]) * O.matvec(e0.up, xr)
    assert (np.abs(h).max() > 65504.0) if log2_scale > 0 else (np.abs(h).max() < 1.0)
    idx, w, eo, y = run_layer_decode(shape, dl, x, ws)
    if check_topk(idx, ref, shape.top_k)[0]:
        ref = O.moe_rows(ol, x, idx=idx.reshape(1, -1))
    assert rel_err(y, ref["y"][0]) <= REL_TOL
    for j in range(shape.top_k):
        assert rel_err(eo[j], ref["expert_out"][0, j]) <= REL_TOL
    assert q.moe_check_device_error() == 0


def test_layer_decode_onehot_is_one_dense_ffn():
    shape = synth.TINY
    L, ol, dl = get_layer(shape, variant=synth.Variant(shared_zero=True))
    x = synth.make_x(shape, 1, seed=5, dtype="f32")
    off = synth.onehot_offset(shape, 17)
    ref = O.moe_rows(ol, x, offset=off)
    ws = workspace(shape, 1)
    idx, w, eo, y = run_layer_decode(shape, dl, x, ws, offset=torch.from_numpy(off).to(device()))
    assert idx[0] == 17 and w[0] == 1.0 and np.all(w[1:] == 0.0)
    assert rel_err(y, ref["y"][0]) <= REL_TOL


def test_layer_decode_deterministic():
    shape = synth.GEMMA4
    L, ol, dl = get_layer(shape)
    ws = workspace(shape, 1)
    x = synth.make_x(shape, 1, seed=6, dtype="bf16")
    a = run_layer_decode(shape, dl, x, ws)
    b = run_layer_decode(shape, dl, x, ws)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_slot_table_placement_does_not_change_results():
    """Experts placed at permuted pool positions (and the table permuted to match): bit-identical."""
    from quantized_mixture_experts_bit_amd.weights import ExpertPool
    shape = synth.TINY
    L, ol, dl = get_layer(shape)
    perm = np.random.default_rng(7).permutation(shape.n_experts)
    pool = ExpertPool(shape, shape.n_experts + 5, device())
    dl2 = pool.add_layer(L, 5, placement=perm)
    ws = workspace(shape, 1)
    x = synth.make_x(shape, 1, seed=7, dtype="f32")
    a = run_layer_decode(shape, dl, x, ws)
    b = run_layer_decode(shape, dl2, x, ws)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_residual_add_is_bf16_rne_of_fp32_sum():
    shape = synth.TINY
    L, ol, dl = get_layer(shape)
    ws = workspace(shape, 1)
    x = synth.make_x(shape, 1, seed=8, dtype="bf16")
    res = to_dev_x(x).clone()
    idx, w, eo, y = run_layer_decode(shape, dl, x, ws, residual=res.view(torch.int16).view(torch.bfloat16))
    got = res.view(torch.int16).cpu().numpy().view(np.uint16)
    want = O.residual_bf16(x[0], y)
    np.testing.assert_array_equal(got[0], want)


def test_bad_slot_entry_is_reported_not_followed():
    """A slot-table entry past the pool end: the kernels skip it and set the device error word."""
    shape = synth.TINY
    L, ol, dl = get_layer(shape)
    from quantized_mixture_experts_bit_amd.weights import DeviceLayer
    table = dl.slot_table.clone()
    table[:] = dl.pool.n_blobs + 3  # every expert out of range
    bad = DeviceLayer(dl.pool, dl.router, dl.shared, table)
    ws = workspace(shape, 1)
    x = synth.make_x(shape, 1, seed=9, dtype="f32")
    q.moe_check_device_error()
    idx, w, eo, y = run_layer_decode(shape, bad, x, ws)
    assert q.moe_check_device_error() & q.MOE_DEVERR_BAD_SLOT
    assert np.all(eo == 0.0)
    assert q.moe_check_device_error() == 0  # cleared by the read
