"""GPU parity of the prefill-chunk path (grouping + grouped MFMA GEMMs + combine)
against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _harness import (BEYOND_FF, NARROW, REL_TOL, WIDE, check_topk, device, empty_f32, empty_i32, get_layer, rel_err,
                      to_dev_x, workspace)

pytestmark = pytest.mark.gpu
q = pytest.importorskip("quantized_mixture_experts_bit_amd")


def zipf(shape):
    return synth.make_zipf_offset(shape, seed=0)


@pytest.mark.parametrize("rows,E,k", [(1, 128, 8), (8, 128, 8), (128, 128, 8), (256, 128, 8), (37, 64, 1),
                                      (200, 256, 16), (3, 64, 16), (1000, 64, 16), (4095, 128, 16)])
def test_grouping_bit_exact(rows, E, k):
    rng = np.random.default_rng(rows * 31 + E + k)
    skew = np.exp(-np.arange(E) / 8.0)
    idx = np.stack([rng.choice(E, size=k, replace=False, p=skew / skew.sum()) for _ in range(rows)]).astype(np.int32)
    shape = q.MoeShape(512, 256, 512, n_experts=E, top_k=k)
    cnt, off = empty_i32(E), empty_i32(E + 1)
    perm, inv = empty_i32(rows * k), empty_i32(rows * k)
    ws = torch.empty(q.moe_workspace_bytes(shape, rows), dtype=torch.uint8, device=device())
    q.moe_group_by_expert(shape, torch.from_numpy(idx).to(device()), rows, cnt, off, perm, inv, ws)
    torch.cuda.synchronize()
    rc, ro, rp, ri = O.group_by_expert(idx, E)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(off.cpu().numpy(), ro)
    np.testing.assert_array_equal(perm.cpu().numpy(), rp)
    np.testing.assert_array_equal(inv.cpu().numpy(), ri)


@pytest.mark.parametrize("rows,E,k", [(40, 128, 8), (600, 64, 8)])
def test_grouping_drops_invalid_ids(rows, E, k):
    """Ids outside [0, E) are reported and their pairs left out: the valid pairs sort as
    the oracle sorts them alone, an invalid pair's inv_perm is -1."""
    rng = np.random.default_rng(rows + E)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(rows)]).astype(np.int32)
    bad = rng.random(idx.shape) < 0.04
    idx[bad] = rng.choice([-1, -100, E, E + 7], size=int(bad.sum()))
    shape = q.MoeShape(512, 256, 512, n_experts=E, top_k=k)
    cnt, off = empty_i32(E), empty_i32(E + 1)
    perm, inv = empty_i32(rows * k), empty_i32(rows * k)
    ws = torch.empty(q.moe_workspace_bytes(shape, rows), dtype=torch.uint8, device=device())
    q.moe_group_by_expert(shape, torch.from_numpy(idx).to(device()), rows, cnt, off, perm, inv, ws)
    assert q.moe_check_device_error() & q.MOE_DEVERR_BAD_EXPERT_ID
    flat = idx.reshape(-1)
    valid = np.flatnonzero(~bad.reshape(-1))
    rc, ro, rp, ri = O.group_by_expert(flat[valid].reshape(-1, 1), E)  # the valid pairs as rows of one pick
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(off.cpu().numpy(), ro)
    np.testing.assert_array_equal(perm.cpu().numpy()[:valid.size], valid[rp])
    want_inv = np.full(rows * k, -1, dtype=np.int32)
    want_inv[valid] = ri
    np.testing.assert_array_equal(inv.cpu().numpy(), want_inv)
    assert q.moe_check_device_error() == 0


def run_layer_prefill(shape, dl, x, ws, offset=None, residual=None):
    rows = x.shape[0]
    k, d, E = shape.top_k, shape.d_model, shape.n_experts
    out = dict(idx=empty_i32(rows, k), w=empty_f32(rows, k), cnt=empty_i32(E), off=empty_i32(E + 1),
               perm=empty_i32(rows * k), inv=empty_i32(rows * k), eo=empty_f32(rows * k, d), y=empty_f32(rows, d))
    q.moe_layer_prefill(shape, dl.c, to_dev_x(x), rows, offset, out["idx"], out["w"], out["cnt"], out["off"],
                        out["perm"], out["inv"], out["eo"], out["y"], residual, ws)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in out.items()}


PREFILL_CASES = [
    pytest.param(synth.TINY, 8, "f32", None, None, id="tiny-8rows-f32"),
    pytest.param(synth.TINY, 8, "f32", synth.Variant(router_scale_log2=-6), None, id="tiny-8rows-f32-soft"),
    pytest.param(synth.TINY, 65, "bf16", synth.Variant(router_scale_log2=-6), None, id="tiny-65rows-bf16-soft"),
    pytest.param(synth.TINY, 130, "bf16", None, "zipf", id="tiny-130rows-bf16-zipf"),
    pytest.param(synth.GEMMA4, 128, "bf16", None, "zipf", id="gemma4-128rows-bf16-zipf"),
    pytest.param(synth.GEMMA4, 256, "bf16", None, "zipf", id="gemma4-256rows-bf16-zipf"),
    pytest.param(synth.GEMMA4, 19, "bf16", synth.Variant(router_scale_log2=-6), None, id="gemma4-19rows-soft"),
    pytest.param(synth.GEMMA4, 64, "f32", None, "zipf", id="gemma4-64rows-f32-zipf"),
    pytest.param(WIDE, 40, "bf16", synth.Variant(router_scale_log2=-6), None, id="wide256x16-40rows-soft"),
    pytest.param(NARROW, 33, "f32", synth.Variant(router_scale_log2=-6), None, id="narrow64x4-33rows-f32-soft"),
    pytest.param(BEYOND_FF, 21, "f32", synth.Variant(router_scale_log2=-6), None, id="dff832-21rows-f32-soft"),
    # the most rows a call takes (rows * top_k < 65536): every expert gets many 64-row tiles
    pytest.param(synth.GEMMA4, 65535 // 8, "bf16", None, None, id="gemma4-8191rows-max"),
]


def sample_rows(rows, n=24):
    """Every row of chunks up to 256 rows (the workload chunks are compared in full);
    the first, the last and n - 2 drawn rows of larger chunks."""
    if rows <= 256:
        return np.arange(rows)
    return np.unique(np.concatenate([[0, rows - 1], np.random.default_rng(rows).choice(rows, n - 2, replace=False)]))


@pytest.mark.parametrize("shape,rows,dt,variant,skew", PREFILL_CASES)
def test_layer_prefill(shape, rows, dt, variant, skew):
    L, ol, dl = get_layer(shape, variant=variant or synth.Variant())
    x = synth.make_x(shape, rows, seed=11, dtype=dt)
    off_np = zipf(shape) if skew == "zipf" else None
    off = None if off_np is None else torch.from_numpy(off_np).to(device())
    ws = workspace(shape, rows)
    got = run_layer_prefill(shape, dl, x, ws, offset=off)
    k = shape.top_k
    # grouping of the GPU's own picks is exact
    rc, ro, rp, ri = O.group_by_expert(got["idx"], shape.n_experts)
    np.testing.assert_array_equal(got["perm"], rp)
    np.testing.assert_array_equal(got["inv"], ri)
    sel = sample_rows(rows)
    ref = O.moe_rows(ol, x[sel], offset=off_np)
    flagged = check_topk(got["idx"][sel], ref, k)
    if flagged.any():
        ref = O.moe_rows(ol, x[sel], offset=off_np, idx=got["idx"][sel])
    for i, r in enumerate(sel):
        assert rel_err(got["y"][r], ref["y"][i]) <= REL_TOL, "row %d" % r
        for j in range(k):
            pos = got["inv"][r * k + j]
            e = rel_err(got["eo"][pos], ref["expert_out"][i, j])
            assert e <= REL_TOL, "row %d slot %d expert %d: %g" % (r, j, got["idx"][r, j], e)
    assert q.moe_check_device_error() == 0
    if skew == "zipf" and shape is synth.GEMMA4:
        # the skew really makes experts repeat across rows
        assert (got["cnt"] > 0).sum() < 60 and got["cnt"].max() >= rows // 2


@pytest.mark.parametrize("log2_scale", [6, -10], ids=["x-times-64", "x-over-1024"])
def test_layer_prefill_far_from_unit_scale(log2_scale):
    """Rows scaled by powers of two (H past the fp16 range, or far below 1), each row by
    a different power within a factor of 8 of the next: the per-row H scale keeps every
    row within the tolerance of the oracle."""
    shape = synth.GEMMA4
    L, ol, dl = get_layer(shape)
    rows = 24
    row_scale = np.float32(2.0) ** (log2_scale + np.arange(rows) % 4 - 2).astype(np.float32)
    x = synth.make_x(shape, rows, seed=13, dtype="f32") * row_scale[:, None]
    ws = workspace(shape, rows)
    got = run_layer_prefill(shape, dl, x, ws)
    sel = np.arange(rows)
    ref = O.moe_rows(ol, x[sel])
    if check_topk(got["idx"][sel], ref, shape.top_k).any():
        ref = O.moe_rows(ol, x[sel], idx=got["idx"][sel])
    for i, r in enumerate(sel):
        assert rel_err(got["y"][r], ref["y"][i]) <= REL_TOL, "row %d" % r
    assert q.moe_check_device_error() == 0


def test_prefill_chunk_split_calls_match_fused():
    shape = synth.GEMMA4
    L, ol, dl = get_layer(shape)
    rows, k, d, E = 40, shape.top_k, shape.d_model, shape.n_experts
    x = synth.make_x(shape, rows, seed=12, dtype="bf16")
    xd = to_dev_x(x)
    ws = workspace(shape, rows)
    fused = run_layer_prefill(shape, dl, x, ws)
    idx, w = empty_i32(rows, k), empty_f32(rows, k)
    q.moe_router_topk(shape, dl.c, xd, rows, None, idx, w, None, ws)
    cnt, off, perm, inv = empty_i32(E), empty_i32(E + 1), empty_i32(rows * k), empty_i32(rows * k)
    q.moe_group_by_expert(shape, idx, rows, cnt, off, perm, inv, ws)
    eo, y = empty_f32(rows * k, d), empty_f32(rows, d)
    q.moe_expert_ffn_prefill_chunk(shape, dl.c, xd, rows, off, perm, eo, ws)
    q.moe_combine(shape, dl.c, xd, rows, eo, inv, w, y, None, ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), fused["idx"])
    assert np.array_equal(eo.cpu().numpy(), fused["eo"])
    assert np.array_equal(y.cpu().numpy(), fused["y"])


def test_prefill_rows_match_decode():
    """Row r of a prefill chunk and a decode call on x_r agree within the tolerance."""
    shape = synth.GEMMA4
    L, ol, dl = get_layer(shape)
    rows = 24
    x = synth.make_x(shape, rows, seed=13, dtype="bf16")
    ws = workspace(shape, rows)
    got = run_layer_prefill(shape, dl, x, ws)
    k, d = shape.top_k, shape.d_model
    for r in (0, 7, 23):
        idx, w, eo, y = empty_i32(k), empty_f32(k), empty_f32(k, d), empty_f32(d)
        q.moe_layer_decode(shape, dl.c, to_dev_x(x[r:r + 1]), None, idx, w, eo, y, None, ws)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), got["idx"][r])
        assert rel_err(got["y"][r], y.cpu().numpy()) <= REL_TOL


def test_empty_chunk_is_a_no_op():
    shape = synth.TINY
    L, ol, dl = get_layer(shape)
    ws = workspace(shape, 1)
    x = torch.zeros(1, shape.d_model, dtype=torch.bfloat16, device=device())
    y = torch.full((1, shape.d_model), 7.0, device=device())
    k, E = shape.top_k, shape.n_experts
    q.moe_layer_prefill(shape, dl.c, x, 0, None, empty_i32(1, k), empty_f32(1, k), empty_i32(E), empty_i32(E + 1),
                        empty_i32(k), empty_i32(k), empty_f32(k, shape.d_model), y, None, ws)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


def test_prefill_deterministic():
    shape = synth.GEMMA4
    L, ol, dl = get_layer(shape)
    x = synth.make_x(shape, 128, seed=14, dtype="bf16")
    off = torch.from_numpy(zipf(shape)).to(device())
    ws = workspace(shape, 128)
    a = run_layer_prefill(shape, dl, x, ws, offset=off)
    b = run_layer_prefill(shape, dl, x, ws, offset=off)
    for n in a:
        assert np.array_equal(a[n].view(np.uint8), b[n].view(np.uint8)), n
