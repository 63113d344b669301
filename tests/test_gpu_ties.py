"""An exact tie at the top-k boundary: experts 3 and 10 get identical router rows,
so their logits are equal bit for bit on every path, and a logit offset puts seven
other experts far above them and the pair in 8th/9th place. The pick goes to the
lower id (3) and in rank order, as the oracle's (logit desc, id asc) order says."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import synth
from _harness import REL_TOL, device, empty_f32, empty_i32, rel_err, to_dev_x, workspace

pytestmark = pytest.mark.gpu
q = pytest.importorskip("quantized_mixture_experts_bit_amd")
from quantized_mixture_experts_bit_amd.weights import upload_layers  # noqa: E402

TOP7 = [0, 20, 30, 40, 50, 60, 70]


def tied_layer(shape):
    L = synth.make_layer(shape, seed=3, layer=0)
    r = L.router
    q8, s, b = r.q.copy(), r.s.copy(), r.b.copy()
    q8[3], s[3], b[3] = q8[10], s[10], b[10]
    L = dataclasses.replace(L, router=dataclasses.replace(r, q=q8, s=s, b=b))
    off = np.zeros(shape.n_experts, dtype=np.float32)
    off[TOP7] = 1.0e5
    off[[3, 10]] = 5.0e4
    return L, off


@pytest.fixture(scope="module")
def tied():
    shape = synth.GEMMA4
    L, off = tied_layer(shape)
    (dl,) = upload_layers(shape, [L], device())
    return shape, L, O.OracleLayer(L), dl, off


def test_oracle_breaks_the_tie_by_id(tied):
    shape, L, ol, dl, off = tied
    x = synth.make_x(shape, 3, seed=21, dtype="bf16")
    ref = O.moe_rows(ol, x, offset=off)
    assert np.all(ref["logits"][:, 3] == ref["logits"][:, 10])
    for r in range(3):
        assert set(ref["idx"][r][:7].tolist()) == set(TOP7) and ref["idx"][r][7] == 3


def test_decode_and_router_pick_the_lower_id(tied):
    shape, L, ol, dl, off = tied
    k, d = shape.top_k, shape.d_model
    offd = torch.from_numpy(off).to(device())
    ws = workspace(shape, 1)
    for r in range(3):
        x = synth.make_x(shape, 3, seed=21, dtype="bf16")[r:r + 1]
        ref = O.moe_rows(ol, x, offset=off)
        idx, w, eo, y = empty_i32(k), empty_f32(k), empty_f32(k, d), empty_f32(d)
        q.moe_layer_decode(shape, dl.c, to_dev_x(x), offd, idx, w, eo, y, None, ws)
        ri, rw, lg = empty_i32(1, k), empty_f32(1, k), torch.empty(1, shape.n_experts, dtype=torch.float64,
                                                                   device=device())
        q.moe_router_topk(shape, dl.c, to_dev_x(x), 1, offd, ri, rw, lg, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"][0])
        np.testing.assert_array_equal(ri.cpu().numpy()[0], ref["idx"][0])
        lgh = lg.cpu().numpy()[0]
        assert lgh[3] == lgh[10]
        assert rel_err(y.cpu().numpy(), ref["y"][0]) <= REL_TOL
    assert q.moe_check_device_error() == 0


def test_prefill_picks_the_lower_id(tied):
    shape, L, ol, dl, off = tied
    rows, k, d, E = 20, shape.top_k, shape.d_model, shape.n_experts
    x = synth.make_x(shape, rows, seed=22, dtype="bf16")
    ref = O.moe_rows(ol, x, offset=off)
    ws = workspace(shape, rows)
    out = dict(idx=empty_i32(rows, k), w=empty_f32(rows, k), cnt=empty_i32(E), off=empty_i32(E + 1),
               perm=empty_i32(rows * k), inv=empty_i32(rows * k), eo=empty_f32(rows * k, d), y=empty_f32(rows, d))
    q.moe_layer_prefill(shape, dl.c, to_dev_x(x), rows, torch.from_numpy(off).to(device()), out["idx"], out["w"],
                        out["cnt"], out["off"], out["perm"], out["inv"], out["eo"], out["y"], None, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["idx"].cpu().numpy(), ref["idx"])
    y = out["y"].cpu().numpy()
    for r in range(0, rows, 5):
        assert rel_err(y[r], ref["y"][r]) <= REL_TOL
    assert q.moe_check_device_error() == 0
