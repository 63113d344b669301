"""Non-finite activations through the block (a stack without norms overflows to
inf/NaN, so the path must stay well defined there): a NaN router logit ranks
below every number, ties by id, so every row still gets k distinct valid picks,
equal to the oracle's; rows holding non-finite values do not disturb other rows;
nothing is flagged and nothing is read out of bounds."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _harness import REL_TOL, check_topk, device, empty_f32, empty_i32, get_layer, rel_err, to_dev_x, workspace

pytestmark = pytest.mark.gpu
q = pytest.importorskip("quantized_mixture_experts_bit_amd")


def poison(x, rows):
    """bf16 rows: rows[0] gets one NaN, rows[1] one +inf and one -inf (bits)."""
    x = x.copy()
    x[rows[0], 5] = 0x7FC0
    x[rows[1], 7] = 0x7F80
    x[rows[1], 300] = 0xFF80
    return x


@pytest.mark.parametrize("shape", [synth.TINY, synth.GEMMA4], ids=["tiny", "gemma4"])
def test_decode_nonfinite_row_picks_valid(shape):
    L, ol, dl = get_layer(shape)
    k, d = shape.top_k, shape.d_model
    x = poison(synth.make_x(shape, 2, seed=51, dtype="bf16"), (0, 1))
    ws = workspace(shape, 1)
    for r in range(2):
        idx, w, eo, y = empty_i32(k), empty_f32(k), empty_f32(k, d), empty_f32(d)
        q.moe_layer_decode(shape, dl.c, to_dev_x(x[r:r + 1]), None, idx, w, eo, y, None, ws)
        torch.cuda.synchronize()
        ref = O.moe_rows(ol, x[r:r + 1], want=("logits", "idx", "p", "gap"))
        got = idx.cpu().numpy()
        np.testing.assert_array_equal(got, ref["idx"][0])
        assert len(set(got.tolist())) == k and got.min() >= 0 and got.max() < shape.n_experts
    assert q.moe_check_device_error() == 0
    # a finite row after the poisoned ones is unaffected
    xf = synth.make_x(shape, 1, seed=52, dtype="bf16")
    idx, w, eo, y = empty_i32(k), empty_f32(k), empty_f32(k, d), empty_f32(d)
    q.moe_layer_decode(shape, dl.c, to_dev_x(xf), None, idx, w, eo, y, None, ws)
    torch.cuda.synchronize()
    ref = O.moe_rows(ol, xf)
    check_topk(idx.cpu().numpy()[None], ref, k)
    assert rel_err(y.cpu().numpy(), ref["y"][0]) <= REL_TOL


def test_prefill_nonfinite_rows_isolated():
    shape = synth.GEMMA4
    L, ol, dl = get_layer(shape)
    rows, k, d, E = 48, shape.top_k, shape.d_model, shape.n_experts
    bad = (3, 40)
    x = poison(synth.make_x(shape, rows, seed=53, dtype="bf16"), bad)
    ws = workspace(shape, rows)
    out = dict(idx=empty_i32(rows, k), w=empty_f32(rows, k), cnt=empty_i32(E), off=empty_i32(E + 1),
               perm=empty_i32(rows * k), inv=empty_i32(rows * k), eo=empty_f32(rows * k, d), y=empty_f32(rows, d))
    q.moe_layer_prefill(shape, dl.c, to_dev_x(x), rows, None, out["idx"], out["w"], out["cnt"], out["off"],
                        out["perm"], out["inv"], out["eo"], out["y"], None, ws)
    torch.cuda.synchronize()
    assert q.moe_check_device_error() == 0
    got = {n: t.cpu().numpy() for n, t in out.items()}
    assert got["cnt"].sum() == rows * k  # every pair grouped
    sel = np.array([0, 3, 17, 40, 47])
    ref = O.moe_rows(ol, x[sel])
    for i, r in enumerate(sel):
        np.testing.assert_array_equal(got["idx"][r], ref["idx"][i])
        if r in bad:
            continue
        assert rel_err(got["y"][r], ref["y"][i]) <= REL_TOL, "row %d" % r
