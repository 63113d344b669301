"""Pins of the fp64 oracle against facts that do not come from the oracle itself:
hand-computed dequantisation bytes, hand-worked top-k cases, closed forms,
invariants, brute force on tiny inputs, and special cases that reduce to
library routines (numpy float64 matmul and sort, torch's tanh-GELU and bf16
rounding). All CPU-only."""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth import MoeShape

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SMALL = MoeShape(d_model=128, d_ff=64, d_ff_shared=128, n_experts=16, top_k=4)


def bf16_f64(h):
    return synth.bf16_bits_to_f32(h).astype(np.float64)


def np_dequant(m):
    """Dense fp64 matrix from the canonical arrays, written with numpy slicing."""
    if m.bits == 4:
        codes = np.empty((m.rows, m.cols), dtype=np.float64)
        codes[:, 0::2] = m.q & 0x0F
        codes[:, 1::2] = m.q >> 4
    else:
        codes = m.q.astype(np.float64)
    s = np.repeat(bf16_f64(m.s), 64, axis=1)
    b = np.repeat(bf16_f64(m.b), 64, axis=1)
    return s * codes + b


def torch_gelu_tanh(z):
    return torch.nn.functional.gelu(torch.from_numpy(np.asarray(z, dtype=np.float64)), approximate="tanh").numpy()


def dense_ffn(expert, x64):
    """Dense GeGLU FFN with library routines: numpy float64 matmul + torch tanh-GELU."""
    g = x64 @ np_dequant(expert.gate).T
    u = x64 @ np_dequant(expert.up).T
    return (torch_gelu_tanh(g) * u) @ np_dequant(expert.down).T


def one_group_mat(bits, s_bits, b_bits, byte, cols=64):
    rows = 1
    q = np.full((rows, cols // 2 if bits == 4 else cols), byte, dtype=np.uint8)
    s = np.full((rows, cols // 64), s_bits, dtype=np.uint16)
    b = np.full((rows, cols // 64), b_bits, dtype=np.uint16)
    return synth.QMat(q, s, b, bits)


# ---------------------------------------------------------------- dequantisation

def load_dequant_golden():
    rows = []
    with open(os.path.join(GOLDEN, "dequant_examples.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                bits, s, b, byte, elem, w = line.split()
                rows.append((int(bits), int(s, 16), int(b, 16), int(byte, 16), int(elem), float(w)))
    return rows


@pytest.mark.parametrize("case", load_dequant_golden())
def test_dequant_hand_computed(case):
    bits, s, b, byte, elem, w = case
    m = one_group_mat(bits, s, b, byte)
    assert O.weight(m, 0, elem) == w
    # the same byte repeated: every even (odd) element decodes alike
    assert O.weight(m, 0, elem + 2 * 7) == w


def test_dequant_constant_code_closed_form():
    rng = np.random.default_rng(1)
    for bits, cmax in ((4, 15), (8, 255)):
        for c in (0, 1, cmax // 2, cmax):
            m = synth.draw_qmat(rng, 8, 256, bits)
            byte = (c | (c << 4)) if bits == 4 else c
            m.q[...] = byte
            W = O.dequant(m)
            want = np.repeat(bf16_f64(m.s) * c + bf16_f64(m.b), 64, axis=1)
            np.testing.assert_array_equal(W, want)


def test_dequant_groups_and_rows_at_scale():
    """Group index i/64 and row strides: matches the numpy-sliced decode exactly."""
    rng = np.random.default_rng(2)
    for bits in (4, 8):
        m = synth.draw_qmat(rng, 40, 512, bits)
        np.testing.assert_array_equal(O.dequant(m), np_dequant(m))


def test_dequant_group_boundary():
    """Element 63 takes group 0's (s, b); element 64 takes group 1's."""
    q = np.full((1, 64), 0x55, dtype=np.uint8)  # every code 5
    s = np.array([[0x3F80, 0x4000]], dtype=np.uint16)  # 1.0, 2.0
    b = np.array([[0x0000, 0x3F80]], dtype=np.uint16)  # 0.0, 1.0
    m = synth.QMat(q, s, b, 4)
    assert O.weight(m, 0, 63) == 5.0
    assert O.weight(m, 0, 64) == 11.0


# ---------------------------------------------------------------- router GEMV

def test_matvec_basis_vector_returns_column():
    rng = np.random.default_rng(3)
    m = synth.draw_qmat(rng, 16, 256, 8)
    W = np_dequant(m)
    for i in (0, 1, 63, 64, 255):
        e = np.zeros(256)
        e[i] = 1.0
        np.testing.assert_array_equal(O.matvec(m, e), W[:, i])


def test_matvec_constant_weights_closed_form():
    rng = np.random.default_rng(4)
    m = synth.draw_qmat(rng, 4, 192, 8)
    m.q[...] = 17
    m.s[...] = 0x3C80  # 2^-6
    m.b[...] = 0xBD80  # -2^-4
    x = rng.standard_normal(192)
    got = O.matvec(m, x)
    want = (17 * 2.0 ** -6 - 2.0 ** -4) * x.sum()
    np.testing.assert_allclose(got, want, rtol=1e-13)


def test_router_logits_match_numpy_matmul():
    rng = np.random.default_rng(5)
    layer = synth.make_layer(SMALL, seed=3)
    x = synth.make_x(SMALL, 5, seed=3)
    off = rng.standard_normal(SMALL.n_experts).astype(np.float32)
    got = O.router_logits(layer, x, off)
    want = O.x_to_f64(x) @ np_dequant(layer.router).T + off.astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- top-k + softmax

def load_topk_golden():
    out = []
    with open(os.path.join(GOLDEN, "topk_examples.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                lg, idx, gap = [t.strip() for t in line.split(";")]
                out.append(([float(v) for v in lg.split(",")], [int(v) for v in idx.split(",")], float(gap)))
    return out


@pytest.mark.parametrize("case", load_topk_golden())
def test_topk_hand_worked(case):
    logits, want_idx, want_gap = case
    idx, p, gap = O.topk_softmax(np.array(logits), 4)
    assert list(idx) == want_idx
    assert gap == want_gap


def test_topk_brute_force_against_library_sort():
    rng = np.random.default_rng(6)
    for trial in range(200):
        E, k = 128, 8
        lg = rng.standard_normal(E) * 50
        if trial % 4 == 0:  # planted ties
            lg[rng.integers(0, E, 20)] = lg[0]
        order = np.lexsort((np.arange(E), -lg))  # primary: -logit, secondary: id
        idx, p, gap = O.topk_softmax(lg, k)
        np.testing.assert_array_equal(idx, order[:k])
        assert gap == lg[order[k - 1]] - lg[order[k]]


def test_topk_nan_logits_rank_last():
    """A NaN logit ranks below every number, ties by id (the reading for non-finite
    activations): brute force against a library sort with NaN replaced by -inf."""
    rng = np.random.default_rng(9)
    for trial in range(100):
        E, k = 64, 8
        lg = rng.standard_normal(E) * 10
        lg[rng.integers(0, E, trial % 70)] = np.nan
        if trial % 5 == 0:
            lg[rng.integers(0, E, 4)] = -np.inf
        key = np.where(np.isnan(lg), -np.inf, lg)
        order = np.lexsort((np.arange(E), -key))
        idx, p, gap = O.topk_softmax(lg, k)
        np.testing.assert_array_equal(idx, order[:k])
        assert len(set(idx.tolist())) == k
    idx, _, _ = O.topk_softmax(np.full(16, np.nan), 4)
    np.testing.assert_array_equal(idx, [0, 1, 2, 3])
    idx, _, _ = O.topk_softmax(np.array([np.nan, 1.0, np.nan, 3.0, -np.inf]), 3)
    np.testing.assert_array_equal(idx, [3, 1, 0])  # NaN at id 0 ties the -inf at id 4; lower id first


def test_topk_relabelling_permutes_selection():
    rng = np.random.default_rng(7)
    lg = rng.standard_normal(128)
    perm = rng.permutation(128)
    idx, _, _ = O.topk_softmax(lg, 8)
    lg2 = np.empty_like(lg)
    lg2[perm] = lg  # expert e is now called perm[e]
    idx2, _, _ = O.topk_softmax(lg2, 8)
    np.testing.assert_array_equal(idx2, perm[idx])


def test_softmax_properties_and_library():
    import scipy.special
    rng = np.random.default_rng(8)
    for _ in range(100):
        lg = rng.standard_normal(128) * rng.choice([0.5, 5, 100])
        idx, p, _ = O.topk_softmax(lg, 8)
        assert abs(p.sum() - 1.0) <= 8 * 2.0 ** -52
        assert np.all(np.diff(p) <= 0)
        np.testing.assert_allclose(p, scipy.special.softmax(lg[idx]), rtol=1e-14, atol=1e-300)
    idx, p, _ = O.topk_softmax(np.zeros(128), 8)
    np.testing.assert_array_equal(p, np.full(8, 0.125))


# ---------------------------------------------------------------- GeGLU expert

def test_gelu_tanh_matches_torch():
    z = np.concatenate([np.linspace(-12, 12, 2001), [0.0, -50.0, 50.0, 1e-8, -1e-8]])
    got = np.array([O.gelu_tanh(v) for v in z])
    np.testing.assert_allclose(got, torch_gelu_tanh(z), rtol=1e-13, atol=1e-15)
    assert O.gelu_tanh(0.0) == 0.0


def test_expert_matches_dense_ffn():
    layer = synth.make_layer(SMALL, seed=9)
    x = synth.make_x(SMALL, 3, seed=9)
    for e in (0, 5, 15):
        got = O.expert_rows(layer.experts[e], x)
        want = dense_ffn(layer.experts[e], O.x_to_f64(x))
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-9 * np.abs(want).max())


def test_expert_zero_codes_zero_bias_is_zero():
    layer = synth.make_layer(SMALL, seed=10)
    ex = layer.experts[2]
    ex.gate.q[...] = 0
    ex.gate.b[...] = 0
    x = synth.make_x(SMALL, 2, seed=10)
    np.testing.assert_array_equal(O.expert_rows(ex, x), 0.0)


def test_gate_and_up_are_not_interchangeable():
    """GELU acts on the gate projection only: swapping gate and up changes the output."""
    layer = synth.make_layer(SMALL, seed=11)
    ex = layer.experts[1]
    x = synth.make_x(SMALL, 2, seed=11)
    swapped = synth.Expert(ex.up, ex.gate, ex.down)
    a, b = O.expert_rows(ex, x), O.expert_rows(swapped, x)
    assert np.abs(a - b).max() > 1e-3 * np.abs(a).max()


# ---------------------------------------------------------------- whole block

@pytest.mark.parametrize("shape", [SMALL, synth.TINY], ids=["small", "tiny"])
def test_onehot_router_reduces_to_dense_ffn(shape):
    j = 3
    layer = synth.make_layer(shape, seed=12, variant=synth.Variant(shared_zero=True))
    ol = O.OracleLayer(layer)
    x = synth.make_x(shape, 2, seed=12, dtype="f32")
    res = O.moe_rows(ol, x, offset=synth.onehot_offset(shape, j))
    assert np.all(res["idx"][:, 0] == j)
    np.testing.assert_array_equal(res["p"][:, 0], 1.0)
    np.testing.assert_array_equal(res["p"][:, 1:], 0.0)
    np.testing.assert_array_equal(res["shared_out"], 0.0)
    want = dense_ffn(layer.experts[j], O.x_to_f64(x))
    np.testing.assert_allclose(res["y"], want, rtol=1e-11, atol=1e-10 * np.abs(want).max())


def test_block_is_shared_plus_weighted_experts():
    """y - S(x) is linear in the weights, and every E_k is the dense FFN of expert idx_k."""
    layer = synth.make_layer(SMALL, seed=13, variant=synth.Variant(router_scale_log2=-6))
    ol = O.OracleLayer(layer)
    x = synth.make_x(SMALL, 4, seed=13)
    res = O.moe_rows(ol, x)
    x64 = O.x_to_f64(x)
    np.testing.assert_allclose(res["shared_out"], dense_ffn(layer.shared, x64), rtol=1e-11,
                               atol=1e-10 * np.abs(res["shared_out"]).max())
    for r in range(4):
        for k in range(SMALL.top_k):
            e = res["idx"][r, k]
            want = dense_ffn(layer.experts[e], x64[r:r + 1])[0]
            np.testing.assert_allclose(res["expert_out"][r, k], want, rtol=1e-11, atol=1e-10 * np.abs(want).max())
    y_lin = res["shared_out"] + np.einsum("rk,rkd->rd", res["p"], res["expert_out"])
    np.testing.assert_allclose(res["y"], y_lin, rtol=1e-13, atol=1e-12 * np.abs(y_lin).max())
    # the soft router really spreads weight, so experts 2..k are exercised
    assert res["p"][:, 1:].min() > 1e-3


def test_conditional_oracle_uses_given_picks():
    layer = synth.make_layer(SMALL, seed=14, variant=synth.Variant(router_scale_log2=-6))
    ol = O.OracleLayer(layer)
    x = synth.make_x(SMALL, 3, seed=14)
    free = O.moe_rows(ol, x)
    given = free["idx"][:, ::-1].copy()  # same set, reversed order
    cond = O.moe_rows(ol, x, idx=given)
    np.testing.assert_allclose(cond["p"], free["p"][:, ::-1], rtol=1e-14)
    np.testing.assert_allclose(cond["y"], free["y"], rtol=1e-12, atol=1e-12 * np.abs(free["y"]).max())


def test_prefill_rows_equal_single_row_calls():
    layer = synth.make_layer(SMALL, seed=15)
    ol = O.OracleLayer(layer)
    x = synth.make_x(SMALL, 6, seed=15)
    batch = O.moe_rows(ol, x)
    for r in range(6):
        one = O.moe_rows(ol, x[r:r + 1])
        np.testing.assert_array_equal(one["y"][0], batch["y"][r])
        np.testing.assert_array_equal(one["idx"][0], batch["idx"][r])


# ---------------------------------------------------------------- grouping

def test_grouping_against_python_sorted():
    rng = np.random.default_rng(16)
    for rows, E, k in ((1, 128, 8), (128, 128, 8), (37, 16, 4), (256, 128, 8)):
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(rows)]).astype(np.int32)
        count, offset, perm, inv = O.group_by_expert(idx, E)
        pairs = [(int(idx[r, j]), r, j) for r in range(rows) for j in range(k)]
        want = [r * k + j for (_, r, j) in sorted(pairs)]
        np.testing.assert_array_equal(perm, want)
        np.testing.assert_array_equal(count, np.bincount(idx.ravel(), minlength=E))
        np.testing.assert_array_equal(offset, np.concatenate([[0], np.cumsum(count)]))
        assert count.sum() == rows * k
        np.testing.assert_array_equal(np.sort(perm), np.arange(rows * k))
        np.testing.assert_array_equal(inv[perm], np.arange(rows * k))


# ---------------------------------------------------------------- residual

def test_residual_matches_torch_bf16_rounding():
    rng = np.random.default_rng(17)
    x = synth.f32_to_bf16_bits(rng.standard_normal(100000).astype(np.float32) * 10)
    y = (rng.standard_normal(100000) * 1000).astype(np.float32)
    y[:100] = 0.0
    got = O.residual_bf16(x, y)
    t = torch.from_numpy(synth.bf16_bits_to_f32(x)) + torch.from_numpy(y)  # fp32 add
    want = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(got[:100], x[:100])
