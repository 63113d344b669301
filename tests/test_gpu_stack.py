"""The 30-layer stacks of the Gemma-4-shaped MoE block, through the C ABI.

Every layer has its own seeded weights; all 30 x 128 experts sit in one
HBM-resident pool (12.85 GB) behind per-layer slot tables, and the residual
add between layers runs in the block's combine, in place (x and the residual
buffer are one tensor):
  - decode: one row through the 30 blocks;
  - prefill: chunks of 256 rows with Zipf-skewed routing through the 30 blocks.

Parity is checked teacher-forced: after the GPU has run layer l, the oracle
runs layer l on the GPU's own bf16 input x_l and the layer's outputs are
compared (the picks exactly on unflagged rows, y and the unweighted expert
outputs within the tolerance; flagged rows through the conditional oracle at the
GPU's picks). The residual store is checked bit-exact against RNE_bf16(RNE_fp32(
x_l + y_l)) of the GPU's own x_l and y_l.

Two stacks run:
  - literal: the workload weights. Without a norm between layers the residual
    stream gains a large common mode after the first layer: on most rows every
    gate pre-activation is then far below zero, tanh-GELU is exactly 0 and y is
    exactly 0; on some rows the common mode has the other sign and the row
    leaves fp32 range within a few layers. Layers whose input is finite are
    still compared, but they carry little numerics;
  - live (synth.LIVE_STACK, test-only weights): expert biases centred on the
    codes' mean and the experts scaled by 2^-3, the router by 2^-6. The residual
    stream stays near unit scale over all 30 layers, every gate is live and
    picks 2..k carry weight, so every layer of both stacks is checked on
    non-trivial values.
A HIP graph of the whole literal stack replays to the same bits as the eager calls.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _harness import FLAG_GAP, REL_TOL, check_topk, device, empty_f32, empty_i32, rel_err, to_dev_x, workspace

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]
q = pytest.importorskip("quantized_mixture_experts_bit_amd")

N_LAYERS = 30
PF_ROWS = 256
PF_SAMPLE = np.array([0, 37, 101, 128, 200, 255])  # prefill rows the oracle evaluates in full on every layer


def bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def residual_property(x_bits, y):
    """RNE_bf16(RNE_fp32(fp32(x) + y)) on the host (numpy), as uint16 bits."""
    s = (x_bits.astype(np.uint32) << 16).view(np.float32) + y.astype(np.float32)
    u = s.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def is_nan_bf16(v):
    return ((v & 0x7F80) == 0x7F80) & ((v & 0x007F) != 0)


def finite_rows(x_bits):
    return np.all((x_bits & 0x7F80) != 0x7F80, axis=-1)


def run_stack(variant, zipf_sigma_scale):
    """Runs both stacks layer by layer on the GPU and the oracle teacher-forced on each
    layer's GPU input. Returns the per-layer records and the device state."""
    from quantized_mixture_experts_bit_amd.weights import ExpertPool
    shape = synth.GEMMA4
    E, k, d = shape.n_experts, shape.top_k, shape.d_model
    dev = device()
    pool = ExpertPool(shape, N_LAYERS * E, dev)
    x0_dec = synth.make_x(shape, 1, seed=41, dtype="bf16")
    x0_pf = synth.make_x(shape, PF_ROWS, seed=42, dtype="bf16")
    h_dec, h_pf = to_dev_x(x0_dec).clone(), to_dev_x(x0_pf).clone()
    ws_dec, ws_pf = workspace(shape, 1), workspace(shape, PF_ROWS)
    idx_d, w_d, eo_d, y_d = empty_i32(1, k), empty_f32(1, k), empty_f32(k, d), empty_f32(1, d)
    pf = dict(idx=empty_i32(PF_ROWS, k), w=empty_f32(PF_ROWS, k), cnt=empty_i32(E), off=empty_i32(E + 1),
              perm=empty_i32(PF_ROWS * k), inv=empty_i32(PF_ROWS * k), eo=empty_f32(PF_ROWS * k, d),
              y=empty_f32(PF_ROWS, d))
    sigma = synth.router_logit_std(shape) * 2.0 ** variant.router_scale_log2 * zipf_sigma_scale
    layers, zipf, rec = [], [], []
    for l in range(N_LAYERS):
        L = synth.make_layer(shape, seed=0, layer=l, variant=variant)
        dl = pool.add_layer(L, l * E)
        zo = synth.make_zipf_offset(shape, seed=0, layer=l, sigma=sigma)
        zd = torch.from_numpy(zo).to(dev)
        layers.append(dl)
        zipf.append(zd)
        xin_d, xin_p = bf16_bits(h_dec), bf16_bits(h_pf)
        q.moe_layer_decode(shape, dl.c, h_dec, None, idx_d, w_d, eo_d, y_d, h_dec, ws_dec)
        q.moe_layer_prefill(shape, dl.c, h_pf, PF_ROWS, zd, pf["idx"], pf["w"], pf["cnt"], pf["off"], pf["perm"],
                            pf["inv"], pf["eo"], pf["y"], h_pf, ws_pf)
        torch.cuda.synchronize()
        g = dict(dec=dict(idx=idx_d.cpu().numpy(), w=w_d.cpu().numpy(), eo=eo_d.cpu().numpy()[None],
                          y=y_d.cpu().numpy(), x=xin_d, h=bf16_bits(h_dec), rows=np.array([0])),
                 pf=dict(idx=pf["idx"].cpu().numpy(), w=pf["w"].cpu().numpy(), cnt=pf["cnt"].cpu().numpy(),
                         perm=pf["perm"].cpu().numpy(), inv=pf["inv"].cpu().numpy(), y=pf["y"].cpu().numpy(),
                         x=xin_p, h=bf16_bits(h_pf), rows=PF_SAMPLE))
        eo_pf = pf["eo"].cpu().numpy()
        g["pf"]["eo"] = np.stack([eo_pf[g["pf"]["inv"][r * k:(r + 1) * k]] for r in PF_SAMPLE])
        ol = O.OracleLayer(L)
        # teacher-forced: the oracle runs this layer on the GPU's own input rows
        for key, off in (("dec", None), ("pf", zo)):
            c = g[key]
            xs = c["x"][c["rows"]]
            ref = O.moe_rows(ol, xs, offset=off)
            flagged = ref["gap"] < FLAG_GAP
            c["ref"] = ref
            c["ref_cond"] = O.moe_rows(ol, xs, offset=off, idx=c["idx"][c["rows"]]) if flagged.any() else None
        # the picks of every prefill row against the oracle's router on the GPU's input
        lg = O.router_logits(L, g["pf"]["x"], offset=zo)
        tk = [O.topk_softmax(lg[r], k) for r in range(PF_ROWS)]
        g["pf"]["ref_all"] = dict(idx=np.stack([t[0] for t in tk]), gap=np.array([t[2] for t in tk]), logits=lg)
        rec.append(g)
        print("stack %s: layer %d done" % ("live" if variant.center_bias else "literal", l), flush=True)
        del L, ol
    assert q.moe_check_device_error() == 0
    return dict(shape=shape, layers=layers, zipf=zipf, rec=rec, x0_dec=x0_dec, x0_pf=x0_pf, ws_dec=ws_dec,
                ws_pf=ws_pf, pf=pf, dec=(idx_d, w_d, eo_d, y_d), pool=pool)


@pytest.fixture(scope="module")
def literal():
    return run_stack(synth.Variant(), 1.0)


@pytest.fixture(scope="module")
def live():
    return run_stack(synth.LIVE_STACK, 1.0)


def check_layer(c, l, key, k):
    """One layer's outputs against the oracle evaluated on the GPU's input. Returns the
    number of rows compared (rows whose input is finite and whose oracle output fits fp32)."""
    compared = 0
    xs = c["x"][c["rows"]]
    ok = finite_rows(xs)
    for i, r in enumerate(c["rows"]):
        ref = c["ref"]
        if not ok[i] or not np.all(np.abs(ref["y"][i]) < 1e30):
            continue
        sub = {n: (v[i:i + 1] if v is not None else None) for n, v in ref.items()}
        if check_topk(c["idx"][r][None], sub, k)[0]:
            ref, i_ref = c["ref_cond"], i  # flagged: the oracle at the GPU's picks
        else:
            i_ref = i
        y_ref = ref["y"][i_ref]
        if np.abs(y_ref).max() == 0.0:
            assert np.all(c["y"][r] == 0.0), "%s layer %d row %d: oracle y is 0, GPU is not" % (key, l, r)
        else:
            e = rel_err(c["y"][r], y_ref)
            assert e <= REL_TOL, "%s layer %d row %d: y %.3g" % (key, l, r, e)
        # each pick's weight and unweighted output, matched by expert id (the order inside
        # the set may differ only where two picked logits tie)
        slot_of = {int(e): j for j, e in enumerate(ref["idx"][i_ref])}
        for j, e in enumerate(c["idx"][r]):
            jr = slot_of[int(e)]
            assert abs(float(c["w"][r][j]) - ref["p"][i_ref, jr]) <= 1e-6, \
                "%s layer %d row %d expert %d: weight %g vs %g" % (key, l, r, e, c["w"][r][j], ref["p"][i_ref, jr])
            eo_ref = ref["expert_out"][i_ref, jr]
            if np.abs(eo_ref).max() > 0.0:
                err = rel_err(c["eo"][i, j], eo_ref)
                assert err <= REL_TOL, "%s layer %d row %d expert %d: %.3g" % (key, l, r, e, err)
        compared += 1
    return compared


@pytest.mark.parametrize("key", ["dec", "pf"])
def test_live_stack_teacher_forced_every_layer(live, key):
    """All 30 layers of the live stack: picks, weights, y and every unweighted expert
    output of the decode row and the sampled prefill rows, on non-trivial values."""
    k = synth.GEMMA4.top_k
    total = 0
    for l, g in enumerate(live["rec"]):
        c = g[key]
        n = check_layer(c, l, key, k)
        assert n == len(c["rows"]), "%s layer %d: only %d of %d rows compared" % (key, l, n, len(c["rows"]))
        total += n
        # the layer is live: y is a real fraction of the residual stream on every checked row
        xs = O.x_to_f64(c["x"][c["rows"]])
        ys = c["y"][c["rows"]]
        assert np.all(np.abs(ys).max(axis=1) > 0.05 * np.sqrt((xs ** 2).mean(axis=1))), "%s layer %d" % (key, l)
    assert total == N_LAYERS * len(live["rec"][0][key]["rows"])


@pytest.mark.parametrize("which", ["literal", "live"])
def test_stack_prefill_picks_every_row(request, which):
    """The picks of all 256 rows on every layer against the oracle's router on the GPU's
    input (bit-exact sets and order on unflagged rows), and the grouping of those picks."""
    st = request.getfixturevalue(which)
    k, E = synth.GEMMA4.top_k, synth.GEMMA4.n_experts
    checked = 0
    for l, g in enumerate(st["rec"]):
        c = g["pf"]
        fin = finite_rows(c["x"])
        ra = c["ref_all"]
        for r in np.flatnonzero(fin):
            sub = dict(idx=ra["idx"][r:r + 1], gap=ra["gap"][r:r + 1], logits=ra["logits"][r:r + 1])
            check_topk(c["idx"][r][None], sub, k)
            checked += 1
        rc, ro, rp, ri = O.group_by_expert(c["idx"], E)
        np.testing.assert_array_equal(c["cnt"], rc, err_msg="layer %d" % l)
        np.testing.assert_array_equal(c["perm"], rp, err_msg="layer %d" % l)
        np.testing.assert_array_equal(c["inv"], ri, err_msg="layer %d" % l)
    if which == "live":
        assert checked == N_LAYERS * PF_ROWS


def test_live_stack_prefill_routing_is_skewed(live):
    """The Zipf offset makes experts repeat across the 256 rows on every layer."""
    for l, g in enumerate(live["rec"]):
        cnt = g["pf"]["cnt"]
        assert (cnt > 0).sum() < 90 and cnt.max() >= 64, "layer %d: %d experts, busiest %d" % (
            l, (cnt > 0).sum(), cnt.max())


@pytest.mark.parametrize("key", ["dec", "pf"])
def test_literal_stack_teacher_forced(literal, key):
    """Every layer of the literal stack whose input is finite, against the oracle on the
    GPU's input; the first layer carries real numerics."""
    k = synth.GEMMA4.top_k
    total = sum(check_layer(g[key], l, key, k) for l, g in enumerate(literal["rec"]))
    print("literal stack, %s: %d (row, layer) pairs compared" % (key, total))
    assert total >= N_LAYERS
    assert np.abs(literal["rec"][0][key]["y"]).max() > 1.0


@pytest.mark.parametrize("which", ["literal", "live"])
def test_stack_routing_stays_valid(request, which):
    """Whatever the activations hold (the literal stack leaves fp32 range on some rows),
    every layer's picks are k distinct valid expert ids on every row."""
    st = request.getfixturevalue(which)
    E, k = synth.GEMMA4.n_experts, synth.GEMMA4.top_k
    for l, r in enumerate(st["rec"]):
        for key in ("dec", "pf"):
            idx = r[key]["idx"].reshape(-1, k)
            assert idx.min() >= 0 and idx.max() < E, "layer %d %s" % (l, key)
            assert all(len(set(row.tolist())) == k for row in idx), "layer %d %s" % (l, key)


@pytest.mark.parametrize("which", ["literal", "live"])
@pytest.mark.parametrize("key", ["dec", "pf"])
def test_stack_residual_store_property(request, which, key):
    st = request.getfixturevalue(which)
    for l, r in enumerate(st["rec"]):
        c = r[key]
        exp = residual_property(c["x"], c["y"])
        same = (c["h"] == exp) | (is_nan_bf16(c["h"]) & is_nan_bf16(exp))  # NaN payloads may differ
        assert same.all(), "layer %d" % l


def test_stack_decode_graph_replay_bit_exact(literal):
    stack = literal
    shape, layers = stack["shape"], stack["layers"]
    idx_d, w_d, eo_d, y_d = stack["dec"]
    h = torch.empty(1, shape.d_model, dtype=torch.bfloat16, device=device())
    x0 = to_dev_x(stack["x0_dec"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        h.copy_(x0)
        q.moe_layer_decode(shape, layers[0].c, h, None, idx_d, w_d, eo_d, y_d, h, stack["ws_dec"], stream=s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for dl in layers:
                q.moe_layer_decode(shape, dl.c, h, None, idx_d, w_d, eo_d, y_d, h, stack["ws_dec"], stream=s)
    torch.cuda.current_stream().wait_stream(s)
    want = stack["rec"][-1]["dec"]["h"]
    for rep in range(3):
        h.copy_(x0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(h), want), "replay %d" % rep
    assert q.moe_check_device_error() == 0


def test_stack_prefill_graph_replay_bit_exact(live):
    stack = live
    shape, layers, zipf, pf = stack["shape"], stack["layers"], stack["zipf"], stack["pf"]
    h = torch.empty(PF_ROWS, shape.d_model, dtype=torch.bfloat16, device=device())
    x0 = to_dev_x(stack["x0_pf"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()

    def step(l):
        q.moe_layer_prefill(shape, layers[l].c, h, PF_ROWS, zipf[l], pf["idx"], pf["w"], pf["cnt"], pf["off"],
                            pf["perm"], pf["inv"], pf["eo"], pf["y"], h, stack["ws_pf"], stream=s)

    with torch.cuda.stream(s):
        h.copy_(x0)
        step(0)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for l in range(N_LAYERS):
                step(l)
    torch.cuda.current_stream().wait_stream(s)
    want = stack["rec"][-1]["pf"]["h"]
    for rep in range(2):
        h.copy_(x0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(h), want), "replay %d" % rep
    assert q.moe_check_device_error() == 0


@pytest.mark.parametrize("which", ["literal", "live"])
def test_stack_decode_one_launch_matches_layer_calls(request, which):
    """moe_stack_decode (all 30 layers in one launch) gives the bits of the 30
    moe_layer_decode calls the fixture recorded: every layer's input, picks, weights,
    unweighted expert outputs and y, and the final row. With those equal, the
    teacher-forced oracle checks above hold for the one-launch stack as well."""
    st = request.getfixturevalue(which)
    shape, layers = st["shape"], st["layers"]
    k, d, L = shape.top_k, shape.d_model, N_LAYERS
    x = to_dev_x(st["x0_dec"]).clone()
    idx, w = empty_i32(L, k), empty_f32(L, k)
    eo, y = empty_f32(L, k, d), empty_f32(L, d)
    xl = torch.empty(L, d, dtype=torch.bfloat16, device=device())
    q.moe_stack_decode(shape, [dl.c for dl in layers], x, None, idx, w, eo, y, xl, st["ws_dec"])
    torch.cuda.synchronize()
    assert q.moe_check_device_error() == 0
    xl_b, idx_n, w_n, eo_n, y_n = bf16_bits(xl), idx.cpu().numpy(), w.cpu().numpy(), eo.cpu().numpy(), y.cpu().numpy()
    for l, r in enumerate(st["rec"]):
        c = r["dec"]
        assert np.array_equal(xl_b[l], c["x"][0]), "layer %d input" % l
        assert np.array_equal(idx_n[l], c["idx"][0]), "layer %d picks" % l
        assert np.array_equal(w_n[l].view(np.uint32), c["w"][0].view(np.uint32)), "layer %d weights" % l
        assert np.array_equal(eo_n[l].view(np.uint32), c["eo"][0].view(np.uint32)), "layer %d expert outputs" % l
        assert np.array_equal(y_n[l].view(np.uint32), c["y"][0].view(np.uint32)), "layer %d y" % l
    assert np.array_equal(bf16_bits(x)[0], st["rec"][-1]["dec"]["h"][0])


def test_stack_decode_graph_replay_bit_exact(live):
    """The one-launch stack captured in a HIP graph replays to the eager bits, with eager
    calls between the replays."""
    st = live
    shape, layers = st["shape"], st["layers"]
    k, d, L = shape.top_k, shape.d_model, N_LAYERS
    cl = [dl.c for dl in layers]
    idx, w, y = empty_i32(L, k), empty_f32(L, k), empty_f32(L, d)
    h = torch.empty(1, d, dtype=torch.bfloat16, device=device())
    x0 = to_dev_x(st["x0_dec"])
    want = st["rec"][-1]["dec"]["h"]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        h.copy_(x0)
        q.moe_stack_decode(shape, cl, h, None, idx, w, None, y, None, st["ws_dec"], stream=s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            q.moe_stack_decode(shape, cl, h, None, idx, w, None, y, None, st["ws_dec"], stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        h.copy_(x0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(h), want), "replay %d" % rep
        # an eager call between the replays
        h.copy_(x0)
        q.moe_stack_decode(shape, cl, h, None, idx, w, None, y, None, st["ws_dec"])
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(h), want), "eager after replay %d" % rep
    assert q.moe_check_device_error() == 0
