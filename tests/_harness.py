"""Helpers shared by the GPU tests: device copies of synthetic layers, runners for
the C-ABI calls, and the comparison rules.

Parity bar (fixed by the block's contract):
  - router top-k indices and the grouping: bit-exact, except rows whose oracle
    gap between the k-th and (k+1)-th logit is below FLAG_GAP (flagged rows: the
    conditional oracle then evaluates the block with the GPU's picks);
  - FFN outputs: max|err| / ||ref||_inf <= REL_TOL against the fp64 oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import synth

FLAG_GAP = 1e-4
REL_TOL = 2e-3

_layer_cache = {}


def device():
    return torch.device("cuda:0")


# shapes at the edges of what the library accepts: the most experts and picks (256, 16)
# and few experts, few picks, groups that do not fill a 4-group block
WIDE = synth.MoeShape(1024, 256, 768, n_experts=256, top_k=16)
NARROW = synth.MoeShape(768, 192, 320, n_experts=64, top_k=4)
# shapes past the whole-block decode kernel's tiling (d_ff <= 768; d_model <= 3072 and
# d_ff_shared <= 2560), which moe_layer_decode serves with its three-launch path
BEYOND_FF = synth.MoeShape(1024, 832, 512, n_experts=64, top_k=4)
BEYOND_D = synth.MoeShape(3200, 256, 2624, n_experts=64, top_k=2)


def get_layer(shape, seed=0, layer=0, variant=synth.Variant()):
    """(canonical layer, oracle layer, device layer), cached per process."""
    key = (shape, seed, layer, variant)
    if key not in _layer_cache:
        from quantized_mixture_experts_bit_amd.weights import upload_layers
        L = synth.make_layer(shape, seed=seed, layer=layer, variant=variant)
        (dl,) = upload_layers(shape, [L], device())
        _layer_cache[key] = (L, O.OracleLayer(L), dl)
    return _layer_cache[key]


def to_dev_x(x):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device())


def workspace(shape, rows):
    import quantized_mixture_experts_bit_amd as q
    ws = torch.empty(q.moe_workspace_bytes(shape, max(rows, 1)), dtype=torch.uint8, device=device())
    q.moe_workspace_init(ws)
    return ws


def rel_err(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(np.asarray(got, dtype=np.float64) - ref).max() / max(np.abs(ref).max(), 1e-300))


def empty_i32(*shape):
    return torch.empty(*shape, dtype=torch.int32, device=device())


def empty_f32(*shape):
    return torch.empty(*shape, dtype=torch.float32, device=device())


def check_topk(got_idx, ref, k):
    """Bit-exact picks (ordered) on unflagged rows; returns the flagged-row mask."""
    flagged = ref["gap"] < FLAG_GAP
    got_idx = np.asarray(got_idx).reshape(-1, k)
    for r in range(got_idx.shape[0]):
        if flagged[r]:
            continue
        assert np.array_equal(np.sort(got_idx[r]), np.sort(ref["idx"][r])), \
            "row %d: GPU picks %s, oracle %s (gap %.3g)" % (r, got_idx[r], ref["idx"][r], ref["gap"][r])
        lg = ref["logits"][r][ref["idx"][r]]
        # the order inside the set is fixed unless two picked logits nearly tie
        if k == 1 or np.min(np.abs(np.diff(lg))) > FLAG_GAP:
            assert np.array_equal(got_idx[r], ref["idx"][r]), "row %d: order %s vs %s" % (r, got_idx[r],
                                                                                          ref["idx"][r])
    return flagged
