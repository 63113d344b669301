"""fp64 CPU oracle of the quantized MoE FFN block -- TEST INFRASTRUCTURE.

Only the tests, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package. The HIP product path never imports it and
shares no code with it; the two meet only at the seeded input generators in
`synth`.

The arithmetic lives in plain C (`moe_oracle.c`, fp64, one loop per step of the
method); this module builds it with gcc, loads it with ctypes and marshals
numpy arrays. Widening bf16/fp32 activations to float64 is exact.

Every function is pinned by CPU tests against hand-computed values, closed
forms, invariants and library routines (numpy matmul/sort, torch's tanh-GELU
and bf16 rounding); see tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False, out: Optional[str] = None, extra_flags=()) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction) into `out` (the
    in-tree liboracle.so by default); extra_flags are added to the command (e.g. a
    host sanitizer)."""
    target = out or _LIB
    if force or out or not os.path.exists(target) or os.path.getmtime(target) < os.path.getmtime(_SRC):
        tmp = target + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-D_GNU_SOURCE"] + list(extra_flags) + ["-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, target)
    return target


class _Mat(C.Structure):
    _fields_ = [("q", C.c_void_p), ("s", C.c_void_p), ("b", C.c_void_p),
                ("rows", C.c_int32), ("cols", C.c_int32), ("bits", C.c_int32)]


class _Layer(C.Structure):
    _fields_ = [("router", _Mat), ("sgate", _Mat), ("sup", _Mat), ("sdown", _Mat),
                ("gate", C.POINTER(_Mat)), ("up", C.POINTER(_Mat)), ("down", C.POINTER(_Mat)),
                ("n_experts", C.c_int32), ("top_k", C.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        # QMOE_ORACLE_LIB names another build of the same source (e.g. a sanitizer build)
        _lib = C.CDLL(os.environ.get("QMOE_ORACLE_LIB") or build())
        P = C.POINTER
        d = P(C.c_double)
        _lib.oracle_code.restype = C.c_int
        _lib.oracle_code.argtypes = [P(_Mat), C.c_int32, C.c_int32]
        _lib.oracle_weight.restype = C.c_double
        _lib.oracle_weight.argtypes = [P(_Mat), C.c_int32, C.c_int32]
        _lib.oracle_dequant.argtypes = [P(_Mat), d]
        _lib.oracle_matvec.argtypes = [P(_Mat), d, d]
        _lib.oracle_gelu_tanh.restype = C.c_double
        _lib.oracle_gelu_tanh.argtypes = [C.c_double]
        _lib.oracle_topk_softmax.argtypes = [d, C.c_int32, C.c_int32, P(C.c_int32), d, d]
        _lib.oracle_softmax_at.argtypes = [d, P(C.c_int32), C.c_int32, d]
        _lib.oracle_moe_rows.argtypes = [P(_Layer), d, C.c_int32, P(C.c_float), C.c_int32, d,
                                         P(C.c_int32), d, d, d, d, d]
        _lib.oracle_router_rows.argtypes = [P(_Mat), d, C.c_int32, P(C.c_float), d]
        _lib.oracle_expert_rows.argtypes = [P(_Mat), P(_Mat), P(_Mat), d, C.c_int32, d]
        _lib.oracle_group_by_expert.argtypes = [P(C.c_int32), C.c_int32, C.c_int32, C.c_int32,
                                                P(C.c_int32), P(C.c_int32), P(C.c_int32), P(C.c_int32)]
        _lib.oracle_residual_bf16.argtypes = [P(C.c_uint16), P(C.c_float), C.c_int64, P(C.c_uint16)]
        _lib.oracle_set_threads.argtypes = [C.c_int32]
        _lib.oracle_threads.restype = C.c_int32
    return _lib


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def threads() -> int:
    return int(lib().oracle_threads())


def _ptr(a: Optional[np.ndarray], ctype=C.c_double):
    if a is None:
        return None
    assert a.flags.c_contiguous
    return a.ctypes.data_as(C.POINTER(ctype))


def _mat(m) -> _Mat:
    """ctypes view of a synth.QMat (arrays must stay alive while used)."""
    for a in (m.q, m.s, m.b):
        assert a.flags.c_contiguous
    return _Mat(m.q.ctypes.data, m.s.ctypes.data, m.b.ctypes.data, m.rows, m.cols, m.bits)


def x_to_f64(x: np.ndarray) -> np.ndarray:
    """Exact fp64 values of stored activations: float32 array, or uint16 bf16 bit patterns."""
    if x.dtype == np.uint16:
        return np.ascontiguousarray((x.astype(np.uint32) << 16).view(np.float32), dtype=np.float64)
    if x.dtype == np.float32:
        return np.ascontiguousarray(x, dtype=np.float64)
    raise TypeError(x.dtype)


class OracleLayer:
    """Holds the ctypes description of one synth.Layer."""

    def __init__(self, layer):
        self.layer = layer
        sh = layer.shape
        E = sh.n_experts
        self._gate = (_Mat * E)(*[_mat(e.gate) for e in layer.experts])
        self._up = (_Mat * E)(*[_mat(e.up) for e in layer.experts])
        self._down = (_Mat * E)(*[_mat(e.down) for e in layer.experts])
        self.c = _Layer(_mat(layer.router), _mat(layer.shared.gate), _mat(layer.shared.up),
                        _mat(layer.shared.down), self._gate, self._up, self._down, E, sh.top_k)


def code(m, n: int, i: int) -> int:
    cm = _mat(m)
    return lib().oracle_code(C.byref(cm), n, i)


def weight(m, n: int, i: int) -> float:
    cm = _mat(m)
    return lib().oracle_weight(C.byref(cm), n, i)


def dequant(m) -> np.ndarray:
    W = np.empty((m.rows, m.cols), dtype=np.float64)
    cm = _mat(m)
    lib().oracle_dequant(C.byref(cm), _ptr(W))
    return W


def matvec(m, v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(m.rows, dtype=np.float64)
    cm = _mat(m)
    lib().oracle_matvec(C.byref(cm), _ptr(v), _ptr(out))
    return out


def gelu_tanh(z: float) -> float:
    return lib().oracle_gelu_tanh(float(z))


def topk_softmax(logits: np.ndarray, k: int):
    """Returns (idx int32[k], p float64[k], gap float)."""
    lg = np.ascontiguousarray(logits, dtype=np.float64)
    idx = np.empty(k, dtype=np.int32)
    p = np.empty(k, dtype=np.float64)
    gap = np.empty(1, dtype=np.float64)
    lib().oracle_topk_softmax(_ptr(lg), lg.shape[0], k, _ptr(idx, C.c_int32), _ptr(p), _ptr(gap))
    return idx, p, float(gap[0])


def router_logits(layer_or_router, x: np.ndarray, offset: Optional[np.ndarray] = None) -> np.ndarray:
    router = getattr(layer_or_router, "router", layer_or_router)
    xf = x_to_f64(x)
    rows = xf.shape[0]
    out = np.empty((rows, router.rows), dtype=np.float64)
    off = None if offset is None else np.ascontiguousarray(offset, dtype=np.float32)
    cm = _mat(router)
    lib().oracle_router_rows(C.byref(cm), _ptr(xf), rows, _ptr(off, C.c_float), _ptr(out))
    return out


def expert_rows(expert, x: np.ndarray) -> np.ndarray:
    """Unweighted expert output E(x) for each row of x (fp64 [rows, d_out])."""
    xf = x_to_f64(x) if x.dtype != np.float64 else np.ascontiguousarray(x)
    rows = xf.shape[0]
    out = np.empty((rows, expert.down.rows), dtype=np.float64)
    g, u, dn = _mat(expert.gate), _mat(expert.up), _mat(expert.down)
    lib().oracle_expert_rows(C.byref(g), C.byref(u), C.byref(dn), _ptr(xf), rows, _ptr(out))
    return out


def moe_rows(olayer: OracleLayer, x: np.ndarray, offset: Optional[np.ndarray] = None,
             idx: Optional[np.ndarray] = None, want=("logits", "idx", "p", "gap", "expert_out", "shared_out", "y")):
    """The whole block for rows of x. If idx is given, the picks are taken from it
    (conditional oracle) and p is this oracle's softmax at those picks."""
    sh = olayer.layer.shape
    xf = x_to_f64(x) if x.dtype != np.float64 else np.ascontiguousarray(x)
    rows, d = xf.shape
    E, k = sh.n_experts, sh.top_k
    res = {}
    res["logits"] = np.empty((rows, E)) if "logits" in want else None
    if idx is not None:
        res["idx"] = np.ascontiguousarray(idx, dtype=np.int32).reshape(rows, k).copy()
    else:
        res["idx"] = np.empty((rows, k), dtype=np.int32)
    res["p"] = np.empty((rows, k))
    res["gap"] = np.full(rows, np.nan) if "gap" in want else None
    res["expert_out"] = np.empty((rows, k, d)) if "expert_out" in want else None
    res["shared_out"] = np.empty((rows, d)) if "shared_out" in want else None
    res["y"] = np.empty((rows, d)) if "y" in want else None
    off = None if offset is None else np.ascontiguousarray(offset, dtype=np.float32)
    lib().oracle_moe_rows(C.byref(olayer.c), _ptr(xf), rows, _ptr(off, C.c_float), 1 if idx is not None else 0,
                          _ptr(res["logits"]), _ptr(res["idx"], C.c_int32), _ptr(res["p"]), _ptr(res["gap"]),
                          _ptr(res["expert_out"]), _ptr(res["shared_out"]), _ptr(res["y"]))
    return res


def group_by_expert(idx: np.ndarray, n_experts: int):
    """Returns (count[E], offset[E+1], perm[P], inv_perm[P]) for idx [rows, k]."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    rows, k = idx.shape
    P = rows * k
    count = np.empty(n_experts, dtype=np.int32)
    offset = np.empty(n_experts + 1, dtype=np.int32)
    perm = np.empty(P, dtype=np.int32)
    inv = np.empty(P, dtype=np.int32)
    i32 = C.c_int32
    lib().oracle_group_by_expert(_ptr(idx, i32), rows, k, n_experts, _ptr(count, i32), _ptr(offset, i32),
                                 _ptr(perm, i32), _ptr(inv, i32))
    return count, offset, perm, inv


def residual_bf16(x_bits: np.ndarray, y: np.ndarray) -> np.ndarray:
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty_like(x_bits)
    lib().oracle_residual_bf16(_ptr(x_bits, C.c_uint16), _ptr(y, C.c_float), x_bits.size,
                               _ptr(out, C.c_uint16))
    return out
