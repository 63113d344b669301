"""Seeded synthetic inputs for the quantized MoE FFN block.

This module draws random numbers and lays them out in the canonical storage
format. It holds none of the block's arithmetic (no dequantisation, no dot
products, no routing). Both the HIP path and the fp64 oracle take their inputs
from here, and nothing else is shared between them.

Canonical format of one quantized matrix W[rows x cols] (MLX-style affine
quantisation, group 64 along the input dimension; the TurboFieldfare pages,
"quantisation" paragraph of the system-design summary on the ai-heartland
review and the 4-bit/8-bit paragraph of the rebasdaily article):

  q  uint8  4-bit: [rows, cols/2], element 2j in the LOW nibble of byte j,
                   element 2j+1 in the high nibble;
            8-bit: [rows, cols], one byte per element
  s  uint16 bf16 bit patterns [rows, cols/64]  (scale of each group)
  b  uint16 bf16 bit patterns [rows, cols/64]  (bias of each group)

Weight distributions follow the tiny-layer workload: q uniform over its code
range, s ~ U(0.005, 0.02), b ~ U(-0.1, 0.1), both rounded to bf16 (RNE), and
the rounded values are the truth. Every (layer, kind, expert, matrix) has its
own numpy SeedSequence stream, so any single expert can be regenerated alone.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np

GROUP = 64

# stream kinds (part of the SeedSequence spawn key)
KIND_ROUTER = 0
KIND_EXPERT = 1
KIND_SHARED = 2
KIND_X = 3
KIND_ZIPF = 4

S_RANGE = (0.005, 0.02)
B_RANGE = (-0.1, 0.1)


@dataclass(frozen=True)
class MoeShape:
    d_model: int
    d_ff: int
    d_ff_shared: int
    n_experts: int = 128
    top_k: int = 8
    group: int = GROUP


# tiny single layer: d_model 512, experts 512x256 / 256x512, shared d_ff 512
TINY = MoeShape(512, 256, 512)
# Gemma-4-26B-A4B-like layer: d_model 2816, expert d_ff 704, shared d_ff 2112
GEMMA4 = MoeShape(2816, 704, 2112)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest even); returns uint16 bit patterns.

    Input preparation only (finite inputs assumed)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class QMat:
    """Canonical quantized matrix W[rows x cols]."""
    q: np.ndarray
    s: np.ndarray
    b: np.ndarray
    bits: int

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    @property
    def cols(self) -> int:
        return self.q.shape[1] * (2 if self.bits == 4 else 1)

    @property
    def nbytes(self) -> int:
        return self.q.nbytes + self.s.nbytes + self.b.nbytes


@dataclass
class Expert:
    gate: QMat  # [d_ff x d_model]
    up: QMat    # [d_ff x d_model]
    down: QMat  # [d_model x d_ff]


@dataclass
class Layer:
    shape: MoeShape
    router: QMat            # 8-bit [n_experts x d_model]
    shared: Expert          # 4-bit, d_ff_shared
    experts: List[Expert]   # 4-bit, d_ff each
    index: int = 0


@dataclass(frozen=True)
class Variant:
    """Test-only changes to the drawn weights (the workloads use the default)."""
    router_scale_log2: int = 0      # multiply router s and b by 2**k (exact in bf16)
    shared_zero: bool = False       # shared expert with s = b = 0 (contributes exactly 0)
    s_range: tuple = S_RANGE
    b_range: tuple = B_RANGE
    # Live-stack weights: expert and shared-expert biases centred on the codes' mean
    # (b' = bf16(b - 7.5 s), so each weight s*q + b' has mean b ~ 0 over q instead of
    # about +0.09), then s and b' of those matrices multiplied by 2**expert_scale_log2
    # (exact in bf16). Without a norm between layers the literal weights drive a
    # 30-layer residual stream into a large common mode (every gate pre-activation
    # far below 0, so y = 0) or out of fp32 range; these keep it at unit scale.
    center_bias: bool = False
    expert_scale_log2: int = 0


# the stacked-layer test variant: centred 4-bit biases, experts scaled by 2**-3, and the
# router's s and b scaled by 2**-6 so that picks 2..k carry weight in the softmax
LIVE_STACK = Variant(router_scale_log2=-6, center_bias=True, expert_scale_log2=-3)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence(entropy=seed, spawn_key=tuple(key))))


def draw_qmat(rng: np.random.Generator, rows: int, cols: int, bits: int,
              s_range=S_RANGE, b_range=B_RANGE) -> QMat:
    assert cols % GROUP == 0
    if bits == 4:
        # one random byte = two independent uniform 4-bit codes
        q = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    elif bits == 8:
        q = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    else:
        raise ValueError(bits)
    ng = cols // GROUP
    s = f32_to_bf16_bits(rng.uniform(s_range[0], s_range[1], size=(rows, ng)).astype(np.float32))
    b = f32_to_bf16_bits(rng.uniform(b_range[0], b_range[1], size=(rows, ng)).astype(np.float32))
    return QMat(q, s, b, bits)


def _scale_bits(h: np.ndarray, log2: int) -> np.ndarray:
    if log2 == 0:
        return h
    f = bf16_bits_to_f32(h) * np.float32(2.0 ** log2)
    return f32_to_bf16_bits(f)


def make_router(shape: MoeShape, seed: int, layer: int, variant: Variant = Variant()) -> QMat:
    m = draw_qmat(_rng(seed, layer, KIND_ROUTER, 0, 0), shape.n_experts, shape.d_model, 8,
                  variant.s_range, variant.b_range)
    if variant.router_scale_log2:
        m = replace(m, s=_scale_bits(m.s, variant.router_scale_log2), b=_scale_bits(m.b, variant.router_scale_log2))
    return m


def _live(m: QMat, variant: Variant) -> QMat:
    """A 4-bit matrix under the variant's centring and power-of-two scaling."""
    if variant.center_bias:
        s = bf16_bits_to_f32(m.s)
        m = replace(m, b=f32_to_bf16_bits(bf16_bits_to_f32(m.b) - np.float32(7.5) * s))
    if variant.expert_scale_log2:
        m = replace(m, s=_scale_bits(m.s, variant.expert_scale_log2), b=_scale_bits(m.b, variant.expert_scale_log2))
    return m


def make_expert(shape: MoeShape, seed: int, layer: int, e: int, variant: Variant = Variant()) -> Expert:
    d, f = shape.d_model, shape.d_ff
    mats = [_live(draw_qmat(_rng(seed, layer, KIND_EXPERT, e, j), r, c, 4, variant.s_range, variant.b_range), variant)
            for j, (r, c) in enumerate(((f, d), (f, d), (d, f)))]
    return Expert(*mats)


def make_shared(shape: MoeShape, seed: int, layer: int, variant: Variant = Variant()) -> Expert:
    d, f = shape.d_model, shape.d_ff_shared
    mats = [_live(draw_qmat(_rng(seed, layer, KIND_SHARED, 0, j), r, c, 4, variant.s_range, variant.b_range), variant)
            for j, (r, c) in enumerate(((f, d), (f, d), (d, f)))]
    if variant.shared_zero:
        mats = [replace(m, s=np.zeros_like(m.s), b=np.zeros_like(m.b)) for m in mats]
    return Expert(*mats)


def make_layer(shape: MoeShape, seed: int = 0, layer: int = 0, variant: Variant = Variant()) -> Layer:
    return Layer(shape=shape,
                 router=make_router(shape, seed, layer, variant),
                 shared=make_shared(shape, seed, layer, variant),
                 experts=[make_expert(shape, seed, layer, e, variant) for e in range(shape.n_experts)],
                 index=layer)


def make_x(shape: MoeShape, rows: int, seed: int = 0, stream: int = 0, dtype: str = "bf16") -> np.ndarray:
    """Activations x ~ N(0, 1): float32 [rows, d_model] for dtype "f32", else bf16 bits (uint16)."""
    x = _rng(seed, stream, KIND_X, 0, 0).standard_normal((rows, shape.d_model)).astype(np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def router_logit_std(shape: MoeShape, s_range=S_RANGE, b_range=B_RANGE) -> float:
    """Standard deviation of one router logit over x ~ N(0, I), in closed form from
    the weight distribution: Var = d * E[w^2], w = s*q + b with independent
    s ~ U(s_range), q ~ U{0..255}, b ~ U(b_range). A property of the input
    distribution, not of any drawn weights."""
    s0, s1 = s_range
    b0, b1 = b_range
    es = 0.5 * (s0 + s1)
    es2 = (s1 ** 3 - s0 ** 3) / (3.0 * (s1 - s0))
    eq, eq2 = 127.5, 255.0 * 511.0 / 6.0
    eb = 0.5 * (b0 + b1)
    eb2 = (b1 ** 3 - b0 ** 3) / (3.0 * (b1 - b0))
    ew2 = es2 * eq2 + 2.0 * es * eq * eb + eb2
    return math.sqrt(shape.d_model * ew2)


def make_zipf_offset(shape: MoeShape, seed: int = 0, layer: int = 0, s_exp: float = 1.1,
                     sigma: Optional[float] = None) -> np.ndarray:
    """Per-expert router-logit offset that makes the selected experts repeat across
    rows: a seeded permutation ranks the experts and expert e of rank r(e) gets
    o[e] = -s_exp * sigma * ln(r(e) + 1), float32 [n_experts]. sigma defaults to the
    closed-form logit standard deviation, so the offset is on the scale of the
    logits (a raw -1.1*ln(r+1) would be negligible next to logits of std ~100)."""
    if sigma is None:
        sigma = router_logit_std(shape)
    rank = _rng(seed, layer, KIND_ZIPF, 0, 0).permutation(shape.n_experts)
    return (-s_exp * sigma * np.log(rank.astype(np.float64) + 1.0)).astype(np.float32)


def onehot_offset(shape: MoeShape, expert: int, big: float = 1.0e6) -> np.ndarray:
    """Offset that forces `expert` to rank first with softmax weight exactly 1 (in fp64,
    the other seven picks sit ~1e6 lower, so their weights underflow to 0)."""
    o = np.zeros(shape.n_experts, dtype=np.float32)
    o[expert] = big
    return o
