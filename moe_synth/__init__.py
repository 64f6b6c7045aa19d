"""Seeded synthetic inputs for the routed 4-bit MoE expert FFN.

This module is shared by the tests, the benchmark and the smoke check.  It only
draws random inputs in the layouts that both the HIP library and the CPU oracle
consume.  It computes nothing of the expert FFN itself (no dequantisation, no
matmul, no activation, no sort, no combine).

Layouts (row-major, K contiguous, the "transposed" weight layout of the
Layr-Labs/mlx PR #4 page, section "What"):

  x            bf16 bits  uint16 [T, H]
  topk_ids     int32             [T, k]   expert id of each routed copy
  topk_weights float32           [T, k]   routing weight of each copy
  w_gateup     uint32            [E, 2I, H/8]   rows [0,I) gate, [I,2I) up
                                                (H/4 with 8-bit codes)
  s_gateup     bf16 bits  uint16 [E, 2I, H/gs]
  b_gateup     bf16 bits  uint16 [E, 2I, H/gs]
  w_down       uint32            [E, H, I/8]    (I/4 with 8-bit codes)
  s_down       bf16 bits  uint16 [E, H, I/gs]
  b_down       bf16 bits  uint16 [E, H, I/gs]

Each uint32 word holds 8 four-bit codes.  Drawing every word uniformly from
[0, 2^32) makes each of its eight nibbles an independent uniform draw from
0..15, so the generator never has to choose a nibble order.

Recipe (one numpy ``default_rng(seed)`` per problem, draws in this order):

  1. router: per-expert bias (biased router) or popularity ranks (Zipf router),
     then logits N(0,1) of shape [T, E];
  2. x = bf16(N(0,1)) of shape [T, H] (round to nearest even);
  3. gate|up words, then gate|up scales bf16(|N(0, 0.02)|);
  4. down words, then down scales bf16(|N(0, 0.02)|);
  biases are -8 * scale (exact in bf16), so every dequantised weight is
  scale * (q - 8); or, with bias="independent", bf16(N(0, 0.05)) drawn right
  after each scale array (the general affine format).

Routing: softmax over all E experts in float32, the k largest logits (ties to
the lower expert id, per-token order by descending logit), weights divided by
the sum of the k selected probabilities.  The library takes ids and weights
as given; this step only produces inputs.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

__all__ = [
    "CONFIGS",
    "Problem",
    "make_problem",
    "make_config",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "route_topk",
]

# The five synthetic workloads.  Geometry E=128, H=2816, I=704 is the exact
# production geometry named on the Layr-Labs/mlx PR #4 page ("What": packed
# gate/up [128, 1408, 352], down [128, 2816, 88]).
CONFIGS: Dict[str, dict] = {
    "tiny": dict(E=8, H=256, I=128, T=64, k=2, router="normal"),
    "decode": dict(E=128, H=2816, I=704, T=8, k=8, router="normal"),
    "prefill4k": dict(E=128, H=2816, I=704, T=512, k=8, router="normal"),
    "prefill8k": dict(E=128, H=2816, I=704, T=1024, k=8, router="biased"),
    "prefill16k": dict(E=128, H=2816, I=704, T=2048, k=8, router="zipf"),
}
CONFIG_ORDER = ["tiny", "decode", "prefill4k", "prefill8k", "prefill16k"]

GROUP_SIZE = 64
SCALE_STD = 0.02


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Problem:
    name: str
    seed: int
    E: int
    H: int
    I: int
    T: int
    k: int
    gs: int
    x: np.ndarray
    topk_ids: np.ndarray
    topk_weights: np.ndarray
    w_gateup: np.ndarray
    s_gateup: np.ndarray
    b_gateup: np.ndarray
    w_down: np.ndarray
    s_down: np.ndarray
    b_down: np.ndarray
    logits: Optional[np.ndarray] = field(default=None, repr=False)
    bits: int = 4
    bias: str = "centred"

    @property
    def A(self) -> int:
        return self.T * self.k

    def shapes(self) -> dict:
        return dict(E=self.E, H=self.H, I=self.I, T=self.T, k=self.k, gs=self.gs, bits=self.bits)


def route_topk(logits: np.ndarray, k: int):
    """Softmax top-k routing in float32 with renormalised weights.

    Ties go to the lower expert id; each token's k ids are ordered by
    descending logit.
    """
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    mx = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mx, dtype=np.float32)
    p = p / p.sum(axis=1, keepdims=True, dtype=np.float32)
    sel = np.take_along_axis(p, order, axis=1).astype(np.float32)
    w = (sel / sel.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return order.astype(np.int32), w


def _router_logits(rng: np.random.Generator, router: str, T: int, E: int) -> np.ndarray:
    if router == "normal":
        return rng.standard_normal((T, E), dtype=np.float32)
    if router == "biased":
        # one N(0,1) bias per expert gives moderately skewed expert loads
        bias = rng.standard_normal(E).astype(np.float32)
        return rng.standard_normal((T, E), dtype=np.float32) + bias[None, :]
    if router == "zipf":
        # Zipf(s=1.1) popularity over a seeded ranking of the experts, added to
        # the logits as log-probabilities: some experts stay empty, a few are hot
        rank = rng.permutation(E) + 1
        pr = rank.astype(np.float64) ** -1.1
        pr /= pr.sum()
        return (rng.standard_normal((T, E), dtype=np.float32)
                + np.log(pr).astype(np.float32)[None, :])
    raise ValueError(f"unknown router {router!r}")


BIAS_STD = 0.05


def _scales(rng: np.random.Generator, shape, bits: int = 4, bias: str = "centred"):
    """Scales |N(0, std)|; 8-bit scales are 16x smaller so that the weights
    keep the 4-bit spread.  Biases: "centred" -2^(bits-1) * scale (exact), or
    "independent" bf16(N(0, 0.05)) drawn right after the scales, unrelated to
    them (the general affine format: any bias with any scale)."""
    std = SCALE_STD if bits == 4 else SCALE_STD / 16
    s = f32_to_bf16_bits(np.abs(rng.normal(0.0, std, size=shape)).astype(np.float32))
    if bias == "centred":
        b = f32_to_bf16_bits(bf16_bits_to_f32(s) * np.float32(-(2 ** (bits - 1))))
    elif bias == "independent":
        b = f32_to_bf16_bits(rng.normal(0.0, BIAS_STD, size=shape).astype(np.float32))
    else:
        raise ValueError(f"unknown bias mode {bias!r}")
    return s, b


def make_problem(E: int, H: int, I: int, T: int, k: int, seed: int = 0,
                 router: str = "normal", gs: int = GROUP_SIZE, name: str = "custom",
                 topk_ids: Optional[np.ndarray] = None,
                 topk_weights: Optional[np.ndarray] = None, bits: int = 4,
                 bias: str = "centred", routing_only: bool = False) -> Problem:
    """Draw one problem.  ``topk_ids``/``topk_weights`` override the router draw
    (the logits are still drawn so the rest of the stream is unchanged).
    ``bits``: 4 (8 codes per uint32 word) or 8 (4 codes per word).
    ``bias``: "centred" (-2^(bits-1) * scale) or "independent" (see _scales).
    ``routing_only``: stop after the router draw (x and the weights are left
    None): the same ids and routing weights, for checks that need no data."""
    if H % 8 or I % 8 or H % gs or I % gs:
        raise ValueError("H and I must be multiples of 8 and of the group size")
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    rng = np.random.default_rng(seed)
    logits = _router_logits(rng, router, T, E)
    if k <= E:
        ids, w = route_topk(logits, k)
    else:
        ids = np.zeros((T, k), np.int32)
        w = np.full((T, k), 1.0 / k, np.float32)
    if topk_ids is not None:
        ids = np.ascontiguousarray(topk_ids, dtype=np.int32).reshape(T, k)
    if topk_weights is not None:
        w = np.ascontiguousarray(topk_weights, dtype=np.float32).reshape(T, k)
    if routing_only:
        return Problem(name=name, seed=seed, E=E, H=H, I=I, T=T, k=k, gs=gs, x=None,
                       topk_ids=ids, topk_weights=w, w_gateup=None, s_gateup=None,
                       b_gateup=None, w_down=None, s_down=None, b_down=None, logits=logits,
                       bits=bits, bias=bias)
    x = f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w_gu = rng.integers(0, 2**32, size=(E, 2 * I, H * bits // 32), dtype=np.uint32)
    s_gu, b_gu = _scales(rng, (E, 2 * I, H // gs), bits, bias)
    w_d = rng.integers(0, 2**32, size=(E, H, I * bits // 32), dtype=np.uint32)
    s_d, b_d = _scales(rng, (E, H, I // gs), bits, bias)
    return Problem(name=name, seed=seed, E=E, H=H, I=I, T=T, k=k, gs=gs, x=x,
                   topk_ids=ids, topk_weights=w, w_gateup=w_gu, s_gateup=s_gu,
                   b_gateup=b_gu, w_down=w_d, s_down=s_d, b_down=b_d, logits=logits,
                   bits=bits, bias=bias)


def make_config(name: str, seed: int = 0, routing_only: bool = False) -> Problem:
    """One of the five named workloads (see CONFIGS)."""
    c = CONFIGS[name]
    return make_problem(c["E"], c["H"], c["I"], c["T"], c["k"], seed=seed,
                        router=c["router"], name=name, routing_only=routing_only)
