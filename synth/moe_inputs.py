"""Seeded synthetic MoE-layer inputs (storage formats only, no layer arithmetic).

Workload shapes follow the Qwen3.6-35B-A3B MoE layer the pages describe (the
router picks 8 of 256 experts and one shared expert is added; page
"Perplexity Open Sources Lily", section Technical Details). Hidden size 2048 and
expert intermediate size 512 are assumed; the pages do not print them.

Storage formats:
  * bf16 tensors are numpy ``uint16`` bit patterns.
  * a 4-bit weight matrix of shape [N, K] is stored as ``q`` uint32 [N, K/8]
    (nibble i of word w, bits 4i..4i+3, holds element 8w+i), plus ``s`` and
    ``b`` bf16 [N, K/64]: one scale and one bias per 64 consecutive elements
    along K (page "Perplexity Open Sources Lily", Technical Details: groupwise
    affine 4-bit, 64 weights per group, bfloat16 scale).

Recipe (numpy PCG64 ``default_rng(seed)``, draws in this order):
  1. x = bf16(N(0, 1))                       [T, H]
  2. router_w = bf16(N(0, 1) / sqrt(H))      [E, H]
  3. for gate, up, down of the E routed experts, then gate, up, down of the
     shared expert: q words uniform over all 32-bit values (so every nibble is
     an independent U{0..15}), then s = bf16(|N(0, 1)| * 0.02), then
     b = -8 s (exact in bf16) or, for the "random" bias mode,
     b = bf16(-s * U(0, 15)).
  4. optional logit bias (a Zipf(1.2) skew over expert index):
     beta[e] = -1.2 * ln(e + 1) as float32 (no draw).
  5. optional shared-expert gate vector (gated_shared=True), drawn last so that
     every earlier draw is unchanged: shared_gate = bf16(N(0, 1) / sqrt(H)) [H].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

GROUP = 64


@dataclasses.dataclass
class Q4Weights:
    """A stack of n 4-bit matrices of shape [N, K] in the storage format."""
    q: np.ndarray  # uint32 [n, N, K//8]
    s: np.ndarray  # uint16 (bf16 bits) [n, N, K//64]
    b: np.ndarray  # uint16 (bf16 bits) [n, N, K//64]

    @property
    def n(self) -> int:
        return self.q.shape[0]

    @property
    def N(self) -> int:
        return self.q.shape[1]

    @property
    def K(self) -> int:
        return self.q.shape[2] * 8


@dataclasses.dataclass
class MoEInputs:
    T: int
    H: int
    I: int
    E: int
    k: int
    x: np.ndarray              # uint16 [T, H]
    router_w: np.ndarray       # uint16 [E, H]
    logit_bias: Optional[np.ndarray]  # float32 [E] or None
    gate: Q4Weights            # n=E, [I, H]
    up: Q4Weights              # n=E, [I, H]
    down: Q4Weights            # n=E, [H, I]
    sh_gate: Q4Weights         # n=1, [I, H]
    sh_up: Q4Weights           # n=1, [I, H]
    sh_down: Q4Weights         # n=1, [H, I]
    seed: int = 0
    bias_mode: str = "sym"
    shared_gate: Optional[np.ndarray] = None   # uint16 [H] or None (ungated shared expert)


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Store float values as bf16 bit patterns (torch's float32->bfloat16 cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _draw_q4(rng: np.random.Generator, n: int, N: int, K: int, bias_mode: str) -> Q4Weights:
    if K % GROUP:
        raise ValueError(f"K={K} must be a multiple of {GROUP}")
    q = rng.integers(0, 2**32, size=(n, N, K // 8), dtype=np.uint32)
    s_f = np.abs(rng.standard_normal((n, N, K // GROUP))) * 0.02
    s = _to_bf16_bits(s_f)
    if bias_mode == "sym":
        # -8 * s only moves the exponent, so it is exact in bf16: flip the sign
        # bit and add 3 to the exponent field through a float32 round trip.
        s32 = (s.astype(np.uint32) << 16).view(np.float32)
        b = _to_bf16_bits(-8.0 * s32)
    elif bias_mode == "random":
        s32 = (s.astype(np.uint32) << 16).view(np.float32)
        u = rng.uniform(0.0, 15.0, size=s.shape)
        b = _to_bf16_bits(-s32.astype(np.float64) * u)
    else:
        raise ValueError(f"unknown bias_mode {bias_mode!r}")
    return Q4Weights(q=q, s=s, b=b)


def make_layer(T: int, H: int, I: int, E: int, k: int, seed: int = 0,
               bias_mode: str = "sym", zipf: Optional[float] = None,
               gated_shared: bool = False) -> MoEInputs:
    """Draw one MoE layer's inputs in the documented order."""
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    rng = np.random.default_rng(seed)
    x = _to_bf16_bits(rng.standard_normal((T, H)))
    router_w = _to_bf16_bits(rng.standard_normal((E, H)) / math.sqrt(H))
    gate = _draw_q4(rng, E, I, H, bias_mode)
    up = _draw_q4(rng, E, I, H, bias_mode)
    down = _draw_q4(rng, E, H, I, bias_mode)
    sh_gate = _draw_q4(rng, 1, I, H, bias_mode)
    sh_up = _draw_q4(rng, 1, I, H, bias_mode)
    sh_down = _draw_q4(rng, 1, H, I, bias_mode)
    logit_bias = None
    if zipf is not None:
        logit_bias = (-float(zipf) * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)
    shared_gate = _to_bf16_bits(rng.standard_normal(H) / math.sqrt(H)) if gated_shared else None
    return MoEInputs(T=T, H=H, I=I, E=E, k=k, x=x, router_w=router_w, logit_bias=logit_bias,
                     gate=gate, up=up, down=down, sh_gate=sh_gate, sh_up=sh_up, sh_down=sh_down,
                     seed=seed, bias_mode=bias_mode, shared_gate=shared_gate)


def redraw_token_rows(inp: MoEInputs, rows: np.ndarray, seed: int) -> None:
    """Replace x[rows] with fresh bf16(N(0,1)) draws from ``default_rng(seed)``.

    Used to resample tokens whose routing boundary is too close to a tie; the
    caller decides which rows (that decision needs the router, which is not
    part of this module)."""
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size == 0:
        return
    rng = np.random.default_rng(seed)
    inp.x[rows] = _to_bf16_bits(rng.standard_normal((rows.size, inp.H)))


# Named workloads: sizes of the layer and of the batch.
CONFIGS = {
    # tiny layer for exhaustive parity: T=64, hidden 256, 16 experts top-2 + shared, I=128
    "tiny": dict(T=64, H=256, I=128, E=16, k=2),
    # full-shape layer (H=2048, I=512, 256 experts top-8 + shared) at several batch sizes
    "prefill512": dict(T=512, H=2048, I=512, E=256, k=8),
    "prefill4096": dict(T=4096, H=2048, I=512, E=256, k=8),
    "prefill4096_zipf": dict(T=4096, H=2048, I=512, E=256, k=8, zipf=1.2),
    "decode1": dict(T=1, H=2048, I=512, E=256, k=8),
    "decode8": dict(T=8, H=2048, I=512, E=256, k=8),
    "prefill32768": dict(T=32768, H=2048, I=512, E=256, k=8),
}


def make_config(name: str, seed: int = 0, bias_mode: str = "sym", **over) -> MoEInputs:
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    return make_layer(seed=seed, bias_mode=bias_mode, **cfg)
