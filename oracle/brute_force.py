"""Per-token brute force for the MoE layer, written independently of moe_oracle.

TEST INFRASTRUCTURE ONLY (used to pin the sort-based oracle; never by the
product path). It computes the same layer the plain way: for every token, pick
its experts with Python's ``sorted``, weight them with scipy's softmax,
dequantise each chosen expert from the raw bytes of the packed words, run the
dense SwiGLU FFN, and add the shared expert. No histogram, scan, scatter or
block map is involved, and no code is shared with moe_oracle.py: every helper
here is a separate formulation (byte-wise nibble unpacking, math.frexp-based
rounding), so a mistake in one is unlikely to be repeated in the other.

Page references as in moe_oracle.py (P1 Technical Details: a router picks 8 of
256 experts, one shared expert, groupwise affine 4-bit weights, 64 per group).
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import expit, softmax


def _bf16_value(bits: int) -> float:
    """Value of one bf16 bit pattern, decoded field by field."""
    sign = -1.0 if bits & 0x8000 else 1.0
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0xFF:
        return sign * math.inf if man == 0 else math.nan
    if exp == 0:
        return sign * man * 2.0 ** -133
    return sign * (1.0 + man / 128.0) * 2.0 ** (exp - 127)


_BF16_TABLE = np.array([_bf16_value(b) for b in range(1 << 16)], dtype=np.float64)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    return _BF16_TABLE[np.asarray(bits, dtype=np.uint16).astype(np.int64)]


def bf16_round_scalar(v: float) -> float:
    """Nearest bf16 value to v (ties to even), via math.frexp and Python's round()."""
    if not math.isfinite(v) or v == 0.0:
        return v
    m, e = math.frexp(abs(v))             # |v| = m * 2**e, m in [0.5, 1)
    q = max(e - 8, -133)
    r = round(abs(v) / 2.0 ** q) * 2.0 ** q   # round(): half to even, exact here
    if r >= 2.0 ** 128:
        r = math.inf
    return math.copysign(r, v)


def dequant_bytes(q_words: np.ndarray, s_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """[N, K/8] uint32 words -> fp64 [N, K] via the little-endian byte view:
    byte j of word w carries element 8w+2j in its low nibble and 8w+2j+1 in its high nibble."""
    N = q_words.shape[0]
    by = np.ascontiguousarray(q_words, dtype="<u4").view(np.uint8).reshape(N, -1)
    q = np.empty((N, by.shape[1] * 2), dtype=np.float64)
    q[:, 0::2] = by & 0x0F
    q[:, 1::2] = by >> 4
    K = q.shape[1]
    s = bf16_decode(s_bits)
    b = bf16_decode(b_bits)
    gidx = np.arange(K) // 64
    return q * s[:, gidx] + b[:, gidx]


def token_output(xt: np.ndarray, logits_row: np.ndarray, k: int, experts, shared,
                 round_h: bool = True, gate_w=None) -> np.ndarray:
    """One token's layer output before the final rounding (fp64).

    ``experts(e)`` and ``shared()`` return (Wg, Wu, Wd) as fp64 arrays;
    ``gate_w`` (fp64 [H] or None) gates the shared expert by the logistic
    function of x . gate_w (scipy's expit of a math.fsum dot product)."""
    E = logits_row.shape[0]
    lrow = [float(v) for v in logits_row]
    chosen = sorted(range(E), key=lambda e: (-lrow[e], e))[:k]
    w = softmax(np.array([lrow[e] for e in chosen], dtype=np.float64))

    def ffn(mats):
        wg, wu, wd = mats
        g = wg @ xt
        u = wu @ xt
        h = np.array([gi / (1.0 + math.exp(-gi)) * ui if gi > -700 else 0.0 * ui
                      for gi, ui in zip(g, u)])
        if round_h:
            h = np.array([bf16_round_scalar(v) for v in h])
        return wd @ h

    out = ffn(shared())
    if gate_w is not None:
        out = out * float(expit(math.fsum(xt * gate_w)))
    for wj, e in zip(w, chosen):
        out = out + wj * ffn(experts(e))
    return out, chosen, w


def layer_brute_force(inp, logits: np.ndarray, tokens=None, round_h: bool = True):
    """Brute-force y (fp64, before the final rounding) for the given tokens (default: all)."""
    tokens = range(inp.T) if tokens is None else tokens
    cache = {}

    def experts(e):
        if e not in cache:
            cache[e] = tuple(dequant_bytes(w.q[e], w.s[e], w.b[e]) for w in (inp.gate, inp.up, inp.down))
        return cache[e]

    def shared():
        if "sh" not in cache:
            cache["sh"] = tuple(dequant_bytes(w.q[0], w.s[0], w.b[0])
                                for w in (inp.sh_gate, inp.sh_up, inp.sh_down))
        return cache["sh"]

    gate_w = None
    if getattr(inp, "shared_gate", None) is not None:
        gate_w = bf16_decode(inp.shared_gate)
    ys, ids, ws = [], [], []
    for t in tokens:
        xt = bf16_decode(inp.x[t])
        y, chosen, w = token_output(xt, np.asarray(logits[t], dtype=np.float32).astype(np.float64),
                                    inp.k, experts, shared, round_h, gate_w)
        ys.append(y)
        ids.append(chosen)
        ws.append(w)
    return np.array(ys), np.array(ids, dtype=np.int32), np.array(ws)
