"""CPU oracle of the 4-bit groupwise-affine quantiser (bf16 weights -> q, s, b).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
cpu_baseline leg may use it; it shares no code with the HIP path.

The pages name the format (P1 = "Perplexity Open Sources Lily ...", Technical
Details, prefill bullet: groupwise affine 4-bit weights, 64 per group; its
Chinese 技术解析: a bf16 scale per 64 weights) but not how weights are
quantised. The reading taken here is the plain min-max affine quantiser,
computed step by step in fp32 so that a GPU implementation can reproduce every
integer exactly:

  for each row n and group g (64 consecutive elements along K):
    lo = min, hi = max of the group (fp32 values of the bf16 weights; -0 -> +0)
    s  = bf16(fp32(fp32(hi - lo) / 15))          round to nearest even
    b  = lo                                       (already a bf16 value)
    q  = 0                                        if s == 0
         min(15, max(0, rint(fp32(fp32(w - b) / s))))   otherwise (rint: ties to even)

so that W = s*q + b reproduces w within s/2 (plus the bf16 rounding of s, at
most 15 * 2^-9 * s at the top of the group). Output layout: q packed 8 per
uint32 word, nibble i = element 8w+i; s and b as bf16 bit patterns [rows][K/64].
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import GROUP, f64_to_bf16_bits


def pack_q4(q: np.ndarray) -> np.ndarray:
    """uint8 [..., K] with values 0..15 -> uint32 [..., K/8]; element 8w+i in nibble i of word w."""
    q = np.asarray(q, dtype=np.uint32)
    K = q.shape[-1]
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    nib = q.reshape(*q.shape[:-1], K // 8, 8)
    shifts = 4 * np.arange(8, dtype=np.uint32)
    return np.bitwise_or.reduce(nib << shifts, axis=-1).astype(np.uint32)


def quantize_q4(w_bits: np.ndarray):
    """bf16 weights [..., K] (uint16 bit patterns) -> (q words uint32 [..., K/8],
    s bits uint16 [..., K/64], b bits uint16 [..., K/64])."""
    wb = np.asarray(w_bits, dtype=np.uint16)
    K = wb.shape[-1]
    if K % GROUP:
        raise ValueError("K must be a multiple of 64")
    w = (wb.astype(np.uint32) << 16).view(np.float32)
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")
    g = w.reshape(*w.shape[:-1], K // GROUP, GROUP)
    lo = g.min(axis=-1) + np.float32(0.0)          # -0 -> +0
    hi = g.max(axis=-1)
    s32 = (hi - lo) / np.float32(15.0)              # float32 arithmetic throughout
    s_bits = f64_to_bf16_bits(s32.astype(np.float64))
    s = (s_bits.astype(np.uint32) << 16).view(np.float32)
    b_bits = (lo.view(np.uint32) >> 16).astype(np.uint16)
    d = g - lo[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(d / s[..., None])
    q = np.where(s[..., None] == 0, np.float32(0), np.clip(r, 0, 15)).astype(np.uint8)
    q = q.reshape(*w.shape)
    return pack_q4(q), s_bits, b_bits
