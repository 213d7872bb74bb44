"""Shared test helpers: workload construction and the parity metrics."""
from __future__ import annotations

import numpy as np

import oracle.moe_oracle as om
from synth import make_config, make_layer, redraw_token_rows

# bf16 outputs vs the fp64-accumulated reference
REL_L2_TOL = 1e-3
MAX_ABS_FRAC_TOL = 2e-2
LOGIT_ABS_TOL = 1e-4
WEIGHT_ABS_TOL = 1e-6
GAP_MIN = 1e-3


def resample_close_calls(inp, gap_min: float = GAP_MIN, max_rounds: int = 50):
    """Redraw tokens whose k-th and (k+1)-th largest router logits are within gap_min."""
    for it in range(max_rounds):
        l = om.router_logits(inp.x, inp.router_w, inp.logit_bias).astype(np.float64)
        if inp.k >= inp.E:
            return inp
        srt = -np.sort(-l, axis=1)
        gap = srt[:, inp.k - 1] - srt[:, inp.k]
        bad = np.nonzero(gap <= gap_min)[0]
        if bad.size == 0:
            return inp
        redraw_token_rows(inp, bad, seed=10_000 * (inp.seed + 1) + it)
    raise RuntimeError("could not separate the top-k boundary")


def tiny_layer(seed: int = 0, bias_mode: str = "sym", **over):
    """The tiny configuration with close routing calls resampled."""
    inp = make_config("tiny", seed=seed, bias_mode=bias_mode, **over)
    return resample_close_calls(inp)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def max_abs_frac(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / den) if den > 0 else float(np.max(np.abs(a - b)))


def assert_close_bf16(got, ref, what: str):
    r = rel_l2(got, ref)
    m = max_abs_frac(got, ref)
    assert r <= REL_L2_TOL and m <= MAX_ABS_FRAC_TOL, f"{what}: rel L2 {r:.3e}, max-abs/max|ref| {m:.3e}"
    return r, m


__all__ = ["make_config", "make_layer", "tiny_layer", "resample_close_calls", "rel_l2", "max_abs_frac",
           "assert_close_bf16", "REL_L2_TOL", "MAX_ABS_FRAC_TOL", "LOGIT_ABS_TOL", "WEIGHT_ABS_TOL"]
