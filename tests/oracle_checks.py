"""Pins for the fp64 oracle: checks against facts that do not come from the oracle itself.

Each ``check_*`` takes the oracle module (possibly with a planted mistake) and
raises AssertionError when the oracle disagrees with a closed form, a library
routine applied to a special case, a hand-derived fixture, an invariant, or the
independent per-token brute force. The tests run every check on the real
oracle (all must pass) and on planted mistakes (each must be caught).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
from scipy.special import softmax

from oracle import brute_force
from synth import Q4Weights, make_layer

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bits_of(values):
    """float32 values that are bf16-exact -> bf16 bit patterns (library cast)."""
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------
# bf16
# ----------------------------------------------------------------------------

def check_bf16(om):
    # hand-derived bit patterns
    cases = {1.0: 0x3F80, -2.0: 0xC000, 0.0: 0x0000, 1.0 + 2**-7: 0x3F81,
             1.0 + 2**-8: 0x3F80,              # tie -> even (down)
             1.0 + 3 * 2**-8: 0x3F82,          # tie -> even (up)
             1.0 + 2**-8 + 2**-40: 0x3F81,     # not a tie in fp64 (through fp32 it would be)
             3.3895313892515355e38: 0x7F7F,    # largest finite bf16
             3.4e38: 0x7F80}                   # rounds past it -> +inf
    for v, bits in cases.items():
        got = int(om.f64_to_bf16_bits(np.array([v]))[0])
        assert got == bits, f"bf16({v!r}) = {got:#06x}, expected {bits:#06x}"
    # every finite bf16 pattern decodes like the field-by-field decoder
    pats = np.arange(1 << 16, dtype=np.uint16)
    fin = ((pats >> 7) & 0xFF) != 0xFF
    a = om.bf16_bits_to_f64(pats[fin])
    b = brute_force.bf16_decode(pats[fin])
    assert np.array_equal(a, b), "bf16 decode mismatch"
    # on float32 inputs (no double rounding possible) rounding equals torch's cast
    rng = np.random.default_rng(7)
    f = (rng.standard_normal(20000) * np.exp2(rng.integers(-60, 60, 20000))).astype(np.float32)
    # add exact ties: a bf16 value plus half a bf16 ulp
    base = f[:2000].view(np.uint32) & np.uint32(0xFFFF0000)
    f[:2000] = (base | np.uint32(0x8000)).view(np.float32)
    ref = torch.tensor(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = om.f64_to_bf16_bits(f.astype(np.float64))
    assert np.array_equal(got, ref), "bf16 rounding differs from torch on float32 inputs"
    # subnormal grid: 2**-133 is the smallest positive bf16; 1.5 * that ties to even (2 * 2**-133)
    assert om.round_bf16(np.array([1.5 * 2.0 ** -133]))[0] == 2 * 2.0 ** -133
    assert om.round_bf16(np.array([0.5 * 2.0 ** -133]))[0] == 0.0


# ----------------------------------------------------------------------------
# 4-bit weights
# ----------------------------------------------------------------------------

def check_unpack(om):
    w = np.array([[0x76543210, 0xFEDCBA98]], dtype=np.uint32)
    got = om.unpack_q4(w)
    assert got.tolist() == [list(range(16))], f"nibble order wrong: {got.tolist()}"


def check_dequant(om):
    # constants: q = 3 everywhere, s = 0.5, b = -1 -> W = 0.5
    N, K = 4, 128
    q = np.full((N, K // 8), 0x33333333, dtype=np.uint32)
    s = np.full((N, K // 64), 0x3F00, dtype=np.uint16)
    b = np.full((N, K // 64), 0xBF80, dtype=np.uint16)
    assert np.all(om.dequant_q4(q, s, b) == 0.5)
    # one group per column block: group g has scale 2**g, bias -g; q = element index mod 16
    K = 256
    idx = np.arange(K)
    words = np.zeros((1, K // 8), dtype=np.uint32)
    for kk in range(K):
        words[0, kk // 8] |= np.uint32((kk % 16) << (4 * (kk % 8)))
    s = _bits_of([[2.0 ** g for g in range(K // 64)]])
    b = _bits_of([[-float(g) for g in range(K // 64)]])
    want = (2.0 ** (idx // 64)) * (idx % 16) - (idx // 64)
    assert np.array_equal(om.dequant_q4(words, s, b)[0], want), "group scale/bias placement wrong"
    # symmetric special case b = -8 s gives s * (q - 8)
    rng = np.random.default_rng(3)
    qw = rng.integers(0, 2**32, size=(8, 32), dtype=np.uint32)
    sv = np.abs(rng.standard_normal((8, 4))).astype(np.float32) * 0.02
    s_b = _bits_of(sv)
    b_b = _bits_of((-8.0 * om.bf16_bits_to_f64(s_b)).astype(np.float32))
    qn = brute_force.dequant_bytes(qw, np.full((8, 4), 0x3F80, np.uint16), np.zeros((8, 4), np.uint16))
    want = np.repeat(om.bf16_bits_to_f64(s_b), 64, axis=1) * (qn - 8)
    assert np.array_equal(om.dequant_q4(qw, s_b, b_b), want)
    # random case against the byte-wise decoder
    b_r = _bits_of((-om.bf16_bits_to_f64(s_b) * rng.uniform(0, 15, (8, 4))).astype(np.float32))
    assert np.array_equal(om.dequant_q4(qw, s_b, b_r), brute_force.dequant_bytes(qw, s_b, b_r))


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------

def check_logits(om):
    # integer-valued x and W_r: every product and partial sum is an exact
    # integer far below 2**24, so fp64 and float32 both hold the int64 result
    rng = np.random.default_rng(5)
    T, H, E = 16, 256, 12
    xi = rng.integers(-16, 17, size=(T, H))
    wi = rng.integers(-8, 9, size=(E, H))
    l = om.router_logits(_bits_of(xi.astype(np.float32)), _bits_of(wi.astype(np.float32)))
    assert l.dtype == np.float32
    assert np.array_equal(l.astype(np.int64), xi @ wi.T), "router logits wrong"
    beta = np.arange(E, dtype=np.float32) * 0.5
    lb = om.router_logits(_bits_of(xi.astype(np.float32)), _bits_of(wi.astype(np.float32)), beta)
    assert np.array_equal(lb, (xi @ wi.T).astype(np.float32) + beta)


def check_topk(om):
    # all-zero logits: experts 0..k-1 with weight 1/k
    ids, w = om.select_topk(np.zeros((5, 9), np.float32), 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 5
    assert np.allclose(w, 0.25, rtol=0, atol=1e-15)
    # constructed ties: lowest index first
    l = np.array([[1, 3, 3, 0, 3], [2, 2, 2, 2, 2]], np.float32)
    ids, _ = om.select_topk(l, 3)
    assert ids.tolist() == [[1, 2, 4], [0, 1, 2]], ids.tolist()
    # negative zero ties with zero
    ids, _ = om.select_topk(np.array([[-0.0, 0.0, -1.0]], np.float32), 1)
    assert ids.tolist() == [[0]]
    # k == E: a full descending sort, weights = softmax over all logits
    rng = np.random.default_rng(11)
    l = rng.standard_normal((6, 10)).astype(np.float32)
    ids, w = om.select_topk(l, 10)
    for t in range(6):
        assert ids[t].tolist() == sorted(range(10), key=lambda e: (-float(l[t, e]), e))
        assert np.allclose(w[t], softmax(l[t].astype(np.float64)[ids[t]]), rtol=0, atol=1e-15)
    # many ties (logits on a coarse grid) against Python's sorted
    l = (rng.integers(0, 4, size=(40, 16)) * 0.25).astype(np.float32)
    ids, w = om.select_topk(l, 5)
    for t in range(40):
        assert ids[t].tolist() == sorted(range(16), key=lambda e: (-float(l[t, e]), e))[:5]
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
    # closed form: logits a and a - ln 2 -> weights 2/3 and 1/3
    a = 1.25
    l = np.array([[a - math.log(2.0), -5.0, a]], np.float32)
    ids, w = om.select_topk(l, 2)
    assert ids.tolist() == [[2, 0]]
    assert abs(w[0, 0] - 2 / 3) < 1e-7 and abs(w[0, 1] - 1 / 3) < 1e-7
    # -inf logits get weight 0
    ids, w = om.select_topk(np.array([[0.0, -np.inf, 1.0]], np.float32), 3)
    assert ids.tolist() == [[2, 0, 1]] and w[0, 2] == 0.0


def check_golden_routing(om):
    with open(os.path.join(GOLDEN, "routing_small.json")) as f:
        g = json.load(f)
    l = np.array(g["logits"], dtype=np.float32)
    ids, w = om.select_topk(l, g["k"])
    assert ids.tolist() == g["topk_ids"]
    assert np.max(np.abs(w - np.array(g["topk_w"]))) <= g["topk_w_tol"]
    for bm, tiles in g["tile_map"].items():
        tab = om.routing_tables(ids, g["E"], int(bm))
        assert tab["counts"].tolist() == g["counts"]
        assert tab["offsets"].tolist() == g["offsets"]
        assert tab["sorted_rows"].tolist() == g["sorted_rows"]
        assert tab["row_of_pair"].tolist() == g["row_of_pair"]
        assert tab["tile_map"].tolist() == tiles, (bm, tab["tile_map"].tolist())
        assert int(tab["num_tiles"]) == len(tiles)


def check_routing_invariants(om, cases=((64, 16, 2, 64), (512, 256, 8, 64), (37, 5, 5, 3),
                                        (1, 256, 8, 32), (300, 32, 4, 16))):
    rng = np.random.default_rng(13)
    for T, E, k, bm in cases:
        l = rng.standard_normal((T, E)).astype(np.float32)
        if T > 10:
            l[::7] = np.round(l[::7])          # plenty of exact ties
        ids, _ = om.select_topk(l, k)
        tab = om.routing_tables(ids, E, bm)
        c, o, sr, rp, tm = (tab[n] for n in ("counts", "offsets", "sorted_rows", "row_of_pair", "tile_map"))
        assert c.sum() == T * k
        assert o[0] == 0 and o[-1] == T * k and np.array_equal(np.diff(o), c)
        assert np.array_equal(np.sort(sr), np.arange(T * k)), "scatter is not a permutation"
        assert np.array_equal(rp[sr], np.arange(T * k))
        flat = ids.ravel()
        for e in range(E):
            seg = sr[o[e]:o[e + 1]]
            assert np.all(flat[seg] == e)
            assert np.all(np.diff(seg) > 0), "scatter is not stable"
        assert np.all(np.bincount(sr // k, minlength=T) == k), "a token does not appear k times"
        for t in range(T):
            assert len(set(ids[t].tolist())) == k, "repeated expert in one token"
        want = [(e, int(o[e]) + i * bm) for e in range(E) for i in range(-(-int(c[e]) // bm))]
        assert [tuple(r) for r in tm.tolist()] == want
        assert int(tab["num_tiles"]) == sum(-(-int(ce) // bm) for ce in c)


# ----------------------------------------------------------------------------
# FFN and the layer
# ----------------------------------------------------------------------------

def _one_expert_layer(T=8, H=128, I=64, seed=21, same_shared=True):
    inp = make_layer(T, H, I, E=1, k=1, seed=seed, bias_mode="random")
    if same_shared:
        inp.sh_gate, inp.sh_up, inp.sh_down = inp.gate, inp.up, inp.down
    return inp


def check_dense_ffn(om):
    # E = 1, k = 1 with the shared expert equal to the routed one: the layer is
    # twice a dense SwiGLU FFN, which torch computes independently in fp64
    inp = _one_expert_layer()
    out = om.moe_layer(inp, round_h=False, round_y=False)
    xb = torch.tensor(inp.x.astype(np.int16)).view(torch.bfloat16).double()

    def deq(w):
        return torch.tensor(brute_force.dequant_bytes(w.q[0], w.s[0], w.b[0]))
    h = torch.nn.functional.silu(xb @ deq(inp.gate).T) * (xb @ deq(inp.up).T)
    ref = 2.0 * (h @ deq(inp.down).T)
    err = (torch.tensor(out["y"]) - ref).abs().max() / ref.abs().max()
    assert float(err) < 1e-13, f"dense FFN mismatch {float(err)}"
    assert out["topk_w"].tolist() == [[1.0]] * inp.T


def check_integer_ffn(om):
    # s = 1, b = 0 and integer x: gate and up products are exact integers; pick
    # the down weights so that the whole expert is exactly checkable
    T, H, I = 4, 128, 64
    inp = make_layer(T, H, I, E=1, k=1, seed=2)
    rng = np.random.default_rng(2)
    xi = rng.integers(-16, 17, size=(T, H))
    inp.x = _bits_of(xi.astype(np.float32))
    one = np.full_like(inp.gate.s, 0x3F80)
    zero = np.zeros_like(inp.gate.b)
    inp.gate = Q4Weights(inp.gate.q, one, zero)
    g_int = xi @ brute_force.dequant_bytes(inp.gate.q[0], one[0], zero[0]).astype(np.int64).T
    wg = om.dequant_q4(inp.gate.q[0], one[0], zero[0])
    assert np.array_equal(om.bf16_bits_to_f64(inp.x) @ wg.T, g_int.astype(np.float64))


def check_brute(om, cfg=dict(T=64, H=256, I=128, E=16, k=2), seeds=(0,), modes=("sym", "random"),
                zipf=(None,), tokens=None):
    for seed in seeds:
        for mode in modes:
            for z in zipf:
                inp = make_layer(seed=seed, bias_mode=mode, zipf=z, **cfg)
                out = om.moe_layer(inp)
                l_ref = brute_force_logits(inp)
                assert np.array_equal(out["logits"], l_ref), "router logits differ from the brute force"
                toks = list(range(inp.T)) if tokens is None else tokens
                yb, ids, w = brute_force.layer_brute_force(inp, l_ref, toks)
                assert np.array_equal(out["topk_ids"][toks], ids), "top-k ids differ"
                assert np.max(np.abs(out["topk_w"][toks] - w)) < 1e-15
                ya = out["y_unrounded"][toks]
                err = np.linalg.norm(ya - yb) / np.linalg.norm(yb)
                assert err < 1e-12, f"layer differs from per-token brute force: rel {err:.3g}"


def check_layer_tokens(om, cases=(dict(T=64, H=256, I=128, E=16, k=2, seed=0, bias_mode="random"),
                                  dict(T=24, H=128, I=64, E=4, k=4, seed=1, bias_mode="random"),
                                  dict(T=12, H=128, I=64, E=64, k=32, seed=2, bias_mode="random"),
                                  dict(T=48, H=256, I=128, E=16, k=2, seed=3, bias_mode="sym", zipf=1.2),
                                  dict(T=32, H=256, I=128, E=16, k=4, seed=4, bias_mode="random",
                                       gated_shared=True))):
    """The per-token oracle (``moe_layer_tokens``, the reference for sampled and
    decode-shaped layer checks) against the independent per-token brute force
    and against the sort-based layer on the same logits: tiny, k = E, k = 32,
    a Zipf logit bias, both bias modes, all tokens and a shuffled subset."""
    for cfg in cases:
        inp = make_layer(**cfg)
        rng = np.random.default_rng(cfg["seed"] + 40)
        l = om.router_logits(inp.x, inp.router_w, inp.logit_bias)
        # exact ties inside the top-k and at its boundary on some tokens
        l[::5] = np.round(l[::5] * 2) / 2
        full = om.moe_layer(inp, logits=l)["y_unrounded"]
        toks = list(range(inp.T))
        sub = rng.permutation(inp.T)[: max(3, inp.T // 3)].tolist()
        for tk in (toks, sub):
            got = om.moe_layer_tokens(inp, tk, l)
            yb, _, _ = brute_force.layer_brute_force(inp, l, tk)
            err_b = np.linalg.norm(got - yb) / np.linalg.norm(yb)
            assert err_b < 1e-12, f"per-token oracle differs from the brute force: rel {err_b:.3g}"
            err_f = np.max(np.abs(got - full[tk])) / np.max(np.abs(full))
            assert err_f < 1e-14, f"per-token oracle differs from the layer oracle: rel {err_f:.3g}"


def check_gated_shared(om):
    """The gated shared expert: against the independent brute force (scipy's
    expit of a math.fsum dot product), and against two closed forms on the
    dense special case E = k = 1 with the shared expert equal to the routed
    one: a zero gate vector gives the factor 1/2 exactly, so y = 1.5 * FFN(x);
    a one-hot gate vector e_0 gives y = (1 + sigmoid(x_0)) * FFN(x), with the
    FFN and the sigmoid from torch in fp64."""
    for cfg in (dict(T=40, H=256, I=128, E=16, k=2, seed=5, bias_mode="random"),
                dict(T=24, H=128, I=64, E=8, k=8, seed=6, bias_mode="sym", zipf=1.2)):
        inp = make_layer(gated_shared=True, **cfg)
        out = om.moe_layer(inp)
        l_ref = brute_force_logits(inp)
        yb, _, _ = brute_force.layer_brute_force(inp, l_ref)
        err = np.linalg.norm(out["y_unrounded"] - yb) / np.linalg.norm(yb)
        assert err < 1e-12, f"gated layer differs from the per-token brute force: rel {err:.3g}"
    inp = _one_expert_layer(seed=31)
    xb = torch.tensor(inp.x.astype(np.int16)).view(torch.bfloat16).double()

    def deq(w):
        return torch.tensor(brute_force.dequant_bytes(w.q[0], w.s[0], w.b[0]))
    ffn = (torch.nn.functional.silu(xb @ deq(inp.gate).T) * (xb @ deq(inp.up).T)) @ deq(inp.down).T
    inp.shared_gate = np.zeros(inp.H, np.uint16)
    y = torch.tensor(om.moe_layer(inp, round_h=False, round_y=False)["y"])
    assert float((y - 1.5 * ffn).abs().max() / ffn.abs().max()) < 1e-13, "zero gate vector: factor is not 1/2"
    inp.shared_gate = _bits_of(np.eye(1, inp.H, 0, dtype=np.float32)[0])
    y = torch.tensor(om.moe_layer(inp, round_h=False, round_y=False)["y"])
    want = (1.0 + torch.sigmoid(xb[:, :1])) * ffn
    assert float((y - want).abs().max() / want.abs().max()) < 1e-13, "one-hot gate vector"


def brute_force_logits(inp):
    """Router logits computed token by token with Python floats -> fp64 dot -> fp32."""
    x = brute_force.bf16_decode(inp.x)
    w = brute_force.bf16_decode(inp.router_w)
    l = np.empty((inp.T, inp.E), np.float32)
    for t in range(inp.T):
        for e in range(inp.E):
            l[t, e] = np.float32(math.fsum(x[t] * w[e]))
    if inp.logit_bias is not None:
        l = l + inp.logit_bias.astype(np.float32)
    return l


ALL_CHECKS = [check_bf16, check_unpack, check_dequant, check_logits, check_topk, check_golden_routing,
              check_routing_invariants, check_dense_ffn, check_integer_ffn, check_brute, check_layer_tokens,
               check_gated_shared]
