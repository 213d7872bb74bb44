"""CPU tests: the fp64 oracle against its pins, and planted mistakes that the pins must catch."""
import numpy as np
import pytest

import oracle.moe_oracle as om
from tests import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(om)


def test_oracle_brute_force_zipf_and_seeds():
    oc.check_brute(om, seeds=(1, 2), modes=("random",), zipf=(1.2,))


def test_oracle_brute_force_full_shape_sampled_tokens():
    # full hidden/intermediate sizes with fewer experts keeps this CPU test short
    oc.check_brute(om, cfg=dict(T=32, H=2048, I=512, E=8, k=8), modes=("random",), tokens=[0, 7, 31])


# ----------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ----------------------------------------------------------------------------

def _unpack_high_first(words):
    w = np.asarray(words, dtype=np.uint32)
    shifts = 4 * (7 - np.arange(8, dtype=np.uint32))
    return ((w[..., None] >> shifts) & np.uint32(0xF)).reshape(*w.shape[:-1], w.shape[-1] * 8).astype(np.uint8)


def _dequant_no_bias(q, s, b):
    return np.asarray(om.unpack_q4(q), np.float64) * np.repeat(om.bf16_bits_to_f64(s), 64, axis=-1)


def _dequant_group32(q, s, b):
    qq = om.unpack_q4(q).astype(np.float64)
    K = qq.shape[-1]
    gi = np.minimum(np.arange(K) // 32, s.shape[-1] - 1)
    return qq * om.bf16_bits_to_f64(s)[..., gi] + om.bf16_bits_to_f64(b)[..., gi]


def _topk_high_index_ties(logits, k):
    l = np.asarray(logits, np.float32).astype(np.float64)
    idx = np.broadcast_to(np.arange(l.shape[1]), l.shape)
    ids = np.lexsort((-idx, -l), axis=-1)[:, :k].astype(np.int32)
    sel = np.take_along_axis(l, ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    return ids, ex / ex.sum(1, keepdims=True)


def _topk_no_renorm(logits, k):
    l = np.asarray(logits, np.float32).astype(np.float64)
    idx = np.broadcast_to(np.arange(l.shape[1]), l.shape)
    ids = np.lexsort((idx, -l), axis=-1)[:, :k].astype(np.int32)
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    return ids, np.take_along_axis(p, ids.astype(np.int64), axis=1)


_real_ffn = om.swiglu_ffn
_real_tables = om.routing_tables
_real_logits = om.router_logits


def _ffn_no_h_round(x, wg, wu, wd, round_h=True):
    return _real_ffn(x, wg, wu, wd, round_h=False)


def _ffn_swapped(x, wg, wu, wd, round_h=True):
    return _real_ffn(x, wu, wg, wd, round_h)


def _tables_unstable(ids, E, bm):
    t = _real_tables(ids, E, bm)
    sr = t["sorted_rows"].copy()
    o = t["offsets"]
    for e in range(E):
        sr[o[e]:o[e + 1]] = sr[o[e]:o[e + 1]][::-1]
    rp = np.empty_like(sr)
    rp[sr] = np.arange(sr.size)
    t["sorted_rows"], t["row_of_pair"] = sr, rp
    return t


def _tables_inclusive_scan(ids, E, bm):
    t = _real_tables(ids, E, bm)
    t["offsets"] = np.concatenate([np.cumsum(t["counts"]), [int(t["counts"].sum())]]).astype(np.int32)
    return t


def _tables_tile_off_by_one(ids, E, bm):
    return _real_tables(ids, E, bm + 1)


def _logits_reversed_experts(x, w, beta=None):
    return _real_logits(x, np.asarray(w)[::-1], beta)


def _round_bf16_truncate(v):
    v = np.asarray(v, np.float64)
    r = v.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return r.view(np.float32).astype(np.float64)


_real_layer_tokens = om.moe_layer_tokens


def _tokens_slot_weights_swapped(inp, tokens, logits, round_h=True):
    # the weights of each token's chosen experts applied in reverse slot order
    real = om.select_topk

    def swapped(l, k):
        ids, w = real(l, k)
        return ids, w[:, ::-1]
    om.select_topk = swapped
    try:
        return _real_layer_tokens(inp, tokens, logits, round_h)
    finally:
        om.select_topk = real


def _tokens_expert_off_by_one(inp, tokens, logits, round_h=True):
    # expert e's output computed with expert (e + 1) % E's weights
    import copy
    shifted = copy.copy(inp)
    for name in ("gate", "up", "down"):
        w = getattr(inp, name)
        setattr(shifted, name, type(w)(np.roll(w.q, -1, 0), np.roll(w.s, -1, 0), np.roll(w.b, -1, 0)))
    return _real_layer_tokens(shifted, tokens, logits, round_h)


def _tokens_no_shared(inp, tokens, logits, round_h=True):
    import copy
    zeroed = copy.copy(inp)
    w = inp.sh_down
    zeroed.sh_down = type(w)(w.q, np.zeros_like(w.s), np.zeros_like(w.b))
    return _real_layer_tokens(zeroed, tokens, logits, round_h)


_real_shared_gate = om.shared_gate


def _gate_sign_flipped(inp, x):
    g = _real_shared_gate(inp, x)
    return g if getattr(inp, "shared_gate", None) is None else 1.0 - g


def _gate_ignored(inp, x):
    return np.ones(x.shape[0])


def _gate_without_sigmoid(inp, x):
    if getattr(inp, "shared_gate", None) is None:
        return np.ones(x.shape[0])
    return x @ om.bf16_bits_to_f64(inp.shared_gate)


MUTANTS = {
    "nibble order": ("unpack_q4", _unpack_high_first),
    "bias dropped": ("dequant_q4", _dequant_no_bias),
    "group size 32": ("dequant_q4", _dequant_group32),
    "ties to high index": ("select_topk", _topk_high_index_ties),
    "softmax not renormalised": ("select_topk", _topk_no_renorm),
    "h not rounded": ("swiglu_ffn", _ffn_no_h_round),
    "gate/up swapped": ("swiglu_ffn", _ffn_swapped),
    "unstable scatter": ("routing_tables", _tables_unstable),
    "inclusive scan": ("routing_tables", _tables_inclusive_scan),
    "tile size off by one": ("routing_tables", _tables_tile_off_by_one),
    "router rows reversed": ("router_logits", _logits_reversed_experts),
    "bf16 truncation": ("round_bf16", _round_bf16_truncate),
    "per-token oracle: slot weights swapped": ("moe_layer_tokens", _tokens_slot_weights_swapped),
    "per-token oracle: expert index off by one": ("moe_layer_tokens", _tokens_expert_off_by_one),
    "per-token oracle: shared expert dropped": ("moe_layer_tokens", _tokens_no_shared),
    "shared gate: 1 - sigmoid": ("shared_gate", _gate_sign_flipped),
    "shared gate ignored": ("shared_gate", _gate_ignored),
    "shared gate without the sigmoid": ("shared_gate", _gate_without_sigmoid),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(om, attr, fn)
    failed = []
    for check in oc.ALL_CHECKS:
        try:
            if check is oc.check_brute:
                check(om, modes=("random",), tokens=list(range(16)))
            else:
                check(om)
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    assert failed, f"planted mistake '{name}' passed every pin"
