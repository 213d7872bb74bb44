"""CPU tests: the quantiser oracle (oracle/quantize.py) against its pins, and
planted mistakes in it that the pins must catch.

Pins (none of them re-states the quantiser's formula):
  - reconstruction error: |w - (s q + b)| <= s/2, up to the bf16 rounding of s
    (at most 15 * 2^-9 * s above the grid's top) and fp32 rounding;
  - exact round trip: weights that lie on a bf16-exact 16-level grid and reach
    both its ends come back as the same codes, scale and bias;
  - constant groups: s = 0, q = 0, b = the value;
  - order: within a group the codes never decrease as the weight increases,
    the minimum gets code 0 and (up to rounding) the maximum code 15;
  - packing: element 8w+i sits in nibble i of word w (checked on a hand-built
    pattern).
"""
import numpy as np
import pytest

import oracle.moe_oracle as om
import oracle.quantize as oq


def _weights(seed, shape=(3, 16, 256), std=0.02):
    rng = np.random.default_rng(seed)
    return om.f64_to_bf16_bits(rng.normal(0.0, std, size=shape))


def check_error_bound(quantize):
    for seed, std in ((0, 0.02), (1, 1.0), (2, 1e-3)):
        w = _weights(seed, std=std)
        q, s, b = quantize(w)
        deq = om.dequant_q4(q, s, b)
        wf = om.bf16_bits_to_f64(w)
        sf = np.repeat(om.bf16_bits_to_f64(s), 64, axis=-1)
        err = np.abs(deq - wf)
        assert np.all(err <= 0.5 * sf * (1 + 2.0 ** -20) + 2.0 ** -24 * np.abs(wf)), float(np.max(err / sf))


def check_grid_round_trip(quantize):
    rng = np.random.default_rng(5)
    N, K = 8, 256
    q0 = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    q0[:, ::64] = 0                                   # every group reaches both ends of the grid
    q0[:, 1::64] = 15
    s0 = 2.0 ** rng.integers(-9, -3, size=(N, K // 64))
    b0 = -8 * s0 + s0 * rng.integers(-3, 4, size=(N, K // 64))
    w = s0.repeat(64, -1) * q0 + b0.repeat(64, -1)    # exact in bf16: 4-bit code times a power of two
    wb = om.f64_to_bf16_bits(w)
    assert np.array_equal(om.bf16_bits_to_f64(wb), w)
    q, s, b = quantize(wb)
    assert np.array_equal(om.unpack_q4(q), q0)
    assert np.array_equal(om.bf16_bits_to_f64(s), s0)
    assert np.array_equal(om.bf16_bits_to_f64(b), b0)


def check_constant_groups(quantize):
    w = np.full((2, 128), 0x3F40, np.uint16)          # 0.75 everywhere
    w[1, 64:] = 0xBC00                                # -0.0078125 in the second group of row 1
    q, s, b = quantize(w)
    assert np.all(om.unpack_q4(q) == 0)
    assert np.all(s == 0)
    assert np.array_equal(b, np.array([[0x3F40, 0x3F40], [0x3F40, 0xBC00]], np.uint16))


def check_order(quantize):
    w = _weights(7, shape=(4, 512))
    q, s, b = quantize(w)
    qq = om.unpack_q4(q).reshape(4, 8, 64)
    wf = om.bf16_bits_to_f64(w).reshape(4, 8, 64)
    for r in range(4):
        for g in range(8):
            o = np.argsort(wf[r, g], kind="stable")
            assert np.all(np.diff(qq[r, g][o].astype(int)) >= 0)
            assert qq[r, g][o[0]] == 0
            assert qq[r, g][o[-1]] >= 14


def check_packing(quantize):
    # weights 0..15 in one group (levels of the exact grid s = 1, b = 0),
    # repeated four times; element 8w+i must land in nibble i of word w
    vals = np.tile(np.arange(16, dtype=np.float64), 4)
    q, s, b = quantize(om.f64_to_bf16_bits(vals[None, :]))
    assert q.dtype == np.uint32 and q.shape == (1, 8)
    assert q[0, 0] == 0x76543210 and q[0, 1] == 0xFEDCBA98
    assert om.bf16_bits_to_f64(s)[0, 0] == 1.0 and om.bf16_bits_to_f64(b)[0, 0] == 0.0


def check_ties_to_even(quantize):
    # A hand-built group whose quotients (w - b)/s land exactly half-way between
    # two codes: lo = 0 and hi = 15 give s = 1 and b = 0 exactly, and every
    # value k + 1/2 (k = 0..14) is a bf16 number. Round half to even sends
    # 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, 3.5 -> 4, ..., 13.5 -> 14, 14.5 -> 14.
    # A second group is the same grid moved by -8 (lo = -8, hi = 7: b = -8, s = 1).
    halves = [k + 0.5 for k in range(15)]
    want = [0, 2, 2, 4, 4, 6, 6, 8, 8, 10, 10, 12, 12, 14, 14]
    g0 = [0.0, 15.0] + halves + [0.0] * (64 - 17)
    g1 = [v - 8.0 for v in g0]
    q, s, b = quantize(om.f64_to_bf16_bits(np.array([g0 + g1])))
    codes = om.unpack_q4(q)[0]
    assert om.bf16_bits_to_f64(s)[0].tolist() == [1.0, 1.0]
    assert om.bf16_bits_to_f64(b)[0].tolist() == [0.0, -8.0]
    for grp in (0, 1):
        c = codes[64 * grp: 64 * grp + 64]
        assert c[0] == 0 and c[1] == 15
        assert c[2:17].tolist() == want, c[2:17].tolist()


CHECKS = [check_error_bound, check_grid_round_trip, check_constant_groups, check_order, check_packing,
          check_ties_to_even]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_quantize_oracle_pin(check):
    check(oq.quantize_q4)


# ----------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ----------------------------------------------------------------------------

def _mut_divide_by_16(w_bits):
    wb = np.asarray(w_bits, np.uint16)
    w = (wb.astype(np.uint32) << 16).view(np.float32)
    g = w.reshape(*w.shape[:-1], -1, 64)
    lo = g.min(-1) + np.float32(0)
    s32 = (g.max(-1) - lo) / np.float32(16.0)
    s_bits = om.f64_to_bf16_bits(s32.astype(np.float64))
    s = (s_bits.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s[..., None] == 0, 0, np.clip(np.rint((g - lo[..., None]) / s[..., None]), 0, 15))
    return oq.pack_q4(q.reshape(w.shape).astype(np.uint8)), s_bits, (lo.view(np.uint32) >> 16).astype(np.uint16)


def _mut_truncate(w_bits):
    q, s, b = oq.quantize_q4(w_bits)
    wb = np.asarray(w_bits, np.uint16)
    w = (wb.astype(np.uint32) << 16).view(np.float32).reshape(*wb.shape[:-1], -1, 64)
    sf = (s.astype(np.uint32) << 16).view(np.float32)[..., None]
    lo = (b.astype(np.uint32) << 16).view(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        qq = np.where(sf == 0, 0, np.clip(np.floor((w - lo) / sf), 0, 15))
    return oq.pack_q4(qq.reshape(wb.shape).astype(np.uint8)), s, b


def _mut_nibbles_reversed(w_bits):
    q, s, b = oq.quantize_q4(w_bits)
    nib = om.unpack_q4(q)
    nib = nib.reshape(*nib.shape[:-1], -1, 8)[..., ::-1].reshape(nib.shape)
    return oq.pack_q4(nib), s, b


def _mut_max_as_bias(w_bits):
    q, s, b = oq.quantize_q4(w_bits)
    nib = 15 - om.unpack_q4(q)
    wb = np.asarray(w_bits, np.uint16)
    w = (wb.astype(np.uint32) << 16).view(np.float32).reshape(*wb.shape[:-1], -1, 64)
    hi = w.max(-1)
    neg = om.f64_to_bf16_bits(-om.bf16_bits_to_f64(s))
    return oq.pack_q4(nib.astype(np.uint8)), neg, (hi.view(np.uint32) >> 16).astype(np.uint16)


def _mut_round_half_up(w_bits):
    q, s, b = oq.quantize_q4(w_bits)
    wb = np.asarray(w_bits, np.uint16)
    w = (wb.astype(np.uint32) << 16).view(np.float32).reshape(*wb.shape[:-1], -1, 64)
    sf = (s.astype(np.uint32) << 16).view(np.float32)[..., None]
    lo = (b.astype(np.uint32) << 16).view(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        qq = np.where(sf == 0, 0, np.clip(np.floor((w - lo) / sf + np.float32(0.5)), 0, 15))
    return oq.pack_q4(qq.reshape(wb.shape).astype(np.uint8)), s, b


MUTANTS = [_mut_divide_by_16, _mut_truncate, _mut_nibbles_reversed, _mut_max_as_bias, _mut_round_half_up]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_planted_quantiser_mistake_is_caught(mutant):
    failed = 0
    for check in CHECKS:
        try:
            check(mutant)
        except AssertionError:
            failed += 1
    assert failed > 0, f"{mutant.__name__} passed every pin"


# ----------------------------------------------------------------------------
# prepacked layout (oracle/prepack.py)
# ----------------------------------------------------------------------------

def test_prepack_hand_worked_example():
    import json
    import os
    import oracle.prepack as op
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "prepack_small.json")))
    codes, sp, bp = op.prepack_q4(np.array(g["q"], np.uint32), np.array(g["s"], np.uint16),
                                  np.array(g["b"], np.uint16))
    assert codes.tolist() == g["codes"]
    assert sp.tolist() == g["s_pairs"]
    assert bp.tolist() == g["b_pairs"]


def test_prepack_is_a_permutation_that_keeps_the_weights():
    # every word and every scale/bias moves and none changes: the dequantised
    # matrices rebuilt from the prepacked arrays by index are the canonical ones
    import oracle.prepack as op
    rng = np.random.default_rng(3)
    n, N, K = 3, 48, 256
    G = K // 64
    q = rng.integers(0, 2**32, size=(n, N, K // 8), dtype=np.uint32)
    s = rng.integers(0, 2**16, size=(n, N, G), dtype=np.uint16)
    b = rng.integers(0, 2**16, size=(n, N, G), dtype=np.uint16)
    codes, sp, bp = op.prepack_q4(q, s, b)
    assert codes.shape == (n, G, N, 8) and sp.shape == (n, G // 2, N) and bp.shape == (n, G // 2, N)
    assert sorted(codes.ravel().tolist()) == sorted(q.ravel().tolist())
    for e, r, w in ((0, 0, 0), (2, 47, 31), (1, 17, 13)):
        assert codes[e, w // 8, r, w % 8] == q[e, r, w]
    for e, r, gg in ((0, 0, 0), (2, 47, 3), (1, 5, 2)):
        assert (sp[e, gg // 2, r] >> (16 * (gg % 2))) & 0xFFFF == s[e, r, gg]
        assert (bp[e, gg // 2, r] >> (16 * (gg % 2))) & 0xFFFF == b[e, r, gg]
    with pytest.raises(ValueError):
        op.prepack_q4(q[:, :, :24], s[:, :, :3], b[:, :, :3])   # an odd number of groups


def test_prepack_planted_mistakes_fail_the_hand_worked_example():
    import json
    import os
    import oracle.prepack as op
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "prepack_small.json")))
    q, s, b = np.array(g["q"], np.uint32), np.array(g["s"], np.uint16), np.array(g["b"], np.uint16)

    def halves_swapped(q, s, b):
        c, sp, bp = op.prepack_q4(q, s, b)
        return c, (sp >> 16) | (sp << 16), bp

    def rows_then_groups(q, s, b):   # [n][N][G][8] left in row-major order
        c, sp, bp = op.prepack_q4(q, s, b)
        return q.reshape(q.shape[0], q.shape[1], -1, 8), sp, bp

    for mut in (halves_swapped, rows_then_groups):
        c, sp, bp = mut(q, s, b)
        assert (c.tolist() != g["codes"]) or (sp.tolist() != g["s_pairs"]) or (bp.tolist() != g["b_pairs"])
