"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Routing tables are compared bit for bit given the same fp32 logits; bf16 layer
outputs must be within relative L2 <= 1e-3 and max-abs <= 2e-2 * max|ref| of
the oracle (which rounds only h and y to bf16); logits within 1e-4 of the
oracle's own; routing weights within 1e-6.
"""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as om
from int4_expert_routing_amd import _lib, ops
from synth import Q4Weights, make_config, make_layer
from tests.helpers import (LOGIT_ABS_TOL, WEIGHT_ABS_TOL, assert_close_bf16, rel_l2, max_abs_frac,
                           resample_close_calls, tiny_layer)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    _lib.load()   # raises when the library has not been built
    return torch.device("cuda:0")


def _np(t):
    return t.detach().cpu().numpy()


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------

def _logits(kind, T, E, seed):
    rng = np.random.default_rng(seed)
    if kind == "zeros":
        return np.zeros((T, E), np.float32)
    l = rng.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":
        l = (np.round(l * 2) / 2).astype(np.float32)
    if kind == "neginf":
        # -inf logits (weight 0): a random third of the entries, and on every
        # fourth token all but three experts, so that -inf entries fill the
        # end of the top-k (they tie and go in expert order)
        l[rng.random((T, E)) < 1 / 3] = -np.inf
        l[::4, 3:] = -np.inf
        l[::4, :3] = rng.standard_normal((l[::4].shape[0], 3))
    return l


ROUTE_CASES = [
    (4096, 256, 8, 64, "gauss"), (4096, 256, 8, 64, "zipf"), (37, 16, 2, 64, "gauss"),
    (64, 16, 2, 3, "ties"), (1, 256, 8, 64, "gauss"), (200, 8, 8, 16, "gauss"),
    (100, 32, 4, 64, "zeros"), (513, 256, 8, 64, "ties"), (32768, 256, 8, 64, "gauss"),
    (33, 256, 32, 1, "ties"), (257, 5, 3, 7, "gauss"),
    (3, 256, 8, 128, "neginf"), (16, 64, 8, 128, "neginf"), (1000, 256, 8, 128, "neginf"),
    # one token: the single-token tables (every count 0 or 1)
    (1, 8, 8, 1, "ties"), (1, 64, 32, 3, "neginf"), (1, 5, 3, 7, "gauss"), (1, 256, 32, 128, "zeros"),
    (1, 256, 1, 64, "zipf"),
    # one routing block of at most 64 pairs: the one-wave tables (repeated experts, several tiles per expert)
    (8, 16, 8, 3, "gauss"), (4, 8, 4, 1, "ties"), (16, 32, 4, 5, "zipf"), (2, 5, 3, 2, "gauss"),
    (8, 256, 8, 64, "zeros"), (6, 64, 8, 2, "neginf"), (32, 256, 2, 64, "gauss"),
    # scan and scatter in one launch at up to 256 routing blocks of 16 tokens (T <= 4096), as two launches
    # above: both sides of that boundary, and of 64 blocks (T = 1024, the router kernel's switch)
    (1024, 256, 8, 32, "gauss"), (1025, 256, 8, 32, "zipf"), (1024, 200, 32, 32, "ties"),
    (4097, 256, 8, 32, "zipf"), (4097, 200, 32, 32, "ties"), (4096, 256, 8, 128, "neginf"),
]


@pytest.mark.parametrize("T,E,k,bm,kind", ROUTE_CASES)
def test_route_matches_oracle_bit_exact(dev, T, E, k, bm, kind):
    print(f"route case T={T} E={E} k={k} bm={bm} {kind}", flush=True)
    l = _logits(kind, T, E, seed=T + E)
    bias = None
    if kind == "zipf":
        bias = (-1.2 * np.log(np.arange(1, E + 1))).astype(np.float32)
    out = ops.moe_route(torch.from_numpy(l).to(dev), k, bm,
                        logit_bias=None if bias is None else torch.from_numpy(bias).to(dev))
    torch.cuda.synchronize()
    lb = l if bias is None else (l + bias[None, :]).astype(np.float32)
    ids, w = om.select_topk(lb, k)
    tab = om.routing_tables(ids, E, bm)
    assert np.array_equal(_np(out["topk_ids"]), ids)
    assert np.max(np.abs(_np(out["topk_w"]) - w)) <= WEIGHT_ABS_TOL
    for name in ("counts", "offsets", "sorted_rows", "row_of_pair"):
        assert np.array_equal(_np(out[name]), tab[name]), name
    n = int(_np(out["num_tiles"])[0])
    assert n == int(tab["num_tiles"])
    assert np.array_equal(_np(out["tile_map"])[:n], tab["tile_map"])


# Seeded random routing calls (1 to 3000 tokens, 1 to 256 experts, top-k up to
# 32, any tile height, every logit kind, with and without a bias): the tables
# bit for bit against the oracle, through the same checks as the cases above.
def test_route_random_calls(dev):
    rng = np.random.default_rng(77)
    for case in range(60):
        E = int(rng.integers(1, 257))
        k = int(rng.integers(1, min(E, 32) + 1))
        T = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 1025)), int(rng.integers(1025, 3000))]))
        bm = int(rng.integers(1, 129))
        kind = str(rng.choice(["gauss", "ties", "zeros", "neginf", "zipf"]))
        test_route_matches_oracle_bit_exact(dev, T, E, k, bm, kind)


def test_route_is_deterministic(dev):
    l = torch.from_numpy(_logits("ties", 4096, 256, 3)).to(dev)
    a = ops.moe_route(l, 8, 64)
    b = ops.moe_route(l, 8, 64)
    torch.cuda.synchronize()
    for name in a:
        assert torch.equal(a[name], b[name]), name


# ----------------------------------------------------------------------------
# grouped GEMM (public entry point)
# ----------------------------------------------------------------------------

def _route_for(dev, T, E, k, seed):
    l = torch.from_numpy(_logits("gauss", T, E, seed)).to(dev)
    return ops.moe_route(l, k, ops.BLOCK_ROWS)


def test_gemm_integer_case_is_exact(dev):
    # s = 1, b = 0 and integer activations: every partial sum is an integer below
    # 2**24, so the fp32 result must equal the int64 product exactly
    T, E, k, N, K = 150, 4, 2, 256, 512
    rng = np.random.default_rng(1)
    xi = rng.integers(-16, 17, size=(T, K)).astype(np.float32)
    A = torch.from_numpy(xi).to(torch.bfloat16).to(dev)
    q = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32)
    one = np.full((E, N, K // 64), 0x3F80, np.uint16)
    zero = np.zeros((E, N, K // 64), np.uint16)
    W = ops.Q4Stack.from_host(Q4Weights(q, one, zero), dev)
    r = _route_for(dev, T, E, k, 5)
    out = ops.moe_grouped_gemm_q4(A, W, r["offsets"], r["tile_map"], r["num_tiles"], ops.MOE_EPI_STORE_F32,
                                  T * k, sorted_rows=r["sorted_rows"], row_div=k)
    torch.cuda.synchronize()
    got = _np(out).astype(np.float64)
    srt = _np(r["sorted_rows"])
    offs = _np(r["offsets"])
    qn = om.unpack_q4(q).astype(np.int64)
    want = np.zeros((T * k, N), np.int64)
    for e in range(E):
        rows = np.arange(offs[e], offs[e + 1])
        want[rows] = xi[srt[rows] // k].astype(np.int64) @ qn[e].T
    assert np.array_equal(got, want.astype(np.float64))


@pytest.mark.parametrize("bias_mode", ["sym", "random"])
def test_gemm_f32_matches_oracle(dev, bias_mode):
    T, E, k, N, K = 300, 8, 2, 256, 512
    inp = make_layer(T, K, N, E, k, seed=7, bias_mode=bias_mode)
    A = ops.bf16_from_bits(inp.x, dev)
    W = ops.Q4Stack.from_host(inp.gate, dev)   # gate is [E][N=I][K=H]: here N=256, K=512
    r = _route_for(dev, T, E, k, 9)
    out = ops.moe_grouped_gemm_q4(A, W, r["offsets"], r["tile_map"], r["num_tiles"], ops.MOE_EPI_STORE_F32,
                                  T * k, sorted_rows=r["sorted_rows"], row_div=k)
    torch.cuda.synchronize()
    got = _np(out).astype(np.float64)
    srt = _np(r["sorted_rows"])
    offs = _np(r["offsets"])
    x = om.bf16_bits_to_f64(inp.x)
    want = np.zeros((T * k, N))
    for e in range(E):
        rows = np.arange(offs[e], offs[e + 1])
        want[rows] = x[srt[rows] // k] @ om.expert_weights(inp.gate, e).T
    assert rel_l2(got, want) < 1e-5, rel_l2(got, want)
    assert max_abs_frac(got, want) < 1e-4


@pytest.mark.parametrize("K", [128, 256, 512, 640, 768, 1280, 2048])
def test_gemm_f32_small_tiles_every_group_count(dev, K):
    # ~6 rows per expert: every tile has one 32-row block and streams through
    # the deeper small-tile ring, whose waits differ for the first steps, the
    # last steps and K below 512
    print(f"gemm f32 small tiles K={K}", flush=True)
    T, E, k, N = 96, 32, 2, 256
    inp = make_layer(T, K, N, E, k, seed=K, bias_mode="random")
    A = ops.bf16_from_bits(inp.x, dev)
    W = ops.Q4Stack.from_host(inp.gate, dev)
    r = _route_for(dev, T, E, k, 21)
    out = ops.moe_grouped_gemm_q4(A, W, r["offsets"], r["tile_map"], r["num_tiles"], ops.MOE_EPI_STORE_F32,
                                  T * k, sorted_rows=r["sorted_rows"], row_div=k)
    torch.cuda.synchronize()
    got = _np(out).astype(np.float64)
    srt = _np(r["sorted_rows"])
    offs = _np(r["offsets"])
    assert np.diff(offs).max() <= 32
    x = om.bf16_bits_to_f64(inp.x)
    want = np.zeros((T * k, N))
    for e in range(E):
        rows = np.arange(offs[e], offs[e + 1])
        want[rows] = x[srt[rows] // k] @ om.expert_weights(inp.gate, e).T
    assert rel_l2(got, want) < 1e-5, rel_l2(got, want)
    assert max_abs_frac(got, want) < 1e-4


def test_gemm_f32_zero_and_spread_scales(dev):
    # Scales that are exactly 0 (a group, a column's first group, every group of
    # a column) and scales spread over 2^-12..2^12 inside one column: the
    # accumulator's unit must skip the zeros and follow the spread exactly
    # enough; the bias terms of zero-scale groups still count.
    T, E, k, N, K = 300, 8, 2, 256, 512
    inp = make_layer(T, K, N, E, k, seed=17, bias_mode="random")
    s = om.bf16_bits_to_f64(inp.gate.s).copy()
    G = K // 64
    rng = np.random.default_rng(3)
    s[:, 0:8, 0] = 0.0                      # first group of columns 0..7
    s[:, 8:16, :] = 0.0                     # every group of columns 8..15
    s[:, 16:64, 3] = 0.0                    # one middle group
    spread = 2.0 ** rng.integers(-12, 13, size=(E, 64, G))
    s[:, 64:128, :] *= spread               # power-of-two spread (exact in bf16)
    gate = Q4Weights(inp.gate.q, om.f64_to_bf16_bits(s), inp.gate.b)
    A = ops.bf16_from_bits(inp.x, dev)
    W = ops.Q4Stack.from_host(gate, dev)
    r = _route_for(dev, T, E, k, 19)
    out = ops.moe_grouped_gemm_q4(A, W, r["offsets"], r["tile_map"], r["num_tiles"], ops.MOE_EPI_STORE_F32,
                                  T * k, sorted_rows=r["sorted_rows"], row_div=k)
    torch.cuda.synchronize()
    got = _np(out).astype(np.float64)
    srt = _np(r["sorted_rows"])
    offs = _np(r["offsets"])
    x = om.bf16_bits_to_f64(inp.x)
    want = np.zeros((T * k, N))
    for e in range(E):
        rows = np.arange(offs[e], offs[e + 1])
        want[rows] = x[srt[rows] // k] @ om.expert_weights(gate, e).T
    for lo, hi in ((0, 16), (16, 64), (64, 128), (128, N)):
        assert rel_l2(got[:, lo:hi], want[:, lo:hi]) < 1e-5, (lo, hi, rel_l2(got[:, lo:hi], want[:, lo:hi]))


def test_gemm_swiglu_matches_oracle(dev):
    T, E, k, I, H = 200, 8, 2, 128, 512
    inp = make_layer(T, H, I, E, k, seed=11, bias_mode="random")
    A = ops.bf16_from_bits(inp.x, dev)
    Wg = ops.Q4Stack.from_host(inp.gate, dev)
    Wu = ops.Q4Stack.from_host(inp.up, dev)
    r = _route_for(dev, T, E, k, 13)
    out = ops.moe_grouped_gemm_q4(A, Wg, r["offsets"], r["tile_map"], r["num_tiles"], ops.MOE_EPI_SWIGLU_BF16,
                                  T * k, W1=Wu, sorted_rows=r["sorted_rows"], row_div=k)
    torch.cuda.synchronize()
    got = ops.bits_from_bf16(out)
    srt = _np(r["sorted_rows"])
    offs = _np(r["offsets"])
    x = om.bf16_bits_to_f64(inp.x)
    want = np.zeros((T * k, I))
    for e in range(E):
        rows = np.arange(offs[e], offs[e + 1])
        xs = x[srt[rows] // k]
        g = xs @ om.expert_weights(inp.gate, e).T
        u = xs @ om.expert_weights(inp.up, e).T
        want[rows] = om.round_bf16(om.silu(g) * u)
    gotf = om.bf16_bits_to_f64(got)
    assert_close_bf16(gotf, want, "SwiGLU h")
    # nearly every element rounds to the same bf16 value as the exact reference
    assert np.mean(gotf == want) > 0.98


# Seeded random grouped GEMM calls through the C ABI: 1 to 64 experts, 1 to
# 700 tokens, reduction lengths 128..2048, both epilogues, both weight layouts
# (canonical and prepacked give the same bits), against the fp64 oracle.
def test_gemm_random_calls(dev):
    rng = np.random.default_rng(99)
    for case in range(24):
        E = int(rng.integers(1, 65))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 701))
        K = 128 * int(rng.integers(1, 17))
        swiglu = bool(rng.random() < 0.5)
        N = 64 * int(rng.integers(1, 11)) if swiglu else 128 * int(rng.integers(1, 6))
        bias_mode = str(rng.choice(["sym", "random"]))
        print(f"gemm random case {case}: T={T} E={E} k={k} N={N} K={K} swiglu={swiglu} {bias_mode}", flush=True)
        inp = make_layer(T, K, N, E, k, seed=5000 + case, bias_mode=bias_mode)
        A = ops.bf16_from_bits(inp.x, dev)
        Wg = ops.Q4Stack.from_host(inp.gate, dev)
        Wu = ops.Q4Stack.from_host(inp.up, dev)
        r = _route_for(dev, T, E, k, 6000 + case)
        epi = ops.MOE_EPI_SWIGLU_BF16 if swiglu else ops.MOE_EPI_STORE_F32
        outs = []
        for packed in (False, True):
            w0 = ops.prepack_q4(Wg) if packed else Wg
            w1 = (ops.prepack_q4(Wu) if packed else Wu) if swiglu else None
            out = ops.moe_grouped_gemm_q4(A, w0, r["offsets"], r["tile_map"], r["num_tiles"], epi, T * k, W1=w1,
                                          sorted_rows=r["sorted_rows"], row_div=k)
            torch.cuda.synchronize()
            outs.append(out.clone())
        assert torch.equal(outs[0], outs[1]), (case, "layouts differ")
        srt, offs = _np(r["sorted_rows"]), _np(r["offsets"])
        x = om.bf16_bits_to_f64(inp.x)
        want = np.zeros((T * k, N))
        for e in range(E):
            rows = np.arange(offs[e], offs[e + 1])
            if rows.size == 0:
                continue
            xs = x[srt[rows] // k]
            g = xs @ om.expert_weights(inp.gate, e).T
            want[rows] = om.round_bf16(om.silu(g) * (xs @ om.expert_weights(inp.up, e).T)) if swiglu else g
        if swiglu:
            assert_close_bf16(om.bf16_bits_to_f64(ops.bits_from_bf16(outs[0])), want, f"case {case} h")
        else:
            got = _np(outs[0]).astype(np.float64)
            assert rel_l2(got, want) < 1e-5 and max_abs_frac(got, want) < 1e-4, case


@pytest.mark.parametrize("I", [64, 192])
def test_gemm_swiglu_half_column_tile(dev, I):
    # N % 128 == 64: the last 128-column slice has two live waves; the other
    # two stream the last 32 columns again and store nothing
    print(f"gemm swiglu N={I}", flush=True)
    T, E, k, H = 150, 8, 2, 256
    inp = make_layer(T, H, I, E, k, seed=23 + I, bias_mode="random")
    A = ops.bf16_from_bits(inp.x, dev)
    Wg = ops.Q4Stack.from_host(inp.gate, dev)
    Wu = ops.Q4Stack.from_host(inp.up, dev)
    r = _route_for(dev, T, E, k, 29)
    out = torch.full((T * k + 1, I), -7.0, dtype=torch.bfloat16, device=dev)   # one guard row
    ops.moe_grouped_gemm_q4(A, Wg, r["offsets"], r["tile_map"], r["num_tiles"], ops.MOE_EPI_SWIGLU_BF16,
                            T * k, W1=Wu, sorted_rows=r["sorted_rows"], row_div=k, out=out)
    torch.cuda.synchronize()
    gotf = om.bf16_bits_to_f64(ops.bits_from_bf16(out))
    assert np.all(gotf[T * k] == -7.0), "a store ran past the last row"
    srt = _np(r["sorted_rows"])
    offs = _np(r["offsets"])
    x = om.bf16_bits_to_f64(inp.x)
    want = np.zeros((T * k, I))
    for e in range(E):
        rows = np.arange(offs[e], offs[e + 1])
        xs = x[srt[rows] // k]
        want[rows] = om.round_bf16(om.silu(xs @ om.expert_weights(inp.gate, e).T) * (xs @ om.expert_weights(inp.up, e).T))
    assert_close_bf16(gotf[:T * k], want, "SwiGLU h, N % 128 == 64")


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------

def run_layer(dev, inp, block_rows=0):
    w = ops.MoEWeights.from_host(inp, dev)
    x = ops.bf16_from_bits(inp.x, dev)
    logits = torch.empty(inp.T, inp.E, dtype=torch.float32, device=dev)
    ids = torch.empty(inp.T, inp.k, dtype=torch.int32, device=dev)
    wts = torch.empty(inp.T, inp.k, dtype=torch.float32, device=dev)
    y = ops.moe_layer_forward(x, w, inp.k, logits_out=logits, topk_ids_out=ids, topk_w_out=wts,
                              block_rows=block_rows)
    torch.cuda.synchronize()
    return dict(y=om.bf16_bits_to_f64(ops.bits_from_bf16(y)), logits=_np(logits), ids=_np(ids), w=_np(wts))


def check_layer(inp, g, tokens=None):
    """Compare a GPU layer run with the oracle (routing from the GPU's own logits)."""
    own = om.router_logits(inp.x, inp.router_w, inp.logit_bias)
    assert np.max(np.abs(g["logits"].astype(np.float64) - own)) <= LOGIT_ABS_TOL
    ids, w = om.select_topk(g["logits"], inp.k)
    assert np.array_equal(g["ids"], ids), "top-k ids differ from the oracle on the same logits"
    assert np.max(np.abs(g["w"] - w)) <= WEIGHT_ABS_TOL
    if tokens is None:
        ref = om.moe_layer(inp, logits=g["logits"])["y"]
        got = g["y"]
    else:
        ref = om.round_bf16(om.moe_layer_tokens(inp, tokens, g["logits"]))
        got = g["y"][tokens]
    return assert_close_bf16(got, ref, "layer y")


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("bias_mode", ["sym", "random"])
def test_layer_tiny(dev, seed, bias_mode):
    print(f"layer tiny seed={seed} bias={bias_mode}", flush=True)
    inp = tiny_layer(seed, bias_mode)
    g = run_layer(dev, inp)
    check_layer(inp, g)
    # with the close calls resampled the GPU routes exactly like the fp64 logits
    ids_own, _ = om.select_topk(om.router_logits(inp.x, inp.router_w), inp.k)
    assert np.array_equal(g["ids"], ids_own)


def test_layer_tiny_zipf(dev):
    inp = tiny_layer(3, "random", zipf=1.2)
    check_layer(inp, run_layer(dev, inp))


@pytest.mark.parametrize("T", [1, 31, 33, 65, 100, 257])
def test_layer_ragged_token_counts(dev, T):
    print(f"layer ragged T={T}", flush=True)
    inp = make_layer(T, 256, 128, 16, 2, seed=T, bias_mode="random")
    check_layer(inp, run_layer(dev, inp))


@pytest.mark.parametrize("T,H,E,zipf", [(600, 512, 16, None), (1000, 256, 16, None), (1100, 512, 16, None),
                                         (3000, 256, 16, 1.2), (5000, 128, 16, None), (9000, 256, 16, 1.2),
                                         (2500, 256, 200, None)])
def test_layer_router_split_ranges(dev, T, H, E, zipf):
    # single-wave router tiles with K split 8 / 4 ways (T <= 1024), then the
    # 64 x 128 tile kernel with 8, 4, 2 and 1 K ranges; the logit bias is added
    # by the top-k kernel after a split and by the router without one; E = 200
    # leaves the last expert tile partly empty
    print(f"layer router split T={T} H={H} E={E} zipf={zipf}", flush=True)
    inp = make_layer(T, H, 128, E, 2, seed=T, bias_mode="random", zipf=zipf)
    check_layer(inp, run_layer(dev, inp))


def test_layer_k_equals_E(dev):
    inp = make_layer(40, 256, 128, 4, 4, seed=4, bias_mode="random")
    check_layer(inp, run_layer(dev, inp))


@pytest.mark.parametrize("T", [3, 40])
def test_layer_max_topk(dev, T):
    # k at its maximum (32 of 64 experts): the one-launch routing, the decode
    # kernels' 16-wave down+combine (T = 3) and the generic combine (T = 40)
    print(f"layer k=32 T={T}", flush=True)
    inp = make_layer(T, 256, 128, 64, 32, seed=50 + T, bias_mode="random")
    check_layer(inp, run_layer(dev, inp))


@pytest.mark.parametrize("T", [1, 3, 8, 40, 600])
def test_layer_graph_replays_match_eager(dev, T):
    # One layer call captured in a HIP graph (it records no allocation or
    # memset) and replayed three times, each after an eager call on other
    # tokens that overwrites the workspace: every replay gives the eager call's
    # bits, and the one-launch routing's counter (T <= 4) is back at zero.
    # Covers the one-launch, decode and prefill paths.
    print(f"layer graph T={T}", flush=True)
    H, I, E, k = 256, 128, 16, 2
    inp = make_layer(T, H, I, E, k, seed=70 + T, bias_mode="random")
    w = ops.MoEWeights.from_host(inp, dev)
    layer = ops.MoELayer(w, k, T)
    x = ops.bf16_from_bits(inp.x, dev)
    x2 = ops.bf16_from_bits(make_layer(T, H, I, E, k, seed=170 + T).x, dev)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    y2 = torch.empty_like(y)
    ids2 = torch.empty_like(ids)
    layer(x, y=y, topk_ids_out=ids)
    torch.cuda.synchronize()
    y_eager, ids_eager = y.clone(), ids.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer(x, y=y, topk_ids_out=ids)
    torch.cuda.synchronize()
    for _ in range(3):
        y.fill_(0)
        ids.fill_(-1)
        layer(x2, y=y2, topk_ids_out=ids2)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager) and torch.equal(ids, ids_eager)
        assert int(layer.workspace[:_lib.MOE_WORKSPACE_HEAD_BYTES].count_nonzero()) == 0
    ref = run_layer(dev, inp)
    assert np.array_equal(om.bf16_bits_to_f64(ops.bits_from_bf16(y)), ref["y"])
    # and the replayed output against the oracle, routed from the GPU's logits
    check_layer(inp, dict(ref, y=om.bf16_bits_to_f64(ops.bits_from_bf16(y))))


def test_layer_zero_tokens_is_a_noop(dev):
    inp = make_layer(3, 256, 128, 16, 2, seed=0)
    w = ops.MoEWeights.from_host(inp, dev)
    x = torch.empty(0, 256, dtype=torch.bfloat16, device=dev)
    y = ops.moe_layer_forward(x, w, 2)
    torch.cuda.synchronize()
    assert y.shape == (0, 256)


# Seeded random shapes across the supported range (H and I multiples of 128,
# E from 8 to 256, k up to 8, 9 to ~1800 tokens, both bias modes, some with a
# Zipf logit skew): the layer against the oracle, and the 32-row and 128-row
# tile geometries (one-column-block and two-block launches) bit for bit.
def test_layer_random_shapes(dev):
    rng = np.random.default_rng(2024)
    for case in range(30):
        E = int(rng.choice([8, 16, 24, 64, 100, 256]))
        k = int(rng.integers(1, min(E, 8) + 1))
        H = int(rng.choice([128, 256, 384, 512, 1024, 2048]))
        I = int(rng.choice([128, 256, 384, 512]))
        T = int(rng.integers(9, 1800 if H * I <= 256 * 512 else 500))
        bias_mode = str(rng.choice(["sym", "random"]))
        zipf = None if rng.random() < 0.7 else 1.2
        print(f"layer random case {case}: T={T} H={H} I={I} E={E} k={k} {bias_mode} zipf={zipf}", flush=True)
        inp = resample_close_calls(make_layer(T, H, I, E, k, seed=3000 + case, bias_mode=bias_mode, zipf=zipf))
        g = run_layer(dev, inp)
        g32 = run_layer(dev, inp, block_rows=32)
        g128 = run_layer(dev, inp, block_rows=128)
        assert np.array_equal(g32["y"], g128["y"]), (case, "32-row and 128-row tiles differ")
        assert np.array_equal(g["y"], g32["y"]), (case, "default tiles differ")
        check_layer(inp, g)


# Seeded random few-token calls (1 to 16 tokens: the one-launch routing, the
# decode kernels and the single routing block), some with a gate vector, each
# also through the persistent decode kernel where it applies: both against
# the oracle.
def test_layer_random_few_tokens(dev):
    rng = np.random.default_rng(4242)
    for case in range(30):
        E = int(rng.choice([8, 16, 32, 64, 128, 256]))
        k = int(rng.integers(1, min(E, 8) + 1))
        H = int(rng.choice([256, 512, 1024, 2048, 2560]))
        I = int(rng.choice([128, 256, 384, 512]))
        T = int(rng.integers(1, 17))
        gated = bool(rng.random() < 0.3)
        print(f"layer random few tokens {case}: T={T} H={H} I={I} E={E} k={k} gated={gated}", flush=True)
        inp = resample_close_calls(make_layer(T, H, I, E, k, seed=8000 + case,
                                              bias_mode=str(rng.choice(["sym", "random"])), gated_shared=gated))
        g = run_layer(dev, inp)
        check_layer(inp, g)
        w = ops.MoEWeights.from_host(inp, dev)
        yp = ops.moe_layer_forward(ops.bf16_from_bits(inp.x, dev), w, k, persistent_decode=True)
        torch.cuda.synchronize()
        ref = om.moe_layer(inp, logits=g["logits"])["y"]
        assert_close_bf16(om.bf16_bits_to_f64(ops.bits_from_bf16(yp)), ref, f"case {case} persistent")


def test_layer_is_deterministic(dev):
    inp = make_layer(300, 256, 128, 16, 2, seed=5, bias_mode="random")
    a = run_layer(dev, inp)
    b = run_layer(dev, inp)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_layer_workspace_reused_across_token_counts(dev):
    # Calls with T <= 4 route in one launch that counts finished workgroups in
    # and parks logits in the workspace's head and leaves it zero; reusing one
    # workspace across token counts (one-launch, decode and general paths)
    # must give the same bits as a fresh zeroed workspace, and end zeroed.
    # E = 12 leaves the last expert slice of the router half empty.
    print("layer workspace reuse, E=12 k=3, T = 1, 16, 40, 9, 3, 12", flush=True)
    H, I, E, k = 256, 256, 12, 3
    ws = torch.zeros(ops.workspace_bytes(40, H, I, E, k), dtype=torch.uint8, device=dev)
    for i, T in enumerate((1, 16, 40, 9, 3, 12)):
        inp = make_layer(T, H, I, E, k, seed=100 + i, bias_mode="random")
        w = ops.MoEWeights.from_host(inp, dev)
        x = ops.bf16_from_bits(inp.x, dev)
        logits = torch.empty(T, E, dtype=torch.float32, device=dev)
        ids = torch.empty(T, k, dtype=torch.int32, device=dev)
        wts = torch.empty(T, k, dtype=torch.float32, device=dev)
        y = ops.moe_layer_forward(x, w, k, logits_out=logits, topk_ids_out=ids, topk_w_out=wts, workspace=ws)
        torch.cuda.synchronize()
        g = dict(y=om.bf16_bits_to_f64(ops.bits_from_bf16(y)), logits=_np(logits), ids=_np(ids), w=_np(wts))
        fresh = run_layer(dev, inp)
        for key in g:
            assert np.array_equal(g[key], fresh[key]), (T, key)
        check_layer(inp, g)
        assert int(ws[:_lib.MOE_WORKSPACE_HEAD_BYTES].count_nonzero()) == 0, T


@pytest.mark.parametrize("name", ["decode1", "decode8"])
def test_layer_full_shape_decode(dev, name):
    print(f"layer {name}", flush=True)
    inp = make_config(name, seed=0, bias_mode="random")
    g = run_layer(dev, inp)
    check_layer(inp, g, tokens=list(range(inp.T)))


# Few-token calls (T <= 8) run the decode-shaped kernels; these shapes cover each
# of their reduction lengths (K = 256, 512, 1024, 2048) and every row count 1..8
# of a tile, with the general path just above the threshold (T = 9) beside them.
@pytest.mark.parametrize("T,H,I,E,k,bias_mode,seed", [
    (1, 256, 256, 16, 2, "random", 0),
    (2, 256, 256, 16, 2, "sym", 1),
    (3, 256, 256, 16, 2, "random", 2),
    (5, 1024, 512, 16, 4, "random", 3),
    (8, 256, 256, 16, 2, "random", 4),
    (8, 256, 256, 16, 16, "random", 5),      # k = E: every expert gets all 8 rows
    (7, 512, 1024, 32, 8, "sym", 6),
    (6, 256, 256, 5, 3, "random", 10),       # one-launch routing, 8-expert workgroups past E = 5
    (3, 512, 256, 5, 2, "random", 11),       # rows staged in LDS (3..4 tokens), experts past E
    (6, 4096, 256, 8, 2, "random", 12),      # H above the staged rows' limit: router + top-k launches
    (2, 2560, 256, 8, 2, "random", 13),      # H = 2560 (not a power of two), rows in registers
    (9, 256, 256, 16, 2, "random", 7),       # above the threshold: grouped GEMM path
])
def test_layer_few_tokens(dev, T, H, I, E, k, bias_mode, seed):
    print(f"layer few tokens T={T} H={H} I={I} E={E} k={k} {bias_mode} seed={seed}", flush=True)
    inp = resample_close_calls(make_layer(T=T, H=H, I=I, E=E, k=k, seed=seed, bias_mode=bias_mode))
    g = run_layer(dev, inp)
    check_layer(inp, g)


def test_layer_largest_reduction_sizes(dev):
    # H = I = 2048: both grouped GEMMs at their largest reduction length
    print("layer H=2048 I=2048 E=8 k=2 T=100", flush=True)
    inp = resample_close_calls(make_layer(T=100, H=2048, I=2048, E=8, k=2, seed=11, bias_mode="random"))
    check_layer(inp, run_layer(dev, inp))


@pytest.mark.parametrize("T,H,I", [(100, 4096, 512), (60, 2048, 2560), (5, 2560, 384), (3, 4096, 256)])
def test_layer_reduction_sizes_above_2048(dev, T, H, I):
    # reductions past 2048 (64 and 40 groups) in both grouped GEMMs; at T <= 8
    # these sizes run the grouped GEMM instead of the decode kernels
    print(f"layer T={T} H={H} I={I}", flush=True)
    inp = resample_close_calls(make_layer(T=T, H=H, I=I, E=8, k=2, seed=H + I, bias_mode="random"))
    check_layer(inp, run_layer(dev, inp))


@pytest.mark.parametrize("bm", [32, 64, 128])
@pytest.mark.parametrize("T,E,k", [(300, 16, 2), (700, 64, 8), (6, 16, 2)])
def test_layer_routed_tile_heights(dev, bm, T, E, k):
    # routed tiles of 32, 64 or 128 rows (the shared expert: 32-row tiles in the
    # one-column-block launches of bm = 32, else 128-row tiles)
    print(f"layer block_rows={bm} T={T} E={E} k={k}", flush=True)
    inp = make_layer(T, 256, 128, E, k, seed=bm + T, bias_mode="random")
    g = run_layer(dev, inp, block_rows=bm)
    check_layer(inp, g)
    if bm != 128:
        ref = run_layer(dev, inp, block_rows=128)
        assert np.array_equal(g["ids"], ref["ids"])


# 32-row tiles run the grouped GEMMs as one-column-block launches (five
# workgroups per CU, gate and up meeting in LDS); 128-row tiles as two-block
# launches. Each output element is the same chain of operations either way,
# so the two agree bit for bit, and both match the oracle: shared tiles of 32
# rows with a ragged last one, experts spread over several 32-row tiles (Zipf),
# reduction lengths with 2 to 32 groups.
@pytest.mark.parametrize("T,H,I,E,k,zipf", [(300, 512, 256, 32, 4, None), (161, 256, 128, 8, 2, 1.2),
                                            (97, 2048, 512, 64, 8, None), (40, 128, 1024, 16, 2, None),
                                            (1200, 2048, 512, 256, 8, None)])
def test_layer_one_block_launches_match_two_block(dev, T, H, I, E, k, zipf):
    print(f"layer one-block vs two-block T={T} H={H} I={I} E={E} k={k} zipf={zipf}", flush=True)
    inp = resample_close_calls(make_layer(T, H, I, E, k, seed=70 + T, bias_mode="random", zipf=zipf))
    g32 = run_layer(dev, inp, block_rows=32)
    g128 = run_layer(dev, inp, block_rows=128)
    assert np.array_equal(g32["ids"], g128["ids"])
    assert np.array_equal(g32["y"], g128["y"]), "32-row and 128-row tiles give different bits"
    check_layer(inp, g32)


@pytest.mark.parametrize("T,H,I,E,k", [(64, 256, 128, 16, 2), (1, 256, 256, 16, 2), (3, 512, 256, 16, 4),
                                       (8, 256, 256, 16, 2), (300, 512, 256, 32, 4)])
def test_layer_gated_shared_expert(dev, T, H, I, E, k):
    # the shared expert scaled by sigmoid(x . w_sg): combine kernel (T > 8)
    # and fused down + combine (T <= 8)
    print(f"layer gated shared T={T} H={H} I={I} E={E} k={k}", flush=True)
    inp = resample_close_calls(make_layer(T, H, I, E, k, seed=90 + T, bias_mode="random", gated_shared=True))
    g = run_layer(dev, inp)
    check_layer(inp, g)
    # the gate matters: the ungated layer differs
    plain = dict(vars(inp))
    plain["shared_gate"] = None
    ref_plain = om.moe_layer(type(inp)(**plain), logits=g["logits"])["y"]
    assert rel_l2(g["y"], ref_plain) > 1e-2


@pytest.mark.parametrize("name", ["decode1", "decode8", "prefill512", "prefill4096"])
def test_layer_full_shape_gated_shared_expert(dev, name):
    print(f"layer {name} gated shared expert", flush=True)
    inp = make_config(name, seed=3, bias_mode="random", gated_shared=True)
    check_layer(inp, run_layer(dev, inp))


def _run_layer_streams(dev, inp, side, k_graph=False):
    w = ops.MoEWeights.from_host(inp, dev)
    layer = ops.MoELayer(w, inp.k, inp.T, side_stream=side)
    x = ops.bf16_from_bits(inp.x, dev)
    logits = torch.empty(inp.T, inp.E, dtype=torch.float32, device=dev)
    ids = torch.empty(inp.T, inp.k, dtype=torch.int32, device=dev)
    wts = torch.empty(inp.T, inp.k, dtype=torch.float32, device=dev)
    y = torch.empty(inp.T, inp.H, dtype=torch.bfloat16, device=dev)
    layer(x, y=y, logits_out=logits, topk_ids_out=ids, topk_w_out=wts)
    torch.cuda.synchronize()
    return dict(y=om.bf16_bits_to_f64(ops.bits_from_bf16(y)), logits=_np(logits), ids=_np(ids), w=_np(wts)), layer


@pytest.mark.parametrize("name,T,gated", [("tiny", None, False), ("tiny", 1, False), ("tiny", 6, True),
                                          ("tiny", 200, True), ("prefill4096", None, False),
                                          ("decode1", None, True), ("decode8", None, False)])
def test_layer_side_stream_matches_one_stream(dev, name, T, gated):
    # the shared expert's tiles on a second stream (forked after the activation
    # prep, joined before the combine) give the one-stream bits
    print(f"layer side stream {name} T={T} gated={gated}", flush=True)
    over = {} if T is None else {"T": T}
    inp = make_config(name, seed=7, bias_mode="random", gated_shared=gated, **over)
    one, _ = _run_layer_streams(dev, inp, False)
    two, _ = _run_layer_streams(dev, inp, True)
    for key in one:
        assert np.array_equal(one[key], two[key]), key
    check_layer(inp, two, tokens=None if inp.T <= 512 else list(range(0, inp.T, 97)))


@pytest.mark.parametrize("T", [2, 8, 300])
def test_layer_side_stream_graph_replays(dev, T):
    # captured with the side stream forked and joined inside the capture;
    # every replay (after eager calls on other tokens) matches the eager bits
    print(f"layer side stream graph T={T}", flush=True)
    H, I, E, k = 256, 128, 16, 2
    inp = make_layer(T, H, I, E, k, seed=80 + T, bias_mode="random", gated_shared=True)
    g, layer = _run_layer_streams(dev, inp, True)
    x = ops.bf16_from_bits(inp.x, dev)
    x2 = ops.bf16_from_bits(make_layer(T, H, I, E, k, seed=180 + T).x, dev)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    y2 = torch.empty_like(y)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer(x, y=y)
    torch.cuda.synchronize()
    for _ in range(3):
        y.fill_(0)
        layer(x2, y=y2)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(om.bf16_bits_to_f64(ops.bits_from_bf16(y)), g["y"])
    check_layer(inp, g)


def _head_ok(ws):
    """The one-launch routing's part of the workspace head is back at zero and
    the persistent decode kernel's status word is clear."""
    st = int(ws[_lib.MOE_WORKSPACE_STATUS_OFFSET:_lib.MOE_WORKSPACE_STATUS_OFFSET + 4].view(torch.int32).item())
    return int(ws[:8448].count_nonzero()) == 0 and st == 0


@pytest.mark.parametrize("T,I,E,k,bias_mode", [(1, 512, 256, 8, "random"), (2, 512, 256, 8, "sym"),
                                               (3, 256, 64, 4, "random"), (4, 512, 256, 8, "random"),
                                               (5, 512, 32, 8, "random"), (6, 256, 16, 2, "random"),
                                               (7, 512, 256, 8, "sym"), (8, 512, 256, 8, "random"),
                                               (8, 512, 8, 8, "random"), (3, 512, 256, 1, "random")])
def test_layer_persistent_decode_kernel(dev, T, I, E, k, bias_mode):
    # H = 2048, T <= 8, persistent_decode: the whole layer runs as one
    # persistent launch; it must match the oracle, and (T <= 4, where both
    # routers sum the logits in the same order) its bits must equal the
    # three-launch path's
    print(f"persistent decode T={T} I={I} E={E} k={k} {bias_mode}", flush=True)
    inp = resample_close_calls(make_layer(T, 2048, I, E, k, seed=300 + T + k, bias_mode=bias_mode))
    w = ops.MoEWeights.from_host(inp, dev)
    x = ops.bf16_from_bits(inp.x, dev)
    one = ops.MoELayer(w, k, T, persistent_decode=True)
    outs = []
    for layer, kw in ((one, {}), (ops.MoELayer(w, k, T), {})):
        y = torch.empty(T, 2048, dtype=torch.bfloat16, device=dev)
        lg = torch.empty(T, E, dtype=torch.float32, device=dev)
        ids = torch.empty(T, k, dtype=torch.int32, device=dev)
        wt = torch.empty(T, k, dtype=torch.float32, device=dev)
        layer(x, y=y, logits_out=lg, topk_ids_out=ids, topk_w_out=wt)
        torch.cuda.synchronize()
        outs.append(dict(y=om.bf16_bits_to_f64(ops.bits_from_bf16(y)), logits=_np(lg), ids=_np(ids), w=_np(wt)))
    assert _head_ok(one.workspace)
    check_layer(inp, outs[0])
    check_layer(inp, outs[1])
    if T <= 4:
        for key in outs[0]:
            assert np.array_equal(outs[0][key], outs[1][key]), key


def test_layer_persistent_decode_graph_replays(dev):
    # the tags of one call never serve the next: a captured call replayed
    # between eager calls of other token counts (1 .. 8) in the same workspace
    print("persistent decode graph replays", flush=True)
    H, I, E, k = 2048, 512, 64, 4
    inp = make_layer(8, H, I, E, k, seed=61, bias_mode="random", gated_shared=True)
    w = ops.MoEWeights.from_host(inp, dev)
    layer = ops.MoELayer(w, k, 8, persistent_decode=True)
    xs = {T: ops.bf16_from_bits(make_layer(T, H, I, E, k, seed=400 + T).x, dev) for T in range(1, 9)}
    x = ops.bf16_from_bits(inp.x, dev)
    y = torch.empty(8, H, dtype=torch.bfloat16, device=dev)
    lg = torch.empty(8, E, dtype=torch.float32, device=dev)
    ids = torch.empty(8, k, dtype=torch.int32, device=dev)
    wt = torch.empty(8, k, dtype=torch.float32, device=dev)
    layer(x, y=y, logits_out=lg, topk_ids_out=ids, topk_w_out=wt)
    torch.cuda.synchronize()
    y_eager = y.clone()
    g = dict(y=om.bf16_bits_to_f64(ops.bits_from_bf16(y_eager)), logits=_np(lg), ids=_np(ids), w=_np(wt))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer(x, y=y)
    torch.cuda.synchronize()
    for T in (1, 5, 8, 2, 3):
        y.fill_(0)
        layer(xs[T], y=torch.empty(T, H, dtype=torch.bfloat16, device=dev))
        graph.replay()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), T
    assert _head_ok(layer.workspace)
    check_layer(inp, g)


def test_layer_decode8_zipf_seeds(dev):
    print("layer decode8 zipf seeds 1, 2", flush=True)
    for seed in (1, 2):
        inp = make_config("decode8", seed=seed, bias_mode="random", zipf=1.2)
        check_layer(inp, run_layer(dev, inp), tokens=list(range(inp.T)))


@pytest.mark.parametrize("bias_mode", ["sym", "random"])
def test_layer_full_shape_prefill512_all_tokens(dev, bias_mode):
    print(f"layer prefill512 {bias_mode}", flush=True)
    inp = make_config("prefill512", seed=1, bias_mode=bias_mode)
    check_layer(inp, run_layer(dev, inp))


@pytest.mark.parametrize("name,bias_mode", [("prefill4096", "sym"), ("prefill4096", "random"),
                                            ("prefill4096_zipf", "sym"), ("prefill4096_zipf", "random")])
def test_layer_full_shape_prefill4096_all_tokens(dev, name, bias_mode):
    # every token of the benchmark workload against the full fp64 layer oracle
    print(f"layer {name} {bias_mode}", flush=True)
    inp = make_config(name, seed=0, bias_mode=bias_mode)
    check_layer(inp, run_layer(dev, inp))


def _tile_covering_tokens(logits, k, bm, n_random, seed):
    """Tokens whose rows sit at the first, a middle and the last row of routed
    tiles of every live 32-row block count (1..4), at the edges of the shared
    expert's 128-row tiles, plus random ones."""
    ids, _ = om.select_topk(logits, k)
    tab = om.routing_tables(ids, logits.shape[1], bm)
    offs, srt = tab["offsets"], tab["sorted_rows"]
    T = logits.shape[0]
    picked = set()
    by_blocks = {1: [], 2: [], 3: [], 4: []}
    for e, r0 in tab["tile_map"].tolist():
        r1 = min(r0 + bm, int(offs[e + 1]))
        by_blocks[-(-(r1 - r0) // 32)].append((r0, r1))
    for nb, tiles in by_blocks.items():
        for r0, r1 in tiles[:: max(1, len(tiles) // 12)]:
            for r in (r0, (r0 + r1) // 2, r1 - 1):
                picked.add(int(srt[r]) // k)
    for t0 in range(0, T, 128 * 37):
        picked.update({t0, min(t0 + 127, T - 1)})
    picked.update({0, T - 1})
    rng = np.random.default_rng(seed)
    picked.update(rng.choice(T, n_random, replace=False).tolist())
    return sorted(picked), by_blocks


def test_layer_full_shape_prefill32768_sampled(dev):
    print("layer prefill32768", flush=True)
    inp = make_config("prefill32768", seed=0, bias_mode="random")
    g = run_layer(dev, inp)
    toks, by_blocks = _tile_covering_tokens(g["logits"], inp.k, ops.BLOCK_ROWS, 360, 0)
    assert all(by_blocks[n] for n in (1, 2, 3, 4)), {n: len(v) for n, v in by_blocks.items()}
    assert len(toks) >= 512, len(toks)
    check_layer(inp, g, tokens=toks)
