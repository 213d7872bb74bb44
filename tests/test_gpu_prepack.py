"""GPU: the prepacked 4-bit layout. moe_prepack_q4 against the CPU oracle of
the permutation (bit for bit), and every entry point on prepacked weights
against the same call on canonical weights (bit for bit: the values and the
arithmetic are the same) and against the layer oracle."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as om
import oracle.prepack as op
from int4_expert_routing_amd import _lib, ops
from synth import Q4Weights, make_config, make_layer
from tests.helpers import resample_close_calls
from tests.test_gpu_parity import _route_for, check_layer, run_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    _lib.load()
    return torch.device("cuda:0")


@pytest.mark.parametrize("n,N,K", [(1, 2, 128), (3, 48, 256), (5, 512, 2048), (2, 2048, 512), (257, 64, 384)])
def test_prepack_matches_oracle(dev, n, N, K):
    print(f"prepack n={n} N={N} K={K}", flush=True)
    rng = np.random.default_rng(n * N + K)
    q = rng.integers(0, 2**32, size=(n, N, K // 8), dtype=np.uint32)
    s = rng.integers(0, 2**16, size=(n, N, K // 64), dtype=np.uint16)
    b = rng.integers(0, 2**16, size=(n, N, K // 64), dtype=np.uint16)
    packed = ops.prepack_q4(ops.Q4Stack.from_host(Q4Weights(q, s, b), dev))
    torch.cuda.synchronize()
    codes, sp, bp = op.prepack_q4(q, s, b)
    assert np.array_equal(packed.q.cpu().numpy().view(np.uint32), codes)
    assert np.array_equal(packed.s.cpu().numpy().view(np.uint32), sp)
    assert np.array_equal(packed.b.cpu().numpy().view(np.uint32), bp)


def _layer(dev, inp, w, **kw):
    x = ops.bf16_from_bits(inp.x, dev)
    logits = torch.empty(inp.T, inp.E, dtype=torch.float32, device=dev)
    ids = torch.empty(inp.T, inp.k, dtype=torch.int32, device=dev)
    wts = torch.empty(inp.T, inp.k, dtype=torch.float32, device=dev)
    y = ops.moe_layer_forward(x, w, inp.k, logits_out=logits, topk_ids_out=ids, topk_w_out=wts, **kw)
    torch.cuda.synchronize()
    return dict(y=om.bf16_bits_to_f64(ops.bits_from_bf16(y)), logits=logits.cpu().numpy(), ids=ids.cpu().numpy(),
                w=wts.cpu().numpy())


@pytest.mark.parametrize("name,T,gated,stacks", [
    ("tiny", None, False, "all"), ("tiny", 3, True, "all"), ("tiny", 8, False, "gate_up"),
    ("decode1", None, False, "all"), ("decode8", None, True, "all"), ("prefill512", None, False, "all"),
    ("prefill4096", None, False, "all"), ("prefill4096", 700, False, "down"),
])
def test_layer_prepacked_matches_canonical(dev, name, T, gated, stacks):
    print(f"layer prepacked {name} T={T} gated={gated} stacks={stacks}", flush=True)
    over = {} if T is None else {"T": T}
    inp = make_config(name, seed=5, bias_mode="random", gated_shared=gated, **over)
    w = ops.MoEWeights.from_host(inp, dev)
    sel = {"all": ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"), "gate_up": ("gate", "up", "sh_gate", "sh_up"),
           "down": ("down", "sh_down")}[stacks]
    a = _layer(dev, inp, w)
    b = _layer(dev, inp, w.prepacked(sel))
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    check_layer(inp, b, tokens=None if inp.T <= 512 else list(range(0, inp.T, 31)))


@pytest.mark.parametrize("epi", [ops.MOE_EPI_STORE_F32, ops.MOE_EPI_SWIGLU_BF16])
@pytest.mark.parametrize("K", [128, 512, 2048])
def test_grouped_gemm_prepacked_matches_canonical(dev, epi, K):
    T, E, k, N = 200, 8, 2, 256
    inp = make_layer(T, K, N, E, k, seed=K + epi, bias_mode="random")
    A = ops.bf16_from_bits(inp.x, dev)
    Wg, Wu = ops.Q4Stack.from_host(inp.gate, dev), ops.Q4Stack.from_host(inp.up, dev)
    r = _route_for(dev, T, E, k, 41)
    outs = []
    for g_, u_ in ((Wg, Wu), (ops.prepack_q4(Wg), ops.prepack_q4(Wu))):
        outs.append(ops.moe_grouped_gemm_q4(A, g_, r["offsets"], r["tile_map"], r["num_tiles"], epi, T * k,
                                            W1=u_ if epi == ops.MOE_EPI_SWIGLU_BF16 else None,
                                            sorted_rows=r["sorted_rows"], row_div=k))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_layer_rejects_mixed_gate_up_layouts(dev):
    inp = make_config("tiny", seed=1)
    w = ops.MoEWeights.from_host(inp, dev)
    with pytest.raises(_lib.MoeError) as e:
        _layer(dev, inp, w.prepacked(("gate",)))
    assert e.value.status == _lib.MOE_ERR_SHAPE
