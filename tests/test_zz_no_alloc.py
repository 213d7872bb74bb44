"""GPU: the no-allocation layer entry point (moe_layer_forward_noalloc, for
callers that cannot allocate) against the workspace entry point, through the
C ABI: identical bits on consecutive calls, the second one smaller, on the
prefill and decode paths, and the size limit reported before any launch."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as om
from int4_expert_routing_amd import _lib, ops
from synth import make_config, make_layer
from tests.test_gpu_parity import check_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    _lib.load()
    return torch.device("cuda:0")


def _outs(dev, T, E, k, H):
    return (torch.full((T, H), -3.0, dtype=torch.bfloat16, device=dev), torch.empty(T, E, dtype=torch.float32, device=dev),
            torch.empty(T, k, dtype=torch.int32, device=dev), torch.empty(T, k, dtype=torch.float32, device=dev))


def _both(dev, inp):
    w = ops.MoEWeights.from_host(inp, dev)
    x = ops.bf16_from_bits(inp.x, dev)
    y, l, i, wt = _outs(dev, inp.T, inp.E, inp.k, inp.H)
    ops.moe_layer_forward_noalloc(x, w, inp.k, y, logits_out=l, topk_ids_out=i, topk_w_out=wt)
    y2, l2, i2, wt2 = _outs(dev, inp.T, inp.E, inp.k, inp.H)
    ops.moe_layer_forward(x, w, inp.k, y=y2, logits_out=l2, topk_ids_out=i2, topk_w_out=wt2)
    torch.cuda.synchronize()
    for a, b, n in ((y, y2, "y"), (l, l2, "logits"), (i, i2, "ids"), (wt, wt2, "weights")):
        assert torch.equal(a, b), n
    g = dict(y=om.bf16_bits_to_f64(ops.bits_from_bf16(y)), logits=l.cpu().numpy(), ids=i.cpu().numpy(),
             w=wt.cpu().numpy())
    return g


@pytest.mark.parametrize("shapes", [
    [("prefill4096", 300), ("prefill4096", 40)],     # grouped-GEMM path, then a smaller call
    [("decode8", None), ("decode1", None)],          # decode path, then the one-launch routing
    [("tiny", None), ("tiny", 3), ("tiny", 1)],
])
def test_noalloc_matches_workspace_entry_point(dev, shapes):
    for name, T in shapes:
        print(f"noalloc {name} T={T}", flush=True)
        over = {} if T is None else {"T": T}
        inp = make_config(name, seed=11, bias_mode="random", **over)
        g = _both(dev, inp)
        check_layer(inp, g, tokens=None if inp.T <= 64 else list(range(0, inp.T, 7)))


def test_noalloc_rejects_sizes_beyond_its_array(dev):
    inp = make_layer(4096, 2048, 512, 256, 8, seed=0)
    assert ops.workspace_bytes(4096, 2048, 512, 256, 8) > _lib.MOE_NOALLOC_SCRATCH_BYTES
    w = ops.MoEWeights.from_host(make_layer(1, 2048, 512, 256, 8, seed=0), dev)
    x = torch.zeros(4096, 2048, dtype=torch.bfloat16, device=dev)
    y = torch.full((4096, 2048), 5.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(_lib.MoeError) as e:
        ops.moe_layer_forward_noalloc(x, w, 8, y)
    assert e.value.status == _lib.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 5.0).all()), "a rejected call launched work"
    del inp
