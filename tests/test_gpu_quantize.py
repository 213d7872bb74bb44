"""GPU parity of the quantiser (moe_quantize_q4) with its oracle: codes, scales
and biases must be bit-identical; the quantised stack must then run in the
layer like any other weights."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as om
import oracle.quantize as oq
from int4_expert_routing_amd import _lib, ops

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    _lib.load()
    return torch.device("cuda:0")


def _gpu_quantize(dev, w_bits):
    shape = w_bits.shape
    w3 = np.ascontiguousarray(w_bits).reshape(-1, shape[-2], shape[-1]) if len(shape) > 2 else w_bits[None]
    w = torch.from_numpy(np.ascontiguousarray(w3).view(np.int16)).view(torch.bfloat16).to(dev)
    st = ops.quantize_q4(w)
    torch.cuda.synchronize()
    q = st.q.cpu().numpy().view(np.uint32).reshape(*shape[:-1], -1)
    s = st.s.view(torch.int16).cpu().numpy().view(np.uint16).reshape(*shape[:-1], -1)
    b = st.b.view(torch.int16).cpu().numpy().view(np.uint16).reshape(*shape[:-1], -1)
    return q, s, b


def _check(dev, w_bits):
    qg, sg, bg = _gpu_quantize(dev, w_bits)
    qo, so, bo = oq.quantize_q4(w_bits)
    assert np.array_equal(sg, so), "scales differ"
    assert np.array_equal(bg, bo), "biases differ"
    assert np.array_equal(qg, qo), f"codes differ in {int(np.sum(qg != qo))} words"


@pytest.mark.parametrize("std", [0.02, 1.0, 1e-3, 300.0])
def test_quantize_matches_oracle_bit_exact(dev, std):
    print(f"quantize random std={std}", flush=True)
    rng = np.random.default_rng(int(std * 1000) % 97)
    _check(dev, om.f64_to_bf16_bits(rng.normal(0.0, std, size=(3, 64, 512))))


@pytest.mark.parametrize("rows,K", [(37, 192), (1, 64), (129, 128), (5, 2048)])
def test_quantize_ragged_group_counts(dev, rows, K):
    # group counts that leave the last workgroup's 128 groups partly empty
    print(f"quantize ragged rows={rows} K={K}", flush=True)
    rng = np.random.default_rng(rows * 31 + K)
    _check(dev, om.f64_to_bf16_bits(rng.normal(0.0, 0.05, size=(1, rows, K))))


def test_quantize_edge_groups(dev):
    # constant groups, signed zeros, exact grid values with half-way points
    # (ties to even), a single outlier, and groups of two values
    rng = np.random.default_rng(4)
    w = om.f64_to_bf16_bits(rng.normal(0.0, 0.02, size=(16, 512)))
    w[0, :64] = 0x3F40                       # constant 0.75
    w[0, 64:128] = 0x8000                    # all -0
    w[0, 128:192] = np.where(np.arange(64) % 2 == 0, 0x8000, 0x0000)   # -0 / +0 mixed
    grid = (np.arange(64) % 31) * 0.5        # 0, 0.5, ..., 15: code boundaries at the half-way points
    w[1, :64] = om.f64_to_bf16_bits(grid * 2.0 ** -6 - 0.125)
    w[1, 64:128] = om.f64_to_bf16_bits(np.where(np.arange(64) == 5, 1.0, 0.0))   # one outlier
    w[1, 128:192] = om.f64_to_bf16_bits(np.where(np.arange(64) % 3 == 0, -2.0, 3.0))
    w[2, :] = om.f64_to_bf16_bits(np.linspace(-1.0, 1.0, 512))
    _check(dev, w)


def test_quantize_full_expert_stack(dev):
    # one gate stack slice at the full shape: 8 experts x 512 x 2048
    print("quantize 8 x 512 x 2048", flush=True)
    rng = np.random.default_rng(9)
    _check(dev, om.f64_to_bf16_bits(rng.normal(0.0, 0.02, size=(8, 512, 2048))))


def test_quantize_zero_rows_is_a_noop(dev):
    w = torch.empty(0, 4, 128, dtype=torch.bfloat16, device=dev)
    st = ops.quantize_q4(w)
    torch.cuda.synchronize()
    assert st.q.shape == (0, 4, 16)
