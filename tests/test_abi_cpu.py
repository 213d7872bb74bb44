"""CPU tests of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments before launching anything (no compute call is made)."""
import ctypes
import os
import re

import pytest

from int4_expert_routing_amd import _lib
from int4_expert_routing_amd._lib import MoeDims, MoeQ4Weights

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_q4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    for must in ("moe_route", "moe_grouped_gemm_q4", "moe_layer_forward", "moe_layer_forward_ex",
                 "moe_workspace_bytes", "moe_status_string"):
        assert must in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in moe_q4.h but not exported"
    assert set(declared_functions()) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def test_status_strings(lib):
    for st in range(0, -7, -1):
        assert lib.moe_status_string(st).decode().startswith("MOE_")
    assert b"unknown" in lib.moe_status_string(5)


def test_check_dims_and_workspace(lib):
    good = MoeDims(4096, 2048, 512, 256, 8, 0)
    assert lib.moe_check_dims(ctypes.byref(good)) == _lib.MOE_OK
    ws = lib.moe_workspace_bytes(ctypes.byref(good))
    # the fp32 per-row outputs dominate: (T*k + T) rows * H * 4 bytes
    assert ws >= (4096 * 9) * 2048 * 4
    assert lib.moe_workspace_bytes(ctypes.byref(MoeDims(0, 2048, 512, 256, 8, 0))) == 0
    cases = {
        (4096, 2048, 512, 256, 0, 0): _lib.MOE_ERR_SHAPE,        # k = 0
        (4096, 2048, 512, 8, 9, 0): _lib.MOE_ERR_SHAPE,          # k > E
        (4096, 2048, 512, 257, 8, 0): _lib.MOE_ERR_SHAPE,        # E too large
        (4096, 2000, 512, 256, 8, 0): _lib.MOE_ERR_SHAPE,        # H not a multiple of 64
        (4096, 2048, 544, 256, 8, 0): _lib.MOE_ERR_SHAPE,        # I not a multiple of 64
        (-1, 2048, 512, 256, 8, 0): _lib.MOE_ERR_SHAPE,          # negative T
        (4096, 2112, 512, 256, 8, 0): _lib.MOE_ERR_UNSUPPORTED,  # H: an odd number of 64-groups
        (4096, 2048, 576, 256, 8, 0): _lib.MOE_ERR_UNSUPPORTED,  # I: an odd number of 64-groups
        (4096, 2048, 512, 256, 8, 96): _lib.MOE_ERR_UNSUPPORTED,  # tile height other than 32, 64, 128
        (4096, 2048, 512, 256, 8, 32): _lib.MOE_OK,              # routed tiles of 32 rows
        (4096, 2048, 512, 256, 8, 64): _lib.MOE_OK,
        (16, 4096, 512, 256, 8, 0): _lib.MOE_OK,                 # reductions above 2048
        (16, 8192, 4096, 256, 8, 0): _lib.MOE_OK,
        # operands addressed with 32-bit byte offsets must stay below 2 GiB:
        (262144, 2048, 512, 256, 8, 0): _lib.MOE_ERR_UNSUPPORTED,  # h: T*(k+1)*I*2 = 2.4 GB
        (600000, 2048, 128, 256, 1, 0): _lib.MOE_ERR_UNSUPPORTED,  # x: T*H*2 = 2.5 GB
        (200000, 2048, 512, 256, 8, 0): _lib.MOE_OK,               # h = 1.84 GB, x = 0.8 GB
        (1, 4194304, 128, 256, 8, 0): _lib.MOE_ERR_UNSUPPORTED,    # W_r: E*H*2 = 2 GiB
    }
    for dims, want in cases.items():
        assert lib.moe_check_dims(ctypes.byref(MoeDims(*dims))) == want, dims
    assert lib.moe_check_dims(None) == _lib.MOE_ERR_NULL


def test_workspace_holds_router_partials(lib):
    # the router GEMM splits K into fp32 partial-sum planes [T, E]: 8 up to
    # 1024 tokens, then as many (up to 8) as keep its 64 x 128 tiles at about
    # 512 workgroups, fewer when H is not a multiple of 64 * planes
    def ws(T, H=2048):
        return lib.moe_workspace_bytes(ctypes.byref(MoeDims(T, H, 512, 256, 8, 0)))

    for T, planes in ((8, 8), (512, 8), (1024, 8), (2048, 8), (4096, 4), (8192, 2)):
        without = ws(T) - planes * T * 256 * 4
        assert without >= (T * 9) * 2048 * 4 + T * 256 * 4, T     # Y and the logits still fit
    # splits fall back when H is not a multiple of 64 * planes
    assert ws(1024, 256) < ws(1024, 512)
    assert ws(16384) >= (16384 * 9) * 2048 * 4 + 16384 * 256 * 4


def test_max_tiles_bound(lib):
    assert lib.moe_max_tiles(ctypes.byref(MoeDims(4096, 0, 0, 256, 8, 128))) == 4096 * 8 // 128 + 256
    assert lib.moe_max_tiles(ctypes.byref(MoeDims(1, 0, 0, 256, 8, 64))) == 0 + 8


def test_calls_reject_bad_arguments_before_launching(lib):
    # every call below fails validation, so nothing reaches the GPU runtime
    d = MoeDims(64, 256, 128, 16, 2, 64)
    null = None
    st = lib.moe_route(null, null, ctypes.byref(d), *([null] * 8), null, 0, null)
    assert st == _lib.MOE_ERR_NULL
    bad = MoeDims(64, 256, 128, 16, 0, 64)
    assert lib.moe_route(null, null, ctypes.byref(bad), *([null] * 8), null, 0, null) == _lib.MOE_ERR_SHAPE
    fake = ctypes.c_void_p(0x1000)     # never dereferenced: validation fails first
    st = lib.moe_route(fake, null, ctypes.byref(d), *([fake] * 8), null, 0, null)
    assert st == _lib.MOE_ERR_WORKSPACE
    w = MoeQ4Weights(0x1000, 0x2000, 0x3000, 16, 128, 256)
    dl = MoeDims(64, 256, 128, 16, 2, 0)
    st = lib.moe_layer_forward(null, null, null, *([ctypes.byref(w)] * 6), ctypes.byref(dl), null, null, null,
                               null, null, 0, null)
    assert st == _lib.MOE_ERR_NULL
    # wrong weight shapes
    st = lib.moe_layer_forward(fake, fake, null, *([ctypes.byref(w)] * 6), ctypes.byref(dl), fake, null, null,
                               null, null, 0, null)
    assert st == _lib.MOE_ERR_SHAPE
    # misaligned activations
    d2 = MoeDims(64, 256, 128, 16, 2, 0)
    ws = [MoeQ4Weights(0x1000, 0x2000, 0x3000, n, N, K)
          for n, N, K in ((16, 128, 256), (16, 128, 256), (16, 256, 128), (1, 128, 256), (1, 128, 256),
                          (1, 256, 128))]
    st = lib.moe_layer_forward(ctypes.c_void_p(0x1002), fake, null, *[ctypes.byref(x) for x in ws],
                               ctypes.byref(d2), fake, null, null, null, null, 0, null)
    assert st == _lib.MOE_ERR_ALIGN
    # scales or biases not 16-byte aligned
    ws_s = [MoeQ4Weights(w_.q, 0x2004, w_.b, w_.n_experts, w_.N, w_.K) for w_ in ws]
    st = lib.moe_layer_forward(fake, fake, null, *[ctypes.byref(x) for x in ws_s], ctypes.byref(d2), fake, null,
                               null, null, fake, 1 << 30, null)
    assert st == _lib.MOE_ERR_ALIGN
    ws_b = [MoeQ4Weights(w_.q, w_.s, 0x3008, w_.n_experts, w_.N, w_.K) for w_ in ws]
    st = lib.moe_layer_forward(fake, fake, null, *[ctypes.byref(x) for x in ws_b], ctypes.byref(d2), fake, null,
                               null, null, fake, 1 << 30, null)
    assert st == _lib.MOE_ERR_ALIGN
    # workspace too small
    st = lib.moe_layer_forward(fake, fake, null, *[ctypes.byref(x) for x in ws], ctypes.byref(d2), fake, null,
                               null, null, fake, 16, null)
    assert st == _lib.MOE_ERR_WORKSPACE
    # options: a side stream needs both events; the gate vector must be 16-byte aligned
    opts = _lib.MoeLayerOptions(0, 0x5000, 0x6000, 0)
    st = lib.moe_layer_forward_ex(fake, fake, null, *[ctypes.byref(x) for x in ws], ctypes.byref(d2), fake, null,
                                  null, null, fake, 1 << 30, null, ctypes.byref(opts))
    assert st == _lib.MOE_ERR_NULL
    opts = _lib.MoeLayerOptions(0x5008, 0, 0, 0)
    st = lib.moe_layer_forward_ex(fake, fake, null, *[ctypes.byref(x) for x in ws], ctypes.byref(d2), fake, null,
                                  null, null, fake, 1 << 30, null, ctypes.byref(opts))
    assert st == _lib.MOE_ERR_ALIGN
    # T = 0 is a no-op
    d0 = MoeDims(0, 256, 128, 16, 2, 0)
    st = lib.moe_layer_forward(fake, fake, null, *[ctypes.byref(x) for x in ws], ctypes.byref(d0), fake, null,
                               null, null, null, 0, null)
    assert st == _lib.MOE_OK
    # grouped GEMM: unsupported width, bad epilogue
    w0 = MoeQ4Weights(0x1000, 0x2000, 0x3000, 4, 96, 256)
    st = lib.moe_grouped_gemm_q4(fake, 8, null, 1, ctypes.byref(w0), null, fake, fake, fake, 4, 0, fake, null, 0,
                                 null)
    assert st == _lib.MOE_ERR_UNSUPPORTED
    st = lib.moe_grouped_gemm_q4(fake, 8, null, 1, ctypes.byref(w0), null, fake, fake, fake, 4, 7, fake, null, 0,
                                 null)
    assert st == _lib.MOE_ERR_SHAPE
    # grouped GEMM: an odd number of 64-groups, and A beyond 32-bit byte offsets
    w3 = MoeQ4Weights(0x1000, 0x2000, 0x3000, 4, 128, 192)
    st = lib.moe_grouped_gemm_q4(fake, 8, null, 1, ctypes.byref(w3), null, fake, fake, fake, 4, 0, fake, null, 0,
                                 null)
    assert st == _lib.MOE_ERR_UNSUPPORTED
    w4 = MoeQ4Weights(0x1000, 0x2000, 0x3000, 4, 128, 4096)
    st = lib.moe_grouped_gemm_q4(fake, 1 << 18, null, 1, ctypes.byref(w4), null, fake, fake, fake, 4, 0, fake,
                                 null, 0, null)
    assert st == _lib.MOE_ERR_UNSUPPORTED    # 2^18 rows x 4096 x 2 bytes = 2 GiB


def test_noalloc_rejects_sizes_beyond_its_array_before_any_hip_call(lib):
    # validation and the size check come before the device is touched
    fake = ctypes.c_void_p(0x100000)
    ws = [MoeQ4Weights(0x1000, 0x2000, 0x3000, n, N, K)
          for n, N, K in ((256, 512, 2048), (256, 512, 2048), (256, 2048, 512), (1, 512, 2048), (1, 512, 2048),
                          (1, 2048, 512))]
    big = MoeDims(4096, 2048, 512, 256, 8, 0)
    assert lib.moe_workspace_bytes(ctypes.byref(big)) > _lib.MOE_NOALLOC_SCRATCH_BYTES
    st = lib.moe_layer_forward_noalloc(fake, fake, None, *[ctypes.byref(x) for x in ws], ctypes.byref(big), fake,
                                       None, None, None, None)
    assert st == _lib.MOE_ERR_WORKSPACE
    bad = MoeDims(4096, 2048, 512, 256, 0, 0)
    st = lib.moe_layer_forward_noalloc(fake, fake, None, *[ctypes.byref(x) for x in ws], ctypes.byref(bad), fake,
                                       None, None, None, None)
    assert st == _lib.MOE_ERR_SHAPE
    hdr = open(HEADER).read()
    assert "#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)" in hdr and _lib.MOE_NOALLOC_SCRATCH_BYTES == 32 << 20
    assert "#define MOE_WORKSPACE_HEAD_BYTES 190080" in hdr and _lib.MOE_WORKSPACE_HEAD_BYTES == 190080
    assert "#define MOE_WORKSPACE_STATUS_OFFSET 16768" in hdr and _lib.MOE_WORKSPACE_STATUS_OFFSET == 16768


def test_quantize_validation_launches_nothing(lib):
    # shape and pointer errors are reported before any launch (no GPU needed)
    P = ctypes.c_void_p
    fake = P(0x100000)   # never dereferenced: every call below fails validation or is a no-op
    assert lib.moe_quantize_q4(fake, 4, 100, fake, fake, fake, None) == -2      # K % 64
    assert lib.moe_quantize_q4(fake, -1, 64, fake, fake, fake, None) == -2      # rows < 0
    assert lib.moe_quantize_q4(fake, 4, 0, fake, fake, fake, None) == -2        # K == 0
    assert lib.moe_quantize_q4(fake, 1 << 40, 2048, fake, fake, fake, None) == -2
    assert lib.moe_quantize_q4(None, 0, 64, None, None, None, None) == 0        # rows == 0: no-op
    assert lib.moe_quantize_q4(None, 4, 64, fake, fake, fake, None) == -1
    assert lib.moe_quantize_q4(P(0x100008), 4, 64, fake, fake, fake, None) == -3  # w not 16-byte aligned
    assert lib.moe_quantize_q4(fake, 4, 64, fake, P(0x100001), fake, None) == -3  # s not 2-byte aligned
