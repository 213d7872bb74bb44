"""Python binding over the C ABI (include/moe_q4.h) using torch tensors for device memory.

Only argument marshalling happens here: tensors are checked for device, dtype
and contiguity, their pointers and the current HIP stream are passed to the
library, and the library's status code is turned into an exception. Every
step of the MoE layer runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import numpy as np
import torch

from . import _lib
from ._lib import MoeDims, MoeLayerOptions, MoeQ4Weights, check

MOE_EPI_STORE_F32 = _lib.MOE_EPI_STORE_F32
MOE_EPI_SWIGLU_BF16 = _lib.MOE_EPI_SWIGLU_BF16
BLOCK_ROWS = _lib.MOE_GEMM_BLOCK_ROWS


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, dtype, name: str, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclasses.dataclass
class Q4Stack:
    """A stack of 4-bit matrices on the GPU.

    Canonical layout (layout 0): q int32 (bit patterns of uint32 words)
    [n][N][K/8], s and b bf16 [n][N][K/64]. Prepacked layout (layout 1, from
    prepack_q4): q int32 [n][G][N][8], s and b int32 [n][G/2][N] (bf16 pairs),
    all views of one buffer; dims holds (n, N, K)."""
    q: torch.Tensor
    s: torch.Tensor
    b: torch.Tensor
    layout: int = _lib.MOE_Q4_CANONICAL
    dims: Optional[tuple] = None

    @property
    def n(self) -> int:
        return self.dims[0] if self.dims else self.q.shape[0]

    @property
    def N(self) -> int:
        return self.dims[1] if self.dims else self.q.shape[1]

    @property
    def K(self) -> int:
        return self.dims[2] if self.dims else self.q.shape[2] * 8

    def c_struct(self) -> MoeQ4Weights:
        _need(self.q, torch.int32, "q")
        if self.layout == _lib.MOE_Q4_CANONICAL:
            _need(self.s, torch.bfloat16, "s", self.q.device)
            _need(self.b, torch.bfloat16, "b", self.q.device)
        else:
            _need(self.s, torch.int32, "s", self.q.device)
            _need(self.b, torch.int32, "b", self.q.device)
        return MoeQ4Weights(self.q.data_ptr(), self.s.data_ptr(), self.b.data_ptr(), self.n, self.N, self.K,
                            self.layout)

    @staticmethod
    def from_host(w, device) -> "Q4Stack":
        """From any object with numpy fields q (uint32), s and b (uint16 bf16 bits)."""
        q = torch.from_numpy(np.ascontiguousarray(w.q).view(np.int32)).to(device)
        s = torch.from_numpy(np.ascontiguousarray(w.s).view(np.int16)).view(torch.bfloat16).to(device)
        b = torch.from_numpy(np.ascontiguousarray(w.b).view(np.int16)).view(torch.bfloat16).to(device)
        return Q4Stack(q, s, b)


def prepack_q4(w: Q4Stack) -> Q4Stack:
    """The stack in the prepacked layout (a new buffer; w is unchanged)."""
    if w.layout != _lib.MOE_Q4_CANONICAL:
        raise ValueError("prepack_q4 takes a canonical stack")
    lib = _lib.load()
    n, N, K = w.n, w.N, w.K
    nbytes = int(lib.moe_prepack_q4_bytes(n, N, K))
    if nbytes == 0:
        raise ValueError("prepack needs K a positive multiple of 128")
    dev = w.q.device
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src = w.c_struct()
    out = MoeQ4Weights()
    check(lib.moe_prepack_q4(ctypes.byref(src), _ptr(buf), nbytes, ctypes.byref(out), _stream(dev)), "moe_prepack_q4")
    G = K // 64
    base = buf.data_ptr()

    def view(ptr, count, shape):
        off = ptr - base
        return buf[off: off + 4 * count].view(torch.int32).view(*shape)
    return Q4Stack(view(out.q, n * G * N * 8, (n, G, N, 8)), view(out.s, n * (G // 2) * N, (n, G // 2, N)),
                   view(out.b, n * (G // 2) * N, (n, G // 2, N)), layout=_lib.MOE_Q4_PREPACKED, dims=(n, N, K))


def bf16_from_bits(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def bits_from_bf16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def workspace_bytes(T: int, H: int, I: int, E: int, k: int, block_rows: int = 0) -> int:
    d = MoeDims(T, H, I, E, k, block_rows)
    return int(_lib.load().moe_workspace_bytes(ctypes.byref(d)))


def max_tiles(T: int, E: int, k: int, block_rows: int) -> int:
    d = MoeDims(T, 0, 0, E, k, block_rows)
    return int(_lib.load().moe_max_tiles(ctypes.byref(d)))


def moe_route(logits: torch.Tensor, k: int, block_rows: int = BLOCK_ROWS,
              logit_bias: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> dict:
    """Top-k, softmax weights and routing tables from fp32 logits [T][E]."""
    _need(logits, torch.float32, "logits")
    dev = logits.device
    T, E = logits.shape
    if logit_bias is not None:
        _need(logit_bias, torch.float32, "logit_bias", dev)
    d = MoeDims(T, 0, 0, E, k, block_rows)
    lib = _lib.load()
    mt = max(int(lib.moe_max_tiles(ctypes.byref(d))), 1)
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(topk_ids=torch.empty(T, k, **i32), topk_w=torch.empty(T, k, dtype=torch.float32, device=dev),
               counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
               sorted_rows=torch.empty(T * k, **i32), row_of_pair=torch.empty(T * k, **i32),
               tile_map=torch.full((mt, 2), -1, **i32), num_tiles=torch.zeros(1, **i32))
    wsb = int(lib.moe_workspace_bytes(ctypes.byref(d)))
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    st = lib.moe_route(_ptr(logits), _ptr(logit_bias), ctypes.byref(d), _ptr(out["topk_ids"]),
                       _ptr(out["topk_w"]), _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["sorted_rows"]),
                       _ptr(out["row_of_pair"]), _ptr(out["tile_map"]), _ptr(out["num_tiles"]),
                       _ptr(workspace), workspace.numel(), _stream(dev))
    check(st, "moe_route")
    return out


def moe_grouped_gemm_q4(A: torch.Tensor, W0: Q4Stack, offsets: torch.Tensor, tile_map: torch.Tensor,
                        num_tiles: torch.Tensor, epilogue: int, out_rows: int,
                        W1: Optional[Q4Stack] = None, sorted_rows: Optional[torch.Tensor] = None,
                        row_div: int = 1, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Grouped GEMM over a tile map: fp32 [out_rows][N] or SwiGLU bf16 [out_rows][N]."""
    _need(A, torch.bfloat16, "A")
    dev = A.device
    for t, n in ((offsets, "offsets"), (tile_map, "tile_map"), (num_tiles, "num_tiles")):
        _need(t, torch.int32, n, dev)
    if sorted_rows is not None:
        _need(sorted_rows, torch.int32, "sorted_rows", dev)
    w0 = W0.c_struct()
    w1 = W1.c_struct() if W1 is not None else None
    if out is None:
        dt = torch.float32 if epilogue == MOE_EPI_STORE_F32 else torch.bfloat16
        out = torch.zeros(out_rows, W0.N, dtype=dt, device=dev)
    lib = _lib.load()
    wsb = int(lib.moe_gemm_workspace_bytes(A.shape[0], W0.K))
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    st = lib.moe_grouped_gemm_q4(_ptr(A), A.shape[0], _ptr(sorted_rows), row_div, ctypes.byref(w0),
                                 ctypes.byref(w1) if w1 is not None else None, _ptr(offsets), _ptr(tile_map),
                                 _ptr(num_tiles), tile_map.shape[0], epilogue, _ptr(out), _ptr(workspace),
                                 workspace.numel(), _stream(dev))
    check(st, "moe_grouped_gemm_q4")
    return out


def quantize_q4(w: torch.Tensor, out: Optional["Q4Stack"] = None) -> "Q4Stack":
    """bf16 weights [n][N][K] (a stack of n matrices, K a multiple of 64) -> the
    4-bit groupwise-affine stack the GEMMs read (min-max affine per 64 elements)."""
    _need(w, torch.bfloat16, "w")
    if w.dim() != 3 or w.shape[2] % 64:
        raise ValueError("w must be [n][N][K] with K a multiple of 64")
    n, N, K = w.shape
    dev = w.device
    if out is None:
        out = Q4Stack(torch.empty(n, N, K // 8, dtype=torch.int32, device=dev),
                      torch.empty(n, N, K // 64, dtype=torch.bfloat16, device=dev),
                      torch.empty(n, N, K // 64, dtype=torch.bfloat16, device=dev))
    st = _lib.load().moe_quantize_q4(_ptr(w), n * N, K, _ptr(out.q), _ptr(out.s), _ptr(out.b), _stream(dev))
    check(st, "moe_quantize_q4")
    return out


@dataclasses.dataclass
class MoEWeights:
    """Device weights of one layer."""
    router_w: torch.Tensor   # bf16 [E][H]
    gate: Q4Stack
    up: Q4Stack
    down: Q4Stack
    sh_gate: Q4Stack
    sh_up: Q4Stack
    sh_down: Q4Stack
    logit_bias: Optional[torch.Tensor] = None   # float [E]
    shared_gate: Optional[torch.Tensor] = None  # bf16 [H]: gated shared expert

    @property
    def E(self) -> int:
        return self.router_w.shape[0]

    @property
    def H(self) -> int:
        return self.router_w.shape[1]

    @property
    def I(self) -> int:
        return self.gate.N

    def prepacked(self, stacks=("gate", "up", "down", "sh_gate", "sh_up", "sh_down")) -> "MoEWeights":
        """The same layer with the named stacks in the prepacked layout."""
        return dataclasses.replace(self, **{n: prepack_q4(getattr(self, n)) for n in stacks})

    @staticmethod
    def from_host(inp, device) -> "MoEWeights":
        """From an object with numpy fields router_w, logit_bias, gate, up, down, sh_gate, sh_up, sh_down."""
        lb = None
        if getattr(inp, "logit_bias", None) is not None:
            lb = torch.from_numpy(np.asarray(inp.logit_bias, np.float32)).to(device)
        sg = None
        if getattr(inp, "shared_gate", None) is not None:
            sg = bf16_from_bits(inp.shared_gate, device)
        return MoEWeights(router_w=bf16_from_bits(inp.router_w, device), shared_gate=sg,
                          gate=Q4Stack.from_host(inp.gate, device), up=Q4Stack.from_host(inp.up, device),
                          down=Q4Stack.from_host(inp.down, device),
                          sh_gate=Q4Stack.from_host(inp.sh_gate, device),
                          sh_up=Q4Stack.from_host(inp.sh_up, device),
                          sh_down=Q4Stack.from_host(inp.sh_down, device), logit_bias=lb)


def moe_layer_forward(x: torch.Tensor, w: MoEWeights, k: int, y: Optional[torch.Tensor] = None,
                      logits_out: Optional[torch.Tensor] = None, topk_ids_out: Optional[torch.Tensor] = None,
                      topk_w_out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, block_rows: int = 0,
                      side_stream: Optional["torch.cuda.Stream"] = None, events=None,
                      persistent_decode: bool = False) -> torch.Tensor:
    """y = MoE layer(x), bf16 [T][H]; optional outputs are filled when given.
    block_rows: routed tile height (0 = the library default, or 32, 64, 128).
    side_stream: run the shared expert on this stream (events: a (fork, join)
    pair of torch.cuda.Event already recorded once, so that they exist).
    A gate vector in w.shared_gate gates the shared expert. persistent_decode:
    few-token calls run as one persistent launch (where supported)."""
    _need(x, torch.bfloat16, "x")
    dev = x.device
    T, H = x.shape
    _need(w.router_w, torch.bfloat16, "router_w", dev)
    if w.logit_bias is not None:
        _need(w.logit_bias, torch.float32, "logit_bias", dev)
    for t, n, dt in ((logits_out, "logits_out", torch.float32), (topk_ids_out, "topk_ids_out", torch.int32),
                     (topk_w_out, "topk_w_out", torch.float32)):
        if t is not None:
            _need(t, dt, n, dev)
    d = MoeDims(T, H, w.I, w.E, k, block_rows)
    lib = _lib.load()
    if y is None:
        y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    _need(y, torch.bfloat16, "y", dev)
    wsb = int(lib.moe_workspace_bytes(ctypes.byref(d)))
    if workspace is None:
        workspace = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)
    structs = [s.c_struct() for s in (w.gate, w.up, w.down, w.sh_gate, w.sh_up, w.sh_down)]
    args = (_ptr(x), _ptr(w.router_w), _ptr(w.logit_bias), *[ctypes.byref(s) for s in structs], ctypes.byref(d),
            _ptr(y), _ptr(logits_out), _ptr(topk_ids_out), _ptr(topk_w_out), _ptr(workspace), workspace.numel(),
            _stream(dev))
    if w.shared_gate is None and side_stream is None and not persistent_decode:
        check(lib.moe_layer_forward(*args), "moe_layer_forward")
        return y
    opts = MoeLayerOptions()
    if w.shared_gate is not None:
        _need(w.shared_gate, torch.bfloat16, "shared_gate", dev)
        opts.shared_gate = w.shared_gate.data_ptr()
    if side_stream is not None:
        if events is None or len(events) != 2:
            raise ValueError("side_stream needs a (fork, join) pair of recorded torch.cuda.Event")
        opts.side_stream = side_stream.cuda_stream
        opts.fork_event = events[0].cuda_event
        opts.join_event = events[1].cuda_event
    opts.persistent_decode = 1 if persistent_decode else 0
    check(lib.moe_layer_forward_ex(*args, ctypes.byref(opts)), "moe_layer_forward_ex")
    return y


def moe_layer_forward_noalloc(x: torch.Tensor, w: MoEWeights, k: int, y: torch.Tensor,
                              logits_out: Optional[torch.Tensor] = None,
                              topk_ids_out: Optional[torch.Tensor] = None,
                              topk_w_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The layer with the library's per-GPU scratch array instead of a
    workspace: allocates nothing (y and the optional outputs are the caller's)."""
    _need(x, torch.bfloat16, "x")
    dev = x.device
    T, H = x.shape
    _need(y, torch.bfloat16, "y", dev)
    for t, n, dt in ((logits_out, "logits_out", torch.float32), (topk_ids_out, "topk_ids_out", torch.int32),
                     (topk_w_out, "topk_w_out", torch.float32)):
        if t is not None:
            _need(t, dt, n, dev)
    d = MoeDims(T, H, w.I, w.E, k, 0)
    structs = [s.c_struct() for s in (w.gate, w.up, w.down, w.sh_gate, w.sh_up, w.sh_down)]
    st = _lib.load().moe_layer_forward_noalloc(_ptr(x), _ptr(w.router_w), _ptr(w.logit_bias),
                                               *[ctypes.byref(s) for s in structs], ctypes.byref(d), _ptr(y),
                                               _ptr(logits_out), _ptr(topk_ids_out), _ptr(topk_w_out),
                                               _stream(dev))
    check(st, "moe_layer_forward_noalloc")
    return y


class MoELayer:
    """A layer with its weights and workspace resident on one GPU."""

    def __init__(self, weights: MoEWeights, k: int, max_tokens: int, block_rows: int = 0,
                 side_stream: bool = False, persistent_decode: bool = False):
        self.w = weights
        self.k = k
        self.block_rows = block_rows
        self.persistent_decode = persistent_decode
        dev = weights.router_w.device
        self.side_stream = None
        self.events = None
        if side_stream:
            # a second stream at the default priority and two events that exist
            # (torch creates an event's HIP handle when it is first recorded)
            self.side_stream = torch.cuda.Stream(device=dev)
            self.events = (torch.cuda.Event(), torch.cuda.Event())
            for e in self.events:
                e.record(torch.cuda.current_stream(dev))
        wsb = workspace_bytes(max_tokens, weights.H, weights.I, weights.E, k, block_rows)
        self.workspace = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)
        self.max_tokens = max_tokens

    def __call__(self, x: torch.Tensor, **outs) -> torch.Tensor:
        if x.shape[0] > self.max_tokens:
            raise ValueError("more tokens than the workspace was sized for")
        return moe_layer_forward(x, self.w, self.k, workspace=self.workspace, block_rows=self.block_rows,
                                 side_stream=self.side_stream, events=self.events,
                                 persistent_decode=self.persistent_decode, **outs)
