"""fp64 CPU oracle for the int4 expert-routed prefill MoE layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
``cpu_baseline`` leg use it. It shares no code with the HIP path; its inputs
come from the ``synth`` package, which holds none of the layer's arithmetic.

What it computes (the plain per-token definition; the method on the pages only
reorders this work). Page references are to the three pages on the subject:
  P1 = "Perplexity Open Sources Lily: A Rust + Metal Inference Engine for
       Qwen3.6-35B-A3B on Apple Silicon" (aitrending.vip, English and Chinese)
  P2 = the itinai.com post on the Lily engine (one untitled body)
  P3 = the labomaru.com post on the Lily engine

  1. router logits   l[t,e] = fp32(fp32(sum_h x[t,h] W_r[e,h]) + beta[e])
                     (P1 Technical Details: a router picks 8 of 256 experts)
  2. selection       the k largest logits per token, ties to the lower expert
                     index (reading: order by the key (-l, e))
  3. weights         softmax over the k chosen logits (reading: softmax over all
                     E followed by renormalisation over the chosen k, which is
                     the same number)
  4. histogram       counts[e] = number of (token, slot) pairs routed to e
  5. prefix scan     offsets = exclusive scan of counts, offsets[E] = T*k
  6. scatter         stable counting sort of pair ids f = t*k + j by expert:
                     sorted_rows[r] = f, row_of_pair[f] = r
  7. block map       for each expert in ascending order, one tile per
                     block_rows rows: (expert, first row)
                     (steps 4-7: P1 Technical Details, prefill bullet, keeps
                     all four on the GPU in one command buffer; P1 技术解析,
                     预填充优化 paragraph; P2 body)
  8. dequantisation  W[n,k] = s[n, k//64] * q[n,k] + b[n, k//64], exact in fp64
                     (P1 Technical Details: groupwise affine 4-bit, 64 weights
                     per group; P1 技术解析: a bfloat16 scale per 64 weights;
                     reading: an affine form has a bias too, stored as bf16)
  9. expert FFN      g = x W_g^T, u = x W_u^T, h = bf16(silu(g) * u),
                     Y = h W_d^T  (SwiGLU; reading: h is rounded to bf16 because
                     it is the bf16 operand of the down projection)
 10. shared expert   the same FFN on every token with weight 1
                     (P1 Technical Details, Model bullet: one shared expert
                     besides the 8 routed ones; reading: added ungated)
 10'. gated variant  optional: with a gate vector w_sg (bf16 [H]) the shared
                     expert's output of token t is scaled by
                     g[t] = sigmoid(x[t] . w_sg), exact in fp64 (reading: the
                     pages do not say how the shared expert is weighted; a
                     sigmoid gate from the token's activations is the common
                     form of a gated shared expert)
 11. combine         y[t] = bf16(sum_j w[t,j] Y[row_of_pair[t*k+j]] + g[t] S[t]),
                     g[t] = 1 for the ungated layer

Only h and y are rounded (to bf16, round-to-nearest-even); everything else is
exact fp64. Routing can be driven from caller-supplied fp32 logits so that the
HIP path's exported logits and this oracle route identically.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

GROUP = 64          # weights per quantisation group (P1 Technical Details)
BF16_MANT_BITS = 8  # significant bits of bfloat16 (1 implicit + 7 stored)


# ----------------------------------------------------------------------------
# bfloat16 helpers
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    Done directly from fp64 (not through fp32, which could round twice)."""
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    fin = np.isfinite(v)
    a = np.abs(v[fin])
    _, e = np.frexp(a)                           # a = m * 2**e, 0.5 <= m < 1
    # quantum of the bf16 grid: 2**(e-8) for normal numbers; bf16 shares
    # float32's exponent range, so subnormals have the fixed quantum 2**-133
    qexp = np.maximum(e - BF16_MANT_BITS, -133)
    r = np.ldexp(np.rint(np.ldexp(a, -qexp)), qexp)   # np.rint: half to even
    r[r >= 2.0 ** 128] = np.inf                       # past the largest finite bf16
    out[fin] = np.copysign(r, v[fin])
    return out


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 (nearest, ties to even) and return the bit patterns."""
    r = round_bf16(v).astype(np.float32)   # exact: every bf16 value is a float32
    return (r.view(np.uint32) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
# 4-bit groupwise affine weights (step 8)
# ----------------------------------------------------------------------------

def unpack_q4(words: np.ndarray) -> np.ndarray:
    """uint32 [..., K/8] -> uint8 [..., K]; nibble i (bits 4i..4i+3) of word w is element 8w+i."""
    w = np.asarray(words, dtype=np.uint32)
    shifts = (4 * np.arange(8, dtype=np.uint32))
    nib = (w[..., None] >> shifts) & np.uint32(0xF)
    return nib.reshape(*w.shape[:-1], w.shape[-1] * 8).astype(np.uint8)


def dequant_q4(q_words: np.ndarray, s_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Exact fp64 dequantisation W = s * q + b of one [N, K] matrix (or a stack)."""
    q = unpack_q4(q_words).astype(np.float64)
    s = np.repeat(bf16_bits_to_f64(s_bits), GROUP, axis=-1)
    b = np.repeat(bf16_bits_to_f64(b_bits), GROUP, axis=-1)
    if s.shape != q.shape:
        raise ValueError(f"scale shape {s.shape} does not cover weights {q.shape}")
    return s * q + b


# ----------------------------------------------------------------------------
# routing (steps 1-7)
# ----------------------------------------------------------------------------

def router_logits(x_bits: np.ndarray, wr_bits: np.ndarray,
                  logit_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """fp32 logits: the fp64 product rounded once to fp32, then + beta in fp32."""
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(wr_bits)
    l = (x @ w.T).astype(np.float32)
    if logit_bias is not None:
        l = l + np.asarray(logit_bias, dtype=np.float32)[None, :]   # float32 + float32
    return l


def select_topk(logits: np.ndarray, k: int):
    """Top-k ids by the key (-logit, expert) and softmax weights over the chosen k.

    Returns (ids int32 [T,k], weights float64 [T,k])."""
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    if np.isnan(l).any() or np.isposinf(l).any():
        raise ValueError("logits must be finite or -inf")
    idx = np.broadcast_to(np.arange(E), l.shape)
    order = np.lexsort((idx, -l), axis=-1)      # primary: -l ascending; then index
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(l, ids.astype(np.int64), axis=1)
    top = sel[:, :1]
    if np.isneginf(top).any():
        raise ValueError("every token needs at least one finite logit")
    ex = np.exp(sel - top)
    w = ex / ex.sum(axis=1, keepdims=True)
    return ids, w


def routing_tables(ids: np.ndarray, E: int, block_rows: int) -> Dict[str, np.ndarray]:
    """Histogram, exclusive scan, stable scatter and block map of the (token, slot) pairs."""
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.ravel()                                   # pair f = t*k + j
    counts = np.bincount(flat, minlength=E)
    if counts.size != E:
        raise ValueError("expert id out of range")
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_rows = np.argsort(flat, kind="stable")        # pairs grouped by expert, f ascending
    row_of_pair = np.empty_like(sorted_rows)
    row_of_pair[sorted_rows] = np.arange(flat.size)
    tiles = []
    for e in range(E):
        for i in range(-(-int(counts[e]) // block_rows)):
            tiles.append((e, int(offsets[e]) + i * block_rows))
    tile_map = np.asarray(tiles, dtype=np.int32).reshape(-1, 2)
    return dict(counts=counts.astype(np.int32), offsets=offsets.astype(np.int32),
                sorted_rows=sorted_rows.astype(np.int32), row_of_pair=row_of_pair.astype(np.int32),
                tile_map=tile_map, num_tiles=np.int32(len(tiles)))


# ----------------------------------------------------------------------------
# expert FFN and the layer (steps 9-11)
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
               round_h: bool = True) -> np.ndarray:
    """Y = bf16(silu(x Wg^T) * (x Wu^T)) Wd^T in fp64 (h rounded unless round_h=False)."""
    g = x @ wg.T
    u = x @ wu.T
    h = silu(g) * u
    if round_h:
        h = round_bf16(h)
    return h @ wd.T


def shared_gate(inp, x: np.ndarray) -> np.ndarray:
    """Per-token factor of the shared expert: 1, or sigmoid(x . w_sg) in fp64 (step 10')."""
    if getattr(inp, "shared_gate", None) is None:
        return np.ones(x.shape[0])
    z = x @ bf16_bits_to_f64(inp.shared_gate)
    return 1.0 / (1.0 + np.exp(-z))


def expert_weights(w, e: int):
    """fp64 dequantised matrix of expert e from a Q4Weights-like stack."""
    return dequant_q4(w.q[e], w.s[e], w.b[e])


def moe_layer(inp, logits: Optional[np.ndarray] = None, block_rows: int = 64,
              round_h: bool = True, round_y: bool = True) -> Dict[str, np.ndarray]:
    """The whole layer. ``inp`` is a synth.MoEInputs; ``logits`` (fp32 [T,E]) overrides step 1.

    Returns every intermediate the HIP path exposes plus y (fp64 values on the
    bf16 grid when round_y) and y_bits (bf16 patterns)."""
    T, E, k = inp.T, inp.E, inp.k
    l_own = router_logits(inp.x, inp.router_w, inp.logit_bias)
    l = l_own if logits is None else np.asarray(logits, dtype=np.float32)
    ids, w = select_topk(l, k)
    tabs = routing_tables(ids, E, block_rows)
    x = bf16_bits_to_f64(inp.x)
    Y = np.zeros((T * k, inp.H), dtype=np.float64)
    offs, srt = tabs["offsets"], tabs["sorted_rows"]
    for e in range(E):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        if r0 == r1:
            continue
        tok = srt[r0:r1] // k
        Y[r0:r1] = swiglu_ffn(x[tok], expert_weights(inp.gate, e), expert_weights(inp.up, e),
                              expert_weights(inp.down, e), round_h)
    S = swiglu_ffn(x, expert_weights(inp.sh_gate, 0), expert_weights(inp.sh_up, 0),
                   expert_weights(inp.sh_down, 0), round_h)
    rop = tabs["row_of_pair"].reshape(T, k)
    y = shared_gate(inp, x)[:, None] * S
    for j in range(k):
        y += w[:, j:j + 1] * Y[rop[:, j]]
    y_out = round_bf16(y) if round_y else y
    out = dict(logits=l_own, route_logits=l, topk_ids=ids, topk_w=w, Y=Y, S=S, y_unrounded=y,
               y=y_out, y_bits=f64_to_bf16_bits(y) if round_y else None)
    out.update(tabs)
    return out


def moe_layer_tokens(inp, tokens: Sequence[int], logits: np.ndarray,
                     round_h: bool = True) -> np.ndarray:
    """y (unrounded fp64) for a subset of tokens, routed from the given fp32 logits rows.

    Each token's output depends only on its own activations, its logits row and
    the weights, so large layers can be checked one sampled token at a time."""
    tokens = np.asarray(tokens, dtype=np.int64)
    l = np.asarray(logits, dtype=np.float32)[tokens]
    ids, w = select_topk(l, inp.k)
    x = bf16_bits_to_f64(inp.x[tokens])
    sh = (expert_weights(inp.sh_gate, 0), expert_weights(inp.sh_up, 0), expert_weights(inp.sh_down, 0))
    y = shared_gate(inp, x)[:, None] * swiglu_ffn(x, *sh, round_h=round_h)
    for e in np.unique(ids):
        mats = (expert_weights(inp.gate, e), expert_weights(inp.up, e), expert_weights(inp.down, e))
        rows, slots = np.nonzero(ids == e)
        y[rows] += w[rows, slots][:, None] * swiglu_ffn(x[rows], *mats, round_h=round_h)
    return y


def layer_flops(T: int, H: int, I: int, E: int, k: int) -> int:
    """Algorithmic flops of one layer: router plus (k+1) SwiGLU experts per token."""
    return T * (2 * H * E + (k + 1) * 2 * H * 3 * I)


def q4_bytes(N: int, K: int) -> int:
    """Bytes of one 4-bit matrix: packed nibbles plus a bf16 scale and bias per 64 weights."""
    return N * K // 2 + 2 * 2 * N * (K // GROUP)

