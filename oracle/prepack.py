"""CPU oracle of the prepacked 4-bit layout (a permutation of the canonical one).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
cpu_baseline leg may use it; it shares no code with the HIP path.

The pages give the weight format (page "Perplexity Open Sources Lily ...",
Technical Details, prefill bullet: groupwise affine 4-bit, 64 weights per
group) and say the weights are expanded only on chip (the itinai.com post), but
not how they are laid out in memory. The canonical layout of this library is
row-major: codes [n][N][K/8] u32, scales and biases [n][N][G] bf16 (G = K/64).
The prepacked layout holds the same values reordered for loads that read one
64-wide group of many consecutive output rows at once:

  codes   [n][G][N][8] u32   codes[e][g][r][j]  = q[e][r][8g + j]
  s pairs [n][G/2][N]  u32   spair[e][p][r]     = s[e][r][2p] | s[e][r][2p+1] << 16
  b pairs [n][G/2][N]  u32   bpair[e][p][r]     = b[e][r][2p] | b[e][r][2p+1] << 16

(G even). No value changes, so every product computed from it is the one
computed from the canonical layout.
"""
from __future__ import annotations

import numpy as np


def prepack_q4(q: np.ndarray, s: np.ndarray, b: np.ndarray):
    """Canonical stack (q uint32 [n][N][K/8], s and b uint16 [n][N][G]) ->
    (codes uint32 [n][G][N][8], s pairs uint32 [n][G/2][N], b pairs uint32 [n][G/2][N])."""
    q = np.asarray(q, dtype=np.uint32)
    s = np.asarray(s, dtype=np.uint16)
    b = np.asarray(b, dtype=np.uint16)
    n, N, W = q.shape
    G = W // 8
    if W % 8 or s.shape != (n, N, G) or b.shape != (n, N, G) or G % 2:
        raise ValueError("need q [n][N][8G], s and b [n][N][G] with G even")
    codes = np.empty((n, G, N, 8), dtype=np.uint32)
    for g in range(G):
        codes[:, g, :, :] = q[:, :, 8 * g: 8 * g + 8]

    def pairs(v):
        lo = v[:, :, 0::2].astype(np.uint32)
        hi = v[:, :, 1::2].astype(np.uint32)
        return np.ascontiguousarray((lo | (hi << 16)).transpose(0, 2, 1))

    return codes, pairs(s), pairs(b)
