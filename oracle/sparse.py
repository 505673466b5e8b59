"""CPU oracle of the token-sparse decode -- test infrastructure only (tests/,
the smoke entry point and bench.py's CPU baseline may import it; the product
library never does).  Plain numpy in fp64 on the exact bf16 values; it shares
no code with the HIP path.

The "Flash MLA: efficient MLA decoding kernel library for variable-length
sequences" page (developer.baidu.com, §三.3) adds a token-level sparse mode:
each query keeps only its top-k key tokens, the selection stored in CSR form;
its account of how the tokens are scored is garbled, so the selection is an
input here.  Reading: query row v = b * s_q + s attends, with every head, to
the cached tokens of sequence b listed in indices[indptr[v]:indptr[v+1]]
(logical positions).  Entries outside [0, L_b) or on a page id outside the
cache are ignored; a token listed twice counts twice; there is no causal mask.
Then for each head h, with keys K_t (576 dims) and values K_t[:512]:

  x_t = scale * q . K_t,  out = sum_t softmax(x)_t K_t[:512],  lse = ln sum_t e^{x_t}

and a row with no kept entry has out = 0, lse = -inf (as the dense decode).

``prepare`` is the integer step the GPU does first (the kept entries, in order,
as byte offsets of their cache rows, and their counts).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

PAGE = 64
ROW_BYTES = 576 * 2


def _f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def kept(w, indices: np.ndarray, indptr: np.ndarray, v: int):
    """Logical positions and physical pages of the entries row v keeps, in order."""
    b = v // w.s_q
    L = max(int(w.cache_seqlens[b]), 0)
    pos, pid = [], []
    for t in indices[int(indptr[v]):int(indptr[v + 1])]:
        t = int(t)
        if t < 0 or t >= L or t // PAGE >= w.block_table.shape[1]:
            continue
        p = int(w.block_table[b, t // PAGE])
        if p < 0 or p >= w.kcache.shape[0]:
            continue
        pos.append(t)
        pid.append(p)
    return pos, pid


def prepare(w, indices: np.ndarray, indptr: np.ndarray):
    """(offsets of the kept entries per row, concatenated as in the CSR ranges, counts)."""
    R = w.batch * w.s_q
    offs = np.zeros(int(indptr[R]), dtype=np.uint32)
    counts = np.zeros(R, dtype=np.int32)
    for v in range(R):
        pos, pid = kept(w, indices, indptr, v)
        counts[v] = len(pos)
        for i, (t, p) in enumerate(zip(pos, pid)):
            offs[int(indptr[v]) + i] = ((p * PAGE + t % PAGE) * w.h_kv) * ROW_BYTES
    return offs, counts


def decode(w, indices: np.ndarray, indptr: np.ndarray, scale: Optional[float] = None,
           sel: Optional[Sequence[int]] = None):
    """fp64 (out [n, 512], lse [n]) for all flat query rows (b*s_q + s)*h_q + h, or ``sel``."""
    scale = w.scale if scale is None else scale
    group = w.h_q // w.h_kv
    flat = range(w.batch * w.s_q * w.h_q) if sel is None else list(sel)
    outs, lses = [], []
    cache = {}
    for idx in flat:
        v, h = divmod(int(idx), w.h_q)
        b, s = divmod(v, w.s_q)
        k = h // group
        if v not in cache:
            pos, pid = kept(w, indices, indptr, v)
            cache[v] = _f64(np.array([w.kcache[p, t % PAGE] for t, p in zip(pos, pid)],
                                     dtype=np.uint16).reshape(len(pos), w.h_kv, 576)) if pos else None
        K = cache[v]
        if K is None:
            outs.append(np.zeros(512))
            lses.append(-math.inf)
            continue
        K = K[:, k, :]
        x = scale * (K @ _f64(w.q[b, s, h]))
        m = x.max()
        e = np.exp(x - m)
        z = e.sum()
        outs.append((e / z) @ K[:, :512])
        lses.append(m + math.log(z))
    return np.array(outs), np.array(lses)
