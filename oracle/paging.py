"""CPU oracle of the paged KV cache step before the decode -- test
infrastructure only (tests/, the smoke entry point and bench.py's CPU baseline
may import it; the product library never does).  Plain numpy on bf16 bit
patterns (uint16), integer work only, so the GPU must match it bit for bit.
It shares no code with the HIP path.

The "Flash MLA: efficient MLA decoding kernel library for variable-length
sequences" page (developer.baidu.com, §三.1, §四 steps 2 and 5): the cache is a
set of fixed-size pages, each sequence reaches its pages through its own page
table, a sequence of n tokens needs ceil(n / page_size) pages, pages are taken
as it grows and handed back when it ends.  The page size is 64 tokens (the
page's 4096 in its listing is read as the decode's 64).
"""
from __future__ import annotations

import numpy as np

PAGE = 64


def pages_needed(n_tokens: int) -> int:
    """Pages a sequence of n_tokens occupies: ceil(n / page_size)."""
    return (int(n_tokens) + PAGE - 1) // PAGE


def kv_append(kcache: np.ndarray, block_table: np.ndarray, seqlens: np.ndarray, new_kv: np.ndarray):
    """Append new_kv [b, s_new, h_kv, 576] after each sequence's current tokens.

    Token j of sequence b goes to logical position t = L_b + j: page
    block_table[b, t // 64], slot t % 64.  Positions whose page entry is
    missing (negative, past the table or past the cache) are not written.
    Returns (new kcache copy, new lengths)."""
    out = kcache.copy()
    b, s_new, h_kv, _ = new_kv.shape
    num_pages, max_blocks = kcache.shape[0], block_table.shape[1]
    for i in range(b):
        L = max(int(seqlens[i]), 0)
        for j in range(s_new):
            t = L + j
            blk = t // PAGE
            if blk >= max_blocks:
                continue
            pid = int(block_table[i, blk])
            if pid < 0 or pid >= num_pages:
                continue
            out[pid, t % PAGE, :, :] = new_kv[i, j, :, :]
    new_lens = np.maximum(seqlens.astype(np.int64), 0) + s_new
    return out, new_lens.astype(np.int32)


def logical_rows(kcache: np.ndarray, block_table: np.ndarray, seq: int, length: int) -> np.ndarray:
    """The first `length` cache rows of sequence `seq` in logical order [length, h_kv, 576]."""
    rows = [kcache[block_table[seq, t // PAGE], t % PAGE] for t in range(length)]
    return np.array(rows, dtype=kcache.dtype).reshape((length,) + kcache.shape[2:])
