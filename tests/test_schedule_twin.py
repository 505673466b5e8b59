"""The scheduler twin (oracle side) against a hand-derived example and the
invariants any valid split-KV partition must satisfy."""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def expand(md, ns, seqlens):
    """Per sequence, the ordered list of (part, first_block, end_block, ordinal)."""
    b = len(seqlens)
    nblk = [(int(L) + 63) // 64 for L in seqlens]
    units = [max(n, 1) for n in nblk]
    per = {i: [] for i in range(b)}
    for p, row in enumerate(md):
        i, f, j, e, o = (int(x) for x in row[:5])
        if i == b:
            assert (f, j, e, o) == (0, b, 0, 0)
            continue
        for k in range(i, j + 1):
            lo = f if k == i else 0
            hi = e if k == j else units[k]
            per[k].append((p, lo, hi, o if k == i else 0))
    return per, nblk, units


def check_invariants(md, ns, seqlens, num_parts):
    b = len(seqlens)
    per, nblk, units = expand(md, ns, seqlens)
    assert md.shape == (num_parts, 8) and ns.shape == (b + 1,)
    assert ns[0] == 0 and np.all(np.diff(ns) >= 1)
    assert np.all(md[:, 5:] == 0)
    seen_empty = False
    for row in md:
        if row[0] == b:
            seen_empty = True
        else:
            assert not seen_empty, "an empty part precedes a non-empty one"
    for k in range(b):
        chunks = per[k]
        assert len(chunks) == ns[k + 1] - ns[k], (k, chunks)
        assert [c[3] for c in chunks] == list(range(len(chunks)))
        # blocks covered exactly once, in order, by consecutive parts
        pos = 0
        for idx, (p, lo, hi, o) in enumerate(chunks):
            assert lo == pos and hi > lo
            pos = hi
            if idx:
                assert p == chunks[idx - 1][0] + 1
        assert pos == units[k]
    return per


def test_golden_tiny(oracle_lib):
    fx = json.load(open(os.path.join(GOLDEN, "schedule_tiny.json")))
    md, ns = oracle_lib.schedule(fx["seqlens"], fx["rows"], fx["num_parts"])
    assert md.tolist() == fx["tile_metadata"]
    assert ns.tolist() == fx["num_splits"]
    check_invariants(md, ns, fx["seqlens"], fx["num_parts"])


@pytest.mark.parametrize("seed", range(12))
def test_random_invariants(oracle_lib, seed):
    rng = np.random.default_rng(seed)
    b = int(rng.integers(1, 200))
    hi = int(rng.choice([1, 64, 300, 5000, 70000]))
    seqlens = rng.integers(0, hi + 1, size=b)
    rows = int(rng.choice([1, 16, 32, 64, 128, 256]))
    P = int(rng.choice([1, 3, 8, 128, 256, 1000]))
    md, ns = oracle_lib.schedule(seqlens, rows, P)
    check_invariants(md, ns, seqlens, P)


@pytest.mark.parametrize("seqlens,rows,P", [
    ([0], 16, 1), ([0, 0, 0], 16, 4), ([1], 128, 256), ([64], 16, 2), ([65], 16, 256),
    ([4096] * 128, 128, 256), ([65536, 32768], 64, 256), ([1] * 500, 16, 7),
])
def test_edge_invariants(oracle_lib, seqlens, rows, P):
    md, ns = oracle_lib.schedule(seqlens, rows, P)
    check_invariants(md, ns, seqlens, P)


def test_chunk_count_closed_form(oracle_lib):
    """chunks_i = part(B_i - 1) - part(A_i) + 1, recomputed from the partition line."""
    seqlens = [218, 1, 0, 5000, 64, 65, 4096]
    for rows, ovh in [(1, 3), (16, 3), (17, 4), (32, 4), (64, 4), (65, 4), (128, 4), (129, 8), (256, 8)]:
        for P in (3, 16, 256):
            md, ns = oracle_lib.schedule(seqlens, rows, P)
            c, A, B = 0, [], []
            for L in seqlens:
                m = max((L + 63) // 64, 1)
                A.append(c + ovh)
                B.append(c + ovh + m)
                c = B[-1]
            q = max(-(-c // P), 2 * ovh)
            chunks = [(Bi - 1) // q - Ai // q + 1 for Ai, Bi in zip(A, B)]
            assert np.diff(ns).tolist() == chunks


def test_balanced_parts(oracle_lib):
    """With many parts, no part carries more than q units of work plus overhead."""
    rng = np.random.default_rng(3)
    seqlens = rng.integers(1, 2561, size=64)
    md, ns = oracle_lib.schedule(seqlens, 16, 256)
    per, nblk, units = expand(md, ns, seqlens)
    work = np.zeros(256, dtype=np.int64)
    for k, chunks in per.items():
        for p, lo, hi, o in chunks:
            work[p] += hi - lo
    ovh = 3  # the 16-row tile's per-chunk overhead, in page units
    T = sum(max((L + 63) // 64, 1) + ovh for L in seqlens)
    q = max(-(-T // 256), 2 * ovh)
    assert work.max() <= q
