"""CPU pins of the token-sparse decode oracle (oracle/sparse.py), independent
of its own formulas, and the C ABI's argument checks of the sparse calls.

* Selecting every cached token reproduces the dense decode oracle (oracle.c),
  and selecting each query's causal prefix reproduces the causal dense decode:
  a wrong gather, head mapping or row order fails.
* The result does not depend on the order of a row's list.
* Entries that address no cached token change nothing; a token listed twice
  weighs twice (checked against a closed form on one head).
* Empty rows give out = 0, lse = -inf; ``prepare`` keeps exactly the valid
  entries, in order, at the offsets of their cache rows.
"""
import ctypes
import dataclasses
import math
import os

import numpy as np
import pytest

import workloads
from oracle import sparse
from workloads import make_sparse_indices, make_workload


def full_lists(w, causal=False):
    idx, ptr = [], [0]
    for v in range(w.batch * w.s_q):
        b, s = divmod(v, w.s_q)
        L = int(w.cache_seqlens[b])
        n = max(0, L - w.s_q + s + 1) if causal else L
        idx.extend(range(n))
        ptr.append(len(idx))
    return np.array(idx, dtype=np.int32), np.array(ptr, dtype=np.int32)


def test_full_selection_is_the_dense_decode(oracle_lib):
    w = make_workload([70, 1, 130], s_q=1, h_q=8, h_kv=2, seed=3)
    idx, ptr = full_lists(w)
    so, sl = sparse.decode(w, idx, ptr)
    do, dl = oracle_lib.decode(w)
    np.testing.assert_allclose(so, do, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(sl, dl, rtol=0, atol=1e-10)


def test_causal_prefix_selection_is_the_causal_decode(oracle_lib):
    w = make_workload([70, 3, 130], s_q=3, h_q=4, causal=True, seed=4)
    idx, ptr = full_lists(w, causal=True)
    so, sl = sparse.decode(w, idx, ptr)
    do, dl = oracle_lib.decode(w)
    np.testing.assert_allclose(so, do, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(sl, dl, rtol=0, atol=1e-10)


def test_order_invalid_entries_and_empty_rows():
    w = make_workload([200, 90, 64], s_q=2, h_q=4, seed=5)
    idx, ptr = make_sparse_indices(w, 40, seed=5)
    base_o, base_l = sparse.decode(w, idx, ptr)
    rng = np.random.default_rng(0)
    rows = [idx[ptr[v]:ptr[v + 1]] for v in range(len(ptr) - 1)]

    def csr(rs):
        return np.concatenate(rs).astype(np.int32), np.cumsum([0] + [len(r) for r in rs]).astype(np.int32)
    o2, l2 = sparse.decode(w, *csr([rng.permutation(r) for r in rows]))
    np.testing.assert_allclose(o2, base_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, base_l, rtol=0, atol=1e-12)
    bad = []
    for v, r in enumerate(rows):
        L = int(w.cache_seqlens[v // w.s_q])
        bad.append(rng.permutation(np.concatenate([r, [-1, L, L + 63, w.max_blocks * 64 + 5, -7]])))
    o3, l3 = sparse.decode(w, *csr(bad))
    np.testing.assert_allclose(o3, base_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l3, base_l, rtol=0, atol=1e-12)
    o4, l4 = sparse.decode(w, *csr([r if v not in (1, 4) else r[:0] for v, r in enumerate(rows)]))
    for v in (1, 4):
        sl = slice(v * w.h_q, (v + 1) * w.h_q)
        assert np.all(o4[sl] == 0) and np.all(np.isneginf(l4[sl]))
    other = np.ones(len(o4), dtype=bool)
    other[w.h_q:2 * w.h_q] = other[4 * w.h_q:5 * w.h_q] = False
    np.testing.assert_allclose(o4[other], base_o[other], rtol=1e-12, atol=1e-14)


def test_duplicates_count_twice():
    w = make_workload([10], s_q=1, h_q=1, seed=6)
    idx = np.array([2, 7, 2], dtype=np.int32)
    ptr = np.array([0, 3], dtype=np.int32)
    o, l = sparse.decode(w, idx, ptr)
    q = sparse._f64(w.q[0, 0, 0])
    K = sparse._f64(np.array([w.kcache[w.block_table[0, 0], t, 0] for t in (2, 7)]))
    x = w.scale * (K @ q)
    wts = np.array([2 * math.exp(x[0]), math.exp(x[1])])
    np.testing.assert_allclose(o[0], (wts[0] * K[0, :512] + wts[1] * K[1, :512]) / wts.sum(), rtol=1e-12)
    assert abs(l[0] - math.log(wts.sum())) < 1e-12


def test_prepare_keeps_valid_entries_in_order():
    w = make_workload([200, 90], s_q=1, h_q=4, seed=7)
    idx, ptr = make_sparse_indices(w, 30, seed=7, invalid=0.4)
    offs, counts = sparse.prepare(w, idx, ptr)
    for v in range(2):
        row = idx[ptr[v]:ptr[v + 1]]
        good = [int(t) for t in row if 0 <= t < w.cache_seqlens[v]]
        assert counts[v] == len(good)
        for i, t in enumerate(good):
            assert offs[ptr[v] + i] == (w.block_table[v, t // 64] * 64 + t % 64) * 1152


# ---- C ABI argument checks --------------------------------------------------

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "paged_mla_decode_02_amd", "libmla.so")
FAKE = 0x100000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libmla.so not built")
    lib = ctypes.CDLL(LIB)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.mla_sparse_prepare.argtypes = [P, P, I, I, P, I, P, ctypes.c_int64, I, P, P, P]
    lib.mla_sparse_decode.argtypes = [P, P, ctypes.c_int64, P, P, P, I, I, I, I, I, I, I, P, I, P, ctypes.c_float,
                                      P, P, P, SZ, P]
    lib.mla_last_error.restype = ctypes.c_char_p
    return lib


def test_sparse_calls_reject(lib):
    pr = lambda **o: lib.mla_sparse_prepare(*[dict(dict(idx=FAKE, ptr=FAKE, b=4, s_q=1, bt=FAKE, mb=8, sl=FAKE,
                                                        np_=100, hkv=1, off=FAKE, cnt=FAKE), **o)[k]
                                              for k in ("idx", "ptr", "b", "s_q", "bt", "mb", "sl", "np_", "hkv",
                                                        "off", "cnt")], None)
    assert pr(b=-1) == -1 and pr(s_q=0) == -1 and pr(hkv=0) == -1 and pr(idx=None) == -1 and pr(off=None) == -1
    assert pr(np_=1 << 20, hkv=64) == -2          # cache beyond 32-bit row offsets
    assert pr(b=0, idx=None, ptr=None, bt=None, sl=None, off=None, cnt=None) == 0

    def dec(**o):
        a = dict(q=FAKE, kc=FAKE, np_=100, off=FAKE, ptr=FAKE, cnt=FAKE, b=4, s_q=1, h_q=16, hkv=1, scale=0.1,
                 ws=1 << 30)
        a.update(o)
        return lib.mla_sparse_decode(a["q"], a["kc"], a["np_"], a["off"], a["ptr"], a["cnt"], a["b"], a["s_q"],
                                     a["h_q"], a["hkv"], 576, 512, 64, FAKE, 256, FAKE, a["scale"], FAKE, FAKE, FAKE,
                                     a["ws"], None)
    assert dec(off=None) == -1 and dec(ptr=None) == -1 and dec(cnt=None) == -1
    assert dec(b=0) == -1 and dec(scale=0.0) == -1 and dec(h_q=15, hkv=2) == -1
    assert dec(b=8192, s_q=2) == -2               # query rows beyond MLA_MAX_BATCH
    assert dec(np_=1 << 20, h_q=64, hkv=64) == -2
    assert dec(ws=16) == -3
