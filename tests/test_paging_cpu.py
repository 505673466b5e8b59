"""CPU pins of the paged-cache step before the decode: the append oracle
(oracle/paging.py) against what the pages fix -- a sequence read back through
its page table is its old tokens followed by the new ones, ceil(n / 64) pages
per sequence -- and the host page allocator of libmla.so (mla_pager_*, plain
host code, no GPU) against the invariants of a page pool: every page owned by
at most one sequence, each sequence holding exactly ceil(len / 64) pages, a
failed request leaving the state unchanged, released pages reused first.
"""
import ctypes

import numpy as np
import pytest

from oracle import paging
from workloads import make_append_case

MLA_ERR_INVALID, MLA_ERR_WORKSPACE, MLA_ERR_CAPACITY, MLA_ERR_RANGE = -1, -3, -5, -6


def test_pages_needed_closed_form():
    for n, want in [(0, 0), (1, 1), (63, 1), (64, 1), (65, 2), (128, 2), (129, 3), (4096, 64)]:
        assert paging.pages_needed(n) == want


@pytest.mark.parametrize("lens,s_new,h_kv", [([0, 1, 63, 64, 130], 1, 1), ([5, 62, 200], 3, 2),
                                             ([0, 0], 70, 1)])
def test_append_reads_back_as_concatenation(lens, s_new, h_kv):
    w, before, new_kv = make_append_case(lens, s_new, h_kv=h_kv, h_q=2 * h_kv, seed=len(lens), extra_pages=3)
    out, new_lens = paging.kv_append(w.kcache, w.block_table, before, new_kv)
    assert np.array_equal(new_lens, before + s_new)
    touched = np.zeros(w.kcache.shape[:2], dtype=bool)
    for i, L in enumerate(before):
        got = paging.logical_rows(out, w.block_table, i, L + s_new)
        old = paging.logical_rows(w.kcache, w.block_table, i, L)
        assert np.array_equal(got[:L], old)
        assert np.array_equal(got[L:], new_kv[i])
        for t in range(L, L + s_new):
            touched[w.block_table[i, t // 64], t % 64] = True
    # nothing else moved (other sequences' rows, tails, spare pages)
    assert np.array_equal(out[~touched], w.kcache[~touched])


def test_append_skips_missing_pages():
    w, before, new_kv = make_append_case([60], 10, seed=3)
    bt = w.block_table.copy()
    bt[0, 1] = -1  # tokens 64.. have no page
    out, _ = paging.kv_append(w.kcache, bt, before, new_kv)
    got = paging.logical_rows(out, w.block_table, 0, 64)
    assert np.array_equal(got[60:64], new_kv[0, :4])
    assert np.array_equal(out[w.block_table[0, 1]], w.kcache[w.block_table[0, 1]])


# ---- host page allocator --------------------------------------------------

@pytest.fixture(scope="module")
def mla():
    import paged_mla_decode_02_amd as m
    return m


def check_invariants(pg, lens):
    bt = pg.block_table().numpy()
    held = []
    for s, L in lens.items():
        n = paging.pages_needed(L)
        assert pg.seq_pages(s) == n
        row = bt[s]
        assert np.all(row[:n] >= 0) and np.all(row[n:] == -1)
        for pid in row[:n]:
            assert pg.page_owner(int(pid)) == s
        held.extend(int(x) for x in row[:n])
    assert len(held) == len(set(held)), "a page is owned twice"
    assert pg.free_pages() == pg.num_pages - len(held)
    free = [p for p in range(pg.num_pages) if pg.page_owner(p) == -1]
    assert len(free) == pg.free_pages() and not set(free) & set(held)


def test_pager_random_ops_keep_invariants(mla):
    rng = np.random.default_rng(5)
    pg = mla.Pager(num_pages=40, max_seqs=6, max_blocks=12)
    lens = {s: 0 for s in range(6)}
    for _ in range(400):
        s = int(rng.integers(6))
        if rng.random() < 0.25:
            pg.release(s)
            lens[s] = 0
        else:
            want = lens[s] + int(rng.integers(0, 150))
            free_before, bt_before = pg.free_pages(), pg.block_table().clone()
            extra = paging.pages_needed(want) - paging.pages_needed(lens[s])
            if paging.pages_needed(want) > 12 or extra > free_before:
                with pytest.raises(mla.MlaError) as e:
                    pg.reserve(s, want)
                assert e.value.code == MLA_ERR_CAPACITY
                assert pg.free_pages() == free_before
                assert np.array_equal(pg.block_table().numpy(), bt_before.numpy())
            else:
                pg.reserve(s, want)
                lens[s] = max(lens[s], want)
        check_invariants(pg, lens)


def test_pager_fresh_pool_ascending_and_lifo_reuse(mla):
    pg = mla.Pager(num_pages=8, max_seqs=3, max_blocks=8)
    pg.reserve(0, 130)   # 3 pages
    pg.reserve(1, 64)    # 1 page
    bt = pg.block_table().numpy()
    assert list(bt[0, :3]) == [0, 1, 2] and bt[1, 0] == 3
    pg.release(0)
    pg.reserve(2, 129)   # takes the released pages first, in their order
    assert list(pg.block_table().numpy()[2, :3]) == [0, 1, 2]
    pg.reserve(2, 100)   # shrinking request: no change
    assert pg.seq_pages(2) == 3


def test_pager_rejects_bad_calls(mla):
    lib = mla._lib
    assert lib.mla_pager_bytes(0, 1, 1) == 0
    n = lib.mla_pager_bytes(4, 2, 2)
    buf = (ctypes.c_int32 * (n // 4))()
    assert lib.mla_pager_init(ctypes.addressof(buf), n - 1, 4, 2, 2) == MLA_ERR_WORKSPACE
    assert lib.mla_pager_reserve(ctypes.addressof(buf), 0, 10) == MLA_ERR_INVALID  # not initialised
    assert lib.mla_pager_init(ctypes.addressof(buf), n, 4, 2, 2) == 0
    p = ctypes.addressof(buf)
    assert lib.mla_pager_reserve(p, 2, 10) == MLA_ERR_INVALID
    assert lib.mla_pager_reserve(p, 0, -1) == MLA_ERR_INVALID
    assert lib.mla_pager_reserve(p, 0, 129) == MLA_ERR_CAPACITY  # 3 pages > max_blocks 2
    assert lib.mla_pager_page_owner(p, 4) == MLA_ERR_RANGE  # distinct from -1 (= free)
    assert lib.mla_pager_page_owner(p, -1) == MLA_ERR_RANGE
    assert lib.mla_pager_release(p, -1) == MLA_ERR_INVALID
    assert lib.mla_pager_reserve(p, 0, 128) == 0 and lib.mla_pager_reserve(p, 1, 128) == 0
    assert lib.mla_pager_free_pages(p) == 0
    assert lib.mla_pager_reserve(p, 1, 128) == 0  # already held


def test_page_owner_out_of_range_raises():
    """An out-of-range page id is an error, not the -1 of a free page."""
    import paged_mla_decode_02_amd as mla
    pg = mla.Pager(8, 2, 4)
    assert pg.page_owner(3) == -1
    with pytest.raises(mla.MlaError):
        pg.page_owner(8)
    with pytest.raises(mla.MlaError):
        pg.page_owner(-1)
