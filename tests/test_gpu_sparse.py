"""GPU parity of the token-sparse decode through the C ABI: the preparation
step bit-exact against oracle/sparse.py's ``prepare`` (integer work), and the
decode against the fp64 sparse oracle (out rel-L2 <= 1e-2, lse <= 1e-3) over
head counts that use one or two 64-row tiles, KV-head groups, invalid and
shuffled entries, empty rows, forced splits and a large sampled workload.
"""
import numpy as np
import pytest

import workloads
from workloads import make_sparse_indices, make_workload

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 1e-3


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oracle import sparse
    import paged_mla_decode_02_amd as mla
    return torch, mla, sparse, torch.device("cuda:0")


def upload(torch, w, idx, ptr, dev):
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kc = torch.from_numpy(w.kcache.view(np.int16)).to(dev).view(torch.bfloat16)
    return (q, kc, torch.from_numpy(w.block_table).to(dev), torch.from_numpy(w.cache_seqlens).to(dev),
            torch.from_numpy(idx).to(dev), torch.from_numpy(ptr).to(dev))


def check(go, gl, ro, rl, what):
    ninf = np.isneginf(rl)
    assert np.all(np.isfinite(go)), what
    assert np.array_equal(np.isneginf(gl), ninf), what
    assert np.all(go[ninf] == 0), what
    nr = np.linalg.norm(ro)
    rel = np.linalg.norm(go - ro) / nr if nr > 0 else np.linalg.norm(go)  # all rows empty: exact zeros
    err = np.max(np.abs(gl[~ninf] - rl[~ninf])) if np.any(~ninf) else 0.0
    assert rel <= OUT_TOL and err <= LSE_TOL, f"{what}: rel {rel:.2e} lse {err:.2e}"


@pytest.mark.parametrize("lens,s_q,h_kv,topk,invalid", [([300, 70, 1000], 1, 1, 64, 0.0),
                                                       ([5, 2000], 2, 2, 700, 0.3)])
def test_prepare_bit_exact(env, lens, s_q, h_kv, topk, invalid):
    torch, mla, sparse, dev = env
    w = make_workload(lens, s_q=s_q, h_q=2 * h_kv, h_kv=h_kv, seed=len(lens))
    idx, ptr = make_sparse_indices(w, topk, seed=3, invalid=invalid)
    q, kc, bt, sl, ti, tp = upload(torch, w, idx, ptr, dev)
    offs, counts = mla.mla_sparse_prepare(ti, tp, s_q, bt, sl, w.num_pages, h_kv)
    torch.cuda.synchronize()
    ro, rc = sparse.prepare(w, idx, ptr)
    gc = counts.cpu().numpy()
    go = offs.cpu().numpy().view(np.uint32)
    assert np.array_equal(gc, rc)
    for v in range(len(rc)):
        assert np.array_equal(go[ptr[v]:ptr[v] + rc[v]], ro[ptr[v]:ptr[v] + rc[v]]), v


@pytest.mark.parametrize("lens,s_q,h_q,h_kv,topk,invalid,empty,parts", [
    ([300, 70, 1000], 1, 16, 1, 64, 0.0, (), None),
    ([300, 70, 1000, 5], 2, 64, 1, 200, 0.3, (3,), None),
    ([2500, 900], 1, 128, 1, 1000, 0.0, (), 9),      # two row tiles, forced splits
    ([640, 33], 2, 32, 2, 130, 0.1, (0,), None),
    # <= 16 rows per KV head (the 16-row kernel's gathered slices): many pages
    # per row, several rows per part, forced splits, ragged 8- and 12-row tiles
    ([5000, 3, 64, 129, 2000], 2, 16, 1, 1500, 0.1, (1,), 3),
    ([4100, 700], 1, 8, 1, 1400, 0.0, (), None),
    ([3000, 65, 1, 2048], 3, 24, 2, 700, 0.2, (4,), 7),
])
def test_sparse_decode_small(env, lens, s_q, h_q, h_kv, topk, invalid, empty, parts):
    torch, mla, sparse, dev = env
    w = make_workload(lens, s_q=s_q, h_q=h_q, h_kv=h_kv, seed=sum(lens) % 97)
    idx, ptr = make_sparse_indices(w, topk, seed=h_q, invalid=invalid, empty_rows=empty)
    q, kc, bt, sl, ti, tp = upload(torch, w, idx, ptr, dev)
    out, lse = mla.flash_mla_sparse_with_kvcache(q, kc, bt, sl, ti, tp, softmax_scale=w.scale, num_parts=parts)
    torch.cuda.synchronize()
    ro, rl = sparse.decode(w, idx, ptr)
    go = out.float().cpu().numpy().astype(np.float64).reshape(-1, 512)
    gl = lse.cpu().numpy().astype(np.float64).reshape(-1)
    check(go, gl, ro, rl, f"{lens} h_q={h_q}")


def test_sparse_decode_large_sampled(env):
    """64 sequences of 4K-16K tokens, 128 heads, top-2048 per query (sampled rows)."""
    torch, mla, sparse, dev = env
    rng = np.random.default_rng(12)
    lens = rng.integers(4096, 16385, size=64)
    w = make_workload(lens, s_q=1, h_q=128, seed=12)
    idx, ptr = make_sparse_indices(w, 2048, seed=12)
    q, kc, bt, sl, ti, tp = upload(torch, w, idx, ptr, dev)
    out, lse = mla.flash_mla_sparse_with_kvcache(q, kc, bt, sl, ti, tp, softmax_scale=w.scale)
    torch.cuda.synchronize()
    n = w.batch * w.h_q
    sel = np.sort(rng.choice(n, size=40, replace=False))
    ro, rl = sparse.decode(w, idx, ptr, sel=sel)
    go = out.float().cpu().numpy().astype(np.float64).reshape(-1, 512)[sel]
    gl = lse.cpu().numpy().astype(np.float64).reshape(-1)[sel]
    check(go, gl, ro, rl, "large sparse")


@pytest.mark.parametrize("seed", range(8))
def test_sparse_decode_random_shapes(env, seed):
    """Seeded draws of lengths, s_q, heads, top-k, invalid entries, shuffled and
    empty rows, and part count."""
    torch, mla, sparse, dev = env
    g = np.random.Generator(np.random.PCG64(4000 + seed))
    batch = int(g.integers(1, 7))
    lens = [int(g.choice([0, 1, 64, 65])) if g.random() < 0.25 else int(g.integers(1, 3000)) for _ in range(batch)]
    s_q = int(g.integers(1, 4))
    h_kv = int(g.choice([1, 1, 2]))
    h_q = h_kv * int(g.choice([8, 16, 64, 128]))
    topk = int(g.integers(1, 1500))
    invalid = float(g.choice([0.0, 0.2]))
    empty = tuple(int(v) for v in g.choice(batch * s_q, size=int(g.integers(0, 2)), replace=False))
    parts = None if g.random() < 0.5 else int(g.integers(1, 24))
    w = make_workload(lens, s_q=s_q, h_q=h_q, h_kv=h_kv, seed=5000 + seed)
    idx, ptr = make_sparse_indices(w, topk, seed=seed, invalid=invalid, shuffle=bool(seed % 2), empty_rows=empty)
    q, kc, bt, sl, ti, tp = upload(torch, w, idx, ptr, dev)
    out, lse = mla.flash_mla_sparse_with_kvcache(q, kc, bt, sl, ti, tp, softmax_scale=w.scale, num_parts=parts)
    torch.cuda.synchronize()
    ro, rl = sparse.decode(w, idx, ptr)
    go = out.float().cpu().numpy().astype(np.float64).reshape(-1, 512)
    gl = lse.cpu().numpy().astype(np.float64).reshape(-1)
    check(go, gl, ro, rl, f"sparse random seed={seed}: lens={lens} s_q={s_q} h_q={h_q} h_kv={h_kv} "
                          f"topk={topk} invalid={invalid} empty={empty} parts={parts}")
