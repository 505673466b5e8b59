"""Race reference: the pipelined decode against libmla_sync.so, the same
kernels built with every HBM -> LDS page transfer waited for right after it is
issued (MLA_SYNC_DEBUG), so that no page data is ever in flight while a kernel
computes.  The kernels wait for their own transfers by count (the transfers are
not visible to the compiler); a miscounted wait would let a wave read a page
slot before its bytes land, which is a timing-dependent race that can pass a
parity check by luck.  Here the arithmetic is identical, so out and lse must be
bit-identical on every case: every decode kernel (16-row token-split, 64-row
split-wave on pages and gathered rows, 128-row), bf16 and FP8 pages,
the token-sparse gather, forced splits, ragged tiles and chunks longer than 64 pages.  Each
pipelined result is also computed twice (run-to-run determinism)."""

import numpy as np
import pytest

import workloads
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mla_decode_02_amd as mla
    return torch, mla, torch.device("cuda:0")


def upload(torch, w, dev, kc8=None):
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kc = (torch.from_numpy(kc8).to(dev) if kc8 is not None
          else torch.from_numpy(w.kcache.view(np.int16)).to(dev).view(torch.bfloat16))
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.cache_seqlens).to(dev)
    return q, kc, bt, sl


def decode(env, w, t, num_parts, fp8):
    torch, mla, dev = env
    q, kc, bt, sl = t
    md, ns = mla.mla_get_metadata(sl, w.rows, w.h_kv, num_parts=num_parts)
    P = md.shape[0]
    ws = torch.full(((w.batch + P) * w.h_kv * w.rows * 513,), float("nan"), dtype=torch.float32, device=dev)
    fn = mla.mla_decode_paged_fp8 if fp8 else mla.mla_decode_paged
    out, lse = fn(q, kc, bt, sl, w.dv, md, ns, w.causal, w.scale, workspace=ws)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy(), lse.view(torch.int32).cpu().numpy()


def compare(env, w, num_parts=None, kc8=None, what=""):
    torch, mla, dev = env
    t = upload(torch, w, dev, kc8)
    fp8 = kc8 is not None
    o1, l1 = decode(env, w, t, num_parts, fp8)
    o2, l2 = decode(env, w, t, num_parts, fp8)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), f"{what}: pipelined build not deterministic"
    with mla.library(mla.SYNC_LIB_PATH):
        os_, ls_ = decode(env, w, t, num_parts, fp8)
    assert np.array_equal(l1, ls_), f"{what}: lse differs from the synchronous build"
    assert np.array_equal(o1, os_), f"{what}: out differs from the synchronous build " \
                                    f"({np.count_nonzero(o1 != os_)} elements)"


CASES = [
    # lens, s_q, h_q, h_kv, causal, num_parts
    ([63, 64, 65, 1, 0, 128], 1, 16, 1, False, None),
    ([0, 0], 2, 64, 1, True, None),
    ([65, 129, 1, 2, 3], 2, 16, 1, True, None),
    ([65, 129, 1, 2, 3], 2, 64, 1, True, 3),
    ([1000, 1, 70], 1, 16, 2, False, None),
    ([300, 77], 2, 32, 2, True, 5),
    ([4096, 100], 1, 128, 1, False, 7),
    ([513, 2049, 64], 2, 128, 1, True, 16),
    ([700, 900], 1, 17, 1, False, 9),
    ([700, 900], 3, 32, 1, True, 11),
    ([5000], 1, 64, 1, False, 64),
    ([5000], 1, 16, 1, False, 64),
    ([10000, 300], 1, 64, 1, False, 1),   # a 157-page chunk: page ids fetched inside the loop
    ([10000], 2, 128, 1, True, 1),
]


@pytest.mark.parametrize("lens,s_q,h_q,h_kv,causal,P", CASES)
def test_sync_reference_edge(env, lens, s_q, h_q, h_kv, causal, P):
    w = make_workload(lens, s_q=s_q, h_q=h_q, h_kv=h_kv, causal=causal, seed=sum(lens) + s_q,
                      extra_pages=2, poison_tail=True, outliers=True)
    compare(env, w, num_parts=P, what=f"{lens} s_q={s_q} h_q={h_q} h_kv={h_kv} P={P}")


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_sync_reference_workloads(env, cfg):
    compare(env, workloads.config_workload(cfg), what=workloads.CONFIGS[cfg]["name"])


@pytest.mark.parametrize("lens,s_q,h_q,h_kv,causal,P", [
    ([218, 164, 0, 2000], 1, 16, 1, False, None),   # 16-row kernel
    ([1000, 3, 577], 1, 16, 1, False, 7),
    ([1, 70, 300], 2, 64, 1, True, None),           # 64-row kernel
    ([0, 129, 64], 1, 128, 2, False, None),
    ([1000, 3, 577], 1, 128, 1, False, 7),
])
def test_sync_reference_fp8(env, lens, s_q, h_q, h_kv, causal, P):
    w = make_workload(lens, s_q=s_q, h_q=h_q, h_kv=h_kv, causal=causal, seed=sum(lens) + h_q)
    kc8 = workloads.make_fp8_cache(w, seed=len(lens))
    compare(env, w, num_parts=P, kc8=kc8, what=f"fp8 {lens} rows {w.rows}")


@pytest.mark.parametrize("cfg", [1, 4])
def test_sync_reference_fp8_workloads(env, cfg):
    w = workloads.config_workload(cfg)
    compare(env, w, kc8=workloads.make_fp8_cache(w, seed=cfg), what=f"fp8 {workloads.CONFIGS[cfg]['name']}")


@pytest.mark.parametrize("lens,h_q,topk,P", [([3000, 70, 1], 64, 700, None), ([5000, 2000], 128, 1500, 9),
                                             ([200, 1000, 64], 16, 100, 3)])
def test_sync_reference_sparse(env, lens, h_q, topk, P):
    torch, mla, dev = env
    w = make_workload(lens, s_q=1, h_q=h_q, seed=len(lens) + topk)
    idx, ptr = workloads.make_sparse_indices(w, topk, seed=topk, invalid=0.05, shuffle=True)
    q, kc, bt, sl = upload(torch, w, dev)
    ti = torch.from_numpy(idx).to(dev)
    tp = torch.from_numpy(ptr).to(dev)

    def run():
        offs, counts = mla.mla_sparse_prepare(ti, tp, 1, bt, sl, w.num_pages, 1)
        md, ns = mla.mla_get_metadata(counts, h_q, 1, num_parts=P)
        out, lse = mla.mla_sparse_decode(q, kc, offs, tp, counts, 512, md, ns, w.scale, nnz=ti.shape[0])
        torch.cuda.synchronize()
        return out.view(torch.int16).cpu().numpy(), lse.view(torch.int32).cpu().numpy()

    o1, l1 = run()
    o2, l2 = run()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    with mla.library(mla.SYNC_LIB_PATH):
        os_, ls_ = run()
    assert np.array_equal(o1, os_) and np.array_equal(l1, ls_), "sparse: differs from the synchronous build"
