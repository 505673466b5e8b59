"""GPU parity of the paged KV append (mla_kv_append, through the C ABI) with
the CPU oracle (oracle/paging.py): the whole cache after the append must match
bit for bit, and so must the new lengths.  Then the step before the decode end
to end: the host page allocator grows every sequence, the append writes the
new rows, and the decode of those newest tokens (causal, s_q = s_new) matches
the decode oracle on the oracle-appended cache (rel-L2 <= 1e-2, lse <= 1e-3).
"""
import numpy as np
import pytest

import workloads
from workloads import make_append_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    from oracle import paging
    import paged_mla_decode_02_amd as mla
    oracle.build(force=False)
    return torch, mla, oracle, paging, torch.device("cuda:0")


def dev16(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)


@pytest.mark.parametrize("lens,s_new,h_kv", [([0, 1, 63, 64, 130], 1, 1), ([5, 62, 200], 3, 2),
                                             ([0, 0], 70, 1), (list(range(0, 640, 37)), 2, 1)])
def test_append_bit_exact(env, lens, s_new, h_kv):
    torch, mla, _, paging, dev = env
    w, before, new_kv = make_append_case(lens, s_new, h_kv=h_kv, h_q=2 * h_kv, seed=len(lens) + s_new,
                                         extra_pages=2)
    kc = dev16(torch, w.kcache, dev).view(torch.bfloat16)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(before).to(dev)
    new_lens = mla.mla_kv_append(dev16(torch, new_kv, dev).view(torch.bfloat16), sl, bt, kc)
    torch.cuda.synchronize()
    ref, ref_lens = paging.kv_append(w.kcache, w.block_table, before, new_kv)
    assert np.array_equal(kc.view(torch.int16).cpu().numpy().view(np.uint16), ref)
    assert np.array_equal(new_lens.cpu().numpy(), ref_lens)
    assert np.array_equal(sl.cpu().numpy(), before)  # the input lengths are untouched


def test_append_skips_missing_pages(env):
    torch, mla, _, paging, dev = env
    w, before, new_kv = make_append_case([60, 10], 10, seed=3)
    btn = w.block_table.copy()
    btn[0, 1] = -1          # tokens 64.. of sequence 0 have no page
    btn[1, 0] = 10 ** 6     # past the cache
    kc = dev16(torch, w.kcache, dev).view(torch.bfloat16)
    mla.mla_kv_append(dev16(torch, new_kv, dev).view(torch.bfloat16), torch.from_numpy(before).to(dev),
                      torch.from_numpy(btn).to(dev), kc)
    torch.cuda.synchronize()
    ref, _ = paging.kv_append(w.kcache, btn, before, new_kv)
    assert np.array_equal(kc.view(torch.int16).cpu().numpy().view(np.uint16), ref)


def test_append_then_decode(env):
    """Pager -> append -> decode of the appended tokens, against the oracles."""
    torch, mla, oracle, paging, dev = env
    rng = np.random.default_rng(8)
    b, s_new, h_q = 6, 2, 16
    lens = rng.integers(0, 400, size=b).astype(np.int32)
    num_pages, max_blocks = 64, 16
    pg = mla.Pager(num_pages, b, max_blocks)
    for i, L in enumerate(lens):
        pg.reserve(i, int(L))
    kc_np = workloads.bf16_bits(rng.standard_normal((num_pages, 64, 1, 576), dtype=np.float32))
    new_kv = workloads.bf16_bits(rng.standard_normal((b, s_new, 1, 576), dtype=np.float32))
    q = workloads.bf16_bits(rng.standard_normal((b, s_new, h_q, 576), dtype=np.float32))
    for i, L in enumerate(lens):
        pg.reserve(i, int(L) + s_new)   # grow each sequence by the new tokens
    bt_np = pg.block_table().numpy()
    kc = dev16(torch, kc_np, dev).view(torch.bfloat16)
    bt = torch.from_numpy(bt_np).to(dev)
    new_lens = mla.mla_kv_append(dev16(torch, new_kv, dev).view(torch.bfloat16), torch.from_numpy(lens).to(dev),
                                 bt, kc)
    md, ns = mla.get_mla_metadata(new_lens, s_new * h_q, 1)
    out, lse = mla.flash_mla_with_kvcache(dev16(torch, q, dev).view(torch.bfloat16), kc, bt, new_lens, 512, md, ns,
                                          causal=True, softmax_scale=workloads.SCALE)
    torch.cuda.synchronize()
    ref_kc, ref_lens = paging.kv_append(kc_np, bt_np, lens, new_kv)
    assert np.array_equal(kc.view(torch.int16).cpu().numpy().view(np.uint16), ref_kc)
    w = workloads.Workload(batch=b, s_q=s_new, h_q=h_q, h_kv=1, causal=True, scale=workloads.SCALE,
                           cache_seqlens=ref_lens, block_table=bt_np, q=q, kcache=ref_kc, seed=8)
    ro, rl = oracle.decode(w)
    go = out.float().cpu().numpy().astype(np.float64)
    gl = lse.cpu().numpy().astype(np.float64)
    ro = ro.reshape(go.shape)
    rl = rl.reshape(gl.shape)
    assert np.linalg.norm(go - ro) / np.linalg.norm(ro) < 1e-2
    assert np.max(np.abs(gl - rl)) < 1e-3


def test_append_empty_batch(env):
    torch, mla, _, _, dev = env
    kc = torch.zeros((2, 64, 1, 576), dtype=torch.bfloat16, device=dev)
    e = torch.empty((0,), dtype=torch.int32, device=dev)
    out = mla.mla_kv_append(torch.empty((0, 1, 1, 576), dtype=torch.bfloat16, device=dev), e,
                            torch.empty((0, 4), dtype=torch.int32, device=dev), kc)
    assert out.shape == (0,)


@pytest.mark.parametrize("seed", range(6))
def test_append_random_shapes(env, seed):
    """Seeded draws of batch, lengths (page edges mixed in), tokens per append and
    KV heads; the whole cache after the append is compared byte for byte."""
    torch, mla, _, paging, dev = env
    g = np.random.Generator(np.random.PCG64(6000 + seed))
    batch = int(g.integers(1, 12))
    lens = [int(g.choice([0, 1, 63, 64, 127, 128])) if g.random() < 0.4 else int(g.integers(0, 700))
            for _ in range(batch)]
    s_new = int(g.choice([1, 1, 2, 5, 64, 65]))
    h_kv = int(g.choice([1, 2]))
    w, before, new_kv = make_append_case(lens, s_new, h_kv=h_kv, h_q=2 * h_kv, seed=7000 + seed, extra_pages=1)
    kc = dev16(torch, w.kcache, dev).view(torch.bfloat16)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(before).to(dev)
    new_lens = mla.mla_kv_append(dev16(torch, new_kv, dev).view(torch.bfloat16), sl, bt, kc)
    torch.cuda.synchronize()
    ref, ref_lens = paging.kv_append(w.kcache, w.block_table, before, new_kv)
    what = f"append random seed={seed}: lens={lens} s_new={s_new} h_kv={h_kv}"
    assert np.array_equal(kc.view(torch.int16).cpu().numpy().view(np.uint16), ref), what
    assert np.array_equal(new_lens.cpu().numpy(), ref_lens), what
