"""mla_decode_paged_noalloc through the C ABI against mla_decode_paged on the
same inputs: out and lse bit-identical (the same kernels run; only where the
split partials live differs), on calls in a row on one GPU, each later one
smaller than the one before, so that a later call runs over what the earlier
one left in the shared scratch array.  The reference call gets a NaN-filled
workspace, so a result that depended on stale partials could not match it."""
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


def tensors(torch, w, dev):
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kc = torch.from_numpy(w.kcache.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.cache_seqlens).to(dev)
    return q, kc, bt, sl


def both(env, w, num_parts=None):
    torch, mla, dev = env
    q, kc, bt, sl = tensors(torch, w, dev)
    md, ns = mla.mla_get_metadata(sl, w.rows, w.h_kv, num_parts=num_parts)
    P = md.shape[0]
    need = (w.batch + P) * w.h_kv * w.rows * 513 * 4
    assert need <= mla.NOALLOC_SCRATCH_BYTES
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev)
    ref_out, ref_lse = mla.mla_decode_paged(q, kc, bt, sl, w.dv, md, ns, w.causal, w.scale, workspace=ws)
    out = torch.full_like(ref_out, 3.0)
    lse = torch.full_like(ref_lse, 3.0)
    mla.mla_decode_paged_noalloc(q, kc, bt, sl, w.dv, md, ns, w.causal, w.scale, out, lse)
    torch.cuda.synchronize()
    assert int(ns[-1].item()) > w.batch, "the case must split some sequence (the scratch holds partials)"
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "out differs"
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), "lse differs"
    return need


def test_noalloc_matches_decode_paged_calls_in_a_row(env):
    sizes = []
    # long_context: 64 rows, ~32 chunks per sequence
    sizes.append(both(env, workloads.config_workload(4)))
    # smaller: memory_bound_varlen, 16 rows
    sizes.append(both(env, workloads.config_workload(1)))
    # smaller again, forced splits, causal s_q = 2: 256 rows on the 128-row kernel
    sizes.append(both(env, make_workload([700, 3, 129], s_q=2, h_q=128, causal=True, seed=7, outliers=True),
                      num_parts=9))
    # smaller again, forced splits, causal s_q = 2 on the 64-row kernel
    sizes.append(both(env, make_workload([700, 3, 129], s_q=2, h_q=64, causal=True, seed=5, outliers=True),
                      num_parts=9))
    assert sizes[0] > sizes[1] > sizes[2] > sizes[3]


def test_noalloc_rejects_a_call_beyond_the_scratch(env):
    torch, mla, dev = env
    w = make_workload([70] * 700, s_q=2, h_q=128, seed=6)  # (700 + P) * 256 rows * 513 * 4 B > 256 MiB
    q, kc, bt, sl = tensors(torch, w, dev)
    md, ns = mla.mla_get_metadata(sl, w.rows, w.h_kv)
    out = torch.empty((w.batch, w.s_q, w.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.s_q, w.h_q), dtype=torch.float32, device=dev)
    with pytest.raises(mla.MlaError, match="scratch"):
        mla.mla_decode_paged_noalloc(q, kc, bt, sl, w.dv, md, ns, w.causal, w.scale, out, lse)
