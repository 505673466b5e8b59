"""GPU parity of the absorption GEMMs and of the whole MLA decode layer
(absorb -> schedule -> latent decode -> up-projection), through the C ABI,
against the CPU oracle (oracle/mla_layer.py) on the same seeded inputs.

Bars: relative L2 <= 1e-2 on every floating-point output (the decode's bar;
the GEMMs accumulate in fp32 and round once to bf16, so they land near 2e-3);
the rope part of the absorbed query is a bit-exact copy.  The layer output is
compared with attention computed WITHOUT absorption (per-head keys and values),
for every row on small workloads and on a seeded sample of rows at full size.
"""
import numpy as np
import pytest

import workloads
from workloads import make_layer_inputs, make_workload

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    from oracle import mla_layer
    import paged_mla_decode_02_amd as mla
    oracle.build(force=False)
    return torch, mla, mla_layer, torch.device("cuda:0")


def dev_bf16(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    n = np.linalg.norm(ref)
    return np.linalg.norm(got - ref) / (n if n > 0 else 1.0)


@pytest.mark.parametrize("batch,s_q,h_q", [(1, 1, 1), (2, 1, 16), (3, 11, 5), (64, 1, 16), (132, 2, 128)])
def test_absorb_and_unabsorb(env, batch, s_q, h_q):
    torch, mla, ml, dev = env
    lay = make_layer_inputs(batch, s_q, h_q, seed=batch * 7 + h_q)
    qn, qr = dev_bf16(torch, lay.q_nope, dev), dev_bf16(torch, lay.q_rope, dev)
    wuk, wuv = dev_bf16(torch, lay.w_uk, dev), dev_bf16(torch, lay.w_uv, dev)
    q_abs = mla.mla_absorb_q(qn, qr, wuk)
    rng = np.random.default_rng(batch + h_q)
    o_bits = workloads.bf16_bits(rng.standard_normal((batch, s_q, h_q, 512), dtype=np.float32))
    out = mla.mla_unabsorb_out(dev_bf16(torch, o_bits, dev), wuv)
    torch.cuda.synchronize()
    ref_q = ml.absorb_q(lay.q_nope, lay.q_rope, lay.w_uk)
    got_q = q_abs.float().cpu().numpy()
    assert rel_l2(got_q[..., :512], ref_q[..., :512]) < TOL
    assert np.array_equal(q_abs.view(torch.int16).cpu().numpy()[..., 512:].view(np.uint16), lay.q_rope)
    ref_o = ml.unabsorb_out(workloads.bf16_to_f32(o_bits).astype(np.float64), lay.w_uv)
    assert rel_l2(out.float().cpu().numpy(), ref_o) < TOL


def test_zero_tokens_launches_nothing(env):
    torch, mla, _, dev = env
    e = torch.empty((0, 4, 128), dtype=torch.bfloat16, device=dev)
    r = torch.empty((0, 4, 64), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((4, 128, 512), dtype=torch.bfloat16, device=dev)
    assert mla.mla_absorb_q(e, r, w).shape == (0, 4, 576)
    o = torch.empty((0, 4, 512), dtype=torch.bfloat16, device=dev)
    assert mla.mla_unabsorb_out(o, w).shape == (0, 4, 128)


def run_layer(env, w, lay):
    torch, mla, _, dev = env
    q_abs = mla.mla_absorb_q(dev_bf16(torch, lay.q_nope, dev), dev_bf16(torch, lay.q_rope, dev),
                             dev_bf16(torch, lay.w_uk, dev))
    kc = dev_bf16(torch, w.kcache, dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.cache_seqlens).to(dev)
    md, ns = mla.get_mla_metadata(sl, w.rows, w.h_kv)
    o_lat, lse = mla.flash_mla_with_kvcache(q_abs, kc, bt, sl, 512, md, ns, softmax_scale=w.scale, causal=w.causal)
    out = mla.mla_unabsorb_out(o_lat, dev_bf16(torch, lay.w_uv, dev))
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("lens,s_q,h_q,causal", [([218, 164], 1, 16, False), ([1, 70, 300], 2, 8, True),
                                                 ([0, 129], 1, 4, False)])
def test_layer_small(env, lens, s_q, h_q, causal):
    _, _, ml, _ = env
    w = make_workload(lens, s_q=s_q, h_q=h_q, causal=causal, seed=31)
    lay = make_layer_inputs(len(lens), s_q, h_q, seed=32)
    got_o, got_l = run_layer(env, w, lay)
    ref_o, ref_l = ml.unabsorbed_attention(w, lay)
    assert rel_l2(got_o, ref_o) < TOL
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(got_l))
    assert np.max(np.abs(got_l[fin] - ref_l[fin]), initial=0.0) < 1e-2


@pytest.mark.parametrize("cfg", [1, 3])
def test_layer_full_size_sampled(env, cfg):
    _, _, ml, _ = env
    w = workloads.config_workload(cfg)
    lay = make_layer_inputs(w.batch, w.s_q, w.h_q, seed=100 + cfg)
    got_o, got_l = run_layer(env, w, lay)
    n = w.batch * w.s_q * w.h_q
    sel = np.random.default_rng(cfg).choice(n, size=24, replace=False)
    ref_o, ref_l = ml.unabsorbed_attention(w, lay, sel=sel)
    assert rel_l2(got_o.reshape(n, -1)[sel], ref_o) < TOL
    assert np.max(np.abs(got_l.reshape(-1)[sel] - ref_l)) < 1e-2
