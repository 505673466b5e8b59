"""GPU parity of the absorption GEMMs and of the whole MLA decode layer
(absorb -> schedule -> latent decode -> up-projection), through the C ABI,
against the CPU oracle (oracle/mla_layer.py) on the same seeded inputs.

Bars:
* each GEMM output is one fp32 dot product of n products rounded once to bf16:
  per element within 2^-8 of the exact value plus the worst-case fp32
  accumulation error n 2^-24 sum |a_i b_i| (which matters only where the sum
  cancels), and equal to the exact result rounded to nearest-even (oracle
  round_bf16) in all but at most 1e-3 of the elements (a GEMM that truncated
  instead of rounding would miss about half of them); the rope part of the
  absorbed query is a bit-exact copy;
* the layer: the ABI's query is bf16, so the oracle chain rounds the fp64
  absorbed query to bf16 before the C decode oracle and then up-projects in
  fp64; against that chain out rel-L2 <= 1e-2 and lse abs <= 1e-3, the decode's
  own bars;
* against attention computed WITHOUT absorption (per-head keys and values) the
  output keeps rel-L2 <= 1e-2, and lse may differ by the bf16 rounding of the
  absorbed query: per row at most 1e-3 + scale * 2^-9 * max_t sum_i |q~_i K_t,i|
  (each query element moves by at most 2^-9 of itself, and lse moves by at most
  the largest score change).
"""
import numpy as np
import pytest

import workloads
from workloads import make_layer_inputs, make_workload

pytestmark = pytest.mark.gpu

TOL = 1e-2
LSE_TOL = 1e-3


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


def check_rounded_once(got_bits, ref64, absdot, n_terms, ml, what):
    """got = one fp32 dot product of n_terms products, rounded once to bf16.
    Per element |got - exact| <= 2^-8 |exact| (the bf16 rounding, with margin)
    + n_terms 2^-24 sum_i |a_i b_i| (the worst-case fp32 accumulation error,
    which dominates where the sum cancels); and got differs from the exact
    result rounded to nearest-even in at most 1e-3 of the elements."""
    got = workloads.bf16_to_f32(got_bits).astype(np.float64)
    err = np.abs(got - ref64)
    tol = 2.0 ** -8 * np.abs(ref64) + n_terms * 2.0 ** -24 * absdot
    assert np.all(err <= tol), f"{what}: error {np.max(err - tol):.3e} over the bound"
    off = np.count_nonzero(np.asarray(got_bits) != ml.round_bf16(ref64)) / max(ref64.size, 1)
    assert off <= 1e-3, f"{what}: {off:.2e} of the elements differ from the rounded fp64 result"


def bits_of(torch, t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


# Each GEMM has a form for few tokens and one for many, picked by the grid size:
# absorb takes 32-column workgroups while h_q * 4 * ceil(T / 128) < 512 and the
# up-projection splits its reduction over the waves while h_q * ceil(T / 32) <
# 256.  T = 128, h_q = 64 takes the narrow absorb with the wide up-projection;
# T = 264, h_q = 128 the wide form of both; the others the narrow forms.
@pytest.mark.parametrize("batch,s_q,h_q", [(1, 1, 1), (2, 1, 16), (3, 11, 5), (64, 1, 16), (64, 2, 64),
                                           (132, 2, 128)])
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
    got_q = bits_of(torch, q_abs)
    f = workloads.bf16_to_f32
    absdot_q = np.einsum("...hn,hnc->...hc", np.abs(f(lay.q_nope).astype(np.float64)),
                         np.abs(f(lay.w_uk).astype(np.float64)))
    check_rounded_once(got_q[..., :512], ref_q[..., :512], absdot_q, 128, ml, "absorb_q")
    assert np.array_equal(got_q[..., 512:], lay.q_rope)
    ref_o = ml.unabsorb_out(workloads.bf16_to_f32(o_bits).astype(np.float64), lay.w_uv)
    absdot_o = np.einsum("hvc,...hc->...hv", np.abs(f(lay.w_uv).astype(np.float64)),
                         np.abs(f(o_bits).astype(np.float64)))
    check_rounded_once(bits_of(torch, out), ref_o, absdot_o, 512, ml, "unabsorb_out")


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


def check_layer(got_o, got_l, ref_o, ref_l, what, lse_tol):
    assert rel_l2(got_o, ref_o) < TOL, what
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(got_l)), what
    err = np.abs(got_l[fin] - ref_l[fin])
    tol = np.broadcast_to(lse_tol, ref_l.shape)[fin]
    assert np.all(err <= tol), f"{what}: lse error {np.max(err - tol):.2e} over the bar"


@pytest.mark.parametrize("lens,s_q,h_q,causal", [([218, 164], 1, 16, False), ([1, 70, 300], 2, 8, True),
                                                 ([0, 129], 1, 4, False)])
def test_layer_small(env, lens, s_q, h_q, causal):
    _, _, ml, _ = env
    w = make_workload(lens, s_q=s_q, h_q=h_q, causal=causal, seed=31)
    lay = make_layer_inputs(len(lens), s_q, h_q, seed=32)
    got_o, got_l = run_layer(env, w, lay)
    n = w.batch * w.s_q * w.h_q
    got_o, got_l = got_o.reshape(n, -1), got_l.reshape(n)
    ref_o, ref_l, q64 = ml.bf16_query_chain(w, lay)
    check_layer(got_o, got_l, ref_o, ref_l, "layer vs bf16-query chain", LSE_TOL)
    un_o, un_l = ml.unabsorbed_attention(w, lay)
    check_layer(got_o, got_l, un_o.reshape(n, -1), un_l.reshape(n), "layer vs unabsorbed attention",
                LSE_TOL + ml.query_rounding_bound(w, q64, range(n)))


@pytest.mark.parametrize("cfg", [1, 3])
def test_layer_full_size(env, cfg):
    """Full-size workloads: every row against the chain oracle; a seeded sample
    of rows against the unabsorbed attention (computed per head, one by one)."""
    _, _, ml, _ = env
    w = workloads.config_workload(cfg)
    lay = make_layer_inputs(w.batch, w.s_q, w.h_q, seed=100 + cfg)
    got_o, got_l = run_layer(env, w, lay)
    n = w.batch * w.s_q * w.h_q
    got_o, got_l = got_o.reshape(n, -1), got_l.reshape(n)
    ref_o, ref_l, q64 = ml.bf16_query_chain(w, lay)
    check_layer(got_o, got_l, ref_o, ref_l, f"config {cfg} vs bf16-query chain", LSE_TOL)
    sel = np.sort(np.random.default_rng(cfg).choice(n, size=24, replace=False))
    un_o, un_l = ml.unabsorbed_attention(w, lay, sel=sel)
    check_layer(got_o[sel], got_l[sel], un_o, un_l, f"config {cfg} vs unabsorbed attention",
                LSE_TOL + ml.query_rounding_bound(w, q64, sel))
