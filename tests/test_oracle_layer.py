"""Pins of the MLA layer oracle (oracle/mla_layer.py) against what the pages and
the mathematics fix, independently of its own formulas:

* the absorption GEMM and the up-projection against explicit loops on a few
  heads and tokens (a transposed or mis-indexed weight fails);
* a closed form: W_UK[h] = [I_128 | 0] makes the absorbed latent query the
  nope query followed by zeros;
* the layer identity of the "FlashMLA inference acceleration" notes
  (dpshk.com/news/5996785), §2.1: absorb -> latent decode (the C oracle) ->
  up-projection equals per-head attention with up-projected keys and values.
"""
import math

import numpy as np
import pytest

from oracle import mla_layer
from workloads import bf16_bits, make_layer_inputs, make_workload

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def f64(bits):
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def test_absorb_against_loops():
    lay = make_layer_inputs(1, 3, 2, seed=11)
    got = mla_layer.absorb_q(lay.q_nope, lay.q_rope, lay.w_uk)
    qn, qr, w = f64(lay.q_nope), f64(lay.q_rope), f64(lay.w_uk)
    for s in range(3):
        for h in range(2):
            for c in range(0, 512, 37):
                acc = 0.0
                for n in range(128):
                    acc += qn[0, s, h, n] * w[h, n, c]
                assert abs(got[0, s, h, c] - acc) < 1e-12 * (1 + abs(acc))
            for r in range(64):
                assert got[0, s, h, 512 + r] == qr[0, s, h, r]


def test_unabsorb_against_loops():
    lay = make_layer_inputs(1, 2, 2, seed=12)
    rng = np.random.default_rng(3)
    o = rng.standard_normal((1, 2, 2, 512))
    got = mla_layer.unabsorb_out(o, lay.w_uv)
    w = f64(lay.w_uv)
    for s in range(2):
        for h in range(2):
            for v in range(0, 128, 9):
                acc = 0.0
                for c in range(512):
                    acc += w[h, v, c] * o[0, s, h, c]
                assert abs(got[0, s, h, v] - acc) < 1e-12 * (1 + abs(acc))


def test_absorb_identity_weight_closed_form():
    lay = make_layer_inputs(2, 1, 3, seed=13)
    eye = np.zeros((3, 128, 512), dtype=np.float32)
    for h in range(3):
        eye[h, :, :128] = np.eye(128, dtype=np.float32)
    got = mla_layer.absorb_q(lay.q_nope, lay.q_rope, bf16_bits(eye))
    assert np.array_equal(got[..., :128], f64(lay.q_nope))
    assert not np.any(got[..., 128:512])


@pytest.mark.parametrize("causal,s_q", [(False, 1), (True, 2)])
def test_layer_identity(oracle_lib, causal, s_q):
    """absorb -> latent decode -> up-projection == unabsorbed attention.

    W_UK and q_nope are small integers so that the absorbed query is exact in
    bf16 and the two sides agree to rounding of fp64 sums."""
    rng = np.random.default_rng(21)
    H, lens = 4, [130, 64, 1]
    w = make_workload(lens, s_q=s_q, h_q=H, causal=causal, seed=5)
    lay = make_layer_inputs(len(lens), s_q, H, seed=6)
    lay.q_nope = bf16_bits(rng.integers(-1, 2, size=lay.q_nope.shape).astype(np.float32))
    lay.w_uk = bf16_bits(rng.integers(-1, 2, size=lay.w_uk.shape).astype(np.float32))
    q_abs = mla_layer.absorb_q(lay.q_nope, lay.q_rope, lay.w_uk)
    qb = bf16_bits(q_abs.astype(np.float32))
    assert np.array_equal(f64(qb), q_abs), "absorbed query must be exact in bf16 here"
    w.q = qb
    o_lat, lse_lat = oracle_lib.decode(w)
    o_lat = o_lat.reshape(w.batch, s_q, H, 512)
    lse_lat = lse_lat.reshape(w.batch, s_q, H)
    out = mla_layer.unabsorb_out(o_lat, lay.w_uv)
    ref_out, ref_lse = mla_layer.unabsorbed_attention(w, lay)
    np.testing.assert_allclose(out, ref_out, rtol=1e-10, atol=1e-10)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse_lat))
    np.testing.assert_allclose(lse_lat[fin], ref_lse[fin], rtol=0, atol=1e-10)
    # sampled rows agree with the full evaluation
    sel = [0, 5, w.batch * s_q * H - 1]
    so, sl = mla_layer.unabsorbed_attention(w, lay, sel=sel)
    np.testing.assert_allclose(so, ref_out.reshape(-1, 128)[sel], rtol=0, atol=0)
    assert math.isclose(sl[0], ref_lse.reshape(-1)[0], rel_tol=0, abs_tol=0)


def test_round_bf16_hand_values():
    """bf16 keeps 7 stored mantissa bits: near 1 its spacing is 2^-7, so 1 + 2^-8
    is a tie (to the even 1.0), 1 + 3*2^-8 a tie between odd 1 + 2^-7 and even
    1 + 2^-6, and 2 - 2^-9 lies nearer 2 than 2 - 2^-7."""
    cases = {
        1.0 + 2.0 ** -8: 0x3F80,
        1.0 + 3 * 2.0 ** -8: 0x3F82,
        -(1.0 + 2.0 ** -8): 0xBF80,
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,
        2.0 - 2.0 ** -9: 0x4000,
        2.0 - 2.0 ** -7: 0x3FFF,
        0.0: 0x0000,
        3.0: 0x4040,
        2.0 ** -100 * (1 + 2.0 ** -7): 0x0D81,
    }
    got = mla_layer.round_bf16(np.array(list(cases.keys())))
    assert [int(g) for g in got] == list(cases.values())


def test_round_bf16_against_fp32_bit_rounding():
    """On fp32 values (exact in fp64) one rounding to bf16 is the integer
    round-to-nearest-even of the fp32 bit pattern (workloads.bf16_bits)."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-40, 40, 200000))).astype(np.float32)
    x[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.5, 2.0 ** -126]
    assert np.array_equal(mla_layer.round_bf16(x.astype(np.float64)), bf16_bits(x))


def test_round_bf16_keeps_bf16_values():
    rng = np.random.default_rng(6)
    bits = rng.integers(0x0080, 0x7F80, 50000).astype(np.uint16) | (rng.integers(0, 2, 50000) << 15).astype(np.uint16)
    assert np.array_equal(mla_layer.round_bf16(f64(bits)), bits)


def test_bf16_query_chain_within_the_rounding_bound():
    """The chain (bf16-rounded absorbed query -> C decode oracle -> up-projection)
    and the unabsorbed per-head attention differ only by the query's rounding:
    lse within the derived per-row bound, and the bound is not vacuous (it is
    small against the lse values and the two results do differ)."""
    w = make_workload([218, 1, 70], s_q=2, h_q=8, causal=True, seed=41)
    lay = make_layer_inputs(3, 2, 8, seed=42)
    n = w.batch * w.s_q * w.h_q
    out_c, lse_c, q64 = mla_layer.bf16_query_chain(w, lay)
    out_u, lse_u = mla_layer.unabsorbed_attention(w, lay)
    out_u, lse_u = out_u.reshape(n, -1), lse_u.reshape(n)
    bound = mla_layer.query_rounding_bound(w, q64, range(n))
    fin = np.isfinite(lse_u)
    assert np.array_equal(fin, np.isfinite(lse_c))
    diff = np.abs(lse_c[fin] - lse_u[fin])
    assert np.all(diff <= bound[fin] * (1 + 1e-9))
    assert 0 < np.max(diff) and np.max(bound) < 0.05
    rel = np.linalg.norm(out_c - out_u) / np.linalg.norm(out_u)
    assert 0 < rel < 1e-2


def test_truncation_fails_the_rounded_once_bar():
    """The GPU GEMM bar (at most 1e-3 of the elements one ulp away from the
    fp64 result rounded to nearest-even) rejects a GEMM that truncates."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal(20000) * 0.5
    rne = mla_layer.round_bf16(x).astype(np.int64)
    trunc = (np.abs(x).astype(np.float32).view(np.uint32) >> 16).astype(np.int64)  # toward zero, magnitude
    mag_rne = rne & 0x7FFF
    frac_off = np.count_nonzero(trunc != mag_rne) / x.size
    assert frac_off > 0.3
