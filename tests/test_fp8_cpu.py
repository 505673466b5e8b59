"""CPU pins of the FP8 cache oracle (oracle/fp8.py) against the e4m3 (OCP
E4M3FN) definition and the properties its quantiser must have, plus the C ABI's
argument checks of the FP8 calls (no GPU).

Pins, chosen so that a wrong exponent bias, a dropped subnormal branch, a
wrong tie rule, an off-by-one scale or a misplaced field fails one of them:
values the format fixes (0, 2^-9, 2^-6, 1, 448, NaN, negative zero); exact
round trip of values that are already e4m3 x 2^e with the group maximum at
448 x 2^e; the half-spacing error bound; ties to the even code; minimality of
the power-of-two scale; the rope bytes copied unchanged; all-zero groups.
"""
import ctypes
import math
import os

import numpy as np
import pytest

from oracle import fp8
from workloads import bf16_bits, bf16_to_f32


def test_e4m3_values_fixed_by_the_format():
    v = fp8.e4m3_value
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9
    assert v(0x08) == 2.0 ** -6 and v(0x38) == 1.0 and v(0x39) == 1.125
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0 and math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    pos = [v(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:])), "codes 0..0x7e increase"
    assert v(0x77) == 240.0  # 1.875 * 2^7


def rows_with_latent(lat, rng=None):
    """bf16 bits [n, 576] with the given latent values (exact in bf16) and random rope."""
    rng = rng or np.random.default_rng(0)
    x = np.zeros((lat.shape[0], 576), dtype=np.float32)
    x[:, :512] = lat
    x[:, 512:] = rng.standard_normal((lat.shape[0], 64))
    return bf16_bits(x)


def test_round_trip_exact_for_representable_rows():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 0x7F, size=(8, 512))
    codes[:, ::128] = 0x7E                           # group max 448 -> scale exactly 2^e
    vals = np.array([fp8.e4m3_value(int(c)) for c in codes.ravel()]).reshape(codes.shape)
    sgn = np.where(rng.random(codes.shape) < 0.5, -1.0, 1.0)
    e = rng.integers(-12, 6, size=(8, 4))
    lat = (sgn * vals * np.repeat(2.0 ** e, 128, axis=1)).astype(np.float32)
    bits = rows_with_latent(lat, rng)
    q = fp8.quantize_rows(bits)
    assert np.array_equal(fp8.dequantize_rows(q), bits)
    sc = q[:, 512:528].copy().view(np.float32)
    assert np.array_equal(sc, (2.0 ** e).astype(np.float32))


def test_error_bound_scale_minimality_and_layout():
    rng = np.random.default_rng(2)
    lat = (rng.standard_normal((16, 512)) * np.exp(rng.uniform(-6, 6, size=(16, 1)))).astype(np.float32)
    lat[3, 128:256] = 0.0                            # an all-zero group
    bits = rows_with_latent(lat, rng)
    x = bf16_to_f32(bits).astype(np.float64)
    q = fp8.quantize_rows(bits)
    d = fp8.dequantize_values(q)
    sc = q[:, 512:528].copy().view(np.float32).astype(np.float64)
    for i in range(16):
        for g in range(4):
            blk = x[i, 128 * g:128 * (g + 1)]
            s = sc[i, g]
            amax = np.max(np.abs(blk))
            assert amax <= 448 * s
            assert amax == 0 and s == 1.0 or amax > 448 * s / 2
            y = np.abs(blk) / s
            # half the spacing of e4m3 around y: 2^(floor(log2 y) - 4), or 2^-10 below 2^-6
            half = np.where(y < 2 ** -6, 2.0 ** -10, 2.0 ** (np.floor(np.log2(np.maximum(y, 2 ** -6))) - 4))
            err = np.abs(d[i, 128 * g:128 * (g + 1)] - blk) / s
            assert np.all(err <= half * (1 + 1e-12))
    assert not np.any(q[3, 128:256]) and sc[3, 1] == 1.0
    assert np.array_equal(q[:, 528:].copy().view(np.uint16), bits[:, 512:])   # rope unchanged


def test_ties_go_to_the_even_code():
    # group max 448 keeps the scale at 1; the other entries sit exactly between codes
    lat = np.zeros((1, 512), dtype=np.float32)
    lat[0, 0] = 448.0
    lat[0, 1] = 1.0625      # between 1.0 (0x38) and 1.125 (0x39) -> 0x38
    lat[0, 2] = 1.1875      # between 1.125 (0x39) and 1.25 (0x3a) -> 0x3a
    lat[0, 3] = 7.5 * 2 ** -9   # between 0x07 and 0x08 -> 0x08
    lat[0, 4] = 0.5 * 2 ** -9   # between 0 and 0x01 -> 0
    lat[0, 5] = -1.0625     # -> 0xb8
    lat[0, 6] = 232.0       # between 224 (0x76) and 240 (0x77) -> 0x76
    q = fp8.quantize_rows(rows_with_latent(lat))
    assert list(q[0, :7]) == [0x7E, 0x38, 0x3A, 0x08, 0x00, 0xB8, 0x76]


def test_fp8_cache_generator_is_valid():
    import workloads
    w = workloads.make_workload([70, 3], s_q=1, h_q=16, seed=1)
    c = workloads.make_fp8_cache(w, 1)
    assert c.shape == w.kcache.shape[:-1] + (656,)
    b = fp8.bf16_cache(c)              # exact dequantisation (asserts representability)
    assert np.array_equal(b[..., 512:], w.kcache[..., 512:])
    assert np.all(np.isfinite(bf16_to_f32(b)))


# ---- C ABI argument checks of the FP8 calls -------------------------------

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "paged_mla_decode_02_amd", "libmla.so")
FAKE = 0x100000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libmla.so not built")
    lib = ctypes.CDLL(LIB)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    for n in ("mla_decode_paged_fp8", "mla_decode_splitkv_fp8"):
        getattr(lib, n).argtypes = [P, P, ctypes.c_int64, P, I, P, I, I, I, I, I, I, I, P, I, P, I,
                                    ctypes.c_float, P, P, P, SZ, P]
    lib.mla_kv_append_fp8.argtypes = [P, I, I, I, P, P, I, P, ctypes.c_int64, P, P]
    lib.mla_last_error.restype = ctypes.c_char_p
    return lib


def test_fp8_decode_rejects(lib):
    def call(fn, h_q=16, s_q=1, ws=1 << 30, kc=FAKE):
        return fn(FAKE, kc, 100, FAKE, 8, FAKE, 4, s_q, h_q, 1, 576, 512, 64, FAKE, 256, FAKE, 0, 0.1,
                  FAKE, FAKE, FAKE, ws, None)
    for fn in (lib.mla_decode_paged_fp8, lib.mla_decode_splitkv_fp8):
        assert call(fn, kc=None) == -1
        assert call(fn, kc=FAKE + 4) == -1      # alignment
        assert call(fn, ws=16) == -3


def test_fp8_append_rejects(lib):
    f = lib.mla_kv_append_fp8
    assert f(FAKE, -1, 1, 1, FAKE, FAKE, 8, FAKE, 10, None, None) == -1
    assert f(None, 4, 1, 1, FAKE, FAKE, 8, FAKE, 10, None, None) == -1
    assert f(FAKE, 4, 1, 1, FAKE, FAKE, 8, FAKE + 8, 10, None, None) == -1
    assert f(None, 0, 1, 1, None, None, 8, None, 10, None, None) == 0
