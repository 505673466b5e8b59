"""CPU oracle of the FP8 latent cache -- test infrastructure only (tests/, the
smoke entry point and bench.py's CPU baseline may import it; the product
library never does).  Plain numpy; it shares no code with the HIP path.

The pages name FP8 as the kernel's low-precision mode (FP8/FP16 mixed
precision on the FP8 instruction set: "Flash MLA: efficient MLA decoding kernel
library for variable-length sequences", developer.baidu.com, §三.2 and §四
step 3) and say nothing of the number format or the scale granularity.  The
reading used here:

  * row of one token and KV head: 656 bytes =
      512 x e4m3 (OCP "E4M3FN": 1 sign, 4 exponent bits with bias 7, 3 mantissa
                  bits; no infinities, S.1111.111 is NaN, largest finite 448)
      4 x fp32 scale, one per 128 latent dims (little endian)
      64 x bf16 rope dims, copied unchanged;
  * each scale is a power of two, the smallest 2^e with max|x| <= 448 * 2^e over
    its 128 dims (2^0 for an all-zero group), so q * 2^e is exactly a bf16
    value and dequantisation is exact;
  * quantisation rounds x / 2^e to the nearest e4m3 value, ties to the even
    code (the one with a zero last mantissa bit).

Functions: ``e4m3_value(code)`` (the format's definition), ``quantize_rows``,
``dequantize_rows`` (to bf16 bits), ``fp8_cache(kcache_bits)`` (a whole bf16
cache in this format) and ``bf16_cache(kcache_fp8)`` (its exact bf16 view, for
the fp64 decode oracle).
"""
from __future__ import annotations

import math

import numpy as np

LATENT, ROPE, GROUP = 512, 64, 128
ROW_BYTES = LATENT + 4 * (LATENT // GROUP) + 2 * ROPE  # 656
E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of an e4m3 (E4M3FN) byte, from the format's definition."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# non-negative finite codes 0x00 .. 0x7e, increasing in value
_POS = np.array([e4m3_value(c) for c in range(0x7F)], dtype=np.float64)


def _round_e4m3(y: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code to each |y| <= 448 (ties to the even code), with sign."""
    a = np.abs(y)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, len(_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    d_hi = np.abs(_POS[hi] - a)
    d_lo = np.abs(a - _POS[lo])
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (lo != hi)
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    return (pick.astype(np.uint8) | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)).astype(np.uint8)


def _scale_exponent(amax: float) -> int:
    """Smallest e with amax <= 448 * 2^e (0 when amax == 0)."""
    if amax == 0.0:
        return 0
    e = math.ceil(math.log2(amax / E4M3_MAX))
    while amax > E4M3_MAX * 2.0 ** e:       # guard the float log at exact powers of two
        e += 1
    while e > -200 and amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return e


def _f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def quantize_rows(bits: np.ndarray) -> np.ndarray:
    """bf16 bits [..., 576] -> fp8 rows uint8 [..., 656]."""
    bits = np.asarray(bits, dtype=np.uint16)
    lead = bits.shape[:-1]
    x = _f64(bits.reshape(-1, LATENT + ROPE))
    n = x.shape[0]
    out = np.zeros((n, ROW_BYTES), dtype=np.uint8)
    scales = np.zeros((n, LATENT // GROUP), dtype=np.float32)
    for g in range(LATENT // GROUP):
        blk = x[:, g * GROUP:(g + 1) * GROUP]
        for i in range(n):
            e = _scale_exponent(float(np.max(np.abs(blk[i]))))
            scales[i, g] = np.float32(2.0 ** e)
            out[i, g * GROUP:(g + 1) * GROUP] = _round_e4m3(blk[i] / 2.0 ** e)
    out[:, LATENT:LATENT + 16] = scales.view(np.uint8).reshape(n, 16)
    rope = np.ascontiguousarray(bits.reshape(-1, LATENT + ROPE)[:, LATENT:])
    out[:, LATENT + 16:] = rope.view(np.uint8).reshape(n, 2 * ROPE)
    return out.reshape(lead + (ROW_BYTES,))


def dequantize_values(rows: np.ndarray) -> np.ndarray:
    """fp8 rows uint8 [..., 656] -> fp64 values [..., 576] (q * scale, rope as is)."""
    rows = np.asarray(rows, dtype=np.uint8)
    lead = rows.shape[:-1]
    r = rows.reshape(-1, ROW_BYTES)
    table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    q = table[r[:, :LATENT]]
    sc = np.ascontiguousarray(r[:, LATENT:LATENT + 16]).view(np.float32).astype(np.float64)
    lat = q * np.repeat(sc, GROUP, axis=1)
    rope = _f64(np.ascontiguousarray(r[:, LATENT + 16:]).view(np.uint16))
    return np.concatenate([lat, rope], axis=1).reshape(lead + (LATENT + ROPE,))


def dequantize_rows(rows: np.ndarray) -> np.ndarray:
    """fp8 rows -> bf16 bits [..., 576]; exact (every q * 2^e is a bf16 value)."""
    v = dequantize_values(rows).astype(np.float32)
    b = v.view(np.uint32)
    # exact: truncation is rounding here because the low 16 bits are zero
    assert not np.any(b & np.uint32(0xFFFF)), "dequantised value not representable in bf16"
    return (b >> np.uint32(16)).astype(np.uint16)


def fp8_cache(kcache_bits: np.ndarray) -> np.ndarray:
    """bf16 cache [pages, 64, h_kv, 576] -> fp8 cache uint8 [pages, 64, h_kv, 656]."""
    return quantize_rows(kcache_bits)


def bf16_cache(kcache_fp8: np.ndarray) -> np.ndarray:
    """fp8 cache -> the bf16 cache it stands for (exact)."""
    return dequantize_rows(kcache_fp8)
