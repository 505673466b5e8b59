"""CPU oracle for the MLA decode layer around the latent decode -- test
infrastructure only (tests/, the smoke entry point and bench.py's CPU baseline
may import it; the product library never does).  Plain numpy in fp64 on the
exact bf16 input values; it shares no code with the HIP path.

What it computes, per query head h (d_nope = d_v = 128, latent 512, rope 64):

  absorb_q:      q~[t,h,0:512] = sum_n q_nope[t,h,n] W_UK[h,n,:],  q~[t,h,512:] = q_rope[t,h,:]
  round_bf16:    the bf16 value the decode's query argument holds (round to
                 nearest, ties to even, from the exact fp64 value)
  unabsorb_out:  out[t,h,v]    = sum_c W_UV[h,v,c] o_lat[t,h,c]
  bf16_query_chain: absorb_q, round_bf16, the C latent-decode oracle and the
      up-projection in a row: what the library's absorb -> decode -> unabsorb
      chain computes up to its own rounding.
  unabsorbed_attention: the MLA attention the two GEMMs and the latent decode
      must reproduce, computed WITHOUT absorption: every head gets its own keys
      k_t = [W_UK[h] c_t ; k_rope_t] and values v_t = W_UV[h] c_t from the cached
      latent c_t = K_t[0:512] and rope key K_t[512:576], and
      out = sum_t softmax(scale q.k)_t v_t over the visible keys (bottom-right
      causal when s_q > 1), lse = ln sum_t exp(scale q.k_t).

The absorption identity q.(W_UK c) = (W_UK^T q).c and the commuting of W_UV
with the softmax-weighted sum are the "FlashMLA inference acceleration" notes
(dpshk.com/news/5996785), §2.1; the unabsorbed form is the per-head attention
those notes start from.  Matrix products use numpy's matmul as a library step.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

_PAGE = 64
_LATENT = 512


def _f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 values -> bf16 bit patterns (uint16), one rounding to nearest with
    ties to even (bf16 keeps 8 significant bits: 1 implicit + 7 stored).

    x is scaled by a power of two so that its 8 significant bits are the integer
    part, rounded with numpy's round-half-to-even, and scaled back: every step
    is exact in fp64.  Values in bf16's normal range only (the layer's queries)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.float64)
    nz = x != 0
    e = np.floor(np.log2(np.abs(x[nz])))
    # guard the floor(log2) of values just below a power of two
    e = np.where(np.abs(x[nz]) < np.ldexp(1.0, e.astype(np.int64)), e - 1, e)
    ulp = np.ldexp(1.0, (e - 7).astype(np.int64))
    out[nz] = np.round(x[nz] / ulp) * ulp
    f = out.astype(np.float32)  # exact: 8 significant bits
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def absorb_q(q_nope_bits: np.ndarray, q_rope_bits: np.ndarray, w_uk_bits: np.ndarray) -> np.ndarray:
    """q~ [..., h, 576] in fp64 from q_nope [..., h, 128], q_rope [..., h, 64], W_UK [h, 128, 512]."""
    qn = _f64(q_nope_bits)
    w = _f64(w_uk_bits)
    lat = np.einsum("...hn,hnc->...hc", qn, w)
    return np.concatenate([lat, _f64(q_rope_bits)], axis=-1)


def unabsorb_out(o_lat: np.ndarray, w_uv_bits: np.ndarray) -> np.ndarray:
    """out [..., h, 128] in fp64 from o_lat [..., h, 512] (fp64 values) and W_UV [h, 128, 512]."""
    w = _f64(w_uv_bits)
    return np.einsum("hvc,...hc->...hv", w, np.asarray(o_lat, dtype=np.float64))


def unabsorbed_attention(w, layer, scale: Optional[float] = None,
                         sel: Optional[Sequence[int]] = None):
    """Reference MLA decode attention without absorption.

    ``w`` is a workloads.Workload (paged latent cache, lengths, block table,
    causal flag, h_kv must be 1); ``layer`` a workloads.LayerInputs.  Returns
    (out [b, s_q, h_q, 128], lse [b, s_q, h_q]) in fp64, or, with ``sel`` (flat
    indices (b * s_q + s) * h_q + h), the selected rows only as ([n, 128], [n])."""
    if w.h_kv != 1:
        raise ValueError("the layer reference covers one latent KV head")
    scale = w.scale if scale is None else scale
    qn = _f64(layer.q_nope)
    qr = _f64(layer.q_rope)
    w_uk = _f64(layer.w_uk)
    w_uv = _f64(layer.w_uv)
    b, s_q, h_q = w.batch, w.s_q, w.h_q
    flat = range(b * s_q * h_q) if sel is None else list(sel)
    outs, lses = [], []
    cache = {}
    for idx in flat:
        bi, rem = divmod(int(idx), s_q * h_q)
        s, h = divmod(rem, h_q)
        L = int(w.cache_seqlens[bi])
        n = L if not w.causal else max(0, L - s_q + s + 1)
        if bi not in cache:
            rows = [w.kcache[w.block_table[bi, t // _PAGE], t % _PAGE, 0] for t in range(L)]
            cache[bi] = _f64(np.array(rows, dtype=np.uint16).reshape(L, -1)) if L else np.zeros((0, 576))
        K = cache[bi][:n]
        if n == 0:
            outs.append(np.zeros(w_uv.shape[1]))
            lses.append(-math.inf)
            continue
        c, k_rope = K[:, :_LATENT], K[:, _LATENT:]
        k_nope = c @ w_uk[h].T          # per-head keys [n, 128]
        v = c @ w_uv[h].T               # per-head values [n, 128]
        x = scale * (k_nope @ qn[bi, s, h] + k_rope @ qr[bi, s, h])
        m = x.max()
        p = np.exp(x - m)
        z = p.sum()
        outs.append((p / z) @ v)
        lses.append(m + math.log(z))
    out = np.array(outs)
    lse = np.array(lses)
    if sel is None:
        return out.reshape(b, s_q, h_q, -1), lse.reshape(b, s_q, h_q)
    return out, lse


def bf16_query_chain(w, layer, sel: Optional[Sequence[int]] = None):
    """The layer as the decode's ABI runs it: the absorbed query in fp64
    (absorb_q), rounded to bf16 (round_bf16: the decode takes a bf16 query),
    the C latent-decode oracle on that query, and the up-projection in fp64.

    Returns (out [n, 128], lse [n], q~ fp64 [b, s_q, h_q, 576]) for all rows
    (n = b * s_q * h_q) or the flat indices in ``sel``."""
    import dataclasses

    from oracle import default

    q64 = absorb_q(layer.q_nope, layer.q_rope, layer.w_uk)
    wq = dataclasses.replace(w, q=round_bf16(q64))
    o_lat, lse = default().decode(wq, sel=sel)
    w_uv = _f64(layer.w_uv)
    rows = np.arange(w.batch * w.s_q * w.h_q) if sel is None else np.asarray(sel, dtype=np.int64)
    heads = rows % w.h_q
    out = np.empty((rows.shape[0], w_uv.shape[1]))
    for h in np.unique(heads):
        m = heads == h
        out[m] = o_lat[m] @ w_uv[h].T
    return out, lse, q64


def query_rounding_bound(w, q64: np.ndarray, sel: Sequence[int]) -> np.ndarray:
    """How far lse may move when every element of the absorbed query q~ is
    rounded to bf16 (relative change at most 2^-9 per element): each score
    scale * q~ . K_t moves by at most scale * 2^-9 * sum_i |q~_i K_t,i|, and lse
    (a log-sum-exp) moves by at most its largest score change.  Per flat row
    index in ``sel`` over the row's visible keys (0 for a row without keys)."""
    bound = []
    cache = {}
    for idx in sel:
        b, rem = divmod(int(idx), w.s_q * w.h_q)
        s, h = divmod(rem, w.h_q)
        L = int(w.cache_seqlens[b])
        n = L if not w.causal else max(0, L - w.s_q + s + 1)
        if n == 0:
            bound.append(0.0)
            continue
        if b not in cache:
            rows = [w.kcache[w.block_table[b, t // _PAGE], t % _PAGE, 0] for t in range(L)]
            cache[b] = np.abs(_f64(np.array(rows, dtype=np.uint16).reshape(L, -1)))
        bound.append(w.scale * 2.0 ** -9 * float(np.max(cache[b][:n] @ np.abs(q64[b, s, h]))))
    return np.array(bound)
