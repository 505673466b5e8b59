"""Seeded synthetic inputs for paged MLA decode.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, so both the CPU oracle and the HIP path can take their
inputs from it without sharing any of the method.

Shapes follow the FlashMLA API as the "OpenSourceWeek Day 1 — Demystifying
DeepSeek's FlashMLA" page (deepseekonline.chat) shows it in §V.2: absorbed
queries ``q[b, s_q, h_q, d_qk]``, a paged cache ``k_cache[num_pages, 64, h_kv,
d_qk]`` with 64-token pages (§II.1, §II.2), ``block_table[b, max_blocks]`` and
``cache_seqlens[b]``.  The latent width 576 = 512 latent + 64 rope and
dv = 512 come from the problem statement of this path; the page size 64 is the
one the Day-1 page and the "Flash MLA: an efficient MLA decoding kernel library
for variable-length sequences" page (developer.baidu.com) agree on.

Draw order (fixed, numpy ``Generator(PCG64(seed))``):
  1. ``cache_seqlens``  (integers, inclusive ends; the long-context config draws
     a fair coin per sequence between two lengths),
  2. a permutation of all physical pages, dealt to sequences in order,
  3. ``q`` ~ N(0, 1) float32, rounded to bf16 (round-to-nearest-even),
  4. ``k_cache`` ~ N(0, 1) float32 in 1024-page chunks, rounded to bf16,
  5. (long-context config only) an independent Bernoulli(0.01) per physical
     slot; a selected slot's whole 576-wide row is scaled by 8 (exact in bf16).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

PAGE = 64
D_QK = 576
DV = 512
SCALE = 1.0 / math.sqrt(192.0)

# The five workloads.  ``lens`` is ("uniform", lo, hi) inclusive, ("const", L) or
# ("choice", a, b) (fair coin per sequence).
CONFIGS = {
    0: dict(name="tiny", batch=2, s_q=1, h_q=16, h_kv=1, lens=("uniform", 1, 256),
            causal=False, outliers=False),
    1: dict(name="memory_bound_varlen", batch=64, s_q=1, h_q=16, h_kv=1,
            lens=("uniform", 1, 2560), causal=False, outliers=False),
    2: dict(name="compute_bound_full_heads", batch=128, s_q=1, h_q=128, h_kv=1,
            lens=("const", 4096), causal=False, outliers=False),
    3: dict(name="spec_decode_causal", batch=132, s_q=2, h_q=128, h_kv=1,
            lens=("uniform", 2048, 16384), causal=True, outliers=False),
    4: dict(name="long_context", batch=8, s_q=1, h_q=64, h_kv=1,
            lens=("choice", 32768, 65536), causal=False, outliers=True),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs here are finite normal draws, so no NaN handling is needed."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    batch: int
    s_q: int
    h_q: int
    h_kv: int
    causal: bool
    scale: float
    cache_seqlens: np.ndarray  # int32 [b]
    block_table: np.ndarray  # int32 [b, max_blocks]; -1 for unused entries
    q: np.ndarray  # uint16 bf16 bits [b, s_q, h_q, 576]
    kcache: np.ndarray  # uint16 bf16 bits [num_pages, 64, h_kv, 576]
    seed: int
    name: str = "custom"
    d_qk: int = D_QK
    dv: int = DV
    page: int = PAGE

    @property
    def rows(self) -> int:
        return self.s_q * self.h_q // self.h_kv

    @property
    def num_pages(self) -> int:
        return int(self.kcache.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def n_blocks(self) -> np.ndarray:
        return (self.cache_seqlens.astype(np.int64) + PAGE - 1) // PAGE


def _draw_lens(rng: np.random.Generator, spec, batch: int) -> np.ndarray:
    kind = spec[0]
    if kind == "uniform":
        return rng.integers(spec[1], spec[2], size=batch, endpoint=True).astype(np.int32)
    if kind == "const":
        return np.full(batch, spec[1], dtype=np.int32)
    if kind == "choice":
        coin = rng.integers(0, 2, size=batch)
        return np.where(coin == 0, spec[1], spec[2]).astype(np.int32)
    raise ValueError(f"unknown length spec {spec}")


def make_workload(seqlens: Sequence[int] | np.ndarray, *, s_q: int = 1, h_q: int = 16,
                  h_kv: int = 1, causal: bool = False, seed: int = 0,
                  outliers: bool = False, rng: Optional[np.random.Generator] = None,
                  extra_pages: int = 0, poison_tail: bool = False,
                  scale: float = SCALE, name: str = "custom") -> Workload:
    """Build a workload from explicit sequence lengths (steps 2-5 of the draw order).

    ``extra_pages`` appends physical pages that no sequence references (their
    contents must not matter).  ``poison_tail`` writes NaN into every slot at or
    beyond a sequence's length in its last page, and into all extra pages; a
    correct implementation never lets those bits reach its result."""
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.asarray(seqlens, dtype=np.int32)
    b = int(lens.shape[0])
    if b <= 0:
        raise ValueError("batch must be positive")
    if h_q % h_kv != 0:
        raise ValueError("h_q must be a multiple of h_kv")
    nblk = (lens.astype(np.int64) + PAGE - 1) // PAGE
    n_used = int(nblk.sum())
    n_pages = n_used + int(extra_pages)
    perm = rng.permutation(n_pages).astype(np.int32) if n_pages > 0 else np.zeros(0, np.int32)
    max_blocks = max(1, int(nblk.max()) if b else 1)
    block_table = np.full((b, max_blocks), -1, dtype=np.int32)
    off = 0
    for i in range(b):
        block_table[i, : nblk[i]] = perm[off: off + nblk[i]]
        off += int(nblk[i])
    q = bf16_bits(rng.standard_normal((b, s_q, h_q, D_QK), dtype=np.float32))
    pages_alloc = max(n_pages, 1)
    kcache = np.empty((pages_alloc, PAGE, h_kv, D_QK), dtype=np.uint16)
    chunk = 1024
    for p0 in range(0, n_pages, chunk):
        p1 = min(n_pages, p0 + chunk)
        kcache[p0:p1] = bf16_bits(rng.standard_normal((p1 - p0, PAGE, h_kv, D_QK), dtype=np.float32))
    if n_pages == 0:
        kcache[:] = 0
    if outliers and n_pages > 0:
        sel = rng.random(n_pages * PAGE) < 0.01
        idx = np.nonzero(sel)[0]
        flat = kcache.reshape(n_pages * PAGE, h_kv * D_QK)
        vals = bf16_to_f32(flat[idx]) * np.float32(8.0)
        flat[idx] = bf16_bits(vals)
    if poison_tail:
        nan = np.uint16(0x7FC0)
        for i in range(b):
            L = int(lens[i])
            if L % PAGE and nblk[i] > 0:
                kcache[block_table[i, nblk[i] - 1], L % PAGE:] = nan
        if extra_pages:
            used = set(block_table[block_table >= 0].tolist())
            for p in range(n_pages):
                if p not in used:
                    kcache[p] = nan
    return Workload(batch=b, s_q=s_q, h_q=h_q, h_kv=h_kv, causal=bool(causal), scale=scale,
                    cache_seqlens=lens, block_table=block_table, q=q, kcache=kcache,
                    seed=seed, name=name)


def config_workload(index: int, seed: Optional[int] = None) -> Workload:
    """One of the five workloads, seeded by its index unless ``seed`` is given."""
    cfg = CONFIGS[index]
    seed = index if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = _draw_lens(rng, cfg["lens"], cfg["batch"])
    return make_workload(lens, s_q=cfg["s_q"], h_q=cfg["h_q"], h_kv=cfg["h_kv"],
                         causal=cfg["causal"], seed=seed, outliers=cfg["outliers"], rng=rng,
                         name=cfg["name"])


def make_append_case(lens: Sequence[int], s_new: int, *, h_q: int = 16, h_kv: int = 1, seed: int = 0,
                     extra_pages: int = 0):
    """A cache whose block table already covers each sequence's next s_new
    tokens, plus the rows to append: returns (w, lens_before, new_kv).

    ``w`` is a causal workload with s_q = s_new and lengths lens + s_new (its
    cache holds random rows at the new positions, which the append overwrites);
    ``new_kv`` is bf16 bits [b, s_new, h_kv, 576], drawn after everything in w
    from PCG64(seed + 7919)."""
    lens_before = np.asarray(lens, dtype=np.int32)
    w = make_workload(lens_before + s_new, s_q=max(s_new, 1), h_q=h_q, h_kv=h_kv, causal=True, seed=seed,
                      extra_pages=extra_pages)
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    new_kv = bf16_bits(rng.standard_normal((len(lens_before), s_new, h_kv, D_QK), dtype=np.float32))
    return w, lens_before, new_kv


FP8_ROW_BYTES = 656


def make_fp8_cache(w: Workload, seed: int, scale_exp: int = -2) -> np.ndarray:
    """A random cache in the 656-byte FP8 row format with w's shape: uint8
    [pages, 64, h_kv, 656].  Latent bytes are e4m3 codes with random sign,
    exponent field 4..10 and mantissa (values 2^-3 .. 3.75 before scaling), one
    in 16 of them zero; the four scales of a row are 2^(scale_exp + u), u in
    {-1, 0, 1}; the rope dims are w's rope bits.  Drawn from PCG64(seed + 104729)
    in that order; nothing here quantises."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    shape = w.kcache.shape[:-1]
    n = int(np.prod(shape))
    sign = rng.integers(0, 2, size=(n, 512), dtype=np.uint8) << 7
    ex = rng.integers(4, 11, size=(n, 512), dtype=np.uint8)
    man = rng.integers(0, 8, size=(n, 512), dtype=np.uint8)
    codes = sign | (ex << 3) | man
    codes[rng.random((n, 512)) < 1.0 / 16] = 0
    scales = np.ldexp(np.float32(1.0), scale_exp + rng.integers(-1, 2, size=(n, 4))).astype(np.float32)
    out = np.empty((n, FP8_ROW_BYTES), dtype=np.uint8)
    out[:, :512] = codes
    out[:, 512:528] = scales.view(np.uint8).reshape(n, 16)
    out[:, 528:] = np.ascontiguousarray(w.kcache.reshape(n, D_QK)[:, 512:]).view(np.uint8).reshape(n, 128)
    return out.reshape(shape + (FP8_ROW_BYTES,))


def make_sparse_indices(w: Workload, topk: int, seed: int, invalid: float = 0.0, shuffle: bool = False,
                        empty_rows: Sequence[int] = ()):
    """CSR selections for a token-sparse decode of workload w: (indices int32,
    indptr int32 [b*s_q + 1]).

    Row v = b*s_q + s lists min(topk, L_b) distinct positions drawn uniformly
    from [0, L_b), ascending; with ``invalid`` > 0 about that fraction of extra
    entries that address no cached token (-1, L_b, L_b + 63, past the table) is
    added and the row is shuffled; ``shuffle`` shuffles every row; rows in
    ``empty_rows`` list nothing.  Drawn from PCG64(seed + 7727)."""
    rng = np.random.Generator(np.random.PCG64(seed + 7727))
    rows, ptr = [], [0]
    for v in range(w.batch * w.s_q):
        L = int(w.cache_seqlens[v // w.s_q])
        if v in empty_rows or L <= 0:
            sel = np.zeros(0, dtype=np.int64)
        else:
            sel = np.sort(rng.choice(L, size=min(topk, L), replace=False))
        if invalid > 0:
            n_bad = int(rng.binomial(max(len(sel), 1), invalid))
            bad = rng.choice(np.array([-1, L, L + 63, w.max_blocks * PAGE + 5]), size=n_bad)
            sel = rng.permutation(np.concatenate([sel, bad]))
        elif shuffle:
            sel = rng.permutation(sel)
        rows.append(sel.astype(np.int32))
        ptr.append(ptr[-1] + len(sel))
    return np.concatenate(rows).astype(np.int32), np.array(ptr, dtype=np.int32)


def permute_pages(w: Workload, seed: int) -> Workload:
    """Same logical cache with physical pages relabelled by a random permutation.

    Page p moves to slot perm[p] and block_table entries are rewritten to match;
    attention over the logical sequence is unchanged by construction."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = w.num_pages
    perm = rng.permutation(n).astype(np.int32)
    kc = np.empty_like(w.kcache)
    kc[perm] = w.kcache
    bt = w.block_table.copy()
    m = bt >= 0
    bt[m] = perm[bt[m]]
    return dataclasses.replace(w, kcache=kc, block_table=bt)


D_NOPE = 128
D_ROPE = 64
D_VHEAD = 128


@dataclasses.dataclass
class LayerInputs:
    """Per-head query parts and up-projection weights of one MLA decode layer
    (bf16 bits): the absorbed query of the decode is built from these."""
    q_nope: np.ndarray  # [b, s_q, h_q, 128]
    q_rope: np.ndarray  # [b, s_q, h_q, 64]
    w_uk: np.ndarray    # [h_q, 128, 512]: the nope key of head h is w_uk[h] . c
    w_uv: np.ndarray    # [h_q, 128, 512]: the value of head h is w_uv[h] . c


def make_layer_inputs(batch: int, s_q: int, h_q: int, seed: int) -> LayerInputs:
    """Seeded draws, in this order: q_nope ~ N(0,1), q_rope ~ N(0,1),
    w_uk ~ N(0, 1/512), w_uv ~ N(0, 1/512) (fan-in of the 512-wide latent), each
    rounded to bf16 (nearest even)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q_nope = bf16_bits(rng.standard_normal((batch, s_q, h_q, D_NOPE), dtype=np.float32))
    q_rope = bf16_bits(rng.standard_normal((batch, s_q, h_q, D_ROPE), dtype=np.float32))
    s = np.float32(1.0 / math.sqrt(DV))
    w_uk = bf16_bits(rng.standard_normal((h_q, D_NOPE, DV), dtype=np.float32) * s)
    w_uv = bf16_bits(rng.standard_normal((h_q, D_VHEAD, DV), dtype=np.float32) * s)
    return LayerInputs(q_nope=q_nope, q_rope=q_rope, w_uk=w_uk, w_uv=w_uv)
