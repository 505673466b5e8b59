"""Paged MLA decode for AMD MI355X (gfx950).

Thin Python binding over libmla.so (see include/mla.h).  Every step of the
decode runs in the library's HIP kernels; this module only marshals torch
tensors (device memory and the current stream) into the C ABI.  Importing it
fails loudly when the library has not been built.

The paged cache (same names as the C ABI):
    mla_kv_append(new_kv, cache_seqlens, block_table, kcache) -> new_seqlens
    Pager(num_pages, max_seqs, max_blocks): host page allocator (reserve,
        release, block_table)
Token-sparse decode (same names as the C ABI):
    mla_sparse_prepare(indices, indptr, s_q, block_table, cache_seqlens, num_pages, h_kv)
        -> (row offsets, counts)
    mla_sparse_decode(q, kcache, offsets, indptr, counts, dv, tile_metadata, num_splits, scale)
    flash_mla_sparse_with_kvcache(q, k_cache, block_table, cache_seqlens, indices, indptr)
        -> (out, lse): prepare + schedule + decode
The absorption GEMMs around the decode (same names as the C ABI):
    mla_absorb_q(q_nope, q_rope, w_uk) -> q_abs      (the decode's query)
    mla_unabsorb_out(o_lat, w_uv) -> out             (per-head values)
Low-level calls, same names as the C ABI:
    mla_plan, mla_tile_rows, mla_get_metadata, mla_decode_paged,
    mla_decode_splitkv + mla_combine_splits (the two stages of mla_decode_paged)
The two-call FlashMLA-style API ("OpenSourceWeek Day 1 -- Demystifying
DeepSeek's FlashMLA", deepseekonline.chat, §V.2):
    get_mla_metadata(cache_seqlens, s_q * h_q // h_kv, h_kv) -> (tile_metadata, num_splits)
    flash_mla_with_kvcache(q, k_cache, block_table, cache_seqlens, dv,
                           tile_metadata, num_splits, causal=False,
                           softmax_scale=None) -> (out, lse)
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "LIB_PATH", "MlaError", "mla_plan", "mla_tile_rows", "mla_get_metadata", "mla_decode_paged",
    "mla_decode_splitkv", "mla_combine_splits", "get_mla_metadata", "flash_mla_with_kvcache",
    "mla_absorb_q", "mla_unabsorb_out", "mla_kv_append", "Pager", "mla_decode_paged_fp8",
    "mla_decode_splitkv_fp8", "FP8_ROW_BYTES", "mla_sparse_prepare", "mla_sparse_decode",
    "flash_mla_sparse_with_kvcache", "mla_decode_paged_noalloc", "NOALLOC_SCRATCH_BYTES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")
# the same library with every page transfer synchronous (a race reference for
# tests; built beside libmla.so, never used unless selected with library())
SYNC_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_sync.so")
PAGE_BLOCK_SIZE = 64
FP8_ROW_BYTES = 656
D_QK = 576
DV = 512
NOALLOC_SCRATCH_BYTES = 256 << 20  # MLA_NOALLOC_SCRATCH_BYTES of include/mla.h


class MlaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libmla error {code}: {msg}")
        self.code = code


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -m paged_mla_decode_02_amd.build)")
    lib = ctypes.CDLL(path)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.mla_plan.argtypes = [I, I, I, I, I, ctypes.POINTER(I), ctypes.POINTER(SZ)]
    lib.mla_plan.restype = I
    lib.mla_tile_rows.argtypes = [I]
    lib.mla_tile_rows.restype = I
    lib.mla_get_metadata.argtypes = [P, I, I, I, I, P, P, P]
    lib.mla_get_metadata.restype = I
    for name in ("mla_decode_paged", "mla_decode_splitkv", "mla_combine_splits", "mla_decode_paged_fp8",
                 "mla_decode_splitkv_fp8"):
        fn = getattr(lib, name)
        fn.argtypes = [P, P, ctypes.c_int64, P, I, P, I, I, I, I, I, I, I, P, I, P, I,
                       ctypes.c_float, P, P, P, SZ, P]
        fn.restype = I
    lib.mla_decode_paged_noalloc.argtypes = [P, P, ctypes.c_int64, P, I, P, I, I, I, I, I, I, I, P, I, P, I,
                                             ctypes.c_float, P, P, P]
    lib.mla_decode_paged_noalloc.restype = I
    lib.mla_absorb_q.argtypes = [P, P, P, I, I, P, P]
    lib.mla_absorb_q.restype = I
    lib.mla_unabsorb_out.argtypes = [P, P, I, I, P, P]
    lib.mla_unabsorb_out.restype = I
    for name in ("mla_kv_append", "mla_kv_append_fp8"):
        getattr(lib, name).argtypes = [P, I, I, I, P, P, I, P, ctypes.c_int64, P, P]
        getattr(lib, name).restype = I
    lib.mla_sparse_prepare.argtypes = [P, P, I, I, P, I, P, ctypes.c_int64, I, P, P, P]
    lib.mla_sparse_prepare.restype = I
    lib.mla_sparse_decode.argtypes = [P, P, ctypes.c_int64, P, P, P, I, I, I, I, I, I, I, P, I, P, ctypes.c_float,
                                      P, P, P, SZ, P]
    lib.mla_sparse_decode.restype = I
    lib.mla_pager_bytes.argtypes = [I, I, I]
    lib.mla_pager_bytes.restype = SZ
    lib.mla_pager_init.argtypes = [P, SZ, I, I, I]
    lib.mla_pager_init.restype = I
    lib.mla_pager_reserve.argtypes = [P, I, ctypes.c_int64]
    lib.mla_pager_reserve.restype = I
    lib.mla_pager_release.argtypes = [P, I]
    lib.mla_pager_release.restype = I
    for name in ("mla_pager_free_pages",):
        getattr(lib, name).argtypes = [P]
        getattr(lib, name).restype = I
    for name in ("mla_pager_seq_pages", "mla_pager_page_owner"):
        getattr(lib, name).argtypes = [P, I]
        getattr(lib, name).restype = I
    lib.mla_pager_block_table.argtypes = [P]
    lib.mla_pager_block_table.restype = ctypes.POINTER(ctypes.c_int32)
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()
_libs = {LIB_PATH: _lib}


@contextlib.contextmanager
def library(path: str):
    """Calls inside the block go to another build of the library at ``path``
    (e.g. SYNC_LIB_PATH, the synchronous-transfer reference build)."""
    global _lib
    if path not in _libs:
        _libs[path] = _load(path)
    prev = _lib
    _lib = _libs[path]
    try:
        yield
    finally:
        _lib = prev


def _check(rc: int) -> None:
    if rc != 0:
        raise MlaError(rc, _lib.mla_last_error().decode(errors="replace"))


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _require(t: torch.Tensor, name: str, dtype: torch.dtype, on_device: bool = True) -> None:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if on_device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _shape(t: torch.Tensor, name: str, shape) -> None:
    """The kernels index these tensors by batch, row and part: any other shape
    would send them outside the buffer, so it is refused on the host."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_device(dev: torch.device, **tensors) -> None:
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, q on {dev}")


def mla_tile_rows(rows_per_kv: int) -> int:
    r = _lib.mla_tile_rows(int(rows_per_kv))
    _check(min(r, 0))
    return r


def mla_plan(batch: int, rows_per_kv: int, h_kv: int, dv: int = DV, num_cus: int = 0) -> Tuple[int, int]:
    """(num_parts, workspace_bytes) for a decode step."""
    parts = ctypes.c_int(0)
    ws = ctypes.c_size_t(0)
    _check(_lib.mla_plan(int(batch), int(rows_per_kv), int(h_kv), int(dv), int(num_cus),
                         ctypes.byref(parts), ctypes.byref(ws)))
    return parts.value, ws.value


def mla_get_metadata(cache_seqlens: torch.Tensor, rows_per_kv: int, h_kv: int,
                     num_parts: Optional[int] = None, num_cus: int = 0, out=None):
    """Split-KV schedule: (tile_metadata int32 [P, 8], num_splits int32 [b + 1]).

    ``out`` may pass preallocated (tile_metadata, num_splits) tensors."""
    _require(cache_seqlens, "cache_seqlens", torch.int32)
    b = cache_seqlens.numel()
    dev = cache_seqlens.device
    if out is not None:
        md, ns = out
        _require(md, "tile_metadata", torch.int32)
        _require(ns, "num_splits", torch.int32)
        if md.dim() != 2 or md.shape[1] != 8 or ns.numel() != b + 1:
            raise ValueError("tile_metadata must be [P, 8] and num_splits [b + 1]")
        if num_parts is not None and num_parts != md.shape[0]:
            raise ValueError("num_parts does not match tile_metadata")
        num_parts = md.shape[0]
    else:
        if num_parts is None:
            num_parts, _ = mla_plan(b, rows_per_kv, h_kv, DV, num_cus)
        md = torch.empty((num_parts, 8), dtype=torch.int32, device=dev)
        ns = torch.empty((b + 1,), dtype=torch.int32, device=dev)
    _check(_lib.mla_get_metadata(cache_seqlens.data_ptr(), b, int(rows_per_kv), int(h_kv),
                                 int(num_parts), md.data_ptr(), ns.data_ptr(), _stream(dev)))
    return md, ns


def _decode_call(fn, q, kcache, block_table, cache_seqlens, dv, tile_metadata, num_splits, causal,
                 softmax_scale, out, lse, workspace, fp8=False):
    # dtypes and shapes first (host metadata only), then devices
    _require(q, "q", torch.bfloat16, on_device=False)
    _require(kcache, "kcache", torch.uint8 if fp8 else torch.bfloat16, on_device=False)
    _require(block_table, "block_table", torch.int32, on_device=False)
    _require(cache_seqlens, "cache_seqlens", torch.int32, on_device=False)
    _require(tile_metadata, "tile_metadata", torch.int32, on_device=False)
    _require(num_splits, "num_splits", torch.int32, on_device=False)
    if q.dim() != 4 or kcache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("q must be [b, s_q, h_q, d], kcache [pages, 64, h_kv, d], block_table [b, n]")
    b, s_q, h_q, d_qk = q.shape
    num_pages, page, h_kv, d_k = kcache.shape
    if d_k != (FP8_ROW_BYTES if fp8 else d_qk):
        raise ValueError("kcache rows must be the head dim of q (bf16) or FP8_ROW_BYTES bytes (fp8)")
    if h_kv <= 0 or h_q % h_kv:
        raise ValueError("h_q must be a multiple of h_kv")
    if block_table.shape[0] != b:
        raise ValueError(f"block_table must have one row per sequence ({b}), got {block_table.shape[0]}")
    _shape(cache_seqlens, "cache_seqlens", (b,))
    _shape(num_splits, "num_splits", (b + 1,))
    if tile_metadata.dim() != 2 or tile_metadata.shape[1] != 8 or tile_metadata.shape[0] < 1:
        raise ValueError(f"tile_metadata must be [num_parts, 8], got {tuple(tile_metadata.shape)}")
    num_parts = tile_metadata.shape[0]
    rows = s_q * h_q // h_kv
    dev = q.device
    if out is not None:
        _require(out, "out", torch.bfloat16, on_device=False)
        _shape(out, "out", (b, s_q, h_q, dv))
    if lse is not None:
        _require(lse, "lse", torch.float32, on_device=False)
        _shape(lse, "lse", (b, s_q, h_q))
    need = (b + num_parts) * h_kv * rows * (dv + 1) * 4
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor")
        if workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace must hold {need} bytes, got {workspace.numel() * workspace.element_size()}")
    _same_device(dev, q=q, kcache=kcache, block_table=block_table, cache_seqlens=cache_seqlens,
                 tile_metadata=tile_metadata, num_splits=num_splits)
    if out is None:
        out = torch.empty((b, s_q, h_q, dv), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((b, s_q, h_q), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _same_device(dev, out=out, lse=lse, workspace=workspace)
    _check(fn(q.data_ptr(), kcache.data_ptr(), num_pages, block_table.data_ptr(), block_table.shape[1],
              cache_seqlens.data_ptr(), b, s_q, h_q, h_kv, d_qk, dv, page, tile_metadata.data_ptr(),
              num_parts, num_splits.data_ptr(), int(bool(causal)), float(softmax_scale),
              out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
              workspace.numel() * workspace.element_size(), _stream(dev)))
    return out, lse


def mla_decode_paged(q: torch.Tensor, kcache: torch.Tensor, block_table: torch.Tensor,
                     cache_seqlens: torch.Tensor, dv: int, tile_metadata: torch.Tensor,
                     num_splits: torch.Tensor, causal: bool, softmax_scale: float,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None):
    """Paged decode; returns (out bf16 [b, s_q, h_q, dv], lse fp32 [b, s_q, h_q])."""
    return _decode_call(_lib.mla_decode_paged, q, kcache, block_table, cache_seqlens, dv, tile_metadata,
                        num_splits, causal, softmax_scale, out, lse, workspace)


def mla_decode_paged_noalloc(q: torch.Tensor, kcache: torch.Tensor, block_table: torch.Tensor,
                             cache_seqlens: torch.Tensor, dv: int, tile_metadata: torch.Tensor,
                             num_splits: torch.Tensor, causal: bool, softmax_scale: float,
                             out: torch.Tensor, lse: torch.Tensor):
    """mla_decode_paged without a workspace and without allocating: the split
    partials use the library's fixed per-GPU scratch array (at most
    NOALLOC_SCRATCH_BYTES).  ``out`` and ``lse`` are the caller's.  Calls that
    overlap on one GPU race on that array."""
    for t, n, dt in ((q, "q", torch.bfloat16), (kcache, "kcache", torch.bfloat16),
                     (block_table, "block_table", torch.int32), (cache_seqlens, "cache_seqlens", torch.int32),
                     (tile_metadata, "tile_metadata", torch.int32), (num_splits, "num_splits", torch.int32),
                     (out, "out", torch.bfloat16), (lse, "lse", torch.float32)):
        _require(t, n, dt, on_device=False)
    if q.dim() != 4 or kcache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("q must be [b, s_q, h_q, d], kcache [pages, 64, h_kv, d], block_table [b, n]")
    b, s_q, h_q, d_qk = q.shape
    num_pages, page, h_kv, d_k = kcache.shape
    if d_k != d_qk or h_kv <= 0 or h_q % h_kv:
        raise ValueError("q / kcache shapes do not match")
    if block_table.shape[0] != b:
        raise ValueError(f"block_table must have one row per sequence ({b}), got {block_table.shape[0]}")
    _shape(cache_seqlens, "cache_seqlens", (b,))
    _shape(num_splits, "num_splits", (b + 1,))
    if tile_metadata.dim() != 2 or tile_metadata.shape[1] != 8 or tile_metadata.shape[0] < 1:
        raise ValueError(f"tile_metadata must be [num_parts, 8], got {tuple(tile_metadata.shape)}")
    _shape(out, "out", (b, s_q, h_q, dv))
    _shape(lse, "lse", (b, s_q, h_q))
    dev = q.device
    _same_device(dev, q=q, kcache=kcache, block_table=block_table, cache_seqlens=cache_seqlens,
                 tile_metadata=tile_metadata, num_splits=num_splits, out=out, lse=lse)
    _check(_lib.mla_decode_paged_noalloc(
        q.data_ptr(), kcache.data_ptr(), num_pages, block_table.data_ptr(), block_table.shape[1],
        cache_seqlens.data_ptr(), b, s_q, h_q, h_kv, d_qk, dv, page, tile_metadata.data_ptr(),
        tile_metadata.shape[0], num_splits.data_ptr(), int(bool(causal)), float(softmax_scale),
        out.data_ptr(), lse.data_ptr(), _stream(dev)))
    return out, lse


def mla_decode_splitkv(q, kcache, block_table, cache_seqlens, dv, tile_metadata, num_splits, causal,
                       softmax_scale, out, lse, workspace):
    """Decode kernel only (split sequences leave partials in ``workspace``)."""
    return _decode_call(_lib.mla_decode_splitkv, q, kcache, block_table, cache_seqlens, dv, tile_metadata,
                        num_splits, causal, softmax_scale, out, lse, workspace)


def mla_combine_splits(q, kcache, block_table, cache_seqlens, dv, tile_metadata, num_splits, causal,
                       softmax_scale, out, lse, workspace):
    """LSE combine of the partials mla_decode_splitkv left in ``workspace``."""
    return _decode_call(_lib.mla_combine_splits, q, kcache, block_table, cache_seqlens, dv, tile_metadata,
                        num_splits, causal, softmax_scale, out, lse, workspace, fp8=kcache.dtype == torch.uint8)


def mla_decode_paged_fp8(q: torch.Tensor, kcache_fp8: torch.Tensor, block_table: torch.Tensor,
                         cache_seqlens: torch.Tensor, dv: int, tile_metadata: torch.Tensor,
                         num_splits: torch.Tensor, causal: bool, softmax_scale: float,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None):
    """Paged decode over the FP8 cache (uint8 [pages, 64, h_kv, 656]), any rows per KV head."""
    return _decode_call(_lib.mla_decode_paged_fp8, q, kcache_fp8, block_table, cache_seqlens, dv, tile_metadata,
                        num_splits, causal, softmax_scale, out, lse, workspace, fp8=True)


def mla_decode_splitkv_fp8(q, kcache_fp8, block_table, cache_seqlens, dv, tile_metadata, num_splits, causal,
                           softmax_scale, out, lse, workspace):
    """Decode kernel only, FP8 cache (finish with mla_combine_splits)."""
    return _decode_call(_lib.mla_decode_splitkv_fp8, q, kcache_fp8, block_table, cache_seqlens, dv,
                        tile_metadata, num_splits, causal, softmax_scale, out, lse, workspace, fp8=True)


def get_mla_metadata(cache_seqlens: torch.Tensor, num_heads_per_head_k: int, num_heads_k: int):
    """FlashMLA-style metadata call: (tile_metadata, num_splits)."""
    return mla_get_metadata(cache_seqlens, num_heads_per_head_k, num_heads_k)


def flash_mla_with_kvcache(q: torch.Tensor, k_cache: torch.Tensor, block_table: torch.Tensor,
                           cache_seqlens: torch.Tensor, head_dim_v: int, tile_metadata: torch.Tensor,
                           num_splits: torch.Tensor, softmax_scale: Optional[float] = None,
                           causal: bool = False):
    """FlashMLA-style decode: (out, lse).  softmax_scale defaults to d_qk ** -0.5.
    A uint8 k_cache is the FP8 format (mla_decode_paged_fp8)."""
    if softmax_scale is None:
        softmax_scale = q.shape[-1] ** -0.5
    if k_cache.dtype == torch.uint8:
        return mla_decode_paged_fp8(q, k_cache, block_table, cache_seqlens, head_dim_v, tile_metadata,
                                    num_splits, causal, softmax_scale)
    return mla_decode_paged(q, k_cache, block_table, cache_seqlens, head_dim_v, tile_metadata,
                            num_splits, causal, softmax_scale)


D_NOPE = 128
D_ROPE = 64
D_VHEAD = 128


def _tokens_view(t: torch.Tensor, last: int, name: str):
    """[..., h, last] -> (tokens, h) of a contiguous bf16 device tensor."""
    _require(t, name, torch.bfloat16)
    if t.dim() < 2 or t.shape[-1] != last:
        raise ValueError(f"{name} must be [..., h, {last}]")
    h = t.shape[-2]
    return t.numel() // (h * last), h


def mla_absorb_q(q_nope: torch.Tensor, q_rope: torch.Tensor, w_uk: torch.Tensor,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q_abs[..., h, 0:512] = W_UK[h]^T q_nope[..., h, :], q_abs[..., h, 512:] = q_rope.

    q_nope [..., h_q, 128], q_rope [..., h_q, 64], w_uk [h_q, 128, 512] (bf16)."""
    tokens, h_q = _tokens_view(q_nope, D_NOPE, "q_nope")
    if _tokens_view(q_rope, D_ROPE, "q_rope") != (tokens, h_q) or q_rope.shape[:-1] != q_nope.shape[:-1]:
        raise ValueError("q_rope must match q_nope's leading shape")
    _require(w_uk, "w_uk", torch.bfloat16)
    if tuple(w_uk.shape) != (h_q, D_NOPE, DV):
        raise ValueError(f"w_uk must be [{h_q}, {D_NOPE}, {DV}]")
    if out is None:
        out = torch.empty(tuple(q_nope.shape[:-1]) + (D_QK,), dtype=torch.bfloat16, device=q_nope.device)
    _require(out, "out", torch.bfloat16)
    if out.shape[:-1] != q_nope.shape[:-1] or out.shape[-1] != D_QK:
        raise ValueError("out must be [..., h_q, 576]")
    _check(_lib.mla_absorb_q(q_nope.data_ptr(), q_rope.data_ptr(), w_uk.data_ptr(), tokens, h_q,
                             out.data_ptr(), _stream(q_nope.device)))
    return out


def mla_unabsorb_out(o_lat: torch.Tensor, w_uv: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[..., h, v] = sum_c W_UV[h, v, c] o_lat[..., h, c].

    o_lat [..., h_q, 512] (the decode's output), w_uv [h_q, 128, 512] (bf16)."""
    tokens, h_q = _tokens_view(o_lat, DV, "o_lat")
    _require(w_uv, "w_uv", torch.bfloat16)
    if tuple(w_uv.shape) != (h_q, D_VHEAD, DV):
        raise ValueError(f"w_uv must be [{h_q}, {D_VHEAD}, {DV}]")
    if out is None:
        out = torch.empty(tuple(o_lat.shape[:-1]) + (D_VHEAD,), dtype=torch.bfloat16, device=o_lat.device)
    _require(out, "out", torch.bfloat16)
    if out.shape[:-1] != o_lat.shape[:-1] or out.shape[-1] != D_VHEAD:
        raise ValueError("out must be [..., h_q, 128]")
    _check(_lib.mla_unabsorb_out(o_lat.data_ptr(), w_uv.data_ptr(), tokens, h_q, out.data_ptr(),
                                 _stream(o_lat.device)))
    return out


def mla_kv_append(new_kv: torch.Tensor, cache_seqlens: torch.Tensor, block_table: torch.Tensor,
                  kcache: torch.Tensor, new_seqlens: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Write new_kv [b, s_new, h_kv, 576] at positions cache_seqlens[b] + j of
    each sequence's pages (in place in kcache); returns cache_seqlens + s_new.
    A uint8 kcache [pages, 64, h_kv, 656] is the FP8 format: rows are quantised."""
    _require(new_kv, "new_kv", torch.bfloat16)
    fp8 = kcache.dtype == torch.uint8
    _require(kcache, "kcache", torch.uint8 if fp8 else torch.bfloat16)
    _require(cache_seqlens, "cache_seqlens", torch.int32)
    _require(block_table, "block_table", torch.int32)
    if new_kv.dim() != 4 or new_kv.shape[-1] != D_QK:
        raise ValueError("new_kv must be [batch, s_new, h_kv, 576]")
    b, s_new, h_kv, _ = new_kv.shape
    row = FP8_ROW_BYTES if fp8 else D_QK
    if kcache.dim() != 4 or kcache.shape[1] != PAGE_BLOCK_SIZE or kcache.shape[2] != h_kv or kcache.shape[3] != row:
        raise ValueError(f"kcache must be [num_pages, 64, {h_kv}, {row}]")
    if cache_seqlens.shape != (b,) or block_table.dim() != 2 or block_table.shape[0] != b:
        raise ValueError("cache_seqlens must be [batch] and block_table [batch, max_blocks]")
    if new_seqlens is None:
        new_seqlens = torch.empty_like(cache_seqlens)
    _require(new_seqlens, "new_seqlens", torch.int32)
    fn = _lib.mla_kv_append_fp8 if fp8 else _lib.mla_kv_append
    _check(fn(new_kv.data_ptr(), b, s_new, h_kv, cache_seqlens.data_ptr(), block_table.data_ptr(),
              block_table.shape[1], kcache.data_ptr(), kcache.shape[0], new_seqlens.data_ptr(),
              _stream(kcache.device)))
    return new_seqlens


class Pager:
    """Host page allocator of the paged cache (mla_pager_* of the C ABI).

    Its state, including the block table [max_seqs, max_blocks] int32 (-1 = no
    page), lives in a host buffer owned by this object."""

    def __init__(self, num_pages: int, max_seqs: int, max_blocks: int):
        n = _lib.mla_pager_bytes(num_pages, max_seqs, max_blocks)
        if n == 0:
            raise ValueError("num_pages, max_seqs and max_blocks must be positive")
        self._buf = (ctypes.c_int32 * ((n + 3) // 4))()
        self._ptr = ctypes.addressof(self._buf)
        _check(_lib.mla_pager_init(self._ptr, n, num_pages, max_seqs, max_blocks))
        self.num_pages, self.max_seqs, self.max_blocks = num_pages, max_seqs, max_blocks

    def reserve(self, seq: int, new_len: int) -> None:
        """Make sequence seq hold new_len tokens (ceil(new_len / 64) pages)."""
        _check(_lib.mla_pager_reserve(self._ptr, seq, new_len))

    def release(self, seq: int) -> None:
        _check(_lib.mla_pager_release(self._ptr, seq))

    def free_pages(self) -> int:
        r = _lib.mla_pager_free_pages(self._ptr)
        _check(min(r, 0))
        return r

    def seq_pages(self, seq: int) -> int:
        r = _lib.mla_pager_seq_pages(self._ptr, seq)
        _check(min(r, 0))
        return r

    def page_owner(self, page: int) -> int:
        r = _lib.mla_pager_page_owner(self._ptr, page)
        if r < -1:
            _check(r)
        return r

    def block_table(self) -> torch.Tensor:
        """A CPU copy of the block table [max_seqs, max_blocks] int32."""
        p = _lib.mla_pager_block_table(self._ptr)
        n = self.max_seqs * self.max_blocks
        arr = (ctypes.c_int32 * n).from_address(ctypes.addressof(p.contents))
        return torch.frombuffer(bytearray(arr), dtype=torch.int32).reshape(self.max_seqs, self.max_blocks)


def mla_sparse_prepare(indices: torch.Tensor, indptr: torch.Tensor, s_q: int, block_table: torch.Tensor,
                       cache_seqlens: torch.Tensor, num_pages: int, h_kv: int,
                       offsets: Optional[torch.Tensor] = None, counts: Optional[torch.Tensor] = None):
    """Keep each query row's valid index entries as cache-row byte offsets.

    indices int32 [nnz] (logical positions), indptr int32 [batch*s_q + 1] (CSR);
    returns (offsets uint32-as-int32 [nnz + 64], counts int32 [batch*s_q])."""
    for t, n in ((indices, "indices"), (indptr, "indptr"), (block_table, "block_table"),
                 (cache_seqlens, "cache_seqlens")):
        _require(t, n, torch.int32, on_device=False)
    if cache_seqlens.dim() != 1 or indices.dim() != 1 or indptr.dim() != 1 or block_table.dim() != 2:
        raise ValueError("cache_seqlens, indices and indptr must be 1-D and block_table [batch, max_blocks]")
    b = cache_seqlens.shape[0]
    rows = indptr.shape[0] - 1
    if rows != b * s_q:
        raise ValueError("indptr must have batch * s_q + 1 entries")
    if block_table.shape[0] != b:
        raise ValueError(f"block_table must have one row per sequence ({b}), got {block_table.shape[0]}")
    if offsets is not None:
        _require(offsets, "offsets", torch.int32, on_device=False)
        if offsets.dim() != 1 or offsets.shape[0] < indices.shape[0] + 64:
            raise ValueError("offsets needs nnz + 64 entries")
    if counts is not None:
        _require(counts, "counts", torch.int32, on_device=False)
        _shape(counts, "counts", (rows,))
    dev = indices.device
    _same_device(dev, indices=indices, indptr=indptr, block_table=block_table, cache_seqlens=cache_seqlens)
    if offsets is None:
        offsets = torch.empty(indices.shape[0] + 64, dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty(rows, dtype=torch.int32, device=dev)
    _same_device(dev, offsets=offsets, counts=counts)
    if indices.numel() == 0:
        # no row lists anything: the kernel reads no entry, but the C ABI takes
        # no null pointer (an empty tensor has none)
        indices = torch.zeros(1, dtype=torch.int32, device=dev)
    _check(_lib.mla_sparse_prepare(indices.data_ptr(), indptr.data_ptr(), b, s_q, block_table.data_ptr(),
                                   block_table.shape[1], cache_seqlens.data_ptr(), num_pages, h_kv,
                                   offsets.data_ptr(), counts.data_ptr(), _stream(dev)))
    return offsets, counts


def mla_sparse_decode(q: torch.Tensor, kcache: torch.Tensor, offsets: torch.Tensor, indptr: torch.Tensor,
                      counts: torch.Tensor, dv: int, tile_metadata: torch.Tensor, num_splits: torch.Tensor,
                      softmax_scale: float, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, nnz: Optional[int] = None):
    """Decode of every query row over its kept cache rows (after mla_sparse_prepare).

    ``nnz`` is the number of index entries (indptr[-1]); the kernel reads up to
    64 offsets past a row's kept entries, so offsets must hold nnz + 64.  When
    it is not given it is read from indptr, which synchronises with the device
    and is refused while a graph is being captured."""
    _require(q, "q", torch.bfloat16, on_device=False)
    _require(kcache, "kcache", torch.bfloat16, on_device=False)
    for t, n in ((offsets, "offsets"), (indptr, "indptr"), (counts, "counts"), (tile_metadata, "tile_metadata"),
                 (num_splits, "num_splits")):
        _require(t, n, torch.int32, on_device=False)
    if q.dim() != 4 or kcache.dim() != 4:
        raise ValueError("q must be [b, s_q, h_q, d] and kcache [pages, 64, h_kv, d]")
    b, s_q, h_q, d_qk = q.shape
    num_pages, page, h_kv, d_k = kcache.shape
    if d_k != d_qk or h_kv <= 0 or h_q % h_kv:
        raise ValueError("q / kcache shapes do not match")
    nq = b * s_q  # every query token is a sequence of its own
    _shape(indptr, "indptr", (nq + 1,))
    _shape(counts, "counts", (nq,))
    _shape(num_splits, "num_splits", (nq + 1,))
    if tile_metadata.dim() != 2 or tile_metadata.shape[1] != 8 or tile_metadata.shape[0] < 1:
        raise ValueError(f"tile_metadata must be [num_parts, 8], got {tuple(tile_metadata.shape)}")
    if offsets.dim() != 1:
        raise ValueError("offsets must be 1-D")
    rows = h_q // h_kv
    num_parts = tile_metadata.shape[0]
    if out is not None:
        _require(out, "out", torch.bfloat16, on_device=False)
        _shape(out, "out", (b, s_q, h_q, dv))
    if lse is not None:
        _require(lse, "lse", torch.float32, on_device=False)
        _shape(lse, "lse", (b, s_q, h_q))
    need = (nq + num_parts) * h_kv * rows * (dv + 1) * 4
    if workspace is not None and workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold {need} bytes")
    def check_nnz(n):
        if n < 0 or offsets.shape[0] < n + 64:
            raise ValueError(f"offsets must hold nnz + 64 = {n + 64} entries, got {offsets.shape[0]}")

    if nnz is not None:
        check_nnz(int(nnz))
    dev = q.device
    _same_device(dev, q=q, kcache=kcache, offsets=offsets, indptr=indptr, counts=counts,
                 tile_metadata=tile_metadata, num_splits=num_splits)
    if nnz is None:
        if torch.cuda.is_current_stream_capturing():
            raise ValueError("pass nnz (indptr[-1]) when capturing mla_sparse_decode into a graph")
        check_nnz(int(indptr[-1].item()))
    if out is None:
        out = torch.empty((b, s_q, h_q, dv), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((b, s_q, h_q), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _same_device(dev, out=out, lse=lse, workspace=workspace)
    _check(_lib.mla_sparse_decode(q.data_ptr(), kcache.data_ptr(), num_pages, offsets.data_ptr(), indptr.data_ptr(),
                                  counts.data_ptr(), b, s_q, h_q, h_kv, d_qk, dv, page, tile_metadata.data_ptr(),
                                  num_parts, num_splits.data_ptr(), float(softmax_scale), out.data_ptr(),
                                  lse.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream(dev)))
    return out, lse


def flash_mla_sparse_with_kvcache(q: torch.Tensor, k_cache: torch.Tensor, block_table: torch.Tensor,
                                  cache_seqlens: torch.Tensor, indices: torch.Tensor, indptr: torch.Tensor,
                                  head_dim_v: int = DV, softmax_scale: Optional[float] = None,
                                  num_parts: Optional[int] = None):
    """Token-sparse decode: query row b*s_q+s attends to the cached tokens listed
    in indices[indptr[v]:indptr[v+1]].  Returns (out, lse)."""
    if softmax_scale is None:
        softmax_scale = q.shape[-1] ** -0.5
    b, s_q, h_q, _ = q.shape
    h_kv = k_cache.shape[2]
    offsets, counts = mla_sparse_prepare(indices, indptr, s_q, block_table, cache_seqlens, k_cache.shape[0], h_kv)
    md, ns = mla_get_metadata(counts, h_q // h_kv, h_kv, num_parts=num_parts)
    return mla_sparse_decode(q, k_cache, offsets, indptr, counts, head_dim_v, md, ns, softmax_scale,
                             nnz=indices.shape[0])
