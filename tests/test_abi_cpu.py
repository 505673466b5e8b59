"""The C ABI without a GPU: every symbol include/mla.h declares is exported, and
argument validation returns the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")
LIB = os.path.join(ROOT, "paged_mla_decode_02_amd", "libmla.so")

MLA_OK, MLA_ERR_INVALID, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE = 0, -1, -2, -3
FAKE = 0x100000  # never dereferenced: every call below fails validation first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libmla.so not built")
    lib = ctypes.CDLL(LIB)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.mla_plan.argtypes = [I, I, I, I, I, ctypes.POINTER(I), ctypes.POINTER(SZ)]
    lib.mla_get_metadata.argtypes = [P, I, I, I, I, P, P, P]
    lib.mla_decode_paged.argtypes = [P, P, ctypes.c_int64, P, I, P, I, I, I, I, I, I, I, P, I, P, I,
                                     ctypes.c_float, P, P, P, SZ, P]
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_tile_rows.argtypes = [I]
    return lib


def test_header_declares_the_two_calls():
    names = declared_functions()
    assert {"mla_get_metadata", "mla_decode_paged", "mla_plan", "mla_last_error", "mla_tile_rows"} <= set(names)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in mla.h but not exported"


def plan(lib, batch, rows, h_kv, dv=512, cus=256):
    parts = ctypes.c_int(-7)
    ws = ctypes.c_size_t(0)
    rc = lib.mla_plan(batch, rows, h_kv, dv, cus, ctypes.byref(parts), ctypes.byref(ws))
    return rc, parts.value, ws.value


def test_plan(lib):
    rc, P, ws = plan(lib, 64, 16, 1)
    assert rc == MLA_OK and P == 256 and ws == (64 + 256) * 16 * 513 * 4
    rc, P, ws = plan(lib, 128, 128, 1)  # two 64-row tiles per part, parts a multiple of 8
    assert rc == MLA_OK and P == 128 and ws == (128 + 128) * 128 * 513 * 4
    rc, P, _ = plan(lib, 132, 256, 1)  # two 128-row tiles per part, parts a multiple of 8
    assert rc == MLA_OK and P == 128
    rc, P, _ = plan(lib, 8, 64, 1)
    assert rc == MLA_OK and P == 256
    rc, P, _ = plan(lib, 1, 16, 3, cus=2)
    assert rc == MLA_OK and P == 1
    assert lib.mla_tile_rows(16) == 16 and lib.mla_tile_rows(17) == 64 and lib.mla_tile_rows(64) == 64
    assert lib.mla_tile_rows(128) == 64 and lib.mla_tile_rows(129) == 128 and lib.mla_tile_rows(256) == 128


@pytest.mark.parametrize("args,code", [
    ((0, 16, 1, 512, 256), MLA_ERR_INVALID),
    ((4, 0, 1, 512, 256), MLA_ERR_INVALID),
    ((4, 16, 0, 512, 256), MLA_ERR_INVALID),
    ((4, 16, 1, 256, 256), MLA_ERR_UNSUPPORTED),
    ((9000, 16, 1, 512, 256), MLA_ERR_UNSUPPORTED),
    ((4, 16, 1, 512, -1), MLA_ERR_INVALID),
])
def test_plan_rejects(lib, args, code):
    parts = ctypes.c_int(0)
    ws = ctypes.c_size_t(0)
    assert lib.mla_plan(*args, ctypes.byref(parts), ctypes.byref(ws)) == code
    assert lib.mla_last_error()


def test_metadata_rejects(lib):
    assert lib.mla_get_metadata(None, 4, 16, 1, 8, FAKE, FAKE, None) == MLA_ERR_INVALID
    assert lib.mla_get_metadata(FAKE, 4, 16, 1, 0, FAKE, FAKE, None) == MLA_ERR_INVALID
    assert lib.mla_get_metadata(FAKE, 0, 16, 1, 8, FAKE, FAKE, None) == MLA_ERR_INVALID
    assert lib.mla_get_metadata(FAKE, 10000, 16, 1, 8, FAKE, FAKE, None) == MLA_ERR_UNSUPPORTED


def decode_args(**over):
    a = dict(q=FAKE, kcache=FAKE, num_pages=10, block_table=FAKE, max_blocks=4, seqlens=FAKE,
             batch=2, s_q=1, h_q=16, h_kv=1, d_qk=576, dv=512, page=64, md=FAKE, num_parts=8,
             ns=FAKE, causal=0, scale=0.07, out=FAKE, lse=FAKE, ws=FAKE,
             ws_bytes=(2 + 8) * 16 * 513 * 4, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,code", [
    (dict(q=None), MLA_ERR_INVALID),
    (dict(out=None), MLA_ERR_INVALID),
    (dict(d_qk=512), MLA_ERR_UNSUPPORTED),
    (dict(dv=576), MLA_ERR_UNSUPPORTED),
    (dict(page=128), MLA_ERR_UNSUPPORTED),
    (dict(h_q=15, h_kv=2), MLA_ERR_INVALID),
    (dict(s_q=0), MLA_ERR_INVALID),
    (dict(max_blocks=0), MLA_ERR_INVALID),
    (dict(num_pages=0), MLA_ERR_INVALID),
    (dict(num_parts=0), MLA_ERR_INVALID),
    (dict(causal=2), MLA_ERR_INVALID),
    (dict(scale=float("nan")), MLA_ERR_INVALID),
    (dict(q=FAKE + 8), MLA_ERR_INVALID),
    (dict(ws=None), MLA_ERR_WORKSPACE),
    (dict(ws_bytes=100), MLA_ERR_WORKSPACE),
    (dict(batch=9000), MLA_ERR_UNSUPPORTED),
])
def test_decode_rejects(lib, over, code):
    assert lib.mla_decode_paged(*decode_args(**over)) == code
    assert lib.mla_last_error()


def test_python_binding_imports():
    import paged_mla_decode_02_amd as mla
    assert mla.mla_plan(64, 16, 1, 512, 256) == (256, (64 + 256) * 16 * 513 * 4)
    with pytest.raises(mla.MlaError):
        mla.mla_plan(0, 16, 1, 512, 256)


def test_absorb_calls_reject(lib):
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.mla_absorb_q.argtypes = [P, P, P, I, I, P, P]
    lib.mla_unabsorb_out.argtypes = [P, P, I, I, P, P]
    assert lib.mla_absorb_q(None, FAKE, FAKE, 4, 16, FAKE, None) == MLA_ERR_INVALID
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, -1, 16, FAKE, None) == MLA_ERR_INVALID
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, 4, 0, FAKE, None) == MLA_ERR_INVALID
    assert lib.mla_absorb_q(FAKE, FAKE + 2, FAKE, 4, 16, FAKE, None) == MLA_ERR_INVALID
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, 0, 16, FAKE, None) == MLA_OK  # nothing to do, no launch
    assert lib.mla_unabsorb_out(FAKE, None, 4, 16, FAKE, None) == MLA_ERR_INVALID
    assert lib.mla_unabsorb_out(FAKE, FAKE, 4, -3, FAKE, None) == MLA_ERR_INVALID
    assert lib.mla_unabsorb_out(FAKE, FAKE, 4, 16, FAKE + 8, None) == MLA_ERR_INVALID
    assert lib.mla_unabsorb_out(FAKE, FAKE, 4, 16, FAKE + 8, None) == MLA_ERR_INVALID
    assert lib.mla_last_error()
    assert lib.mla_unabsorb_out(FAKE, FAKE, 0, 16, FAKE, None) == MLA_OK
    assert lib.mla_unabsorb_out(None, None, 0, 16, None, None) == MLA_OK  # no tokens: pointers unused
    assert lib.mla_absorb_q(None, None, None, 0, 16, None, None) == MLA_OK


def test_kv_append_rejects(lib):
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.mla_kv_append.argtypes = [P, I, I, I, P, P, I, P, ctypes.c_int64, P, P]
    good = dict(new_kv=FAKE, batch=4, s_new=1, h_kv=1, lens=FAKE + 64, bt=FAKE + 128, max_blocks=8, kc=FAKE,
                num_pages=10, new_lens=FAKE + 256)

    def call(**over):
        a = dict(good, **over)
        return lib.mla_kv_append(a["new_kv"], a["batch"], a["s_new"], a["h_kv"], a["lens"], a["bt"],
                                 a["max_blocks"], a["kc"], a["num_pages"], a["new_lens"], None)

    assert call(batch=-1) == MLA_ERR_INVALID
    assert call(s_new=-2) == MLA_ERR_INVALID
    assert call(h_kv=0) == MLA_ERR_INVALID
    assert call(max_blocks=0) == MLA_ERR_INVALID
    assert call(num_pages=0) == MLA_ERR_INVALID
    assert call(new_kv=None) == MLA_ERR_INVALID
    assert call(kc=None) == MLA_ERR_INVALID
    assert call(lens=None) == MLA_ERR_INVALID
    assert call(bt=None) == MLA_ERR_INVALID
    assert call(new_lens=FAKE + 64) == MLA_ERR_INVALID  # aliases cache_seqlens
    assert call(new_kv=FAKE + 4) == MLA_ERR_INVALID     # misaligned
    assert call(kc=FAKE + 8) == MLA_ERR_INVALID
    assert call(batch=1 << 20, s_new=1 << 10, h_kv=8) == MLA_ERR_UNSUPPORTED
    assert lib.mla_last_error()
    assert call(batch=0, new_kv=None, kc=None, lens=None, bt=None) == MLA_OK  # nothing to do, no launch


@pytest.mark.parametrize("scale", [0.0, -0.5, float("inf"), float("nan")])
def test_decode_rejects_scale(lib, scale):
    args = [FAKE, FAKE, 100, FAKE, 8, FAKE, 4, 1, 16, 1, 576, 512, 64, FAKE, 256, FAKE, 0, scale,
            FAKE, FAKE, FAKE, 1 << 30, None]
    assert lib.mla_decode_paged(*args) == MLA_ERR_INVALID
    assert b"softmax_scale" in lib.mla_last_error()


@pytest.mark.parametrize("over,code", [
    (dict(q=None), MLA_ERR_INVALID),
    (dict(s_q=0), MLA_ERR_INVALID),
    (dict(d_qk=512), MLA_ERR_UNSUPPORTED),
    (dict(ws_bytes=100), MLA_ERR_WORKSPACE),
    (dict(batch=9000), MLA_ERR_UNSUPPORTED),
])
def test_decode_fp8_rejects(lib, over, code):
    lib.mla_decode_paged_fp8.argtypes = lib.mla_decode_paged.argtypes
    assert lib.mla_decode_paged_fp8(*decode_args(**over)) == code
    assert lib.mla_last_error()


def sparse_prepare_args(**over):
    a = dict(indices=FAKE, indptr=FAKE, batch=2, s_q=1, bt=FAKE, max_blocks=4, seqlens=FAKE, num_pages=10,
             h_kv=1, offsets=FAKE, counts=FAKE, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,code", [
    (dict(batch=-1), MLA_ERR_INVALID),
    (dict(s_q=0), MLA_ERR_INVALID),
    (dict(indices=None), MLA_ERR_INVALID),  # also when every list is empty
    (dict(counts=None), MLA_ERR_INVALID),
    (dict(num_pages=60000), MLA_ERR_UNSUPPORTED),  # 4.4 GB: beyond 32-bit row offsets
    (dict(batch=0), MLA_OK),  # nothing to do, no HIP call
])
def test_sparse_prepare_rejects(lib, over, code):
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.mla_sparse_prepare.argtypes = [P, P, I, I, P, I, P, ctypes.c_int64, I, P, P, P]
    assert lib.mla_sparse_prepare(*sparse_prepare_args(**over)) == code


def sparse_decode_args(**over):
    a = dict(q=FAKE, kcache=FAKE, num_pages=10, offsets=FAKE, indptr=FAKE, counts=FAKE, batch=2, s_q=1,
             h_q=16, h_kv=1, d_qk=576, dv=512, page=64, md=FAKE, num_parts=8, ns=FAKE, scale=0.07,
             out=FAKE, lse=FAKE, ws=FAKE, ws_bytes=(2 + 8) * 16 * 513 * 4, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,code", [
    (dict(batch=0), MLA_ERR_INVALID),
    (dict(batch=4097, s_q=2), MLA_ERR_UNSUPPORTED),  # batch * s_q query rows above MLA_MAX_BATCH
    (dict(d_qk=512), MLA_ERR_UNSUPPORTED),
    (dict(ws_bytes=100), MLA_ERR_WORKSPACE),
    (dict(num_pages=60000), MLA_ERR_UNSUPPORTED),
])
def test_sparse_decode_rejects(lib, over, code):
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.mla_sparse_decode.argtypes = [P, P, ctypes.c_int64, P, P, P, I, I, I, I, I, I, I, P, I, P,
                                      ctypes.c_float, P, P, P, SZ, P]
    assert lib.mla_sparse_decode(*sparse_decode_args(**over)) == code
    assert lib.mla_last_error()


def noalloc_args(**over):
    a = dict(q=FAKE, kc=FAKE, np_=100, bt=FAKE, mb=8, sl=FAKE, b=64, s_q=1, h_q=16, h_kv=1, d_qk=576, dv=512,
             page=64, md=FAKE, P=256, ns=FAKE, causal=0, scale=0.07, out=FAKE, lse=FAKE, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,code", [
    (dict(q=None), MLA_ERR_INVALID),
    (dict(d_qk=512), MLA_ERR_UNSUPPORTED),
    (dict(h_q=17, h_kv=2), MLA_ERR_INVALID),
    # (8192 + 256) * 256 rows * 513 * 4 bytes is far above the 256 MiB array
    (dict(b=8192, s_q=2, h_q=128), MLA_ERR_WORKSPACE),
    (dict(b=600, s_q=2, h_q=128), MLA_ERR_WORKSPACE),
])
def test_decode_noalloc_rejects(lib, over, code):
    """Validation, including the scratch limit, runs before any HIP call."""
    lib.mla_decode_paged_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                             ctypes.c_int, ctypes.c_void_p] + [ctypes.c_int] * 7 + [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p]
    assert lib.mla_decode_paged_noalloc(*noalloc_args(**over)) == code
    msg = lib.mla_last_error().decode()
    assert msg
    if code == MLA_ERR_WORKSPACE:
        assert "268435456" in msg and "scratch" in msg
