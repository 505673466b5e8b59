"""The Python binding refuses tensors whose shapes do not match the batch it
derives from q, before any device call: the kernels index block_table,
cache_seqlens, num_splits, tile_metadata, out, lse and the sparse offset list by
sequence, row and part, so a short tensor would become an out-of-bounds read or
write on the GPU.  Runs without a GPU (host tensors; the shape checks come
before the device checks)."""
import pytest
import torch

mla = pytest.importorskip("paged_mla_decode_02_amd")

B, S_Q, H_Q, H_KV = 3, 2, 16, 1


def good():
    return dict(
        q=torch.zeros((B, S_Q, H_Q, 576), dtype=torch.bfloat16),
        kcache=torch.zeros((5, 64, H_KV, 576), dtype=torch.bfloat16),
        block_table=torch.zeros((B, 4), dtype=torch.int32),
        cache_seqlens=torch.zeros((B,), dtype=torch.int32),
        tile_metadata=torch.zeros((7, 8), dtype=torch.int32),
        num_splits=torch.zeros((B + 1,), dtype=torch.int32),
    )


def call(**over):
    a = good()
    extra = {k: over.pop(k) for k in ("out", "lse", "workspace") if k in over}
    a.update(over)
    return mla.mla_decode_paged(a["q"], a["kcache"], a["block_table"], a["cache_seqlens"], 512,
                                a["tile_metadata"], a["num_splits"], False, 0.07, **extra)


def test_well_formed_call_reaches_the_device_check():
    with pytest.raises(ValueError, match="device tensor"):
        call()


@pytest.mark.parametrize("over,msg", [
    (dict(block_table=torch.zeros((B - 1, 4), dtype=torch.int32)), "block_table"),
    (dict(cache_seqlens=torch.zeros((B + 1,), dtype=torch.int32)), "cache_seqlens"),
    (dict(cache_seqlens=torch.zeros((B, 1), dtype=torch.int32)), "cache_seqlens"),
    (dict(num_splits=torch.zeros((B,), dtype=torch.int32)), "num_splits"),
    (dict(tile_metadata=torch.zeros((7, 7), dtype=torch.int32)), "tile_metadata"),
    (dict(tile_metadata=torch.zeros((56,), dtype=torch.int32)), "tile_metadata"),
    (dict(out=torch.zeros((B, S_Q, H_Q, 511), dtype=torch.bfloat16)), "out"),
    (dict(out=torch.zeros((B - 1, S_Q, H_Q, 512), dtype=torch.bfloat16)), "out"),
    (dict(lse=torch.zeros((B, S_Q, H_Q + 1), dtype=torch.float32)), "lse"),
    (dict(lse=torch.zeros((B, S_Q, H_Q), dtype=torch.float64)), "lse"),
    (dict(workspace=torch.zeros(100, dtype=torch.uint8)), "workspace"),
    (dict(kcache=torch.zeros((5, 64, 3, 576), dtype=torch.bfloat16)), "multiple of h_kv"),
])
def test_decode_rejects_mismatched_shapes(over, msg):
    with pytest.raises(ValueError, match=msg):
        call(**over)


def sparse_args(**over):
    nq = B * S_Q
    a = dict(q=torch.zeros((B, S_Q, H_Q, 576), dtype=torch.bfloat16),
             kcache=torch.zeros((5, 64, H_KV, 576), dtype=torch.bfloat16),
             offsets=torch.zeros((10 + 64,), dtype=torch.int32),
             indptr=torch.zeros((nq + 1,), dtype=torch.int32),
             counts=torch.zeros((nq,), dtype=torch.int32),
             tile_metadata=torch.zeros((7, 8), dtype=torch.int32),
             num_splits=torch.zeros((nq + 1,), dtype=torch.int32))
    a.update(over)
    return a


def sparse_call(nnz=10, **over):
    a = sparse_args(**over)
    return mla.mla_sparse_decode(a["q"], a["kcache"], a["offsets"], a["indptr"], a["counts"], 512,
                                 a["tile_metadata"], a["num_splits"], 0.07, nnz=nnz)


def test_sparse_well_formed_reaches_the_device_check():
    with pytest.raises(ValueError, match="device tensor"):
        sparse_call()


@pytest.mark.parametrize("over,msg", [
    (dict(indptr=torch.zeros((B * S_Q,), dtype=torch.int32)), "indptr"),
    (dict(counts=torch.zeros((B,), dtype=torch.int32)), "counts"),
    (dict(num_splits=torch.zeros((B + 1,), dtype=torch.int32)), "num_splits"),
    (dict(tile_metadata=torch.zeros((3, 4), dtype=torch.int32)), "tile_metadata"),
])
def test_sparse_decode_rejects_mismatched_shapes(over, msg):
    with pytest.raises(ValueError, match=msg):
        sparse_call(**over)


def test_sparse_decode_rejects_short_offsets():
    # a given nnz is host metadata: checked before any device check
    a = sparse_args()
    with pytest.raises(ValueError, match="nnz"):
        mla.mla_sparse_decode(a["q"], a["kcache"], a["offsets"][:20], a["indptr"], a["counts"], 512,
                              a["tile_metadata"], a["num_splits"], 0.07, nnz=10)


def test_sparse_prepare_rejects_mismatched_shapes():
    idx = torch.zeros((10,), dtype=torch.int32)
    ptr = torch.zeros((B * S_Q + 1,), dtype=torch.int32)
    bt = torch.zeros((B, 4), dtype=torch.int32)
    sl = torch.zeros((B,), dtype=torch.int32)
    with pytest.raises(ValueError, match="indptr"):
        mla.mla_sparse_prepare(idx, ptr[:-1], S_Q, bt, sl, 5, 1)
    with pytest.raises(ValueError, match="block_table"):
        mla.mla_sparse_prepare(idx, ptr, S_Q, bt[:-1], sl, 5, 1)
    with pytest.raises(ValueError, match="offsets"):
        mla.mla_sparse_prepare(idx, ptr, S_Q, bt, sl, 5, 1, offsets=torch.zeros((70,), dtype=torch.int32))
    with pytest.raises(ValueError, match="counts"):
        mla.mla_sparse_prepare(idx, ptr, S_Q, bt, sl, 5, 1, counts=torch.zeros((B,), dtype=torch.int32))
