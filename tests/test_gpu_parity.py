"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: out relative L2 <= 1e-2, lse absolute <= 1e-3 (rows the oracle gives -inf
must be -inf), tile metadata and num_splits bit-exact against the oracle twin.
Every case compares every output element: the five workloads at full size, the
maximum sizes (8192 sequences, a 2^20-token sequence), edge cases and random
shapes.
"""

import dataclasses

import numpy as np
import pytest

import workloads
from workloads import make_workload

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 1e-3


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    import paged_mla_decode_02_amd as mla
    oracle.build(force=False)
    return torch, mla, oracle.default(), torch.device("cuda:0")


def upload(torch, w, dev):
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kc = torch.from_numpy(w.kcache.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.cache_seqlens).to(dev)
    return q, kc, bt, sl


def run(env, w, num_parts=None, tensors=None):
    torch, mla, _, dev = env
    q, kc, bt, sl = tensors if tensors is not None else upload(torch, w, dev)
    md, ns = mla.mla_get_metadata(sl, w.rows, w.h_kv, num_parts=num_parts)
    out, lse = mla.mla_decode_paged(q, kc, bt, sl, w.dv, md, ns, w.causal, w.scale)
    torch.cuda.synchronize()
    return md.cpu().numpy(), ns.cpu().numpy(), out, lse


def as_np(out, lse):
    o = out.float().cpu().numpy().astype(np.float64)
    return o.reshape(-1, o.shape[-1]), lse.cpu().numpy().astype(np.float64).reshape(-1)


def check(out, lse, ref_out, ref_lse, sel=None, what=""):
    go, gl = as_np(out, lse)
    if sel is not None:
        go, gl = go[sel], gl[sel]
    assert np.all(np.isfinite(go)), f"{what}: non-finite output"
    ninf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(gl), ninf), f"{what}: -inf lse rows differ"
    assert np.all(go[ninf] == 0), f"{what}: rows without keys must be zero"
    denom = np.linalg.norm(ref_out)
    rel = np.linalg.norm(go - ref_out) / denom if denom > 0 else np.linalg.norm(go)
    err = np.max(np.abs(gl[~ninf] - ref_lse[~ninf])) if np.any(~ninf) else 0.0
    assert rel <= OUT_TOL, f"{what}: out rel L2 {rel:.3e} > {OUT_TOL}"
    assert err <= LSE_TOL, f"{what}: lse abs err {err:.3e} > {LSE_TOL}"
    return rel, err


# ------------------------------------------------------------------ metadata
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_metadata_bit_exact_configs(env, cfg):
    torch, mla, orc, dev = env
    w = workloads.config_workload(cfg)
    sl = torch.from_numpy(w.cache_seqlens).to(dev)
    md, ns = mla.mla_get_metadata(sl, w.rows, w.h_kv)
    md_ref, ns_ref = orc.schedule(w.cache_seqlens, w.rows, md.shape[0])
    assert np.array_equal(md.cpu().numpy(), md_ref)
    assert np.array_equal(ns.cpu().numpy(), ns_ref)


@pytest.mark.parametrize("seed", range(8))
def test_metadata_bit_exact_random(env, seed):
    torch, mla, orc, dev = env
    rng = np.random.default_rng(100 + seed)
    b = int(rng.integers(1, 3000))
    lens = rng.integers(0, int(rng.choice([2, 65, 5000, 100000])), size=b).astype(np.int32)
    rows = int(rng.choice([1, 16, 17, 64, 128, 256]))
    P = int(rng.choice([1, 7, 64, 256, 1500]))
    md, ns = mla.mla_get_metadata(torch.from_numpy(lens).to(dev), rows, 1, num_parts=P)
    md_ref, ns_ref = orc.schedule(lens, rows, P)
    assert np.array_equal(md.cpu().numpy(), md_ref)
    assert np.array_equal(ns.cpu().numpy(), ns_ref)


# ------------------------------------------------------------------ the five workloads
def test_config0_tiny_full(env):
    w = workloads.config_workload(0)
    md, ns, out, lse = run(env, w)
    ref = env[2].decode(w)
    check(out, lse, *ref, what="tiny")


def test_config1_memory_bound_full(env):
    w = workloads.config_workload(1)
    md, ns, out, lse = run(env, w)
    ref = env[2].decode(w)
    check(out, lse, *ref, what="memory-bound")


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_large_configs_full(env, cfg):
    """compute_bound_full_heads, spec_decode_causal and long_context at full size,
    every output row against the oracle (the fp64 oracle runs these in seconds
    on the host cores)."""
    w = workloads.config_workload(cfg)
    md, ns, out, lse = run(env, w)
    md_ref, ns_ref = env[2].schedule(w.cache_seqlens, w.rows, md.shape[0])
    assert np.array_equal(md, md_ref) and np.array_equal(ns, ns_ref)
    ref_out, ref_lse = env[2].decode(w)
    check(out, lse, ref_out, ref_lse, what=f"config {cfg}")
    # and per sequence: a wrong row tile, part or head mapping that the global
    # relative L2 would average away still fails here
    go, _ = as_np(out, lse)
    per_b = w.s_q * w.h_q
    for b in range(w.batch):
        r = slice(b * per_b, (b + 1) * per_b)
        den = np.linalg.norm(ref_out[r])
        assert np.linalg.norm(go[r] - ref_out[r]) <= OUT_TOL * den, f"config {cfg}: sequence {b}"


# ------------------------------------------------------------------ combine over many chunks
@pytest.mark.parametrize("h_q,L", [(16, 1 << 17), (64, 1 << 18)])
def test_combine_more_than_256_chunks(env, h_q, L):
    """One sequence cut into ~290 chunks (300 parts): the combine stages chunk
    weights 256 at a time, so its second tile runs.  16 rows (token-split
    kernel) and 64 rows (split-wave kernel), every row against the oracle."""
    w = make_workload([L], s_q=1, h_q=h_q, seed=90 + h_q, outliers=True)
    md, ns, out, lse = run(env, w, num_parts=300)
    md_ref, ns_ref = env[2].schedule(w.cache_seqlens, w.rows, md.shape[0])
    assert np.array_equal(md, md_ref) and np.array_equal(ns, ns_ref)
    assert ns[-1] > 256, f"only {ns[-1]} chunks: the second weight tile would not run"
    check(out, lse, *env[2].decode(w), what=f"{ns[-1]} chunks, {h_q} rows")


# ------------------------------------------------------------------ maximum sizes
def test_max_batch(env):
    """MLA_MAX_BATCH = 8192 sequences (the metadata kernel's on-chip prefix sums
    at their limit): metadata bit-exact, every output row against the oracle."""
    w = make_workload(np.random.default_rng(81).integers(0, 131, size=8192), s_q=1, h_q=16, seed=81)
    md, ns, out, lse = run(env, w)
    md_ref, ns_ref = env[2].schedule(w.cache_seqlens, w.rows, md.shape[0])
    assert np.array_equal(md, md_ref) and np.array_equal(ns, ns_ref)
    check(out, lse, *env[2].decode(w), what="8192 sequences")


@pytest.mark.parametrize("h_q", [16, 64])
def test_one_long_sequence(env, h_q):
    """One sequence of 2^20 tokens (16384 pages, split across every part), 16
    rows (token-split kernel) and 64 rows (split-wave kernel)."""
    w = make_workload([1 << 20], s_q=1, h_q=h_q, seed=82 + h_q)
    md, ns, out, lse = run(env, w)
    md_ref, ns_ref = env[2].schedule(w.cache_seqlens, w.rows, md.shape[0])
    assert np.array_equal(md, md_ref) and np.array_equal(ns, ns_ref)
    assert ns[-1] == np.count_nonzero(md[:, 0] < w.batch)  # one chunk per non-empty part
    check(out, lse, *env[2].decode(w), what=f"2^20 tokens, {h_q} rows")


@pytest.mark.parametrize("P", [1, 2])
@pytest.mark.parametrize("s_q,h_q", [(1, 16), (1, 64), (1, 128), (2, 128)])
def test_long_chunk_page_id_windows(env, s_q, h_q, P):
    """Chunks of more than 64 pages in one part (a 10000-token sequence, 157
    pages, with 1 or 2 parts): every kernel reads a sequence's block-table
    entries 64 at a time and fetches the next 64 inside its page loop (16, 64,
    128 and 256 rows per KV head)."""
    w = make_workload([10000, 300], s_q=s_q, h_q=h_q, causal=s_q > 1, seed=900 + h_q + s_q,
                      extra_pages=2, poison_tail=True, outliers=True)
    md, ns, out, lse = run(env, w, num_parts=P)
    md_ref, ns_ref = env[2].schedule(w.cache_seqlens, w.rows, md.shape[0])
    assert np.array_equal(md, md_ref) and np.array_equal(ns, ns_ref)
    # the first part starts at page 0 of sequence 0 and ends more than 64 pages later
    assert md[0, 0] == 0 and md[0, 1] == 0 and (md[0, 2] > 0 or md[0, 3] > 64)
    check(out, lse, *env[2].decode(w), what=f"10000 tokens, {w.rows} rows, P={P}")


# ------------------------------------------------------------------ edge cases
EDGE = [
    # lens, s_q, h_q, h_kv, causal, num_parts
    ([1], 1, 16, 1, False, None),
    ([63, 64, 65, 1, 0, 128], 1, 16, 1, False, None),
    ([0, 0], 1, 16, 1, False, None),
    ([0, 0], 2, 64, 1, True, None),
    ([65, 129, 1, 2, 3], 2, 16, 1, True, None),        # L % 64 == 1 with causal s_q = 2
    ([65, 129, 1, 2, 3], 2, 64, 1, True, 3),
    ([1000, 1, 70], 1, 8, 1, False, 2),
    ([1000, 1, 70], 1, 16, 2, False, None),            # two KV heads, 8 q heads each
    ([300, 77], 2, 32, 2, True, 5),
    ([4096, 100], 1, 128, 1, False, 7),
    ([513, 2049, 64], 2, 128, 1, True, 16),
    ([700, 900], 1, 17, 1, False, 9),                  # 17 rows: one ragged 64-row tile
    ([700, 900], 3, 32, 1, True, 11),                  # 96 rows: two tiles, second ragged
    ([5000], 1, 64, 1, False, 64),                     # many splits of one sequence
    ([5000], 1, 16, 1, False, 64),
    ([2, 3000, 1, 640], 1, 1, 1, False, None),         # a single query row
    # more than 128 rows per KV head: 128-row tiles, the last one ragged
    ([700, 900, 33], 3, 64, 1, True, 9),               # 192 rows
    ([1200, 5], 2, 100, 1, True, None),                # 200 rows
    ([4100], 1, 129, 1, False, 32),                    # 129 rows: a one-row second tile, many splits
    ([300, 2000], 5, 64, 2, True, 6),                  # two KV heads of 160 rows
    # the combine's two-row form (num_parts <= 8 * batch) on rows with more
    # than 8 chunks: 24 chunks, and 313 (lse values re-read, two weight tiles)
    ([9000, 100, 100, 100], 1, 16, 1, False, 32),
    ([120000] + [64] * 63, 1, 16, 1, False, 500),
]


@pytest.mark.parametrize("lens,s_q,h_q,h_kv,causal,P", EDGE)
def test_edge_cases(env, lens, s_q, h_q, h_kv, causal, P):
    w = make_workload(lens, s_q=s_q, h_q=h_q, h_kv=h_kv, causal=causal, seed=sum(lens) + s_q,
                      extra_pages=2, poison_tail=True, outliers=True)
    md, ns, out, lse = run(env, w, num_parts=P)
    md_ref, ns_ref = env[2].schedule(w.cache_seqlens, w.rows, md.shape[0])
    assert np.array_equal(md, md_ref) and np.array_equal(ns, ns_ref)
    ref = env[2].decode(w)
    check(out, lse, *ref, what=f"edge {lens} s_q={s_q} h_q={h_q} h_kv={h_kv} P={P}")


# ------------------------------------------------------------ random shapes
def random_shape(seed):
    """A seeded draw of batch, lengths (with 0, 1 and page-edge lengths mixed
    in), s_q, heads, causal mask and part count."""
    g = np.random.Generator(np.random.PCG64(1000 + seed))
    batch = int(g.integers(1, 13))
    pool = [0, 1, 63, 64, 65, 127, 128, 129]
    lens = [int(g.choice(pool)) if g.random() < 0.3 else int(g.integers(1, 3000)) for _ in range(batch)]
    s_q = int(g.integers(1, 5))
    h_kv = int(g.choice([1, 1, 2]))
    h_q = h_kv * int(g.choice([1, 4, 8, 16, 17, 32, 64]))
    causal = bool(g.random() < 0.5)
    P = None if g.random() < 0.5 else int(g.integers(1, 40))
    return lens, s_q, h_q, h_kv, causal, P


@pytest.mark.parametrize("seed", range(16))
def test_random_shapes(env, seed):
    lens, s_q, h_q, h_kv, causal, P = random_shape(seed)
    w = make_workload(lens, s_q=s_q, h_q=h_q, h_kv=h_kv, causal=causal, seed=seed,
                      extra_pages=1, poison_tail=True, outliers=bool(seed % 2))
    md, ns, out, lse = run(env, w, num_parts=P)
    md_ref, ns_ref = env[2].schedule(w.cache_seqlens, w.rows, md.shape[0])
    assert np.array_equal(md, md_ref) and np.array_equal(ns, ns_ref)
    ref = env[2].decode(w)
    check(out, lse, *ref, what=f"random seed={seed}: lens={lens} s_q={s_q} h_q={h_q} h_kv={h_kv} "
                               f"causal={causal} P={P}")


@pytest.mark.parametrize("h_q", [8, 16, 64, 128])
def test_large_scores_rescale(env, h_q):
    """Scores far apart (|x| up to ~300 in log2 units) force the lazy rescale
    path of every kernel: 16 rows per KV head (token-split), 32 and 128 rows
    (split-wave 64-row tiles, rescale threshold 2^64), 256 rows (128-row
    tiles, 2^8)."""
    w = make_workload([3000, 640, 129], s_q=2, h_q=h_q, causal=True, seed=21)
    ramp = np.linspace(0, 40, 3000 * 0 + w.num_pages * 64).astype(np.float32)
    kc = workloads.bf16_to_f32(w.kcache).reshape(w.num_pages * 64, -1)
    kc = kc * ramp[:, None]
    w.kcache = workloads.bf16_bits(kc).reshape(w.kcache.shape)
    md, ns, out, lse = run(env, w, num_parts=6)
    ref = env[2].decode(w)
    check(out, lse, *ref, what="rescale")


# ------------------------------------------------------------------ determinism / invariance
def test_determinism_bitwise(env):
    torch = env[0]
    w = workloads.config_workload(1)
    t = upload(torch, w, env[3])
    _, _, o1, l1 = run(env, w, tensors=t)
    _, _, o2, l2 = run(env, w, tensors=t)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("cfg,rows_h", [(0, None), (None, 64)])
def test_page_permutation_bitwise(env, cfg, rows_h):
    torch = env[0]
    if cfg is not None:
        w = workloads.config_workload(cfg)
    else:
        w = make_workload([1000, 77, 4000], s_q=1, h_q=rows_h, seed=3)
    _, _, o1, l1 = run(env, w)
    wp = workloads.permute_pages(w, 9)
    _, _, o2, l2 = run(env, wp)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("bad", ["past_end", "negative"])
@pytest.mark.parametrize("s_q,h_q", [(1, 16), (1, 64), (1, 128), (2, 128)])
def test_out_of_range_page_ids_are_safe(env, s_q, h_q, bad):
    """A block-table entry outside [0, num_pages) reads as a page of zeros in
    every kernel (16, 64, 128 and 256 rows), never outside the cache: the
    result equals the oracle's on the same table with that entry pointing at
    an all-zero page appended to the cache."""
    w = make_workload([200, 100], s_q=s_q, h_q=h_q, causal=s_q > 1, seed=4)
    w.block_table[0, 1] = w.num_pages + 1000 if bad == "past_end" else -5
    _, _, out, lse = run(env, w)
    zero = np.zeros((1,) + w.kcache.shape[1:], dtype=w.kcache.dtype)
    bt = w.block_table.copy()
    bt[0, 1] = w.num_pages
    ref = env[2].decode(dataclasses.replace(w, kcache=np.concatenate([w.kcache, zero]), block_table=bt))
    check(out, lse, *ref, what=f"{bad} page id, {w.rows} rows")


# ------------------------------------------------------------------ HIP graphs
@pytest.mark.parametrize("cfg", [1, 4])
def test_graph_replay_matches_eager(env, cfg):
    """A captured step (metadata + decode + combine) replayed several times, with
    eager work and synchronisations between replays, matches the eager result
    bit for bit on every replay.  The workspace is refilled with NaNs between
    replays: partials of an earlier call must never be read."""
    torch, mla, _, dev = env
    w = workloads.config_workload(cfg)
    q, kc, bt, sl = upload(torch, w, dev)
    P, ws_bytes = mla.mla_plan(w.batch, w.rows, w.h_kv)
    md = torch.empty((P, 8), dtype=torch.int32, device=dev)
    ns = torch.empty((w.batch + 1,), dtype=torch.int32, device=dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((w.batch, w.s_q, w.h_q, w.dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.s_q, w.h_q), dtype=torch.float32, device=dev)

    def step():
        mla.mla_get_metadata(sl, w.rows, w.h_kv, num_parts=P, out=(md, ns))
        mla.mla_decode_paged(q, kc, bt, sl, w.dv, md, ns, w.causal, w.scale, out, lse, ws)

    step()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(4):
        out.zero_()
        lse.fill_(7.0)
        ws.fill_(255)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}: out differs"
        assert torch.equal(lse, ref_lse), f"replay {r}: lse differs"
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
