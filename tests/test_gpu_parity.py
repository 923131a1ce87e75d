"""GPU parity: every stage of libmsa against the CPU oracle on identical
seeded inputs, through the C ABI (ctypes binding).  Stage-wise tests feed
the oracle and the library the same stored inputs; the chain tests run
pool -> route -> gather -> decode end to end."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import sparse_latent_memory_amd as msa
from parity_util import (TAU, check_decode, check_pool, check_scores, check_topk, check_topk_order, lse_bound,
                         np64, storage)
from sparse_latent_memory_amd import _lib, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
THETA = 1e6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    _lib.load()   # raises when libmsa.so is missing: no fallback exists


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _randn(gen, *shape, dtype=torch.float32, scale=1.0):
    return (torch.randn(*shape, generator=gen) * scale).to(dtype)


def _dev(x):
    return torch.as_tensor(x).to(DEV)


# ==========================================================================
# stage 1: pooling
# ==========================================================================

def _pool_check(k, v, kr, lens, P, dtype, what, theta=THETA):
    tok_off = synth.token_offsets(lens)
    pool_off = synth.row_offsets(lens, P)
    kv_g, kr_g = msa.pool_encode(_dev(k), _dev(v), _dev(kr), _dev(tok_off), _dev(pool_off), P, theta,
                                 int(pool_off[-1]))
    torch.cuda.synchronize()
    kv_r, kr_r, off_r = oracle.pool(np64(k), np64(v), np64(kr), tok_off, P, theta, "f64")
    assert np.array_equal(off_r, pool_off)
    check_pool(np64(kv_g[:, 0]), kv_r[:, 0], dtype, what + " K_bar")
    check_pool(np64(kv_g[:, 1]), kv_r[:, 1], dtype, what + " V_bar")
    check_pool(np64(kr_g), kr_r, dtype, what + " Kr_bar")


def test_pool_tiny_config_fp32():
    cfg = synth.config(1)
    _say("pool: 64 docs x 512 tokens fp32, pool 64")
    bank = synth.raw_bank(cfg)
    _pool_check(bank["k"], bank["v"], bank["kr"], bank["lens"], cfg.pool, torch.float32, "tiny")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("P", [1, 7, 64, 100])
def test_pool_ragged_documents(dtype, P):
    g = torch.Generator().manual_seed(1000 + P)
    lens = np.concatenate([[1, 2, P, P + 1, 2 * P - 1], torch.randint(1, 300, (20,), generator=g).numpy()])
    n = int(lens.sum())
    _say(f"pool: ragged {len(lens)} docs ({n} tokens), P={P}, {dtype}")
    _pool_check(_randn(g, n, 8, 128, dtype=dtype), _randn(g, n, 8, 128, dtype=dtype),
                _randn(g, n, 8, 128, dtype=dtype), lens, P, dtype, f"ragged P={P}")


def test_pool_small_heads_and_long_document():
    # one 70,000-token document: in-document positions far beyond one RoPE period
    g = torch.Generator().manual_seed(7)
    lens = np.array([70_000, 3, 1025])
    n = int(lens.sum())
    _say("pool: 70K-token document, Hkv=1, D=64, Hr=2, dr=64, P=1024, fp32")
    _pool_check(_randn(g, n, 1, 64), _randn(g, n, 1, 64), _randn(g, n, 2, 64), lens, 1024, torch.float32,
                "long doc", theta=1e4)


def test_pool_constant_chunk_and_zero_input_on_gpu():
    g = torch.Generator().manual_seed(3)
    lens = np.array([64, 64, 10])
    c = _randn(g, 1, 8, 128, dtype=torch.bfloat16)
    v = c.repeat(138, 1, 1)
    _say("pool: constant V/Kr chunks pool to themselves; zero K pools to zero")
    kv_g, kr_g = msa.pool_encode(_dev(torch.zeros(138, 8, 128, dtype=torch.bfloat16)), _dev(v), _dev(v),
                                 _dev(synth.token_offsets(lens)), _dev(synth.row_offsets(lens, 64)), 64, THETA, 3)
    torch.cuda.synchronize()
    assert torch.equal(kv_g[:, 1].cpu(), c.repeat(3, 1, 1))
    assert torch.equal(kr_g.cpu(), c.repeat(3, 1, 1))
    assert torch.count_nonzero(kv_g[:, 0]).item() == 0


def test_pool_routing_layer_config_sampled():
    """Full 2048-document bf16 bank (~1.3M tokens, lengths U[256,1024]);
    32 sampled documents checked against the oracle one by one."""
    cfg = synth.config(2)
    _say("pool: routing-layer bank, 2048 docs, bf16, sampled docs")
    bank = synth.raw_bank(cfg, device=DEV)
    lens = bank["lens"]
    pool_off = synth.row_offsets(lens, cfg.pool)
    kv_g, kr_g = msa.pool_encode(bank["k"], bank["v"], bank["kr"], bank["doc_tok_off"], _dev(pool_off),
                                 cfg.pool, cfg.rope_theta, int(pool_off[-1]))
    torch.cuda.synchronize()
    tok_off = synth.token_offsets(lens)
    rng = np.random.default_rng(2)
    for d in np.concatenate([[0, len(lens) - 1], rng.choice(len(lens), 30, replace=False)]):
        a, b = tok_off[d], tok_off[d + 1]
        kb, vb, rb = oracle.pool_doc(np64(bank["k"][a:b]), np64(bank["v"][a:b]), np64(bank["kr"][a:b]),
                                     cfg.pool, cfg.rope_theta, "f64")
        r0, r1 = pool_off[d], pool_off[d + 1]
        check_pool(np64(kv_g[r0:r1, 0]), kb, torch.bfloat16, f"doc {d} K_bar")
        check_pool(np64(kv_g[r0:r1, 1]), vb, torch.bfloat16, f"doc {d} V_bar")
        check_pool(np64(kr_g[r0:r1]), rb, torch.bfloat16, f"doc {d} Kr_bar")


def test_pool_into_pinned_host_tier():
    """Pooled K/V written straight into pinned host memory (the content
    tier) equal, bit for bit, the same call into device memory; a batch is
    written at its row offset inside a larger host tier."""
    cfg = synth.config(2, n_docs=96)
    bank = synth.raw_bank(cfg, device=DEV)
    lens = bank["lens"]
    off = _dev(synth.row_offsets(lens, cfg.pool))
    n_pool = int(synth.row_offsets(lens, cfg.pool)[-1])
    _say(f"pool: {len(lens)} docs into pinned host memory ({n_pool} rows)")
    kv_d, kr_d = msa.pool_encode(bank["k"], bank["v"], bank["kr"], bank["doc_tok_off"], off, cfg.pool,
                                 cfg.rope_theta, n_pool)
    tier = torch.zeros((n_pool + 50, 2, 8, 128), dtype=torch.bfloat16, pin_memory=True)
    kr_h = torch.zeros((n_pool, 8, 128), dtype=torch.bfloat16, pin_memory=True)
    msa.pool_encode(bank["k"], bank["v"], bank["kr"], bank["doc_tok_off"], off, cfg.pool, cfg.rope_theta,
                    n_pool, tier[50:], kr_h)
    torch.cuda.synchronize()
    assert torch.equal(tier[50:].view(torch.int16), kv_d.cpu().view(torch.int16))
    assert torch.equal(kr_h.view(torch.int16), kr_d.cpu().view(torch.int16))
    assert not tier[:50].view(torch.int16).any()
    pageable = torch.zeros(tuple(tier[50:].shape), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="not pinned"):
        msa.pool_encode(bank["k"], bank["v"], bank["kr"], bank["doc_tok_off"], off, cfg.pool, cfg.rope_theta,
                        n_pool, pageable, kr_h)
    # the library refuses pageable memory by itself too (straight through the C ABI)
    a = _lib.PoolArgs(dtype=_lib.MSA_BF16, n_docs=len(lens), n_tokens=bank["k"].shape[0], n_pool=n_pool,
                      pool_size=cfg.pool, n_kv_heads=8, head_dim=128, n_router_heads=8, router_dim=128,
                      rope_theta=cfg.rope_theta, doc_tok_off=_lib._ptr(bank["doc_tok_off"]),
                      doc_pool_off=_lib._ptr(off), k=_lib._ptr(bank["k"]), v=_lib._ptr(bank["v"]),
                      kr=_lib._ptr(bank["kr"]), kv_pooled=_lib._ptr(pageable), kr_pooled=_lib._ptr(kr_h))
    lib = _lib.load()
    assert lib.msa_pool_encode(ctypes.byref(a), _lib._stream(None)) == _lib.MSA_ERR_INVALID_ARG
    assert b"must be device memory" in lib.msa_last_error()
    torch.cuda.synchronize()
    assert not pageable.view(torch.int16).any()


def test_pool_tiled_router_bank_at_row_offsets():
    """Kr_bar written into a tiled bank at an unaligned first row equals the
    row-major output bit for bit, rows outside the call untouched; the bank
    encoded in two batches (each at its own first row) equals the one-call
    bank."""
    cfg = synth.config(2, n_docs=96)
    bank = synth.raw_bank(cfg, device=DEV)
    lens = bank["lens"]
    off_h = synth.row_offsets(lens, cfg.pool)
    n_pool = int(off_h[-1])
    _say(f"pool: tiled router bank, {len(lens)} docs, {n_pool} rows at row 5")
    kv_r, kr_r = msa.pool_encode(bank["k"], bank["v"], bank["kr"], bank["doc_tok_off"], _dev(off_h), cfg.pool,
                                 cfg.rope_theta, n_pool)
    base = 5
    sentinel = torch.full((msa.bank_rows(base + n_pool, "tiled"), 8, 128), -3.0, dtype=torch.bfloat16, device=DEV)
    kt = sentinel.clone()
    kv_t, _ = msa.pool_encode(bank["k"], bank["v"], bank["kr"], bank["doc_tok_off"], _dev(off_h), cfg.pool,
                              cfg.rope_theta, n_pool, kr_pooled=kt, kr_layout="tiled", kr_row_base=base)
    torch.cuda.synchronize()
    rows = synth.untile_router_bank(kt, kt.shape[0])
    assert torch.equal(rows[base:base + n_pool].view(torch.int16), kr_r.view(torch.int16))
    assert torch.equal(rows[:base].view(torch.int16), sentinel[:base].view(torch.int16))
    assert torch.equal(rows[base + n_pool:].view(torch.int16), sentinel[base + n_pool:].view(torch.int16))
    assert torch.equal(kv_t.view(torch.int16), kv_r.view(torch.int16))
    # two batches: documents [0, 37) and [37, 96), the second at the first's end
    whole = synth.tile_router_bank(kr_r, pad_value=-3.0)
    kt2 = torch.full_like(whole, -3.0)
    tok = synth.token_offsets(lens)
    d1 = 37
    for d0, d_end in [(0, d1), (d1, len(lens))]:
        t0, t1 = int(tok[d0]), int(tok[d_end])
        toff = _dev(tok[d0:d_end + 1] - tok[d0])
        poff = off_h[d0:d_end + 1] - off_h[d0]
        msa.pool_encode(bank["k"][t0:t1], bank["v"][t0:t1], bank["kr"][t0:t1], toff, _dev(poff), cfg.pool,
                        cfg.rope_theta, int(poff[-1]), kr_pooled=kt2, kr_layout="tiled", kr_row_base=int(off_h[d0]))
    torch.cuda.synchronize()
    assert int(off_h[d1]) % 16 != 0
    assert torch.equal(kt2.view(torch.int16), whole.view(torch.int16))


@pytest.mark.parametrize("hr,dr,host", [(2, 64, False), (1, 128, True), (16, 64, False)])
def test_pool_tiled_router_bank_shapes_and_pinned_output(hr, dr, host):
    """The tiled writer at other router shapes (2, 1 and 16 heads), and into
    pinned host memory: always the row-major output, permuted."""
    g = torch.Generator().manual_seed(40 + hr * dr)
    lens = np.concatenate([[1, 63, 64, 65], torch.randint(1, 400, (30,), generator=g).numpy()])
    n = int(lens.sum())
    P = 64
    pool_off = synth.row_offsets(lens, P)
    n_pool = int(pool_off[-1])
    k = _randn(g, n, 2, 64, dtype=torch.bfloat16).to(DEV)
    v = _randn(g, n, 2, 64, dtype=torch.bfloat16).to(DEV)
    kr = _randn(g, n, hr, dr, dtype=torch.bfloat16).to(DEV)
    _say(f"pool: tiled router bank Hr={hr} dr={dr}, {n_pool} rows at row 3, {'pinned host' if host else 'device'}")
    tok = _dev(synth.token_offsets(lens))
    _, kr_r = msa.pool_encode(k, v, kr, tok, _dev(pool_off), P, THETA, n_pool)
    shape = (msa.bank_rows(3 + n_pool, "tiled"), hr, dr)
    kt = torch.zeros(shape, dtype=torch.bfloat16, pin_memory=True) if host else \
        torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
    msa.pool_encode(k, v, kr, tok, _dev(pool_off), P, THETA, n_pool, kr_pooled=kt, kr_layout="tiled", kr_row_base=3)
    torch.cuda.synchronize()
    rows = synth.untile_router_bank(kt.to(DEV), kt.shape[0])
    assert torch.equal(rows[3:3 + n_pool].view(torch.int16), kr_r.view(torch.int16))
    assert not rows[:3].view(torch.int16).any() and not rows[3 + n_pool:].view(torch.int16).any()


# ==========================================================================
# stage 2: routing
# ==========================================================================

def _route_check(kr_pooled, pool_off, qr, k, what):
    idx, sc, dsc = msa.route(qr, kr_pooled, _dev(pool_off), k)
    torch.cuda.synchronize()
    ref = oracle.doc_scores(np64(qr), np64(kr_pooled), pool_off)
    check_scores(np64(dsc), ref, what)
    check_topk(np64(idx), ref, k, what)
    check_topk_order(np64(idx), np64(sc), what)
    assert np.array_equal(np64(sc), np.take_along_axis(np64(dsc), np64(idx), 1))
    return np64(idx), ref


def _ragged_bank(gen, n_docs, max_rows, hr, dr, dtype):
    rows = torch.randint(1, max_rows + 1, (n_docs,), generator=gen).numpy()
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    return _randn(gen, int(off[-1]), hr, dr, dtype=dtype).to(DEV), off


def test_route_tiny_config_fp32():
    cfg = synth.config(1)
    _say("route: tiny config, fp32, 16 query tokens, top-4")
    lens = synth.doc_lengths(cfg)
    off = synth.row_offsets(lens, cfg.pool)
    g = torch.Generator().manual_seed(11)
    kr = _randn(g, int(off[-1]), cfg.n_router_heads, cfg.router_dim).to(DEV)
    qr = synth.router_queries(cfg).to(DEV)
    _route_check(kr, off, qr, cfg.top_k, "tiny fp32")


@pytest.mark.parametrize("hr,dr", [(8, 128), (4, 64), (1, 128), (16, 64), (2, 128)])
@pytest.mark.parametrize("b,tq", [(1, 1), (8, 1), (2, 4), (3, 2), (1, 8)])
def test_route_matrix_core_path(hr, dr, b, tq):
    g = torch.Generator().manual_seed(hr * 100 + dr + b * 7 + tq)
    kr, off = _ragged_bank(g, 700, 5, hr, dr, torch.bfloat16)       # ~2100 rows, ragged last tile
    qr = _randn(g, b, tq, hr, dr, dtype=torch.bfloat16).to(DEV)
    _say(f"route: MFMA path Hr={hr} dr={dr} B={b} Tq={tq} rows={off[-1]}")
    _route_check(kr, off, qr, 16, f"mfma {hr}x{dr} B{b} Tq{tq}")


@pytest.mark.parametrize("b,tq", [(1, 16), (4, 3), (9, 1)])
def test_route_vector_path_fp32(b, tq):
    g = torch.Generator().manual_seed(b * 31 + tq)
    kr, off = _ragged_bank(g, 500, 4, 8, 128, torch.float32)
    qr = _randn(g, b, tq, 8, 128).to(DEV)
    _say(f"route: fp32 vector path B={b} Tq={tq}")
    _route_check(kr, off, qr, 8, f"valu B{b} Tq{tq}")


@pytest.mark.parametrize("hr,dr", [(8, 128), (4, 64), (16, 64), (1, 128), (8, 64), (2, 64)])
@pytest.mark.parametrize("b,tq", [(1, 16), (4, 3), (9, 1), (20, 1), (3, 40), (100, 1), (1, 256)])
def test_route_many_tokens_matrix_core_path(hr, dr, b, tq):
    """More than 8 query tokens: bf16 query M-tiles held in LDS, tokens of a
    query padded to whole tiles.  The shapes cover one and several chunks of
    resident tiles (4 or 8 per chunk, by head shape), chunks of whole
    queries, and one query cut into partial maxima over several chunks."""
    g = torch.Generator().manual_seed(hr * 1000 + dr + b * 7 + tq)
    kr, off = _ragged_bank(g, 600, 4, hr, dr, torch.bfloat16)
    qr = _randn(g, b, tq, hr, dr, dtype=torch.bfloat16).to(DEV)
    _say(f"route: wide MFMA path Hr={hr} dr={dr} B={b} Tq={tq} rows={off[-1]}")
    _route_check(kr, off, qr, 8, f"wide {hr}x{dr} B{b} Tq{tq}")


@pytest.mark.parametrize("b,tq", [(257, 64), (65, 256), (129, 256)])
def test_route_more_query_chunks_than_workgroups(b, tq):
    """More chunks of query tiles than workgroups (one per compute unit):
    each workgroup walks several chunks, restaging the query tiles between
    them; with 256 tokens every query is also cut into partial maxima (four
    chunks of four tiles per query: 260 and 516 chunks)."""
    g = torch.Generator().manual_seed(b + tq)
    kr, off = _ragged_bank(g, 100, 4, 8, 128, torch.bfloat16)
    qr = _randn(g, b, tq, 8, 128, dtype=torch.bfloat16).to(DEV)
    _say(f"route: wide MFMA path B={b} Tq={tq} rows={off[-1]}")
    _route_check(kr, off, qr, 8, f"wide chunks B{b} Tq{tq}")


@pytest.mark.parametrize("b,tq,n_docs", [(1, 256, 2460), (64, 1, 10240), (1, 256, 8200), (256, 1, 10240)])
def test_route_heads_outer_and_tile_loops_in_one_launch(b, tq, n_docs):
    """Workgroups that take the wide scan's loops differently, in one launch
    on a 256-CU device.  One 256-token query (four chunks of query tiles,
    64 workgroups per chunk) over 24,600 rows (193 groups of 8 tiles):
    workgroups 1..63 walk three groups (one heads-outer batch), workgroup 0
    four (batches of three and one); over 82,000 rows (641 groups) they walk
    10 or 11 groups in batches of three and a shorter last one.  64
    one-token queries (one chunk, 256 workgroups) over 102,400 rows (800
    groups): workgroups 0..31 walk four groups (the tile loop), the others
    three (heads outer).  256 one-token queries (four chunks, 64 workgroups
    per chunk) over the same rows: 12 or 13 groups per workgroup in
    heads-outer batches, each run's per-document maxima stored per chunk.
    Row-major and tiled banks identical, and checked against the oracle."""
    g = torch.Generator().manual_seed(4242 + b)
    rows = np.full(n_docs, 10, dtype=np.int64)
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    kr = _randn(g, int(off[-1]), 8, 128, dtype=torch.bfloat16).to(DEV)
    qr = _randn(g, b, tq, 8, 128, dtype=torch.bfloat16).to(DEV)
    _say(f"route: heads-outer and tile loops in one launch, {int(off[-1])} rows, B={b} Tq={tq}")
    idx, dsc = _route_both_layouts(qr, kr, off, 16, f"loop boundary B={b} Tq={tq}")
    ref = oracle.doc_scores(np64(qr), np64(kr), off)
    check_scores(np64(dsc), ref, f"loop boundary B={b} Tq={tq} vs oracle")
    check_topk(np64(idx), ref, 16, f"loop boundary B={b} Tq={tq} vs oracle")


def test_route_prefill_config_full_size():
    """Routing layer of a 4B-parameter backbone: 2048 documents (lengths
    U[256,1024], ~21.8K pooled rows), a 256-token query prefill, top-16;
    every document score checked against the oracle."""
    cfg = synth.config(2)
    lens = synth.doc_lengths(cfg)
    off = synth.row_offsets(lens, cfg.pool)
    _say(f"route: prefill routing, {len(lens)} docs, {off[-1]} rows, Tq=256")
    kr = synth.pooled_router_bank(cfg, lens, device=DEV)
    qr = synth.router_queries(cfg, device=DEV)
    _route_check(kr, off, qr, cfg.top_k, "prefill 256")


def test_route_interleave_batch_shape():
    """64 queries of one token against a ragged lognormal bank (the
    multi-hop workload's routing shape, smaller bank)."""
    cfg = synth.config(5, total_tokens=3_000_000)
    lens = synth.doc_lengths(cfg)
    off = synth.row_offsets(lens, cfg.pool)
    _say(f"route: 64 queries, {len(lens)} docs, {off[-1]} rows")
    kr = synth.pooled_router_bank(cfg, lens, device=DEV)
    qr = synth.router_queries(cfg, device=DEV)
    _route_check(kr, off, qr, cfg.top_k, "64 queries")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_route_ties_go_to_lower_document_id(dtype):
    g = torch.Generator().manual_seed(5)
    kr, off = _ragged_bank(g, 300, 3, 8, 128, dtype)
    hot = _randn(g, 1, 8, 128, dtype=dtype).to(DEV)
    twins = [17, 18, 90, 200, 299]
    for d in twins:                              # identical best rows: bit-identical scores
        kr[off[d]] = hot[0]
    qr = hot[None].clone()
    _say(f"route: exact ties across documents {twins}, {dtype}")
    idx, sc, dsc = msa.route(qr, kr, _dev(off), 8)
    torch.cuda.synchronize()
    idx = np64(idx)[0]
    assert idx[:5].tolist() == twins
    assert len(set(np64(sc)[0, :5].tolist())) == 1
    check_topk(idx[None], oracle.doc_scores(np64(qr), np64(kr), off), 8, "ties")


@pytest.mark.parametrize("b", [9, 17, 64])
@pytest.mark.parametrize("k", [1, 16, 64, 65, 300])
def test_route_document_path(b, k):
    """One-token batches (the scan reduces each tile per document itself):
    documents of 1 to 70 rows (runs within a tile, documents over many
    tiles), every selection branch (k up to 64 uses the block bound; 65 and
    all documents the radix select), checked against the oracle and, tiled
    with NaN in its padding rows, against the row-major bank bit for bit."""
    g = torch.Generator().manual_seed(3000 + b * 11 + k)
    rows = np.where(torch.rand(300, generator=g).numpy() < 0.2,
                    torch.randint(17, 71, (300,), generator=g).numpy(),
                    torch.randint(1, 5, (300,), generator=g).numpy())
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    kr = _randn(g, int(off[-1]), 8, 128, dtype=torch.bfloat16).to(DEV)
    qr = _randn(g, b, 1, 8, 128, dtype=torch.bfloat16).to(DEV)
    _say(f"route: document path B={b} k={k}, 300 docs, {off[-1]} rows")
    _route_check(kr, off, qr, k, f"docs B{b} k{k}")
    _route_both_layouts(qr, kr, off, k, f"docs tiled B{b} k{k}")


def test_route_document_path_ties_and_whole_tiles():
    """Exact ties between documents on the document path, and a bank whose
    documents are 16-row multiples (every tile starts a document or
    continues one whole)."""
    g = torch.Generator().manual_seed(8)
    rows = np.array([16, 32, 16, 48, 16] * 20)
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    kr = _randn(g, int(off[-1]), 8, 128, dtype=torch.bfloat16).to(DEV)
    hot = _randn(g, 1, 8, 128, dtype=torch.bfloat16).to(DEV)
    twins = [3, 4, 41, 77, 99]
    for d in twins:
        kr[int(off[d + 1]) - 1] = hot[0]         # the last row of each twin
    qr = hot[None].repeat(12, 1, 1, 1).clone()
    _say("route: document path, ties, 16-row documents, B=12")
    idx, _ = _route_check(kr, off, qr, 8, "docs ties")
    assert all(idx[b, :5].tolist() == twins for b in range(12))


def _doc_map_reference(off):
    """The document map written out from its definition: per 16-row tile,
    the document holding the tile's first row, and bit r set where row
    16 t + r starts a document or is row n_pool."""
    off = np.asarray(off, dtype=np.int64)
    n_pool = int(off[-1])
    n_tiles = (n_pool + 15) // 16
    starts = set(off[:-1].tolist()) | {n_pool}
    doc = np.searchsorted(off, 16 * np.arange(n_tiles), side="right") - 1
    bits = np.array([sum(1 << r for r in range(16) if 16 * t + r in starts) for t in range(n_tiles)],
                    dtype=np.uint32)
    return doc.astype(np.int32), bits


@pytest.mark.parametrize("seed", [0, 1])
def test_doc_map_matches_its_definition(seed):
    """msa_doc_map, bit for bit against the map written out in Python: 400
    documents of 1 to 70 rows (many starts in one tile, documents spanning
    many tiles) and a bank that ends inside its last tile."""
    g = torch.Generator().manual_seed(70 + seed)
    rows = np.where(torch.rand(400, generator=g).numpy() < 0.3,
                    torch.randint(17, 71, (400,), generator=g).numpy(),
                    torch.randint(1, 4, (400,), generator=g).numpy())
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    n_pool = int(off[-1])
    _say(f"doc map: 400 documents, {n_pool} rows")
    m = msa.doc_map(_dev(off), n_pool)
    torch.cuda.synchronize()
    n_tiles = (n_pool + 15) // 16
    raw = m.cpu().numpy()
    doc = raw[:4 * n_tiles].view(np.int32)
    bits_at = (4 * n_tiles + 255) // 256 * 256
    bits = raw[bits_at:bits_at + 4 * n_tiles].view(np.uint32)
    want_doc, want_bits = _doc_map_reference(off)
    assert np.array_equal(doc, want_doc)
    assert np.array_equal(bits, want_bits)


@pytest.mark.parametrize("b", [1, 8, 17, 64])
@pytest.mark.parametrize("lay", ["rows", "tiled"])
def test_route_with_a_prebuilt_doc_map_is_identical(b, lay):
    """Routing with the document map built once by msa_doc_map gives the
    results of routing that builds it per call, bit for bit (narrow and
    wide scans, both bank layouts), over repeated calls and fresh queries."""
    g = torch.Generator().manual_seed(500 + b)
    rows = torch.randint(1, 40, (600,), generator=g).numpy()
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    n_pool = int(off[-1])
    kr = _randn(g, n_pool, 8, 128, dtype=torch.bfloat16).to(DEV)
    bank = synth.tile_router_bank(kr) if lay == "tiled" else kr
    offd = _dev(off)
    m = msa.doc_map(offd, n_pool)
    _say(f"route with a prebuilt document map: B={b}, {lay} bank, {n_pool} rows")
    for rep in range(2):
        qr = _randn(g, b, 1, 8, 128, dtype=torch.bfloat16).to(DEV)
        i0, s0, d0 = msa.route(qr, bank, offd, 16, kr_layout=lay, n_pool=n_pool)
        i1, s1, d1 = msa.route(qr, bank, offd, 16, kr_layout=lay, n_pool=n_pool, doc_map=m)
        torch.cuda.synchronize()
        assert torch.equal(d0.view(torch.int32), d1.view(torch.int32)), f"rep {rep}: document scores differ"
        assert torch.equal(i0, i1) and torch.equal(s0.view(torch.int32), s1.view(torch.int32))
    ref = oracle.doc_scores(np64(qr), np64(kr), off)
    check_scores(np64(d1), ref, "prebuilt doc map")
    check_topk(np64(i1), ref, 16, "prebuilt doc map")


def test_route_top_k_bound_when_block_maxima_tie():
    """250,000 one-row documents (977 blocks of 256): 300 blocks share one
    tied maximum and the 16 blocks above it all sit in the same lane of the
    bound's search (blocks 0, 64, ..., 960), so more than 128 block maxima
    reach the lane bound and the selection takes its every-list search; the
    winners are exactly the 16 planted documents, in score order."""
    g = torch.Generator().manual_seed(41)
    n_docs = 250_000
    off = np.arange(n_docs + 1, dtype=np.int64)
    kr = torch.randn(n_docs, 1, 128, generator=g)
    q = torch.randn(128, generator=g)
    u = torch.randn(128, generator=g)
    qh = q / q.norm()
    u = u - (u @ qh) * qh
    uh = u / u.norm()
    row = lambda c: c * qh + (1 - c * c) ** 0.5 * uh  # noqa: E731  (cosine c with q)
    tied = [b for b in range(977) if b % 64 != 0][:300]
    for b in tied:
        kr[256 * b + 5, 0] = row(0.6)
    high = [256 * 64 * j + 7 for j in range(16)]
    for j, d in enumerate(high):
        kr[d, 0] = row(0.7 + 0.01 * j)
    kr = kr.to(torch.bfloat16).to(DEV)
    qr = q.reshape(1, 1, 1, 128).to(torch.bfloat16).to(DEV)
    _say("route: 250,000 documents, 300 tied block maxima under 16 in one lane")
    idx, ref = _route_check(kr, off, qr, 16, "tied block maxima")
    assert idx[0].tolist() == high[::-1]
    _route_both_layouts(qr, kr, off, 16, "tied block maxima, tiled")


@pytest.mark.parametrize("k", [16, 4096])
def test_route_top_k_over_more_than_4096_blocks(k):
    """1,100,000 one-row documents (4,297 blocks of 256, more than the block
    bound orders): the selection takes its radix select over every document
    key, at k = 16 and at the largest k the library takes (4,096), and with
    the device-side assembly at that k the copy plan drops every rank from the
    first document that no longer fits (capacity 3,000 rows); scores, top-k,
    order and the gathered memory against the oracle."""
    g = torch.Generator().manual_seed(4100 + k)
    n_docs, cap = 1_100_000, 3000
    off = np.arange(n_docs + 1, dtype=np.int64)
    kr = torch.randn(n_docs, 1, 128, generator=g).to(torch.bfloat16).to(DEV)
    qr = torch.randn(2, 1, 1, 128, generator=g).to(torch.bfloat16).to(DEV)
    host_kv = torch.randn(n_docs, 2, 1, 64, generator=g).to(torch.bfloat16).pin_memory()
    _say(f"route: {n_docs} one-row documents, top-{k}, radix selection, assembly cap {cap}")
    idx, ref = _route_check(kr, off, qr, k, f"{n_docs} documents, top-{k}")
    asm = msa.Assembly.allocate(host_kv, torch.as_tensor(off), 2, k, cap, DEV, mode="kernel")
    idx_a, _, _ = msa.route(qr, kr, _dev(off), k, assembly=asm)
    torch.cuda.synchronize()
    assert np.array_equal(np64(idx_a), idx)
    src = host_kv.view(torch.int16).numpy()
    ref_mem, ref_len, ref_taken = oracle.assemble(src, off, idx, cap)
    assert np.array_equal(np64(asm.mem_len), ref_len)
    assert ref_taken.tolist() == [min(k, cap)] * 2
    got = asm.mem_kv.view(torch.int16).cpu().numpy()
    for b in range(2):
        assert np.array_equal(got[b, :ref_len[b]], ref_mem[b, :ref_len[b]]), f"memory of query {b}"
    _route_both_layouts(qr, kr, off, k, f"{n_docs} documents, top-{k}, tiled")


def test_route_all_documents_and_degenerate_rows():
    g = torch.Generator().manual_seed(6)
    kr, off = _ragged_bank(g, 37, 3, 8, 128, torch.bfloat16)
    kr[off[4]:off[5]] = 0                        # a document of zero vectors scores exactly 0
    qr = _randn(g, 2, 1, 8, 128, dtype=torch.bfloat16).to(DEV)
    _say("route: k = n_docs (a permutation), a zero-vector document")
    idx, ref = _route_check(kr, off, qr, 37, "k=all")
    for row in idx:
        assert sorted(row.tolist()) == list(range(37))
    dsc = msa.route(qr, kr, _dev(off), 1)[2]
    assert np64(dsc)[:, 4].tolist() == [0.0, 0.0]


def test_route_single_document_bank():
    g = torch.Generator().manual_seed(8)
    kr, off = _ragged_bank(g, 1, 1, 8, 128, torch.bfloat16)
    qr = _randn(g, 1, 1, 8, 128, dtype=torch.bfloat16).to(DEV)
    _say("route: one document with one row")
    idx, ref = _route_check(kr, off, qr, 1, "single")
    assert idx.tolist() == [[0]]


def test_route_needle_bank_full_size():
    """16M-token bank (32768 lognormal docs, ~276K pooled rows, bf16), 8
    queries of one token; each planted needle (cosine 0.6) is in its top-16
    and every document score matches the oracle."""
    cfg = synth.config(3)
    lens = synth.doc_lengths(cfg)
    off = synth.row_offsets(lens, cfg.pool)
    _say(f"route: needle bank, {len(lens)} docs, {off[-1]} rows, B=8")
    kr = synth.pooled_router_bank(cfg, lens, device=DEV)
    qr = synth.router_queries(cfg, device=DEV)
    needles = synth.plant_needles(cfg, qr, kr, off)
    idx, sc, dsc = msa.route(qr, kr, _dev(off), cfg.top_k)
    torch.cuda.synchronize()
    idx = np64(idx)
    for b, d in enumerate(needles):
        assert d in idx[b].tolist(), f"needle {d} missing for query {b}"
        assert idx[b, 0] == d
    qn = np64(qr)
    ref = np.empty((cfg.batch, len(lens)))
    step = 4096
    for d0 in range(0, len(lens), step):
        d1 = min(d0 + step, len(lens))
        ref[:, d0:d1] = oracle.doc_scores(qn, np64(kr[off[d0]:off[d1]]), off[d0:d1 + 1] - off[d0])
    check_scores(np64(dsc), ref, "needle bank")
    check_topk(idx, ref, cfg.top_k, "needle bank")
    assert np.all(np.abs(ref[np.arange(cfg.batch), needles] - 0.6) < 5e-3)


def _oracle_doc_scores(qr, kr, off, block_docs=2048):
    """The oracle's score of every document of a bank held on the GPU,
    computed block by block (documents never straddle a block)."""
    qn = np64(qr)
    n_docs = len(off) - 1
    ref = np.empty((qn.shape[0], n_docs))
    for d0 in range(0, n_docs, block_docs):
        d1 = min(d0 + block_docs, n_docs)
        ref[:, d0:d1] = oracle.doc_scores(qn, np64(kr[off[d0]:off[d1]]), off[d0:d1 + 1] - off[d0])
    return ref


def _bf16_bits_to_f64(bits):
    """int16 bit patterns of bf16 values (numpy) -> float64."""
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).double().numpy()


@pytest.mark.slow
def test_route_decode_100m_bank_whole_bank_against_oracle():
    """The 100M-token step at full size, called as the benchmark times it:
    195,313 documents x 512 tokens (1,562,504 pooled rows, 3.2 GB bf16) in
    the tiled layout with its document map built once, one query token,
    top-16 with the device-side gather from the 6.4 GB pinned host tier,
    then decode GQA 32/8 x 128 over 128 memory rows + 4096 local tokens.
    For two steps' queries: all 195,313 document scores against the oracle,
    the top-k by the full-bank rule, the memory byte for byte, and the
    decode output on it.  The row-major bank routed alone gives the same
    results bit for bit."""
    cfg = synth.config(4)
    lens = synth.doc_lengths(cfg)
    off = synth.row_offsets(lens, cfg.pool)
    n_pool = int(off[-1])
    _say(f"route+decode: 100M-token bank, {len(lens)} docs, {n_pool} rows, whole bank vs oracle")
    kr = synth.pooled_router_bank(cfg, lens, device=DEV)
    kt = synth.tile_router_bank(kr)
    off_d = _dev(off)
    dmap = msa.doc_map(off_d, n_pool)
    host_kv = synth.pooled_content_bank(cfg, lens, device=DEV, pin=True)
    k = cfg.top_k
    mem_cap = k * (512 // cfg.pool)
    asm = msa.Assembly.allocate(host_kv, torch.as_tensor(off), cfg.batch, k, mem_cap, DEV)
    lk, lv = synth.local_context(cfg, device=DEV)
    loc_len = np.full(cfg.batch, cfg.local_len, dtype=np.int32)
    pos = np.full(cfg.batch, k, dtype=np.int32)
    src = host_kv.view(torch.int16).numpy()
    for step in (0, 1):
        qr = synth.router_queries(cfg, step=step, device=DEV)
        q = synth.decode_queries(cfg, step=step, device=DEV)
        idx, sc, dsc = msa.route(qr, kt, off_d, k, assembly=asm, kr_layout="tiled", n_pool=n_pool, doc_map=dmap)
        out, _ = msa.sparse_decode(q, asm.mem_kv, asm.mem_len, lk, lv, _dev(loc_len), _dev(pos), cfg.rope_theta)
        idx_r, sc_r, dsc_r = msa.route(qr, kr, off_d, k)
        torch.cuda.synchronize()
        assert torch.equal(dsc.view(torch.int32), dsc_r.view(torch.int32)), "tiled and row-major scores differ"
        assert torch.equal(idx, idx_r), "tiled and row-major top-k differ"
        _say(f"  step {step}: oracle scores of {len(lens)} documents")
        ref = _oracle_doc_scores(qr, kr, off)
        check_scores(np64(dsc), ref, f"100M step {step} scores")
        check_topk(np64(idx), ref, k, f"100M step {step} top-k")
        check_topk_order(np64(idx), np64(sc), f"100M step {step} order")
        mem_r, mlen_r, _ = oracle.assemble(src, off, np64(idx), mem_cap)
        assert np.array_equal(np64(asm.mem_len), mlen_r), f"100M step {step} memory length"
        got = asm.mem_kv.view(torch.int16).cpu().numpy()
        assert np.array_equal(got[0, :mlen_r[0]], mem_r[0, :mlen_r[0]]), f"100M step {step} memory bytes"
        ro, _ = oracle.decode(np64(q), _bf16_bits_to_f64(mem_r), mlen_r, np64(lk), np64(lv), loc_len, pos,
                              cfg.rope_theta, None, "bf16")
        check_decode(np64(out), ro, torch.bfloat16, f"100M step {step} decode")


def _route_both_layouts(qr, kr, off, k, what, pad_value=float("nan")):
    """Route the row-major bank and its tiled copy (padding rows hold
    pad_value): every output must be identical, bit for bit."""
    n_pool = int(off[-1])
    kt = synth.tile_router_bank(kr, pad_value=pad_value)
    assert kt.shape[0] == msa.bank_rows(n_pool, "tiled")
    idx_r, sc_r, dsc_r = msa.route(qr, kr, _dev(off), k)
    idx_t, sc_t, dsc_t = msa.route(qr, kt, _dev(off), k, kr_layout="tiled", n_pool=n_pool)
    torch.cuda.synchronize()
    assert torch.equal(dsc_t.view(torch.int32), dsc_r.view(torch.int32)), f"{what}: doc scores differ"
    assert torch.equal(idx_t, idx_r), f"{what}: top-k differs"
    assert torch.equal(sc_t.view(torch.int32), sc_r.view(torch.int32)), f"{what}: top-k scores differ"
    return idx_t, dsc_t


@pytest.mark.parametrize("hr,dr", [(8, 128), (4, 64), (1, 128), (16, 64), (2, 64)])
@pytest.mark.parametrize("b,tq", [(1, 1), (3, 2), (8, 1), (16, 1), (2, 100), (1, 200)])
def test_route_tiled_bank_matches_row_major(hr, dr, b, tq):
    """The tiled router bank gives the row-major bank's results bit for bit
    (narrow and wide scans), with NaN in the padding rows of its last tile;
    one case is also checked against the oracle."""
    g = torch.Generator().manual_seed(900 + hr * dr + b * 7 + tq)
    kr, off = _ragged_bank(g, 301, 17, hr, dr, torch.bfloat16)
    qr = _randn(g, b, tq, hr, dr, dtype=torch.bfloat16).to(DEV)
    _say(f"route: tiled bank, Hr={hr} dr={dr} B={b} Tq={tq}, {int(off[-1])} rows")
    idx, dsc = _route_both_layouts(qr, kr, off, 16, f"tiled Hr={hr} dr={dr} B={b} Tq={tq}")
    if hr == 8 and b * tq in (1, 200):
        ref = oracle.doc_scores(np64(qr), np64(kr), off)
        check_scores(np64(dsc), ref, "tiled vs oracle")
        check_topk(np64(idx), ref, 16, "tiled vs oracle")


@pytest.mark.parametrize("b,tq", [(1, 256), (1, 1)])
def test_route_tiled_bank_ragged_tail_sizes(b, tq):
    """Banks of 1..33 rows (a partial last tile of every size) and a bank
    whose last tile is whole."""
    g = torch.Generator().manual_seed(77 + tq)
    for n_rows in [1, 2, 15, 16, 17, 31, 33]:
        rows = np.ones(n_rows, dtype=np.int64)
        off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
        kr = _randn(g, n_rows, 8, 128, dtype=torch.bfloat16).to(DEV)
        qr = _randn(g, b, tq, 8, 128, dtype=torch.bfloat16).to(DEV)
        _route_both_layouts(qr, kr, off, min(4, n_rows), f"{n_rows} rows, B={b} Tq={tq}")


def test_route_tiled_needle_bank_full_size():
    """The 16.8M-token needle bank (275K rows) tiled: identical to the
    row-major results, and every needle is selected."""
    cfg = synth.config(3)
    lens = synth.doc_lengths(cfg)
    off = synth.row_offsets(lens, cfg.pool)
    kr = synth.pooled_router_bank(cfg, lens, device=DEV)
    qr = synth.router_queries(cfg, device=DEV)
    needles = synth.plant_needles(cfg, qr, kr, off)
    _say(f"route: tiled needle bank, {off[-1]} rows, B={cfg.batch}")
    idx, _ = _route_both_layouts(qr, kr, off, cfg.top_k, "tiled needle bank")
    idx = np64(idx)
    assert all(needles[b] in idx[b] for b in range(cfg.batch))


# ==========================================================================
# stage 3: decode
# ==========================================================================

def _decode_check(b, hq, hkv, d, mem_cap, loc_cap, mem_len, loc_len, pos, dtype, what, mem_scale=1.0, seed=0,
                  theta=THETA):
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, b, hq, d, dtype=dtype)
    mem = None
    if mem_cap:
        mem = torch.randn(b, mem_cap, 2, hkv, d, generator=g)
        mem[:, :, 0] *= mem_scale
        mem = mem.to(dtype)
    lk = _randn(g, b, loc_cap, hkv, d, dtype=dtype)
    lv = _randn(g, b, loc_cap, hkv, d, dtype=dtype)
    i32 = lambda x: torch.as_tensor(np.asarray(x, dtype=np.int32)).to(DEV)  # noqa: E731
    out, lse = msa.sparse_decode(_dev(q), None if mem is None else _dev(mem), i32(mem_len), _dev(lk), _dev(lv),
                                 i32(loc_len), i32(pos), theta)
    torch.cuda.synchronize()
    mem_np = np64(mem) if mem is not None else np.zeros((b, 0, 2, hkv, d))
    ro, rl = oracle.decode(np64(q), mem_np, mem_len, np64(lk), np64(lv), loc_len, pos, theta, None, storage(dtype))
    check_decode(np64(out), ro, dtype, what)
    gl = np64(lse)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(gl), fin)
    bound = lse_bound(np64(q), mem_np[:, :, 0], mem_len, np64(lk), loc_len, dtype)
    assert np.all(np.abs(gl[fin] - rl[fin]) <= bound[fin]), what
    return np64(out), gl


def test_decode_tiny_config_fp32():
    _say("decode: 8/2 x 64 fp32, memory 32 rows, local 128")
    _decode_check(1, 8, 2, 64, 32, 128, [32], [128], [4], torch.float32, "tiny")


@pytest.mark.parametrize("mem_scale", [1.0, 8.0])
def test_decode_100m_config_shape_bf16(mem_scale):
    _say(f"decode: 32/8 x 128 bf16, memory 128 rows (K x{mem_scale}), local 4096")
    _decode_check(1, 32, 8, 128, 128, 4096, [128], [4096], [16], torch.bfloat16, "100M shape",
                  mem_scale=mem_scale, seed=int(mem_scale))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_ragged_batch(dtype):
    _say(f"decode: batch of 5 with ragged lengths, {dtype}")
    _decode_check(5, 32, 8, 128, 200, 300, [0, 5, 128, 77, 200], [1, 64, 65, 300, 0], [0, 3, 16, 1000, 7],
                  dtype, "ragged", mem_scale=8.0, seed=3)


def test_decode_head_dim_64_and_group_8():
    _say("decode: D=64, 8 query heads per KV head, bf16")
    _decode_check(2, 16, 2, 64, 64, 130, [64, 10], [130, 1], [16, 5], torch.bfloat16, "d64 g8", mem_scale=4.0)


def test_decode_empty_contexts():
    _say("decode: no keys at all, and memory only")
    out, lse = _decode_check(2, 8, 2, 64, 16, 8, [0, 16], [0, 0], [0, 4], torch.float32, "empty")
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    _say("decode: no memory buffer (capacity 0)")
    _decode_check(1, 8, 2, 64, 0, 70, [0], [70], [3], torch.float32, "no memory")


def test_decode_large_position_offset():
    _say("decode: position offset 1e6 (RoPE angle reduction)")
    _decode_check(1, 8, 2, 128, 8, 100, [8], [100], [1_000_000], torch.float32, "big offset", mem_scale=4.0)


def test_decode_local_only_is_offset_invariant():
    g = torch.Generator().manual_seed(9)
    q = _randn(g, 1, 32, 128, dtype=torch.bfloat16).to(DEV)
    lk = _randn(g, 1, 500, 8, 128, dtype=torch.bfloat16).to(DEV)
    lv = _randn(g, 1, 500, 8, 128, dtype=torch.bfloat16).to(DEV)
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=DEV)  # noqa: E731
    _say("decode: empty memory, offsets 0 and 12345 agree")
    a, _ = msa.sparse_decode(q, None, i32([0]), lk, lv, i32([500]), i32([0]), THETA)
    b, _ = msa.sparse_decode(q, None, i32([0]), lk, lv, i32([500]), i32([12345]), THETA)
    torch.cuda.synchronize()
    check_decode(np64(a), np64(b), torch.bfloat16, "offset invariance")


# ==========================================================================
# stage 3 for a block of query tokens (prefill through the sparse context)
# ==========================================================================

def _attend_check(b, tq, hq, hkv, d, mem_cap, loc_cap, mem_len, loc_len, pos, what, mem_scale=1.0, seed=0,
                  theta=THETA):
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, b, tq, hq, d, dtype=torch.bfloat16)
    mem = None
    if mem_cap:
        mem = torch.randn(b, mem_cap, 2, hkv, d, generator=g)
        mem[:, :, 0] *= mem_scale
        mem = mem.to(torch.bfloat16)
    lk = _randn(g, b, loc_cap, hkv, d, dtype=torch.bfloat16)
    lv = _randn(g, b, loc_cap, hkv, d, dtype=torch.bfloat16)
    i32 = lambda x: torch.as_tensor(np.asarray(x, dtype=np.int32)).to(DEV)  # noqa: E731
    out, lse = msa.sparse_attend(_dev(q), None if mem is None else _dev(mem), i32(mem_len), _dev(lk), _dev(lv),
                                 i32(loc_len), i32(pos), theta)
    torch.cuda.synchronize()
    mem_np = np64(mem) if mem is not None else np.zeros((b, 0, 2, hkv, d))
    ro, rl = oracle.attend(np64(q), mem_np, mem_len, np64(lk), np64(lv), loc_len, pos, theta, None, "bf16")
    check_decode(np64(out).reshape(b * tq, hq, d), ro.reshape(b * tq, hq, d), torch.bfloat16, what)
    gl = np64(lse)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(gl), fin), what
    assert np.all(np.abs(gl[fin] - rl[fin]) <= 2e-2), f"{what}: lse off by {np.abs(gl[fin] - rl[fin]).max():.3g}"
    return np64(out), gl, q, mem, lk, lv


@pytest.mark.parametrize("mem_scale", [1.0, 8.0])
def test_attend_one_token_at_the_100m_decode_shape(mem_scale):
    """One query token: the decode step over 128 memory rows and 4096 local
    tokens, checked against the oracle (and so against msa_sparse_decode's
    definition)."""
    _say(f"attend: Tq=1, 32/8 x 128, memory 128 rows (K x{mem_scale}), local 4096")
    _attend_check(1, 1, 32, 8, 128, 128, 4096, [128], [4096], [16], "attend decode shape", mem_scale=mem_scale,
                  seed=int(mem_scale))


def test_attend_prefill_routing_layer_shape():
    """256 prefill tokens (the last 256 of 2048 local tokens) over ~170
    memory rows, GQA 32/8 x 128: 64 query tiles per KV head, causal."""
    _say("attend: Tq=256 prefill, 32/8 x 128, memory 170 rows, local 2048")
    _attend_check(1, 256, 32, 8, 128, 256, 2048, [170], [2048], [16], "prefill", mem_scale=8.0, seed=5)


@pytest.mark.parametrize("tq,t_loc", [(2048, 2048), (1000, 1500)])
def test_attend_long_prefill_blocks(tq, t_loc):
    """Long prefill blocks: every local token a query token (2,048 tokens,
    512 query tiles per KV head) and 1,000 of 1,500; causal over the whole
    block, ~170 memory rows, GQA 32/8 x 128, against the oracle."""
    _say(f"attend: Tq={tq} prefill over local {t_loc}, 32/8 x 128, memory 170 rows")
    _attend_check(1, tq, 32, 8, 128, 256, t_loc, [170], [t_loc], [16], f"prefill Tq={tq}", mem_scale=4.0,
                  seed=tq)


def test_attend_interleave_batch_shape():
    _say("attend: 64 queries x 1 token, memory 600 rows, local 1024")
    _attend_check(64, 1, 32, 8, 128, 700, 1024, list(range(540, 604)), [1024] * 64, [8] * 64, "batch 64",
                  mem_scale=4.0, seed=6)


@pytest.mark.parametrize("hq,hkv,d,tq", [(32, 8, 128, 5), (16, 2, 64, 7), (16, 1, 64, 3), (8, 8, 128, 20),
                                         (4, 2, 64, 33), (32, 8, 128, 13), (32, 4, 128, 9), (32, 8, 128, 40),
                                         (16, 4, 64, 40), (8, 2, 64, 70), (32, 8, 128, 70), (32, 8, 128, 67),
                                         (32, 4, 128, 35)])
def test_attend_ragged_batch_and_head_shapes(hq, hkv, d, tq):
    """Ragged memory and local lengths (one query with fewer local tokens
    than query tokens, one without memory), groups of 1 to 16 query heads,
    head dims 64 and 128, token counts that leave a partial last tile."""
    _say(f"attend: ragged batch of 4, Hq={hq} Hkv={hkv} D={d} Tq={tq}")
    _attend_check(4, tq, hq, hkv, d, 150, 300, [0, 37, 150, 64], [300, tq, 2, 129], [0, 9, 1000, 16],
                  f"ragged {hq}/{hkv}x{d} Tq{tq}", mem_scale=4.0, seed=hq + d + tq)


def test_attend_empty_contexts_and_large_offset():
    _say("attend: no keys at all / memory only / offset 1e6")
    out, lse, *_ = _attend_check(3, 2, 8, 2, 128, 16, 8, [0, 16, 5], [0, 0, 8], [0, 4, 1_000_000],
                                 "empty and offset", mem_scale=4.0)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    _say("attend: no memory buffer (capacity 0)")
    _attend_check(1, 3, 8, 2, 64, 0, 70, [0], [70], [3], "no memory")


def test_attend_is_causal_on_the_gpu():
    """Changing the last local token (the last query token's own key and
    value) leaves every earlier query token's output bit for bit."""
    g = torch.Generator().manual_seed(12)
    tq, t = 6, 200
    q = _randn(g, 1, tq, 32, 128, dtype=torch.bfloat16).to(DEV)
    mem = _randn(g, 1, 40, 2, 8, 128, dtype=torch.bfloat16).to(DEV)
    lk = _randn(g, 1, t, 8, 128, dtype=torch.bfloat16).to(DEV)
    lv = _randn(g, 1, t, 8, 128, dtype=torch.bfloat16).to(DEV)
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=DEV)  # noqa: E731
    _say("attend: causality, last local token perturbed")
    a, _ = msa.sparse_attend(q, mem, i32([40]), lk, lv, i32([t]), i32([16]), THETA)
    lk2, lv2 = lk.clone(), lv.clone()
    lk2[0, -1] += 1.0
    lv2[0, -1] -= 1.0
    b, _ = msa.sparse_attend(q, mem, i32([40]), lk2, lv2, i32([t]), i32([16]), THETA)
    torch.cuda.synchronize()
    assert torch.equal(a[0, :tq - 1], b[0, :tq - 1])
    assert not torch.equal(a[0, tq - 1], b[0, tq - 1])


# ==========================================================================
# context assembly (gather)
# ==========================================================================

def _bank_with_host_tier(gen, n_docs, max_rows, hkv, d, dtype):
    rows = torch.randint(1, max_rows + 1, (n_docs,), generator=gen).numpy()
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    host_kv = _randn(gen, int(off[-1]), 2, hkv, d, dtype=dtype).pin_memory()
    kr = _randn(gen, int(off[-1]), 8, 128, dtype=torch.bfloat16).to(DEV)
    return off, host_kv, kr


@pytest.mark.parametrize("mode", ["kernel", "copies"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gather_is_byte_exact_in_rank_order(dtype, mode):
    g = torch.Generator().manual_seed(21)
    off, host_kv, kr = _bank_with_host_tier(g, 400, 9, 8, 128, dtype)
    qr = _randn(g, 3, 1, 8, 128, dtype=torch.bfloat16).to(DEV)
    k, cap = 12, 40
    asm = msa.Assembly.allocate(host_kv, torch.as_tensor(off), 3, k, cap, DEV, copy_stream=torch.cuda.Stream(),
                                mode=mode)
    _say(f"gather ({mode}): 3 queries, top-{k}, cap {cap} rows, {dtype}")
    idx, _, _ = msa.route(qr, kr, _dev(off), k, assembly=asm)
    torch.cuda.synchronize()
    idx = np64(idx)
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    src = host_kv.view(bits).numpy()
    ref_mem, ref_len, ref_taken = oracle.assemble(src, off, idx, cap)
    got = asm.mem_kv.view(bits).cpu().numpy()
    assert np.array_equal(np64(asm.mem_len), ref_len)
    if mode == "copies":
        assert np.array_equal(asm.host_topk_idx.numpy(), idx)
        assert np.array_equal(asm.host_mem_len.numpy(), ref_len)
        assert np.array_equal(asm.host_mem_docs.numpy(), ref_taken)
    for b in range(3):
        assert np.array_equal(got[b, :ref_len[b]], ref_mem[b, :ref_len[b]])
    assert ref_taken.min() < k, "the capacity should force a drop in this case"
    assert np.array_equal(ref_len, [int(off[idx[b, :ref_taken[b]] + 1].sum() - off[idx[b, :ref_taken[b]]].sum())
                                    for b in range(3)])


@pytest.mark.parametrize("mode", ["kernel", "copies"])
def test_route_call_matches_route(mode):
    """RouteCall (every argument but the query bound once) gives route()'s
    results bit for bit - scores, top-k and the gathered memory - with the
    tiled bank, its document map and the assembly, for two queries in a
    row; a query of another shape is refused before any launch."""
    g = torch.Generator().manual_seed(23)
    off, host_kv, kr = _bank_with_host_tier(g, 400, 9, 8, 128, torch.bfloat16)
    n_pool = int(off[-1])
    kt = synth.tile_router_bank(kr)
    off_d = _dev(off)
    dmap = msa.doc_map(off_d, n_pool)
    k, cap = 12, 40
    kw = dict(kr_layout="tiled", n_pool=n_pool, doc_map=dmap)
    asm_a = msa.Assembly.allocate(host_kv, torch.as_tensor(off), 3, k, cap, DEV, copy_stream=torch.cuda.Stream(),
                                  mode=mode)
    asm_b = msa.Assembly.allocate(host_kv, torch.as_tensor(off), 3, k, cap, DEV, copy_stream=torch.cuda.Stream(),
                                  mode=mode)
    call = msa.RouteCall((3, 1, 8, 128), torch.bfloat16, kt, off_d, k, assembly=asm_b, **kw)
    _say(f"route call ({mode}): 3 queries, top-{k}, two calls")
    for step in range(2):
        qr = _randn(g, 3, 1, 8, 128, dtype=torch.bfloat16).to(DEV)
        idx_a, sc_a, dsc_a = msa.route(qr, kt, off_d, k, assembly=asm_a, **kw)
        idx_b, sc_b, dsc_b = call(qr)
        torch.cuda.synchronize()
        assert torch.equal(idx_a, idx_b) and torch.equal(sc_a.view(torch.int32), sc_b.view(torch.int32))
        assert torch.equal(dsc_a.view(torch.int32), dsc_b.view(torch.int32))
        assert torch.equal(asm_a.mem_len, asm_b.mem_len)
        assert torch.equal(asm_a.mem_kv.view(torch.int16), asm_b.mem_kv.view(torch.int16))
    with pytest.raises(ValueError, match="qr must be"):
        call(_randn(g, 2, 1, 8, 128, dtype=torch.bfloat16).to(DEV))


@pytest.mark.parametrize("mode", ["kernel", "copies"])
def test_two_stream_schedule_matches_one_stream(mode):
    """The serving schedule the benchmark's pipelined pass runs: consecutive
    queries alternate between two streams, each with its own outputs,
    workspaces and memory, so one query's selection, assembly and decode run
    beside the next query's bank scan (kernel mode: msa_route with the
    assembly; copies: msa_route without it, then msa_assemble for the
    previous query, whose copies cross the host link while the next query is
    scored).  Scores, top-k, the assembled memory and the decode output equal
    those of the same queries run one at a time on one stream, bit for bit,
    and every query's memory and decode match the oracle."""
    g = torch.Generator().manual_seed(31)
    off, host_kv, kr = _bank_with_host_tier(g, 3000, 9, 8, 128, torch.bfloat16)
    n_docs, n_pool = len(off) - 1, int(off[-1])
    kt = synth.tile_router_bank(kr)
    off_d, off_h = _dev(off), torch.as_tensor(off)
    dmap = msa.doc_map(off_d, n_pool)
    k, cap, n_q, hq, hkv, d, t_loc = 16, 144, 6, 32, 8, 128, 300
    kw = dict(kr_layout="tiled", n_pool=n_pool, doc_map=dmap)
    lk = _randn(g, 1, t_loc, hkv, d, dtype=torch.bfloat16)
    lv = _randn(g, 1, t_loc, hkv, d, dtype=torch.bfloat16)
    lk_d, lv_d = _dev(lk), _dev(lv)
    loc_len = torch.full((1,), t_loc, dtype=torch.int32, device=DEV)
    pos = torch.full((1,), k, dtype=torch.int32, device=DEV)
    qrs = [_randn(g, 1, 1, 8, 128, dtype=torch.bfloat16).to(DEV) for _ in range(n_q)]
    qs = [_randn(g, 1, hq, d, dtype=torch.bfloat16).to(DEV) for _ in range(n_q)]
    rws_bytes = msa.route_workspace_bytes(torch.bfloat16, 1, 1, 8, 128, n_docs, n_pool, k)
    dws_bytes = msa.decode_workspace_bytes(1, hq, d, cap, t_loc)

    def lane(stream):
        return {"s": stream, "asm": msa.Assembly.allocate(host_kv, off_h, 1, k, cap, DEV,
                                                          copy_stream=torch.cuda.Stream(), mode=mode),
                "rws": torch.empty(rws_bytes, dtype=torch.uint8, device=DEV),
                "dws": torch.empty(dws_bytes, dtype=torch.uint8, device=DEV),
                "dsc": torch.empty(1, n_docs, dtype=torch.float32, device=DEV),
                "idx": torch.empty(1, k, dtype=torch.int32, device=DEV),
                "sc": torch.empty(1, k, dtype=torch.float32, device=DEV),
                "out": torch.empty(1, hq, d, dtype=torch.bfloat16, device=DEV),
                "lse": torch.empty(1, hq, dtype=torch.float32, device=DEV)}

    def route(i, L, assembled):
        msa.route(qrs[i], kt, off_d, k, L["dsc"], L["idx"], L["sc"], L["rws"],
                  assembly=L["asm"] if assembled else None, stream=L["s"], **kw)

    def finish(i, L, assemble, res):
        if assemble:
            msa.assemble(L["idx"], off_d, L["asm"], stream=L["s"])
        msa.sparse_decode(qs[i], L["asm"].mem_kv, L["asm"].mem_len, lk_d, lv_d, loc_len, pos, THETA, L["out"],
                          L["lse"], L["dws"], stream=L["s"])
        with torch.cuda.stream(L["s"]):    # this query's results, before the lane's next query
            res[i] = [t.clone() for t in (L["dsc"], L["idx"], L["sc"], L["asm"].mem_len, L["asm"].mem_kv,
                                          L["out"], L["lse"])]

    _say(f"two-stream schedule ({mode}): {n_q} queries over {n_docs} documents, top-{k}, cap {cap}")
    main = torch.cuda.current_stream()
    one, two = {}, {}
    solo = lane(main)
    for i in range(n_q):                   # one at a time on one stream
        route(i, solo, mode == "kernel")
        finish(i, solo, mode == "copies", one)
        torch.cuda.synchronize()
    lanes = [lane(main), lane(torch.cuda.Stream())]
    prev = None
    for n in range(n_q):                   # alternating lanes, no synchronisation between queries
        L = lanes[n % 2]
        route(n, L, mode == "kernel")
        if mode == "kernel":
            finish(n, L, False, two)
        else:
            if prev is not None:
                finish(*prev, True, two)
            prev = (n, L)
    if prev is not None:
        finish(*prev, True, two)
    torch.cuda.synchronize()

    bits = lambda t: t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)  # noqa: E731
    src = host_kv.view(torch.int16).numpy()
    for i in range(n_q):
        dsc1, idx1, sc1, len1, mem1, out1, lse1 = one[i]
        dsc2, idx2, sc2, len2, mem2, out2, lse2 = two[i]
        m = int(len1[0])
        assert torch.equal(bits(dsc1), bits(dsc2)) and torch.equal(idx1, idx2) and torch.equal(bits(sc1), bits(sc2))
        assert torch.equal(len1, len2) and torch.equal(bits(mem1[:, :m]), bits(mem2[:, :m]))
        assert torch.equal(bits(out1), bits(out2)) and torch.equal(bits(lse1), bits(lse2)), f"query {i}"
        ref_mem, ref_len, _ = oracle.assemble(src, off, np64(idx2), cap)
        assert np.array_equal(np64(len2), ref_len)
        assert np.array_equal(bits(mem2).cpu().numpy()[:, :m], ref_mem[:, :m])
        ro, _ = oracle.decode(np64(qs[i]), np64(mem2), np64(len2), np64(lk), np64(lv), [t_loc], [k], THETA, None,
                              storage(torch.bfloat16))
        check_decode(np64(out2), ro, torch.bfloat16, f"two-stream decode, query {i}")
    # the routing itself against the oracle for the first query
    ref_scores = oracle.doc_scores(np64(qrs[0]), np64(kr), off)
    check_scores(np64(two[0][0]), ref_scores, "two-stream doc scores")
    check_topk(np64(two[0][1]), ref_scores, k, "two-stream top-k")


@pytest.mark.parametrize("mode", ["kernel", "copies"])
def test_gather_append_mode(mode):
    g = torch.Generator().manual_seed(22)
    off, host_kv, kr = _bank_with_host_tier(g, 300, 6, 8, 128, torch.bfloat16)
    asm = msa.Assembly.allocate(host_kv, torch.as_tensor(off), 2, 4, 60, DEV, mode=mode)
    src = host_kv.view(torch.int16).numpy()
    ref_mem = np.zeros((2, 60) + src.shape[1:], dtype=np.int16)
    ref_len = np.zeros(2, dtype=np.int64)
    for rnd in range(4):
        qr = _randn(g, 2, 1, 8, 128, dtype=torch.bfloat16).to(DEV)
        asm.append = rnd > 0
        _say(f"gather ({mode}): append round {rnd}")
        idx, _, _ = msa.route(qr, kr, _dev(off), 4, assembly=asm)
        torch.cuda.synchronize()
        ref_mem, ref_len, _ = oracle.assemble(src, off, np64(idx), 60, start_len=ref_len, mem=ref_mem)
        assert np.array_equal(np64(asm.mem_len), ref_len)
        if mode == "copies":
            assert np.array_equal(asm.host_mem_len.numpy(), ref_len)
        got = asm.mem_kv.view(torch.int16).cpu().numpy()
        for b in range(2):
            assert np.array_equal(got[b, :ref_len[b]], ref_mem[b, :ref_len[b]])


@pytest.mark.parametrize("mode", ["kernel", "copies"])
@pytest.mark.parametrize("k", [12, 100])
def test_assemble_on_its_own_matches_the_oracle(mode, k):
    """msa_assemble with ids from an earlier msa_route (no assembly there),
    4 appending rounds, capacity drops, and an id outside the bank in one
    query's list, which ends that list: byte-exact against the oracle."""
    g = torch.Generator().manual_seed(23 + k)
    off, host_kv, kr = _bank_with_host_tier(g, 500, 7, 8, 128, torch.bfloat16)
    cap = 3 * k
    asm = msa.Assembly.allocate(host_kv, torch.as_tensor(off), 3, k, cap, DEV, copy_stream=torch.cuda.Stream(),
                                mode=mode)
    src = host_kv.view(torch.int16).numpy()
    ref_mem = np.zeros((3, cap) + src.shape[1:], dtype=np.int16)
    ref_len = np.zeros(3, dtype=np.int64)
    for rnd in range(4):
        qr = _randn(g, 3, 1, 8, 128, dtype=torch.bfloat16).to(DEV)
        idx, _, _ = msa.route(qr, kr, _dev(off), k)
        if rnd == 2:
            idx[1, k // 2] = len(off) + 5                 # not a document: the list of query 1 ends there
        asm.append = rnd > 0
        _say(f"assemble ({mode}): round {rnd}, top-{k}, cap {cap}")
        msa.assemble(idx, _dev(off), asm)
        torch.cuda.synchronize()
        ids = np64(idx)
        if rnd == 2:
            ids_q1 = ids[1, :k // 2]
            m1, l1, _ = oracle.assemble(src, off, ids_q1[None], cap, start_len=ref_len[1:2], mem=ref_mem[1:2])
            rest = [0, 2]
            m2, l2, _ = oracle.assemble(src, off, ids[rest], cap, start_len=ref_len[rest], mem=ref_mem[rest])
            ref_mem[1:2], ref_len[1] = m1, l1[0]
            ref_mem[rest], ref_len[rest] = m2, l2
        else:
            ref_mem, ref_len, _ = oracle.assemble(src, off, ids, cap, start_len=ref_len, mem=ref_mem)
        assert np.array_equal(np64(asm.mem_len), ref_len), f"round {rnd} lengths"
        if mode == "copies":
            assert np.array_equal(asm.host_mem_len.numpy(), ref_len)
        got = asm.mem_kv.view(torch.int16).cpu().numpy()
        for b in range(3):
            assert np.array_equal(got[b, :ref_len[b]], ref_mem[b, :ref_len[b]]), f"round {rnd} query {b}"
    assert ref_len.max() > 2 * k // 2, "the rounds should fill the memory past the first round"


# ==========================================================================
# end to end
# ==========================================================================

def _chain(cfg, lens, k, mem_cap, P, pos_offset):
    bank = synth.raw_bank(cfg, lens=lens)
    tok_off = synth.token_offsets(lens)
    pool_off = synth.row_offsets(lens, P)
    n_pool = int(pool_off[-1])
    kv_g, kr_g = msa.pool_encode(_dev(bank["k"]), _dev(bank["v"]), _dev(bank["kr"]), _dev(tok_off),
                                 _dev(pool_off), P, cfg.rope_theta, n_pool)
    host_kv = kv_g.cpu().pin_memory()             # the content tier lives in pinned host memory
    qr = synth.router_queries(cfg).to(DEV)
    asm = msa.Assembly.allocate(host_kv, torch.as_tensor(pool_off), cfg.batch, k, mem_cap, DEV)
    idx, _, dsc = msa.route(qr, kr_g, _dev(pool_off), k, assembly=asm)
    q = synth.decode_queries(cfg).to(DEV)
    lk, lv = synth.local_context(cfg)
    loc_len = np.full(cfg.batch, cfg.local_len, dtype=np.int32)
    pos = np.full(cfg.batch, pos_offset, dtype=np.int32)
    out, lse = msa.sparse_decode(q, asm.mem_kv, asm.mem_len, _dev(lk), _dev(lv), _dev(loc_len), _dev(pos),
                                 cfg.rope_theta)
    torch.cuda.synchronize()

    kv_u, kr_u, _ = oracle.pool(np64(bank["k"]), np64(bank["v"]), np64(bank["kr"]), tok_off, P, cfg.rope_theta,
                                "f64")
    check_pool(np64(kv_g[:, 0]), kv_u[:, 0], cfg.torch_dtype, "chain K_bar")
    kv_r = oracle.round_to_storage(kv_u, storage(cfg.torch_dtype))
    kr_r = oracle.round_to_storage(kr_u, storage(cfg.torch_dtype))
    dsc_r = oracle.doc_scores(np64(qr), kr_r, pool_off)
    check_scores(np64(dsc), dsc_r, "chain scores")
    check_topk(np64(idx), dsc_r, k, "chain top-k")
    # decode is checked on the GPU-selected documents (oracle-pooled rows)
    mem_r, mlen_r, _ = oracle.assemble(kv_r, pool_off, np64(idx), mem_cap)
    assert np.array_equal(np64(asm.mem_len), mlen_r)
    ro, _ = oracle.decode(np64(q), mem_r, mlen_r, np64(lk), np64(lv), loc_len, pos, cfg.rope_theta, None,
                          storage(cfg.torch_dtype))
    check_decode(np64(out), ro, cfg.torch_dtype, "chain decode")
    return kv_r, kv_g, out


def test_end_to_end_tiny_config():
    cfg = synth.config(1)
    _say("chain: tiny config pool -> route -> gather -> decode")
    _chain(cfg, synth.doc_lengths(cfg), cfg.top_k, 64, cfg.pool, cfg.top_k)


def test_end_to_end_bf16_ragged():
    cfg = synth.config(2, batch=2, q_tokens=3, local_len=300)
    lens = np.random.default_rng(5).integers(1, 500, 60)
    _say("chain: bf16 ragged bank, 2 queries x 3 tokens")
    _chain(cfg, lens, 6, 64, 64, 6)


@pytest.mark.parametrize("mem_cap", [12288, 200])
def test_interleave_rounds_end_to_end(mem_cap):
    """Memory interleave: 3 rounds of route -> append -> decode for 64
    queries over a ragged lognormal bank.  Round r routes a fresh query,
    appends its top-8 documents to the query's memory (documents that no
    longer fit are dropped with every lower-ranked one) and decodes with the
    query offset by 8 per round so far.  Every round is checked against the
    oracle: scores, top-k, the assembled memory byte for byte, and the decode
    output on that memory.  mem_cap 200 forces drops in later rounds."""
    cfg = synth.config(5, total_tokens=1_500_000, local_len=256)
    lens = synth.doc_lengths(cfg)
    off = synth.row_offsets(lens, cfg.pool)
    _say(f"interleave: 64 queries x 3 rounds, {len(lens)} docs, {off[-1]} rows, mem_cap {mem_cap}")
    kr = synth.pooled_router_bank(cfg, lens, device=DEV)
    host_kv = synth.pooled_content_bank(cfg, lens, device=DEV, pin=True)
    k = cfg.top_k
    asm = msa.Assembly.allocate(host_kv, torch.as_tensor(off), cfg.batch, k, mem_cap, DEV)
    lk, lv = synth.local_context(cfg)
    loc_len = np.full(cfg.batch, cfg.local_len, dtype=np.int32)
    kr_n = np64(kr)
    src = host_kv.view(torch.int16).numpy()
    ref_mem = np.zeros((cfg.batch, mem_cap) + src.shape[1:], dtype=np.int16)
    ref_len = np.zeros(cfg.batch, dtype=np.int64)
    dropped = 0
    for rnd in range(cfg.rounds):
        qr = synth.router_queries(cfg, step=rnd, device=DEV)
        q = synth.decode_queries(cfg, step=rnd, device=DEV)
        asm.append = rnd > 0
        pos = np.full(cfg.batch, k * (rnd + 1), dtype=np.int32)
        idx, _, dsc = msa.route(qr, kr, _dev(off), k, assembly=asm)
        out, _ = msa.sparse_decode(q, asm.mem_kv, asm.mem_len, _dev(lk), _dev(lv), _dev(loc_len), _dev(pos),
                                   cfg.rope_theta)
        torch.cuda.synchronize()
        ref = oracle.doc_scores(np64(qr), kr_n, off)
        check_scores(np64(dsc), ref, f"round {rnd} scores")
        check_topk(np64(idx), ref, k, f"round {rnd} top-k")
        ref_mem, ref_len, taken = oracle.assemble(src, off, np64(idx), mem_cap, start_len=ref_len, mem=ref_mem)
        dropped += int((taken < k).sum())
        assert np.array_equal(np64(asm.mem_len), ref_len), f"round {rnd} memory lengths"
        got = asm.mem_kv.view(torch.int16).cpu().numpy()
        for b in range(cfg.batch):
            assert np.array_equal(got[b, :ref_len[b]], ref_mem[b, :ref_len[b]]), f"round {rnd} memory of query {b}"
        mem_f = np64(asm.mem_kv)
        ro, _ = oracle.decode(np64(q), mem_f, ref_len, np64(lk), np64(lv), loc_len, pos, cfg.rope_theta, None,
                              "bf16")
        check_decode(np64(out), ro, torch.bfloat16, f"round {rnd} decode")
    if mem_cap < 1000:
        assert dropped > 0, "the small memory should force drops"


def test_interleave_pipeline_matches_the_oracle():
    """The pipelined interleave schedule (routing, assembly and decode on
    three streams, ordered by events): three groups of 3 rounds for 64
    queries, so both memory buffers are used and one is refilled.  Every
    round's top-k, memory lengths and decode output against the oracle, the
    decode on memory the oracle assembles from the same ids, and the two
    final memories byte for byte."""
    from sparse_latent_memory_amd.interleave import InterleavePipeline
    cfg = synth.config(5, total_tokens=1_500_000, local_len=256)
    lens = synth.doc_lengths(cfg)
    off = synth.row_offsets(lens, cfg.pool)
    n_pool = int(off[-1])
    B, k, R = cfg.batch, cfg.top_k, cfg.rounds
    mem_cap = 600
    _say(f"interleave pipeline: 3 groups x {R} rounds x {B} queries, {len(lens)} docs, mem_cap {mem_cap}")
    kr = synth.pooled_router_bank(cfg, lens, device=DEV)
    kt = synth.tile_router_bank(kr)
    off_d = _dev(off)
    rkw = {"kr_layout": "tiled", "n_pool": n_pool, "doc_map": msa.doc_map(off_d, n_pool)}
    host_kv = synth.pooled_content_bank(cfg, lens, device=DEV, pin=True)
    lk, lv = synth.local_context(cfg, device=DEV)
    loc_len = np.full(B, cfg.local_len, dtype=np.int32)
    pipe = InterleavePipeline(kt, off_d, rkw, host_kv, torch.as_tensor(off), B, k, mem_cap, lk, lv, _dev(loc_len),
                              cfg.rope_theta, cfg.n_q_heads)
    qrs = [synth.router_queries(cfg, step=r, device=DEV) for r in range(R)]
    qs = [synth.decode_queries(cfg, step=r, device=DEV) for r in range(R)]
    pos = [np.full(B, k * (r + 1), dtype=np.int32) for r in range(R)]
    keep = []
    mems = [pipe.run(qrs, qs, [_dev(p_) for p_ in pos], keep=keep) for _ in range(3)]
    torch.cuda.synchronize()
    src = host_kv.view(torch.int16).numpy()
    refs = [oracle.doc_scores(np64(q), np64(kr), off) for q in qrs]
    lk_n, lv_n = np64(lk), np64(lv)
    for grp in range(3):
        ref_mem = np.zeros((B, mem_cap) + src.shape[1:], dtype=np.int16)
        ref_len = np.zeros(B, dtype=np.int64)
        for r in range(R):
            out, mlen, idx = keep[grp * R + r]
            ids = np64(idx)
            check_topk(ids, refs[r], k, f"group {grp} round {r} top-k")
            ref_mem, ref_len, _ = oracle.assemble(src, off, ids, mem_cap, start_len=ref_len, mem=ref_mem)
            assert np.array_equal(np64(mlen), ref_len), f"group {grp} round {r} lengths"
            ro, _ = oracle.decode(np64(qs[r]), _bf16_bits_to_f64(ref_mem), ref_len, lk_n, lv_n, loc_len, pos[r],
                                  cfg.rope_theta, None, "bf16")
            check_decode(np64(out), ro, torch.bfloat16, f"group {grp} round {r} decode")
        if grp >= 1:                              # groups 1 and 2 own the two buffers at the end
            got = mems[grp].mem_kv.view(torch.int16).cpu().numpy()
            for b in range(B):
                assert np.array_equal(got[b, :ref_len[b]], ref_mem[b, :ref_len[b]]), f"group {grp} memory {b}"
    assert mems[0] is mems[2]


@pytest.mark.slow
def test_interleave_50m_bank_full_size():
    """Memory interleave at its full size, called as the benchmark times it:
    the 50M-token lognormal bank (tiled, document map built once), 64
    one-token queries x 3 rounds of top-8 on the wide matrix-core scan, the
    device-side gather appending into a 12,288-row memory per query, and
    decode over [memory ; 4096 local tokens] with the query offset by 8 per
    round.  Every round: all document scores and the top-k against the
    oracle, the memory byte for byte, and all 64 decode outputs."""
    cfg = synth.config(5)
    lens = synth.doc_lengths(cfg)
    off = synth.row_offsets(lens, cfg.pool)
    n_pool = int(off[-1])
    B, k = cfg.batch, cfg.top_k
    mem_cap = cfg.ctx_cap - cfg.local_len
    _say(f"interleave: full size, {len(lens)} docs, {n_pool} rows, 64 queries x {cfg.rounds} rounds, "
         f"mem_cap {mem_cap}, {cfg.local_len} local")
    kr = synth.pooled_router_bank(cfg, lens, device=DEV)
    kt = synth.tile_router_bank(kr)
    off_d = _dev(off)
    dmap = msa.doc_map(off_d, n_pool)
    host_kv = synth.pooled_content_bank(cfg, lens, device=DEV, pin=True)
    asm = msa.Assembly.allocate(host_kv, torch.as_tensor(off), B, k, mem_cap, DEV)
    lk, lv = synth.local_context(cfg, device=DEV)
    lk_n, lv_n = np64(lk), np64(lv)
    loc_len = np.full(B, cfg.local_len, dtype=np.int32)
    src = host_kv.view(torch.int16).numpy()
    ref_mem = np.zeros((B, mem_cap) + src.shape[1:], dtype=np.int16)
    ref_len = np.zeros(B, dtype=np.int64)
    for rnd in range(cfg.rounds):
        qr = synth.router_queries(cfg, step=rnd, device=DEV)
        q = synth.decode_queries(cfg, step=rnd, device=DEV)
        asm.append = rnd > 0
        pos = np.full(B, k * (rnd + 1), dtype=np.int32)
        idx, sc, dsc = msa.route(qr, kt, off_d, k, assembly=asm, kr_layout="tiled", n_pool=n_pool, doc_map=dmap)
        out, _ = msa.sparse_decode(q, asm.mem_kv, asm.mem_len, lk, lv, _dev(loc_len), _dev(pos), cfg.rope_theta)
        torch.cuda.synchronize()
        _say(f"  round {rnd}: oracle scores of {len(lens)} documents x {B} queries")
        ref = _oracle_doc_scores(qr, kr, off)
        check_scores(np64(dsc), ref, f"round {rnd} scores")
        check_topk(np64(idx), ref, k, f"round {rnd} top-k")
        check_topk_order(np64(idx), np64(sc), f"round {rnd} order")
        ref_mem, ref_len, _ = oracle.assemble(src, off, np64(idx), mem_cap, start_len=ref_len, mem=ref_mem)
        assert np.array_equal(np64(asm.mem_len), ref_len), f"round {rnd} memory lengths"
        got = asm.mem_kv.view(torch.int16).cpu().numpy()
        for b in range(B):
            assert np.array_equal(got[b, :ref_len[b]], ref_mem[b, :ref_len[b]]), f"round {rnd} memory of query {b}"
        del got
        _say(f"  round {rnd}: oracle decode of {B} queries over up to {int(ref_len.max())} memory rows")
        ro = np.empty((B, cfg.n_q_heads, cfg.head_dim))
        for b in range(B):
            m = _bf16_bits_to_f64(ref_mem[b:b + 1, :ref_len[b]])
            ro[b], _ = oracle.decode(np64(q[b:b + 1]), m, ref_len[b:b + 1], lk_n[b:b + 1], lv_n[b:b + 1],
                                     loc_len[b:b + 1], pos[b:b + 1], cfg.rope_theta, None, "bf16")
        check_decode(np64(out), ro, torch.bfloat16, f"round {rnd} decode")


def test_dense_special_case_equals_sdpa():
    """Pool size 1 and k = all documents: the whole path is dense attention
    over [every document's rotated keys ; the locally rotated keys], checked
    against torch's scaled_dot_product_attention in float64 on the CPU."""
    cfg = synth.config(1, local_len=37)
    lens = np.array([3, 9, 5, 1, 7, 4])
    _say("chain: P=1, k=n_docs vs dense SDPA")
    kv_r, kv_g, out = _chain(cfg, lens, len(lens), int(lens.sum()), 1, len(lens))
    bank = synth.raw_bank(cfg, lens=lens)
    tok_off = synth.token_offsets(lens)
    keys = [oracle.rope(np64(bank["k"][tok_off[i]:tok_off[i + 1]]), np.arange(lens[i]), cfg.rope_theta)
            for i in range(len(lens))]
    lk, lv = synth.local_context(cfg)
    o = len(lens)
    keys.append(oracle.rope(np64(lk[0]), o + np.arange(cfg.local_len), cfg.rope_theta))
    vals = [np64(bank["v"][tok_off[i]:tok_off[i + 1]]) for i in range(len(lens))] + [np64(lv[0])]
    rep = cfg.n_q_heads // cfg.n_kv_heads
    kk = torch.from_numpy(np.concatenate(keys)).permute(1, 0, 2).repeat_interleave(rep, 0).contiguous()
    vv = torch.from_numpy(np.concatenate(vals)).permute(1, 0, 2).repeat_interleave(rep, 0).contiguous()
    q = synth.decode_queries(cfg)
    qq = torch.from_numpy(oracle.rope(np64(q[0])[None], [o + cfg.local_len - 1], cfg.rope_theta)[0])[:, None, :]
    want = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[:, 0].numpy()
    check_decode(np64(out)[0], want, torch.float32, "dense special case")
