"""Pins of the CPU oracle against things other than itself: hand-derived
worked examples (tests/golden), closed forms, invariants, library routines
(torch's bfloat16 cast, cosine_similarity, scaled_dot_product_attention,
Python's sorted) and a pure-Python brute-force twin on tiny inputs."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import loops

RNG = np.random.default_rng(20261203)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# bfloat16 rounding: equals torch's round-to-nearest-even cast
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_cast():
    x = np.concatenate([
        RNG.standard_normal(20000) * 10.0 ** RNG.integers(-30, 30, 20000),
        np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 2 ** -130, 3 * 2 ** -134,
                    3.3e38, 0.0, -0.0, 1e-45]),
    ]).astype(np.float32)
    ours = oracle.round_to_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_bf16_rounding_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0)
    assert oracle.round_to_bf16(1.0 + 2 ** -8) == 1.0
    assert oracle.round_to_bf16(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6
    # a hair above the tie rounds up
    assert oracle.round_to_bf16(1.0 + 2 ** -8 + 2 ** -30) == 1.0 + 2 ** -7


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------

def test_rope_equals_complex_rotation_twin():
    x = RNG.standard_normal((5, 3, 8))
    pos = np.array([0, 1, 7, 1000, 65535])
    got = oracle.rope(x, pos, 1e6)
    for n in range(5):
        for h in range(3):
            np.testing.assert_allclose(got[n, h], loops._rot(list(x[n, h]), int(pos[n]), 1e6),
                                       rtol=0, atol=1e-12)


def test_rope_closed_form_single_pair():
    # D = 2: one frequency theta^0 = 1, so position p rotates by p radians
    for p in [0, 1, 2, 3, 100]:
        got = oracle.rope(np.array([[[1.0, 0.0]]]), [p], 12345.0)[0, 0]
        np.testing.assert_allclose(got, [math.cos(p), math.sin(p)], atol=1e-15)


def test_rope_worked_example_exact_frequencies(golden_dir):
    # theta chosen so that every frequency theta^(-2j/D) is a power of 1/4:
    # pins the schedule's exponent and the rotate-half pairing for j >= 1
    g = _load(golden_dir, "rope_worked_example.json")
    assert len(g["cases"]) == 12
    for c in g["cases"]:
        x = np.array(c["x"], dtype=np.float64)[None, None, :]
        got = oracle.rope(x, [c["pos"]], c["theta"])[0, 0]
        np.testing.assert_allclose(got, c["rope"], rtol=0, atol=1e-15, err_msg=c["formula"])


@pytest.mark.parametrize("head_dim,theta", [(128, 1e6), (64, 1e4)])
def test_rope_matches_transformers_qwen3_rotary(head_dim, theta):
    # an implementation written by others: the Qwen3 rotary embedding of the
    # transformers library (rotate-half, theta^(-2j/D) in float32).  Its float32
    # frequencies move an angle by at most p * 2^-24 * omega, so positions stay
    # below 4096 and the bound is 1e-3 of each vector's norm; a wrong exponent
    # or interleaved pairs give errors of order one.
    tf = pytest.importorskip("transformers")
    from transformers.models.qwen3 import modeling_qwen3 as q3
    cfg = tf.Qwen3Config(head_dim=head_dim, rope_theta=theta, hidden_size=2 * head_dim, num_attention_heads=2,
                         num_key_value_heads=1)
    emb = q3.Qwen3RotaryEmbedding(cfg)
    pos = torch.arange(0, 4096, 37)[None]
    x = torch.from_numpy(RNG.standard_normal((1, 2, pos.shape[1], head_dim)))
    cos, sin = emb(x, pos)
    ref, _ = q3.apply_rotary_pos_emb(x, x, cos, sin)
    got = np.stack([oracle.rope(x[0, h].numpy(), pos[0].numpy(), theta) for h in range(2)])
    err = np.linalg.norm(got - ref[0].numpy(), axis=-1) / np.linalg.norm(got, axis=-1)
    assert err.max() < 1e-3, err.max()
    np.testing.assert_allclose(oracle.rope_inv_freq(head_dim, theta), emb.inv_freq.double().numpy(), rtol=2e-7)


def test_rope_invariants():
    d = 64
    x = RNG.standard_normal((1, 1, d))
    y = RNG.standard_normal((1, 1, d))
    # position 0 is the identity
    np.testing.assert_array_equal(oracle.rope(x, [0], 1e6), x)
    # norm preserved
    for p in [1, 17, 4096]:
        assert abs(np.linalg.norm(oracle.rope(x, [p], 1e6)) - np.linalg.norm(x)) < 1e-12
    # inner product depends only on the position difference
    base = float(np.sum(oracle.rope(x, [10], 1e4) * oracle.rope(y, [3], 1e4)))
    for shift in [1, 50, 9000]:
        other = float(np.sum(oracle.rope(x, [10 + shift], 1e4) * oracle.rope(y, [3 + shift], 1e4)))
        assert abs(base - other) < 1e-10


# --------------------------------------------------------------------------
# pooling
# --------------------------------------------------------------------------

def test_pool_worked_example(golden_dir):
    g = _load(golden_dir, "pool_worked_example.json")
    kb, vb, rb = oracle.pool_doc(np.array(g["k"]), np.array(g["v"]), np.array(g["kr"]),
                                 g["pool"], g["theta"])
    np.testing.assert_allclose(kb, g["k_bar"], atol=1e-15)
    np.testing.assert_allclose(vb, g["v_bar"], atol=1e-15)
    np.testing.assert_allclose(rb, g["kr_bar"], atol=1e-15)


def test_pool_constant_chunk_pools_to_itself():
    c = RNG.standard_normal((1, 2, 16))
    k = RNG.standard_normal((10, 2, 16))
    kb, vb, rb = oracle.pool_doc(k, np.repeat(c, 10, axis=0), np.repeat(c, 10, axis=0), 4, 1e6)
    assert vb.shape == (3, 2, 16)
    np.testing.assert_allclose(vb, np.repeat(c, 3, axis=0), atol=1e-14)
    np.testing.assert_allclose(rb, np.repeat(c, 3, axis=0), atol=1e-14)


@pytest.mark.parametrize("theta", [1e4, 1e6])
def test_pool_rope_mean_phasor_closed_form(theta):
    # constant x over positions a..a+n-1: each pair rotates by the mean phasor
    # (1/n) sum_p e^{i p w} = e^{i (a + (n-1)/2) w} sin(n w / 2) / (n sin(w / 2))
    d, n_tok, pool = 16, 37, 8
    x = RNG.standard_normal(d)
    kb, _, _ = oracle.pool_doc(np.tile(x, (n_tok, 1, 1)), np.zeros((n_tok, 1, d)),
                               np.zeros((n_tok, 1, d)), pool, theta)
    h = d // 2
    for c in range(kb.shape[0]):
        a = c * pool
        n = min(pool, n_tok - a)
        for j in range(h):
            w = theta ** (-2.0 * j / d)
            amp = math.sin(n * w / 2) / (n * math.sin(w / 2))
            z = complex(x[j], x[j + h]) * amp * complex(math.cos((a + (n - 1) / 2) * w),
                                                        math.sin((a + (n - 1) / 2) * w))
            assert abs(kb[c, 0, j] - z.real) < 1e-12
            assert abs(kb[c, 0, j + h] - z.imag) < 1e-12


def test_pool_size_one_is_identity_up_to_rope():
    k = RNG.standard_normal((9, 2, 8))
    v = RNG.standard_normal((9, 2, 8))
    kr = RNG.standard_normal((9, 3, 4))
    kb, vb, rb = oracle.pool_doc(k, v, kr, 1, 1e6)
    np.testing.assert_array_equal(vb, v)
    np.testing.assert_array_equal(rb, kr)
    for t in range(9):
        np.testing.assert_allclose(kb[t, 0], loops._rot(list(k[t, 0]), t, 1e6), atol=1e-12)


def test_pool_linearity():
    a, b = 0.7, -2.5
    x = [RNG.standard_normal((13, 2, 8)) for _ in range(3)]
    y = [RNG.standard_normal((13, 2, 8)) for _ in range(3)]
    px = oracle.pool_doc(*x, 5, 1e6)
    py = oracle.pool_doc(*y, 5, 1e6)
    pz = oracle.pool_doc(*[a * u + b * w for u, w in zip(x, y)], 5, 1e6)
    for i in range(3):
        np.testing.assert_allclose(pz[i], a * px[i] + b * py[i], atol=1e-12)


def test_pool_matches_brute_force_twin_with_tail():
    k = RNG.standard_normal((11, 2, 4))
    v = RNG.standard_normal((11, 2, 4))
    kr = RNG.standard_normal((11, 1, 6))
    got = oracle.pool_doc(k, v, kr, 4, 1e4)
    want = loops.pool_doc(k, v, kr, 4, 1e4)
    assert got[0].shape[0] == 3     # 4 + 4 + tail of 3
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, np.array(w), atol=1e-12)


def test_pool_bank_document_independence_and_offsets():
    lens = np.array([5, 1, 12, 8, 3])
    off = np.concatenate([[0], np.cumsum(lens)])
    k = RNG.standard_normal((off[-1], 2, 8))
    v = RNG.standard_normal((off[-1], 2, 8))
    kr = RNG.standard_normal((off[-1], 2, 4))
    kv, krp, pool_off = oracle.pool(k, v, kr, off, 4, 1e6)
    np.testing.assert_array_equal(pool_off, [0, 2, 3, 6, 8, 9])
    for d in range(len(lens)):
        a, b = off[d], off[d + 1]
        kb, vb, rb = oracle.pool_doc(k[a:b], v[a:b], kr[a:b], 4, 1e6)
        r0, r1 = pool_off[d], pool_off[d + 1]
        np.testing.assert_array_equal(kv[r0:r1, 0], kb)
        np.testing.assert_array_equal(kv[r0:r1, 1], vb)
        np.testing.assert_array_equal(krp[r0:r1], rb)


# --------------------------------------------------------------------------
# routing scores
# --------------------------------------------------------------------------

def test_route_worked_example(golden_dir):
    g = _load(golden_dir, "route_worked_example.json")
    qr = np.array(g["qr"], dtype=float)
    kr = np.array(g["kr_pooled"], dtype=float)
    off = np.array(g["doc_pool_off"])
    np.testing.assert_allclose(oracle.row_scores(qr, kr), g["row_scores_by_token"], atol=1e-15)
    dsc = oracle.doc_scores(qr, kr, off)
    np.testing.assert_allclose(dsc, g["doc_scores"], atol=1e-15)
    assert oracle.topk(dsc, 3)[0].tolist() == g["topk_3"]
    assert oracle.topk(dsc, 4)[0].tolist() == g["topk_4"]


def _bank(n_docs, max_rows, hr, dr, rng=RNG):
    rows = rng.integers(1, max_rows + 1, n_docs)
    off = np.concatenate([[0], np.cumsum(rows)])
    return rng.standard_normal((off[-1], hr, dr)), off


def test_scores_match_brute_force_twin():
    kr, off = _bank(5, 3, 3, 4)
    qr = RNG.standard_normal((2, 3, 3, 4))
    got = oracle.doc_scores(qr, kr, off)
    want = loops.doc_scores(qr, kr, list(zip(off[:-1], off[1:])))
    np.testing.assert_allclose(got, want, atol=1e-13)


def test_scores_library_cosine_special_case():
    # one router head, one query token, one row per document: the score is
    # exactly torch's cosine_similarity
    kr = RNG.standard_normal((50, 1, 32))
    qr = RNG.standard_normal((1, 1, 1, 32))
    got = oracle.doc_scores(qr, kr, np.arange(51))[0]
    want = torch.nn.functional.cosine_similarity(torch.from_numpy(qr[0, 0]), torch.from_numpy(kr[:, 0]),
                                                 dim=-1).numpy()
    np.testing.assert_allclose(got, want, atol=1e-14)


def test_scores_range_and_self_match():
    kr, off = _bank(40, 4, 8, 16)
    qr = RNG.standard_normal((3, 2, 8, 16))
    dsc = oracle.doc_scores(qr, kr, off)
    assert np.all(dsc <= 1 + 1e-12) and np.all(dsc >= -1 - 1e-12)
    # a query equal to a stored row scores 1 for that document, which ranks first
    d = 17
    qr2 = kr[off[d]][None, None] * 3.0
    dsc2 = oracle.doc_scores(qr2, kr, off)
    assert abs(dsc2[0, d] - 1.0) < 1e-12
    assert oracle.topk(dsc2, 1)[0][0, 0] == d


def test_scores_norm_clamp_closed_form():
    # cos(x, y) = <x,y> / (max(|x|, 1e-8) max(|y|, 1e-8)): a key c * q_hat scores
    # c / 1e-8 below the clamp and exactly 1 above it, per head, so the head
    # mean is the mean of those values
    q = RNG.standard_normal((1, 1, 2, 8))
    qhat = q / np.linalg.norm(q, axis=-1, keepdims=True)
    for c, want in [(1e-9, 0.1), (2.5e-9, 0.25), (1e-6, 1.0), (1e-3, 1.0)]:
        kr = (c * qhat[0, 0])[None]                                   # one row, both heads scaled by c
        np.testing.assert_allclose(oracle.doc_scores(q, kr, [0, 1]), [[want]], rtol=1e-9)
    kr = np.stack([1e-9 * qhat[0, 0, 0], 5.0 * qhat[0, 0, 1]])[None]   # heads 0.1 and 1
    np.testing.assert_allclose(oracle.doc_scores(q, kr, [0, 1]), [[0.55]], rtol=1e-9)


def test_scores_invariances():
    kr, off = _bank(30, 5, 4, 8)
    qr = RNG.standard_normal((2, 3, 4, 8))
    base = oracle.doc_scores(qr, kr, off)
    # positive per-head scaling of Qr and of Kr
    sq = RNG.uniform(0.1, 10, (1, 1, 4, 1))
    sk = RNG.uniform(0.1, 10, (1, 4, 1))
    np.testing.assert_allclose(oracle.doc_scores(qr * sq, kr * sk, off), base, atol=1e-13)
    # joint permutation of heads
    p = RNG.permutation(4)
    np.testing.assert_allclose(oracle.doc_scores(qr[:, :, p], kr[:, p], off), base, atol=1e-13)
    # duplicating query tokens changes nothing; adding a token never lowers a score
    qd = np.concatenate([qr, qr[:, :1]], axis=1)
    np.testing.assert_allclose(oracle.doc_scores(qd, kr, off), base, atol=1e-13)
    qa = np.concatenate([qr, RNG.standard_normal((2, 1, 4, 8))], axis=1)
    assert np.all(oracle.doc_scores(qa, kr, off) >= base - 1e-13)


def test_scores_bank_order_invariance_through_pooling():
    # permuting documents, re-pooling and re-scoring permutes the scores
    lens = np.array([7, 3, 12, 9, 4, 6])
    off = np.concatenate([[0], np.cumsum(lens)])
    k = RNG.standard_normal((off[-1], 2, 8))
    v = RNG.standard_normal((off[-1], 2, 8))
    kr = RNG.standard_normal((off[-1], 4, 8))
    qr = RNG.standard_normal((2, 2, 4, 8))
    kv, krp, poff = oracle.pool(k, v, kr, off, 4, 1e6)
    base = oracle.doc_scores(qr, krp, poff)
    perm = RNG.permutation(len(lens))
    idx = np.concatenate([np.arange(off[d], off[d + 1]) for d in perm])
    off2 = np.concatenate([[0], np.cumsum(lens[perm])])
    kv2, krp2, poff2 = oracle.pool(k[idx], v[idx], kr[idx], off2, 4, 1e6)
    np.testing.assert_allclose(oracle.doc_scores(qr, krp2, poff2), base[:, perm], atol=1e-13)
    # pooled K is identical per document too (positions restart per document)
    for new, d in enumerate(perm):
        np.testing.assert_array_equal(kv2[poff2[new]:poff2[new + 1]], kv[poff[d]:poff[d + 1]])


def test_planted_needle_scores_point_six():
    from sparse_latent_memory_amd import synth
    cfg = synth.config(3, batch=2)
    lens = np.array([64, 128, 300, 64, 64, 100, 64, 200])
    off = synth.row_offsets(lens, 64)
    kr = torch.randn(int(off[-1]), 8, 128, dtype=torch.float64) * 0.125
    qr = torch.randn(2, 1, 8, 128, dtype=torch.float64)
    docs = synth.plant_needles(cfg, qr, kr, off)
    dsc = oracle.doc_scores(qr.numpy(), kr.numpy(), off)
    for b, d in enumerate(docs):
        # the planted row is written through float32, hence 1e-7 and not 1e-15
        assert abs(dsc[b, d] - 0.6) < 1e-7
        assert oracle.topk(dsc, 1)[0][b, 0] == d


# --------------------------------------------------------------------------
# top-k
# --------------------------------------------------------------------------

def test_topk_matches_sorted_with_ties():
    s = RNG.integers(0, 6, (4, 200)).astype(float) / 5.0     # many exact ties
    for k in [1, 7, 50, 200]:
        idx, sc = oracle.topk(s, k)
        want = loops.topk(s.tolist(), k)
        assert idx.tolist() == want
        np.testing.assert_array_equal(sc, np.take_along_axis(s, np.array(want), 1))


def test_topk_all_is_permutation():
    s = RNG.standard_normal((3, 33))
    idx, sc = oracle.topk(s, 33)
    for row in idx:
        assert sorted(row.tolist()) == list(range(33))
    assert np.all(np.diff(sc, axis=1) <= 0)


# --------------------------------------------------------------------------
# assembly
# --------------------------------------------------------------------------

def test_assemble_copies_rows_in_rank_order_and_drops_overflow():
    kv = RNG.integers(-2 ** 15, 2 ** 15, (20, 2, 2, 4)).astype(np.int16)   # raw bf16 bit patterns
    off = np.array([0, 3, 4, 9, 11, 20])
    idx = np.array([[2, 0, 3], [4, 1, 0]])
    mem, mlen, taken = oracle.assemble(kv, off, idx, mem_cap=10)
    # query 0: docs 2 (5 rows), 0 (3 rows) fit (8), doc 3 (2 rows) fits (10)
    assert mlen.tolist()[0] == 10 and taken[0] == 3
    assert np.array_equal(mem[0, :5], kv[4:9]) and np.array_equal(mem[0, 5:8], kv[0:3])
    assert np.array_equal(mem[0, 8:10], kv[9:11])
    # query 1: doc 4 has 9 rows, doc 1 fits (10), doc 0 overflows: dropped
    assert mlen[1] == 10 and taken[1] == 2
    assert np.array_equal(mem[1, :9], kv[11:20]) and np.array_equal(mem[1, 9], kv[3])
    # a lower-ranked document that would still fit is dropped with the one
    # that overflowed: docs 2 (5 rows) and 4 (9 rows) leave 1 row of 7 free
    # after doc 2, doc 4 does not fit, doc 1 (1 row) would, but is not taken
    mem3, mlen3, taken3 = oracle.assemble(kv, off, np.array([[2, 4, 1]]), mem_cap=7)
    assert mlen3.tolist() == [5] and taken3.tolist() == [1]
    assert not mem3[0, 5:].any()
    # appending after existing rows
    mem2, mlen2, _ = oracle.assemble(kv, off, idx[:, :1], mem_cap=12, start_len=[2, 0])
    assert mlen2.tolist() == [7, 9]
    assert np.array_equal(mem2[0, 2:7], kv[4:9])


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------

def test_decode_worked_example(golden_dir):
    g = _load(golden_dir, "decode_worked_example.json")
    mem = np.stack([np.array(g["mem_k"]), np.array(g["mem_v"])], axis=2)[:, :, :, None, :]
    out, lse = oracle.decode(np.array(g["q"]), mem, [1], np.array(g["local_k"])[:, :, None, :],
                             np.array(g["local_v"])[:, :, None, :], [1], [g["pos_offset"]], 1e4)
    np.testing.assert_allclose(out[0], g["out"], atol=1e-14)
    np.testing.assert_allclose(lse[0], g["lse"], atol=1e-14)


def test_decode_relative_position_closed_form():
    # D = 2: local key (a, 0) at position o and a zero key at o + 1; the query
    # (1, 0) sits at o + 1.  The logit of the first key is a cos(1) / sqrt(2)
    # whatever o is.
    a = 1.7
    for o in [0, 3, 1000]:
        lk = np.array([[[[a, 0.0]], [[0.0, 0.0]]]])
        lv = np.array([[[[1.0, 0.0]], [[0.0, 1.0]]]])
        out, lse = oracle.decode(np.array([[[1.0, 0.0]]]), np.zeros((1, 0, 2, 1, 2)), [0], lk, lv,
                                 [2], [o], 1e6)
        z = a * math.cos(1.0) / math.sqrt(2.0)
        w0 = math.exp(z) / (math.exp(z) + 1.0)
        np.testing.assert_allclose(out[0, 0], [w0, 1 - w0], atol=1e-14)
        assert abs(lse[0, 0] - math.log(math.exp(z) + 1.0)) < 1e-14


def test_decode_matches_brute_force_twin():
    hq, hkv, d = 4, 2, 8
    q = RNG.standard_normal((1, hq, d))
    mem = RNG.standard_normal((1, 5, 2, hkv, d))
    lk = RNG.standard_normal((1, 6, hkv, d))
    lv = RNG.standard_normal((1, 6, hkv, d))
    out, lse = oracle.decode(q, mem, [3], lk, lv, [4], [7], 1e4)
    o2, l2 = loops.decode(q[0], mem[0, :3, 0], mem[0, :3, 1], lk[0, :4], lv[0, :4], 7, 1e4)
    np.testing.assert_allclose(out[0], o2, atol=1e-12)
    np.testing.assert_allclose(lse[0], l2, atol=1e-12)


def test_decode_dense_special_case_equals_sdpa():
    """Pool size 1 and k = all documents: sparse decode is dense attention
    (torch's scaled_dot_product_attention, float64, GQA by repeating KV
    heads) over every document's rotated keys followed by the local keys."""
    hq, hkv, d, theta = 8, 2, 16, 1e6
    lens = np.array([3, 5, 2, 4])
    off = np.concatenate([[0], np.cumsum(lens)])
    k = RNG.standard_normal((off[-1], hkv, d))
    v = RNG.standard_normal((off[-1], hkv, d))
    kr = RNG.standard_normal((off[-1], 2, 4))
    kv, krp, poff = oracle.pool(k, v, kr, off, 1, theta)
    qr = RNG.standard_normal((1, 1, 2, 4))
    idx, _ = oracle.topk(oracle.doc_scores(qr, krp, poff), len(lens))
    mem, mlen, taken = oracle.assemble(kv, poff, idx, mem_cap=int(off[-1]))
    assert mlen[0] == off[-1] and taken[0] == len(lens)
    t_loc = 6
    q = RNG.standard_normal((1, hq, d))
    lk = RNG.standard_normal((1, t_loc, hkv, d))
    lv = RNG.standard_normal((1, t_loc, hkv, d))
    o = len(lens)
    out, _ = oracle.decode(q, mem, mlen, lk, lv, [t_loc], [o], theta)

    keys = [oracle.rope(k[off[i]:off[i + 1]], np.arange(lens[i]), theta) for i in range(len(lens))]
    keys.append(oracle.rope(lk[0], o + np.arange(t_loc), theta))
    vals = [v[off[i]:off[i + 1]] for i in range(len(lens))] + [lv[0]]
    kk = torch.from_numpy(np.concatenate(keys)).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    vv = torch.from_numpy(np.concatenate(vals)).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    qq = torch.from_numpy(oracle.rope(q[0][None], [o + t_loc - 1], theta)[0])[:, None, :]
    want = torch.nn.functional.scaled_dot_product_attention(qq, kk.contiguous(), vv.contiguous())
    np.testing.assert_allclose(out[0], want[:, 0].numpy(), atol=1e-12)


def test_decode_special_cases():
    hq, hkv, d = 4, 2, 8
    q = RNG.standard_normal((1, hq, d))
    lk = RNG.standard_normal((1, 5, hkv, d))
    lv = RNG.standard_normal((1, 5, hkv, d))
    empty = np.zeros((1, 0, 2, hkv, d))
    # empty memory: the offset cancels (RoPE is relative)
    a, la = oracle.decode(q, empty, [0], lk, lv, [5], [0], 1e6)
    b, lb = oracle.decode(q, empty, [0], lk, lv, [5], [123], 1e6)
    np.testing.assert_allclose(a, b, atol=1e-12)
    np.testing.assert_allclose(la, lb, atol=1e-12)
    # a single key gives its value
    one, _ = oracle.decode(q, empty, [0], lk, lv, [1], [4], 1e6)
    np.testing.assert_allclose(one[0], np.repeat(lv[0, 0], hq // hkv, axis=0), atol=1e-14)
    # zero keys give the mean of the values
    zero, lz = oracle.decode(q, empty, [0], np.zeros_like(lk), lv, [5], [2], 1e6)
    np.testing.assert_allclose(zero[0], np.repeat(lv[0].mean(0), hq // hkv, axis=0), atol=1e-14)
    np.testing.assert_allclose(lz, math.log(5.0), atol=1e-14)
    # no keys at all
    nil, ln = oracle.decode(q, empty, [0], lk, lv, [0], [0], 1e6)
    assert np.all(nil == 0) and np.all(np.isneginf(ln))


# --------------------------------------------------------------------------
# a block of query tokens through the sparse context (reading R13)
# --------------------------------------------------------------------------

def test_attend_worked_example(golden_dir):
    g = _load(golden_dir, "attend_worked_example.json")
    out, lse = oracle.attend(np.array(g["q"]), np.array(g["mem_kv"]), g["mem_len"], np.array(g["local_k"]),
                             np.array(g["local_v"]), g["local_len"], g["pos_offset"], g["theta"])
    np.testing.assert_allclose(out, g["out"], atol=1e-14)
    np.testing.assert_allclose(lse, g["lse"], atol=1e-14)


def test_attend_one_token_is_the_decode_step():
    hq, hkv, d = 8, 2, 16
    q = RNG.standard_normal((2, hq, d))
    mem = RNG.standard_normal((2, 5, 2, hkv, d))
    lk = RNG.standard_normal((2, 7, hkv, d))
    lv = RNG.standard_normal((2, 7, hkv, d))
    a, la = oracle.attend(q[:, None], mem, [3, 5], lk, lv, [7, 2], [16, 1000], 1e6)
    b, lb = oracle.decode(q, mem, [3, 5], lk, lv, [7, 2], [16, 1000], 1e6)
    np.testing.assert_allclose(a[:, 0], b, atol=1e-12)
    np.testing.assert_allclose(la[:, 0], lb, atol=1e-12)


def test_attend_matches_brute_force_twin():
    hq, hkv, d, tq = 4, 2, 8, 3
    q = RNG.standard_normal((1, tq, hq, d))
    mem = RNG.standard_normal((1, 4, 2, hkv, d))
    lk = RNG.standard_normal((1, 6, hkv, d))
    lv = RNG.standard_normal((1, 6, hkv, d))
    out, lse = oracle.attend(q, mem, [2], lk, lv, [5], [9], 1e4)
    o2, l2 = loops.attend(q[0], mem[0, :2, 0], mem[0, :2, 1], lk[0, :5], lv[0, :5], 9, 1e4)
    np.testing.assert_allclose(out[0], o2, atol=1e-12)
    np.testing.assert_allclose(lse[0], l2, atol=1e-12)


def test_attend_dense_causal_equals_sdpa():
    """Pool size 1, k = all documents: a block of query tokens over the
    assembled context is torch's scaled_dot_product_attention (float64, GQA
    by repeating KV heads) with a mask that shows every memory key and the
    local keys up to each token."""
    hq, hkv, d, theta = 8, 2, 16, 1e6
    lens = np.array([3, 5, 2])
    off = np.concatenate([[0], np.cumsum(lens)])
    k = RNG.standard_normal((off[-1], hkv, d))
    v = RNG.standard_normal((off[-1], hkv, d))
    kr = RNG.standard_normal((off[-1], 2, 4))
    kv, krp, poff = oracle.pool(k, v, kr, off, 1, theta)
    idx, _ = oracle.topk(oracle.doc_scores(RNG.standard_normal((1, 1, 2, 4)), krp, poff), len(lens))
    mem, mlen, _ = oracle.assemble(kv, poff, idx, mem_cap=int(off[-1]))
    t_loc, tq = 9, 4
    q = RNG.standard_normal((1, tq, hq, d))
    lk = RNG.standard_normal((1, t_loc, hkv, d))
    lv = RNG.standard_normal((1, t_loc, hkv, d))
    o = len(lens)
    out, _ = oracle.attend(q, mem, mlen, lk, lv, [t_loc], [o], theta)

    order = idx[0]
    keys = [oracle.rope(k[off[i]:off[i + 1]], np.arange(lens[i]), theta) for i in order]
    keys.append(oracle.rope(lk[0], o + np.arange(t_loc), theta))
    vals = [v[off[i]:off[i + 1]] for i in order] + [lv[0]]
    kk = torch.from_numpy(np.concatenate(keys)).permute(1, 0, 2).repeat_interleave(hq // hkv, 0).contiguous()
    vv = torch.from_numpy(np.concatenate(vals)).permute(1, 0, 2).repeat_interleave(hq // hkv, 0).contiguous()
    i_t = t_loc - tq + np.arange(tq)
    qq = torch.from_numpy(oracle.rope(q[0], o + i_t, theta)).permute(1, 0, 2).contiguous()   # [Hq, Tq, D]
    m = int(off[-1])
    j = np.arange(m + t_loc)
    mask = torch.from_numpy((j[None, :] < m) | ((j[None, :] - m) <= i_t[:, None]))
    want = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)   # [Hq, Tq, D]
    np.testing.assert_allclose(out[0], want.permute(1, 0, 2).numpy(), atol=1e-12)


def test_attend_is_causal_and_relative():
    hq, hkv, d, tq, t_loc = 4, 2, 8, 3, 6
    q = RNG.standard_normal((1, tq, hq, d))
    mem = RNG.standard_normal((1, 3, 2, hkv, d))
    lk = RNG.standard_normal((1, t_loc, hkv, d))
    lv = RNG.standard_normal((1, t_loc, hkv, d))
    base, _ = oracle.attend(q, mem, [3], lk, lv, [t_loc], [5], 1e6)
    # changing the last local token moves only the last query token
    lk2, lv2 = lk.copy(), lv.copy()
    lk2[0, -1] += 1.0
    lv2[0, -1] -= 2.0
    moved, _ = oracle.attend(q, mem, [3], lk2, lv2, [t_loc], [5], 1e6)
    np.testing.assert_allclose(moved[0, :tq - 1], base[0, :tq - 1], atol=1e-14)
    assert np.abs(moved[0, tq - 1] - base[0, tq - 1]).max() > 1e-3
    # without memory the position offset cancels
    empty = np.zeros((1, 0, 2, hkv, d))
    a, _ = oracle.attend(q, empty, [0], lk, lv, [t_loc], [0], 1e6)
    b, _ = oracle.attend(q, empty, [0], lk, lv, [t_loc], [777], 1e6)
    np.testing.assert_allclose(a, b, atol=1e-12)
    # the first local token as the only visible key gives its value
    one, _ = oracle.attend(q[:, :1], empty, [0], lk, lv, [1], [3], 1e6)
    np.testing.assert_allclose(one[0, 0], np.repeat(lv[0, 0], hq // hkv, axis=0), atol=1e-14)
