"""Comparison rules shared by the GPU parity tests.

Tolerances (floating point; integer/byte work is compared exactly):
* pooled vectors: fp32 per (row, head) ||g - u|| <= 1e-3 ||u||, u the exact
  oracle value; bf16 see check_pool (one bf16 step of u elementwise, and at
  most 1% of elements off the correctly rounded value).
* document scores: |g - r| <= 2e-3 absolute.
* top-k: with tau = 2e-3 and the oracle's k-th score s_k, every document with
  oracle score > s_k + tau is selected and every selected document has
  oracle score >= s_k - tau; where the gap exceeds tau the sets agree.
* decode: per (query, head) ||g - r|| <= 2e-2 ||r|| for bf16, 1e-4 for fp32;
  the log-sum-exp within lse_bound (the rounding the arithmetic allows).
"""

import numpy as np
import torch

TAU = 2e-3
POOL_REL = 1e-3
DECODE_REL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def np64(t):
    """Tensor (any device, fp32/bf16/int) -> numpy float64 / int64 copy."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    if t.is_floating_point():
        return t.double().numpy()
    return t.long().numpy()


def storage(dtype):
    return "bf16" if dtype == torch.bfloat16 else "f32"


def bf16_step(x):
    """Spacing of bf16 numbers at |x| (float64)."""
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def check_pool(got, ref_exact, dtype, what=""):
    """got: GPU pooled vectors [..., D]; ref_exact: the oracle's unrounded
    float64 values.

    fp32 storage: per vector ||g - u|| <= 1e-3 ||u||.
    bf16 storage: every element lies within one bf16 step of the exact value
    (slack 1e-5 ||u|| per vector for fp32 cancellation), and at most 1% of
    the elements differ from the correctly rounded oracle value.  A bf16
    result rounded from an fp32 accumulation equals the rounded oracle except
    where the two pre-rounding values straddle a rounding boundary (about 3
    in 10^4 elements); a pre-rounding error of 1e-3 relative would flip about
    a quarter of them, so the rate cap is the stricter test.
    """
    got = np.asarray(got, dtype=np.float64)
    u = np.asarray(ref_exact, dtype=np.float64)
    assert got.shape == u.shape, (got.shape, u.shape)
    norm = np.linalg.norm(u, axis=-1, keepdims=True)
    if dtype != torch.bfloat16:
        err = np.linalg.norm(got - u, axis=-1)
        lim = POOL_REL * norm[..., 0] + 1e-6
        bad = err > lim
        assert not bad.any(), f"{what}: {bad.sum()} vectors over the normwise bound; worst ratio " \
                              f"{np.max(err / lim):.3g} at {np.argwhere(bad)[:3].tolist()}"
        return
    r = oracle_round_bf16(u)
    off = np.abs(got - u) > bf16_step(u) * (1 + 1e-9) + 1e-5 * norm
    assert not off.any(), f"{what}: {off.sum()} elements beyond one bf16 step, e.g. at " \
                          f"{np.argwhere(off)[:3].tolist()}"
    rate = float(np.mean(got != r))
    assert rate <= 0.01, f"{what}: {rate:.2%} of elements differ from the correctly rounded value"
    return rate


def oracle_round_bf16(x):
    import oracle
    return oracle.round_to_bf16(x)


def check_scores(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    assert d.max() <= TAU, f"{what}: score error {d.max():.3g} > {TAU} at {np.unravel_index(d.argmax(), d.shape)}"


def check_topk(idx_gpu, dsc_ref, k, what=""):
    """idx_gpu: [B, k] selected ids; dsc_ref: [B, n_docs] oracle scores."""
    idx_gpu = np.asarray(idx_gpu)
    for b in range(idx_gpu.shape[0]):
        sel = idx_gpu[b]
        assert len(set(sel.tolist())) == k, f"{what}: query {b} repeats a document"
        assert sel.min() >= 0 and sel.max() < dsc_ref.shape[1]
        s = dsc_ref[b]
        s_k = np.sort(s)[::-1][k - 1]
        must = np.nonzero(s > s_k + TAU)[0]
        assert set(must.tolist()) <= set(sel.tolist()), f"{what}: query {b} misses clear winners"
        assert np.all(s[sel] >= s_k - TAU), f"{what}: query {b} selected a clear loser"


def check_topk_order(idx_gpu, score_gpu, what=""):
    """Returned in score-descending order, ties by ascending id."""
    idx_gpu = np.asarray(idx_gpu)
    score_gpu = np.asarray(score_gpu)
    for b in range(idx_gpu.shape[0]):
        for i in range(idx_gpu.shape[1] - 1):
            s0, s1 = score_gpu[b, i], score_gpu[b, i + 1]
            assert s0 > s1 or (s0 == s1 and idx_gpu[b, i] < idx_gpu[b, i + 1]), f"{what}: order at {b},{i}"


def check_decode(got, ref, dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.array_equal(np.isfinite(got), np.isfinite(ref)), f"{what}: non-finite values where the reference has none"
    err = np.linalg.norm(got - ref, axis=-1)
    lim = DECODE_REL[dtype] * np.linalg.norm(ref, axis=-1) + 1e-6
    bad = err > lim
    assert not bad.any(), f"{what}: {bad.sum()} heads over bound; worst ratio {np.max(err / lim):.3g} " \
                          f"at {np.argwhere(bad)[:3].tolist()}"


def lse_bound(q, mem_k, mem_len, local_k, local_len, dtype):
    """Per (query, head): the largest log-sum-exp error the decode's
    arithmetic allows.  bf16: each locally rotated key is rounded to bf16
    once (|dk| <= 2^-9 |k|) and the rotated, scaled query is kept as two bf16
    terms (|dq| <= 2^-16 |q|), so a logit moves by at most
    scale |q| (2^-9 max|k_local| + 2^-16 max|k|), and the log-sum-exp by at
    most the largest logit change; plus 1e-5 for fp32 sums.  fp32 inputs:
    1e-4 (fp32 logits, exp2 and log2 of the vector units).
    q [B, Hq, D]; mem_k [B, M_cap, Hkv, D] (or None); local_k [B, T_cap, Hkv, D]."""
    q = np.asarray(q, dtype=np.float64)
    n_b, n_q, d = q.shape
    if dtype != torch.bfloat16:
        return np.full((n_b, n_q), 1e-4)
    n_kv = np.asarray(local_k).shape[2]
    grp = n_q // n_kv
    out = np.empty((n_b, n_q))
    for b in range(n_b):
        kl = np.linalg.norm(np.asarray(local_k[b, :local_len[b]], dtype=np.float64), axis=-1)   # [T, Hkv]
        km = (np.linalg.norm(np.asarray(mem_k[b, :mem_len[b]], dtype=np.float64), axis=-1)
              if mem_k is not None and mem_len[b] > 0 else np.zeros((0, n_kv)))
        for h in range(n_q):
            g = h // grp
            ml = kl[:, g].max() if kl.shape[0] else 0.0
            ma = max(ml, km[:, g].max() if km.shape[0] else 0.0)
            out[b, h] = np.linalg.norm(q[b, h]) / np.sqrt(d) * (2.0 ** -9 * ml + 2.0 ** -16 * ma) + 1e-5
    return out
