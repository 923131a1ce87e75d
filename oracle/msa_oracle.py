"""Plain float64 definition of the MSA hot path (test infrastructure only).

The method, restated from the pages (see the package docstring for the page
titles [HL], [TM], [GF]):

1. Offline memory encoding: each document's keys K, values V and router
   keys Kr are mean-pooled over fixed-size chunks, giving the cached pooled
   triples (K_bar, V_bar, Kr_bar) ([HL] "How MSA compresses and routes
   documents"; [TM] "Architectural Design and Inference", stage 1).
   Positions restart at zero inside every document (document-wise RoPE,
   same sections).
2. Online routing: the projected query Qr is compared with every pooled
   router key by cosine similarity, averaged over router heads, maximised
   over tokens, and the top-k documents are selected ([HL], [TM] stage 2).
3. Context assembly: the pooled K/V of the chosen documents, in rank
   order, followed by the query's own K/V ([HL]; [TM] stage 2).
4. Sparse generation: attention over that assembled context, with the
   query's start position offset by k, the number of retrieved documents,
   keeping the order background -> query -> generation ([HL]; [TM] stage 3).

Readings where the pages are silent:

* R1 chunk = P consecutive tokens of one document; a tail chunk of n < P
  tokens is the plain mean of those n tokens; chunks never cross documents.
* R2 only K is rotated before pooling (each token at its in-document
  position, then averaged); V and Kr are not rotated.
* R3 RoPE is the rotate-half form with inverse frequencies
  theta^(-2j/D), j < D/2.
* R4 the maximum over tokens covers the query tokens and the pooled rows
  of a document (max of max, so both readings agree).
* R5 cosine uses max(||x||, 1e-8) per vector.
* R6 top-k orders by score descending, then document id ascending.
* R7 assembled memory = the selected documents' pooled rows in rank order;
  a document that would overflow the memory capacity is dropped together
  with every lower-ranked one.
* R8 decode: the query token sits at position o + T - 1 and local token i
  at o + i, where o is the position offset (k by default) and T the local
  length; pooled memory keys are used as stored (already document-wise
  rotated); one softmax over [memory ; local] with scale 1/sqrt(D); query
  head h reads KV head h // (Hq / Hkv).
* R9 every cast to bfloat16 rounds to nearest, ties to even.
* R13 a block of Tq query tokens (prefill through the sparse context) is
  the last Tq tokens of the local context: with T local tokens, token t of
  the block is local token i_t = T - Tq + t at position o + i_t; it sees
  every memory row and the local tokens 0 .. i_t (causal); Tq = 1 is the
  decode step of R8.  The pages order the context background -> query ->
  generation and give no block form, so this is the plainest extension.
"""

import numpy as np

EPS = 1e-8

F64 = np.float64


# --------------------------------------------------------------------------
# storage rounding (reading R9)
# --------------------------------------------------------------------------

def round_to_bf16(x):
    """Round to the nearest bfloat16 value (ties to even); returns float64.

    bfloat16 keeps 8 significant bits with float32's exponent range, so in
    the binade 2^(e-1) <= |x| < 2^e the spacing is 2^(e-8); below the
    smallest normal (2^-126) the spacing is the subnormal step 2^-133.
    """
    x = np.asarray(x, dtype=F64)
    _, e = np.frexp(x)
    shift = np.maximum(e - 8, -133)
    q = np.rint(np.ldexp(x, -shift))          # exact power-of-two scaling
    out = np.ldexp(q, shift)
    big = np.abs(out) >= 2.0 ** 128           # beyond the largest finite bf16
    return np.where(big, np.copysign(np.inf, x), out)


def round_to_storage(x, dtype):
    """Round float64 values to the storage type 'f32' or 'bf16'."""
    x = np.asarray(x, dtype=F64)
    if dtype == "f32":
        return x.astype(np.float32).astype(F64)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f64":
        return x
    raise ValueError(f"unknown storage dtype {dtype!r}")


# --------------------------------------------------------------------------
# RoPE (reading R3); document-wise positions from [HL]/[TM]
# --------------------------------------------------------------------------

def rope_inv_freq(head_dim, theta):
    """omega_j = theta^(-2j/D) for j = 0 .. D/2-1, in float64."""
    j = np.arange(head_dim // 2, dtype=F64)
    return np.power(F64(theta), -2.0 * j / head_dim)


def rope(x, pos, theta):
    """Rotate x[n, ..., D] at positions pos[n] (rotate-half pairs j, j+D/2)."""
    x = np.asarray(x, dtype=F64)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(pos, dtype=F64)[:, None] * rope_inv_freq(d, theta)[None, :]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (h,)
    c = np.cos(ang).reshape(shape)
    s = np.sin(ang).reshape(shape)
    x1 = x[..., :h]
    x2 = x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# --------------------------------------------------------------------------
# stage 1: chunk-mean pooling with document-wise RoPE (readings R1, R2)
# --------------------------------------------------------------------------

def pool_offsets(doc_lens, pool_size):
    """Row offsets of each document in the pooled bank: prefix of ceil(L/P)."""
    doc_lens = np.asarray(doc_lens, dtype=np.int64)
    if np.any(doc_lens < 1):
        raise ValueError("every document needs at least one token")
    rows = -(-doc_lens // pool_size)
    return np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)


def pool_doc(k, v, kr, pool_size, theta, out_dtype="f64"):
    """Pool one document.  k, v: [L, Hkv, D]; kr: [L, Hr, dr].

    Token t of the document is rotated at position t (positions restart at
    zero per document), then every chunk [cP, min((c+1)P, L)) is averaged.
    Returns (k_bar, v_bar, kr_bar) rounded to out_dtype.
    """
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    kr = np.asarray(kr, dtype=F64)
    n_tok = k.shape[0]
    n_chunks = -(-n_tok // pool_size)
    k_rot = rope(k, np.arange(n_tok), theta)
    k_bar = np.empty((n_chunks,) + k.shape[1:], dtype=F64)
    v_bar = np.empty((n_chunks,) + v.shape[1:], dtype=F64)
    kr_bar = np.empty((n_chunks,) + kr.shape[1:], dtype=F64)
    for c in range(n_chunks):
        a, b = c * pool_size, min((c + 1) * pool_size, n_tok)
        k_bar[c] = k_rot[a:b].mean(axis=0)
        v_bar[c] = v[a:b].mean(axis=0)
        kr_bar[c] = kr[a:b].mean(axis=0)
    return (round_to_storage(k_bar, out_dtype),
            round_to_storage(v_bar, out_dtype),
            round_to_storage(kr_bar, out_dtype))


def pool(k, v, kr, doc_tok_off, pool_size, theta, out_dtype="f64"):
    """Pool a packed bank of documents.

    k, v: [T, Hkv, D]; kr: [T, Hr, dr]; doc_tok_off: [n_docs+1] token
    offsets.  Returns (kv_pooled [n_pool, 2, Hkv, D], kr_pooled
    [n_pool, Hr, dr], doc_pool_off [n_docs+1]); K and V of one pooled row
    sit next to each other so that a document is one contiguous range.
    """
    doc_tok_off = np.asarray(doc_tok_off, dtype=np.int64)
    lens = np.diff(doc_tok_off)
    pool_off = pool_offsets(lens, pool_size)
    n_pool = int(pool_off[-1])
    kv = np.empty((n_pool, 2) + tuple(k.shape[1:]), dtype=F64)
    krp = np.empty((n_pool,) + tuple(kr.shape[1:]), dtype=F64)
    for d in range(len(lens)):
        a, b = doc_tok_off[d], doc_tok_off[d + 1]
        kb, vb, rb = pool_doc(k[a:b], v[a:b], kr[a:b], pool_size, theta, out_dtype)
        r0, r1 = pool_off[d], pool_off[d + 1]
        kv[r0:r1, 0] = kb
        kv[r0:r1, 1] = vb
        krp[r0:r1] = rb
    return kv, krp, pool_off


# --------------------------------------------------------------------------
# stage 2: routing (readings R4, R5, R6)
# --------------------------------------------------------------------------

def _unit(x):
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    return x / np.maximum(n, EPS)


def row_scores(qr, kr_pooled):
    """s[b, t, j] = mean over router heads h of cos(Qr[b,t,h], Kr_bar[j,h]).

    qr: [B, Tq, Hr, dr]; kr_pooled: [n_pool, Hr, dr].
    """
    q = _unit(np.asarray(qr, dtype=F64))
    k = _unit(np.asarray(kr_pooled, dtype=F64))
    n_heads = q.shape[2]
    # the sum over h and d of the unit vectors' products = sum of per-head cosines
    return np.einsum("bthd,nhd->btn", q, k, optimize=True) / n_heads


def doc_scores(qr, kr_pooled, doc_pool_off):
    """Dsc[b, d] = max over query tokens t and over the rows j of document d
    of s[b, t, j].  Slicing a bank at document boundaries gives exactly the
    scores of those documents, which is how large banks are scored in
    blocks."""
    pool_off = np.asarray(doc_pool_off, dtype=np.int64)
    if np.any(np.diff(pool_off) < 1):
        raise ValueError("every document needs at least one pooled row")
    s = row_scores(qr, kr_pooled).max(axis=1)                 # [B, n_pool]
    return np.maximum.reduceat(s, pool_off[:-1], axis=1)      # [B, n_docs]


def topk(dsc, k):
    """Per query: the k documents with the highest score, ties to the lower
    document id, in that order.  Returns (idx int64 [B, k], score [B, k])."""
    dsc = np.asarray(dsc, dtype=F64)
    n = dsc.shape[1]
    if not 1 <= k <= n:
        raise ValueError("need 1 <= k <= n_docs")
    ids = np.arange(n)
    idx = np.stack([np.lexsort((ids, -row))[:k] for row in dsc])
    return idx.astype(np.int64), np.take_along_axis(dsc, idx, axis=1)


# --------------------------------------------------------------------------
# context assembly (reading R7)
# --------------------------------------------------------------------------

def assemble(kv_pooled, doc_pool_off, idx, mem_cap, start_len=None, mem=None):
    """Concatenate the selected documents' pooled rows in rank order.

    kv_pooled: [n_pool, 2, Hkv, D] (any dtype, copied bit for bit);
    idx: [B, k] document ids.  Rows are appended after start_len[b] (0 by
    default) into mem [B, mem_cap, 2, Hkv, D] (zero-filled when not given).
    Documents are taken in rank order while they fit; the first one that
    does not fit is dropped with every lower-ranked one.
    Returns (mem, mem_len [B], n_taken [B]).
    """
    kv_pooled = np.asarray(kv_pooled)
    pool_off = np.asarray(doc_pool_off, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    n_b = idx.shape[0]
    if mem is None:
        mem = np.zeros((n_b, mem_cap) + kv_pooled.shape[1:], dtype=kv_pooled.dtype)
    lens = np.zeros(n_b, dtype=np.int64) if start_len is None else np.array(start_len, dtype=np.int64)
    taken = np.zeros(n_b, dtype=np.int64)
    for b in range(n_b):
        for d in idx[b]:
            r0, r1 = pool_off[d], pool_off[d + 1]
            if lens[b] + (r1 - r0) > mem_cap:
                break
            mem[b, lens[b]:lens[b] + (r1 - r0)] = kv_pooled[r0:r1]
            lens[b] += r1 - r0
            taken[b] += 1
    return mem, lens, taken


# --------------------------------------------------------------------------
# stage 3: sparse decode attention (reading R8)
# --------------------------------------------------------------------------

def decode(q, mem_kv, mem_len, local_k, local_v, local_len, pos_offset,
           theta, scale=None, out_dtype="f64"):
    """One decode-attention step over [pooled memory ; local context].

    q: [B, Hq, D] (before RoPE); mem_kv: [B, M_cap, 2, Hkv, D];
    local_k, local_v: [B, T_cap, Hkv, D] (K before RoPE);
    mem_len, local_len, pos_offset: [B].
    Returns (out [B, Hq, D] rounded to out_dtype, lse [B, Hq] float64);
    a query with no keys at all gets out = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=F64)
    n_b, n_q, d = q.shape
    n_kv = np.asarray(local_k).shape[2]
    group = n_q // n_kv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((n_b, n_q, d), dtype=F64)
    lse = np.full((n_b, n_q), -np.inf, dtype=F64)
    for b in range(n_b):
        o, t_loc, m_len = int(pos_offset[b]), int(local_len[b]), int(mem_len[b])
        q_rot = rope(q[b][None], [o + t_loc - 1], theta)[0]                     # [Hq, D]
        k_loc = rope(np.asarray(local_k[b, :t_loc], dtype=F64), o + np.arange(t_loc), theta)
        keys = np.concatenate([np.asarray(mem_kv[b, :m_len, 0], dtype=F64), k_loc], axis=0)
        vals = np.concatenate([np.asarray(mem_kv[b, :m_len, 1], dtype=F64),
                               np.asarray(local_v[b, :t_loc], dtype=F64)], axis=0)
        if keys.shape[0] == 0:
            continue
        for h in range(n_q):
            g = h // group
            logits = scale * (keys[:, g, :] @ q_rot[h])
            m = logits.max()
            w = np.exp(logits - m)
            den = w.sum()
            out[b, h] = (w @ vals[:, g, :]) / den
            lse[b, h] = m + np.log(den)
    return round_to_storage(out, out_dtype), lse


# --------------------------------------------------------------------------
# a block of query tokens through the sparse context (reading R13)
# --------------------------------------------------------------------------

def attend(q, mem_kv, mem_len, local_k, local_v, local_len, pos_offset,
           theta, scale=None, out_dtype="f64"):
    """Attention of Tq query tokens over [pooled memory ; causal local].

    q: [B, Tq, Hq, D] (before RoPE), the last Tq tokens of each local
    context; mem_kv: [B, M_cap, 2, Hkv, D]; local_k, local_v:
    [B, T_cap, Hkv, D] (K before RoPE); mem_len, local_len, pos_offset: [B].
    Written as the masked definition: logits of every query row against
    every key, keys a token may not see set to -inf, one softmax per row.
    Returns (out [B, Tq, Hq, D] rounded to out_dtype, lse [B, Tq, Hq]
    float64); a row that sees no key gets out = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=F64)
    n_b, n_t, n_q, d = q.shape
    n_kv = np.asarray(local_k).shape[2]
    group = n_q // n_kv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((n_b, n_t, n_q, d), dtype=F64)
    lse = np.full((n_b, n_t, n_q), -np.inf, dtype=F64)
    for b in range(n_b):
        o, t_loc, m_len = int(pos_offset[b]), int(local_len[b]), int(mem_len[b])
        i_t = t_loc - n_t + np.arange(n_t)                                  # local index of each token
        q_rot = rope(q[b], o + i_t, theta)                                  # [Tq, Hq, D]
        k_loc = rope(np.asarray(local_k[b, :t_loc], dtype=F64), o + np.arange(t_loc), theta)
        keys = np.concatenate([np.asarray(mem_kv[b, :m_len, 0], dtype=F64), k_loc], axis=0)
        vals = np.concatenate([np.asarray(mem_kv[b, :m_len, 1], dtype=F64),
                               np.asarray(local_v[b, :t_loc], dtype=F64)], axis=0)
        j = np.arange(m_len + t_loc)
        visible = (j[None, :] < m_len) | ((j[None, :] - m_len) <= i_t[:, None])   # [Tq, M + T]
        for h in range(n_q):
            g = h // group
            logits = scale * (q_rot[:, h, :] @ keys[:, g, :].T)             # [Tq, M + T]
            logits = np.where(visible, logits, -np.inf)
            for t in range(n_t):
                if not visible[t].any():
                    continue
                m = logits[t].max()
                w = np.exp(logits[t] - m)
                den = w.sum()
                out[b, t, h] = (w @ vals[:, g, :]) / den
                lse[b, t, h] = m + np.log(den)
    return round_to_storage(out, out_dtype), lse

