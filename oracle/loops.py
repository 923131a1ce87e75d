"""Pure-Python brute-force twin of the oracle for tiny inputs (test infra).

Written independently of ``msa_oracle``: RoPE is done as a complex product
(pair (x_j, x_{j+D/2}) as x_j + i*x_{j+D/2}, times exp(i*p*omega_j)),
cosines as explicit dot products, top-k by sorting on the definition's key,
attention with an explicit softmax loop.  Only for banks of a few documents
of a few tokens; inputs are nested lists or NumPy arrays.
"""

import cmath
import math


def _rot(vec, pos, theta):
    d = len(vec)
    h = d // 2
    out = [0.0] * d
    for j in range(h):
        w = theta ** (-2.0 * j / d)
        z = complex(vec[j], vec[j + h]) * cmath.exp(1j * pos * w)
        out[j] = z.real
        out[j + h] = z.imag
    return out


def pool_doc(k, v, kr, pool_size, theta):
    """k, v: [L][Hkv][D], kr: [L][Hr][dr] -> lists of pooled rows."""
    n_tok = len(k)
    k_bar, v_bar, kr_bar = [], [], []
    c0 = 0
    while c0 < n_tok:
        toks = range(c0, min(c0 + pool_size, n_tok))
        n = len(toks)
        k_bar.append([[sum(_rot(list(k[t][hh]), t, theta)[i] for t in toks) / n
                       for i in range(len(k[0][0]))] for hh in range(len(k[0]))])
        v_bar.append([[sum(float(v[t][hh][i]) for t in toks) / n
                       for i in range(len(v[0][0]))] for hh in range(len(v[0]))])
        kr_bar.append([[sum(float(kr[t][hh][i]) for t in toks) / n
                        for i in range(len(kr[0][0]))] for hh in range(len(kr[0]))])
        c0 += pool_size
    return k_bar, v_bar, kr_bar


def _cos(a, b, eps=1e-8):
    dot = sum(float(x) * float(y) for x, y in zip(a, b))
    na = math.sqrt(sum(float(x) ** 2 for x in a))
    nb = math.sqrt(sum(float(y) ** 2 for y in b))
    return dot / (max(na, eps) * max(nb, eps))


def doc_scores(qr, kr_rows, doc_rows):
    """qr: [B][Tq][Hr][dr]; kr_rows: [n_pool][Hr][dr]; doc_rows: list of
    (first_row, end_row) per document.  Returns [B][n_docs]."""
    out = []
    for qb in qr:
        per_doc = []
        for r0, r1 in doc_rows:
            best = -math.inf
            for j in range(r0, r1):
                for qt in qb:
                    hs = [_cos(qt[h], kr_rows[j][h]) for h in range(len(qt))]
                    best = max(best, sum(hs) / len(hs))
            per_doc.append(best)
        out.append(per_doc)
    return out


def topk(scores, k):
    """scores: [B][n] -> [B][k] document ids (score desc, id asc)."""
    return [sorted(range(len(row)), key=lambda d: (-row[d], d))[:k] for row in scores]


def decode(q, mem_k, mem_v, loc_k, loc_v, pos_offset, theta):
    """One query.  q: [Hq][D]; mem_k/mem_v: [M][Hkv][D]; loc_k/loc_v:
    [T][Hkv][D].  Returns (out [Hq][D], lse [Hq])."""
    n_q, d = len(q), len(q[0])
    n_kv = len(loc_k[0]) if len(loc_k) else len(mem_k[0])
    t_loc = len(loc_k)
    outs, lses = [], []
    for h in range(n_q):
        g = h // (n_q // n_kv)
        qh = _rot(list(q[h]), pos_offset + t_loc - 1, theta)
        keys = [list(map(float, mk[g])) for mk in mem_k]
        keys += [_rot(list(loc_k[i][g]), pos_offset + i, theta) for i in range(t_loc)]
        vals = [list(map(float, mv[g])) for mv in mem_v] + [list(map(float, lv[g])) for lv in loc_v]
        logits = [sum(a * b for a, b in zip(qh, kk)) / math.sqrt(d) for kk in keys]
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        s = sum(w)
        outs.append([sum(w[i] * vals[i][e] for i in range(len(w))) / s for e in range(d)])
        lses.append(m + math.log(s))
    return outs, lses


def attend(q, mem_k, mem_v, loc_k, loc_v, pos_offset, theta):
    """A block of query tokens, one at a time.  q: [Tq][Hq][D] are the last
    Tq of the T local tokens; token t is local token i = T - Tq + t and reads
    the memory and the local tokens 0 .. i.  Returns (out [Tq][Hq][D],
    lse [Tq][Hq])."""
    n_t, t_loc = len(q), len(loc_k)
    outs, lses = [], []
    for t in range(n_t):
        i = t_loc - n_t + t
        n_q, d = len(q[t]), len(q[t][0])
        n_kv = len(loc_k[0]) if len(loc_k) else len(mem_k[0])
        o_t, l_t = [], []
        for h in range(n_q):
            g = h // (n_q // n_kv)
            qh = _rot(list(q[t][h]), pos_offset + i, theta)
            keys = [list(map(float, mk[g])) for mk in mem_k]
            keys += [_rot(list(loc_k[j][g]), pos_offset + j, theta) for j in range(i + 1)]
            vals = [list(map(float, mv[g])) for mv in mem_v] + [list(map(float, loc_v[j][g])) for j in range(i + 1)]
            logits = [sum(a * b for a, b in zip(qh, kk)) / math.sqrt(d) for kk in keys]
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            s = sum(w)
            o_t.append([sum(w[j] * vals[j][e] for j in range(len(w))) / s for e in range(d)])
            l_t.append(m + math.log(s))
        outs.append(o_t)
        lses.append(l_t)
    return outs, lses
