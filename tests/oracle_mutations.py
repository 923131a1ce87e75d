"""Planted mistakes in the CPU oracle, for checking that its pins catch them.

Each mutation is a textual edit of oracle/msa_oracle.py: a plausible slip
(a dropped term, a wrong sign, exponent or index, a transposed rule).
apply(name) executes the edited source in place of the oracle's module, so
every later `oracle.<function>` call runs the mutated code; the pure-Python
twin in oracle/loops.py is left as it is.  tests/conftest.py applies the
mutation named by the ORACLE_MUTATION environment variable, and
tests/test_oracle_mutations.py runs the pins once per mutation, each in a
process of its own, expecting a failure every time.  Only the tests
use this; it runs on the CPU.
"""

# name -> [(old text, new text, how many occurrences to replace (0 = all))]
MUTATIONS = {
    # RoPE
    "rope_exponent_half": [("-2.0 * j / head_dim", "-1.0 * j / head_dim", 0)],
    "rope_interleaved_pairs": [("    x1 = x[..., :h]\n    x2 = x[..., h:]\n    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)",
                                "    x1 = x[..., 0::2]\n    x2 = x[..., 1::2]\n    o = np.empty_like(x)\n"
                                "    o[..., 0::2] = x1 * c - x2 * s\n    o[..., 1::2] = x2 * c + x1 * s\n    return o", 0)],
    "rope_sign": [("x1 * c - x2 * s, x2 * c + x1 * s", "x1 * c + x2 * s, x2 * c - x1 * s", 0)],
    "rope_dropped_in_pool": [("k_rot = rope(k, np.arange(n_tok), theta)", "k_rot = k", 0)],
    "rope_positions_not_reset": [("k_rot = rope(k, np.arange(n_tok), theta)", "k_rot = rope(k, np.arange(n_tok) + 3, theta)", 0)],
    # pooling
    "pool_sum_not_mean": [("k_bar[c] = k_rot[a:b].mean(axis=0)", "k_bar[c] = k_rot[a:b].sum(axis=0)", 0),
                          ("v_bar[c] = v[a:b].mean(axis=0)", "v_bar[c] = v[a:b].sum(axis=0)", 0),
                          ("kr_bar[c] = kr[a:b].mean(axis=0)", "kr_bar[c] = kr[a:b].sum(axis=0)", 0)],
    "pool_tail_divides_by_P": [("v_bar[c] = v[a:b].mean(axis=0)", "v_bar[c] = v[a:b].sum(axis=0) / pool_size", 0)],
    "pool_chunk_off_by_one": [("a, b = c * pool_size, min((c + 1) * pool_size, n_tok)",
                               "a, b = c * pool_size, min((c + 1) * pool_size + 1, n_tok)", 0)],
    # routing
    "no_head_mean": [('q, k, optimize=True) / n_heads', 'q, k, optimize=True)', 0)],
    "token_mean_not_max": [("s = row_scores(qr, kr_pooled).max(axis=1)", "s = row_scores(qr, kr_pooled).mean(axis=1)", 0)],
    "doc_sum_not_max": [("np.maximum.reduceat(s, pool_off[:-1], axis=1)", "np.add.reduceat(s, pool_off[:-1], axis=1)", 0)],
    "unnormalised_key": [("    k = _unit(np.asarray(kr_pooled, dtype=F64))", "    k = np.asarray(kr_pooled, dtype=F64)", 0)],
    "eps_clamp_large": [("EPS = 1e-8", "EPS = 1e-1", 0)],
    # top-k and assembly
    "topk_ties_to_higher_id": [("np.lexsort((ids, -row))", "np.lexsort((-ids, -row))", 0)],
    "topk_ascending": [("np.lexsort((ids, -row))", "np.lexsort((ids, row))", 0)],
    "assemble_skips_instead_of_dropping": [("            if lens[b] + (r1 - r0) > mem_cap:\n                break",
                                            "            if lens[b] + (r1 - r0) > mem_cap:\n                continue", 0)],
    "assemble_capacity_off_by_one": [("if lens[b] + (r1 - r0) > mem_cap:", "if lens[b] + (r1 - r0) >= mem_cap:", 0)],
    # decode
    "decode_query_position_off_by_one": [("q_rot = rope(q[b][None], [o + t_loc - 1], theta)[0]",
                                          "q_rot = rope(q[b][None], [o + t_loc], theta)[0]", 0)],
    "decode_local_keys_without_offset": [("k_loc = rope(np.asarray(local_k[b, :t_loc], dtype=F64), o + np.arange(t_loc), theta)",
                                          "k_loc = rope(np.asarray(local_k[b, :t_loc], dtype=F64), np.arange(t_loc), theta)", 1)],
    "decode_gqa_modulo": [("            g = h // group", "            g = h % n_kv", 1)],
    "decode_scale_one_over_d": [("scale = 1.0 / np.sqrt(d)", "scale = 1.0 / d", 1)],
    "decode_values_from_keys": [("vals = np.concatenate([np.asarray(mem_kv[b, :m_len, 1], dtype=F64),",
                                 "vals = np.concatenate([np.asarray(mem_kv[b, :m_len, 0], dtype=F64),", 1)],
    # block attention
    "attend_not_causal": [("((j[None, :] - m_len) <= i_t[:, None])", "((j[None, :] - m_len) < t_loc)", 0)],
    "attend_token_position_off_by_one": [("i_t = t_loc - n_t + np.arange(n_t)", "i_t = t_loc - n_t + 1 + np.arange(n_t)", 0)],
    # storage rounding
    "bf16_truncates": [("q = np.rint(np.ldexp(x, -shift))", "q = np.trunc(np.ldexp(x, -shift))", 0)],
    "bf16_one_bit_short": [("shift = np.maximum(e - 8, -133)", "shift = np.maximum(e - 7, -133)", 0)],
}


def apply(name):
    """Replace the oracle's functions by those of the mutated source."""
    import oracle
    import oracle.msa_oracle as mo

    with open(mo.__file__) as f:
        src = f.read()
    for old, new, count in MUTATIONS[name]:
        n = src.count(old)
        if n == 0:
            raise RuntimeError(f"mutation {name}: text not found in the oracle: {old[:60]!r}")
        src = src.replace(old, new, count if count else n)
    exec(compile(src, mo.__file__, "exec"), mo.__dict__)
    for attr in dir(oracle):
        if not attr.startswith("_") and hasattr(mo, attr):
            setattr(oracle, attr, getattr(mo, attr))
