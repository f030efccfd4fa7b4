"""Pin strength: copies of the oracle with one planted mistake each must fail
at least one pin.  The mutants are compiled from the oracle source with gcc
into a temporary directory; nothing here touches a GPU."""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

# (name, exact text in mla_oracle.c, replacement, which occurrence (0-based) or None for all)
MUTANTS = [
    ("drop_rope_term", "s[t] = scale * (content + rope);", "s[t] = scale * (content);", 0),
    ("rope_sign", "s[t] = scale * (content + rope);", "s[t] = scale * (content - rope);", 0),
    ("latent_no_scale", "s[t] = scale * acc;", "s[t] = acc;", 0),
    ("latent_drop_rope_cols", "for (int i = 0; i < d; ++i) acc += q[i] * row[i];",
     "for (int i = 0; i < d_c; ++i) acc += q[i] * row[i];", 0),
    ("uk_transposed_in_expanded", "w_uk[IDX3(hi, j, c, d_k, d_c)]", "w_uk[IDX3(hi, c, j, d_c, d_k)]", 0),
    ("uk_transposed_in_absorb", "w_uk[IDX3(hi, j, c, d_k, d_c)]", "w_uk[IDX3(hi, c, j, d_c, d_k)]", 1),
    ("uv_transposed_in_expanded", "w_uv[IDX3(hi, c, j, d_c, d_v)]", "w_uv[IDX3(hi, j, c, d_v, d_c)]", 0),
    ("uv_transposed_in_absorb", "w_uv[IDX3(hi, c, j, d_c, d_v)]", "w_uv[IDX3(hi, j, c, d_v, d_c)]", 1),
    ("lse_without_max", "return m + log(l);", "return log(l);", 0),
    ("softmax_unnormalised", "for (int t = 0; t < n; ++t) p[t] /= l;", "", 0),
    ("max_sign", "p[t] = exp(s[t] - m);", "p[t] = exp(m - s[t]);", 0),
    ("value_uses_shifted_cols", "o[c] += p[t] * row[c];", "o[c] += p[t] * row[c + 1];", 0),
    ("last_token_dropped", "const int L = clamp_len(seqlens[bi], t_max);",
     "const int L = clamp_len(seqlens[bi] - 1, t_max);", None),
    ("rope_copy_wrong_offset", "qp[d_c + r] = q_rope[IDX2(bh, r, d_r)];",
     "qp[d_c + r] = q_rope[IDX2(bh, 0, d_r)];", 0),
    ("wrong_head_in_expanded_query", "const double* qn = q_nope + IDX3(bi, hi, 0, h, d_k);",
     "const double* qn = q_nope + IDX3(bi, 0, 0, h, d_k);", 0),
    ("causal_limit_off_by_one", "int n = L - q_len + 1 + qi;", "int n = L - q_len + qi;", 0),
    ("causal_no_mask", "int n = L - q_len + 1 + qi;", "int n = L;", 0),
    ("causal_reversed_tokens", "int n = L - q_len + 1 + qi;", "int n = L - qi;", 0),
    ("append_rope_sign", "row[d_c + 2 * j] = r0 * cs - r1 * sn;", "row[d_c + 2 * j] = r0 * cs + r1 * sn;", 0),
    ("append_rope_pairs_swapped", "row[d_c + 2 * j + 1] = r0 * sn + r1 * cs;",
     "row[d_c + 2 * j + 1] = r1 * sn + r0 * cs;", 0),
    ("append_wrong_row", "double* row = cache + IDX3(bi, pos, 0, t_max, d);",
     "double* row = cache + IDX3(bi, pos > 0 ? pos - 1 : 0, 0, t_max, d);", 0),
    ("append_wrong_table_row", "const double cs = cos_tab[IDX2(pos, j, d_r / 2)]",
     "const double cs = cos_tab[IDX2(0, j, d_r / 2)]", 0),
]


def _mutate(src, old, new, which):
    assert old in src, old
    if which is None:
        return src.replace(old, new)
    idx = -1
    for _ in range(which + 1):
        idx = src.index(old, idx + 1)
    return src[:idx] + new + src[idx + len(old):]


@pytest.mark.parametrize("name,old,new,which", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, which):
    src = open(oracle.SRC).read()
    msrc = tmp_path / ("mutant_%s.c" % name)
    msrc.write_text(_mutate(src, old, new, which))
    so = oracle.compile_source(str(msrc), str(tmp_path / ("mutant_%s.so" % name)))
    mut = oracle.Oracle(so)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mut)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "planted mistake %r passed every pin" % name
