"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with what the pages or the mathematics fix.  ``test_oracle_pins``
runs every pin on the real oracle; ``test_oracle_mutants`` runs them on copies
of the oracle with a planted mistake and requires that some pin fails.

Kinds of pin used (none re-types the oracle's own loops):
  * the two absorption identities the glossary page asserts to 1e-10
    (latent scores == expanded scores, (sum p c) W_UV == sum p (c W_UV)),
    comparing the oracle's two independent forms;
  * a library routine on a special case: torch's scaled_dot_product_attention
    in fp64 on the CPU (one shared K/V "head" = the latent rows), and numpy
    einsum for the absorbs;
  * closed forms: zero query (uniform softmax), one token, identical rows,
    identity up-projections;
  * invariants: constant score shift, token permutation, equal heads,
    split-and-merge of the token set (log-sum-exp combine), rows summing to 1.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
SCALE = 1.0 / math.sqrt(192.0)


def _rng(seed):
    return np.random.default_rng(seed)


def _toy(seed, b, t, h, dc, dk, dr, dv):
    """Inputs at the glossary check's toy widths, drawn directly from one
    generator: t cached latent rows [c (dc) ; k_R (dr)] per batch row, each
    head's query split into its no-RoPE part (dk) and RoPE part (dr), and the
    two up-projections in this library's layouts, W_UK [h, dk, dc] and
    W_UV [h, dc, dv], scaled by 1/sqrt(contracted width)."""
    g = _rng(seed)
    cache = g.standard_normal((b, t, dc + dr))
    q_nope = g.standard_normal((b, h, dk))
    q_rope = g.standard_normal((b, h, dr))
    w_uk = g.standard_normal((h, dk, dc)) / math.sqrt(dk)
    w_uv = g.standard_normal((h, dc, dv)) / math.sqrt(dc)
    return dict(cache=cache, q_nope=q_nope, q_rope=q_rope, w_uk=w_uk, w_uv=w_uv,
                seqlens=np.full((b,), t, np.int32), scale=1.0 / math.sqrt(dk + dr), dc=dc)


def _close(a, b, tol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, "%s: max|diff| = %.3e > %.1e" % (what, err, tol)
    return err


def pin_glossary_toy_identities(orc):
    """Glossary check at its own dims: expanded and absorbed forms agree to 1e-10."""
    gold = json.load(open(os.path.join(GOLDEN, "glossary_expanded_vs_absorbed.json")))
    d = gold["dims"]
    assert 2 * d["hq"] * d["dv"] == gold["printed_per_token_standard_kv_elements"]
    assert d["dc"] + d["dr"] == gold["printed_mla_cached_elements"]
    tol = gold["assert_atol"]
    for seed in (3, 41, 2024):
        z = _toy(seed, b=d["b"], t=d["t"], h=d["hq"], dc=d["dc"], dk=d["dk"], dr=d["dr"],
                 dv=d["dv"])
        y, lse_x, s_x, _ = orc.decode_unabsorbed(z["q_nope"], z["q_rope"], z["w_uk"], z["w_uv"],
                                                 z["cache"], z["seqlens"], z["scale"],
                                                 want_scores=True)
        qp = orc.absorb_q(z["q_nope"], z["w_uk"], z["q_rope"])
        out, lse_l, s_l = orc.decode_latent(qp, z["cache"], z["seqlens"], z["scale"], d_c=z["dc"],
                                            want_scores=True)
        # content-only scores: zero the rope query on both sides
        zr = np.zeros_like(z["q_rope"])
        _, _, sc_x, _ = orc.decode_unabsorbed(z["q_nope"], zr, z["w_uk"], z["w_uv"], z["cache"],
                                              z["seqlens"], z["scale"], want_scores=True)
        qp0 = orc.absorb_q(z["q_nope"], z["w_uk"], zr)
        _, _, sc_l = orc.decode_latent(qp0, z["cache"], z["seqlens"], z["scale"], d_c=z["dc"],
                                       want_scores=True)
        _close(sc_l, sc_x, tol, "content scores latent vs expanded")
        _close(s_l, s_x, tol, "full scores latent vs expanded")
        _close(lse_l, lse_x, tol, "lse latent vs expanded")
        y_abs = orc.absorb_o(out, z["w_uv"])
        _close(y_abs, y, tol, "absorbed output vs expanded output")


def pin_identities_c1_dims(orc, seed=11):
    """The same identities at production widths (d_c=512, d_r=64, d_k=d_v=128),
    ragged lengths, relative to the magnitude."""
    g = _rng(seed)
    b, h, t_max = 2, 4, 40
    lens = np.array([17, 40], np.int32)
    cache = g.standard_normal((b, t_max, 576))
    q_nope = g.standard_normal((b, h, 128))
    q_rope = g.standard_normal((b, h, 64))
    w_uk = g.standard_normal((h, 128, 512)) / math.sqrt(128)
    w_uv = g.standard_normal((h, 512, 128)) / math.sqrt(512)
    y, lse_x, s_x, _ = orc.decode_unabsorbed(q_nope, q_rope, w_uk, w_uv, cache, lens, SCALE,
                                             want_scores=True)
    qp = orc.absorb_q(q_nope, w_uk, q_rope)
    out, lse_l, s_l = orc.decode_latent(qp, cache, lens, SCALE, want_scores=True)
    m = np.isfinite(s_x)
    assert np.array_equal(m, np.isfinite(s_l))
    _close(s_l[m], s_x[m], 1e-10 * max(1.0, np.abs(s_x[m]).max()), "scores")
    _close(lse_l, lse_x, 1e-10 * max(1.0, np.abs(lse_x).max()), "lse")
    _close(orc.absorb_o(out, w_uv), y, 1e-10 * max(1.0, np.abs(y).max()), "output")


def _sdpa_rows(qp, cache, lens, scale, d_c):
    """torch SDPA (fp64, CPU) with one shared K/V head: K = latent rows, V = rows[:, :d_c]."""
    b, h, _ = qp.shape
    outs = np.zeros((b, h, d_c))
    for i in range(b):
        L = int(lens[i])
        if L == 0:
            continue
        q = torch.from_numpy(qp[i][None, :, None, :])  # [1, h, 1, d]
        k = torch.from_numpy(cache[i, :L])[None, None].expand(1, h, L, cache.shape[2])
        v = torch.from_numpy(cache[i, :L, :d_c])[None, None].expand(1, h, L, d_c)
        o = torch.nn.functional.scaled_dot_product_attention(q, k.contiguous(), v.contiguous(),
                                                             scale=scale)
        outs[i] = o[0, :, 0, :].numpy()
    return outs


def pin_latent_vs_sdpa(orc, seed=12):
    """Latent form == torch SDPA on the special case of one shared K/V head."""
    g = _rng(seed)
    b, h, t_max = 3, 5, 70
    lens = np.array([1, 33, 70], np.int32)
    cache = g.standard_normal((b, t_max, 576))
    qp = g.standard_normal((b, h, 576))
    out, lse = orc.decode_latent(qp, cache, lens, SCALE)
    ref = _sdpa_rows(qp, cache, lens, SCALE, 512)
    _close(out, ref, 1e-12, "latent out vs SDPA")
    # small widths too (generic d_c / d_r)
    cache2 = g.standard_normal((2, 9, 7))
    qp2 = g.standard_normal((2, 3, 7))
    lens2 = np.array([9, 4], np.int32)
    out2, _ = orc.decode_latent(qp2, cache2, lens2, 0.3, d_c=5)
    _close(out2, _sdpa_rows(qp2, cache2, lens2, 0.3, 5), 1e-12, "latent out vs SDPA (small)")


def pin_zero_query(orc, seed=13):
    """q' = 0: uniform softmax, lse = ln L, out = column mean of the latent rows."""
    g = _rng(seed)
    lens = np.array([257, 128, 5], np.int32)
    cache = g.standard_normal((3, 257, 576))
    qp = np.zeros((3, 4, 576))
    out, lse = orc.decode_latent(qp, cache, lens, SCALE)
    for i, L in enumerate(lens):
        _close(lse[i], np.full(4, math.log(L)), 1e-12, "lse = ln L")
        _close(out[i], np.broadcast_to(cache[i, :L, :512].mean(0), (4, 512)), 1e-12, "out = mean")
    assert abs(math.log(4096) - 8.317766166719343) < 1e-12


def pin_single_token(orc, seed=14):
    """L = 1: out = c_0 exactly and lse = the single score."""
    g = _rng(seed)
    cache = g.standard_normal((2, 3, 576))
    qp = g.standard_normal((2, 6, 576))
    lens = np.array([1, 1], np.int32)
    out, lse = orc.decode_latent(qp, cache, lens, SCALE)
    for i in range(2):
        _close(out[i], np.broadcast_to(cache[i, 0, :512], (6, 512)), 0.0, "out = c_0")
        _close(lse[i], SCALE * (qp[i] @ cache[i, 0]), 1e-12, "lse = s_0")


def pin_identical_rows(orc, seed=15):
    """Every cached row identical: out = that row for any query; lse = s + ln L."""
    g = _rng(seed)
    row = g.standard_normal(576)
    L = 37
    cache = np.broadcast_to(row, (1, L, 576)).copy()
    qp = g.standard_normal((1, 3, 576)) * 4.0
    out, lse = orc.decode_latent(qp, cache, np.array([L], np.int32), SCALE)
    _close(out[0], np.broadcast_to(row[:512], (3, 512)), 1e-12, "out = row")
    _close(lse[0], SCALE * (qp[0] @ row) + math.log(L), 1e-12, "lse = s + ln L")


def pin_shift_invariance(orc, seed=16):
    """A constant added to every score leaves out unchanged and moves lse by
    that constant (set cache[..., 575] = 1 and add delta to q'[..., 575])."""
    g = _rng(seed)
    cache = g.standard_normal((2, 50, 576))
    cache[:, :, 575] = 1.0
    qp = g.standard_normal((2, 4, 576))
    lens = np.array([50, 21], np.int32)
    out0, lse0 = orc.decode_latent(qp, cache, lens, SCALE)
    for delta in (3.0, -11.5, 40.0):
        q2 = qp.copy()
        q2[:, :, 575] += delta
        out1, lse1 = orc.decode_latent(q2, cache, lens, SCALE)
        _close(out1, out0, 1e-12, "out under shift")
        _close(lse1 - lse0, np.full_like(lse0, SCALE * delta), 1e-11, "lse shift")


def pin_permutation(orc, seed=17):
    """Permuting the cached tokens changes nothing."""
    g = _rng(seed)
    cache = g.standard_normal((1, 64, 576))
    qp = g.standard_normal((1, 3, 576))
    lens = np.array([64], np.int32)
    out0, lse0 = orc.decode_latent(qp, cache, lens, SCALE)
    perm = g.permutation(64)
    out1, lse1 = orc.decode_latent(qp, cache[:, perm], lens, SCALE)
    _close(out1, out0, 1e-13, "out under permutation")
    _close(lse1, lse0, 1e-13, "lse under permutation")


def pin_equal_heads(orc, seed=18):
    """Heads with equal q' give bit-identical outputs; different heads differ."""
    g = _rng(seed)
    cache = g.standard_normal((1, 30, 576))
    q = g.standard_normal((1, 1, 576))
    qp = np.concatenate([q, q, g.standard_normal((1, 1, 576)), q], axis=1)
    out, lse = orc.decode_latent(qp, cache, np.array([30], np.int32), SCALE)
    assert np.array_equal(out[0, 0], out[0, 1]) and np.array_equal(out[0, 0], out[0, 3])
    assert not np.allclose(out[0, 0], out[0, 2])


def pin_split_merge(orc, seed=19):
    """Splitting the token set A | B: lse = logaddexp(lse_A, lse_B) and
    out = e^(lse_A - lse) out_A + e^(lse_B - lse) out_B."""
    g = _rng(seed)
    L = 90
    cache = g.standard_normal((1, L, 576))
    qp = g.standard_normal((1, 6, 576)) * 2.0
    full_out, full_lse = orc.decode_latent(qp, cache, np.array([L], np.int32), SCALE)
    for cut in (1, 31, 64, 89):
        oa, la = orc.decode_latent(qp, cache[:, :cut], np.array([cut], np.int32), SCALE)
        ob, lb = orc.decode_latent(qp, cache[:, cut:], np.array([L - cut], np.int32), SCALE)
        lse = np.logaddexp(la, lb)
        _close(lse, full_lse, 1e-12, "merged lse")
        out = np.exp(la - lse)[..., None] * oa + np.exp(lb - lse)[..., None] * ob
        _close(out, full_out, 1e-12, "merged out")


def pin_probs_sum_to_one(orc, seed=20):
    """The expanded form's softmax rows sum to 1 and are non-negative."""
    z = _toy(seed, b=1, t=9, h=4, dc=4, dk=5, dr=2, dv=6)
    _, _, _, p = orc.decode_unabsorbed(z["q_nope"], z["q_rope"], z["w_uk"], z["w_uv"], z["cache"],
                                       z["seqlens"], z["scale"], want_scores=True)
    assert np.all(p >= 0.0)
    _close(p.sum(-1), np.ones(p.shape[:2]), 1e-12, "sum p")


def pin_absorbs_vs_numpy(orc, seed=21):
    """Absorbs against numpy einsum, and against the identity up-projections:
    W_UK[h] = [I | 0] gives q' = [q_nope, 0, q_rope]; W_UV[h] = [I ; 0] gives y = out[:, :128]."""
    g = _rng(seed)
    b, h = 3, 5
    qn = g.standard_normal((b, h, 128))
    qr = g.standard_normal((b, h, 64))
    wk = g.standard_normal((h, 128, 512))
    o = g.standard_normal((b, h, 512))
    wv = g.standard_normal((h, 512, 128))
    qp = orc.absorb_q(qn, wk, qr)
    _close(qp[..., :512], np.einsum("bhj,hjc->bhc", qn, wk), 1e-11, "absorb_q vs einsum")
    _close(qp[..., 512:], qr, 0.0, "absorb_q rope copy")
    _close(orc.absorb_o(o, wv), np.einsum("bhc,hcj->bhj", o, wv), 1e-11, "absorb_o vs einsum")
    eye_k = np.zeros((h, 128, 512))
    eye_k[:, :, :128] = np.eye(128)
    qp = orc.absorb_q(qn, eye_k, qr)
    _close(qp[..., :128], qn, 0.0, "identity W_UK")
    _close(qp[..., 128:512], np.zeros((b, h, 384)), 0.0, "identity W_UK zeros")
    eye_v = np.zeros((h, 512, 128))
    eye_v[:, :128, :] = np.eye(128)
    _close(orc.absorb_o(o, eye_v), o[..., :128], 0.0, "identity W_UV")
    # non-square small shapes catch a transposed operand
    qn2 = g.standard_normal((2, 3, 5))
    wk2 = g.standard_normal((3, 5, 4))
    qr2 = g.standard_normal((2, 3, 2))
    _close(orc.absorb_q(qn2, wk2, qr2)[..., :4], np.einsum("bhj,hjc->bhc", qn2, wk2), 1e-12,
           "absorb_q small")
    o2 = g.standard_normal((2, 3, 4))
    wv2 = g.standard_normal((3, 4, 6))
    _close(orc.absorb_o(o2, wv2), np.einsum("bhc,hcj->bhj", o2, wv2), 1e-12, "absorb_o small")


def pin_unabsorbed_identity_weights_vs_sdpa(orc, seed=22):
    """With W_UK[h] = [I | 0] and W_UV[h] = [I ; 0] the expanded form is plain
    attention with k = [c[:d_k] ; k_R] and v = c[:d_v]: compare with torch SDPA."""
    g = _rng(seed)
    b, h, t_max, dc, dk, dr, dv = 2, 3, 11, 7, 4, 2, 3
    cache = g.standard_normal((b, t_max, dc + dr))
    qn = g.standard_normal((b, h, dk))
    qr = g.standard_normal((b, h, dr))
    wk = np.zeros((h, dk, dc))
    wk[:, :, :dk] = np.eye(dk)
    wv = np.zeros((h, dc, dv))
    wv[:, :dv, :] = np.eye(dv)
    lens = np.array([11, 6], np.int32)
    scale = 0.41
    y, _ = orc.decode_unabsorbed(qn, qr, wk, wv, cache, lens, scale)
    for i in range(b):
        L = int(lens[i])
        q = torch.from_numpy(np.concatenate([qn[i], qr[i]], -1)[None, :, None, :])
        kk = np.concatenate([cache[i, :L, :dk], cache[i, :L, dc:]], -1)
        k = torch.from_numpy(kk)[None, None].expand(1, h, L, dk + dr).contiguous()
        v = torch.from_numpy(cache[i, :L, :dv])[None, None].expand(1, h, L, dv).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
        _close(y[i], ref[0, :, 0, :].numpy(), 1e-12, "expanded vs SDPA (identity weights)")


def pin_empty_sequence(orc, seed=23):
    """seqlens = 0: out = 0 and lse = -inf, for both forms."""
    g = _rng(seed)
    cache = g.standard_normal((2, 4, 576))
    qp = g.standard_normal((2, 3, 576))
    lens = np.array([0, 4], np.int32)
    out, lse = orc.decode_latent(qp, cache, lens, SCALE)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


def _causal_counts(lens, q_len):
    """Rows new token i of each batch row may see: L - q_len + 1 + i, clamped to [0, L]."""
    return np.clip(np.asarray(lens)[:, None] - q_len + 1 + np.arange(q_len)[None, :], 0,
                   np.asarray(lens)[:, None])


def pin_causal_vs_sdpa(orc, seed=24):
    """Several query tokens per row == torch SDPA (fp64) with an explicit
    boolean mask that lets new token i see rows t <= L - q_len + i."""
    g = _rng(seed)
    b, q_len, h, t_max = 3, 4, 3, 40
    lens = np.array([40, 9, 2], np.int32)  # the last row has fewer rows than new tokens
    cache = g.standard_normal((b, t_max, 576))
    qp = g.standard_normal((b, q_len, h, 576))
    out, lse = orc.decode_latent_causal(qp, cache, lens, SCALE)
    n = _causal_counts(lens, q_len)
    for i in range(b):
        L = int(lens[i])
        q = torch.from_numpy(qp[i].transpose(1, 0, 2).copy())[None]  # [1, h, q_len, d]
        k = torch.from_numpy(cache[i, :L])[None, None].expand(1, h, L, 576).contiguous()
        v = torch.from_numpy(cache[i, :L, :512])[None, None].expand(1, h, L, 512).contiguous()
        mask = torch.from_numpy(np.arange(L)[None, :] < n[i][:, None])  # [q_len, L]
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=SCALE)
        o = o[0].numpy().transpose(1, 0, 2)  # [q_len, h, 512]
        for qi in range(q_len):
            if n[i, qi] > 0:
                _close(out[i, qi], o[qi], 1e-12, "causal out vs masked SDPA")
                s = SCALE * (qp[i, qi] @ cache[i, :n[i, qi]].T)  # [h, n]
                m = s.max(1)
                _close(lse[i, qi], m + np.log(np.exp(s - m[:, None]).sum(1)), 1e-12, "causal lse")
            else:
                assert np.all(out[i, qi] == 0.0) and np.all(np.isneginf(lse[i, qi])), "empty prefix"


def pin_causal_zero_query(orc, seed=25):
    """q' = 0 with several new tokens: token i averages exactly its visible
    prefix of n_i rows and lse = ln n_i."""
    g = _rng(seed)
    lens = np.array([10, 3], np.int32)
    q_len = 3
    cache = g.standard_normal((2, 10, 576))
    out, lse = orc.decode_latent_causal(np.zeros((2, q_len, 2, 576)), cache, lens, SCALE)
    n = _causal_counts(lens, q_len)
    for i in range(2):
        for qi in range(q_len):
            _close(lse[i, qi], np.full(2, math.log(n[i, qi])), 1e-12, "lse = ln n_i")
            _close(out[i, qi], np.broadcast_to(cache[i, :n[i, qi], :512].mean(0), (2, 512)), 1e-12,
                   "out = mean of the visible prefix")


def pin_causal_future_rows_unseen(orc, seed=26):
    """A NaN written into the row of new token j reaches exactly the new tokens
    j, j+1, ... and leaves every earlier one unchanged."""
    g = _rng(seed)
    L, q_len, h = 12, 4, 2
    cache = g.standard_normal((1, L, 576))
    qp = g.standard_normal((1, q_len, h, 576))
    lens = np.array([L], np.int32)
    ref, _ = orc.decode_latent_causal(qp, cache, lens, SCALE)
    for j in range(q_len):
        bad = cache.copy()
        bad[0, L - q_len + j] = np.nan
        out, _ = orc.decode_latent_causal(qp, bad, lens, SCALE)
        for qi in range(q_len):
            if qi < j:
                _close(out[0, qi], ref[0, qi], 0.0, "earlier token unaffected")
            else:
                assert np.all(np.isnan(out[0, qi])), "token %d must see row of token %d" % (qi, j)


def _rope_tables(n_pos, half, base=10000.0):
    """Rotation tables of the RoFormer form: angle pos * base^(-j/half)."""
    ang = np.arange(n_pos)[:, None] * base ** (-np.arange(half)[None, :] / half)
    return np.cos(ang), np.sin(ang)


def pin_append_projection_vs_matmul(orc, seed=27):
    """Identity rotation (cos = 1, sin = 0): the appended row is exactly
    [x W_DKV ; x W_KR] (numpy matmul), written at row seqlens[i] only."""
    g = _rng(seed)
    b, d_model, t_max = 3, 40, 9
    x = g.standard_normal((b, d_model))
    wd = g.standard_normal((d_model, 512))
    wr = g.standard_normal((d_model, 64))
    cache = g.standard_normal((b, t_max, 576))
    lens = np.array([0, 5, 8], np.int32)
    out = orc.cache_append(x, wd, wr, np.ones((t_max, 32)), np.zeros((t_max, 32)), lens, cache)
    for i in range(b):
        ref = np.concatenate([x[i] @ wd, x[i] @ wr])
        _close(out[i, lens[i]], ref, 1e-12, "appended row = [x W_DKV ; x W_KR]")
        keep = np.ones(t_max, bool)
        keep[lens[i]] = False
        assert np.array_equal(out[i, keep], cache[i, keep]), "other rows untouched"


def pin_append_rope_properties(orc, seed=28):
    """RoPE as rotations: each pair keeps its length, the content part does not
    move, and the dot product of two keys rotated at positions m and n depends
    only on m - n (shift both rows by 5 positions: same dot product)."""
    g = _rng(seed)
    d_model, t_max = 16, 40
    cos_t, sin_t = _rope_tables(t_max, 32)
    x = g.standard_normal((2, d_model))
    wd = g.standard_normal((d_model, 512))
    wr = g.standard_normal((d_model, 64))
    cache = np.zeros((2, t_max, 576))
    ident = orc.cache_append(x, wd, wr, np.ones((t_max, 32)), np.zeros((t_max, 32)),
                             np.array([3, 11], np.int32), cache)
    rot = orc.cache_append(x, wd, wr, cos_t, sin_t, np.array([3, 11], np.int32), cache)
    for i, pos in enumerate((3, 11)):
        _close(rot[i, pos, :512], ident[i, pos, :512], 0.0, "content part not rotated")
        r = ident[i, pos, 512:].reshape(32, 2)
        k = rot[i, pos, 512:].reshape(32, 2)
        _close(np.hypot(k[:, 0], k[:, 1]), np.hypot(r[:, 0], r[:, 1]), 1e-12, "pair length kept")
    shifted = orc.cache_append(x, wd, wr, cos_t, sin_t, np.array([8, 16], np.int32), cache)
    d0 = rot[0, 3, 512:] @ rot[1, 11, 512:]
    d1 = shifted[0, 8, 512:] @ shifted[1, 16, 512:]
    _close(np.array([d1]), np.array([d0]), 1e-10, "relative-position dot product")
    # the rotation itself, position 3 of pair 0 written out
    r0, r1 = ident[0, 3, 512], ident[0, 3, 513]
    _close(np.array([rot[0, 3, 512], rot[0, 3, 513]]),
           np.array([r0 * math.cos(3.0) - r1 * math.sin(3.0), r0 * math.sin(3.0) + r1 * math.cos(3.0)]),
           1e-12, "pair 0 turned by its angle")


def pin_append_out_of_range_rows(orc, seed=29):
    """A length at or past the cache (or the tables) or negative writes nothing."""
    g = _rng(seed)
    x = g.standard_normal((3, 8))
    cache = g.standard_normal((3, 6, 576))
    out = orc.cache_append(x, g.standard_normal((8, 512)), g.standard_normal((8, 64)),
                           np.ones((5, 32)), np.zeros((5, 32)), np.array([6, -1, 5], np.int32), cache)
    assert np.array_equal(out, cache)


ALL_PINS = [
    pin_glossary_toy_identities,
    pin_identities_c1_dims,
    pin_latent_vs_sdpa,
    pin_zero_query,
    pin_single_token,
    pin_identical_rows,
    pin_shift_invariance,
    pin_permutation,
    pin_equal_heads,
    pin_split_merge,
    pin_probs_sum_to_one,
    pin_absorbs_vs_numpy,
    pin_unabsorbed_identity_weights_vs_sdpa,
    pin_empty_sequence,
    pin_causal_vs_sdpa,
    pin_causal_zero_query,
    pin_causal_future_rows_unseen,
    pin_append_projection_vs_matmul,
    pin_append_rope_properties,
    pin_append_out_of_range_rows,
]
