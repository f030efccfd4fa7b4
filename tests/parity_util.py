"""Shared helpers for the GPU parity tests: tolerance checks and sampled oracle runs.

Tolerances (stated once, used everywhere):
  bf16 inputs: max|out - ref| <= 2e-2 * max|ref|, max|lse - ref| <= 1e-3 (absolute),
               absorbs (q', y) use the out rule;
  fp32 inputs: max|x - ref| <= 1e-5 * max|ref| for q', out, lse and y.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

BF16_OUT_REL = 2e-2
BF16_LSE_ABS = 1e-3
F32_REL = 1e-5


def to_np(t):
    return t.detach().to(device="cpu", dtype=torch.float64).numpy()


def max_rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return err, scale


def assert_out(got, ref, rel, what="out"):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), "%s has non-finite values" % what
    err, scale = max_rel_err(got, ref)
    assert err <= rel * scale, "%s: max|err| %.3e > %.1e * max|ref| (%.3e)" % (what, err, rel, scale)
    return err / max(scale, 1e-300)


def assert_lse(got, ref, tol, what="lse"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    empty = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), empty), "%s: -inf pattern differs" % what
    fin = ~empty
    assert np.all(np.isfinite(got[fin])), "%s has non-finite values" % what
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    assert err <= tol, "%s: max|err| %.3e > %.1e" % (what, err, tol)
    return err


def oracle_decode_rows(q_prime, cache, seqlens, scale, rows, heads=None):
    """Latent-form oracle on a subset of batch rows (and optionally heads).

    Inputs are the GPU tensors; only the needed rows are copied back and
    widened to fp64.  Returns (out [len(rows), n_heads, 512], lse [...])."""
    rows = list(rows)
    lens = seqlens.cpu().tolist()
    L = max(1, max(int(lens[r]) for r in rows))
    q = q_prime[rows] if heads is None else q_prime[rows][:, list(heads)]
    c = cache[rows, :L]
    sl = np.array([min(int(lens[r]), L) for r in rows], np.int32)
    return oracle.decode_latent(q.cpu(), c.cpu(), sl, scale)


def check_decode(q_prime, cache, seqlens, scale, out, lse, rows, heads=None, bf16=True):
    ref_out, ref_lse = oracle_decode_rows(q_prime, cache, seqlens, scale, rows, heads)
    o = out[list(rows)] if heads is None else out[list(rows)][:, list(heads)]
    l = lse[list(rows)] if heads is None else lse[list(rows)][:, list(heads)]
    o, l = to_np(o), to_np(l)
    if bf16:
        e1 = assert_out(o, ref_out, BF16_OUT_REL)
        e2 = assert_lse(l, ref_lse, BF16_LSE_ABS)
    else:
        e1 = assert_out(o, ref_out, F32_REL)
        fin = np.isfinite(ref_lse)
        e2 = assert_out(l[fin], ref_lse[fin], F32_REL, "lse")
    return e1, e2
