"""fp64 CPU oracle for absorbed MLA decode -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product library
(``head_latent_attention_decode_amd``) never imports, links or calls it, and
this package imports nothing from the product library: the two share no code.

The arithmetic lives in ``mla_oracle.c`` (plain C loops in double precision,
OpenMP over independent (batch, head) pairs).  This module only marshals numpy
arrays into that shared object.  See the C file's header for the definitions
and the pages each routine follows.

``Oracle(path)`` binds one compiled copy of the C file; the module-level
functions use the default build ``libmla_oracle.so`` next to this file.  (The
pin-strength tests bind deliberately broken copies compiled to a temporary
directory, to show that the pins catch each planted mistake.)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "mla_oracle.c")
LIB = os.path.join(_HERE, "libmla_oracle.so")
_lock = threading.Lock()
_default = None

D_C = 512
D_R = 64
D_K = 128
D_V = 128

GCC_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off"]


def compile_source(src: str, out: str) -> str:
    """Compile an oracle C source into a shared object at `out` (gcc, IEEE fp64)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile mla_oracle.c into libmla_oracle.so."""
    if force or not os.path.exists(LIB):
        compile_source(SRC, LIB)
    return LIB


def _f64(a) -> np.ndarray:
    """Widen an array-like (numpy, or a torch tensor of any float dtype) to C-contiguous fp64."""
    if hasattr(a, "detach"):  # torch tensor: widen on the torch side (bf16 has no numpy dtype)
        import torch
        a = a.detach().to(device="cpu", dtype=torch.float64).contiguous().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def _dp(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if a is not None else None


def _ip(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if a is not None else None


class Oracle:
    """One loaded copy of the fp64 oracle."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        ci, cd = ctypes.c_int, ctypes.c_double
        lib.oracle_decode_latent.argtypes = [ci, ci, ci, ci, ci, dp, dp, ip, cd, dp, dp, dp]
        lib.oracle_decode_latent.restype = None
        lib.oracle_decode_latent_causal.argtypes = [ci, ci, ci, ci, ci, ci, dp, dp, ip, cd, dp, dp]
        lib.oracle_decode_latent_causal.restype = None
        lib.oracle_decode_unabsorbed.argtypes = [ci, ci, ci, ci, ci, ci, ci, dp, dp, dp, dp,
                                                 dp, ip, cd, ip, ci, dp, dp, dp, dp]
        lib.oracle_decode_unabsorbed.restype = None
        lib.oracle_cache_append.argtypes = [ci, ci, ci, ci, ci, ci, dp, dp, dp, dp, dp, ip, dp]
        lib.oracle_cache_append.restype = None
        lib.oracle_absorb_q.argtypes = [ci, ci, ci, ci, ci, dp, dp, dp, dp]
        lib.oracle_absorb_q.restype = None
        lib.oracle_absorb_o.argtypes = [ci, ci, ci, ci, dp, dp, dp]
        lib.oracle_absorb_o.restype = None
        lib.oracle_abi_version.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def decode_latent(self, q_prime, cache, seqlens, scale, d_c=D_C, want_scores=False):
        """Latent form.  q_prime [b,h,d_c+d_r], cache [b,t_max,d_c+d_r], seqlens [b].

        Returns (out [b,h,d_c], lse [b,h]) or, with want_scores, also scores
        [b,h,t_max] (NaN at t >= seqlens[b]).
        """
        q = _f64(q_prime)
        c = _f64(cache)
        sl = _i32(seqlens)
        b, h, d = q.shape
        assert c.ndim == 3 and c.shape[0] == b and c.shape[2] == d, (q.shape, c.shape)
        assert sl.shape == (b,)
        t_max = c.shape[1]
        d_r = d - d_c
        out = np.empty((b, h, d_c), np.float64)
        lse = np.empty((b, h), np.float64)
        sc = np.full((b, h, t_max), np.nan) if want_scores else None
        self.lib.oracle_decode_latent(b, h, t_max, d_c, d_r, _dp(q), _dp(c), _ip(sl),
                                      float(scale), _dp(out), _dp(lse), _dp(sc))
        return (out, lse, sc) if want_scores else (out, lse)

    def decode_latent_causal(self, q_prime, cache, seqlens, scale, d_c=D_C):
        """Latent form with several query tokens per row (causal reading).

        q_prime [b,q_len,h,d_c+d_r], cache [b,t_max,d_c+d_r], seqlens [b]: new
        token i attends to the first seqlens[b] - q_len + 1 + i rows.  Returns
        (out [b,q_len,h,d_c], lse [b,q_len,h]).
        """
        q = _f64(q_prime)
        c = _f64(cache)
        sl = _i32(seqlens)
        b, q_len, h, d = q.shape
        assert c.ndim == 3 and c.shape[0] == b and c.shape[2] == d, (q.shape, c.shape)
        assert sl.shape == (b,)
        t_max = c.shape[1]
        out = np.empty((b, q_len, h, d_c), np.float64)
        lse = np.empty((b, q_len, h), np.float64)
        self.lib.oracle_decode_latent_causal(b, q_len, h, t_max, d_c, d - d_c, _dp(q), _dp(c),
                                             _ip(sl), float(scale), _dp(out), _dp(lse))
        return out, lse

    def decode_unabsorbed(self, q_nope, q_rope, w_uk, w_uv, cache, seqlens, scale, heads=None,
                          want_scores=False):
        """Expanded form.  q_nope [b,h,d_k], q_rope [b,h,d_r], w_uk [h,d_k,d_c],
        w_uv [h,d_c,d_v], cache [b,t_max,d_c+d_r].  heads: optional head subset.

        Returns (y [b,n_sel,d_v], lse [b,n_sel]) or, with want_scores, also
        (scores, probs) [b,n_sel,t_max] (NaN at t >= seqlens[b]).
        """
        qn, qr, wk, wv, c = (_f64(x) for x in (q_nope, q_rope, w_uk, w_uv, cache))
        sl = _i32(seqlens)
        b, h, d_k = qn.shape
        d_r = qr.shape[2]
        d_c = wk.shape[2]
        d_v = wv.shape[2]
        assert qr.shape[:2] == (b, h) and wk.shape == (h, d_k, d_c) and wv.shape == (h, d_c, d_v)
        assert c.shape[0] == b and c.shape[2] == d_c + d_r and sl.shape == (b,)
        t_max = c.shape[1]
        hs = None if heads is None else _i32(np.asarray(heads))
        n_sel = h if hs is None else int(hs.shape[0])
        y = np.empty((b, n_sel, d_v), np.float64)
        lse = np.empty((b, n_sel), np.float64)
        sc = np.full((b, n_sel, t_max), np.nan) if want_scores else None
        pr = np.full((b, n_sel, t_max), np.nan) if want_scores else None
        self.lib.oracle_decode_unabsorbed(b, h, t_max, d_c, d_r, d_k, d_v, _dp(qn), _dp(qr),
                                          _dp(wk), _dp(wv), _dp(c), _ip(sl), float(scale),
                                          _ip(hs), n_sel, _dp(y), _dp(lse), _dp(sc), _dp(pr))
        return (y, lse, sc, pr) if want_scores else (y, lse)

    def cache_append(self, x, w_dkv, w_kr, cos_tab, sin_tab, seqlens, cache):
        """Write the new token's latent row [x W_DKV ; RoPE(x W_KR)] into row
        seqlens[i] of each batch row.  x [b,d_model], w_dkv [d_model,d_c],
        w_kr [d_model,d_r], cos_tab/sin_tab [n_pos,d_r/2], cache [b,t_max,d_c+d_r].
        Returns the updated cache (a new fp64 array)."""
        xx, wd, wr, ct, st = (_f64(a) for a in (x, w_dkv, w_kr, cos_tab, sin_tab))
        c = _f64(cache).copy()
        sl = _i32(seqlens)
        b, d_model = xx.shape
        d_c, d_r = wd.shape[1], wr.shape[1]
        n_pos = ct.shape[0]
        assert wd.shape[0] == d_model and wr.shape[0] == d_model and st.shape == ct.shape
        assert ct.shape[1] == d_r // 2 and c.shape[0] == b and c.shape[2] == d_c + d_r
        self.lib.oracle_cache_append(b, d_model, d_c, d_r, c.shape[1], n_pos, _dp(xx), _dp(wd),
                                     _dp(wr), _dp(ct), _dp(st), _ip(sl), _dp(c))
        return c

    def absorb_q(self, q_nope, w_uk, q_rope):
        """q'[b,h,:d_c] = q_nope[b,h,:] @ w_uk[h] ; q'[b,h,d_c:] = q_rope[b,h,:]."""
        qn, wk, qr = _f64(q_nope), _f64(w_uk), _f64(q_rope)
        b, h, d_k = qn.shape
        d_c = wk.shape[2]
        d_r = qr.shape[2]
        assert wk.shape == (h, d_k, d_c) and qr.shape[:2] == (b, h)
        qp = np.empty((b, h, d_c + d_r), np.float64)
        self.lib.oracle_absorb_q(b, h, d_k, d_c, d_r, _dp(qn), _dp(wk), _dp(qr), _dp(qp))
        return qp

    def absorb_o(self, o, w_uv):
        """y[b,h,:] = o[b,h,:] @ w_uv[h]."""
        oo, wv = _f64(o), _f64(w_uv)
        b, h, d_c = oo.shape
        d_v = wv.shape[2]
        assert wv.shape == (h, d_c, d_v)
        y = np.empty((b, h, d_v), np.float64)
        self.lib.oracle_absorb_o(b, h, d_c, d_v, _dp(oo), _dp(wv), _dp(y))
        return y


def default() -> Oracle:
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(LIB):
                build(force=False)
            _default = Oracle(LIB)
    return _default


def decode_latent(*a, **k):
    return default().decode_latent(*a, **k)


def decode_unabsorbed(*a, **k):
    return default().decode_unabsorbed(*a, **k)


def decode_latent_causal(*a, **k):
    return default().decode_latent_causal(*a, **k)


def cache_append(*a, **k):
    return default().cache_append(*a, **k)


def absorb_q(*a, **k):
    return default().absorb_q(*a, **k)


def absorb_o(*a, **k):
    return default().absorb_o(*a, **k)
