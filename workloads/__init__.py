"""Seeded synthetic inputs for absorbed MLA decode.

This module only draws random numbers and fixes shapes.  It holds none of the
method's arithmetic, so the oracle and the HIP path can both be fed from it
without sharing any computation.

Dimensions follow DeepSeek-V2/V3 as the pages give them: a 512-wide latent
c_KV plus a 64-wide decoupled RoPE key per cached token (576 per row), a
128-wide per-head query/value width, and a softmax scale of 1/sqrt(128 + 64).

Recipe (one CPU ``torch.Generator`` per workload, seed = 1000 + config
number; every tensor is drawn on the CPU and then moved to the requested
device, so one seed gives the same numbers on every device): draw order is
sequence lengths (ragged configs only), cache, query side, then weights.
Values are fp32 N(0,1) draws, rounded to nearest-even into bf16 where the
config is bf16; weights are divided by sqrt(fan_in) (128 for W_UK, 512 for
W_UV).  In parity runs every cache row at or past a sequence's length holds
NaN, so a kernel that reads past the end cannot go unnoticed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

D_C = 512
D_R = 64
D_QK = D_C + D_R
D_K = 128
D_V = 128
SCALE = 1.0 / math.sqrt(D_K + D_R)


@dataclass
class Config:
    cid: int
    name: str
    dtype: torch.dtype
    b: int
    h: int
    t_max: int
    lengths: str  # "fixed" (all t_max), "list", or "uniform" (U[1, t_max])
    length_list: Optional[list] = None
    raw_query: bool = False  # True: q_nope/q_rope + weights; False: absorbed q' given


CONFIGS = {
    1: Config(1, "tiny_fp32_b2_h16_L128_257", torch.float32, 2, 16, 257, "list", [128, 257],
              raw_query=True),
    2: Config(2, "dsv3_decode_b64_h128_T4096", torch.bfloat16, 64, 128, 4096, "fixed"),
    3: Config(3, "few_heads_b128_h16_T8192", torch.bfloat16, 128, 16, 8192, "fixed"),
    4: Config(4, "ragged_b132_h128_Tmax32768", torch.bfloat16, 132, 128, 32768, "uniform"),
    5: Config(5, "long_e2e_b4_h128_T131072", torch.bfloat16, 4, 128, 131072, "fixed",
              raw_query=True),
}


@dataclass
class Workload:
    name: str
    dtype: torch.dtype
    b: int
    h: int
    t_max: int
    seqlens: torch.Tensor  # int32 [b], on `device`
    cache: torch.Tensor  # [b, t_max, 576]
    q_prime: Optional[torch.Tensor] = None  # [b, h, 576]
    q_nope: Optional[torch.Tensor] = None  # [b, h, 128]
    q_rope: Optional[torch.Tensor] = None  # [b, h, 64]
    w_uk: Optional[torch.Tensor] = None  # [h, 128, 512]
    w_uv: Optional[torch.Tensor] = None  # [h, 512, 128]
    scale: float = SCALE
    seed: int = 0
    extra: dict = field(default_factory=dict)

    def seqlens_host(self):
        return [int(x) for x in self.seqlens.cpu().tolist()]


def _randn(shape, gen, device, dtype, divisor=1.0, chunk_rows=None):
    """fp32 N(0,1) draws from the CPU generator `gen` (optionally / divisor),
    rounded to `dtype` and placed on `device`.  Large tensors are drawn in
    consecutive blocks of `chunk_rows` leading rows (the block size is a
    function of the shape only, so a given shape always gets the same
    numbers)."""
    if chunk_rows is None or shape[0] <= chunk_rows:
        x = torch.randn(shape, generator=gen, dtype=torch.float32)
        if divisor != 1.0:
            x.div_(divisor)
        return x.to(dtype).to(device)
    out = torch.empty(shape, device=device, dtype=dtype)
    for i in range(0, shape[0], chunk_rows):
        n = min(chunk_rows, shape[0] - i)
        x = torch.randn((n,) + tuple(shape[1:]), generator=gen, dtype=torch.float32)
        if divisor != 1.0:
            x.div_(divisor)
        out[i:i + n].copy_(x.to(dtype))
        del x
    return out


def poison_tail(cache: torch.Tensor, seqlens) -> None:
    """Fill every row at or past each sequence's length with NaN (in place)."""
    lens = seqlens.cpu().tolist() if hasattr(seqlens, "cpu") else list(seqlens)
    t_max = cache.shape[1]
    for i, L in enumerate(lens):
        L = max(0, min(int(L), t_max))
        if L < t_max:
            cache[i, L:].fill_(float("nan"))


def make_custom(b, h, seqlens, t_max=None, dtype=torch.bfloat16, seed=0, device="cpu",
                raw_query=False, poison=True, name="custom"):
    """A workload of arbitrary shape with the same recipe as the named configs.

    seqlens: list of ints (one per batch row).  t_max defaults to max(seqlens)
    (at least 1).  raw_query=True draws q_nope, q_rope, W_UK, W_UV instead of q'.
    """
    assert len(seqlens) == b
    if t_max is None:
        t_max = max(1, max(seqlens))
    gen = torch.Generator()
    gen.manual_seed(seed)
    sl = torch.tensor([int(x) for x in seqlens], dtype=torch.int32, device=device)
    chunk = max(1, (1 << 26) // max(1, t_max * D_QK))
    cache = _randn((b, t_max, D_QK), gen, device, dtype, chunk_rows=chunk)
    w = Workload(name=name, dtype=dtype, b=b, h=h, t_max=t_max, seqlens=sl, cache=cache,
                 seed=seed)
    if raw_query:
        w.q_nope = _randn((b, h, D_K), gen, device, dtype)
        w.q_rope = _randn((b, h, D_R), gen, device, dtype)
        w.w_uk = _randn((h, D_K, D_C), gen, device, dtype, divisor=math.sqrt(D_K))
        w.w_uv = _randn((h, D_C, D_V), gen, device, dtype, divisor=math.sqrt(D_C))
    else:
        w.q_prime = _randn((b, h, D_QK), gen, device, dtype)
    if poison:
        poison_tail(cache, sl)
    return w


def _draw_lengths(cfg, gen, bb):
    """The sequence lengths of a configuration: the first draw from its
    generator (ragged configs only)."""
    if cfg.lengths == "fixed":
        return torch.full((bb,), cfg.t_max, dtype=torch.int32)
    if cfg.lengths == "list":
        return torch.tensor(cfg.length_list[:bb], dtype=torch.int32)
    return torch.randint(1, cfg.t_max + 1, (bb,), generator=gen, dtype=torch.int64).to(torch.int32)


def lengths(cid: int) -> list:
    """Sequence lengths of configuration `cid` exactly as make() draws them,
    without building the cache."""
    cfg = CONFIGS[cid]
    gen = torch.Generator()
    gen.manual_seed(1000 + cid)
    return [int(x) for x in _draw_lengths(cfg, gen, cfg.b).tolist()]


def make(cid: int, device="cpu", poison=True, b=None) -> Workload:
    """Build configuration `cid` (1..5).  `b` optionally truncates the batch
    (the first b rows of the same draw order are not reproduced; it is a
    smaller workload of the same recipe, used for CPU-sized samples)."""
    cfg = CONFIGS[cid]
    seed = 1000 + cid
    bb = cfg.b if b is None else b
    gen = torch.Generator()
    gen.manual_seed(seed)
    sl = _draw_lengths(cfg, gen, bb).to(device)
    chunk = max(1, (1 << 26) // (cfg.t_max * D_QK))
    cache = _randn((bb, cfg.t_max, D_QK), gen, device, cfg.dtype, chunk_rows=chunk)
    w = Workload(name=cfg.name, dtype=cfg.dtype, b=bb, h=cfg.h, t_max=cfg.t_max, seqlens=sl,
                 cache=cache, seed=seed)
    if cfg.raw_query:
        w.q_nope = _randn((bb, cfg.h, D_K), gen, device, cfg.dtype)
        w.q_rope = _randn((bb, cfg.h, D_R), gen, device, cfg.dtype)
        w.w_uk = _randn((cfg.h, D_K, D_C), gen, device, cfg.dtype, divisor=math.sqrt(D_K))
        w.w_uv = _randn((cfg.h, D_C, D_V), gen, device, cfg.dtype, divisor=math.sqrt(D_C))
    else:
        w.q_prime = _randn((bb, cfg.h, D_QK), gen, device, cfg.dtype)
    if poison:
        poison_tail(cache, sl)
    return w


def make_step_weights(b, h, dtype=torch.bfloat16, seed=2002, device="cpu"):
    """q_nope, q_rope, W_UK, W_UV for a full absorb -> decode -> absorb step at
    a decode-only config's shape (same recipe as the end-to-end config)."""
    gen = torch.Generator()
    gen.manual_seed(seed)
    q_nope = _randn((b, h, D_K), gen, device, dtype)
    q_rope = _randn((b, h, D_R), gen, device, dtype)
    w_uk = _randn((h, D_K, D_C), gen, device, dtype, divisor=math.sqrt(D_K))
    w_uv = _randn((h, D_C, D_V), gen, device, dtype, divisor=math.sqrt(D_C))
    return q_nope, q_rope, w_uk, w_uv
