"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Small cases run the oracle on every output; the full-size configurations
(the same launch configuration the benchmark times) check sampled batch rows
(and heads) against the oracle, plus properties that hold at any size.
Every cache row at or past a sequence's length holds NaN, so any read past
the end shows up as a non-finite output.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import (BF16_LSE_ABS, BF16_OUT_REL, F32_REL, assert_lse, assert_out,
                         check_decode, to_np)

pytestmark = pytest.mark.gpu

SCALE = workloads.SCALE


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_latent_attention_decode_amd as m
    return m


def _run(mla, w, config=None):
    out, lse = mla.mla_decode(w.q_prime, w.cache, w.seqlens, w.scale, config=config)
    torch.cuda.synchronize()
    return out, lse


# ---------------------------------------------------------------- fp32 (tiny config)

def test_tiny_fp32_pipeline(mla):
    w = workloads.make(1, device="cuda")
    # q absorb against the oracle's absorb
    qp_gpu = mla.mla_absorb_q(w.q_nope, w.w_uk, w.q_rope)
    qp_ref = oracle.absorb_q(w.q_nope.cpu(), w.w_uk.cpu(), w.q_rope.cpu())
    torch.cuda.synchronize()
    assert_out(to_np(qp_gpu), qp_ref, F32_REL, "q'")
    # decode fed the oracle's q' (never the HIP path's)
    qp_in = torch.from_numpy(qp_ref).to(torch.float32).cuda()
    ref_out, ref_lse = oracle.decode_latent(qp_in.cpu(), w.cache.cpu(), w.seqlens.cpu(), w.scale)
    for cfg in (None, {"n_chunks": 8}, {"n_chunks": 64}, {"n_chunks": 256}):
        out, lse = mla.mla_decode(qp_in, w.cache, w.seqlens, w.scale, config=cfg)
        torch.cuda.synchronize()
        assert_out(to_np(out), ref_out, F32_REL, "out %s" % cfg)
        assert_out(to_np(lse), ref_lse, F32_REL, "lse %s" % cfg)
    # end to end against the expanded (un-absorbed) form
    bufs = mla.alloc_step(w.b, w.h, w.t_max, torch.float32)
    y = mla.mla_step(w.q_nope, w.q_rope, w.w_uk, w.w_uv, w.cache, w.seqlens, w.scale, bufs)
    torch.cuda.synchronize()
    y_ref, lse_x = oracle.decode_unabsorbed(w.q_nope.cpu(), w.q_rope.cpu(), w.w_uk.cpu(),
                                            w.w_uv.cpu(), w.cache.cpu(), w.seqlens.cpu(), w.scale)
    assert_out(to_np(y), y_ref, F32_REL, "y")
    assert_out(to_np(bufs.lse), lse_x, F32_REL, "lse vs expanded form")


@pytest.mark.parametrize("h", [3, 20, 40])
def test_fp32_partial_head_groups(mla, h):
    # fp32 kernels with h not a multiple of their 16-head group (the last
    # group partly empty), edge lengths with NaN tails: every stage against
    # the oracle, and the step end to end against the expanded form
    lens = [1, 15, 16, 17, 33, 0, 257]
    w = workloads.make_custom(len(lens), h, lens, dtype=torch.float32, seed=150 + h, device="cuda",
                              raw_query=True)
    qp_gpu = mla.mla_absorb_q(w.q_nope, w.w_uk, w.q_rope)
    torch.cuda.synchronize()
    qp_ref = oracle.absorb_q(w.q_nope.cpu(), w.w_uk.cpu(), w.q_rope.cpu())
    assert_out(to_np(qp_gpu), qp_ref, F32_REL, "q'")
    qp_in = torch.from_numpy(qp_ref).to(torch.float32).cuda()
    ref_out, ref_lse = oracle.decode_latent(qp_in.cpu(), w.cache.cpu(), w.seqlens.cpu(), w.scale)
    fin = np.isfinite(ref_lse)
    for cfg in (None, {"n_chunks": 8}, {"n_chunks": 64}):
        out, lse = mla.mla_decode(qp_in, w.cache, w.seqlens, w.scale, config=cfg)
        torch.cuda.synchronize()
        assert_out(to_np(out), ref_out, F32_REL, "out %s" % cfg)
        assert_out(to_np(lse)[fin], ref_lse[fin], F32_REL, "lse %s" % cfg)
        assert torch.all(out[lens.index(0)] == 0) and torch.all(torch.isneginf(lse[lens.index(0)]))
    bufs = mla.alloc_step(w.b, w.h, w.t_max, torch.float32)
    y = mla.mla_step(w.q_nope, w.q_rope, w.w_uk, w.w_uv, w.cache, w.seqlens, w.scale, bufs)
    torch.cuda.synchronize()
    y_ref, lse_x = oracle.decode_unabsorbed(w.q_nope.cpu(), w.q_rope.cpu(), w.w_uk.cpu(),
                                            w.w_uv.cpu(), w.cache.cpu(), w.seqlens.cpu(), w.scale)
    assert_out(to_np(y), y_ref, F32_REL, "y vs expanded form")
    assert_out(to_np(bufs.lse)[fin], lse_x[fin], F32_REL, "lse vs expanded form")


@pytest.mark.parametrize("b,h", [(40, 3), (40, 16), (17, 20)])
def test_fp32_absorbs_many_rows(mla, b, h):
    # fp32 absorbs over more batch rows than one 16-row block (the last block ragged)
    g = torch.Generator().manual_seed(160 + b + h)
    q_nope = torch.randn(b, h, 128, generator=g).cuda()
    q_rope = torch.randn(b, h, 64, generator=g).cuda()
    w_uk = (torch.randn(h, 128, 512, generator=g) / math.sqrt(128)).cuda()
    o = torch.randn(b, h, 512, generator=g).cuda()
    w_uv = (torch.randn(h, 512, 128, generator=g) / math.sqrt(512)).cuda()
    qp = mla.mla_absorb_q(q_nope, w_uk, q_rope)
    y = mla.mla_absorb_o(o, w_uv)
    torch.cuda.synchronize()
    assert_out(to_np(qp), oracle.absorb_q(q_nope.cpu(), w_uk.cpu(), q_rope.cpu()), F32_REL, "q'")
    np.testing.assert_array_equal(to_np(qp[..., 512:]), to_np(q_rope))
    assert_out(to_np(y), oracle.absorb_o(o.cpu(), w_uv.cpu()), F32_REL, "y")


# ---------------------------------------------------------------- bf16, small, every output

EDGE_LENS = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 0, 700]

BF16_CASES = [
    # (h, config)
    (1, None), (3, None), (16, None), (16, {"heads_per_group": 16, "variant": 2}),
    (32, None), (32, {"heads_per_group": 32, "variant": 2}), (64, None),
    (64, {"heads_per_group": 64, "variant": 2}), (128, None),
    (128, {"heads_per_group": 128, "variant": 2}), (128, {"heads_per_group": 64}),
    (128, {"heads_per_group": 16}), (40, {"heads_per_group": 16}),
    (64, {"heads_per_group": 64, "variant": 3}),
    pytest.param(64, {"heads_per_group": 64, "variant": 4}, marks=pytest.mark.skip(
        reason="three-stage pair kernel switched off after an unexplained GPU memory fault")),
    (32, {"heads_per_group": 32, "variant": 3}),
    (100, None), (16, {"heads_per_group": 16, "variant": 1}),
    # wide-wave kernels (32 heads per wave)
    (128, {"heads_per_group": 128, "variant": 3}), (128, {"heads_per_group": 128, "variant": 4}),
    (128, {"heads_per_group": 128, "variant": 5}),
    (100, {"heads_per_group": 128, "variant": 3}), (64, {"heads_per_group": 64, "variant": 5}),
    (64, {"heads_per_group": 64, "variant": 6}), (32, {"heads_per_group": 32, "variant": 4}),
    (20, {"heads_per_group": 32, "variant": 4}),
    # column-split, pipelined kernel (128 heads per workgroup)
    (128, {"heads_per_group": 128, "variant": 6}), (100, {"heads_per_group": 128, "variant": 6}),
    (3, {"heads_per_group": 128, "variant": 6}),
]


def _case_id(c):
    h, cfg = c.values if hasattr(c, "values") else c
    return f"h{h}-{cfg}"


@pytest.mark.parametrize("h,cfg", BF16_CASES, ids=[_case_id(c) for c in BF16_CASES])
def test_bf16_edges_every_output(mla, h, cfg):
    w = workloads.make_custom(len(EDGE_LENS), h, EDGE_LENS, seed=100 + h, device="cuda")
    # 2560 chunks: more than a wide kernel plans in its own LDS (plan kernel)
    for extra in ({}, {"n_chunks": 8}, {"n_chunks": 64}, {"n_chunks": 256}, {"n_chunks": 2560}):
        c = dict(cfg or {})
        c.update(extra)
        out, lse = _run(mla, w, c or None)
        check_decode(w.q_prime, w.cache, w.seqlens, w.scale, out, lse, range(w.b))
        # empty row: out = 0, lse = -inf
        assert torch.all(out[EDGE_LENS.index(0)] == 0)
        assert torch.all(torch.isneginf(lse[EDGE_LENS.index(0)]))


RESCALE_CASES = [
    (128, None), (128, {"heads_per_group": 128, "variant": 3}), (128, {"heads_per_group": 128, "variant": 5}),
    (64, {"heads_per_group": 64, "variant": 6}), (64, {"heads_per_group": 64, "variant": 2}),
    (32, {"heads_per_group": 32, "variant": 4}), (128, {"heads_per_group": 16}),
    (128, {"heads_per_group": 128, "variant": 6}), (100, {"heads_per_group": 128, "variant": 6}),
]


@pytest.mark.parametrize("h,cfg", RESCALE_CASES, ids=[_case_id(c) for c in RESCALE_CASES])
def test_bf16_running_max_growth(mla, h, cfg):
    # Scores that grow along the tokens for some heads only: the running max
    # of those heads jumps by more than the lazy-rescale threshold tile after
    # tile, while the other heads never rescale.
    w = workloads.make_custom(4, h, [700, 257, 1000, 33], seed=61 + h, device="cuda")
    t = torch.arange(w.t_max, device="cuda", dtype=torch.float32)
    w.cache[:, :, 575] = (0.25 * t).to(torch.bfloat16)[None, :]
    slope = torch.tensor([16.0, 4.0, 1.0, 0.0, -4.0, 0.5, 8.0, -1.0], device="cuda")
    per_head = slope[torch.arange(h, device="cuda") % 8]
    # heads 32..63 and 96..127 (second and fourth group of 32) never grow
    per_head = torch.where((torch.arange(h, device="cuda") // 32) % 2 == 1, -per_head.abs(), per_head)
    w.q_prime[:, :, 575] = per_head.to(torch.bfloat16)[None, :]
    workloads.poison_tail(w.cache, w.seqlens)
    for extra in ({}, {"n_chunks": 8}, {"n_chunks": 64}):
        c = dict(cfg or {})
        c.update(extra)
        out, lse = _run(mla, w, c or None)
        check_decode(w.q_prime, w.cache, w.seqlens, w.scale, out, lse, range(w.b))


TILE_MAX_CASES = [
    (128, None), (128, {"heads_per_group": 128, "variant": 6}), (64, {"heads_per_group": 64, "variant": 6}),
    (64, {"heads_per_group": 64, "variant": 3}), (32, {"heads_per_group": 32, "variant": 4}),
    (128, {"heads_per_group": 128, "variant": 2}),
]


@pytest.mark.parametrize("h,cfg", TILE_MAX_CASES, ids=[_case_id(c) for c in TILE_MAX_CASES])
def test_bf16_tile_max_spans_both_lane_halves(mla, h, cfg):
    # In the 32-wide MFMA layouts lane l holds tokens 8i + 0..3 of a head and
    # lane l + 32 tokens 8i + 4..7.  Here the second kind score about 1280
    # above the first (q' and k agree in channel 575), so a tile maximum
    # taken over one lane's tokens only sits ~133 below the true one in base 2
    # and exp2 overflows; the true maximum keeps every probability <= 1.
    lens = [64, 33, 700]
    w = workloads.make_custom(len(lens), h, lens, seed=90 + h, device="cuda", poison=False)
    t = torch.arange(w.t_max, device="cuda")
    w.cache[:, :, 575] = torch.where((t % 8) >= 4, 40.0, 0.0).to(torch.bfloat16)[None, :]
    w.q_prime[:, :, 575] = 32.0
    workloads.poison_tail(w.cache, w.seqlens)
    for extra in ({}, {"n_chunks": 8}):
        c = dict(cfg or {})
        c.update(extra)
        out, lse = _run(mla, w, c or None)
        check_decode(w.q_prime, w.cache, w.seqlens, w.scale, out, lse, range(w.b))


def test_fp8_wide_tile_max_spans_both_lane_halves(mla):
    # the same construction through the FP8-MFMA kernel (its tile maximum and
    # the per-head query maximum both combine the two lanes of a head)
    h, lens = 128, [64, 33, 700]
    w = workloads.make_custom(len(lens), h, lens, seed=95, device="cuda", poison=False)
    t = torch.arange(w.t_max, device="cuda")
    w.cache[:, :, 575] = torch.where((t % 8) >= 4, 40.0, 0.0).to(torch.bfloat16)[None, :]
    w.q_prime[:, :, 575] = 32.0
    codes, scale, deq = _fp8_from(w)
    qd = _fp8_query_deq(w.q_prime)
    ref_out, ref_lse = oracle.decode_latent(qd, deq, w.seqlens.cpu(), w.scale)
    out, lse = mla.mla_decode_fp8(w.q_prime, codes, scale, w.seqlens, w.scale)
    torch.cuda.synchronize()
    check_fp8_mfma(out, lse, qd, deq, lens, w.scale, ref_out, ref_lse)


def test_bf16_split_invariance_and_determinism(mla):
    w = workloads.make_custom(5, 128, [3000, 17, 4096, 1, 2500], seed=7, device="cuda")
    outs = []
    for n in (8, 16, 64, 256, 1024):
        out, lse = _run(mla, w, {"n_chunks": n})
        check_decode(w.q_prime, w.cache, w.seqlens, w.scale, out, lse, range(w.b))
        outs.append((out.clone(), lse.clone()))
        out2, lse2 = _run(mla, w, {"n_chunks": n})
        assert torch.equal(out, out2) and torch.equal(lse, lse2), "not deterministic"
    # different schedules agree with each other to the same tolerance
    ref_o, ref_l = to_np(outs[0][0]), to_np(outs[0][1])
    for o, l in outs[1:]:
        assert_out(to_np(o), ref_o, BF16_OUT_REL)
        assert_lse(to_np(l), ref_l, BF16_LSE_ABS)


def test_bf16_closed_forms(mla):
    # zero query: lse = ln L exactly (up to fp32), out = mean of the latent rows
    lens = [1, 77, 1024]
    w = workloads.make_custom(3, 16, lens, seed=9, device="cuda")
    w.q_prime.zero_()
    out, lse = _run(mla, w)
    for i, L in enumerate(lens):
        np.testing.assert_allclose(to_np(lse[i]), math.log(L), atol=1e-5)
        mean = to_np(w.cache[i, :L, :512].float()).mean(0)
        assert_out(to_np(out[i]), np.broadcast_to(mean, (16, 512)), BF16_OUT_REL)
    # constant score shift: cache[..., 575] = 1, q'[..., 575] += delta
    w = workloads.make_custom(2, 32, [500, 333], seed=10, device="cuda")
    w.cache[:, :, 575] = 1.0
    workloads.poison_tail(w.cache, w.seqlens)
    out0, lse0 = _run(mla, w)
    q575_before = w.q_prime[:, :, 575].float().clone()
    w.q_prime[:, :, 575] += 8.0
    out1, lse1 = _run(mla, w)
    # the bf16 addition rounds, so each head's actual shift is read back exactly
    shift = (w.q_prime[:, :, 575].float() - q575_before).cpu().double().numpy()
    assert_out(to_np(out1), to_np(out0), BF16_OUT_REL, "out under shift")
    np.testing.assert_allclose(to_np(lse1 - lse0), SCALE * shift, atol=2e-3)


def test_bf16_combine_many_segments(mla):
    # two long rows cut into ~40 segments each (several rounds of the combine's
    # per-wave slot loop); 100 heads leave the last 32-head group partly empty
    w = workloads.make_custom(3, 100, [20000, 13001, 5], seed=21, device="cuda")
    heads = [0, 31, 32, 63, 64, 95, 96, 99]
    out, lse = _run(mla, w, {"n_chunks": 96})
    check_decode(w.q_prime, w.cache, w.seqlens, w.scale, out, lse, range(w.b), heads)


def _plan_model(lens, t_max, n_chunks, min_chunk):
    """The split rule written out in Python: the batch as one concatenated
    token sequence cut into n_chunks equal chunks (at least min_chunk tokens)."""
    L = [min(max(x, 0), t_max) for x in lens]
    cu = [0]
    for x in L:
        cu.append(cu[-1] + x)
    total = cu[-1]
    chunk = max(-(-total // n_chunks), min_chunk)
    ns = [((cu[i + 1] - 1) // chunk - cu[i] // chunk + 1) if L[i] > 0 else 0 for i in range(len(L))]
    base = [sum(ns[:i]) for i in range(len(L))]
    row_of = []
    for k in range(n_chunks):
        t = k * chunk
        row_of.append(next(i for i in range(len(L)) if cu[i] <= t < cu[i + 1]) if t < total else -1)
    return [total, chunk, n_chunks, 0] + cu + base + ns + row_of


@pytest.mark.parametrize("n_chunks", [256, 4096], ids=["in-kernel", "plan-kernel"])
@pytest.mark.parametrize("lens", [
    [4096] * 64,                                    # uniform: four chunks per row
    [131072] * 4,                                   # long rows: 64 chunk starts per row
    [0, 5, 0, 700, 33, 0, 9000, 1] + [17] * 120,    # ragged, empty rows, b > 64
    [0, 0, 0],                                      # nothing to attend
    [-3, 10**9, 40],                                # out-of-range lengths are clamped
], ids=["uniform", "long", "ragged", "empty", "clamped"])
def test_plan_bit_exact(mla, lens, n_chunks):
    # The plan sits at the start of the workspace; integer data, compared
    # exactly.  At 128 heads the attention kernel builds the plan itself when
    # it fits its LDS (256 chunks here) and leaves a copy in the workspace;
    # 4096 chunks go through the separate plan kernel.
    b, h = len(lens), 128
    t_max = min(max(max(lens), 1), 131072)
    cache = torch.zeros(b, t_max, 576, dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(b, h, 576, dtype=torch.bfloat16, device="cuda")
    seqlens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    cfg = {"n_chunks": n_chunks}
    ws = torch.zeros(mla.mla_decode_workspace_bytes(torch.bfloat16, b, h, t_max, cfg), dtype=torch.uint8,
                     device="cuda")
    out, lse = mla.mla_decode(q, cache, seqlens, SCALE, workspace=ws, config=cfg)
    torch.cuda.synchronize()
    ref = _plan_model(lens, t_max, n_chunks, 32)
    got = ws[:4 * len(ref)].cpu().view(torch.int32).tolist()
    assert got == ref
    # empty rows are written by whichever kernel holds the plan
    for i, L in enumerate(lens):
        if min(max(L, 0), t_max) == 0:
            assert torch.all(out[i] == 0) and torch.all(torch.isneginf(lse[i]))


# ---------------------------------------------------------------- paged latent cache

def _paginate(w, block_size, seed, spare=3, unused_entry=None):
    """Scatter every row's cache rows into randomly permuted blocks of a pool.
    Spare blocks and the rows past each sequence end hold NaN (the cache tail
    is NaN-poisoned), so a read of any row the method does not use shows up."""
    b, t = w.b, w.t_max
    mb = -(-t // block_size)
    nb = b * mb + spare
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(nb, generator=g)[: b * mb].reshape(b, mb)
    padded = torch.full((b, mb * block_size, 576), float("nan"), dtype=w.cache.dtype, device="cuda")
    padded[:, :t] = w.cache
    pool = torch.full((nb, block_size, 576), float("nan"), dtype=w.cache.dtype, device="cuda")
    pool[perm.reshape(-1).cuda()] = padded.reshape(b * mb, block_size, 576)
    bt = perm.to(torch.int32)
    if unused_entry is not None:
        # entries past a sequence's last block are never read, whatever they hold
        lens = w.seqlens.cpu().tolist()
        for i, L in enumerate(lens):
            bt[i, -(-max(L, 0) // block_size):] = unused_entry
    return pool, bt.cuda()


PAGED_CASES = [
    (128, 64, None), (128, 32, None), (128, 256, None), (100, 64, None), (64, 64, None),
    (16, 64, None), (20, 32, None),
    (128, 64, {"heads_per_group": 128, "variant": 3}), (64, 128, {"heads_per_group": 64, "variant": 5}),
    (128, 64, {"heads_per_group": 128, "variant": 6}), (100, 32, {"heads_per_group": 128, "variant": 6}),
]


@pytest.mark.parametrize("h,bs,cfg", PAGED_CASES, ids=["h%d-bs%d-%s" % c for c in PAGED_CASES])
def test_paged_edges_every_output(mla, h, bs, cfg):
    w = workloads.make_custom(len(EDGE_LENS), h, EDGE_LENS, seed=300 + h + bs, device="cuda")
    pool, bt = _paginate(w, bs, seed=h + bs, unused_entry=-12345)
    for extra in ({}, {"n_chunks": 8}, {"n_chunks": 64}, {"n_chunks": 256}):
        c = dict(cfg or {})
        c.update(extra)
        out, lse = mla.mla_decode_paged(w.q_prime, pool, bt, w.seqlens, w.scale, config=c or None)
        torch.cuda.synchronize()
        check_decode(w.q_prime, w.cache, w.seqlens, w.scale, out, lse, range(w.b))
        assert torch.all(out[EDGE_LENS.index(0)] == 0)
        assert torch.all(torch.isneginf(lse[EDGE_LENS.index(0)]))


def test_paged_clamps_block_entries_and_is_deterministic(mla):
    # an out-of-range entry that is read is clamped into the pool: the result is
    # the decode over the rows gathered with the clamped table
    # t_max = 5 whole blocks and no poisoning: every pool row is finite
    w = workloads.make_custom(3, 128, [300, 64, 129], t_max=320, seed=41, device="cuda",
                              poison=False)
    pool, bt = _paginate(w, 64, seed=5, spare=0)
    nb = pool.shape[0]
    bt[0, 1] = nb + 17   # -> block nb - 1
    bt[2, 0] = -4        # -> block 0
    bt_c = bt.clamp(0, nb - 1).long().cpu()
    gathered = pool[bt_c.reshape(-1).cuda()].reshape(3, -1, 576)[:, : w.t_max].contiguous()
    out, lse = mla.mla_decode_paged(w.q_prime, pool, bt, w.seqlens, w.scale)
    out2, lse2 = mla.mla_decode_paged(w.q_prime, pool, bt, w.seqlens, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    check_decode(w.q_prime, gathered, w.seqlens, w.scale, out, lse, range(3))


# ---------------------------------------------------------------- fp8 latent cache

def _fp8_from(w, poison=True):
    """Quantise w's cache with the oracle's quantiser (test input); codes and
    scales past each sequence end are NaN (0x7F, NaN scale) when poisoned."""
    from oracle import fp8 as ofp8
    lens = w.seqlens.cpu().tolist()
    x = w.cache.float().cpu().numpy()
    x = np.nan_to_num(x, nan=0.0)
    codes, scale = ofp8.quantize_rows(x)
    if poison:
        for i, L in enumerate(lens):
            codes[i, max(L, 0):] = 0x7F
            scale[i, max(L, 0):] = np.nan
    return (torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda(),
            ofp8.dequantize(codes, np.nan_to_num(scale)))


def test_fp8_quantiser_bit_exact(mla):
    # integer codes decided in fp32 on both sides: compared exactly
    from oracle import fp8 as ofp8
    w = workloads.make_custom(3, 16, [700, 1, 333], seed=51, device="cuda", poison=False)
    w.cache[1, 5] = 0.0                       # an all-zero row
    w.cache[2, 7, 9] = -0.0
    codes, scale = mla.mla_quantize_cache_fp8(w.cache)
    torch.cuda.synchronize()
    rc, rs = ofp8.quantize_rows(w.cache.float().cpu().numpy())
    np.testing.assert_array_equal(scale.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


FP8_CASES = [16, 1, 3, 20, 128]


@pytest.mark.parametrize("h", FP8_CASES, ids=["h%d" % h for h in FP8_CASES])
def test_fp8_edges_every_output(mla, h):
    w = workloads.make_custom(len(EDGE_LENS), h, EDGE_LENS, seed=500 + h, device="cuda")
    codes, scale, deq = _fp8_from(w)
    ref_out, ref_lse = oracle.decode_latent(w.q_prime.cpu(), deq, w.seqlens.cpu(), w.scale)
    # the 16-head kernel (exact bf16 queries) also at more than 64 heads, where
    # the automatic choice is the FP8-MFMA kernel
    base = {"heads_per_group": 16} if h > 64 else {}
    assert mla.mla_decode_fp8_kernel_name(h, base or None).startswith("decode_bf16_kernel<16")
    for extra in ({}, {"n_chunks": 8}, {"n_chunks": 64}, {"n_chunks": 256}):
        cfg = dict(base, **extra)
        out, lse = mla.mla_decode_fp8(w.q_prime, codes, scale, w.seqlens, w.scale, config=cfg or None)
        torch.cuda.synchronize()
        assert_out(to_np(out), ref_out, BF16_OUT_REL, "out %s" % extra)
        assert_lse(to_np(lse), ref_lse, BF16_LSE_ABS)
        assert torch.all(out[EDGE_LENS.index(0)] == 0)
        assert torch.all(torch.isneginf(lse[EDGE_LENS.index(0)]))


def test_full_few_heads_fp8_b128_h16_T8192(mla):
    # the few-heads configuration with its cache quantised on the GPU; sampled
    # rows against the oracle fed the same codes (decoded exactly)
    from oracle import fp8 as ofp8
    w = workloads.make(3, device="cuda", poison=False)
    codes, scale = mla.mla_quantize_cache_fp8(w.cache)
    out, lse = mla.mla_decode_fp8(w.q_prime, codes, scale, w.seqlens, w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    rows = [0, 1, 77, 127]
    deq = ofp8.dequantize(codes[rows].cpu().numpy(), scale[rows].cpu().numpy())
    ref_out, ref_lse = oracle.decode_latent(w.q_prime[rows].cpu(), deq, w.seqlens[rows].cpu(), w.scale)
    assert_out(to_np(out[rows]), ref_out, BF16_OUT_REL)
    assert_lse(to_np(lse[rows]), ref_lse, BF16_LSE_ABS)


# ------------------------------------------- fp8 cache, 128-head FP8-MFMA kernel

def _fp8_query_deq(q_prime):
    """The FP8-MFMA path's quantised queries (the oracle's quantiser, the same
    fp32 steps the kernel takes), dequantised exactly in fp64."""
    from oracle import fp8 as ofp8
    codes, sigma = ofp8.quantize_query(q_prime.float().cpu().numpy())
    return ofp8.decode(codes) * sigma[..., None].astype(np.float64)


# The FP8 MFMA adds its 64 exact code products with less than fp32
# precision: a probe of v_mfma_scale_f32_32x32x64_f8f6f4 on random codes put
# the error of one score at up to 2^-15.4 of sum |a b|, and the large-score
# test below at 2^-13.8.  The FP8-MFMA checks allow 2^-12 of
# scale * sum_i |q8_i k_i| per score.
FP8_MFMA_SUM_REL = 2.0 ** -12


def check_fp8_mfma(out, lse, qdeq, kdeq, lens, scale, ref_out, ref_lse, extra_d=None, what="out"):
    """out/lse of the FP8-MFMA kernel against the oracle fed the same query
    and cache codes.  Each score may be off by d_t = 2^-12 * scale *
    sum_i |q_i k_t,i|; with D = max_t d_t for a (row, head) the lse may move by
    D and every softmax weight by a factor within [e^-2D, e^2D], so out by
    (e^2D - 1) * max_t |v_t| per column -- on top of the bf16 bar.  extra_d
    [b, h] adds to D (a further bounded score perturbation)."""
    got_o, got_l = to_np(out), to_np(lse)
    assert np.all(np.isfinite(got_o)), "%s has non-finite values" % what
    bar = BF16_OUT_REL * float(np.max(np.abs(ref_out)))
    for r, L in enumerate(lens):
        if L <= 0:
            assert np.all(got_o[r] == 0) and np.all(np.isneginf(got_l[r]))
            continue
        k = kdeq[r, :L]
        D = FP8_MFMA_SUM_REL * scale * (np.abs(qdeq[r]) @ np.abs(k).T).max(axis=1)   # [h]
        if extra_d is not None:
            D = D + extra_d[r]
        vmax = np.abs(k[:, :512]).max(axis=0)
        err = np.abs(got_o[r] - ref_out[r])
        bound = np.expm1(2 * D)[:, None] * vmax[None, :] + bar
        assert np.all(err <= bound), "%s row %d: max|err| %.3e beyond the bound" % (what, r, err.max())
        lerr = np.abs(got_l[r] - ref_lse[r])
        assert np.all(lerr <= D + BF16_LSE_ABS), "%s row %d: lse err %.3e" % (what, r, lerr.max())


FP8_WIDE_CASES = [128, 100, 65, 256]


@pytest.mark.parametrize("h", FP8_WIDE_CASES, ids=["h%d" % h for h in FP8_WIDE_CASES])
def test_fp8_wide_every_output(mla, h):
    # Query codes decided in fp32 on both sides: against the oracle fed the
    # same codes (and the same cache codes), what is left is the bf16
    # probabilities, fp32 accumulation and the bf16 output -- the bf16 bar.
    w = workloads.make_custom(len(EDGE_LENS), h, EDGE_LENS, seed=800 + h, device="cuda")
    codes, scale, deq = _fp8_from(w)
    assert mla.mla_decode_fp8_kernel_name(h) == "decode_wide_fp8_kernel"
    qd = _fp8_query_deq(w.q_prime)
    ref_out, ref_lse = oracle.decode_latent(qd, deq, w.seqlens.cpu(), w.scale)
    # 2560 chunks: more than the kernel plans in its own LDS (plan kernel)
    for extra in ({}, {"n_chunks": 8}, {"n_chunks": 64}, {"n_chunks": 256}, {"n_chunks": 2560}):
        out, lse = mla.mla_decode_fp8(w.q_prime, codes, scale, w.seqlens, w.scale, config=extra or None)
        torch.cuda.synchronize()
        check_fp8_mfma(out, lse, qd, deq, EDGE_LENS, w.scale, ref_out, ref_lse, what="out %s" % extra)
        assert torch.all(out[EDGE_LENS.index(0)] == 0)
        assert torch.all(torch.isneginf(lse[EDGE_LENS.index(0)]))
        out2, lse2 = mla.mla_decode_fp8(w.q_prime, codes, scale, w.seqlens, w.scale, config=extra or None)
        assert torch.equal(out, out2) and torch.equal(lse, lse2), "not deterministic"


def test_fp8_wide_running_max_growth(mla):
    # The bf16 rescale construction on the fp8 path: scores that grow tile
    # after tile for some heads (lazy rescale of the AGPR outputs), not for others.
    h = 128
    w = workloads.make_custom(4, h, [700, 257, 1000, 33], seed=61 + h, device="cuda", poison=False)
    t = torch.arange(w.t_max, device="cuda", dtype=torch.float32)
    w.cache[:, :, 575] = (0.25 * t).to(torch.bfloat16)[None, :]
    slope = torch.tensor([16.0, 4.0, 1.0, 0.0, -4.0, 0.5, 8.0, -1.0], device="cuda")
    per_head = slope[torch.arange(h, device="cuda") % 8]
    per_head = torch.where((torch.arange(h, device="cuda") // 32) % 2 == 1, -per_head.abs(), per_head)
    w.q_prime[:, :, 575] = per_head.to(torch.bfloat16)[None, :]
    codes, scale, deq = _fp8_from(w)
    qd = _fp8_query_deq(w.q_prime)
    ref_out, ref_lse = oracle.decode_latent(qd, deq, w.seqlens.cpu(), w.scale)
    for extra in ({}, {"n_chunks": 8}, {"n_chunks": 64}):
        out, lse = mla.mla_decode_fp8(w.q_prime, codes, scale, w.seqlens, w.scale, config=extra or None)
        torch.cuda.synchronize()
        check_fp8_mfma(out, lse, qd, deq, [700, 257, 1000, 33], w.scale, ref_out, ref_lse, what="out %s" % extra)


def test_fp8_wide_query_quantisation_bound(mla):
    # Against the oracle with the exact bf16 queries (and the same cache
    # codes).  Quantising a query moves its score with token t by
    # d_t = scale * (q - q8) . k_t; with D = max_t |d_t| for a (row, head),
    # every softmax weight moves by a factor within [e^-2D, e^2D], so
    # |out - out_exact| <= (e^2D - 1) * max_t |v_t| per column and
    # |lse - lse_exact| <= D.  Checked per (row, head), with D added to the
    # FP8-MFMA allowance, on top of the bf16 bar.
    h = 128
    lens = [700, 1, 257, 64, 1000]
    w = workloads.make_custom(len(lens), h, lens, seed=77, device="cuda")
    codes, scale, deq = _fp8_from(w)
    out, lse = mla.mla_decode_fp8(w.q_prime, codes, scale, w.seqlens, w.scale)
    torch.cuda.synchronize()
    q = w.q_prime.double().cpu().numpy()
    qd = _fp8_query_deq(w.q_prime)
    ref_out, ref_lse = oracle.decode_latent(q, deq, w.seqlens.cpu(), w.scale)
    d_quant = np.zeros((len(lens), h))
    for r, L in enumerate(lens):
        d_quant[r] = (w.scale * np.abs((q[r] - qd[r]) @ deq[r, :L].T)).max(axis=1)
    print("largest score move from quantising the queries: %.4f" % d_quant.max())
    check_fp8_mfma(out, lse, qd, deq, lens, w.scale, ref_out, ref_lse, extra_d=d_quant)


def test_full_dsv3_decode_fp8_b64_h128_T4096(mla):
    # the 128-head configuration with its cache quantised on the GPU; sampled
    # rows against the oracle fed the same cache and query codes
    from oracle import fp8 as ofp8
    w = workloads.make(2, device="cuda", poison=False)
    codes, scale = mla.mla_quantize_cache_fp8(w.cache)
    out, lse = mla.mla_decode_fp8(w.q_prime, codes, scale, w.seqlens, w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    rows = [0, 1, 33, 63]
    deq = ofp8.dequantize(codes[rows].cpu().numpy(), scale[rows].cpu().numpy())
    qd = _fp8_query_deq(w.q_prime[rows])
    ref_out, ref_lse = oracle.decode_latent(qd, deq, w.seqlens[rows].cpu(), w.scale)
    check_fp8_mfma(out[rows], lse[rows], qd, deq, w.seqlens[rows].tolist(), w.scale, ref_out, ref_lse)


# ---------------------------------------------------------------- engine-clock stamps

def test_record_clock_stamps(mla):
    # the measurement hook: stamps only when asked for, a plausible engine
    # clock, and the same results either way
    w = workloads.make_custom(4, 128, [700, 1, 2048, 300], seed=5, device="cuda", poison=False)
    cases = [({}, "decode_wide_kernel"), ({"heads_per_group": 16}, "decode_bf16_kernel"),
             ({"heads_per_group": 128, "variant": 6}, "decode_colsplit_kernel")]
    for cfg, name in cases:
        assert mla.mla_decode_kernel_name(torch.bfloat16, 128, cfg or None).startswith(name)
        ws = torch.zeros(mla.mla_decode_workspace_bytes(torch.bfloat16, 4, 128, w.t_max, cfg or None),
                         dtype=torch.uint8, device="cuda")
        out, lse = mla.mla_decode(w.q_prime, w.cache, w.seqlens, w.scale, workspace=ws, config=cfg or None)
        torch.cuda.synchronize()
        assert mla.read_clock_mhz(ws) is None, name   # not asked for: the area stays zero
        c = dict(cfg, record_clock=True)
        out2, lse2 = mla.mla_decode(w.q_prime, w.cache, w.seqlens, w.scale, workspace=ws, config=c)
        torch.cuda.synchronize()
        mhz = mla.read_clock_mhz(ws)
        assert mhz is not None and 300.0 < mhz < 4000.0, (name, mhz)
        assert torch.equal(out, out2) and torch.equal(lse, lse2), name
    codes, scale = mla.mla_quantize_cache_fp8(w.cache)
    ws = torch.zeros(mla.mla_decode_fp8_workspace_bytes(4, 128, w.t_max), dtype=torch.uint8, device="cuda")
    mla.mla_decode_fp8(w.q_prime, codes, scale, w.seqlens, w.scale, workspace=ws, config={"record_clock": True})
    torch.cuda.synchronize()
    mhz = mla.read_clock_mhz(ws)
    assert mhz is not None and 300.0 < mhz < 4000.0, ("fp8", mhz)


# ---------------------------------------------------------------- absorbs, bf16

@pytest.mark.parametrize("b,h", [(64, 128), (100, 16), (3, 8), (70, 13)])
def test_absorbs_bf16(mla, b, h):
    # b = 100: two rounds of the 64-row load groups, the second one ragged;
    # h = 13: workgroups past the last whole group of 8 heads keep their ids
    q_nope, q_rope, w_uk, w_uv = workloads.make_step_weights(b, h, device="cuda")
    qp = mla.mla_absorb_q(q_nope, w_uk, q_rope)
    o = torch.randn(b, h, 512, device="cuda").to(torch.bfloat16)
    y = mla.mla_absorb_o(o, w_uv)
    torch.cuda.synchronize()
    ref_q = oracle.absorb_q(q_nope.cpu(), w_uk.cpu(), q_rope.cpu())
    assert_out(to_np(qp), ref_q, BF16_OUT_REL, "q'")
    np.testing.assert_array_equal(to_np(qp[..., 512:]), to_np(q_rope))
    ref_y = oracle.absorb_o(o.cpu(), w_uv.cpu())
    assert_out(to_np(y), ref_y, BF16_OUT_REL, "y")


# ---------------------------------------------------------------- full-size configurations

def _full(mla, cid, rows):
    w = workloads.make(cid, device="cuda")
    out, lse = _run(mla, w)
    assert torch.isfinite(out).all(), "non-finite output (read past a sequence end?)"
    check_decode(w.q_prime, w.cache, w.seqlens, w.scale, out, lse, rows)
    return w, out, lse


def test_full_dsv3_decode_b64_h128_T4096(mla):
    _full(mla, 2, [0, 17, 42, 63])


def test_full_dsv3_decode_colsplit_kernel(mla):
    # the 128-head configuration through the column-split kernel explicitly,
    # sampled rows, run-to-run bit equality
    w = workloads.make(2, device="cuda")
    cfg = {"heads_per_group": 128, "variant": 6}
    out, lse = _run(mla, w, cfg)
    out2, lse2 = _run(mla, w, cfg)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    assert torch.isfinite(out).all()
    check_decode(w.q_prime, w.cache, w.seqlens, w.scale, out, lse, [0, 17, 42, 63])


def test_full_dsv3_decode_paged_bs64(mla):
    # the same configuration through a paged pool (64-token blocks, shuffled)
    w = workloads.make(2, device="cuda")
    pool, bt = _paginate(w, 64, seed=77)
    out, lse = mla.mla_decode_paged(w.q_prime, pool, bt, w.seqlens, w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    check_decode(w.q_prime, w.cache, w.seqlens, w.scale, out, lse, [0, 17, 42, 63])


def test_full_few_heads_b128_h16_T8192(mla):
    _full(mla, 3, [0, 1, 77, 127])


def test_full_ragged_b132_h128(mla):
    w = workloads.make(4, device="cuda")
    lens = w.seqlens.cpu().tolist()
    rows = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 131, 66})
    out, lse = _run(mla, w)
    assert torch.isfinite(out).all()
    check_decode(w.q_prime, w.cache, w.seqlens, w.scale, out, lse, rows)


def test_full_long_context_end_to_end(mla):
    w = workloads.make(5, device="cuda")
    # absorbs in full
    qp_gpu = mla.mla_absorb_q(w.q_nope, w.w_uk, w.q_rope)
    torch.cuda.synchronize()
    qp_ref = oracle.absorb_q(w.q_nope.cpu(), w.w_uk.cpu(), w.q_rope.cpu())
    assert_out(to_np(qp_gpu), qp_ref, BF16_OUT_REL, "q'")
    # decode fed the oracle's q' rounded to bf16; heads sampled
    qp_in = torch.from_numpy(qp_ref).to(torch.bfloat16).cuda()
    out, lse = mla.mla_decode(qp_in, w.cache, w.seqlens, w.scale)
    torch.cuda.synchronize()
    heads = [0, 1, 63, 64, 126, 127]
    check_decode(qp_in, w.cache, w.seqlens, w.scale, out, lse, range(4), heads)
    # end to end (absorb -> decode -> absorb) against the oracle's own pipeline
    bufs = mla.alloc_step(w.b, w.h, w.t_max)
    y = mla.mla_step(w.q_nope, w.q_rope, w.w_uk, w.w_uv, w.cache, w.seqlens, w.scale, bufs)
    torch.cuda.synchronize()
    ref_out, _ = oracle.decode_latent(torch.from_numpy(qp_ref)[:, heads], w.cache.cpu(),
                                      w.seqlens.cpu(), w.scale)
    ref_y = oracle.absorb_o(ref_out, w.w_uv.cpu()[heads])
    assert_out(to_np(y[:, heads]), ref_y, BF16_OUT_REL, "y")


def test_long_context_step_vs_expanded_form(mla):
    # The long-context step (absorb q -> decode -> absorb o, all on the GPU)
    # against the oracle's un-absorbed form -- per-head keys and values
    # expanded from the latent rows, the RoPE score term added, softmax,
    # weighted sum -- on heads 0, 63 and 127 of all four rows.
    w = workloads.make(5, device="cuda")
    heads = [0, 63, 127]
    bufs = mla.alloc_step(w.b, w.h, w.t_max)
    y = mla.mla_step(w.q_nope, w.q_rope, w.w_uk, w.w_uv, w.cache, w.seqlens, w.scale, bufs)
    torch.cuda.synchronize()
    cache = w.cache.cpu()
    y_x, lse_x = oracle.decode_unabsorbed(w.q_nope.cpu(), w.q_rope.cpu(), w.w_uk.cpu(), w.w_uv.cpu(),
                                          cache, w.seqlens.cpu(), w.scale, heads=heads)
    assert_out(to_np(y[:, heads]), y_x, BF16_OUT_REL, "y vs expanded form")
    # The step stores the absorbed query in bf16 (the decode's input dtype);
    # that rounding alone moves the lse by about 1e-3 at this length.  The lse
    # bound is the decode's own (1e-3) on top of that shift, which the oracle
    # computes by itself: its latent form fed its own q' rounded to bf16.
    qp_ref = oracle.absorb_q(w.q_nope.cpu(), w.w_uk.cpu(), w.q_rope.cpu())
    qp_b = torch.from_numpy(qp_ref[:, heads]).to(torch.bfloat16)
    _, lse_b = oracle.decode_latent(qp_b, cache, w.seqlens.cpu(), w.scale)
    shift = float(np.max(np.abs(lse_b - lse_x)))
    assert_lse(to_np(bufs.lse[:, heads]), lse_x, BF16_LSE_ABS + shift, "lse vs expanded form")
    # and the decode itself against the latent form fed the GPU's own q'
    check_decode(bufs.q_prime, w.cache, w.seqlens, w.scale, bufs.out, bufs.lse, range(w.b), heads)


# ---- several causal query tokens per row (mla_decode_mtp) ---------------------

MTP_CASES = [
    # (q_len, h, lengths)
    (2, 128, [700, 257, 1000, 33, 2]),   # 256 query rows: two groups of 128
    (3, 16, [100, 3, 1, 0, 64]),         # 48 rows; lengths below q_len and an empty row
    (4, 8, [129, 32, 31, 5]),            # 32 rows
    (2, 100, [513, 96]),                 # 200 rows, the last group padded
    (8, 16, [300, 40, 8]),               # 128 rows, a row of exactly q_len
    (160, 8, [700, 300, 160]),           # prefill-sized: 1280 query rows per batch row, tiles
                                         # past a query group's causal limits skipped
    (96, 16, [2000, 97, 96]),            # 1536 query rows; most chunks of the long row hold
                                         # tokens only the later query groups see
]


def _mtp_workload(b, q_len, h, lens, seed):
    w = workloads.make_custom(b, q_len * h, lens, seed=seed, device="cuda")
    return w, w.q_prime.view(b, q_len, h, 576)


@pytest.mark.parametrize("q_len,h,lens", MTP_CASES, ids=["q%d-h%d" % (c[0], c[1]) for c in MTP_CASES])
def test_mtp_every_output(mla, q_len, h, lens):
    b = len(lens)
    w, q = _mtp_workload(b, q_len, h, lens, seed=700 + q_len * h)
    ref_o, ref_l = oracle.decode_latent_causal(q.cpu(), w.cache.cpu(), w.seqlens.cpu().numpy(), w.scale)
    n = np.clip(np.array(lens)[:, None] - q_len + 1 + np.arange(q_len)[None, :], 0, None)
    # default schedule (the kernel builds its own plan) and 2560 chunks (too
    # many for its LDS: the separate plan kernel)
    for cfg in (None, {"n_chunks": 2560}):
        out, lse = mla.mla_decode_mtp(q, w.cache, w.seqlens, w.scale, config=cfg)
        torch.cuda.synchronize()
        assert_out(to_np(out), ref_o, BF16_OUT_REL)
        assert_lse(to_np(lse), ref_l, BF16_LSE_ABS)
        # tokens with nothing to attend to: exactly zero output
        for i in range(b):
            for t in range(q_len):
                if n[i, t] == 0:
                    assert torch.all(out[i, t] == 0) and torch.all(torch.isneginf(lse[i, t]))


def test_mtp_one_token_is_decode(mla):
    w = workloads.make_custom(3, 128, [400, 1, 77], seed=81, device="cuda")
    q = w.q_prime.view(3, 1, 128, 576)
    out, lse = mla.mla_decode_mtp(q, w.cache, w.seqlens, w.scale)
    out_d, lse_d = mla.mla_decode(w.q_prime, w.cache, w.seqlens, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(3, 128, 512), out_d) and torch.equal(lse.view(3, 128), lse_d)


def test_mtp_token_matches_decode_of_its_prefix(mla):
    # new token i of a row equals plain decode of the same query over the
    # first L - q_len + 1 + i rows (both within tolerance of the oracle, and
    # of each other)
    b, q_len, h = 2, 4, 64
    lens = [900, 130]
    w, q = _mtp_workload(b, q_len, h, lens, seed=82)
    out, lse = mla.mla_decode_mtp(q, w.cache, w.seqlens, w.scale)
    for i in range(q_len):
        sl = torch.tensor([L - q_len + 1 + i for L in lens], dtype=torch.int32, device="cuda")
        od, ld = mla.mla_decode(q[:, i].contiguous(), w.cache, sl, w.scale)
        assert_out(to_np(out[:, i]), to_np(od), BF16_OUT_REL)
        assert_lse(to_np(lse[:, i]), to_np(ld), BF16_LSE_ABS)


def test_full_dsv3_decode_mtp2_b64_h128_T4096(mla):
    # the 128-head configuration with two query tokens per row; sampled rows
    b, q_len, h, T = 64, 2, 128, 4096
    w = workloads.make_custom(b, q_len * h, [T] * b, seed=83, device="cuda", poison=False)
    q = w.q_prime.view(b, q_len, h, 576)
    out, lse = mla.mla_decode_mtp(q, w.cache, w.seqlens, w.scale)
    torch.cuda.synchronize()
    rows = [0, 37, 63]
    ref_o, ref_l = oracle.decode_latent_causal(q[rows].cpu(), w.cache[rows].cpu(),
                                               w.seqlens[rows].cpu().numpy(), w.scale)
    assert_out(to_np(out[rows]), ref_o, BF16_OUT_REL)
    assert_lse(to_np(lse[rows]), ref_l, BF16_LSE_ABS)


# ---- appending a token's latent row (mla_cache_append) ------------------------

def _append_inputs(b, d_model, t_max, n_pos, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(b, d_model, generator=g).to(torch.bfloat16)
    wd = (torch.randn(d_model, 512, generator=g) / math.sqrt(d_model)).to(torch.bfloat16)
    wr = (torch.randn(d_model, 64, generator=g) / math.sqrt(d_model)).to(torch.bfloat16)
    cache = torch.randn(b, t_max, 576, generator=g).to(torch.bfloat16)
    # caller-chosen rotation tables (RoFormer-style angles, base 10000)
    ang = np.arange(n_pos)[:, None] * 10000.0 ** (-np.arange(32)[None, :] / 32.0)
    cos_t = torch.from_numpy(np.cos(ang).astype(np.float32))
    sin_t = torch.from_numpy(np.sin(ang).astype(np.float32))
    return [t.cuda() for t in (x, wd, wr, cos_t, sin_t, cache)]


def _check_append(before, after, ref, lens, t_max, n_pos):
    written = [(i, L) for i, L in enumerate(lens) if 0 <= L < min(t_max, n_pos)]
    got = np.stack([to_np(after[i, L]) for i, L in written])
    want = np.stack([ref[i, L] for i, L in written])
    assert_out(got, want, BF16_OUT_REL, "appended rows")
    mask = torch.ones(after.shape[:2], dtype=torch.bool, device=after.device)
    for i, L in written:
        mask[i, L] = False
    assert torch.equal(after[mask], before[mask]), "rows other than the appended ones changed"


@pytest.mark.parametrize("d_model", [256, 7168])
def test_cache_append_every_row(mla, d_model):
    lens = [0, 7, 47, 48, -3, 20]
    b, t_max, n_pos = len(lens), 48, 48
    x, wd, wr, cos_t, sin_t, cache = _append_inputs(b, d_model, t_max, n_pos, seed=90 + d_model)
    before = cache.clone()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sl_out = torch.empty_like(sl)
    mla.mla_cache_append(x, wd, wr, cos_t, sin_t, cache, sl, sl_out)
    torch.cuda.synchronize()
    ref = oracle.cache_append(x.cpu(), wd.cpu(), wr.cpu(), cos_t.cpu(), sin_t.cpu(), np.array(lens, np.int32),
                              before.cpu())
    _check_append(before, cache, ref, lens, t_max, n_pos)
    assert sl_out.cpu().tolist() == [1, 8, 48, 48, -3, 21]
    assert sl.cpu().tolist() == lens


def test_cache_append_more_than_64_rows(mla):
    # 100 rows: the projection's second block of 64 input rows (ragged: 36),
    # with its fp32 partial sums staged and stored as 256-byte row pieces
    rng = np.random.default_rng(97)
    b, t_max, n_pos, d_model = 100, 24, 24, 768
    lens = [int(v) for v in rng.integers(-2, t_max + 2, size=b)]
    x, wd, wr, cos_t, sin_t, cache = _append_inputs(b, d_model, t_max, n_pos, seed=97)
    before = cache.clone()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sl_out = torch.empty_like(sl)
    mla.mla_cache_append(x, wd, wr, cos_t, sin_t, cache, sl, sl_out)
    torch.cuda.synchronize()
    ref = oracle.cache_append(x.cpu(), wd.cpu(), wr.cpu(), cos_t.cpu(), sin_t.cpu(), np.array(lens, np.int32),
                              before.cpu())
    _check_append(before, cache, ref, lens, t_max, n_pos)
    assert sl_out.cpu().tolist() == [L + 1 if 0 <= L < t_max else L for L in lens]


def test_cache_append_in_place_lengths_and_table_bound(mla):
    # seqlens updated in place; a position past the tables (n_pos < t_max) is not written
    lens = [3, 10, 9]
    b, t_max, n_pos = 3, 16, 10
    x, wd, wr, cos_t, sin_t, cache = _append_inputs(b, 512, t_max, n_pos, seed=95)
    before = cache.clone()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    mla.mla_cache_append(x, wd, wr, cos_t, sin_t, cache, sl, sl)
    torch.cuda.synchronize()
    ref = oracle.cache_append(x.cpu(), wd.cpu(), wr.cpu(), cos_t.cpu(), sin_t.cpu(), np.array(lens, np.int32),
                              before.cpu())
    _check_append(before, cache, ref, lens, t_max, n_pos)
    assert sl.cpu().tolist() == [4, 10, 10]


def test_cache_append_then_decode(mla):
    # one decode step: append the new token, then attend with it included
    b, h, d_model, t_max = 4, 128, 7168, 600
    lens = [599, 0, 257, 31]
    x, wd, wr, cos_t, sin_t, cache = _append_inputs(b, d_model, t_max, t_max, seed=96)
    before = cache.clone()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    mla.mla_cache_append(x, wd, wr, cos_t, sin_t, cache, sl, sl)
    g = torch.Generator().manual_seed(97)
    q = torch.randn(b, h, 576, generator=g).to(torch.bfloat16).cuda()
    out, lse = mla.mla_decode(q, cache, sl, 1.0 / math.sqrt(192.0))
    torch.cuda.synchronize()
    ref = oracle.cache_append(x.cpu(), wd.cpu(), wr.cpu(), cos_t.cpu(), sin_t.cpu(), np.array(lens, np.int32),
                              before.cpu())
    _check_append(before, cache, ref, lens, t_max, t_max)
    # attention over the cache as the GPU wrote it (the appended row included)
    check_decode(q, cache, sl, 1.0 / math.sqrt(192.0), out, lse, range(b))


def test_cache_append_dsv3_b64(mla):
    # the hidden width of the glossary's example (7168), 64 rows at position 4095
    b, d_model, t_max = 64, 7168, 4096
    x, wd, wr, cos_t, sin_t, cache = _append_inputs(b, d_model, t_max, t_max, seed=98)
    before = cache.clone()
    lens = [4095] * b
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    mla.mla_cache_append(x, wd, wr, cos_t, sin_t, cache, sl)
    torch.cuda.synchronize()
    rows = [0, 33, 63]
    ref = oracle.cache_append(x[rows].cpu(), wd.cpu(), wr.cpu(), cos_t.cpu(), sin_t.cpu(),
                              np.array([4095] * 3, np.int32), before[rows].cpu())
    got = np.stack([to_np(cache[r, 4095]) for r in rows])
    assert_out(got, ref[:, 4095], BF16_OUT_REL, "appended rows")
    assert torch.equal(cache[:, :4095], before[:, :4095])


# ---- paged forms of the multi-token decode and the append ---------------------

@pytest.mark.parametrize("q_len,h,lens,bs", [
    (2, 128, [700, 257, 1000, 33, 2], 64), (3, 16, [100, 3, 1, 0, 64], 32), (4, 32, [129, 4, 96], 128),
], ids=["q2-h128-bs64", "q3-h16-bs32", "q4-h32-bs128"])
def test_mtp_paged_every_output(mla, q_len, h, lens, bs):
    b = len(lens)
    w, q = _mtp_workload(b, q_len, h, lens, seed=710 + q_len * h + bs)
    pool, bt = _paginate(w, bs, seed=q_len + bs, unused_entry=-777)
    out, lse = mla.mla_decode_mtp_paged(q, pool, bt, w.seqlens, w.scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.decode_latent_causal(q.cpu(), w.cache.cpu(), w.seqlens.cpu().numpy(), w.scale)
    assert_out(to_np(out), ref_o, BF16_OUT_REL)
    assert_lse(to_np(lse), ref_l, BF16_LSE_ABS)
    # the contiguous call agrees within the same tolerance
    out_c, lse_c = mla.mla_decode_mtp(q, w.cache, w.seqlens, w.scale)
    assert_out(to_np(out), to_np(out_c), BF16_OUT_REL)


def test_cache_append_paged(mla):
    # rows scattered over a shuffled pool; the written block comes from the table
    lens = [0, 70, 127, 128, 200, 63]
    b, bs, mb, d_model = len(lens), 64, 4, 512
    nb = b * mb + 2
    x, wd, wr, cos_t, sin_t, _ = _append_inputs(b, d_model, 1, bs * mb, seed=99)
    g = torch.Generator().manual_seed(100)
    pool = torch.randn(nb, bs, 576, generator=g).to(torch.bfloat16).cuda()
    bt = torch.randperm(nb, generator=g)[: b * mb].reshape(b, mb).to(torch.int32)
    bt[5, 0] = nb + 3   # row 5 writes at position 63 of block 0: out of the pool, no write
    bt = bt.cuda()
    before = pool.clone()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sl_out = torch.empty_like(sl)
    mla.mla_cache_append_paged(x, wd, wr, cos_t, sin_t, pool, bt, sl, sl_out)
    torch.cuda.synchronize()
    assert sl_out.cpu().tolist() == [1, 71, 128, 129, 201, 63]
    # the oracle appends into the gathered contiguous view; compare the written rows
    btc = bt.long().cpu()
    gathered = torch.zeros(b, mb * bs, 576, dtype=torch.bfloat16)
    for i in range(b):
        for k in range(mb):
            if 0 <= btc[i, k] < nb:
                gathered[i, k * bs:(k + 1) * bs] = before[btc[i, k]].cpu()
    ref = oracle.cache_append(x.cpu(), wd.cpu(), wr.cpu(), cos_t.cpu(), sin_t.cpu(), np.array(lens, np.int32),
                              gathered)
    changed = torch.zeros(nb, bs, dtype=torch.bool)
    got, want = [], []
    for i, L in enumerate(lens):
        if i == 5:
            continue
        blk, r = int(btc[i, L // bs]), L % bs
        changed[blk, r] = True
        got.append(to_np(pool[blk, r]))
        want.append(ref[i, L])
    assert_out(np.stack(got), np.stack(want), BF16_OUT_REL, "appended rows")
    assert torch.equal(pool.cpu()[~changed], before.cpu()[~changed]), "other pool rows changed"


@pytest.mark.parametrize("h", [16, 128])
def test_large_batch_short_rows(mla, h):
    # more batch rows than the plan kernel's grid (its workgroups then loop over
    # rows): many short and empty rows; sampled rows against the oracle, every
    # empty row exactly zero
    b = 3000
    g = torch.Generator().manual_seed(120 + h)
    lens = torch.randint(0, 101, (b,), generator=g)
    lens[::7] = 0
    w = workloads.make_custom(b, h, lens.tolist(), seed=121 + h, device="cuda")
    out, lse = mla.mla_decode(w.q_prime, w.cache, w.seqlens, w.scale)
    torch.cuda.synchronize()
    rows = [0, 1, 2, 1499, 2047, 2048, 2049, 2998, 2999] + list(range(3, 3000, 97))
    check_decode(w.q_prime, w.cache, w.seqlens, w.scale, out, lse, rows)
    empty = (lens == 0).nonzero().flatten().tolist()
    assert torch.all(out[empty] == 0) and torch.all(torch.isneginf(lse[empty]))


@pytest.mark.parametrize("b,n_chunks", [(256, 2048), (257, 2048), (256, 2056)],
                         ids=["lds-plan-full", "rows-past-lds-plan", "chunks-past-lds-plan"])
def test_wide_kernel_plan_limits(mla, b, n_chunks):
    # At 128 heads the attention kernel builds the split plan in its LDS for up
    # to 256 rows and 2048 chunks (256 x 2048 fills that array exactly); one
    # row or one chunk group more and the separate plan kernel runs instead.
    # Short rows, every seventh empty: each row is compared with the oracle
    # and every empty row must be exactly zero on both sides of the limit.
    h = 128
    g = torch.Generator().manual_seed(130 + b + n_chunks)
    lens = torch.randint(0, 300, (b,), generator=g)
    lens[::7] = 0
    w = workloads.make_custom(b, h, lens.tolist(), seed=131 + b, device="cuda")
    cfg = {"n_chunks": n_chunks}
    ws = torch.zeros(mla.mla_decode_workspace_bytes(torch.bfloat16, b, h, w.t_max, cfg), dtype=torch.uint8,
                     device="cuda")
    out, lse = mla.mla_decode(w.q_prime, w.cache, w.seqlens, w.scale, workspace=ws, config=cfg)
    torch.cuda.synchronize()
    check_decode(w.q_prime, w.cache, w.seqlens, w.scale, out, lse, range(b), [0, 31, 64, 127])
    empty = (lens == 0).nonzero().flatten().tolist()
    assert torch.all(out[empty] == 0) and torch.all(torch.isneginf(lse[empty]))
    # the plan left in the workspace is the split rule exactly
    ref = _plan_model(lens.tolist(), w.t_max, n_chunks, 32)
    assert ws[:4 * len(ref)].cpu().view(torch.int32).tolist() == ref


def test_two_head_groups_with_empty_rows(mla):
    # 256 heads: two groups of 128, each its own attention workgroup per chunk
    # (both build the same plan); empty rows must be zero across all 256 heads.
    lens = [0, 700, 33, 0, 1, 4096, 257, 0]
    w = workloads.make_custom(len(lens), 256, lens, seed=141, device="cuda")
    for cfg in (None, {"n_chunks": 64}, {"n_chunks": 2560}):
        out, lse = _run(mla, w, cfg)
        check_decode(w.q_prime, w.cache, w.seqlens, w.scale, out, lse, range(w.b),
                     [0, 1, 127, 128, 129, 200, 255])
        for i, L in enumerate(lens):
            if L == 0:
                assert torch.all(out[i] == 0) and torch.all(torch.isneginf(lse[i]))
