"""mla_decode_noalloc (the library's own device array as the workspace)
against mla_decode with a caller workspace, through the C ABI: two calls in a
row, the second on a smaller problem, each bit-identical to mla_decode (same
kernels, same schedule) and within the bf16 tolerance of the fp64 oracle."""
import pytest
import torch

import workloads
from parity_util import check_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_latent_attention_decode_amd as m
    return m


def test_noalloc_matches_decode_twice(mla):
    cases = [
        (128, [4096, 700, 1, 0, 3000, 257, 33, 1500], 11),   # larger first
        (64, [500, 33, 1], 12),                               # then smaller: stale contents must not matter
    ]
    for h, lens, seed in cases:
        w = workloads.make_custom(len(lens), h, lens, seed=seed, device="cuda")
        ref_out, ref_lse = mla.mla_decode(w.q_prime, w.cache, w.seqlens, w.scale)
        out = torch.full_like(ref_out, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        mla.mla_decode_noalloc(w.q_prime, w.cache, w.seqlens, w.scale, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        check_decode(w.q_prime, w.cache, w.seqlens, w.scale, out, lse, range(w.b))


def test_noalloc_rejects_problems_past_its_array(mla):
    # 300 rows of 128 heads need more workspace than the array holds: refused
    # on the host with MLA_ERR_WORKSPACE_TOO_SMALL before anything is launched
    b, h, t = 300, 128, 64
    need = mla.mla_decode_workspace_bytes(torch.bfloat16, b, h, t)
    assert need > mla.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(b, h, 576, dtype=torch.bfloat16, device="cuda")
    c = torch.zeros(b, t, 576, dtype=torch.bfloat16, device="cuda")
    sl = torch.full((b,), t, dtype=torch.int32, device="cuda")
    out = torch.empty(b, h, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(b, h, dtype=torch.float32, device="cuda")
    with pytest.raises(mla.MLAError) as e:
        mla.mla_decode_noalloc(q, c, sl, workloads.SCALE, out, lse)
    assert e.value.status == 3
