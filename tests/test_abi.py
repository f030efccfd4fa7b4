"""C ABI checks that need no GPU: the library loads, exports every entry point
include/mla355.h declares, computes workspace sizes on the host, and rejects
bad arguments with the documented status before launching anything."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla355.h")


@pytest.fixture(scope="module")
def mla():
    import head_latent_attention_decode_amd as m
    return m


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_three_calls():
    names = _declared_functions()
    for n in ("mla_absorb_q", "mla_decode", "mla_absorb_o", "mla_decode_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(mla):
    lib = ctypes.CDLL(mla.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), "missing export %s" % name
    assert set(_declared_functions()) == set(mla.EXPORTED_SYMBOLS)


def test_library_exports_nothing_but_the_c_abi(mla):
    # dynamic symbols the library defines (functions): exactly the header's
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    res = subprocess.run([nm, "-D", "--defined-only", mla.LIB_PATH], capture_output=True, text=True,
                         check=True)
    funcs = {ln.split()[-1] for ln in res.stdout.splitlines() if len(ln.split()) == 3 and ln.split()[1] == "T"}
    assert funcs == set(_declared_functions()), sorted(funcs ^ set(_declared_functions()))


def test_abi_version_and_status_strings(mla):
    assert mla.abi_version() == 1
    assert mla.status_string(0) == "ok"
    assert mla.status_string(3) == "workspace too small"


def test_workspace_bytes_host_only(mla):
    ws = mla.mla_decode_workspace_bytes(torch.bfloat16, 64, 128, 4096)
    assert ws > 0 and ws % 256 == 0
    # partial slots: at least (chunks + rows) * heads * (512 outputs in dtype + one fp32 lse)
    assert ws >= (8 + 64) * 128 * (512 * 2 + 4)
    n = {"n_chunks": 256, "heads_per_group": 64}
    assert mla.mla_decode_workspace_bytes(torch.bfloat16, 64, 128, 4096, n) >= (256 + 64) * 128 * (512 * 2 + 4)
    assert mla.mla_decode_workspace_bytes(torch.float32, 64, 16, 4096) >= (8 + 64) * 16 * (512 * 4 + 4)
    assert mla.mla_decode_workspace_bytes(torch.bfloat16, 0, 128, 4096) == 0
    assert mla.mla_decode_workspace_bytes(torch.bfloat16, 4, 0, 4096) == 0
    assert mla.mla_decode_workspace_bytes(torch.bfloat16, 4, 8, -1) == 0
    assert mla.mla_decode_workspace_bytes(torch.float32, 2, 16, 257) > 0
    cfg = {"n_chunks": 64, "heads_per_group": 16}
    assert mla.mla_decode_workspace_bytes(torch.bfloat16, 3, 16, 100, cfg) > 0
    assert mla.mla_decode_workspace_bytes(torch.bfloat16, 3, 16, 100, {"n_chunks": 12}) == 0
    assert mla.mla_decode_workspace_bytes(torch.bfloat16, 3, 16, 100, {"heads_per_group": 48}) == 0


# Raw C calls with fake (never dereferenced) device pointers: exactly one
# argument is wrong in each case, so the call must fail in host validation.
A = 0x10000  # aligned fake pointer
SCALE = 0.0721


def _decode(lib, dt=1, b=2, h=16, t=100, q=A, c=A, sl=A, scale=SCALE, out=A, lse=A, ws=A,
            wsb=1 << 30):
    vp = ctypes.c_void_p
    return lib.mla_decode(dt, b, h, t, vp(q), vp(c), vp(sl), ctypes.c_float(scale), vp(out),
                          vp(lse), vp(ws), ctypes.c_size_t(wsb), vp(0))


@pytest.mark.parametrize("kw,status", [
    ({"q": 0}, 1), ({"c": 0}, 1), ({"sl": 0}, 1), ({"out": 0}, 1), ({"lse": 0}, 1),
    ({"ws": 0}, 1), ({"b": 0}, 1), ({"h": -1}, 1), ({"t": -5}, 1), ({"dt": 7}, 1),
    ({"q": A + 8}, 1), ({"c": A + 2}, 1), ({"out": A + 4}, 1), ({"ws": A + 16}, 1),
    ({"scale": 0.0}, 1), ({"scale": -1.0}, 1), ({"scale": float("nan")}, 1),
    ({"scale": float("inf")}, 1), ({"wsb": 1024}, 3), ({"b": 1 << 20, "t": 1 << 12}, 1),
])
def test_decode_validation(mla, kw, status):
    lib = ctypes.CDLL(mla.LIB_PATH)
    assert _decode(lib, **kw) == status


def test_decode_ex_rejects_bad_config(mla):
    lib = ctypes.CDLL(mla.LIB_PATH)
    vp = ctypes.c_void_p
    for cfg in ({"n_chunks": 12}, {"n_chunks": 1 << 20}, {"heads_per_group": 24},
                {"variant": 9}, {"reserved": (ctypes.c_int * 5)(2, 0, 0, 0, 0)},
                {"reserved": (ctypes.c_int * 5)(1, 1, 0, 0, 0)}):
        c = mla.MLAConfig()
        for k, v in cfg.items():
            setattr(c, k, v)
        st = lib.mla_decode_ex(1, 2, 16, 100, vp(A), vp(A), vp(A), ctypes.c_float(SCALE), vp(A),
                               vp(A), vp(A), ctypes.c_size_t(1 << 30), ctypes.byref(c), vp(0))
        assert st == 2, cfg


def test_record_clock_flag(mla):
    # reserved[0] = MLA_CONFIG_RECORD_CLOCK is the one accepted non-zero
    # reserved value; the workspace always ends with the stamp area
    assert mla.CONFIG_RECORD_CLOCK == 1 and mla.CLOCK_BYTES == 256
    text = open(os.path.join(ROOT, "include", "mla355.h")).read()
    assert "#define MLA_CONFIG_RECORD_CLOCK 1" in text and "#define MLA_CLOCK_BYTES 256" in text
    plain = mla.mla_decode_workspace_bytes(torch.bfloat16, 64, 128, 4096)
    assert plain == mla.mla_decode_workspace_bytes(torch.bfloat16, 64, 128, 4096, {"record_clock": True})
    assert plain % 256 == 0 and plain >= 256
    assert mla.mla_decode_kernel_name(torch.bfloat16, 128, {"record_clock": True}) == \
        mla.mla_decode_kernel_name(torch.bfloat16, 128)
    assert mla.mla_decode_mtp_workspace_bytes(4, 2, 16, 100, {"record_clock": True}) > 0


def test_absorb_validation(mla):
    lib = ctypes.CDLL(mla.LIB_PATH)
    vp = ctypes.c_void_p
    assert lib.mla_absorb_q(1, 4, 8, vp(0), vp(A), vp(A), vp(A), vp(0)) == 1
    assert lib.mla_absorb_q(1, 4, 8, vp(A), vp(A + 4), vp(A), vp(A), vp(0)) == 1
    assert lib.mla_absorb_q(1, 0, 8, vp(A), vp(A), vp(A), vp(A), vp(0)) == 1
    assert lib.mla_absorb_q(5, 4, 8, vp(A), vp(A), vp(A), vp(A), vp(0)) == 1
    assert lib.mla_absorb_o(1, 4, 8, vp(A), vp(0), vp(A), vp(0)) == 1
    assert lib.mla_absorb_o(1, 4, 0, vp(A), vp(A), vp(A), vp(0)) == 1
    assert lib.mla_absorb_o(0, 4, 8, vp(A), vp(A), vp(A + 2), vp(0)) == 1


def test_python_binding_checks_tensors(mla):
    q = torch.zeros(2, 16, 576, dtype=torch.bfloat16)  # CPU tensor: rejected before any call
    with pytest.raises(ValueError):
        mla.mla_decode(q, torch.zeros(2, 8, 576, dtype=torch.bfloat16),
                       torch.zeros(2, dtype=torch.int32), 0.07)
    with pytest.raises(TypeError):
        mla.mla_decode_workspace_bytes(torch.float16, 2, 16, 8)


def test_decode_kernel_name_host_only(mla):
    # the schedule picks a kernel per head count; the query makes no HIP call
    assert mla.mla_decode_kernel_name(torch.bfloat16, 128) == "decode_wide_kernel<4, 2, false>"
    assert mla.mla_decode_kernel_name(torch.bfloat16, 16).startswith("decode_bf16_kernel<16,")
    assert mla.mla_decode_kernel_name(torch.float32, 16) == "decode_f32_kernel"
    assert mla.mla_decode_kernel_name(torch.bfloat16, 64, {"heads_per_group": 64, "variant": 3}) == \
        "decode_pair_kernel<2, 4>"
    # rejected configurations give no name
    assert mla.mla_decode_kernel_name(torch.bfloat16, 0) is None
    assert mla.mla_decode_kernel_name(torch.bfloat16, 64, {"heads_per_group": 64, "variant": 4}) is None
    assert mla.mla_decode_kernel_name(torch.bfloat16, 64, {"variant": 99}) is None


def _decode_paged(lib, dt=1, b=2, h=16, q=A, pool=A, nb=8, bs=64, bt=A, mb=4, sl=A, scale=SCALE,
                  out=A, lse=A, ws=A, wsb=1 << 30):
    vp = ctypes.c_void_p
    return lib.mla_decode_paged(dt, b, h, vp(q), vp(pool), nb, bs, vp(bt), mb, vp(sl),
                                ctypes.c_float(scale), vp(out), vp(lse), vp(ws),
                                ctypes.c_size_t(wsb), vp(0))


@pytest.mark.parametrize("kw,status", [
    ({"dt": 0}, 2), ({"dt": 5}, 1), ({"bs": 48}, 1), ({"bs": 0}, 1), ({"bs": 16}, 1),
    ({"nb": 0}, 1), ({"mb": 0}, 1), ({"b": 0}, 1), ({"h": 0}, 1), ({"bt": 0}, 1), ({"pool": 0}, 1),
    ({"sl": 0}, 1), ({"pool": A + 8}, 1), ({"bt": A + 4}, 1), ({"ws": A + 64}, 1),
    ({"scale": 0.0}, 1), ({"wsb": 1024}, 3), ({"b": 1 << 15, "mb": 1 << 10}, 1),
])
def test_decode_paged_validation(mla, kw, status):
    lib = ctypes.CDLL(mla.LIB_PATH)
    assert _decode_paged(lib, **kw) == status


def test_decode_paged_host_queries(mla):
    # only the wide kernels address a block pool; the query makes no HIP call
    assert mla.mla_decode_paged_kernel_name(128) == "decode_wide_kernel<4, 2, true>"
    assert mla.mla_decode_paged_kernel_name(100) == "decode_wide_kernel<4, 2, true>"
    assert mla.mla_decode_paged_kernel_name(64) == "decode_wide_kernel<2, 2, true>"
    assert mla.mla_decode_paged_kernel_name(16) == "decode_wide_kernel<1, 3, true>"
    assert mla.mla_decode_paged_kernel_name(128, {"heads_per_group": 128, "variant": 3}) == \
        "decode_wide_kernel<4, 3, true>"
    assert mla.mla_decode_paged_kernel_name(16, {"heads_per_group": 16}) is None
    assert mla.mla_decode_paged_kernel_name(64, {"heads_per_group": 64, "variant": 3}) is None
    lib = ctypes.CDLL(mla.LIB_PATH)
    lib.mla_decode_paged_kernel_name.restype = ctypes.c_char_p
    assert lib.mla_decode_paged_kernel_name(0, 16, None) is None  # fp32 has no paged form
    # same workspace as the contiguous call of the same schedule
    assert mla.mla_decode_paged_workspace_bytes(64, 128, 4096, 64, 64) == \
        mla.mla_decode_workspace_bytes(torch.bfloat16, 64, 128, 4096)
    assert mla.mla_decode_paged_workspace_bytes(64, 128, 4096, 48, 64) == 0
    assert mla.mla_decode_paged_workspace_bytes(64, 128, 4096, 64, 64, {"heads_per_group": 16}) == 0


def test_fp8_validation_and_queries(mla):
    lib = ctypes.CDLL(mla.LIB_PATH)
    vp = ctypes.c_void_p
    lib.mla_quantize_cache_fp8.argtypes = [ctypes.c_longlong, vp, vp, vp, vp]
    assert lib.mla_quantize_cache_fp8(0, vp(A), vp(A), vp(A), vp(0)) == 1
    assert lib.mla_quantize_cache_fp8(-5, vp(A), vp(A), vp(A), vp(0)) == 1
    assert lib.mla_quantize_cache_fp8(10, vp(0), vp(A), vp(A), vp(0)) == 1
    assert lib.mla_quantize_cache_fp8(10, vp(A + 8), vp(A), vp(A), vp(0)) == 1
    assert lib.mla_quantize_cache_fp8(10, vp(A), vp(A), vp(A + 2), vp(0)) == 1
    assert lib.mla_quantize_cache_fp8(1 << 40, vp(A), vp(A), vp(A), vp(0)) == 1

    def dec(b=2, h=16, t=100, q=A, c=A, s=A, sl=A, scale=SCALE, out=A, lse=A, ws=A, wsb=1 << 30):
        return lib.mla_decode_fp8(b, h, t, vp(q), vp(c), vp(s), vp(sl), ctypes.c_float(scale),
                                  vp(out), vp(lse), vp(ws), ctypes.c_size_t(wsb), vp(0))
    for kw, st in (({"q": 0}, 1), ({"c": 0}, 1), ({"s": 0}, 1), ({"s": A + 2}, 1), ({"c": A + 4}, 1),
                   ({"b": 0}, 1), ({"t": -1}, 1), ({"scale": -1.0}, 1), ({"wsb": 100}, 3),
                   ({"ws": A + 128}, 1), ({"b": 1 << 20, "t": 1 << 12}, 1)):
        assert dec(**kw) == st, kw
    # two kernels read e4m3 codes: the 16-head one (up to 64 heads by default)
    # and the 128-head FP8-MFMA one (more heads)
    assert mla.mla_decode_fp8_kernel_name(16) == "decode_bf16_kernel<16, 1, 2, 32, 2, true>"
    assert mla.mla_decode_fp8_kernel_name(64) == "decode_bf16_kernel<16, 1, 2, 32, 2, true>"
    assert mla.mla_decode_fp8_kernel_name(65) == "decode_wide_fp8_kernel"
    assert mla.mla_decode_fp8_kernel_name(128) == "decode_wide_fp8_kernel"
    assert mla.mla_decode_fp8_kernel_name(128, {"heads_per_group": 128}) == "decode_wide_fp8_kernel"
    assert mla.mla_decode_fp8_kernel_name(128, {"heads_per_group": 16}) == \
        "decode_bf16_kernel<16, 1, 2, 32, 2, true>"
    assert mla.mla_decode_fp8_kernel_name(128, {"heads_per_group": 128, "variant": 3}) is None
    assert mla.mla_decode_fp8_kernel_name(16, {"heads_per_group": 16, "variant": 2}) is None
    assert mla.mla_decode_fp8_kernel_name(64, {"heads_per_group": 64}) is None
    # the 128-head kernel: one workgroup per CU, the bf16 schedule's chunks
    assert mla.mla_decode_fp8_workspace_bytes(64, 128, 4096) == \
        mla.mla_decode_workspace_bytes(torch.bfloat16, 64, 128, 4096)
    # two resident workgroups per CU: twice the chunks of the bf16 schedule
    assert mla.mla_decode_fp8_workspace_bytes(128, 16, 8192) == \
        mla.mla_decode_workspace_bytes(torch.bfloat16, 128, 16, 8192, {"n_chunks": 512})


def _decode_mtp(lib, dt=1, b=2, ql=2, h=16, t=100, q=A, c=A, sl=A, scale=SCALE, out=A, lse=A, ws=A,
                wsb=1 << 30):
    vp = ctypes.c_void_p
    return lib.mla_decode_mtp(dt, b, ql, h, t, vp(q), vp(c), vp(sl), ctypes.c_float(scale), vp(out),
                              vp(lse), vp(ws), ctypes.c_size_t(wsb), vp(0))


@pytest.mark.parametrize("kw,status", [
    ({"dt": 0}, 2), ({"dt": 5}, 1), ({"ql": 0}, 1), ({"ql": -3}, 1), ({"ql": 1 << 20}, 1),
    ({"b": 0}, 1), ({"h": 0}, 1), ({"t": -1}, 1), ({"q": 0}, 1), ({"c": 0}, 1), ({"sl": 0}, 1),
    ({"out": 0}, 1), ({"lse": 0}, 1), ({"ws": 0}, 1), ({"q": A + 8}, 1), ({"lse": A + 4}, 1),
    ({"ws": A + 16}, 1), ({"scale": 0.0}, 1), ({"scale": float("nan")}, 1), ({"wsb": 1024}, 3),
    ({"b": 1 << 20, "t": 1 << 12}, 1),
    # one query token: the same validation as mla_decode
    ({"ql": 1, "q": 0}, 1), ({"ql": 1, "scale": -1.0}, 1), ({"ql": 1, "wsb": 1024}, 3),
])
def test_decode_mtp_validation(mla, kw, status):
    lib = ctypes.CDLL(mla.LIB_PATH)
    assert _decode_mtp(lib, **kw) == status


def test_decode_mtp_host_queries(mla):
    # query rows = q_len * h; 32 per wave, up to 4 waves per workgroup
    assert mla.mla_decode_mtp_kernel_name(2, 128) == "decode_wide_causal_kernel<4, 2, false>"
    assert mla.mla_decode_mtp_kernel_name(3, 16) == "decode_wide_causal_kernel<2, 2, false>"
    assert mla.mla_decode_mtp_kernel_name(2, 16) == "decode_wide_causal_kernel<1, 3, false>"
    assert mla.mla_decode_mtp_kernel_name(1, 128) == mla.mla_decode_kernel_name(torch.bfloat16, 128)
    assert mla.mla_decode_mtp_kernel_name(0, 128) is None
    assert mla.mla_decode_mtp_kernel_name(1 << 14, 128) is None
    # one token: exactly mla_decode's workspace; more: that of q_len*h heads
    assert mla.mla_decode_mtp_workspace_bytes(64, 1, 128, 4096) == \
        mla.mla_decode_workspace_bytes(torch.bfloat16, 64, 128, 4096)
    assert mla.mla_decode_mtp_workspace_bytes(64, 2, 128, 4096) == \
        mla.mla_decode_workspace_bytes(torch.bfloat16, 64, 256, 4096,
                                       {"heads_per_group": 128, "n_chunks": 128})
    assert mla.mla_decode_mtp_workspace_bytes(64, 0, 128, 4096) == 0
    lib = ctypes.CDLL(mla.LIB_PATH)
    lib.mla_decode_mtp_workspace_bytes.restype = ctypes.c_size_t
    assert lib.mla_decode_mtp_workspace_bytes(0, 4, 2, 16, 100) == 0  # fp32 has no causal form


def test_decode_mtp_ex_config(mla):
    lib = ctypes.CDLL(mla.LIB_PATH)
    vp = ctypes.c_void_p
    lib.mla_decode_mtp_workspace_bytes_ex.restype = ctypes.c_size_t
    for cfg in ({"n_chunks": 12}, {"n_chunks": -8}, {"heads_per_group": 128}, {"variant": 1},
                {"reserved": (ctypes.c_int * 5)(0, 0, 1, 0, 0)}):
        c = mla.MLAConfig()
        for k, v in cfg.items():
            setattr(c, k, v)
        for ql in (1, 2):
            st = lib.mla_decode_mtp_ex(1, 2, ql, 16, 100, vp(A), vp(A), vp(A), ctypes.c_float(SCALE),
                                       vp(A), vp(A), vp(A), ctypes.c_size_t(1 << 30), ctypes.byref(c),
                                       vp(0))
            assert st == 2, (cfg, ql)
            assert lib.mla_decode_mtp_workspace_bytes_ex(1, 2, ql, 16, 100, ctypes.byref(c)) == 0
    # a split count of its own changes the workspace like mla_decode_ex's does
    assert mla.mla_decode_mtp_workspace_bytes(64, 2, 128, 4096, {"n_chunks": 256}) == \
        mla.mla_decode_workspace_bytes(torch.bfloat16, 64, 256, 4096,
                                       {"heads_per_group": 128, "n_chunks": 256})


def _append(lib, dt=1, b=4, dm=512, t=64, x=A, wd=A, wr=A, cs=A, sn=A, npos=64, c=A, sl=A, so=0,
            ws=A, wsb=1 << 30):
    vp = ctypes.c_void_p
    return lib.mla_cache_append(dt, b, dm, t, vp(x), vp(wd), vp(wr), vp(cs), vp(sn), npos, vp(c), vp(sl),
                                vp(so), vp(ws), ctypes.c_size_t(wsb), vp(0))


@pytest.mark.parametrize("kw,status", [
    ({"dt": 0}, 2), ({"dt": 4}, 1), ({"b": 0}, 1), ({"dm": 0}, 1), ({"dm": 100}, 1), ({"dm": 384}, 1),
    ({"t": 0}, 1), ({"npos": 0}, 1), ({"x": 0}, 1), ({"wd": 0}, 1), ({"wr": 0}, 1), ({"cs": 0}, 1),
    ({"sn": 0}, 1), ({"c": 0}, 1), ({"sl": 0}, 1), ({"ws": 0}, 1), ({"x": A + 8}, 1), ({"wr": A + 4}, 1),
    ({"c": A + 2}, 1), ({"cs": A + 2}, 1), ({"sl": A + 2}, 1), ({"so": A + 1}, 1), ({"ws": A + 16}, 1),
    ({"wsb": 1024}, 3), ({"b": 1 << 20, "t": 1 << 12}, 1),
])
def test_cache_append_validation(mla, kw, status):
    lib = ctypes.CDLL(mla.LIB_PATH)
    assert _append(lib, **kw) == status


def test_cache_append_workspace(mla):
    # fp32 partial sums (one 576-wide row per batch row and 256-wide hidden
    # chunk) and a copy of the b positions, each rounded up to 256 bytes
    up = lambda n: -(-n // 256) * 256
    assert mla.mla_cache_append_workspace_bytes(64, 7168) == 64 * 28 * 576 * 4 + 256
    assert mla.mla_cache_append_workspace_bytes(3, 256) == 3 * 576 * 4 + 256
    assert mla.mla_cache_append_workspace_bytes(5, 256) == up(5 * 576 * 4) + 256
    assert mla.mla_cache_append_workspace_bytes(100, 512) == up(100 * 2 * 576 * 4) + up(400)
    assert mla.mla_cache_append_workspace_bytes(64, 7000) == 0
    assert mla.mla_cache_append_workspace_bytes(0, 7168) == 0


def _append_paged(lib, dt=1, b=4, dm=512, x=A, wd=A, wr=A, cs=A, sn=A, npos=64, pool=A, nb=8, bs=64,
                  bt=A, mb=4, sl=A, so=0, ws=A, wsb=1 << 30):
    vp = ctypes.c_void_p
    return lib.mla_cache_append_paged(dt, b, dm, vp(x), vp(wd), vp(wr), vp(cs), vp(sn), npos, vp(pool), nb,
                                      bs, vp(bt), mb, vp(sl), vp(so), vp(ws), ctypes.c_size_t(wsb), vp(0))


@pytest.mark.parametrize("kw,status", [
    ({"dt": 0}, 2), ({"dt": 3}, 1), ({"b": 0}, 1), ({"dm": 300}, 1), ({"npos": 0}, 1), ({"nb": 0}, 1),
    ({"bs": 48}, 1), ({"bs": 0}, 1), ({"mb": 0}, 1), ({"pool": 0}, 1), ({"bt": 0}, 1), ({"sl": 0}, 1),
    ({"x": 0}, 1), ({"pool": A + 8}, 1), ({"bt": A + 2}, 1), ({"so": A + 2}, 1), ({"ws": A + 64}, 1),
    ({"wsb": 100}, 3),
])
def test_cache_append_paged_validation(mla, kw, status):
    lib = ctypes.CDLL(mla.LIB_PATH)
    assert _append_paged(lib, **kw) == status


def _mtp_paged(lib, dt=1, b=2, ql=2, h=16, q=A, pool=A, nb=8, bs=64, bt=A, mb=4, sl=A, scale=SCALE,
               out=A, lse=A, ws=A, wsb=1 << 30):
    vp = ctypes.c_void_p
    return lib.mla_decode_mtp_paged(dt, b, ql, h, vp(q), vp(pool), nb, bs, vp(bt), mb, vp(sl),
                                    ctypes.c_float(scale), vp(out), vp(lse), vp(ws), ctypes.c_size_t(wsb),
                                    vp(0))


@pytest.mark.parametrize("kw,status", [
    ({"dt": 0}, 2), ({"dt": 7}, 1), ({"ql": 0}, 1), ({"h": 0}, 1), ({"bs": 40}, 1), ({"nb": 0}, 1),
    ({"mb": 0}, 1), ({"q": 0}, 1), ({"pool": 0}, 1), ({"bt": 0}, 1), ({"sl": 0}, 1), ({"out": 0}, 1),
    ({"lse": 0}, 1), ({"ws": 0}, 1), ({"q": A + 8}, 1), ({"ws": A + 16}, 1), ({"scale": 0.0}, 1),
    ({"wsb": 1024}, 3),
    # one query token: the same validation as mla_decode_paged
    ({"ql": 1, "bs": 40}, 1), ({"ql": 1, "pool": 0}, 1), ({"ql": 1, "wsb": 1024}, 3),
])
def test_decode_mtp_paged_validation(mla, kw, status):
    lib = ctypes.CDLL(mla.LIB_PATH)
    assert _mtp_paged(lib, **kw) == status


def test_decode_mtp_paged_workspace(mla):
    lib = ctypes.CDLL(mla.LIB_PATH)
    lib.mla_decode_mtp_paged_workspace_bytes.restype = ctypes.c_size_t
    # the same workspace as the contiguous multi-token call of the same rows
    assert lib.mla_decode_mtp_paged_workspace_bytes(1, 64, 2, 128, 4096, 64, 64) == \
        mla.mla_decode_mtp_workspace_bytes(64, 2, 128, 4096)
    assert lib.mla_decode_mtp_paged_workspace_bytes(1, 64, 1, 128, 4096, 64, 64) == \
        mla.mla_decode_paged_workspace_bytes(64, 128, 4096, 64, 64)
    assert lib.mla_decode_mtp_paged_workspace_bytes(1, 64, 2, 128, 4096, 48, 64) == 0
    assert lib.mla_decode_mtp_paged_workspace_bytes(0, 64, 2, 128, 4096, 64, 64) == 0
