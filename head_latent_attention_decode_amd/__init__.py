"""libmla355: absorbed Multi-head Latent Attention (MLA) decode on one AMD MI355X.

Thin ctypes binding over the C ABI in ``include/mla355.h``.  Every function
takes torch tensors (device memory and streams are torch's), checks dtype,
device, shape and contiguity, and passes raw pointers plus the current HIP
stream to the library.  No arithmetic happens here: every step of the path
runs in the library's HIP kernels.

The shared object ``libmla355.so`` is built in-tree by ``build.py``; importing
this package without it raises immediately (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla355.so")

D_C, D_R, D_QK, D_K, D_V = 512, 64, 576, 128, 128

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_HIP = 4
MLA_DTYPE_F32 = 0
MLA_DTYPE_BF16 = 1
# mla_decode_config_t.reserved[0] bit: record engine-clock stamps in the last
# CLOCK_BYTES of the workspace (include/mla355.h)
CONFIG_RECORD_CLOCK = 1
CLOCK_BYTES = 256

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libmla355.so is not built (expected at %s); run "
        "`python -m head_latent_attention_decode_amd.build` first" % LIB_PATH)


class MLAConfig(ctypes.Structure):
    """Mirror of mla_decode_config_t (scheduling overrides; zero = automatic)."""
    _fields_ = [("n_chunks", ctypes.c_int), ("heads_per_group", ctypes.c_int),
                ("variant", ctypes.c_int), ("reserved", ctypes.c_int * 5),
                ("profile_events", ctypes.c_void_p * 2)]


_lib = ctypes.CDLL(LIB_PATH)
_vp, _ci, _cf, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_lib.mla_abi_version.restype = _ci
_lib.mla_status_string.restype = ctypes.c_char_p
_lib.mla_status_string.argtypes = [_ci]
_lib.mla_absorb_q.restype = _ci
_lib.mla_absorb_q.argtypes = [_ci, _ci, _ci, _vp, _vp, _vp, _vp, _vp]
_lib.mla_absorb_o.restype = _ci
_lib.mla_absorb_o.argtypes = [_ci, _ci, _ci, _vp, _vp, _vp, _vp]
_lib.mla_decode_workspace_bytes.restype = _sz
_lib.mla_decode_workspace_bytes.argtypes = [_ci, _ci, _ci, _ci]
_lib.mla_decode_workspace_bytes_ex.restype = _sz
_lib.mla_decode_workspace_bytes_ex.argtypes = [_ci, _ci, _ci, _ci, ctypes.POINTER(MLAConfig)]
_lib.mla_decode.restype = _ci
_lib.mla_decode.argtypes = [_ci, _ci, _ci, _ci, _vp, _vp, _vp, _cf, _vp, _vp, _vp, _sz, _vp]
_lib.mla_decode_kernel_name.restype = ctypes.c_char_p
_lib.mla_decode_kernel_name.argtypes = [_ci, _ci, ctypes.POINTER(MLAConfig)]
_lib.mla_decode_noalloc.restype = _ci
_lib.mla_decode_noalloc.argtypes = [_ci, _ci, _ci, _ci, _vp, _vp, _vp, _cf, _vp, _vp, _vp]
_lib.mla_decode_ex.restype = _ci
_lib.mla_decode_ex.argtypes = [_ci, _ci, _ci, _ci, _vp, _vp, _vp, _cf, _vp, _vp, _vp, _sz,
                               ctypes.POINTER(MLAConfig), _vp]
_lib.mla_decode_paged_workspace_bytes.restype = _sz
_lib.mla_decode_paged_workspace_bytes.argtypes = [_ci, _ci, _ci, _ci, _ci, _ci,
                                                  ctypes.POINTER(MLAConfig)]
_lib.mla_decode_paged_kernel_name.restype = ctypes.c_char_p
_lib.mla_decode_paged_kernel_name.argtypes = [_ci, _ci, ctypes.POINTER(MLAConfig)]
_lib.mla_decode_paged.restype = _ci
_lib.mla_decode_paged.argtypes = [_ci, _ci, _ci, _vp, _vp, _ci, _ci, _vp, _ci, _vp, _cf, _vp, _vp,
                                  _vp, _sz, _vp]
_lib.mla_quantize_cache_fp8.restype = _ci
_lib.mla_quantize_cache_fp8.argtypes = [ctypes.c_longlong, _vp, _vp, _vp, _vp]
_lib.mla_decode_fp8_workspace_bytes.restype = _sz
_lib.mla_decode_fp8_workspace_bytes.argtypes = [_ci, _ci, _ci, ctypes.POINTER(MLAConfig)]
_lib.mla_decode_fp8_kernel_name.restype = ctypes.c_char_p
_lib.mla_decode_fp8_kernel_name.argtypes = [_ci, ctypes.POINTER(MLAConfig)]
_lib.mla_decode_fp8.restype = _ci
_lib.mla_decode_fp8.argtypes = [_ci, _ci, _ci, _vp, _vp, _vp, _vp, _cf, _vp, _vp, _vp, _sz, _vp]
_lib.mla_decode_fp8_ex.restype = _ci
_lib.mla_decode_fp8_ex.argtypes = [_ci, _ci, _ci, _vp, _vp, _vp, _vp, _cf, _vp, _vp, _vp, _sz,
                                   ctypes.POINTER(MLAConfig), _vp]
_lib.mla_decode_paged_ex.restype = _ci
_lib.mla_decode_paged_ex.argtypes = [_ci, _ci, _ci, _vp, _vp, _ci, _ci, _vp, _ci, _vp, _cf, _vp,
                                     _vp, _vp, _sz, ctypes.POINTER(MLAConfig), _vp]
_lib.mla_decode_mtp_workspace_bytes.restype = _sz
_lib.mla_decode_mtp_workspace_bytes.argtypes = [_ci, _ci, _ci, _ci, _ci]
_lib.mla_decode_mtp_kernel_name.restype = ctypes.c_char_p
_lib.mla_decode_mtp_kernel_name.argtypes = [_ci, _ci, _ci]
_lib.mla_decode_mtp.restype = _ci
_lib.mla_decode_mtp.argtypes = [_ci, _ci, _ci, _ci, _ci, _vp, _vp, _vp, _cf, _vp, _vp, _vp, _sz, _vp]
_lib.mla_decode_mtp_workspace_bytes_ex.restype = _sz
_lib.mla_decode_mtp_workspace_bytes_ex.argtypes = [_ci, _ci, _ci, _ci, _ci, ctypes.POINTER(MLAConfig)]
_lib.mla_decode_mtp_ex.restype = _ci
_lib.mla_decode_mtp_ex.argtypes = [_ci, _ci, _ci, _ci, _ci, _vp, _vp, _vp, _cf, _vp, _vp, _vp, _sz,
                                   ctypes.POINTER(MLAConfig), _vp]
_lib.mla_cache_append_workspace_bytes.restype = _sz
_lib.mla_cache_append_workspace_bytes.argtypes = [_ci, _ci]
_lib.mla_cache_append.restype = _ci
_lib.mla_cache_append.argtypes = [_ci, _ci, _ci, _ci, _vp, _vp, _vp, _vp, _vp, _ci, _vp, _vp, _vp, _vp,
                                  _sz, _vp]
_lib.mla_cache_append_paged.restype = _ci
_lib.mla_cache_append_paged.argtypes = [_ci, _ci, _ci, _vp, _vp, _vp, _vp, _vp, _ci, _vp, _ci, _ci, _vp, _ci,
                                        _vp, _vp, _vp, _sz, _vp]
_lib.mla_decode_mtp_paged_workspace_bytes.restype = _sz
_lib.mla_decode_mtp_paged_workspace_bytes.argtypes = [_ci, _ci, _ci, _ci, _ci, _ci, _ci]
_lib.mla_decode_mtp_paged.restype = _ci
_lib.mla_decode_mtp_paged.argtypes = [_ci, _ci, _ci, _ci, _vp, _vp, _ci, _ci, _vp, _ci, _vp, _cf, _vp, _vp,
                                      _vp, _sz, _vp]

EXPORTED_SYMBOLS = ("mla_abi_version", "mla_status_string", "mla_absorb_q", "mla_absorb_o",
                    "mla_decode_workspace_bytes", "mla_decode_workspace_bytes_ex", "mla_decode",
                    "mla_decode_ex", "mla_decode_kernel_name", "mla_decode_paged_workspace_bytes",
                    "mla_decode_paged", "mla_decode_paged_ex", "mla_decode_paged_kernel_name",
                    "mla_quantize_cache_fp8", "mla_decode_fp8_workspace_bytes", "mla_decode_fp8",
                    "mla_decode_fp8_ex", "mla_decode_fp8_kernel_name",
                    "mla_decode_mtp_workspace_bytes", "mla_decode_mtp", "mla_decode_mtp_kernel_name",
                    "mla_decode_mtp_workspace_bytes_ex", "mla_decode_mtp_ex",
                    "mla_cache_append_workspace_bytes", "mla_cache_append", "mla_cache_append_paged",
                    "mla_decode_mtp_paged_workspace_bytes", "mla_decode_mtp_paged", "mla_decode_noalloc")

# Size of the library's own device array used by mla_decode_noalloc.
NOALLOC_SCRATCH_BYTES = 64 << 20


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" %
                         (where, _lib.mla_status_string(status).decode(), status))


def _check(status: int, where: str):
    if status != MLA_OK:
        raise MLAError(status, where)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return MLA_DTYPE_BF16
    if dt == torch.float32:
        return MLA_DTYPE_F32
    raise TypeError("libmla355 supports bfloat16 and float32, got %s" % dt)


def _dev(t: torch.Tensor, name: str, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def abi_version() -> int:
    return _lib.mla_abi_version()


def status_string(status: int) -> str:
    return _lib.mla_status_string(status).decode()


def _cfg(config):
    if config is None:
        return None
    if isinstance(config, MLAConfig):
        return ctypes.pointer(config)
    c = MLAConfig()
    for k, v in dict(config).items():
        if k == "profile_events":
            c.profile_events[0] = v[0]
            c.profile_events[1] = v[1]
        elif k == "record_clock":
            c.reserved[0] = CONFIG_RECORD_CLOCK if v else 0
        else:
            setattr(c, k, int(v))
    return ctypes.pointer(c)


def read_clock_mhz(workspace, workspace_bytes=None):
    """Engine clock (MHz) of the last attention launch made with the config key
    record_clock: the library's workspace ends with four uint64 stamps (shader
    clock and 100 MHz real-time counter at the start and the end of the
    kernel's first workgroup).  workspace_bytes: the size the library reported
    for the call (default: the whole tensor).  None if nothing was recorded."""
    n = workspace.numel() if workspace_bytes is None else int(workspace_bytes)
    st = workspace[n - CLOCK_BYTES:n - CLOCK_BYTES + 32].view(torch.int64).cpu().tolist()
    c0, r0, c1, r1 = st
    if r1 <= r0 or c1 <= c0 or r0 == 0:
        return None
    return 100.0 * (c1 - c0) / (r1 - r0)


def mla_decode_kernel_name(dtype: torch.dtype, h: int, config=None):
    """Name of the attention kernel mla_decode would launch (pure host, no GPU); None if rejected."""
    name = _lib.mla_decode_kernel_name(_dtype_code(dtype), h, _cfg(config))
    return None if name is None else name.decode()


def mla_decode_workspace_bytes(dtype: torch.dtype, b: int, h: int, t_max: int, config=None) -> int:
    """Bytes of workspace mla_decode needs (pure host computation, no GPU)."""
    if config is None:
        return int(_lib.mla_decode_workspace_bytes(_dtype_code(dtype), b, h, t_max))
    return int(_lib.mla_decode_workspace_bytes_ex(_dtype_code(dtype), b, h, t_max, _cfg(config)))


def mla_absorb_q(q_nope, w_uk, q_rope, q_prime=None, stream=None):
    """q'[b,h,:512] = q_nope[b,h,:] @ W_UK[h];  q'[b,h,512:] = q_rope[b,h,:]."""
    b, h, _ = q_nope.shape
    dt = q_nope.dtype
    if q_prime is None:
        q_prime = torch.empty((b, h, D_QK), dtype=dt, device=q_nope.device)
    args = (_dev(q_nope, "q_nope", (b, h, D_K), dt), _dev(w_uk, "w_uk", (h, D_K, D_C), dt),
            _dev(q_rope, "q_rope", (b, h, D_R), dt), _dev(q_prime, "q_prime", (b, h, D_QK), dt))
    _check(_lib.mla_absorb_q(_dtype_code(dt), b, h, *args, _stream(stream)), "mla_absorb_q")
    return q_prime


def mla_absorb_o(o, w_uv, y=None, stream=None):
    """y[b,h,:] = o[b,h,:] @ W_UV[h]."""
    b, h, _ = o.shape
    dt = o.dtype
    if y is None:
        y = torch.empty((b, h, D_V), dtype=dt, device=o.device)
    args = (_dev(o, "o", (b, h, D_C), dt), _dev(w_uv, "w_uv", (h, D_C, D_V), dt),
            _dev(y, "y", (b, h, D_V), dt))
    _check(_lib.mla_absorb_o(_dtype_code(dt), b, h, *args, _stream(stream)), "mla_absorb_o")
    return y


def mla_decode(q_prime, cache, seqlens, softmax_scale, out=None, lse=None, workspace=None,
               config=None, stream=None):
    """Latent-form MLA decode.  Returns (out [b,h,512], lse [b,h] fp32).

    q_prime [b,h,576], cache [b,t_max,576] (same dtype), seqlens [b] int32 on the GPU.
    workspace: optional uint8 GPU tensor of at least mla_decode_workspace_bytes bytes.
    config: optional scheduling overrides (dict or MLAConfig).
    """
    b, h, _ = q_prime.shape
    t_max = cache.shape[1]
    dt = q_prime.dtype
    dev = q_prime.device
    _dev(q_prime, "q_prime", (b, h, D_QK), dt)
    _dev(cache, "cache", (b, t_max, D_QK), dt)
    if out is None:
        out = torch.empty((b, h, D_C), dtype=dt, device=dev)
    if lse is None:
        lse = torch.empty((b, h), dtype=torch.float32, device=dev)
    need = mla_decode_workspace_bytes(dt, b, h, t_max, config)
    if need == 0:
        raise ValueError("invalid decode problem or config: b=%d h=%d t_max=%d" % (b, h, t_max))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device.type != "cuda":
        raise TypeError("workspace must be a uint8 GPU tensor")
    args = (_dev(q_prime, "q_prime", (b, h, D_QK), dt), _dev(cache, "cache", (b, t_max, D_QK), dt),
            _dev(seqlens, "seqlens", (b,), torch.int32), ctypes.c_float(float(softmax_scale)),
            _dev(out, "out", (b, h, D_C), dt), _dev(lse, "lse", (b, h), torch.float32),
            ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()))
    if config is None:
        st = _lib.mla_decode(_dtype_code(dt), b, h, t_max, *args, _stream(stream))
    else:
        st = _lib.mla_decode_ex(_dtype_code(dt), b, h, t_max, *args, _cfg(config), _stream(stream))
    _check(st, "mla_decode")
    return out, lse


def mla_decode_noalloc(q_prime, cache, seqlens, softmax_scale, out, lse, stream=None):
    """mla_decode with the library's own fixed device array as its workspace
    (the C call allocates nothing).  out [b,h,512] and lse [b,h] fp32 are
    the caller's; returns (out, lse).  Calls on one GPU share that array."""
    b, h, _ = q_prime.shape
    t_max = cache.shape[1]
    dt = q_prime.dtype
    args = (_dev(q_prime, "q_prime", (b, h, D_QK), dt), _dev(cache, "cache", (b, t_max, D_QK), dt),
            _dev(seqlens, "seqlens", (b,), torch.int32), ctypes.c_float(float(softmax_scale)),
            _dev(out, "out", (b, h, D_C), dt), _dev(lse, "lse", (b, h), torch.float32))
    _check(_lib.mla_decode_noalloc(_dtype_code(dt), b, h, t_max, *args, _stream(stream)), "mla_decode_noalloc")
    return out, lse


def mla_decode_mtp_kernel_name(q_len: int, h: int):
    """Name of the attention kernel mla_decode_mtp would launch (pure host); None if rejected."""
    name = _lib.mla_decode_mtp_kernel_name(MLA_DTYPE_BF16, q_len, h)
    return None if name is None else name.decode()


def mla_decode_mtp_workspace_bytes(b: int, q_len: int, h: int, t_max: int, config=None) -> int:
    """Bytes of workspace mla_decode_mtp needs (pure host computation, no GPU)."""
    return int(_lib.mla_decode_mtp_workspace_bytes_ex(MLA_DTYPE_BF16, b, q_len, h, t_max, _cfg(config)))


def mla_decode_mtp(q_prime, cache, seqlens, softmax_scale, out=None, lse=None, workspace=None,
                   config=None, stream=None):
    """Latent-form decode of q_len causal query tokens per row (bf16).

    q_prime [b,q_len,h,576], cache [b,t_max,576], seqlens [b] int32 on the GPU
    (cached rows, the q_len new ones included).  Returns (out [b,q_len,h,512],
    lse [b,q_len,h] fp32).
    """
    b, q_len, h, _ = q_prime.shape
    t_max = cache.shape[1]
    dt = q_prime.dtype
    dev = q_prime.device
    if dt != torch.bfloat16:
        raise TypeError("mla_decode_mtp takes bf16 tensors")
    if out is None:
        out = torch.empty((b, q_len, h, D_C), dtype=dt, device=dev)
    if lse is None:
        lse = torch.empty((b, q_len, h), dtype=torch.float32, device=dev)
    need = mla_decode_mtp_workspace_bytes(b, q_len, h, t_max, config)
    if need == 0:
        raise ValueError("invalid problem or config: b=%d q_len=%d h=%d t_max=%d" % (b, q_len, h, t_max))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device.type != "cuda":
        raise TypeError("workspace must be a uint8 GPU tensor")
    st = _lib.mla_decode_mtp_ex(MLA_DTYPE_BF16, b, q_len, h, t_max,
                             _dev(q_prime, "q_prime", (b, q_len, h, D_QK), dt),
                             _dev(cache, "cache", (b, t_max, D_QK), dt),
                             _dev(seqlens, "seqlens", (b,), torch.int32),
                             ctypes.c_float(float(softmax_scale)),
                             _dev(out, "out", (b, q_len, h, D_C), dt),
                             _dev(lse, "lse", (b, q_len, h), torch.float32),
                             ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()),
                             _cfg(config), _stream(stream))
    _check(st, "mla_decode_mtp")
    return out, lse


def mla_cache_append_workspace_bytes(b: int, d_model: int) -> int:
    """Bytes of workspace mla_cache_append needs (pure host computation, no GPU)."""
    return int(_lib.mla_cache_append_workspace_bytes(b, d_model))


def mla_cache_append(x, w_dkv, w_kr, rope_cos, rope_sin, cache, seqlens, seqlens_out=None,
                     workspace=None, stream=None):
    """Write [x W_DKV ; RoPE(x W_KR)] (bf16) into row seqlens[i] of each batch row.

    x [b,d_model], w_dkv [d_model,512], w_kr [d_model,64] bf16; rope_cos /
    rope_sin [n_pos,32] fp32; cache [b,t_max,576] bf16 (updated in place);
    seqlens [b] int32; seqlens_out: optional int32 [b] (may be seqlens itself)
    that receives the lengths including the new token.  Returns cache.
    """
    b, d_model = x.shape
    t_max = cache.shape[1]
    n_pos = rope_cos.shape[0]
    dev = x.device
    need = mla_cache_append_workspace_bytes(b, d_model)
    if need == 0:
        raise ValueError("invalid append problem: b=%d d_model=%d" % (b, d_model))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device.type != "cuda":
        raise TypeError("workspace must be a uint8 GPU tensor")
    so = None if seqlens_out is None else _dev(seqlens_out, "seqlens_out", (b,), torch.int32)
    st = _lib.mla_cache_append(MLA_DTYPE_BF16, b, d_model, t_max,
                               _dev(x, "x", (b, d_model), torch.bfloat16),
                               _dev(w_dkv, "w_dkv", (d_model, D_C), torch.bfloat16),
                               _dev(w_kr, "w_kr", (d_model, D_R), torch.bfloat16),
                               _dev(rope_cos, "rope_cos", (n_pos, D_R // 2), torch.float32),
                               _dev(rope_sin, "rope_sin", (n_pos, D_R // 2), torch.float32), n_pos,
                               _dev(cache, "cache", (b, t_max, D_QK), torch.bfloat16),
                               _dev(seqlens, "seqlens", (b,), torch.int32), so,
                               ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()),
                               _stream(stream))
    _check(st, "mla_cache_append")
    return cache


def mla_cache_append_paged(x, w_dkv, w_kr, rope_cos, rope_sin, kv_pool, block_table, seqlens,
                           seqlens_out=None, workspace=None, stream=None):
    """mla_cache_append into a paged pool [num_blocks, block_size, 576] through
    block_table [b, max_blocks] int32.  Returns kv_pool."""
    b, d_model = x.shape
    nb, bs = kv_pool.shape[0], kv_pool.shape[1]
    mb = block_table.shape[1]
    n_pos = rope_cos.shape[0]
    dev = x.device
    need = mla_cache_append_workspace_bytes(b, d_model)
    if need == 0:
        raise ValueError("invalid append problem: b=%d d_model=%d" % (b, d_model))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    so = None if seqlens_out is None else _dev(seqlens_out, "seqlens_out", (b,), torch.int32)
    st = _lib.mla_cache_append_paged(MLA_DTYPE_BF16, b, d_model,
                                     _dev(x, "x", (b, d_model), torch.bfloat16),
                                     _dev(w_dkv, "w_dkv", (d_model, D_C), torch.bfloat16),
                                     _dev(w_kr, "w_kr", (d_model, D_R), torch.bfloat16),
                                     _dev(rope_cos, "rope_cos", (n_pos, D_R // 2), torch.float32),
                                     _dev(rope_sin, "rope_sin", (n_pos, D_R // 2), torch.float32), n_pos,
                                     _dev(kv_pool, "kv_pool", (nb, bs, D_QK), torch.bfloat16), nb, bs,
                                     _dev(block_table, "block_table", (b, mb), torch.int32), mb,
                                     _dev(seqlens, "seqlens", (b,), torch.int32), so,
                                     ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()),
                                     _stream(stream))
    _check(st, "mla_cache_append_paged")
    return kv_pool


def mla_decode_mtp_paged(q_prime, kv_pool, block_table, seqlens, softmax_scale, out=None, lse=None,
                         workspace=None, stream=None):
    """mla_decode_mtp over a paged pool.  q_prime [b,q_len,h,576] bf16, kv_pool
    [num_blocks,block_size,576], block_table [b,max_blocks] int32."""
    b, q_len, h, _ = q_prime.shape
    nb, bs = kv_pool.shape[0], kv_pool.shape[1]
    mb = block_table.shape[1]
    dt = q_prime.dtype
    dev = q_prime.device
    if dt != torch.bfloat16:
        raise TypeError("mla_decode_mtp_paged takes bf16 tensors")
    if out is None:
        out = torch.empty((b, q_len, h, D_C), dtype=dt, device=dev)
    if lse is None:
        lse = torch.empty((b, q_len, h), dtype=torch.float32, device=dev)
    need = int(_lib.mla_decode_mtp_paged_workspace_bytes(MLA_DTYPE_BF16, b, q_len, h, nb, bs, mb))
    if need == 0:
        raise ValueError("invalid paged problem: b=%d q_len=%d h=%d block_size=%d" % (b, q_len, h, bs))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = _lib.mla_decode_mtp_paged(MLA_DTYPE_BF16, b, q_len, h,
                                   _dev(q_prime, "q_prime", (b, q_len, h, D_QK), dt),
                                   _dev(kv_pool, "kv_pool", (nb, bs, D_QK), dt), nb, bs,
                                   _dev(block_table, "block_table", (b, mb), torch.int32), mb,
                                   _dev(seqlens, "seqlens", (b,), torch.int32),
                                   ctypes.c_float(float(softmax_scale)),
                                   _dev(out, "out", (b, q_len, h, D_C), dt),
                                   _dev(lse, "lse", (b, q_len, h), torch.float32),
                                   ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()),
                                   _stream(stream))
    _check(st, "mla_decode_mtp_paged")
    return out, lse


def mla_decode_paged_kernel_name(h: int, config=None):
    """Name of the attention kernel mla_decode_paged would launch (pure host); None if rejected."""
    name = _lib.mla_decode_paged_kernel_name(MLA_DTYPE_BF16, h, _cfg(config))
    return None if name is None else name.decode()


def mla_decode_paged_workspace_bytes(b: int, h: int, num_blocks: int, block_size: int,
                                     max_blocks: int, config=None) -> int:
    """Bytes of workspace mla_decode_paged needs (pure host computation, no GPU)."""
    return int(_lib.mla_decode_paged_workspace_bytes(MLA_DTYPE_BF16, b, h, num_blocks, block_size,
                                                     max_blocks, _cfg(config)))


def mla_decode_paged(q_prime, kv_pool, block_table, seqlens, softmax_scale, out=None, lse=None,
                     workspace=None, config=None, stream=None):
    """Latent-form MLA decode over a paged cache.  Returns (out [b,h,512], lse [b,h] fp32).

    q_prime [b,h,576] bf16; kv_pool [num_blocks, block_size, 576] bf16; block_table
    [b, max_blocks] int32 and seqlens [b] int32 on the GPU.  Token t of row i is row
    t % block_size of block block_table[i, t // block_size].
    """
    b, h, _ = q_prime.shape
    num_blocks, block_size, _ = kv_pool.shape
    max_blocks = block_table.shape[1]
    dev = q_prime.device
    dt = torch.bfloat16
    if out is None:
        out = torch.empty((b, h, D_C), dtype=dt, device=dev)
    if lse is None:
        lse = torch.empty((b, h), dtype=torch.float32, device=dev)
    need = mla_decode_paged_workspace_bytes(b, h, num_blocks, block_size, max_blocks, config)
    if need == 0:
        raise ValueError("invalid paged decode problem or config: b=%d h=%d blocks=%d x %d, "
                         "max_blocks=%d" % (b, h, num_blocks, block_size, max_blocks))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device.type != "cuda":
        raise TypeError("workspace must be a uint8 GPU tensor")
    args = (_dev(q_prime, "q_prime", (b, h, D_QK), dt),
            _dev(kv_pool, "kv_pool", (num_blocks, block_size, D_QK), dt),
            ctypes.c_int(num_blocks), ctypes.c_int(block_size),
            _dev(block_table, "block_table", (b, max_blocks), torch.int32), ctypes.c_int(max_blocks),
            _dev(seqlens, "seqlens", (b,), torch.int32), ctypes.c_float(float(softmax_scale)),
            _dev(out, "out", (b, h, D_C), dt), _dev(lse, "lse", (b, h), torch.float32),
            ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()))
    if config is None:
        st = _lib.mla_decode_paged(MLA_DTYPE_BF16, b, h, *args, _stream(stream))
    else:
        st = _lib.mla_decode_paged_ex(MLA_DTYPE_BF16, b, h, *args, _cfg(config), _stream(stream))
    _check(st, "mla_decode_paged")
    return out, lse


def mla_quantize_cache_fp8(cache, codes=None, scale=None, stream=None):
    """Per-token OCP e4m3 form of bf16 latent rows [..., 576] -> (codes uint8 [..., 576],
    scale fp32 [...]), with row ~ e4m3(codes) * scale."""
    if cache.dtype != torch.bfloat16 or cache.shape[-1] != D_QK:
        raise TypeError("cache must be bf16 [..., 576]")
    lead = tuple(cache.shape[:-1])
    n = 1
    for x in lead:
        n *= x
    if codes is None:
        codes = torch.empty(lead + (D_QK,), dtype=torch.uint8, device=cache.device)
    if scale is None:
        scale = torch.empty(lead, dtype=torch.float32, device=cache.device)
    args = (_dev(cache, "cache", lead + (D_QK,), torch.bfloat16),
            _dev(codes, "codes", lead + (D_QK,), torch.uint8), _dev(scale, "scale", lead, torch.float32))
    _check(_lib.mla_quantize_cache_fp8(n, *args, _stream(stream)), "mla_quantize_cache_fp8")
    return codes, scale


def mla_decode_fp8_kernel_name(h: int, config=None):
    """Name of the attention kernel mla_decode_fp8 would launch (pure host); None if rejected."""
    name = _lib.mla_decode_fp8_kernel_name(h, _cfg(config))
    return None if name is None else name.decode()


def mla_decode_fp8_workspace_bytes(b: int, h: int, t_max: int, config=None) -> int:
    return int(_lib.mla_decode_fp8_workspace_bytes(b, h, t_max, _cfg(config)))


def mla_decode_fp8(q_prime, cache_codes, cache_scale, seqlens, softmax_scale, out=None, lse=None,
                   workspace=None, config=None, stream=None):
    """Latent-form MLA decode over an fp8 cache.  Returns (out [b,h,512] bf16, lse [b,h] fp32).

    q_prime [b,h,576] bf16; cache_codes [b,t_max,576] uint8 (OCP e4m3); cache_scale
    [b,t_max] fp32; seqlens [b] int32 on the GPU.
    """
    b, h, _ = q_prime.shape
    t_max = cache_codes.shape[1]
    dev = q_prime.device
    if out is None:
        out = torch.empty((b, h, D_C), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((b, h), dtype=torch.float32, device=dev)
    need = mla_decode_fp8_workspace_bytes(b, h, t_max, config)
    if need == 0:
        raise ValueError("invalid fp8 decode problem or config: b=%d h=%d t_max=%d" % (b, h, t_max))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    args = (_dev(q_prime, "q_prime", (b, h, D_QK), torch.bfloat16),
            _dev(cache_codes, "cache_codes", (b, t_max, D_QK), torch.uint8),
            _dev(cache_scale, "cache_scale", (b, t_max), torch.float32),
            _dev(seqlens, "seqlens", (b,), torch.int32), ctypes.c_float(float(softmax_scale)),
            _dev(out, "out", (b, h, D_C), torch.bfloat16), _dev(lse, "lse", (b, h), torch.float32),
            ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()))
    if config is None:
        st = _lib.mla_decode_fp8(b, h, t_max, *args, _stream(stream))
    else:
        st = _lib.mla_decode_fp8_ex(b, h, t_max, *args, _cfg(config), _stream(stream))
    _check(st, "mla_decode_fp8")
    return out, lse


@dataclass
class StepBuffers:
    """Pre-allocated buffers for a full absorb -> decode -> absorb step."""
    q_prime: torch.Tensor
    out: torch.Tensor
    lse: torch.Tensor
    y: torch.Tensor
    workspace: torch.Tensor


def alloc_step(b, h, t_max, dtype=torch.bfloat16, device="cuda", config=None) -> StepBuffers:
    need = mla_decode_workspace_bytes(dtype, b, h, t_max, config)
    return StepBuffers(
        q_prime=torch.empty((b, h, D_QK), dtype=dtype, device=device),
        out=torch.empty((b, h, D_C), dtype=dtype, device=device),
        lse=torch.empty((b, h), dtype=torch.float32, device=device),
        y=torch.empty((b, h, D_V), dtype=dtype, device=device),
        workspace=torch.empty(need, dtype=torch.uint8, device=device))


def mla_step(q_nope, q_rope, w_uk, w_uv, cache, seqlens, softmax_scale, bufs: StepBuffers,
             config=None, stream=None):
    """mla_absorb_q -> mla_decode -> mla_absorb_o on one stream (no allocation)."""
    mla_absorb_q(q_nope, w_uk, q_rope, bufs.q_prime, stream=stream)
    mla_decode(bufs.q_prime, cache, seqlens, softmax_scale, bufs.out, bufs.lse, bufs.workspace,
               config=config, stream=stream)
    mla_absorb_o(bufs.out, w_uv, bufs.y, stream=stream)
    return bufs.y


def default_scale() -> float:
    return 1.0 / math.sqrt(D_K + D_R)
