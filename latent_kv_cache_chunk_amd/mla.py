"""ctypes binding of libmla_hip.so (declared in include/mla.h).

Argument marshalling only: shapes, dtypes, devices and contiguity are checked
here, then raw device pointers and the current HIP stream are handed to the C
ABI.  Every step of the path runs in the library's HIP kernels.  There is no
fallback: if the library is missing or fails to load, importing this module
raises ImportError.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_LIB_PATH = os.environ.get("MLA_HIP_LIB", os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_hip.so"))
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m latent_kv_cache_chunk_amd.build` "
                      "(there is no CPU or PyTorch fallback)")
_lib = ctypes.CDLL(_LIB_PATH)

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = 0, -1, -2, -3, -4
MLA_BF16, MLA_F32 = 0, 1

LIB_PATH = _LIB_PATH
EXPORTED = ("mla_cache_append", "mla_chunk_attend_workspace_bytes", "mla_chunk_attend",
            "mla_chunk_attend_causal", "mla_query_absorb", "mla_latent_attend", "mla_latent_attend_causal",
            "mla_value_upproj", "mla_status_string", "mla_last_error", "mla_version",
            "mla_ring_init", "mla_ring_current", "mla_ring_commit", "mla_ring_slot_chunks",
            "mla_cache_bytes", "mla_dense_kv_bytes", "mla_ring_last_error",
            "mla_mha_attend_workspace_bytes", "mla_mha_attend",
            "mla_chunk_attend_expanded_workspace_bytes", "mla_chunk_attend_expanded",
            "mla_chunk_attend_form", "mla_chunk_attend_auto_workspace_bytes", "mla_chunk_attend_auto",
            "mla_chunk_attend_noalloc")


class MlaDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("d_c", ctypes.c_int32), ("d_r", ctypes.c_int32), ("rope_t", ctypes.c_int32),
                ("rope_h", ctypes.c_int32), ("rope_w", ctypes.c_int32), ("rope_theta", ctypes.c_double)]


class MlaCausal(ctypes.Structure):
    _fields_ = [("q_start", ctypes.c_int32), ("chunk_len", ctypes.c_int32)]


class MlaRing(ctypes.Structure):
    _fields_ = [("chunk_tokens", ctypes.c_int32), ("sink_chunks", ctypes.c_int32),
                ("window_chunks", ctypes.c_int32), ("capacity", ctypes.c_int32), ("committed", ctypes.c_int64)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_DIMS = ctypes.POINTER(MlaDims)

_lib.mla_cache_append.argtypes = [_DIMS, _I32, _P, _I32, _I32, _P, _P, _P, _P, _I32, _I32, _P]
_lib.mla_cache_append.restype = _I32
_lib.mla_chunk_attend_workspace_bytes.argtypes = [_DIMS, _I32, _I32, _I32]
_lib.mla_chunk_attend_workspace_bytes.restype = _I64
_lib.mla_chunk_attend.argtypes = [_DIMS, _I32, _I32, _P, _P, _P, _I32, _P, _P, _P, _I32, _I32,
                                  ctypes.c_float, _P, _P, _I64, _P]
_lib.mla_chunk_attend.restype = _I32
_lib.mla_chunk_attend_causal.argtypes = [_DIMS, _I32, _I32, _P, _P, _P, _I32, _P, _P, _P, _I32, _I32,
                                         ctypes.POINTER(MlaCausal), ctypes.c_float, _P, _P, _I64, _P]
_lib.mla_chunk_attend_causal.restype = _I32
_lib.mla_query_absorb.argtypes = [_DIMS, _I32, _P, _P, _P, _I32, _P, ctypes.c_float, _I32, _P, _I64, _P]
_lib.mla_query_absorb.restype = _I32
_lib.mla_latent_attend.argtypes = [_DIMS, _I32, _P, _I32, _I32, _I32, _P, _I64, _P]
_lib.mla_latent_attend.restype = _I32
_lib.mla_latent_attend_causal.argtypes = [_DIMS, _I32, _P, _I32, _I32, _I32, ctypes.POINTER(MlaCausal), _P, _I64,
                                          _P]
_lib.mla_latent_attend_causal.restype = _I32
_lib.mla_value_upproj.argtypes = [_DIMS, _I32, _I32, _I32, _I32, _P, _P, _P, _I64, _P]
_lib.mla_value_upproj.restype = _I32
_RING = ctypes.POINTER(MlaRing)
_lib.mla_mha_attend_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32, _I32]
_lib.mla_mha_attend_workspace_bytes.restype = _I64
_lib.mla_mha_attend.argtypes = [_I32, _I32, _I32, _I32, _P, _I32, _P, _P, _I32, _I32, ctypes.c_float, _P, _P, _I64,
                                _P]
_lib.mla_mha_attend.restype = _I32
_lib.mla_chunk_attend_expanded_workspace_bytes.argtypes = [_DIMS, _I32, _I32]
_lib.mla_chunk_attend_expanded_workspace_bytes.restype = _I64
_lib.mla_chunk_attend_expanded.argtypes = [_DIMS, _I32, _P, _P, _P, _I32, _P, _P, _P, _I32, _I32, ctypes.c_float,
                                           _P, _P, _I64, _P]
_lib.mla_chunk_attend_expanded.restype = _I32

_lib.mla_chunk_attend_form.argtypes = [_DIMS, _I32, _I32, _I32]
_lib.mla_chunk_attend_form.restype = _I32
_lib.mla_chunk_attend_auto_workspace_bytes.argtypes = [_DIMS, _I32, _I32, _I32]
_lib.mla_chunk_attend_auto_workspace_bytes.restype = _I64
_lib.mla_chunk_attend_auto.argtypes = list(_lib.mla_chunk_attend.argtypes)
_lib.mla_chunk_attend_auto.restype = _I32

_lib.mla_chunk_attend_noalloc.argtypes = [_DIMS, _I32, _I32, _P, _P, _P, _I32, _P, _P, _P, _I32, _I32, ctypes.c_float,
                                          _P, _P]
_lib.mla_chunk_attend_noalloc.restype = _I32
NOALLOC_SCRATCH_BYTES = 128 << 20     # MLA_NOALLOC_SCRATCH_BYTES in mla.h

_lib.mla_ring_init.argtypes = [_RING, _I32, _I32, _I32]
_lib.mla_ring_init.restype = _I32
_lib.mla_ring_current.argtypes = [_RING, ctypes.POINTER(_I32), ctypes.POINTER(_I32)]
_lib.mla_ring_current.restype = _I32
_lib.mla_ring_commit.argtypes = [_RING]
_lib.mla_ring_commit.restype = _I32
_lib.mla_ring_slot_chunks.argtypes = [_RING, ctypes.POINTER(_I64)]
_lib.mla_ring_slot_chunks.restype = _I32
_lib.mla_cache_bytes.argtypes = [_DIMS, _I32, _I32]
_lib.mla_cache_bytes.restype = _I64
_lib.mla_dense_kv_bytes.argtypes = [_DIMS, _I32, _I32]
_lib.mla_dense_kv_bytes.restype = _I64
_lib.mla_ring_last_error.argtypes = []
_lib.mla_ring_last_error.restype = ctypes.c_char_p
_lib.mla_status_string.argtypes = [_I32]
_lib.mla_status_string.restype = ctypes.c_char_p
_lib.mla_last_error.argtypes = []
_lib.mla_last_error.restype = ctypes.c_char_p
_lib.mla_version.argtypes = []
_lib.mla_version.restype = ctypes.c_char_p


class MLAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = _lib.mla_last_error().decode()
        super().__init__(f"{where}: {_lib.mla_status_string(code).decode()} ({code}): {msg}")


@dataclass(frozen=True)
class Dims:
    batch: int
    n_heads: int = 12
    head_dim: int = 128
    d_c: int = 192
    d_r: int = 32
    rope: tuple = (8, 12, 12)
    rope_theta: float = 1e4

    def c(self) -> MlaDims:
        return MlaDims(self.batch, self.n_heads, self.head_dim, self.d_c, self.d_r,
                       self.rope[0], self.rope[1], self.rope[2], float(self.rope_theta))


def version() -> str:
    return _lib.mla_version().decode()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return MLA_BF16
    if t == torch.float32:
        return MLA_F32
    raise TypeError(f"unsupported dtype {t} (bfloat16 or float32)")


def _check(t: torch.Tensor, name: str, shape, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, but the library launches on the current device "
                         f"cuda:{torch.cuda.current_device()}")


def _ws(workspace):
    """(device pointer, size in bytes) of a workspace tensor of any dtype."""
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    _check(workspace, "workspace", tuple(workspace.shape))
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    if s.device.index != torch.cuda.current_device():
        raise ValueError(f"stream is on {s.device}, not on the current device cuda:{torch.cuda.current_device()}")
    return s.cuda_stream


def _raise(code: int, where: str):
    if code != MLA_OK:
        raise MLAError(code, where)


def cache_append(dims: Dims, x, w_dkv, w_kr, pos, cache, offset: int, stream=None) -> None:
    """Write [W_DKV x || RoPE3D(pos) W_KR x] rows of the new tokens into cache[:, offset:offset+n]."""
    B, n_new, D = x.shape
    dt = x.dtype
    _check(x, "x", (dims.batch, n_new, D), dt)
    _check(w_dkv, "w_dkv", (dims.d_c, D), dt)
    _check(w_kr, "w_kr", (dims.d_r, D), dt)
    _check(pos, "pos", (n_new, 3), torch.int32)
    cap = cache.shape[1]
    _check(cache, "cache", (dims.batch, cap, dims.d_c + dims.d_r), dt)
    d = dims.c()
    code = _lib.mla_cache_append(ctypes.byref(d), _dtype_code(dt), x.data_ptr(), D, n_new, w_dkv.data_ptr(),
                                 w_kr.data_ptr(), pos.data_ptr(), cache.data_ptr(), cap, int(offset),
                                 _stream(stream))
    _raise(code, "mla_cache_append")


def workspace_bytes(dims: Dims, dtype: torch.dtype, n_q: int, n_k: int) -> int:
    d = dims.c()
    n = _lib.mla_chunk_attend_workspace_bytes(ctypes.byref(d), _dtype_code(dtype), int(n_q), int(n_k))
    if n < 0:
        _raise(int(n), "mla_chunk_attend_workspace_bytes")
    return int(n)


def alloc_workspace(dims: Dims, dtype: torch.dtype, n_q: int, n_k: int, device="cuda") -> torch.Tensor:
    n = workspace_bytes(dims, dtype, n_q, n_k)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _attend_checks(dims, q, q_r, q_pos, w_uk, w_uv, cache, n_k):
    B, n_q, H, dh = q.shape
    dt = q.dtype
    _check(q, "q", (dims.batch, n_q, dims.n_heads, dims.head_dim), dt)
    _check(q_r, "q_r", (dims.batch, n_q, dims.n_heads, dims.d_r), dt)
    _check(q_pos, "q_pos", (n_q, 3), torch.int32)
    if w_uk is not None:
        _check(w_uk, "w_uk", (dims.n_heads, dims.head_dim, dims.d_c), dt)
    if w_uv is not None:
        _check(w_uv, "w_uv", (dims.n_heads, dims.head_dim, dims.d_c), dt)
    if cache is not None:
        _check(cache, "cache", (dims.batch, cache.shape[1], dims.d_c + dims.d_r), dt)
    return n_q, dt


def chunk_attend(dims: Dims, q, q_r, q_pos, w_uk, w_uv, cache, n_k: int, scale: float,
                 out=None, out_dtype=None, workspace=None, stream=None, causal=None) -> torch.Tensor:
    """out[b,i,h] = sum_j softmax_j(scale*(q.k_h + RoPE(p_i)q_r.k_R)) W_UV[h] c_j over the visible keys.

    causal=None: every query sees keys [0, n_k).  causal=(q_start, chunk_len):
    query i is token q_start + i and sees the keys of every chunk up to its own
    (mla_chunk_attend_causal)."""
    n_q, dt = _attend_checks(dims, q, q_r, q_pos, w_uk, w_uv, cache, n_k)
    odt = dt if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((dims.batch, n_q, dims.n_heads, dims.head_dim), dtype=odt, device=q.device)
    _check(out, "out", (dims.batch, n_q, dims.n_heads, dims.head_dim), odt)
    if workspace is None:
        workspace = alloc_workspace(dims, dt, n_q, n_k, q.device)
    d = dims.c()
    args = (_dtype_code(dt), _dtype_code(odt), q.data_ptr(), q_r.data_ptr(), q_pos.data_ptr(), n_q,
            w_uk.data_ptr(), w_uv.data_ptr(), cache.data_ptr(), cache.shape[1], int(n_k))
    tail = (float(scale), out.data_ptr(), *_ws(workspace), _stream(stream))
    if causal is None:
        code = _lib.mla_chunk_attend(ctypes.byref(d), *args, *tail)
        _raise(code, "mla_chunk_attend")
    else:
        cz = MlaCausal(int(causal[0]), int(causal[1]))
        code = _lib.mla_chunk_attend_causal(ctypes.byref(d), *args, ctypes.byref(cz), *tail)
        _raise(code, "mla_chunk_attend_causal")
    return out


def chunk_attend_noalloc(dims: Dims, q, q_r, q_pos, w_uk, w_uv, cache, n_k: int, scale: float, out,
                         stream=None) -> torch.Tensor:
    """chunk_attend through mla_chunk_attend_noalloc: the library's static scratch
    replaces the workspace and nothing is allocated (out is the caller's)."""
    n_q, dt = _attend_checks(dims, q, q_r, q_pos, w_uk, w_uv, cache, n_k)
    _check(out, "out", (dims.batch, n_q, dims.n_heads, dims.head_dim), out.dtype)
    d = dims.c()
    code = _lib.mla_chunk_attend_noalloc(ctypes.byref(d), _dtype_code(dt), _dtype_code(out.dtype), q.data_ptr(),
                                         q_r.data_ptr(), q_pos.data_ptr(), n_q, w_uk.data_ptr(), w_uv.data_ptr(),
                                         cache.data_ptr(), cache.shape[1], int(n_k), float(scale), out.data_ptr(),
                                         _stream(stream))
    _raise(code, "mla_chunk_attend_noalloc")
    return out


def query_absorb(dims: Dims, q, q_r, q_pos, w_uk, scale: float, n_k: int, workspace, stream=None) -> None:
    n_q, dt = _attend_checks(dims, q, q_r, q_pos, w_uk, None, None, n_k)
    d = dims.c()
    code = _lib.mla_query_absorb(ctypes.byref(d), _dtype_code(dt), q.data_ptr(), q_r.data_ptr(), q_pos.data_ptr(),
                                 n_q, w_uk.data_ptr(), float(scale), int(n_k),
                                 *_ws(workspace), _stream(stream))
    _raise(code, "mla_query_absorb")


def latent_attend(dims: Dims, cache, n_q: int, n_k: int, workspace, stream=None, causal=None) -> None:
    _check(cache, "cache", (dims.batch, cache.shape[1], dims.d_c + dims.d_r), cache.dtype)
    d = dims.c()
    args = (_dtype_code(cache.dtype), cache.data_ptr(), cache.shape[1], int(n_q), int(n_k))
    tail = (*_ws(workspace), _stream(stream))
    if causal is None:
        _raise(_lib.mla_latent_attend(ctypes.byref(d), *args, *tail), "mla_latent_attend")
    else:
        cz = MlaCausal(int(causal[0]), int(causal[1]))
        _raise(_lib.mla_latent_attend_causal(ctypes.byref(d), *args, ctypes.byref(cz), *tail),
               "mla_latent_attend_causal")


def value_upproj(dims: Dims, w_uv, out, n_q: int, n_k: int, workspace, stream=None) -> None:
    _check(w_uv, "w_uv", (dims.n_heads, dims.head_dim, dims.d_c), w_uv.dtype)
    _check(out, "out", (dims.batch, n_q, dims.n_heads, dims.head_dim), out.dtype)
    d = dims.c()
    code = _lib.mla_value_upproj(ctypes.byref(d), _dtype_code(w_uv.dtype), _dtype_code(out.dtype), int(n_q),
                                 int(n_k), w_uv.data_ptr(), out.data_ptr(),
                                 *_ws(workspace), _stream(stream))
    _raise(code, "mla_value_upproj")


def mha_workspace_bytes(batch: int, n_heads: int, head_dim: int, n_q: int, n_k: int) -> int:
    n = _lib.mla_mha_attend_workspace_bytes(int(batch), int(n_heads), int(head_dim), int(n_q), int(n_k))
    if n < 0:
        _raise(int(n), "mla_mha_attend_workspace_bytes")
    return int(n)


def mha_attend(q, k, v, n_k: int, scale: float, out=None, out_dtype=None, workspace=None,
               stream=None) -> torch.Tensor:
    """Dense per-head attention (mla_mha_attend): out[b,i,h] = softmax_j(scale q.k_j) v_j, j < n_k.

    q [B, n_q, H, d_h]; k, v [B, capacity, H, d_h]; bf16."""
    B, n_q, H, dh = q.shape
    cap = k.shape[1]
    _check(q, "q", (B, n_q, H, dh), torch.bfloat16)
    _check(k, "k", (B, cap, H, dh), torch.bfloat16)
    _check(v, "v", (B, cap, H, dh), torch.bfloat16)
    odt = torch.bfloat16 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, n_q, H, dh), dtype=odt, device=q.device)
    _check(out, "out", (B, n_q, H, dh), odt)
    if workspace is None:
        workspace = torch.empty(mha_workspace_bytes(B, H, dh, n_q, n_k), dtype=torch.uint8, device=q.device)
    code = _lib.mla_mha_attend(B, H, dh, _dtype_code(odt), q.data_ptr(), n_q, k.data_ptr(), v.data_ptr(), cap,
                               int(n_k), float(scale), out.data_ptr(), *_ws(workspace),
                               _stream(stream))
    _raise(code, "mla_mha_attend")
    return out


def expanded_workspace_bytes(dims: Dims, n_q: int, n_k: int) -> int:
    d = dims.c()
    n = _lib.mla_chunk_attend_expanded_workspace_bytes(ctypes.byref(d), int(n_q), int(n_k))
    if n < 0:
        _raise(int(n), "mla_chunk_attend_expanded_workspace_bytes")
    return int(n)


def chunk_attend_expanded(dims: Dims, q, q_r, q_pos, w_uk, w_uv, cache, n_k: int, scale: float,
                          out=None, out_dtype=None, workspace=None, stream=None) -> torch.Tensor:
    """chunk_attend in the non-absorbed form (mla_chunk_attend_expanded): per-head K_h, V_h are
    materialised from the latent cache, then standard attention runs over them.  bf16."""
    n_q, dt = _attend_checks(dims, q, q_r, q_pos, w_uk, w_uv, cache, n_k)
    if dt != torch.bfloat16:
        raise TypeError("chunk_attend_expanded takes bfloat16 inputs")
    odt = dt if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((dims.batch, n_q, dims.n_heads, dims.head_dim), dtype=odt, device=q.device)
    _check(out, "out", (dims.batch, n_q, dims.n_heads, dims.head_dim), odt)
    if workspace is None:
        workspace = torch.empty(expanded_workspace_bytes(dims, n_q, n_k), dtype=torch.uint8, device=q.device)
    d = dims.c()
    code = _lib.mla_chunk_attend_expanded(ctypes.byref(d), _dtype_code(odt), q.data_ptr(), q_r.data_ptr(),
                                          q_pos.data_ptr(), n_q, w_uk.data_ptr(), w_uv.data_ptr(), cache.data_ptr(),
                                          cache.shape[1], int(n_k), float(scale), out.data_ptr(),
                                          *_ws(workspace), _stream(stream))
    _raise(code, "mla_chunk_attend_expanded")
    return out


MLA_FORM_ABSORBED, MLA_FORM_EXPANDED = 0, 1


def chunk_attend_form(dims: Dims, dtype: torch.dtype, n_q: int, n_k: int) -> int:
    """MLA_FORM_ABSORBED or MLA_FORM_EXPANDED: the form mla_chunk_attend_auto runs for this shape."""
    d = dims.c()
    f = _lib.mla_chunk_attend_form(ctypes.byref(d), _dtype_code(dtype), int(n_q), int(n_k))
    if f < 0:
        _raise(int(f), "mla_chunk_attend_form")
    return int(f)


def chunk_attend_auto(dims: Dims, q, q_r, q_pos, w_uk, w_uv, cache, n_k: int, scale: float,
                      out=None, out_dtype=None, workspace=None, stream=None) -> torch.Tensor:
    """chunk_attend through the faster evaluation order for the shape (mla_chunk_attend_auto)."""
    n_q, dt = _attend_checks(dims, q, q_r, q_pos, w_uk, w_uv, cache, n_k)
    odt = dt if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((dims.batch, n_q, dims.n_heads, dims.head_dim), dtype=odt, device=q.device)
    _check(out, "out", (dims.batch, n_q, dims.n_heads, dims.head_dim), odt)
    d = dims.c()
    if workspace is None:
        n = _lib.mla_chunk_attend_auto_workspace_bytes(ctypes.byref(d), _dtype_code(dt), n_q, int(n_k))
        if n < 0:
            _raise(int(n), "mla_chunk_attend_auto_workspace_bytes")
        workspace = torch.empty(int(n), dtype=torch.uint8, device=q.device)
    code = _lib.mla_chunk_attend_auto(ctypes.byref(d), _dtype_code(dt), _dtype_code(odt), q.data_ptr(),
                                      q_r.data_ptr(), q_pos.data_ptr(), n_q, w_uk.data_ptr(), w_uv.data_ptr(),
                                      cache.data_ptr(), cache.shape[1], int(n_k), float(scale), out.data_ptr(),
                                      *_ws(workspace), _stream(stream))
    _raise(code, "mla_chunk_attend_auto")
    return out


class Ring:
    """Rolling latent cache bookkeeping (mla_ring_*): sink chunks kept for the
    whole rollout, a window of recent chunks, one slot for the current chunk."""

    def __init__(self, chunk_tokens: int, sink_chunks: int, window_chunks: int):
        self._r = MlaRing()
        code = _lib.mla_ring_init(ctypes.byref(self._r), int(chunk_tokens), int(sink_chunks), int(window_chunks))
        if code != MLA_OK:
            raise ValueError(_lib.mla_ring_last_error().decode())

    @property
    def capacity(self) -> int:
        return self._r.capacity

    @property
    def committed(self) -> int:
        return self._r.committed

    def current(self):
        """(write_offset, n_k) of the chunk being denoised."""
        off, n_k = _I32(), _I32()
        _raise(_lib.mla_ring_current(ctypes.byref(self._r), ctypes.byref(off), ctypes.byref(n_k)), "mla_ring_current")
        return off.value, n_k.value

    def commit(self) -> None:
        _raise(_lib.mla_ring_commit(ctypes.byref(self._r)), "mla_ring_commit")

    def state(self) -> tuple:
        """The ring's whole state (mla_ring is plain caller-owned data): with the
        cache slots [0, capacity) of its sample it checkpoints the rollout."""
        r = self._r
        return (r.chunk_tokens, r.sink_chunks, r.window_chunks, r.capacity, r.committed)

    @classmethod
    def from_state(cls, state: tuple) -> "Ring":
        """A ring that resumes from state(): the same slots and n_k from here on."""
        ring = cls.__new__(cls)
        ring._r = MlaRing(*(int(v) for v in state))
        return ring

    def slot_chunks(self):
        n = self._r.sink_chunks + self._r.window_chunks + 1
        arr = (_I64 * n)()
        _raise(_lib.mla_ring_slot_chunks(ctypes.byref(self._r), arr), "mla_ring_slot_chunks")
        return list(arr)


def cache_bytes(dims: Dims, dtype: torch.dtype, capacity: int) -> int:
    d = dims.c()
    return int(_lib.mla_cache_bytes(ctypes.byref(d), _dtype_code(dtype), int(capacity)))


def dense_kv_bytes(dims: Dims, dtype: torch.dtype, capacity: int) -> int:
    d = dims.c()
    return int(_lib.mla_dense_kv_bytes(ctypes.byref(d), _dtype_code(dtype), int(capacity)))


def raw():
    """The loaded ctypes library (for tests of the C ABI itself)."""
    return _lib
