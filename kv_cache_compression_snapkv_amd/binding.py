"""ctypes binding of libanchorkv.so (the C ABI in include/anchorkv.h).

Argument marshalling only: device buffers are torch tensors (for allocation
and streams); every step of the compress and decode paths runs in the HIP
library.  There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes as ct
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libanchorkv.so")

BF16, F32 = 1, 2
CODEC_AFFINE, CODEC_HADAMARD_LM = 0, 1
ANCHORS_UNIFORM, ANCHORS_COVER = 0, 1

ERRORS = {-1: "E_ARG", -2: "E_DTYPE", -3: "E_SHAPE", -4: "E_BUDGET", -5: "E_SMALL_BUFFER", -6: "E_HIP", -7: "E_LAYOUT"}


class AnchorKVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class Dims(ct.Structure):
    _fields_ = [("units", ct.c_int32), ("kv_heads", ct.c_int32), ("q_per_kv", ct.c_int32), ("n_tokens", ct.c_int32),
                ("head_dim", ct.c_int32), ("n_obs", ct.c_int32), ("dtype", ct.c_int32)]


class Params(ct.Structure):
    _fields_ = [("theta", ct.c_float), ("window", ct.c_int32), ("anchor_div", ct.c_int32), ("pool", ct.c_int32),
                ("rho", ct.c_double), ("group", ct.c_int32), ("pool_kv_jointly", ct.c_int32),
                ("codec", ct.c_int32), ("hadamard_signs", ct.c_uint32 * 4), ("anchor_mode", ct.c_int32),
                ("cover_rounds", ct.c_int32), ("rope", ct.c_int32), ("rope_theta", ct.c_float),
                ("reserved", ct.c_int32 * 2)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_ if f not in ("reserved", "hadamard_signs")}
        d["hadamard_signs"] = list(self.hadamard_signs)
        return d


class Layout(ct.Structure):
    _fields_ = [(f, ct.c_int64) for f in ("off_anchor_k", "off_anchor_v", "off_res_k", "off_res_v", "off_words",
                                           "off_chunk_k", "off_chunk_v", "off_positions", "unit_bytes",
                                           "unit_stride")] + \
               [(f, ct.c_int32) for f in ("A", "R_K", "R_V", "n_chunks", "record_bytes")] + [("reserved", ct.c_int32 * 3)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_ if f != "reserved"}


class PlanInfo(ct.Structure):
    _fields_ = [
        ("units", ct.c_int32), ("H", ct.c_int32), ("G", ct.c_int32), ("N", ct.c_int32), ("D", ct.c_int32),
        ("n_obs", ct.c_int32), ("dtype", ct.c_int32), ("elem_bytes", ct.c_int32), ("window", ct.c_int32),
        ("theta", ct.c_float), ("params", Params),
        ("A", ct.c_int32), ("k_scored", ct.c_int32), ("k_uniform", ct.c_int32), ("R_K", ct.c_int32),
        ("R_V", ct.c_int32), ("n_chunks", ct.c_int32),
        ("budget_bytes_per_side", ct.c_int64), ("used_bytes_k", ct.c_int64), ("used_bytes_v", ct.c_int64),
        ("compression_ratio", ct.c_double),
        ("off_anchor_k", ct.c_int64), ("off_anchor_v", ct.c_int64), ("off_res_k", ct.c_int64),
        ("off_res_v", ct.c_int64), ("off_words", ct.c_int64), ("off_chunk_k", ct.c_int64),
        ("off_chunk_v", ct.c_int64), ("off_positions", ct.c_int64),
        ("unit_bytes", ct.c_int64), ("unit_stride", ct.c_int64), ("cache_bytes", ct.c_int64),
        ("compress_workspace_bytes", ct.c_int64), ("decode_workspace_bytes", ct.c_int64),
        ("decode_splits", ct.c_int32), ("joint", ct.c_int32), ("R_total", ct.c_int32), ("reserved", ct.c_int32 * 5),
    ]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_ if f not in ("reserved", "params")}
        d.update({"param_" + k: v for k, v in self.params.as_dict().items()})
        return d


class UnitArrays(ct.Structure):
    _fields_ = [("positions", ct.c_void_p), ("anchors_k", ct.c_void_p), ("anchors_v", ct.c_void_p),
                ("idx", ct.c_void_p), ("gamma16", ct.c_void_p), ("flag", ct.c_void_p), ("codes", ct.c_void_p),
                ("scale16", ct.c_void_p), ("zero16", ct.c_void_p)]


_lib = None


def lib():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(f"{LIB_PATH} is missing: build it with "
                                    "`python -m kv_cache_compression_snapkv_amd.build`")
        L = ct.CDLL(LIB_PATH)
        L.anchorkv_version.restype = ct.c_char_p
        L.anchorkv_last_error.restype = ct.c_char_p
        L.anchorkv_params_default.argtypes = [ct.POINTER(Params), ct.c_float, ct.c_int32]
        L.anchorkv_params_default.restype = None
        L.anchorkv_plan.argtypes = [ct.POINTER(Dims), ct.POINTER(Params), ct.POINTER(PlanInfo)]
        L.anchorkv_plan_from_header.argtypes = [ct.c_void_p, ct.c_int32, ct.POINTER(PlanInfo)]
        L.anchorkv_cache_layout.argtypes = [ct.c_void_p, ct.POINTER(Layout)]
        L.anchorkv_decode_workspace_bytes.argtypes = [ct.c_void_p, ct.c_int32, ct.POINTER(ct.c_size_t)]
        L.anchorkv_compress.argtypes = [ct.POINTER(PlanInfo), ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                        ct.c_size_t, ct.c_void_p, ct.c_size_t, ct.c_void_p]
        L.anchorkv_workspace_offsets.argtypes = [ct.POINTER(PlanInfo), ct.POINTER(ct.c_int64)]
        L.anchorkv_decode_attn.argtypes = [ct.POINTER(PlanInfo), ct.c_void_p, ct.c_size_t, ct.c_void_p, ct.c_void_p,
                                           ct.c_void_p, ct.c_size_t, ct.c_void_p]
        L.anchorkv_decode_attn_tail.argtypes = [ct.POINTER(PlanInfo), ct.c_void_p, ct.c_size_t, ct.c_void_p,
                                                ct.c_void_p, ct.c_void_p, ct.c_int32, ct.c_int32, ct.c_void_p,
                                                ct.c_void_p, ct.c_size_t, ct.c_void_p]
        L.anchorkv_decode_attn_noalloc.argtypes = [ct.POINTER(PlanInfo), ct.c_void_p, ct.c_size_t, ct.c_void_p,
                                                   ct.c_void_p, ct.c_void_p]
        L.anchorkv_unit_pack_host.argtypes = [ct.POINTER(PlanInfo), ct.POINTER(UnitArrays), ct.c_void_p]
        L.anchorkv_unit_unpack_host.argtypes = [ct.POINTER(PlanInfo), ct.c_void_p, ct.POINTER(UnitArrays)]
        L.anchorkv_profile_enable.argtypes = [ct.c_int]
        L.anchorkv_profile_read.argtypes = [ct.POINTER(ct.c_char_p), ct.POINTER(ct.c_float), ct.c_int,
                                            ct.POINTER(ct.c_int)]
        _lib = L
    return _lib


EXPORTED = ["anchorkv_version", "anchorkv_last_error", "anchorkv_params_default", "anchorkv_plan",
            "anchorkv_plan_from_header", "anchorkv_cache_layout", "anchorkv_decode_workspace_bytes",
            "anchorkv_compress", "anchorkv_workspace_offsets", "anchorkv_decode_attn", "anchorkv_decode_attn_tail",
            "anchorkv_decode_attn_noalloc",
            "anchorkv_unit_pack_host",
            "anchorkv_unit_unpack_host", "anchorkv_profile_enable", "anchorkv_profile_read"]


def _check(rc: int):
    if rc != 0:
        raise AnchorKVError(rc, lib().anchorkv_last_error().decode())


def version() -> str:
    return lib().anchorkv_version().decode()


def params(theta, window, **kw) -> Params:
    """The method's parameters: defaults (anchorkv_params_default) with the
    given theta and window, then any of anchor_div, rho, pool, group,
    pool_kv_jointly, codec, hadamard_signs (four 32-bit words), anchor_mode,
    cover_rounds, rope, rope_theta replaced."""
    q = Params()
    lib().anchorkv_params_default(ct.byref(q), ct.c_float(theta), int(window))
    for k, v in kw.items():
        if k == "hadamard_signs":
            for i, x in enumerate(v):
                q.hadamard_signs[i] = int(x)
            continue
        if k not in ("anchor_div", "rho", "pool", "group", "pool_kv_jointly", "codec", "anchor_mode", "cover_rounds",
                     "rope", "rope_theta"):
            raise TypeError(f"unknown parameter {k}")
        setattr(q, k, v)
    return q


def plan(units, kv_heads, q_per_kv, n_tokens, head_dim, n_obs, dtype, theta, window, **kw) -> PlanInfo:
    """anchorkv_plan for the dims and params(theta, window, **kw)."""
    d = Dims(units, kv_heads, q_per_kv, n_tokens, head_dim, n_obs, dtype)
    q = params(theta, window, **kw)
    p = PlanInfo()
    _check(lib().anchorkv_plan(ct.byref(d), ct.byref(q), ct.byref(p)))
    return p


def plan_from_header(header: bytes, units: int) -> PlanInfo:
    p = PlanInfo()
    buf = ct.create_string_buffer(bytes(header[:256]), 256)
    _check(lib().anchorkv_plan_from_header(buf, units, ct.byref(p)))
    return p


def cache_layout(header: bytes) -> dict:
    """Section offsets of a unit, from a host copy of its header."""
    lay = Layout()
    buf = ct.create_string_buffer(bytes(header[:256]), 256)
    _check(lib().anchorkv_cache_layout(buf, ct.byref(lay)))
    return lay.as_dict()


def decode_workspace_bytes(header: bytes, units: int) -> int:
    n = ct.c_size_t(0)
    buf = ct.create_string_buffer(bytes(header[:256]), 256)
    _check(lib().anchorkv_decode_workspace_bytes(buf, units, ct.byref(n)))
    return int(n.value)


def workspace_offsets(p: PlanInfo) -> dict:
    out = (ct.c_int64 * 8)()
    _check(lib().anchorkv_workspace_offsets(ct.byref(p), out))
    keys = ["score", "ml", "o", "util", "gamma", "rn2", "aidx", "GQp"]
    return dict(zip(keys, list(out)))


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _expect(fn, name, t, shape, dtype):
    """The C ABI takes bare pointers: check what the kernels will index."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{fn}: {name} must be {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def _elem_dtype(p: PlanInfo):
    import torch
    return torch.bfloat16 if p.dtype == BF16 else torch.float32


def compress(p: PlanInfo, K, V, Q, cache, workspace, stream=None):
    """Enqueue the compression of all units (torch CUDA tensors, contiguous)."""
    for t in (K, V, Q, cache, workspace):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("compress: inputs must be contiguous device tensors")
    dt = _elem_dtype(p)
    _expect("compress", "K", K, (p.units, p.H, p.N, p.D), dt)
    _expect("compress", "V", V, (p.units, p.H, p.N, p.D), dt)
    _expect("compress", "Q_obs", Q, (p.units, p.H * p.G, p.n_obs, p.D), dt)
    _check(lib().anchorkv_compress(ct.byref(p), _ptr(K), _ptr(V), _ptr(Q), _ptr(cache), _nbytes(cache),
                                   _ptr(workspace), _nbytes(workspace), _stream(stream)))


def _check_cache(fn, p: PlanInfo, cache):
    import torch
    if cache.dtype != torch.uint8 or cache.numel() < p.cache_bytes:
        raise ValueError(f"{fn}: cache must be a uint8 tensor of >= {p.cache_bytes} bytes, "
                         f"got {cache.dtype} with {cache.numel()} elements")


def decode_attn(p: PlanInfo, cache, q, o, workspace, stream=None):
    """Enqueue decode attention: q [U, H*G, D] cache dtype -> o [U, H*G, D] float32."""
    for t in (cache, q, o, workspace):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("decode_attn: inputs must be contiguous device tensors")
    import torch
    _check_cache("decode_attn", p, cache)
    _expect("decode_attn", "q", q, (p.units, p.H * p.G, p.D), _elem_dtype(p))
    _expect("decode_attn", "o", o, (p.units, p.H * p.G, p.D), torch.float32)
    _check(lib().anchorkv_decode_attn(ct.byref(p), _ptr(cache), _nbytes(cache), _ptr(q), _ptr(o), _ptr(workspace),
                                      _nbytes(workspace), _stream(stream)))


def decode_attn_noalloc(p: PlanInfo, cache, q, o, stream=None):
    """decode_attn with the library's static device workspace (no workspace
    tensor; calls that overlap on one GPU race)."""
    for t in (cache, q, o):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("decode_attn_noalloc: inputs must be contiguous device tensors")
    import torch
    _check_cache("decode_attn_noalloc", p, cache)
    _expect("decode_attn_noalloc", "q", q, (p.units, p.H * p.G, p.D), _elem_dtype(p))
    _expect("decode_attn_noalloc", "o", o, (p.units, p.H * p.G, p.D), torch.float32)
    _check(lib().anchorkv_decode_attn_noalloc(ct.byref(p), _ptr(cache), _nbytes(cache), _ptr(q), _ptr(o),
                                              _stream(stream)))


def decode_attn_tail(p: PlanInfo, cache, q, K_tail, V_tail, n_tail: int, o, workspace, stream=None):
    """Enqueue decode attention over the compressed cache plus an exact tail:
    K_tail, V_tail [U, H, tail_cap, D] cache dtype (rows [0, n_tail) used);
    q [U, H*G, D] cache dtype -> o [U, H*G, D] float32."""
    for t in (cache, q, o, workspace, K_tail, V_tail):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("decode_attn_tail: inputs must be contiguous device tensors")
    import torch
    if K_tail.dim() != 4:
        raise ValueError("decode_attn_tail: K_tail must be [U, H, tail_cap, D]")
    cap = int(K_tail.shape[2])
    _check_cache("decode_attn_tail", p, cache)
    _expect("decode_attn_tail", "q", q, (p.units, p.H * p.G, p.D), _elem_dtype(p))
    _expect("decode_attn_tail", "o", o, (p.units, p.H * p.G, p.D), torch.float32)
    _expect("decode_attn_tail", "K_tail", K_tail, (p.units, p.H, cap, p.D), _elem_dtype(p))
    _expect("decode_attn_tail", "V_tail", V_tail, (p.units, p.H, cap, p.D), _elem_dtype(p))
    _check(lib().anchorkv_decode_attn_tail(ct.byref(p), _ptr(cache), _nbytes(cache), _ptr(q), _ptr(K_tail), _ptr(V_tail),
                                           int(n_tail), int(K_tail.shape[2]), _ptr(o), _ptr(workspace),
                                           _nbytes(workspace), _stream(stream)))


def alloc(p: PlanInfo, device):
    """Cache, compress workspace and decode workspace as uint8 device tensors."""
    import torch
    cache = torch.empty(int(p.cache_bytes), dtype=torch.uint8, device=device)
    ws = torch.empty(int(p.compress_workspace_bytes), dtype=torch.uint8, device=device)
    dws = torch.empty(int(p.decode_workspace_bytes), dtype=torch.uint8, device=device)
    return cache, ws, dws


def profile_enable(on: bool = True):
    """Record HIP events between the stages of every compress / decode call."""
    _check(lib().anchorkv_profile_enable(1 if on else 0))


def profile_read(max_stages: int = 1024):
    """[(stage, ms), ...] for the calls since the last read (waits for them)."""
    names = (ct.c_char_p * max_stages)()
    ms = (ct.c_float * max_stages)()
    n = ct.c_int(0)
    _check(lib().anchorkv_profile_read(names, ms, max_stages, ct.byref(n)))
    return [(names[i].decode(), float(ms[i])) for i in range(n.value)]


# ---------------------------------------------------------------- host packer
def _unit_arrays(p: PlanInfo):
    H, N, D, A = p.H, p.N, p.D, p.A
    adt = np.uint16 if p.dtype == BF16 else np.float32
    arr = dict(
        positions=np.zeros((H, A), np.int32),
        anchors_k=np.zeros((H, A, D), adt), anchors_v=np.zeros((H, A, D), adt),
        idx=np.zeros((2, H, N), np.int32), gamma16=np.zeros((2, H, N), np.uint16),
        flag=np.zeros((2, H, N), np.uint8), codes=np.zeros((2, H, N, D), np.uint8),
        scale16=np.zeros((2, H, N, D // 32), np.uint16), zero16=np.zeros((2, H, N, D // 32), np.uint16))
    return arr


def _struct(arr) -> UnitArrays:
    s = UnitArrays()
    for k in arr:
        a = arr[k]
        assert a.flags["C_CONTIGUOUS"]
        setattr(s, k, a.ctypes.data)
    return s


def pack_unit(p: PlanInfo, arrays: dict) -> bytes:
    """Pack one unit from host numpy arrays (see anchorkv_unit_arrays)."""
    base = _unit_arrays(p)
    for k in base:
        base[k] = np.ascontiguousarray(arrays[k], dtype=base[k].dtype).reshape(base[k].shape)
    out = ct.create_string_buffer(int(p.unit_bytes))
    _check(lib().anchorkv_unit_pack_host(ct.byref(p), ct.byref(_struct(base)), out))
    return out.raw


def unpack_unit(p: PlanInfo, unit: bytes) -> dict:
    """Decode one unit's bytes into host numpy arrays."""
    arr = _unit_arrays(p)
    buf = ct.create_string_buffer(bytes(unit[:int(p.unit_bytes)]), int(p.unit_bytes))
    _check(lib().anchorkv_unit_unpack_host(ct.byref(p), buf, ct.byref(_struct(arr))))
    return arr
