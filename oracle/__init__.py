"""fp64 CPU oracle for one flash-decoding attention step (ctypes wrapper of ``oracle.c``).

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only ``tests/``, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` may import this package.
It shares no code with the HIP library and never imports it; inputs are plain host arrays
(numpy or CPU torch tensors).

What it computes -- softmax(q . K^T * scale) . V over each sequence's dequantised cache -- and
the passages each function follows are documented in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F16, BF16, E4M3, I8 = 1, 2, 3, 4
_DTYPE = {"f16": F16, "bf16": BF16, "fp8_e4m3": E4M3, "int8": I8}
_SCALE = {"none": 0, "tensor": 1, "token_head": 2}


class _Problem(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("kv_start", ctypes.c_void_p),
        ("seq_len", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("d", ctypes.c_int32), ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32), ("scale_mode", ctypes.c_int32),
        ("softmax_scale", ctypes.c_double), ("nq", ctypes.c_int32),
    ]


class _Append(ctypes.Structure):
    _fields_ = [
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p), ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("kv_start", ctypes.c_void_p), ("pos", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("hkv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("scale_mode", ctypes.c_int32),
    ]


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (no fast-math: IEEE double semantics)."""
    with _lock:
        if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            tmp = _LIB + f".tmp{os.getpid()}"
            subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                                   "-o", tmp, _SRC, "-lm", "-lpthread"])
            os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # ORACLE_LIB: a separately built copy (e.g. a sanitizer build) to load instead
        path = os.environ.get("ORACLE_LIB")
        if not path:
            build()
            path = _LIB
        lib = ctypes.CDLL(path)
        lib.orc_e4m3_to_double.restype = ctypes.c_double
        lib.orc_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.orc_f16_to_double.restype = ctypes.c_double
        lib.orc_f16_to_double.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_double.restype = ctypes.c_double
        lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.orc_attend_range.restype = ctypes.c_int
        lib.orc_attend_range.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
        lib.orc_merge.restype = None
        lib.orc_merge.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)]
        lib.orc_decode_attention.restype = ctypes.c_int
        lib.orc_decode_attention.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
        lib.orc_f16_encode.restype = ctypes.c_uint16
        lib.orc_f16_encode.argtypes = [ctypes.c_float]
        lib.orc_bf16_encode.restype = ctypes.c_uint16
        lib.orc_bf16_encode.argtypes = [ctypes.c_float]
        lib.orc_quantize_row_e4m3.restype = ctypes.c_float
        lib.orc_quantize_row_e4m3.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_void_p]
        lib.orc_quantize_row_i8.restype = ctypes.c_float
        lib.orc_quantize_row_i8.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_void_p]
        lib.orc_kv_append.restype = ctypes.c_int
        lib.orc_kv_append.argtypes = [ctypes.POINTER(_Append)]
        _lib = lib
    return _lib


def _host(x, dtype=None):
    """Host numpy view (contiguous) of a numpy array or torch tensor (16-bit floats as raw bits)."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        import torch
        t = x.detach()
        if t.device.type != "cpu":
            t = t.cpu()
        t = t.contiguous()
        if t.dtype in (torch.float16, torch.bfloat16):
            t = t.view(torch.int16)
        x = t.numpy()
    x = np.ascontiguousarray(x)
    if dtype is not None:
        x = x.astype(dtype, copy=False)
    return x


class Problem:
    """Host-side copy of one decode step's inputs, laid out for oracle.c."""

    def __init__(self, *, q, k_cache, v_cache, seq_len, batch, hq, hkv, d, q_dtype, kv_dtype,
                 scale_mode="none", k_scale=None, v_scale=None, block_table=None, kv_start=None,
                 block_size=0, softmax_scale, nq=1):
        self._keep = dict(q=_host(q), k=_host(k_cache), v=_host(v_cache),
                          bt=_host(block_table, np.int32), ks=_host(kv_start, np.int32),
                          sl=_host(seq_len, np.int32), ksc=_host(k_scale, np.float32),
                          vsc=_host(v_scale, np.float32))
        k = self._keep
        ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
        self.d = d
        self.batch = batch
        self.hq = hq
        self.nq = int(nq)
        self.seq_lens = [int(x) for x in k["sl"]]
        self.s = _Problem(ptr(k["q"]), ptr(k["k"]), ptr(k["v"]), ptr(k["bt"]), ptr(k["ks"]),
                          ptr(k["sl"]), ptr(k["ksc"]), ptr(k["vsc"]), batch, hq, hkv, d,
                          block_size, 0 if k["bt"] is None else k["bt"].shape[1],
                          _DTYPE[q_dtype], _DTYPE[kv_dtype], _SCALE[scale_mode],
                          float(softmax_scale), int(nq))

    @classmethod
    def from_case(cls, case):
        """Build from a ``workloads.Case`` (duck-typed; any device)."""
        return cls(q=case.q, k_cache=case.k_cache, v_cache=case.v_cache, seq_len=case.seq_len,
                   batch=case.batch, hq=case.hq, hkv=case.hkv, d=case.d, q_dtype=case.q_dtype,
                   kv_dtype=case.kv_dtype, scale_mode=case.scale_mode, k_scale=case.k_scale,
                   v_scale=case.v_scale, block_table=case.block_table, kv_start=case.kv_start,
                   block_size=case.block_size, softmax_scale=case.softmax_scale,
                   nq=getattr(case, "nq", 1))


def host_threads() -> int:
    """Threads for the oracle: the CPUs this process may run on (its affinity mask), capped by
    OMP_NUM_THREADS when the environment sets one (a machine that shares its cores between jobs
    gives each its count there)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def decode_attention(prob: Problem, seqs=None, nthreads: int | None = None):
    """(out [B][Hq][D], lse [B][Hq]) in float64 -- or [B][nq][Hq][D], [B][nq][Hq] for a window of
    nq > 1 query tokens per sequence.  ``seqs``: optional iterable of sequence ids to compute
    (others are NaN)."""
    lib = _load()
    rows = (prob.batch, prob.nq, prob.hq) if prob.nq > 1 else (prob.batch, prob.hq)
    out = np.full(rows + (prob.d,), np.nan, dtype=np.float64)
    lse = np.full(rows, np.nan, dtype=np.float64)
    mask = None
    if seqs is not None:
        mask = np.zeros(prob.batch, dtype=np.uint8)
        mask[list(seqs)] = 1
    nthreads = nthreads or host_threads()
    rc = lib.orc_decode_attention(ctypes.byref(prob.s), None if mask is None else mask.ctypes.data,
                                  out.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return out, lse


def attend_range(prob: Problem, b: int, h: int, t0: int, t1: int):
    """Unnormalised partial state (m, l, acc[D]) of head h of sequence b over tokens [t0, t1)."""
    lib = _load()
    m, l_ = ctypes.c_double(), ctypes.c_double()
    acc = np.zeros(prob.d, dtype=np.float64)
    if lib.orc_attend_range(ctypes.byref(prob.s), b, h, t0, t1, ctypes.byref(m), ctypes.byref(l_),
                            acc.ctypes.data):
        raise ValueError("bad range")
    return m.value, l_.value, acc


def merge(ms, ls, accs):
    """Log-sum-exp merge of partial states -> (out[D], lse)."""
    lib = _load()
    ms = np.ascontiguousarray(ms, dtype=np.float64)
    ls = np.ascontiguousarray(ls, dtype=np.float64)
    accs = np.ascontiguousarray(accs, dtype=np.float64)
    d = accs.shape[-1]
    out = np.zeros(d, dtype=np.float64)
    lse = ctypes.c_double()
    lib.orc_merge(len(ms), ms.ctypes.data, ls.ctypes.data, accs.ctypes.data, d, out.ctypes.data,
                  ctypes.byref(lse))
    return out, lse.value


def e4m3_to_double(byte: int) -> float:
    return _load().orc_e4m3_to_double(byte)


def f16_to_double(bits: int) -> float:
    return _load().orc_f16_to_double(bits)


def bf16_to_double(bits: int) -> float:
    return _load().orc_bf16_to_double(bits)


# ---------------------------------------------------------------- KV-cache append (oracle.c)
def e4m3_encode(x: float) -> int:
    """Nearest E4M3 code of the fp32 value x (clamped to +-448, ties to even)."""
    return int(_load().orc_e4m3_encode(float(np.float32(x))))


def f16_encode(x: float) -> int:
    return int(_load().orc_f16_encode(float(np.float32(x))))


def bf16_encode(x: float) -> int:
    return int(_load().orc_bf16_encode(float(np.float32(x))))


def quantize_row_e4m3(x, scale: float = 0.0):
    """(bytes uint8[n], scale) for one fp32 row: scale = amax/448 unless a scale > 0 is given."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.shape[0], dtype=np.uint8)
    sc = _load().orc_quantize_row_e4m3(x.ctypes.data, int(x.shape[0]), float(scale), out.ctypes.data)
    return out, float(np.float32(sc))


def quantize_row_i8(x, scale: float = 0.0):
    """(codes int8[n], scale) for one fp32 row: scale = amax/127 unless a scale > 0 is given."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.shape[0], dtype=np.int8)
    sc = _load().orc_quantize_row_i8(x.ctypes.data, int(x.shape[0]), float(scale), out.ctypes.data)
    return out, float(np.float32(sc))


def kv_append(*, k_new, v_new, k_cache, v_cache, pos, kv_dtype, scale_mode="none", k_scale=None,
              v_scale=None, block_table=None, kv_start=None, block_size=0):
    """Host copies (k_cache, v_cache, k_scale, v_scale) after appending k_new / v_new
    ([batch][hkv][d], any float dtype -- converted to fp32 exactly) at token pos[b] of each
    sequence.  Caches are returned as raw bits (uint8 for E4M3, int16 for f16 / bf16)."""
    def f32(t):
        if hasattr(t, "detach"):
            t = t.detach().float().cpu().numpy()
        return np.ascontiguousarray(t, dtype=np.float32)
    kn, vn = f32(k_new), f32(v_new)
    batch, hkv, d = kn.shape
    keep = dict(kn=kn, vn=vn, kc=_host(k_cache).copy(), vc=_host(v_cache).copy(),
                ks=None if k_scale is None else _host(k_scale, np.float32).copy(),
                vs=None if v_scale is None else _host(v_scale, np.float32).copy(),
                bt=_host(block_table, np.int32), st=_host(kv_start, np.int32), pos=_host(pos, np.int32))
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    bt = keep["bt"]
    a = _Append(ptr(keep["kn"]), ptr(keep["vn"]), ptr(keep["kc"]), ptr(keep["vc"]), ptr(keep["ks"]),
                ptr(keep["vs"]), ptr(bt), ptr(keep["st"]), ptr(keep["pos"]), batch, hkv, d,
                block_size, 0 if bt is None else bt.shape[1], _DTYPE[kv_dtype], _SCALE[scale_mode])
    if _load().orc_kv_append(ctypes.byref(a)) != 0:
        raise ValueError("oracle rejected the append")
    return keep["kc"], keep["vc"], keep["ks"], keep["vs"]
