"""Python binding of the flash-decoding C ABI (``include/fd.h``), via ctypes.

Argument marshalling only: every step of the attention runs in the HIP kernels of
``libfd.so``.  PyTorch provides device memory and the current HIP stream.  If the library
cannot be loaded (or built) the calls raise -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfd.so")

FD_OK, FD_ERR_INVALID_ARG, FD_ERR_UNSUPPORTED, FD_ERR_WORKSPACE, FD_ERR_LAUNCH, FD_ERR_CONTRACT = 0, 1, 2, 3, 4, 5
FD_ERR_SCRATCH = 6
FD_SCRATCH_BYTES = 48 << 20  # include/fd.h
FD_F32, FD_F16, FD_BF16, FD_FP8_E4M3, FD_INT8 = 0, 1, 2, 3, 4
FD_SCALE_NONE, FD_SCALE_PER_TENSOR, FD_SCALE_PER_TOKEN_HEAD = 0, 1, 2

DTYPE_CODES = {"f32": FD_F32, "f16": FD_F16, "bf16": FD_BF16, "fp8_e4m3": FD_FP8_E4M3, "int8": FD_INT8}
SCALE_CODES = {"none": FD_SCALE_NONE, "tensor": FD_SCALE_PER_TENSOR, "token_head": FD_SCALE_PER_TOKEN_HEAD}
EXPORTS = ("fd_decode_attention", "fd_workspace_bytes", "fd_plan_partitions", "fd_status_string",
           "fd_version", "fd_fp8_e4m3_decode", "fd_set_profile_events", "fd_hbm_read_probe",
           "fd_kv_append", "fd_fp8_e4m3_encode", "fd_decode_attention_mq", "fd_workspace_bytes_mq",
           "fd_plan_partitions_mq", "fd_check_inputs", "fd_decode_attention_noalloc")

_lock = threading.Lock()
_lib = None


class FdError(RuntimeError):
    def __init__(self, status: int, what: str = "fd_decode_attention"):
        self.status = status
        super().__init__(f"{what} failed: {status_string(status)} ({status})")


def _c_int(x):
    return ctypes.c_int(int(x))


def lib() -> ctypes.CDLL:
    """Load libfd.so, building it first if it is not there."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        # FD_LIB: a separately built copy of the library (e.g. a host-sanitizer build) to load
        path = os.environ.get("FD_LIB") or LIB_PATH
        if not os.path.exists(path):
            if path != LIB_PATH:
                raise RuntimeError(f"FD_LIB names {path}, which does not exist")
            from . import _build
            _build.build()
        L = ctypes.CDLL(path)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.fd_decode_attention.restype = i32
        L.fd_decode_attention.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                          i32, i32, i32, vp, vp, ctypes.c_float, vp, i32, vp, vp, sz,
                                          i32, vp]
        L.fd_decode_attention_mq.restype = i32
        L.fd_decode_attention_mq.argtypes = [vp, i32] + L.fd_decode_attention.argtypes[1:]
        L.fd_decode_attention_noalloc.restype = i32
        # the _mq arguments without (workspace, workspace_bytes)
        L.fd_decode_attention_noalloc.argtypes = L.fd_decode_attention_mq.argtypes[:23] + \
            L.fd_decode_attention_mq.argtypes[25:]
        L.fd_workspace_bytes_mq.restype = sz
        L.fd_workspace_bytes_mq.argtypes = [i32] * 9
        L.fd_plan_partitions_mq.restype = i32
        L.fd_plan_partitions_mq.argtypes = [i32] * 9
        L.fd_workspace_bytes.restype = sz
        L.fd_workspace_bytes.argtypes = [i32] * 8
        L.fd_plan_partitions.restype = i32
        L.fd_plan_partitions.argtypes = [i32] * 8
        L.fd_status_string.restype = ctypes.c_char_p
        L.fd_status_string.argtypes = [i32]
        L.fd_version.restype = i32
        L.fd_version.argtypes = []
        L.fd_fp8_e4m3_decode.restype = i32
        L.fd_fp8_e4m3_decode.argtypes = [vp, vp, i32, vp]
        L.fd_hbm_read_probe.restype = i32
        L.fd_hbm_read_probe.argtypes = [vp, sz, vp, i32, i32, vp]
        L.fd_set_profile_events.restype = i32
        L.fd_set_profile_events.argtypes = [vp, vp]
        L.fd_kv_append.restype = i32
        L.fd_kv_append.argtypes = [vp, vp, i32, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                   vp, vp, vp]
        L.fd_fp8_e4m3_encode.restype = i32
        L.fd_fp8_e4m3_encode.argtypes = [vp, vp, i32, vp]
        L.fd_check_inputs.restype = i32
        L.fd_check_inputs.argtypes = [vp, vp, i32, vp, i32, i32, i32, ctypes.c_int64, vp, vp]
        _lib = L
        return L


def status_string(status: int) -> str:
    return lib().fd_status_string(int(status)).decode()


def version() -> int:
    return lib().fd_version()


def workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, block_size=0,
                    kv_dtype="fp8_e4m3", num_partitions=0, num_query=1) -> int:
    n = lib().fd_workspace_bytes_mq(batch, num_query, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                    block_size, DTYPE_CODES.get(kv_dtype, kv_dtype), num_partitions)
    if n == ctypes.c_size_t(-1).value:
        raise FdError(FD_ERR_INVALID_ARG, "fd_workspace_bytes")
    return n


def plan_partitions(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, block_size=0,
                    kv_dtype="fp8_e4m3", num_partitions=0, num_query=1) -> int:
    """Number of partitions (partition-kernel waves) the library will use."""
    n = lib().fd_plan_partitions_mq(batch, num_query, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                    block_size, DTYPE_CODES.get(kv_dtype, kv_dtype), num_partitions)
    if n < 0:
        raise FdError(FD_ERR_INVALID_ARG, "fd_plan_partitions")
    return n


def decode_attention_raw(q, k_cache, v_cache, block_table, max_blocks_per_seq, kv_start, seq_len,
                         batch, max_seq_len, num_q_heads, num_kv_heads, head_dim, block_size,
                         kv_dtype, q_dtype, scale_mode, k_scale, v_scale, softmax_scale, out,
                         out_dtype, lse, workspace, workspace_bytes_, num_partitions, stream) -> int:
    """Direct call of fd_decode_attention with integer pointers/codes; returns the status."""
    return lib().fd_decode_attention(q, k_cache, v_cache, block_table, max_blocks_per_seq, kv_start,
                                     seq_len, batch, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                                     block_size, kv_dtype, q_dtype, scale_mode, k_scale, v_scale,
                                     ctypes.c_float(softmax_scale), out, out_dtype, lse, workspace,
                                     workspace_bytes_, num_partitions, stream)


def decode_attention_mq_raw(q, num_query, *args) -> int:
    """Direct call of fd_decode_attention_mq: the arguments of ``decode_attention_raw`` with the
    window size after q; returns the status."""
    a = list(args)
    a[17] = ctypes.c_float(a[17])  # softmax_scale
    return lib().fd_decode_attention_mq(q, num_query, *a)


def decode_attention_noalloc_raw(q, num_query, *args) -> int:
    """Direct call of fd_decode_attention_noalloc: the arguments of ``decode_attention_mq_raw``
    without (workspace, workspace_bytes); returns the status."""
    a = list(args)
    a[17] = ctypes.c_float(a[17])  # softmax_scale
    return lib().fd_decode_attention_noalloc(q, num_query, *a)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _require_cuda(**tensors):
    for name, t in tensors.items():
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor (got {t.device})")


def _cache_dtypes(kv_dtype):
    import torch

    return {"f16": (torch.float16,), "bf16": (torch.bfloat16,),
            "fp8_e4m3": (torch.uint8, torch.float8_e4m3fn), "int8": (torch.int8,)}[kv_dtype]


def _int32_vector(name, t, n):
    import torch

    if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{name} must be a contiguous int32 tensor of {n} elements "
                         f"(got {t.dtype}, {tuple(t.shape)}, contiguous={t.is_contiguous()})")


def check_decode_args(q, k_cache, v_cache, seq_len, *, block_table, kv_start, kv_dtype, scale_mode,
                      k_scale, v_scale, num_kv_heads, block_size, max_seq_len):
    """Host-side checks of what the kernels assume of the tensors but the C ABI (plain pointers)
    cannot see: dtypes, contiguity, shapes and element counts.  Raises ValueError; launches
    nothing and needs no GPU (the tensors may live anywhere)."""
    import torch

    if kv_dtype not in DTYPE_CODES or kv_dtype == "f32":
        raise ValueError(f"kv_dtype must be one of f16, bf16, fp8_e4m3, int8 (got {kv_dtype!r})")
    if scale_mode not in SCALE_CODES:
        raise ValueError(f"scale_mode must be one of {tuple(SCALE_CODES)} (got {scale_mode!r})")
    if q.dtype not in (torch.float16, torch.bfloat16) or not q.is_contiguous() or q.dim() not in (3, 4):
        raise ValueError(f"q must be a contiguous f16/bf16 tensor [batch][heads][head_dim] or "
                         f"[batch][num_query][heads][head_dim] (got {q.dtype}, {tuple(q.shape)})")
    batch, d = q.shape[0], q.shape[-1]
    hkv = num_kv_heads if num_kv_heads is not None else k_cache.shape[-2]
    if (block_table is None) == (kv_start is None):
        raise ValueError("give exactly one of block_table (paged cache) and kv_start (contiguous cache)")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype not in _cache_dtypes(kv_dtype):
            raise ValueError(f"{name} dtype {t.dtype} does not hold kv_dtype {kv_dtype!r}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        want = 4 if block_table is not None else 3
        if t.dim() != want or t.shape[-1] != d or t.shape[-2] != hkv:
            raise ValueError(f"{name} must be [{'num_blocks][block_size' if want == 4 else 'rows'}]"
                             f"[{hkv}][{d}] (got {tuple(t.shape)})")
        if block_table is not None and t.shape[1] != block_size:
            raise ValueError(f"{name} blocks hold {t.shape[1]} tokens, block_size is {block_size}")
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError(f"k_cache and v_cache shapes differ ({tuple(k_cache.shape)} vs {tuple(v_cache.shape)})")
    _int32_vector("seq_len", seq_len, batch)
    if block_table is not None:
        if block_table.dtype != torch.int32 or not block_table.is_contiguous() or block_table.dim() != 2 \
                or block_table.shape[0] != batch:
            raise ValueError(f"block_table must be a contiguous int32 tensor [{batch}][max_blocks_per_seq] "
                             f"(got {block_table.dtype}, {tuple(block_table.shape)})")
        if max_seq_len > block_table.shape[1] * block_size:
            raise ValueError(f"max_seq_len {max_seq_len} exceeds the table's {block_table.shape[1]} "
                             f"blocks of {block_size} tokens")
    else:
        _int32_vector("kv_start", kv_start, batch)
    rows = k_cache.numel() // max(1, hkv * d)  # cache rows (tokens), all kv heads
    quant = kv_dtype in ("fp8_e4m3", "int8")
    if quant and scale_mode == "none":
        raise ValueError(f"kv_dtype {kv_dtype!r} needs k and v scales (scale_mode 'tensor' or 'token_head')")
    if not quant and scale_mode != "none":
        raise ValueError(f"kv_dtype {kv_dtype!r} takes no scales (scale_mode must be 'none')")
    if quant:
        n = 1 if scale_mode == "tensor" else rows * hkv
        for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
            if t is None or t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
                raise ValueError(f"{name} must be a contiguous fp32 tensor of {n} elements for scale_mode "
                                 f"{scale_mode!r} (got {None if t is None else (t.dtype, tuple(t.shape))})")


def decode_attention(q, k_cache, v_cache, seq_len, *, max_seq_len: int, block_table=None,
                     kv_start=None, kv_dtype: str, scale_mode: str = "none", k_scale=None,
                     v_scale=None, softmax_scale: float, num_kv_heads: int | None = None,
                     block_size: int = 0, out=None, out_dtype: str = "f32", lse=None,
                     workspace=None, num_partitions: int = 0, stream=None):
    """One decode step on the GPU.  Shapes follow ``include/fd.h``; sizes are read from the
    tensors.  A 4-d q [batch][num_query][heads][head_dim] is a window of query tokens per
    sequence (fd_decode_attention_mq; out and lse get the same leading dims).  ``out``/``workspace``
    are allocated with torch when not given (pass them in to keep the call allocation-free).
    Returns ``out``."""
    import torch

    check_decode_args(q, k_cache, v_cache, seq_len, block_table=block_table, kv_start=kv_start,
                      kv_dtype=kv_dtype, scale_mode=scale_mode, k_scale=k_scale, v_scale=v_scale,
                      num_kv_heads=num_kv_heads, block_size=block_size, max_seq_len=max_seq_len)
    _require_cuda(q=q, k_cache=k_cache, v_cache=v_cache, seq_len=seq_len, block_table=block_table,
                  kv_start=kv_start, k_scale=k_scale, v_scale=v_scale, out=out, lse=lse,
                  workspace=workspace)
    window = q.dim() == 4
    if window:
        batch, nq, hq, d = q.shape
    else:
        (batch, hq, d), nq = q.shape, 1
    hkv = num_kv_heads if num_kv_heads is not None else k_cache.shape[-2]
    q_code = {torch.float16: FD_F16, torch.bfloat16: FD_BF16}[q.dtype]
    kv_code = DTYPE_CODES[kv_dtype]
    out_code = DTYPE_CODES[out_dtype]
    if out is None:
        out = torch.empty(tuple(q.shape), dtype={"f32": torch.float32, "f16": torch.float16,
                                                 "bf16": torch.bfloat16}[out_dtype], device=q.device)
    # the kernels write one out row (and one lse value) per query row of q: refuse buffers of
    # another size before anything is launched
    if tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous tensor of q's shape {tuple(q.shape)} (got {tuple(out.shape)})")
    if lse is not None and (lse.numel() != q.numel() // d or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous fp32 tensor of {q.numel() // d} elements")
    if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor")
    max_blocks = 0 if block_table is None else block_table.shape[1]
    need = workspace_bytes(batch, hq, hkv, d, max_seq_len, block_size, kv_dtype, num_partitions, nq)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    args = (_ptr(k_cache), _ptr(v_cache), _ptr(block_table), max_blocks, _ptr(kv_start), _ptr(seq_len),
            batch, max_seq_len, hq, hkv, d, block_size, kv_code, q_code, SCALE_CODES[scale_mode],
            _ptr(k_scale), _ptr(v_scale), float(softmax_scale), _ptr(out), out_code, _ptr(lse),
            _ptr(workspace), ws_bytes, num_partitions, stream)
    if window:
        st = decode_attention_mq_raw(_ptr(q), nq, *args)
    else:
        st = decode_attention_raw(_ptr(q), *args)
    if st != FD_OK:
        raise FdError(st, "fd_decode_attention_mq" if window else "fd_decode_attention")
    return out


def decode_case(case, *, out=None, out_dtype="f32", lse=None, workspace=None, num_partitions=0,
                stream=None):
    """Convenience: run one ``workloads.Case`` (duck-typed) through the library."""
    return decode_attention(case.q, case.k_cache, case.v_cache, case.seq_len,
                            max_seq_len=case.max_seq_len, block_table=case.block_table,
                            kv_start=case.kv_start, kv_dtype=case.kv_dtype,
                            scale_mode=case.scale_mode, k_scale=case.k_scale, v_scale=case.v_scale,
                            softmax_scale=case.softmax_scale, num_kv_heads=case.hkv,
                            block_size=case.block_size, out=out, out_dtype=out_dtype, lse=lse,
                            workspace=workspace, num_partitions=num_partitions, stream=stream)


def fp8_e4m3_decode(x, stream=None):
    """Diagnostic: decode a uint8 GPU tensor with the kernels' conversions -> float32 [n][2]
    (column 0 via f16, column 1 via bf16)."""
    import torch

    _require_cuda(x=x)
    out = torch.empty((x.numel(), 2), dtype=torch.float32, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = lib().fd_fp8_e4m3_decode(x.data_ptr(), out.data_ptr(), x.numel(), stream)
    if st != FD_OK:
        raise FdError(st, "fd_fp8_e4m3_decode")
    return out


def kv_append_raw(k_new, v_new, new_dtype, k_cache, v_cache, block_table, max_blocks_per_seq, kv_start,
                  pos, batch, num_kv_heads, head_dim, block_size, kv_dtype, scale_mode, k_scale,
                  v_scale, stream) -> int:
    """Direct call of fd_kv_append with integer pointers/codes; returns the status."""
    return lib().fd_kv_append(k_new, v_new, new_dtype, k_cache, v_cache, block_table, max_blocks_per_seq,
                              kv_start, pos, batch, num_kv_heads, head_dim, block_size, kv_dtype,
                              scale_mode, k_scale, v_scale, stream)


def kv_append(k_new, v_new, k_cache, v_cache, pos, *, kv_dtype: str, block_table=None, kv_start=None,
              block_size: int = 0, scale_mode: str = "none", k_scale=None, v_scale=None, stream=None):
    """Write the current token's K/V rows ``k_new``/``v_new`` ([batch][num_kv_heads][head_dim],
    f32/f16/bf16 GPU tensors) into the cache at token ``pos[b]`` of each sequence (in place;
    per-token E4M3 / INT8 scales are written too).  Layouts and codes as ``include/fd.h``."""
    import torch

    if k_new.dim() != 3 or k_new.dtype not in (torch.float32, torch.float16, torch.bfloat16):
        raise ValueError(f"k_new must be an f32/f16/bf16 tensor [batch][num_kv_heads][head_dim] "
                         f"(got {k_new.dtype}, {tuple(k_new.shape)})")
    batch, hkv, d = k_new.shape
    new_code = {torch.float32: FD_F32, torch.float16: FD_F16, torch.bfloat16: FD_BF16}[k_new.dtype]
    if v_new.dtype != k_new.dtype or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must have the same shape and dtype")
    if not (k_new.is_contiguous() and v_new.is_contiguous()):
        raise ValueError("k_new and v_new must be contiguous")
    _int32_vector("pos", pos, batch)
    if (block_table is None) == (kv_start is None):
        raise ValueError("give exactly one of block_table (paged cache) and kv_start (contiguous cache)")
    if block_table is not None and (block_table.dtype != torch.int32 or block_table.dim() != 2
                                    or not block_table.is_contiguous() or block_table.shape[0] != batch):
        raise ValueError(f"block_table must be a contiguous int32 tensor [{batch}][max_blocks_per_seq]")
    if kv_start is not None:
        _int32_vector("kv_start", kv_start, batch)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype not in _cache_dtypes(kv_dtype) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor holding kv_dtype {kv_dtype!r} (got {t.dtype})")
        if t.shape[-1] != d or t.shape[-2] != hkv:
            raise ValueError(f"{name} rows must be [{hkv}][{d}] like k_new (got {tuple(t.shape)})")
    if kv_dtype in ("fp8_e4m3", "int8"):
        rows = k_cache.numel() // (hkv * d)
        n = 1 if scale_mode == "tensor" else rows * hkv
        for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
            if t is None or t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
                raise ValueError(f"{name} must be a contiguous fp32 tensor of {n} elements")
    _require_cuda(k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, pos=pos,
                  block_table=block_table, kv_start=kv_start, k_scale=k_scale, v_scale=v_scale)
    max_blocks = 0 if block_table is None else block_table.shape[1]
    if stream is None:
        stream = torch.cuda.current_stream(k_new.device).cuda_stream
    st = kv_append_raw(_ptr(k_new), _ptr(v_new), new_code, _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                       max_blocks, _ptr(kv_start), _ptr(pos), batch, hkv, d, block_size,
                       DTYPE_CODES[kv_dtype], SCALE_CODES[scale_mode], _ptr(k_scale), _ptr(v_scale), stream)
    if st != FD_OK:
        raise FdError(st, "fd_kv_append")


def fp8_e4m3_encode(x, stream=None):
    """Diagnostic: the E4M3 codes fd_kv_append stores for the fp32 quotients in GPU tensor x."""
    import torch

    _require_cuda(x=x)
    out = torch.empty(x.numel(), dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = lib().fd_fp8_e4m3_encode(x.data_ptr(), out.data_ptr(), x.numel(), stream)
    if st != FD_OK:
        raise FdError(st, "fd_fp8_e4m3_encode")
    return out


def set_profile_events(begin=None, end=None):
    """Diagnostic: record torch.cuda.Event ``begin``/``end`` around the partition kernel of the
    following calls from this thread (None, None clears)."""
    if (begin is None) != (end is None):
        raise ValueError("pass both events or neither")
    bp = None if begin is None else begin.cuda_event
    ep = None if end is None else end.cuda_event
    st = lib().fd_set_profile_events(bp, ep)
    if st != FD_OK:
        raise FdError(st, "fd_set_profile_events")


CHECK_KINDS = {0: "none", 1: "seq_len", 2: "block_table", 3: "kv_start"}


def check_inputs_raw(seq_len, block_table, max_blocks_per_seq, kv_start, batch, max_seq_len, block_size,
                     extent, result, stream) -> int:
    """Direct call of fd_check_inputs with integer pointers; returns the status."""
    return lib().fd_check_inputs(seq_len, block_table, max_blocks_per_seq, kv_start, batch, max_seq_len,
                                 block_size, extent, result, stream)


def check_inputs(seq_len, *, max_seq_len: int, extent: int, block_table=None, kv_start=None,
                 block_size: int = 0, result=None, stream=None) -> dict:
    """Debug validation of the device-side contract (see ``fd_check_inputs`` in include/fd.h):
    seq_len range, the used block-table entries against ``extent`` physical blocks (paged) or
    kv_start + seq_len against ``extent`` rows (contiguous).  ``result``: optional int32 GPU
    tensor of 4 elements to write into.  Synchronises the device and returns
    {"violations", "first_sequence", "kind", "value"}."""
    import torch

    _require_cuda(seq_len=seq_len, block_table=block_table, kv_start=kv_start)
    batch = seq_len.numel()
    max_blocks = 0 if block_table is None else block_table.shape[1]
    if stream is None:
        stream = torch.cuda.current_stream(seq_len.device).cuda_stream
    if result is None:
        result = torch.empty(4, dtype=torch.int32, device=seq_len.device)
    elif result.dtype != torch.int32 or result.numel() < 4 or result.device != seq_len.device:
        raise ValueError("result must be an int32 GPU tensor of at least 4 elements")
    st = check_inputs_raw(seq_len.data_ptr(), None if block_table is None else block_table.data_ptr(),
                          max_blocks, None if kv_start is None else kv_start.data_ptr(), batch, max_seq_len,
                          block_size, extent, result.data_ptr(), stream)
    if st != FD_OK:
        raise FdError(st, "fd_check_inputs")
    torch.cuda.synchronize(seq_len.device)
    n, first, kind, value = result[:4].cpu().tolist()
    return {"violations": n, "first_sequence": first, "kind": CHECK_KINDS.get(kind, kind), "value": value}


def hbm_read_probe(buf, out, blocks: int, kind: int = 0, stream=None):
    """Diagnostic: stream-read GPU tensor ``buf`` (uint8, 16-byte multiple; 1 KB multiple for
    kinds 1 and 2) once with load design ``kind`` (see fd_hbm_read_probe); ``out`` is a uint32
    GPU tensor of at least blocks*256 elements."""
    import torch

    _require_cuda(buf=buf, out=out)
    nbytes = buf.numel() * buf.element_size()
    if out.numel() < blocks * 256:
        raise ValueError("out too small")
    if stream is None:
        stream = torch.cuda.current_stream(buf.device).cuda_stream
    st = lib().fd_hbm_read_probe(buf.data_ptr(), nbytes, out.data_ptr(), blocks, kind, stream)
    if st != FD_OK:
        raise FdError(st, "fd_hbm_read_probe")
