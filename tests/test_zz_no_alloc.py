"""fd_decode_attention_noalloc (partial states in the library's static per-GPU scratch array)
against fd_decode_attention_mq with a caller workspace, through the C ABI.

The two run the same kernels on the same plan, so their outputs must be equal bit for bit; both
are also held to the oracle's bar.  Calls come in pairs, the second smaller than the first, so
the second runs on whatever the first left in the shared scratch array."""
import numpy as np
import pytest
import torch

import decode_attention_06_amd as fd
import oracle
import workloads
from test_gpu_parity import TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    fd.lib()
    yield


def _args(case, out, lse, num_partitions):
    """Arguments after (q, num_query) shared by both entry points, up to the workspace."""
    bt = case.block_table
    return ([case.k_cache.data_ptr(), case.v_cache.data_ptr(), None if bt is None else bt.data_ptr(),
             case.max_blocks, None if case.kv_start is None else case.kv_start.data_ptr(),
             case.seq_len.data_ptr(), case.batch, case.max_seq_len, case.hq, case.hkv, case.d,
             case.block_size, fd.DTYPE_CODES[case.kv_dtype], fd.DTYPE_CODES[case.q_dtype],
             fd.SCALE_CODES[case.scale_mode],
             None if case.k_scale is None else case.k_scale.data_ptr(),
             None if case.v_scale is None else case.v_scale.data_ptr(),
             case.softmax_scale, out.data_ptr(), fd.FD_F32, lse.data_ptr()], num_partitions)


def _run_both(name, case, num_partitions=0):
    print(f"[{name}] lens={case.seq_lens} G={case.group} nq={case.nq} kv={case.kv_dtype} "
          f"scale={case.scale_mode} partitions={num_partitions}", flush=True)
    stream = torch.cuda.current_stream().cuda_stream
    rows = tuple(case.q.shape[:-1])
    out_ws = torch.full(tuple(case.q.shape), float("nan"), dtype=torch.float32, device="cuda")
    lse_ws = torch.full(rows, float("nan"), dtype=torch.float32, device="cuda")
    out_na, lse_na = torch.full_like(out_ws, float("nan")), torch.full_like(lse_ws, float("nan"))
    need = fd.workspace_bytes(case.batch, case.hq, case.hkv, case.d, case.max_seq_len, case.block_size,
                              case.kv_dtype, num_partitions, case.nq)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    head, np_ = _args(case, out_ws, lse_ws, num_partitions)
    st = fd.decode_attention_mq_raw(case.q.data_ptr(), case.nq, *head, ws.data_ptr(), need, np_, stream)
    assert st == fd.FD_OK, fd.status_string(st)
    head, np_ = _args(case, out_na, lse_na, num_partitions)
    st = fd.decode_attention_noalloc_raw(case.q.data_ptr(), case.nq, *head, np_, stream)
    assert st == fd.FD_OK, fd.status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(out_na, out_ws), f"{name}: out differs from the workspace entry point"
    assert torch.equal(lse_na, lse_ws), f"{name}: lse differs from the workspace entry point"
    ref, _ = oracle.decode_attention(oracle.Problem.from_case(case))
    got = out_na.double().cpu().numpy()
    err = got - ref
    max_abs, rel = float(np.abs(err).max()), float(np.linalg.norm(err) / np.linalg.norm(ref))
    tol_abs, tol_rel = TOL[case.kv_dtype]
    print(f"[{name}] bitwise equal; oracle max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert max_abs <= tol_abs and rel <= tol_rel


PAIRS = [
    # (first call, second smaller call): 16-head kernel E4M3 with pieces, then f16 (fp32 rows)
    ("g8_fp8_then_f16",
     dict(batch=4, hq=16, hkv=2, d=128, seq_lens=[3000, 700, 64, 1500], kv="fp8_e4m3", scale="token_head",
          block_size=64), 0,
     dict(batch=2, hq=4, hkv=1, d=64, seq_lens=[200, 33], kv="f16", q="f16", scale="none", block_size=32), 5),
    # wide-group kernel (128 heads on one kv head), then a window of 3 query tokens on INT8
    ("wide_then_window_i8",
     dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[4000, 900], kv="fp8_e4m3", scale="tensor",
          block_size=64), 0,
     dict(batch=2, hq=8, hkv=2, d=128, seq_lens=[300, 40], kv="int8", scale="token_head", block_size=16,
          nq=3), 3),
]


@pytest.mark.parametrize("name,first,p1,second,p2", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_equals_workspace_entry_point_on_two_calls(name, first, p1, second, p2):
    kw1 = dict(q="bf16", **first) if "q" not in first else first
    kw2 = dict(q="bf16", **second) if "q" not in second else second
    _run_both(f"{name}/1", workloads.custom_case(seed=21, device="cuda", **kw1), p1)
    _run_both(f"{name}/2", workloads.custom_case(seed=22, device="cuda", **kw2), p2)


def test_noalloc_oversized_step_rejected_without_writing():
    case = workloads.custom_case(seed=2, device="cuda", batch=2, hq=8, hkv=2, d=128, seq_lens=[60000, 10],
                                 kv="fp8_e4m3", q="bf16", scale="token_head", block_size=64)
    big = 100000
    assert fd.workspace_bytes(case.batch, case.hq, case.hkv, case.d, case.max_seq_len, 64, "fp8_e4m3",
                              big) > fd.FD_SCRATCH_BYTES
    out = torch.full(tuple(case.q.shape), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full(tuple(case.q.shape[:-1]), 7.0, dtype=torch.float32, device="cuda")
    head, np_ = _args(case, out, lse, big)
    st = fd.decode_attention_noalloc_raw(case.q.data_ptr(), 1, *head, np_, torch.cuda.current_stream().cuda_stream)
    assert st == fd.FD_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())
