"""fd_check_inputs on the GPU: the debug validation of the step's device-side contract reports
nothing for valid inputs (unused table entries hold -1 in every workload) and names the first
offending sequence, what is wrong and the value for broken ones.  The validator reads only
seq_len, the used entries inside each table row and kv_start, so the broken inputs below are
safe to hand it; no decode step is run on them."""
import pytest
import torch

import decode_attention_06_amd as fd
import workloads

pytestmark = pytest.mark.gpu


def paged_case(bs=64):
    return workloads.custom_case(seed=3, device="cuda", batch=4, hq=8, hkv=2, d=128,
                                 seq_lens=[700, 0, 129, 64], kv="fp8_e4m3", q="bf16",
                                 scale="token_head", block_size=bs)


def check(case, **kw):
    seq_len = kw.pop("seq_len", case.seq_len)
    table = kw.pop("block_table", case.block_table)
    kv_start = kw.pop("kv_start", case.kv_start)
    result = kw.pop("result", None)
    assert not kw
    extent = case.k_cache.shape[0]
    print(f"[check] {case.name} bs={case.block_size} extent={extent}", flush=True)
    return fd.check_inputs(seq_len, max_seq_len=case.max_seq_len, extent=extent, block_table=table,
                           kv_start=kv_start, block_size=case.block_size if case.paged else 0,
                           result=result)


@pytest.mark.parametrize("bs", [16, 32, 64])
def test_valid_paged_inputs_pass(bs):
    case = paged_case(bs)
    assert (case.block_table < 0).any()          # unused entries are poisoned and must not count
    r = check(case)
    assert r == {"violations": 0, "first_sequence": -1, "kind": "none", "value": 0}


def test_valid_contiguous_inputs_pass():
    case = workloads.custom_case(seed=4, device="cuda", batch=3, hq=8, hkv=2, d=64, seq_lens=[40, 1, 129],
                                 kv="f16", q="f16", scale="none", paged=False, block_size=0)
    assert check(case)["violations"] == 0


def test_workloads_pass():
    for name in ("tiny_mqa_f16", "gqa_bf16"):
        case = workloads.make_case(name, device="cuda")
        assert check(case)["violations"] == 0, name


def test_seq_len_out_of_range():
    case = paged_case()
    sl = case.seq_len.clone()
    sl[2] = case.max_seq_len + 1
    r = check(case, seq_len=sl)
    assert r == {"violations": 1, "first_sequence": 2, "kind": "seq_len", "value": case.max_seq_len + 1}
    sl = case.seq_len.clone()
    sl[3] = -3
    sl[1] = case.max_seq_len + 5
    r = check(case, seq_len=sl)
    assert r == {"violations": 2, "first_sequence": 1, "kind": "seq_len", "value": case.max_seq_len + 5}


def test_used_table_entry_out_of_range():
    case = paged_case()
    nb = case.k_cache.shape[0]
    t = case.block_table.clone()
    t[2, 2] = nb                                 # logical block 2 of a 129-token sequence: used
    r = check(case, block_table=t)
    assert r == {"violations": 1, "first_sequence": 2, "kind": "block_table", "value": nb}
    t[0, 5] = -7                                 # and one of sequence 0
    t[0, 9] = nb + 3                             # a later entry of the same sequence
    r = check(case, block_table=t)
    assert r == {"violations": 2, "first_sequence": 0, "kind": "block_table", "value": -7}


def test_unused_table_entries_are_not_read():
    case = paged_case()
    t = case.block_table.clone()
    t[3, 1:] = 1 << 30                           # 64 tokens use logical block 0 only
    t[1, :] = -1                                 # empty sequence: no entry used
    assert check(case, block_table=t)["violations"] == 0


def test_contiguous_rows_out_of_range():
    case = workloads.custom_case(seed=4, device="cuda", batch=3, hq=8, hkv=2, d=64, seq_lens=[40, 1, 129],
                                 kv="f16", q="f16", scale="none", paged=False, block_size=0)
    rows = case.k_cache.shape[0]
    ks = case.kv_start.clone()
    ks[1] = rows                                 # one row past the end
    r = check(case, kv_start=ks)
    assert r == {"violations": 1, "first_sequence": 1, "kind": "kv_start", "value": rows}
    ks = case.kv_start.clone()
    ks[0] = -1
    r = check(case, kv_start=ks)
    assert r == {"violations": 1, "first_sequence": 0, "kind": "kv_start", "value": -1}


def test_result_rewritten_on_every_call():
    case = paged_case()
    res = torch.full((4,), 12345, dtype=torch.int32, device="cuda")
    sl = case.seq_len.clone()
    sl[0] = -1
    assert check(case, seq_len=sl, result=res)["violations"] == 1
    # the same buffer again: the previous verdict is overwritten, not accumulated
    assert check(case, result=res) == {"violations": 0, "first_sequence": -1, "kind": "none", "value": 0}


def test_debug_mode_rejects_a_broken_contract_before_launching(monkeypatch):
    # FD_CHECK=1: the step validates first, synchronises, and refuses a broken contract with
    # FD_ERR_CONTRACT without launching.  The first broken input (seq_len past max_seq_len) is one
    # the kernels would clamp safely anyway: it proves the mode is on before the second one (a -1
    # table entry in a used position, never safe to launch on) is handed over.
    case = paged_case()
    out_plain = fd.decode_case(case).clone()
    monkeypatch.setenv("FD_CHECK", "1")
    out_checked = fd.decode_case(case)
    torch.cuda.synchronize()
    assert torch.equal(out_plain, out_checked)   # a valid step is unchanged
    sl = case.seq_len.clone()
    sl[2] = case.max_seq_len + 1
    good_sl = case.seq_len
    case.seq_len = sl
    with pytest.raises(fd.FdError) as e:
        fd.decode_case(case)
    assert e.value.status == fd.FD_ERR_CONTRACT
    case.seq_len = good_sl
    t = case.block_table.clone()
    t[0, 3] = -1                                 # used by the 700-token sequence
    good_t = case.block_table
    case.block_table = t
    with pytest.raises(fd.FdError) as e:
        fd.decode_case(case)
    assert e.value.status == fd.FD_ERR_CONTRACT
    case.block_table = good_t
    assert torch.equal(fd.decode_case(case), out_plain)
