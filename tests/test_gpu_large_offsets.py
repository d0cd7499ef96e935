"""Cache offsets past 4 GiB: the same step with its KV rows (contiguous mode) or blocks (paged
mode) placed beyond 4 GiB of a larger cache, on each partition kernel.

The kernels form every cache address from a 64-bit row or block base; a 32-bit product anywhere
in that arithmetic would wrap at 2^31 or 2^32 bytes.  Two placements: "shift" moves every row or
block past 4 GiB; "split" (paged) keeps a copy of the blocks at the front and maps every second
block of each sequence to the copy past 4 GiB, so consecutive blocks -- and the two halves of a
32-token tile over 16-token pages -- lie more than 4 GiB apart.  The relocated step must equal the
step on the compact cache bitwise (same values, same work split) and match the oracle within the
bar.
Cases: the 16-head kernel (E4M3 with per-token scales, contiguous; bf16 with 16-token pages),
the wide-group kernel (E4M3 per-tensor and INT8 per-token, 128 heads per kv head, paged) and the
32-column kernel (a 4-token window, paged).  Each case allocates about 9 GB of device memory.
"""
import dataclasses

import numpy as np
import pytest
import torch

import decode_attention_06_amd as fd
import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"f16": (2e-3, 1e-3), "bf16": (2e-3, 1e-3), "fp8_e4m3": (5e-3, 3e-3), "int8": (5e-3, 3e-3)}
FOUR_GIB = 4 << 30

CASES = [
    # name, placement, kwargs for workloads.custom_case
    ("g8_fp8_tok_contig", "shift", dict(batch=3, hq=16, hkv=2, d=128, seq_lens=[700, 65, 0],
                                        kv="fp8_e4m3", q="bf16", scale="token_head", paged=False,
                                        block_size=0)),
    ("g8_fp8_tok_bs64", "split", dict(batch=2, hq=16, hkv=2, d=128, seq_lens=[700, 130],
                                      kv="fp8_e4m3", q="bf16", scale="token_head", block_size=64)),
    ("g4_bf16_bs16", "shift", dict(batch=2, hq=8, hkv=2, d=128, seq_lens=[333, 1000], kv="bf16",
                                   q="bf16", scale="none", block_size=16)),
    ("g4_bf16_bs16", "split", dict(batch=2, hq=8, hkv=2, d=128, seq_lens=[333, 1000], kv="bf16",
                                   q="bf16", scale="none", block_size=16)),
    ("wide_g128_fp8_tensor_bs64", "shift", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[2049, 40],
                                                kv="fp8_e4m3", q="bf16", scale="tensor", block_size=64)),
    ("wide_g128_fp8_tok_bs16", "split", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[700, 33],
                                             kv="fp8_e4m3", q="bf16", scale="token_head",
                                             block_size=16)),
    ("wide_g128_i8_tok_bs32", "shift", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[900, 33],
                                            kv="int8", q="bf16", scale="token_head", block_size=32)),
    ("direct_g8_nq4_fp8_tok_bs32", "shift", dict(batch=2, hq=16, hkv=2, d=128, seq_lens=[1000, 70],
                                                 nq=4, kv="fp8_e4m3", q="bf16", scale="token_head",
                                                 block_size=32)),
    ("direct_g8_nq4_fp8_tok_bs16", "split", dict(batch=2, hq=16, hkv=2, d=128, seq_lens=[500, 70],
                                                 nq=4, kv="fp8_e4m3", q="bf16", scale="token_head",
                                                 block_size=16)),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    fd.lib()
    yield


def _relocate(t, lead, keep_front):
    """t with `lead` entries of its first dimension in front: zeros, or a copy of t followed by
    zeros when keep_front."""
    big = torch.zeros((lead + t.shape[0],) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
    big[lead:] = t
    if keep_front:
        big[:t.shape[0]] = t
    return big


def relocated(case, placement):
    """The same step with its rows (contiguous) or blocks (paged) placed past 4 GiB of K cache:
    all of them ("shift"), or every second block of each sequence ("split", paged)."""
    unit_bytes = case.k_cache[0].numel() * case.k_cache.element_size()  # one row or one block
    lead = FOUR_GIB // unit_bytes + 1000
    split = placement == "split"
    assert not split or case.paged
    kw = dict(k_cache=_relocate(case.k_cache, lead, split), v_cache=_relocate(case.v_cache, lead, split))
    if case.scale_mode == "token_head":
        kw.update(k_scale=_relocate(case.k_scale, lead, split), v_scale=_relocate(case.v_scale, lead, split))
    if case.paged:
        table = case.block_table.clone()
        moved = table >= 0
        if split:
            moved &= (torch.arange(table.shape[1], device=table.device) % 2 == 1)[None, :]
        table[moved] += lead
        kw["block_table"] = table
    else:
        kw["kv_start"] = case.kv_start + lead
    big = dataclasses.replace(case, **kw)
    assert lead * unit_bytes > FOUR_GIB and big.k_cache.numel() * big.k_cache.element_size() > FOUR_GIB
    return big


def run(case):
    lse = torch.empty(tuple(case.q.shape[:-1]), dtype=torch.float32, device="cuda")
    out = fd.decode_case(case, lse=lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("name,placement,kw", CASES, ids=[f"{c[0]}-{c[1]}" for c in CASES])
def test_cache_offsets_beyond_4gib(name, placement, kw):
    case = workloads.custom_case(seed=31, device="cuda", **kw)
    print(f"[{name}/{placement}] lens={case.seq_lens} G={case.group} nq={case.nq} kv={case.kv_dtype} "
          f"scale={case.scale_mode} bs={case.block_size}", flush=True)
    out, lse = run(case)
    big = relocated(case, placement)
    out_big, lse_big = run(big)
    assert torch.equal(out_big, out), f"{name}: output changed when the cache moved past 4 GiB"
    assert torch.equal(torch.nan_to_num(lse_big, neginf=-1e30), torch.nan_to_num(lse, neginf=-1e30))
    del big, out_big, lse_big
    torch.cuda.empty_cache()
    ref, _ = oracle.decode_attention(oracle.Problem.from_case(case))
    got = out.double().cpu().numpy()
    err = got - ref
    max_abs = float(np.max(np.abs(err)))
    rel_l2 = float(np.linalg.norm(err) / np.linalg.norm(ref))
    tol_abs, tol_rel = TOL[case.kv_dtype]
    print(f"[{name}] relocated bitwise equal; oracle max_abs={max_abs:.3e} rel_l2={rel_l2:.3e}", flush=True)
    assert max_abs <= tol_abs and rel_l2 <= tol_rel, f"{name}: max_abs={max_abs:.3e} rel_l2={rel_l2:.3e}"
