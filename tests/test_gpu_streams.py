"""Calls on different streams with their own outputs and workspaces may overlap: four different
steps (the 16-head, wide-group and 32-column kernels; E4M3, INT8 and bf16 KV) issued three times
each on four streams of default priority, with no synchronisation between them, must each equal
the same step run alone, bitwise (outputs and lse).  Nothing in the library may be shared between
concurrent calls."""
import pytest
import torch

import decode_attention_06_amd as fd
import workloads

pytestmark = pytest.mark.gpu

CASES = [
    dict(seed=41, batch=3, hq=64, hkv=8, d=128, seq_lens=[3000, 700, 65], kv="fp8_e4m3", q="bf16",
         scale="token_head", block_size=64),
    dict(seed=42, batch=2, hq=128, hkv=1, d=128, seq_lens=[4000, 900], kv="int8", q="bf16",
         scale="tensor", block_size=32),
    dict(seed=43, batch=4, hq=32, hkv=8, d=128, seq_lens=[1000, 1, 0, 2500], kv="bf16", q="bf16",
         scale="none", paged=False, block_size=0),
    dict(seed=44, batch=2, hq=16, hkv=2, d=128, seq_lens=[1500, 300], nq=4, kv="fp8_e4m3", q="bf16",
         scale="token_head", block_size=16),
]
REPEATS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    fd.lib()
    yield


def _lse_like(case):
    return torch.empty(tuple(case.q.shape[:-1]), dtype=torch.float32, device="cuda")


def test_concurrent_streams_bitwise():
    cases = []
    for kw in CASES:
        kw = dict(kw)
        cases.append(workloads.custom_case(device="cuda", seed=kw.pop("seed"), **kw))
    # each step alone
    refs = []
    for c in cases:
        lse = _lse_like(c)
        out = fd.decode_case(c, lse=lse)
        torch.cuda.synchronize()
        refs.append((out, lse))
    # all of them at once: own stream, workspace and outputs per step
    wss = [torch.empty(fd.workspace_bytes(c.batch, c.hq, c.hkv, c.d, c.max_seq_len, c.block_size,
                                          c.kv_dtype, 0, c.nq), dtype=torch.uint8, device="cuda")
           for c in cases]
    outs = [[torch.empty_like(r[0]) for _ in range(REPEATS)] for r in refs]
    lses = [[torch.empty_like(r[1]) for _ in range(REPEATS)] for r in refs]
    streams = [torch.cuda.Stream(device="cuda") for _ in cases]
    torch.cuda.synchronize()
    for rep in range(REPEATS):
        for i, (c, s) in enumerate(zip(cases, streams)):
            with torch.cuda.stream(s):
                fd.decode_case(c, out=outs[i][rep], lse=lses[i][rep], workspace=wss[i])
    torch.cuda.synchronize()
    for i, (out, lse) in enumerate(refs):
        for rep in range(REPEATS):
            assert torch.equal(outs[i][rep], out), f"step {i} repeat {rep}: output differs"
            assert torch.equal(torch.nan_to_num(lses[i][rep], neginf=-1e30),
                               torch.nan_to_num(lse, neginf=-1e30)), f"step {i} repeat {rep}: lse differs"
    print(f"[streams] {len(cases)} steps x {REPEATS} on {len(streams)} streams: bitwise equal", flush=True)
