"""The decode step captured once in a HIP graph and replayed (GPU).

A serving loop captures the step's launches once and replays them every token ("第 15 章 · GPU
Profiling 与 LLM 推理优化实战", section 15.20): the library must be capture-safe -- no allocation,
no host synchronisation, no memset nodes, every size and pointer fixed at capture, every value
that changes per step (seq_len, pos, the new token's K/V, q) read from device memory at run time.
Here the append of the new token and the attention over the grown cache are captured together,
then replayed several times with the per-step inputs rewritten between replays (eager copies and
host synchronisations in between); every replay is compared bitwise with the same step run eagerly
on a copy of the cache, and the first one also with the oracle.
"""
import numpy as np
import pytest
import torch

import decode_attention_06_amd as fd
import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    fd.lib()
    yield


def _grown_case(seed, nq, spare_tokens):
    # a batch whose tables have room for `spare_tokens` more tokens per sequence
    lens = [700, 33, 64, 2000]
    case = workloads.custom_case(seed=seed, device="cpu", batch=4, hq=16, hkv=2, d=128, seq_lens=lens,
                                 kv="fp8_e4m3", q="bf16", scale="token_head", block_size=16,
                                 max_seq_len=max(lens) + spare_tokens, nq=nq)
    bt = case.block_table.clone()
    nb = case.k_cache.shape[0]
    used = set(int(x) for x in bt[bt >= 0].tolist())
    spare = [i for i in range(nb) if i not in used]
    need = 0
    for b, n in enumerate(lens):
        for j in range((n + 15) // 16, (n + spare_tokens + 15) // 16):
            need += 1
    # grow the pool so every sequence can take `spare_tokens` more rows
    extra = max(0, need - len(spare))
    if extra:
        pad = torch.full((extra,) + tuple(case.k_cache.shape[1:]), 0x7F, dtype=case.k_cache.dtype)
        case.k_cache = torch.cat([case.k_cache, pad])
        case.v_cache = torch.cat([case.v_cache, pad.clone()])
        spad = torch.full((extra,) + tuple(case.k_scale.shape[1:]), float("nan"))
        case.k_scale = torch.cat([case.k_scale, spad])
        case.v_scale = torch.cat([case.v_scale, spad.clone()])
        spare += list(range(nb, nb + extra))
    for b, n in enumerate(lens):
        for j in range((n + 15) // 16, (n + spare_tokens + 15) // 16):
            bt[b, j] = spare.pop()
    case.block_table = bt
    case.k_scale = torch.nan_to_num(case.k_scale, nan=1.0)
    case.v_scale = torch.nan_to_num(case.v_scale, nan=1.0)
    return case


@pytest.mark.parametrize("nq", [1, 3])
def test_captured_append_and_attend_replays_match_eager(nq):
    steps = 4
    case = _grown_case(seed=60 + nq, nq=nq, spare_tokens=steps * nq + 1)
    dev = "cuda"
    g = torch.Generator().manual_seed(7)
    # per-step inputs, fixed buffers (the graph reads them at replay time)
    k_new_all = torch.randn(steps, nq, case.batch, case.hkv, case.d, generator=g).to(torch.bfloat16)
    v_new_all = torch.randn(steps, nq, case.batch, case.hkv, case.d, generator=g).to(torch.bfloat16)
    q_all = torch.randn((steps,) + tuple(case.q.shape), generator=g).to(torch.bfloat16)
    base = case.seq_len.clone()

    def buffers():
        b = dict(k=case.k_cache.to(dev), v=case.v_cache.to(dev), ks=case.k_scale.to(dev), vs=case.v_scale.to(dev),
                 bt=case.block_table.to(dev), seq=case.seq_len.to(dev).clone(), pos=torch.zeros(case.batch, dtype=torch.int32, device=dev),
                 k_new=torch.empty(case.batch, case.hkv, case.d, dtype=torch.bfloat16, device=dev),
                 v_new=torch.empty(case.batch, case.hkv, case.d, dtype=torch.bfloat16, device=dev),
                 q=torch.empty(tuple(case.q.shape), dtype=torch.bfloat16, device=dev),
                 out=torch.empty(tuple(case.q.shape), dtype=torch.float32, device=dev),
                 lse=torch.empty(tuple(case.q.shape[:-1]), dtype=torch.float32, device=dev))
        nbytes = fd.workspace_bytes(case.batch, case.hq, case.hkv, case.d, case.max_seq_len, 16, "fp8_e4m3", 0, nq)
        b["ws"] = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        return b

    def step_calls(b, stream):
        # the window's nq new tokens are appended one row at a time, then the window attends
        for r in range(nq):
            fd.kv_append(b["k_new_r"][r], b["v_new_r"][r], b["k"], b["v"], b["pos_r"][r], kv_dtype="fp8_e4m3",
                         block_table=b["bt"], block_size=16, scale_mode="token_head", k_scale=b["ks"],
                         v_scale=b["vs"], stream=stream)
        fd.decode_attention(b["q"], b["k"], b["v"], b["seq"], max_seq_len=case.max_seq_len, block_table=b["bt"],
                            kv_dtype="fp8_e4m3", scale_mode="token_head", k_scale=b["ks"], v_scale=b["vs"],
                            softmax_scale=case.softmax_scale, num_kv_heads=case.hkv, block_size=16,
                            out=b["out"], lse=b["lse"], workspace=b["ws"], stream=stream)

    def set_inputs(b, s):
        # step s: rows base + s*nq .. base + s*nq + nq - 1 are appended, seq_len grows by nq
        for r in range(nq):
            b["k_new_r"][r].copy_(k_new_all[s, r])
            b["v_new_r"][r].copy_(v_new_all[s, r])
            b["pos_r"][r].copy_(base + s * nq + r)
        b["seq"].copy_(base + (s + 1) * nq)
        b["q"].copy_(q_all[s])

    def add_row_buffers(b):
        b["k_new_r"] = [torch.empty(case.batch, case.hkv, case.d, dtype=torch.bfloat16, device=dev) for _ in range(nq)]
        b["v_new_r"] = [torch.empty(case.batch, case.hkv, case.d, dtype=torch.bfloat16, device=dev) for _ in range(nq)]
        b["pos_r"] = [torch.empty(case.batch, dtype=torch.int32, device=dev) for _ in range(nq)]

    gb, eb = buffers(), buffers()
    add_row_buffers(gb)
    add_row_buffers(eb)
    # capture (warm the library up on a side stream first, as torch recommends)
    set_inputs(gb, 0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    capture_k, capture_v = gb["k"].clone(), gb["v"].clone()  # the capture itself must not change the cache
    with torch.cuda.graph(graph):
        step_calls(gb, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(gb["k"], capture_k) and torch.equal(gb["v"], capture_v)

    for s in range(steps):
        set_inputs(gb, s)
        set_inputs(eb, s)
        torch.cuda.synchronize()
        graph.replay()
        step_calls(eb, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        print(f"[graph nq={nq}] step {s}: replay vs eager", flush=True)
        assert torch.equal(gb["k"], eb["k"]) and torch.equal(gb["ks"], eb["ks"]), f"step {s}: cache differs"
        assert torch.equal(gb["out"], eb["out"]) and torch.equal(gb["lse"], eb["lse"]), f"step {s}: output differs"
        if s == 0:
            prob = oracle.Problem(q=gb["q"], k_cache=gb["k"], v_cache=gb["v"], seq_len=gb["seq"], batch=case.batch,
                                  hq=case.hq, hkv=case.hkv, d=case.d, q_dtype="bf16", kv_dtype="fp8_e4m3",
                                  scale_mode="token_head", k_scale=gb["ks"], v_scale=gb["vs"],
                                  block_table=gb["bt"], block_size=16, softmax_scale=case.softmax_scale, nq=nq)
            ref, _ = oracle.decode_attention(prob)
            err = np.abs(gb["out"].double().cpu().numpy() - ref).max()
            print(f"[graph nq={nq}] step 0 vs oracle max_abs={err:.3e}", flush=True)
            assert err < 5e-3
