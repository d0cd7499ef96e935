"""Seeded random shapes against the oracle: KV dtype, head_dim, kv heads, group, window length,
batch, per-sequence lengths (empty, single-token, short, long), paged (16/32/64-token pages) or
contiguous, q dtype, scale mode and partition count are drawn per case from a fixed seed, so the
set is the same on every run.  Complements the hand-picked shapes with combinations no single
test names; every draw is a valid input.  out, lse and the workspace sit between guard bytes that
must be unchanged after every call.  A second set draws only wide groups (32 to 256 heads per kv
head, head_dim 128), the shapes of the wide-group and 32-column kernels, windows included."""
import random

import numpy as np
import pytest
import torch

import decode_attention_06_amd as fd
import oracle
import workloads

pytestmark = pytest.mark.gpu

N_CASES = 120


def draw(rng: random.Random):
    kv = rng.choice(["fp8_e4m3", "int8", "f16", "bf16"])
    d = rng.choice([64, 128])
    hkv = rng.choice([1, 2, 4, 8])
    g = rng.choice([1, 2, 4, 8, 16, 32] + ([64, 128] if d == 128 else []))
    nq = rng.choice([1, 1, 1, 2, 4])
    if g * nq > 256:
        nq = 1
    batch = rng.choice([1, 2, 3, 5, 9, 17])
    lens = [rng.choice([0, 1, rng.randint(1, 70), rng.randint(1, 700), rng.randint(1, 3000)]) for _ in range(batch)]
    if max(lens) == 0:
        lens[0] = 5
    paged = rng.random() < 0.8
    return dict(batch=batch, hq=hkv * g, hkv=hkv, d=d, seq_lens=lens, kv=kv,
                q="f16" if kv == "f16" else ("bf16" if kv == "bf16" else rng.choice(["bf16", "f16"])),
                scale="none" if kv in ("f16", "bf16") else rng.choice(["tensor", "token_head"]),
                paged=paged, block_size=rng.choice([16, 32, 64]) if paged else 0, nq=nq), \
        rng.choice([0, 0, 1, 2, 3, 7, 50, 100000])


CASES = []
_rng = random.Random(20261203)
for _i in range(N_CASES):
    CASES.append(draw(_rng))

N_WIDE = 48


def draw_wide(rng: random.Random):
    kv = rng.choice(["fp8_e4m3", "int8", "f16", "bf16"])
    hkv = rng.choice([1, 1, 2])
    g = rng.choice([32, 64, 96, 128, 192, 256] if kv in ("fp8_e4m3", "int8") else [128, 256])
    nq = rng.choice([1, 1, 2, 3, 4])
    batch = rng.choice([1, 2, 3, 5])
    lens = [rng.choice([0, 1, 2, rng.randint(1, 70), rng.randint(1, 700), rng.randint(1, 4000)])
            for _ in range(batch)]
    if max(lens) == 0:
        lens[0] = 5
    paged = rng.random() < 0.8
    return dict(batch=batch, hq=hkv * g, hkv=hkv, d=128, seq_lens=lens, kv=kv,
                q="f16" if kv == "f16" else ("bf16" if kv == "bf16" else rng.choice(["bf16", "f16"])),
                scale="none" if kv in ("f16", "bf16") else rng.choice(["tensor", "token_head"]),
                paged=paged, block_size=rng.choice([16, 32, 64]) if paged else 0, nq=nq), \
        rng.choice([0, 0, 1, 3, 50, 100000])


WIDE_CASES = []
_rng_w = random.Random(20261204)
for _i in range(N_WIDE):
    WIDE_CASES.append(draw_wide(_rng_w))


GUARD = 4096  # guard bytes on each side of out, lse and the workspace
GUARD_BYTE = 0xA5


def guarded(nbytes):
    """A uint8 GPU buffer of nbytes between two guard regions of GUARD bytes filled with
    GUARD_BYTE; returns (whole buffer, interior view).  The interior starts 4 KB in, so it keeps
    the 256-byte alignment the workspace needs."""
    whole = torch.full((GUARD + nbytes + GUARD,), GUARD_BYTE, dtype=torch.uint8, device="cuda")
    return whole, whole[GUARD:GUARD + nbytes]


def guards_intact(whole):
    g = torch.cat([whole[:GUARD], whole[-GUARD:]])
    return bool((g == GUARD_BYTE).all())


@pytest.mark.parametrize("idx", range(N_CASES))
def test_random_shape(idx):
    kw, parts = CASES[idx]
    print(f"[random {idx}] {kw} partitions={parts}", flush=True)
    run_case(kw, parts, seed=5000 + idx)


@pytest.mark.parametrize("idx", range(N_WIDE))
def test_random_wide_shape(idx):
    kw, parts = WIDE_CASES[idx]
    print(f"[random wide {idx}] {kw} partitions={parts}", flush=True)
    run_case(kw, parts, seed=7000 + idx)


def run_case(kw, parts, seed):
    case = workloads.custom_case(seed=seed, device="cuda", **kw)
    # out, lse and the workspace sit between guard bytes: no kernel may write outside them
    q_shape = tuple(case.q.shape)
    n_out, n_lse = int(np.prod(q_shape)), int(np.prod(q_shape[:-1]))
    out_whole, out_bytes = guarded(4 * n_out)
    lse_whole, lse_bytes = guarded(4 * n_lse)
    need = fd.workspace_bytes(case.batch, case.hq, case.hkv, case.d, case.max_seq_len, case.block_size,
                              case.kv_dtype, parts, case.nq)
    ws_whole, ws = guarded(need)
    out = out_bytes.view(torch.float32).view(q_shape)
    lse = lse_bytes.view(torch.float32).view(q_shape[:-1])
    fd.decode_case(case, out=out, lse=lse, workspace=ws, num_partitions=parts)
    torch.cuda.synchronize()
    assert guards_intact(out_whole), "write outside out"
    assert guards_intact(lse_whole), "write outside lse"
    assert guards_intact(ws_whole), "write outside the workspace"
    ref, _ = oracle.decode_attention(oracle.Problem.from_case(case))
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    err = got - ref
    max_abs = float(np.abs(err).max())
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    tol_abs, tol_rel = (2e-3, 1e-3) if kw["kv"] in ("f16", "bf16") else (5e-3, 3e-3)
    assert max_abs <= tol_abs and rel <= tol_rel, (max_abs, rel)
