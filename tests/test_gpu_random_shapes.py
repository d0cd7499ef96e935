"""Seeded random shapes against the oracle: KV dtype, head_dim, kv heads, group, window length,
batch, per-sequence lengths (empty, single-token, short, long), paged (16/32/64-token pages) or
contiguous, q dtype, scale mode and partition count are drawn per case from a fixed seed, so the
set is the same on every run.  Complements the hand-picked shapes with combinations no single
test names; every draw is a valid input."""
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


@pytest.mark.parametrize("idx", range(N_CASES))
def test_random_shape(idx):
    kw, parts = CASES[idx]
    print(f"[random {idx}] {kw} partitions={parts}", flush=True)
    case = workloads.custom_case(seed=5000 + idx, device="cuda", **kw)
    out = fd.decode_case(case, num_partitions=parts)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_attention(oracle.Problem.from_case(case))
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    err = got - ref
    max_abs = float(np.abs(err).max())
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    tol_abs, tol_rel = (2e-3, 1e-3) if kw["kv"] in ("f16", "bf16") else (5e-3, 3e-3)
    assert max_abs <= tol_abs and rel <= tol_rel, (max_abs, rel)
