"""Pins of the oracle's window of query tokens per sequence (CPU).

Reading (the pages give the window -- several query rows per block, a verify pass over a window
of draft tokens -- but not its mask): the window's nq tokens are the last nq tokens already in
the cache, so query row m sits at position seq_len - nq + m and attends to tokens
[0, seq_len - nq + m]; a row whose range is empty gives out = 0, lse = -inf.  Pinned against a
pure-Python brute force on dense logical data (tests/bruteforce.py) and against reductions to
the single-token step.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from bruteforce import attention_window
from dense_cases import Dense

WINDOW_SHAPES = [
    # seed, lens, nq, hq, hkv, d, kv, q, scale, bs
    (0, [5, 9, 17], 4, 4, 2, 8, "fp8_e4m3", "bf16", "token_head", 4),
    (1, [3, 33], 5, 6, 3, 16, "int8", "f16", "tensor", 8),   # 3 < 5: rows 0, 1 of seq 0 empty
    (2, [12, 2, 7], 3, 4, 1, 8, "bf16", "bf16", "none", 4),
    (3, [16, 40], 16, 2, 2, 8, "f16", "f16", "none", 8),     # the window is the whole of seq 0
]


def _window_q(seed, batch, nq, hq, d, qd):
    g = torch.Generator().manual_seed(1000 + seed)
    return torch.randn(batch, nq, hq, d, generator=g).to({"f16": torch.float16, "bf16": torch.bfloat16}[qd])


def _case(shape, paged=True):
    seed, lens, nq, hq, hkv, d, kv, qd, scale, bs = shape
    dn = Dense(seed, lens, hq, hkv, d, kv=kv, q=qd, scale=scale)
    kw = dn.paged(bs, seed=seed + 10) if paged else dn.contiguous()
    qw = _window_q(seed, len(lens), nq, hq, d, qd)
    kw.update(q=qw, nq=nq)
    return dn, kw, qw


@pytest.mark.parametrize("paged", [True, False])
@pytest.mark.parametrize("shape", WINDOW_SHAPES, ids=lambda s: f"seed{s[0]}-nq{s[2]}-{s[6]}")
def test_window_vs_bruteforce(shape, paged):
    dn, kw, qw = _case(shape, paged)
    out, lse = oracle.decode_attention(oracle.Problem(**kw), nthreads=2)
    _, K, V = dn.dense_values()
    bo, bl = attention_window(qw.to(torch.float64), K, V, 1.0 / math.sqrt(shape[5]))
    assert out.shape == (len(shape[1]), shape[2], shape[3], shape[5])
    np.testing.assert_allclose(out, np.array(bo), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, np.array(bl), rtol=1e-12, atol=1e-13)


def test_window_of_one_is_the_decode_step():
    dn, kw, _ = _case(WINDOW_SHAPES[0])
    one = dict(kw, q=dn.q.unsqueeze(1), nq=1)
    plain = dict(kw, q=dn.q)
    plain.pop("nq")
    o1, l1 = oracle.decode_attention(oracle.Problem(**one), nthreads=1)
    o0, l0 = oracle.decode_attention(oracle.Problem(**plain), nthreads=1)
    assert np.array_equal(o1, o0) and np.array_equal(l1, l0)


@pytest.mark.parametrize("shape", WINDOW_SHAPES[:3], ids=lambda s: f"seed{s[0]}")
def test_row_m_is_the_decode_step_of_its_prefix(shape):
    seed, lens, nq = shape[0], shape[1], shape[2]
    _, kw, qw = _case(shape)
    out, lse = oracle.decode_attention(oracle.Problem(**kw), nthreads=1)
    for m in range(nq):
        pre = [max(0, n - nq + m + 1) for n in lens]
        single = dict(kw, q=qw[:, m].contiguous(), nq=1, seq_len=torch.tensor(pre, dtype=torch.int32))
        o, l_ = oracle.decode_attention(oracle.Problem(**single), nthreads=1)
        assert np.array_equal(out[:, m], o) and np.array_equal(lse[:, m], l_), f"row {m}"


def test_rows_before_the_cache_are_empty():
    shape = WINDOW_SHAPES[1]  # seq 0 has 3 tokens, window of 5
    _, kw, _ = _case(shape)
    out, lse = oracle.decode_attention(oracle.Problem(**kw), nthreads=1)
    assert np.all(out[0, :2] == 0.0) and np.all(np.isneginf(lse[0, :2]))
    assert np.all(np.isfinite(lse[0, 2:])) and np.all(np.isfinite(lse[1]))


def test_rows_differ_only_by_their_prefix():
    # with identical query rows, row m and row m+1 differ exactly by one more token
    shape = WINDOW_SHAPES[0]
    _, kw, qw = _case(shape)
    same = qw[:, :1].expand(-1, shape[2], -1, -1).contiguous()
    out, lse = oracle.decode_attention(oracle.Problem(**dict(kw, q=same)), nthreads=1)
    assert not np.array_equal(out[:, 0], out[:, 1])
    assert np.all(lse[:, 1:] > lse[:, :-1])  # one more positive term in the sum of exp
