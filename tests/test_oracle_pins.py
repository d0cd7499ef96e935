"""Pins of the fp64 oracle against things other than itself (no GPU needed).

* element decoders: exhaustive against library conversions and the OCP spot values;
* attention: hand-worked closed forms, pure-Python brute force on tiny dense inputs, and the
  library routine torch SDPA in float64;
* invariants the definition fixes: uniform scores -> mean of V, one token -> its V row, a split
  and log-sum-exp merge equals the unsplit result, block placement / paged vs contiguous /
  GQA vs replicated-KV MHA / scaling of V, huge scores stay finite, empty sequences.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from bruteforce import attention as brute_attention
from dense_cases import Dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- element decoders
def test_e4m3_exhaustive_vs_torch():
    allb = torch.arange(256, dtype=torch.uint8)
    ref = allb.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.e4m3_to_double(i) for i in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(mine[ok]))


def test_e4m3_spec_spot_values():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "e4m3_spot_values.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for hx, val in rows:
        got = oracle.e4m3_to_double(int(hx, 16))
        if val == "nan":
            assert math.isnan(got), hx
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), hx


def test_f16_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    mine = np.array([oracle.f16_to_double(int(b)) for b in bits])
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])


def test_bf16_exhaustive_vs_torch():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    mine = np.array([oracle.bf16_to_double(int(b) & 0xFFFF) for b in bits.tolist()])
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])


# ---------------------------------------------------------------- hand-worked closed forms
def _problem_from_rows(q, K, V, scale, kv="bf16"):
    d = len(q)
    n = len(K)
    qt = torch.tensor([[q]], dtype=torch.bfloat16)
    Kt = torch.tensor(K, dtype=torch.bfloat16).view(n, 1, d)
    Vt = torch.tensor(V, dtype=torch.bfloat16).view(n, 1, d)
    return oracle.Problem(q=qt, k_cache=Kt, v_cache=Vt, seq_len=torch.tensor([n], dtype=torch.int32),
                          batch=1, hq=1, hkv=1, d=d, q_dtype="bf16", kv_dtype=kv,
                          kv_start=torch.tensor([0], dtype=torch.int32), softmax_scale=scale)


def test_handworked_cases():
    cases = json.load(open(os.path.join(GOLDEN, "handworked_attention.json")))["cases"]
    assert len(cases) >= 4
    for c in cases:
        p = _problem_from_rows(c["q"], c["K"], c["V"], c["scale"])
        out, lse = oracle.decode_attention(p, nthreads=1)
        np.testing.assert_allclose(out[0, 0], c["out"], rtol=0, atol=1e-13, err_msg=c["name"])
        assert abs(lse[0, 0] - c["lse"]) < 1e-13, c["name"]


# ---------------------------------------------------------------- brute force and SDPA
BRUTE_SHAPES = [
    # seed, lens, hq, hkv, d, kv, q, scale, bs
    (0, [5, 1, 17], 4, 2, 8, "fp8_e4m3", "bf16", "token_head", 4),
    (1, [9, 33], 6, 3, 16, "fp8_e4m3", "bf16", "tensor", 8),
    (2, [12, 7], 4, 1, 8, "bf16", "bf16", "none", 4),
    (3, [3, 20, 1], 2, 2, 8, "f16", "f16", "none", 8),
    (4, [40], 8, 1, 64, "fp8_e4m3", "f16", "token_head", 32),
    (5, [7, 30], 4, 2, 16, "int8", "bf16", "token_head", 8),
    (6, [13, 2], 2, 1, 8, "int8", "f16", "tensor", 4),
]


@pytest.mark.parametrize("shape", BRUTE_SHAPES, ids=lambda s: f"seed{s[0]}-{s[5]}-{s[7]}")
def test_oracle_vs_bruteforce_paged(shape):
    seed, lens, hq, hkv, d, kv, qd, scale, bs = shape
    dn = Dense(seed, lens, hq, hkv, d, kv=kv, q=qd, scale=scale)
    prob = oracle.Problem(**dn.paged(bs, seed=seed + 10))
    out, lse = oracle.decode_attention(prob, nthreads=2)
    q64, K, V = dn.dense_values()
    bo, bl = brute_attention(q64, K, V, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(out, np.array(bo), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, np.array(bl), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("shape", BRUTE_SHAPES[:3] + BRUTE_SHAPES[5:], ids=lambda s: f"seed{s[0]}")
def test_oracle_vs_bruteforce_contiguous(shape):
    seed, lens, hq, hkv, d, kv, qd, scale, _ = shape
    dn = Dense(seed, lens, hq, hkv, d, kv=kv, q=qd, scale=scale)
    out, lse = oracle.decode_attention(oracle.Problem(**dn.contiguous()), nthreads=1)
    bo, bl = brute_attention(*dn.dense_values(), 1.0 / math.sqrt(d))
    np.testing.assert_allclose(out, np.array(bo), rtol=1e-12, atol=1e-13)


def test_oracle_vs_torch_sdpa_f64():
    """Library routine: torch's scaled_dot_product_attention in float64 with a key padding mask."""
    lens = [30, 64, 1, 45]
    hq, hkv, d = 8, 2, 64
    dn = Dense(7, lens, hq, hkv, d, kv="fp8_e4m3", q="bf16", scale="token_head")
    out, lse = oracle.decode_attention(oracle.Problem(**dn.paged(16, seed=3)), nthreads=2)
    q64, K, V = dn.dense_values()
    nmax = max(lens)
    G = hq // hkv
    for b, n in enumerate(lens):
        Kb = torch.zeros(hq, nmax, d, dtype=torch.float64)
        Vb = torch.zeros(hq, nmax, d, dtype=torch.float64)
        Kb[:, :n] = K[b].permute(1, 0, 2).repeat_interleave(G, dim=0)
        Vb[:, :n] = V[b].permute(1, 0, 2).repeat_interleave(G, dim=0)
        mask = torch.zeros(hq, 1, nmax, dtype=torch.bool)
        mask[:, :, :n] = True
        ref = torch.nn.functional.scaled_dot_product_attention(
            q64[b].unsqueeze(1), Kb, Vb, attn_mask=mask, scale=1.0 / math.sqrt(d))
        np.testing.assert_allclose(out[b], ref[:, 0].numpy(), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- invariants
def test_zero_query_gives_mean_of_v():
    lens = [13, 64, 100]
    dn = Dense(11, lens, 4, 2, 32, kv="fp8_e4m3", scale="token_head")
    dn.q.zero_()
    out, lse = oracle.decode_attention(oracle.Problem(**dn.paged(32)), nthreads=2)
    _, _, V = dn.dense_values()
    for b, n in enumerate(lens):
        mean = V[b].mean(dim=0).numpy()  # [hkv][d]
        for h in range(4):
            np.testing.assert_allclose(out[b, h], mean[h // 2], rtol=1e-13, atol=1e-15)
            assert abs(lse[b, h] - math.log(n)) < 1e-13


def test_single_token_returns_its_v_row_exactly():
    dn = Dense(12, [1, 1], 4, 1, 64, kv="fp8_e4m3", scale="token_head")
    out, _ = oracle.decode_attention(oracle.Problem(**dn.paged(64)), nthreads=1)
    _, _, V = dn.dense_values()
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, h], V[b][0, 0].numpy())


def test_dominant_score_selects_one_row():
    dn = Dense(13, [50], 1, 1, 16, kv="bf16", q="bf16")
    dn.q.zero_()
    dn.q[0, 0, 0] = 64.0
    for t in range(50):
        dn.k[0][t].zero_()
    dn.k[0][21, 0, 0] = 16.0     # score 64*16/4 = 256, every other score 0
    out, _ = oracle.decode_attention(oracle.Problem(**dn.contiguous()), nthreads=1)
    v = dn.v[0][21, 0].to(torch.float64).numpy()
    np.testing.assert_allclose(out[0, 0], v, rtol=1e-15, atol=1e-100 + 1e-60)


@pytest.mark.parametrize("cut", [0, 1, 31, 32, 63, 64, 65, 150, 199, 200])
def test_split_and_merge_equals_unsplit(cut):
    dn = Dense(14, [200], 8, 2, 64, kv="fp8_e4m3", scale="token_head")
    prob = oracle.Problem(**dn.paged(64))
    out, lse = oracle.decode_attention(prob, nthreads=1)
    for h in (0, 5):
        a = oracle.attend_range(prob, 0, h, 0, cut)
        b = oracle.attend_range(prob, 0, h, cut, 200)
        mo, ml = oracle.merge([a[0], b[0]], [a[1], b[1]], np.stack([a[2], b[2]]))
        np.testing.assert_allclose(mo, out[0, h], rtol=1e-13, atol=1e-15)
        assert abs(ml - lse[0, h]) < 1e-12


def test_many_way_split_merge():
    dn = Dense(15, [333], 4, 1, 64, kv="bf16", q="bf16")
    prob = oracle.Problem(**dn.paged(32))
    out, lse = oracle.decode_attention(prob, nthreads=1)
    cuts = [0, 32, 64, 65, 130, 200, 333, 333]
    parts = [oracle.attend_range(prob, 0, 2, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    mo, ml = oracle.merge([p[0] for p in parts], [p[1] for p in parts], np.stack([p[2] for p in parts]))
    np.testing.assert_allclose(mo, out[0, 2], rtol=1e-13, atol=1e-15)


def test_block_placement_is_bitwise_invariant():
    dn = Dense(16, [70, 129, 5], 4, 2, 32, kv="fp8_e4m3", scale="token_head")
    o1, l1 = oracle.decode_attention(oracle.Problem(**dn.paged(32, seed=1)), nthreads=2)
    o2, l2 = oracle.decode_attention(oracle.Problem(**dn.paged(32, seed=99, spare=9)), nthreads=3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_paged_equals_contiguous_bitwise():
    dn = Dense(17, [37, 100], 4, 1, 64, kv="f16", q="f16")
    oc, lc = oracle.decode_attention(oracle.Problem(**dn.contiguous()), nthreads=1)
    for bs in (32, 64):
        op, lp = oracle.decode_attention(oracle.Problem(**dn.paged(bs)), nthreads=1)
        assert np.array_equal(oc, op) and np.array_equal(lc, lp)


def test_gqa_equals_replicated_mha_bitwise():
    dn = Dense(18, [45, 90], 8, 2, 32, kv="fp8_e4m3", scale="token_head")
    og, lg = oracle.decode_attention(oracle.Problem(**dn.paged(32)), nthreads=1)
    rep = Dense(18, [45, 90], 8, 2, 32, kv="fp8_e4m3", scale="token_head")
    rep.hkv = 8
    for b in range(2):
        rep.k[b] = dn.k[b].repeat_interleave(4, dim=1)
        rep.v[b] = dn.v[b].repeat_interleave(4, dim=1)
        rep.ks[b] = dn.ks[b].repeat_interleave(4, dim=1)
        rep.vs[b] = dn.vs[b].repeat_interleave(4, dim=1)
    om, lm = oracle.decode_attention(oracle.Problem(**rep.paged(32)), nthreads=1)
    assert np.array_equal(og, om) and np.array_equal(lg, lm)


def test_token_permutation_invariance():
    dn = Dense(19, [77], 4, 1, 32, kv="bf16", q="bf16")
    o1, _ = oracle.decode_attention(oracle.Problem(**dn.contiguous()), nthreads=1)
    perm = torch.from_numpy(np.random.default_rng(5).permutation(77))
    dn.k[0] = dn.k[0][perm]
    dn.v[0] = dn.v[0][perm]
    o2, _ = oracle.decode_attention(oracle.Problem(**dn.contiguous()), nthreads=1)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)


def test_v_scale_doubling_doubles_output_bitwise():
    dn = Dense(20, [64, 31], 4, 2, 32, kv="fp8_e4m3", scale="token_head")
    o1, l1 = oracle.decode_attention(oracle.Problem(**dn.paged(32)), nthreads=1)
    dn.vs = [s * 2 for s in dn.vs]
    o2, l2 = oracle.decode_attention(oracle.Problem(**dn.paged(32)), nthreads=1)
    assert np.array_equal(o2, 2 * o1) and np.array_equal(l1, l2)


def test_huge_scores_stay_finite():
    dn = Dense(21, [300], 4, 1, 128, kv="fp8_e4m3", scale="token_head", qmul=100.0)
    out, lse = oracle.decode_attention(oracle.Problem(**dn.paged(64)), nthreads=1)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


def test_empty_sequence():
    dn = Dense(22, [0, 10, 0], 4, 1, 32, kv="fp8_e4m3", scale="token_head")
    out, lse = oracle.decode_attention(oracle.Problem(**dn.paged(32)), nthreads=1)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isfinite(lse[1]))


def test_seq_mask_computes_only_selected():
    dn = Dense(23, [10, 20, 30], 2, 1, 16, kv="bf16", q="bf16")
    prob = oracle.Problem(**dn.contiguous())
    full, _ = oracle.decode_attention(prob, nthreads=1)
    part, _ = oracle.decode_attention(prob, seqs=[1], nthreads=1)
    assert np.array_equal(part[1], full[1]) and np.all(np.isnan(part[0]))


@pytest.mark.parametrize("mult", [0.0, -1.0, -6.0, 6.0])
@pytest.mark.parametrize("kv,qd,scale", [("fp8_e4m3", "bf16", "token_head"), ("int8", "f16", "tensor"),
                                         ("bf16", "bf16", "none")])
def test_oracle_vs_bruteforce_any_softmax_scale(kv, qd, scale, mult):
    """Any finite softmax scale: zero (uniform weights), negative (the ranking reversed) and large
    ones, against the literal brute force (which subtracts no maximum)."""
    d = 16
    dn = Dense(33, [19, 40, 1], 4, 2, d, kv=kv, q=qd, scale=scale)
    kw = dn.paged(8, seed=34)
    kw["softmax_scale"] = mult / math.sqrt(d)
    out, lse = oracle.decode_attention(oracle.Problem(**kw), nthreads=2)
    bo, bl = brute_attention(*dn.dense_values(), mult / math.sqrt(d))
    np.testing.assert_allclose(out, np.array(bo), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(bl), rtol=1e-11, atol=1e-12)
