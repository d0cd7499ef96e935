"""Per-(token, kv head) scales are caller data: any finite value is valid, zero and negative
included.  Scales of E4M3 and INT8 caches are rewritten so that a fifth of the rows have zero k
and/or v scales, a fifth have negated ones, and whole 32-token tiles have zero v scales (a tile
whose weights all vanish), on the 16-head, wide-group and 32-column kernels, against the oracle.
"""
import numpy as np
import pytest
import torch

import decode_attention_06_amd as fd
import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"fp8_e4m3": (5e-3, 3e-3), "int8": (5e-3, 3e-3)}

KERNELS = [
    ("g8_fp8", dict(batch=3, hq=16, hkv=2, d=128, seq_lens=[900, 70, 5], kv="fp8_e4m3", q="bf16",
                    block_size=64)),
    ("g8_i8_bs16", dict(batch=3, hq=16, hkv=2, d=128, seq_lens=[900, 70, 5], kv="int8", q="f16",
                        block_size=16)),
    ("wide_g128_fp8", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[1100, 40], kv="fp8_e4m3",
                           q="bf16", block_size=32)),
    ("wide_g64_i8", dict(batch=2, hq=64, hkv=1, d=128, seq_lens=[1100, 40], kv="int8", q="bf16",
                         block_size=64)),
    ("direct_g8_nq4_fp8", dict(batch=2, hq=16, hkv=2, d=128, seq_lens=[900, 70], nq=4, kv="fp8_e4m3",
                               q="bf16", block_size=32)),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    fd.lib()
    yield


def _rewrite(scale, rng, zero_tiles):
    """Zero a fifth of the entries, negate another fifth; with zero_tiles, also zero every row
    of tokens 32..63 and 256..287 of the cache rows (a whole tile of the sequences that own them)."""
    flat = scale.reshape(-1, scale.shape[-1]).clone()
    n = flat.shape[0]
    pick = torch.from_numpy(rng.random(n)).to(flat.device)
    flat[pick < 0.2] = 0.0
    flat[(pick >= 0.2) & (pick < 0.4)] *= -1.0
    if zero_tiles:
        flat[32:64] = 0.0
        flat[256:288] = 0.0
    return flat.reshape(scale.shape)


@pytest.mark.parametrize("name,kw", KERNELS, ids=[k[0] for k in KERNELS])
def test_zero_and_negative_token_scales(name, kw):
    case = workloads.custom_case(seed=61, device="cuda", scale="token_head", **kw)
    rng = np.random.default_rng(61)
    case.k_scale = _rewrite(case.k_scale, rng, zero_tiles=False)
    case.v_scale = _rewrite(case.v_scale, rng, zero_tiles=True)
    print(f"[{name}] lens={case.seq_lens} G={case.group} nq={case.nq} kv={case.kv_dtype}", flush=True)
    lse = torch.empty(tuple(case.q.shape[:-1]), dtype=torch.float32, device="cuda")
    out = fd.decode_case(case, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode_attention(oracle.Problem.from_case(case))
    got = out.double().cpu().numpy()
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = got - ref
    max_abs = float(np.max(np.abs(err)))
    rel_l2 = float(np.linalg.norm(err) / np.linalg.norm(ref))
    tol_abs, tol_rel = TOL[case.kv_dtype]
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lg)), f"{name}: lse finiteness differs"
    lse_err = float(np.max(np.abs(lg[fin] - ref_lse[fin]))) if fin.any() else 0.0
    print(f"[{name}] max_abs={max_abs:.3e} rel_l2={rel_l2:.3e} lse_err={lse_err:.2e}", flush=True)
    assert max_abs <= tol_abs and rel_l2 <= tol_rel, f"{name}: max_abs={max_abs:.3e} rel_l2={rel_l2:.3e}"
    assert lse_err < 1e-3, f"{name}: lse error {lse_err:.2e}"
