"""Any finite softmax_scale is a valid input: zero (every weight equal: the mean of V), negative
(the ranking of the scores reversed) and large (a near one-hot softmax), on every partition
kernel and KV type, against the oracle.  Large negative scales with large K are the hard case
for a kernel that takes a tile's maximum on unscaled scores: its multiplier must stay >= 0, so a
negative one flips q instead."""
import math

import numpy as np
import pytest
import torch

import decode_attention_06_amd as fd
import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"f16": (2e-3, 1e-3), "bf16": (2e-3, 1e-3), "fp8_e4m3": (5e-3, 3e-3), "int8": (5e-3, 3e-3)}

KERNELS = [
    # name, kwargs for workloads.custom_case
    ("g8_fp8_tok", dict(batch=2, hq=16, hkv=2, d=128, seq_lens=[700, 40], kv="fp8_e4m3", q="bf16",
                        scale="token_head", block_size=64)),
    ("g8_bf16", dict(batch=2, hq=16, hkv=2, d=128, seq_lens=[700, 40], kv="bf16", q="bf16",
                     scale="none", block_size=32)),
    ("wide_g128_fp8_tensor", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[900, 33], kv="fp8_e4m3",
                                  q="bf16", scale="tensor", block_size=64)),
    ("wide_g128_i8_tok", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[900, 33], kv="int8", q="bf16",
                              scale="token_head", block_size=32)),
    ("wide_g128_bf16", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[900, 33], kv="bf16", q="bf16",
                            scale="none", block_size=64)),
    ("wide_g128_f16", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[900, 33], kv="f16", q="f16",
                           scale="none", block_size=16)),
    ("direct_g8_nq4_fp8_tok", dict(batch=2, hq=16, hkv=2, d=128, seq_lens=[700, 40], nq=4,
                                   kv="fp8_e4m3", q="bf16", scale="token_head", block_size=32)),
    ("direct_g32_fp8_tensor", dict(batch=2, hq=64, hkv=2, d=128, seq_lens=[700, 40], kv="fp8_e4m3",
                                   q="f16", scale="tensor", block_size=64)),
    ("g8_i8_tensor_f16q", dict(batch=2, hq=16, hkv=2, d=128, seq_lens=[700, 40], kv="int8", q="f16",
                               scale="tensor", block_size=16)),
]
# (multiple of 1/sqrt(head_dim), K source magnitude): at 8 x 4 the scaled scores of a tile span
# ~2^200 in base 2, past fp32's range for weights taken against anything but the tile's true max;
# the near one-hot softmax there sits within the bar (its output error is the f16 rounding of the
# winning weights and of the partial rows)
SCALES = [(0.0, 1.0), (-1.0, 1.0), (8.0, 1.0), (-8.0, 1.0), (8.0, 4.0), (-8.0, 4.0)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    fd.lib()
    yield


@pytest.mark.parametrize("mult,k_mag", SCALES, ids=[f"s{m:g}_k{k:g}" for m, k in SCALES])
@pytest.mark.parametrize("name,kw", KERNELS, ids=[k[0] for k in KERNELS])
def test_softmax_scale_values(name, kw, mult, k_mag):
    case = workloads.custom_case(seed=51, device="cuda", k_mag=k_mag, **kw)
    case.softmax_scale = mult / math.sqrt(case.d)
    print(f"[{name}] softmax_scale={case.softmax_scale:.4g} k_mag={k_mag}", flush=True)
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
    lse_err = float(np.max(np.abs(lg[fin] - ref_lse[fin]) / np.maximum(1.0, np.abs(ref_lse[fin]))))
    print(f"[{name}] max_abs={max_abs:.3e} rel_l2={rel_l2:.3e} lse_err={lse_err:.2e}", flush=True)
    assert max_abs <= tol_abs and rel_l2 <= tol_rel, f"{name}: max_abs={max_abs:.3e} rel_l2={rel_l2:.3e}"
    assert lse_err < 1e-4, f"{name}: lse error {lse_err:.2e}"
