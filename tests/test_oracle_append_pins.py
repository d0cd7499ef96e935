"""Pins of the oracle's KV-cache append (current token written into its cache row, FP8 row
quantisation) against things other than itself (no GPU needed).

* E4M3 encoder: every code round-trips; all midpoints tie to the even code; saturation;
  agreement with torch's float8_e4m3fn cast (round to nearest even) on random values;
* f16 / bf16 encoders: agreement with numpy's float16 and torch's bfloat16 casts;
* row quantisation: the absmax element maps to +-448, the fp32 scale is amax / 448, the
  dequantisation error stays within half an E4M3 step, zero rows, fixed scales saturate;
* append: only the target rows (and their scales) change, paged and contiguous addressing,
  skipped sequences; a one-token sequence read back through the attention oracle returns the
  dequantised appended V row.
"""
import numpy as np
import pytest
import torch

import oracle

FINITE_CODES = [c for c in range(256) if (c & 0x7F) != 0x7F]


def e4m3_value(c: int) -> float:
    return oracle.e4m3_to_double(c)


# ---------------------------------------------------------------- E4M3 encoder
def test_e4m3_encode_roundtrips_every_finite_code():
    for c in FINITE_CODES:
        assert oracle.e4m3_encode(np.float32(e4m3_value(c))) == c, hex(c)


def test_e4m3_encode_midpoints_tie_to_even_and_neighbours_round_correctly():
    for sign in (0, 0x80):
        for c in range(0, 0x7E):
            lo, hi = e4m3_value(sign | c), e4m3_value(sign | (c + 1))
            mid = np.float32((lo + hi) / 2)          # exact: E4M3 midpoints need 5 bits
            assert float(mid) == (lo + hi) / 2
            even = (sign | c) if c % 2 == 0 else (sign | (c + 1))
            assert oracle.e4m3_encode(mid) == even, (hex(sign | c), float(mid))
            toward_hi = np.nextafter(mid, np.float32(np.inf) if not sign else np.float32(-np.inf))
            toward_lo = np.nextafter(mid, np.float32(0.0))
            assert oracle.e4m3_encode(toward_hi) == sign | (c + 1)
            assert oracle.e4m3_encode(toward_lo) == sign | c


def test_e4m3_encode_saturates_and_keeps_sign():
    for x, code in [(448.0, 0x7E), (448.5, 0x7E), (464.0, 0x7E), (1e6, 0x7E), (np.inf, 0x7E),
                    (-448.0, 0xFE), (-1e30, 0xFE), (-np.inf, 0xFE), (0.0, 0x00), (-0.0, 0x80)]:
        assert oracle.e4m3_encode(np.float32(x)) == code, x
    assert oracle.e4m3_encode(np.float32(np.nan)) == 0x7F


def test_e4m3_encode_matches_torch_round_to_nearest_even():
    g = np.random.default_rng(5)
    mags = np.exp(g.uniform(np.log(2.0 ** -12), np.log(448.0), size=20000)).astype(np.float32)
    x = (mags * g.choice([-1.0, 1.0], size=mags.size)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([oracle.e4m3_encode(v) for v in x], dtype=np.uint8)
    assert np.array_equal(mine, ref)


# ---------------------------------------------------------------- f16 / bf16 encoders
def _edge_floats():
    g = np.random.default_rng(6)
    x = g.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    extra = np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 65519.0, 65520.0, 70000.0, -65520.0,
                      2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26, 1e-30,
                      3.0e38, -3.0e38, 2.0 ** -126, 2.0 ** -133, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9],
                     dtype=np.float32)
    tiny = (g.standard_normal(2000) * 2.0 ** -20).astype(np.float32)
    huge = (g.standard_normal(2000) * 2.0 ** 100).astype(np.float32)
    return np.concatenate([x, extra, tiny, huge])


def test_f16_encode_matches_numpy_cast():
    x = _edge_floats()
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    mine = np.array([oracle.f16_encode(v) for v in x], dtype=np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_encode_matches_torch_cast():
    x = _edge_floats()
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = np.array([oracle.bf16_encode(v) for v in x], dtype=np.uint16)
    assert np.array_equal(mine, ref)


# ---------------------------------------------------------------- row quantisation
@pytest.mark.parametrize("mag", [1e-3, 1.0, 37.0, 1e4])
def test_quantize_row_absmax_maps_to_448_and_scale_is_fp32_amax_over_448(mag):
    g = np.random.default_rng(int(mag * 1000) % 2 ** 31)
    for _ in range(50):
        x = (g.standard_normal(128) * mag).astype(np.float32)
        b, s = oracle.quantize_row_e4m3(x)
        i = int(np.argmax(np.abs(x)))
        assert e4m3_value(int(b[i])) == (448.0 if x[i] > 0 else -448.0)
        assert s == float(np.float32(np.abs(x).max()) / np.float32(448.0))


def test_quantize_row_error_within_half_step():
    g = np.random.default_rng(8)
    for _ in range(200):
        x = (g.standard_normal(128) * g.uniform(0.01, 100)).astype(np.float32)
        b, s = oracle.quantize_row_e4m3(x)
        q = np.array([float(np.float32(v) / np.float32(s)) for v in x])
        dq = np.array([e4m3_value(int(c)) for c in b])
        # half a step of the E4M3 grid at |q|: 2^(floor(log2|q|) - 4) for normals, 2^-10 below 2^-6
        with np.errstate(divide="ignore"):
            half = np.where(np.abs(q) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.abs(q))) - 4), 2.0 ** -10)
        assert np.all(np.abs(dq - q) <= half)


def test_quantize_zero_row_and_fixed_scale():
    b, s = oracle.quantize_row_e4m3(np.zeros(64, np.float32))
    assert s == 1.0 and not b.any()
    x = np.array([0.0, 1.0, -1.0, 10.0, -10.0, 0.25], np.float32)
    b, s = oracle.quantize_row_e4m3(x, scale=0.01)
    assert s == np.float32(0.01)
    assert [e4m3_value(int(c)) for c in b] == [0.0, 96.0, -96.0, 448.0, -448.0, 24.0]


@pytest.mark.parametrize("mag", [1e-3, 1.0, 50.0])
def test_quantize_row_i8_matches_numpy_round_half_even(mag):
    g = np.random.default_rng(int(mag * 100) + 3)
    for _ in range(100):
        x = (g.standard_normal(128) * mag).astype(np.float32)
        codes, s = oracle.quantize_row_i8(x)
        want_s = np.float32(np.abs(x).max()) / np.float32(127.0)
        assert s == want_s
        want = np.clip(np.rint(x / want_s), -127, 127).astype(np.int8)   # fp32 quotient, half to even
        assert np.array_equal(codes, want)
        i = int(np.argmax(np.abs(x)))
        assert int(codes[i]) == (127 if x[i] > 0 else -127)


def test_quantize_row_i8_ties_zero_row_and_fixed_scale():
    codes, _ = oracle.quantize_row_i8(np.array([0.5, 1.5, 2.5, -0.5, -2.5], np.float32), scale=1.0)
    assert codes.tolist() == [0, 2, 2, 0, -2]                                   # ties to even
    codes, s = oracle.quantize_row_i8(np.zeros(32, np.float32))
    assert s == 1.0 and not codes.any()
    codes, _ = oracle.quantize_row_i8(np.array([300.0, -1e9, 12.0], np.float32), scale=0.5)
    assert codes.tolist() == [127, -127, 24]                                    # saturation


# ---------------------------------------------------------------- append
def _paged_cache(kv, nblocks, bs, hkv, d, g):
    if kv == "int8":
        k = torch.from_numpy(g.integers(-127, 128, size=(nblocks, bs, hkv, d), dtype=np.int8))
        v = torch.from_numpy(g.integers(-127, 128, size=(nblocks, bs, hkv, d), dtype=np.int8))
    elif kv == "fp8_e4m3":
        k = torch.from_numpy(g.integers(0, 0x7E, size=(nblocks, bs, hkv, d), dtype=np.uint8))
        v = torch.from_numpy(g.integers(0, 0x7E, size=(nblocks, bs, hkv, d), dtype=np.uint8))
    else:
        dt = torch.float16 if kv == "f16" else torch.bfloat16
        k = torch.from_numpy(g.standard_normal((nblocks, bs, hkv, d)).astype(np.float32)).to(dt)
        v = torch.from_numpy(g.standard_normal((nblocks, bs, hkv, d)).astype(np.float32)).to(dt)
    return k, v


@pytest.mark.parametrize("kv,scale", [("fp8_e4m3", "token_head"), ("fp8_e4m3", "tensor"),
                                      ("int8", "token_head"), ("int8", "tensor"),
                                      ("f16", "none"), ("bf16", "none")])
def test_append_writes_exactly_the_target_rows(kv, scale):
    g = np.random.default_rng(9)
    batch, hkv, d, bs, nblocks, maxb = 4, 2, 64, 32, 12, 3
    k, v = _paged_cache(kv, nblocks, bs, hkv, d, g)
    table = torch.from_numpy(g.permutation(nblocks)[: batch * maxb].reshape(batch, maxb).astype(np.int32))
    pos = torch.tensor([0, 31, 32, -1], dtype=torch.int32)
    k_new = torch.randn(batch, hkv, d, generator=torch.Generator().manual_seed(1))
    v_new = torch.randn(batch, hkv, d, generator=torch.Generator().manual_seed(2))
    ks = vs = None
    if scale == "token_head":
        ks = torch.full((nblocks, bs, hkv), 7.0)
        vs = torch.full((nblocks, bs, hkv), 7.0)
    elif scale == "tensor":
        ks, vs = torch.tensor([0.02]), torch.tensor([0.03])
    kc, vc, ksc, vsc = oracle.kv_append(k_new=k_new, v_new=v_new, k_cache=k, v_cache=v, pos=pos,
                                        kv_dtype=kv, scale_mode=scale, k_scale=ks, v_scale=vs,
                                        block_table=table, block_size=bs)
    k0 = oracle._host(k).reshape(nblocks * bs, hkv, d)
    kc = kc.reshape(nblocks * bs, hkv, d)
    vc = vc.reshape(nblocks * bs, hkv, d)
    touched = set()
    for b in range(batch):
        t = int(pos[b])
        if t < 0:
            continue
        row = int(table[b, t // bs]) * bs + t % bs
        touched.add(row)
        for h in range(hkv):
            for new, cache, sc, fixed in ((k_new, kc, ksc, 0.02), (v_new, vc, vsc, 0.03)):
                x = new[b, h].numpy()
                if kv in ("fp8_e4m3", "int8"):
                    quant = oracle.quantize_row_e4m3 if kv == "fp8_e4m3" else oracle.quantize_row_i8
                    want, s = quant(x, fixed if scale == "tensor" else 0.0)
                    assert np.array_equal(cache[row, h], want)
                    if scale == "token_head":
                        assert sc.reshape(-1, hkv)[row, h] == s
                else:
                    enc = oracle.f16_encode if kv == "f16" else oracle.bf16_encode
                    assert [int(w) & 0xFFFF for w in cache[row, h]] == [enc(e) for e in x]
    others = [r for r in range(nblocks * bs) if r not in touched]
    assert np.array_equal(kc[others], k0[others])
    if scale == "token_head":
        keep = np.ones(nblocks * bs, bool)
        keep[list(touched)] = False
        assert np.all(ksc.reshape(-1, hkv)[keep] == 7.0) and np.all(vsc.reshape(-1, hkv)[keep] == 7.0)
    if scale == "tensor":
        assert ksc[0] == np.float32(0.02) and vsc[0] == np.float32(0.03)


def test_append_contiguous_rows():
    g = np.random.default_rng(10)
    batch, hkv, d, rows = 3, 1, 16, 40
    k = torch.zeros(rows, hkv, d, dtype=torch.float16)
    v = torch.zeros(rows, hkv, d, dtype=torch.float16)
    start = torch.tensor([0, 10, 25], dtype=torch.int32)
    pos = torch.tensor([3, 0, 14], dtype=torch.int32)
    k_new = torch.from_numpy(g.standard_normal((batch, hkv, d)).astype(np.float32))
    kc, vc, _, _ = oracle.kv_append(k_new=k_new, v_new=k_new * 2, k_cache=k, v_cache=v, pos=pos,
                                    kv_dtype="f16", kv_start=start)
    kc = kc.view(np.float16).astype(np.float32)
    for b in range(batch):
        row = int(start[b]) + int(pos[b])
        assert np.array_equal(kc[row, 0], k_new[b, 0].numpy().astype(np.float16).astype(np.float32))
    assert np.count_nonzero(np.abs(kc).sum(axis=(1, 2))) == batch


def test_appended_token_read_back_through_attention_oracle():
    # a sequence whose only token is the appended one attends to exactly that dequantised V row
    g = np.random.default_rng(11)
    batch, hq, hkv, d, bs, nblocks = 2, 4, 2, 64, 32, 4
    k = torch.zeros(nblocks, bs, hkv, d, dtype=torch.uint8)
    v = torch.zeros(nblocks, bs, hkv, d, dtype=torch.uint8)
    ks = torch.ones(nblocks, bs, hkv)
    vs = torch.ones(nblocks, bs, hkv)
    table = torch.tensor([[2, 0], [3, 1]], dtype=torch.int32)
    k_new = torch.from_numpy(g.standard_normal((batch, hkv, d)).astype(np.float32))
    v_new = torch.from_numpy(g.standard_normal((batch, hkv, d)).astype(np.float32) * 5)
    kc, vc, ksc, vsc = oracle.kv_append(k_new=k_new, v_new=v_new, k_cache=k, v_cache=v,
                                        pos=torch.zeros(batch, dtype=torch.int32), kv_dtype="fp8_e4m3",
                                        scale_mode="token_head", k_scale=ks, v_scale=vs,
                                        block_table=table, block_size=bs)
    q = torch.randn(batch, hq, d).to(torch.bfloat16)
    prob = oracle.Problem(q=q, k_cache=kc, v_cache=vc, seq_len=torch.ones(batch, dtype=torch.int32),
                          batch=batch, hq=hq, hkv=hkv, d=d, q_dtype="bf16", kv_dtype="fp8_e4m3",
                          scale_mode="token_head", k_scale=ksc, v_scale=vsc, block_table=table,
                          block_size=bs, softmax_scale=d ** -0.5)
    out, _ = oracle.decode_attention(prob, nthreads=1)
    for b in range(batch):
        for h in range(hq):
            gk = h // (hq // hkv)
            bytes_, s = oracle.quantize_row_e4m3(v_new[b, gk].numpy())
            want = np.array([e4m3_value(int(c)) for c in bytes_]) * s
            assert np.array_equal(out[b, h], want)
