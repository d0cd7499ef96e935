"""GPU parity of the KV-cache append (fd_kv_append) against the oracle, through the C ABI.

The bar is bit-exact: the stored E4M3 / INT8 codes, f16/bf16 values and per-token scales are integer /
byte results decided in fp32, the same precision on both sides.  Every byte of the caches and
every scale is compared (rows not appended must be left untouched).  An end-to-end case appends
a token to every sequence of a decode batch and runs the attention over the grown sequences.
"""
import random

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


def test_fp8_encode_matches_format_definition():
    vals = []
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        v = np.float32(oracle.e4m3_to_double(c))
        vals += [v, np.nextafter(v, np.float32(np.inf)), np.nextafter(v, np.float32(-np.inf))]
    for sign in (1.0, -1.0):
        for c in range(0x7E):
            lo, hi = oracle.e4m3_to_double(c), oracle.e4m3_to_double(c + 1)
            mid = np.float32(sign * (lo + hi) / 2)
            vals += [mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(-np.inf))]
    g = np.random.default_rng(3)
    mags = np.exp(g.uniform(np.log(2.0 ** -14), np.log(600.0), size=50000))
    vals += list((mags * g.choice([-1.0, 1.0], size=mags.size)).astype(np.float32))
    vals += [np.float32(x) for x in (0.0, -0.0, 448.0, -448.0, 449.0, 463.9, 464.0, 1e6, -1e30, 1e-30)]
    x = np.array(vals, dtype=np.float32)
    got = fd.fp8_e4m3_encode(torch.from_numpy(x).cuda()).cpu().numpy()
    want = np.array([oracle.e4m3_encode(v) for v in x], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def _append_case(seed, *, batch, hkv, d, kv, scale, new, paged, bs=64, nblocks=None):
    g = torch.Generator().manual_seed(seed)
    rows_per_seq = 3 * max(bs, 32)
    if kv == "fp8_e4m3":
        mk = lambda shape: torch.randint(0, 0x7E, shape, generator=g, dtype=torch.uint8)  # noqa: E731
    elif kv == "int8":
        mk = lambda shape: torch.randint(-127, 128, shape, generator=g, dtype=torch.int8)  # noqa: E731
    else:
        dt = {"f16": torch.float16, "bf16": torch.bfloat16}[kv]
        mk = lambda shape: torch.randn(shape, generator=g).to(dt)  # noqa: E731
    if paged:
        nblocks = nblocks or batch * 3 + 2
        k, v = mk((nblocks, bs, hkv, d)), mk((nblocks, bs, hkv, d))
        table = torch.randperm(nblocks, generator=g)[: batch * 3].reshape(batch, 3).to(torch.int32)
        start = None
        rows = nblocks * bs
    else:
        rows = batch * rows_per_seq + 7
        k, v = mk((rows, hkv, d)), mk((rows, hkv, d))
        table = None
        start = (torch.arange(batch, dtype=torch.int32) * rows_per_seq + 3)
    ks = vs = None
    if scale == "token_head":
        ks = torch.rand(rows * hkv, generator=g) + 0.5
        vs = torch.rand(rows * hkv, generator=g) + 0.5
    elif scale == "tensor":
        ks, vs = torch.tensor([0.013]), torch.tensor([0.021])
    # positions: block starts and ends, a skipped sequence, mid-block
    cand = [0, bs - 1, bs, 2 * bs - 1, 2 * bs, 5, -1, bs + 7]
    pos = torch.tensor([cand[i % len(cand)] for i in range(batch)], dtype=torch.int32)
    ndt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[new]
    k_new = (torch.randn(batch, hkv, d, generator=g) * 3).to(ndt)
    v_new = (torch.randn(batch, hkv, d, generator=g) * 0.2).to(ndt)
    k_new[0, 0] = 0.0  # an all-zero row (scale 1)
    return dict(k_new=k_new, v_new=v_new, k=k, v=v, table=table, start=start, ks=ks, vs=vs, pos=pos, bs=bs)


APPEND_CASES = [
    # name, kwargs
    ("fp8_tok_bf16in_bs64", dict(batch=8, hkv=2, d=128, kv="fp8_e4m3", scale="token_head", new="bf16", paged=True)),
    ("fp8_tok_f32in_bs32", dict(batch=8, hkv=4, d=128, kv="fp8_e4m3", scale="token_head", new="f32", paged=True, bs=32)),
    ("fp8_tok_f16in_d64_contig", dict(batch=5, hkv=1, d=64, kv="fp8_e4m3", scale="token_head", new="f16", paged=False)),
    ("fp8_tensor_bf16in", dict(batch=8, hkv=8, d=128, kv="fp8_e4m3", scale="tensor", new="bf16", paged=True)),
    ("fp8_tensor_f32in_d64_bs32", dict(batch=3, hkv=2, d=64, kv="fp8_e4m3", scale="tensor", new="f32", paged=True, bs=32)),
    ("f16_f32in", dict(batch=6, hkv=2, d=128, kv="f16", scale="none", new="f32", paged=True)),
    ("bf16_f32in_contig", dict(batch=4, hkv=2, d=128, kv="bf16", scale="none", new="f32", paged=False)),
    ("bf16_bf16in_d64", dict(batch=4, hkv=3, d=64, kv="bf16", scale="none", new="bf16", paged=True, bs=32)),
    ("fp8_tok_bf16in_bs16", dict(batch=8, hkv=2, d=128, kv="fp8_e4m3", scale="token_head", new="bf16", paged=True, bs=16)),
    ("i8_tok_bf16in_bs64", dict(batch=8, hkv=2, d=128, kv="int8", scale="token_head", new="bf16", paged=True)),
    ("i8_tok_f32in_d64_bs16", dict(batch=8, hkv=3, d=64, kv="int8", scale="token_head", new="f32", paged=True, bs=16)),
    ("i8_tensor_f16in_contig", dict(batch=5, hkv=2, d=128, kv="int8", scale="tensor", new="f16", paged=False)),
    ("i8_tensor_f32in_d64_bs32", dict(batch=4, hkv=1, d=64, kv="int8", scale="tensor", new="f32", paged=True, bs=32)),
]


@pytest.mark.parametrize("name,kw", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_kv_append_bitwise_equals_oracle(name, kw):
    _check_append(name, kw, 7)


def _random_append_configs(n, seed):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        kv = rng.choice(["fp8_e4m3", "int8", "f16", "bf16"])
        paged = rng.random() < 0.75
        out.append(dict(batch=rng.randint(1, 12), hkv=rng.choice([1, 2, 3, 4, 8]), d=rng.choice([64, 128]), kv=kv,
                        scale="none" if kv in ("f16", "bf16") else rng.choice(["tensor", "token_head"]),
                        new=rng.choice(["f32", "f16", "bf16"]), paged=paged,
                        bs=rng.choice([16, 32, 64]) if paged else 64))
    return out


RANDOM_APPEND = _random_append_configs(60, 20261203)


@pytest.mark.parametrize("idx", range(len(RANDOM_APPEND)))
def test_kv_append_random_configs_bitwise(idx):
    # seeded random (cache dtype, scale mode, input dtype, head_dim, kv heads, batch, paging)
    _check_append(f"random{idx} {RANDOM_APPEND[idx]}", RANDOM_APPEND[idx], 100 + idx)


def _check_append(name, kw, seed):
    c = _append_case(seed, **kw)
    print(f"[{name}] pos={c['pos'].tolist()}", flush=True)
    want_k, want_v, want_ks, want_vs = oracle.kv_append(
        k_new=c["k_new"], v_new=c["v_new"], k_cache=c["k"], v_cache=c["v"], pos=c["pos"],
        kv_dtype=kw["kv"], scale_mode=kw["scale"], k_scale=c["ks"], v_scale=c["vs"],
        block_table=c["table"], kv_start=c["start"], block_size=c["bs"] if kw["paged"] else 0)
    dev = lambda t: None if t is None else t.cuda()  # noqa: E731
    k, v, ks, vs = dev(c["k"]), dev(c["v"]), dev(c["ks"]), dev(c["vs"])
    fd.kv_append(dev(c["k_new"]), dev(c["v_new"]), k, v, dev(c["pos"]), kv_dtype=kw["kv"],
                 block_table=dev(c["table"]), kv_start=dev(c["start"]),
                 block_size=c["bs"] if kw["paged"] else 0, scale_mode=kw["scale"], k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    assert np.array_equal(oracle._host(k), want_k), f"{name}: K cache differs"
    assert np.array_equal(oracle._host(v), want_v), f"{name}: V cache differs"
    if kw["scale"] != "none":
        assert np.array_equal(ks.cpu().numpy(), want_ks) and np.array_equal(vs.cpu().numpy(), want_vs), \
            f"{name}: scales differ"
    print(f"[{name}] PASS bitwise", flush=True)


@pytest.mark.parametrize("wname", ["fp8_32k_small", "wide_mqa", "int8_small"])
def test_append_then_attend(wname):
    # append one token to each sequence, then attend over the grown sequences (both paths)
    if wname == "fp8_32k_small":
        case = workloads.custom_case(seed=31, device="cpu", batch=4, hq=64, hkv=8, d=128,
                                     seq_lens=[127, 64, 1000, 5], kv="fp8_e4m3", q="bf16",
                                     scale="token_head", block_size=64, max_seq_len=1100)
    elif wname == "wide_mqa":
        case = workloads.custom_case(seed=32, device="cpu", batch=3, hq=128, hkv=1, d=128,
                                     seq_lens=[63, 700, 32], kv="fp8_e4m3", q="bf16",
                                     scale="tensor", block_size=64, max_seq_len=800)
    else:
        case = workloads.custom_case(seed=33, device="cpu", batch=4, hq=32, hkv=4, d=128,
                                     seq_lens=[15, 16, 900, 3], kv="int8", q="bf16",
                                     scale="token_head", block_size=16, max_seq_len=1000)
    # every sequence gets a block for its next token (the spare blocks of the generator)
    bt = case.block_table.clone()
    nb = case.k_cache.shape[0]
    used = set(int(x) for x in bt[bt >= 0].tolist())
    spare = [i for i in range(nb) if i not in used]
    for b, n in enumerate(case.seq_lens):
        if n % case.block_size == 0:
            bt[b, n // case.block_size] = spare.pop()
    case.block_table = bt
    if case.scale_mode == "token_head":  # the spare blocks' scales were poisoned: give them values
        case.k_scale = torch.nan_to_num(case.k_scale, nan=1.0)
        case.v_scale = torch.nan_to_num(case.v_scale, nan=1.0)
    g = torch.Generator().manual_seed(5)
    k_new = torch.randn(case.batch, case.hkv, case.d, generator=g).to(torch.bfloat16)
    v_new = torch.randn(case.batch, case.hkv, case.d, generator=g).to(torch.bfloat16)
    pos = case.seq_len.clone()
    kc, vc, ksc, vsc = oracle.kv_append(k_new=k_new, v_new=v_new, k_cache=case.k_cache, v_cache=case.v_cache,
                                        pos=pos, kv_dtype=case.kv_dtype, scale_mode=case.scale_mode,
                                        k_scale=case.k_scale, v_scale=case.v_scale,
                                        block_table=case.block_table, block_size=case.block_size)
    grown = case.seq_len + 1
    prob = oracle.Problem(q=case.q, k_cache=torch.from_numpy(kc), v_cache=torch.from_numpy(vc), seq_len=grown,
                          batch=case.batch, hq=case.hq, hkv=case.hkv, d=case.d, q_dtype=case.q_dtype,
                          kv_dtype=case.kv_dtype, scale_mode=case.scale_mode,
                          k_scale=None if ksc is None else torch.from_numpy(ksc),
                          v_scale=None if vsc is None else torch.from_numpy(vsc),
                          block_table=case.block_table, block_size=case.block_size,
                          softmax_scale=case.softmax_scale)
    ref, _ = oracle.decode_attention(prob)
    dev = lambda t: None if t is None else t.cuda()  # noqa: E731
    k, v, ks, vs, btd = dev(case.k_cache), dev(case.v_cache), dev(case.k_scale), dev(case.v_scale), dev(case.block_table)
    fd.kv_append(dev(k_new), dev(v_new), k, v, dev(pos), kv_dtype=case.kv_dtype, block_table=btd,
                 block_size=case.block_size, scale_mode=case.scale_mode, k_scale=ks, v_scale=vs)
    out = fd.decode_attention(dev(case.q), k, v, dev(grown), max_seq_len=case.max_seq_len + 1,
                              block_table=btd, kv_dtype=case.kv_dtype, scale_mode=case.scale_mode,
                              k_scale=ks, v_scale=vs, softmax_scale=case.softmax_scale,
                              num_kv_heads=case.hkv, block_size=case.block_size)
    torch.cuda.synchronize()
    err = out.double().cpu().numpy() - ref
    max_abs = float(np.abs(err).max())
    rel = float(np.linalg.norm(err) / np.linalg.norm(ref))
    print(f"[append_then_attend/{wname}] max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert max_abs <= 5e-3 and rel <= 3e-3
