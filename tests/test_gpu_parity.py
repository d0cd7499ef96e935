"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded inputs.

Bar (per KV type): max |gpu - oracle| over all output elements and relative L2 error
||gpu - oracle|| / ||oracle|| must stay within 2e-3 / 1e-3 for f16/bf16 KV and 5e-3 / 3e-3 for
E4M3 and INT8 KV (the oracle dequantises the same bytes with the same scales).  Results are printed as
``[case] PASS max_abs=... rel_l2=...`` lines.
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_06_amd as fd
import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"f16": (2e-3, 1e-3), "bf16": (2e-3, 1e-3), "fp8_e4m3": (5e-3, 3e-3), "int8": (5e-3, 3e-3)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    fd.lib()
    yield


def compare(name, got, ref, kv_dtype, seqs=None):
    got = got.detach().float().cpu().numpy().astype(np.float64)
    if seqs is not None:
        got, ref = got[list(seqs)], ref[list(seqs)]
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = got - ref
    max_abs = float(np.max(np.abs(err))) if err.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel_l2 = float(np.linalg.norm(err) / nref) if nref > 0 else float(np.linalg.norm(err))
    tol_abs, tol_rel = TOL[kv_dtype]
    ok = max_abs <= tol_abs and rel_l2 <= tol_rel
    print(f"[{name}] {'PASS' if ok else 'FAIL'} max_abs={max_abs:.3e} rel_l2={rel_l2:.3e}", flush=True)
    assert ok, f"{name}: max_abs={max_abs:.3e} rel_l2={rel_l2:.3e} (tol {tol_abs}, {tol_rel})"
    return max_abs, rel_l2


def run_gpu(case, **kw):
    lse = torch.empty(tuple(case.q.shape[:-1]), dtype=torch.float32, device="cuda")
    out = fd.decode_case(case, lse=lse, **kw)
    torch.cuda.synchronize()
    return out, lse


def check_case(name, case, seqs=None, num_partitions=0, out_dtype="f32"):
    print(f"[{name}] lens={case.seq_lens[:8]}{'...' if case.batch > 8 else ''} G={case.group} "
          f"D={case.d} kv={case.kv_dtype} scale={case.scale_mode} bs={case.block_size} "
          f"partitions={num_partitions}", flush=True)
    out, lse = run_gpu(case, num_partitions=num_partitions, out_dtype=out_dtype)
    prob = oracle.Problem.from_case(case)
    ref, ref_lse = oracle.decode_attention(prob, seqs=seqs)
    compare(name, out, ref, case.kv_dtype, seqs)
    lg = lse.cpu().numpy().astype(np.float64)
    rl = ref_lse if seqs is None else ref_lse[list(seqs)]
    lg = lg if seqs is None else lg[list(seqs)]
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lg)), f"{name}: lse finiteness differs"
    if fin.any():
        assert np.max(np.abs(lg[fin] - rl[fin])) < 1e-3, f"{name}: lse mismatch"
    return out


# ------------------------------------------------------------------ E4M3 conversion
def test_fp8_hardware_decode_matches_format_definition():
    allb = torch.arange(256, dtype=torch.uint8, device="cuda")
    got = fd.fp8_e4m3_decode(allb).cpu().numpy()
    for byte in range(256):
        ref = oracle.e4m3_to_double(byte)
        for col in range(2):
            if math.isnan(ref):
                assert math.isnan(got[byte, col]), (hex(byte), col)
            else:
                assert got[byte, col] == ref, (hex(byte), col, got[byte, col], ref)


# ------------------------------------------------------------------ small shapes
SMALL = [
    # name, kwargs for workloads.custom_case
    ("mqa_f16_d64_contig", dict(batch=2, hq=4, hkv=1, d=64, seq_lens=[37, 100], kv="f16", q="f16",
                                scale="none", paged=False, block_size=0)),
    ("gqa4_bf16_d128", dict(batch=3, hq=8, hkv=2, d=128, seq_lens=[1, 100, 777], kv="bf16", q="bf16",
                            scale="none", block_size=64)),
    ("gqa8_fp8_tok", dict(batch=3, hq=16, hkv=2, d=128, seq_lens=[65, 1500, 31], kv="fp8_e4m3",
                          q="bf16", scale="token_head", block_size=64)),
    ("gqa8_fp8_tok_f16q", dict(batch=2, hq=8, hkv=1, d=128, seq_lens=[300, 64], kv="fp8_e4m3",
                               q="f16", scale="token_head", block_size=32)),
    ("mqa128_fp8_tensor", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[2049, 333], kv="fp8_e4m3",
                               q="bf16", scale="tensor", block_size=64)),
    ("g32_fp8_tensor_d64", dict(batch=2, hq=32, hkv=1, d=64, seq_lens=[513, 7], kv="fp8_e4m3",
                                q="bf16", scale="tensor", block_size=32)),
    ("mha_f16_d64_paged", dict(batch=2, hq=4, hkv=4, d=64, seq_lens=[33, 250], kv="f16", q="f16",
                               scale="none", block_size=32)),
    ("g16_bf16_d64", dict(batch=2, hq=16, hkv=1, d=64, seq_lens=[95, 64], kv="bf16", q="bf16",
                          scale="none", block_size=64)),
    ("g4_fp8_tok_d64_contig", dict(batch=3, hq=8, hkv=2, d=64, seq_lens=[40, 1, 129], kv="fp8_e4m3",
                                   q="bf16", scale="token_head", paged=False, block_size=0)),
    ("g2_fp8_tok_bs32", dict(batch=2, hq=4, hkv=2, d=128, seq_lens=[1000, 2], kv="fp8_e4m3", q="bf16",
                             scale="token_head", block_size=32)),
    # several head blocks per kv head (cached, shared loads) in contiguous mode
    ("g32_bf16_contig", dict(batch=2, hq=64, hkv=2, d=128, seq_lens=[200, 1], kv="bf16", q="bf16",
                             scale="none", paged=False, block_size=0)),
    # wide-group kernel (E4M3, head_dim 128, group a multiple of 64): 2 and 4 waves per workgroup,
    # both scale modes, both q types, paged and contiguous, two workgroups per kv head (G = 256)
    ("wide_g64_tok", dict(batch=3, hq=128, hkv=2, d=128, seq_lens=[1000, 33, 4097], kv="fp8_e4m3",
                          q="bf16", scale="token_head", block_size=64)),
    ("wide_g128_tok_contig_f16q", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[300, 1], kv="fp8_e4m3",
                                       q="f16", scale="token_head", paged=False, block_size=0)),
    ("wide_g256_tensor_bs32", dict(batch=2, hq=256, hkv=1, d=128, seq_lens=[700, 64], kv="fp8_e4m3",
                                   q="bf16", scale="tensor", block_size=32)),
    ("wide_g64_tensor_f16q", dict(batch=2, hq=64, hkv=1, d=128, seq_lens=[2500, 95], kv="fp8_e4m3",
                                  q="f16", scale="tensor", block_size=64)),
    # 16-token pages: every 32-token tile spans two blocks
    ("bs16_fp8_tok_g8", dict(batch=3, hq=16, hkv=2, d=128, seq_lens=[700, 17, 48], kv="fp8_e4m3",
                             q="bf16", scale="token_head", block_size=16)),
    ("bs16_bf16_g4_d64", dict(batch=2, hq=8, hkv=2, d=64, seq_lens=[333, 16], kv="bf16", q="bf16",
                              scale="none", block_size=16)),
    ("bs16_wide_g128_tok", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[1000, 31], kv="fp8_e4m3",
                                q="bf16", scale="token_head", block_size=16)),
    # 32-column units, K/V straight into registers (E4M3 KV, head_dim 128, 32 MFMA columns per kv head)
    ("direct_g32_tok", dict(batch=3, hq=64, hkv=2, d=128, seq_lens=[1000, 33, 4097], kv="fp8_e4m3",
                            q="bf16", scale="token_head", block_size=64)),
    ("direct_g32_tensor_bs16", dict(batch=2, hq=32, hkv=1, d=128, seq_lens=[700, 31], kv="fp8_e4m3",
                                    q="bf16", scale="tensor", block_size=16)),
    ("direct_g32_tok_contig_f16q", dict(batch=2, hq=64, hkv=2, d=128, seq_lens=[300, 1], kv="fp8_e4m3",
                                        q="f16", scale="token_head", paged=False, block_size=0)),
    ("direct_g96_tok_bs32", dict(batch=2, hq=96, hkv=1, d=128, seq_lens=[1500, 64], kv="fp8_e4m3",
                                 q="bf16", scale="token_head", block_size=32)),
    # wide-group kernel with INT8 KV (K and V staged once per workgroup as exact f16)
    ("wide_i8_g64_tok", dict(batch=3, hq=128, hkv=2, d=128, seq_lens=[1000, 33, 4097], kv="int8",
                             q="bf16", scale="token_head", block_size=64)),
    ("wide_i8_g128_tok_contig_f16q", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[300, 1], kv="int8",
                                          q="f16", scale="token_head", paged=False, block_size=0)),
    ("wide_i8_g256_tensor_bs32", dict(batch=2, hq=256, hkv=1, d=128, seq_lens=[700, 64], kv="int8",
                                      q="bf16", scale="tensor", block_size=32)),
    ("bs16_wide_i8_g128_tensor", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[1000, 31], kv="int8",
                                      q="bf16", scale="tensor", block_size=16)),
    ("bs16_wide_g64_tensor", dict(batch=3, hq=128, hkv=2, d=128, seq_lens=[65, 300, 1], kv="fp8_e4m3",
                                  q="bf16", scale="tensor", block_size=16)),
    # wide-group kernel with f16 / bf16 KV (groups of 128+: K read from the ring as is, V re-laid
    # without conversion, bf16 P in two terms): both types, paged (64, 32, 16) and contiguous, two
    # workgroups per kv head (G = 256), two kv heads
    ("wide16_bf16_g128", dict(batch=3, hq=128, hkv=1, d=128, seq_lens=[1000, 33, 4097], kv="bf16",
                              q="bf16", scale="none", block_size=64)),
    ("wide16_f16_g128_contig", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[300, 1], kv="f16", q="f16",
                                    scale="none", paged=False, block_size=0)),
    ("wide16_bf16_g256_bs32", dict(batch=2, hq=256, hkv=1, d=128, seq_lens=[700, 64], kv="bf16",
                                   q="bf16", scale="none", block_size=32)),
    ("wide16_f16_g128_hkv2_bs16", dict(batch=3, hq=256, hkv=2, d=128, seq_lens=[65, 300, 1], kv="f16",
                                       q="f16", scale="none", block_size=16)),
    ("wide16_bf16_g128_hkv2", dict(batch=2, hq=256, hkv=2, d=128, seq_lens=[2500, 95], kv="bf16",
                                   q="bf16", scale="none", block_size=64)),
    # one long sequence over few units: many pieces per row, merged by several combine waves
    ("mqa8_d64_long_f16", dict(batch=1, hq=8, hkv=1, d=64, seq_lens=[4000], kv="f16", q="f16",
                               scale="none", block_size=32)),
    ("mqa16_d128_long_fp8", dict(batch=2, hq=16, hkv=1, d=128, seq_lens=[5000, 3], kv="fp8_e4m3",
                                 q="bf16", scale="token_head", block_size=64)),
    # INT8 KV: both scale modes and q types, both head dims, every page size and contiguous, a
    # group of 128 (eight 16-head blocks per kv head)
    ("gqa8_i8_tok", dict(batch=3, hq=16, hkv=2, d=128, seq_lens=[65, 1500, 31], kv="int8",
                         q="bf16", scale="token_head", block_size=64)),
    ("g8_i8_tok_f16q_bs32", dict(batch=2, hq=8, hkv=1, d=128, seq_lens=[300, 64], kv="int8",
                                 q="f16", scale="token_head", block_size=32)),
    ("mqa128_i8_tensor", dict(batch=2, hq=128, hkv=1, d=128, seq_lens=[2049, 333], kv="int8",
                              q="bf16", scale="tensor", block_size=64)),
    ("g4_i8_tok_d64_contig", dict(batch=3, hq=8, hkv=2, d=64, seq_lens=[40, 1, 129], kv="int8",
                                  q="bf16", scale="token_head", paged=False, block_size=0)),
    ("g32_i8_tensor_f16q_d64", dict(batch=2, hq=32, hkv=1, d=64, seq_lens=[513, 7], kv="int8",
                                    q="f16", scale="tensor", block_size=32)),
    ("bs16_i8_tok_g8", dict(batch=3, hq=16, hkv=2, d=128, seq_lens=[700, 17, 48], kv="int8",
                            q="bf16", scale="token_head", block_size=16)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("parts", [0, 1, 2, 7, 100000])
def test_small_shapes(name, kw, parts):
    case = workloads.custom_case(seed=3, device="cuda", **kw)
    check_case(f"{name}/p{parts}", case, num_partitions=parts)


@pytest.mark.parametrize("n", [0, 1, 31, 32, 33, 63, 64, 65, 255, 256, 257, 4095])
def test_length_edges(n):
    lens = [n, 5, n]
    case = workloads.custom_case(seed=n, device="cuda", batch=3, hq=16, hkv=2, d=128, seq_lens=lens,
                                 kv="fp8_e4m3", q="bf16", scale="token_head", block_size=64,
                                 max_seq_len=max(lens + [1]))
    for parts in (0, 3):
        check_case(f"len{n}/p{parts}", case, num_partitions=parts)


@pytest.mark.parametrize("bs", [16, 64])
@pytest.mark.parametrize("n", [0, 1, 31, 32, 33, 63, 64, 65, 4095])
def test_int8_length_edges(n, bs):
    lens = [n, 5, n]
    case = workloads.custom_case(seed=300 + n, device="cuda", batch=3, hq=16, hkv=2, d=128, seq_lens=lens,
                                 kv="int8", q="bf16", scale="token_head", block_size=bs,
                                 max_seq_len=max(lens + [1]))
    for parts in (0, 3):
        check_case(f"i8_len{n}_bs{bs}/p{parts}", case, num_partitions=parts)


@pytest.mark.parametrize("kv", ["fp8_e4m3", "int8", "bf16"])
@pytest.mark.parametrize("n", [0, 1, 31, 32, 33, 191, 192, 193, 4095])
def test_wide_length_edges(n, kv):
    lens = [n, 7, n]
    case = workloads.custom_case(seed=100 + n, device="cuda", batch=3, hq=128, hkv=1, d=128, seq_lens=lens,
                                 kv=kv, q="bf16", scale="none" if kv == "bf16" else "token_head",
                                 block_size=64, max_seq_len=max(lens + [1]))
    for parts in (0, 3):
        check_case(f"wide_{kv}_len{n}/p{parts}", case, num_partitions=parts)


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("n", [1, 15, 16, 17, 31, 32, 33, 47, 48, 49])
def test_block16_length_edges(n, wide):
    lens = [n, 16, n + 16]
    hq = 128 if wide else 16
    case = workloads.custom_case(seed=200 + n, device="cuda", batch=3, hq=hq, hkv=1 if wide else 2, d=128,
                                 seq_lens=lens, kv="fp8_e4m3", q="bf16", scale="token_head", block_size=16,
                                 max_seq_len=max(lens))
    for parts in (0, 5):
        check_case(f"bs16_len{n}{'_wide' if wide else ''}/p{parts}", case, num_partitions=parts)


def test_block16_ragged_mix():
    lens = [0, 1, 5000, 33, 0, 64, 2047, 12000, 31, 0, 700, 96]
    case = workloads.custom_case(seed=23, device="cuda", batch=len(lens), hq=32, hkv=8, d=128,
                                 seq_lens=lens, kv="fp8_e4m3", q="bf16", scale="token_head",
                                 block_size=16)
    for parts in (3, 256):
        check_case(f"bs16_ragged/p{parts}", case, num_partitions=parts)


@pytest.mark.parametrize("kv", ["fp8_e4m3", "int8", "f16"])
def test_wide_ragged_mix(kv):
    lens = [0, 1, 5000, 33, 0, 64, 2047, 12000, 31, 0, 700, 96]
    case = workloads.custom_case(seed=22, device="cuda", batch=len(lens), hq=256 if kv == "f16" else 128,
                                 hkv=2, d=128, seq_lens=lens, kv=kv, q="f16" if kv == "f16" else "bf16",
                                 scale="none" if kv == "f16" else "token_head", block_size=32)
    for parts in (1, 7, 100, 1024):
        check_case(f"wide_{kv}_ragged/p{parts}", case, num_partitions=parts)


def test_more_partitions_than_tiles():
    # 3 partitions per tile on average: many idle waves, every unit cut into one-tile pieces
    case = workloads.custom_case(seed=9, device="cuda", batch=3, hq=8, hkv=1, d=128,
                                 seq_lens=[32 * 40 + 3, 200, 0], kv="fp8_e4m3", q="bf16",
                                 scale="token_head", block_size=64)
    tiles = sum(-(-n // 32) for n in case.seq_lens)
    check_case("overpartitioned", case, num_partitions=3 * tiles)
    check_case("one_tile_each", case, num_partitions=tiles)


@pytest.mark.parametrize("parts", [1, 5, 64, 333, 2048])
def test_ragged_mix_partition_counts(parts):
    lens = [0, 1, 5000, 33, 0, 64, 2047, 12000, 31, 0, 700, 96]
    case = workloads.custom_case(seed=21, device="cuda", batch=len(lens), hq=32, hkv=8, d=128,
                                 seq_lens=lens, kv="fp8_e4m3", q="bf16", scale="token_head",
                                 block_size=32)
    check_case(f"ragged_mix/p{parts}", case, num_partitions=parts)


@pytest.mark.parametrize("kv", ["fp8_e4m3", "bf16"])
@pytest.mark.parametrize("parts", [40, 160, 600])
def test_combine_many_pieces_per_row(parts, kv):
    # one long sequence among short ones, over 10 to 150 partitions per sequence: rows of the long
    # sequence hold up to ~250 pieces, merged by 1, 4 or 8 combine waves, in several rounds of
    # loads per lane group (16-bit pieces of E4M3 KV, fp32 pieces of bf16 KV)
    case = workloads.custom_case(seed=21, device="cuda", batch=4, hq=16, hkv=2, d=128,
                                 seq_lens=[8000, 40, 700, 1], kv=kv, q="bf16",
                                 scale="token_head" if kv == "fp8_e4m3" else "none", block_size=64)
    check_case(f"many_pieces/{kv}/p{parts}", case, num_partitions=parts)


def test_wide_kernel_batch_beyond_lds_prefix_table():
    # more sequences (300) than the wide kernel keeps tile prefix sums for in LDS (256): tiles are
    # located by wave scans of seq_len instead, in the partition kernel and the combine
    lens = [int(x) for x in np.random.default_rng(7).integers(0, 200, size=300)]
    lens[5], lens[0], lens[299] = 0, 1, 1000
    case = workloads.custom_case(seed=7, device="cuda", batch=300, hq=64, hkv=1, d=128, seq_lens=lens,
                                 kv="fp8_e4m3", q="bf16", scale="tensor", block_size=64)
    for parts in (0, 97):
        check_case(f"wide_batch300/p{parts}", case, num_partitions=parts)


def test_largest_batch():
    # 65535 sequences (the interface's limit; the combine's grid has one row of workgroups per
    # sequence), lengths 0..40, every fifth one empty
    rng = np.random.default_rng(12)
    lens = [int(x) for x in rng.integers(0, 41, size=65535)]
    for i in range(0, 65535, 5):
        lens[i] = 0
    case = workloads.custom_case(seed=12, device="cuda", batch=65535, hq=2, hkv=1, d=64, seq_lens=lens,
                                 kv="f16", q="f16", scale="none", block_size=16)
    check_case("batch65535", case)


def test_longest_sequence():
    # one sequence of 2^24 tokens (the interface's largest max_seq_len; 4.3 GB of E4M3 K and V)
    # beside a short one: every workgroup takes a piece of it, so its row merges 256 pieces (one
    # head: the oracle's single thread for the sequence takes ~35 s)
    case = workloads.custom_case(seed=14, device="cuda", batch=2, hq=1, hkv=1, d=128,
                                 seq_lens=[1 << 24, 100], kv="fp8_e4m3", q="bf16", scale="token_head",
                                 block_size=64)
    check_case("seq_2^24", case)


def test_partition_kernel_batch_beyond_lds_prefix_table():
    # 4100 sequences: past the 4096 the 16-head kernel keeps in LDS
    lens = [int(x) for x in np.random.default_rng(8).integers(0, 40, size=4100)]
    lens[4099] = 300
    case = workloads.custom_case(seed=8, device="cuda", batch=4100, hq=4, hkv=1, d=64, seq_lens=lens,
                                 kv="f16", q="f16", scale="none", block_size=32)
    for parts in (0, 333):
        check_case(f"batch4100/p{parts}", case, num_partitions=parts)


@pytest.mark.parametrize("kv", ["fp8_e4m3", "int8"])
@pytest.mark.parametrize("k_mult,v_mult", [(-1.0, 1.0), (-1.0, -1.0), (0.0, 1.0)])
@pytest.mark.parametrize("hq", [16, 32, 128])
def test_per_tensor_scale_signs(k_mult, v_mult, hq, kv):
    # negative or zero per-tensor scales (hq 128: the wide kernel, which scales scores inside the
    # exponent and flips q's sign for a negative scale; hq 32 with E4M3: the 32-column kernel, which
    # flips it the same way; hq 16: the 16-head kernel).  A zero k
    # scale makes every score 0: out is the plain mean of the dequantised V rows
    case = workloads.custom_case(seed=31, device="cuda", batch=2, hq=hq, hkv=1, d=128,
                                 seq_lens=[3000, 77], kv=kv, q="bf16", scale="tensor",
                                 block_size=64)
    case.k_scale = case.k_scale * k_mult
    case.v_scale = case.v_scale * v_mult
    for parts in (0, 7):
        check_case(f"scale_signs {kv} k{k_mult} v{v_mult} hq{hq}/p{parts}", case, num_partitions=parts)


@pytest.mark.parametrize("hq,kv", [(16, "fp8_e4m3"), (128, "fp8_e4m3"), (128, "int8"), (16, "int8")])
def test_peaky_scores(hq, kv):
    # q x 4: scores four times larger, the running max moves and the softmax is sharp (hq 128:
    # the wide kernel, whose q terms then carry more of the score)
    case = workloads.custom_case(seed=10, device="cuda", batch=2, hq=hq, hkv=2, d=128,
                                 seq_lens=[3000, 700], kv=kv, q="bf16", scale="token_head",
                                 block_size=64)
    case.q.mul_(4.0)
    check_case(f"peaky_q4_hq{hq}_{kv}", case, num_partitions=0)


@pytest.mark.parametrize("parts", [0, 1])
@pytest.mark.parametrize("kern", [
    dict(hq=16, hkv=2, kv="fp8_e4m3", scale="token_head"),
    dict(hq=128, hkv=1, kv="fp8_e4m3", scale="tensor"),
    dict(hq=128, hkv=1, kv="bf16", scale="none"),
    dict(hq=16, hkv=2, kv="fp8_e4m3", scale="token_head", nq=4),
], ids=["g8_fp8", "wide_fp8", "wide_bf16", "direct_nq4"])
@pytest.mark.parametrize("out_dtype", ["f16", "bf16"])
def test_half_outputs_are_rounded_f32(out_dtype, kern, parts):
    # rows finished by a partition kernel (the short sequence; everything with one partition) and
    # rows merged by the combine (the long sequence cut into pieces) both round the fp32 result
    kw = dict(kern)
    q = "bf16" if kw["kv"] != "f16" else "f16"
    case = workloads.custom_case(seed=11, device="cuda", batch=2, d=128, seq_lens=[900, 3], q=q,
                                 block_size=64, **kw)
    o32, _ = run_gpu(case, out_dtype="f32", num_partitions=parts)
    oh, _ = run_gpu(case, out_dtype=out_dtype, num_partitions=parts)
    ref = o32.to({"f16": torch.float16, "bf16": torch.bfloat16}[out_dtype])
    assert torch.equal(oh, ref)


# ------------------------------------------------------------------ properties
def test_run_to_run_bitwise_deterministic():
    case = workloads.make_case("fp8_32k", seed=1, device="cuda", batch=4)
    a, la = run_gpu(case)
    b, lb = run_gpu(case)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_run_to_run_bitwise_deterministic_many_pieces():
    # one MQA sequence over hundreds of workgroups: each row's pieces are split over the eight
    # waves of its combine workgroup and merged through LDS in a fixed order
    case = workloads.custom_case(seed=5, device="cuda", batch=1, hq=128, hkv=1, d=128,
                                 seq_lens=[40000], kv="fp8_e4m3", q="bf16", scale="tensor",
                                 block_size=64)
    a, la = run_gpu(case)
    b, lb = run_gpu(case)
    assert torch.equal(a, b) and torch.equal(la, lb)
    check_case("mqa_one_long_seq", case)


def test_block_placement_bitwise_invariant():
    case = workloads.custom_case(seed=12, device="cuda", batch=3, hq=16, hkv=2, d=128,
                                 seq_lens=[1000, 64, 333], kv="fp8_e4m3", q="bf16", scale="token_head",
                                 block_size=64)
    a, _ = run_gpu(case)
    # move every block to a new physical slot and rewrite the table
    nb = case.k_cache.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(4)).cuda()
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(nb, device="cuda")
    k2, v2 = torch.empty_like(case.k_cache), torch.empty_like(case.v_cache)
    k2[perm] = case.k_cache
    v2[perm] = case.v_cache
    ks2, vs2 = torch.empty_like(case.k_scale), torch.empty_like(case.v_scale)
    ks2[perm] = case.k_scale
    vs2[perm] = case.v_scale
    bt = case.block_table.clone()
    live = bt >= 0
    bt[live] = perm[bt[live].long()].int()
    case.k_cache, case.v_cache, case.k_scale, case.v_scale, case.block_table = k2, v2, ks2, vs2, bt
    b, _ = run_gpu(case)
    assert torch.equal(a, b)


# ------------------------------------------------------------------ full-size workloads
def test_workload_tiny_mqa_f16():
    check_case("tiny_mqa_f16", workloads.make_case("tiny_mqa_f16", device="cuda"))


def test_workload_gqa_bf16_full():
    check_case("gqa_bf16", workloads.make_case("gqa_bf16", device="cuda"))


def test_workload_fp8_32k_full():
    check_case("fp8_32k", workloads.make_case("fp8_32k", device="cuda"))


def test_workload_int8_32k_full():
    check_case("int8_32k", workloads.make_case("int8_32k", device="cuda"))


def test_workload_mqa_fp8_128k_full():
    # every output row (4 sequences x 128 heads) against the oracle on the host's threads
    check_case("mqa_fp8_128k", workloads.make_case("mqa_fp8_128k", device="cuda"))


def test_workload_mqa_i8_128k_full():
    # INT8 KV, the same shape (the wide-group kernel's int8 path)
    check_case("mqa_i8_128k", workloads.make_case("mqa_i8_128k", device="cuda"))


def test_workload_mqa_bf16_64k_full():
    # bf16 KV, 128 heads on one kv head (the wide-group kernel's 16-bit path), every output row
    check_case("mqa_bf16_64k", workloads.make_case("mqa_bf16_64k", device="cuda"))


def test_workload_ragged_fp8_full():
    # every output row (256 sequences x 32 heads, 2.4M tokens)
    check_case("ragged_fp8", workloads.make_case("ragged_fp8", device="cuda"))


@pytest.mark.parametrize("kw", [
    dict(hq=16, hkv=2, kv="fp8_e4m3", scale="token_head", block_size=32),
    dict(hq=128, hkv=1, kv="bf16", scale="none", block_size=16),
    dict(hq=128, hkv=1, kv="fp8_e4m3", scale="tensor", block_size=64),
    dict(hq=16, hkv=2, kv="fp8_e4m3", scale="token_head", block_size=16, nq=4),
], ids=["g8_fp8_bs32", "wide_bf16_bs16", "wide_fp8_bs64", "direct_nq4_bs16"])
def test_shared_and_repeated_blocks(kw):
    # block tables may point several sequences at the same physical blocks (a shared prefix, a
    # whole duplicated sequence) or one sequence at one block many times: all reads, no writes
    kw = dict(kw)
    q = "bf16"
    case = workloads.custom_case(seed=71, device="cuda", batch=4, d=128, seq_lens=[900, 700, 900, 500],
                                 q=q, **kw)
    bs = case.block_size
    table = case.block_table.clone()
    full0 = 900 // bs  # whole blocks of sequence 0
    share = min(full0, 700 // bs) - 1
    table[1, :share] = table[0, :share]          # sequence 1 starts with sequence 0's blocks
    table[2] = table[0]                          # sequence 2 is sequence 0's table (same length)
    nb3 = -(-500 // bs)
    table[3, :nb3] = table[3, 0]                 # sequence 3 reads its first block over and over
    case.block_table = table
    check_case(f"shared_blocks/{kw['kv']}/bs{bs}", case)


@pytest.mark.parametrize("kv", ["int8", "fp8_e4m3"])
@pytest.mark.parametrize("hq,hkv,nq", [(16, 2, 1), (128, 1, 1), (16, 2, 4)], ids=["g8", "wide_g128", "direct_nq4"])
def test_every_code_in_the_cache(kv, hq, hkv, nq):
    # K and V bytes drawn uniformly over every code the format has (INT8: -128..127, -128 included,
    # which row-absmax quantisation never writes; E4M3: every byte but the two NaNs, so +-448 and
    # the subnormals too), with per-token scales: the in-kernel conversions of the whole code set
    # against the oracle's decoder
    case = workloads.custom_case(seed=81, device="cuda", batch=2, hq=hq, hkv=hkv, d=128, seq_lens=[700, 45],
                                 nq=nq, kv=kv, q="bf16", scale="token_head", block_size=32)
    g = torch.Generator(device="cuda").manual_seed(81)
    for t in (case.k_cache, case.v_cache):
        raw = torch.randint(0, 256, t.shape, generator=g, device="cuda", dtype=torch.int32)
        if kv == "fp8_e4m3":
            raw = torch.where((raw & 0x7F) == 0x7F, raw ^ 0x01, raw)  # 0x7F / 0xFF (NaN) -> 0x7E / 0xFE
            t.copy_(raw.to(torch.uint8))
        else:
            t.copy_((raw - 128).to(torch.int8))
    # scales that keep the dequantised values near unit size (codes reach 448 / 128)
    f = 1.0 / 448.0 if kv == "fp8_e4m3" else 1.0 / 128.0
    case.k_scale = f * (0.5 + torch.rand(case.k_scale.shape, generator=g, device="cuda"))
    case.v_scale = f * (0.5 + torch.rand(case.v_scale.shape, generator=g, device="cuda"))
    if kv == "int8":
        assert int(case.k_cache.min()) == -128 and int(case.v_cache.min()) == -128
    check_case(f"every_code/{kv}/g{hq // hkv}/nq{nq}", case)


@pytest.mark.parametrize("hq,hkv,kv,scale", [
    (1024, 1, "fp8_e4m3", "tensor"),    # wide kernel, 32 head blocks of one kv head (8 unit groups)
    (512, 2, "bf16", "none"),           # wide 16-bit path, 256 heads per kv head
    (64, 64, "fp8_e4m3", "token_head"), # one head per kv head, 64 kv heads (16-head kernel)
    (256, 32, "int8", "token_head"),    # 32 kv heads of 8 heads
], ids=["wide_g1024_fp8", "wide_g256x2_bf16", "g1_hkv64_fp8", "g8_hkv32_i8"])
def test_many_heads(hq, hkv, kv, scale):
    case = workloads.custom_case(seed=91, device="cuda", batch=2, hq=hq, hkv=hkv, d=128, seq_lens=[600, 37],
                                 kv=kv, q="bf16", scale=scale, block_size=64)
    check_case(f"heads/{hq}x{hkv}/{kv}", case)
    check_case(f"heads/{hq}x{hkv}/{kv}/p9", case, num_partitions=9)
