"""Host-side argument checks of the Python binding (CPU only, nothing is launched).

The C ABI takes plain pointers, so it cannot see a tensor's dtype, layout or element count; the
binding checks them before any call.  Each test takes a valid seeded case and breaks one thing:
the call must raise ValueError naming it, before anything reaches the GPU."""
import pytest
import torch

import decode_attention_06_amd as fd
import workloads


def _case(**kw):
    base = dict(batch=3, hq=16, hkv=2, d=128, seq_lens=[70, 1, 200], kv="fp8_e4m3", q="bf16",
                scale="token_head", block_size=64)
    base.update(kw)
    return workloads.custom_case(seed=0, device="cpu", **base)


def _call(c, **over):
    args = dict(q=c.q, k_cache=c.k_cache, v_cache=c.v_cache, seq_len=c.seq_len,
                block_table=c.block_table, kv_start=c.kv_start, kv_dtype=c.kv_dtype,
                scale_mode=c.scale_mode, k_scale=c.k_scale, v_scale=c.v_scale, num_kv_heads=c.hkv,
                block_size=c.block_size, max_seq_len=c.max_seq_len)
    args.update(over)
    q, k, v, sl = args.pop("q"), args.pop("k_cache"), args.pop("v_cache"), args.pop("seq_len")
    fd.check_decode_args(q, k, v, sl, **args)


@pytest.mark.parametrize("kw", [
    {}, dict(kv="int8"), dict(scale="tensor"), dict(kv="bf16", scale="none"), dict(kv="f16", q="f16"),
    dict(paged=False, block_size=0), dict(block_size=16), dict(nq=3),
])
def test_valid_inputs_pass(kw):
    c = _case(**kw)
    _call(c)
    # and the full call gets past the checks to the device test (these are CPU tensors)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        fd.decode_case(c)


def test_int64_seq_len_rejected():
    c = _case()
    with pytest.raises(ValueError, match="seq_len must be a contiguous int32"):
        _call(c, seq_len=c.seq_len.long())


def test_seq_len_wrong_length_rejected():
    c = _case()
    with pytest.raises(ValueError, match="seq_len"):
        _call(c, seq_len=c.seq_len[:2].contiguous())


def test_non_contiguous_seq_len_rejected():
    c = _case()
    sl = torch.stack([c.seq_len, c.seq_len], 1)[:, 0]
    assert not sl.is_contiguous()
    with pytest.raises(ValueError, match="seq_len"):
        _call(c, seq_len=sl)


def test_block_table_dtype_and_shape_rejected():
    c = _case()
    with pytest.raises(ValueError, match="block_table"):
        _call(c, block_table=c.block_table.long())
    with pytest.raises(ValueError, match="block_table"):
        _call(c, block_table=c.block_table[:2].contiguous())
    with pytest.raises(ValueError, match="block_table"):
        _call(c, block_table=c.block_table.t())


def test_block_table_too_short_for_max_seq_len_rejected():
    c = _case()
    with pytest.raises(ValueError, match="exceeds the table"):
        _call(c, max_seq_len=c.block_table.shape[1] * c.block_size + 1)


def test_both_or_neither_table_and_kv_start_rejected():
    c = _case()
    with pytest.raises(ValueError, match="exactly one of"):
        _call(c, kv_start=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="exactly one of"):
        _call(c, block_table=None)


def test_kv_start_dtype_rejected():
    c = _case(paged=False, block_size=0)
    with pytest.raises(ValueError, match="kv_start"):
        _call(c, kv_start=c.kv_start.long())


def test_cache_dtype_must_hold_kv_dtype():
    c = _case()
    # an FP8 cache labelled bf16 (would be read as twice as many bytes)
    with pytest.raises(ValueError, match="does not hold kv_dtype"):
        _call(c, kv_dtype="bf16", scale_mode="none", k_scale=None, v_scale=None)
    ci = _case(kv="int8")
    with pytest.raises(ValueError, match="does not hold kv_dtype"):
        _call(ci, kv_dtype="fp8_e4m3")


def test_cache_shape_rejected():
    c = _case()
    with pytest.raises(ValueError, match="k_cache must be"):
        _call(c, num_kv_heads=4)
    with pytest.raises(ValueError, match="k_cache must be"):
        _call(c, k_cache=c.k_cache[..., :64].contiguous(), v_cache=c.v_cache[..., :64].contiguous())
    with pytest.raises(ValueError, match="block_size is"):
        _call(c, block_size=32)
    with pytest.raises(ValueError, match="shapes differ"):
        _call(c, v_cache=c.v_cache[:-1].contiguous())
    with pytest.raises(ValueError, match="contiguous"):
        _call(c, k_cache=c.k_cache.transpose(0, 1))


def test_scale_counts_rejected():
    c = _case()
    # a per-tensor-sized scale with per-token mode would be read past its end
    with pytest.raises(ValueError, match="k_scale must be"):
        _call(c, k_scale=torch.ones(1))
    with pytest.raises(ValueError, match="v_scale must be"):
        _call(c, v_scale=c.v_scale.double())
    with pytest.raises(ValueError, match="v_scale must be"):
        _call(c, v_scale=None)
    ct = _case(scale="tensor")
    with pytest.raises(ValueError, match="k_scale must be"):
        _call(ct, k_scale=torch.ones(2))


def test_scale_mode_consistent_with_kv_dtype():
    c = _case()
    with pytest.raises(ValueError, match="needs k and v scales"):
        _call(c, scale_mode="none")
    cb = _case(kv="bf16", scale="none")
    with pytest.raises(ValueError, match="takes no scales"):
        _call(cb, scale_mode="tensor")


def test_q_dtype_and_layout_rejected():
    c = _case()
    with pytest.raises(ValueError, match="q must be"):
        _call(c, q=c.q.float())
    with pytest.raises(ValueError, match="q must be"):
        _call(c, q=c.q.transpose(0, 1))


def test_kv_append_checks():
    c = _case()
    kn = torch.zeros(3, 2, 128)
    pos = torch.tensor([70, 1, 200], dtype=torch.int32)
    kw = dict(kv_dtype="fp8_e4m3", block_table=c.block_table, block_size=64, scale_mode="token_head",
              k_scale=c.k_scale, v_scale=c.v_scale)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        fd.kv_append(kn, kn, c.k_cache, c.v_cache, pos, **kw)
    with pytest.raises(ValueError, match="pos must be"):
        fd.kv_append(kn, kn, c.k_cache, c.v_cache, pos.long(), **kw)
    with pytest.raises(ValueError, match="k_cache must be"):
        fd.kv_append(kn, kn, c.k_cache.view(torch.int8), c.v_cache, pos, **kw)
    with pytest.raises(ValueError, match="rows must be"):
        fd.kv_append(torch.zeros(3, 2, 64), torch.zeros(3, 2, 64), c.k_cache, c.v_cache, pos, **kw)
    with pytest.raises(ValueError, match="k_scale must be"):
        fd.kv_append(kn, kn, c.k_cache, c.v_cache, pos, **{**kw, "k_scale": torch.ones(1)})
