"""Seeded synthetic inputs for one flash-decoding attention step.

This module only *makes data*: sequence lengths, Q, paged or contiguous K/V caches
(optionally FP8 E4M3 with fp32 scales), block tables.  It holds none of the
attention arithmetic, and both the HIP path and the fp64 oracle consume exactly
the tensors it returns.  Nothing here imports either side.

Workloads (sizes as specified for the decode workloads this library targets):

* ``tiny_mqa_f16``      batch 2, 4 q heads / 1 kv head, head_dim 64, seq_len {37, 100},
                        contiguous fp16 KV.
* ``gqa_bf16``          batch 16, 32 q / 8 kv heads, head_dim 128, seq_len ~ U[512, 4096],
                        bf16 KV, block_size 64, randomly permuted block table.
* ``fp8_32k``           batch 32, 64 q / 8 kv heads, head_dim 128, seq_len ~ logU[1K, 32K],
                        E4M3 KV with per-(token, kv-head) fp32 scales, block_size 64.
* ``mqa_fp8_128k``      batch 4, seq_len 131072, 128 q / 1 kv head, head_dim 128,
                        E4M3 KV with one per-tensor scale, block_size 64.
* ``ragged_fp8``        batch 256, 90 % seq_len ~ U[256, 2048] and 10 % ~ U[32K, 128K],
                        32 q / 8 kv heads, head_dim 128, E4M3 KV, block_size 32, shuffled blocks.
* ``int8_32k``          ``fp8_32k`` with INT8 KV (per-(token, kv-head) scales).
* ``mqa_i8_128k``       ``mqa_fp8_128k`` with INT8 KV (one per-tensor scale).
* ``mqa_bf16_64k``      batch 4, seq_len 65536, 128 q / 1 kv head, head_dim 128, bf16 KV
                        (the same KV bytes as ``mqa_fp8_128k``), block_size 64.
* ``verify_fp8_32k``    ``fp8_32k`` with a window of 4 query tokens per sequence (a speculative-
                        decoding verify pass over 4 draft tokens already in the cache).

Recipe (readings where the pages leave the inputs open):

* Sequence lengths come from ``numpy.random.Generator(PCG64(seed))``; integer bounds are
  inclusive; log-uniform is ``round(exp(U(ln a, ln b)))``; the ragged mix has exactly
  ``round(0.1 * batch)`` long sequences at seeded positions.
* Q, K, V source values are N(0, 1) fp32 from ``torch.Generator(device).manual_seed(seed)``
  (the stream depends on the device; every consumer gets the same tensors, so this is fine),
  times optional magnitudes ``q_mag`` / ``k_mag`` / ``v_mag`` (default 1) applied before
  rounding or quantisation: range tests of the kernels at data far from unit size.
* FP8 rows are quantised row-absmax style, the way activations are quantised in the
  "小算子融合 residual + RMSNorm + quant" passage of the ch.15 profiling page:
  ``scale = amax / 448`` (1 if amax is 0), ``byte = RNE(x / scale)`` via torch's own
  ``float8_e4m3fn`` cast.  Per-tensor scale takes amax over the whole tensor.  INT8 rows the
  same way with ``scale = amax / 127`` and ``code = round-half-even(x / scale)`` in [-127, 127].
* Paged caches hold ``sum(ceil(n_b / bs))`` live blocks plus 8 spare blocks, placed by a random
  permutation (the "fragmented" page placement of the ch.15 paged-KV scan passage).
  Everything the kernels must never read is poisoned: slots past ``seq_len`` in the last block,
  spare blocks (NaN payload, NaN scales) and unused block-table entries (-1).
* Contiguous caches put sequences back to back with 3 NaN rows between them (``kv_start``).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

FP8_MAX = 448.0
SPARE_BLOCKS = 8
CONTIG_GAP_ROWS = 3

# dtype names shared by the binding, the oracle wrapper and the tests
KV_DTYPES = ("f16", "bf16", "fp8_e4m3", "int8")
QUANTISED = ("fp8_e4m3", "int8")
INT8_MAX = 127.0
Q_DTYPES = ("f16", "bf16")
SCALE_MODES = ("none", "tensor", "token_head")

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}

WORKLOADS = {
    "tiny_mqa_f16": dict(batch=2, hq=4, hkv=1, d=64, lens=("fixed_list", [37, 100]), kv="f16",
                         q="f16", block_size=0, scale="none", paged=False),
    "gqa_bf16": dict(batch=16, hq=32, hkv=8, d=128, lens=("uniform", 512, 4096), kv="bf16",
                     q="bf16", block_size=64, scale="none", paged=True),
    "fp8_32k": dict(batch=32, hq=64, hkv=8, d=128, lens=("loguniform", 1024, 32768), kv="fp8_e4m3",
                    q="bf16", block_size=64, scale="token_head", paged=True),
    "mqa_fp8_128k": dict(batch=4, hq=128, hkv=1, d=128, lens=("fixed", 131072), kv="fp8_e4m3",
                         q="bf16", block_size=64, scale="tensor", paged=True),
    "ragged_fp8": dict(batch=256, hq=32, hkv=8, d=128,
                       lens=("mix", 0.1, (256, 2048), (32768, 131072)), kv="fp8_e4m3",
                       q="bf16", block_size=32, scale="token_head", paged=True),
    "int8_32k": dict(batch=32, hq=64, hkv=8, d=128, lens=("loguniform", 1024, 32768), kv="int8",
                     q="bf16", block_size=64, scale="token_head", paged=True),
    "mqa_i8_128k": dict(batch=4, hq=128, hkv=1, d=128, lens=("fixed", 131072), kv="int8",
                        q="bf16", block_size=64, scale="tensor", paged=True),
    "mqa_bf16_64k": dict(batch=4, hq=128, hkv=1, d=128, lens=("fixed", 65536), kv="bf16",
                         q="bf16", block_size=64, scale="none", paged=True),
    "verify_fp8_32k": dict(batch=32, hq=64, hkv=8, d=128, lens=("loguniform", 1024, 32768),
                           kv="fp8_e4m3", q="bf16", block_size=64, scale="token_head", paged=True,
                           nq=4),
}


@dataclasses.dataclass
class Case:
    """One decode step's inputs.  Tensors live on ``device``; ``seq_lens`` is a host list."""
    name: str
    batch: int
    hq: int
    hkv: int
    d: int
    kv_dtype: str
    q_dtype: str
    scale_mode: str
    block_size: int            # 0 in contiguous mode
    paged: bool
    seq_lens: list
    max_seq_len: int
    q: torch.Tensor            # [B][Hq][D] f16/bf16
    k_cache: torch.Tensor      # paged [NB][bs][Hkv][D] / contiguous [rows][Hkv][D]; uint8 for FP8
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor]   # fp32: [1] or paged [NB][bs][Hkv] / contiguous [rows][Hkv]
    v_scale: Optional[torch.Tensor]
    block_table: Optional[torch.Tensor]  # int32 [B][max_blocks] (paged)
    kv_start: Optional[torch.Tensor]     # int32 [B] (contiguous)
    seq_len: torch.Tensor                # int32 [B]
    max_blocks: int
    softmax_scale: float
    nq: int = 1                          # query tokens per sequence (q is [B][nq][Hq][D] when > 1)

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    def kv_elem_bytes(self) -> int:
        return 1 if self.kv_dtype in QUANTISED else 2

    def kv_read_bytes(self) -> int:
        """K+V payload plus scale bytes the method must read for this step."""
        toks = sum(self.seq_lens)
        b = toks * self.hkv * self.d * self.kv_elem_bytes() * 2
        if self.scale_mode == "token_head":
            b += toks * self.hkv * 4 * 2
        elif self.scale_mode == "tensor":
            b += 8
        return b

    def to(self, device) -> "Case":
        kw = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            kw[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Case(**kw)


def draw_seq_lens(spec, batch: int, rng: np.random.Generator) -> list:
    kind = spec[0]
    if kind == "fixed_list":
        lens = list(spec[1])
        assert len(lens) == batch
        return [int(x) for x in lens]
    if kind == "fixed":
        return [int(spec[1])] * batch
    if kind == "uniform":
        return [int(x) for x in rng.integers(spec[1], spec[2], size=batch, endpoint=True)]
    if kind == "loguniform":
        u = rng.uniform(math.log(spec[1]), math.log(spec[2]), size=batch)
        return [int(x) for x in np.clip(np.rint(np.exp(u)), spec[1], spec[2])]
    if kind == "mix":
        frac, short, long_ = spec[1], spec[2], spec[3]
        n_long = int(round(frac * batch))
        long_pos = set(int(x) for x in rng.choice(batch, size=n_long, replace=False))
        short_l = rng.integers(short[0], short[1], size=batch, endpoint=True)
        long_l = rng.integers(long_[0], long_[1], size=batch, endpoint=True)
        return [int(long_l[i]) if i in long_pos else int(short_l[i]) for i in range(batch)]
    raise ValueError(f"unknown length spec {spec!r}")


def _nan_bits(dtype: str) -> int:
    # int8 has no NaN: -128 lies outside the quantised range [-127, 127] (and its scales are NaN)
    return {"f16": 0x7E00, "bf16": 0x7FC0, "fp8_e4m3": 0x7F, "int8": 0x80}[dtype]


def _quant_rows(x: torch.Tensor):
    """Row-absmax FP8 quantisation of the last dim: returns (uint8 bytes, fp32 scales)."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp_(-FP8_MAX, FP8_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8), scale.to(torch.float32)


def _quant_tensor(x: torch.Tensor, amax: float):
    scale = amax / FP8_MAX if amax > 0 else 1.0
    scale = float(np.float32(scale))
    y = (x / scale).clamp_(-FP8_MAX, FP8_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8), scale


def _quant_rows_i8(x: torch.Tensor):
    """Row-absmax INT8 quantisation of the last dim: returns (int8 codes, fp32 scales)."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / INT8_MAX, torch.ones_like(amax))
    y = torch.round(x / scale.unsqueeze(-1)).clamp_(-INT8_MAX, INT8_MAX)
    return y.to(torch.int8), scale.to(torch.float32)


def _quant_tensor_i8(x: torch.Tensor, amax: float):
    scale = float(np.float32(amax / INT8_MAX if amax > 0 else 1.0))
    y = torch.round(x / scale).clamp_(-INT8_MAX, INT8_MAX)
    return y.to(torch.int8), scale


def _fill_store(n_rows: int, hkv: int, d: int, kv: str, scale: str, device, gen,
                chunk_rows: int = 1 << 19, k_mag: float = 1.0, v_mag: float = 1.0):
    """Generate K and V row stores ([n_rows][hkv][d]) plus scales, chunk by chunk; the N(0, 1)
    sources are multiplied by k_mag / v_mag first."""
    storage_dtype = {"fp8_e4m3": torch.uint8, "int8": torch.int8}.get(kv) or _TORCH[kv]
    k = torch.empty((n_rows, hkv, d), dtype=storage_dtype, device=device)
    v = torch.empty_like(k)
    ks = vs = None
    if scale == "token_head":
        ks = torch.empty((n_rows, hkv), dtype=torch.float32, device=device)
        vs = torch.empty_like(ks)
    if scale == "tensor":
        # per-tensor amax needs the whole tensor: generate at once (sizes here allow it)
        ksrc = torch.randn((n_rows, hkv, d), generator=gen, device=device, dtype=torch.float32) * k_mag
        vsrc = torch.randn((n_rows, hkv, d), generator=gen, device=device, dtype=torch.float32) * v_mag
        quant = _quant_tensor_i8 if kv == "int8" else _quant_tensor
        kb, kscale = quant(ksrc, float(ksrc.abs().max()))
        vb, vscale = quant(vsrc, float(vsrc.abs().max()))
        k.copy_(kb)
        v.copy_(vb)
        del ksrc, vsrc
        ks = torch.tensor([kscale], dtype=torch.float32, device=device)
        vs = torch.tensor([vscale], dtype=torch.float32, device=device)
        return k, v, ks, vs
    for r0 in range(0, n_rows, chunk_rows):
        r1 = min(n_rows, r0 + chunk_rows)
        for dst, sdst, mag in ((k, ks, k_mag), (v, vs, v_mag)):
            src = torch.randn((r1 - r0, hkv, d), generator=gen, device=device, dtype=torch.float32)
            if mag != 1.0:
                src *= mag
            if kv in QUANTISED:
                b, s = (_quant_rows_i8 if kv == "int8" else _quant_rows)(src)
                dst[r0:r1] = b
                sdst[r0:r1] = s
            else:
                dst[r0:r1] = src.to(storage_dtype)
    return k, v, ks, vs


def _poison_rows(t: torch.Tensor, rows: torch.Tensor, nan_bits: int):
    if rows.numel() == 0:
        return
    if t.dtype == torch.uint8:
        t[rows] = nan_bits
    elif t.dtype == torch.int8:
        t[rows] = int(np.uint8(nan_bits).view(np.int8))
    elif t.dtype == torch.float32:
        t[rows] = float("nan")
    else:
        t.view(torch.int16)[rows] = np.int16(np.uint16(nan_bits).view(np.int16))


def make_case(name: str = "fp8_32k", seed: int = 0, device="cpu", seq_lens=None,
              **overrides) -> Case:
    """Build the inputs of one named workload (fields can be overridden, e.g. batch, lens)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    return _build(name, cfg, seed, device, seq_lens)


def _build(name, cfg, seed, device, seq_lens) -> Case:
    rng = np.random.Generator(np.random.PCG64(seed))
    batch = cfg["batch"]
    if seq_lens is None:
        seq_lens = draw_seq_lens(cfg["lens"], batch, rng)
    seq_lens = [int(x) for x in seq_lens]
    assert len(seq_lens) == batch
    hq, hkv, d = cfg["hq"], cfg["hkv"], cfg["d"]
    kv, qd, scale, paged = cfg["kv"], cfg["q"], cfg["scale"], cfg["paged"]
    bs = cfg["block_size"] if paged else 0
    if kv not in QUANTISED:
        scale = "none"
    max_seq_len = int(cfg.get("max_seq_len", max(seq_lens) if seq_lens else 0))
    gen = torch.Generator(device=device).manual_seed(seed)
    nq = int(cfg.get("nq", 1))
    qshape = (batch, nq, hq, d) if nq > 1 else (batch, hq, d)
    q = (torch.randn(qshape, generator=gen, device=device, dtype=torch.float32) *
         float(cfg.get("q_mag", 1.0))).to(_TORCH[qd])
    mags = dict(k_mag=float(cfg.get("k_mag", 1.0)), v_mag=float(cfg.get("v_mag", 1.0)))
    nan = _nan_bits(kv)
    if paged:
        nb_per = [(n + bs - 1) // bs for n in seq_lens]
        live = sum(nb_per)
        num_blocks = live + SPARE_BLOCKS
        max_blocks = max(1, (max_seq_len + bs - 1) // bs)
        perm = rng.permutation(num_blocks) if cfg.get("shuffle", True) else np.arange(num_blocks)
        table = np.full((batch, max_blocks), -1, dtype=np.int32)
        off = 0
        for b, nb in enumerate(nb_per):
            table[b, :nb] = perm[off:off + nb]
            off += nb
        spare = perm[live:]
        k, v, ks, vs = _fill_store(num_blocks * bs, hkv, d, kv, scale, device, gen, **mags)
        # poison rows that must never be read
        dead = [np.arange(p * bs, (p + 1) * bs) for p in spare]
        for b, n in enumerate(seq_lens):
            if n % bs:
                p = table[b, nb_per[b] - 1]
                dead.append(np.arange(p * bs + n % bs, (p + 1) * bs))
        dead_rows = torch.from_numpy(np.concatenate(dead) if dead else np.zeros(0, np.int64)).to(device)
        for t in (k, v):
            _poison_rows(t, dead_rows, nan)
        if scale == "token_head":
            for t in (ks, vs):
                _poison_rows(t, dead_rows, 0)
            ks = ks.view(num_blocks, bs, hkv)
            vs = vs.view(num_blocks, bs, hkv)
        k = k.view(num_blocks, bs, hkv, d)
        v = v.view(num_blocks, bs, hkv, d)
        block_table = torch.from_numpy(table).to(device)
        kv_start = None
    else:
        starts, rows = [], 0
        for n in seq_lens:
            rows += CONTIG_GAP_ROWS
            starts.append(rows)
            rows += n
        rows += CONTIG_GAP_ROWS
        k, v, ks, vs = _fill_store(rows, hkv, d, kv, scale, device, gen, **mags)
        live = np.zeros(rows, dtype=bool)
        for s, n in zip(starts, seq_lens):
            live[s:s + n] = True
        dead_rows = torch.from_numpy(np.nonzero(~live)[0]).to(device)
        for t in (k, v):
            _poison_rows(t, dead_rows, nan)
        if scale == "token_head":
            for t in (ks, vs):
                _poison_rows(t, dead_rows, 0)
        block_table = None
        max_blocks = 0
        kv_start = torch.tensor(starts, dtype=torch.int32, device=device)
    seq_len = torch.tensor(seq_lens, dtype=torch.int32, device=device)
    return Case(name=name, batch=batch, hq=hq, hkv=hkv, d=d, kv_dtype=kv, q_dtype=qd,
                scale_mode=scale, block_size=bs, paged=paged, seq_lens=seq_lens,
                max_seq_len=max_seq_len, q=q, k_cache=k, v_cache=v, k_scale=ks, v_scale=vs,
                block_table=block_table, kv_start=kv_start, seq_len=seq_len,
                max_blocks=max_blocks, softmax_scale=1.0 / math.sqrt(d), nq=nq)


def custom_case(seed=0, device="cpu", *, batch, hq, hkv, d, seq_lens, kv="fp8_e4m3", q="bf16",
                block_size=64, scale="token_head", paged=True, shuffle=True, max_seq_len=None, nq=1,
                q_mag=1.0, k_mag=1.0, v_mag=1.0):
    """A case with explicit shapes (edge cases and small parity sizes); ``*_mag`` multiply the
    N(0, 1) sources of q, K and V."""
    cfg = dict(batch=batch, hq=hq, hkv=hkv, d=d, lens=("fixed_list", list(seq_lens)), kv=kv,
               q=q, block_size=block_size, scale=scale, paged=paged, shuffle=shuffle, nq=nq,
               q_mag=q_mag, k_mag=k_mag, v_mag=v_mag)
    if max_seq_len is not None:
        cfg["max_seq_len"] = max_seq_len
    return _build("custom", cfg, seed, device, list(seq_lens))
