"""Tiny cases built from *logical* dense K/V, then paged with this file's own scatter.

Used to pin the oracle: the brute force reads the dense tensors, the oracle reads the paged
copy through its block table, so a paging / indexing mistake on either side shows up.
"""
import numpy as np
import torch

FP8_MAX = 448.0
I8_MAX = 127.0


def quant_rows(x):
    amax = x.abs().amax(dim=-1)
    s = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).to(torch.float32)
    y = (x / s.unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    return y, s


def quant_rows_i8(x):
    amax = x.abs().amax(dim=-1)
    s = torch.where(amax > 0, amax / I8_MAX, torch.ones_like(amax)).to(torch.float32)
    y = torch.round(x / s.unsqueeze(-1)).clamp(-I8_MAX, I8_MAX).to(torch.int8)
    return y, s


def _fill(kv):
    """(storage dtype, poison value) of a quantised cache"""
    return (torch.uint8, 0x7F) if kv == "fp8_e4m3" else (torch.int8, -128)


class Dense:
    """Logical per-sequence data: k[b], v[b] stored [n_b][hkv][d]; ks[b], vs[b] scales."""

    def __init__(self, seed, lens, hq, hkv, d, kv="fp8_e4m3", q="bf16", scale="token_head",
                 qmul=1.0):
        g = torch.Generator().manual_seed(seed)
        self.lens, self.hq, self.hkv, self.d = list(lens), hq, hkv, d
        self.kv, self.qd, self.scale = kv, q, (scale if kv in ("fp8_e4m3", "int8") else "none")
        qdt = {"f16": torch.float16, "bf16": torch.bfloat16}[q]
        self.q = (torch.randn(len(lens), hq, d, generator=g) * qmul).to(qdt)
        self.k, self.v, self.ks, self.vs = [], [], [], []
        tensor_scale = None
        qmax = I8_MAX if kv == "int8" else FP8_MAX
        if self.scale == "tensor":
            tensor_scale = (float(np.float32(2.7 / qmax)), float(np.float32(3.1 / qmax)))
        for n in lens:
            for store, sstore, which in ((self.k, self.ks, 0), (self.v, self.vs, 1)):
                x = torch.randn(n, hkv, d, generator=g)
                if kv == "fp8_e4m3":
                    if self.scale == "tensor":
                        s = tensor_scale[which]
                        b = (x / s).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
                        store.append(b)
                        sstore.append(s)
                    else:
                        b, s = quant_rows(x)
                        store.append(b)
                        sstore.append(s)
                elif kv == "int8":
                    if self.scale == "tensor":
                        s = tensor_scale[which]
                        store.append(torch.round(x / s).clamp(-I8_MAX, I8_MAX).to(torch.int8))
                        sstore.append(s)
                    else:
                        b, s = quant_rows_i8(x)
                        store.append(b)
                        sstore.append(s)
                else:
                    store.append(x.to({"f16": torch.float16, "bf16": torch.bfloat16}[kv]))
                    sstore.append(None)
        self.tensor_scale = tensor_scale

    def dense_values(self):
        from bruteforce import dequant
        K = [dequant(self.k[b], self.kv, self.ks[b]) for b in range(len(self.lens))]
        V = [dequant(self.v[b], self.kv, self.vs[b]) for b in range(len(self.lens))]
        return self.q.to(torch.float64), K, V

    def paged(self, bs, seed=1, spare=3, max_blocks=None):
        """Scatter into [num_blocks][bs][hkv][d] at a random block placement; returns kwargs for
        oracle.Problem (unused storage is NaN / 0x7F, unused table entries -1)."""
        rng = np.random.default_rng(seed)
        nb = [(n + bs - 1) // bs for n in self.lens]
        total = sum(nb) + spare
        place = rng.permutation(total)
        mb = max_blocks or max(1, max(nb) if nb else 1)
        table = np.full((len(self.lens), mb), -1, dtype=np.int32)
        quant = self.kv in ("fp8_e4m3", "int8")
        sdt = _fill(self.kv)[0] if quant else self.k[0].dtype
        K = torch.empty(total, bs, self.hkv, self.d, dtype=sdt)
        V = torch.empty_like(K)
        if quant:
            K.fill_(_fill(self.kv)[1])
            V.fill_(_fill(self.kv)[1])
        else:
            K.fill_(float("nan"))
            V.fill_(float("nan"))
        KS = torch.full((total, bs, self.hkv), float("nan"))
        VS = torch.full((total, bs, self.hkv), float("nan"))
        off = 0
        for b, n in enumerate(self.lens):
            for j in range(nb[b]):
                p = int(place[off + j])
                table[b, j] = p
                t0, t1 = j * bs, min(n, (j + 1) * bs)
                K[p, : t1 - t0] = self.k[b][t0:t1]
                V[p, : t1 - t0] = self.v[b][t0:t1]
                if self.scale == "token_head":
                    KS[p, : t1 - t0] = self.ks[b][t0:t1]
                    VS[p, : t1 - t0] = self.vs[b][t0:t1]
            off += nb[b]
        kw = self._common()
        kw.update(k_cache=K, v_cache=V, block_table=torch.from_numpy(table), block_size=bs)
        if self.scale == "token_head":
            kw.update(k_scale=KS, v_scale=VS)
        return kw

    def contiguous(self, gap=2):
        quant = self.kv in ("fp8_e4m3", "int8")
        rows = sum(self.lens) + gap * (len(self.lens) + 1)
        sdt = _fill(self.kv)[0] if quant else self.k[0].dtype
        K = torch.empty(rows, self.hkv, self.d, dtype=sdt)
        V = torch.empty_like(K)
        if quant:
            K.fill_(_fill(self.kv)[1])
            V.fill_(_fill(self.kv)[1])
        else:
            K.fill_(float("nan"))
            V.fill_(float("nan"))
        KS = torch.full((rows, self.hkv), float("nan"))
        VS = torch.full((rows, self.hkv), float("nan"))
        starts, r = [], gap
        for b, n in enumerate(self.lens):
            starts.append(r)
            K[r:r + n] = self.k[b]
            V[r:r + n] = self.v[b]
            if self.scale == "token_head":
                KS[r:r + n] = self.ks[b]
                VS[r:r + n] = self.vs[b]
            r += n + gap
        kw = self._common()
        kw.update(k_cache=K, v_cache=V, kv_start=torch.tensor(starts, dtype=torch.int32))
        if self.scale == "token_head":
            kw.update(k_scale=KS, v_scale=VS)
        return kw

    def _common(self):
        kw = dict(q=self.q, seq_len=torch.tensor(self.lens, dtype=torch.int32), batch=len(self.lens),
                  hq=self.hq, hkv=self.hkv, d=self.d, q_dtype=self.qd, kv_dtype=self.kv,
                  scale_mode=self.scale, softmax_scale=1.0 / float(np.sqrt(self.d)))
        if self.scale == "tensor":
            kw.update(k_scale=torch.tensor([self.tensor_scale[0]], dtype=torch.float32),
                      v_scale=torch.tensor([self.tensor_scale[1]], dtype=torch.float32))
        return kw
