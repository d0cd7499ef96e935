"""Dense brute-force attention in pure Python (math.fsum / math.exp), for tiny inputs only.

Independent of both the oracle and the HIP path: it takes *logical* per-sequence K/V (no block
table, no paging), dequantises with torch's own float8/f16/bf16 conversions and evaluates
softmax(q . K^T * scale) . V literally, without subtracting the running max.
"""
import math

import torch


def dequant(x, kind, scale=None):
    """Dense float64 values of a stored K or V tensor [n][hkv][d] (scale: None, float or [n][hkv])."""
    if kind == "fp8_e4m3":
        v = x.view(torch.float8_e4m3fn).to(torch.float64)
    else:
        v = x.to(torch.float64)
    if scale is None:
        return v
    if isinstance(scale, float):
        return v * scale
    return v * scale.to(torch.float64).unsqueeze(-1)


def attention(q, ks, vs, scale):
    """q: [B][Hq][D] float64; ks/vs: list over b of float64 [n_b][Hkv][D].  Returns (out, lse)
    as nested Python lists."""
    B, Hq, D = q.shape
    outs, lses = [], []
    for b in range(B):
        K, V = ks[b], vs[b]
        n = K.shape[0]
        hkv = K.shape[1] if n else 1
        G = Hq // hkv
        ob, lb = [], []
        for h in range(Hq):
            g = h // G
            qh = q[b, h].tolist()
            if n == 0:
                ob.append([0.0] * D)
                lb.append(-math.inf)
                continue
            w = []
            for t in range(n):
                kt = K[t, g].tolist()
                w.append(math.exp(scale * math.fsum(a * c for a, c in zip(qh, kt))))
            L = math.fsum(w)
            Vg = V[:, g].tolist()
            ob.append([math.fsum(w[t] * Vg[t][i] for t in range(n)) / L for i in range(D)])
            lb.append(math.log(L))
        outs.append(ob)
        lses.append(lb)
    return outs, lses


def attention_window(q, ks, vs, scale):
    """A window of M query tokens per sequence: q [B][M][Hq][D] float64; row m of sequence b sits
    at position n_b - M + m and sees tokens [0, n_b - M + m] (none: out 0, lse -inf).  Returns
    (out [B][M][Hq][D], lse [B][M][Hq]) as nested lists, from `attention` on each row's prefix."""
    B, M = q.shape[0], q.shape[1]
    outs, lses = [], []
    for b in range(B):
        n = ks[b].shape[0]
        ob, lb = [], []
        for m in range(M):
            L = max(0, n - M + m + 1)
            o, ls = attention(q[b:b + 1, m], [ks[b][:L]], [vs[b][:L]], scale)
            ob.append(o[0])
            lb.append(ls[0])
        outs.append(ob)
        lses.append(lb)
    return outs, lses
