// fd_direct.hip -- gfx950 partition kernel for 32-column units with K/V loaded straight into
// registers: one wave per unit (one kv head's 32 MFMA columns, e.g. a window of 4 query tokens
// x 8 heads, or 32 heads), E4M3 KV, head_dim 128.
//
// Method (pages): the same online-softmax flash-decoding step as the other partition kernels
// ("从 SGLang Kernel源码到 GPU Trace：DeepSeek V4.1 Flash-Decode", sections 2.2 / 3.1 / 3.2; "第 15
// 章 · GPU Profiling 与 LLM 推理优化实战", sections 15.11-15.13, 15.21 for the verify window of
// several query tokens, each seeing the sequence up to its own position).
//
// gfx950 design:
//   * The 16-head kernel splits 32 columns of a kv head over two waves that both load and
//     convert every K/V tile of that kv head; here one wave covers all 32 columns with the wide
//     kernel's 32x32 MFMA blocks, so each tile is loaded and converted once.  No LDS ring: each
//     wave's unit has its own kv head (or head block), so there is nothing to share, and the
//     operands are loaded straight into the MFMA register layouts, one tile ahead of the compute.
//   * q.k^T: v_mfma_scale_f32_32x32x64_f8f6f4 on the raw E4M3 bytes of K (lane (i, hh) loads 32
//     bytes of token i's row per 64-deep k-step) and q split exactly into E4M3 terms, as in the
//     wide kernel.
//   * p.V: v_mfma_f32_32x32x16_f16; lane (i, hh) loads 4 bytes (d = 4i .. 4i + 3) of 8 token
//     rows per 16-token k-step (two full 128-byte rows per load instruction) and converts them
//     with a byte permute + the hardware E4M3 -> f16 convert.
//   * A window's column (query row m, head h) sees tokens up to seq_len - nq + m: scores past a
//     column's limit are masked before the tile max.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_device.h"

namespace fd {
namespace {

// sequences whose tile prefix sums the workgroup keeps in LDS (larger batches: a wave scan)
constexpr int kDirectLdsBatch = 256;

// K: plain (cached) loads.  A K row's 128-byte line is read by four load instructions of the wave
// (32 bytes of each of 32 rows per instruction), which find it cached; nontemporal loads, which do
// not keep it, streamed this pattern at 5.2 TB/s against 6.1 in an isolated probe, and made the
// 4-token verify kernel 172 us against 143 us.
template <typename T>
__device__ __forceinline__ T ld_dir(const uint8_t *src) {
    return *(const T *)src;
}

// V: nontemporal loads.  Each V load instruction reads two whole 128-byte rows, so nothing of a
// line is read again; streaming them past the caches made the 4-token verify kernel 135 us
// against 143 us with plain loads.
__device__ __forceinline__ uint32_t ld_dir_v(const uint8_t *src) {
    return __builtin_nontemporal_load((const uint32_t *)src);
}

// Four 16-byte LDS reads at a + 0, 32, 64, 96 bytes, complete on return.
__device__ __forceinline__ void lds_read_4x16_d(u32x4_t (&r)[4], uint32_t a) {
    asm volatile(
        "ds_read_b128 %0, %4 offset:0\n\t"
        "ds_read_b128 %1, %4 offset:32\n\t"
        "ds_read_b128 %2, %4 offset:64\n\t"
        "ds_read_b128 %3, %4 offset:96\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a)
        : "memory");
}

// One 16-byte LDS read, complete on return.
__device__ __forceinline__ void lds_read_1x16_d(u32x4_t (&r)[1], uint32_t a) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r[0]) : "v"(a) : "memory");
}

// Two 16-byte LDS reads at a + 0 and a + 32 bytes, complete on return.
__device__ __forceinline__ void lds_read_2x16_d(u32x4_t (&r)[2], uint32_t a) {
    asm volatile(
        "ds_read_b128 %0, %2 offset:0\n\t"
        "ds_read_b128 %1, %2 offset:32\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1])
        : "v"(a)
        : "memory");
}

// Largest of x over lanes i and i ^ 32 (one v_permlane32_swap).  (Elements of the returned pair
// are copied to scalars before any bit cast: a bit cast straight from a vector element reads
// element 0 with this compiler.)
__device__ __forceinline__ float max_halves_d(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t a = r[0], b = r[1];
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

// One tile of one unit in registers, lane (li, lh):
//   k[2 ks + q]: token li's K row, bytes 64 ks + 32 lh + 16 q .. + 15 (FP8 MFMA A operand of k-step ks)
//   v[ks][j]:    token 16 ks + 4 lh + (j < 4 ? j : j + 4)'s V row, bytes 4 li .. 4 li + 3
//   sc:          lane < 32: the k scale of token lane; else the v scale of token lane - 32
struct DTile {
    u32x4_t k[4];
    uint32_t v[2][8];
    float sc;
};

}  // namespace

template <int QT, int SCALE, bool PAGED, bool B16>
__global__ __launch_bounds__(64 * kMaxWavesPerGroup) __attribute__((amdgpu_waves_per_eu(2)))
void direct_partition_kernel(Params p) {
    constexpr int D = 128;
    constexpr int HB = kWideHeadBlock;  // 32 columns per unit
    constexpr int NQT = QT == KV_BF16 ? 2 : 3;  // E4M3 terms of q
    __shared__ __attribute__((aligned(16))) float sh_sc_all[kMaxWavesPerGroup][64];
    __shared__ int sh_prefix[kDirectLdsBatch + 1];
    // q's E4M3 terms of each wave's current segment, [wave][term][k-step][lane] x 32 bytes (held
    // here, not in registers, between the q.k^T steps); sized at launch for the workgroup's waves
    extern __shared__ __attribute__((aligned(32))) i32x8_t sh_q_all[];

    const int wave = uni((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
    const int li = lane & 31, lh = lane >> 5, lh4 = 4 * lh;
    i32x8_t *sh_q = sh_q_all + (size_t)wave * (NQT * 2 * 64);  // [2 t + ks][lane] at (2 t + ks) * 64 + lane
    const int64_t wg = blockIdx.x, W = gridDim.x;
    const int groups = p.groups;
    const bool lds_prefix = p.batch <= kDirectLdsBatch;
    const uint32_t sh_sc = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)sh_sc_all[wave];

    // ---- per-sequence tile prefix sums, once per workgroup
    if (lds_prefix) {
        if (wave == 0) {
            int base = 0;
            for (int b0 = 0; b0 < p.batch; b0 += 64) {
                const int bb = b0 + lane;
                const int t = bb < p.batch ? seq_tiles(p, bb) : 0;
                const int incl = wave_incl_scan(t, lane);
                if (bb < p.batch) sh_prefix[bb] = base + incl - t;
                base += __shfl(incl, 63, 64);
            }
            if (lane == 0) sh_prefix[p.batch] = base;
        }
        __syncthreads();
    }
    const int64_t TT = uni(lds_prefix ? (int64_t)sh_prefix[p.batch] * groups : total_seq_tiles(p, lane) * groups);
    const Split sp = make_split(TT, W);
    const int64_t lo = split_lo(sp, wg), hi = split_lo(sp, wg + 1);
    if (lo >= hi) return;  // workgroup-uniform

    float tensor_k = 1.0f, tensor_v = 1.0f;
    if constexpr (SCALE == SC_TENSOR) {
        tensor_k = p.k_scale[0];
        tensor_v = p.v_scale[0];
    }
    const float qk_scale = p.qk_scale * tensor_k;
    const float sc_floor = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(
                   uint32_t, fmaxf(fabsf(SCALE == SC_TENSOR ? tensor_v : 1.0f) * kMinNormal, kMinNormal))));
    const uint32_t row_bytes = (uint32_t)p.hkv * D;
    const int bsh = PAGED ? (B16 ? 4 : uni(__builtin_ctz((unsigned)p.block_size))) : 0;
    // lane byte offsets in a full tile: K token li, bytes 32 lh ..; V token 4 lh, bytes 4 li ..
    const uint32_t k_lane = __umul24((uint32_t)li, row_bytes) + 32 * lh;
    const uint32_t v_lane = __umul24((uint32_t)lh4, row_bytes) + 4 * li;

    // ---- tile cursor (the same tiles for every wave; each wave its own unit of the unit group)
    int64_t pos = lo;
    int b = 0, Tb = 0, grp = 0, tt = 0, seg = 0, seg_start = 0, n = 0;
    auto locate = [&](int64_t at) {
        if (lds_prefix) {
            int l0 = 0, h0 = p.batch;
            while (h0 - l0 > 1) {
                const int mid = (l0 + h0) >> 1;
                if ((int64_t)sh_prefix[mid] * groups <= at) l0 = mid;
                else h0 = mid;
            }
            b = uni(l0);
            Tb = uni(sh_prefix[b + 1] - sh_prefix[b]);
            const int64_t rel = at - (int64_t)sh_prefix[b] * groups;
            grp = uni((int)(rel / Tb));
            tt = uni((int)(rel % Tb));
        } else {
            int64_t base = 0;
            for (int b0 = 0; b0 < p.batch; b0 += 64) {
                const int bb = b0 + lane;
                const int t = bb < p.batch ? seq_tiles(p, bb) : 0;
                const int incl = wave_incl_scan(t, lane);
                const int64_t excl = base + incl - t;
                const bool here = t > 0 && excl * groups <= at && (excl + t) * groups > at;
                const uint64_t mask = __ballot(here);
                if (mask) {
                    const int src = __builtin_ctzll(mask);
                    b = uni(b0 + src);
                    Tb = uni(__shfl(t, src, 64));
                    const int64_t Pb = base + uni(__shfl(incl, src, 64)) - Tb;
                    const int64_t rel = at - Pb * groups;
                    grp = uni((int)(rel / Tb));
                    tt = uni((int)(rel % Tb));
                    break;
                }
                base += uni(__shfl(incl, 63, 64));
            }
        }
        n = max(0, min(ld_uniform(p.seq_len, b), p.max_seq_len));
    };
    int pf_b = -1, pf_bi = -1;  // block-table entry (sequence, block) read ahead, and its value
    int32_t pf_val = 0;
    struct Desc {
        int64_t row0, row1;  // first cache rows of the tile's two 16-token halves
        int b, kvh, ub, t0, last, nrel, seg;
        bool first, lastseg, whole;
    };
    auto describe = [&](Desc &d) {
        const int u_in = grp * p.wpg + wave;
        d.b = b;
        d.kvh = u_in / p.nhb;
        d.ub = u_in % p.nhb;
        d.t0 = tt * kTile;
        d.nrel = n - d.t0;
        d.last = min(d.nrel, kTile) - 1;
        if constexpr (PAGED && !B16) {
            // the block-table entry was read one tile ahead when it is the one the previous tile
            // asked for, so the tile's loads do not wait for a scalar load
            const int bi = d.t0 >> bsh;
            const int32_t e = (pf_b == b && pf_bi == bi) ? pf_val
                                                        : ld_uniform(p.block_table, (size_t)b * p.max_blocks + bi);
            d.row0 = ((int64_t)e << bsh) + (d.t0 & ((1 << bsh) - 1));
            d.row1 = d.row0 + 16;
            // the next tile's block (an entry of the same table row even past the sequence's end)
            pf_b = b;
            pf_bi = min((d.t0 + kTile) >> bsh, p.max_blocks - 1);
            pf_val = ld_uniform(p.block_table, (size_t)b * p.max_blocks + pf_bi);
        } else if constexpr (PAGED) {
            d.row0 = (int64_t)ld_uniform(p.block_table, (size_t)b * p.max_blocks + (d.t0 >> 4)) << 4;
            d.row1 = d.last < 16 ? d.row0 + 16
                                 : (int64_t)ld_uniform(p.block_table, (size_t)b * p.max_blocks + (d.t0 >> 4) + 1) << 4;
        } else {
            d.row0 = (int64_t)ld_uniform(p.kv_start, b) + d.t0;
            d.row1 = d.row0 + 16;
        }
        d.seg = seg;
        d.first = (tt == seg_start);
        d.lastseg = (tt + 1 == Tb) || (pos + 1 == hi);
        d.whole = (seg_start == 0) && (tt + 1 == Tb);
    };
    auto advance = [&](Desc &d) {
        ++pos;
        if (++tt == Tb) {
            tt = 0;
            seg++;
            seg_start = 0;
            if (++grp == groups) {
                grp = 0;
                do {
                    b++;
                } while ((Tb = lds_prefix ? uni(sh_prefix[b + 1] - sh_prefix[b]) : seq_tiles_u(p, b)) == 0);
                n = max(0, min(ld_uniform(p.seq_len, b), p.max_seq_len));
            }
        }
        describe(d);
    };

    // ---- lane column li of a unit: column col = 32 ub + li of its kv head = query row m of the
    // window, head h of the kv head's group
    struct Col {
        bool valid;
        int m, h;
    };
    auto col_of = [&](int ub) -> Col {
        const int col = ub * HB + li;
        Col r;
        r.valid = col < p.cols;
        if (p.nq == 1) {
            r.m = 0;
            r.h = col;
        } else {
            r.m = col / p.group;
            r.h = col - r.m * p.group;
        }
        return r;
    };

    // ---- per-segment state.  q as exact E4M3 terms (q * 2^eq = t1 + t2 (+ t3)), d = 64 ks + 32 lh
    // + j in byte j of term t, k-step ks (sh_q); the score multiplier carries 2^-eq (and a negative
    // per-tensor scale's sign goes into q)
    float qk_head = qk_scale;
    f32x16_t acc[4];
    float m_run = -INFINITY, l_run = 0.0f;
    int ev = 0;  // per-token v scales: the accumulator holds values / 2^ev
    int win_off = 0;  // a window column's tokens end this many before the sequence's end
    auto load_q = [&](const Desc &d) {
        const Col cl = col_of(d.ub);
        win_off = p.nq - 1 - cl.m;
        const uint16_t *qrow =
            (const uint16_t *)p.q + (((size_t)d.b * p.nq + cl.m) * p.hq + d.kvh * p.group + cl.h) * D + 32 * lh;
        u32x4_t raw[8];
#pragma unroll
        for (int i = 0; i < 8; i++)
            raw[i] = cl.valid ? *(const u32x4_t *)(qrow + 64 * (i >> 2) + 8 * (i & 3)) : u32x4_t{0, 0, 0, 0};
        uint32_t mx = 0;
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const uint32_t w = raw[i][e] & 0x7FFF7FFFu;
                mx = max(mx, max(w & 0xFFFFu, w >> 16));
            }
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32, 64));
        // 2^eq puts the largest |q| of the column in [2^7, 2^8), inside E4M3's range
        int eq = 0;
        if (mx != 0) eq = QT == KV_BF16 ? 7 + 127 - (int)(mx >> 7) : 7 + 15 - (int)(mx >> 10);
        const bool flip = SCALE == SC_TENSOR && qk_scale < 0.0f;
        qk_head = __builtin_amdgcn_ldexpf(flip ? -qk_scale : qk_scale, -eq);
        auto to_f32 = [](uint32_t h) -> float {
            if constexpr (QT == KV_BF16) return __builtin_bit_cast(float, h << 16);
            else return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
        };
        i32x8_t qf8[NQT][2];
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int e2 = 0; e2 < 2; e2++) {
                float x[4];
#pragma unroll
                for (int h = 0; h < 4; h++) {
                    const uint32_t w = raw[i][2 * e2 + (h >> 1)];
                    const float v = to_f32((h & 1) ? (w >> 16) : (w & 0xFFFFu));
                    x[h] = __builtin_amdgcn_ldexpf(flip ? -v : v, eq);
                }
#pragma unroll
                for (int t = 0; t < NQT; t++) {
                    // nearest E4M3 values (exact hardware convert); the remainder is exact in fp32
                    // and has few enough significant bits for the next term
                    i16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2_t{0, 0}, x[0], x[1], 1.0f, false);
                    c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, x[2], x[3], 1.0f, true);
                    const uint32_t cw = __builtin_bit_cast(uint32_t, c);
                    qf8[t][i >> 2][2 * (i & 3) + e2] = (int)cw;
                    if (t + 1 < NQT) {
                        const auto lo2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw, 1.0f, false);
                        const auto hi2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw, 1.0f, true);
                        x[0] -= lo2[0];
                        x[1] -= lo2[1];
                        x[2] -= hi2[0];
                        x[3] -= hi2[1];
                    }
                }
            }
#pragma unroll
        for (int t = 0; t < NQT; t++)
#pragma unroll
            for (int ks = 0; ks < 2; ks++) sh_q[(2 * t + ks) * 64 + lane] = qf8[t][ks];
    };
    auto reset_state = [&]() {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][r] = 0.0f;
        m_run = -INFINITY;
        l_run = 0.0f;
        ev = 0;
    };

    // ---- one tile's loads (rows of a partial last tile past `last` repeat row `last`).  Each
    // load takes a wave-uniform base and a 32-bit lane offset; with 16-token blocks the tile's
    // second half has its own base (the whole tile is in block 0 when it ends before token 16).
    auto issue = [&](DTile &r, const Desc &d) {
        const uint8_t *kb = (const uint8_t *)p.k + (size_t)d.kvh * D + d.row0 * row_bytes;
        const uint8_t *vb = (const uint8_t *)p.v + (size_t)d.kvh * D + d.row0 * row_bytes;
        const int64_t jump = B16 ? (d.row1 - d.row0 - 16) * (int64_t)row_bytes : 0;
        if (d.last == kTile - 1) {
            // a full tile (wave-uniform): the lane offsets are the kernel's fixed ones and each V
            // load's row goes into its scalar base, so no per-load address arithmetic
            const uint8_t *kt = kb + ((B16 && li >= 16) ? jump : 0);
#pragma unroll
            for (int i = 0; i < 4; i++) r.k[i] = ld_dir<u32x4_t>(kt + k_lane + 64 * (i >> 1) + 16 * (i & 1));
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const uint8_t *vrow = vb + (ks ? jump : 0) + (size_t)(16 * ks + (j < 4 ? j : j + 4)) * row_bytes;
                    r.v[ks][j] = ld_dir_v(vrow + v_lane);
                }
            }
        } else {
            {
                const int t = min(li, d.last);
                const uint32_t ko = __umul24((uint32_t)t, row_bytes) + 32 * lh;
                const uint8_t *kt = kb + ((B16 && t >= 16) ? jump : 0);
#pragma unroll
                for (int i = 0; i < 4; i++) r.k[i] = ld_dir<u32x4_t>(kt + ko + 64 * (i >> 1) + 16 * (i & 1));
            }
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const uint8_t *vt = vb + (ks ? jump : 0);  // tokens 16 ks ..: block 1 for ks = 1
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const int t = min(16 * ks + lh4 + (j < 4 ? j : j + 4), d.last);
                    r.v[ks][j] = ld_dir_v(vt + __umul24((uint32_t)t, row_bytes) + 4 * li);
                }
            }
        }
        if constexpr (SCALE == SC_TOKEN_HEAD) {
            const int t = min(li, d.last);
            const int64_t crow = (B16 && t >= 16) ? d.row1 + (t - 16) : d.row0 + t;
            r.sc = (lh ? p.v_scale : p.k_scale)[(size_t)crow * p.hkv + d.kvh];
        }
        // the next tile's loads go out before the current tile's compute (and its waits)
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- one tile: lane (li, lh) holds the scores of tokens 8(r/4) + 4lh + r%4 for column li
    auto compute = [&](const DTile &r, const Desc &d) {
        // the lane's scales through LDS: k scales of the 32 tokens, then the v scales
        if constexpr (SCALE == SC_TOKEN_HEAD) sh_sc_all[wave][lane] = r.sc;
        // ---- scores S[token][column] on FP8 MFMAs from the raw E4M3 bytes
        f32x16_t S;
#pragma unroll
        for (int q = 0; q < 16; q++) S[q] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
            const u32x4_t k0 = r.k[2 * ks], k1 = r.k[2 * ks + 1];
            const i32x8_t a = {(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3],
                               (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
#pragma unroll
            for (int t = 0; t < NQT; t++)
                S = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, sh_q[(2 * t + ks) * 64 + lane], S, 0, 0, 0, 127, 0, 127);
        }
        // scaled in place (per-token k scales four at a time: tokens 8c + 4lh + 0..3)
        if constexpr (SCALE == SC_TOKEN_HEAD) {
#pragma unroll
            for (int c4 = 0; c4 < 4; c4++) {
                u32x4_t raw[1];
                lds_read_1x16_d(raw, sh_sc + 32 * c4 + 16 * lh);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const uint32_t w = raw[0][e];
                    S[4 * c4 + e] *= __builtin_bit_cast(float, w) * qk_head;
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < 16; q++) S[q] *= qk_head;
        }
        float s[16];
#pragma unroll
        for (int q = 0; q < 16; q++) s[q] = S[q];
        // last token column li may see in this tile: a window row m stops nq - 1 - m tokens before
        // the sequence's end (a plain step: the tile's last valid token, whose copies fill the rest)
        int lastc = d.last;
        if (p.nq > 1) lastc = min(d.nrel - win_off, kTile) - 1;
        const bool masked = __any(lastc < kTile - 1);  // wave-uniform
        if (masked) {
#pragma unroll
            for (int q = 0; q < 16; q++)
                if (8 * (q >> 2) + lh4 + (q & 3) > lastc) s[q] = -INFINITY;
        }
        float mt = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
        for (int q = 3; q < 15; q += 2) mt = fmaxf(fmaxf(mt, s[q]), s[q + 1]);
        mt = fmaxf(mt, s[15]);
        mt = max_halves_d(mt);
        int evt = ev;
        if constexpr (SCALE == SC_TOKEN_HEAD) {
            u32x4_t raw[4];
            lds_read_4x16_d(raw, sh_sc + 128 + 16 * lh);
            float vm = 0.0f;
#pragma unroll
            for (int q = 0; q < 16; q += 2) {
                const uint32_t w0 = raw[q >> 2][q & 3], w1 = raw[q >> 2][(q & 3) + 1];
                vm = fmaxf(vm, fmaxf(fabsf(__builtin_bit_cast(float, w0)), fabsf(__builtin_bit_cast(float, w1))));
            }
            vm = max_halves_d(vm);
            evt = uni(vm > 0.0f ? exp2_ceil(vm) : ev);
        }
        const bool emove = evt > ev + kVrefHigh || evt < ev - kVrefLow;
        // (a column with no visible token yet keeps m_run = -inf: the max with -kMaxFloat keeps its
        // weights 0 and its alpha 1 instead of NaN)
        if (__any(mt > m_run + kRescaleSlack) || emove) {  // wave-uniform
            const float m_new = fmaxf(m_run, mt);
            const float dm = fmaxf(m_run, -kMaxFloat) - fmaxf(m_new, -kMaxFloat);
            const float alpha = __builtin_amdgcn_exp2f(dm);
            const float alpha_acc = SCALE == SC_TOKEN_HEAD ? __builtin_amdgcn_exp2f(dm + (float)(ev - evt)) : alpha;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int q = 0; q < 16; q++) acc[i][q] *= alpha_acc;
            m_run = m_new;
            ev = evt;
        }
        float pj[16];
        const float m_ref = fmaxf(m_run, -kMaxFloat) + (SCALE == SC_TOKEN_HEAD ? (float)ev : 0.0f);
#pragma unroll
        for (int q = 0; q < 16; q++) pj[q] = __builtin_amdgcn_exp2f(s[q] - m_ref);
        if constexpr (SCALE == SC_TOKEN_HEAD) {
            float psum = 0.0f;
#pragma unroll
            for (int q = 0; q < 16; q++) psum += pj[q];
            l_run += __builtin_amdgcn_ldexpf(psum, ev);
        } else {
            // l sums the f16 weights p.V multiplies
            float psum = 0.0f;
#pragma unroll
            for (int u = 0; u < 8; u++)
                psum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pack_f16(pj[2 * u], pj[2 * u + 1])),
                                              f16x2_t{(_Float16)1.0f, (_Float16)1.0f}, psum, false);
            l_run += psum;
        }
        // ---- p.V, two 16-token k-steps
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
            float vsc[8];
            if constexpr (SCALE == SC_TOKEN_HEAD) {
                u32x4_t raw[2];
                lds_read_2x16_d(raw, sh_sc + 128 + 64 * ks + 16 * lh);
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const uint32_t w = raw[j >> 2][j & 3];
                    vsc[j] = __builtin_bit_cast(float, w);
                }
            }
            uint32_t pp[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                float p0 = pj[8 * ks + 2 * u], p1 = pj[8 * ks + 2 * u + 1];
                if constexpr (SCALE == SC_TOKEN_HEAD) {
                    p0 *= vsc[2 * u];
                    p1 *= vsc[2 * u + 1];
                }
                pp[u] = pack_f16(p0, p1);
            }
            const u32x4_t pop = {pp[0], pp[1], pp[2], pp[3]};
            uint32_t a[4][4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const uint32_t x = __builtin_amdgcn_perm(r.v[ks][2 * u + 1], r.v[ks][2 * u], 0x05010400u);
                const uint32_t y = __builtin_amdgcn_perm(r.v[ks][2 * u + 1], r.v[ks][2 * u], 0x07030602u);
                a[0][u] = cvt_fp8x2<KV_F16, false>(x);
                a[1][u] = cvt_fp8x2<KV_F16, true>(x);
                a[2][u] = cvt_fp8x2<KV_F16, false>(y);
                a[3][u] = cvt_fp8x2<KV_F16, true>(y);
            }
#pragma unroll
            for (int dt = 0; dt < 4; dt++)
                acc[dt] = mfma32_f16(u32x4_t{a[dt][0], a[dt][1], a[dt][2], a[dt][3]}, pop, acc[dt]);
        }
    };

    // ---- segment result (lane (li, lh) holds d = 4i + dt, i = 8(r/4) + 4lh + r%4, in acc[dt][r])
    auto finalize = [&](const Desc &d) {
        const Col cl = col_of(d.ub);
        const size_t orow_idx = ((size_t)d.b * p.nq + cl.m) * p.hq + d.kvh * p.group + cl.h;
        const float l_tot = l_run + shfl_xor_f(l_run, 32);
        const float sv = (SCALE == SC_TENSOR) ? tensor_v : __builtin_bit_cast(float, (uint32_t)(ev + 127) << 23);
        if (d.whole) {
            if (cl.valid) {
                const size_t orow = orow_idx * D;
                // 0: a window row that sees no token (l_tot >= 1 otherwise)
                const float inv = l_tot > 0.0f ? sv / l_tot : 0.0f;
#pragma unroll
                for (int q = 0; q < 16; q++) {
                    const float v[4] = {acc[0][q] * inv, acc[1][q] * inv, acc[2][q] * inv, acc[3][q] * inv};
                    store_row_chunk<4>(p.out, p.out_dtype, orow + 4 * (8 * (q >> 2) + 4 * lh + (q & 3)), v);
                }
                if (p.lse && lh == 0) p.lse[orow_idx] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
            }
        } else {
            // slot 0: the range's first segment; slot 1: its last.  f16 of value / (largest |value|
            // of the column's row), the scale beside it
            const size_t slot = (((size_t)wg * 2 + (d.seg == 0 ? 0 : 1)) * p.wpg + wave) * HB + li;
            float mx = 0.0f;
#pragma unroll
            for (int q = 0; q < 16; q++)
#pragma unroll
                for (int dt = 0; dt < 4; dt++) mx = fmaxf(mx, fabsf(acc[dt][q] * sv));
            mx = fmaxf(mx, shfl_xor_f(mx, 32));
            const float floor_sc = SCALE == SC_TENSOR ? sc_floor : fmaxf(sv * kMinNormal, kMinNormal);
            const float sc = fmaxf(mx, floor_sc), inv = sv / sc;
            if (cl.valid) {
                uint16_t *dst = (uint16_t *)p.ws_acc + slot * D;
#pragma unroll
                for (int q = 0; q < 16; q++)
                    *(u32x2_t *)(dst + 4 * (8 * (q >> 2) + 4 * lh + (q & 3))) =
                        u32x2_t{pack_f16(acc[0][q] * inv, acc[1][q] * inv), pack_f16(acc[2][q] * inv, acc[3][q] * inv)};
                if (lh == 0) {
                    p.ws_ml[slot] = make_float2(m_run, l_tot);
                    p.ws_sc[slot] = sc;
                }
            }
        }
    };

    // ---- tile stream: two register sets, the next tile's loads in flight while the current
    // one is computed (the same fixed-count loop as the 16-head kernel, so that the compiler's
    // wait before a compute covers only the tile being computed)
    locate(lo);
    seg_start = tt;
    DTile ra, rb;
    Desc da, db;
    const int ntiles = (int)(hi - lo);
    describe(da);
    load_q(da);
    reset_state();
    issue(ra, da);
    for (int step = 0; step < (ntiles - 1) >> 1; step++) {
        advance(db);
        issue(rb, db);
        if ((step & 7) == 0) __builtin_amdgcn_s_barrier();  // bounds the drift between the waves
        compute(ra, da);
        if (da.lastseg) finalize(da);
        if (db.first) {
            load_q(db);
            reset_state();
        }
        advance(da);
        issue(ra, da);
        compute(rb, db);
        if (db.lastseg) finalize(db);
        if (da.first) {
            load_q(da);
            reset_state();
        }
    }
    if ((ntiles & 1) == 0) {
        advance(db);
        issue(rb, db);
        compute(ra, da);
        if (da.lastseg) finalize(da);
        if (db.first) {
            load_q(db);
            reset_state();
        }
        compute(rb, db);
        finalize(db);
    } else {
        compute(ra, da);
        finalize(da);
    }
}

// ---------------------------------------------------------------- host-side dispatch
// Launches one instantiation with `lds` bytes of dynamic LDS; the limit on dynamic LDS is raised
// to the most any launch asks for (8 waves, three q terms), once per instantiation.
template <int QT, int SCALE, bool PAGED, bool B16>
static hipError_t launch_one(const Params &p, size_t lds, hipStream_t stream) {
    auto kern = direct_partition_kernel<QT, SCALE, PAGED, B16>;
    static const hipError_t attr = hipFuncSetAttribute(
        (const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)(kMaxWavesPerGroup * 3 * 2 * 64 * sizeof(i32x8_t)));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3(p.nparts), dim3(64 * p.wpg), lds, stream, p);
    return hipGetLastError();
}

template <int QT, int SCALE>
static hipError_t launch_ds(const Params &p, hipStream_t stream) {
    const size_t lds_q = (size_t)p.wpg * (QT == KV_BF16 ? 2 : 3) * 2 * 64 * sizeof(i32x8_t);
    if (p.block_table && p.block_size == 16) return launch_one<QT, SCALE, true, true>(p, lds_q, stream);
    if (p.block_table) return launch_one<QT, SCALE, true, false>(p, lds_q, stream);
    return launch_one<QT, SCALE, false, false>(p, lds_q, stream);
}

hipError_t launch_direct_partition(const Params &p, int q_dtype, int scale_mode, hipStream_t stream) {
    if (p.d != 128 || p.hb != kWideHeadBlock || p.wpg < 1 || p.wpg > kMaxWavesPerGroup) return hipErrorInvalidValue;
    if (q_dtype == KV_BF16) {
        if (scale_mode == SC_TENSOR) return launch_ds<KV_BF16, SC_TENSOR>(p, stream);
        return launch_ds<KV_BF16, SC_TOKEN_HEAD>(p, stream);
    }
    if (scale_mode == SC_TENSOR) return launch_ds<KV_F16, SC_TENSOR>(p, stream);
    return launch_ds<KV_F16, SC_TOKEN_HEAD>(p, stream);
}

}  // namespace fd
