// fd_kernels.hip -- gfx950 (MI355X, CDNA4) kernels of one flash-decoding attention step.
//
// Method (pages):
//   * "SGLang Prefill 性能优化：用 GPU Trace 剖析 FlashAttention 内核瓶颈", section 2.2: keys and
//     values are consumed block by block; per block the scores q.k^T*scale update a running
//     max m, the previous accumulator and running sum are rescaled by exp(m_old - m_new), and
//     exp(s - m_new) weights are summed into l and multiplied into V.
//   * "从 SGLang Kernel源码到 GPU Trace：DeepSeek V4.1 Flash-Decode", sections 2.2 / 3.1 / 3.2:
//     ragged batch located by seq_len (work follows each sequence's own length), KV processed
//     in 32/64-token blocks, FP8 KV converted to wider floats right after the load, and
//     per-block partial results written out before the final normalisation.
//   * "第 15 章 · GPU Profiling 与 LLM 推理优化实战", sections 15.11-15.13 and 15.26: per-token
//     KV scales read with the payload, one KV head serving a group of query heads, paged
//     addressing through the block table, split-K partials.
//
// The split-KV combine (log-sum-exp merge of per-split (m, l, acc)) is the same recurrence
// applied to whole partial states.
//
// gfx950 design (differs from the pages' Hopper kernel, which stages KV through shared memory
// with async copies and runs mma.sync on 32-wide warps):
//   * Persistent workgroups of up to 8 wave64s, one wave per unit (sequence, kv head, 16-head
//     block) of a unit group; each workgroup streams an equal share of the step's 32-token tiles
//     (balanced over the sum of all sequences' lengths, computed on the device).  KV is never
//     staged in LDS: every MFMA operand is loaded straight from HBM into the register layout the
//     instruction wants, one tile ahead of the compute.
//   * q.k^T runs on v_mfma_f32_16x16x32_{bf16,f16}: A = 16 tokens x 32 d of K (converted to
//     q's type -- exact for E4M3), B = 32 d x 16 heads of q.  Lane (g = lane/16, c = lane%16)
//     of the C tile holds the scores of tokens 4g..4g+3 of the 16-token half for head c.
//   * p.V runs on v_mfma_f32_16x16x32_f16 (E4M3 and f16 V; bf16 V uses bf16 with p split in
//     hi + lo parts): A = V^T (16 d x 32 tokens), B = P^T (32 tokens x 16 heads).  The token
//     order of the contraction is chosen so that the q.k^T C tile *is* the B operand of p.V
//     (lane g holds tokens {4g..4g+3, 16+4g..16+4g+3}), and the d order so that each lane's
//     V operand is one contiguous 8-element chunk of 8 token rows (one coalesced load per row;
//     a byte/half permute plus the hardware E4M3 -> f16 convert builds the operand).
//   * Scores are kept in log2 units (scale folded with log2 e) and exponentiated with v_exp_f32.
#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include "fd_device.h"

namespace fd {

// Element index (within a head_dim row) of MFMA k-slot (group g, step kk, position j) of the
// q.k^T contraction.  E = elements per 16-byte load of K; each lane loads 16 bytes at element
// offset 4E*L + E*g for L = 0 .. D/(4E)-1, so one load instruction covers 4E contiguous
// elements of 16 rows.
template <int E>
__device__ __forceinline__ int qk_elem(int g, int kk) {
    constexpr int steps_per_load = E / 8;
    return 4 * E * (kk / steps_per_load) + E * g + 8 * (kk % steps_per_load);
}

// Tile-relative token of k-slot j (0..7) of lane group g in the p.V contraction; equals the
// token whose score sits in C slot (j & 3) of half (j >> 2) of the q.k^T result.
__device__ __forceinline__ int pv_token(int g, int j) { return (j < 4) ? 4 * g + j : 12 + 4 * g + j; }

// ---------------------------------------------------------------- split-KV partition kernel
//
// Grid: W workgroups of wpg waves.  Workgroup w takes tile range w of the balanced split; wave i
// runs unit i of each unit group in it.  The range is one stream of tiles that crosses unit and
// sequence boundaries ("segments"): per segment a wave accumulates the unnormalised softmax state
// of the segment's tokens for its head block and writes either the final output (whole unit) or
// a partial state (m, l, acc) to its workspace slot.
//
// Per 32-token tile a lane loads: K -- 16 bytes x KLOADS from each of its two token rows
// (16*half + c); V -- one DT-element chunk of each of its 8 token rows pv_token(g, j); and, with
// per-(token, head) scales, one fp32 scale (lane 16g+i holds the k (i < 8) or v (i >= 8) scale
// of token pv_token(g, i & 7)), shared through LDS.  The next tile's loads are issued before the
// current tile is computed (two register sets, used alternately).

template <int D, int KVT>
struct Geometry {
    static constexpr int EB = (KVT == KV_FP8 || KVT == KV_I8) ? 1 : 2;  // bytes per KV element
    static constexpr int E = 16 / EB;                   // elements per 16-byte load
    static constexpr int KSTEPS = D / 32;               // MFMA k-steps of q.k^T
    static constexpr int KLOADS = (D / 4) / E;          // 16-byte K loads per lane per 16-token half
    static constexpr int DT = D / 16;                   // d-tiles of p.V == elements per V chunk
    static constexpr int VDW = (DT * EB) / 4;           // dwords per V chunk (1, 2 or 4)
};

template <int KLOADS, int VDW>
struct TileRaw {
    u32x4_t k[2][KLOADS];
    uint32_t v[8][VDW];
    float sc;
};

// Lane-dependent byte offsets of a full tile's loads (the rest of each address is wave-uniform
// and folded into the scalar base pointer of the token's 16-row half -- the two halves of a tile
// are 16 rows apart in one block, or in two blocks of 16 tokens):
//   K  row c of half `half`, elements 4E*L + E*g:  k = c*row_bytes + E*g*EB   (+ 4E*L*EB)
//   V  row 4g + (j & 3) of half j >> 2, elements DT*c ..:  v = 4g*row_bytes + DT*c*EB  (+ (j & 3)*row_bytes)
//   scale of token pv_token(g, c & 7) (half (c & 7) >> 2), in floats: s = (4g + (c & 3)) * hkv
struct LaneOffsets {
    uint32_t k, v, s;
};

template <int D, int KVT>
__device__ __forceinline__ LaneOffsets lane_offsets(int g, int c, uint32_t row_bytes, int hkv) {
    using G = Geometry<D, KVT>;
    LaneOffsets o;
    o.k = (uint32_t)c * row_bytes + (uint32_t)(G::E * g * G::EB);
    o.v = (uint32_t)(4 * g) * row_bytes + (uint32_t)(G::DT * c * G::EB);
    o.s = (uint32_t)(4 * g + (c & 3)) * (uint32_t)hkv;
    return o;
}

// KV payload load.  NT: streaming (nontemporal) hint, used for V when every KV byte has exactly
// one reader in the grid, so the stream does not displace lines that other loads still need.  K
// stays on cached loads: each 128-byte K row is read by two load instructions of the wave (64
// bytes of 16 rows each), and a nontemporal first read made the second one miss (the 32K FP8
// step's kernel 120.0 us with nontemporal K, 118.0 with cached K; the ragged mix 768 -> 735 us).
template <bool NT, typename T>
__device__ __forceinline__ T ld_kv(const uint8_t *src) {
    if constexpr (NT) return __builtin_nontemporal_load((const T *)src);
    else return *(const T *)src;
}

template <int VDW, bool NT>
__device__ __forceinline__ void load_v_chunk(uint32_t (&dst)[VDW], const uint8_t *src) {
    if constexpr (VDW == 4) {
        const u32x4_t x = ld_kv<NT, u32x4_t>(src);
        dst[0] = x[0]; dst[1] = x[1]; dst[2] = x[2]; dst[3] = x[3];
    } else if constexpr (VDW == 2) {
        const u32x2_t x = ld_kv<NT, u32x2_t>(src);
        dst[0] = x[0]; dst[1] = x[1];
    } else {
        dst[0] = ld_kv<NT, uint32_t>(src);
    }
}

// First rows of a tile's two 16-token halves: K/V bytes of half 1 start h1 bytes (scales h1s
// floats) after those of half 0 -- 16 rows, unless the cache has blocks of 16 tokens (B16).
struct TileBase {
    const uint8_t *k, *v;
    const float *s;
    int64_t h1, h1s;
};

// One tile's loads.  Rows of a partial last tile past `last` are clamped to `last` (valid rows;
// masked later).  Only the per-lane byte offsets differ between a full and a partial tile: both
// kinds then issue the same loads from one place, so the compiler's count of loads in flight
// after a tile is the same on every path (a path with fewer loads would make it wait for more).
template <int D, int KVT, int SCALE, bool NT, bool B16>
__device__ __forceinline__ void load_tile(TileRaw<Geometry<D, KVT>::KLOADS, Geometry<D, KVT>::VDW> &r,
                                          const TileBase &t, int g, int c, const LaneOffsets &o,
                                          uint32_t row_bytes, int hkv, int last) {
    using G = Geometry<D, KVT>;
    // 32-bit offsets unless half 1 may lie in another block (a tile of one block spans < 2^32 bytes)
    using Off = typename std::conditional<B16, int64_t, uint32_t>::type;
    Off kofs[2], vofs[8], sofs = 0;
    if (last >= kTile - 1) {
        // offset of half 1: 16 rows in one block, or wherever the next 16-token block lies
        const Off h1 = B16 ? (Off)t.h1 : (Off)(16 * row_bytes);
        const Off h1s = B16 ? (Off)t.h1s : (Off)(16 * hkv);
        kofs[0] = o.k;
        kofs[1] = h1 + o.k;
#pragma unroll
        for (int j = 0; j < 8; j++) vofs[j] = (j < 4 ? (Off)0 : h1) + (Off)((j & 3) * row_bytes) + o.v;
        if constexpr (SCALE == SC_TOKEN_HEAD) sofs = ((c & 4) ? h1s : (Off)0) + o.s;
    } else {
        // byte offset of tile-relative token `tok` (< 32) from the half-0 base
        auto row_off = [&](int tok) -> Off {
            if constexpr (!B16) return (uint32_t)tok * row_bytes;
            else return tok < 16 ? (int64_t)tok * row_bytes : t.h1 + (int64_t)(tok - 16) * row_bytes;
        };
#pragma unroll
        for (int half = 0; half < 2; half++)
            kofs[half] = row_off(min(16 * half + c, last)) + (Off)(G::E * g * G::EB);
#pragma unroll
        for (int j = 0; j < 8; j++) vofs[j] = row_off(min(pv_token(g, j), last)) + (Off)(G::DT * c * G::EB);
        if constexpr (SCALE == SC_TOKEN_HEAD) {
            const int tok = min(pv_token(g, c & 7), last);
            if constexpr (!B16) sofs = (uint32_t)tok * (uint32_t)hkv;
            else sofs = tok < 16 ? (int64_t)tok * hkv : t.h1s + (int64_t)(tok - 16) * hkv;
        }
    }
#pragma unroll
    for (int half = 0; half < 2; half++)
#pragma unroll
        for (int L = 0; L < G::KLOADS; L++)
            r.k[half][L] = ld_kv<false, u32x4_t>(t.k + kofs[half] + 4 * G::E * L * G::EB);
#pragma unroll
    for (int j = 0; j < 8; j++) load_v_chunk<G::VDW, NT>(r.v[j], t.v + vofs[j]);
    if constexpr (SCALE == SC_TOKEN_HEAD) r.sc = t.s[sofs];
}

template <int D, int KVT, int QT, int SCALE, bool PAGED, bool NT, bool B16>
__global__ __launch_bounds__(64 * kMaxWavesPerGroup) __attribute__((amdgpu_waves_per_eu(2)))
void partition_kernel(Params p) {
    using G = Geometry<D, KVT>;
    constexpr int EB = G::EB, E = G::E, KSTEPS = G::KSTEPS, KLOADS = G::KLOADS, DT = G::DT, VDW = G::VDW;
    // q.k^T operand type: q's own, except against INT8 KV (codes become f16 exactly; a bf16 q is
    // scaled by a power of two into f16's range and converted once per segment)
    constexpr int QM = (KVT == KV_I8) ? KV_F16 : QT;
    constexpr bool QCVT = (KVT == KV_I8 && QT == KV_BF16);
    // quantised KV: partial outputs in 16 bits (the host sets Params::part16 by the same rule)
    constexpr bool PART16 = (KVT == KV_FP8 || KVT == KV_I8);
    __shared__ __attribute__((aligned(16))) float sh_scale_all[kMaxWavesPerGroup][64];
    __shared__ int sh_prefix[kLdsBatch + 1];  // tiles of the sequences before b (b <= batch)
    __shared__ int sh_len[kLdsBatch];         // the sequences' lengths, clamped to max_seq_len

    const int wave = uni((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;  // wave index kept scalar
    float *sh_scale = sh_scale_all[wave];
    const int c = lane & 15, g = lane >> 4;
    const int64_t wg = blockIdx.x, W = gridDim.x;
    const int groups = p.groups;  // unit groups per sequence
    const bool lds_prefix = p.batch <= kLdsBatch;

    // ---- per-sequence tile prefix sums, once per workgroup (then every lookup is an LDS read)
    if (lds_prefix) {
        if (wave == 0) {
            int base = 0;
            for (int b0 = 0; b0 < p.batch; b0 += 64) {
                const int bb = b0 + lane;
                const int nb = bb < p.batch ? max(0, min(p.seq_len[bb], p.max_seq_len)) : 0;
                const int t = (nb + kTile - 1) / kTile;
                const int incl = wave_incl_scan(t, lane);
                if (bb < p.batch) {
                    sh_prefix[bb] = base + incl - t;
                    sh_len[bb] = nb;
                }
                base += __shfl(incl, 63, 64);
            }
            if (lane == 0) sh_prefix[p.batch] = base;
        }
        __syncthreads();
    }
    // length of (wave-uniform) sequence b, clamped: from LDS when the table is there
    auto seq_n = [&](int bq) -> int {
        return lds_prefix ? uni(sh_len[bq]) : max(0, min(ld_uniform(p.seq_len, bq), p.max_seq_len));
    };
    // block sizes are 16, 32 or 64: block index and offset by shift and mask
    const int bsh = PAGED ? (B16 ? 4 : uni(__builtin_ctz((unsigned)p.block_size))) : 0;
    // block-table entry of the next tile's block, read one tile ahead (its scalar load is then
    // complete when that tile is described, instead of stalling the issue of its loads)
    int pf_b = -1, pf_bi = -1;
    int32_t pf_val = 0;

    // ---- this workgroup's tile range [lo, hi) of the concatenation of all unit groups
    const int64_t TT = uni(lds_prefix ? (int64_t)sh_prefix[p.batch] * groups : total_seq_tiles(p, lane) * groups);
    const Split sp = make_split(TT, W);
    const int64_t lo = split_lo(sp, wg), hi = split_lo(sp, wg + 1);
    if (lo >= hi) return;  // every wave of the workgroup takes this branch together

    float tensor_k = 1.0f, tensor_v = 1.0f;
    if constexpr (SCALE == SC_TENSOR) {
        tensor_k = p.k_scale[0];
        tensor_v = p.v_scale[0];
    }
    const float qk_scale = p.qk_scale * tensor_k;
    const uint32_t row_bytes = (uint32_t)p.hkv * D * EB;  // bytes per cache row (all kv heads)
    const LaneOffsets lofs = lane_offsets<D, KVT>(g, c, row_bytes, p.hkv);

    // ---- tile cursor.  Every wave of the workgroup walks the same tiles (its own unit of each
    // unit group), so the cursor is identical across the waves.
    int64_t pos = lo;
    int b = 0, Tb = 0, grp = 0, tt = 0, seg = 0, seg_start = 0, n = 0;

    // place the cursor on global tile `at`
    auto locate = [&](int64_t at) {
        if (lds_prefix) {  // largest b with P_b * groups <= at; it owns a tile, so T_b > 0
            int lo = 0, hi2 = p.batch;
            while (hi2 - lo > 1) {
                const int mid = (lo + hi2) >> 1;
                if ((int64_t)sh_prefix[mid] * groups <= at) lo = mid;
                else hi2 = mid;
            }
            b = uni(lo);
            const int64_t Pb = sh_prefix[b];
            Tb = uni(sh_prefix[b + 1] - sh_prefix[b]);
            const int64_t rel = at - Pb * groups;
            grp = uni((int)(rel / Tb));
            tt = uni((int)(rel % Tb));
            n = seq_n(b);
            return;
        }
        int64_t base = 0;
        Tb = 0;
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
        n = seq_n(b);
    };
    struct Desc {
        int64_t row0, row1;       // first cache rows of the tile's two 16-token halves
        int b, u_in, t0, last;    // sequence, unit in sequence, first token, last valid token in tile
        int nrel;                 // tokens of the sequence from t0 on (> last)
        int seg;                  // segment index within the workgroup's range
        bool first, lastseg, whole;
    };
    auto describe = [&](Desc &d) {
        d.b = b;
        d.u_in = grp * p.wpg + wave;
        d.t0 = tt * kTile;
        d.nrel = n - d.t0;
        d.last = min(d.nrel, kTile) - 1;
        if constexpr (PAGED && !B16) {
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
            d.row0 = (int64_t)ld_uniform(p.block_table, (size_t)b * p.max_blocks + (d.t0 >> 4)) * 16;
            // blocks of 16 tokens: the second half sits in the next block (if the tile reaches it)
            d.row1 = d.last < 16 ? d.row0 + 16
                                 : (int64_t)ld_uniform(p.block_table, (size_t)b * p.max_blocks + (d.t0 >> 4) + 1) * 16;
        } else {
            d.row0 = (int64_t)ld_uniform(p.kv_start, b) + d.t0;
            d.row1 = d.row0 + 16;
        }
        d.seg = seg;
        d.first = (tt == seg_start);
        d.lastseg = (tt + 1 == Tb) || (pos + 1 == hi);
        d.whole = (seg_start == 0) && (tt + 1 == Tb);
    };
    // advance the cursor one tile (crossing units and sequences); false at the end of the range
    auto advance = [&](Desc &d) -> bool {
        if (++pos == hi) return false;
        if (++tt == Tb) {
            tt = 0;
            seg++;
            seg_start = 0;
            if (++grp == groups) {
                grp = 0;
                do {
                    b++;
                } while ((Tb = lds_prefix ? uni(sh_prefix[b + 1] - sh_prefix[b]) : seq_tiles_u(p, b)) == 0);
                n = seq_n(b);
            }
        }
        describe(d);
        return true;
    };

    // ---- per-segment state
    u32x4_t qop[KSTEPS], qnext[KSTEPS];  // q operand of the current segment / of the next one
    f32x4_t acc[DT];
    float m_run = -INFINITY, l_run = 0.0f;
    // per-token v scales: the accumulator holds values / 2^ev (wave-uniform reference exponent)
    int ev = 0;
    // score multiplier of the lane's column: qk_scale, times 2^-eq when q was scaled by 2^eq
    float qk_col = qk_scale;
    // Lane column c of unit u_in: column col = hb * 16 + c of its kv head, i.e. query row
    // m = col / group of the sequence's window and head hl = col % group of the kv head's group
    struct Col {
        bool valid;
        int m, hl;
    };
    auto col_of = [&](int u_in) -> Col {
        const int col = (u_in % p.nhb) * kHeadBlock + c;
        Col r;
        r.valid = col < p.cols;
        if (p.nq == 1) {  // wave-uniform
            r.m = 0;
            r.hl = col;
        } else {
            r.m = col / p.group;
            r.hl = col - r.m * p.group;
        }
        return r;
    };
    // q operand (B of q.k^T) of segment d's unit: lane column c, k-slots of lane group g
    auto load_q = [&](u32x4_t (&dst)[KSTEPS], const Desc &d) {
        const int kvh = d.u_in / p.nhb;
        const Col cl = col_of(d.u_in);
        const uint16_t *qrow =
            (const uint16_t *)p.q + (((size_t)d.b * p.nq + cl.m) * p.hq + kvh * p.group + cl.hl) * D;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; kk++)
            dst[kk] = cl.valid ? *(const u32x4_t *)(qrow + qk_elem<E>(g, kk)) : u32x4_t{0, 0, 0, 0};
    };
    auto reset_state = [&]() {
#pragma unroll
        for (int i = 0; i < DT; i++) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_run = 0.0f;
        ev = 0;
    };
    auto convert_q = [&](u32x4_t (&dst)[KSTEPS], const u32x4_t (&src)[KSTEPS]) {
        if constexpr (QCVT) {
            // largest |q| of column c (its D values lie in the four lane groups): the bf16 bit
            // patterns with the sign cleared order like the magnitudes
            uint32_t mx = 0;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; kk++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const uint32_t w = src[kk][i] & 0x7FFF7FFFu;
                    mx = max(mx, max(w & 0xFFFFu, w >> 16));
                }
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16, 64));
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32, 64));
            // 2^eq puts the largest |q| in [2^14, 2^15) (bf16 biased exponent in bits 7..14)
            const int eq = mx == 0 ? 0 : 141 - (int)(mx >> 7);
#pragma unroll
            for (int kk = 0; kk < KSTEPS; kk++)
                dst[kk] = u32x4_t{bf16x2_to_f16x2_scaled(src[kk][0], eq), bf16x2_to_f16x2_scaled(src[kk][1], eq),
                                  bf16x2_to_f16x2_scaled(src[kk][2], eq), bf16x2_to_f16x2_scaled(src[kk][3], eq)};
            qk_col = __builtin_amdgcn_ldexpf(qk_scale, -eq);
        } else {
#pragma unroll
            for (int kk = 0; kk < KSTEPS; kk++) dst[kk] = src[kk];
        }
    };
    auto next_segment = [&]() {
        convert_q(qop, qnext);
        reset_state();
    };

    auto issue = [&](TileRaw<KLOADS, VDW> &r, const Desc &d) {
        const int kvh = d.u_in / p.nhb;
        TileBase t;
        t.k = (const uint8_t *)p.k + (size_t)kvh * D * EB + (size_t)d.row0 * row_bytes;
        t.v = (const uint8_t *)p.v + (size_t)kvh * D * EB + (size_t)d.row0 * row_bytes;
        t.h1 = (d.row1 - d.row0) * (int64_t)row_bytes;
        t.h1s = (d.row1 - d.row0) * (int64_t)p.hkv;
        t.s = nullptr;
        // lane 16g+i holds the k (i < 8) or v (i >= 8) scale of token pv_token(g, i & 7)
        if constexpr (SCALE == SC_TOKEN_HEAD) t.s = ((c & 8) ? p.v_scale : p.k_scale) + kvh + (size_t)d.row0 * p.hkv;
        load_tile<D, KVT, SCALE, NT, B16>(r, t, g, c, lofs, row_bytes, p.hkv, d.last);
        // keep the instruction scheduler from pulling the current tile's compute (and its waits)
        // above these loads: the next tile's loads go out first
        __builtin_amdgcn_sched_barrier(0);
    };

    auto compute = [&](const TileRaw<KLOADS, VDW> &r, const Desc &d) {
        const int last = d.last;  // last valid tile-relative token (>= 0)
        // ---- per-token scales of the lane's 8 score slots, through LDS
        float ksc[8], vsc[8];
        if constexpr (SCALE == SC_TOKEN_HEAD) {
            sh_scale[lane] = r.sc;
            __builtin_amdgcn_wave_barrier();
            const float4 k0 = *(const float4 *)&sh_scale[16 * g + 0];
            const float4 k1 = *(const float4 *)&sh_scale[16 * g + 4];
            const float4 v0 = *(const float4 *)&sh_scale[16 * g + 8];
            const float4 v1 = *(const float4 *)&sh_scale[16 * g + 12];
            __builtin_amdgcn_wave_barrier();
            ksc[0] = k0.x; ksc[1] = k0.y; ksc[2] = k0.z; ksc[3] = k0.w;
            ksc[4] = k1.x; ksc[5] = k1.y; ksc[6] = k1.z; ksc[7] = k1.w;
            vsc[0] = v0.x; vsc[1] = v0.y; vsc[2] = v0.z; vsc[3] = v0.w;
            vsc[4] = v1.x; vsc[5] = v1.y; vsc[6] = v1.z; vsc[7] = v1.w;
        }

        // ---- scores: S[token][head] = K . q over two 16-token halves
        f32x4_t sacc[2];
#pragma unroll
        for (int half = 0; half < 2; half++) {
            sacc[half] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KSTEPS; kk++) {
                u32x4_t a;
                if constexpr (KVT == KV_FP8) {
                    const u32x4_t wv = r.k[half][kk / 2];
                    const uint32_t w0 = wv[2 * (kk % 2)], w1 = wv[2 * (kk % 2) + 1];
                    a = u32x4_t{cvt_fp8x2<QT, false>(w0), cvt_fp8x2<QT, true>(w0),
                                cvt_fp8x2<QT, false>(w1), cvt_fp8x2<QT, true>(w1)};
                } else if constexpr (KVT == KV_I8) {
                    // bytes 0,1 / 2,3 of each dword -> 0x00bb 16-bit halves (zero bytes: selector 0x0C)
                    const u32x4_t wv = r.k[half][kk / 2];
                    const uint32_t w0 = wv[2 * (kk % 2)], w1 = wv[2 * (kk % 2) + 1];
                    a = u32x4_t{i8x2_to_f16x2(__builtin_amdgcn_perm(0u, w0, 0x0C010C00u)),
                                i8x2_to_f16x2(__builtin_amdgcn_perm(0u, w0, 0x0C030C02u)),
                                i8x2_to_f16x2(__builtin_amdgcn_perm(0u, w1, 0x0C010C00u)),
                                i8x2_to_f16x2(__builtin_amdgcn_perm(0u, w1, 0x0C030C02u))};
                } else {
                    a = r.k[half][kk];
                }
                sacc[half] = mfma_qk<QM>(a, qop[kk], sacc[half]);
            }
        }

        // ---- online softmax (log2 units)
        float s[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            float x = sacc[j >> 2][j & 3];
            if constexpr (SCALE == SC_TOKEN_HEAD) x *= ksc[j] * qk_col;
            else x *= qk_col;
            s[j] = x;
        }
        // last token of this tile column c may see: query row m of a window of nq rows stops
        // nq - 1 - m tokens before the sequence's end (a plain step: the tile's last valid token)
        int lastc = last;
        if (p.nq > 1) lastc = min(d.nrel - (p.nq - 1 - col_of(d.u_in).m), kTile) - 1;
        if (__any(lastc < kTile - 1)) {
#pragma unroll
            for (int j = 0; j < 8; j++) s[j] = (pv_token(g, j) <= lastc) ? s[j] : -INFINITY;
        }
        float mt = s[0];
#pragma unroll
        for (int j = 1; j < 8; j++) mt = fmaxf(mt, s[j]);
        mt = fmaxf(mt, shfl_xor_f(mt, 16));
        mt = fmaxf(mt, shfl_xor_f(mt, 32));
        // per-token v scales: reference exponent of the tile's largest |v scale| (all 32 tokens:
        // the lane's 8, then the four lane groups); it replaces ev when out of ev's window
        int evt = ev;
        if constexpr (SCALE == SC_TOKEN_HEAD) {
            float vm = fmaxf(fmaxf(fabsf(vsc[0]), fabsf(vsc[1])), fmaxf(fabsf(vsc[2]), fabsf(vsc[3])));
            vm = fmaxf(vm, fmaxf(fmaxf(fabsf(vsc[4]), fabsf(vsc[5])), fmaxf(fabsf(vsc[6]), fabsf(vsc[7]))));
            vm = fmaxf(vm, shfl_xor_f(vm, 16));
            vm = fmaxf(vm, shfl_xor_f(vm, 32));
            evt = uni(vm > 0.0f ? exp2_ceil(vm) : ev);  // all-zero scales: keep ev
        }
        const bool emove = evt > ev + kVrefHigh || evt < ev - kVrefLow;
        // move the reference max only when some head exceeds it by more than kRescaleSlack
        // (a column with no visible token yet keeps m_run = -inf: the max with -kMaxFloat below keeps
        // its weights 0 and its alpha 1 instead of NaN)
        if (__any(mt > m_run + kRescaleSlack) || emove) {  // wave-uniform
            const float m_new = fmaxf(m_run, mt);
            const float dm = fmaxf(m_run, -kMaxFloat) - fmaxf(m_new, -kMaxFloat);
            const float alpha = __builtin_amdgcn_exp2f(dm);
            // the accumulator also moves from units of 2^ev to units of 2^evt (exact for a power of two)
            const float alpha_acc = SCALE == SC_TOKEN_HEAD ? __builtin_amdgcn_exp2f(dm + (float)(ev - evt)) : alpha;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < DT; i++) acc[i] *= alpha_acc;
            m_run = m_new;
            ev = evt;
        }
        // token-head scales: weights 2^(s - m - ev), i.e. divided by 2^ev (their sum is scaled back
        // for l, which stays in units of 2^m)
        float pj[8], psum = 0.0f;
        const float m_ref = fmaxf(m_run, -kMaxFloat) + (SCALE == SC_TOKEN_HEAD ? (float)ev : 0.0f);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            pj[j] = __builtin_amdgcn_exp2f(s[j] - m_ref);
            psum += pj[j];
        }
        l_run += SCALE == SC_TOKEN_HEAD ? __builtin_amdgcn_ldexpf(psum, ev) : psum;

        // ---- p.V
        if constexpr (KVT == KV_BF16) {
            uint32_t hi2[4], lo2[4];
#pragma unroll
            for (int u = 0; u < 4; u++) split_bf16_pair(pj[2 * u], pj[2 * u + 1], hi2[u], lo2[u]);
            const u32x4_t phi = {hi2[0], hi2[1], hi2[2], hi2[3]}, plo = {lo2[0], lo2[1], lo2[2], lo2[3]};
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                uint32_t a[4];
#pragma unroll
                for (int u = 0; u < 4; u++)
                    a[u] = __builtin_amdgcn_perm(r.v[2 * u + 1][dt >> 1], r.v[2 * u][dt >> 1],
                                                 (dt & 1) ? 0x07060302u : 0x05040100u);
                const u32x4_t av = {a[0], a[1], a[2], a[3]};
                acc[dt] = mfma_bf16(av, phi, acc[dt]);
                acc[dt] = mfma_bf16(av, plo, acc[dt]);
            }
        } else {
            uint32_t pp[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                float p0 = pj[2 * u], p1 = pj[2 * u + 1];
                if constexpr (SCALE == SC_TOKEN_HEAD) { p0 *= vsc[2 * u]; p1 *= vsc[2 * u + 1]; }
                pp[u] = pack_f16(p0, p1);
            }
            const u32x4_t pop = {pp[0], pp[1], pp[2], pp[3]};
            if constexpr (KVT == KV_I8) {
#pragma unroll
                for (int wd = 0; wd < VDW; wd++) {
                    uint32_t a[4][4];
#pragma unroll
                    for (int u = 0; u < 4; u++)
#pragma unroll
                        for (int k = 0; k < 4; k++)  // byte k of rows 2u, 2u+1 -> f16 pair (token 2u, 2u+1)
                            a[k][u] = i8x2_to_f16x2(__builtin_amdgcn_perm(r.v[2 * u + 1][wd], r.v[2 * u][wd],
                                                                          0x0C000C00u | ((4u + k) << 16) | (uint32_t)k));
#pragma unroll
                    for (int k = 0; k < 4; k++)
                        acc[4 * wd + k] = mfma_f16(u32x4_t{a[k][0], a[k][1], a[k][2], a[k][3]}, pop, acc[4 * wd + k]);
                }
            } else if constexpr (KVT == KV_FP8) {
#pragma unroll
                for (int wd = 0; wd < VDW; wd++) {
                    uint32_t a[4][4];
#pragma unroll
                    for (int u = 0; u < 4; u++) {
                        const uint32_t x = __builtin_amdgcn_perm(r.v[2 * u + 1][wd], r.v[2 * u][wd], 0x05010400u);
                        const uint32_t y = __builtin_amdgcn_perm(r.v[2 * u + 1][wd], r.v[2 * u][wd], 0x07030602u);
                        a[0][u] = cvt_fp8x2<KV_F16, false>(x);
                        a[1][u] = cvt_fp8x2<KV_F16, true>(x);
                        a[2][u] = cvt_fp8x2<KV_F16, false>(y);
                        a[3][u] = cvt_fp8x2<KV_F16, true>(y);
                    }
#pragma unroll
                    for (int k = 0; k < 4; k++)
                        acc[4 * wd + k] = mfma_f16(u32x4_t{a[k][0], a[k][1], a[k][2], a[k][3]}, pop, acc[4 * wd + k]);
                }
            } else {
#pragma unroll
                for (int dt = 0; dt < DT; dt++) {
                    uint32_t a[4];
#pragma unroll
                    for (int u = 0; u < 4; u++)
                        a[u] = __builtin_amdgcn_perm(r.v[2 * u + 1][dt >> 1], r.v[2 * u][dt >> 1],
                                                     (dt & 1) ? 0x07060302u : 0x05040100u);
                    acc[dt] = mfma_f16(u32x4_t{a[0], a[1], a[2], a[3]}, pop, acc[dt]);
                }
            }
        }
    };

    // ---- segment result: total running sum over the four lane groups of head c
    auto finalize = [&](const Desc &d) {
        const int kvh = d.u_in / p.nhb;
        const Col cl = col_of(d.u_in);
        const bool hvalid = cl.valid;
        const size_t orow_idx = ((size_t)d.b * p.nq + cl.m) * p.hq + kvh * p.group + cl.hl;  // out / lse row
        float l_tot = l_run + shfl_xor_f(l_run, 16);
        l_tot += shfl_xor_f(l_tot, 32);
        f32x4_t o[DT];
#pragma unroll
        for (int i = 0; i < DT; i++) o[i] = (SCALE == SC_TENSOR) ? acc[i] * tensor_v : acc[i];
        // lane (g, c) holds d = DT*(4g + r) + dt in o[dt][r]; with per-token scales the values are
        // o * 2^ev
        if (d.whole) {
            if (hvalid) {
                const size_t orow = orow_idx * D;
                // 0: a window row with no token.  l_tot >= 1 otherwise (the weight of the token
                // that set m is 1), so the factor stays finite
                float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
                if constexpr (SCALE == SC_TOKEN_HEAD) inv = __builtin_amdgcn_ldexpf(inv, ev);
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    float v[DT];
#pragma unroll
                    for (int dt = 0; dt < DT; dt++) v[dt] = o[dt][r] * inv;
                    store_row_chunk<DT>(p.out, p.out_dtype, orow + DT * (4 * g + r), v);
                }
                if (p.lse && g == 0) p.lse[orow_idx] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
            }
        } else {
            // slot 0: the range's first segment; slot 1: its last (a middle one is always whole)
            const size_t slot = (((size_t)wg * 2 + (d.seg == 0 ? 0 : 1)) * p.wpg + wave) * kHeadBlock + c;
            if constexpr (PART16) {
                // f16 of value / (largest |value| of the head's row): the row spans the four lane
                // groups of column c (every lane joins the shuffles)
                float mx = 0.0f;
#pragma unroll
                for (int r = 0; r < 4; r++)
#pragma unroll
                    for (int dt = 0; dt < DT; dt++) mx = fmaxf(mx, fabsf(o[dt][r]));
                mx = fmaxf(mx, shfl_xor_f(mx, 16));
                mx = fmaxf(mx, shfl_xor_f(mx, 32));
                if (hvalid) {
                    // at least the smallest normal float: its reciprocal stays finite
                    const float sc = fmaxf(mx, kMinNormal), inv = 1.0f / sc;
                    uint16_t *dst = (uint16_t *)p.ws_acc + slot * D;
#pragma unroll
                    for (int r = 0; r < 4; r++) {
#pragma unroll
                        for (int dt = 0; dt < DT; dt += 4)
                            *(u32x2_t *)(dst + DT * (4 * g + r) + dt) =
                                u32x2_t{pack_f16(o[dt][r] * inv, o[dt + 1][r] * inv),
                                        pack_f16(o[dt + 2][r] * inv, o[dt + 3][r] * inv)};
                    }
                    if (g == 0) {
                        p.ws_ml[slot] = make_float2(m_run, l_tot);
                        p.ws_sc[slot] = SCALE == SC_TOKEN_HEAD ? __builtin_amdgcn_ldexpf(sc, ev) : sc;
                    }
                }
            } else if (hvalid) {
                float *dst = p.ws_acc + slot * D;
#pragma unroll
                for (int r = 0; r < 4; r++) {
#pragma unroll
                    for (int dt = 0; dt < DT; dt += 4)
                        *(float4 *)(dst + DT * (4 * g + r) + dt) =
                            make_float4(o[dt][r], o[dt + 1][r], o[dt + 2][r], o[dt + 3][r]);
                }
                if (g == 0) p.ws_ml[slot] = make_float2(m_run, l_tot);
            }
        }
    };

    // ---- start
    locate(lo);
    seg_start = tt;

    // ---- tile stream: two register sets; the next tile's loads (possibly of the next unit or
    // sequence) are in flight while the current one is computed.  A new segment's q operand is
    // loaded just before its first tile.  The range's tile count is known, so the loop runs a
    // fixed number of two-tile steps, each an issue followed by a compute, and the last one or two
    // tiles are finished after it.  The compiler's wait before a compute then covers only the tile
    // being computed: an exit or a skipped issue inside the loop would, on the paths its control
    // flow merges, make it wait for the tile just issued as well.
    TileRaw<KLOADS, VDW> ra, rb;
    Desc da, db;
    const int ntiles = (int)(hi - lo);  // >= 1
    describe(da);
    load_q(qnext, da);
    issue(ra, da);
    convert_q(qop, qnext);
    reset_state();
    for (int step = 0; step < (ntiles - 1) >> 1; step++) {
        advance(db);
        if (db.first) load_q(qnext, db);
        issue(rb, db);
        // The waves of a workgroup stream the same token rows but are not otherwise tied; left
        // alone, the first waves run ahead and the last ones finish with few loads in flight on
        // their CU.  A barrier every 16 tiles bounds that drift (measured: 3-4 % faster kernels
        // than with no barrier or with one per tile).
        if ((step & 7) == 0) __builtin_amdgcn_s_barrier();
        compute(ra, da);
        if (da.lastseg) finalize(da);
        if (db.first) next_segment();
        advance(da);
        if (da.first) load_q(qnext, da);
        issue(ra, da);
        compute(rb, db);
        if (db.lastseg) finalize(db);
        if (da.first) next_segment();
    }
    if ((ntiles & 1) == 0) {  // two tiles left
        advance(db);
        if (db.first) load_q(qnext, db);
        issue(rb, db);
        compute(ra, da);
        if (da.lastseg) finalize(da);
        if (db.first) next_segment();
        compute(rb, db);
        finalize(db);  // the range's last tile ends its segment
    } else {
        compute(ra, da);
        finalize(da);
    }
}

// ---------------------------------------------------------------- combine kernel
//
// Grid: x = window row * hq + q head, y = sequence.  Block: NW waves.  For a unit cut by
// workgroup boundaries, merges its pieces -- slot 1 (or 0) of the first workgroup, slot 0 of the
// later ones -- with the log-sum-exp rule for two partial states (m_a, l_a, acc_a), (m_b, l_b, acc_b):
//   M = max(m_a, m_b),  w = 2^(m - M),  l = w_a l_a + w_b l_b,  acc = w_a acc_a + w_b acc_b
// (an empty state has m = -inf and weight 0), then out = acc / l, lse = (M + log2 l) ln 2 (a
// window row that sees no token: out = 0, lse = -inf).
// Lane group j = lane / 8 of wave w (global group g = 8 w + j) folds pieces g, g + 8 NW, ... in
// order over output elements [k*D/8, (k+1)*D/8), k = lane % 8, NF pieces' loads in flight at a
// time; the eight lane-group states of a wave are merged by a fixed butterfly (both partners
// compute the same sums), and the NW wave states, in wave order, through LDS.  A row of at most
// 32 pieces is merged by wave 0 alone (in rounds of 8 * NF pieces' loads).  Many pieces per row
// (a few very long sequences over many workgroups) make the single-wave merge a chain of
// dependent load rounds; NW > 1 splits that chain.  Also writes out = 0, lse = -inf for empty sequences.  Fixed order
// throughout: deterministic for a given NW.
template <int D, int NW, bool P16>
__global__ __launch_bounds__(64 * NW) void combine_kernel(Params p) {
    constexpr int PER = D / 8;  // output elements per lane
    // per-wave merged state: D outputs, then m and l; rows padded to a 16-byte multiple
    __shared__ __attribute__((aligned(16))) float sh_state[NW > 1 ? NW : 1][D + 4];
    const int mq = blockIdx.x / p.hq, h = blockIdx.x % p.hq, b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = NW > 1 ? uni((int)(threadIdx.x >> 6)) : 0;
    const int j = lane >> 3, k = lane & 7;
    const int kvh = h / p.group, col = mq * p.group + h % p.group;  // column of the kv head
    const int u_in = kvh * p.nhb + col / p.hb;
    const int grp = u_in / p.wpg, uw = u_in % p.wpg, c = col % p.hb;
    const size_t orow_idx = ((size_t)b * p.nq + mq) * p.hq + h;  // out / lse row
    const size_t obase = orow_idx * D + PER * k;

    auto store = [&](const float *v) {
        if (p.out_dtype == 0) {
            float *o = (float *)p.out + obase;
#pragma unroll
            for (int i = 0; i < PER; i += 4) *(float4 *)(o + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
        } else {
            uint32_t w[PER / 2];
#pragma unroll
            for (int i = 0; i < PER / 2; i++) {
                if (p.out_dtype == 1) w[i] = pack_f16(v[2 * i], v[2 * i + 1]);
                else w[i] = f32_to_bf16_bits(v[2 * i]) | (f32_to_bf16_bits(v[2 * i + 1]) << 16);
            }
            uint16_t *o = (uint16_t *)p.out + obase;
#pragma unroll
            for (int i = 0; i < PER / 2; i += 4) *(u32x4_t *)(o + 2 * i) = u32x4_t{w[i], w[i + 1], w[i + 2], w[i + 3]};
        }
    };

    // one pass over seq_len: tiles of all sequences, of those before b, and of b
    int64_t tot = 0, bef = 0;
    int mine = 0;
#pragma unroll 4
    for (int bb = lane; bb < p.batch; bb += 64) {
        const int t = seq_tiles(p, bb);
        tot += t;
        bef += bb < b ? t : 0;
        mine = bb == b ? t : mine;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        tot += __shfl_xor(tot, off, 64);
        bef += __shfl_xor(bef, off, 64);
        mine += __shfl_xor(mine, off, 64);
    }
    const int64_t TT = tot * p.groups, Pb = bef;
    const int Tb = mine;
    if (Tb == 0) {
        if (wave != 0) return;
        if (j == 0) {
            float z[PER];
#pragma unroll
            for (int i = 0; i < PER; i++) z[i] = 0.0f;
            store(z);
        }
        if (p.lse && lane == 0) p.lse[orow_idx] = -INFINITY;
        return;
    }
    const int64_t U0 = Pb * p.groups + (int64_t)grp * Tb;
    const Split sp = make_split(TT, p.nparts);
    const int64_t wlo = split_owner(sp, U0), whi = split_owner(sp, U0 + Tb - 1);
    if (wlo == whi) return;  // finished by the partition kernel
    // pieces: the ranges wlo..whi in order (never empty: with fewer tiles than workgroups every
    // non-empty range holds one tile and split_owner(t) = t)
    const int np = (int)(whi - wlo + 1);
    // the same for every wave of the workgroup: the split-up merge (and its barrier) runs in all
    // of them or in none
    const int nw = np <= 32 ? 1 : NW;
    if (wave >= nw) return;
    const int first_slot = split_lo(sp, wlo) == U0 ? 0 : 1;  // unit began inside wlo's range
    auto slot_of = [&](int i) -> size_t {
        return (((size_t)(wlo + i) * 2 + (i == 0 ? first_slot : 0)) * p.wpg + uw) * p.hb + c;
    };

    // ---- this lane group's pieces g, g + 8 nw, ..., four at a time
    const int g = 8 * wave + j, gstride = 8 * nw;
    float m = -INFINITY, l = 0.0f, o[PER];
#pragma unroll
    for (int i = 0; i < PER; i++) o[i] = 0.0f;
    // NF, pieces in flight per lane group and round: a single-wave row with 16-bit pieces takes
    // two (8 + 3 registers each), which keeps the kernel within 64 VGPRs -- eight resident waves
    // per SIMD, so the many one-wave workgroups of a multi-token window or a large batch run in
    // one residency round; otherwise four
    constexpr int NF = (NW == 1 && P16) ? 2 : 4;
    for (int i0 = g; i0 < np; i0 += NF * gstride) {
        float2 ml[NF];
        float sc[NF];
        u32x4_t raw[NF][P16 ? PER / 8 : PER / 4];  // f16 words, or fp32 bit patterns
#pragma unroll
        for (int u = 0; u < NF; u++) {
            const size_t slot = slot_of(min(i0 + gstride * u, np - 1));
            ml[u] = p.ws_ml[slot];
            if constexpr (P16) {  // f16 of value / row scale
                sc[u] = p.ws_sc[slot];
                const uint16_t *src = (const uint16_t *)p.ws_acc + slot * D + PER * k;
#pragma unroll
                for (int e = 0; e < PER / 8; e++) raw[u][e] = *(const u32x4_t *)(src + 8 * e);
            } else {
                const float *src = p.ws_acc + slot * D + PER * k;
#pragma unroll
                for (int e = 0; e < PER / 4; e++) raw[u][e] = *(const u32x4_t *)(src + 4 * e);
            }
        }
#pragma unroll
        for (int u = 0; u < NF; u++) {
            if (i0 + gstride * u < np) {
                float x[PER];
                if constexpr (P16) {
#pragma unroll
                    for (int e = 0; e < PER / 8; e++)
#pragma unroll
                        for (int h2 = 0; h2 < 4; h2++) {
                            const uint32_t wh = raw[u][e][h2];
                            x[8 * e + 2 * h2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wh & 0xFFFFu)) * sc[u];
                            x[8 * e + 2 * h2 + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wh >> 16)) * sc[u];
                        }
                } else {
#pragma unroll
                    for (int e = 0; e < PER / 4; e++)
#pragma unroll
                        for (int h2 = 0; h2 < 4; h2++) {
                            // through a scalar: a bit cast of the vector element itself reads
                            // element 0 (hipcc, ROCm 7.2)
                            const uint32_t w = raw[u][e][h2];
                            x[4 * e + h2] = __builtin_bit_cast(float, w);
                        }
                }
                // a piece of a window row can hold no visible token (m = -inf, l = 0): the max with
                // -kMaxFloat gives it weight 0 (and an all-empty state weight 1 on zeros), not NaN
                const float mn = fmaxf(m, ml[u].x);
                const float ma = fmaxf(m, -kMaxFloat), mb = fmaxf(ml[u].x, -kMaxFloat), mc = fmaxf(mn, -kMaxFloat);
                const float wa = __builtin_amdgcn_exp2f(ma - mc), wb = __builtin_amdgcn_exp2f(mb - mc);
                l = l * wa + ml[u].y * wb;
#pragma unroll
                for (int e = 0; e < PER; e++) o[e] = o[e] * wa + x[e] * wb;
                m = mn;
            }
        }
    }
    // ---- merge the eight lane-group states of the wave
#pragma unroll
    for (int off = 8; off < 64; off <<= 1) {
        const float mo = shfl_xor_f(m, off), lo = shfl_xor_f(l, off);
        const float mn = fmaxf(m, mo);
        const float wa = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
        const float wb = mo == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
        l = l * wa + lo * wb;
#pragma unroll
        for (int e = 0; e < PER; e++) o[e] = o[e] * wa + shfl_xor_f(o[e], off) * wb;
        m = mn;
    }
    if constexpr (NW > 1) {
        // ---- then the wave states, in wave order (lanes 0..7 of a wave hold its state)
        if (nw > 1) {
            if (j == 0) {
#pragma unroll
                for (int e = 0; e < PER; e += 4)
                    *(float4 *)&sh_state[wave][PER * k + e] = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
                if (k == 0) {
                    sh_state[wave][D] = m;
                    sh_state[wave][D + 1] = l;
                }
            }
            __syncthreads();
            if (wave != 0) return;
            if (j == 0) {
                for (int w2 = 1; w2 < nw; w2++) {
                    const float mo = sh_state[w2][D], lo = sh_state[w2][D + 1];
                    const float mn = fmaxf(m, mo);
                    const float wa = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
                    const float wb = mo == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
                    l = l * wa + lo * wb;
#pragma unroll
                    for (int e = 0; e < PER; e++) o[e] = o[e] * wa + sh_state[w2][PER * k + e] * wb;
                    m = mn;
                }
            }
        }
    }
    if (j == 0) {
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
        for (int e = 0; e < PER; e++) o[e] *= inv;
        store(o);
        if (p.lse && lane == 0) p.lse[orow_idx] = l > 0.0f ? (m + log2f(l)) * kLn2 : -INFINITY;
    }
}

// ---------------------------------------------------------------- E4M3 decode (diagnostic)
// The same hardware conversion the partition kernel uses for K (to bf16) and V (to f16),
// widened to fp32; lets the tests compare it against the format definition on all 256 bytes.
__global__ void fp8_decode_kernel(const uint8_t *in, float *out, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t w = in[i];
    const uint32_t hb = cvt_fp8x2<KV_F16, false>(w);
    const uint32_t bb = cvt_fp8x2<KV_BF16, false>(w);
    const float fh = (float)__builtin_bit_cast(_Float16, (uint16_t)(hb & 0xFFFF));
    const float fb = __builtin_bit_cast(float, (bb & 0xFFFF) << 16);
    out[2 * i] = fh;
    out[2 * i + 1] = fb;
}

// ---------------------------------------------------------------- HBM read probe (diagnostic)
// Streams `n16` 16-byte words with coalesced 128-bit loads (four independent loads in flight per
// lane per iteration, grid-stride) and folds them with XOR so the loads cannot be dropped.
// The measured rate is the read bandwidth a plain stream reaches on this device.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4_t *__restrict__ in, size_t n16,
                                                         uint32_t *__restrict__ out) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4_t acc = {0, 0, 0, 0};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4_t a = in[i], b = in[i + stride], c = in[i + 2 * stride], d = in[i + 3 * stride];
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= in[i];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Second probe design: each wave streams whole 1 KB chunks (lane i the 16 bytes at 16 i),
// chunks c = 4 * block + wave + k * (4 * grid), INFL nontemporal loads per lane in flight.
// Covers the first n1k * 1024 bytes.
template <int INFL>
__global__ __launch_bounds__(256) void read_probe_chunks_kernel(const u32x4_t *__restrict__ in, size_t n1k,
                                                                uint32_t *__restrict__ out) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const size_t nw = (size_t)gridDim.x * 4;
    size_t c = (size_t)blockIdx.x * 4 + wave;
    u32x4_t acc = {0, 0, 0, 0};
    for (; c + (INFL - 1) * nw < n1k; c += INFL * nw) {
        u32x4_t v[INFL];
#pragma unroll
        for (int i = 0; i < INFL; i++) v[i] = __builtin_nontemporal_load(in + (c + i * nw) * 64 + lane);
#pragma unroll
        for (int i = 0; i < INFL; i++) acc ^= v[i];
    }
    for (; c < n1k; c += nw) acc ^= __builtin_nontemporal_load(in + c * 64 + lane);
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// ---------------------------------------------------------------- host-side dispatch
template <int D, int KVT, int QT, int SCALE>
static hipError_t launch_p(const Params &p, hipStream_t stream) {
    dim3 grid(p.nparts), block(64 * p.wpg);
    // with one head block per kv head every KV byte is read by one wave only: stream it
    const bool nt = p.nhb == 1;
    if (p.block_table && p.block_size == 16) {  // 32-token tiles span two blocks
        if (nt) hipLaunchKernelGGL((partition_kernel<D, KVT, QT, SCALE, true, true, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((partition_kernel<D, KVT, QT, SCALE, true, false, true>), grid, block, 0, stream, p);
    } else if (p.block_table) {
        if (nt) hipLaunchKernelGGL((partition_kernel<D, KVT, QT, SCALE, true, true, false>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((partition_kernel<D, KVT, QT, SCALE, true, false, false>), grid, block, 0, stream, p);
    } else {
        if (nt) hipLaunchKernelGGL((partition_kernel<D, KVT, QT, SCALE, false, true, false>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((partition_kernel<D, KVT, QT, SCALE, false, false, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const Params &p, int kv, int qt, int sc, hipStream_t stream) {
    if (kv == KV_F16) return launch_p<D, KV_F16, KV_F16, SC_NONE>(p, stream);
    if (kv == KV_BF16) return launch_p<D, KV_BF16, KV_BF16, SC_NONE>(p, stream);
    if (kv == KV_I8) {
        if (qt == KV_BF16) {
            if (sc == SC_TENSOR) return launch_p<D, KV_I8, KV_BF16, SC_TENSOR>(p, stream);
            return launch_p<D, KV_I8, KV_BF16, SC_TOKEN_HEAD>(p, stream);
        }
        if (sc == SC_TENSOR) return launch_p<D, KV_I8, KV_F16, SC_TENSOR>(p, stream);
        return launch_p<D, KV_I8, KV_F16, SC_TOKEN_HEAD>(p, stream);
    }
    if (qt == KV_BF16) {
        if (sc == SC_TENSOR) return launch_p<D, KV_FP8, KV_BF16, SC_TENSOR>(p, stream);
        return launch_p<D, KV_FP8, KV_BF16, SC_TOKEN_HEAD>(p, stream);
    }
    if (sc == SC_TENSOR) return launch_p<D, KV_FP8, KV_F16, SC_TENSOR>(p, stream);
    return launch_p<D, KV_FP8, KV_F16, SC_TOKEN_HEAD>(p, stream);
}

hipError_t launch_partition(const Params &p, int kv_dtype, int q_dtype, int scale_mode, hipStream_t stream) {
    if (p.d == 128) return launch_d<128>(p, kv_dtype, q_dtype, scale_mode, stream);
    return launch_d<64>(p, kv_dtype, q_dtype, scale_mode, stream);
}

// Waves per combine workgroup: the partition workgroups per sequence bound the pieces of a row
// from above on average; past 16 of them rows of the longer sequences exceed the 32 pieces one
// wave merges in a single round of loads.
static int combine_waves(const Params &p) {
    const long per_seq = (long)p.nparts / p.batch;
    return per_seq > 64 ? 8 : per_seq > 16 ? 4 : 1;
}

template <int D, bool P16>
static void launch_combine_d(const Params &p, int nw, hipStream_t stream) {
    dim3 grid(p.hq * p.nq, p.batch);
    if (nw == 8) hipLaunchKernelGGL((combine_kernel<D, 8, P16>), grid, dim3(512), 0, stream, p);
    else if (nw == 4) hipLaunchKernelGGL((combine_kernel<D, 4, P16>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((combine_kernel<D, 1, P16>), grid, dim3(64), 0, stream, p);
}

hipError_t launch_combine(const Params &p, hipStream_t stream) {
    const int nw = combine_waves(p);
    if (p.d == 128) {
        if (p.part16) launch_combine_d<128, true>(p, nw, stream);
        else launch_combine_d<128, false>(p, nw, stream);
    } else {
        if (p.part16) launch_combine_d<64, true>(p, nw, stream);
        else launch_combine_d<64, false>(p, nw, stream);
    }
    return hipGetLastError();
}

hipError_t launch_read_probe(const void *in, size_t n16, uint32_t *out, int blocks, int kind, hipStream_t stream) {
    if (kind == 0)
        hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, stream, (const u32x4_t *)in, n16, out);
    else if (kind == 1)
        hipLaunchKernelGGL(read_probe_chunks_kernel<4>, dim3(blocks), dim3(256), 0, stream, (const u32x4_t *)in,
                           n16 / 64, out);
    else
        hipLaunchKernelGGL(read_probe_chunks_kernel<8>, dim3(blocks), dim3(256), 0, stream, (const u32x4_t *)in,
                           n16 / 64, out);
    return hipGetLastError();
}

hipError_t launch_fp8_decode(const uint8_t *in, float *out, int n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fp8_decode_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, in, out, n);
    return hipGetLastError();
}

}  // namespace fd
