// fd_wide.hip -- gfx950 partition kernel for wide query groups: 64 or more query heads per kv
// head (MQA / wide GQA), E4M3 or INT8 KV (128 or more heads: also f16 / bf16 KV), head_dim 128.
//
// Method: the split-KV online-softmax recurrence of the 16-head partition kernel in
// fd_kernels.hip (same pages: "SGLang Prefill 性能优化" section 2.2 for the block recurrence;
// "从 SGLang Kernel源码到 GPU Trace：DeepSeek V4.1 Flash-Decode" sections 2.2 / 3.1 for the ragged,
// block-wise KV walk and FP8 conversion right after the load; the ch.15 profiling page, sections
// 15.11-15.13, for per-token scales, one kv head serving a query-head group, paged addressing and
// split-K partials).  Same work split (unit groups concatenated into 32-token tiles, equal tile
// ranges per workgroup) and the same partial-slot layout, so the same combine kernel finishes it.
//
// gfx950 design:
//   * One workgroup runs WPG waves on WPG head blocks of 32 heads of ONE kv head: the K/V tile is
//     the same for all of them, so it is fetched once per workgroup, straight into LDS by
//     direct-to-LDS copies (global_load_lds_dwordx4: no VGPRs held while a copy is in flight),
//     into a ring of NSLOT tiles with NSLOT-1 tiles in flight.  Every wave issues its share of each
//     tile's copies.  Before reading a tile a wave waits for its own copies of it (an explicit
//     vmcnt, which counts only what this wave issued), and one workgroup barrier per tile then
//     publishes the tile and frees the slot read one tile earlier, which the next copies refill.
//     LDS reads of the ring are issued as inline ds_read so the compiler does not add its own
//     (conservative: every in-flight copy) waits for the direct-to-LDS writes.
//   * q.k^T, E4M3 KV: v_mfma_scale_f32_32x32x64_f8f6f4 straight on the ring's E4M3 bytes (no K
//     conversion), q split exactly into E4M3 terms (two for a bf16 q, three for f16) scaled per
//     head by a power of two the score multiplier takes back.  Lane (i = l % 32, hh = l / 32) reads
//     d = 64 ks + 32 hh + 0..31 of token i at k-step ks (two 16-byte chunks); chunk c of K row r
//     is stored at c ^ (r & 7), so the lanes of each LDS read phase hit different bank groups.
//     INT8 KV: each wave converts a quarter of a tile's K into an exact-f16 staging buffer in the
//     A-operand order, two tiles ahead; 32x32x16 f16 MFMAs against q scaled exactly into f16.
//     f16 / bf16 KV (q of the same type): rows of 256 bytes; the 32x32x16 MFMA of that type reads
//     K from the ring as is (k-step kk: d = 64 hh + 8 kk + 0..7, one 16-byte chunk, chunk c of
//     row r at c ^ (r & 15)).
//   * p.V: O^T (128 d x 32 heads) = V^T . P^T, four 32-row d-tiles, two 16-token k-steps.  The
//     score C tile holds, in lane l register r, token 8(r/4) + 4hh + r%4 of head i; registers
//     8s..8s+7 are exactly the B operand (P^T) of k-step s when k-slot j of lane half hh means
//     token 16s + 8(j/4) + 4hh + j%4, so P never moves between lanes.  The A operand (V^T) of lane
//     (i, hh) for d-tile dt holds d = 4i + dt of those 8 tokens: each wave re-lays a quarter of the
//     next tile's V into a staging buffer in that order (E4M3 and INT8: converted to f16; f16 and
//     bf16: a halfword permute), so each d-tile's operand is one 16-byte LDS read.  bf16 V takes P
//     as two bf16 terms (hi + lo), so the weights keep f32-like precision against exact V.
//   * Softmax in log2 units with v_exp_f32, as in the 16-head kernel; per-token v scales move the
//     accumulator's power-of-two reference exponent lazily, like the running max.
//   * A window of query tokens (a separate instantiation) adds a per-column limit: scores past a
//     column's last visible token are kept out of the tile max and get weight 0.
//   * Partial rows: f16 of value / row scale for E4M3 and INT8, fp32 for f16 / bf16 KV.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fd_device.h"

namespace fd {
namespace {

// Largest batch whose per-sequence tile prefix sums a wide workgroup keeps in LDS (the ring and
// the staging buffers take most of the LDS, two workgroups share one CU's 160 KB; larger batches,
// and 16-bit KV, whose ring and staging fill 80 KB, locate tiles with a wave scan of seq_len).
constexpr int kWideLdsBatch = 256;

// Tile max of a window column that sees none of the tile's tokens (log2 units): finite, and far
// below any score a finite input can give.
constexpr float kNoScore = -1.0e30f;

// s_waitcnt immediate that waits for vmcnt <= n and nothing else (gfx9 field layout:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at bits 15:14).
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// s_waitcnt lgkmcnt(0) alone
constexpr int waitcnt_lgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

// f16 staging of a tile's V in p.V operand order: 2 k-steps x 4 d-tiles, 1 KB each
constexpr int kVStageBlock = 1024;
constexpr int kVStageBytes = 8 * kVStageBlock;
// INT8 KV: f16 staging of a tile's K in q.k^T operand order: 8 k-steps of 16 d, 1 KB each
constexpr int kKStageBlock = 1024;
constexpr int kKStageBytes = 8 * kKStageBlock;

template <int KVT, int WPG, int SCALE>
struct WideLayout {
    static constexpr bool KV16 = KVT == KV_F16 || KVT == KV_BF16;
    static constexpr int ROWB = KV16 ? 256 : 128;    // bytes of one token's K (or V) row, one kv head
    static constexpr int KV_BYTES = kTile * ROWB;    // one tile of K (or V)
    static constexpr int RPC = 1024 / ROWB;          // rows per 1 KB copy
    static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
    static constexpr int NCK = KV_BYTES / 1024;      // 1 KB copies per tile of K (or V)
    static constexpr int SC_BYTES = 256;             // per wave: 32 k then 32 v scales of a tile
    static constexpr int SLOT = 2 * KV_BYTES + (SCALE == SC_TOKEN_HEAD ? WPG * SC_BYTES : 0);
    static constexpr int OPS_KV = 2 * NCK / WPG;     // 1 KB copies per wave per tile
    static constexpr int OPS = OPS_KV + (SCALE == SC_TOKEN_HEAD ? 1 : 0);
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

// Direct-to-LDS copies: lane i moves 16 (or 4) bytes from its own global address to
// dst + 16 i (dst + 4 i); dst is wave-uniform.
__device__ __forceinline__ void copy16_to_lds(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds((gbl_void_t *)src, (lds_void_t *)dst, 16, 0, 0);
}
__device__ __forceinline__ void copy4_to_lds(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds((gbl_void_t *)src, (lds_void_t *)dst, 4, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(lds_void_t *)p; }

// Four 16-byte LDS reads at a + 0, 32, 64, 96 bytes, complete on return.
__device__ __forceinline__ void lds_read_4x16_s32(u32x4_t (&r)[4], uint32_t a) {
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

// Two 16-byte LDS reads at a + 0 and a + 32 bytes, complete on return.
__device__ __forceinline__ void lds_read_2x16_s32(u32x4_t (&r)[2], uint32_t a) {
    asm volatile(
        "ds_read_b128 %0, %2 offset:0\n\t"
        "ds_read_b128 %1, %2 offset:32\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1])
        : "v"(a)
        : "memory");
}

// x = 0 unless thr >= lh4 (a token is kept when its offset within the lane's run, subtracted from
// the tile's last valid token, is still at least the lane-half offset 4 lh).  Inline, so that the
// compare stays inside the rarely taken branch of a partial tile instead of being hoisted into
// every tile.  x may come straight from a transcendental op (v_exp_f32), whose result a following
// VALU read must wait for: the asm starts with wait states of its own (the compiler does not pad
// inline asm for that hazard).
__device__ __forceinline__ void keep_if_ge(float &x, int thr, int lh4) {
    asm volatile("s_nop 1\n\tv_cmp_ge_i32 vcc, %1, %2\n\tv_cndmask_b32 %0, 0, %0, vcc" : "+v"(x) : "s"(thr), "v"(lh4) : "vcc");
}

// Four 16-byte LDS reads, complete on return.
__device__ __forceinline__ void lds_read_4x16(u32x4_t (&r)[4], uint32_t a0, uint32_t a1, uint32_t a2,
                                              uint32_t a3) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
        : "memory");
}

// Four 4-byte LDS reads from four consecutive 128-byte rows past a, complete on return.
__device__ __forceinline__ void lds_read_rows4(uint32_t (&w)[4], uint32_t a) {
    asm volatile(
        "ds_read_b32 %0, %4 offset:0\n\t"
        "ds_read_b32 %1, %4 offset:128\n\t"
        "ds_read_b32 %2, %4 offset:256\n\t"
        "ds_read_b32 %3, %4 offset:384\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3])
        : "v"(a)
        : "memory");
}

// Four 8-byte LDS reads from four consecutive 256-byte rows past a, complete on return.
__device__ __forceinline__ void lds_read_rows4_b64(u32x2_t (&w)[4], uint32_t a) {
    asm volatile(
        "ds_read_b64 %0, %4 offset:0\n\t"
        "ds_read_b64 %1, %4 offset:256\n\t"
        "ds_read_b64 %2, %4 offset:512\n\t"
        "ds_read_b64 %3, %4 offset:768\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3])
        : "v"(a)
        : "memory");
}

// One 16-byte LDS read, complete on return.
__device__ __forceinline__ void lds_read_1x16(u32x4_t (&r)[1], uint32_t a) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r[0]) : "v"(a) : "memory");
}

// One 16-byte LDS write (not waited for here, as the 8-byte one below).
__device__ __forceinline__ void lds_write_16(uint32_t a, uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
    const u32x4_t v = {x0, x1, x2, x3};
    asm volatile("ds_write_b128 %0, %1" : : "v"(a), "v"(v) : "memory");
}

// One 8-byte LDS write (not waited for here: LDS operations of a wave complete in order, and the
// next LDS read's wait, or the wait before the workgroup barrier, covers it).
__device__ __forceinline__ void lds_write_8(uint32_t a, uint32_t lo, uint32_t hi) {
    const u32x2_t v = {lo, hi};
    asm volatile("ds_write_b64 %0, %1" : : "v"(a), "v"(v) : "memory");
}

// Largest of x over lanes i and i ^ 32 (the two lane halves): one v_permlane32_swap, no LDS.
// (Elements of the returned pair are copied to scalars before any bit cast: a bit cast straight
// from a vector element reads element 0 with this compiler.)
__device__ __forceinline__ float max_halves(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t a = r[0], b = r[1];
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

// Workgroup barrier that the compiler may not move memory operations across.
__device__ __forceinline__ void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace

template <int KVT, int WPG, int NSLOT, int QT, int SCALE, bool PAGED, bool B16, bool WIN>
__global__ __launch_bounds__(64 * WPG) __attribute__((amdgpu_waves_per_eu(2)))
void wide_partition_kernel(Params p) {
    using LY = WideLayout<KVT, WPG, SCALE>;
    constexpr int D = 128;
    constexpr bool KV16 = LY::KV16;
    constexpr int EB = KV16 ? 2 : 1;  // bytes per KV element
    static_assert(!KV16 || (QT == KVT && SCALE == SC_NONE && WPG == 4), "16-bit KV: q of the same type, no scales");
    // tiles whose data is consumed ahead of the computed one: V one tile ahead; INT8 K two
    constexpr int AHEAD = KVT == KV_I8 ? 2 : 1;
    static_assert(NSLOT >= 3 + AHEAD, "the ring holds the tile being read, the ones being converted, one "
                                      "being refilled and at least one more in flight");
    static_assert((NSLOT - 2) * LY::OPS < 64, "vmcnt field is 6 bits");
    __shared__ __attribute__((aligned(16))) uint8_t ring[NSLOT * LY::SLOT];
    // V of a tile as f16 (bf16 KV: bf16) in p.V's MFMA operand order, two buffers (the tile being
    // computed and the next one, converted by all waves of the workgroup together, a quarter each)
    __shared__ __attribute__((aligned(16))) uint8_t vstage[2 * kVStageBytes];
    // INT8 KV: K the same way, as exact f16 for q.k^T on f16 MFMAs
    __shared__ __attribute__((aligned(16))) uint8_t kstage[KVT == KV_I8 ? 2 * kKStageBytes : 16];
    // (16-bit KV: ring and staging alone fill 80 KB, two workgroups per CU; the arrays below are
    // then never referenced and take no LDS, and tiles are located by a wave scan)
    constexpr int LDS_BATCH = KV16 ? 0 : kWideLdsBatch;
    __shared__ int sh_prefix[kWideLdsBatch + 1];

    // (the wave index is uniform: kept in a scalar register, so per-wave choices are scalar)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int li = lane & 31, lh = lane >> 5;
    const int64_t wg = blockIdx.x, W = gridDim.x;
    const int groups = p.groups;
    const bool lds_prefix = LDS_BATCH > 0 && p.batch <= LDS_BATCH;

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
    // floor of a 16-bit partial row's scale sc: sv / sc stays finite for any v scale sv (rows of
    // denormal magnitude), and the stored values acc * sv / sc still lie in [-1, 1]
    // (wave-uniform: kept in a scalar register for the whole kernel)
    const float sc_floor = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(
                   uint32_t, fmaxf(fabsf(SCALE == SC_TENSOR ? tensor_v : 1.0f) * kMinNormal, kMinNormal))));
    const uint32_t row_bytes = (uint32_t)p.hkv * D * EB;  // bytes per cache row (all kv heads)

    // ---- tile cursors: one issuing copies NSLOT-1 tiles ahead, one computing
    // kvh: kv head of the unit group grp (kept with the cursor: it changes only with the group)
    struct Cursor {
        int64_t pos;
        int b, Tb, grp, tt, n, kvh;
    };
    auto group_kvh = [&](int grp) -> int { return uni((grp * WPG) / p.nhb); };
    auto locate = [&](Cursor &k, int64_t at) {
        k.pos = at;
        if (lds_prefix) {
            int l0 = 0, h0 = p.batch;
            while (h0 - l0 > 1) {
                const int mid = (l0 + h0) >> 1;
                if ((int64_t)sh_prefix[mid] * groups <= at) l0 = mid;
                else h0 = mid;
            }
            k.b = uni(l0);
            k.Tb = uni(sh_prefix[k.b + 1] - sh_prefix[k.b]);
            const int64_t rel = at - (int64_t)sh_prefix[k.b] * groups;
            k.grp = uni((int)(rel / k.Tb));
            k.tt = uni((int)(rel % k.Tb));
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
                    k.b = uni(b0 + src);
                    k.Tb = uni(__shfl(t, src, 64));
                    const int64_t Pb = base + uni(__shfl(incl, src, 64)) - k.Tb;
                    const int64_t rel = at - Pb * groups;
                    k.grp = uni((int)(rel / k.Tb));
                    k.tt = uni((int)(rel % k.Tb));
                    break;
                }
                base += uni(__shfl(incl, 63, 64));
            }
        }
        k.n = max(0, min(ld_uniform(p.seq_len, k.b), p.max_seq_len));
        k.kvh = group_kvh(k.grp);
    };
    // one tile forward (crossing unit groups and sequences); false, unmoved, at the range end
    auto step = [&](Cursor &k) -> bool {
        if (k.pos + 1 >= hi) return false;
        k.pos++;
        if (++k.tt == k.Tb) {
            k.tt = 0;
            if (++k.grp == groups) {
                k.grp = 0;
                do {
                    k.b++;
                } while ((k.Tb = lds_prefix ? uni(sh_prefix[k.b + 1] - sh_prefix[k.b]) : seq_tiles_u(p, k.b)) == 0);
                k.n = max(0, min(ld_uniform(p.seq_len, k.b), p.max_seq_len));
            }
            k.kvh = group_kvh(k.grp);
        }
        return true;
    };
    auto next_slot = [](int si) -> int { return si + 1 == NSLOT ? 0 : si + 1; };

    // ---- copies of one tile into a ring slot (this wave's share)
    // block sizes are 16, 32 or 64: block index and offset by shift and mask
    const int bsh = PAGED ? (B16 ? 4 : uni(__builtin_ctz((unsigned)p.block_size))) : 0;
    auto issue = [&](const Cursor &k, int si) {
        const int t0 = k.tt * kTile;
        const int last = min(k.n - t0, kTile) - 1;  // rows past it repeat it (valid; masked later)
        // first cache rows of the tile's two 16-token halves (blocks of 16 tokens: two blocks)
        int64_t row0, row1;
        if constexpr (PAGED) {
            row0 = ((int64_t)ld_uniform(p.block_table, (size_t)k.b * p.max_blocks + (t0 >> bsh)) << bsh) +
                   (t0 & ((1 << bsh) - 1));
            if constexpr (B16)
                row1 = last < 16 ? row0 + 16
                                 : (int64_t)ld_uniform(p.block_table, (size_t)k.b * p.max_blocks + (t0 >> 4) + 1) << 4;
            else
                row1 = row0 + 16;
        } else {
            row0 = (int64_t)ld_uniform(p.kv_start, k.b) + t0;
            row1 = row0 + 16;
        }
        uint8_t *slot = ring + si * LY::SLOT;
        // uniform base of the tile's first row; each lane adds a 32-bit offset (a tile of 32 rows
        // inside one block, or two 16-row blocks, each contiguous)
        const uint8_t *kb = (const uint8_t *)p.k + (size_t)k.kvh * D * EB + row0 * row_bytes;
        const uint8_t *vb = (const uint8_t *)p.v + (size_t)k.kvh * D * EB + row0 * row_bytes;
        const int64_t jump = B16 ? (row1 - row0 - 16) * row_bytes : 0;  // second block's shift
#pragma unroll
        for (int u = 0; u < LY::OPS_KV; u++) {
            // copies 0..NCK-1: K rows RPC oo .. RPC oo + RPC-1; NCK..2 NCK-1: V rows (oo = o % NCK);
            // lane L writes chunk position L % CPR of row RPC oo + L / CPR (a K chunk c sits at
            // position c ^ (row % CPR))
            const int o = wave * LY::OPS_KV + u;
            const int oo = o % LY::NCK;
            const int row = LY::RPC * oo + lane / LY::CPR, pos = lane % LY::CPR;
            const int r = min(row, last);
            const uint32_t off = __umul24((uint32_t)r, row_bytes);
            const int64_t shift = (B16 && r >= 16) ? jump : 0;
            if (o < LY::NCK)
                copy16_to_lds(kb + shift + off + 16 * (pos ^ (row & (LY::CPR - 1))), slot + oo * 1024);
            else
                copy16_to_lds(vb + shift + off + 16 * pos, slot + LY::KV_BYTES + oo * 1024);
        }
        if constexpr (SCALE == SC_TOKEN_HEAD) {
            const int t = min(lane & 31, last);
            const int64_t crow = B16 && t >= 16 ? row1 + (t - 16) : row0 + t;
            const float *sb = (lane < 32 ? p.k_scale : p.v_scale) + k.kvh + (size_t)crow * p.hkv;
            copy4_to_lds(sb, slot + 2 * LY::KV_BYTES + wave * LY::SC_BYTES);
        }
    };

    // ---- per-lane LDS offsets within a slot
    const uint32_t ring0 = lds_addr(ring);
    // K operand of the E4M3 q.k^T MFMA: token li; k-step ks = q / 2 (32x32x64): d = 64 ks + 32 lh
    // + 0..31, the row's 16-byte chunks 4 ks + 2 lh and 4 ks + 2 lh + 1.  Chunk c of row r is
    // stored at c ^ (r & 7).  (INT8 KV reads K from its f16 staging instead.)
    // 16-bit KV: k-step kk (32x32x16) takes d = 64 lh + 8 kk + 0..7, chunk 8 lh + kk of token li,
    // stored at (8 lh + kk) ^ (li & 15).
    constexpr bool I8 = KVT == KV_I8;
    constexpr int NKR = KV16 ? 8 : 4;  // K operand reads per tile
    uint32_t koff[NKR];
#pragma unroll
    for (int q = 0; q < NKR; q++)
        koff[q] = KV16 ? li * LY::ROWB + 16 * ((8 * lh + q) ^ (li & 15))
                       : li * LY::ROWB + 16 * ((4 * (q >> 1) + 2 * lh + (q & 1)) ^ (li & 7));
    const uint32_t vst0 = lds_addr(vstage);
    const uint32_t soff = 2 * LY::KV_BYTES + wave * LY::SC_BYTES + 16 * lh;

    // ---- per-segment state
    // q operand of q.k^T, for head li; the head's score multiplier qk_head carries 2^-eq (and, for
    // a negative per-tensor k scale, q carries the sign):
    //   E4M3 KV: NQT E4M3 terms whose sum is q * 2^eq exactly (bf16 q: 2 terms, f16 q: 3), d =
    //            64 ks + 32 lh + j in byte j of qf8[t][ks] (32 bytes per term and k-step);
    //   INT8 KV: f16 of q * 2^eq (the largest |q * 2^eq| lies in [2^14, 2^15): every value within
    //            2^28 of it is an f16 normal number and converts exactly, bf16's 8-bit or f16's
    //            11-bit significand fitting f16's), d = 16 ks + 8 lh + j in half j of qh[ks].
    //   16-bit KV: q as is, d = 64 lh + 8 kk + j in half j of qh[kk].
    constexpr int NQT = QT == KV_BF16 ? 2 : 3;
    i32x8_t qf8[(I8 || KV16) ? 1 : NQT][2];
    u32x4_t qh[(I8 || KV16) ? 8 : 1];
    float qk_head = qk_scale;
    f32x16_t acc[4];
    float m_run = -INFINITY, l_run = 0.0f;
    // per-token v scales: the accumulator holds values / 2^ev (wave-uniform reference exponent)
    int ev = 0;
    // a window of nq query tokens: column (row m, head h) of the kv head sees the sequence up to
    // nq - 1 - m tokens before its end
    int win_off = 0;
    // lane column li of head block hb: column col = 32 hb + li of the kv head = query row m of the
    // window, head h of the group; its out / lse row
    auto out_row = [&](int b, int u_in) -> size_t {
        const int kvh = u_in / p.nhb, col = (u_in % p.nhb) * kWideHeadBlock + li;
        const int m = col / p.group, h = kvh * p.group + col % p.group;
        return ((size_t)b * p.nq + m) * p.hq + h;
    };
    auto load_q = [&](int b, int grp) {
        const int u_in = grp * WPG + wave;
        if constexpr (WIN) win_off = p.nq - 1 - ((u_in % p.nhb) * kWideHeadBlock + li) / p.group;
        const size_t qrow_idx = out_row(b, u_in);
        if constexpr (KV16) {
            const uint16_t *qrow = (const uint16_t *)p.q + qrow_idx * D + 64 * lh;
#pragma unroll
            for (int kk = 0; kk < 8; kk++) qh[kk] = *(const u32x4_t *)(qrow + 8 * kk);
            // complete here (once per segment; see below)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            // the multiplier is kept >= 0 (the tile max is taken on raw scores): a negative softmax
            // scale flips q's sign bits instead (exact)
            if (qk_scale < 0.0f) {
#pragma unroll
                for (int kk = 0; kk < 8; kk++) qh[kk] ^= u32x4_t{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
            }
            qk_head = fabsf(qk_scale);
        } else {
            const uint16_t *qrow = (const uint16_t *)p.q + qrow_idx * D + (I8 ? 8 : 32) * lh;
            // E4M3: raw[4 ks + c] holds d = 64 ks + 32 lh + 8 c + 0..7; INT8: raw[ks] holds
            // d = 16 ks + 8 lh + 0..7
            u32x4_t raw[8];
#pragma unroll
            for (int i = 0; i < 8; i++)
                raw[i] = *(const u32x4_t *)(qrow + (I8 ? 16 * i : 64 * (i >> 2) + 8 * (i & 3)));
            // complete here (a drain, once per segment), so that no load is pending at the top of the
            // tile loop and the compiler adds no wait on the in-flight tile copies there
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            // largest |q| of head li over its 128 values (this lane's 64 and lane li + 32 * (1 - lh)'s):
            // bf16 / f16 bit patterns with the sign cleared order like the magnitudes
            uint32_t mx = 0;
#pragma unroll
            for (int i = 0; i < 8; i++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const uint32_t w = raw[i][e] & 0x7FFF7FFFu;
                    mx = max(mx, max(w & 0xFFFFu, w >> 16));
                }
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32, 64));
            // 2^eq puts the largest |q| in [2^7, 2^8), inside E4M3's range (largest finite 448); for
            // INT8 KV (f16 q) in [2^14, 2^15)
            const int target = I8 ? 14 : 7;
            int eq = 0;
            if (mx != 0) eq = QT == KV_BF16 ? target + 127 - (int)(mx >> 7) : target + 15 - (int)(mx >> 10);
            // per-tensor scale: the multiplier is kept >= 0 (the tile max is then taken on raw scores)
            const bool flip = SCALE == SC_TENSOR && qk_scale < 0.0f;
            qk_head = __builtin_amdgcn_ldexpf(flip ? -qk_scale : qk_scale, -eq);
            auto to_f32 = [](uint32_t h) -> float {
                if constexpr (QT == KV_BF16) return __builtin_bit_cast(float, h << 16);
                else return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
            };
#pragma unroll
            for (int i = 0; i < 8; i++)
#pragma unroll
                for (int e2 = 0; e2 < 2; e2++) {
                    // values 4 e2 .. 4 e2 + 3 of raw[i]: d = 8 c + 4 e2 + 0..3 -> dword 2 c + e2 of a term
                    float x[4];
#pragma unroll
                    for (int h = 0; h < 4; h++) {
                        const uint32_t w = raw[i][2 * e2 + (h >> 1)];
                        const float v = to_f32((h & 1) ? (w >> 16) : (w & 0xFFFFu));
                        x[h] = __builtin_amdgcn_ldexpf(flip ? -v : v, eq);
                    }
                    if constexpr (I8) {
                        // exact f16 pairs (d = 8 lh + 4 e2 + 0..3 of k-step i)
                        qh[i][2 * e2] = pack_f16(x[0], x[1]);
                        qh[i][2 * e2 + 1] = pack_f16(x[2], x[3]);
                    } else {
#pragma unroll
                        for (int t = 0; t < NQT; t++) {
                            // nearest E4M3 values (exact hardware convert, ties to even); the remainder is
                            // exact in fp32 and has few enough significant bits for the next term
                            i16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2_t{0, 0}, x[0], x[1], 1.0f, false);
                            c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, x[2], x[3], 1.0f, true);
                            const uint32_t cw = __builtin_bit_cast(uint32_t, c);
                            qf8[t][i >> 2][2 * (i & 3) + e2] = (int)cw;
                            if (t + 1 < NQT) {
                                const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw, 1.0f, false);
                                const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw, 1.0f, true);
                                x[0] -= lo[0];
                                x[1] -= lo[1];
                                x[2] -= hi[0];
                                x[3] -= hi[1];
                            }
                        }
                    }
                }
        }
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

    const int lh4 = 4 * lh;
    // ---- V of the tile in ring slot si -> f16 staging buffer buf, this wave's share.  Operand
    // layout: block (ks, dt) of 1 KB holds, for each lane l = (i, hh) of the reading wave, the 8 f16
    // of d = 4i + dt at tokens 16 ks + 4 hh + {0, 1, 2, 3, 8, 9, 10, 11} (16 bytes at 16 l).  The
    // tile is four passes j = (ks, hh): in a pass, lane L converts for reader lane 32 hh + L % 32 the
    // four tokens 16 ks + 4 hh + 8 (L / 32) + 0..3 (one 4-byte read per token row, d = 4 (L % 32) +
    // 0..3) and writes 8 bytes per d-tile.  Waves take 4 / WPG passes each.
    auto convert_v = [&](int si, int buf) {
        const uint32_t vsrc = ring0 + si * LY::SLOT + LY::KV_BYTES;
        const uint32_t vdst = vst0 + buf * kVStageBytes;
        const int th = lane >> 5, lv = lane & 31;
#pragma unroll 1  // (2-wave workgroups: one pass after the other, not both held in registers)
        for (int jj = 0; jj < 4 / WPG; jj++) {
            const int j = wave * (4 / WPG) + jj;  // wave-uniform
            const int ks = j >> 1, hh = j & 1;
            uint32_t o[4][2];  // [dt][token pair]
            if constexpr (KV16) {
                // 16-bit V: 8 bytes (d = 4 lv .. 4 lv + 3) of each of the four token rows; the pair
                // (token 2u, token 2u + 1) of one d is a halfword permute, no conversion
                u32x2_t w2[4];
                lds_read_rows4_b64(w2, vsrc + (16 * ks + 4 * hh + 8 * th) * LY::ROWB + 8 * lv);
#pragma unroll
                for (int u = 0; u < 2; u++) {
                    const u32x2_t a = w2[2 * u + 1], b = w2[2 * u];
                    const uint32_t a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
                    o[0][u] = __builtin_amdgcn_perm(a0, b0, 0x05040100u);
                    o[1][u] = __builtin_amdgcn_perm(a0, b0, 0x07060302u);
                    o[2][u] = __builtin_amdgcn_perm(a1, b1, 0x05040100u);
                    o[3][u] = __builtin_amdgcn_perm(a1, b1, 0x07060302u);
                }
            } else {
                uint32_t w[4];
                lds_read_rows4(w, vsrc + (16 * ks + 4 * hh + 8 * th) * LY::ROWB + 4 * lv);
#pragma unroll
                for (int u = 0; u < 2; u++) {
                    if constexpr (I8) {
                        // byte k of rows 2u, 2u+1 -> bytes 0 and 2 of a dword (zeros between: selector
                        // 0x0C) -> the exact f16 pair of the two codes
#pragma unroll
                        for (int k = 0; k < 4; k++)
                            o[k][u] = i8x2_to_f16x2(__builtin_amdgcn_perm(w[2 * u + 1], w[2 * u],
                                                                              0x0C000C00u | ((4u + k) << 16) | (uint32_t)k));
                    } else {
                        const uint32_t x = __builtin_amdgcn_perm(w[2 * u + 1], w[2 * u], 0x05010400u);
                        const uint32_t y = __builtin_amdgcn_perm(w[2 * u + 1], w[2 * u], 0x07030602u);
                        o[0][u] = cvt_fp8x2<KV_F16, false>(x);
                        o[1][u] = cvt_fp8x2<KV_F16, true>(x);
                        o[2][u] = cvt_fp8x2<KV_F16, false>(y);
                        o[3][u] = cvt_fp8x2<KV_F16, true>(y);
                    }
                }
            }
            const uint32_t at = vdst + ks * 4 * kVStageBlock + 16 * (32 * hh + lv) + 8 * th;
#pragma unroll
            for (int dt = 0; dt < 4; dt++) lds_write_8(at + dt * kVStageBlock, o[dt][0], o[dt][1]);
        }
    };

    // K operand of q.k^T for the tile about to be computed (read one tile ahead): E4M3 raw bytes
    // from the ring; INT8 exact f16 from its staging buffer
    u32x4_t kr[NKR];
    u32x4_t kf[KVT == KV_I8 ? 8 : 1];
    auto read_kf = [&](int kbuf) {
        const u32x4_t *kp = (const u32x4_t *)(kstage + kbuf * kKStageBytes) + lane;
#pragma unroll
        for (int ks = 0; ks < 8; ks++) kf[ks] = kp[ks * (kKStageBlock / 16)];
    };
    auto read_k = [&](int si) {
        const uint32_t b = ring0 + si * LY::SLOT;
#pragma unroll
        for (int h = 0; h < NKR / 4; h++) {
            u32x4_t r4[4];
            lds_read_4x16(r4, b + koff[4 * h], b + koff[4 * h + 1], b + koff[4 * h + 2], b + koff[4 * h + 3]);
#pragma unroll
            for (int i = 0; i < 4; i++) kr[4 * h + i] = r4[i];
        }
    };
    // ---- INT8 KV: K of the tile in ring slot si -> exact f16 staging buffer buf, this wave's share.
    // Operand layout: block ks of 1 KB holds, for each lane l = (i, hh) of the reading wave, the 8
    // f16 of token i at d = 16 ks + 8 hh + 0..7 (16 bytes at 16 l).  The ring's row t holds 16-byte
    // chunk c (d = 16 c .. 16 c + 15) at c ^ (t & 7); lane L converts token L % 32's chunk
    // c = 2 j + L / 32 in each of its passes j and writes both halves (hh = 0, 1) of block c.
    auto convert_k = [&](int si, int buf) {
        const uint32_t ksrc = ring0 + si * LY::SLOT;
        const uint32_t kdst = lds_addr(kstage) + buf * kKStageBytes;
        const int t = lane & 31, half = lane >> 5;
#pragma unroll 1
        for (int jj = 0; jj < 4 / WPG; jj++) {
            const int c = 2 * (wave * (4 / WPG) + jj) + half;
            u32x4_t w[1];
            lds_read_1x16(w, ksrc + t * LY::ROWB + 16 * (c ^ (t & 7)));
            uint32_t o[8];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                // bytes 0, 1 and 2, 3 of the dword -> bytes 0 and 2 of a dword (zeros between)
                o[2 * e] = i8x2_to_f16x2(__builtin_amdgcn_perm(w[0][e], w[0][e], 0x0C010C00u));
                o[2 * e + 1] = i8x2_to_f16x2(__builtin_amdgcn_perm(w[0][e], w[0][e], 0x0C030C02u));
            }
            const uint32_t at = kdst + c * kKStageBlock + 16 * t;
            lds_write_16(at, o[0], o[1], o[2], o[3]);
            lds_write_16(at + 16 * 32, o[4], o[5], o[6], o[7]);
        }
    };

    // the tile in ring slot si (its K already in kr), its V staged in buffer buf; the next tile's V
    // (ring slot si_next) is converted into the other buffer while the q.k^T MFMAs run, and the
    // next tile's K is read while the p.V MFMAs run (that tile has landed and was published by
    // this step's barrier; its slot is refilled two steps later)
    auto compute = [&](int si, int buf, int nrel, int si_next) {
        const int last = min(nrel, kTile) - 1;  // rows past it repeat it (valid; masked later)
        const uint32_t sbase = ring0 + si * LY::SLOT;
        // p.V's A operands of both k-steps, read now (plain loads: the staging buffer is never a
        // copy target, so the compiler waits for these reads only where p.V uses them)
        u32x4_t va[2][4];
        {
            const u32x4_t *vp = (const u32x4_t *)(vstage + buf * kVStageBytes) + lane;
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
#pragma unroll
                for (int dt = 0; dt < 4; dt++) va[ks][dt] = vp[(ks * 4 + dt) * (kVStageBlock / 16)];
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_sched_barrier(0);
        // the next tile's conversions, placed after the q.k^T MFMAs are issued: their LDS waits and
        // VALU work run while the matrix unit is busy
        auto convert_next = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            convert_v(si_next, buf ^ 1);
            // INT8: K two tiles ahead, into the K buffer this tile's K was read from
            if constexpr (I8) convert_k(next_slot(si_next), buf);
            __builtin_amdgcn_sched_barrier(0);
        };
        // per-token scales: element to a scalar before the bit cast (a bit cast straight from a
        // vector element reads element 0 with this compiler)
        auto read_scales = [&](float (&sc)[16], uint32_t at) {
            u32x4_t raw[4];
            lds_read_4x16_s32(raw, at);
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const uint32_t w = raw[r >> 2][r & 3];
                sc[r] = __builtin_bit_cast(float, w);
            }
        };

        // ---- scores S[token][head] = K . (q * 2^eq) straight from the ring's bytes (no conversion)
        f32x16_t S;
        if constexpr (I8) {
            // INT8: exact f16 K (staged) times exact f16 q on 32x32x16 f16 MFMAs, eight 16-deep k-steps
#pragma unroll
            for (int r = 0; r < 16; r++) S[r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 8; ks++) S = mfma32_f16(kf[ks], qh[ks], S);
            convert_next();
        } else if constexpr (KV16) {
            // 16-bit KV: K from the ring times q, both of q's type, eight 16-deep k-steps
#pragma unroll
            for (int r = 0; r < 16; r++) S[r] = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 8; kk++) S = mfma32_qk<KVT>(kr[kk], qh[kk], S);
            convert_next();
        } else {
            // E4M3: FP8 MFMAs, two 64-deep k-steps, NQT terms of q each
#pragma unroll
            for (int r = 0; r < 16; r++) S[r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const u32x4_t k0 = kr[2 * ks], k1 = kr[2 * ks + 1];
                const i32x8_t a = {(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3],
                                   (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
#pragma unroll
                for (int t = 0; t < NQT; t++)  // E4M3 x E4M3, both block scales 2^0 (E8M0 127)
                    S = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf8[t][ks], S, 0, 0, 0, 127, 0, 127);
            }
            convert_next();
        }
        float ksc[16];
        if constexpr (SCALE == SC_TOKEN_HEAD) read_scales(ksc, sbase + soff);
        // ---- online softmax (log2 units); lane holds tokens 8(r/4) + 4lh + r%4 of head li.
        // Per-tensor scale: s = S * qk_head with qk_head >= 0, so the tile max is qk_head times the
        // max of the raw scores and the multiply folds into the exponent's FMA below; per-token
        // scales: s = S * k_scale * qk_head per token.
        // A partial tile's rows past `last` are copies of row `last` (the copies clamp the row), so
        // they cannot raise the tile max; only their weights are zeroed below.
        float s[16];
#pragma unroll
        for (int r = 0; r < 16; r++) s[r] = (SCALE == SC_TOKEN_HEAD) ? S[r] * (ksc[r] * qk_head) : S[r];
        // a window's column stops nq - 1 - m tokens before the sequence's end: its later tokens are
        // real rows (of other columns) and are kept out of the max and the weights
        // (a separate instantiation: the one-token step keeps none of this in its registers)
        const int lastc = WIN ? min(nrel - win_off, kTile) - 1 : last;
        const bool wmask = WIN && __any(lastc < kTile - 1);  // wave-uniform
        if (wmask) {
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (8 * (r >> 2) + lh4 + (r & 3) > lastc) s[r] = -INFINITY;
        }
        float mt = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) mt = fmaxf(fmaxf(mt, s[r]), s[r + 1]);
        mt = fmaxf(mt, s[15]);
        mt = max_halves(mt);
        if constexpr (WIN) {
            // (-inf only for a window column that sees nothing of the tile: a finite stand-in far
            // below any score keeps m_run finite -- no -inf - -inf below -- and its weights are zeroed)
            if constexpr (SCALE != SC_TOKEN_HEAD) mt = mt > -INFINITY ? mt * qk_head : kNoScore;
            else mt = mt > -INFINITY ? mt : kNoScore;
        } else if constexpr (SCALE != SC_TOKEN_HEAD) {
            mt *= qk_head;  // finite: token 0 of the tile is valid
        }
        // per-token v scales: reference exponent of the tile's largest |v scale| (the lane's 16
        // tokens, then the other lane half); it replaces ev when out of ev's window
        int evt = ev;
        if constexpr (SCALE == SC_TOKEN_HEAD) {
            // (read here for the max only and again per k-step below: holding all 16 across the
            // softmax costs registers the kernel does not have)
            float vsc[16];
            read_scales(vsc, sbase + soff + 128);  // v scales lie 128 bytes after the k scales
            float vm = fabsf(vsc[0]);
#pragma unroll
            for (int r = 1; r < 16; r++) vm = fmaxf(vm, fabsf(vsc[r]));
            vm = max_halves(vm);
            evt = uni(vm > 0.0f ? exp2_ceil(vm) : ev);  // all-zero scales: keep ev
        }
        const bool emove = evt > ev + kVrefHigh || evt < ev - kVrefLow;
        if (__any(mt > m_run + kRescaleSlack) || emove) {  // wave-uniform; always taken on a segment's first tile
            const float m_new = fmaxf(m_run, mt);  // finite (mt is)
            const float dm = m_run - m_new;
            const float alpha = __builtin_amdgcn_exp2f(dm);
            // the accumulator also moves from units of 2^ev to units of 2^evt (exact for a power of two)
            const float alpha_acc = SCALE == SC_TOKEN_HEAD ? __builtin_amdgcn_exp2f(dm + (float)(ev - evt)) : alpha;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[i][r] *= alpha_acc;
            m_run = m_new;
            ev = evt;
        }
        // token-head scales: weights 2^(s - m - ev), i.e. divided by 2^ev (their sum is scaled back
        // for l, which stays in units of 2^m)
        float pj[16];
        const float m_ref = m_run + (SCALE == SC_TOKEN_HEAD ? (float)ev : 0.0f);
#pragma unroll
        for (int r = 0; r < 16; r++)
            pj[r] = __builtin_amdgcn_exp2f((SCALE == SC_TOKEN_HEAD) ? s[r] - m_ref : __builtin_fmaf(WIN ? s[r] : S[r], qk_head, -m_ref));
        if (last < kTile - 1) {  // a partial tile: weight 0 for tokens 8(r/4) + 4lh + r%4 past `last`
#pragma unroll
            for (int r = 0; r < 16; r++) keep_if_ge(pj[r], last - 8 * (r >> 2) - (r & 3), lh4);
        }
        if (wmask) {
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (8 * (r >> 2) + lh4 + (r & 3) > lastc) pj[r] = 0.0f;
        }
        if constexpr (SCALE == SC_TOKEN_HEAD || KVT == KV_BF16) {
            // (bf16 KV: the weights p.V multiplies are hi + lo, the f32 weights to ~2^-16)
            float psum = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; r++) psum += pj[r];
            l_run += __builtin_amdgcn_ldexpf(psum, ev);
        } else {
            // l sums the f16 weights p.V multiplies (acc and l then carry the same rounded weights)
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
            // v scales of this k-step's 8 tokens (registers 8ks .. 8ks+7)
            float vsc[8];
            if constexpr (SCALE == SC_TOKEN_HEAD) {
                u32x4_t raw[2];
                lds_read_2x16_s32(raw, sbase + soff + 128 + 64 * ks);
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const uint32_t w = raw[j >> 2][j & 3];
                    vsc[j] = __builtin_bit_cast(float, w);
                }
            }
            if constexpr (KVT == KV_BF16) {
                // P as bf16 hi + lo against the staged bf16 V: two MFMAs per d-tile
                uint32_t hi2[4], lo2[4];
#pragma unroll
                for (int u = 0; u < 4; u++) split_bf16_pair(pj[8 * ks + 2 * u], pj[8 * ks + 2 * u + 1], hi2[u], lo2[u]);
                const u32x4_t phi = {hi2[0], hi2[1], hi2[2], hi2[3]}, plo = {lo2[0], lo2[1], lo2[2], lo2[3]};
#pragma unroll
                for (int dt = 0; dt < 4; dt++) {
                    acc[dt] = mfma32_qk<KV_BF16>(va[ks][dt], phi, acc[dt]);
                    acc[dt] = mfma32_qk<KV_BF16>(va[ks][dt], plo, acc[dt]);
                }
            } else {
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
#pragma unroll
                for (int dt = 0; dt < 4; dt++) acc[dt] = mfma32_f16(va[ks][dt], pop, acc[dt]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (I8) read_kf(buf ^ 1);  // converted last step, published by this step's barrier
        else read_k(si_next);
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- segment result (lane (li, lh) holds d = 4i + dt, i = 8(r/4) + 4lh + r%4, in acc[dt][r])
    auto finalize = [&](const Cursor &k, int seg, bool whole) {
        const size_t orow_idx = out_row(k.b, k.grp * WPG + wave);
        const float l_tot = l_run + shfl_xor_f(l_run, 32);
        // factor of the accumulator: the tensor v scale, or 2^ev with per-token scales
        // (2^ev is a normal float: |ev| <= 100)
        const float sv = (SCALE == SC_TENSOR) ? tensor_v : __builtin_bit_cast(float, (uint32_t)(ev + 127) << 23);
        if (whole) {
            const size_t orow = orow_idx * D;
            const float inv = l_tot > 0.0f ? sv / l_tot : 0.0f;  // 0: a window row that sees no token
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const float v[4] = {acc[0][r] * inv, acc[1][r] * inv, acc[2][r] * inv, acc[3][r] * inv};
                store_row_chunk<4>(p.out, p.out_dtype, orow + 4 * (8 * (r >> 2) + 4 * lh + (r & 3)), v);
            }
            if (p.lse && lh == 0) p.lse[orow_idx] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
        } else {
            // slot 0: the range's first segment; slot 1: its last (a middle one is always whole).
            // E4M3 KV: f16 of value / (largest |value| of the head's row, spread over the two lane
            // halves), the scale beside it
            const size_t slot = (((size_t)wg * 2 + (seg == 0 ? 0 : 1)) * WPG + wave) * kWideHeadBlock + li;
            if constexpr (KV16) {
                // 16-bit KV: fp32 rows (no scales: the accumulator is the value)
                float *dst = p.ws_acc + slot * D;
#pragma unroll
                for (int r = 0; r < 16; r++)
                    *(float4 *)(dst + 4 * (8 * (r >> 2) + 4 * lh + (r & 3))) =
                        make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
                if (lh == 0) p.ws_ml[slot] = make_float2(m_run, l_tot);
                return;
            }
            float mx = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; r++)
#pragma unroll
                for (int dt = 0; dt < 4; dt++) mx = fmaxf(mx, fabsf(acc[dt][r] * sv));
            mx = fmaxf(mx, shfl_xor_f(mx, 32));
            // per-token scales: the floor follows 2^ev like sc_floor follows the tensor v scale
            const float floor_sc = SCALE == SC_TENSOR ? sc_floor : fmaxf(sv * kMinNormal, kMinNormal);
            const float sc = fmaxf(mx, floor_sc), inv = sv / sc;
            uint16_t *dst = (uint16_t *)p.ws_acc + slot * D;
#pragma unroll
            for (int r = 0; r < 16; r++)
                *(u32x2_t *)(dst + 4 * (8 * (r >> 2) + 4 * lh + (r & 3))) =
                    u32x2_t{pack_f16(acc[0][r] * inv, acc[1][r] * inv), pack_f16(acc[2][r] * inv, acc[3][r] * inv)};
            if (lh == 0) {
                p.ws_ml[slot] = make_float2(m_run, l_tot);
                p.ws_sc[slot] = sc;
            }
        }
    };

    // ---- pipeline: copies of tiles lo .. lo+NSLOT-2 in flight before the first compute; each
    // step waits for the tile after its own, barriers, refills the slot freed by the previous
    // tile (past the range end the issue cursor repeats its last tile, so every wave always has
    // the same number of copies in flight), converts its share of the next tile's V and computes
    // its tile from the ring's K and the staged V.
    Cursor ic, cc;
    locate(ic, lo);
    cc = ic;
    issue(ic, 0);
#pragma unroll
    for (int k = 1; k <= NSLOT - 2; k++) {
        step(ic);
        issue(ic, k);
    }
    int seg = 0, seg_start = cc.tt;
    int slot_c = 0, slot_i = NSLOT - 1;  // ring slots of the computed tile and of the next copies
    int buf = 0;                         // staging buffer holding the computed tile's V
    bool stores_pending = false;
    load_q(cc.b, cc.grp);  // (drains this wave's copies: the first tiles have landed)
    reset_state();
    // the first tile's V and K, once every wave's copies of it have landed
    wg_barrier();
    convert_v(slot_c, buf);
    if constexpr (I8) {
        convert_k(slot_c, 0);
        convert_k(next_slot(slot_c), 1);
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0);
        wg_barrier();
        read_kf(0);
    } else {
        read_k(slot_c);
    }
    for (;;) {
        // own copies of the tile AHEAD of this one done (younger ones may still be in flight);
        // after stores, wait for everything (loads and stores need not retire in order).  The
        // barrier then publishes that tile, this tile's converted V (and INT8: the next tile's
        // converted K), and frees the ring slot and staging buffers read in the previous step.
        if (stores_pending) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm((NSLOT - 2 - AHEAD) * LY::OPS));
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0);  // this wave's staging writes
        stores_pending = false;
        wg_barrier();
        step(ic);
        issue(ic, slot_i);
        slot_i = next_slot(slot_i);
        // (computing converts the next tile's V; past the range end that slot holds a repeat of the
        // last tile: converted, never read)
        const int t0 = cc.tt * kTile;
        compute(slot_c, buf, cc.n - t0, next_slot(slot_c));
        slot_c = next_slot(slot_c);
        buf ^= 1;
        const bool end_unit = cc.tt + 1 == cc.Tb;
        if (end_unit || cc.pos + 1 == hi) {
            finalize(cc, seg, seg_start == 0 && end_unit);
            stores_pending = true;
        }
        if (!step(cc)) break;
        if (cc.tt == 0) {  // a new unit group begins
            seg++;
            seg_start = 0;
            load_q(cc.b, cc.grp);
            reset_state();
        }
    }
    // no copy may still be landing in LDS when the workgroup retires
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// ---------------------------------------------------------------- host-side dispatch
template <int KVT, int WPG, int QT, int SCALE>
static hipError_t launch_w(const Params &p, hipStream_t stream) {
    // Ring slots (tiles in flight per workgroup: up to NSLOT-1).  E4M3: 6 (5 with per-token scales,
    // 4 for 2-wave workgroups); ring + V staging (16 KB) fit two 4-wave workgroups, or three 2-wave
    // ones, in one CU's 160 KB of LDS.  INT8: 5, with its K staging (16 KB more) two workgroups
    // of either size.  16-bit KV: slots of 16 KB, four of them and the staging fill 80 KB, two
    // workgroups per CU.
    constexpr int NSLOT = (KVT == KV_I8 || KVT == KV_F16 || KVT == KV_BF16) ? (KVT == KV_I8 ? 5 : 4)
                                                                           : (WPG == 2 ? 4 : (SCALE == SC_TOKEN_HEAD ? 5 : 6));
    dim3 grid(p.nparts), block(64 * WPG);
    if (p.nq > 1) {  // a window of query tokens: per-column limits
        if (p.block_table && p.block_size == 16)
            hipLaunchKernelGGL((wide_partition_kernel<KVT, WPG, NSLOT, QT, SCALE, true, true, true>), grid, block, 0, stream, p);
        else if (p.block_table)
            hipLaunchKernelGGL((wide_partition_kernel<KVT, WPG, NSLOT, QT, SCALE, true, false, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((wide_partition_kernel<KVT, WPG, NSLOT, QT, SCALE, false, false, true>), grid, block, 0, stream, p);
    } else if (p.block_table && p.block_size == 16) {  // 32-token tiles span two blocks
        hipLaunchKernelGGL((wide_partition_kernel<KVT, WPG, NSLOT, QT, SCALE, true, true, false>), grid, block, 0, stream, p);
    } else if (p.block_table) {
        hipLaunchKernelGGL((wide_partition_kernel<KVT, WPG, NSLOT, QT, SCALE, true, false, false>), grid, block, 0, stream, p);
    } else {
        hipLaunchKernelGGL((wide_partition_kernel<KVT, WPG, NSLOT, QT, SCALE, false, false, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

template <int KVT, int WPG>
static hipError_t launch_wq(const Params &p, int qt, int sc, hipStream_t stream) {
    if (qt == KV_BF16) {
        if (sc == SC_TENSOR) return launch_w<KVT, WPG, KV_BF16, SC_TENSOR>(p, stream);
        return launch_w<KVT, WPG, KV_BF16, SC_TOKEN_HEAD>(p, stream);
    }
    if (sc == SC_TENSOR) return launch_w<KVT, WPG, KV_F16, SC_TENSOR>(p, stream);
    return launch_w<KVT, WPG, KV_F16, SC_TOKEN_HEAD>(p, stream);
}

hipError_t launch_wide_partition(const Params &p, int kv_dtype, int q_dtype, int scale_mode, hipStream_t stream) {
    if (p.d != 128 || p.hb != kWideHeadBlock || (p.wpg != 2 && p.wpg != 4) || p.nhb % p.wpg)
        return hipErrorInvalidValue;
    if (kv_dtype == KV_F16 || kv_dtype == KV_BF16) {
        // 16-bit KV: q of the same type, no scales, four head blocks per workgroup
        if (q_dtype != kv_dtype || scale_mode != SC_NONE || p.wpg != 4) return hipErrorInvalidValue;
        if (kv_dtype == KV_F16) return launch_w<KV_F16, 4, KV_F16, SC_NONE>(p, stream);
        return launch_w<KV_BF16, 4, KV_BF16, SC_NONE>(p, stream);
    }
    if (kv_dtype != KV_FP8 && kv_dtype != KV_I8) return hipErrorInvalidValue;
    if (kv_dtype == KV_I8) {
        if (p.wpg == 4) return launch_wq<KV_I8, 4>(p, q_dtype, scale_mode, stream);
        return launch_wq<KV_I8, 2>(p, q_dtype, scale_mode, stream);
    }
    if (p.wpg == 4) return launch_wq<KV_FP8, 4>(p, q_dtype, scale_mode, stream);
    return launch_wq<KV_FP8, 2>(p, q_dtype, scale_mode, stream);
}

}  // namespace fd
