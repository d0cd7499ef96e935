// fd_device.h -- gfx950 device helpers shared by the flash-decoding kernels: vector types,
// MFMA wrappers, E4M3 conversion, wave-uniform loads, output stores and the balanced split of a
// step's KV tiles over partition workgroups.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_internal.h"

namespace fd {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(16))) int i32x16_t;
typedef __attribute__((ext_vector_type(2))) short i16x2_t;

enum { KV_F16 = 1, KV_BF16 = 2, KV_FP8 = 3, KV_I8 = 4 };
enum { SC_NONE = 0, SC_TENSOR = 1, SC_TOKEN_HEAD = 2 };

constexpr float kLn2 = 0.69314718055994530942f;

// The running max m that the accumulator is scaled to moves only when a tile's max exceeds it
// by more than this (log2 units): weights 2^(s - m) then stay <= 2^8, exact to represent in
// fp32 and f16, and acc / l is unchanged (both carry the same reference m), while the rescale
// of the accumulator is skipped on most tiles.
constexpr float kRescaleSlack = 8.0f;
// Largest finite float: m = max(m_run, -kMaxFloat) keeps exp2 of (score - m) at 0, not NaN, while a
// column has seen no token (m_run = -inf).
constexpr float kMaxFloat = 3.40282347e38f;
// Smallest normal float: the floor of a 16-bit partial row's scale (its reciprocal is finite).
constexpr float kMinNormal = 1.17549435e-38f;

// Per-(token, head) v scales enter p.V through the f16 P operand, whose range (normal numbers
// 2^-14 .. 65504) is narrower than that of the scales.  A wave therefore keeps a power-of-two
// reference 2^ev near the largest |v scale| it has seen and forms 2^(s - m - ev) * v_scale, the
// weight times v_scale / 2^ev; the accumulator holds the sum divided by 2^ev, which is multiplied
// back when the segment ends.  ev moves (an exact power-of-two rescale of the accumulator, merged
// with the running-max rescale) when a tile's largest |v scale| leaves
// [2^(ev - kVrefLow), 2^(ev + kVrefHigh)]: the f16 operand then stays below
// 2^(kRescaleSlack + kVrefHigh) = 2^14, and the largest-scale tokens of a tile with weights down to
// 2^-5 stay f16-normal, whatever the magnitude of the data.
constexpr int kVrefHigh = 6;
constexpr int kVrefLow = 8;
constexpr int kVrefLimit = 100;  // |ev| bound: 2^(s - m - ev) stays finite

// e with x <= 2^e < 2x for a positive normal float x, clamped to [-kVrefLimit, kVrefLimit]
// (denormals give the lower bound; inf and NaN the upper one).
__device__ __forceinline__ int exp2_ceil(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x) & 0x7FFFFFFFu;
    const int e = (int)((u + 0x007FFFFFu) >> 23) - 127;
    return min(max(e, -kVrefLimit), kVrefLimit);
}
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// ---------------------------------------------------------------- small helpers
template <int QT>
__device__ __forceinline__ f32x4_t mfma_qk(u32x4_t a, u32x4_t b, f32x4_t c) {
    if constexpr (QT == KV_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_f16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two E4M3 bytes (bytes 0,1 or 2,3 of w) -> two values of type QT packed in one dword.
// Exact: every E4M3 value is representable in f16 and bf16.
template <int QT, bool HI>
__device__ __forceinline__ uint32_t cvt_fp8x2(uint32_t w) {
    if constexpr (QT == KV_BF16)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// Two int8 codes -> two f16 values (exact), for codes placed in bytes 0 and 2 of x with bytes 1
// and 3 zero: each 16-bit half 0x00bb becomes 0x64 | (bb ^ 0x80), i.e. the f16 value 1024 +
// (code + 128), and subtracting 1152 leaves the code.
__device__ __forceinline__ uint32_t i8x2_to_f16x2(uint32_t x) {
    const f16x2_t biased = __builtin_bit_cast(f16x2_t, x ^ 0x64806480u);
    return __builtin_bit_cast(uint32_t, biased - f16x2_t{(_Float16)1152.0f, (_Float16)1152.0f});
}

// bf16 pair times 2^e -> f16 pair, for a bf16 q against INT8 KV.  The caller picks e so that the
// largest |q| of the column lands in [2^14, 2^15): every value within 2^28 of it is then an f16
// normal number and converts exactly (bf16's 8-bit significand fits f16's 11 bits); smaller ones
// keep an absolute error below 2^-25 of the largest.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2_scaled(uint32_t w, int e) {
    const float lo = __builtin_amdgcn_ldexpf(__builtin_bit_cast(float, w << 16), e);
    const float hi = __builtin_amdgcn_ldexpf(__builtin_bit_cast(float, w & 0xFFFF0000u), e);
    f16x2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even
    return u >> 16;
}

// bf16 pair, a in the low half: round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// A pair of p.V weights as two bf16 terms: hi = bf16(p), lo = bf16(p - hi) (p - hi is exact in
// fp32), so hi + lo carries p to ~2^-16 against a bf16 V operand.
__device__ __forceinline__ void split_bf16_pair(float p0, float p1, uint32_t &hi, uint32_t &lo) {
    hi = pack_bf16(p0, p1);
    const float r0 = p0 - __builtin_bit_cast(float, hi << 16);
    const float r1 = p1 - __builtin_bit_cast(float, hi & 0xFFFF0000u);
    lo = pack_bf16(r0, r1);
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    f16x2_t v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Scalar load of a wave-uniform int32 the kernel never writes (seq_len, block table, kv start):
// through the constant address space, so it is an s_load, independent of the vector-memory
// counter that the KV prefetch uses.
__device__ __forceinline__ int32_t ld_uniform(const int32_t *ptr, size_t i) {
    return *((const __attribute__((address_space(4))) int32_t *)ptr + i);
}

// Wave-uniform copies (the value is the same in every lane; this keeps it in scalar registers
// so that loads addressed by it are scalar loads, counted apart from the KV vector loads).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// 32x32x16 MFMA (one wave): A = 32 rows x 16 k, B = 16 k x 32 columns, C 32 x 32.
// Lane l holds A[l % 32][8*(l/32) + 0..7] and B[8*(l/32) + 0..7][l % 32]; C register r of lane l
// is C[8*(r/4) + 4*(l/32) + r%4][l % 32].
template <int QT>
__device__ __forceinline__ f32x16_t mfma32_qk(u32x4_t a, u32x4_t b, f32x16_t c) {
    if constexpr (QT == KV_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma32_f16(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Store DT consecutive output elements starting at element `d0` of row `dst`.
template <int DT>
__device__ __forceinline__ void store_row_chunk(void *out, int out_dtype, size_t base, const float *v) {
    if (out_dtype == 0) {
        float *o = (float *)out + base;
#pragma unroll
        for (int i = 0; i < DT; i += 4) *(float4 *)(o + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
    } else if (out_dtype == 1) {
        uint32_t w[DT / 2];
#pragma unroll
        for (int i = 0; i < DT / 2; i++) w[i] = pack_f16(v[2 * i], v[2 * i + 1]);
        uint16_t *o = (uint16_t *)out + base;
        if constexpr (DT == 8) *(u32x4_t *)o = u32x4_t{w[0], w[1], w[2], w[3]};
        else *(u32x2_t *)o = u32x2_t{w[0], w[1]};
    } else {
        uint32_t w[DT / 2];
#pragma unroll
        for (int i = 0; i < DT / 2; i++)
            w[i] = f32_to_bf16_bits(v[2 * i]) | (f32_to_bf16_bits(v[2 * i + 1]) << 16);
        uint16_t *o = (uint16_t *)out + base;
        if constexpr (DT == 8) *(u32x4_t *)o = u32x4_t{w[0], w[1], w[2], w[3]};
        else *(u32x2_t *)o = u32x2_t{w[0], w[1]};
    }
}

// ---------------------------------------------------------------- work split helpers
//
// Balanced split of one step's KV work.  A *unit* is (sequence b, kv head, head block): the
// G <= 16 query heads of one head block that share one kv head.  The units of a sequence are
// taken in groups of `wpg` by the `wpg` waves of one workgroup (wave i takes unit grp*wpg + i),
// so the waves of a workgroup stream the same token rows of the cache at the same time.
// Unit group (b, grp) owns T_b = ceil(seq_len[b] / 32) tiles; groups are concatenated
// sequence-major into TT tiles, and workgroup w of W takes tiles [lo_w, lo_{w+1}) with
// lo_w = w*q + min(w, r), q = TT / W, r = TT % W: every workgroup gets the same amount of KV
// (up to one tile) whatever the length mix.  A group cut by workgroup boundaries leaves one
// partial state per piece: slot 0 of a workgroup holds its first piece, slot 1 its last one.

__device__ __forceinline__ int seq_tiles(const Params &p, int b) {
    int n = p.seq_len[b];
    n = max(0, min(n, p.max_seq_len));
    return (n + kTile - 1) / kTile;
}

// Same, for a wave-uniform b (scalar load).
__device__ __forceinline__ int seq_tiles_u(const Params &p, int b) {
    int n = ld_uniform(p.seq_len, b);
    n = max(0, min(n, p.max_seq_len));
    return (n + kTile - 1) / kTile;
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

struct Split {
    int64_t q, r;
};

__device__ __forceinline__ Split make_split(int64_t TT, int64_t W) { return Split{TT / W, TT % W}; }

__device__ __forceinline__ int64_t split_lo(const Split &s, int64_t w) { return w * s.q + min(w, s.r); }

// Workgroup whose range holds tile t (0 <= t < TT).
__device__ __forceinline__ int64_t split_owner(const Split &s, int64_t t) {
    const int64_t big = s.r * (s.q + 1);
    return t < big ? t / (s.q + 1) : s.r + (t - big) / s.q;
}

// Total tiles over all sequences (one unit group each); every lane gets the same value.
__device__ __forceinline__ int64_t total_seq_tiles(const Params &p, int lane) {
    int64_t tot = 0;
    for (int b0 = 0; b0 < p.batch; b0 += 64) {
        const int b = b0 + lane;
        int t = b < p.batch ? seq_tiles(p, b) : 0;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off, 64);
        tot += t;
    }
    return tot;
}


}  // namespace fd
