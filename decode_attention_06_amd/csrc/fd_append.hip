// fd_append.hip -- gfx950 kernel that writes the current decode token's K and V rows of every
// sequence into its cache row: the step before the attention scan.
//
// Pages: "第 15 章 · GPU Profiling 与 LLM 推理优化实战" -- section 15.9 (paged cache writes; its
// exercises add a single-token decode append), 15.11 (quantised KV with per-token k/v scales)
// and 15.18 (row-wise absmax -> scale -> quantise); the row address is the 15.26 paged form.
//
// One wave per (sequence, kv head); lane i holds elements [E*i, E*i + E) of the D-element row
// (E = D / 64), so loads and stores are coalesced.  E4M3 rows: the wave's max |x| (a butterfly)
// gives scale = amax / 448 (1 for an all-zero row), q = x / scale in IEEE fp32 (correctly
// rounded division), clamped to +-448, then the hardware convert rounds to the nearest E4M3
// value (ties to even).  INT8 rows: scale = amax / 127, the code is x / scale rounded to the
// nearest integer (ties to even), clamped to +-127.  f16 / bf16 caches take the value rounded
// to nearest even.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_device.h"

namespace fd {

typedef __attribute__((ext_vector_type(2))) short v2i16_t;

// Two fp32 values -> two E4M3 codes (bytes 0 and 1), round to nearest even; |q| <= 448 here.
__device__ __forceinline__ uint32_t e4m3_rne_x2(float q0, float q1) {
    const v2i16_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2i16_t{0, 0}, q0, q1, 1.0f, false);
    return __builtin_bit_cast(uint32_t, r) & 0xFFFFu;
}

// Clamp to the E4M3 range by comparisons (a NaN passes through unchanged).
__device__ __forceinline__ float clamp448(float q) { return q > 448.0f ? 448.0f : (q < -448.0f ? -448.0f : q); }
// Clamp to the symmetric INT8 range [-127, 127].
__device__ __forceinline__ float clamp127(float q) { return q > 127.0f ? 127.0f : (q < -127.0f ? -127.0f : q); }

template <int NT>
__device__ __forceinline__ float load_new(const void *src, size_t i) {
    if constexpr (NT == 0) return ((const float *)src)[i];
    else if constexpr (NT == 1) return (float)((const _Float16 *)src)[i];
    else return __builtin_bit_cast(float, (uint32_t)((const uint16_t *)src)[i] << 16);
}

template <int D, int NT, int KVT, int SCALE, bool PAGED>
__global__ __launch_bounds__(64) void append_kernel(AppendParams a) {
    constexpr int E = D / 64;
    const int b = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv, lane = threadIdx.x;
    const int t = a.pos[b];
    if (t < 0) return;  // sequence skipped (wave-uniform)
    int64_t row;
    if constexpr (PAGED)
        row = (int64_t)a.block_table[(size_t)b * a.max_blocks + t / a.block_size] * a.block_size + t % a.block_size;
    else
        row = (int64_t)a.kv_start[b] + t;
    const size_t src0 = ((size_t)b * a.hkv + g) * D + E * lane;
    const size_t dst0 = ((size_t)row * a.hkv + g) * D + E * lane;
#pragma unroll
    for (int which = 0; which < 2; which++) {
        const void *src = which ? a.v_new : a.k_new;
        void *cache = which ? a.v_cache : a.k_cache;
        float x[E];
#pragma unroll
        for (int i = 0; i < E; i++) x[i] = load_new<NT>(src, src0 + i);
        if constexpr (KVT == KV_FP8 || KVT == KV_I8) {
            constexpr float qmax = (KVT == KV_FP8) ? 448.0f : 127.0f;
            float *sc = which ? a.v_scale : a.k_scale;
            float scale;
            if constexpr (SCALE == SC_TOKEN_HEAD) {
                float amax = fabsf(x[0]);
#pragma unroll
                for (int i = 1; i < E; i++) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, shfl_xor_f(amax, off));
                scale = amax > 0.0f ? amax / qmax : 1.0f;
                if (lane == 0) sc[row * a.hkv + g] = scale;
            } else {
                scale = sc[0];
            }
            uint8_t *dst = (uint8_t *)cache + dst0;
            uint32_t code;
            if constexpr (KVT == KV_FP8) {
                code = e4m3_rne_x2(clamp448(x[0] / scale), E == 2 ? clamp448(x[1] / scale) : 0.0f);
            } else {
                code = (uint32_t)(uint8_t)(int8_t)(int)clamp127(__builtin_rintf(x[0] / scale));
                if constexpr (E == 2) code |= (uint32_t)(uint8_t)(int8_t)(int)clamp127(__builtin_rintf(x[1] / scale)) << 8;
            }
            if constexpr (E == 2) *(uint16_t *)dst = (uint16_t)code;
            else dst[0] = (uint8_t)code;
        } else {
            uint16_t h[E];
#pragma unroll
            for (int i = 0; i < E; i++) {
                if constexpr (KVT == KV_F16) h[i] = __builtin_bit_cast(uint16_t, (_Float16)x[i]);
                else h[i] = (uint16_t)f32_to_bf16_bits(x[i]);
            }
            uint16_t *dst = (uint16_t *)cache + dst0;
            if constexpr (E == 2) *(uint32_t *)dst = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
            else dst[0] = h[0];
        }
    }
}

// The same conversion the append kernel applies to an E4M3 row, element by element
// (diagnostic: lets the tests compare it with the format definition).
__global__ void fp8_encode_kernel(const float *in, uint8_t *out, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    out[i] = (uint8_t)e4m3_rne_x2(clamp448(in[i]), 0.0f);
}

// ---------------------------------------------------------------- host-side dispatch
template <int D, int NT, int KVT, int SCALE>
static hipError_t launch_a4(const AppendParams &a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.batch * a.hkv)), block(64);
    if (a.block_table) hipLaunchKernelGGL((append_kernel<D, NT, KVT, SCALE, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((append_kernel<D, NT, KVT, SCALE, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <int D, int NT>
static hipError_t launch_a3(const AppendParams &a, int kv, int sc, hipStream_t stream) {
    if (kv == KV_F16) return launch_a4<D, NT, KV_F16, SC_NONE>(a, stream);
    if (kv == KV_BF16) return launch_a4<D, NT, KV_BF16, SC_NONE>(a, stream);
    if (kv == KV_I8) {
        if (sc == SC_TENSOR) return launch_a4<D, NT, KV_I8, SC_TENSOR>(a, stream);
        return launch_a4<D, NT, KV_I8, SC_TOKEN_HEAD>(a, stream);
    }
    if (sc == SC_TENSOR) return launch_a4<D, NT, KV_FP8, SC_TENSOR>(a, stream);
    return launch_a4<D, NT, KV_FP8, SC_TOKEN_HEAD>(a, stream);
}

template <int D>
static hipError_t launch_a2(const AppendParams &a, int nt, int kv, int sc, hipStream_t stream) {
    if (nt == 0) return launch_a3<D, 0>(a, kv, sc, stream);
    if (nt == 1) return launch_a3<D, 1>(a, kv, sc, stream);
    return launch_a3<D, 2>(a, kv, sc, stream);
}

hipError_t launch_append(const AppendParams &a, int new_dtype, int kv_dtype, int scale_mode, hipStream_t stream) {
    if (a.batch <= 0 || a.hkv <= 0) return hipSuccess;
    if (a.d == 128) return launch_a2<128>(a, new_dtype, kv_dtype, scale_mode, stream);
    return launch_a2<64>(a, new_dtype, kv_dtype, scale_mode, stream);
}

hipError_t launch_fp8_encode(const float *in, uint8_t *out, int n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fp8_encode_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, in, out, n);
    return hipGetLastError();
}

}  // namespace fd
