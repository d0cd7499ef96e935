// fd_internal.h -- parameters shared by the host launcher and the gfx950 kernels.
#pragma once
#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace fd {

// Tokens per wave tile: two 16-row MFMA blocks for q.k^T, one 32-deep MFMA step for p.V.
constexpr int kTile = 32;
// Heads per MFMA column block (a GQA group wider than this takes several head blocks): 16 for
// the 16x16x32 partition kernel, 32 for the wide-group kernel (32x32x16 MFMA, LDS-shared tiles).
constexpr int kHeadBlock = 16;
constexpr int kWideHeadBlock = 32;
// Most waves (units of one sequence) a partition workgroup runs side by side.
constexpr int kMaxWavesPerGroup = 8;
// Largest batch whose per-sequence tile prefix sums a partition workgroup keeps in LDS.
constexpr int kLdsBatch = 4096;

struct Params {
    const void *q;               // [batch][nq][hq][d]
    const void *k;
    const void *v;
    const int32_t *block_table;  // paged mode
    const int32_t *kv_start;     // contiguous mode
    const int32_t *seq_len;
    const float *k_scale;
    const float *v_scale;
    void *out;
    float *lse;
    float *ws_acc;   // [nparts][2][wpg][hb][d]  unnormalised partial outputs (fp32, or f16 when part16)
    float2 *ws_ml;   // [nparts][2][wpg][hb]     (running max in log2 units, running sum)
    float *ws_sc;    // [nparts][2][wpg][hb]     part16: the row's largest |value|, which divides it
    int part16;      // partial outputs stored as f16 of value / row max (quantised KV), else fp32
    int batch, hq, hkv, d;
    int block_size, max_blocks;
    int max_seq_len;  // host bound; seq_len values above it are clamped (never read past it)
    int group;        // hq / hkv
    int nq;           // query tokens per sequence (a window of nq rows; 1 for a plain decode step)
    int cols;         // MFMA columns per kv head: group * nq (column m * group + h: row m, head h)
    int hb;           // columns per head block (kHeadBlock or kWideHeadBlock)
    int nhb;          // head blocks per kv head: ceil(cols / hb)
    int wpg;          // waves per partition workgroup = units per unit group (divides hkv*nhb)
    int groups;       // unit groups per sequence: hkv * nhb / wpg
    int nparts;       // partition workgroups (equal shares of the step's tiles)
    int out_dtype;
    float qk_scale;   // softmax_scale * log2(e): scores are kept in log2 units
};

// KV-cache append of the current token (fd_append.hip).
struct AppendParams {
    const void *k_new;           // [batch][hkv][d], new dtype
    const void *v_new;
    void *k_cache;               // rows of [hkv][d]
    void *v_cache;
    float *k_scale;              // E4M3: [1] (per tensor, read) or [rows][hkv] (per token, written)
    float *v_scale;
    const int32_t *block_table;  // paged mode
    const int32_t *kv_start;     // contiguous mode
    const int32_t *pos;          // [batch] token index written; < 0 skips
    int batch, hkv, d, block_size, max_blocks;
};

// Host-side launchers (defined in fd_kernels.hip).  Return hipSuccess or the launch error.
hipError_t launch_partition(const Params &p, int kv_dtype, int q_dtype, int scale_mode,
                            hipStream_t stream);
hipError_t launch_combine(const Params &p, hipStream_t stream);
// Wide-group variant (defined in fd_wide.hip): E4M3 or INT8 KV, head_dim 128, hb = kWideHeadBlock,
// wpg 2 or 4 head blocks of one kv head per workgroup.
hipError_t launch_wide_partition(const Params &p, int kv_dtype, int q_dtype, int scale_mode, hipStream_t stream);
// 32-column units with K/V straight into registers (defined in fd_direct.hip): E4M3 KV, head_dim
// 128, hb = kWideHeadBlock, one unit per wave, up to kMaxWavesPerGroup units per workgroup.
hipError_t launch_direct_partition(const Params &p, int q_dtype, int scale_mode, hipStream_t stream);
hipError_t launch_fp8_decode(const uint8_t *in, float *out, int n, hipStream_t stream);
hipError_t launch_read_probe(const void *in, size_t n16, uint32_t *out, int blocks, int kind, hipStream_t stream);
// fd_append.hip: new_dtype 0 f32 / 1 f16 / 2 bf16; kv_dtype and scale_mode as the FD_ codes.
hipError_t launch_append(const AppendParams &a, int new_dtype, int kv_dtype, int scale_mode, hipStream_t stream);
hipError_t launch_fp8_encode(const float *in, uint8_t *out, int n, hipStream_t stream);

}  // namespace fd
