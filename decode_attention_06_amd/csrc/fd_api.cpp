// fd_api.cpp -- host side of the C ABI declared in include/fd.h: argument validation, the
// split plan for 256 compute units, workspace carve-up and the two kernel launches.
// Nothing here reads device memory or synchronises (no per-step host sync, as the ch.15
// profiling page's section 15.17 asks; no allocation on the hot path, section 15.22).
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "fd.h"
#include "fd_check.h"
#include "fd_internal.h"

namespace {

// Partition-kernel waves per step, all resident at once, each workgroup of `wpg` waves with an
// equal share of the step's KV tiles: 8 per CU on 256 CUs (two per SIMD; the 16-head kernel
// needs up to 256 VGPRs).  The wide-group kernel fits three per SIMD (168 VGPRs) but runs two:
// a group of 128 heads leaves one partial state of 66 KB per workgroup piece, and two
// workgroups per CU instead of three cut those bytes (written, then merged by the combine) by a
// third, for a step measured ~3 % faster on the 128K MQA workload.
constexpr long kDefaultWaves = 2048;
constexpr long kDefaultWavesWide = 2048;    // 4-wave workgroups: two per CU
constexpr long kDefaultWavesWide2 = 1536;   // 2-wave workgroups: three per CU (their LDS),
constexpr long kDefaultWavesWide2I8 = 1024; // two with INT8 KV (its K staging)
constexpr int kMaxSeqLen = 1 << 24;
constexpr int kMaxQueryWindow = 64;  // query tokens per sequence in one call

thread_local hipEvent_t t_prof_begin = nullptr, t_prof_end = nullptr;

inline long cdiv(long a, long b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
    bool wide;   // wide-group kernel (32-head blocks, LDS-shared tiles)
    bool direct; // 32-column units with K/V straight into registers, one per wave
    int hb;      // heads per head block
    int nhb;     // head blocks per kv head
    int wpg;     // waves per partition workgroup (units processed side by side)
    int groups;  // unit groups per sequence
    int nparts;  // partition workgroups
};

// Groups of 64+ query heads per kv head with E4M3 or INT8 KV and head_dim 128 take the
// wide-group kernel: 32 columns per wave, and 2 or 4 waves of one kv head share every K/V tile
// through LDS; with f16 or bf16 KV, groups of 128+ (four waves: a 16-bit tile ring fits only two
// workgroups per CU).  A window of nq query tokens multiplies the columns (each 32-column block
// lies in one window row, the group being a multiple of 32).  (The wide kernel forms in-tile row
// offsets with 24-bit multiplies: a cache row of all kv heads, hkv * 256 bytes at most, stays
// below 2^24.)
bool use_wide(int group, int hkv, int head_dim, int kv_dtype, int nq) {
    (void)nq;
    if (head_dim != 128 || hkv >= (1 << 16)) return false;
    if (kv_dtype == FD_FP8_E4M3 || kv_dtype == FD_INT8) return group % 64 == 0;
    return (kv_dtype == FD_F16 || kv_dtype == FD_BF16) && group % 128 == 0;
}

// Otherwise, E4M3 KV with head_dim 128 and a multiple of 32 MFMA columns per kv head (a window of
// 4 query tokens x 8 heads, or 32 heads) takes the 32-column kernel: each wave loads and converts
// its kv head's tiles once, where 16-column blocks would load them once per block.
bool use_direct(int cols, int hkv, int head_dim, int kv_dtype) {
    return kv_dtype == FD_FP8_E4M3 && head_dim == 128 && cols % 32 == 0 && hkv < (1 << 16);
}

bool sizes_ok(int batch, int hq, int hkv, int head_dim, int max_seq_len) {
    if (batch <= 0 || hq <= 0 || hkv <= 0 || max_seq_len < 0) return false;
    if (hq % hkv) return false;
    if (batch > 65535 || max_seq_len > kMaxSeqLen) return false;
    (void)head_dim;
    return true;
}

// Units per sequence (kv head x head block) are grouped `wpg` at a time, wpg the largest
// divisor of their count up to 8 (wide kernel: 4 or 2 head blocks of one kv head); workgroup w
// of the partition kernel takes tiles [w*q + min(w, r), ...) of the concatenation of all unit
// groups (TT tiles of 32 tokens).  The workgroup count is capped by the largest TT the sizes allow.
// A window of nq query tokens multiplies the MFMA columns of a kv head: cols = group * nq.
Plan make_plan(int batch, int nq, int hq, int hkv, int head_dim, int kv_dtype, int max_seq_len,
               int num_partitions) {
    Plan pl;
    const int group = hq / hkv, cols = group * nq;
    pl.wide = use_wide(group, hkv, head_dim, kv_dtype, nq);
    pl.direct = !pl.wide && use_direct(cols, hkv, head_dim, kv_dtype);
    if (pl.wide) {
        pl.hb = fd::kWideHeadBlock;
        pl.nhb = cols / pl.hb;  // every column of the window (cols is a multiple of 64)
        pl.wpg = pl.nhb % 4 == 0 ? 4 : 2;
        pl.groups = hkv * pl.nhb / pl.wpg;
    } else {
        pl.hb = pl.direct ? fd::kWideHeadBlock : fd::kHeadBlock;
        pl.nhb = (int)cdiv(cols, pl.hb);
        const long ups = (long)hkv * pl.nhb;
        pl.wpg = 1;
        for (int d = fd::kMaxWavesPerGroup; d >= 1; d--)
            if (ups % d == 0) { pl.wpg = d; break; }
        pl.groups = (int)(ups / pl.wpg);
    }
    const long tt_max = (long)batch * pl.groups * cdiv(max_seq_len, fd::kTile);
    long W = num_partitions > 0
                 ? num_partitions
                 : (pl.wide ? (pl.wpg == 2 ? (kv_dtype == FD_INT8 ? kDefaultWavesWide2I8 : kDefaultWavesWide2)
                                           : kDefaultWavesWide)
                            : kDefaultWaves) / pl.wpg;
    if (W > tt_max) W = tt_max;
    if (W < 1) W = 1;
    pl.nparts = (int)W;
    return pl;
}

// Workspace: [ml slots][row-scale slots][acc slots]; one slot pair per partition per unit of a
// group per head.  Acc rows are fp32 (f16 and bf16 KV) or f16 (quantised KV: half the bytes).
size_t ws_slots(const Plan &pl) { return (size_t)pl.nparts * 2 * pl.wpg * pl.hb; }

// The last kCheckBytes hold the debug-mode validator's result (FD_CHECK=1).
constexpr size_t kCheckBytes = 256;

// quantised KV keeps its partial outputs in 16 bits (the kernels take the same rule from
// Params::part16)
bool part16_of(int kv_dtype) { return kv_dtype == FD_FP8_E4M3 || kv_dtype == FD_INT8; }

size_t ws_bytes(const Plan &pl, int head_dim, int kv_dtype) {
    const size_t slots = ws_slots(pl);
    const size_t acc_elem = part16_of(kv_dtype) ? sizeof(uint16_t) : sizeof(float);
    return align256(slots * sizeof(float) * 2) + align256(slots * sizeof(float)) +
           align256(slots * head_dim * acc_elem) + kCheckBytes;
}

// ---- static scratch of the allocation-free entry point (fd_decode_attention_noalloc)
//
// One array per GPU, in the library's own code object, that holds the partial states instead of
// a caller's workspace.  In host code `scratch` names a host-side stand-in, never the device
// memory: its device address comes from hipGetSymbolAddress, once per device with that device
// current, and only that address is used.  Every call on a device shares its array.
static __device__ __align__(256) unsigned char scratch[FD_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the scratch array on the device `stream` belongs to (the current device
// for the null stream).
hipError_t scratch_address(hipStream_t stream, void **addr) {
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *a = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!a) {
        std::lock_guard<std::mutex> guard(g_scratch_mu);
        a = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!a) {
            int cur = -1;
            if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
            if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
            e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
            const hipError_t r = cur != dev ? hipSetDevice(cur) : hipSuccess;
            if (e != hipSuccess) return e;
            if (r != hipSuccess) return r;
            if (!a) return hipErrorInvalidSymbol;
            g_scratch_addr[dev].store(a, std::memory_order_release);
        }
    }
    *addr = a;
    return hipSuccess;
}

// Debug mode: FD_CHECK=1 in the environment, read on every call (no cached state).
bool debug_check_enabled() {
    const char *v = getenv("FD_CHECK");
    return v && v[0] == '1' && v[1] == 0;
}

}  // namespace

extern "C" {

int fd_version(void) { return FD_VERSION; }

int fd_check_inputs(const int32_t *seq_len, const int32_t *block_table, int max_blocks_per_seq,
                    const int32_t *kv_start, int batch, int max_seq_len, int block_size,
                    int64_t extent, int32_t *result, hipStream_t stream) {
    if (!seq_len || !result) return FD_ERR_INVALID_ARG;
    if (batch <= 0 || max_seq_len < 0 || extent < 0) return FD_ERR_INVALID_ARG;
    if ((block_table == nullptr) == (kv_start == nullptr)) return FD_ERR_INVALID_ARG;
    if (block_table) {
        if (block_size != 16 && block_size != 32 && block_size != 64) return FD_ERR_UNSUPPORTED;
        if (max_blocks_per_seq <= 0) return FD_ERR_INVALID_ARG;
        // every used entry (logical block < ceil(seq_len / block_size), seq_len <= max_seq_len)
        // then lies inside the table row
        if ((long)max_seq_len > (long)max_blocks_per_seq * block_size) return FD_ERR_INVALID_ARG;
    }
    if (fd::launch_check(seq_len, block_table, max_blocks_per_seq, kv_start, batch, max_seq_len, block_size,
                         extent, result, stream) != hipSuccess)
        return FD_ERR_LAUNCH;
    return FD_OK;
}

const char *fd_status_string(int status) {
    switch (status) {
    case FD_OK: return "FD_OK";
    case FD_ERR_INVALID_ARG: return "FD_ERR_INVALID_ARG";
    case FD_ERR_UNSUPPORTED: return "FD_ERR_UNSUPPORTED";
    case FD_ERR_WORKSPACE: return "FD_ERR_WORKSPACE";
    case FD_ERR_LAUNCH: return "FD_ERR_LAUNCH";
    case FD_ERR_CONTRACT: return "FD_ERR_CONTRACT";
    case FD_ERR_SCRATCH: return "FD_ERR_SCRATCH";
    default: return "FD_UNKNOWN_STATUS";
    }
}

int fd_plan_partitions_mq(int batch, int num_query, int num_q_heads, int num_kv_heads, int head_dim,
                          int max_seq_len, int block_size, int kv_dtype, int num_partitions) {
    (void)block_size;
    if (!sizes_ok(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len) || num_partitions < 0) return -1;
    if (num_query < 1 || num_query > kMaxQueryWindow) return -1;
    return make_plan(batch, num_query, num_q_heads, num_kv_heads, head_dim, kv_dtype, max_seq_len, num_partitions)
        .nparts;
}

int fd_plan_partitions(int batch, int num_q_heads, int num_kv_heads, int head_dim, int max_seq_len,
                       int block_size, int kv_dtype, int num_partitions) {
    return fd_plan_partitions_mq(batch, 1, num_q_heads, num_kv_heads, head_dim, max_seq_len, block_size,
                                 kv_dtype, num_partitions);
}

size_t fd_workspace_bytes_mq(int batch, int num_query, int num_q_heads, int num_kv_heads, int head_dim,
                             int max_seq_len, int block_size, int kv_dtype, int num_partitions) {
    (void)block_size;
    if (!sizes_ok(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len) || num_partitions < 0)
        return (size_t)-1;
    if (num_query < 1 || num_query > kMaxQueryWindow) return (size_t)-1;
    Plan pl = make_plan(batch, num_query, num_q_heads, num_kv_heads, head_dim, kv_dtype, max_seq_len,
                        num_partitions);
    return ws_bytes(pl, head_dim, kv_dtype);
}

size_t fd_workspace_bytes(int batch, int num_q_heads, int num_kv_heads, int head_dim, int max_seq_len,
                          int block_size, int kv_dtype, int num_partitions) {
    return fd_workspace_bytes_mq(batch, 1, num_q_heads, num_kv_heads, head_dim, max_seq_len, block_size,
                                 kv_dtype, num_partitions);
}

}  // extern "C"

namespace {

// One step.  use_scratch: the partial states go to the device's static scratch array instead of
// the caller's workspace (which is then ignored).
int step(const void *q, int num_query, const void *k_cache, const void *v_cache,
         const int32_t *block_table, int max_blocks_per_seq, const int32_t *kv_start,
         const int32_t *seq_len, int batch, int max_seq_len, int num_q_heads, int num_kv_heads,
         int head_dim, int block_size, int kv_dtype, int q_dtype, int scale_mode,
         const float *k_scale, const float *v_scale, float softmax_scale, void *out, int out_dtype,
         float *lse, void *workspace, size_t workspace_bytes, int num_partitions, hipStream_t stream,
         bool use_scratch) {
    // ---- argument validation (host only, nothing launched on failure)
    if (!q || !k_cache || !v_cache || !seq_len || !out) return FD_ERR_INVALID_ARG;
    if (!sizes_ok(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len)) return FD_ERR_INVALID_ARG;
    if (num_query < 1 || num_query > kMaxQueryWindow) return FD_ERR_INVALID_ARG;
    if (num_partitions < 0) return FD_ERR_INVALID_ARG;
    if ((block_table == nullptr) == (kv_start == nullptr)) return FD_ERR_INVALID_ARG;
    if (kv_dtype != FD_F16 && kv_dtype != FD_BF16 && kv_dtype != FD_FP8_E4M3 && kv_dtype != FD_INT8)
        return FD_ERR_INVALID_ARG;
    if (q_dtype != FD_F16 && q_dtype != FD_BF16) return FD_ERR_INVALID_ARG;
    if (out_dtype != FD_F32 && out_dtype != FD_F16 && out_dtype != FD_BF16) return FD_ERR_INVALID_ARG;
    if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return FD_ERR_INVALID_ARG;
    if (kv_dtype == FD_FP8_E4M3 || kv_dtype == FD_INT8) {
        if (scale_mode != FD_SCALE_PER_TENSOR && scale_mode != FD_SCALE_PER_TOKEN_HEAD) return FD_ERR_INVALID_ARG;
        if (!k_scale || !v_scale) return FD_ERR_INVALID_ARG;
    } else {
        if (scale_mode != FD_SCALE_NONE) return FD_ERR_INVALID_ARG;
        if (q_dtype != kv_dtype) return FD_ERR_UNSUPPORTED;
    }
    if (head_dim != 64 && head_dim != 128) return FD_ERR_UNSUPPORTED;
    if (block_table) {
        if (block_size != 16 && block_size != 32 && block_size != 64) return FD_ERR_UNSUPPORTED;
        if (max_blocks_per_seq <= 0) return FD_ERR_INVALID_ARG;
        if ((long)max_seq_len > (long)max_blocks_per_seq * block_size) return FD_ERR_INVALID_ARG;
    }
    const Plan pl = make_plan(batch, num_query, num_q_heads, num_kv_heads, head_dim, kv_dtype, max_seq_len,
                              num_partitions);
    const size_t need = ws_bytes(pl, head_dim, kv_dtype);
    if (use_scratch) {
        if (need > (size_t)FD_SCRATCH_BYTES) return FD_ERR_SCRATCH;
        if (scratch_address(stream, &workspace) != hipSuccess) return FD_ERR_LAUNCH;
        workspace_bytes = FD_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < need) return FD_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 255) return FD_ERR_WORKSPACE;

    if (debug_check_enabled()) {
        // validate the device-side contract first: result in the workspace's last 256 bytes,
        // then a synchronous read of it (debug mode only)
        int32_t *res = (int32_t *)((char *)workspace + need - kCheckBytes);
        if (fd::launch_check(seq_len, block_table, max_blocks_per_seq, kv_start, batch, max_seq_len,
                             block_table ? block_size : 0, (int64_t)INT64_MAX, res, stream) != hipSuccess)
            return FD_ERR_LAUNCH;
        int32_t host[4];
        if (hipMemcpyAsync(host, res, sizeof(host), hipMemcpyDeviceToHost, stream) != hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess)
            return FD_ERR_LAUNCH;
        if (host[0] != 0) return FD_ERR_CONTRACT;
    }

    fd::Params p;
    memset(&p, 0, sizeof(p));
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.block_table = block_table;
    p.kv_start = kv_start;
    p.seq_len = seq_len;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.out = out;
    p.lse = lse;
    p.batch = batch;
    p.hq = num_q_heads;
    p.hkv = num_kv_heads;
    p.d = head_dim;
    p.block_size = block_table ? block_size : 0;
    p.max_blocks = block_table ? max_blocks_per_seq : 0;
    p.max_seq_len = max_seq_len;
    p.group = num_q_heads / num_kv_heads;
    p.nq = num_query;
    p.cols = p.group * num_query;
    p.hb = pl.hb;
    p.nhb = pl.nhb;
    p.wpg = pl.wpg;
    p.groups = pl.groups;
    p.nparts = pl.nparts;
    p.out_dtype = out_dtype;
    // quantised KV (parity bar 5e-3 / 3e-3) keeps its partial outputs in 16 bits: f16 of the value
    // over its row's largest magnitude, relative rounding 2^-12 of that magnitude per piece
    p.part16 = part16_of(kv_dtype) ? 1 : 0;
    p.qk_scale = (float)((double)softmax_scale * 1.4426950408889634074);  // log2(e)
    {
        const size_t slots = ws_slots(pl);
        p.ws_ml = (float2 *)workspace;
        p.ws_sc = (float *)((char *)workspace + align256(slots * sizeof(float) * 2));
        p.ws_acc = (float *)((char *)p.ws_sc + align256(slots * sizeof(float)));
    }

    if (t_prof_begin) (void)hipEventRecord(t_prof_begin, stream);
    const hipError_t perr = pl.wide     ? fd::launch_wide_partition(p, kv_dtype, q_dtype, scale_mode, stream)
                            : pl.direct ? fd::launch_direct_partition(p, q_dtype, scale_mode, stream)
                                        : fd::launch_partition(p, kv_dtype, q_dtype, scale_mode, stream);
    if (perr != hipSuccess) return FD_ERR_LAUNCH;
    if (t_prof_end) (void)hipEventRecord(t_prof_end, stream);
    if (fd::launch_combine(p, stream) != hipSuccess) return FD_ERR_LAUNCH;
    return FD_OK;
}

}  // namespace

extern "C" {

int fd_decode_attention_mq(const void *q, int num_query, const void *k_cache, const void *v_cache,
                           const int32_t *block_table, int max_blocks_per_seq,
                           const int32_t *kv_start, const int32_t *seq_len,
                           int batch, int max_seq_len,
                           int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                           int kv_dtype, int q_dtype, int scale_mode,
                           const float *k_scale, const float *v_scale,
                           float softmax_scale,
                           void *out, int out_dtype, float *lse,
                           void *workspace, size_t workspace_bytes,
                           int num_partitions, hipStream_t stream) {
    return step(q, num_query, k_cache, v_cache, block_table, max_blocks_per_seq, kv_start, seq_len, batch,
                max_seq_len, num_q_heads, num_kv_heads, head_dim, block_size, kv_dtype, q_dtype, scale_mode,
                k_scale, v_scale, softmax_scale, out, out_dtype, lse, workspace, workspace_bytes,
                num_partitions, stream, false);
}

int fd_decode_attention_noalloc(const void *q, int num_query, const void *k_cache, const void *v_cache,
                                const int32_t *block_table, int max_blocks_per_seq,
                                const int32_t *kv_start, const int32_t *seq_len,
                                int batch, int max_seq_len,
                                int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                int kv_dtype, int q_dtype, int scale_mode,
                                const float *k_scale, const float *v_scale,
                                float softmax_scale,
                                void *out, int out_dtype, float *lse,
                                int num_partitions, hipStream_t stream) {
    return step(q, num_query, k_cache, v_cache, block_table, max_blocks_per_seq, kv_start, seq_len, batch,
                max_seq_len, num_q_heads, num_kv_heads, head_dim, block_size, kv_dtype, q_dtype, scale_mode,
                k_scale, v_scale, softmax_scale, out, out_dtype, lse, nullptr, 0, num_partitions, stream, true);
}

int fd_decode_attention(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *block_table, int max_blocks_per_seq,
                        const int32_t *kv_start, const int32_t *seq_len,
                        int batch, int max_seq_len,
                        int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                        int kv_dtype, int q_dtype, int scale_mode,
                        const float *k_scale, const float *v_scale,
                        float softmax_scale,
                        void *out, int out_dtype, float *lse,
                        void *workspace, size_t workspace_bytes,
                        int num_partitions, hipStream_t stream) {
    return fd_decode_attention_mq(q, 1, k_cache, v_cache, block_table, max_blocks_per_seq, kv_start, seq_len,
                                  batch, max_seq_len, num_q_heads, num_kv_heads, head_dim, block_size, kv_dtype,
                                  q_dtype, scale_mode, k_scale, v_scale, softmax_scale, out, out_dtype, lse,
                                  workspace, workspace_bytes, num_partitions, stream);
}

int fd_set_profile_events(hipEvent_t partition_begin, hipEvent_t partition_end) {
    t_prof_begin = partition_begin;
    t_prof_end = partition_end;
    return FD_OK;
}

int fd_hbm_read_probe(const void *buf, size_t bytes, uint32_t *out, int blocks, int kind, hipStream_t stream) {
    if (!buf || !out || blocks <= 0 || (bytes & 15) || ((uintptr_t)buf & 15)) return FD_ERR_INVALID_ARG;
    if (kind < 0 || kind > 2 || (kind > 0 && (bytes & 1023))) return FD_ERR_INVALID_ARG;
    return fd::launch_read_probe(buf, bytes / 16, out, blocks, kind, stream) == hipSuccess ? FD_OK : FD_ERR_LAUNCH;
}

int fd_kv_append(const void *k_new, const void *v_new, int new_dtype, void *k_cache, void *v_cache,
                 const int32_t *block_table, int max_blocks_per_seq, const int32_t *kv_start,
                 const int32_t *pos, int batch, int num_kv_heads, int head_dim, int block_size,
                 int kv_dtype, int scale_mode, float *k_scale, float *v_scale, hipStream_t stream) {
    if (!k_new || !v_new || !k_cache || !v_cache || !pos) return FD_ERR_INVALID_ARG;
    if (batch <= 0 || batch > 65535 || num_kv_heads <= 0 || num_kv_heads > 4096) return FD_ERR_INVALID_ARG;
    if ((block_table == nullptr) == (kv_start == nullptr)) return FD_ERR_INVALID_ARG;
    if (new_dtype != FD_F32 && new_dtype != FD_F16 && new_dtype != FD_BF16) return FD_ERR_INVALID_ARG;
    if (kv_dtype != FD_F16 && kv_dtype != FD_BF16 && kv_dtype != FD_FP8_E4M3 && kv_dtype != FD_INT8)
        return FD_ERR_INVALID_ARG;
    if (kv_dtype == FD_FP8_E4M3 || kv_dtype == FD_INT8) {
        if (scale_mode != FD_SCALE_PER_TENSOR && scale_mode != FD_SCALE_PER_TOKEN_HEAD) return FD_ERR_INVALID_ARG;
        if (!k_scale || !v_scale) return FD_ERR_INVALID_ARG;
    } else if (scale_mode != FD_SCALE_NONE) {
        return FD_ERR_INVALID_ARG;
    }
    if (head_dim != 64 && head_dim != 128) return FD_ERR_UNSUPPORTED;
    if (block_table) {
        if (block_size != 16 && block_size != 32 && block_size != 64) return FD_ERR_UNSUPPORTED;
        if (max_blocks_per_seq <= 0) return FD_ERR_INVALID_ARG;
    }
    fd::AppendParams a;
    memset(&a, 0, sizeof(a));
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_table = block_table;
    a.kv_start = kv_start;
    a.pos = pos;
    a.batch = batch;
    a.hkv = num_kv_heads;
    a.d = head_dim;
    a.block_size = block_table ? block_size : 0;
    a.max_blocks = block_table ? max_blocks_per_seq : 0;
    return fd::launch_append(a, new_dtype, kv_dtype, scale_mode, stream) == hipSuccess ? FD_OK : FD_ERR_LAUNCH;
}

int fd_fp8_e4m3_encode(const float *in, uint8_t *out, int n, hipStream_t stream) {
    if (n < 0 || (n > 0 && (!in || !out))) return FD_ERR_INVALID_ARG;
    return fd::launch_fp8_encode(in, out, n, stream) == hipSuccess ? FD_OK : FD_ERR_LAUNCH;
}

int fd_fp8_e4m3_decode(const uint8_t *in, float *out, int n, hipStream_t stream) {
    if (n < 0 || (n > 0 && (!in || !out))) return FD_ERR_INVALID_ARG;
    return fd::launch_fp8_decode(in, out, n, stream) == hipSuccess ? FD_OK : FD_ERR_LAUNCH;
}

}  // extern "C"
