/*
 * fd.h -- C ABI of the flash-decoding attention library for AMD MI355X (gfx950).
 *
 * One call computes one decode step of attention: a single query token per sequence against
 * that sequence's KV cache, out[b][h][:] = softmax(q[b][h] . K_b^T * softmax_scale) . V_b,
 * where K_b, V_b are the dequantised first seq_len[b] tokens of the sequence's cache and
 * q head h reads kv head h / (num_q_heads / num_kv_heads).
 *
 * Passages this interface follows (page titles; section numbers as on the pages):
 *   - "从 SGLang Kernel源码到 GPU Trace：DeepSeek V4.1 Flash-Decode", section 3.1: the decode
 *     kernel's arguments -- q, uint8 k/v caches, output, per-sequence kv start index and
 *     seq_len, max_seq_len (an upper bound used for sizing only; work follows seq_len),
 *     num_heads, head_dim, block_size (32 or 64, chosen at run time), softmax_scale, batch.
 *   - same page, sections 2.2 and 3.2: FP8 KV dequantised in the load stage of the kernel.
 *   - "SGLang Prefill 性能优化：用 GPU Trace 剖析 FlashAttention 内核瓶颈", section 2.2: the
 *     block-wise online-softmax recurrence (running max, running sum, rescaled accumulator).
 *   - "第 15 章 · GPU Profiling 与 LLM 推理优化实战", section 15.26 (paged KV: physical page
 *     = block_table[b * max_pages + logical_page], row ((page * page_size + slot) * H + h) * D),
 *     15.11 (quantised KV with per-token k/v scales), 15.12 (GQA/MQA head groups),
 *     15.13 (ragged batch: each sequence scans only its own length), 15.22 (no allocation on
 *     the hot path: caller-owned workspace), 15.17 (no host synchronisation per step).
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees, copies to the host or synchronises; it enqueues kernels on `stream`
 *     and returns.  Calls on different streams with different outputs/workspaces may overlap.
 *   - Argument errors are detected on the host, before anything is launched, and reported
 *     as an fd_status; nothing is written in that case.  Device-side contract violations
 *     (see fd_decode_attention) are not detected.
 */
#ifndef FD_H
#define FD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FD_VERSION 1

typedef enum {
    FD_OK = 0,
    FD_ERR_INVALID_ARG = 1, /* null pointer, bad count, inconsistent dtype / scale mode      */
    FD_ERR_UNSUPPORTED = 2, /* head_dim not 64/128, block_size not 16/32/64, dtype combination */
    FD_ERR_WORKSPACE = 3,   /* workspace missing, too small or not 256-byte aligned           */
    FD_ERR_LAUNCH = 4,      /* the HIP runtime refused a kernel launch                        */
    FD_ERR_CONTRACT = 5,    /* debug mode (FD_CHECK=1) found the device-side contract broken  */
    FD_ERR_SCRATCH = 6      /* fd_decode_attention_noalloc: the step's partial states need more
                               than FD_SCRATCH_BYTES                                           */
} fd_status;

/* Bytes of the static per-GPU scratch array of fd_decode_attention_noalloc (48 MiB): above every
 * default plan's workspace (at most ~35 MB for head_dim 128: the 16-head kernel's 65536 fp32
 * partial rows, or the wide-group kernel's 131072 f16 rows). */
#define FD_SCRATCH_BYTES (48u << 20)

typedef enum {
    FD_F32 = 0,      /* output only                                                       */
    FD_F16 = 1,      /* IEEE binary16                                                     */
    FD_BF16 = 2,     /* bfloat16                                                          */
    FD_FP8_E4M3 = 3, /* OCP E4M3FN bytes (KV only): bias 7, no infinities, 0x7F/0xFF = NaN */
    FD_INT8 = 4      /* two's-complement int8 codes (KV only), value = code * scale        */
} fd_dtype;

typedef enum {
    FD_SCALE_NONE = 0,           /* f16 / bf16 KV                                            */
    FD_SCALE_PER_TENSOR = 1,     /* k_scale, v_scale each point at one fp32                  */
    FD_SCALE_PER_TOKEN_HEAD = 2  /* one fp32 per (token row, kv head), laid out like the cache
                                    rows: paged [num_blocks][block_size][num_kv_heads],
                                    contiguous [rows][num_kv_heads]                           */
} fd_scale_mode;

/*
 * fd_decode_attention -- one flash-decoding step (split-KV partition + log-sum-exp combine).
 *
 * Work split: every (sequence, kv head, block of <= 16 query heads) "unit" owns
 * ceil(seq_len / 32) tiles of 32 tokens; the units' tiles are concatenated and cut into
 * `num_partitions` equal ranges, one per partition workgroup, so long and short sequences are
 * balanced without any host-side knowledge of seq_len.  A unit cut by a range boundary leaves
 * partial (max, sum, accumulator) states that the combine kernel merges in a fixed order.
 *
 *   q            [batch][num_q_heads][head_dim], q_dtype (FD_F16 or FD_BF16), contiguous.
 *   k_cache,     paged mode:      [num_blocks][block_size][num_kv_heads][head_dim]
 *   v_cache      contiguous mode: [rows][num_kv_heads][head_dim]
 *                element type kv_dtype.  With f16/bf16 KV, q_dtype must equal kv_dtype.
 *                Each (row, kv head) vector must start 16-byte aligned (true for the layouts
 *                above when the base pointers are 16-byte aligned).
 *   block_table  [batch][max_blocks_per_seq] int32 physical block ids (paged mode), or NULL.
 *   kv_start     [batch] int32 first row of each sequence (contiguous mode), or NULL.
 *                Exactly one of block_table / kv_start must be given.
 *   seq_len      [batch] int32, 0 <= seq_len[b] <= max_seq_len (device memory).
 *   max_seq_len  host-side upper bound of seq_len (<= 2^24); sizes the grid and the workspace
 *                only.
 *                Paged mode needs max_seq_len <= max_blocks_per_seq * block_size.
 *   block_size   16, 32 or 64 in paged mode (16: the 15.9 page size; a 32-token kernel tile then
 *                spans two blocks); ignored (pass 0) in contiguous mode.
 *   scale_mode   FD_SCALE_NONE for f16/bf16 KV; PER_TENSOR or PER_TOKEN_HEAD for FP8 / INT8
 *                KV (15.11: quantised KV, per-token k/v scales).
 *   k_scale,     fp32 dequantisation scales (value = decode(byte) * scale), NULL when none.
 *   v_scale      Per tensor: [1]; per token and kv head: one per cache row and kv head, in the
 *                cache's row order.  Any finite values, zero and negative included.
 *   softmax_scale  multiplies q . k (natural-exp softmax); usually 1/sqrt(head_dim).  Any finite
 *                value (zero and negative included); NaN or infinity is FD_ERR_INVALID_ARG.
 *   out          [batch][num_q_heads][head_dim] in out_dtype (FD_F32, FD_F16 or FD_BF16).
 *   lse          optional [batch][num_q_heads] fp32 natural-log sum of exp(scores); NULL = skip.
 *                An empty sequence (seq_len 0) yields out = 0 and lse = -inf.
 *   workspace    device scratch of at least fd_workspace_bytes(...) bytes, 256-byte aligned.
 *                Contents need no initialisation and are clobbered; one workspace must not be
 *                shared by calls that may overlap.
 *   num_partitions  0 = automatic (one partition workgroup per `wpg` of 2048 resident waves,
 *                8 per CU on 256 CUs, for the 16-head kernel and for the wide-group kernel that
 *                E4M3 KV with head_dim 128 and a multiple of 64 query heads per kv head uses);
 *                > 0 forces that many (testing and tuning).  Capped by the number of tiles the
 *                sizes allow.
 *   stream       HIP stream to enqueue on (0 = null stream).
 *
 * Device-side contract (not checked by the step; violating it is undefined; fd_check_inputs
 * validates it for debugging): seq_len[b] <= max_seq_len, block_table entries for logical
 * blocks < ceil(seq_len[b] / block_size) are valid block ids, kv_start[b] + seq_len[b] rows
 * exist.
 *
 * Debug mode: with the environment variable FD_CHECK=1 (read on every call), the call first runs
 * the fd_check_inputs pass on `stream` (its result in the last 256 bytes of the workspace, which
 * fd_workspace_bytes includes), synchronises the stream and, if the contract is broken, returns
 * FD_ERR_CONTRACT without launching the step.  The cache's block count is not an argument here,
 * so table entries are checked for >= 0 only (contiguous mode: kv_start >= 0).  Synchronising,
 * so not for graph capture; off by default.  The kernels read only those entries and rows, so
 * unused table entries and unused slots of a last block may hold anything.
 *
 * Returns FD_OK or an fd_status.
 */
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
                        int num_partitions, hipStream_t stream);

/*
 * fd_workspace_bytes -- workspace size fd_decode_attention needs for these sizes (partial
 * states: 2 slots x 16 (wide-group kernel: 32) heads per partition and unit of a group, each
 * max and sum (2 fp32), a row scale (fp32) and the accumulator row: head_dim fp32 for f16 / bf16
 * KV, head_dim f16 of value / row scale for E4M3 / INT8 KV; plus 256 bytes for debug mode).
 * The same arguments must be passed to fd_decode_attention.  Returns (size_t)-1 for arguments
 * fd_decode_attention would reject as invalid.
 */
size_t fd_workspace_bytes(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                          int max_seq_len, int block_size, int kv_dtype, int num_partitions);

/*
 * fd_plan_partitions -- the number of partitions (partition-kernel waves) fd_decode_attention
 * will use for these sizes, or -1 for invalid sizes.  Host-only; for tests and tuning.
 */
int fd_plan_partitions(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                       int max_seq_len, int block_size, int kv_dtype, int num_partitions);

/*
 * fd_decode_attention_mq -- the same step for a window of num_query query tokens per sequence,
 * e.g. the draft tokens a speculative-decoding verify pass checks at once ("第 15 章 · GPU
 * Profiling 与 LLM 推理优化实战", section 15.21; "从 SGLang Kernel源码到 GPU Trace：DeepSeek V4.1
 * Flash-Decode", section 2.2, tiles several query rows per block).  The window's tokens are the
 * last num_query tokens already in the cache (seq_len[b] counts them), so query row m sits at
 * position seq_len[b] - num_query + m and attends to tokens [0, seq_len[b] - num_query + m] (a
 * causal window; a row with an empty range gets out = 0, lse = -inf).  All K/V bytes of a
 * sequence are read once for the whole window: row m of every head of a kv head's group is one
 * more MFMA column of that kv head.
 *   q      [batch][num_query][num_q_heads][head_dim], q_dtype, contiguous.
 *   out    [batch][num_query][num_q_heads][head_dim] in out_dtype.
 *   lse    optional [batch][num_query][num_q_heads] fp32.
 *   num_query  1..64; 1 is exactly fd_decode_attention.  Every other argument, the workspace
 *          rule (size from fd_workspace_bytes_mq with the same num_query) and the status codes
 *          are as for fd_decode_attention.  Windows always take the 16-column kernel.
 */
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
                           int num_partitions, hipStream_t stream);

/*
 * fd_decode_attention_noalloc -- fd_decode_attention_mq without a workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The partial states go to a static array of FD_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends; its device address is looked up
 * once per device on the first call there (hipGetSymbolAddress), and no call allocates or frees
 * anything.  The caller still passes q, the caches, out and lse.  Arguments, results and status
 * codes are those of fd_decode_attention_mq (num_query = 1: fd_decode_attention), plus
 * FD_ERR_SCRATCH, before anything is launched, when the step would need more than
 * FD_SCRATCH_BYTES (fd_workspace_bytes_mq tells; every default plan fits; a forced
 * num_partitions may not).  Nothing in the array needs to start at zero.  All calls on one GPU
 * share its array: calls that may overlap on one GPU (different streams without ordering) race
 * and must not be made; calls on one stream are ordered and safe.  The device is the stream's
 * (the current device for the null stream).
 */
int fd_decode_attention_noalloc(const void *q, int num_query, const void *k_cache, const void *v_cache,
                                const int32_t *block_table, int max_blocks_per_seq,
                                const int32_t *kv_start, const int32_t *seq_len,
                                int batch, int max_seq_len,
                                int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                int kv_dtype, int q_dtype, int scale_mode,
                                const float *k_scale, const float *v_scale,
                                float softmax_scale,
                                void *out, int out_dtype, float *lse,
                                int num_partitions, hipStream_t stream);

/* fd_workspace_bytes_mq / fd_plan_partitions_mq -- fd_workspace_bytes / fd_plan_partitions for a
 * window of num_query query tokens ((size_t)-1 / -1 also when num_query is outside 1..64). */
size_t fd_workspace_bytes_mq(int batch, int num_query, int num_q_heads, int num_kv_heads, int head_dim,
                             int max_seq_len, int block_size, int kv_dtype, int num_partitions);
int fd_plan_partitions_mq(int batch, int num_query, int num_q_heads, int num_kv_heads, int head_dim,
                          int max_seq_len, int block_size, int kv_dtype, int num_partitions);

/*
 * fd_fp8_e4m3_decode -- diagnostic: decodes n E4M3 bytes with the exact hardware conversions the
 * attention kernels use and writes out[2*i] = value via the f16 path, out[2*i+1] = value via the
 * bf16 path (both fp32, [2*n]).  Format: OCP 8-bit floating point, E4M3 (as for fd_dtype).
 * Device pointers; asynchronous on `stream`.  Returns FD_OK, FD_ERR_INVALID_ARG or FD_ERR_LAUNCH.
 */
int fd_fp8_e4m3_decode(const uint8_t *in, float *out, int n, hipStream_t stream);

/*
 * fd_kv_append -- writes the current decode token's K and V rows of every sequence into its
 * cache row, the step before the attention scan ("第 15 章 · GPU Profiling 与 LLM 推理优化实战",
 * section 15.9: paged cache writes and the single-token decode append; 15.11: per-token k/v
 * scales; 15.18: row-wise absmax -> scale -> quantise).  All pointers are device pointers owned
 * by the caller; nothing is allocated; asynchronous on `stream`.
 *   k_new, v_new  [batch][num_kv_heads][head_dim] in new_dtype (FD_F32, FD_F16 or FD_BF16).
 *   k_cache, v_cache, block_table / kv_start, max_blocks_per_seq, block_size, kv_dtype,
 *                scale_mode   as for fd_decode_attention (same layouts, same codes).
 *   pos          [batch] int32: the token index each sequence's new row is written at (its length
 *                before this step); a negative value leaves that sequence untouched.  The row is
 *                block_table[b][pos / block_size] * block_size + pos % block_size (paged) or
 *                kv_start[b] + pos (contiguous).
 *   k_scale, v_scale  E4M3 / INT8 only.  FD_SCALE_PER_TOKEN_HEAD: written, per (row, kv head),
 *                as amax |row| / QMAX in fp32 (1 for an all-zero row; QMAX = 448 for E4M3, 127
 *                for INT8), and each value is stored as the code nearest to x / scale (fp32
 *                quotient, ties to even).  FD_SCALE_PER_TENSOR: the given k_scale[0] /
 *                v_scale[0] are used (not written); x / scale saturates at +-QMAX.  f16 / bf16
 *                caches (scale_mode FD_SCALE_NONE) store x rounded to nearest even.
 * Device-side contract (not checked): the table entry of block pos / block_size is a valid block
 * id and pos < max_blocks_per_seq * block_size (paged), the row exists (contiguous); inputs are
 * finite.  Host-checked errors as for fd_decode_attention: FD_ERR_INVALID_ARG (null pointers,
 * batch or heads <= 0, both or neither of block_table / kv_start, a dtype or scale_mode not
 * allowed), FD_ERR_UNSUPPORTED (head_dim not 64 / 128, block_size not 16 / 32 / 64), FD_ERR_LAUNCH.
 */
int fd_kv_append(const void *k_new, const void *v_new, int new_dtype, void *k_cache, void *v_cache,
                 const int32_t *block_table, int max_blocks_per_seq, const int32_t *kv_start,
                 const int32_t *pos, int batch, int num_kv_heads, int head_dim, int block_size,
                 int kv_dtype, int scale_mode, float *k_scale, float *v_scale, hipStream_t stream);

/*
 * fd_fp8_e4m3_encode -- diagnostic: out[i] = the E4M3 code fd_kv_append stores for the
 * quotient in[i] (clamped to +-448, nearest E4M3 value, ties to even), n values, device
 * pointers, asynchronous on `stream`.  Returns FD_OK, FD_ERR_INVALID_ARG or FD_ERR_LAUNCH.
 */
int fd_fp8_e4m3_encode(const float *in, uint8_t *out, int n, hipStream_t stream);

/*
 * fd_set_profile_events -- diagnostic timing hook.  While set (non-NULL), every later
 * fd_decode_attention call made by the calling thread records `partition_begin` right before
 * and `partition_end` right after its split-KV partition kernel, on that call's stream, so
 * hipEventElapsedTime gives that kernel's duration.  Pass NULL, NULL to clear.  The events are
 * owned by the caller.  Thread-local; returns FD_OK.
 */
int fd_set_profile_events(hipEvent_t partition_begin, hipEvent_t partition_end);

/*
 * fd_hbm_read_probe -- diagnostic: reads `bytes` (a multiple of 16) from the device buffer `buf`
 * (16-byte aligned) with coalesced 128-bit loads, `blocks` workgroups of 256 lanes, and writes one
 * XOR fold per lane to out[blocks * 256] (uint32).  Timing it gives the read bandwidth a plain
 * stream reaches on the device, the practical ceiling for the attention kernels' KV reads.
 * `kind` picks the load design, so that the ceiling does not rest on one of them: 0 = plain
 * loads, lanes striding over the buffer, 4 per lane in flight; 1 / 2 = nontemporal loads, each
 * wave reading whole 1 KB chunks, 4 / 8 per lane in flight (`bytes` a multiple of 1024).
 * Asynchronous on `stream`.  Returns FD_OK, FD_ERR_INVALID_ARG or FD_ERR_LAUNCH.
 */
int fd_hbm_read_probe(const void *buf, size_t bytes, uint32_t *out, int blocks, int kind, hipStream_t stream);

/*
 * fd_check_inputs -- debug validation of the device-side contract of fd_decode_attention(_mq)
 * and fd_kv_append: the values a step reads from device memory to locate KV rows, checked
 * against the sizes the caller states.  The step itself never checks them: it would need a host
 * synchronisation per step (15.17); call this while debugging, or in tests.  Paged addressing
 * as in 15.26 (token t of sequence b: block_table[b * max_blocks_per_seq + t / block_size]).
 *
 *   seq_len, block_table, max_blocks_per_seq, kv_start, batch, max_seq_len, block_size
 *                exactly as for fd_decode_attention (one of block_table / kv_start is NULL).
 *   extent       number of physical blocks of the cache (paged) or rows (contiguous).
 *   result       device int32[4], written (not read first):
 *                [0] number of sequences that violate the contract,
 *                [1] the lowest such sequence, or -1 when there is none,
 *                [2] what is wrong with it: 0 nothing, 1 seq_len outside [0, max_seq_len],
 *                    2 a used block-table entry (logical block < ceil(seq_len / block_size))
 *                    outside [0, extent) -- [3] then holds the lowest such entry's value,
 *                    3 kv_start[b] < 0 or kv_start[b] + seq_len[b] > extent,
 *                [3] the offending value (seq_len, table entry or kv_start).
 * Unused table entries are not read.  Asynchronous on `stream` (three small launches, no memset,
 * no allocation); the caller synchronises before reading `result`.  Host-checked errors as for
 * fd_decode_attention (null seq_len / result, batch <= 0, max_seq_len < 0, extent < 0, both or
 * neither of block_table / kv_start, paged max_seq_len above the table, block_size not
 * 16/32/64); FD_ERR_LAUNCH if a launch fails.
 */
int fd_check_inputs(const int32_t *seq_len, const int32_t *block_table, int max_blocks_per_seq,
                    const int32_t *kv_start, int batch, int max_seq_len, int block_size,
                    int64_t extent, int32_t *result, hipStream_t stream);

/* fd_status_string -- static, NUL-terminated name of a status code (never NULL). */
const char *fd_status_string(int status);

/* fd_version -- FD_VERSION of the built library. */
int fd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FD_H */
