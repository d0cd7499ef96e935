// fd_check.hip -- debug validation of the device-side contract of a decode step: the values a
// step reads from device memory to locate its KV rows (seq_len, the used block-table entries,
// kv_start) are checked against the sizes the caller states.  The step itself never checks
// them (no host synchronisation per step, "第 15 章 · GPU Profiling 与 LLM 推理优化实战" section
// 15.17); this pass is for debugging and tests.  Paged addressing as in section 15.26 of that
// page: token t of sequence b is slot t % block_size of physical block
// block_table[b * max_blocks + t / block_size]; contiguous rows start at kv_start[b]
// ("从 SGLang Kernel源码到 GPU Trace：DeepSeek V4.1 Flash-Decode", section 3.1).
//
// Three launches, none of them a memset (capture-safe): one lane initialises the result, one
// wave per sequence counts violations (reading only table entries inside the table row), and
// one lane describes the first offending sequence.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_check.h"

namespace fd {
namespace {

struct CheckArgs {
    const int32_t *seq_len, *block_table, *kv_start;
    int batch, max_seq_len, max_blocks, block_size;
    int64_t extent;   // num_blocks (paged) or rows (contiguous)
    int32_t *result;  // [0] violations, [1] first sequence (INT32_MAX: none), [2] kind, [3] value
};

// Kind of the first violation of sequence b (0: none) and the offending value; lane-parallel over
// the used table entries, the lowest offending entry wins.
__device__ void check_sequence(const CheckArgs &a, int b, int lane, int &kind, int64_t &value) {
    kind = 0;
    value = 0;
    const int n = a.seq_len[b];
    if (n < 0 || n > a.max_seq_len) {
        kind = 1;
        value = n;
        return;
    }
    if (a.block_table) {
        const int used = (n + a.block_size - 1) / a.block_size;  // <= max_blocks: max_seq_len is
        int first = INT32_MAX;                                  // bounded by the table on the host
        for (int j = lane; j < used; j += 64) {
            const int32_t e = a.block_table[(size_t)b * a.max_blocks + j];
            if (e < 0 || (int64_t)e >= a.extent) first = min(first, j);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) first = min(first, __shfl_xor(first, off, 64));
        if (first != INT32_MAX) {
            kind = 2;
            value = a.block_table[(size_t)b * a.max_blocks + first];
        }
    } else {
        const int64_t s = a.kv_start[b];
        if (s < 0 || s + n > a.extent) {
            kind = 3;
            value = s;
        }
    }
}

__global__ void check_init_kernel(int32_t *result) {
    if (threadIdx.x == 0) {
        result[0] = 0;
        result[1] = INT32_MAX;
        result[2] = 0;
        result[3] = 0;
    }
}

__global__ __launch_bounds__(64) void check_kernel(CheckArgs a) {
    const int b = blockIdx.x, lane = threadIdx.x;
    int kind;
    int64_t value;
    check_sequence(a, b, lane, kind, value);
    if (lane == 0 && kind != 0) {
        atomicAdd(&a.result[0], 1);
        atomicMin(&a.result[1], b);
    }
}

__global__ __launch_bounds__(64) void check_describe_kernel(CheckArgs a) {
    const int b = a.result[1];  // written by the previous launch on the same stream
    if (b == INT32_MAX) {
        if (threadIdx.x == 0) a.result[1] = -1;
        return;
    }
    int kind;
    int64_t value;
    check_sequence(a, b, threadIdx.x, kind, value);
    if (threadIdx.x == 0) {
        a.result[2] = kind;
        a.result[3] = (int32_t)value;
    }
}

}  // namespace

hipError_t launch_check(const int32_t *seq_len, const int32_t *block_table, int max_blocks,
                        const int32_t *kv_start, int batch, int max_seq_len, int block_size,
                        int64_t extent, int32_t *result, hipStream_t stream) {
    CheckArgs a{seq_len, block_table, kv_start, batch, max_seq_len, max_blocks, block_size, extent, result};
    hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, stream, result);
    hipLaunchKernelGGL(check_kernel, dim3(batch), dim3(64), 0, stream, a);
    hipLaunchKernelGGL(check_describe_kernel, dim3(1), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace fd
