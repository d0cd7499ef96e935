// fd_check.h -- launcher of the debug validation pass (fd_check.hip).
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace fd {

// Enqueues the three validation launches on `stream`; result: int32[4] on the device.
hipError_t launch_check(const int32_t *seq_len, const int32_t *block_table, int max_blocks,
                        const int32_t *kv_start, int batch, int max_seq_len, int block_size,
                        int64_t extent, int32_t *result, hipStream_t stream);

}  // namespace fd
