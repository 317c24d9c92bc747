// Host-side launchers of the device kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "decode_core.h"
#include "prefill_core.h"

namespace attn {

// Varlen prefill over contiguous K/V. Grid: (head groups, sequences, query tiles), query tiles
// walked heaviest (last) first.
hipError_t launch_prefill(const PrefillParams& p, int head_dim, int max_seqlen, hipStream_t stream);

// Split-KV paged decode, one launch (grid: partitions x kv heads x requests); the last partition
// of each (request, kv head) to finish merges the partitions. rows_max = rows per
// (request, kv head) sizing the LDS combine buffer (<= 16).
hipError_t launch_decode(const PagedParams& p, int head_dim, int kv_type, int rows_max, hipStream_t stream);

// Number of CUs of the current device (cached per device).
int device_cu_count();

}  // namespace attn
