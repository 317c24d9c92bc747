// Host-side launchers of the device kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "decode_core.h"
#include "prefill_core.h"

namespace attn {

// Devices the per-device caches below cover (device ids 0 .. kMaxDevices - 1).
constexpr int kMaxDevices = 64;
// Upper bound on decode partitions (it bounds the workspace: two partial slots per partition).
constexpr int kMaxSplits = 4096;
// Upper bound on requests of a paged call: the partition kernel keeps one chunk offset per
// request in LDS.
constexpr int kMaxPagedSeqs = 16384;

// The current device's id if it is in [0, kMaxDevices), else -1 (a failed query leaves no
// pending error).
int current_device_index();

template <class T>
struct ident {
  using type = T;
};

// Launch a kernel with hipLaunchKernel and return that launch's own status (so an error left
// pending by earlier, unrelated work is neither reported as this launch's nor cleared).
template <typename... KArgs>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                         typename ident<KArgs>::type... args) {
  void* ptrs[] = {static_cast<void*>(&args)..., nullptr};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds, stream);
}

// Raise the dynamic-LDS limit of `kernel` to `bytes` (a constant per kernel: the most any of its
// launches takes) once per device; `done` holds one flag per device. Setting it twice is harmless,
// so concurrent first calls need no lock.
hipError_t ensure_dynamic_lds(const void* kernel, std::atomic<bool>* done, int bytes);

// Varlen prefill over contiguous K/V. Grid: (head groups, sequences, query tiles), query tiles
// walked heaviest (last) first.
hipError_t launch_prefill(const PrefillParams& p, int head_dim, int max_seqlen, hipStream_t stream);

// FP8 varlen prefill over contiguous e4m3fn Q/K/V with per-head scales, head_dim 128 (the
// parameter block is defined in prefill_fp8.h). Grid as launch_prefill's.
struct PrefillFp8Params;
hipError_t launch_prefill_fp8(const PrefillFp8Params& p, int max_seqlen, hipStream_t stream);

// Split-KV paged decode: p.num_wg partition workgroups, each taking an equal share of the batch's
// (request, kv head, key chunk) work, then the LSE merge (grid: rows x kv heads x requests).
// rows_max = rows per (request, kv head) (<= 16); it sizes the LDS combine buffer and the merge
// grid.
hipError_t launch_decode(const PagedParams& p, int head_dim, int kv_type, int rows_max, hipStream_t stream);

// The LSE merge alone (the second launch of a paged decode / mixed call); nu = the partition
// kernel's sub-tiles per chunk (chunk = 16 * nu keys). ensure_merge_attrs raises the merge
// kernel's LDS limit on the current device without launching it.
hipError_t launch_decode_merge(const PagedParams& p, int head_dim, int nu, int rows_max, hipStream_t stream);
hipError_t ensure_merge_attrs(int head_dim, int nu);

// Mixed varlen batch over a paged cache: one launch holding the decode path's p.num_wg shares
// and the prefill q-tiles, then the merge.
// Largest num_seqs a mixed call of this head_dim supports (its LDS holds per-request offsets).
int mixed_max_seqs(int head_dim);
hipError_t launch_mixed(const PrefillParams& pp, const PagedParams& dp, int head_dim, int kv_type, int total_q,
                        hipStream_t stream);

// Paged KV-cache append: new tokens' K rows / V columns into their cache slots (fp8 caches get
// the values quantised with the per-head scales).
struct AppendParams {
  const bf16* k_new;           // [total_new, Hkv, D]
  const bf16* v_new;           // [total_new, Hkv, D]
  void* k_cache;               // [num_blocks, Hkv, bs, D] bf16 or e4m3fn codes
  void* v_cache;               // [num_blocks, Hkv, D, bs]
  const float* k_scale;        // [Hkv] (fp8) or nullptr
  const float* v_scale;        // [Hkv] (fp8) or nullptr
  const int32_t* block_table;  // [B, max_blocks]
  const int32_t* cu_seqlens_new;  // [B + 1]
  const int32_t* seq_lens_k;   // [B] cached tokens after the append
  int num_seqs, total_new, Hkv, bs, max_blocks;
};
hipError_t launch_append(const AppendParams& p, int head_dim, int kv_type, hipStream_t stream);

// Keys per chunk of the decode variant, and its resident workgroups per compute unit.
int decode_chunk_tokens(int head_dim, int kv_type);
int decode_wgs_per_cu(int head_dim, int kv_type);

// Number of CUs of the current device (cached per device).
int device_cu_count();

}  // namespace attn
