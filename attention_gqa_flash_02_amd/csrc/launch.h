// Host-side launchers of the device kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "decode_core.h"
#include "prefill_core.h"

namespace attn {

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
// kernel's sub-tiles per chunk (chunk = 16 * nu keys).
hipError_t launch_decode_merge(const PagedParams& p, int head_dim, int nu, int rows_max, hipStream_t stream);

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
