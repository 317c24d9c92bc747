// Paged decode without a caller-provided workspace, for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops that forbid allocation): the split-KV
// partials live in a fixed device array of this library instead.
//
// The array `scratch` is a file-scope __device__ variable, so every GPU the library runs on holds
// its own copy from the moment the code object is loaded until the process ends. Host code never
// uses the array's name as an address (on the host it is only a stand-in symbol): the device
// address is looked up once per device with hipGetSymbolAddress, with that device current, and
// that pointer is what the kernels receive. Every call on one GPU shares that GPU's array, so
// calls that overlap in time on one GPU (different streams, or different host threads) race on it.
// Nothing in it needs clearing: every slot the merge kernel reads is written earlier in the same
// call (as for attn_decode_paged's workspace).
#include <mutex>

#include "../../include/attn_gqa.h"
#include "launch.h"

namespace attn {

// ATTN_DECODE_NOALLOC_MAX_BYTES (16 MiB): enough for the automatic partition count of every
// supported shape on MI355X (one partition per resident workgroup slot: 256 compute units x 1
// workgroup = 256 partitions need 256 x 2 x 16 x (256 + 1) x 4 bytes = 8.4 MB at head_dim 256, plus
// 4 bytes per request).
constexpr size_t kScratchBytes = ATTN_DECODE_NOALLOC_MAX_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once resolved

// The current device's address of `scratch`, resolved on the first call on that device.
hipError_t scratch_address(void** out) {
  const int dev = current_device_index();
  if (dev < 0) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();   // the failure just reported is this lookup's own
      return e != hipSuccess ? e : hipErrorInvalidSymbol;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace attn

using namespace attn;

extern "C" {

attn_status attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* seq_lens, float scale, void* out,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t num_splits, float* lse,
                                      int32_t kv_dtype, const float* k_scale, const float* v_scale,
                                      int32_t window, void* stream) {
  // Arguments that attn_decode_paged would reject are rejected the same way, before the size
  // check, so the two entry points report the same status for the same invalid call.
  const attn_status probe =
      attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale, out, num_seqs, num_q_heads, num_kv_heads,
                        head_dim, block_size, num_blocks, max_blocks_per_seq, num_splits, lse, nullptr, 0, kv_dtype,
                        k_scale, v_scale, window, stream);
  if (probe != ATTN_ERR_WORKSPACE) return probe;   // a validation error (no valid call passes a NULL workspace)
  const int32_t S = attn_decode_num_splits(num_seqs, num_kv_heads, head_dim, kv_dtype, block_size,
                                           max_blocks_per_seq, num_splits);
  const size_t need = attn_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, S);
  if (need > kScratchBytes) return ATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return ATTN_ERR_LAUNCH;
  return attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale, out, num_seqs, num_q_heads,
                           num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, num_splits, lse, ws,
                           kScratchBytes, kv_dtype, k_scale, v_scale, window, stream);
}

}  // extern "C"
