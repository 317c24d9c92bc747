// C-ABI entry points: argument validation, partition planning and dispatch.
// Validation happens before any HIP call, so an invalid call touches nothing.
#include <atomic>
#include <climits>
#include <cmath>

#include "../../include/attn_gqa.h"
#include "launch.h"
#include "prefill_fp8.h"

namespace attn {

int current_device_index() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  return (dev >= 0 && dev < kMaxDevices) ? dev : -1;
}

hipError_t ensure_dynamic_lds(const void* kernel, std::atomic<bool>* done, int bytes) {
  const int dev = current_device_index();
  if (dev >= 0 && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  if (dev >= 0) done[dev].store(true, std::memory_order_release);
  return hipSuccess;
}

int device_cu_count() {
  static std::atomic<int> cache[kMaxDevices];
  const int dev = current_device_index();
  if (dev < 0) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

static bool supported_block_size(int bs) {
  return bs == 16 || bs == 32 || bs == 64 || bs == 128 || bs == 256;
}

static int gcd_int(int a, int b) {
  while (b) {
    int t = a % b;
    a = b;
    b = t;
  }
  return a;
}


}  // namespace attn

using namespace attn;

extern "C" {

const char* attn_status_string(attn_status status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL: a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE: inconsistent or non-positive sizes";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: head_dim, block_size or kv dtype not supported";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: workspace missing or too small";
    case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH: the HIP runtime rejected the launch";
    default: return "ATTN_ERR_UNKNOWN";
  }
}

attn_status attn_prefill_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                int32_t causal, float scale, void* out, float* lse, int32_t num_seqs,
                                int32_t total_tokens, int32_t max_seqlen, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t window, void* stream) {
  if (num_seqs <= 0 || total_tokens < 0 || max_seqlen < 0 || max_seqlen > total_tokens ||
      num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      (causal != 0 && causal != 1) || !(std::isfinite(scale) && scale >= 0.f) || window < 0)
    return ATTN_ERR_SHAPE;
  if (head_dim != 128 && head_dim != 256) return ATTN_ERR_UNSUPPORTED;
  if ((long long)total_tokens * num_q_heads * head_dim > (long long)INT_MAX * 8) return ATTN_ERR_SHAPE;
  if (total_tokens == 0 || max_seqlen == 0) return ATTN_OK;   // nothing to read or write
  if (!q || !k || !v || !cu_seqlens || !out) return ATTN_ERR_NULL;

  PrefillParams p{};
  p.q = static_cast<const bf16*>(q);
  p.k = static_cast<const bf16*>(k);
  p.v = static_cast<const bf16*>(v);
  p.cu_seqlens_q = cu_seqlens;
  p.out = static_cast<bf16*>(out);
  p.lse = lse;
  p.scale = scale;
  p.window = window;
  p.num_seqs = num_seqs;
  p.Hq = num_q_heads;
  p.Hkv = num_kv_heads;
  p.g = num_q_heads / num_kv_heads;
  p.hpw = gcd_int(p.g, 4);
  p.causal = causal;
  hipError_t e = launch_prefill(p, head_dim, max_seqlen, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status attn_prefill_varlen_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                                    const float* k_scale, const float* v_scale, const int32_t* cu_seqlens,
                                    int32_t causal, float scale, void* out, float* lse,
                                    int32_t num_seqs, int32_t total_tokens, int32_t max_seqlen,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t window,
                                    void* stream) {
  if (num_seqs <= 0 || total_tokens < 0 || max_seqlen < 0 || max_seqlen > total_tokens ||
      num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      (causal != 0 && causal != 1) || !(std::isfinite(scale) && scale >= 0.f) || window < 0)
    return ATTN_ERR_SHAPE;
  if (head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if ((long long)total_tokens * num_q_heads * head_dim > (long long)INT_MAX * 8) return ATTN_ERR_SHAPE;
  if (total_tokens == 0 || max_seqlen == 0) return ATTN_OK;   // nothing to read or write
  if (!q || !k || !v || !q_scale || !k_scale || !v_scale || !cu_seqlens || !out) return ATTN_ERR_NULL;

  PrefillFp8Params p{};
  p.q = static_cast<const uint8_t*>(q);
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.out = static_cast<bf16*>(out);
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.scale = scale;
  p.window = window;
  p.num_seqs = num_seqs;
  p.Hq = num_q_heads;
  p.Hkv = num_kv_heads;
  p.g = num_q_heads / num_kv_heads;
  p.hpw = gcd_int(p.g, 4);
  p.causal = causal;
  hipError_t e = launch_prefill_fp8(p, max_seqlen, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int32_t attn_decode_num_splits(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t kv_dtype,
                               int32_t block_size, int32_t max_blocks_per_seq, int32_t requested) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || requested < 0 ||
      (head_dim != 128 && head_dim != 256) || (kv_dtype != ATTN_KV_BF16 && kv_dtype != ATTN_KV_FP8_E4M3FN))
    return 0;
  const int kvt = kv_dtype == ATTN_KV_BF16 ? KV_BF16 : KV_FP8;
  const long long ch = decode_chunk_tokens(head_dim, kvt);
  const long long max_len = (long long)max_blocks_per_seq * block_size;
  // useful shares: at most one per 4 chunks of the largest possible batch
  const long long max_shares = ((long long)num_seqs * num_kv_heads * ((max_len + ch - 1) / ch) + 3) / 4;
  long long s = requested > 0 ? requested : (long long)decode_wgs_per_cu(head_dim, kvt) * device_cu_count();
  if (s > max_shares) s = max_shares;
  if (s > kMaxSplits) s = kMaxSplits;
  return (int32_t)(s < 1 ? 1 : s);
}

size_t attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                   int32_t num_splits) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || num_splits <= 0) return 0;
  return (size_t)num_splits * 2 * 16 * ((size_t)head_dim + 1) * sizeof(float) +
         ((size_t)num_seqs + 1) * sizeof(int32_t);
}

static attn_status validate_paged(const void* q, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                                  const float* k_scale, const float* v_scale, const int32_t* block_table,
                                  const int32_t* seq_lens, const void* out, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                  int32_t num_splits) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return ATTN_ERR_NULL;
  if (kv_dtype != ATTN_KV_BF16 && kv_dtype != ATTN_KV_FP8_E4M3FN) return ATTN_ERR_UNSUPPORTED;
  if (kv_dtype == ATTN_KV_FP8_E4M3FN && (!k_scale || !v_scale)) return ATTN_ERR_NULL;
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || num_splits < 0)
    return ATTN_ERR_SHAPE;
  if (head_dim != 128 && head_dim != 256) return ATTN_ERR_UNSUPPORTED;
  if (!supported_block_size(block_size)) return ATTN_ERR_UNSUPPORTED;
  if (num_seqs > kMaxPagedSeqs) return ATTN_ERR_UNSUPPORTED;
  if ((long long)max_blocks_per_seq * block_size > INT_MAX / 2) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

attn_status attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, float scale, void* out,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t num_splits, float* lse,
                              void* workspace, size_t workspace_bytes,
                              int32_t kv_dtype, const float* k_scale, const float* v_scale, int32_t window,
                              void* stream) {
  attn_status st = validate_paged(q, k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table, seq_lens,
                                  out, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                  num_blocks, max_blocks_per_seq, num_splits);
  if (st != ATTN_OK) return st;
  if (!(std::isfinite(scale) && scale >= 0.f) || window < 0) return ATTN_ERR_SHAPE;
  const int g = num_q_heads / num_kv_heads;
  if (g > 16) return ATTN_ERR_UNSUPPORTED;
  const int S = attn_decode_num_splits(num_seqs, num_kv_heads, head_dim, kv_dtype, block_size,
                                       max_blocks_per_seq, num_splits);
  const size_t need = attn_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, S);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;

  PagedParams p{};
  p.q = static_cast<const bf16*>(q);
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_table = block_table;
  p.seq_lens_k = seq_lens;
  p.cu_seqlens_q = nullptr;
  p.out = static_cast<bf16*>(out);
  p.lse = lse;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_lse = p.ws_o + (size_t)S * 2 * 16 * head_dim;
  p.ws_prefix = reinterpret_cast<int32_t*>(p.ws_lse + (size_t)S * 2 * 16);
  p.scale = scale;
  p.window = window;
  p.num_seqs = num_seqs;
  p.Hq = num_q_heads;
  p.Hkv = num_kv_heads;
  p.g = g;
  p.bs = block_size;
  p.bs_shift = __builtin_ctz((unsigned)block_size);
  p.max_blocks = max_blocks_per_seq;
  p.num_wg = S;
  p.causal = 1;
  p.max_rows = 16;
  hipError_t e = launch_decode(p, head_dim, kv_dtype == ATTN_KV_BF16 ? KV_BF16 : KV_FP8, g,
                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Rows of a partial-result slot in the mixed batch's workspace: the most rows per (request, kv
// head) that its decode role takes (32 with head_dim 128, 16 with head_dim 256).
static int varlen_slot_rows(int32_t head_dim) { return head_dim == 128 ? 32 : 16; }

size_t attn_varlen_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                   int32_t num_splits) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || num_splits <= 0) return 0;
  return (size_t)num_splits * 2 * varlen_slot_rows(head_dim) * ((size_t)head_dim + 1) * sizeof(float) +
         ((size_t)num_seqs + 1) * sizeof(int32_t);
}

attn_status attn_varlen_paged(const void* q, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                              const float* k_scale, const float* v_scale, const int32_t* block_table,
                              const int32_t* cu_seqlens_q, const int32_t* seq_lens_k, int32_t causal,
                              float scale, void* out, float* lse, int32_t num_seqs, int32_t total_q,
                              int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                              int32_t num_splits, void* workspace, size_t workspace_bytes, int32_t window,
                              void* stream) {
  attn_status st = validate_paged(q, k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table, seq_lens_k,
                                  out, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                  num_blocks, max_blocks_per_seq, num_splits);
  if (st != ATTN_OK) return st;
  if (!cu_seqlens_q) return ATTN_ERR_NULL;
  if (total_q < 0 || max_q_len < 0 || max_q_len > total_q || (causal != 0 && causal != 1) ||
      !(std::isfinite(scale) && scale >= 0.f) || window < 0)
    return ATTN_ERR_SHAPE;
  if ((long long)total_q * num_q_heads * head_dim > (long long)INT_MAX * 8) return ATTN_ERR_SHAPE;
  if (num_seqs > mixed_max_seqs(head_dim)) return ATTN_ERR_UNSUPPORTED;
  const int S = attn_decode_num_splits(num_seqs, num_kv_heads, head_dim, kv_dtype, block_size,
                                       max_blocks_per_seq, num_splits);
  const size_t need = attn_varlen_workspace_bytes(num_seqs, num_q_heads, head_dim, S);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (total_q == 0) return ATTN_OK;
  const int g = num_q_heads / num_kv_heads;
  const int kvt = kv_dtype == ATTN_KV_BF16 ? KV_BF16 : KV_FP8;

  PagedParams dp{};
  dp.q = static_cast<const bf16*>(q);
  dp.k_cache = k_cache;
  dp.v_cache = v_cache;
  dp.k_scale = k_scale;
  dp.v_scale = v_scale;
  dp.block_table = block_table;
  dp.seq_lens_k = seq_lens_k;
  dp.cu_seqlens_q = cu_seqlens_q;
  dp.out = static_cast<bf16*>(out);
  dp.lse = lse;
  // requests with up to 16 rows per kv head (32 with head_dim 128 when some request has more
  // than 16) take the decode role; the workspace slots have that many rows
  dp.max_rows = ((long long)max_q_len * g > 16 && varlen_slot_rows(head_dim) >= 32) ? 32 : 16;
  dp.ws_o = static_cast<float*>(workspace);
  dp.ws_lse = dp.ws_o + (size_t)S * 2 * dp.max_rows * head_dim;
  dp.ws_prefix = reinterpret_cast<int32_t*>(dp.ws_lse + (size_t)S * 2 * dp.max_rows);
  dp.scale = scale;
  dp.window = window;
  dp.num_seqs = num_seqs;
  dp.Hq = num_q_heads;
  dp.Hkv = num_kv_heads;
  dp.g = g;
  dp.bs = block_size;
  dp.bs_shift = __builtin_ctz((unsigned)block_size);
  dp.max_blocks = max_blocks_per_seq;
  dp.num_wg = S;
  dp.causal = causal;

  PrefillParams pp{};
  pp.q = dp.q;
  pp.out = dp.out;
  pp.lse = lse;
  pp.cu_seqlens_q = cu_seqlens_q;
  pp.k_cache = k_cache;
  pp.v_cache = v_cache;
  pp.k_scale = kvt == KV_FP8 ? k_scale : nullptr;
  pp.v_scale = kvt == KV_FP8 ? v_scale : nullptr;
  pp.block_table = block_table;
  pp.seq_lens_k = seq_lens_k;
  pp.scale = scale;
  pp.window = window;
  pp.num_seqs = num_seqs;
  pp.Hq = num_q_heads;
  pp.Hkv = num_kv_heads;
  pp.g = g;
  pp.hpw = gcd_int(g, 4);
  pp.causal = causal;
  pp.bs = block_size;
  pp.bs_shift = __builtin_ctz((unsigned)block_size);
  pp.max_blocks = max_blocks_per_seq;
  hipError_t e = launch_mixed(pp, dp, head_dim, kvt, total_q, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}


attn_status attn_kv_append_paged(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                 int32_t kv_dtype, const float* k_scale, const float* v_scale,
                                 const int32_t* block_table, const int32_t* cu_seqlens_new,
                                 const int32_t* seq_lens_k, int32_t num_seqs, int32_t total_new,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, int32_t max_blocks_per_seq, void* stream) {
  if (!k_cache || !v_cache || !block_table || !cu_seqlens_new || !seq_lens_k) return ATTN_ERR_NULL;
  if (kv_dtype != ATTN_KV_BF16 && kv_dtype != ATTN_KV_FP8_E4M3FN) return ATTN_ERR_UNSUPPORTED;
  if (kv_dtype == ATTN_KV_FP8_E4M3FN && (!k_scale || !v_scale)) return ATTN_ERR_NULL;
  if (num_seqs <= 0 || total_new < 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return ATTN_ERR_SHAPE;
  if (head_dim != 128 && head_dim != 256) return ATTN_ERR_UNSUPPORTED;
  if (!supported_block_size(block_size)) return ATTN_ERR_UNSUPPORTED;
  if (num_seqs > kMaxPagedSeqs) return ATTN_ERR_UNSUPPORTED;
  if ((long long)max_blocks_per_seq * block_size > INT_MAX / 2) return ATTN_ERR_SHAPE;
  if (total_new == 0) return ATTN_OK;                // the new rows may then be NULL
  if (!k_new || !v_new) return ATTN_ERR_NULL;
  AppendParams p{};
  p.k_new = static_cast<const bf16*>(k_new);
  p.v_new = static_cast<const bf16*>(v_new);
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_table = block_table;
  p.cu_seqlens_new = cu_seqlens_new;
  p.seq_lens_k = seq_lens_k;
  p.num_seqs = num_seqs;
  p.total_new = total_new;
  p.Hkv = num_kv_heads;
  p.bs = block_size;
  p.max_blocks = max_blocks_per_seq;
  (void)num_blocks;
  hipError_t e = launch_append(p, head_dim, kv_dtype == ATTN_KV_BF16 ? KV_BF16 : KV_FP8,
                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // extern "C"
