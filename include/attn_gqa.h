/*
 * attn_gqa.h -- exact grouped-query softmax attention over a KV cache for AMD
 * MI355X (gfx950). C ABI: plain pointers and sizes, no framework types.
 *
 * What is computed (every entry point): for request b, query head h and query
 * row i, with kv head = h / (num_q_heads / num_kv_heads) (contiguous groups,
 * "Optimization 1: batching and attention", sections 2.2 and 2.4):
 *     s_ij  = scale * <q_i, k_j>                 over the keys j row i may see
 *     out_i = sum_j softmax(s_i)_j * v_j         ("Attention kernels", section
 *                                                 "Memory round trips of standard attention")
 *     lse_i = ln sum_j exp(s_ij)                 (natural log, scale included)
 * The result is exact softmax attention (no approximation): the kernels tile
 * the key axis and keep running row statistics (online softmax, "Attention
 * kernels", section "FlashAttention"); they never write the score matrix.
 * Causal masking is bottom-right aligned: row i of a request with Lq new rows
 * and Lk keys sees keys j <= Lk - Lq + i. A row that sees no key gets out = 0
 * and lse = -inf.
 *
 * Conventions shared by all calls:
 *   - Every pointer argument is DEVICE memory allocated and owned by the caller
 *     (except where stated). The library allocates nothing, frees nothing,
 *     never synchronises the stream and never changes the current device.
 *   - Inputs are read only. out / lse are overwritten in full (every row of
 *     every head); they must not alias any input or the workspace.
 *   - bf16 means IEEE bfloat16 (2 bytes). fp8 means OCP e4m3fn codes (1 byte):
 *     bias 7, no infinities, max 448; the value is code * per-head scale.
 *   - Layouts are row-major with the last index fastest:
 *       q, out   [tokens, num_q_heads, head_dim]
 *       lse      [tokens, num_q_heads]                  fp32
 *       k, v     [tokens, num_kv_heads, head_dim]       (contiguous prefill)
 *       k_cache  [num_blocks, num_kv_heads, block_size, head_dim]
 *       v_cache  [num_blocks, num_kv_heads, head_dim, block_size]  (tokens innermost)
 *       block_table [num_seqs, max_blocks_per_seq] int32: logical block i of
 *       request b lives in physical block block_table[b][i]; token t is slot
 *       t % block_size of logical block t / block_size ("Optimization 1",
 *       section 3.4 PagedAttention; "Attention kernels", section "Paged KV and kernels").
 *   - The V page departs from the K page order ([block_size, head_dim]): it is
 *     stored transposed. The kernels multiply P by V on the matrix cores with the
 *     keys as the reduction axis; with tokens innermost each lane's operand (8
 *     consecutive keys of one head_dim row) is one contiguous 16-byte load
 *     straight from the page, with no transpose through LDS. A page has the same
 *     byte count either way. When block_size == head_dim the two orders have the
 *     same shape, so nothing can detect a V cache written in the K order: the
 *     attention is then silently wrong. The append call writes this order.
 *   - head_dim must be 128 or 256; num_q_heads must be a multiple of
 *     num_kv_heads; block_size must be 16, 32, 64, 128 or 256; paged calls
 *     take at most 16384 requests.
 *   - scale (every call) must be finite and >= 0; otherwise ATTN_ERR_SHAPE.
 *   - window (every attention call): 0 = no window; W > 0 = sliding window:
 *     row i additionally drops the keys j < Lk - Lq + i - W + 1, so with causal
 *     masking it sees its own position and the W - 1 keys before it (a lower
 *     bound on the visible keys, bottom-right aligned like the causal bound;
 *     "Optimization 1", section 2 on shrinking the KV a token attends to; the
 *     NVIDIA guideline summary, principle 3). Negative: ATTN_ERR_SHAPE.
 *   - stream is a hipStream_t (NULL = the default stream). Calls return once
 *     the work is enqueued; results are valid after the stream synchronises.
 *   - Argument validation is synchronous and happens before anything is
 *     launched: a validation error (ATTN_ERR_NULL, _SHAPE, _UNSUPPORTED,
 *     _WORKSPACE) launches nothing and writes nothing. ATTN_ERR_LAUNCH means the
 *     HIP runtime refused one of the call's kernels; kernels of the call
 *     enqueued before it may then have run, so out / lse / the workspace (or the
 *     caches, for the append) are undefined. An error left pending by earlier,
 *     unrelated HIP work is neither reported as this call's nor cleared.
 *     Device-resident values (cu_seqlens, seq_lens, block-table entries) are
 *     NOT validated: they are the caller's contract (monotone cu_seqlens,
 *     0 <= seq_lens[b] <= max_blocks_per_seq * block_size, table entries in
 *     [0, num_blocks) for every block a request uses).
 */
#ifndef ATTN_GQA_H
#define ATTN_GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t attn_status;

#define ATTN_OK 0
#define ATTN_ERR_NULL 1         /* a required pointer is NULL */
#define ATTN_ERR_SHAPE 2        /* counts <= 0, Hq % Hkv != 0, inconsistent sizes */
#define ATTN_ERR_UNSUPPORTED 3  /* head_dim, block_size or kv dtype not supported */
#define ATTN_ERR_WORKSPACE 4    /* workspace NULL or smaller than required */
#define ATTN_ERR_LAUNCH 5       /* the HIP runtime reported an error at launch */

#define ATTN_KV_BF16 0
#define ATTN_KV_FP8_E4M3FN 1

/* Human-readable name of a status code (static storage; never NULL). */
const char* attn_status_string(attn_status status);

/*
 * Varlen prefill over contiguous K/V ("Attention kernels", section
 * "FlashAttention"; the varlen batch: section "Paged KV and kernels").
 * Request b owns rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of q, k, v, out, lse
 * and attends within itself (Lq = Lk = its length).
 *   q [total_tokens, num_q_heads, head_dim] bf16; k, v [total_tokens, num_kv_heads, head_dim] bf16
 *   cu_seqlens [num_seqs + 1] int32 (device), cu_seqlens[0] = 0, cu_seqlens[num_seqs] = total_tokens
 *   causal: 0 or 1; scale: score multiplier, finite and >= 0 (e.g. 1/sqrt(head_dim))
 *   out [total_tokens, num_q_heads, head_dim] bf16 (round to nearest even)
 *   lse [total_tokens, num_q_heads] fp32, or NULL to skip it
 *   max_seqlen: an upper bound on every request's length (sizes the grid)
 *   window: sliding window (0 = none), see the conventions above
 * Needs no workspace: nothing but out and lse is written. Sizes are checked
 * first; total_tokens = 0 (or max_seqlen = 0) is then a no-op that returns
 * ATTN_OK whatever the pointers (empty tensors may pass NULL).
 */
attn_status attn_prefill_varlen(const void* q, const void* k, const void* v,
                                const int32_t* cu_seqlens, int32_t causal, float scale,
                                void* out, float* lse,
                                int32_t num_seqs, int32_t total_tokens, int32_t max_seqlen,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t window, void* stream);

/*
 * FP8 varlen prefill ("Attention kernels", section "FlashAttention": the third
 * version's FP8 variant) on the gfx950 fp8 matrix cores. Inputs are OCP e4m3fn
 * codes with per-head fp32 scales; the call computes the attention of
 * attn_prefill_varlen on the decoded values
 *   Q[t, h, :] = q_scale[h]   * e4m3(q[t, h, :])
 *   K[t, j, :] = k_scale[j]   * e4m3(k[t, j, :])
 *   V[t, j, :] = v_scale[j]   * e4m3(v[t, j, :])
 * with the exponentials P rounded to e4m3 (round to nearest even) for the P V
 * product; tiles that mask some keys of a row carry P as two e4m3 parts (hi and
 * the rounding remainder). Row sums and the LSE use the unrounded exponentials.
 * Results agree with the exact attention of the decoded inputs to within the
 * fp8 tolerance of the tests (max-abs 3e-2 on out; the LSE to 1e-3).
 *   q [total_tokens, num_q_heads, 128], k, v [total_tokens, num_kv_heads, 128] uint8 codes;
 *   every code must be finite (not 0x7F / 0xFF)
 *   q_scale [num_q_heads], k_scale, v_scale [num_kv_heads] fp32 (device), finite and >= 0
 *   other arguments and the outputs as for attn_prefill_varlen (window: sliding window, 0 = none)
 * head_dim other than 128 returns ATTN_ERR_UNSUPPORTED. Needs no workspace;
 * total_tokens = 0 is a no-op as for attn_prefill_varlen.
 */
attn_status attn_prefill_varlen_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                                    const float* k_scale, const float* v_scale, const int32_t* cu_seqlens,
                                    int32_t causal, float scale, void* out, float* lse,
                                    int32_t num_seqs, int32_t total_tokens, int32_t max_seqlen,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t window, void* stream);

/*
 * Number of partitions (partition workgroups) a paged decode call will use
 * (split-KV, "Attention kernels", section "Prefill and decode attention").
 * The batch's work -- every (request, kv head, chunk of keys) -- is cut into
 * that many contiguous shares of equal planned cost: a chunk counts one, and a
 * (request, kv head) of fewer than 256 chunks counts two more for starting it,
 * so each partition takes about the same time whatever the mix of context
 * lengths; a request whose keys span several shares is merged from their
 * partial results. requested > 0 is
 * returned clamped to the useful count (at most one share per 4 chunks of the
 * largest possible batch) and to 4096; requested == 0 picks one partition per
 * resident workgroup slot of the device (compute units x workgroups per unit
 * for this head_dim and kv_dtype). Returns 0 on invalid arguments.
 */
int32_t attn_decode_num_splits(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t kv_dtype,
                               int32_t block_size, int32_t max_blocks_per_seq, int32_t requested);

/*
 * Workspace bytes a paged decode / varlen-paged call needs for num_splits
 * (resolved, >= 1) partitions: two partial results per partition (16 rows x
 * head_dim fp32 outputs plus 16 fp32 LSEs each) and num_seqs + 1 int32 chunk
 * offsets. The size does not depend on the head count (a partition holds at
 * most 16 rows of one KV group); num_q_heads must only be positive. Returns 0
 * for a non-positive argument. The contents need no initialisation; calls
 * that share one workspace must not overlap in time (enqueue them on one
 * stream).
 */
size_t attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                   int32_t num_splits);

/*
 * Paged decode: one query token per request over its paged KV cache.
 * Each KV head is read once for all num_q_heads / num_kv_heads query heads of
 * its group ("Attention kernels", section "Prefill and decode attention"); the
 * key axis is split across num_splits partitions that take equal shares of
 * the batch's keys (see attn_decode_num_splits), and the pieces of a request
 * are merged with their log-sum-exps.
 *   q [num_seqs, num_q_heads, head_dim] bf16 (the newest token of each request)
 *   k_cache, v_cache: see the layouts above; kv_dtype ATTN_KV_BF16 or ATTN_KV_FP8_E4M3FN
 *   k_scale, v_scale [num_kv_heads] fp32 per-head dequantisation scales (fp8 only; ignored for bf16)
 *   block_table [num_seqs, max_blocks_per_seq] int32; seq_lens [num_seqs] int32 =
 *   number of cached tokens INCLUDING the current one (0 gives out 0, lse -inf)
 *   out [num_seqs, num_q_heads, head_dim] bf16; lse [num_seqs, num_q_heads] fp32 or NULL
 *   num_splits: 0 = automatic (attn_decode_num_splits), else the partition count
 *   workspace: device scratch of >= attn_decode_workspace_bytes(...) bytes.
 *   kv_dtype, k_scale, v_scale, window: as above (they follow the arguments of
 *   the plain bf16 call, so a bf16 caller passes ATTN_KV_BF16, NULL, NULL, 0).
 * A (request, kv head) whose keys lie in one partition's share is written by
 * that partition; otherwise each partition writes a normalised partial output
 * and its LSE to the workspace, and a second kernel, enqueued on the same
 * stream, merges them (it also writes the rows of requests with no key).
 * Requires num_q_heads / num_kv_heads <= 16.
 */
attn_status attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, float scale, void* out,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t num_splits, float* lse,
                              void* workspace, size_t workspace_bytes,
                              int32_t kv_dtype, const float* k_scale, const float* v_scale, int32_t window,
                              void* stream);

/*
 * attn_decode_paged for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid allocation. It
 * takes no workspace: the split-KV partials go to a fixed array of
 * ATTN_DECODE_NOALLOC_MAX_BYTES bytes that the library holds on every GPU it
 * runs on until the process ends. The call allocates nothing (no hipMalloc, no
 * allocating library routine); the array's device address is looked up once
 * per device on the first call there.
 *   Arguments, layouts, results and validation errors: as attn_decode_paged
 *   (without workspace / workspace_bytes).
 *   ATTN_ERR_WORKSPACE: the call would need more than
 *   ATTN_DECODE_NOALLOC_MAX_BYTES of partials (attn_decode_workspace_bytes of
 *   its resolved partition count); nothing is launched. The automatic count
 *   (num_splits = 0) fits every supported shape on MI355X.
 * Every call on one GPU shares that GPU's array and it keeps the last call's
 * contents: calls that overlap in time on one GPU (two streams, two host
 * threads) race and give undefined results. Enqueue them on one stream.
 */
#define ATTN_DECODE_NOALLOC_MAX_BYTES ((size_t)16 << 20)

attn_status attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* seq_lens, float scale, void* out,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t num_splits, float* lse,
                                      int32_t kv_dtype, const float* k_scale, const float* v_scale,
                                      int32_t window, void* stream);

/*
 * Mixed varlen batch over a paged cache in one attention launch ("Attention
 * kernels", section "Paged KV and kernels": prefill chunks and decode requests
 * of different lengths in one step). Request b owns query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and seq_lens_k[b] cached keys, its
 * own new tokens being the last Lq of them (a prefill chunk over a cached
 * prefix, or a decode token). Requests whose Lq * (num_q_heads/num_kv_heads)
 * is at most 16 run on the split-KV decode path (num_splits partitions, as in
 * attn_decode_paged); with head_dim 128 so do requests of up to 32 such rows
 * when max_q_len * (num_q_heads/num_kv_heads) exceeds 16 (several new tokens
 * per request, as in speculative verification); the others run on the tiled
 * prefill path. max_q_len is the largest Lq (a smaller value is not an error:
 * it only sends requests of 17-32 rows to the prefill path).
 *   q, out [total_q, num_q_heads, head_dim] bf16; lse [total_q, num_q_heads] fp32 or NULL
 *   causal: 0 or 1 (bottom-right aligned)
 *   workspace: >= attn_varlen_workspace_bytes(...) bytes of device scratch:
 *     per partition two partial results of 32 rows (head_dim 128) or 16 rows
 *     (head_dim 256) x (head_dim + 1) floats, then num_seqs + 1 int32.
 * With head_dim 256, num_seqs above 7927 returns ATTN_ERR_UNSUPPORTED (the
 * kernel keeps per-request offsets in LDS beside its 129 KB of tiles or
 * partial results).
 */
size_t attn_varlen_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                   int32_t num_splits);

attn_status attn_varlen_paged(const void* q, const void* k_cache, const void* v_cache,
                              int32_t kv_dtype, const float* k_scale, const float* v_scale,
                              const int32_t* block_table, const int32_t* cu_seqlens_q,
                              const int32_t* seq_lens_k, int32_t causal, float scale,
                              void* out, float* lse,
                              int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                              int32_t num_splits, void* workspace, size_t workspace_bytes,
                              int32_t window, void* stream);

/*
 * Append new tokens' K and V to a paged cache, the step before attention in
 * every engine step ("Optimization 1: batching and attention", section 3.4:
 * the cache is a pool of fixed-size blocks reached through a block table;
 * "Attention kernels", section "Paged KV and kernels": an FP8 cache is read
 * directly by the attention kernels).
 * Request b's new tokens are rows cu_seqlens_new[b] .. cu_seqlens_new[b+1]-1
 * of k_new / v_new (n_b of them); they become its cached tokens
 * seq_lens_k[b] - n_b .. seq_lens_k[b] - 1 (seq_lens_k counts them, as the
 * attention calls do). Token t goes to slot t % block_size of physical block
 * block_table[b][t / block_size]: the K row [block][h][slot][:] and the V
 * column [block][h][:][slot] (layouts as above). No other byte of the caches
 * changes.
 *   k_new, v_new [total_new, num_kv_heads, head_dim] bf16 (device, read only)
 *   k_cache, v_cache: bf16 (ATTN_KV_BF16: the values are stored unchanged) or
 *     e4m3fn codes (ATTN_KV_FP8_E4M3FN: code = e4m3fn(x / scale[h]), the
 *     quotient in correctly rounded fp32, rounded to the nearest code with ties
 *     to even, magnitudes beyond 448 saturated); k_scale, v_scale [num_kv_heads]
 *     fp32 (device), required for fp8, ignored for bf16.
 *   cu_seqlens_new [num_seqs + 1], seq_lens_k [num_seqs] int32 (device).
 * Device-resident values are the caller's contract as for the attention calls;
 * in addition n_b <= seq_lens_k[b], distinct new tokens must map to distinct
 * slots, and the new rows must not alias the caches. total_new = 0 is a no-op
 * (k_new and v_new may then be NULL).
 * Errors: ATTN_ERR_NULL (a required pointer is NULL), ATTN_ERR_SHAPE (counts
 * out of range), ATTN_ERR_UNSUPPORTED (head_dim, block_size, kv dtype or more
 * than 16384 requests).
 */
attn_status attn_kv_append_paged(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                 int32_t kv_dtype, const float* k_scale, const float* v_scale,
                                 const int32_t* block_table, const int32_t* cu_seqlens_new,
                                 const int32_t* seq_lens_k, int32_t num_seqs, int32_t total_new,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, int32_t max_blocks_per_seq, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_GQA_H */
