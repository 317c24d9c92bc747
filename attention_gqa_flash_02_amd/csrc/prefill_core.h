// Tiled causal/non-causal prefill for gfx950 on bf16 MFMA, over contiguous or paged K/V.
//
// What it computes ("Attention kernels", section "FlashAttention"): Q, K and V
// are cut into tiles; each workgroup keeps its query rows in registers,
// streams K/V tiles through LDS, and per tile computes the scores, updates each
// row's running maximum and exponential sum (rescaling what it has accumulated
// when the maximum moves) and accumulates P V. Only O and one log-sum-exp per
// row are written; the score matrix never leaves the chip. Causal masking is
// bottom-right aligned: row i of a request with Lq new rows and Lk keys sees
// keys j <= Lk - Lq + i (for self-attention Lq = Lk); a sliding window W also
// drops keys j < Lk - Lq + i - W + 1 (a workgroup's loop starts at the tile
// holding its first visible key; tiles below some row's lower bound mask it).
//
// Layout of the work:
//   * a workgroup is 4 waves; each wave owns 32 query rows = 32 tokens of one
//     query head. The waves of a workgroup are the query heads that share one
//     KV head (up to 4 of them) times consecutive 32-token blocks, so one K/V
//     tile staged in LDS serves every head of the group (GQA sharing).
//   * S^T = K Q^T on 32x32x16 MFMA: the wave's 32 query rows are the MFMA
//     columns, so every lane owns one query row and its softmax state lives in
//     that lane (plus its partner lane 32 apart).
//   * A-row i of a 32-key block loads key pi(i) = i with bits 2 and 3 swapped;
//     then accumulator r of lane half hh holds key 16*(r/8) + 8*hh + r%8, and
//     the 8 k-slots a lane feeds to the P V MFMA are 8 consecutive keys: V^T is
//     read from LDS with one 16-byte read per MFMA operand.
//   * O^T += V^T P^T on 32x32x16 MFMA, P^T being the bf16-rounded S^T
//     accumulator (no shuffle, no LDS round trip for P).
//   * K tiles are stored row-major in LDS, V tiles transposed ([d][key]); row
//     strides are padded by 16 bytes so that the MFMA operand reads are free of
//     bank conflicts. LDS is double-buffered: tile n+1 is fetched into
//     registers while tile n is computed.
//   * softmax state in the base-2 exponent domain (t = c * s, c = scale *
//     log2 e): a reference maximum mc per row that only moves when a tile's
//     maximum exceeds it by more than 2^8 (so the O rescale is skipped on
//     almost every tile); the row sum is kept in fp32 (the log-sum-exp carries no
//     bf16 rounding of P). Tiles crossing the causal diagonal or the end
//     of the keys mask their scores and carry P as hi + lo bf16 parts (there a
//     row sees few keys and the rounding of P would not average out).
//   * K/V come from contiguous [tokens, Hkv, D] bf16 tensors or from a paged
//     cache (K pages [Hkv][bs][D], V pages [Hkv][D][bs], bf16 or OCP e4m3fn
//     codes dequantised to bf16 on the way into LDS; the per-head k_scale is
//     folded into c and v_scale into the final normalisation).
#pragma once

#include <climits>

#include "common.h"

namespace attn {

enum { KVSRC_CONTIG = 0, KVSRC_PAGED_BF16 = 1, KVSRC_PAGED_FP8 = 2 };

struct PrefillParams {
  const bf16* q;               // [Tq, Hq, D]
  bf16* out;                   // [Tq, Hq, D]
  float* lse;                  // [Tq, Hq] or nullptr
  const int32_t* cu_seqlens_q; // [B + 1]
  // contiguous K/V (self-attention: request b owns rows cu_seqlens_q[b] .. of k and v)
  const bf16* k;               // [T, Hkv, D]
  const bf16* v;               // [T, Hkv, D]
  // paged K/V
  const void* k_cache;         // [num_blocks, Hkv, bs, D]
  const void* v_cache;         // [num_blocks, Hkv, D, bs]
  const float* k_scale;        // [Hkv] (fp8) or nullptr
  const float* v_scale;        // [Hkv] (fp8) or nullptr
  const int32_t* block_table;  // [B, max_blocks]
  const int32_t* seq_lens_k;   // [B] keys per request (its Lq new tokens are the last ones)
  float scale;
  int num_seqs, Hq, Hkv, g, hpw, causal, num_qtiles, bs, max_blocks;
  int window;                  // > 0: row i also drops keys j < shift + i - window + 1
  int bs_shift;                // log2(bs) for paged K/V: block sizes are powers of two
};

template <int D, int BN>
struct PrefillShape {
  static constexpr int KS = D + 8;                  // K tile row stride in LDS (elements)
  static constexpr int VS = BN + 8;                 // V^T tile row stride in LDS (elements)
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
  static constexpr int LDS_BYTES = 2 * BUF * 2;     // two buffers of bf16
  static_assert(BN % 32 == 0, "key tiles are whole 32-key MFMA blocks");
};

// Key loaded by A-row i of a 32-key block: bits 2 and 3 of i swapped.
__device__ __forceinline__ int key_perm32(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// ---------------------------------------------------------------------------------------------
// K/V tile loaders: fetch(n) issues the global loads of key tile n into registers, stage(dst)
// writes them into one LDS buffer (K [BN][KS] row-major, V^T [D][VS]). Keys at or past Lk are
// zero in both (their scores are masked, and zero V keeps NaN-carrying slots out of P V).
// ---------------------------------------------------------------------------------------------

// Contiguous bf16 K/V [T, Hkv, D]: K rows are copied, V is transposed 4 keys x 8 d at a time.
// Loads are buffer loads: per tile a resource whose range ends at the request's last key (so
// rows past the keys read as zero, with no branch), and per-thread byte offsets that stay fixed
// for the whole loop (so no register written in the loop is a pending load's address).
template <int D, int BN>
struct ContigLoader {
  static constexpr int KCH = D / 8;                 // 16-byte chunks per K row
  static constexpr int K_LOADS = BN * KCH / 256;
  static constexpr int K_ROWS_PER_PASS = 256 / KCH;
  static constexpr int VKG = BN / 4;                // 4-key groups per V tile
  static constexpr int VB = VKG * (D / 8) / 256;    // 4-key x 8-d blocks of V per thread
  static_assert(VB >= 1 && VKG * (D / 8) % 256 == 0, "V staging splits into whole 4x8 blocks");
  u32x4 kreg[K_LOADS];
  u32x4 vreg[4 * VB];
  const char* kbase;
  const char* vbase;
  long long row_bytes;                              // bytes between consecutive tokens
  long long end_bytes;                              // bytes from the first row to the end of the last key
  int koff[K_LOADS], voff[4 * VB];
  int kch, krow0, vkg, vdc;

  __device__ __forceinline__ void init(const PrefillParams& p, int b, int kvh, int Lk, int first_tile) {
    (void)first_tile;
    const int tid = threadIdx.x;
    const int seq0 = p.cu_seqlens_q[b];
    const long long stride = (long long)p.Hkv * D;
    kbase = reinterpret_cast<const char*>(p.k + (size_t)seq0 * stride + (size_t)kvh * D);
    vbase = reinterpret_cast<const char*>(p.v + (size_t)seq0 * stride + (size_t)kvh * D);
    row_bytes = stride * 2;
    end_bytes = Lk > 0 ? (long long)(Lk - 1) * row_bytes + D * 2 : 0;
    kch = tid % KCH;
    krow0 = tid / KCH;
    vkg = tid % VKG;
    vdc = tid / VKG;
#pragma unroll
    for (int it = 0; it < K_LOADS; ++it) koff[it] = (int)((it * K_ROWS_PER_PASS + krow0) * row_bytes + 16 * kch);
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        voff[4 * vb + s] = (int)((4 * vkg + s) * row_bytes + 16 * (vdc + vb * (256 / VKG)));
  }
  __device__ __forceinline__ void fetch(int n) {
    const long long t = (long long)n * BN * row_bytes;
    long long left = end_bytes - t;
    left = left < 0 ? 0 : (left > (long long)BN * row_bytes ? (long long)BN * row_bytes : left);
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + t), 0, (int)left, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + t), 0, (int)left, kBufferFlags);
#pragma unroll
    for (int it = 0; it < K_LOADS; ++it)
      kreg[it] = bitcast<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(kr, koff[it], 0, 0));
#pragma unroll
    for (int s = 0; s < 4 * VB; ++s) vreg[s] = bitcast<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(vr, voff[s], 0, 0));
  }
  __device__ __forceinline__ void stage(bf16* Ks, bf16* Vt) {
    using S = PrefillShape<D, BN>;
#pragma unroll
    for (int it = 0; it < K_LOADS; ++it)
      *reinterpret_cast<u32x4*>(Ks + (it * K_ROWS_PER_PASS + krow0) * S::KS + 8 * kch) = kreg[it];
    // transpose each 4 keys x 8 d block: d-row 8*dc + e gets keys 4*vkg .. 4*vkg+3
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      const int dc = vdc + vb * (256 / VKG);
      const u32x4* v = vreg + 4 * vb;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo01 = __builtin_amdgcn_perm(v[1][w], v[0][w], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(v[3][w], v[2][w], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(v[1][w], v[0][w], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(v[3][w], v[2][w], 0x07060302u);
        *reinterpret_cast<u32x2*>(Vt + (8 * dc + 2 * w) * S::VS + 4 * vkg) = u32x2{lo01, lo23};
        *reinterpret_cast<u32x2*>(Vt + (8 * dc + 2 * w + 1) * S::VS + 4 * vkg) = u32x2{hi01, hi23};
      }
    }
  }
};

// Paged cache (bf16 or fp8 codes). K: thread loads 16 bytes of one key row (8 bf16 / 16 fp8
// values); V^T: 16 bytes of one d row of one page (8 bf16 / 16 fp8 consecutive tokens). Tokens
// past Lk read the request's last page (a valid address, so the loads are unconditional) and
// are zeroed when the registers are written to LDS.
template <int D, int BN, bool FP8>
struct PagedLoader {
  static constexpr int ELT = FP8 ? 1 : 2;
  static constexpr int VPL = 16 / ELT;              // values per 16-byte load
  static constexpr int K_CH = D / VPL;              // 16-byte loads per K row
  static constexpr int K_LOADS = BN * K_CH / 256;
  static constexpr int V_CH = BN / VPL;             // 16-byte loads per V^T d row of the tile
  static constexpr int V_LOADS = D * V_CH / 256;
  static_assert(K_LOADS >= 1 && V_LOADS >= 1 && BN * K_CH % 256 == 0 && D * V_CH % 256 == 0, "tile split");
  // K: thread t loads K_LOADS consecutive 16-byte chunks of key row t / K_TPR (one page, so one
  // block-table entry); V: thread t loads VPL-key runs starting at the same key for V_LOADS d rows
  // (again one page).
  static constexpr int K_TPR = 256 / BN;            // threads per K row
  static_assert(256 % BN == 0 && K_TPR * K_LOADS == K_CH && 256 % V_CH == 0, "one page per thread");
  u32x4 kreg[K_LOADS];
  u32x4 vreg[V_LOADS];
  const char* kc;
  const char* vc;
  const int32_t* table;
  size_t block_stride;                              // bytes between consecutive blocks
  int Lk, bs, bs_shift;

  __device__ __forceinline__ void init(const PrefillParams& p, int b, int kvh, int Lk_, int first_tile) {
    const size_t page = (size_t)p.bs * D * ELT;
    kc = reinterpret_cast<const char*>(p.k_cache) + (size_t)kvh * page;
    vc = reinterpret_cast<const char*>(p.v_cache) + (size_t)kvh * page;
    block_stride = (size_t)p.Hkv * page;
    table = p.block_table + (size_t)b * p.max_blocks;
    Lk = Lk_;
    bs = p.bs;
    bs_shift = p.bs_shift;
    if (first_tile * BN < Lk) load_table(first_tile);
  }
  // Block-table entries are loaded one tile ahead of the K/V loads that use them, so a fetch
  // never waits on a table load.
  int kphys, vphys;
  int tile0;
  __device__ __forceinline__ void load_table(int n) {
    const int tid = threadIdx.x;
    const int n0 = n * BN;
    const int last = Lk - 1;
    kphys = table[min(n0 + tid / K_TPR, last) >> bs_shift];
    vphys = table[min(n0 + VPL * (tid % V_CH), last & ~(VPL - 1)) >> bs_shift];
  }
  __device__ __forceinline__ void fetch(int n) {                // table entries of tile n are loaded
    const int tid = threadIdx.x;
    const int n0 = n * BN;
    tile0 = n0;
    const int last = Lk - 1;
    {
      const int key = min(n0 + tid / K_TPR, last);
      const char* row = kc + (size_t)kphys * block_stride + (size_t)(key & (bs - 1)) * D * ELT +
                        16 * K_LOADS * (tid % K_TPR);
#pragma unroll
      for (int it = 0; it < K_LOADS; ++it) kreg[it] = ld16(row + 16 * it);   // rows past the keys are zeroed in stage
    }
    {
      const int tt = min(n0 + VPL * (tid % V_CH), last & ~(VPL - 1));   // a VPL-aligned run inside a valid page
      const char* col = vc + (size_t)vphys * block_stride + (size_t)(tt & (bs - 1)) * ELT;
#pragma unroll
      for (int it = 0; it < V_LOADS; ++it) {
        const int d = (it * 256 + tid) / V_CH;
        vreg[it] = ld16(col + (size_t)d * bs * ELT);
      }
    }
    if ((n + 1) * BN < Lk) load_table(n + 1);
  }
  __device__ __forceinline__ void stage(bf16* Ks, bf16* Vt) {
    using S = PrefillShape<D, BN>;
    const int tid = threadIdx.x;
    if (tile0 + BN > Lk) {                          // the last tile: zero keys past the end
      if (tile0 + tid / K_TPR >= Lk) {
#pragma unroll
        for (int it = 0; it < K_LOADS; ++it) kreg[it] = u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int it = 0; it < V_LOADS; ++it) {
        const int t0 = tile0 + VPL * ((it * 256 + tid) % V_CH);
        const int valid = Lk - t0;                  // values of this run that exist (may be <= 0)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int first = e * (4 / ELT);          // first value index held by dword e
          uint32_t keep = 0;
#pragma unroll
          for (int v = 0; v < 4 / ELT; ++v)
            if (first + v < valid) keep |= (FP8 ? 0xFFu : 0xFFFFu) << (8 * ELT * v);
          vreg[it][e] &= keep;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < K_LOADS; ++it) {
      const int key = tid / K_TPR, ch = K_LOADS * (tid % K_TPR) + it;
      bf16* dst = Ks + key * S::KS + VPL * ch;
      if constexpr (FP8) {
        *reinterpret_cast<bf16x8*>(dst) = fp8x8_to_bf16x8(kreg[it][0], kreg[it][1]);
        *reinterpret_cast<bf16x8*>(dst + 8) = fp8x8_to_bf16x8(kreg[it][2], kreg[it][3]);
      } else {
        *reinterpret_cast<u32x4*>(dst) = kreg[it];
      }
    }
#pragma unroll
    for (int it = 0; it < V_LOADS; ++it) {
      const int idx = it * 256 + tid;
      const int d = idx / V_CH, t = VPL * (idx % V_CH);
      bf16* dst = Vt + d * S::VS + t;
      if constexpr (FP8) {
        *reinterpret_cast<bf16x8*>(dst) = fp8x8_to_bf16x8(vreg[it][0], vreg[it][1]);
        *reinterpret_cast<bf16x8*>(dst + 8) = fp8x8_to_bf16x8(vreg[it][2], vreg[it][3]);
      } else {
        *reinterpret_cast<u32x4*>(dst) = vreg[it];
      }
    }
  }
};

// ---------------------------------------------------------------------------------------------
// One workgroup: q-tile qt of request b for head group hgrp.
// ---------------------------------------------------------------------------------------------
template <int D, int BN, class Loader, bool PAGED>
__device__ __forceinline__ void prefill_tile_body(const PrefillParams& p, bf16* smem, int hgrp, int b, int qt) {
  using S = PrefillShape<D, BN>;
  constexpr int NKB = BN / 32;      // 32-key blocks per tile
  constexpr int NDB = D / 32;       // 32-wide d blocks of O^T
  constexpr int NKK = D / 16;       // k-steps of the QK MFMA
  constexpr float kLazyRescale = 8.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane & 31;          // query row of this lane (MFMA column)
  const int hh = lane >> 5;         // lane half

  const int groups_per_kv = p.g / p.hpw;
  const int kvh = hgrp / groups_per_kv;
  const int head = kvh * p.g + (hgrp % groups_per_kv) * p.hpw + (wave % p.hpw);
  const int nwt = 4 / p.hpw;
  const int TQ = 32 * nwt;
  const int q0 = p.cu_seqlens_q[b];
  const int Lq = p.cu_seqlens_q[b + 1] - q0;
  const int Lk = PAGED ? p.seq_lens_k[b] : Lq;
  const int t0 = qt * TQ;
  if (t0 >= Lq) return;
  const int tw = t0 + 32 * (wave / p.hpw);               // first query row of this wave
  const bool wave_active = tw < Lq;
  const int shift = Lk - Lq;                             // row i sees keys <= shift + i (causal)
  // keys any row of the workgroup / of this wave sees
  const int kv_end = p.causal ? min(Lk, shift + min(Lq, t0 + TQ)) : Lk;
  const int wave_kv_end = p.causal ? min(Lk, shift + min(Lq, tw + 32)) : Lk;
  const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  // sliding window: the first key any row of the workgroup / of this wave sees, and the largest
  // first-visible key of the wave's rows (tiles below it mask the lower edge)
  const int win = p.window;
  const int kv_begin = win > 0 ? max(0, shift + t0 - win + 1) : 0;
  const int wave_kv_begin = win > 0 ? max(0, shift + tw - win + 1) : 0;
  const int wave_lower_max = win > 0 ? shift + tw + 31 - win + 1 : INT_MIN;
  const int n_first = min(kv_begin / BN, ntiles);
  float kscale = 1.f, vscale = 1.f;
  if (PAGED && p.k_scale) { kscale = p.k_scale[kvh]; vscale = p.v_scale[kvh]; }
  const float c = p.scale * kscale * kLog2e;

  // ---- Q^T operands: lane (j, hh) holds Q[row tw + j][16*kk + 8*hh .. +7].
  bf16x8 qB[NKK];
  const int qrow_i = tw + j;
  if (qrow_i < Lq) {
    const bf16* qrow = p.q + ((size_t)(q0 + qrow_i) * p.Hq + head) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qB[kk] = *reinterpret_cast<const bf16x8*>(qrow + 16 * kk + 8 * hh);
  } else {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qB[kk] = bf16x8{};
  }
  // An empty asm redefines the Q registers: the loads are waited for here, once, and the loop
  // never sees them as outstanding (it would otherwise wait on the memory counter before each
  // QK MFMA, i.e. on the next tile's prefetch).
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(qB[kk]));
  // last key row j may see, and the first key at which some row of the wave stops seeing keys
  const int lim = p.causal ? min(shift + qrow_i, Lk - 1) : (Lk - 1);
  const int lower = win > 0 ? shift + qrow_i - win + 1 : INT_MIN;   // first key row j may see
  // first key that some row of the wave does not see (tiles reaching it need the mask)
  const int wave_mask_from = p.causal ? max(0, shift + tw + 1) : Lk;

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float mc = kNegInf, l = 0.f;

  Loader ld;
  ld.init(p, b, kvh, Lk, n_first);
  if (n_first < ntiles) {
    ld.fetch(n_first);
    bf16* nb = smem + (n_first & 1) * S::BUF;
    ld.stage(nb, nb + S::K_ELEMS);
  }
  __syncthreads();
  const int kperm = key_perm32(j);

  for (int n = n_first; n < ntiles; ++n) {
    const int cur = n & 1;
    if (n + 1 < ntiles) ld.fetch(n + 1);
    const int n0 = n * BN;
    if (wave_active && n0 < wave_kv_end && n0 + BN > wave_kv_begin) {
      const bf16* Ks = smem + cur * S::BUF;
      const bf16* Vt = Ks + S::K_ELEMS;
      // S^T = K . Q^T
      f32x16 st[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kb][r] = 0.f;
        const bf16* krow = Ks + (32 * kb + kperm) * S::KS + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          st[kb] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(krow + 16 * kk), qB[kk], st[kb]);
      }
      // tiles that cross the causal edge of some row of the wave or the end of the keys
      const bool edge = (n0 + BN > Lk) || (n0 + BN - 1 >= wave_mask_from) || (n0 < wave_lower_max);
      if (edge) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = n0 + 32 * kb + 16 * (r >> 3) + 8 * hh + (r & 7);
            st[kb][r] = (key <= lim && key >= lower) ? st[kb][r] : kNegInf;
          }
      }
      // tile maximum of the raw scores (c >= 0, so it maps to the maximum of t = c * s)
      float tmax = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) tmax = max3(tmax, st[kb][r], st[kb][r + 1]);
      tmax = max_with_other_half(tmax);
      tmax = (tmax == kNegInf) ? kNegInf : tmax * c;
      // move the reference (and rescale what was accumulated) only where the tile maximum is
      // more than kLazyRescale above it; a row's first visible tile always moves it
      const bool move = tmax > mc + kLazyRescale;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        const float alpha = move ? ((mc == kNegInf) ? 0.f : fast_exp2(mc - tmax)) : 1.f;
        mc = move ? tmax : mc;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
      }
      const float nbase = (mc == kNegInf) ? 0.f : -mc;   // p = 2^(c * s - mc)
      if (!edge) {
        bf16x8 pB[NKB][2];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            {
              float e[8];
#pragma unroll
              for (int s = 0; s < 8; ++s) e[s] = fast_exp2(__builtin_fmaf(st[kb][8 * t + s], c, nbase));
#pragma unroll
              for (int s = 0; s < 8; s += 2) {
                const bf16x2 pe = cvt_pk_bf16(e[s], e[s + 1]);
                pB[kb][t][s] = pe[0];
                pB[kb][t][s + 1] = pe[1];
              }
              // pairwise sum: a short dependency chain instead of eight serial adds
              l += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
            }
          }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16* vrow = Vt + (32 * db + j) * S::VS + 8 * hh;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int t = 0; t < 2; ++t)
              acc[db] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(vrow + 32 * kb + 16 * t), pB[kb][t], acc[db]);
        }
      } else {
        // edge tile: P as hi + lo bf16 parts
        bf16x8 pB[NKB][2], pL[NKB][2];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const float x = st[kb][8 * t + s];
              const float e = (x == kNegInf) ? 0.f : fast_exp2(__builtin_fmaf(x, c, nbase));
              l += e;
              pB[kb][t][s] = (bf16)e;
              pL[kb][t][s] = (bf16)(e - (float)pB[kb][t][s]);
            }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16* vrow = Vt + (32 * db + j) * S::VS + 8 * hh;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const bf16x8 va = *reinterpret_cast<const bf16x8*>(vrow + 32 * kb + 16 * t);
              acc[db] = mfma_32x32x16(va, pB[kb][t], acc[db]);
              acc[db] = mfma_32x32x16(va, pL[kb][t], acc[db]);
            }
        }
      }
    }
    if (n + 1 < ntiles) {
      bf16* nb = smem + (cur ^ 1) * S::BUF;
      ld.stage(nb, nb + S::K_ELEMS);
    }
    __syncthreads();
  }

  // ---- epilogue: O / l (bf16, round to nearest even) and the natural-log LSE. The output row
  // index is taken through an empty asm, so that its address is computed here rather than kept
  // live (in registers the tile loop needs) from before the loop.
  const float l_row = l + __shfl_xor(l, 32, kWave);
  int orow_i = q0 + qrow_i;
  asm volatile("" : "+v"(orow_i));
  if (wave_active && qrow_i < Lq) {
    const float inv = (l_row > 0.f) ? vscale / l_row : 0.f;
    bf16* orow = p.out + ((size_t)orow_i * p.Hq + head) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        f32x4 o4 = f32x4{acc[db][4 * rb], acc[db][4 * rb + 1], acc[db][4 * rb + 2], acc[db][4 * rb + 3]} * inv;
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * rb + 4 * hh) = f32x4_to_bf16x4(o4);
      }
    if (p.lse && hh == 0)
      p.lse[(size_t)orow_i * p.Hq + head] = (l_row > 0.f) ? kLn2 * (mc + fast_log2(l_row)) : kNegInf;
  }
}

}  // namespace attn
