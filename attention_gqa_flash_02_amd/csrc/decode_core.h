// Split-KV paged decode for gfx950: one workgroup = (request, kv head, KV partition).
//
// What it computes ("Attention kernels", section "Prefill and decode attention"):
// the few query rows of a request that share one KV head (g query heads x Lq
// new tokens, at most 16 rows) attend over the request's paged cache; each KV
// head is read once for all of them, and the key axis is cut into partitions
// whose results are later merged with their log-sum-exps (same rule as the
// online softmax). Pages are located through the block table ("Optimization 1",
// section 3.4; "Attention kernels", section "Paged KV and kernels").
//
// Work layout inside a workgroup (4 waves):
//   * the partition is walked in 64-token chunks; wave w takes chunks w, w+4, ...
//   * per chunk, S^T = K . Q^T on 16x16x32 MFMA (4 sub-tiles of 16 keys; the 16
//     query rows are the MFMA columns), then an online-softmax update in
//     registers, then O^T += V^T . P^T on 16x16x16 MFMA. V pages are stored
//     token-innermost ([D][block_size]), so the V^T operand is read straight
//     from HBM with the key axis contiguous in each lane; P^T is the S^T
//     accumulator itself (no shuffle, no LDS).
//   * the key held by A-row i of sub-tile u is chunk token 16*(i/4) + 4*u + i%4,
//     so that C-row 4*q + s (lane quad q, accumulator s) of sub-tile u is token
//     16*q + 4*u + s: each lane quad then owns a contiguous 16-token run, which
//     is what its V^T loads need.
//   * the four waves' (max, sum, O) are combined in LDS in a fixed order.
#pragma once

#include "common.h"

namespace attn {

enum { KV_BF16 = 0, KV_FP8 = 1 };

struct PagedParams {
  const bf16* q;               // [Tq, Hq, D]
  const void* k_cache;         // [num_blocks, Hkv, bs, D]
  const void* v_cache;         // [num_blocks, Hkv, D, bs]
  const float* k_scale;        // [Hkv] (fp8) or nullptr
  const float* v_scale;        // [Hkv] (fp8) or nullptr
  const int32_t* block_table;  // [B, max_blocks]
  const int32_t* seq_lens_k;   // [B]
  const int32_t* cu_seqlens_q; // [B + 1], or nullptr: request b owns q row b
  bf16* out;                   // [Tq, Hq, D]
  float* lse;                  // [Tq, Hq] or nullptr
  float* ws_o;                 // [B, Hkv, S, 16, D] partial outputs (normalised)
  float* ws_lse;               // [B, Hkv, S, 16] partial natural-log LSEs
  unsigned* counters;          // [B, Hkv] finished-partition counters (zero between calls)
  float scale;
  int num_seqs, Hq, Hkv, g, bs, max_blocks, num_splits, split_tokens, causal;
};

template <int D>
__device__ void merge_unit(const PagedParams& p, int b, int kvh);

// Rows of a request on this path: r -> (new token r / g, query head kvh*g + r % g).
template <int D, int KVT>
__device__ __forceinline__ void decode_unit(const PagedParams& p, int b, int kvh, int split,
                                            float* lds) {
  constexpr int KK = D / 32;        // QK MFMAs per 16-key sub-tile
  constexpr int NB = D / 16;        // 16-wide d blocks of O^T
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane & 15;          // MFMA column (query row) / A-row (key) index
  const int qd = lane >> 4;         // lane quad

  const int len = p.seq_lens_k[b];
  const int q0 = p.cu_seqlens_q ? p.cu_seqlens_q[b] : b;
  const int qlen = p.cu_seqlens_q ? (p.cu_seqlens_q[b + 1] - q0) : 1;
  const int R = qlen * p.g;
  const int C = p.split_tokens;
  const int n_splits_b = (len + C - 1) / C;          // non-empty partitions of this request
  if (split >= (n_splits_b > 0 ? n_splits_b : 1)) return;
  const bool direct = (n_splits_b <= 1);              // write out/lse here, no merge needed
  const int t_begin = split * C;
  const int t_end = min(len, t_begin + C);

  float kscale = 1.f, vscale = 1.f;
  if (KVT == KV_FP8) { kscale = p.k_scale[kvh]; vscale = p.v_scale[kvh]; }
  const float c = p.scale * kscale * kLog2e;           // base-2 exponent per raw score unit

  // ---- Q^T operands (B of the QK MFMA): lane (j = row, qd) holds Q[row][d-slots].
  bf16x8 qB[KK];
  int limit;                                          // last visible key of row j
  {
    const int r = j;
    const int i = (r < R) ? r / p.g : 0;
    limit = p.causal ? (len - qlen + i) : (len - 1);
    if (r < R) {
      const int h = kvh * p.g + (r % p.g);
      const bf16* qrow = p.q + ((size_t)(q0 + i) * p.Hq + h) * D;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        // bf16 cache: natural d order; fp8 cache: d = 64*(kk/2) + 16*qd + 8*(kk%2), so one
        // 16-byte fp8 load feeds two MFMAs. Q uses the same order as K.
        const int d0 = (KVT == KV_BF16) ? (32 * kk + 8 * qd) : (64 * (kk >> 1) + 16 * qd + 8 * (kk & 1));
        qB[kk] = *reinterpret_cast<const bf16x8*>(qrow + d0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qB[kk] = bf16x8{};
    }
  }

  float m = kNegInf;        // running max of raw scores of row j (same in all 4 quads)
  float l = 0.f;            // this lane's share of the running exp-sum
  f32x4 acc[NB];            // O^T[16n + 4qd + s][row j]
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t head_stride_k = (size_t)p.bs * D;    // elements per (block, kv head) page
  const int32_t* table = p.block_table + (size_t)b * p.max_blocks;
  const int elt = (KVT == KV_BF16) ? 2 : 1;
  const char* kc = reinterpret_cast<const char*>(p.k_cache);
  const char* vc = reinterpret_cast<const char*>(p.v_cache);

  for (int T0 = t_begin + 64 * wave; T0 < t_end; T0 += 256) {
    // ---------------- K: lane (j, qd) reads key 16*(j/4) + 4u + j%4 of the chunk.
    const int ka = j >> 2;
    const int ktok_blk = T0 + 16 * ka;                 // first token of the lane's 16-key run
    const bool kvalid = ktok_blk < len;
    bf16x8 kA[4][KK];
    if (kvalid) {
      const int phys = table[ktok_blk / p.bs];
      const int slot0 = ktok_blk % p.bs + (j & 3);
      const char* kpage = kc + ((size_t)phys * p.Hkv + kvh) * head_stride_k * elt;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const char* krow = kpage + (size_t)(slot0 + 4 * u) * D * elt;
        if (KVT == KV_BF16) {
#pragma unroll
          for (int kk = 0; kk < KK; ++kk)
            kA[u][kk] = bitcast<bf16x8>(ld16(krow + (32 * kk + 8 * qd) * 2));
        } else {
#pragma unroll
          for (int mm = 0; mm < KK / 2; ++mm) {
            u32x4 w = ld16(krow + 64 * mm + 16 * qd);
            kA[u][2 * mm] = fp8x8_to_bf16x8(w[0], w[1]);
            kA[u][2 * mm + 1] = fp8x8_to_bf16x8(w[2], w[3]);
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) kA[u][kk] = bf16x8{};
    }

    // ---------------- V^T: lane (j = d % 16, qd) reads tokens 16*qd .. 16*qd+15 of the chunk.
    const int vtok_blk = T0 + 16 * qd;
    const bool vvalid = vtok_blk < len;
    const int vlimit = len - vtok_blk;                  // tokens of the run that exist
    bf16x4 vA[NB][4];
    if (vvalid) {
      const int phys = table[vtok_blk / p.bs];
      const int slot0 = vtok_blk % p.bs;
      const char* vpage = vc + ((size_t)phys * p.Hkv + kvh) * head_stride_k * elt;
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const char* vrow = vpage + ((size_t)(16 * n + j) * p.bs + slot0) * elt;
        if (KVT == KV_BF16) {
          u32x4 w0 = ld16(vrow);
          u32x4 w1 = ld16(vrow + 16);
          vA[n][0] = bitcast<bf16x4>(u32x2{w0[0], w0[1]});
          vA[n][1] = bitcast<bf16x4>(u32x2{w0[2], w0[3]});
          vA[n][2] = bitcast<bf16x4>(u32x2{w1[0], w1[1]});
          vA[n][3] = bitcast<bf16x4>(u32x2{w1[2], w1[3]});
        } else {
          u32x4 w = ld16(vrow);
#pragma unroll
          for (int u = 0; u < 4; ++u) vA[n][u] = fp8x4_to_bf16x4(w[u]);
        }
      }
      if (vlimit < 16) {                                // tail: zero keys past the end
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int s = 0; s < 4; ++s)
              if (4 * u + s >= vlimit) vA[n][u][s] = (bf16)0.f;
      }
    } else {
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int u = 0; u < 4; ++u) vA[n][u] = bf16x4{};
    }

    // ---------------- S^T = K . Q^T for the 4 sub-tiles; mask; chunk max.
    f32x4 st[4];
    float mloc = kNegInf;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) a = mfma_16x16x32(kA[u][kk], qB[kk], a);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int tok = T0 + 16 * qd + 4 * u + s;
        a[s] = (tok <= limit) ? a[s] : kNegInf;
        mloc = fmaxf(mloc, a[s]);
      }
      st[u] = a;
    }
    const float m_new = fmaxf(m, max_over_quads(mloc));
    const float base = (m_new == kNegInf) ? 0.f : m_new * c;
    const float alpha = (m == kNegInf) ? 0.f : fast_exp2(m * c - base);
    m = m_new;

    // ---------------- P = exp2(c*s - c*m), running sum, rescale, O^T += V^T P^T.
    // P in bf16 for the MFMA; on the request's last chunk (the only chunk of a short request)
    // P is carried as hi + lo bf16 parts so its rounding does not dominate when few keys exist.
    const bool split_p = (T0 + 64 >= len);
    bf16x4 pB[4], pL[4];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f32x4 pv;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        pv[s] = fast_exp2(__builtin_fmaf(st[u][s], c, -base));
        psum += pv[s];
      }
      pB[u] = f32x4_to_bf16x4(pv);
      f32x4 lo;
#pragma unroll
      for (int s = 0; s < 4; ++s) lo[s] = pv[s] - (float)pB[u][s];
      pL[u] = f32x4_to_bf16x4(lo);
    }
    l = l * alpha + psum;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      acc[n] *= alpha;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[n] = mfma_16x16x16(vA[n][u], pB[u], acc[n]);
        if (split_p) acc[n] = mfma_16x16x16(vA[n][u], pL[u], acc[n]);
      }
    }
  }

  // ---------------- combine the four waves (fixed order) through LDS.
  // lds layout: stats[2][4][16] (max, sum) then O[4][R][D].
  float* smax = lds;
  float* ssum = lds + 64;
  float* so = lds + 128;
  const float l_row = sum_over_quads(l);
  if (qd == 0) {
    smax[wave * 16 + j] = m;
    ssum[wave * 16 + j] = l_row;
  }
  __syncthreads();
  float mx = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) mx = fmaxf(mx, smax[w * 16 + j]);
  const float mbase = (mx == kNegInf) ? 0.f : mx * c;
  float ltot = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = smax[w * 16 + j];
    ltot += (mw == kNegInf) ? 0.f : ssum[w * 16 + j] * fast_exp2(mw * c - mbase);
  }
  const float own = (m == kNegInf || ltot == 0.f) ? 0.f : fast_exp2(m * c - mbase) * vscale / ltot;
  if (j < R) {
    float* dst = so + ((size_t)wave * R + j) * D;
#pragma unroll
    for (int n = 0; n < NB; ++n) *reinterpret_cast<f32x4*>(dst + 16 * n + 4 * qd) = acc[n] * own;
  }
  __syncthreads();

  const float row_lse = (ltot == 0.f) ? kNegInf : kLn2 * (mx * c + fast_log2(ltot));
  if (direct) {
    for (int idx = tid; idx < R * D; idx += blockDim.x) {
      const int r = idx / D, d = idx - r * D;
      const float o = so[(0 * R + r) * D + d] + so[(1 * R + r) * D + d] + so[(2 * R + r) * D + d] +
                      so[(3 * R + r) * D + d];
      const int i = r / p.g, h = kvh * p.g + r % p.g;
      p.out[((size_t)(q0 + i) * p.Hq + h) * D + d] = (bf16)o;
    }
    if (p.lse && wave == 0 && qd == 0 && j < R) {
      const int i = j / p.g, h = kvh * p.g + j % p.g;
      p.lse[(size_t)(q0 + i) * p.Hq + h] = row_lse;
    }
  } else {
    const size_t unit = ((size_t)b * p.Hkv + kvh) * p.num_splits + split;
    float* wo = p.ws_o + unit * 16 * D;
    for (int idx = tid; idx < R * D; idx += blockDim.x) {
      const int r = idx / D, d = idx - r * D;
      wo[idx] = so[(0 * R + r) * D + d] + so[(1 * R + r) * D + d] + so[(2 * R + r) * D + d] +
                so[(3 * R + r) * D + d];
    }
    if (wave == 0 && qd == 0 && j < R) p.ws_lse[unit * 16 + j] = row_lse;
    // The last partition of this (request, kv head) to finish merges all of them. atomicInc
    // wraps at n_splits_b - 1, so the counter is back at zero once every partition has counted.
    __threadfence();
    __syncthreads();
    int* flag = reinterpret_cast<int*>(lds);
    if (tid == 0) {
      const unsigned old = atomicInc(p.counters + (size_t)b * p.Hkv + kvh, (unsigned)(n_splits_b - 1));
      *flag = (old == (unsigned)(n_splits_b - 1));
    }
    __syncthreads();
    if (*flag) {
      __threadfence();
      merge_unit<D>(p, b, kvh);
    }
  }
}

// Merge of the partitions of one (request, kv head): natural-log LSE weights.
template <int D>
__device__ void merge_unit(const PagedParams& p, int b, int kvh) {
  const int len = p.seq_lens_k[b];
  const int q0 = p.cu_seqlens_q ? p.cu_seqlens_q[b] : b;
  const int qlen = p.cu_seqlens_q ? (p.cu_seqlens_q[b + 1] - q0) : 1;
  const int R = qlen * p.g;
  if (R > 16) return;                                  // rows written by the prefill path
  const int C = p.split_tokens;
  const int ns = (len + C - 1) / C;
  if (ns <= 1) return;                                 // written directly by the split kernel
  const size_t unit0 = ((size_t)b * p.Hkv + kvh) * p.num_splits;
  for (int idx = threadIdx.x; idx < R * (D / 4); idx += blockDim.x) {
    const int r = idx / (D / 4);
    const int d4 = (idx - r * (D / 4)) * 4;
    float mx = kNegInf;
    for (int s = 0; s < ns; ++s) mx = fmaxf(mx, p.ws_lse[(unit0 + s) * 16 + r]);
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (mx != kNegInf) {
      for (int s = 0; s < ns; ++s) {
        const float ls = p.ws_lse[(unit0 + s) * 16 + r];
        const float w = (ls == kNegInf) ? 0.f : fast_exp2((ls - mx) * kLog2e);
        const f32x4 os = *reinterpret_cast<const f32x4*>(p.ws_o + ((unit0 + s) * 16 + r) * D + d4);
        o += os * w;
        wsum += w;
      }
    }
    const float inv = (wsum > 0.f) ? 1.f / wsum : 0.f;
    const int i = r / p.g, h = kvh * p.g + r % p.g;
    bf16* dst = p.out + ((size_t)(q0 + i) * p.Hq + h) * D + d4;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = (bf16)(o[e] * inv);
    if (p.lse && d4 == 0)
      p.lse[(size_t)(q0 + i) * p.Hq + h] = (wsum > 0.f) ? mx + kLn2 * fast_log2(wsum) : kNegInf;
  }
}

}  // namespace attn
