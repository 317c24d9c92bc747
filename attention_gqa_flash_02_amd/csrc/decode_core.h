// Split-KV paged decode for gfx950: one workgroup = (request, kv head, KV partition).
//
// What it computes ("Attention kernels", section "Prefill and decode attention"):
// the few query rows of a request that share one KV head (g query heads x Lq
// new tokens, at most 16 rows) attend over the request's paged cache; each KV
// head is read once for all of them, and the key axis is cut into partitions
// whose results are merged with their log-sum-exps (the same rule as the
// online softmax). Pages are located through the block table ("Optimization
// 1", section 3.4; "Attention kernels", section "Paged KV and kernels").
//
// Work layout inside a workgroup (4 waves):
//   * the partition is walked in chunks of CH = 16*NU tokens; wave w takes
//     chunks w, w+4, ...
//   * per chunk, S^T = K . Q^T on 16x16x32 MFMA (NU sub-tiles of 16 keys; the
//     16 query rows are the MFMA columns), an online-softmax update in
//     registers, then O^T += V^T . P^T on 16x16x16 MFMA. V pages are stored
//     token-innermost ([D][block_size]), so the V^T operand comes straight from
//     HBM with the key axis contiguous in each lane; P^T is the S^T accumulator
//     itself (no shuffle, no LDS).
//   * the key held by A-row i of sub-tile u is chunk token RUN*(i/4) + 4*u + i%4
//     (RUN = 4*NU), so that C-row 4*q + s of sub-tile u is token RUN*q + 4*u + s:
//     each lane quad then owns one contiguous RUN-token run, which is what its
//     V^T loads need, and a run never crosses a page (block sizes are >= 16).
//   * memory: the block-table entries of the next chunk are loaded while the
//     current chunk computes, and the K and V loads of a chunk are issued back
//     to back with no wait in between. Loads past the end of the request are
//     redirected into its last page (always a valid address) and their values
//     masked, so no load sits behind a branch.
//   * the four waves' (max, sum, O) are combined in LDS in a fixed order. A
//     request that needs one partition writes out/lse directly; otherwise each
//     partition writes a normalised partial and its LSE, and a second small
//     kernel merges them.
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
  float scale;
  int num_seqs, Hq, Hkv, g, bs, max_blocks, num_splits, split_tokens, causal;
};

template <int NU>
struct DecodeShape {
  static constexpr int CH = 16 * NU;   // tokens per wave iteration
  static constexpr int RUN = 4 * NU;   // consecutive tokens owned by one lane quad
};

// Rows of a request on this path: r -> (new token r / g, query head kvh*g + r % g).
template <int D, int KVT, int NU>
__device__ __forceinline__ void decode_unit(const PagedParams& p, int b, int kvh, int split, float* lds) {
  constexpr int CH = DecodeShape<NU>::CH;
  constexpr int RUN = DecodeShape<NU>::RUN;
  constexpr int KK = D / 32;        // QK MFMAs per 16-key sub-tile
  constexpr int NB = D / 16;        // 16-wide d blocks of O^T
  constexpr int ELT = (KVT == KV_BF16) ? 2 : 1;
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

  const size_t page_elems = (size_t)p.bs * D;         // elements per (block, kv head) page
  const int32_t* table = p.block_table + (size_t)b * p.max_blocks;
  const char* kc = reinterpret_cast<const char*>(p.k_cache);
  const char* vc = reinterpret_cast<const char*>(p.v_cache);
  const int last_tok = len - 1;

  // Block-table entries of a chunk: lane (j, qd) reads keys from the run at RUN*(j/4) (K) and
  // the run at RUN*qd (V). Runs past the end of the request read its last page instead.
  auto k_block = [&](int T0) { return min(T0 + RUN * (j >> 2), last_tok) / p.bs; };
  auto v_block = [&](int T0) { return min(T0 + RUN * qd, last_tok) / p.bs; };

  int T0 = t_begin + CH * wave;
  int kphys = 0, vphys = 0;
  if (T0 < t_end) {
    kphys = table[k_block(T0)];
    vphys = table[v_block(T0)];
  }

  for (; T0 < t_end; T0 += 4 * CH) {
    // ---------------- issue the K and V loads of this chunk
    const int kt = T0 + RUN * (j >> 2);                 // first token of the lane's K run
    const int kslot = kt % p.bs;                        // the run never crosses a page
    const char* kpage = kc + ((size_t)kphys * p.Hkv + kvh) * page_elems * ELT;
    constexpr int KW = (KVT == KV_BF16) ? KK : KK / 2;  // 16-byte K loads per key row
    u32x4 kraw[NU][KW];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const char* krow = kpage + (size_t)(kslot + 4 * u + (j & 3)) * D * ELT;
#pragma unroll
      for (int w = 0; w < KW; ++w)
        kraw[u][w] = (KVT == KV_BF16) ? ld16(krow + (32 * w + 8 * qd) * 2) : ld16(krow + 64 * w + 16 * qd);
    }
    const int vt = T0 + RUN * qd;                       // first token of the lane's V run
    const int vslot = vt % p.bs;
    const char* vpage = vc + ((size_t)vphys * p.Hkv + kvh) * page_elems * ELT;
    constexpr int VW = RUN * ELT / 4;                   // dwords of one lane's V run per d row
    uint32_t vraw[NB][VW];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const char* vrow = vpage + ((size_t)(16 * n + j) * p.bs + vslot) * ELT;
      if constexpr (VW == 8) {
        const u32x4 w0 = ld16(vrow), w1 = ld16(vrow + 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) { vraw[n][e] = w0[e]; vraw[n][4 + e] = w1[e]; }
      } else if constexpr (VW == 4) {
        const u32x4 w0 = ld16(vrow);
#pragma unroll
        for (int e = 0; e < 4; ++e) vraw[n][e] = w0[e];
      } else {
        const u32x2 w0 = ld8(vrow);
        vraw[n][0] = w0[0];
        vraw[n][1] = w0[1];
      }
    }
    // ---------------- block-table entries of this wave's next chunk
    const int Tn = T0 + 4 * CH;
    if (Tn < t_end) {
      kphys = table[k_block(Tn)];
      vphys = table[v_block(Tn)];
    }

    // ---------------- S^T = K . Q^T for the NU sub-tiles; mask; chunk max.
    f32x4 st[NU];
    float mloc = kNegInf;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
      if (KVT == KV_BF16) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) a = mfma_16x16x32(bitcast<bf16x8>(kraw[u][kk]), qB[kk], a);
      } else {
#pragma unroll
        for (int w = 0; w < KW; ++w) {
          a = mfma_16x16x32(fp8x8_to_bf16x8(kraw[u][w][0], kraw[u][w][1]), qB[2 * w], a);
          a = mfma_16x16x32(fp8x8_to_bf16x8(kraw[u][w][2], kraw[u][w][3]), qB[2 * w + 1], a);
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int tok = T0 + RUN * qd + 4 * u + s;
        a[s] = (tok <= limit) ? a[s] : kNegInf;
        mloc = fmaxf(mloc, a[s]);
      }
      st[u] = a;
    }
    const float m_new = fmaxf(m, max_over_quads(mloc));
    const float base = (m_new == kNegInf) ? 0.f : m_new * c;
    const float alpha = (m == kNegInf) ? 0.f : fast_exp2(m * c - base);
    m = m_new;

    // ---------------- P = exp2(c*s - c*m), running sum.
    // P is rounded to bf16 for the MFMA. On the request's last chunk (the only chunk of a short
    // request) P is carried as hi + lo bf16 parts, so that its rounding does not dominate the
    // output error when only a few keys exist.
    const bool split_p = (T0 + CH >= len);
    bf16x4 pB[NU], pL[NU];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
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

    // ---------------- V^T operands; keys past the end of the request are zeroed (their P is
    // zero, but the slots may hold anything, including NaN).
    const int vvalid = len - vt;                        // tokens of the lane's run that exist
    // ---------------- O^T = alpha * O^T + V^T . P^T
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      acc[n] *= alpha;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        bf16x4 va;
        if (KVT == KV_BF16) {
          va = bitcast<bf16x4>(u32x2{vraw[n][2 * u], vraw[n][2 * u + 1]});
        } else {
          va = fp8x4_to_bf16x4(vraw[n][u]);
        }
        if (vvalid < RUN) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            if (4 * u + s >= vvalid) va[s] = (bf16)0.f;
        }
        acc[n] = mfma_16x16x16(va, pB[u], acc[n]);
        if (split_p) acc[n] = mfma_16x16x16(va, pL[u], acc[n]);
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
    for (int idx = tid; idx < R * (D / 4); idx += blockDim.x) {
      const int r = idx / (D / 4), d4 = 4 * (idx - r * (D / 4));
      f32x4 o = *reinterpret_cast<const f32x4*>(so + (0 * R + r) * D + d4);
#pragma unroll
      for (int w = 1; w < 4; ++w) o += *reinterpret_cast<const f32x4*>(so + (w * R + r) * D + d4);
      const int i = r / p.g, h = kvh * p.g + r % p.g;
      *reinterpret_cast<bf16x4*>(p.out + ((size_t)(q0 + i) * p.Hq + h) * D + d4) = f32x4_to_bf16x4(o);
    }
    if (p.lse && wave == 0 && qd == 0 && j < R) {
      const int i = j / p.g, h = kvh * p.g + j % p.g;
      p.lse[(size_t)(q0 + i) * p.Hq + h] = row_lse;
    }
  } else {
    const size_t unit = ((size_t)b * p.Hkv + kvh) * p.num_splits + split;
    float* wo = p.ws_o + unit * 16 * D;
    for (int idx = tid; idx < R * (D / 4); idx += blockDim.x) {
      const int r = idx / (D / 4), d4 = 4 * (idx - r * (D / 4));
      f32x4 o = *reinterpret_cast<const f32x4*>(so + (0 * R + r) * D + d4);
#pragma unroll
      for (int w = 1; w < 4; ++w) o += *reinterpret_cast<const f32x4*>(so + (w * R + r) * D + d4);
      *reinterpret_cast<f32x4*>(wo + r * D + d4) = o;
    }
    if (wave == 0 && qd == 0 && j < R) p.ws_lse[unit * 16 + j] = row_lse;
  }
}

// Merge of the partitions of one (request, kv head, row): natural-log LSE weights
// ("Attention kernels", section "Prefill and decode attention": partial results combined the
// same way as the online softmax). 256 threads: thread t sums d-quad t % (D/4) over the
// partitions s = t / (D/4), t / (D/4) + 256/(D/4), ...; the groups are then added in LDS in a
// fixed order. lds: weights[num_splits] then sums[256/(D/4)][D].
template <int D>
__device__ __forceinline__ void merge_row(const PagedParams& p, int b, int kvh, int r, float* lds) {
  constexpr int DQ = D / 4;
  constexpr int GROUPS = 256 / DQ;
  const int len = p.seq_lens_k[b];
  const int q0 = p.cu_seqlens_q ? p.cu_seqlens_q[b] : b;
  const int qlen = p.cu_seqlens_q ? (p.cu_seqlens_q[b + 1] - q0) : 1;
  const int R = qlen * p.g;
  if (R > 16 || r >= R) return;                        // rows written by other paths
  const int C = p.split_tokens;
  const int ns = (len + C - 1) / C;
  if (ns <= 1) return;                                 // written directly by the partition kernel
  const int tid = threadIdx.x;
  const size_t unit0 = ((size_t)b * p.Hkv + kvh) * p.num_splits;
  float* w = lds;
  float* red = lds + p.num_splits;
  __shared__ float s_max, s_sum;
  if (tid < 64) {
    float mx = kNegInf;
    for (int s = tid; s < ns; s += 64) mx = fmaxf(mx, p.ws_lse[(unit0 + s) * 16 + r]);
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    float sum = 0.f;
    for (int s = tid; s < ns; s += 64) {
      const float ls = p.ws_lse[(unit0 + s) * 16 + r];
      const float e = (mx == kNegInf || ls == kNegInf) ? 0.f : fast_exp2((ls - mx) * kLog2e);
      w[s] = e;
      sum += e;
    }
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
    if (tid == 0) { s_max = mx; s_sum = sum; }
  }
  __syncthreads();
  const int dq = tid % DQ, grp = tid / DQ;
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = grp; s < ns; s += GROUPS) {
    const f32x4 os = *reinterpret_cast<const f32x4*>(p.ws_o + ((unit0 + s) * 16 + r) * D + 4 * dq);
    o += os * w[s];
  }
  *reinterpret_cast<f32x4*>(red + grp * D + 4 * dq) = o;
  __syncthreads();
  if (grp == 0) {
    for (int g2 = 1; g2 < GROUPS; ++g2) o += *reinterpret_cast<const f32x4*>(red + g2 * D + 4 * dq);
    const float inv = (s_sum > 0.f) ? 1.f / s_sum : 0.f;
    const int i = r / p.g, h = kvh * p.g + r % p.g;
    *reinterpret_cast<bf16x4*>(p.out + ((size_t)(q0 + i) * p.Hq + h) * D + 4 * dq) = f32x4_to_bf16x4(o * inv);
    if (p.lse && dq == 0)
      p.lse[(size_t)(q0 + i) * p.Hq + h] = (s_sum > 0.f) ? s_max + kLn2 * fast_log2(s_sum) : kNegInf;
  }
}

}  // namespace attn
