// Tiled causal/non-causal varlen prefill for gfx950 on bf16 MFMA.
//
// What it computes ("Attention kernels", section "FlashAttention"): Q, K and V
// are cut into tiles; each workgroup keeps its query rows in registers,
// streams K/V tiles through LDS, and per tile computes the scores, updates each
// row's running maximum and exponential sum (rescaling what it has accumulated
// when the maximum moves) and accumulates P V. Only O and one log-sum-exp per
// row are written; the score matrix never leaves the chip.
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
//     then accumulator r of lane half h holds key 16*(r/8) + 8*h + r%8, and the
//     8 k-slots a lane feeds to the P V MFMA are 8 consecutive keys: V^T is
//     read from LDS with one 16-byte read per MFMA operand.
//   * O^T += V^T P^T on 32x32x16 MFMA, P^T being the bf16-rounded S^T
//     accumulator (no shuffle, no LDS round trip for P).
//   * K tiles are stored row-major in LDS, V tiles transposed ([d][key]); row
//     strides are padded by 16 bytes so that the MFMA operand reads are free of
//     bank conflicts. LDS is double-buffered: tile n+1 is fetched into
//     registers while tile n is computed.
#pragma once

#include "common.h"

namespace attn {

struct PrefillParams {
  const bf16* q;               // [T, Hq, D]
  const bf16* k;               // [T, Hkv, D]
  const bf16* v;               // [T, Hkv, D]
  const int32_t* cu_seqlens;   // [B + 1]
  bf16* out;                   // [T, Hq, D]
  float* lse;                  // [T, Hq] or nullptr
  float scale;
  int num_seqs, Hq, Hkv, g, hpw, causal, num_qtiles;
};

template <int D, int BN>
struct PrefillShape {
  static constexpr int KS = D + 8;                  // K tile row stride in LDS (elements)
  static constexpr int VS = BN + 8;                 // V^T tile row stride in LDS (elements)
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
  static constexpr int LDS_BYTES = 2 * BUF * 2;     // two buffers of bf16
  static constexpr int KCH = D / 8;                 // 16-byte chunks per K row
  static constexpr int K_LOADS = BN * KCH / 256;    // K chunks per thread per tile
  static constexpr int K_ROWS_PER_PASS = 256 / KCH;
  static constexpr int VKG = BN / 4;                // 4-key groups per V tile
  static_assert(VKG * (D / 8) == 256, "V staging assumes one 4x8 block per thread");
  static_assert(BN % 32 == 0, "key tiles are whole 32-key MFMA blocks");
};

// Key loaded by A-row i of a 32-key block: bits 2 and 3 of i swapped.
__device__ __forceinline__ int key_perm32(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

template <int D, int BN>
__device__ __forceinline__ void prefill_tile_body(const PrefillParams& p, bf16* smem, int hgrp, int b,
                                                  int qt) {
  using S = PrefillShape<D, BN>;
  constexpr int NKB = BN / 32;      // 32-key blocks per tile
  constexpr int NDB = D / 32;       // 32-wide d blocks of O^T
  constexpr int NKK = D / 16;       // k-steps of the QK MFMA
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
  const int seq0 = p.cu_seqlens[b];
  const int L = p.cu_seqlens[b + 1] - seq0;
  const int t0 = qt * TQ;
  if (t0 >= L) return;
  const int tw = t0 + 32 * (wave / p.hpw);               // first token of this wave
  const bool wave_active = tw < L;
  const int kv_end = p.causal ? min(L, t0 + TQ) : L;     // keys any row of the workgroup sees
  const int ntiles = (kv_end + BN - 1) / BN;
  const int wave_kv_end = p.causal ? min(L, tw + 32) : L;
  const float c = p.scale * kLog2e;

  // ---- Q^T operands: lane (j, hh) holds Q[token tw + j][16*kk + 8*hh .. +7].
  bf16x8 qB[NKK];
  const int qtok = tw + j;
  if (qtok < L) {
    const bf16* qrow = p.q + ((size_t)(seq0 + qtok) * p.Hq + head) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qB[kk] = *reinterpret_cast<const bf16x8*>(qrow + 16 * kk + 8 * hh);
  } else {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qB[kk] = bf16x8{};
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m = kNegInf, l = 0.f;

  // ---- staging registers
  u32x4 kreg[S::K_LOADS];
  u32x4 vreg[4];
  const int kch = tid % S::KCH;
  const int krow0 = tid / S::KCH;
  const int vkg = tid % S::VKG;
  const int vdc = tid / S::VKG;
  const size_t kv_stride = (size_t)p.Hkv * D;
  const bf16* kbase = p.k + (size_t)seq0 * kv_stride + (size_t)kvh * D;
  const bf16* vbase = p.v + (size_t)seq0 * kv_stride + (size_t)kvh * D;

  auto fetch = [&](int n) {
    const int n0 = n * BN;
#pragma unroll
    for (int it = 0; it < S::K_LOADS; ++it) {
      const int key = n0 + it * S::K_ROWS_PER_PASS + krow0;
      kreg[it] = (key < L) ? ld16(kbase + (size_t)key * kv_stride + 8 * kch) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int key = n0 + 4 * vkg + s;
      vreg[s] = (key < L) ? ld16(vbase + (size_t)key * kv_stride + 8 * vdc) : u32x4{0, 0, 0, 0};
    }
  };
  auto stage = [&](int buf) {
    bf16* Ks = smem + buf * S::BUF;
    bf16* Vt = Ks + S::K_ELEMS;
#pragma unroll
    for (int it = 0; it < S::K_LOADS; ++it)
      *reinterpret_cast<u32x4*>(Ks + (it * S::K_ROWS_PER_PASS + krow0) * S::KS + 8 * kch) = kreg[it];
    // transpose the 4 keys x 8 d block: d-row 8*vdc + e gets keys 4*vkg .. 4*vkg+3
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo01 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x05040100u);
      const uint32_t lo23 = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x07060302u);
      const uint32_t hi23 = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x07060302u);
      *reinterpret_cast<u32x2*>(Vt + (8 * vdc + 2 * w) * S::VS + 4 * vkg) = u32x2{lo01, lo23};
      *reinterpret_cast<u32x2*>(Vt + (8 * vdc + 2 * w + 1) * S::VS + 4 * vkg) = u32x2{hi01, hi23};
    }
  };

  fetch(0);
  stage(0);
  __syncthreads();
  const int kperm = key_perm32(j);

  for (int n = 0; n < ntiles; ++n) {
    const int cur = n & 1;
    if (n + 1 < ntiles) fetch(n + 1);
    const int n0 = n * BN;
    if (wave_active && n0 < wave_kv_end) {
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
      // mask (only tiles that cross the diagonal or the sequence end)
      const bool need_mask = (n0 + BN > L) || (p.causal && n0 + BN - 1 > tw);
      if (need_mask) {
        const int lim = p.causal ? min(qtok, L - 1) : (L - 1);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = n0 + 32 * kb + 16 * (r >> 3) + 8 * hh + (r & 7);
            st[kb][r] = (key <= lim) ? st[kb][r] : kNegInf;
          }
      }
      float mloc = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, st[kb][r]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
      const float m_new = fmaxf(m, mloc);
      const float base = (m_new == kNegInf) ? 0.f : m_new * c;
      const float alpha = (m == kNegInf) ? 0.f : fast_exp2(m * c - base);
      m = m_new;
      // P in bf16 for the MFMA. On tiles that cross the diagonal or the sequence end the rows
      // see few keys, so the rounding of P would not average out: there P is carried as
      // hi + lo bf16 parts and multiplied into V twice.
      bf16x8 pB[NKB][2], pL[NKB][2];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          bf16x8 pv, pl;
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const float e = fast_exp2(__builtin_fmaf(st[kb][8 * t + s], c, -base));
            psum += e;
            pv[s] = (bf16)e;
            pl[s] = (bf16)(e - (float)pv[s]);
          }
          pB[kb][t] = pv;
          pL[kb][t] = pl;
        }
      l = l * alpha + psum;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        acc[db] *= alpha;
        const bf16* vrow = Vt + (32 * db + j) * S::VS + 8 * hh;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(vrow + 32 * kb + 16 * t);
            acc[db] = mfma_32x32x16(va, pB[kb][t], acc[db]);
            if (need_mask) acc[db] = mfma_32x32x16(va, pL[kb][t], acc[db]);
          }
      }
    }
    if (n + 1 < ntiles) stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / l (bf16, round to nearest even) and the natural-log LSE
  const float l_row = l + __shfl_xor(l, 32, kWave);
  if (wave_active && qtok < L) {
    const float inv = (l_row > 0.f) ? 1.f / l_row : 0.f;
    bf16* orow = p.out + ((size_t)(seq0 + qtok) * p.Hq + head) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        f32x4 o4 = f32x4{acc[db][4 * rb], acc[db][4 * rb + 1], acc[db][4 * rb + 2], acc[db][4 * rb + 3]} * inv;
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * rb + 4 * hh) = f32x4_to_bf16x4(o4);
      }
    if (p.lse && hh == 0)
      p.lse[(size_t)(seq0 + qtok) * p.Hq + head] = (l_row > 0.f) ? kLn2 * (m * c + fast_log2(l_row)) : kNegInf;
  }
}

}  // namespace attn
