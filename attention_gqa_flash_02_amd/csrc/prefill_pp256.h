// Ping-pong prefill tile over a paged cache with head_dim 256 (the prefill part of a mixed batch).
// What it computes is the tiled exact attention of prefill_core.h ("Attention kernels", section
// "FlashAttention"): per K/V tile the scores, the running row maximum and exponential sum, and P V;
// only O and the per-row log-sum-exp are written. Causal masking is bottom-right aligned (a chunk of
// Lq new rows over Lk cached keys: row i sees keys j <= Lk - Lq + i), with the optional sliding
// window of prefill_core.h. K/V come from the paged cache (K pages [bs][D], V pages [D][bs], bf16 or
// OCP e4m3fn codes with per-head scales; "Attention kernels", section "Paged KV and kernels").
//
// Work layout. A workgroup is 8 waves in two groups of four (A = waves 0-3, B = 4-7), one wave of
// each group per SIMD, and takes 128 query rows: 4 row blocks of 32 rows (a row block = 32 tokens of
// one query head; the heads of a block set share one KV head, so every K/V tile in LDS serves all
// of them). A row block belongs to a pair of waves of one group (waves 2p and 2p+1 of the group):
// both hold the block's Q^T (the whole head_dim) and compute the same S^T = K Q^T; each accumulates
// one half of O^T (head_dim 0-127 or 128-255). At head_dim 256 a wave cannot hold Q^T (64
// registers), S^T, P and all of O^T (128) within the 256 registers of two waves per SIMD; splitting
// O keeps every wave at two per SIMD, at the price of computing S^T twice (the matrix work per
// useful FLOP is 1.5x). The exponentials are not computed twice: each wave of a pair takes the
// tile's row maximum from the whole S^T but computes P only for its own 16 of the 32 keys, and the
// two halves of P meet in LDS, which shortens the vector work of the slot that sets the pace.
//
// Ping-pong (as in prefill_pp.h). Time is cut into slots that end at a workgroup barrier. In each
// slot one group runs its matrix work (P V of its previous tile, then S^T of its current tile)
// while the other group runs its softmax and stages one tile into LDS, so on every SIMD one wave
// feeds the MFMA pipe while the other feeds the VALU. MFMAs are 32x32x16 bf16 with the key
// permutation of prefill_core.h, so the S^T accumulator is already the B operand of P V.
//
// Tiles are 32 keys. K (32 x 256) and V^T (256 x 32) tiles are bf16 in LDS (rows padded by 16 bytes
// against bank conflicts), three buffers each (tile n in buffer n mod 3). They are staged through
// registers, so fp8 codes are decoded once per workgroup: group A stages K tiles and group B V^T
// tiles, each in its softmax slot. The loads of a tile are issued two slots before its registers
// are decoded and written to LDS:
//   slot 2m   A: P V (m-1), S^T (m)                   B: softmax (m-1); write V (m+1), load V (m+2)
//   slot 2m+1 A: softmax (m); write K (m+2), load K (m+3)   B: P V (m-1), S^T (m)
// K (m+2) goes to buffer (m+2) mod 3 in slot 2m+1, after the last read of K (m-1) (slot 2m-1) and
// before its first read (slot 2m+4); V (m+1) goes to buffer (m+1) mod 3 in slot 2m, after the last
// read of V (m-2) (slot 2m-1) and before its first (slot 2m+4). Every wave runs every tile of its
// workgroup (tiles its rows do not see are masked): the control flow is uniform.
#pragma once

#include "prefill_core.h"

namespace attn {

template <bool FP8>
struct PingPong256Shape {
  static constexpr int D = 256;
  static constexpr int BN = 32;
  static constexpr int KS = D + 8;                  // K row stride in LDS (bf16 elements)
  static constexpr int VS = BN + 8;                 // V^T row stride in LDS (bf16 elements)
  static constexpr int K_BYTES = BN * KS * 2;       // one K tile
  static constexpr int V_BYTES = D * VS * 2;        // one V^T tile
  static constexpr int NBUF = 3;
  static constexpr int XCHG_OFFSET = NBUF * (K_BYTES + V_BYTES);
  static constexpr int XCHG_BYTES = 2 * 8 * 64 * 16;       // P half (hi, lo) per wave and lane
  static constexpr int LDS_BYTES = XCHG_OFFSET + XCHG_BYTES;
  static constexpr int ELT = FP8 ? 1 : 2;
  static constexpr int LOADS = 32 * ELT / 16;       // 16-byte loads per staging thread per tile
};

template <bool FP8>
__device__ __forceinline__ void prefill_pp256_body(const PrefillParams& p, unsigned char* smem, int hgrp, int b,
                                                   int qt) {
  using S = PingPong256Shape<FP8>;
  constexpr int D = 256;
  constexpr int BN = S::BN;
  constexpr int NKK = D / 16;       // k-steps of the QK MFMA (the whole head_dim)
  constexpr int NDB = 4;            // 32-wide d blocks of the wave's half of O^T
  constexpr int ELT = S::ELT;
  constexpr int VPL = 16 / ELT;     // values per 16-byte load
  constexpr int NL = S::LOADS;      // 16-byte loads per staging thread per tile
  constexpr float kLazyRescale = 8.f;
  constexpr float kFastLimit = 4294967296.f;   // 2^32: far inside the bf16 and fp32 ranges
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gp = wave >> 2;
  const int lw = wave & 3;
  const int rblk = 2 * gp + (lw >> 1);   // row block 0..3
  const int dh = lw & 1;                 // half of O^T: head_dim 128 * dh .. + 127
  const int j = lane & 31;
  const int hh = lane >> 5;

  const int groups_per_kv = p.g / p.hpw;
  const int kvh = hgrp / groups_per_kv;
  const int head = kvh * p.g + (hgrp % groups_per_kv) * p.hpw + (rblk % p.hpw);
  const int TQ = 32 * (4 / p.hpw);
  const int q0 = p.cu_seqlens_q[b];
  const int Lq = p.cu_seqlens_q[b + 1] - q0;
  const int Lk = p.seq_lens_k[b];
  const int t0 = qt * TQ;
  if (t0 >= Lq) return;                                  // uniform over the workgroup
  const int tw = t0 + 32 * (rblk / p.hpw);               // first query row of this row block
  const bool wave_active = tw < Lq;
  const int shift = Lk - Lq;                             // row i sees keys <= shift + i (causal)
  const int kv_end = p.causal ? min(Lk, shift + min(Lq, t0 + TQ)) : Lk;
  const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  const int win = p.window;
  const int kv_begin = win > 0 ? max(0, shift + t0 - win + 1) : 0;
  const int wave_lower_max = win > 0 ? shift + tw + 31 - win + 1 : INT_MIN;
  const int n_first = min(kv_begin / BN, ntiles);
  const int N = ntiles - n_first;
  float kscale = 1.f, vscale = 1.f;
  if (FP8) { kscale = p.k_scale[kvh]; vscale = p.v_scale[kvh]; }
  const float c = p.scale * kscale * kLog2e;

  // ---- Q^T operands: lane (j, hh) holds Q[row tw + j][16 kk + 8 hh .. +7] for the whole head_dim
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
  const int lim = p.causal ? min(shift + qrow_i, Lk - 1) : (Lk - 1);
  const int lower = win > 0 ? shift + qrow_i - win + 1 : INT_MIN;
  const int wave_mask_from = p.causal ? max(0, shift + tw + 1) : Lk;

  unsigned char* const kbuf0 = smem;                          // K tiles: [BN][KS] bf16
  unsigned char* const vbuf0 = smem + S::NBUF * S::K_BYTES;   // V^T tiles: [D][VS] bf16

  // ---- staging. Group A thread t (0-255) stages 32 head_dim values of key t / 8 of each K tile:
  // piece i (one 16-byte load) starts at column kcol(t % 8, i), so that the 8 threads of a key
  // read 256 contiguous bytes per pair of loads and the 16 lanes of an LDS write phase (two keys,
  // eight column offsets 32 bytes apart) fall in 16 different bank groups of the padded rows.
  // Group B thread t stages the 32 keys of head_dim row t of each V^T tile.
  // Keys at or past Lk are loaded from a valid page (the last key's) and written as zero.
  const int st_t = tid & 255;
  const int st_key = st_t >> 3;
  auto kcol = [](int cc, int i) {     // first head_dim column of K piece i of staging thread cc
    return FP8 ? 16 * cc + 128 * i : 16 * cc + 8 * (i & 1) + 128 * (i >> 1);
  };
  const size_t page_bytes = (size_t)p.bs * D * ELT;
  const size_t block_stride = (size_t)p.Hkv * page_bytes;
  const char* kc = reinterpret_cast<const char*>(p.k_cache) + (size_t)kvh * page_bytes;
  const char* vc = reinterpret_cast<const char*>(p.v_cache) + (size_t)kvh * page_bytes;
  const int32_t* table = p.block_table + (size_t)b * p.max_blocks;
  const int last = Lk - 1;
  u32x4 sreg[NL];                  // the staged tile in flight
  int sphys[NL];                   // block-table entries of the next tile to load
  // block-table entries of tile n (absolute tile index) for this thread's loads
  auto load_table = [&](int n) {
    const int n0 = n * BN;
    if (gp == 0) {
      sphys[0] = table[min(n0 + st_key, last) >> p.bs_shift];
    } else {
#pragma unroll
      for (int i = 0; i < NL; ++i) sphys[i] = table[min(n0 + VPL * i, last & ~(VPL - 1)) >> p.bs_shift];
    }
  };
  // issue the loads of tile n (the table entries of tile n are in sphys), then fetch tile n+1's
  auto issue = [&](int n) {
    const int n0 = n * BN;
    if (gp == 0) {
      const int key = min(n0 + st_key, last);
      const char* row = kc + (size_t)sphys[0] * block_stride + (size_t)(key & (p.bs - 1)) * D * ELT;
#pragma unroll
      for (int i = 0; i < NL; ++i) sreg[i] = ld16(row + kcol(st_t & 7, i) * ELT);
    } else {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int tt = min(n0 + VPL * i, last & ~(VPL - 1));   // a VPL-aligned run inside a valid page
        sreg[i] = ld16(vc + (size_t)sphys[i] * block_stride + ((size_t)st_t * p.bs + (tt & (p.bs - 1))) * ELT);
      }
    }
    if ((n + 1) * BN < Lk) load_table(n + 1);
  };
  // decode the staged tile n into buffer `buf` (bf16), zeroing keys at or past Lk
  auto write = [&](int n, int buf) {
    const int n0 = n * BN;
    if (gp == 0) {
      const bool live = n0 + st_key < Lk;
      bf16* dst = reinterpret_cast<bf16*>(kbuf0 + buf * S::K_BYTES) + st_key * S::KS;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const u32x4 r = live ? sreg[i] : u32x4{0, 0, 0, 0};
        bf16* d = dst + kcol(st_t & 7, i);
        if constexpr (FP8) {
          *reinterpret_cast<bf16x8*>(d) = fp8x8_to_bf16x8(r[0], r[1]);
          *reinterpret_cast<bf16x8*>(d + 8) = fp8x8_to_bf16x8(r[2], r[3]);
        } else {
          *reinterpret_cast<u32x4*>(d) = r;
        }
      }
    } else {
      bf16* dst = reinterpret_cast<bf16*>(vbuf0 + buf * S::V_BYTES) + st_t * S::VS;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        u32x4 r = sreg[i];
        const int valid = Lk - (n0 + VPL * i);               // values of this run that exist
        if (valid < VPL) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t keep = 0;
#pragma unroll
            for (int v = 0; v < 4 / ELT; ++v)
              if (e * (4 / ELT) + v < valid) keep |= (FP8 ? 0xFFu : 0xFFFFu) << (8 * ELT * v);
            r[e] &= keep;
          }
        }
        if constexpr (FP8) {
          *reinterpret_cast<bf16x8*>(dst + 16 * i) = fp8x8_to_bf16x8(r[0], r[1]);
          *reinterpret_cast<bf16x8*>(dst + 16 * i + 8) = fp8x8_to_bf16x8(r[2], r[3]);
        } else {
          *reinterpret_cast<u32x4*>(dst + 8 * i) = r;
        }
      }
    }
  };

  // ---- operand addresses inside a tile (bytes). The second wave of a pair takes the tile's two
  // 16-key halves in swapped order (A row i of its S^T is key key_perm32(i) ^ 16), so in both waves
  // score slots 0-7 and P half 0 belong to the wave's own keys 16 dh .. 16 dh + 15, and P half t
  // multiplies the V^T columns of key half t ^ dh.
  const int kaddr = (key_perm32(j) ^ (16 * dh)) * S::KS * 2 + 16 * hh;  // + 32 * kk
  const int vbase = (128 * dh + j) * S::VS * 2 + 16 * hh;
  const int vaddr[2] = {vbase + 32 * dh, vbase + 32 * (dh ^ 1)};         // + 32 * db * VS * 2

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float mc = kNegInf, l = 0.f;

  // ---- prologue: V^T buffer 2 zeroed (the first slot's P V reads it with P = 0); K (0), K (1) and
  // V (0) written, the loads of K (2) and V (1) in flight
  {
    u32x4* z = reinterpret_cast<u32x4*>(vbuf0 + 2 * S::V_BYTES);
    for (int i = tid; i < S::V_BYTES / 16; i += 512) z[i] = u32x4{0, 0, 0, 0};
  }
  if (N > 0) {
    load_table(n_first);
    issue(n_first);
    write(n_first, 0);
    if (gp == 0) {
      if (N > 1) { issue(n_first + 1); write(n_first + 1, 1); }
      if (N > 2) issue(n_first + 2);
    } else {
      if (N > 1) issue(n_first + 1);
    }
  }
  __syncthreads();

  f32x16 st = f32x16{};
  bf16x8 pB[2], pL[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) pB[t] = pL[t] = bf16x8{};
  bool pedge = false;
  // P halves of the wave pairs: [hi, lo][wave][lane]. Each wave writes the half of its own keys in
  // its softmax slot and reads its partner's in its next matrix slot (a workgroup barrier between).
  bf16x8* const xp = reinterpret_cast<bf16x8*>(smem + S::XCHG_OFFSET);
  const int xown = wave * 64 + lane, xother = (wave ^ 1) * 64 + lane;

  // Matrix slot: P V of tile m-1 (8 MFMAs on the wave's half of O^T) and S^T of tile m (16 MFMAs),
  // V and K operands interleaved one to two and read AHEAD operands in advance
  // (scheduling barriers keep that order). Edge tiles add P_lo V in a second pass.
  constexpr int NV = NDB * 2;       // V^T operands, one per (db, t)
  constexpr int NK = NKK;           // K operands
  constexpr int NOP = NV + NK;
  constexpr int AHEAD = 6;
  auto is_v = [](int i) { return i % 3 == 0; };
  auto matrix_slot = [&](auto kb_c, bool has_p) {
    constexpr int KB = decltype(kb_c)::value;           // K (m) is in buffer m % 3
    constexpr int VB = (KB + 2) % 3;                    // V (m-1)
    const unsigned char* Ks = kbuf0 + KB * S::K_BYTES;
    const unsigned char* Vt = vbuf0 + VB * S::V_BYTES;
    auto fetch = [&](int i) -> bf16x8 {
      if (is_v(i)) {
        const int v = i / 3, db = v >> 1, t = v & 1;
        return *reinterpret_cast<const bf16x8*>(Vt + vaddr[t] + db * 32 * S::VS * 2);
      }
      const int kk = i - i / 3 - 1;
      return *reinterpret_cast<const bf16x8*>(Ks + kaddr + 32 * kk);
    };
    if (has_p) {                      // the partner's half of P (m-1)
      pB[1] = xp[xother];
      if (pedge) pL[1] = xp[512 + xother];
    }
    bf16x8 ring[AHEAD];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) ring[i] = fetch(i);
#pragma unroll
    for (int i = 0; i < NOP; ++i) {
      const bf16x8 op = ring[i % AHEAD];
      if (i + AHEAD < NOP) ring[i % AHEAD] = fetch(i + AHEAD);
      if (is_v(i)) {
        const int v = i / 3, db = v >> 1, t = v & 1;
        acc[db] = mfma_32x32x16(op, pB[t], acc[db]);
      } else {
        const int kk = i - i / 3 - 1;
        st = mfma_32x32x16(op, qB[kk], kk == 0 ? f32x16{} : st);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (pedge) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int db = v >> 1, t = v & 1;
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vt + vaddr[t] + db * 32 * S::VS * 2);
        acc[db] = mfma_32x32x16(va, pL[t], acc[db]);
      }
    }
  };
  // Softmax of tile m: masks (edge tiles), the tile's row maximum over all 32 keys and the lazy
  // reference move (both waves of a pair hold the same S^T, so they take the same decisions), then
  // P for the wave's own 16 keys only (hi + lo parts on edge tiles), written for the partner. The
  // row sum l takes the own keys; the partner's l holds the others.
  auto softmax_work = [&](int m) {
    const int n0 = (n_first + m) * BN;
    const bool edge = (n0 + BN > Lk) || (n0 + BN - 1 >= wave_mask_from) || (n0 < wave_lower_max);
    if (edge) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = n0 + 16 * ((r >> 3) ^ dh) + 8 * hh + (r & 7);
        st[r] = (key <= lim && key >= lower) ? st[r] : kNegInf;
      }
    }
    float tmax = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; r += 2) tmax = max3(tmax, st[r], st[r + 1]);
    tmax = max_with_other_half(tmax);
    tmax = (tmax == kNegInf) ? kNegInf : tmax * c;
    const bool move = tmax > mc + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      const float alpha = move ? ((mc == kNegInf) ? 0.f : fast_exp2(mc - tmax)) : 1.f;
      mc = move ? tmax : mc;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    }
    const float nbase = (mc == kNegInf) ? 0.f : -mc;
    if (!edge) {
      float e[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) e[q] = fast_exp2(__builtin_fmaf(st[q], c, nbase));
#pragma unroll
      for (int q = 0; q < 8; q += 2) {
        const bf16x2 pe = cvt_pk_bf16(e[q], e[q + 1]);
        pB[0][q] = pe[0];
        pB[0][q + 1] = pe[1];
      }
      l += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float x = st[q];
        const float e = (x == kNegInf) ? 0.f : fast_exp2(__builtin_fmaf(x, c, nbase));
        l += e;
        pB[0][q] = (bf16)e;
        pL[0][q] = (bf16)(e - (float)pB[0][q]);
      }
      xp[512 + xown] = pL[0];
    }
    xp[xown] = pB[0];
    pedge = edge;
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if (gp == 0) {
    auto step = [&](int m, auto kb_c) {
      constexpr int KB = decltype(kb_c)::value;
      if (m > N) return;
      __builtin_amdgcn_s_setprio(1);
      matrix_slot(kb_c, m > 0);
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      if (m < N) softmax_work(m);
      if (m + 2 < N) write(n_first + m + 2, (KB + 2) % 3);
      if (m + 3 < N) issue(n_first + m + 3);
      __syncthreads();
    };
    for (int m = 0; m <= N; m += 3) {
      step(m, I0{});
      step(m + 1, I1{});
      step(m + 2, I2{});
    }
    __syncthreads();
  } else {
    // slot 0: V (1) into buffer 1, V (2) loads issued
    if (1 < N) write(n_first + 1, 1);
    if (2 < N) issue(n_first + 2);
    __syncthreads();
    auto step = [&](int m, auto kb_c) {
      constexpr int KB = decltype(kb_c)::value;
      if (m > N) return;
      __builtin_amdgcn_s_setprio(1);
      matrix_slot(kb_c, m > 0);
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      if (m < N) softmax_work(m);
      if (m + 2 < N) write(n_first + m + 2, (KB + 2) % 3);
      if (m + 3 < N) issue(n_first + m + 3);
      __syncthreads();
    };
    for (int m = 0; m <= N; m += 3) {
      step(m, I0{});
      step(m + 1, I1{});
      step(m + 2, I2{});
    }
  }

  // ---- epilogue: the row sums of the pair's two key halves are added through LDS; then this
  // wave's half of O / l (bf16, round to nearest even) and the natural-log LSE from the first wave
  // of the pair
  float* const xl = reinterpret_cast<float*>(smem + S::XCHG_OFFSET);    // [wave][lane]
  const float l_half = l + __shfl_xor(l, 32, kWave);
  __syncthreads();                    // the last matrix slot's reads of the exchange area are done
  xl[xown] = l_half;
  __syncthreads();
  const float l_row = l_half + xl[xother];
  if (wave_active && qrow_i < Lq) {
    const float inv = (l_row > 0.f) ? vscale / l_row : 0.f;
    bf16* orow = p.out + ((size_t)(q0 + qrow_i) * p.Hq + head) * D + 128 * dh;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        f32x4 o4 = f32x4{acc[db][4 * rb], acc[db][4 * rb + 1], acc[db][4 * rb + 2], acc[db][4 * rb + 3]} * inv;
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * rb + 4 * hh) = f32x4_to_bf16x4(o4);
      }
    if (p.lse && hh == 0 && dh == 0)
      p.lse[(size_t)(q0 + qrow_i) * p.Hq + head] = (l_row > 0.f) ? kLn2 * (mc + fast_log2(l_row)) : kNegInf;
  }
}

}  // namespace attn
