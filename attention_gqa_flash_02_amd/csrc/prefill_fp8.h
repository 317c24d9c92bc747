// FP8 causal/non-causal prefill over contiguous e4m3fn Q/K/V with per-head scales, head_dim 128,
// on the gfx950 fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, unit block scales).
//
// What it computes. This is the attention of prefill_core.h on the decoded inputs
// Q = q_scale[h] * e4m3(q), K = k_scale[kvh] * e4m3(k) and V = v_scale[kvh] * e4m3(v). The per-head
// scales are folded into the score scale and the final normalisation. The exponentials P are
// rounded to e4m3 for the P V product ("Attention kernels", section "FlashAttention", FP8 variant
// of the third version); the row sums stay in fp32. The rounding of one weight (3 mantissa bits)
// only averages out over many keys, so P is carried as hi + lo e4m3 parts (lo = the rounding
// remainder, about 2^-8 relative together) on every tile among the first kSplitKeys keys a wave's
// rows see and on every tile that masks some key of a row (the diagonal, the key tail, a sliding
// window's lower edge); beyond them a row has seen at least kSplitKeys keys.
//
// Structure. This is the ping-pong kernel of prefill_pp.h with one byte per element:
//   * S^T = K Q^T: one 32x32x64 fp8 MFMA per 32-key block and 64-wide half of head_dim. Its A
//     operand is 32 consecutive bytes of a K row (A-row i loads key pi(i), bits 2 and 3 of i
//     swapped), and its B operand is 32 consecutive Q bytes held in registers. The accumulator
//     layout is the 32x32 one of the bf16 MFMA, so lane (j, hh) holds the scores of keys
//     32 kb + 16 (r / 8) + 8 hh + r % 8.
//   * O^T += V^T P^T: one MFMA per 32-wide block of head_dim covers the whole 64-key tile. The
//     B operand is the lane's 32 P values as bytes, in accumulator order (byte p = 16 kb + r). The
//     A operand must give lane (d, hh) V[key(hh, p)][d] for the same byte p, which is 4 runs of 8
//     consecutive keys (16 u + 8 hh + 0..7). Each run is one ds_read_b64_tr_b8: within 16 lanes,
//     lane 8 h + e returns byte e of the 8-byte rows that lanes h, h+2, ..., h+14 point at.
//   * Tiles are 64 rows of 128 bytes, loaded straight into LDS in 1 KB blocks of 8 rows. Chunk c
//     (16 bytes) of row r sits at slot c ^ swz(r), with swz = (r / 2) mod 8 for K and
//     2 ((r / 2) mod 4) for V. That makes both operand reads free of bank conflicts.
#pragma once

#include "prefill_pp.h"

namespace attn {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

struct PrefillFp8Params {
  const uint8_t* q;            // [Tq, Hq, D] e4m3fn codes
  const uint8_t* k;            // [T, Hkv, D]
  const uint8_t* v;            // [T, Hkv, D]
  const float* q_scale;        // [Hq]
  const float* k_scale;        // [Hkv]
  const float* v_scale;        // [Hkv]
  bf16* out;                   // [Tq, Hq, D]
  float* lse;                  // [Tq, Hq] or nullptr
  const int32_t* cu_seqlens;   // [B + 1]
  float scale;
  int num_seqs, Hq, Hkv, g, hpw, causal, num_qtiles, window;
};

__device__ __forceinline__ int swz_k8(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_v8(int r) { return ((r >> 1) & 3) << 1; }

__device__ __forceinline__ f32x16 mfma_f8_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
  // formats 0 / 0 = e4m3 for both operands; block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ i32x2 lds_read_tr8(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}
// Four floats -> four e4m3fn codes in one dword (round to nearest even; the values here are in
// [0, 256], inside the finite range). The first conversion writes the low half of its third
// operand and keeps the high half, which the second overwrites, so any starting value will do
// (a's bits: no register has to be zeroed first).
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}
// The two e4m3fn codes in the low (HI = false) or high half of w, decoded to floats.
template <bool HI>
__device__ __forceinline__ f32x2 unpack_fp8x2(int w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

template <int BN>
struct PingPongFp8Shape {
  static constexpr int D = 128;
  static constexpr int ROW = D;                      // bytes per key row
  static constexpr int TILE = BN * ROW;
  static constexpr int LDS_BYTES = 4 * TILE;         // K0 K1 V0 V1
  static constexpr int BLOCKS = TILE / 1024;         // 1 KB load blocks (8 rows) per tile
  static_assert(BN == 64, "one MFMA covers the 64 keys of a tile in P V");
  static_assert(BLOCKS % 4 == 0, "each of the 4 loading waves fills whole blocks");
};

template <int BN>
__device__ __forceinline__ void prefill_fp8_body(const PrefillFp8Params& p, unsigned char* smem, int hgrp, int b,
                                                 int qt) {
  using S = PingPongFp8Shape<BN>;
  constexpr int D = 128;
  constexpr int NKB = BN / 32;      // 32-key blocks per tile
  constexpr int NDB = D / 32;       // 32-wide d blocks of O^T
  constexpr int NM = D / 64;        // 64-wide d halves of the QK contraction
  constexpr float kLazyRescale = 8.f;   // keeps every unscaled P at most 2^8, inside e4m3's range
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gp = wave >> 2;
  const int j = lane & 31;
  const int hh = lane >> 5;

  const int groups_per_kv = p.g / p.hpw;
  const int kvh = hgrp / groups_per_kv;
  const int head = kvh * p.g + (hgrp % groups_per_kv) * p.hpw + (wave % p.hpw);
  const int TQ = 32 * (8 / p.hpw);
  const int q0 = p.cu_seqlens[b];
  const int Lq = p.cu_seqlens[b + 1] - q0;
  const int Lk = Lq;
  const int t0 = qt * TQ;
  if (t0 >= Lq) return;
  const int tw = t0 + 32 * (wave / p.hpw);
  const bool wave_active = tw < Lq;
  const int kv_end = p.causal ? min(Lk, min(Lq, t0 + TQ)) : Lk;
  const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  const int win = p.window;
  const int kv_begin = win > 0 ? max(0, t0 - win + 1) : 0;
  const int wave_lower_max = win > 0 ? tw + 31 - win + 1 : INT_MIN;
  constexpr int kSplitKeys = 256;
  const int wave_split_end = (win > 0 ? max(0, tw - win + 1) : 0) + kSplitKeys;
  const int n_first = min(kv_begin / BN, ntiles);
  const int N = ntiles - n_first;
  const float c = p.scale * p.q_scale[head] * p.k_scale[kvh] * kLog2e;
  const float vscale = p.v_scale[kvh];

  // ---- Q^T operands: lane (j, hh) holds Q[row tw + j][64 m + 32 hh .. +31] (bytes)
  i32x8 qB[NM];
  const int qrow_i = tw + j;
  if (qrow_i < Lq) {
    const uint8_t* qrow = p.q + ((size_t)(q0 + qrow_i) * p.Hq + head) * D;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(qrow + 64 * m + 32 * hh);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(qrow + 64 * m + 32 * hh + 16);
      qB[m] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  } else {
#pragma unroll
    for (int m = 0; m < NM; ++m) qB[m] = i32x8{};
  }
#pragma unroll
  for (int m = 0; m < NM; ++m) asm volatile("" : "+v"(qB[m]));
  const int lim = p.causal ? min(qrow_i, Lk - 1) : (Lk - 1);
  const int lower = win > 0 ? qrow_i - win + 1 : INT_MIN;
  const int wave_mask_from = p.causal ? max(0, tw + 1) : Lk;

  // ---- tile loads, all issued by group A: its wave w (0-3) fills 1 KB blocks LPW*w .. of each
  // K and V tile; lane l of a block writes slot l & 7 of row 8 * block + l / 8, i.e. it loads
  // global chunk slot ^ swz(row) of that row
  const long long row_bytes = (long long)p.Hkv * D;
  const char* kbase = reinterpret_cast<const char*>(p.k + (size_t)q0 * row_bytes + (size_t)kvh * D);
  const char* vbase = reinterpret_cast<const char*>(p.v + (size_t)q0 * row_bytes + (size_t)kvh * D);
  const long long end_bytes = Lk > 0 ? (long long)(Lk - 1) * row_bytes + D : 0;
  constexpr int LPW = S::BLOCKS / 4;
  const int lw = wave & 3;
  int koff[LPW], voff[LPW];
#pragma unroll
  for (int it = 0; it < LPW; ++it) {
    const int row = 8 * (lw * LPW + it) + (lane >> 3);
    const int slot = lane & 7;
    koff[it] = (int)(row * row_bytes) + 16 * (slot ^ swz_k8(row));
    voff[it] = (int)(row * row_bytes) + 16 * (slot ^ swz_v8(row));
  }
  unsigned char* const kbuf0 = smem;
  unsigned char* const vbuf0 = smem + 2 * S::TILE;
  auto tile_rsrc = [&](const char* base, int n, bool exists) -> u32x4 {
    const long long t = (long long)n * BN * row_bytes;
    long long left = exists ? end_bytes - t : 0;
    left = left < 0 ? 0 : (left > (long long)BN * row_bytes ? (long long)BN * row_bytes : left);
    const uint64_t a = reinterpret_cast<uint64_t>(base + (exists ? t : 0));
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, (uint32_t)left, (uint32_t)kBufferFlags};
  };
  // One 1 KB block from global memory straight into LDS (M0 = LDS byte address of the block); as
  // in prefill_pp.h, issued from inline assembly and waited for by the schedule itself.
  auto load_block = [&](const u32x4& rsrc, int off, unsigned char* dst) {
    const uint32_t lds = (uint32_t)reinterpret_cast<uintptr_t>((lds_byte*)dst);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(off), "s"(rsrc) : "memory", "m0");
#pragma clang diagnostic pop
  };

  // ---- operand addresses inside a tile (bytes)
  const int kperm = key_perm32(j);
  int kaddr[NM][2];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) kaddr[m][h2] = kperm * S::ROW + 16 * ((4 * m + 2 * hh + h2) ^ swz_k8(kperm));
  int vaddr[NDB];
  {
    const int s = lane & 15, g = lane >> 4;
    const int row0 = 8 * (g >> 1) + (s >> 1);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      vaddr[db] = row0 * S::ROW + 16 * ((2 * db + (g & 1)) ^ swz_v8(row0)) + 8 * (s & 1);
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float mc = kNegInf, l = 0.f;

  // LDS starts zeroed, then K of the first tile. As in prefill_pp.h the kernel does not depend on what
  // a range-checked load past the keys leaves in LDS (zero or an earlier tile's finite codes of the same
  // request): those keys' scores are masked and their P is 0.
  {
    u32x4* z = reinterpret_cast<u32x4*>(smem);
    for (int i = tid; i < S::LDS_BYTES / 16; i += 512) z[i] = u32x4{0, 0, 0, 0};
  }
  __syncthreads();
  if (gp == 0 && N > 0) {
    const u32x4 r0 = tile_rsrc(kbase, n_first, true);
#pragma unroll
    for (int it = 0; it < LPW; ++it) load_block(r0, koff[it], kbuf0 + 1024 * (LPW * lw + it));
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  f32x16 st[NKB];
  i32x8 pB = i32x8{}, pL = i32x8{};
  bool psplit = false;

  // Matrix slot: P V of tile m-1 (one MFMA per d block, each over the tile's 64 keys) and S^T of
  // tile m (one MFMA per 32-key block and d half). All LDS operands are read first; the first
  // slot's P V runs with P = 0 on a zeroed V buffer and the last slot's S^T is dropped, so every
  // slot runs the same code. Tiles with P split into hi + lo add P_lo V.
  auto matrix_slot = [&](int m) {
    const unsigned char* Vt = vbuf0 + ((m - 1) & 1) * S::TILE;
    const unsigned char* Ks = kbuf0 + (m & 1) * S::TILE;
    i32x8 vop[NDB], kop[NKB][NM];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      i32x2 r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) r[u] = lds_read_tr8(Vt + 16 * u * S::ROW + vaddr[db]);
      vop[db] = i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int mm = 0; mm < NM; ++mm) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(Ks + 32 * kb * S::ROW + kaddr[mm][0]);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(Ks + 32 * kb * S::ROW + kaddr[mm][1]);
        kop[kb][mm] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
      acc[i] = mfma_f8_32x32x64(vop[i], pB, acc[i]);
      const int kb = i % NKB, mm = i / NKB;
      st[kb] = mfma_f8_32x32x64(kop[kb][mm], qB[mm], mm == 0 ? f32x16{} : st[kb]);
    }
    if (psplit) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] = mfma_f8_32x32x64(vop[db], pL, acc[db]);
    }
    // The scores go into the exponent domain of the current reference here, t = S c - ref (S c
    // while a row has none): the matrix slot has room to spare, the softmax slot beside it sets the
    // pace. (The empty asm keeps each product in this slot; the compiler would otherwise sink it
    // past the barrier.)
    const float tb = (mc == kNegInf) ? 0.f : -mc;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = __builtin_fmaf(st[kb][r], c, tb);
        asm volatile("" : "+v"(x));
        st[kb][r] = x;
      }
  };
  auto softmax_work = [&](int m) {
    const int n0 = (n_first + m) * BN;
    const bool edge = (n0 + BN > Lk) || (n0 + BN - 1 >= wave_mask_from) || (n0 < wave_lower_max);
    const bool split = edge || (n0 < wave_split_end);
    const float tb = (mc == kNegInf) ? 0.f : -mc;    // st holds t = S c + tb (see the matrix slot)
    // Fast path of an unsplit interior tile once every row of the wave has a finite reference
    // maximum: P = 2^t without the tile maximum, kept unless some lane's tile sum exceeds 2^8 (so
    // every P stays at most 2^8, inside e4m3's range; else the tile is redone below, where the
    // reference moves).
    if (!split && __builtin_amdgcn_ballot_w64(mc == kNegInf) == 0) {
      float tsum;
#pragma unroll
      for (int w = 0; w < 2 * NKB * 2; ++w) {
        const int kb = w / 4, r = 4 * (w % 4);
        float e[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) e[q] = fast_exp2(st[kb][r + q]);
        const float s4 = (e[0] + e[1]) + (e[2] + e[3]);   // summed before the packing takes a's register
        tsum = (w == 0) ? s4 : tsum + s4;
        pB[w] = pack_fp8x4(e[0], e[1], e[2], e[3]);
      }
      if (__builtin_amdgcn_ballot_w64(!(tsum <= 256.f)) == 0) {
        l += tsum;
        psplit = false;
        return;
      }
    }
    if (edge) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = n0 + 32 * kb + 16 * (r >> 3) + 8 * hh + (r & 7);
          st[kb][r] = (key <= lim && key >= lower) ? st[kb][r] : kNegInf;
        }
    }
    // tile maximum in t units; the reference moves where it exceeds the current one by more than
    // kLazyRescale (any finite maximum where the row has no reference yet)
    float tmax = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) tmax = max3(tmax, st[kb][r], st[kb][r + 1]);
    tmax = max_with_other_half(tmax);
    const bool move = tmax > ((mc == kNegInf) ? kNegInf : kLazyRescale);
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      const float alpha = move ? ((mc == kNegInf) ? 0.f : fast_exp2(-tmax)) : 1.f;
      mc = move ? tmax - tb : mc;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    }
    const float sh = move ? tmax : 0.f;             // t - sh is relative to the (new) reference
    if (!split) {
#pragma unroll
      for (int w = 0; w < 2 * NKB * 2; ++w) {       // dword w of the B operand: scores 4w .. 4w+3
        const int kb = w / 4, r = 4 * (w % 4);
        float e[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) e[q] = fast_exp2(st[kb][r + q] - sh);
        pB[w] = pack_fp8x4(e[0], e[1], e[2], e[3]);
        l += (e[0] + e[1]) + (e[2] + e[3]);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 2 * NKB * 2; ++w) {
        const int kb = w / 4, r = 4 * (w % 4);
        float e[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float x = st[kb][r + q];
          e[q] = (x == kNegInf) ? 0.f : fast_exp2(x - sh);
        }
        const int hi = pack_fp8x4(e[0], e[1], e[2], e[3]);
        const f32x2 d01 = unpack_fp8x2<false>(hi), d23 = unpack_fp8x2<true>(hi);
        pB[w] = hi;
        pL[w] = pack_fp8x4(e[0] - d01[0], e[1] - d01[1], e[2] - d23[0], e[3] - d23[1]);
        l += (e[0] + e[1]) + (e[2] + e[3]);
      }
    }
    psplit = split;
  };
  // Group A runs slots 2m (matrix) and 2m+1 (softmax) in iteration m; group B, one slot later,
  // runs slots 2m+1 (matrix) and 2m+2 (softmax). Group A issues the tile loads of slot 2m (K m+1,
  // V m) at its start and waits for them at the end of slot 2m+1: its matrix slot has room to
  // spare, while the softmax slot beside it sets the pace.
  auto issue_loads = [&](int jt) {
    const u32x4 rk = tile_rsrc(kbase, n_first + jt + 1, jt + 1 < N);
    const u32x4 rv = tile_rsrc(vbase, n_first + jt, jt < N);
    unsigned char* kdst = kbuf0 + ((jt + 1) & 1) * S::TILE + 1024 * LPW * lw;
    unsigned char* vdst = vbuf0 + (jt & 1) * S::TILE + 1024 * LPW * lw;
#pragma unroll
    for (int q = 0; q < LPW; ++q) load_block(rk, koff[q], kdst + 1024 * q);
#pragma unroll
    for (int q = 0; q < LPW; ++q) load_block(rv, voff[q], vdst + 1024 * q);
  };
  if (gp == 0) {
    for (int m = 0; m <= N; ++m) {
      __builtin_amdgcn_s_setprio(1);
      if (m < N) issue_loads(m);
      matrix_slot(m);
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      if (m < N) softmax_work(m);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    __syncthreads();
  } else {
    __syncthreads();
    for (int m = 0; m <= N; ++m) {
      __builtin_amdgcn_s_setprio(1);
      matrix_slot(m);
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      if (m < N) softmax_work(m);
      __syncthreads();
    }
  }

  // ---- epilogue: O v_scale / l (bf16, round to nearest even) and the natural-log LSE
  const float l_row = l + __shfl_xor(l, 32, kWave);
  if (wave_active && qrow_i < Lq) {
    const float inv = (l_row > 0.f) ? vscale / l_row : 0.f;
    bf16* orow = p.out + ((size_t)(q0 + qrow_i) * p.Hq + head) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        f32x4 o4 = f32x4{acc[db][4 * rb], acc[db][4 * rb + 1], acc[db][4 * rb + 2], acc[db][4 * rb + 3]} * inv;
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * rb + 4 * hh) = f32x4_to_bf16x4(o4);
      }
    if (p.lse && hh == 0)
      p.lse[(size_t)(q0 + qrow_i) * p.Hq + head] = (l_row > 0.f) ? kLn2 * (mc + fast_log2(l_row)) : kNegInf;
  }
}

}  // namespace attn
