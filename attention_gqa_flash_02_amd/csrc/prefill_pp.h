// Ping-pong causal/non-causal prefill over contiguous bf16 K/V, head_dim 128. What it computes is
// the tiled exact attention of prefill_core.h ("Attention kernels", section "FlashAttention"):
// per K/V tile the scores, the running row maximum and exponential sum, and P V; only O and the
// per-row log-sum-exp are written.
//
// Work layout. A workgroup is 8 waves in two groups of four (A = waves 0-3, B = 4-7), one wave of
// each group per SIMD. Every wave owns 32 query rows of one query head, with Q^T in registers;
// S^T = K Q^T and O^T += V^T P^T run on 32x32x16 bf16 MFMA with the key permutation of
// prefill_core.h, so the S^T accumulator is already the B operand of the P V product.
//
// Ping-pong. Time is cut into slots that end at a workgroup barrier. In each slot one group runs
// its matrix work (P V of its previous tile, then S^T of its current tile) while the other group
// runs its softmax. So on every SIMD one wave feeds the MFMA pipe while the other feeds the VALU,
// and the groups swap roles every slot.
//
// K/V tiles. They go from global memory straight into LDS (buffer loads with an LDS destination,
// 16 bytes per lane, one wave writing 1 KB = 4 rows of 128 values per instruction). No register
// holds a tile in flight and no VALU work stages it. A tile is BN rows of 256 bytes. The 16-byte
// chunk c of row r sits at chunk slot c ^ swz(r) of its row: the loads pick their global chunk per
// lane so that this holds. The swizzles keep the operand reads free of LDS bank conflicts:
//   * K is read as MFMA A operands (16 consecutive keys of one chunk per 16 lanes): swz = r mod 16.
//   * V is read with the gfx950 transposing LDS read ds_read_b64_tr_b16 (within 16 lanes, lane
//     4a + b returns element b of the 8-byte rows that lanes a, a+4, a+8 and a+12 point at). That
//     is 4 keys x 4 chunks per 32 lanes: swz = 4 (r mod 4) + (r / 4) mod 4.
// Loads past the request's last key are range-checked (the buffer resource of a tile ends at the
// request's last key). The kernel does not depend on what such a lane leaves in LDS (zero, or the
// bytes already there): LDS is zeroed once before the first tile, so a slot past the keys holds
// either zero or a key of an earlier tile of the same request. Its score is masked (P = 0) and
// 0 times a finite value adds nothing, so the only requirement is the caller's: finite K and V.
//
// Schedule, with m = tile index counted from the first tile the workgroup sees:
//   slot 2m:   A: P V (m-1), S^T (m)        B: issue V (m+1), then softmax (m-1)
//   slot 2m+1: A: issue K (m+2), softmax(m) B: P V (m-1), S^T (m), then wait for V (m)
// and A waits for K (m+1) at the end of slot 2m+1. K and V have three LDS buffers each (tile n in
// buffer n mod 3): V (j) goes out in slot 2j-2 and K (j+1) in slot 2j-1, each overwriting a tile
// last read in slot 2j-3, and both are waited for before the barrier that ends slot 2j+1, ahead
// of their first read in slot 2j+2. Each group issues one tile's loads, so the data lands in two
// smaller bursts. Every wave runs every tile of its workgroup:
// tiles that a wave's rows do not see are masked. The control flow is therefore uniform, and every
// slot runs the same straight-line MFMA stream.
#pragma once

#include "prefill_core.h"

namespace attn {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_byte;

__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <int BN>
struct PingPongShape {
  static constexpr int D = 128;
  static constexpr int ROW = 2 * D;                  // bytes per key row in LDS
  static constexpr int TILE = BN * ROW;              // bytes per K or V tile
  static constexpr int NBUF = 3;                     // LDS buffers per K and V
  static constexpr int LDS_BYTES = 2 * NBUF * TILE;  // K0 K1 K2 V0 V1 V2
  static constexpr int BLOCKS = TILE / 1024;         // 1 KB load blocks per tile
  static_assert(BLOCKS % 4 == 0, "each of the 4 loading waves fills whole 1 KB blocks");
};

__device__ __forceinline__ bf16x8 lds_read_b128(const unsigned char* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ i16x4 lds_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

template <int BN>
__device__ __forceinline__ void prefill_pingpong_body(const PrefillParams& p, unsigned char* smem, int hgrp, int b,
                                                      int qt) {
  using S = PingPongShape<BN>;
  constexpr int D = 128;
  constexpr int NKB = BN / 32;      // 32-key blocks per tile
  constexpr int NDB = D / 32;       // 32-wide d blocks of O^T
  constexpr int NKK = D / 16;       // k-steps of the QK MFMA
  constexpr float kLazyRescale = 8.f;
  constexpr float kFastLimit = 4294967296.f;   // 2^32
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: kept in a scalar register
  const int gp = wave >> 2;
  const int j = lane & 31;
  const int hh = lane >> 5;

  const int groups_per_kv = p.g / p.hpw;
  const int kvh = hgrp / groups_per_kv;
  const int head = kvh * p.g + (hgrp % groups_per_kv) * p.hpw + (wave % p.hpw);
  const int TQ = 32 * (8 / p.hpw);
  const int q0 = p.cu_seqlens_q[b];
  const int Lq = p.cu_seqlens_q[b + 1] - q0;
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
  const int n_first = min(kv_begin / BN, ntiles);
  const int N = ntiles - n_first;
  const float c = p.scale * kLog2e;

  // ---- Q^T operands: lane (j, hh) holds Q[row tw + j][16*kk + 8*hh .. +7]
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
  const int lim = p.causal ? min(qrow_i, Lk - 1) : (Lk - 1);
  const int lower = win > 0 ? qrow_i - win + 1 : INT_MIN;
  const int wave_mask_from = p.causal ? max(0, tw + 1) : Lk;

  // ---- tile loads: group A loads the K tiles and group B the V tiles (and the first K tile); wave
  // w of a group (0-3) fills 1 KB blocks LPW*w .. of the tile; lane l of a block writes slot l & 15
  // of row 4 * block + l / 16, i.e. it loads global chunk slot ^ swz(row) of that row
  const long long stride = (long long)p.Hkv * D;
  const long long row_bytes = stride * 2;
  const char* kbase = reinterpret_cast<const char*>(p.k + (size_t)q0 * stride + (size_t)kvh * D);
  const char* vbase = reinterpret_cast<const char*>(p.v + (size_t)q0 * stride + (size_t)kvh * D);
  const long long end_bytes = Lk > 0 ? (long long)(Lk - 1) * row_bytes + D * 2 : 0;
  constexpr int LPW = S::BLOCKS / 4;                 // blocks per loading wave per tile
  const int lw = wave & 3;
  int koff[LPW], voff[LPW];
#pragma unroll
  for (int it = 0; it < LPW; ++it) {
    const int row = 4 * (lw * LPW + it) + (lane >> 4);
    const int slot = lane & 15;
    koff[it] = (int)(row * row_bytes) + 16 * (slot ^ swz_k(row));
    voff[it] = (int)(row * row_bytes) + 16 * (slot ^ swz_v(row));
  }
  constexpr int NBUF = S::NBUF;
  unsigned char* const kbuf0 = smem;
  unsigned char* const vbuf0 = smem + NBUF * S::TILE;
  // Buffer resource of tile n (no bytes when the tile does not exist: its loads fetch nothing).
  auto tile_rsrc = [&](const char* base, int n, bool exists) -> u32x4 {
    const long long t = (long long)n * BN * row_bytes;
    long long left = exists ? end_bytes - t : 0;
    left = left < 0 ? 0 : (left > (long long)BN * row_bytes ? (long long)BN * row_bytes : left);
    const uint64_t a = reinterpret_cast<uint64_t>(base + (exists ? t : 0));
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, (uint32_t)left, (uint32_t)kBufferFlags};
  };
  // One 1 KB block from global memory straight into LDS (M0 = LDS byte address of the block).
  // Issued from inline assembly: the compiler then does not see LDS written behind its back and
  // does not make every later LDS read wait for the load; the schedule waits for the loads itself
  // (vmcnt) before the barrier that publishes a tile. M0 is written by nothing else in this kernel,
  // so the clobber of that reserved register is safe.
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
  int kaddr[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kaddr[kk] = kperm * S::ROW + 16 * ((2 * kk + hh) ^ swz_k(kperm));
  int vaddr[NDB][2];
  {
    const int s = lane & 15, g = lane >> 4, a = s & 3, k = s >> 2;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int rowb = 8 * (g >> 1) + 4 * r + k;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int chunk = 4 * db + 2 * (g & 1) + (a >> 1);
        vaddr[db][r] = NBUF * S::TILE + rowb * S::ROW + 16 * (chunk ^ swz_v(rowb)) + 8 * (a & 1);
      }
    }
    // The V addresses include the offset of the first V buffer and are kept opaque, so that a read
    // of V buffer b only adds b * TILE (an immediate below 64 KB) to them.
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int db = 0; db < NDB; ++db) asm volatile("" : "+v"(vaddr[db][r]));
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float mc = kNegInf, l = 0.f;

  // LDS starts zeroed (see the top of the file for the slots past the keys), then K of the first tile.
  // The Q loads, issued first, are waited for only here, together with that tile, so the two
  // latencies overlap. An empty asm then redefines the Q registers, so the tile loop never waits on
  // the memory counter for them (which would also wait for the tile loads in flight).
  {
    u32x4* z = reinterpret_cast<u32x4*>(smem);
    for (int i = tid; i < S::LDS_BYTES / 16; i += 512) z[i] = u32x4{0, 0, 0, 0};
  }
  __syncthreads();
  if (gp == 1 && N > 0) {
    const u32x4 r0 = tile_rsrc(kbase, n_first, true);
#pragma unroll
    for (int it = 0; it < LPW; ++it) load_block(r0, koff[it], kbuf0 + 1024 * (LPW * lw + it));
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(qB[kk]));
  __syncthreads();

  f32x16 st[NKB];
  bf16x8 pB[NKB][2], pL[NKB][2];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t) pB[kb][t] = pL[kb][t] = bf16x8{};
  bool pedge = false;
  // Every wave runs every tile of the workgroup (tiles a wave's rows do not see are masked), so
  // the control flow is uniform and the registers of S^T and P are easy to share.
  // Matrix slot: P V of tile m-1 and S^T of tile m as one stream of MFMAs. V and K operands
  // alternate, so consecutive MFMAs never depend on each other. The LDS operands are read AHEAD
  // operands in advance; scheduling barriers keep that order (the compiler would otherwise sink
  // each read next to its MFMA and wait for it). The first slot's P V runs with P = 0 on a zeroed
  // V buffer and the last slot's S^T is computed and dropped, so every slot runs the same code.
  // Edge tiles add P_lo V in a second pass.
  constexpr int NV = NKB * 2 * NDB;                 // V^T operands, one per (kb, t, db)
  constexpr int NK = NKK * NKB;                     // K operands, one per (kk, kb)
  static_assert(NV == NK, "V and K operands alternate");
  constexpr int NOP = NV + NK;
  constexpr int AHEAD = 6;
  auto v_operand = [&](const unsigned char* Vt, int v) -> bf16x8 {
    const int kb = v / (2 * NDB), t = (v / NDB) % 2, db = v % NDB;
    const unsigned char* vt = Vt + (32 * kb + 16 * t) * S::ROW;
    const i16x4 v0 = lds_read_tr(vt + vaddr[db][0]);
    const i16x4 v1 = lds_read_tr(vt + vaddr[db][1]);
    return bitcast<bf16x8>(__builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // The buffer indices are compile-time constants (the slot loop is unrolled by NBUF), so the
  // operand reads address every buffer with an immediate offset.
  auto matrix_slot = [&](auto kb_c) {
    constexpr int KB = decltype(kb_c)::value;          // K (m) is in buffer m % NBUF
    constexpr int VB = (KB + NBUF - 1) % NBUF;         // V (m-1)
    const unsigned char* Vt = smem + VB * S::TILE;     // + vaddr = V buffer VB
    const unsigned char* Ks = kbuf0 + KB * S::TILE;
    auto fetch = [&](int i) -> bf16x8 {
      if ((i & 1) == 0) return v_operand(Vt, i >> 1);
      const int k = i >> 1, kk = k / NKB, kb = k % NKB;
      return lds_read_b128(Ks + 32 * kb * S::ROW + kaddr[kk]);
    };
    bf16x8 ring[AHEAD];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) ring[i] = fetch(i);
#pragma unroll
    for (int i = 0; i < NOP; ++i) {
      const bf16x8 op = ring[i % AHEAD];
      if (i + AHEAD < NOP) ring[i % AHEAD] = fetch(i + AHEAD);
      if ((i & 1) == 0) {
        const int v = i >> 1, kb = v / (2 * NDB), t = (v / NDB) % 2, db = v % NDB;
        acc[db] = mfma_32x32x16(op, pB[kb][t], acc[db]);
      } else {
        const int k = i >> 1, kk = k / NKB, kb = k % NKB;
        st[kb] = mfma_32x32x16(op, qB[kk], kk == 0 ? f32x16{} : st[kb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (pedge) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int kb = v / (2 * NDB), t = (v / NDB) % 2, db = v % NDB;
        acc[db] = mfma_32x32x16(v_operand(Vt, v), pL[kb][t], acc[db]);
      }
    }
  };
  auto softmax_work = [&](int m) {
      const int n0 = (n_first + m) * BN;
      const bool edge = (n0 + BN > Lk) || (n0 + BN - 1 >= wave_mask_from) || (n0 < wave_lower_max);
      // Fast path of an interior tile (no masked key) once every row of the wave has a finite
      // reference maximum: P = 2^(S c - ref) against the current reference, without the tile
      // maximum. It stands when no lane's tile sum exceeds kFastLimit (then every P of the tile is
      // below it, far inside the bf16 and fp32 ranges); otherwise the tile is redone below, where
      // the reference moves. Unless the scores of a row grow by more than 32 / log2(e) after its
      // first tile, the maximum is taken on the first and the masked tiles only.
      if (!edge && __builtin_amdgcn_ballot_w64(mc == kNegInf) == 0) {
        const float nbase = -mc;
        float ts[2];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            float e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) e[q] = fast_exp2(__builtin_fmaf(st[kb][8 * t + q], c, nbase));
#pragma unroll
            for (int q = 0; q < 8; q += 2) {
              const bf16x2 pe = cvt_pk_bf16(e[q], e[q + 1]);
              pB[kb][t][q] = pe[0];
              pB[kb][t][q + 1] = pe[1];
            }
            const float s8 = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
            ts[t] = (kb == 0) ? s8 : ts[t] + s8;
          }
        const float tsum = ts[0] + ts[1];
        if (__builtin_amdgcn_ballot_w64(!(tsum <= kFastLimit)) == 0) {
          l += tsum;
          pedge = false;
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
      float tmax = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) tmax = max3(tmax, st[kb][r], st[kb][r + 1]);
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
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            float e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) e[q] = fast_exp2(__builtin_fmaf(st[kb][8 * t + q], c, nbase));
#pragma unroll
            for (int q = 0; q < 8; q += 2) {
              const bf16x2 pe = cvt_pk_bf16(e[q], e[q + 1]);
              pB[kb][t][q] = pe[0];
              pB[kb][t][q + 1] = pe[1];
            }
            l += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const float x = st[kb][8 * t + q];
              const float e = (x == kNegInf) ? 0.f : fast_exp2(__builtin_fmaf(x, c, nbase));
              l += e;
              pB[kb][t][q] = (bf16)e;
              pL[kb][t][q] = (bf16)(e - (float)pB[kb][t][q]);
            }
      }
      pedge = edge;
  };
  // Group A runs slots 2m (matrix) and 2m+1 (softmax) in iteration m; group B, one slot later,
  // runs slots 2m+1 (matrix) and 2m+2 (softmax). Each group issues its tile's loads at the start
  // of its softmax slot (see the schedule at the top). The matrix work runs at a raised wave
  // priority, so that the SIMD's other wave never holds up an MFMA's issue.
  // K (j+1) into buffer (j+1) mod NBUF, issued by group A; V (j) into buffer j mod NBUF, issued
  // by group B. Each wave writes the 1 KB blocks LPW*lw .. of the tile.
  auto issue_k = [&](int j, auto kb_c) {
    constexpr int KB = decltype(kb_c)::value;          // (j + 1) % NBUF
    const u32x4 rk = tile_rsrc(kbase, n_first + j + 1, j + 1 < N);
    unsigned char* kdst = kbuf0 + KB * S::TILE + 1024 * LPW * lw;
#pragma unroll
    for (int q = 0; q < LPW; ++q) load_block(rk, koff[q], kdst + 1024 * q);
  };
  auto issue_v = [&](int j, auto vb_c) {
    constexpr int VB = decltype(vb_c)::value;          // j % NBUF
    const u32x4 rv = tile_rsrc(vbase, n_first + j, j < N);
    unsigned char* vdst = vbuf0 + VB * S::TILE + 1024 * LPW * lw;
#pragma unroll
    for (int q = 0; q < LPW; ++q) load_block(rv, voff[q], vdst + 1024 * q);
  };
  static_assert(NBUF == 3, "the slot loop below is unrolled by 3");
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  static_assert(LPW == 4, "a group's batch is 4 loads per wave (the vmcnt below)");
  if (gp == 0) {
    // K (j+1) goes out at the start of slot 2j-1 (K 1 before slot 0) and is waited for at the end
    // of slot 2j+1; it overwrites K (j-2), last read in slot 2j-3, and is first read in slot 2j+2.
    issue_k(0, I1{});
    auto step = [&](int m, auto kb_c) {
      constexpr int KB = decltype(kb_c)::value;
      if (m > N) return;
      __builtin_amdgcn_s_setprio(1);
      matrix_slot(kb_c);
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      if (m + 1 <= N) issue_k(m + 1, std::integral_constant<int, (KB + 2) % 3>{});
      if (m < N) softmax_work(m);
      // wait for K (m+1) only: K (m+2), issued after it, may stay in flight
      if (m + 1 <= N) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    };
    for (int m = 0; m <= N; m += 3) {
      step(m, I0{});
      step(m + 1, I1{});
      step(m + 2, I2{});
    }
    __syncthreads();
  } else {
    // V (j) goes out at the start of slot 2j-2 (V 0 and V 1 in slot 0) and is waited for at the
    // end of slot 2j+1; it overwrites V (j-3), last read in slot 2j-3, and is first read in slot
    // 2j+2.
    issue_v(0, I0{});
    if (1 <= N) issue_v(1, I1{});
    __syncthreads();
    auto step = [&](int m, auto kb_c) {
      constexpr int KB = decltype(kb_c)::value;
      if (m > N) return;
      __builtin_amdgcn_s_setprio(1);
      matrix_slot(kb_c);
      __builtin_amdgcn_s_setprio(0);
      // wait for V (m) only: V (m+1), issued after it, may stay in flight
      if (m + 1 <= N) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (m + 2 <= N) issue_v(m + 2, std::integral_constant<int, (KB + 2) % 3>{});
      if (m < N) softmax_work(m);
      __syncthreads();
    };
    for (int m = 0; m <= N; m += 3) {
      step(m, I0{});
      step(m + 1, I1{});
      step(m + 2, I2{});
    }
  }

  // ---- epilogue: O / l (bf16, round to nearest even) and the natural-log LSE
  const float l_row = l + __shfl_xor(l, 32, kWave);
  if (wave_active && qrow_i < Lq) {
    const float inv = (l_row > 0.f) ? 1.f / l_row : 0.f;
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
