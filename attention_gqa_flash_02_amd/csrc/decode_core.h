// Split-KV paged decode for gfx950.
//
// What it computes ("Attention kernels", section "Prefill and decode attention"):
// the few query rows of a request that share one KV head (g query heads x Lq
// new tokens, at most 16 rows, or 32 in the head_dim-128 mixed batch) attend over the
// request's paged cache; each KV
// head is read once for all of them, and the key axis is cut into pieces whose
// results are merged with their log-sum-exps (the same rule as the online
// softmax). Pages are located through the block table ("Optimization 1",
// section 3.4; "Attention kernels", section "Paged KV and kernels").
//
// Work split: the batch's work is the list of (request, kv head, chunk of CH
// keys) items, request-major. The partition kernel's G workgroups take equal
// contiguous shares of that list (a multiple of 4 chunks each), so every
// workgroup streams the same number of KV bytes whatever the mix of context
// lengths. A share covers pieces of one or more (request, kv head) units; a
// unit that lies inside one share is written directly, the pieces of a unit
// that spans shares go to the workspace as normalised partials with their LSEs
// and are merged by a second small kernel.
//
// Work layout inside a workgroup (NW waves: 4 in the decode kernel, 8 in the head_dim-256 mixed
// kernel):
//   * the share's chunks are dealt to the waves round-robin.
//   * per chunk, S^T = K . Q^T on 16x16x32 MFMA (NU sub-tiles of 16 keys; each
//     block of 16 query rows is the MFMA columns), an online-softmax update in
//     registers, then O^T += V^T . P^T on 16x16x32 MFMA. V pages are stored
//     token-innermost ([D][block_size]), so the V^T operand comes straight from
//     HBM with the key axis contiguous in each lane; P^T is the S^T accumulator
//     itself (no shuffle, no LDS).
//   * token layout: in half h (32 tokens) of a chunk, lane quad q owns the
//     8-token run 32h + 8q .. +7. A-row i of QK sub-tile u = 2h + e loads token
//     32h + 8(i/4) + 4e + i%4, so that C-row 4q + s of that sub-tile is token
//     32h + 8q + 4e + s: each lane then holds P for exactly the 8 tokens its own
//     V^T load brings (one 16-byte load per d row for bf16), and a run never
//     crosses a page (block sizes are >= 16).
//   * memory: the block-table entries of the next chunk are loaded while the
//     current chunk computes, and the K and V loads of a chunk are issued back
//     to back with no wait in between. Loads past the end of the request are
//     redirected into its last page (always a valid address) and their values
//     masked, so no load sits behind a branch.
//   * the NW waves' (max, sum, O) are combined in LDS in a fixed order.
#pragma once

#include <climits>
#include <type_traits>

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
  float* ws_o;                 // [G, 2, max_rows, D] partial outputs (normalised)
  float* ws_lse;               // [G, 2, max_rows] partial natural-log LSEs
  int32_t* ws_prefix;          // [B + 1] prefix sums of the planned lengths (decode_plan_len),
                               // written by workgroup 0
  float scale;
  int num_seqs, Hq, Hkv, g, bs, max_blocks, num_wg, causal;
  int max_rows;                // 16 or 32: most query rows of one (request, kv head) on this path,
                               // and the rows of a workspace slot
  int window;                  // > 0: row i of a request also drops keys j < len - qlen + i - window + 1
  int bs_shift;                // log2(bs): block sizes are powers of two
};

// First key any row of a request with qlen new rows and len keys may see (the sliding window's
// lower bound of its first row; 0 without a window).
__device__ __forceinline__ int decode_key_begin(const PagedParams& p, int len, int qlen) {
  return p.window > 0 ? max(0, len - qlen - p.window + 1) : 0;
}

// Chunk count of request b on this path (0 when its rows belong to another path or it has
// no new rows): the chunks from the first visible key to the last key, per kv head.
template <int CH>
__device__ __forceinline__ int decode_chunks(const PagedParams& p, int b) {
  const int len = p.seq_lens_k[b];
  const int qlen = p.cu_seqlens_q ? (p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b]) : 1;
  const int rows = qlen * p.g;
  if (!(rows > 0 && rows <= p.max_rows)) return 0;
  // chunks from the one holding the first visible key (chunk indices of a unit count from there)
  return (len + CH - 1) / CH - decode_key_begin(p, len, qlen) / CH;
}

// Share planning. The batch's work is the request-major list of (request, kv head) units. In
// the plan a unit of 0 < nb < kPieceCostUnits chunks is kPieceCost + nb long: its first
// kPieceCost places stand for the fixed cost of starting a piece of it (the cross-wave combine
// and the block-table and K/V latency before its first chunk: about 1.9 us, 1.5 chunks of 64
// tokens, measured as the extra time of a share per extra piece), and the next nb are its chunks.
// Shares are equal parts of the planned list, so a share that crosses more short units streams
// fewer chunks. Longer units span many shares, where the few extra pieces matter less than
// keeping the list's length (shares are cut in groups of 4 places, and a share's time follows its
// groups: one extra group in a share of 8 is an eighth longer).
constexpr int kPieceCost = 2;
constexpr int kPieceCostUnits = 256;
__device__ __forceinline__ int decode_plan_len(int nb) {
  return (nb > 0 && nb < kPieceCostUnits) ? nb + kPieceCost : nb;
}

// First place of workgroup g's share of T planned places: shares are whole groups of 4 places,
// as equal as possible.
__device__ __forceinline__ long long share_start(long long g, long long T, int G) {
  const long long quads = (T + 3) / 4;
  const long long s = 4 * ((g * quads) / G);
  return s < T ? s : T;
}
// The workgroup whose share holds place x (0 <= x < T).
__device__ __forceinline__ int share_of(long long x, long long T, int G) {
  const long long quads = (T + 3) / 4;
  return (int)(((x / 4 + 1) * G + quads - 1) / quads - 1);
}

template <int NU>
struct DecodeShape {
  static_assert(NU == 2 || NU == 4, "a chunk is one or two 32-token halves");
  static constexpr int CH = 16 * NU;   // tokens per wave iteration
  static constexpr int NH = NU / 2;    // 32-token halves per chunk
};

// One piece of a (request, kv head) unit: places [u0, u1) of the unit's ul planned places (see
// the share planning above), i.e. its chunks [c0, c1); the waves start at chunk c0 + first[w] and
// step by NW chunks. Returns the number of chunks (0: the places hold none, and nothing is done).
// Rows of a request on this path: r -> (new token r / g, query head kvh*g + r % g). A piece that
// is the whole unit is written to out/lse; else it goes to partial slot 0 (the share's first
// piece with a chunk, `first`) or 1 of the workspace. LONGV: V page rows are longer than one
// 32-token half (block size > 32), which decides how the V loads are issued. NR: blocks of 16
// rows (1, or 2 for up to 32 rows: several new tokens of a request at group size 4 and up); each K
// and V operand is loaded and converted once and feeds the MFMAs of every row block.
template <int D, int KVT, int NU, bool LONGV, int NW, int NR = 1>
__device__ __forceinline__ int decode_piece(const PagedParams& p, int b, int kvh, int u0, int u1, int ul,
                                            int wave_first, int share, bool first, float* lds) {
  constexpr int CH = DecodeShape<NU>::CH;
  constexpr int NH = DecodeShape<NU>::NH;
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
  const int kc0 = decode_key_begin(p, len, qlen) / CH;   // chunk c of the unit is key chunk kc0 + c
  const int nb = (len + CH - 1) / CH - kc0;              // the unit's chunks (decode_chunks)
  const int cost = ul - nb;                              // its planned places before them
  const int c0 = max(0, u0 - cost), c1 = max(0, u1 - cost);   // empty: see below
  const bool direct = c0 == 0 && c1 == nb;
  const int slot = direct ? -1 : (first ? 0 : 1);
  const int t_end = min(len, (kc0 + c1) * CH);

  float kscale = 1.f, vscale = 1.f;
  if (KVT == KV_FP8) { kscale = p.k_scale[kvh]; vscale = p.v_scale[kvh]; }
  const float c = p.scale * kscale * kLog2e;           // base-2 exponent per raw score unit
  constexpr float kLazyRescale = 8.f;                  // see the running statistics below

  // ---- Q^T operands (B of the QK MFMA): lane (j, qd) holds Q[row 16 rb + j][d-slots].
  bf16x8 qB[NR][KK];
  int limit[NR];                                      // last visible key of row 16 rb + j
  int lower[NR];                                      // first visible key of row 16 rb + j
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
    const int r = 16 * rb + j;
    const int i = (r < R) ? r / p.g : 0;
    limit[rb] = p.causal ? (len - qlen + i) : (len - 1);
    lower[rb] = p.window > 0 ? (len - qlen + i - p.window + 1) : INT_MIN;
    if (r < R) {
      const int h = kvh * p.g + (r % p.g);
      const bf16* qrow = p.q + ((size_t)(q0 + i) * p.Hq + h) * D;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        // bf16 cache: natural d order; fp8 cache: d = 64*(kk/2) + 16*qd + 8*(kk%2), so one
        // 16-byte fp8 load feeds two MFMAs. Q uses the same order as K.
        const int d0 = (KVT == KV_BF16) ? (32 * kk + 8 * qd) : (64 * (kk >> 1) + 16 * qd + 8 * (kk & 1));
        qB[rb][kk] = *reinterpret_cast<const bf16x8*>(qrow + d0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qB[rb][kk] = bf16x8{};
    }
  }
  // An empty asm redefines the Q registers: their loads are waited for here, once, so the
  // chunk loop never waits on the memory counter for them (which would also wait for the
  // chunk's own K/V loads issued after them).
#pragma unroll
  for (int rb = 0; rb < NR; ++rb)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(qB[rb][kk]));
  // A piece whose places hold no chunk returns here, after the Q loads (which do not wait for the
  // request's length, so they are in flight together with it).
  if (c1 <= c0) return 0;

  // Running statistics of row j, in the base-2 exponent domain t = c * s: mc is a reference
  // maximum (the same in all four quads), l this lane's share of sum 2^(t - mc). The reference
  // is only moved when a row's maximum exceeds it by more than kLazyRescale (so P <= 2^8 and
  // the O rescale is skipped on almost every chunk); any reference gives the same result.
  float mc[NR], l[NR];
  f32x4 acc[NR][NB];        // O^T[16n + 4qd + r][row 16 rb + j], scaled by 2^-mc
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
    mc[rb] = kNegInf;
    l[rb] = 0.f;
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[rb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t page_bytes = (size_t)p.bs * D * ELT;   // bytes per (block, kv head) page
  const int32_t* table = p.block_table + (size_t)b * p.max_blocks;
  const char* kc = reinterpret_cast<const char*>(p.k_cache) + (size_t)kvh * page_bytes;
  const char* vc = reinterpret_cast<const char*>(p.v_cache) + (size_t)kvh * page_bytes;
  const size_t block_stride = (size_t)p.Hkv * page_bytes;
  const int last_tok = len - 1;
  const int min_limit = p.causal ? (len - qlen) : (len - 1);   // smallest last-visible key of any row
  const int max_lower = p.window > 0 ? (len - p.window) : INT_MIN;  // largest first-visible key of any row

  // Token layout of a chunk: in half h (32 tokens), lane quad q owns the 8-token run
  // T0 + 32h + 8q .. +7, and score slot s of sub-tile u = 2h + e is token T0 + 32h + 8q + 4e + s.
  // A K lane j loads the run of quad j/4, a V lane the run of its own quad. Runs past the end of
  // the request read its last page instead (and are masked). Within a page the run starts at
  // slot (T0 + 32h) % bs + 8q % bs (T0 is a multiple of 64 and bs of 16).
  // token -> (page, slot) by shift and mask (block sizes are powers of two; every token index
  // here is non-negative)
  const int bmask = p.bs - 1;
  const int kq8 = (8 * (j >> 2)) & bmask;
  const int vq8 = (8 * qd) & bmask;
  auto k_block = [&](int T0, int h) { return min(T0 + 32 * h + 8 * (j >> 2), last_tok) >> p.bs_shift; };
  auto v_block = [&](int T0, int h) { return min(T0 + 32 * h + 8 * qd, last_tok) >> p.bs_shift; };

  int T0 = (kc0 + c0 + wave_first) * CH;
  int kphys[NH], vphys[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) kphys[h] = vphys[h] = 0;
  if (T0 < t_end) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      kphys[h] = table[k_block(T0, h)];
      vphys[h] = table[v_block(T0, h)];
    }
  }

  constexpr int KW = (KVT == KV_BF16) ? KK : KK / 2;    // 16-byte K loads per key row
  typedef typename std::conditional<KVT == KV_BF16, u32x4, u32x2>::type vword;
  for (; T0 < t_end; T0 += NW * CH) {
    // ---------------- issue the K and V loads of this chunk
    u32x4 kraw[NU][KW];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int kslot = ((T0 + 32 * h) & bmask) + kq8;  // an 8-token run never crosses a page
      const char* krun = kc + (size_t)kphys[h] * block_stride + (size_t)kslot * D * ELT;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const char* krow = krun + (4 * e + (j & 3)) * D * ELT;
#pragma unroll
        for (int w = 0; w < KW; ++w)
          kraw[2 * h + e][w] = (KVT == KV_BF16) ? ld16(krow + (32 * w + 8 * qd) * 2) : ld16(krow + 64 * w + 16 * qd);
      }
    }
    // V: 8 consecutive tokens of one d row per lane and d block (16 bytes bf16, 8 bytes fp8).
    // The V stream is read once, so its loads are nontemporal where every line they touch is
    // read whole by loads issued back to back: with block size <= 32 a half covers whole page
    // rows; with longer rows the two halves of a chunk share each line and are issued in pairs.
    // With one half per chunk the rest of each line belongs to another chunk: plain loads.
    vword vraw[NH][NB];
    const char* vrun[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int vslot = ((T0 + 32 * h) & bmask) + vq8;
      vrun[h] = vc + (size_t)vphys[h] * block_stride + ((size_t)j * p.bs + vslot) * ELT;
    }
    auto vload = [&](int h, int n, bool nt) {
      const char* vrow = vrun[h] + (size_t)16 * n * p.bs * ELT;
      if constexpr (KVT == KV_BF16) vraw[h][n] = nt ? ld16nt(vrow) : ld16(vrow);
      else vraw[h][n] = nt ? ld8nt(vrow) : ld8(vrow);
    };
    // With head_dim 256, bf16 pages and 8 waves (256 registers per lane), the second half of the
    // V loads is issued after the QK products, in the registers the K rows leave free.
    constexpr int NB_EARLY = (D == 256 && KVT == KV_BF16 && NW == 8) ? NB / 2 : NB;
    if constexpr (!LONGV) {
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int n = 0; n < NB_EARLY; ++n) vload(h, n, true);
    } else {
#pragma unroll
      for (int n = 0; n < NB_EARLY; ++n)
#pragma unroll
        for (int h = 0; h < NH; ++h) vload(h, n, NH == 2);
    }
    // ---------------- block-table entries of this wave's next chunk
    const int Tn = T0 + NW * CH;
    if (Tn < t_end) {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        kphys[h] = table[k_block(Tn, h)];
        vphys[h] = table[v_block(Tn, h)];
      }
    }

    // ---------------- S^T = K . Q^T for the NU sub-tiles, in exponent units t = c * s.
    f32x4 st[NR][NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      f32x4 a[NR];
#pragma unroll
      for (int rb = 0; rb < NR; ++rb) a[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (KVT == KV_BF16) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 ka = bitcast<bf16x8>(kraw[u][kk]);
#pragma unroll
          for (int rb = 0; rb < NR; ++rb) a[rb] = mfma_16x16x32(ka, qB[rb][kk], a[rb]);
        }
      } else {
#pragma unroll
        for (int w = 0; w < KW; ++w) {
          const bf16x8 k0 = fp8x8_to_bf16x8(kraw[u][w][0], kraw[u][w][1]);
          const bf16x8 k1 = fp8x8_to_bf16x8(kraw[u][w][2], kraw[u][w][3]);
#pragma unroll
          for (int rb = 0; rb < NR; ++rb) {
            a[rb] = mfma_16x16x32(k0, qB[rb][2 * w], a[rb]);
            a[rb] = mfma_16x16x32(k1, qB[rb][2 * w + 1], a[rb]);
          }
        }
      }
#pragma unroll
      for (int rb = 0; rb < NR; ++rb) st[rb][u] = a[rb] * c;
    }
    if constexpr (NB_EARLY < NB) {
#pragma unroll
      for (int n = NB_EARLY; n < NB; ++n)
#pragma unroll
        for (int h = 0; h < NH; ++h) vload(h, n, !LONGV || NH == 2);
    }
    // A chunk is a tail chunk when some row may not see all of its keys (the end of the request,
    // the causal edge of a multi-token request, or the start of a sliding window). Only tail chunks mask scores, zero V slots
    // past the end, and carry P as hi + lo bf16 parts: there rows see few keys, so the rounding
    // of P would not average out.
    const bool tail = (T0 + CH - 1 > min_limit) || (T0 < max_lower);
    if (tail) {
#pragma unroll
      for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int tok0 = T0 + 32 * (u >> 1) + 8 * qd + 4 * (u & 1);
#pragma unroll
          for (int s = 0; s < 4; ++s)
            st[rb][u][s] = (tok0 + s <= limit[rb] && tok0 + s >= lower[rb]) ? st[rb][u][s] : kNegInf;
        }
    }
    float base[NR];
#pragma unroll
    for (int rb = 0; rb < NR; ++rb) {
      float mloc = kNegInf;
#pragma unroll
      for (int u = 0; u < NU; ++u)
        mloc = fmaxf(fmaxf(mloc, fmaxf(st[rb][u][0], st[rb][u][1])), fmaxf(st[rb][u][2], st[rb][u][3]));
      mloc = max_over_quads(mloc);
      // Move the reference (and rescale what was accumulated) only where the new maximum is
      // more than kLazyRescale above it; the first visible chunk of a row always moves it.
      const bool move = mloc > mc[rb] + kLazyRescale;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        const float alpha = move ? ((mc[rb] == kNegInf) ? 0.f : fast_exp2(mc[rb] - mloc)) : 1.f;
        mc[rb] = move ? mloc : mc[rb];
        l[rb] *= alpha;
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[rb][n] *= alpha;
      }
      base[rb] = (mc[rb] == kNegInf) ? 0.f : mc[rb];
    }

    // ---------------- P = 2^(t - mc), running sum, O^T += V^T . P^T (16x16x32 per d block, half)
    if (!tail) {
      bf16x8 pB[NR][NH];
#pragma unroll
      for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int t = 0; t < 8; t += 2) {
            const float e0 = fast_exp2(st[rb][2 * h + (t >> 2)][t & 3] - base[rb]);
            const float e1 = fast_exp2(st[rb][2 * h + (t >> 2)][(t & 3) + 1] - base[rb]);
            l[rb] += e0 + e1;
            pB[rb][h][t] = (bf16)e0;
            pB[rb][h][t + 1] = (bf16)e1;
          }
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          bf16x8 va;
          if constexpr (KVT == KV_BF16) va = bitcast<bf16x8>(vraw[h][n]);
          else va = fp8x8_to_bf16x8(vraw[h][n][0], vraw[h][n][1]);
#pragma unroll
          for (int rb = 0; rb < NR; ++rb) acc[rb][n] = mfma_16x16x32(va, pB[rb][h], acc[rb][n]);
        }
    } else {
      bf16x8 pB[NR][NH], pL[NR][NH];
#pragma unroll
      for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float e = fast_exp2(st[rb][2 * h + (t >> 2)][t & 3] - base[rb]);
            l[rb] += e;
            pB[rb][h][t] = (bf16)e;
            pL[rb][h][t] = (bf16)(e - (float)pB[rb][h][t]);
          }
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        // Keys past the end of the request are zeroed in V (their P is zero, but the slots may
        // hold anything, including NaN).
        const int vvalid = len - (T0 + 32 * h + 8 * qd);  // tokens of the lane's run that exist
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          bf16x8 va;
          if constexpr (KVT == KV_BF16) va = bitcast<bf16x8>(vraw[h][n]);
          else va = fp8x8_to_bf16x8(vraw[h][n][0], vraw[h][n][1]);
#pragma unroll
          for (int t = 0; t < 8; ++t) va[t] = (t < vvalid) ? va[t] : (bf16)0.f;
#pragma unroll
          for (int rb = 0; rb < NR; ++rb) {
            acc[rb][n] = mfma_16x16x32(va, pB[rb][h], acc[rb][n]);
            acc[rb][n] = mfma_16x16x32(va, pL[rb][h], acc[rb][n]);
          }
        }
      }
    }
  }

  // ---------------- combine the NW waves (fixed order) through LDS.
  // lds layout: stats[2][NW][16 NR] (reference maximum, sum) then O[NW][R][D].
  constexpr int SR = 16 * NR;
  float* smax = lds;
  float* ssum = lds + NW * SR;
  float* so = lds + 2 * NW * SR;
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
    const float l_row = sum_over_quads(l[rb]);
    if (qd == 0) {
      smax[wave * SR + 16 * rb + j] = mc[rb];
      ssum[wave * SR + 16 * rb + j] = l_row;
    }
  }
  __syncthreads();
  float mx[NR], ltot[NR];
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
    const int r = 16 * rb + j;
    mx[rb] = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx[rb] = fmaxf(mx[rb], smax[w * SR + r]);
    const float mbase = (mx[rb] == kNegInf) ? 0.f : mx[rb];
    ltot[rb] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = smax[w * SR + r];
      ltot[rb] += (mw == kNegInf) ? 0.f : ssum[w * SR + r] * fast_exp2(mw - mbase);
    }
    const float own = (mc[rb] == kNegInf || ltot[rb] == 0.f) ? 0.f : fast_exp2(mc[rb] - mbase) * vscale / ltot[rb];
    if (r < R) {
      float* dst = so + ((size_t)wave * R + r) * D;
#pragma unroll
      for (int n = 0; n < NB; ++n) *reinterpret_cast<f32x4*>(dst + 16 * n + 4 * qd) = acc[rb][n] * own;
    }
  }
  __syncthreads();

  float row_lse[NR];
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) row_lse[rb] = (ltot[rb] == 0.f) ? kNegInf : kLn2 * (mx[rb] + fast_log2(ltot[rb]));
  if (direct) {
    for (int idx = tid; idx < R * (D / 4); idx += NW * 64) {
      const int r = idx / (D / 4), d4 = 4 * (idx - r * (D / 4));
      f32x4 o = *reinterpret_cast<const f32x4*>(so + (0 * R + r) * D + d4);
#pragma unroll
      for (int w = 1; w < NW; ++w) o += *reinterpret_cast<const f32x4*>(so + (w * R + r) * D + d4);
      const int i = r / p.g, h = kvh * p.g + r % p.g;
      *reinterpret_cast<bf16x4*>(p.out + ((size_t)(q0 + i) * p.Hq + h) * D + d4) = f32x4_to_bf16x4(o);
    }
#pragma unroll
    for (int rb = 0; rb < NR; ++rb) {
      const int r = 16 * rb + j;
      if (p.lse && wave == 0 && qd == 0 && r < R) {
        const int i = r / p.g, h = kvh * p.g + r % p.g;
        p.lse[(size_t)(q0 + i) * p.Hq + h] = row_lse[rb];
      }
    }
    return c1 - c0;
  }
  const size_t unit = (size_t)share * 2 + slot;
  float* wo = p.ws_o + unit * p.max_rows * D;
  for (int idx = tid; idx < R * (D / 4); idx += NW * 64) {
    const int r = idx / (D / 4), d4 = 4 * (idx - r * (D / 4));
    f32x4 o = *reinterpret_cast<const f32x4*>(so + (0 * R + r) * D + d4);
#pragma unroll
    for (int w = 1; w < NW; ++w) o += *reinterpret_cast<const f32x4*>(so + (w * R + r) * D + d4);
    *reinterpret_cast<f32x4*>(wo + r * D + d4) = o;
  }
#pragma unroll
  for (int rb = 0; rb < NR; ++rb)
    if (wave == 0 && qd == 0 && 16 * rb + j < R) p.ws_lse[unit * p.max_rows + 16 * rb + j] = row_lse[rb];
  return c1 - c0;
}

// Exclusive prefix sums of count(b) over requests b < B into sp[0 .. B] (LDS); threads 0-255 scan
// contiguous segments of requests (any further threads of the workgroup have empty segments);
// wave_tot holds one int per wave of the workgroup. Ends with a barrier.
template <class Count>
__device__ __forceinline__ void block_prefix(int B, Count count, int* sp, int* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (B + 255) / 256;
  const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += count(b);
  int incl = local;                                    // inclusive scan over the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int off = incl - local;
  for (int w = 0; w < wave; ++w) off += wave_tot[w];
  for (int b = b0; b < b1; ++b) {
    sp[b] = off;
    off += count(b);
  }
  if (tid == 255) sp[B] = off;
  __syncthreads();
}

// The partition kernel's body for a workgroup of NW waves: share g of the batch's chunks walks the
// (request, kv head) pieces it covers. lds: the combine buffer of decode_piece
// (decode_combine_floats), then sp[B + 1] and NW scratch ints.
template <int D, int NW, int NR = 1>
constexpr int decode_combine_floats(int rows) { return 2 * NW * 16 * NR + NW * rows * D; }

template <int D, int KVT, int NU, bool LONGV, int NW = 4, int NR = 1>
__device__ __forceinline__ void decode_share(const PagedParams& p, float* lds, int combine_floats, int g) {
  constexpr int CH = DecodeShape<NU>::CH;
  int* sp = reinterpret_cast<int*>(lds + combine_floats);
  int* wave_tot = sp + p.num_seqs + 1;
  block_prefix(p.num_seqs, [&](int b) { return decode_plan_len(decode_chunks<CH>(p, b)); }, sp, wave_tot);
  const int B = p.num_seqs, G = p.num_wg;
  if (g == 0)
    for (int b = threadIdx.x; b <= B; b += NW * 64) p.ws_prefix[b] = sp[b];
  const long long T = (long long)p.Hkv * sp[B];
  const long long r0 = share_start(g, T, G), r1 = share_start(g + 1, T, G);
  if (r0 >= r1) return;
  // request holding place r0: the largest b < B with Hkv * sp[b] <= r0
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((long long)p.Hkv * sp[mid] <= r0) lo = mid; else hi = mid - 1;
  }
  int b = lo;
  long long pos = r0;
  int dealt = 0;                       // chunks of the share so far
  bool first = true;
  const int wave = threadIdx.x >> 6;
  while (pos < r1) {
    const int ul = sp[b + 1] - sp[b];  // planned length of each unit of request b
    if (ul == 0) { ++b; continue; }
    const long long base = (long long)p.Hkv * sp[b];
    const int kvh = (int)((pos - base) / ul);
    const int u0 = (int)(pos - base - (long long)kvh * ul);        // places of the unit in the share:
    const int u1 = (int)min((long long)ul, u0 + (r1 - pos));      // [u0, u1)
    // chunks are dealt to the waves round-robin over the whole share
    const int wave_first = ((wave - dealt) % NW + NW) % NW;
    const int n = decode_piece<D, KVT, NU, LONGV, NW, NR>(p, b, kvh, u0, u1, ul, wave_first, g, first, lds);
    dealt += n;
    first = first && n == 0;
    pos += u1 - u0;
    if (u1 == ul && kvh == p.Hkv - 1) ++b;
  }
}

// Merge of the pieces of one (request, kv head, row) that spans several shares, with
// natural-log LSE weights ("Attention kernels", section "Prefill and decode attention": partial
// results combined the same way as the online softmax). Also writes out = 0, lse = -inf for
// rows of a request with no key. Latency-bound, so it takes two dependent memory round trips:
// the chunk offsets, then every piece's LSE and partial output together. Thread t handles d-quad
// t % (D/4) of the pieces t / (D/4) + k * 256/(D/4) (eight in flight) and folds them into a
// running (max, sum, output); the thread groups are then combined in LDS in a fixed order.
// lds: per group its maximum and sum, then its output row.
template <int D, int CH>
__device__ __forceinline__ void merge_row(const PagedParams& p, int b, int kvh, int r, float* lds) {
  constexpr int DQ = D / 4;
  constexpr int GROUPS = 256 / DQ;
  const int q0 = p.cu_seqlens_q ? p.cu_seqlens_q[b] : b;
  const int qlen = p.cu_seqlens_q ? (p.cu_seqlens_q[b + 1] - q0) : 1;
  const int R = qlen * p.g;
  if (R > p.max_rows || r >= R) return;                // rows of another path, or no such row
  const int tid = threadIdx.x;
  const int i = r / p.g, h = kvh * p.g + r % p.g;
  bf16* orow = p.out + ((size_t)(q0 + i) * p.Hq + h) * D;
  const int ul = p.ws_prefix[b + 1] - p.ws_prefix[b];  // planned length of the unit
  const int nb = decode_chunks<CH>(p, b);
  if (nb == 0) {                                       // no key at all
    if (tid < DQ) *reinterpret_cast<bf16x4*>(orow + 4 * tid) = bf16x4{};
    if (p.lse && tid == 0) p.lse[(size_t)(q0 + i) * p.Hq + h] = kNegInf;
    return;
  }
  const int G = p.num_wg;
  const long long T = (long long)p.Hkv * p.ws_prefix[p.num_seqs];
  const long long ustart = (long long)p.Hkv * p.ws_prefix[b] + (long long)kvh * ul;   // the unit's places
  const long long start = ustart + (ul - nb);          // its first chunk
  const int g_lo = share_of(start, T, G), g_hi = share_of(start + nb - 1, T, G);
  if (g_lo == g_hi) return;                            // written directly by the partition kernel
  const int ns = g_hi - g_lo + 1;
  // piece k lives in share g_lo + k: slot 0 (the unit is that share's first unit with a chunk)
  // except for the first piece when share g_lo began before the unit's places, where it holds the
  // last chunk of an earlier unit first. Empty shares (when there are fewer place groups than
  // shares) hold no piece and are skipped.
  const int slot_lo = (share_start(g_lo, T, G) >= ustart) ? 0 : 1;
  const int dq = tid % DQ, grp = tid / DQ;
  float M = kNegInf, S = 0.f;
  f32x4 O = f32x4{0.f, 0.f, 0.f, 0.f};
  // FULL: every share holds at least one group of 4 places (at least as many groups as shares),
  // so no piece needs the 64-bit divisions of the emptiness test; the choice is uniform.
  auto fold = [&](auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;
    for (int k0 = grp; k0 < ns; k0 += 8 * GROUPS) {
      float lk[8];
      f32x4 ok[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u * GROUPS;
        const int gk = g_lo + k;
        const bool has = k < ns && (FULL || share_start(gk, T, G) < share_start(gk + 1, T, G));
        const size_t piece = (size_t)gk * 2 + (k == 0 ? slot_lo : 0);
        lk[u] = has ? p.ws_lse[piece * p.max_rows + r] : kNegInf;
        ok[u] = has ? *reinterpret_cast<const f32x4*>(p.ws_o + (piece * p.max_rows + r) * D + 4 * dq)
                    : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (lk[u] == kNegInf) continue;
        const float m2 = fmaxf(M, lk[u]);
        const float a = (M == kNegInf) ? 0.f : fast_exp2((M - m2) * kLog2e);
        const float w = fast_exp2((lk[u] - m2) * kLog2e);
        S = S * a + w;
        O = O * a + ok[u] * w;
        M = m2;
      }
    }
  };
  if ((T + 3) / 4 >= G) fold(std::true_type{});
  else fold(std::false_type{});
  float* gstat = lds;                                  // [GROUPS][2]: maximum, sum
  float* gout = lds + 2 * GROUPS;                      // [GROUPS][D]
  if (dq == 0) {
    gstat[2 * grp] = M;
    gstat[2 * grp + 1] = S;
  }
  *reinterpret_cast<f32x4*>(gout + grp * D + 4 * dq) = O;
  __syncthreads();
  if (grp == 0) {
    float mt = kNegInf;
#pragma unroll
    for (int g2 = 0; g2 < GROUPS; ++g2) mt = fmaxf(mt, gstat[2 * g2]);
    float st = 0.f;
    f32x4 ot = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g2 = 0; g2 < GROUPS; ++g2) {
      const float mg = gstat[2 * g2];
      if (mg == kNegInf) continue;
      const float w = fast_exp2((mg - mt) * kLog2e);
      st += gstat[2 * g2 + 1] * w;
      ot += *reinterpret_cast<const f32x4*>(gout + g2 * D + 4 * dq) * w;
    }
    const float inv = (st > 0.f) ? 1.f / st : 0.f;
    *reinterpret_cast<bf16x4*>(orow + 4 * dq) = f32x4_to_bf16x4(ot * inv);
    if (p.lse && dq == 0)
      p.lse[(size_t)(q0 + i) * p.Hq + h] = (st > 0.f) ? mt + kLn2 * fast_log2(st) : kNegInf;
  }
}

}  // namespace attn
