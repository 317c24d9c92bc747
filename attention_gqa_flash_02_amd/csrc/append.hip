// Paged KV-cache append: new tokens' K rows and V columns scattered into their cache slots.
//
// What it computes ("Optimization 1: batching and attention", section 3.4 PagedAttention; "Attention
// kernels", section "Paged KV and kernels"): request b's n_b new tokens become its cached tokens
// seq_lens_k[b] - n_b .. seq_lens_k[b] - 1; token t lands in slot t % bs of physical block
// block_table[b][t / bs]: K as the row [block][h][slot][:], V as the column [block][h][:][slot]
// (the V page keeps tokens innermost, which is what the attention kernels read). An fp8 cache
// stores e4m3fn(x / scale[h]): the quotient in correctly rounded fp32, clamped to +-448, converted
// with round-to-nearest-even.
//
// Work layout: a workgroup takes 64 consecutive new-token rows of one kv head. Waves 1-3 load
// those rows' K and V (32 contiguous bytes per thread and item); these loads do not depend on where
// the rows land. Wave 0 meanwhile finds each row's request (a coarse sample of cu_seqlens_new, then,
// for more than 255 requests, the window that holds the first row, and a search in LDS) and cache
// slot; it loads no K or V itself, since a wave's loads return in order and its three dependent
// lookups would otherwise wait behind them. Then:
//   * K: every row's K row is one contiguous byte range of its page ([bs][D]); each thread converts
//     the 16 bf16 values of each of its items into one 16-byte fp8 store (or stores them as two
//     16-byte bf16 pieces).
//   * V: the rows go to LDS and are written column-wise, the page being [D][bs] (tokens innermost).
//     A 16-slot chunk of a page whose 16 slots are all new rows of one request is written whole:
//     (chunk, head_dim pair) items, one 16-byte piece per d row (two for a bf16 cache). A chunk cut
//     by the boundary between two workgroups is written whole by the first of them, which reads
//     the rows past its range from the new V rows directly; the second one leaves those rows out.
//     Every other row (the first and last rows of a request that share a chunk with cached
//     tokens, a decode token) is written element by element, so that no slot outside the new rows
//     is touched.
#include <type_traits>

#include "launch.h"

namespace attn {

namespace {

constexpr int kAppendRows = 64;    // new-token rows per workgroup

// largest b in [0, B) with cu[b] <= row (the request holding new-token row `row`)
__device__ int request_of_row_global(const int32_t* cu, int B, int row) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// x / s in fp32, correctly rounded. FAST: without a division per value (Markstein's method,
// "Handbook of Floating-Point Arithmetic", division by a correctly rounded reciprocal): with
// r = 1/s correctly rounded, q = x r is within one ulp of x / s, the residual q s - x is exact in
// one fma, and q - (q s - x) r rounded once is the correctly rounded quotient, as long as nothing
// under- or overflows. The caller takes FAST only for scales in [2^-60, 2^60]: the e4m3 code
// depends on the exact quotient only for |x / s| from 2^-10 (half the smallest subnormal) up,
// where then |x| >= 2^-70 and the residual stays a normal number. Quotients past 1024 only need
// their sign (they saturate to 448): q is clamped there first, so nothing overflows to a NaN.
// Written as q - (q s - x) r, a zero x keeps its sign.
template <bool FAST>
__device__ __forceinline__ float quotient(float x, float s, float r) {
  if constexpr (!FAST) {
    return x / s;
  } else {
    const float q = __builtin_amdgcn_fmed3f(x * r, -1024.f, 1024.f);
    return __builtin_fmaf(-__builtin_fmaf(q, s, -x), r, q);
  }
}

// fp32 -> e4m3fn codes of x / s for 4 values (saturated at 448), packed little-endian into one word
template <bool FAST>
__device__ __forceinline__ uint32_t quant4(float x0, float x1, float x2, float x3, float s, float r) {
  const float q0 = __builtin_amdgcn_fmed3f(quotient<FAST>(x0, s, r), -448.f, 448.f);
  const float q1 = __builtin_amdgcn_fmed3f(quotient<FAST>(x1, s, r), -448.f, 448.f);
  const float q2 = __builtin_amdgcn_fmed3f(quotient<FAST>(x2, s, r), -448.f, 448.f);
  const float q3 = __builtin_amdgcn_fmed3f(quotient<FAST>(x3, s, r), -448.f, 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace

template <int D, bool FP8>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
  constexpr int ELT = FP8 ? 1 : 2;
  constexpr int IPR = D / 16;                  // 32-byte source items (16 bf16 values) per row
  constexpr int NITEM = kAppendRows * IPR;     // items of a workgroup
  constexpr int LT = 192;                      // loading threads: waves 1-3 (wave 0 finds the slots)
  constexpr int ITEMS = (NITEM + LT - 1) / LT; // items per loading thread
  constexpr int HD = D / 2;                    // head_dim pairs
  constexpr int VS = D + 2;                    // LDS row stride of the staged V rows (bf16)
  static_assert(kAppendRows == 64, "wave 0 holds one row per lane");
  __shared__ int s_cu[257];
  __shared__ int s_sl[256];                    // seq_lens_k, with at most 255 requests
  __shared__ int s_req[kAppendRows];           // request of each row
  __shared__ int s_pos[kAppendRows];           // cache position of each row
  __shared__ long long s_page[kAppendRows];    // (block, head) page index of each row
  __shared__ int s_full[kAppendRows];          // first row of each whole 16-slot chunk
  __shared__ int s_prow[kAppendRows];          // the rows outside whole chunks
  __shared__ int s_cnt[4];         // whole chunks, other rows, rows left to the previous workgroup,
                                   // first row of the chunk finished past the range (or -1)
  __shared__ __align__(16) bf16 s_v[kAppendRows * VS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int h = blockIdx.y;
  // row blocks from the last one: a batch's single-token (decode) rows usually come last, and
  // their scattered V columns make theirs the slowest workgroups, so they start first
  const int row0 = ((int)gridDim.x - 1 - (int)blockIdx.x) * kAppendRows;
  const int nrows = min(kAppendRows, p.total_new - row0);
  const int B = p.num_seqs;
  const size_t row_stride = (size_t)p.Hkv * D;              // elements between consecutive new rows

  // ---- the rows' K and V into the registers of waves 1-3: item i = lt + 192 u is row i / IPR,
  // values 16 (i % IPR) .. + 15. Wave 0 loads none: a wave's loads return in order, so its search
  // below (three dependent loads) does not wait behind them.
  const bf16* __restrict__ knew = p.k_new;
  const bf16* __restrict__ vnew = p.v_new;
  const int lt = tid - 64;                     // loading thread, negative in wave 0
  u32x4 kin[ITEMS][2], vin[ITEMS][2];
  if (lt >= 0) {
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const int i = min(lt + LT * u, NITEM - 1), r = min(i / IPR, nrows - 1), c = i % IPR;
      const size_t off = (size_t)(row0 + r) * row_stride + (size_t)h * D + 16 * c;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        kin[u][q] = *reinterpret_cast<const u32x4*>(knew + off + 8 * q);
        vin[u][q] = *reinterpret_cast<const u32x4*>(vnew + off + 8 * q);
      }
    }
  }

  // ---- requests of the rows: coarse sample, then the window holding the first row (one round
  // when the whole cu_seqlens_new fits the sample)
  const int step = (B + 256) / 256;            // ceil((B + 1) / 256) requests per sample
  if (tid < 64) {
#pragma unroll
    for (int k = 0; k < 4; ++k) s_cu[tid + 64 * k] = p.cu_seqlens_new[min((tid + 64 * k) * step, B)];
    if (tid == 0) s_cu[256] = p.cu_seqlens_new[B];
    if (step == 1) {                           // then seq_lens_k fits too: one lookup fewer below
#pragma unroll
      for (int k = 0; k < 4; ++k) s_sl[tid + 64 * k] = p.seq_lens_k[min(tid + 64 * k, B - 1)];
    }
  }
  __syncthreads();
  int base = 0;
  if (step > 1) {
    int lo = 0, hi = 255;                      // largest sample t with cu[t * step] <= row0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (mid * step <= B && s_cu[mid] <= row0) lo = mid; else hi = mid - 1;
    }
    base = lo * step;
    __syncthreads();
    if (tid < 64) {
#pragma unroll
      for (int k = 0; k < 4; ++k) s_cu[tid + 64 * k] = p.cu_seqlens_new[min(base + tid + 64 * k, B)];
      if (tid == 0) s_cu[256] = p.cu_seqlens_new[min(base + 256, B)];
    }
    __syncthreads();
  }
  if (tid < nrows) {
    const int row = row0 + tid;
    int b, c0, c1;
    if (row < s_cu[256] || base + 256 >= B) {  // inside the window: search it in LDS
      int l2 = 0, h2 = min(256, B - 1 - base);   // l2 <= 255 here, so s_cu[l2 + 1] exists
      while (l2 < h2) {
        const int mid = (l2 + h2 + 1) >> 1;
        if (s_cu[mid] <= row) l2 = mid; else h2 = mid - 1;
      }
      b = base + l2;
      c0 = s_cu[l2];
      c1 = s_cu[l2 + 1];
    } else {
      b = request_of_row_global(p.cu_seqlens_new, B, row);
      c0 = p.cu_seqlens_new[b];
      c1 = p.cu_seqlens_new[b + 1];
    }
    const int pos = (step == 1 ? s_sl[b] : p.seq_lens_k[b]) - (c1 - c0) + (row - c0);
    const int blk = p.block_table[(size_t)b * p.max_blocks + pos / p.bs];
    s_req[tid] = b;
    s_pos[tid] = pos;
    s_page[tid] = (long long)blk * p.Hkv + h;
    // The 16-slot chunk across the boundary before global row x (a row of request [c0, c1) at
    // position px) is written whole by the workgroup before the boundary when the boundary cuts it
    // (px not a chunk start, row x - 1 of the same request) and all its 16 slots are new rows of
    // the request. Both workgroups take the same decision from the same numbers.
    auto cut_whole = [&](int x, int px) {
      const int cs = x - (px & 15);                       // global row of the chunk's first slot
      return (px & 15) != 0 && c0 < x && cs >= c0 && cs + 15 < c1;
    };
    if (tid == 0) s_cnt[2] = cut_whole(row, pos) ? 16 - (pos & 15) : 0;
    if (tid == nrows - 1) {
      // the boundary after this workgroup: row + 1 (only with a full range; a shorter one is the
      // grid's last workgroup)
      const int x = row + 1;
      s_cnt[3] = (nrows == kAppendRows && x < c1 && cut_whole(x, pos + 1)) ? tid + 1 - ((pos + 1) & 15) : -1;
    }
  }
  // ---- V rows into LDS
  if (lt >= 0) {
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const int i = lt + LT * u, r = i / IPR, c = i % IPR;
      if (i >= NITEM) break;
      bf16* dst = s_v + r * VS + 16 * c;
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int w = 0; w < 4; ++w) *reinterpret_cast<uint32_t*>(dst + 8 * q + 2 * w) = vin[u][q][w];
    }
  }
  __syncthreads();
  // a row lies in a whole chunk when the 16 rows of its 16-slot chunk are all new rows of this
  // workgroup and of its request (then their positions are consecutive and fill the chunk)
  // Rows below `head` belong to a cut chunk the previous workgroup writes; rows from `tail` on to a
  // cut chunk this one finishes past its range.
  const int head = s_cnt[2], tail = s_cnt[3];
  bool whole = false, whole_start = false;
  if (tid < nrows) {
    const int i0 = tid - (s_pos[tid] & 15);
    whole = i0 >= 0 && i0 + 15 < nrows && s_req[i0] == s_req[tid] && s_req[i0 + 15] == s_req[tid];
    whole_start = whole && i0 == tid;
  }
  const bool other = tid < nrows && !whole && tid >= head && !(tail >= 0 && tid >= tail);
  // compact the whole-chunk starts and the other rows (the rows are held by wave 0)
  const uint64_t mw = __builtin_amdgcn_ballot_w64(whole_start);
  const uint64_t mp = __builtin_amdgcn_ballot_w64(other);
  if (tid == 0) {
    s_cnt[0] = __builtin_popcountll(mw);
    s_cnt[1] = __builtin_popcountll(mp);
  }
  if (whole_start)
    s_full[__builtin_amdgcn_mbcnt_hi((uint32_t)(mw >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mw, 0))] = tid;
  if (other)
    s_prow[__builtin_amdgcn_mbcnt_hi((uint32_t)(mp >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mp, 0))] = tid;
  __syncthreads();
  const int nfull = s_cnt[0];
  const int npart = s_cnt[1];

  // ---- the stores. Quantisation without a division per value needs scales in [2^-60, 2^60]
  // (see quotient); the choice is uniform over the workgroup.
  const float ks = FP8 ? p.k_scale[h] : 1.f, vs = FP8 ? p.v_scale[h] : 1.f;
  const float kr = 1.f / ks, vr = 1.f / vs;
  auto in_range = [](float x) { return x >= 0x1p-60f && x <= 0x1p60f; };
  auto emit = [&](auto fast_c) {
    constexpr bool F = decltype(fast_c)::value;
    // ---- K: each item (16 values of one row) becomes one 16-byte fp8 piece or two bf16 pieces
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const int i = lt + LT * u, r = i / IPR, c = i % IPR;
      if (lt < 0 || i >= NITEM || r >= nrows) continue;
      char* dst = reinterpret_cast<char*>(p.k_cache) +
                  (((size_t)s_page[r] * p.bs + (s_pos[r] & (p.bs - 1))) * D + 16 * c) * ELT;
      if constexpr (!FP8) {
        *reinterpret_cast<u32x4*>(dst) = kin[u][0];
        *reinterpret_cast<u32x4*>(dst + 16) = kin[u][1];
      } else {
        const u32x4 a = kin[u][0], e = kin[u][1];
        u32x4 o;
        o[0] = quant4<F>(bf16_lo(a[0]), bf16_hi(a[0]), bf16_lo(a[1]), bf16_hi(a[1]), ks, kr);
        o[1] = quant4<F>(bf16_lo(a[2]), bf16_hi(a[2]), bf16_lo(a[3]), bf16_hi(a[3]), ks, kr);
        o[2] = quant4<F>(bf16_lo(e[0]), bf16_hi(e[0]), bf16_lo(e[1]), bf16_hi(e[1]), ks, kr);
        o[3] = quant4<F>(bf16_lo(e[2]), bf16_hi(e[2]), bf16_lo(e[3]), bf16_hi(e[3]), ks, kr);
        *reinterpret_cast<u32x4*>(dst) = o;
      }
    }

    // ---- V, whole chunks: (chunk, head_dim pair) items. w: bf16 pairs (d, d + 1) of the 16 rows;
    // i0: the chunk's first row in this workgroup
    auto write_chunk = [&](int i0, int d, const uint32_t (&w)[16]) {
      const size_t e0 = ((size_t)s_page[i0] * D + d) * p.bs + (s_pos[i0] & (p.bs - 1));   // (d, first slot)
      if constexpr (!FP8) {
        bf16* v0 = reinterpret_cast<bf16*>(p.v_cache) + e0;
        bf16* v1 = v0 + p.bs;                                   // the d + 1 row
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          u32x4 lo4, hi4;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t x0 = w[8 * q + 2 * c], x1 = w[8 * q + 2 * c + 1];
            lo4[c] = (x0 & 0xffffu) | (x1 << 16);               // d row: slots 2c, 2c + 1
            hi4[c] = (x0 >> 16) | (x1 & 0xffff0000u);           // d + 1 row
          }
          *reinterpret_cast<u32x4*>(v0 + 8 * q) = lo4;
          *reinterpret_cast<u32x4*>(v1 + 8 * q) = hi4;
        }
      } else {
        uint8_t* v0 = reinterpret_cast<uint8_t*>(p.v_cache) + e0;
        uint32_t q0[4], q1[4];                                  // codes of the d and d + 1 rows
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          q0[c] = quant4<F>(bf16_lo(w[4 * c]), bf16_lo(w[4 * c + 1]), bf16_lo(w[4 * c + 2]), bf16_lo(w[4 * c + 3]), vs, vr);
          q1[c] = quant4<F>(bf16_hi(w[4 * c]), bf16_hi(w[4 * c + 1]), bf16_hi(w[4 * c + 2]), bf16_hi(w[4 * c + 3]), vs, vr);
        }
        *reinterpret_cast<u32x4*>(v0) = u32x4{q0[0], q0[1], q0[2], q0[3]};
        *reinterpret_cast<u32x4*>(v0 + p.bs) = u32x4{q1[0], q1[1], q1[2], q1[3]};
      }
    };
    for (int it = tid; it < nfull * HD; it += 256) {
      const int i0 = s_full[it / HD], d = 2 * (it % HD);
      uint32_t w[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) w[t] = *reinterpret_cast<const uint32_t*>(s_v + (i0 + t) * VS + d);
      write_chunk(i0, d, w);
    }
    // ---- V, the chunk cut by the end of the range: its rows past the range come from the new
    // rows in memory
    if (tail >= 0) {
      for (int d2 = tid; d2 < HD; d2 += 256) {
        const int d = 2 * d2;
        uint32_t w[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int r = tail + t;
          w[t] = r < kAppendRows
                     ? *reinterpret_cast<const uint32_t*>(s_v + r * VS + d)
                     : *reinterpret_cast<const uint32_t*>(vnew + (size_t)(row0 + r) * row_stride + (size_t)h * D + d);
        }
        write_chunk(tail, d, w);
      }
    }

    // ---- V, the other rows: (row, head_dim pair) items
    for (int it = tid; it < npart * HD; it += 256) {
      const int r = s_prow[it / HD], d = 2 * (it % HD);
      const uint32_t w = *reinterpret_cast<const uint32_t*>(s_v + r * VS + d);
      const size_t e0 = ((size_t)s_page[r] * D + d) * p.bs + (s_pos[r] & (p.bs - 1));
      if constexpr (!FP8) {
        reinterpret_cast<uint16_t*>(p.v_cache)[e0] = (uint16_t)(w & 0xffffu);
        reinterpret_cast<uint16_t*>(p.v_cache)[e0 + p.bs] = (uint16_t)(w >> 16);
      } else {
        const uint32_t q = quant4<F>(bf16_lo(w), bf16_hi(w), 0.f, 0.f, vs, vr);
        reinterpret_cast<uint8_t*>(p.v_cache)[e0] = (uint8_t)(q & 0xffu);
        reinterpret_cast<uint8_t*>(p.v_cache)[e0 + p.bs] = (uint8_t)((q >> 8) & 0xffu);
      }
    }
  };
  if (in_range(ks) && in_range(vs)) emit(std::true_type{});
  else emit(std::false_type{});
  (void)lane;
}

template <int D, bool FP8>
static hipError_t launch_append_t(const AppendParams& p, hipStream_t stream) {
  dim3 grid((p.total_new + kAppendRows - 1) / kAppendRows, p.Hkv);
  return launch_kernel(&kv_append_kernel<D, FP8>, grid, dim3(256), 0, stream, p);
}

hipError_t launch_append(const AppendParams& p, int head_dim, int kv_type, hipStream_t stream) {
  if (p.total_new <= 0) return hipSuccess;
  if (head_dim == 128) return kv_type == KV_FP8 ? launch_append_t<128, true>(p, stream) : launch_append_t<128, false>(p, stream);
  if (head_dim == 256) return kv_type == KV_FP8 ? launch_append_t<256, true>(p, stream) : launch_append_t<256, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
