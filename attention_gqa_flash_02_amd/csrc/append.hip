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
// Work layout: a workgroup takes 32 consecutive new-token rows of one kv head. Their K and V rows
// are loaded into registers first, while the rows' requests are found: a coarse sample of
// cu_seqlens_new, then (for more than 255 requests) the window that holds the first row, and a
// search in LDS. K rows are written 16 bytes per thread; V rows are staged in LDS and written
// column-wise, consecutive lanes taking consecutive tokens so that each d row of a page is
// written as one contiguous run.
#include "launch.h"

namespace attn {

namespace {

constexpr int kAppendRows = 32;

// largest b in [0, B) with cu[b] <= row (the request holding new-token row `row`)
__device__ int request_of_row_global(const int32_t* cu, int B, int row) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// fp32 -> e4m3fn codes of x / s for 4 values, packed little-endian into one word
__device__ __forceinline__ uint32_t quant4(float x0, float x1, float x2, float x3, float s) {
  const float q0 = fminf(fmaxf(x0 / s, -448.f), 448.f);
  const float q1 = fminf(fmaxf(x1 / s, -448.f), 448.f);
  const float q2 = fminf(fmaxf(x2 / s, -448.f), 448.f);
  const float q3 = fminf(fmaxf(x3 / s, -448.f), 448.f);
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
  constexpr int CPR = D / 8;                   // 16-byte chunks of a bf16 row
  constexpr int OCH = D * ELT / 16;            // 16-byte output chunks of a cache row
  constexpr int IPO = 16 / ELT / 8;            // 16-byte input chunks per output chunk (2 for fp8)
  constexpr int KPT = kAppendRows * OCH / 256; // K output chunks per thread
  constexpr int VPT = kAppendRows * CPR / 256; // V input chunks per thread
  static_assert(kAppendRows * OCH % 256 == 0 && kAppendRows * CPR % 256 == 0, "whole chunks per thread");
  __shared__ int s_cu[257];
  __shared__ long long s_kdst[kAppendRows];   // byte offset of each row's K slot
  __shared__ long long s_vdst[kAppendRows];   // element offset of each row's V column (d = 0)
  __shared__ __align__(16) bf16 s_v[kAppendRows][D];
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int row0 = blockIdx.x * kAppendRows;
  const int nrows = min(kAppendRows, p.total_new - row0);
  const int B = p.num_seqs;

  // ---- the new K and V rows go into registers first: these loads do not depend on where the
  // rows land, so they are in flight while the requests and cache slots are looked up
  u32x4 kin[KPT][IPO], vin[VPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int idx = tid + 256 * i, r = idx / OCH, ch = idx % OCH;
    const bf16* src = p.k_new + ((size_t)(row0 + r) * p.Hkv + h) * D + IPO * 8 * ch;
#pragma unroll
    for (int u = 0; u < IPO; ++u)
      kin[i][u] = r < nrows ? *reinterpret_cast<const u32x4*>(src + 8 * u) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = tid + 256 * i, r = idx / CPR, ch = idx % CPR;
    const bf16* src = p.v_new + ((size_t)(row0 + r) * p.Hkv + h) * D + 8 * ch;
    vin[i] = r < nrows ? *reinterpret_cast<const u32x4*>(src) : u32x4{0, 0, 0, 0};
  }

  // ---- requests of the 32 rows: coarse sample, then the window holding the first row (one round
  // when the whole cu_seqlens_new fits the sample)
  const int step = (B + 256) / 256;            // ceil((B + 1) / 256) requests per sample
  s_cu[tid] = p.cu_seqlens_new[min(tid * step, B)];
  if (tid == 0) s_cu[256] = p.cu_seqlens_new[B];
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
    s_cu[tid] = p.cu_seqlens_new[min(base + tid, B)];
    if (tid == 0) s_cu[256] = p.cu_seqlens_new[min(base + 256, B)];
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
    const int pos = p.seq_lens_k[b] - (c1 - c0) + (row - c0);
    const int blk = p.block_table[(size_t)b * p.max_blocks + pos / p.bs];
    const int slot = pos % p.bs;
    s_kdst[tid] = (((long long)blk * p.Hkv + h) * p.bs + slot) * D * ELT;
    s_vdst[tid] = ((long long)blk * p.Hkv + h) * D * p.bs + slot;
  }
  // ---- V rows into LDS
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = tid + 256 * i, r = idx / CPR, ch = idx % CPR;
    *reinterpret_cast<u32x4*>(&s_v[r][8 * ch]) = vin[i];
  }
  __syncthreads();

  // ---- K rows: 16 output bytes per thread per chunk
  const float ks = FP8 ? p.k_scale[h] : 1.f;
  char* kc = reinterpret_cast<char*>(p.k_cache);
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int idx = tid + 256 * i, r = idx / OCH, ch = idx % OCH;
    if (r >= nrows) continue;
    char* dst = kc + s_kdst[r] + 16 * ch;
    if constexpr (!FP8) {
      *reinterpret_cast<u32x4*>(dst) = kin[i][0];
    } else {
      const u32x4 a = kin[i][0], c = kin[i][IPO - 1];
      u32x4 o;
      o[0] = quant4(bf16_lo(a[0]), bf16_hi(a[0]), bf16_lo(a[1]), bf16_hi(a[1]), ks);
      o[1] = quant4(bf16_lo(a[2]), bf16_hi(a[2]), bf16_lo(a[3]), bf16_hi(a[3]), ks);
      o[2] = quant4(bf16_lo(c[0]), bf16_hi(c[0]), bf16_lo(c[1]), bf16_hi(c[1]), ks);
      o[3] = quant4(bf16_lo(c[2]), bf16_hi(c[2]), bf16_lo(c[3]), bf16_hi(c[3]), ks);
      *reinterpret_cast<u32x4*>(dst) = o;
    }
  }

  // ---- V columns: lane r % 32 takes token r, so a d row's tokens are written side by side
  const float vs = FP8 ? p.v_scale[h] : 1.f;
  const int r = tid % kAppendRows;
  if (r < nrows) {
    const long long vdst = s_vdst[r];
    for (int d = tid / kAppendRows; d < D; d += 256 / kAppendRows) {
      const bf16 x = s_v[r][d];
      if constexpr (!FP8) {
        reinterpret_cast<bf16*>(p.v_cache)[vdst + (long long)d * p.bs] = x;
      } else {
        const float q = fminf(fmaxf((float)x / vs, -448.f), 448.f);
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(q, q, 0, false);
        reinterpret_cast<uint8_t*>(p.v_cache)[vdst + (long long)d * p.bs] = (uint8_t)(w & 0xff);
      }
    }
  }
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
