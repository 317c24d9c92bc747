// Prefill and mixed-batch kernel instantiations and launchers.
#include "launch.h"
#include "prefill_pp.h"
#include "prefill_pp256.h"

namespace attn {

// Varlen self-attention over contiguous K/V with head_dim 256 (head_dim 128 takes the ping-pong
// kernel below). Grid: (head groups, requests, q-tiles), q-tiles walked heaviest (last) first.
// Two workgroups per compute unit (two waves per SIMD, so one wave's softmax overlaps the
// other's MFMAs) when the head dimension leaves room in the register file.
template <int D>
constexpr int prefill_waves_per_eu() { return D <= 128 ? 2 : 1; }

template <int D, int BN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(prefill_waves_per_eu<D>(), prefill_waves_per_eu<D>())))
void prefill_varlen_kernel(PrefillParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  prefill_tile_body<D, BN, ContigLoader<D, BN>, false>(p, reinterpret_cast<bf16*>(smem_raw), blockIdx.x,
                                                        blockIdx.y, p.num_qtiles - 1 - (int)blockIdx.z);
}

// Varlen self-attention over contiguous K/V with head_dim 128: the ping-pong kernel (8 waves,
// 96 KB of LDS: three 16 KB buffers each of K and V; one workgroup per compute unit); a q-tile is
// 32 * 8 / hpw rows. One-dimensional grid over (head group, request, q-tile). The dispatcher deals
// workgroup i to XCD i % 8; when the (head group, request) pairs are a multiple of 8, XCD x takes
// pairs x, x + 8, ... one after the other, each pair's q-tiles heaviest first, so that the
// workgroups an XCD runs at once stream the same K/V tiles through its L2. Otherwise the order is
// (head group, request) fastest, q-tiles heaviest first.
template <int BN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_pingpong_kernel(PrefillParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int id = blockIdx.x;
  const int HG = p.Hkv * (p.g / p.hpw), Z = p.num_qtiles;
  const int P = HG * p.num_seqs;
  int pair, t;
  if (P % 8 == 0) {
    const int k = id >> 3;
    pair = (id & 7) + 8 * (k / Z);
    t = k % Z;
  } else {
    pair = id % P;
    t = id / P;
  }
  prefill_pingpong_body<BN>(p, smem_raw, pair % HG, pair / HG, Z - 1 - t);
}

// Q-tiles of request b on the prefill path of a mixed batch (its rows per KV head exceed
// max_rows, the most the decode path takes).
__device__ __forceinline__ int prefill_qtiles(const PrefillParams& p, int b, int tq, int max_rows) {
  const int lq = p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b];
  return (lq * p.g > max_rows) ? (lq + tq - 1) / tq : 0;
}

// Mixed varlen batch over a paged cache in one launch: workgroups [0, n_dec) are the decode
// path's shares (memory-bound; dispatched first so that they run beside the prefill tiles), the
// rest are prefill q-tiles (compute-bound), heaviest tile of each request first.
template <int D, int BN, int KVT, int NU, bool LONGV, int NR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(prefill_waves_per_eu<D>(), prefill_waves_per_eu<D>())))
void varlen_mixed_kernel(PrefillParams pp, PagedParams dp, int n_dec,
                                                           int combine_floats) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float* lds = reinterpret_cast<float*>(smem_raw);
  if ((int)blockIdx.x < n_dec) {
    decode_share<D, KVT, NU, LONGV, 4, NR>(dp, lds, combine_floats, blockIdx.x);
    return;
  }
  using Loader = PagedLoader<D, BN, KVT == KV_FP8>;
  const int w = blockIdx.x - n_dec;
  const int hg = pp.Hkv * (pp.g / pp.hpw);
  const int hgrp = w % hg, t = w / hg;
  const int tq = 32 * (4 / pp.hpw);
  int* sp = reinterpret_cast<int*>(smem_raw + PrefillShape<D, BN>::LDS_BYTES);
  block_prefix(pp.num_seqs, [&](int b) { return prefill_qtiles(pp, b, tq, dp.max_rows); }, sp, sp + pp.num_seqs + 1);
  if (t >= sp[pp.num_seqs]) return;
  int lo = 0, hi = pp.num_seqs - 1;                    // the largest b with sp[b] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sp[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int nt = sp[lo + 1] - sp[lo];
  const int qt = nt - 1 - (t - sp[lo]);
  __syncthreads();                                     // sp is not read below; the tile reuses LDS
  prefill_tile_body<D, BN, Loader, true>(pp, reinterpret_cast<bf16*>(smem_raw), hgrp, lo, qt);
}

// Mixed varlen batch over a paged cache with head_dim 256: the same one-launch split with 8 waves
// per workgroup. Decode-share workgroups deal their chunks to 8 waves; prefill workgroups run the
// ping-pong tile of prefill_pp256.h (128 query rows, two waves per SIMD).
template <int KVT, int NU, bool LONGV>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void varlen_mixed256_kernel(PrefillParams pp, PagedParams dp, int n_dec, int combine_floats) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float* lds = reinterpret_cast<float*>(smem_raw);
  if ((int)blockIdx.x < n_dec) {
    decode_share<256, KVT, NU, LONGV, 8>(dp, lds, combine_floats, blockIdx.x);
    return;
  }
  const int w = blockIdx.x - n_dec;
  const int hg = pp.Hkv * (pp.g / pp.hpw);
  const int hgrp = w % hg, t = w / hg;
  const int tq = 32 * (4 / pp.hpw);
  int* sp = reinterpret_cast<int*>(smem_raw + PingPong256Shape<KVT == KV_FP8>::LDS_BYTES);
  block_prefix(pp.num_seqs, [&](int b) { return prefill_qtiles(pp, b, tq, dp.max_rows); }, sp, sp + pp.num_seqs + 1);
  if (t >= sp[pp.num_seqs]) return;
  int lo = 0, hi = pp.num_seqs - 1;                    // the largest b with sp[b] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sp[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int nt = sp[lo + 1] - sp[lo];
  const int qt = nt - 1 - (t - sp[lo]);
  __syncthreads();                                     // sp is not read below; the tile reuses LDS
  prefill_pp256_body<KVT == KV_FP8>(pp, smem_raw, hgrp, lo, qt);
}

template <int D, int BN>
static hipError_t launch_prefill_t(const PrefillParams& p, int max_seqlen, hipStream_t stream) {
  using S = PrefillShape<D, BN>;
  static std::atomic<bool> done[kMaxDevices];
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&prefill_varlen_kernel<D, BN>), done, S::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int tq = 32 * (4 / p.hpw);
  PrefillParams q = p;
  q.num_qtiles = (max_seqlen + tq - 1) / tq;
  if (q.num_qtiles <= 0) return hipSuccess;
  dim3 grid(p.Hkv * (p.g / p.hpw), p.num_seqs, q.num_qtiles);
  return launch_kernel(&prefill_varlen_kernel<D, BN>, grid, dim3(256), S::LDS_BYTES, stream, q);
}

template <int BN>
static hipError_t launch_pingpong_t(const PrefillParams& p, int max_seqlen, hipStream_t stream) {
  using S = PingPongShape<BN>;
  static std::atomic<bool> done[kMaxDevices];
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&prefill_pingpong_kernel<BN>), done, S::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int tq = 32 * (8 / p.hpw);
  PrefillParams q = p;
  q.num_qtiles = (max_seqlen + tq - 1) / tq;
  if (q.num_qtiles <= 0) return hipSuccess;
  const long long n = (long long)p.Hkv * (p.g / p.hpw) * p.num_seqs * q.num_qtiles;
  if (n > 0x7fffffffLL) return hipErrorInvalidValue;
  return launch_kernel(&prefill_pingpong_kernel<BN>, dim3((unsigned)n), dim3(512), S::LDS_BYTES, stream, q);
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, int max_seqlen, hipStream_t stream) {
  if (head_dim == 128) return launch_pingpong_t<64>(p, max_seqlen, stream);
  if (head_dim == 256) return launch_prefill_t<256, 64>(p, max_seqlen, stream);
  return hipErrorInvalidValue;
}

// Rows per (request, kv head) that the decode role of the mixed kernel takes at most: 32 with
// head_dim 128 (two 16-row blocks; their combine buffer fits beside the prefill tiles), 16 with
// head_dim 256 (8 waves' combine buffer of 32 rows would not fit the LDS).
template <int D>
constexpr int mixed_max_rows() { return D == 128 ? 32 : 16; }

// Dynamic LDS of the mixed kernel: the larger of the prefill tile buffers and the decode combine
// buffer of its NW waves (for the most rows it takes), then num_seqs + 1 + NW ints (prefix sums and
// per-wave scratch). Head_dim 128: 4 waves and the tiles of prefill_core.h; head_dim 256: 8 waves
// and the tiles of prefill_pp256.h (the same for both cache dtypes).
template <int D>
static size_t mixed_lds_bytes(int num_seqs) {
  constexpr int NW = D == 256 ? 8 : 4;
  constexpr int NR = mixed_max_rows<D>() / 16;
  const size_t tiles = D == 256 ? (size_t)PingPong256Shape<false>::LDS_BYTES : (size_t)PrefillShape<D, 64>::LDS_BYTES;
  const size_t combine = (size_t)decode_combine_floats<D, NW, NR>(16 * NR) * sizeof(float);
  return std::max(tiles, combine) + ((size_t)num_seqs + 1 + NW) * sizeof(int);
}

// Largest request count whose mixed-kernel LDS fits the 160 KB a workgroup may hold.
constexpr long long kMaxWorkgroupLds = 160 * 1024;
template <int D>
static int mixed_max_seqs_t() {
  const long long base = (long long)mixed_lds_bytes<D>(0);
  return (int)std::min<long long>((kMaxWorkgroupLds - base) / 4, kMaxPagedSeqs);
}

int mixed_max_seqs(int head_dim) {
  return head_dim == 128 ? mixed_max_seqs_t<128>() : mixed_max_seqs_t<256>();
}

// NR: 16-row blocks of the decode role (dp.max_rows / 16).
template <int D, int BN, int KVT, int NU, bool LONGV, int NR>
static hipError_t launch_mixed_t(const PrefillParams& pp, const PagedParams& dp, int total_q, hipStream_t stream) {
  static_assert(16 * NR <= mixed_max_rows<D>(), "the decode role's rows fit its combine buffer");
  const int tq = 32 * (4 / pp.hpw);
  // upper bound on prefill q-tiles: every request adds at most one partial tile
  const long long n_pre = (long long)pp.Hkv * (pp.g / pp.hpw) * ((total_q + tq - 1) / tq + pp.num_seqs);
  const int n_dec = dp.num_wg;
  if (n_pre + n_dec > 0x7fffffffLL) return hipErrorInvalidValue;
  // both kernels' LDS limits are raised before the first launch
  static std::atomic<bool> done[kMaxDevices];
  const void* fn;
  if constexpr (D == 256) fn = reinterpret_cast<const void*>(&varlen_mixed256_kernel<KVT, NU, LONGV>);
  else fn = reinterpret_cast<const void*>(&varlen_mixed_kernel<D, BN, KVT, NU, LONGV, NR>);
  hipError_t e = ensure_dynamic_lds(fn, done, (int)mixed_lds_bytes<D>(mixed_max_seqs_t<D>()));
  if (e != hipSuccess) return e;
  e = ensure_merge_attrs(D, NU);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(n_pre + n_dec));
  const size_t lds = mixed_lds_bytes<D>(pp.num_seqs);
  if constexpr (D == 256) {
    e = launch_kernel(&varlen_mixed256_kernel<KVT, NU, LONGV>, grid, dim3(512), lds, stream, pp, dp, n_dec,
                      decode_combine_floats<256, 8, NR>(16 * NR));
  } else {
    e = launch_kernel(&varlen_mixed_kernel<D, BN, KVT, NU, LONGV, NR>, grid, dim3(256), lds, stream, pp, dp, n_dec,
                      decode_combine_floats<D, 4, NR>(16 * NR));
  }
  if (e != hipSuccess) return e;
  return launch_decode_merge(dp, D, NU, dp.max_rows, stream);
}

template <int D, int BN, int KVT, int NU, int NR>
static hipError_t launch_mixed_nr(const PrefillParams& pp, const PagedParams& dp, int total_q, hipStream_t stream) {
  return dp.bs > 32 ? launch_mixed_t<D, BN, KVT, NU, true, NR>(pp, dp, total_q, stream)
                    : launch_mixed_t<D, BN, KVT, NU, false, NR>(pp, dp, total_q, stream);
}

template <int D, int BN, int KVT, int NU>
static hipError_t launch_mixed_bs(const PrefillParams& pp, const PagedParams& dp, int total_q, hipStream_t stream) {
  // two row blocks take 32-token chunks (NU = 2), so that their registers fit beside the prefill
  // role's two waves per SIMD
  if constexpr (mixed_max_rows<D>() >= 32) {
    if (dp.max_rows > 16) return launch_mixed_nr<D, BN, KVT, 2, 2>(pp, dp, total_q, stream);
  }
  if (dp.max_rows != 16) return hipErrorInvalidValue;
  return launch_mixed_nr<D, BN, KVT, NU, 1>(pp, dp, total_q, stream);
}

hipError_t launch_mixed(const PrefillParams& pp, const PagedParams& dp, int head_dim, int kv_type, int total_q,
                        hipStream_t stream) {
  if (head_dim == 128 && kv_type == KV_BF16) return launch_mixed_bs<128, 64, KV_BF16, 4>(pp, dp, total_q, stream);
  if (head_dim == 256 && kv_type == KV_BF16) return launch_mixed_bs<256, 32, KV_BF16, 2>(pp, dp, total_q, stream);
  if (head_dim == 128 && kv_type == KV_FP8) return launch_mixed_bs<128, 64, KV_FP8, 4>(pp, dp, total_q, stream);
  if (head_dim == 256 && kv_type == KV_FP8) return launch_mixed_bs<256, 32, KV_FP8, 2>(pp, dp, total_q, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
