// Paged decode kernel instantiations and launchers.
#include "launch.h"

namespace attn {

template <int D, int KVT, int NU, bool LONGV>
__global__ __launch_bounds__(256) void decode_share_kernel(PagedParams p, int combine_floats) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  decode_share<D, KVT, NU, LONGV>(p, reinterpret_cast<float*>(smem_raw), combine_floats, blockIdx.x);
}

template <int D, int CH>
__global__ __launch_bounds__(256) void decode_merge_kernel(PagedParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  merge_row<D, CH>(p, blockIdx.z, blockIdx.y, blockIdx.x, reinterpret_cast<float*>(smem_raw));
}

// Dynamic LDS of the partition kernel (4 waves): the statistics and the waves' O rows, then the
// chunk prefix sums (num_seqs + 1) and one scratch int per wave.
template <int D>
static size_t decode_lds_bytes(int rows_max, int num_seqs) {
  return (size_t)decode_combine_floats<D, 4>(rows_max) * sizeof(float) + ((size_t)num_seqs + 5) * sizeof(int);
}

template <int D>
static size_t merge_lds_bytes() {
  return (size_t)(256 / (D / 4)) * (D + 2) * sizeof(float);
}

template <int D, int CH>
static hipError_t ensure_merge_t() {
  static std::atomic<bool> done[kMaxDevices];
  return ensure_dynamic_lds(reinterpret_cast<const void*>(&decode_merge_kernel<D, CH>), done,
                            (int)merge_lds_bytes<D>());
}

hipError_t ensure_merge_attrs(int head_dim, int nu) {
  if (head_dim == 128 && nu == 4) return ensure_merge_t<128, 64>();
  if (head_dim == 128 && nu == 2) return ensure_merge_t<128, 32>();
  if (head_dim == 256 && nu == 4) return ensure_merge_t<256, 64>();
  if (head_dim == 256 && nu == 2) return ensure_merge_t<256, 32>();
  return hipErrorInvalidValue;
}

// The dynamic-LDS limits of the partition kernel (its largest launch: 16 rows, the most requests a
// paged call takes) and of the merge kernel, raised once per device before either is launched.
template <int D, int KVT, int NU, bool LONGV>
static hipError_t ensure_decode_attrs() {
  static std::atomic<bool> done[kMaxDevices];
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&decode_share_kernel<D, KVT, NU, LONGV>),
                                    done, (int)decode_lds_bytes<D>(16, kMaxPagedSeqs));
  if (e != hipSuccess) return e;
  return ensure_merge_t<D, DecodeShape<NU>::CH>();
}

template <int D, int KVT, int NU, bool LONGV>
static hipError_t launch_decode_t(const PagedParams& p, int rows_max, hipStream_t stream) {
  hipError_t e = ensure_decode_attrs<D, KVT, NU, LONGV>();
  if (e != hipSuccess) return e;
  const int combine_floats = decode_combine_floats<D, 4>(rows_max);
  e = launch_kernel(&decode_share_kernel<D, KVT, NU, LONGV>, dim3(p.num_wg), dim3(256),
                    decode_lds_bytes<D>(rows_max, p.num_seqs), stream, p, combine_floats);
  if (e != hipSuccess) return e;
  return launch_decode_merge(p, D, NU, rows_max, stream);
}

template <int D, int CH>
static hipError_t launch_merge_t(const PagedParams& p, int rows_max, hipStream_t stream) {
  hipError_t e = ensure_merge_t<D, CH>();
  if (e != hipSuccess) return e;
  dim3 mgrid(rows_max, p.Hkv, p.num_seqs);
  return launch_kernel(&decode_merge_kernel<D, CH>, mgrid, dim3(256), merge_lds_bytes<D>(), stream, p);
}

hipError_t launch_decode_merge(const PagedParams& p, int head_dim, int nu, int rows_max, hipStream_t stream) {
  if (head_dim == 128 && nu == 4) return launch_merge_t<128, 64>(p, rows_max, stream);
  if (head_dim == 128 && nu == 2) return launch_merge_t<128, 32>(p, rows_max, stream);
  if (head_dim == 256 && nu == 4) return launch_merge_t<256, 64>(p, rows_max, stream);
  if (head_dim == 256 && nu == 2) return launch_merge_t<256, 32>(p, rows_max, stream);
  return hipErrorInvalidValue;
}

template <int D, int KVT, int NU>
static hipError_t launch_decode_bs(const PagedParams& p, int rows_max, hipStream_t stream) {
  return p.bs > 32 ? launch_decode_t<D, KVT, NU, true>(p, rows_max, stream)
                   : launch_decode_t<D, KVT, NU, false>(p, rows_max, stream);
}

hipError_t launch_decode(const PagedParams& p, int head_dim, int kv_type, int rows_max, hipStream_t stream) {
  if (head_dim == 128 && kv_type == KV_BF16) return launch_decode_bs<128, KV_BF16, 4>(p, rows_max, stream);
  if (head_dim == 256 && kv_type == KV_BF16) return launch_decode_bs<256, KV_BF16, 2>(p, rows_max, stream);
  if (head_dim == 128 && kv_type == KV_FP8) return launch_decode_bs<128, KV_FP8, 4>(p, rows_max, stream);
  if (head_dim == 256 && kv_type == KV_FP8) return launch_decode_bs<256, KV_FP8, 2>(p, rows_max, stream);
  return hipErrorInvalidValue;
}

int decode_chunk_tokens(int head_dim, int kv_type) {
  (void)kv_type;
  return head_dim == 128 ? DecodeShape<4>::CH : DecodeShape<2>::CH;
}

template <int D, int KVT, int NU>
static int wgs_per_cu_t() {
  // Resident partition workgroups per compute unit (the register-limited occupancy of the
  // variant; the smaller of its two V-load forms), queried once per device; a failed query
  // leaves no pending error and counts as 1.
  static std::atomic<int> cache[kMaxDevices];
  const int dev = current_device_index();
  if (dev >= 0) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = INT_MAX;
  for (const void* fn : {reinterpret_cast<const void*>(&decode_share_kernel<D, KVT, NU, false>),
                         reinterpret_cast<const void*>(&decode_share_kernel<D, KVT, NU, true>)}) {
    int m = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&m, fn, 256, 16 * 1024) != hipSuccess || m < 1) {
      (void)hipGetLastError();
      m = 1;
    }
    n = std::min(n, m);
  }
  if (dev >= 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

int decode_wgs_per_cu(int head_dim, int kv_type) {
  if (head_dim == 128 && kv_type == KV_BF16) return wgs_per_cu_t<128, KV_BF16, 4>();
  if (head_dim == 256 && kv_type == KV_BF16) return wgs_per_cu_t<256, KV_BF16, 2>();
  if (head_dim == 128 && kv_type == KV_FP8) return wgs_per_cu_t<128, KV_FP8, 4>();
  if (head_dim == 256 && kv_type == KV_FP8) return wgs_per_cu_t<256, KV_FP8, 2>();
  return 1;
}

}  // namespace attn
