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

template <int D, int KVT, int NU, bool LONGV>
static hipError_t launch_decode_t(const PagedParams& p, int rows_max, hipStream_t stream) {
  // partition kernel LDS: 128 floats of statistics, four waves' O rows, then the chunk prefix
  // sums and 4 scratch ints
  const int combine_floats = 128 + 4 * rows_max * D;
  const size_t lds = (size_t)combine_floats * sizeof(float) + ((size_t)p.num_seqs + 5) * sizeof(int);
  // the dynamic-LDS limit of each kernel is raised to the largest size launched so far
  static size_t lds_set = 0;
  if (lds > lds_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_share_kernel<D, KVT, NU, LONGV>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_set = lds;
  }
  hipLaunchKernelGGL((decode_share_kernel<D, KVT, NU, LONGV>), dim3(p.num_wg), dim3(256), lds, stream, p, combine_floats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_merge(p, D, NU, rows_max, stream);
}

template <int D, int CH>
static hipError_t launch_merge_t(const PagedParams& p, int rows_max, hipStream_t stream) {
  const size_t merge_lds = (size_t)(256 / (D / 4)) * (D + 2) * sizeof(float);
  static size_t merge_lds_set = 0;
  if (merge_lds > merge_lds_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_merge_kernel<D, CH>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)merge_lds);
    if (e != hipSuccess) return e;
    merge_lds_set = merge_lds;
  }
  dim3 mgrid(rows_max, p.Hkv, p.num_seqs);
  hipLaunchKernelGGL((decode_merge_kernel<D, CH>), mgrid, dim3(256), merge_lds, stream, p);
  return hipGetLastError();
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
  // variant; the smaller of its two V-load forms), queried once; a failed query leaves no
  // pending error and counts as 1.
  static int cached = 0;
  if (cached > 0) return cached;
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
  cached = n;
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
