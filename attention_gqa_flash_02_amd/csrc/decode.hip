// Paged decode kernel instantiations and launchers.
#include "launch.h"

namespace attn {

template <int D, int KVT, int NU>
__global__ __launch_bounds__(256) void decode_split_kernel(PagedParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  decode_unit<D, KVT, NU>(p, blockIdx.z, blockIdx.y, blockIdx.x, reinterpret_cast<float*>(smem_raw));
}

template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(PagedParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  merge_row<D>(p, blockIdx.z, blockIdx.y, blockIdx.x, reinterpret_cast<float*>(smem_raw));
}

// Partition kernel LDS: 128 floats of statistics plus four waves' O rows.
static size_t decode_lds_bytes(int rows_max, int head_dim) {
  return (128 + 4 * (size_t)rows_max * head_dim) * sizeof(float);
}

template <int D, int KVT, int NU>
static hipError_t launch_decode_t(const PagedParams& p, int rows_max, hipStream_t stream) {
  static bool attr_set = false;  // per process; the attribute is a property of the function
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_split_kernel<D, KVT, NU>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)decode_lds_bytes(16, D));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid(p.num_splits, p.Hkv, p.num_seqs);
  hipLaunchKernelGGL((decode_split_kernel<D, KVT, NU>), grid, dim3(256), decode_lds_bytes(rows_max, D), stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_splits <= 1) return e;
  const size_t merge_lds = ((size_t)p.num_splits + (256 / (D / 4)) * D) * sizeof(float);
  dim3 mgrid(rows_max, p.Hkv, p.num_seqs);
  hipLaunchKernelGGL((decode_merge_kernel<D>), mgrid, dim3(256), merge_lds, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode(const PagedParams& p, int head_dim, int kv_type, int rows_max, hipStream_t stream) {
  if (head_dim == 128 && kv_type == KV_BF16) return launch_decode_t<128, KV_BF16, 4>(p, rows_max, stream);
  if (head_dim == 256 && kv_type == KV_BF16) return launch_decode_t<256, KV_BF16, 2>(p, rows_max, stream);
  if (head_dim == 128 && kv_type == KV_FP8) return launch_decode_t<128, KV_FP8, 4>(p, rows_max, stream);
  if (head_dim == 256 && kv_type == KV_FP8) return launch_decode_t<256, KV_FP8, 2>(p, rows_max, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
