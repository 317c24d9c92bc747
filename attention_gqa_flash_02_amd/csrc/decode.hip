// Paged decode kernel instantiations and launcher.
#include "launch.h"

namespace attn {

template <int D, int KVT>
__global__ __launch_bounds__(256) void decode_split_kernel(PagedParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  decode_unit<D, KVT>(p, blockIdx.z, blockIdx.y, blockIdx.x, reinterpret_cast<float*>(smem_raw));
}

template <int D, int KVT>
static hipError_t launch_decode_t(const PagedParams& p, int rows_max, hipStream_t stream) {
  const size_t lds = (128 + 4 * (size_t)rows_max * D) * sizeof(float);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_split_kernel<D, KVT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)((128 + 4 * 16 * D) * sizeof(float)));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid(p.num_splits, p.Hkv, p.num_seqs);
  hipLaunchKernelGGL((decode_split_kernel<D, KVT>), grid, dim3(256), lds, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode(const PagedParams& p, int head_dim, int kv_type, int rows_max, hipStream_t stream) {
  if (head_dim == 128 && kv_type == KV_BF16) return launch_decode_t<128, KV_BF16>(p, rows_max, stream);
  if (head_dim == 256 && kv_type == KV_BF16) return launch_decode_t<256, KV_BF16>(p, rows_max, stream);
  if (head_dim == 128 && kv_type == KV_FP8) return launch_decode_t<128, KV_FP8>(p, rows_max, stream);
  if (head_dim == 256 && kv_type == KV_FP8) return launch_decode_t<256, KV_FP8>(p, rows_max, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
