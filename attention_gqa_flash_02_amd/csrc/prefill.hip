// Prefill kernel instantiations and launcher.
#include "launch.h"

namespace attn {

template <int D, int BN>
__global__ __launch_bounds__(256) void prefill_varlen_kernel(PrefillParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  prefill_tile_body<D, BN>(p, reinterpret_cast<bf16*>(smem_raw), blockIdx.x, blockIdx.y,
                           p.num_qtiles - 1 - (int)blockIdx.z);
}

template <int D, int BN>
static hipError_t launch_prefill_t(const PrefillParams& p, int max_seqlen, hipStream_t stream) {
  using S = PrefillShape<D, BN>;
  static bool attr_set = false;  // per process; the attribute is a property of the function
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_varlen_kernel<D, BN>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int tq = 32 * (4 / p.hpw);
  PrefillParams q = p;
  q.num_qtiles = (max_seqlen + tq - 1) / tq;
  if (q.num_qtiles <= 0) return hipSuccess;
  dim3 grid(p.Hkv * (p.g / p.hpw), p.num_seqs, q.num_qtiles);
  hipLaunchKernelGGL((prefill_varlen_kernel<D, BN>), grid, dim3(256), S::LDS_BYTES, stream, q);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, int max_seqlen, hipStream_t stream) {
  if (head_dim == 128) return launch_prefill_t<128, 64>(p, max_seqlen, stream);
  if (head_dim == 256) return launch_prefill_t<256, 32>(p, max_seqlen, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
