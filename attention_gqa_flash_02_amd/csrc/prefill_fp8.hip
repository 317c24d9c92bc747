// FP8 prefill kernel instantiation and launcher (see prefill_fp8.h).
#include "launch.h"
#include "prefill_fp8.h"

namespace attn {

// Grid: (head groups, requests, q-tiles), q-tiles walked heaviest (last) first; a q-tile is
// 32 * 8 / hpw rows. 8 waves, 32 KB of LDS, one workgroup per compute unit.
template <int BN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_fp8_kernel(PrefillFp8Params p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  prefill_fp8_body<BN>(p, smem_raw, blockIdx.x, blockIdx.y, p.num_qtiles - 1 - (int)blockIdx.z);
}

hipError_t launch_prefill_fp8(const PrefillFp8Params& p, int max_seqlen, hipStream_t stream) {
  using S = PingPongFp8Shape<64>;
  const int tq = 32 * (8 / p.hpw);
  PrefillFp8Params q = p;
  q.num_qtiles = (max_seqlen + tq - 1) / tq;
  if (q.num_qtiles <= 0) return hipSuccess;
  dim3 grid(p.Hkv * (p.g / p.hpw), p.num_seqs, q.num_qtiles);
  return launch_kernel(&prefill_fp8_kernel<64>, grid, dim3(512), S::LDS_BYTES, stream, q);
}

}  // namespace attn
