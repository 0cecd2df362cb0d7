// Key-tile-size variants of the sequential kernel for head dimension 128,
// fp16 and bf16 inputs (device code in attn_fwd_kernel.h): 32- and 128-key
// tiles.  A translation unit of their own: the 128-key bf16 kernel fits its
// registers under the default scheduler but not under the register trackers
// the other d = 128 kernels are built with.
#include "attn_fwd_kernel.h"

namespace attn {
namespace kernels {

template __global__ void attn_fwd_seq_kernel<128, ATTN_F16, false, false, 32>(Params);
template __global__ void attn_fwd_seq_kernel<128, ATTN_F16, true, false, 32>(Params);
template __global__ void attn_fwd_seq_kernel<128, ATTN_BF16, false, false, 32>(Params);
template __global__ void attn_fwd_seq_kernel<128, ATTN_BF16, true, false, 32>(Params);
template __global__ void attn_fwd_seq_kernel<128, ATTN_F16, false, false, 128>(Params);
template __global__ void attn_fwd_seq_kernel<128, ATTN_F16, true, false, 128>(Params);
template __global__ void attn_fwd_seq_kernel<128, ATTN_BF16, false, false, 128>(Params);
template __global__ void attn_fwd_seq_kernel<128, ATTN_BF16, true, false, 128>(Params);

template <int DT, bool CAUSAL>
int launch_bc(const Params& p, int bn, hipStream_t stream) {
  const dim3 grid(p.total_tiles), block(64 * Waves<128, DT>::value);
  if (bn == 32) hipLaunchKernelGGL((attn_fwd_seq_kernel<128, DT, CAUSAL, false, 32>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((attn_fwd_seq_kernel<128, DT, CAUSAL, false, 128>), grid, block, 0, stream, p);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int launch_seq_bc_d128(const Params& p, int dtype, bool causal, int bn, hipStream_t stream) {
  if (dtype == ATTN_F16) return causal ? launch_bc<ATTN_F16, true>(p, bn, stream) : launch_bc<ATTN_F16, false>(p, bn, stream);
  return causal ? launch_bc<ATTN_BF16, true>(p, bn, stream) : launch_bc<ATTN_BF16, false>(p, bn, stream);
}

}  // namespace kernels
}  // namespace attn
