// Wide-wave attention forward kernels (64 query rows per wave) for head
// dimension 128, fp16 and bf16 inputs (device code in attn_fwd_wide.h).  A
// translation unit of its own: its MFMAs keep the compiler's default
// register form, so the output accumulators can live in AGPRs.
#include "attn_fwd_wide.h"

namespace attn {
namespace kernels {

template __global__ void attn_fwd_wide_kernel<128, ATTN_F16, false>(Params);
template __global__ void attn_fwd_wide_kernel<128, ATTN_F16, true>(Params);
template __global__ void attn_fwd_wide_kernel<128, ATTN_BF16, false>(Params);
template __global__ void attn_fwd_wide_kernel<128, ATTN_BF16, true>(Params);

template <int DT, bool CAUSAL>
static void launch_wide(const Params& p, hipStream_t stream) {
  const dim3 grid(p.total_tiles), block(64 * kWideWaves);
  hipLaunchKernelGGL((attn_fwd_wide_kernel<128, DT, CAUSAL>), grid, block, 0, stream, p);
}

int launch_wide_d128(const Params& p, int dtype, bool causal, hipStream_t stream) {
  if (dtype == ATTN_F16) {
    if (causal) launch_wide<ATTN_F16, true>(p, stream);
    else launch_wide<ATTN_F16, false>(p, stream);
  } else {
    if (causal) launch_wide<ATTN_BF16, true>(p, stream);
    else launch_wide<ATTN_BF16, false>(p, stream);
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace kernels
}  // namespace attn
