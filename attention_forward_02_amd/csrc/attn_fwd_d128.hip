// Attention forward kernels for head dimension 128 (device code in
// attn_fwd_kernel.h).  Explicit instantiations make the host pass emit a
// launch stub for every kernel the dispatcher can launch.
#include "attn_fwd_kernel.h"

namespace attn {
namespace kernels {

template __global__ void attn_fwd_kernel<128, ATTN_F16, false>(Params);
template __global__ void attn_fwd_kernel<128, ATTN_F16, true>(Params);
template __global__ void attn_fwd_kernel<128, ATTN_BF16, false>(Params);
template __global__ void attn_fwd_kernel<128, ATTN_BF16, true>(Params);
template __global__ void attn_fwd_kernel<128, ATTN_FP8_E4M3, false>(Params);
template __global__ void attn_fwd_kernel<128, ATTN_FP8_E4M3, true>(Params);

}  // namespace kernels

int launch_forward_d128(const Problem& p, hipStream_t stream) { return kernels::launch_head_dim<128>(p, stream); }

}  // namespace attn
