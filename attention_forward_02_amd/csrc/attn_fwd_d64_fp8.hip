// Attention forward kernels for head dimension 64, E4M3 inputs (device code in
// attn_fwd_kernel.h).  Explicit instantiations make the host pass emit a
// launch stub for every kernel the dispatcher can launch.
#include "attn_fwd_kernel.h"

namespace attn {
namespace kernels {

template __global__ void attn_fwd_kernel<64, ATTN_FP8_E4M3, false>(Params);
template __global__ void attn_fwd_kernel<64, ATTN_FP8_E4M3, true>(Params);

template __global__ void attn_fwd_seq_kernel<64, ATTN_FP8_E4M3, false, true>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_FP8_E4M3, true, true>(Params);

// Tuning variants (attn_fwd_variant).
template __global__ void attn_fwd_kernel<64, ATTN_FP8_E4M3, false, 4>(Params);
template __global__ void attn_fwd_kernel<64, ATTN_FP8_E4M3, true, 4>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_FP8_E4M3, false>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_FP8_E4M3, true>(Params);

// Key-tile-size variant of the sequential kernel.
template __global__ void attn_fwd_seq_kernel<64, ATTN_FP8_E4M3, false, false, 128>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_FP8_E4M3, true, false, 128>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_FP8_E4M3, false, true, 128>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_FP8_E4M3, true, true, 128>(Params);

}  // namespace kernels

int launch_forward_d64_fp8(const Problem& p, hipStream_t stream) { return kernels::launch_fp8<64>(p, stream); }

}  // namespace attn
