// Attention forward kernels for head dimension 64, fp16 and bf16 inputs (device code in
// attn_fwd_kernel.h).  Explicit instantiations make the host pass emit a
// launch stub for every kernel the dispatcher can launch.
#include "attn_fwd_kernel.h"

namespace attn {
namespace kernels {

template __global__ void attn_fwd_kernel<64, ATTN_F16, false>(Params);
template __global__ void attn_fwd_kernel<64, ATTN_F16, true>(Params);
template __global__ void attn_fwd_kernel<64, ATTN_BF16, false>(Params);
template __global__ void attn_fwd_kernel<64, ATTN_BF16, true>(Params);

template __global__ void attn_fwd_split_kernel<64, ATTN_F16, false>(Params);
template __global__ void attn_fwd_split_kernel<64, ATTN_F16, true>(Params);
template __global__ void attn_fwd_split_kernel<64, ATTN_BF16, false>(Params);
template __global__ void attn_fwd_split_kernel<64, ATTN_BF16, true>(Params);
// Tuning variants (attn_fwd_variant).
template __global__ void attn_fwd_kernel<64, ATTN_F16, false, 4>(Params);
template __global__ void attn_fwd_kernel<64, ATTN_F16, true, 4>(Params);
template __global__ void attn_fwd_kernel<64, ATTN_BF16, false, 4>(Params);
template __global__ void attn_fwd_kernel<64, ATTN_BF16, true, 4>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_F16, false>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_F16, true>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_BF16, false>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_BF16, true>(Params);

// Key-tile-size variants of the sequential kernel.
template __global__ void attn_fwd_seq_kernel<64, ATTN_F16, false, false, 32>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_F16, false, false, 128>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_F16, true, false, 32>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_F16, true, false, 128>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_BF16, false, false, 32>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_BF16, false, false, 128>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_BF16, true, false, 32>(Params);
template __global__ void attn_fwd_seq_kernel<64, ATTN_BF16, true, false, 128>(Params);

// Three-stage pipelined variant.
template __global__ void attn_fwd_pipe3_kernel<64, ATTN_F16, false>(Params);
template __global__ void attn_fwd_pipe3_kernel<64, ATTN_F16, true>(Params);
template __global__ void attn_fwd_pipe3_kernel<64, ATTN_BF16, false>(Params);
template __global__ void attn_fwd_pipe3_kernel<64, ATTN_BF16, true>(Params);

}  // namespace kernels

int launch_forward_d64(const Problem& p, hipStream_t stream) { return kernels::launch_16bit<64>(p, stream); }

}  // namespace attn
