// Head-dimension and element-format dispatch of the attention forward
// launch.  Each (head dimension, 16-bit or E4M3) family of kernels lives in
// its own translation unit so that each can be built with the register-form
// options that suit it.
#include "attn.h"
#include "attn_internal.h"

namespace attn {

int launch_forward_d64(const Problem& p, hipStream_t stream);
int launch_forward_d128(const Problem& p, hipStream_t stream);
int launch_forward_d256(const Problem& p, hipStream_t stream);
int launch_forward_d64_fp8(const Problem& p, hipStream_t stream);
int launch_forward_d128_fp8(const Problem& p, hipStream_t stream);
int launch_forward_d256_fp8(const Problem& p, hipStream_t stream);

int launch_forward(const Problem& p, hipStream_t stream) {
  const bool fp8 = p.dtype == ATTN_FP8_E4M3;
  switch (p.d) {
    case 64: return fp8 ? launch_forward_d64_fp8(p, stream) : launch_forward_d64(p, stream);
    case 128: return fp8 ? launch_forward_d128_fp8(p, stream) : launch_forward_d128(p, stream);
    case 256: return fp8 ? launch_forward_d256_fp8(p, stream) : launch_forward_d256(p, stream);
    default: return ATTN_ERR_HEADDIM;
  }
}

}  // namespace attn
