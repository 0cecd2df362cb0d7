// Head-dimension dispatch of the attention forward launch.  Each head
// dimension's kernels live in their own translation unit so that each can
// be built with the register-form options that suit it.
#include "attn.h"
#include "attn_internal.h"

namespace attn {

int launch_forward_d64(const Problem& p, hipStream_t stream);
int launch_forward_d128(const Problem& p, hipStream_t stream);
int launch_forward_d256(const Problem& p, hipStream_t stream);

int launch_forward(const Problem& p, hipStream_t stream) {
  switch (p.d) {
    case 64: return launch_forward_d64(p, stream);
    case 128: return launch_forward_d128(p, stream);
    case 256: return launch_forward_d256(p, stream);
    default: return ATTN_ERR_HEADDIM;
  }
}

}  // namespace attn
