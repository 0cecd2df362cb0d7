// Private interface between the C ABI (attn_api.cpp) and the kernels
// (attn_fwd.hip).  Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

// Everything a launch needs, validated by the C ABI before it gets here.
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Nq, Nk, d;
  int causal;
  int dtype;          // attn_dtype
  float scale;        // multiplies Q K^T (dequantisation of q and k folded in for fp8)
  float v_descale;    // multiplies P V (1 unless fp8)
};

// Launches the forward pass on `stream`.  Returns 0 or a negative ATTN_ERR_*.
int launch_forward(const Problem& p, hipStream_t stream);

}  // namespace attn
