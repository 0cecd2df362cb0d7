// Private interface between the C ABI (attn_api.cpp) and the kernels
// (attn_fwd_d*.hip, attn_quant.hip).  Not installed; not part of the public header.
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
  // Block-scaled E4M3 (attn_fwd_fp8_blockscaled): one descale per
  // ATTN_FP8_BLOCK_ROWS rows of each head, [B][H][ceil(N / rows)]; NULL
  // otherwise.  `scale` then excludes the descales.
  const float* q_descales;
  const float* k_descales;
  const float* v_descales;
  int variant;        // ATTN_VARIANT_*; AUTO for attn_fwd / attn_fwd_fp8
  // Split-key forward (attn_fwd_splitkv) only: splits per query tile (0 =
  // the library's choice) and the device workspace for partial results.
  int num_splits;
  void* workspace;
  size_t workspace_bytes;
};

// Launches the forward pass on `stream`.  Returns 0 or a negative ATTN_ERR_*.
int launch_forward(const Problem& p, hipStream_t stream);

// Split-key forward: workspace bytes a shape needs (0 for an unsupported
// head dim or dtype), and the launch.
size_t splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int causal, int dtype, int num_splits);
int splitkv_splits(int B, int H, int Nq, int Nk, int d, int causal, int dtype, int num_splits);
int launch_splitkv(const Problem& p, hipStream_t stream);
// Device address of the current device's static split-key scratch
// (ATTN_SPLITKV_SCRATCH_BYTES), looked up on the first call per device.
int splitkv_scratch(void** ptr);

// One tensor's block-scaled E4M3 quantisation, validated by the C ABI.
struct QuantProblem {
  const void* x;      // [B][H][N][d] binary16 or bfloat16
  void* codes;        // [B][H][N][d] E4M3 codes
  float* descales;    // [B][H][ceil(N / ATTN_FP8_BLOCK_ROWS)]
  int B, H, N, d;
  int dtype;          // ATTN_F16 or ATTN_BF16
  int hadamard;       // nonzero: 16x16 Walsh-Hadamard transform first
};

int launch_quantize(const QuantProblem& p, hipStream_t stream);

}  // namespace attn
