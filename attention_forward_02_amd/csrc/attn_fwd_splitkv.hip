// Split-key attention forward (device code in attn_fwd_splitkv.h): every
// head dimension and input format, causal or not, in one translation unit;
// and the static scratch of its allocation-free entry point.
#include <mutex>

#include "attn_fwd_splitkv.h"

// Partials of attn_fwd_splitkv_noalloc: one copy per device, held from the
// library's load until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: every host use goes through the
// device address looked up by splitkv_scratch() below.
static __device__ __align__(256) unsigned char scratch[ATTN_SPLITKV_SCRATCH_BYTES];

namespace attn {
namespace kernels {

#define ATTN_SPLITKV_INSTANCES(D)                                                  \
  template __global__ void attn_fwd_splitkv_kernel<D, ATTN_F16, false>(Params);    \
  template __global__ void attn_fwd_splitkv_kernel<D, ATTN_F16, true>(Params);     \
  template __global__ void attn_fwd_splitkv_kernel<D, ATTN_BF16, false>(Params);   \
  template __global__ void attn_fwd_splitkv_kernel<D, ATTN_BF16, true>(Params);    \
  template __global__ void attn_fwd_splitkv_kernel<D, ATTN_FP8_E4M3, false>(Params); \
  template __global__ void attn_fwd_splitkv_kernel<D, ATTN_FP8_E4M3, true>(Params);      \
  template __global__ void attn_splitkv_merge_kernel<D, ATTN_F16, false>(Params);  \
  template __global__ void attn_splitkv_merge_kernel<D, ATTN_F16, true>(Params);   \
  template __global__ void attn_splitkv_merge_kernel<D, ATTN_BF16, false>(Params); \
  template __global__ void attn_splitkv_merge_kernel<D, ATTN_BF16, true>(Params);  \
  template __global__ void attn_splitkv_merge_kernel<D, ATTN_FP8_E4M3, false>(Params); \
  template __global__ void attn_splitkv_merge_kernel<D, ATTN_FP8_E4M3, true>(Params);
ATTN_SPLITKV_INSTANCES(64)
ATTN_SPLITKV_INSTANCES(128)
ATTN_SPLITKV_INSTANCES(256)
#undef ATTN_SPLITKV_INSTANCES

template <int D>
SplitPlan plan_d(int B, int H, int Nq, int Nk, bool causal, int dtype, int num_splits) {
  if (dtype == ATTN_FP8_E4M3) return split_plan<D, ATTN_FP8_E4M3>(B, H, Nq, Nk, causal, num_splits);
  return split_plan<D, ATTN_F16>(B, H, Nq, Nk, causal, num_splits);  // bf16 tiles are the same
}

SplitPlan plan(int B, int H, int Nq, int Nk, int d, bool causal, int dtype, int num_splits) {
  switch (d) {
    case 64: return plan_d<64>(B, H, Nq, Nk, causal, dtype, num_splits);
    case 128: return plan_d<128>(B, H, Nq, Nk, causal, dtype, num_splits);
    default: return plan_d<256>(B, H, Nq, Nk, causal, dtype, num_splits);
  }
}

template <int D>
int launch_d(const Problem& p, hipStream_t s) {
  switch (p.dtype) {
    case ATTN_F16:
      return p.causal ? launch_splitkv_one<D, ATTN_F16, true>(p, s) : launch_splitkv_one<D, ATTN_F16, false>(p, s);
    case ATTN_BF16:
      return p.causal ? launch_splitkv_one<D, ATTN_BF16, true>(p, s) : launch_splitkv_one<D, ATTN_BF16, false>(p, s);
    case ATTN_FP8_E4M3:
      return p.causal ? launch_splitkv_one<D, ATTN_FP8_E4M3, true>(p, s)
                      : launch_splitkv_one<D, ATTN_FP8_E4M3, false>(p, s);
    default:
      return ATTN_ERR_DTYPE;
  }
}

}  // namespace kernels

size_t splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int causal, int dtype, int num_splits) {
  return kernels::plan(B, H, Nq, Nk, d, causal != 0, dtype, num_splits).bytes;
}

int splitkv_splits(int B, int H, int Nq, int Nk, int d, int causal, int dtype, int num_splits) {
  return kernels::plan(B, H, Nq, Nk, d, causal != 0, dtype, num_splits).nsplit;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_address[kMaxDevices];  // per device, once looked up
}  // namespace

int splitkv_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_SCRATCH;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_address[dev]) {
    // with `dev` current: this device's copy of the array
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return ATTN_ERR_SCRATCH;
    scratch_address[dev] = a;
  }
  *ptr = scratch_address[dev];
  return ATTN_OK;
}

int launch_splitkv(const Problem& p, hipStream_t stream) {
  switch (p.d) {
    case 64: return kernels::launch_d<64>(p, stream);
    case 128: return kernels::launch_d<128>(p, stream);
    case 256: return kernels::launch_d<256>(p, stream);
    default: return ATTN_ERR_HEADDIM;
  }
}

}  // namespace attn
