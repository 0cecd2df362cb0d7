// Timeline probe: two of the library's kernels built with their shader-clock
// trace points switched on (Timeline in attn_fwd_kernel.h), as a shared
// library of its own (libattn_timeline.so) for attention_forward_02_amd/
// timeline.py.  The attention library never defines ATTN_TIMELINE, so its
// kernels carry no trace code.  This file is compiled twice, with
// ATTN_TIMELINE_KERNEL 0 or 1 and the register-form options of the
// translation unit that holds the kernel in the library:
//   0: the sequential kernel with 128-key tiles, d = 64, bfloat16, causal
//      (attn_fwd_d64.hip; the default on 64-512 query tiles of 128 rows);
//   1: the producer-wave kernel, d = 128, binary16, not causal
//      (attn_fwd_d128.hip; the binary16 d = 128 default).
#define ATTN_TIMELINE 1
#include "attn_fwd_kernel.h"

namespace attn {
namespace kernels {

#if ATTN_TIMELINE_KERNEL == 0
constexpr int kTlD = 64, kTlDtype = ATTN_BF16, kTlWaves = 4, kTlRows = 128;
template __global__ void attn_fwd_seq_kernel<64, ATTN_BF16, true, false, 128>(Params);
#else
constexpr int kTlD = 128, kTlDtype = ATTN_F16, kTlWaves = 9, kTlRows = 256;
template __global__ void attn_fwd_producer_kernel<128, ATTN_F16, false, 2, 1>(Params);
#endif

namespace {
// Launches the traced kernel on [B, H, Nq, 64 or 128] tensors q and
// [B, H, Nk, same] k, v (device pointers, row-major), writing o and lse as
// attn_fwd does and kTimelineSlots counters per wave to `timeline`.
// Returns ATTN_ERR_SHAPE before launching when the sizes are out of range
// or `timeline_bytes` is smaller than the grid needs.
int timeline_launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                    float scale, unsigned long long* timeline, unsigned long long timeline_bytes,
                    hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !timeline) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (long long)B * H * Nq * kTlD >= (1LL << 31) ||
      (long long)B * H * Nk * kTlD >= (1LL << 31))
    return ATTN_ERR_SHAPE;
  Params p = {};
  p.q = (const unsigned char*)q;
  p.k = (const unsigned char*)k;
  p.v = (const unsigned char*)v;
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.Nq = Nq;
  p.Nk = Nk;
  p.n_qtiles = (Nq + kTlRows - 1) / kTlRows;
  const long long tiles = (long long)B * H * p.n_qtiles;
  if (tiles > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  p.total_tiles = (int)tiles;
  if ((unsigned long long)tiles * kTlWaves * kTimelineSlots * sizeof(unsigned long long) > timeline_bytes)
    return ATTN_ERR_SHAPE;
  set_scale(p, scale, kTlDtype);
  p.o_scale = 1.f;
  p.timeline = timeline;
#if ATTN_TIMELINE_KERNEL == 0
  hipLaunchKernelGGL((attn_fwd_seq_kernel<64, ATTN_BF16, true, false, 128>), dim3(p.total_tiles), dim3(64 * kTlWaves),
                     0, stream, p);
#else
  hipLaunchKernelGGL((attn_fwd_producer_kernel<128, ATTN_F16, false, 2, 1>), dim3(p.total_tiles),
                     dim3(64 * kTlWaves), 0, stream, p);
#endif
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
}  // namespace

}  // namespace kernels
}  // namespace attn

extern "C" {

#if ATTN_TIMELINE_KERNEL == 0
// The sequential 128-key kernel, d = 64, bfloat16, causal (4 waves, 128 query
// rows per workgroup).
int attn_timeline_seq_d64_bf16_causal(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                      int Nq, int Nk, float scale, unsigned long long* timeline,
                                      unsigned long long timeline_bytes, hipStream_t stream) {
  return attn::kernels::timeline_launch(q, k, v, o, lse, B, H, Nq, Nk, scale, timeline, timeline_bytes, stream);
}
#else
// The producer-wave kernel, d = 128, binary16, not causal (8 consumer waves
// and one producer wave, 256 query rows per workgroup).
int attn_timeline_producer_d128_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                    int Nq, int Nk, float scale, unsigned long long* timeline,
                                    unsigned long long timeline_bytes, hipStream_t stream) {
  return attn::kernels::timeline_launch(q, k, v, o, lse, B, H, Nq, Nk, scale, timeline, timeline_bytes, stream);
}
// Counters per wave.
int attn_timeline_slots(void) { return attn::kernels::kTimelineSlots; }
#endif

}  // extern "C"
