// Block-scaled FP8 E4M3 quantisation of one attention input, with optional
// 16x16 Walsh-Hadamard smoothing ("Inside FlashAttention-3", section 5:
// block scaling plus Hadamard outlier smoothing before quantising Q and K;
// since the transform is orthogonal, transforming both Q and K leaves
// Q K^T unchanged while an outlier channel is spread over 16 channels).
//
// One workgroup of 256 threads per block of 64 rows of one (batch, head):
//   1. every thread loads whole 16-element groups of a row (two 16-byte
//      loads each; consecutive threads take consecutive groups, so a wave
//      reads 2 KB contiguously), widens them and, with the transform on,
//      runs the 16-point butterflies in double precision -- exact for
//      binary16 inputs -- before one rounding to float;
//   2. the block's largest magnitude comes from a wave reduction plus one
//      LDS exchange between the four waves; descale = amax / 448 in IEEE
//      float32 (1 for an all-zero block);
//   3. every value is divided by the descale and rounded to E4M3 by
//      v_cvt_pk_fp8_f32 (round to nearest even); each group leaves as one
//      16-byte store.  The quotient is the IEEE float32 one, RN(y / ds),
//      from a multiply and two FMAs per value: with r = RN(1 / ds) (one
//      correctly rounded division per thread), q = RN(y r) is within one ulp
//      of y / ds, the residual y - ds q is exact in an FMA, and q + (y - ds q) r
//      rounds to RN(y / ds) (Markstein's theorem on FMA division).  The
//      theorem needs the residual to stay a normal number wherever it can
//      move a code, which holds for ds >= 2^-90; smaller descales (bfloat16
//      blocks of magnitude below about 1e-25) take the plain division.
// The block stays in registers between the passes, so every input byte is
// read once and every code written once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn.h"
#include "attn_internal.h"

namespace attn {
namespace quant {

constexpr int kRows = ATTN_FP8_BLOCK_ROWS;
constexpr int kThreads = 256;
constexpr float kE4m3Max = 448.0f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ float widen(uint32_t bits16) {
  if constexpr (DT == ATTN_BF16) return __builtin_bit_cast(float, bits16 << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// x <- H16 x / 4 with H16 the Sylvester-ordered Walsh-Hadamard matrix,
// entry (i, j) = (-1)^popcount(i & j): radix-2 butterflies (a + b, a - b).
__device__ __forceinline__ void fwht16(double (&x)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int i = 0; i < 16; i += 2 * h)
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const double a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] *= 0.25;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

template <int D, int DT, bool HAD>
__global__ void __launch_bounds__(kThreads) quantize_kernel(const uint16_t* __restrict__ x,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ descales, int N, int nb) {
  constexpr int kGroups = D / 16;                       // 16-element groups per row
  constexpr int kPer = kRows * kGroups / kThreads;      // groups per thread
  static_assert(kPer * kThreads == kRows * kGroups, "block must split evenly");
  const int bh = blockIdx.x / nb;
  const int r0 = (blockIdx.x - bh * nb) * kRows;
  const size_t head = (size_t)bh * N;

  float y[kPer][16];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int g = threadIdx.x + i * kThreads;
    const int r = r0 + g / kGroups;
    if (r < N) {
      const u32x4* src = (const u32x4*)(x + (head + r) * D + (g % kGroups) * 16);
      const u32x4 a = src[0], b = src[1];
      float v[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v[2 * w] = widen<DT>(a[w] & 0xffffu);
        v[2 * w + 1] = widen<DT>(a[w] >> 16);
        v[8 + 2 * w] = widen<DT>(b[w] & 0xffffu);
        v[8 + 2 * w + 1] = widen<DT>(b[w] >> 16);
      }
      if constexpr (HAD) {
        double t[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) t[e] = (double)v[e];
        fwht16(t);
#pragma unroll
        for (int e = 0; e < 16; ++e) y[i][e] = (float)t[e];
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) y[i][e] = v[e];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(y[i][e]));
    }
  }

  __shared__ float wmax[kThreads / 64];
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float ds = amax > 0.f ? amax / kE4m3Max : 1.f;
  if (threadIdx.x == 0) descales[blockIdx.x] = ds;

  auto emit = [&](auto quot) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int g = threadIdx.x + i * kThreads;
      const int r = r0 + g / kGroups;
      if (r < N) {
        u32x4 out;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float* p = &y[i][4 * w];
          const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(quot(p[0]), quot(p[1]), 0, false);
          out[w] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(quot(p[2]), quot(p[3]), lo, true);
        }
        *(u32x4*)(codes + (head + r) * D + (g % kGroups) * 16) = out;
      }
    }
  };
  if (ds >= 0x1p-90f) {  // block-uniform
    const float rcp = 1.f / ds;
    emit([&](float v) {
      // The residual is formed as ds q - v and subtracted, so that v = -0
      // gives -0 (as v / ds does) rather than +0 + -0 = +0.
      const float q = v * rcp;
      return __builtin_fmaf(-__builtin_fmaf(ds, q, -v), rcp, q);
    });
  } else {
    emit([&](float v) { return v / ds; });
  }
}

template <int D, int DT>
int launch_d(const QuantProblem& p, hipStream_t stream) {
  const int nb = (p.N + kRows - 1) / kRows;
  const dim3 grid((unsigned)((long long)p.B * p.H * nb));
  const uint16_t* x = (const uint16_t*)p.x;
  uint8_t* c = (uint8_t*)p.codes;
  if (p.hadamard)
    hipLaunchKernelGGL((quantize_kernel<D, DT, true>), grid, dim3(kThreads), 0, stream, x, c, p.descales, p.N, nb);
  else
    hipLaunchKernelGGL((quantize_kernel<D, DT, false>), grid, dim3(kThreads), 0, stream, x, c, p.descales, p.N, nb);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

template <int DT>
int launch_dt(const QuantProblem& p, hipStream_t stream) {
  switch (p.d) {
    case 64: return launch_d<64, DT>(p, stream);
    case 128: return launch_d<128, DT>(p, stream);
    case 256: return launch_d<256, DT>(p, stream);
    default: return ATTN_ERR_HEADDIM;
  }
}

}  // namespace quant

int launch_quantize(const QuantProblem& p, hipStream_t stream) {
  switch (p.dtype) {
    case ATTN_F16: return quant::launch_dt<ATTN_F16>(p, stream);
    case ATTN_BF16: return quant::launch_dt<ATTN_BF16>(p, stream);
    default: return ATTN_ERR_DTYPE;
  }
}

}  // namespace attn
