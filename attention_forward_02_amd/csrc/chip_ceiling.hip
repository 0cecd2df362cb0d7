// Chip ceilings behind the attention kernels' roofline figures, measured
// under sustained load on the GPU at hand (a standalone program; the
// attention library does not use it).
//
//   attention_forward_02_amd/chip_ceiling [seconds]
//
// prints a markdown table.  Every test launches one 8-wave workgroup per
// CU (two waves per SIMD: waves w and w + 4 share SIMD w), keeps launching
// for `seconds` (default 1) so that clocks and power management settle,
// then times `seconds` more of launches with HIP events.  Each wave reads
// the shader clock counter around its loop, so the table also gives the
// cycles an iteration takes and the effective shader clock (wave cycles
// over wall time).
//
//   mfma f16   every wave: 4 independent v_mfma_f32_32x32x16_f16 chains
//   mfma bf16  the same with v_mfma_f32_32x32x16_bf16
//   mfma fp8   every wave: 4 independent v_mfma_f32_32x32x64_f8f6f4 chains
//              (E4M3 operands)
//   fma        waves 0-3 only (one wave per SIMD): 16 independent fp32 FMA
//              chains, 32 FMAs per iteration
//   exp        waves 0-3 only: 16 v_exp_f32 (+ 16 multiplies) per iteration
//   exp alone  waves 0-3 only: 16 v_exp_f32 per iteration, nothing else
//   mfma f16 + fma / + exp: waves 0-3 the f16 MFMA loop, waves 4-7 (same
//              SIMDs) the fma or exp loop at the same time
//   mfma f16 + lds (+ fma / + exp): the MFMA waves take their A operands
//              from LDS, one 16-byte read per MFMA (1 KB per wave
//              instruction, 32 bytes per MFMA cycle: the operand rate of
//              the attention kernels' score and P V products), read one
//              iteration ahead
//
// The MFMA operands are distinct per lane and the accumulators feed back,
// so no iteration can be folded away.
//
// A second table models one step of the attention kernels per wave, with
// the step's dependences: S = A B (8 chained 32x32x16 f16 MFMAs, B the
// previous iteration's P), p = exp2(c S - m) (16 FMAs, 16 exp2, 8 packs to
// binary16), O += A' P (8 MFMAs over 4 accumulators): 512 MFMA cycles and
// about 300 VALU cycles per iteration.  It runs with one or two waves per
// SIMD, with the A operands in registers or read from LDS one 16-byte read
// per MFMA (the P V operands optionally by two ds_read_b64_tr_b16, as the
// kernels read V), optionally with a workgroup barrier per iteration, with
// the kernels' full softmax mix (a row max and v_dot2 row sums added), and
// with the LDS reads as the compiler schedules them or pinned ahead of
// their use.  Matrix-core use = 512 cycles x waves per SIMD over the
// slowest wave's cycles per iteration.
//
// A third table gives the CU's LDS read rate: every wave issues `n` reads
// (ds_read_b128 or ds_read_b64_tr_b16, conflict-free addresses), waits for
// them, and repeats.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

enum { kMfmaF16 = 0, kMfmaFp8 = 1, kFma = 2, kExp = 3, kMfmaFma = 4, kMfmaExp = 5, kLds = 6, kLdsFma = 7, kLdsExp = 8,
       kExpOnly = 9, kMfmaBf16 = 10 };
constexpr int kCUs = 256;
constexpr int kWaves = 8;

template <int T>
__global__ void __launch_bounds__(512) ceiling_kernel(float* sink, long long* cycles, int iters) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr bool kPair = T == kMfmaFma || T == kMfmaExp || T == kLdsFma || T == kLdsExp;
  constexpr bool kUsesLds = T == kLds || T == kLdsFma || T == kLdsExp;
  constexpr bool kExpLoop = T == kExp || T == kMfmaExp || T == kLdsExp;
  const bool mfma_wave = (T == kMfmaF16 || T == kMfmaFp8 || T == kMfmaBf16 || T == kLds) || (kPair && w < 4);
  const bool valu_wave = ((T == kFma || T == kExp || T == kExpOnly) && w < 4) || (kPair && w >= 4);
  constexpr int kLdsBytes = 16384;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kUsesLds ? kLdsBytes : 16];
  if constexpr (kUsesLds) {
    for (int i = threadIdx.x; i < kLdsBytes / 2; i += 512)
      ((_Float16*)lds)[i] = (_Float16)(0.001f * (i & 255));
    __syncthreads();
  }
  float acc = 0.f;
  const long long t0 = __builtin_readcyclecounter();
  if (mfma_wave && kUsesLds) {
    f16x8 b;
    for (int i = 0; i < 8; ++i) b[i] = (_Float16)(0.25f - 0.002f * (lane - 3 * i));
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    typedef _Float16 lds_f16x8 __attribute__((ext_vector_type(8), address_space(3)));
    const lds_f16x8* base = (const lds_f16x8*)(lds + 16 * lane);
    // operand of MFMA i of iteration it: 1 KB block (4 it + i) mod 16; two
    // register sets, each read one iteration before its MFMAs
    f16x8 a[4], n[4];
    for (int i = 0; i < 4; ++i) a[i] = base[64 * i];
    auto read = [&](f16x8(&r)[4], int it) {
      const int nb = (it & 3) * 4 * 64;
      for (int i = 0; i < 4; ++i) r[i] = base[nb + 64 * i];
    };
    auto mfma4 = [&](const f16x8(&r)[4]) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(r[0], b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(r[1], b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(r[2], b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(r[3], b, c3, 0, 0, 0);
    };
    for (int it = 0; it < iters; it += 2) {
      read(n, it + 1);
      mfma4(a);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      read(a, it + 2);
      mfma4(n);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    for (int i = 0; i < 16; ++i) acc += c0[i] + c1[i] + c2[i] + c3[i];
  } else if (mfma_wave) {
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    if constexpr (T == kMfmaFp8) {
      i32x8 a, b;
      for (int i = 0; i < 8; ++i) {
        a[i] = 0x38303438 ^ (lane * 0x01010101 * (i + 1) & 0x07070707);  // E4M3 values near 1
        b[i] = 0x30383438 ^ (lane * 0x01030105 * (i + 3) & 0x07070707);
      }
      for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 0, 0, 0, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 0, 0, 0, 0, 0, 0);
      }
    } else if constexpr (T == kMfmaBf16) {
      typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
      bf16x8 a, b;
      for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.5f + 0.001f * (lane + 7 * i));
        b[i] = (__bf16)(0.25f - 0.002f * (lane - 3 * i));
      }
      for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
      }
    } else {
      f16x8 a, b;
      for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(0.5f + 0.001f * (lane + 7 * i));
        b[i] = (_Float16)(0.25f - 0.002f * (lane - 3 * i));
      }
      for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
      }
    }
    for (int i = 0; i < 16; ++i) acc += c0[i] + c1[i] + c2[i] + c3[i];
  } else if (valu_wave) {
    float x[16];
    for (int i = 0; i < 16; ++i) x[i] = 0.01f * lane + i;
    // the VALU waves run twice the MFMA waves' iterations in the overlap
    // tests, so that they are busy for the whole MFMA loop
    const int n = kPair ? 2 * iters : iters;
    for (int it = 0; it < n; ++it) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (T == kExpOnly) {
          x[i] = __builtin_amdgcn_exp2f(-x[i]);  // stays in (0, 1]; the sign is a free operand modifier
        } else if constexpr (!kExpLoop) {
          x[i] = __builtin_fmaf(x[i], 0.999f, 0.001f);
          x[i] = __builtin_fmaf(x[i], 0.999f, 0.001f);
        } else {
          x[i] = __builtin_amdgcn_exp2f(x[i] * -0.001f);
        }
      }
    }
    for (int i = 0; i < 16; ++i) acc += x[i];
  }
  const long long t1 = __builtin_readcyclecounter();
  sink[blockIdx.x * 512 + threadIdx.x] = acc;
  if (lane == 0) cycles[blockIdx.x * kWaves + w] = t1 - t0;
}

// One attention-like step per iteration (see the header).  MODE bits:
// 1 = barrier per iteration, 2 = A operands from LDS (a per-lane base plus
// immediate offsets, two ring stages, as the kernels address K and V),
// 4 = P V operands by transpose reads (with 2), 8 = the kernels' full
// softmax mix (a row max by v_max3 and v_dot2 row sums as well), 16 = the
// LDS reads pinned by sched_group_barrier: two score reads ahead of their
// MFMAs and the first two P V reads issued before the softmax (with 2).
template <int MODE>
__global__ void __launch_bounds__(512) step_kernel(const f16x8* ain, float* sink, long long* cycles, int iters,
                                                   float c, float m) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef _Float16 lds_f16x8 __attribute__((ext_vector_type(8), address_space(3)));
  typedef short lds_i16x4 __attribute__((ext_vector_type(4), address_space(3)));
  constexpr bool kLds = MODE & 2, kTr = (MODE & 6) == 6, kMix = MODE & 8, kPin = (MODE & 18) == 18;
  // 32 KB: two stages of 16 operands of 1 KB (64 lanes x 16 bytes)
  __shared__ __attribute__((aligned(1024))) _Float16 lds[16384];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 16384; i += blockDim.x) lds[i] = (_Float16)(0.001f * ((i * 37) % 97));
  __syncthreads();
  f16x8 a[8], pf[2];
  for (int k = 0; k < 8; ++k) a[k] = ain[lane + 64 * k];
  for (int i = 0; i < 8; ++i) {
    pf[0][i] = (_Float16)0.5f;
    pf[1][i] = (_Float16)0.25f;
  }
  f32x16 o[4] = {};
  float mx = 0.f, l = 0.f;
  const lds_f16x8* L = (const lds_f16x8*)lds + lane;
  auto operand = [&](const lds_f16x8* S, int k) -> f16x8 {
    if constexpr (kTr) {
      const __attribute__((address_space(3))) char* base = (const __attribute__((address_space(3))) char*)(S + 64 * k);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)base);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 8));
      return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return S[64 * k];
    }
  };
  auto step = [&](const lds_f16x8* S) {
    // Without a barrier the operands would be loop-invariant loads that the
    // compiler could hoist out of the loop; the empty asm's memory clobber
    // makes every step read them again.
    if constexpr (MODE & 1) __syncthreads();
    else asm volatile("" ::: "memory");
    f32x16 s = {};
#pragma unroll
    for (int k = 0; k < 8; ++k) s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kLds ? S[64 * k] : a[k], pf[k & 1], s, 0, 0, 0);
    if constexpr (kMix) {
      float ma = s[0], mb = s[1];
#pragma unroll
      for (int r = 2; r < 16; r += 2) {
        ma = fmaxf(fmaxf(ma, s[r]), s[r]);
        mb = fmaxf(fmaxf(mb, s[r + 1]), s[r + 1]);
      }
      mx = fmaxf(mx, fmaxf(ma, mb));
    }
    float pr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m));
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2 t = __builtin_convertvector((f32x2){pr[8 * h + 2 * e], pr[8 * h + 2 * e + 1]}, f16x2);
        pf[h][2 * e] = t[0];
        pf[h][2 * e + 1] = t[1];
        if constexpr (kMix) l = __builtin_amdgcn_fdot2(t, (f16x2){(_Float16)1.0f, (_Float16)1.0f}, l, false);
      }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      o[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kLds ? operand(S, 8 + k) : a[k], pf[k & 1], o[k & 3], 0, 0, 0);
    if constexpr (kPin) {
      // two score reads, then (MFMA, read) x 6, two MFMAs; two P V reads;
      // the softmax; then each P V MFMA with the next read
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, kTr ? 4 : 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 1000, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 6) __builtin_amdgcn_sched_group_barrier(0x100, kTr ? 2 : 1, 0);
      }
    }
  };
  const long long t0 = __builtin_readcyclecounter();
#pragma nounroll
  for (int it = 0; it < iters; it += 2) {
    step(L);
    step(L + 1024);
  }
  const long long t1 = __builtin_readcyclecounter();
  float acc = mx + l;
  for (int j = 0; j < 4; ++j)
    for (int i = 0; i < 16; ++i) acc += o[j][i];
  sink[blockIdx.x * 512 + threadIdx.x] = acc;
  if (lane == 0) cycles[blockIdx.x * kWaves + w] = t1 - t0;
}

// LDS read rate: n reads in flight per wave, then a wait; TR: the
// transpose read instead of ds_read_b128.
template <bool TR, int N>
__global__ void __launch_bounds__(1024) lds_kernel(float* sink, long long* cycles, int iters) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef int lds_i32x4 __attribute__((ext_vector_type(4), address_space(3)));
  typedef short lds_i16x4 __attribute__((ext_vector_type(4), address_space(3)));
  __shared__ __attribute__((aligned(1024))) int lds[16384];  // 64 KB
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 16384; i += blockDim.x) lds[i] = i * 40503;
  __syncthreads();
  const __attribute__((address_space(3))) char* base = (const __attribute__((address_space(3))) char*)lds;
  const long long t0 = __builtin_readcyclecounter();
#pragma nounroll
  for (int it = 0; it < iters; ++it) {
    i32x4 x[N];
    i16x4 y[N];
#pragma unroll
    for (int r = 0; r < N; ++r) {
      const int idx = (lane + 64 * ((r + it) & 15) + 1024 * (w & 3)) & 4095;  // 16-byte units
      if constexpr (TR) y[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 8 * idx));
      else x[r] = *(const lds_i32x4*)(base + 16 * idx);
    }
#pragma unroll
    for (int r = 0; r < N; ++r) {
      if constexpr (TR) asm volatile("" ::"v"(y[r]));
      else asm volatile("" ::"v"(x[r]));
    }
  }
  const long long t1 = __builtin_readcyclecounter();
  sink[blockIdx.x * 1024 + threadIdx.x] = 0.f;
  if (lane == 0) cycles[blockIdx.x * 16 + w] = t1 - t0;
}

struct Result {
  double ms_per_launch, mfma_cycles_per_iter, valu_cycles_per_iter, clock_ghz;
};

#define CHECK(x)                                                                 \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
      std::exit(1);                                                              \
    }                                                                            \
  } while (0)

template <int T>
Result run(int iters, double seconds, float* sink, long long* cyc) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  auto launch = [&]() { hipLaunchKernelGGL((ceiling_kernel<T>), dim3(kCUs), dim3(64 * kWaves), 0, 0, sink, cyc, iters); };
  // settle
  const auto start = std::chrono::steady_clock::now();
  while (std::chrono::duration<double>(std::chrono::steady_clock::now() - start).count() < seconds) {
    launch();
    CHECK(hipDeviceSynchronize());
  }
  // time
  int n = 0;
  float total_ms = 0.f;
  while (total_ms < seconds * 1e3f) {
    CHECK(hipEventRecord(e0));
    launch();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    total_ms += ms;
    ++n;
  }
  CHECK(hipGetLastError());
  std::vector<long long> c(kCUs * kWaves);
  CHECK(hipMemcpy(c.data(), cyc, c.size() * sizeof(long long), hipMemcpyDeviceToHost));
  const bool both = T == kMfmaFma || T == kMfmaExp || T == kLdsFma || T == kLdsExp;
  const bool valu_only = T == kFma || T == kExp || T == kExpOnly;
  double mc = 0, vc = 0, maxc = 0;
  for (int b = 0; b < kCUs; ++b)
    for (int w = 0; w < kWaves; ++w) {
      const double x = (double)c[b * kWaves + w];
      if (x > maxc) maxc = x;
      if (w < 4) (valu_only ? vc : mc) += x;
      else if (both) vc += x;
      else if (!valu_only) mc += x;
    }
  Result r;
  r.ms_per_launch = total_ms / n;
  const int mfma_waves = valu_only ? 0 : (both ? 4 : 8);
  const int valu_waves = valu_only || both ? 4 : 0;
  r.mfma_cycles_per_iter = mfma_waves ? mc / ((double)kCUs * mfma_waves * iters) : 0.0;
  r.valu_cycles_per_iter = valu_waves ? vc / ((double)kCUs * valu_waves * (both ? 2 * iters : iters)) : 0.0;
  r.clock_ghz = maxc / (r.ms_per_launch * 1e-3) / 1e9;  // the slowest wave spans the launch
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return r;
}

// Settle for `seconds` of launches, then time `seconds` more; returns ms
// per launch.
template <typename F>
double timed(F launch, double seconds) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const auto start = std::chrono::steady_clock::now();
  while (std::chrono::duration<double>(std::chrono::steady_clock::now() - start).count() < seconds) {
    launch();
    CHECK(hipDeviceSynchronize());
  }
  int n = 0;
  float total_ms = 0.f;
  while (total_ms < seconds * 1e3f) {
    CHECK(hipEventRecord(e0));
    launch();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    total_ms += ms;
    ++n;
  }
  CHECK(hipGetLastError());
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return total_ms / n;
}

// Largest per-wave cycle count of the last launch (waves < W of each block;
// `stride` entries per block).
double slowest(const long long* cyc, int W, int stride) {
  std::vector<long long> c((size_t)kCUs * stride);
  CHECK(hipMemcpy(c.data(), cyc, c.size() * sizeof(long long), hipMemcpyDeviceToHost));
  long long mx = 0;
  for (int b = 0; b < kCUs; ++b)
    for (int w = 0; w < W; ++w) mx = c[(size_t)b * stride + w] > mx ? c[(size_t)b * stride + w] : mx;
  return (double)mx;
}

template <int MODE>
void step_row(const char* name, int W, const f16x8* ain, float* sink, long long* cyc, double seconds) {
  const int iters = 4000;
  CHECK(hipMemset(cyc, 0, (size_t)kCUs * kWaves * sizeof(long long)));
  const double ms = timed(
      [&]() {
        hipLaunchKernelGGL((step_kernel<MODE>), dim3(kCUs), dim3(64 * W), 0, 0, ain, sink, cyc, iters, 0.05f, 1.0f);
      },
      seconds);
  const double per_iter = slowest(cyc, W, kWaves) / iters;
  const double use = 512.0 * (W / 4) / per_iter;
  std::printf("| %s | %d | %.1f | %.0f%% | %.2f |\n", name, W / 4, per_iter, 100.0 * use,
              slowest(cyc, W, kWaves) / (ms * 1e-3) / 1e9);
  std::fflush(stdout);
}

template <bool TR, int N>
void lds_row(int W, float* sink, long long* cyc, double seconds) {
  const int iters = 20000;
  CHECK(hipMemset(cyc, 0, (size_t)kCUs * 16 * sizeof(long long)));
  timed([&]() { hipLaunchKernelGGL((lds_kernel<TR, N>), dim3(kCUs), dim3(64 * W), 0, 0, sink, cyc, iters); },
        seconds);
  const double bytes = (double)W * iters * N * 64 * (TR ? 8 : 16);
  std::printf("| %s | %d | %d | %.0f |\n", TR ? "ds_read_b64_tr_b16" : "ds_read_b128", W, N,
              bytes / slowest(cyc, W, 16));
  std::fflush(stdout);
}

}  // namespace

int main(int argc, char** argv) {
  const double seconds = argc > 1 ? std::atof(argv[1]) : 1.0;
  const int iters = 20000;
  float* sink;
  long long* cyc;
  CHECK(hipMalloc(&sink, (size_t)kCUs * 512 * sizeof(float)));
  CHECK(hipMalloc(&cyc, (size_t)kCUs * kWaves * sizeof(long long)));
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  std::printf("Device: %s, %d CUs; settle %.1f s, then %.1f s timed per test; %d iterations per wave.\n\n",
              prop.gcnArchName, prop.multiProcessorCount, seconds, seconds, iters);
  std::printf("| test | ms per launch | TFLOP/s | of nominal peak | MFMA-wave cycles / iteration | VALU-wave cycles "
              "/ iteration | shader clock (GHz) |\n|---|---|---|---|---|---|---|\n");
  const double f16_flop = 2.0 * 32 * 32 * 16, fp8_flop = 2.0 * 32 * 32 * 64;
  // The overlap tests give cycles only: their VALU waves outlast the MFMA
  // waves, so work over launch time is not a rate there.
  auto row = [&](const char* name, const Result& r, double flop_per_mfma, double peak_tflops, int mfma_waves,
                 bool rate) {
    char tf[32] = "—", frac[32] = "—", mc[32] = "—", vc[32] = "—";
    if (mfma_waves) {
      const double flop = flop_per_mfma * 4.0 * iters * mfma_waves * kCUs;
      const double t = flop / (r.ms_per_launch * 1e-3) / 1e12;
      if (rate) {
        std::snprintf(tf, sizeof tf, "%.0f", t);
        std::snprintf(frac, sizeof frac, "%.1f%%", 100.0 * t / peak_tflops);
      }
      std::snprintf(mc, sizeof mc, "%.1f", r.mfma_cycles_per_iter);
    }
    if (r.valu_cycles_per_iter > 0) std::snprintf(vc, sizeof vc, "%.1f", r.valu_cycles_per_iter);
    std::printf("| %s | %.3f | %s | %s | %s | %s | %.2f |\n", name, r.ms_per_launch, tf, frac, mc, vc, r.clock_ghz);
    std::fflush(stdout);
  };
  row("mfma f16 (4 x 32x32x16 per iteration)", run<kMfmaF16>(iters, seconds, sink, cyc), f16_flop, 2516.6, 8, true);
  row("mfma bf16 (4 x 32x32x16 per iteration)", run<kMfmaBf16>(iters, seconds, sink, cyc), f16_flop, 2516.6, 8, true);
  row("mfma fp8 (4 x 32x32x64 per iteration)", run<kMfmaFp8>(iters, seconds, sink, cyc), fp8_flop, 5033.2, 8, true);
  row("fma (32 per iteration)", run<kFma>(iters, seconds, sink, cyc), 0, 0, 0, false);
  row("exp (16 exp + 16 mul per iteration)", run<kExp>(iters, seconds, sink, cyc), 0, 0, 0, false);
  row("exp alone (16 per iteration)", run<kExpOnly>(iters, seconds, sink, cyc), 0, 0, 0, false);
  row("mfma f16 + fma on the same SIMDs", run<kMfmaFma>(iters, seconds, sink, cyc), f16_flop, 2516.6, 4, false);
  row("mfma f16 + exp on the same SIMDs", run<kMfmaExp>(iters, seconds, sink, cyc), f16_flop, 2516.6, 4, false);
  row("mfma f16, A operands from LDS", run<kLds>(iters, seconds, sink, cyc), f16_flop, 2516.6, 8, true);
  row("mfma f16 from LDS + fma on the same SIMDs", run<kLdsFma>(iters, seconds, sink, cyc), f16_flop, 2516.6, 4, false);
  row("mfma f16 from LDS + exp on the same SIMDs", run<kLdsExp>(iters, seconds, sink, cyc), f16_flop, 2516.6, 4, false);
  CHECK(hipFree(sink));
  CHECK(hipFree(cyc));

  // Step model and LDS rates: buffers sized for 16 waves per block.
  CHECK(hipMalloc(&sink, (size_t)kCUs * 1024 * sizeof(float)));
  CHECK(hipMalloc(&cyc, (size_t)kCUs * 16 * sizeof(long long)));
  f16x8* ain;
  CHECK(hipMalloc(&ain, 512 * sizeof(f16x8)));
  {
    std::vector<_Float16> h(512 * 8);
    for (size_t i = 0; i < h.size(); ++i) h[i] = (_Float16)(0.01f + 0.0001f * (float)((i * 7) % 50));
    CHECK(hipMemcpy(ain, h.data(), h.size() * sizeof(_Float16), hipMemcpyHostToDevice));
  }
  std::printf("\n| step model (4,000 iterations per wave) | waves per SIMD | cycles / iteration (slowest wave) | "
              "matrix-core use | shader clock (GHz) |\n|---|---|---|---|---|\n");
  step_row<0>("operands in registers", 4, ain, sink, cyc, seconds);
  step_row<0>("operands in registers", 8, ain, sink, cyc, seconds);
  step_row<1>("operands in registers, barrier per iteration", 8, ain, sink, cyc, seconds);
  step_row<2>("operands from LDS", 4, ain, sink, cyc, seconds);
  step_row<2>("operands from LDS", 8, ain, sink, cyc, seconds);
  step_row<3>("operands from LDS, barrier per iteration", 8, ain, sink, cyc, seconds);
  step_row<7>("operands from LDS, P V operands by transpose reads, barrier per iteration", 8, ain, sink, cyc,
              seconds);
  step_row<9>("full softmax mix, operands in registers, barrier", 8, ain, sink, cyc, seconds);
  step_row<15>("full softmax mix, operands from LDS (transpose reads for P V), barrier", 8, ain, sink, cyc, seconds);
  step_row<31>("the same with the LDS reads pinned ahead", 8, ain, sink, cyc, seconds);
  std::printf("\n| LDS read | waves per CU | reads in flight per wave | bytes per clock per CU |\n|---|---|---|---|\n");
  lds_row<false, 2>(8, sink, cyc, seconds);
  lds_row<false, 4>(8, sink, cyc, seconds);
  lds_row<false, 16>(8, sink, cyc, seconds);
  lds_row<false, 16>(16, sink, cyc, seconds);
  lds_row<true, 4>(8, sink, cyc, seconds);
  lds_row<true, 16>(8, sink, cyc, seconds);
  lds_row<true, 16>(16, sink, cyc, seconds);
  CHECK(hipFree(ain));
  CHECK(hipFree(sink));
  CHECK(hipFree(cyc));
  return 0;
}
