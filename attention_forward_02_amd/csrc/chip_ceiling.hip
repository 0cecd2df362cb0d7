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
       kExpOnly = 9 };
constexpr int kCUs = 256;
constexpr int kWaves = 8;

template <int T>
__global__ void __launch_bounds__(512) ceiling_kernel(float* sink, long long* cycles, int iters) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr bool kPair = T == kMfmaFma || T == kMfmaExp || T == kLdsFma || T == kLdsExp;
  constexpr bool kUsesLds = T == kLds || T == kLdsFma || T == kLdsExp;
  constexpr bool kExpLoop = T == kExp || T == kMfmaExp || T == kLdsExp;
  const bool mfma_wave = (T == kMfmaF16 || T == kMfmaFp8 || T == kLds) || (kPair && w < 4);
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
  return 0;
}
