// Fused attention forward for MI355X (gfx950, CDNA4).
//
// Computes, per (batch, head), O = softmax(scale * Q K^T) V and the natural
// log-sum-exp of every score row, one key tile at a time with a running row
// max and row sum ("Warp specialization" concept card, implementation
// sketch, consumer loop; the output rescale uses exp(old max - new max), the
// factor the card gives below its sketch).  Scores and probabilities live
// only in registers.
//
// gfx950 mapping
//   * A workgroup owns 128 query rows: 4 waves x 32 rows.  Each wave keeps
//     its Q rows in VGPRs for the whole key loop.
//   * K and V tiles (64 keys) are streamed into a 2-stage LDS ring with
//     16-byte direct-to-LDS global loads (global_load_lds_dwordx4); a
//     vmcnt wait plus s_barrier publishes a stage.  The 16-byte chunks of a
//     row are XOR-swizzled so MFMA operand reads spread over the banks.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{f16,bf16}: the accumulator then gives every lane
//     32 scores of ONE query row (lanes l and l+32 share a row), so the row
//     max and row sum are in-lane work plus one v_permlane32_swap.
//   * The output is accumulated transposed too, O^T += V^T P^T: P^T is the
//     score accumulator itself after exp2 and rounding (no data movement),
//     and V^T comes from LDS through ds_read_b64_tr_b16 transpose reads.
//   * exp is v_exp_f32 (2^x) on scores pre-multiplied by scale * log2(e);
//     LSE is converted back to natural log at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBlockM = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBlockN = 64;                     // keys per tile
constexpr int kStages = 2;                      // LDS ring depth
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) unsigned char lds_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i16x8 lds_i16x8;

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int Nq, Nk;
  int n_qtiles;     // ceil(Nq / kBlockM)
  int total_tiles;  // B * H * n_qtiles
  float c;          // scale * log2(e): scores -> base-2 exponent units
};

// 16-bit element types: MFMA and float -> element rounding (RNE).
template <int DT>
struct Elt;

template <>
struct Elt<ATTN_F16> {
  static __device__ __forceinline__ f32x16 mma(i16x8 a, i16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float x, float y) {
    f16x2 h = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, h);
  }
};

template <>
struct Elt<ATTN_BF16> {
  static __device__ __forceinline__ f32x16 mma(i16x8 a, i16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float x, float y) {
    bf16x2 h = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, h);
  }
};

// XOR swizzle of the 16-byte chunk index within a row, by the row's low 3
// bits.  Within any 8 consecutive rows the swizzle values are distinct, and
// within any 4-aligned group of 4 rows their bits [2:1] are distinct, which
// spreads both the K operand reads (8 rows, same chunk) and the V transpose
// reads (4 rows x 2 adjacent chunks) over distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

__device__ __forceinline__ float swap_halves_max(float x) {
  // v_permlane32_swap with both operands x: result[0] holds lanes 0..31 of x
  // in both halves, result[1] lanes 32..63 in both halves.
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Workgroup -> (batch*head, query tile).  Workgroups are handed to the 8
// XCDs round-robin, so consecutive ids are remapped to let each XCD work
// through neighbouring query tiles of the same heads (their K/V stream then
// stays in that XCD's L2).  Causal: heaviest (last) query tiles first.
__device__ __forceinline__ void schedule(const Params& p, int bid, bool causal, int& bh, int& qt) {
  const int per = p.total_tiles >> 3;
  int lin = bid;
  if (bid < (per << 3)) lin = (bid & 7) * per + (bid >> 3);
  bh = lin / p.n_qtiles;
  qt = lin - bh * p.n_qtiles;
  if (causal) qt = p.n_qtiles - 1 - qt;
}

// One wave's share of the direct-to-LDS loads of a [kBlockN x D] tile.
// Every wave instruction fills 1 KB of LDS contiguously (lane i -> bytes
// 16i..16i+15), so the swizzle is applied on the global side: LDS chunk
// position pc of row r receives global chunk pc ^ swz(r).  Rows past Nk are
// clamped to row Nk-1 (valid memory; such keys are masked to -inf, so their
// values never reach the output).
template <int D>
__device__ __forceinline__ void load_tile(lds_t* dst, const uint16_t* src, int key0, int Nk, int wave,
                                          int lane) {
  constexpr int kRowBytes = D * 2;
  constexpr int kChunks = D / 8;
  constexpr int kRowsPerKB = 1024 / kRowBytes;
  constexpr int kBlocks = kBlockN * kRowBytes / 1024;
  static_assert(kBlocks % kWaves == 0, "tile must split evenly over waves");
#pragma unroll
  for (int i = 0; i < kBlocks / kWaves; ++i) {
    const int b = i * kWaves + wave;
    const int row = b * kRowsPerKB + lane / kChunks;
    const int chunk = (lane % kChunks) ^ swz(row);
    const int key = min(key0 + row, Nk - 1);
    const uint16_t* g = src + (size_t)key * D + chunk * 8;
    __builtin_amdgcn_global_load_lds((const void*)g, (__attribute__((address_space(3))) void*)(dst + b * 1024),
                                     16, 0, 0);
  }
}

// Per-wave state carried across key tiles.
template <int D>
struct WaveState {
  i16x8 qf[D / 16];       // Q rows of this lane as MFMA B-operand fragments
  f32x16 oacc[D / 32];    // O^T accumulator, 32 output columns per block
  float m2;               // running row max, in units of scale*log2(e)
  float lrun;             // running row sum over this lane's half of the keys
  int koff[4];            // per-lane LDS byte offsets of K operand reads
  int voff[2];            // per-lane LDS byte offsets of V transpose reads
};

// One key tile for one wave: S^T = K Q^T, mask, online softmax update,
// O^T = alpha * O^T + V^T P^T.
template <int D, int DT, bool CAUSAL>
__device__ __forceinline__ void consume_tile(WaveState<D>& st, const lds_t* Ks, const lds_t* Vs, int key0,
                                             int qw0, int qrow, int diag, int Nk, int half, float c) {
  constexpr int kRowBytes = D * 2;
  constexpr int kKSteps = D / 16;
  constexpr int kDBlocks = D / 32;

  f32x16 s0 = {}, s1 = {};
#pragma unroll
  for (int s = 0; s < kKSteps; ++s) {
    const int o = st.koff[s & 3] + (s >> 2) * 128;
    const i16x8 a0 = *(const lds_i16x8*)(Ks + o);
    const i16x8 a1 = *(const lds_i16x8*)(Ks + o + 32 * kRowBytes);
    s0 = Elt<DT>::mma(a0, st.qf[s], s0);
    s1 = Elt<DT>::mma(a1, st.qf[s], s1);
  }

  // Mask keys past Nk and (causal) above the diagonal; wave-uniform test.
  const bool ragged = key0 + kBlockN > Nk;
  const bool on_diag = CAUSAL && (key0 + kBlockN - 1 > qw0 + diag);
  if (ragged || on_diag) {
    const int lim = CAUSAL ? min(qrow + diag, Nk - 1) : Nk - 1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (key > lim) s0[r] = -__builtin_inff();
      if (key + 32 > lim) s1[r] = -__builtin_inff();
    }
  }

  // Online softmax statistics for this lane's query row.
  float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
  mx = swap_halves_max(mx);
  const float m2new = fmaxf(st.m2, mx * c);
  const float mref = (m2new == -__builtin_inff()) ? 0.f : m2new;
  const float alpha = __builtin_amdgcn_exp2f(st.m2 - mref);
  st.m2 = m2new;
  float ls = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c, -mref));
    s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c, -mref));
    ls += s0[r] + s1[r];
  }
  st.lrun = alpha * st.lrun + ls;
#pragma unroll
  for (int i = 0; i < kDBlocks; ++i) st.oacc[i] *= alpha;

  // P^T fragments: k-step ks covers keys 16ks..16ks+15 of the tile.
  i16x8 pf[4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    uint32_t w0[4], w1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0[i] = Elt<DT>::pack(s0[8 * hh + 2 * i], s0[8 * hh + 2 * i + 1]);
      w1[i] = Elt<DT>::pack(s1[8 * hh + 2 * i], s1[8 * hh + 2 * i + 1]);
    }
    pf[hh] = __builtin_bit_cast(i16x8, u32x4{w0[0], w0[1], w0[2], w0[3]});
    pf[2 + hh] = __builtin_bit_cast(i16x8, u32x4{w1[0], w1[1], w1[2], w1[3]});
  }

  // O^T += V^T P^T.
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const lds_t* base = Vs + st.voff[db & 1] + (db >> 1) * 128 + 16 * ks * kRowBytes;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)base);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 8 * kRowBytes));
      const i16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      st.oacc[db] = Elt<DT>::mma(a, pf[ks], st.oacc[db]);
    }
  }
}

template <int D, int DT, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) attn_fwd_kernel(Params p) {
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kBlockN * kRowBytes;
  constexpr int kKSteps = D / 16;
  constexpr int kDBlocks = D / 32;
  // The two ring stages are separate LDS objects and the key loop is
  // unrolled by two, so every LDS read names its stage statically: the
  // compiler can then prove that reads of one stage never alias the
  // in-flight direct-to-LDS loads into the other and does not wait on them.
  __shared__ __attribute__((aligned(1024))) unsigned char k_st0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_st0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k_st1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_st1[kTileBytes];
  lds_t* const K0 = (lds_t*)k_st0;
  lds_t* const V0 = (lds_t*)v_st0;
  lds_t* const K1 = (lds_t*)k_st1;
  lds_t* const V1 = (lds_t*)v_st1;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;  // which k-half of the MFMA operands this lane holds
  const int r32 = lane & 31;   // query row within the wave (S^T / O^T column)

  int bh, qt;
  schedule(p, blockIdx.x, CAUSAL, bh, qt);
  const int q0 = qt * kBlockM;
  const int qw0 = q0 + wave * kRowsPerWave;
  const int qrow = qw0 + r32;
  const int diag = p.Nk - p.Nq;  // key j visible to row i iff j <= i + diag

  int kend = p.Nk;
  if (CAUSAL) kend = min(p.Nk, q0 + kBlockM + diag);
  const int nt = kend > 0 ? (kend + kBlockN - 1) / kBlockN : 0;

  const uint16_t* Qb = p.q + (size_t)bh * p.Nq * D;
  const uint16_t* Kb = p.k + (size_t)bh * p.Nk * D;
  const uint16_t* Vb = p.v + (size_t)bh * p.Nk * D;

  WaveState<D> st;
  {
    const int row = min(qrow, p.Nq - 1);
    const i16x8* src = (const i16x8*)(Qb + (size_t)row * D);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) st.qf[s] = src[2 * s + half];
  }
  // K operand: row r32 (+32 for the second key block), chunk 2s + half.
  {
    const int x = swz(r32);
#pragma unroll
    for (int s = 0; s < 4; ++s) st.koff[s] = r32 * kRowBytes + (((2 * s + half) ^ x) * 16);
  }
  // V transpose reads: 16-lane group G reads rows 4*(G>>1) + t/4 and columns
  // 16*(G&1) + 4*(t&3) of each 32-column block (t = lane & 15).
  {
    const int G = lane >> 4, t = lane & 15;
    const int row = 4 * (G >> 1) + (t >> 2);
    const int x = swz(row);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int chunk = 4 * e + 2 * (G & 1) + ((t & 3) >> 1);
      st.voff[e] = row * kRowBytes + ((chunk ^ x) * 16) + 8 * (t & 1);
    }
  }
#pragma unroll
  for (int i = 0; i < kDBlocks; ++i) st.oacc[i] = f32x16{};
  st.m2 = -__builtin_inff();
  st.lrun = 0.f;

  // Causal: tiles entirely above this wave's diagonal contribute nothing.
  const int wave_kend = qw0 + kRowsPerWave - 1 + diag;  // last key any row of the wave sees

  if (nt > 0) {
    load_tile<D>(K0, Kb, 0, p.Nk, wave, lane);
    load_tile<D>(V0, Vb, 0, p.Nk, wave, lane);
  }
  for (int j = 0; j < nt; j += 2) {
    // stage 0 holds tile j; prefetch tile j+1 into stage 1
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < nt) {
      load_tile<D>(K1, Kb, (j + 1) * kBlockN, p.Nk, wave, lane);
      load_tile<D>(V1, Vb, (j + 1) * kBlockN, p.Nk, wave, lane);
    }
    if (!CAUSAL || j * kBlockN <= wave_kend)
      consume_tile<D, DT, CAUSAL>(st, K0, V0, j * kBlockN, qw0, qrow, diag, p.Nk, half, p.c);
    if (j + 1 >= nt) break;
    // stage 1 holds tile j+1; prefetch tile j+2 into stage 0
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 2 < nt) {
      load_tile<D>(K0, Kb, (j + 2) * kBlockN, p.Nk, wave, lane);
      load_tile<D>(V0, Vb, (j + 2) * kBlockN, p.Nk, wave, lane);
    }
    if (!CAUSAL || (j + 1) * kBlockN <= wave_kend)
      consume_tile<D, DT, CAUSAL>(st, K1, V1, (j + 1) * kBlockN, qw0, qrow, diag, p.Nk, half, p.c);
  }

  // Epilogue: O = O^T / l, LSE = ln2 * (m2 + log2 l).
  const float ltot = swap_halves_sum(st.lrun);
  const bool has_key = ltot > 0.f;
  const float inv = has_key ? 1.0f / ltot : 0.f;
  if (qrow < p.Nq) {
    const size_t row = (size_t)bh * p.Nq + qrow;
    if (half == 0) p.lse[row] = has_key ? (st.m2 + __builtin_amdgcn_logf(ltot)) * kLn2 : -__builtin_inff();
    uint16_t* orow = p.o + row * D;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * half;
        u32x2 w;
        w[0] = Elt<DT>::pack(st.oacc[db][4 * g] * inv, st.oacc[db][4 * g + 1] * inv);
        w[1] = Elt<DT>::pack(st.oacc[db][4 * g + 2] * inv, st.oacc[db][4 * g + 3] * inv);
        *(u32x2*)(orow + d0) = w;
      }
    }
  }
}

template <int D, int DT, bool CAUSAL>
int launch_one(const Problem& pr, hipStream_t stream) {
  Params p;
  p.q = (const uint16_t*)pr.q;
  p.k = (const uint16_t*)pr.k;
  p.v = (const uint16_t*)pr.v;
  p.o = (uint16_t*)pr.o;
  p.lse = pr.lse;
  p.Nq = pr.Nq;
  p.Nk = pr.Nk;
  p.n_qtiles = (pr.Nq + kBlockM - 1) / kBlockM;
  const long long total = (long long)pr.B * pr.H * p.n_qtiles;
  if (total > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  p.total_tiles = (int)total;
  p.c = pr.scale * kLog2e;
  hipLaunchKernelGGL((attn_fwd_kernel<D, DT, CAUSAL>), dim3(p.total_tiles), dim3(kThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

template <int D, int DT>
int launch_causal(const Problem& p, hipStream_t s) {
  return p.causal ? launch_one<D, DT, true>(p, s) : launch_one<D, DT, false>(p, s);
}

template <int DT>
int launch_dtype(const Problem& p, hipStream_t s) {
  switch (p.d) {
    case 64: return launch_causal<64, DT>(p, s);
    case 128: return launch_causal<128, DT>(p, s);
    case 256: return launch_causal<256, DT>(p, s);
    default: return ATTN_ERR_HEADDIM;
  }
}

}  // namespace

int launch_forward(const Problem& p, hipStream_t stream) {
  switch (p.dtype) {
    case ATTN_F16: return launch_dtype<ATTN_F16>(p, stream);
    case ATTN_BF16: return launch_dtype<ATTN_BF16>(p, stream);
    default: return ATTN_ERR_DTYPE;
  }
}

}  // namespace attn
