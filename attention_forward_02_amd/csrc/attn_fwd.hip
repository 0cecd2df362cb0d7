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
namespace kernels {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBlockM = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBlockN = 64;                     // keys per tile
constexpr int kStages = 2;                      // LDS ring depth
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
  static __device__ __forceinline__ uint32_t pack(float x, float y) {  // v_cvt_pk_f16_f32 (RNE)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, f16x2));
  }
};

template <>
struct Elt<ATTN_BF16> {
  static __device__ __forceinline__ f32x16 mma(i16x8 a, i16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float x, float y) {  // v_cvt_pk_bf16_f32 (RNE)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
  }
};

// XOR swizzle of the 16-byte chunk index within a row.  The gfx950 LDS
// serves 256 bytes (64 banks x 4 B) per cycle, i.e. 16 lanes of a 128-bit
// read or 32 lanes of a 64-bit read.  Two access patterns must be
// conflict-free:
//   * K operand reads (ds_read_b128): 16 consecutive rows, one logical chunk;
//   * V transpose reads (ds_read_b64_tr_b16): 4 consecutive rows (a 4-aligned
//     group) x 4 consecutive chunks (a 4-aligned group).
// Rows of >= 256 bytes (d >= 128): f(r) = 4*(r&3) + ((r>>2)&3) is a bijection
// on r mod 16, and inside a 4-row group its values differ in bits [3:2].
// Rows of 128 bytes (d = 64) put two rows in one 256-byte bank window: f(r)
// = 4*((r>>1)&1) + ((r>>2)&3) is distinct over the even and over the odd
// rows of any 16, and rows r, r+2 of a 4-row group differ in bit 2.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D >= 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return ((row & 2) << 1) | ((row >> 2) & 3);
}

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

// Direct-to-LDS tile loader for one wave (buffer_load_dwordx4 ... lds).
// Every wave instruction fills 1 KB of LDS contiguously (lane i -> bytes
// 16i..16i+15), so the swizzle is applied on the global side: LDS chunk
// position pc of row r receives global chunk pc ^ swz(r).  The buffer
// resource spans exactly one head's [Nk x D] rows, so rows past Nk (a ragged
// last tile) fail the hardware range check and arrive as zeros; their
// scores are masked to -inf and their zero values meet P = 0.
template <int D>
struct TileLoader {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;
  static constexpr int kRowsPerKB = 1024 / kRowBytes;
  static constexpr int kBlocks = kBlockN * kRowBytes / 1024;
  static constexpr int kPerWave = kBlocks / kWaves;
  static_assert(kBlocks % kWaves == 0, "tile must split evenly over waves");
  int voff[kPerWave];   // byte offset of this lane's chunk within a tile
  int lds[kPerWave];    // LDS byte offset of the wave instruction's 1 KB block

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int b = i * kWaves + wave;
      const int row = b * kRowsPerKB + lane / kChunks;
      voff[i] = row * kRowBytes + ((lane % kChunks) ^ swz<D>(row)) * 16;
      lds[i] = b * 1024;
    }
  }
  __device__ __forceinline__ void load(lds_t* dst, __amdgpu_buffer_rsrc_t src, int key0) const {
    const int tile = key0 * kRowBytes;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)(dst + lds[i]), 16,
                                               voff[i] + tile, 0, 0, 0);
  }
};

// Buffer resource over `bytes` bytes at `base` (raw, stride 0; gfx9 word 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}

// Per-wave state carried across key tiles.
template <int D>
struct WaveState {
  static constexpr int kKOff = (D / 16 < 8) ? D / 16 : 8;
  i16x8 qf[D / 16];       // Q rows of this lane as MFMA B-operand fragments
  f32x16 oacc[D / 32];    // O^T accumulator, 32 output columns per block
  float m2;               // reference row max for exp2, in units of scale*log2(e)
  float lrun;             // running row sum over this lane's half of the keys
  int koff[kKOff];        // per-lane LDS byte offsets of K operand reads
  int voff[4][2];         // per-lane LDS byte offsets of V transpose reads

  __device__ __forceinline__ void init_offsets(int lane) {
    constexpr int kRowBytes = D * 2;
    const int half = lane >> 5, r32 = lane & 31;
    // K operand: row r32 (+32 for the second key block), chunk 2s + half.
    const int xk = swz<D>(r32);
#pragma unroll
    for (int s = 0; s < kKOff; ++s) koff[s] = r32 * kRowBytes + (((2 * s + half) ^ xk) * 16);
    // V transpose reads: 16-lane group G reads rows 4*(G>>1) + t/4 (+8 for
    // the second read) and columns 16*(G&1) + 4*(t&3) of a 32-column block.
    const int G = lane >> 4, t = lane & 15;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = 4 * (G >> 1) + (t >> 2) + 8 * e;
      const int x = swz<D>(row);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int chunk = (4 * db + 2 * (G & 1) + ((t & 3) >> 1)) ^ x;
        voff[db][e] = row * kRowBytes + chunk * 16 + 8 * (t & 1);
      }
    }
  }
};

// S^T = K Q^T for the 64 keys of one tile: two 32x32 accumulators.
template <int D, int DT>
__device__ __forceinline__ void tile_scores(const WaveState<D>& st, const lds_t* Ks, f32x16& s0, f32x16& s1) {
  constexpr int kRowBytes = D * 2;
  constexpr int kKOff = WaveState<D>::kKOff;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const int o = st.koff[s % kKOff] + (s / kKOff) * 256;
    const i16x8 a0 = *(const lds_i16x8*)(Ks + o);
    const i16x8 a1 = *(const lds_i16x8*)(Ks + o + 32 * kRowBytes);
    s0 = Elt<DT>::mma(a0, st.qf[s], s == 0 ? f32x16{} : s0);
    s1 = Elt<DT>::mma(a1, st.qf[s], s == 0 ? f32x16{} : s1);
  }
}

// Rows may hold p = exp2(s*c - m2) up to 2^kLazy before the reference max
// m2 is raised and O, l rescaled: the final O / l and m2 + log2 l do not
// depend on which reference was used, only the rounding does.
constexpr float kLazy = 8.0f;

// Softmax of one tile's scores (s0, s1), ready for the P V product.
struct SoftmaxOut {
  i16x8 pf[4];   // P^T fragments: k-step ks covers keys 16ks..16ks+15 of the tile
  float alpha;   // factor O and l must be multiplied by before adding this tile
  bool rescale;  // wave-uniform: alpha != 1 for some lane
};

// Phase A of one pipelined step, a single branch-free block: the score
// MFMAs of the NEXT tile (K from `Kn`) interleaved with the softmax of the
// CURRENT tile (mask, row max, reference update, exp2, rounding of P).
// sched_group_barrier lays the block out as [MFMA, ~7 VALU, K read] x 16 so
// that the wave keeps issuing softmax VALU work while each MFMA runs.
template <int D, int DT, bool MASK>
__device__ __forceinline__ SoftmaxOut phase_a(WaveState<D>& st, f32x16 s0, f32x16 s1, const lds_t* Kn,
                                              f32x16& n0, f32x16& n1, int rem, int half, float c) {
  tile_scores<D, DT>(st, Kn, n0, n1);

  if (MASK) {
    // rem = last visible key of this lane's row minus the lane's first key
    // (key0 + 4*half); element r of s0 sits 8*(r>>2) + (r&3) keys later, of
    // s1 another 32.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int o = 8 * (r >> 2) + (r & 3);
      s0[r] = o > rem ? -__builtin_inff() : s0[r];
      s1[r] = o + 32 > rem ? -__builtin_inff() : s1[r];
    }
  }
  float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
  mx = swap_halves_max(mx);
  const float m2t = mx * c;
  SoftmaxOut out;
  out.rescale = __any(m2t > st.m2 + kLazy);
  const float m2new = out.rescale ? fmaxf(st.m2, m2t) : st.m2;
  out.alpha = (m2new == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(st.m2 - m2new);
  st.m2 = m2new;
  const float mref = (m2new == -__builtin_inff()) ? 0.f : m2new;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c, -mref));
    s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c, -mref));
  }
  // row sum from the unrounded probabilities (kept in fp32)
  float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    ls0 += s0[r];
    ls1 += s1[r];
  }
  st.lrun = out.alpha * st.lrun + (ls0 + ls1);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    out.pf[hh] = __builtin_bit_cast(i16x8, u32x4{Elt<DT>::pack(s0[8 * hh + 0], s0[8 * hh + 1]),
                                                 Elt<DT>::pack(s0[8 * hh + 2], s0[8 * hh + 3]),
                                                 Elt<DT>::pack(s0[8 * hh + 4], s0[8 * hh + 5]),
                                                 Elt<DT>::pack(s0[8 * hh + 6], s0[8 * hh + 7])});
    out.pf[2 + hh] = __builtin_bit_cast(i16x8, u32x4{Elt<DT>::pack(s1[8 * hh + 0], s1[8 * hh + 1]),
                                                     Elt<DT>::pack(s1[8 * hh + 2], s1[8 * hh + 3]),
                                                     Elt<DT>::pack(s1[8 * hh + 4], s1[8 * hh + 5]),
                                                     Elt<DT>::pack(s1[8 * hh + 6], s1[8 * hh + 7])});
  }
  // Interleave: 4 K reads up front, then [MFMA, 7 VALU, K read] x 16.
  constexpr int kMfma = 2 * (D / 16);
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < kMfma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
    if (i + 4 < kMfma) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  return out;
}

// Phase B: O^T = alpha * O^T + V^T P^T (the rescale is skipped when no lane
// raised its reference max).
template <int D, int DT>
__device__ __forceinline__ void phase_b(WaveState<D>& st, const SoftmaxOut& sm, const lds_t* Vs) {
  constexpr int kRowBytes = D * 2;
  constexpr int kDBlocks = D / 32;
  if (sm.rescale) {
#pragma unroll
    for (int i = 0; i < kDBlocks; ++i) st.oacc[i] *= sm.alpha;
  }
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const lds_t* base = Vs + (db >> 2) * 256 + 16 * ks * kRowBytes;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + st.voff[db & 3][0]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + st.voff[db & 3][1]));
      const i16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      st.oacc[db] = Elt<DT>::mma(a, sm.pf[ks], st.oacc[db]);
    }
  }
}

// One pipelined step for tile j (scores in s0/s1): next tile's scores into
// n0/n1 from Kn, softmax and P V of tile j with V from Vs.
template <int D, int DT, bool CAUSAL>
__device__ __forceinline__ void step(WaveState<D>& st, f32x16 s0, f32x16 s1, f32x16& n0, f32x16& n1,
                                     const lds_t* Kn, const lds_t* Vs, int key0, int qw0, int qrow, int diag,
                                     int Nk, int half, float c) {
  const bool ragged = key0 + kBlockN > Nk;
  const bool on_diag = CAUSAL && (key0 + kBlockN - 1 > qw0 + diag);
  SoftmaxOut sm;
  if (ragged || on_diag) {
    const int lim = CAUSAL ? min(qrow + diag, Nk - 1) : Nk - 1;
    sm = phase_a<D, DT, true>(st, s0, s1, Kn, n0, n1, lim - key0 - 4 * half, half, c);
  } else {
    sm = phase_a<D, DT, false>(st, s0, s1, Kn, n0, n1, 0, half, c);
  }
  phase_b<D, DT>(st, sm, Vs);
}

template <int D, int DT, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) attn_fwd_kernel(Params p) {
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kBlockN * kRowBytes;
  constexpr int kKSteps = D / 16;
  constexpr int kDBlocks = D / 32;
  // K and V rings of two stages each, as four separate LDS objects.  K runs
  // one tile ahead of V: while a wave applies the softmax of tile j it
  // already multiplies K_{j+1} (the two-stage overlap of score MFMAs with
  // softmax inside one wave).  With every stage a distinct object and the
  // loop unrolled by two, each LDS read names its stage statically, so the
  // compiler can prove it never aliases the in-flight direct-to-LDS loads
  // into another stage and does not wait on them.
  __shared__ __attribute__((aligned(1024))) unsigned char k_st0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k_st1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_st0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_st1[kTileBytes];
  lds_t* const K0 = (lds_t*)k_st0;
  lds_t* const K1 = (lds_t*)k_st1;
  lds_t* const V0 = (lds_t*)v_st0;
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
  // Causal: tiles starting past this wave's last visible key contribute nothing.
  const int wave_kend = CAUSAL ? qw0 + kRowsPerWave - 1 + diag : p.Nk;

  const uint16_t* Qb = p.q + (size_t)bh * p.Nq * D;
  const uint32_t head_bytes = (uint32_t)p.Nk * kRowBytes;
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc(p.k + (size_t)bh * p.Nk * D, head_bytes);
  const __amdgpu_buffer_rsrc_t Vr = make_rsrc(p.v + (size_t)bh * p.Nk * D, head_bytes);

  TileLoader<D> ld;
  ld.init(wave, lane);
  WaveState<D> st;
  st.init_offsets(lane);
  {
    const int row = min(qrow, p.Nq - 1);
    const i16x8* src = (const i16x8*)(Qb + (size_t)row * D);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) st.qf[s] = src[2 * s + half];
  }
#pragma unroll
  for (int i = 0; i < kDBlocks; ++i) st.oacc[i] = f32x16{};
  st.m2 = -__builtin_inff();
  st.lrun = 0.f;

  // Scores of even tiles live in (a0, a1), of odd tiles in (b0, b1).  Each
  // step computes the next tile's scores unconditionally (the K stage it
  // reads always holds valid LDS; after the last tile the result is unused)
  // so that the MFMAs share one branch-free block with the softmax.
  f32x16 a0, a1, b0, b1;
  if (nt > 0) {
    ld.load(K0, Kr, 0);
    ld.load(V0, Vr, 0);
    if (nt > 1) ld.load(K1, Kr, kBlockN);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    tile_scores<D, DT>(st, K0, a0, a1);
  }
  for (int j = 0; j < nt; j += 2) {
    // Even step: (a0, a1) = scores of tile j; K_{j+1} is in K1, V_j in V0.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 2 < nt) ld.load(K0, Kr, (j + 2) * kBlockN);
    if (j + 1 < nt) ld.load(V1, Vr, (j + 1) * kBlockN);
    if (j * kBlockN <= wave_kend)
      step<D, DT, CAUSAL>(st, a0, a1, b0, b1, K1, V0, j * kBlockN, qw0, qrow, diag, p.Nk, half, p.c);
    if (j + 1 >= nt) break;
    // Odd step: (b0, b1) = scores of tile j+1; K_{j+2} is in K0, V_{j+1} in V1.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 3 < nt) ld.load(K1, Kr, (j + 3) * kBlockN);
    if (j + 2 < nt) ld.load(V0, Vr, (j + 2) * kBlockN);
    if ((j + 1) * kBlockN <= wave_kend)
      step<D, DT, CAUSAL>(st, b0, b1, a0, a1, K0, V1, (j + 1) * kBlockN, qw0, qrow, diag, p.Nk, half, p.c);
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

// Explicit instantiations: every kernel the dispatcher can launch, so the
// host pass emits each launch stub.
#define ATTN_INSTANTIATE(D, DT)                                                  \
  template __global__ void attn_fwd_kernel<D, DT, false>(Params);               \
  template __global__ void attn_fwd_kernel<D, DT, true>(Params);
ATTN_INSTANTIATE(64, ATTN_F16)
ATTN_INSTANTIATE(128, ATTN_F16)
ATTN_INSTANTIATE(256, ATTN_F16)
ATTN_INSTANTIATE(64, ATTN_BF16)
ATTN_INSTANTIATE(128, ATTN_BF16)
ATTN_INSTANTIATE(256, ATTN_BF16)
#undef ATTN_INSTANTIATE

}  // namespace kernels

using namespace kernels;

int launch_forward(const Problem& p, hipStream_t stream) {
  switch (p.dtype) {
    case ATTN_F16: return launch_dtype<ATTN_F16>(p, stream);
    case ATTN_BF16: return launch_dtype<ATTN_BF16>(p, stream);
    default: return ATTN_ERR_DTYPE;
  }
}

}  // namespace attn
