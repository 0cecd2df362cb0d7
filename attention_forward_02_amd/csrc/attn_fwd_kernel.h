#pragma once
// Fused attention forward for MI355X (gfx950, CDNA4): device code, shared by
// one translation unit per head dimension (attn_fwd_d{64,128,256}.hip).
//
// Computes, per (batch, head), O = softmax(scale * Q K^T) V and the natural
// log-sum-exp of every score row, one key tile at a time with a running row
// max and row sum ("Warp specialization" concept card, implementation
// sketch, consumer loop; the output rescale uses exp(old max - new max), the
// factor the card gives below its sketch).  Scores and probabilities live
// only in registers.
//
// gfx950 mapping
//   * Every wave owns 32 query rows and keeps them in VGPRs for the whole
//     key loop.
//   * K and V tiles (64 keys) stream into a two-stage LDS ring with 16-byte
//     direct-to-LDS buffer loads; a vmcnt wait plus s_barrier publishes a
//     stage.  The 16-byte chunks of a row are XOR-swizzled so MFMA operand
//     reads spread over the 64 LDS banks.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{f16,bf16}: the accumulator then gives every lane
//     32 scores of ONE query row (lanes l and l+32 share a row), so the row
//     max and row sum are in-lane work plus one v_permlane32_swap.
//   * The output is accumulated transposed too, O^T += V^T P^T: P^T is the
//     score accumulator itself after exp2 and rounding (no data movement),
//     and V^T comes from LDS through ds_read_b64_tr_b16 transpose reads.
//   * exp is v_exp_f32 (2^x) on scores pre-multiplied by scale * log2(e);
//     LSE is converted back to natural log at the end.
//
// Schedule (4 waves, 128 query rows per workgroup, two workgroups per CU at
// d <= 128 so that every SIMD runs two waves): each step overlaps the score
// MFMAs of the next tile with the exponentials of the current one, and the
// P V MFMAs with the row sums and the next tile's row max (the pages'
// two-stage overlap of matrix multiplies and softmax), so a wave issues
// only about five VALU instructions per MFMA and the matrix core stays fed
// from both waves of the SIMD.  Masking is folded into the initial values
// of the score accumulators, so the step is the same branch-free code for
// every tile.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn.h"
#include "attn_internal.h"

namespace attn {
namespace kernels {

constexpr int kRowsPerWave = 32;
constexpr int kBlockN = 64;  // keys per tile
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
  int n_qtiles;     // ceil(Nq / query rows per workgroup)
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

// Direct-to-LDS tile loader for one wave of an NW-wave workgroup
// (buffer_load_dwordx4 ... lds).  Every wave instruction fills 1 KB of LDS
// contiguously (lane i -> bytes 16i..16i+15), so the swizzle is applied on
// the global side: LDS chunk position pc of row r receives global chunk
// pc ^ swz(r).  The buffer resource spans exactly one head's [Nk x D] rows,
// so rows past Nk (a ragged last tile) fail the hardware range check and
// arrive as zeros; their scores are masked to -inf and their zero values
// meet P = 0.
template <int D, int NW>
struct TileLoader {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;
  static constexpr int kRowsPerKB = 1024 / kRowBytes;
  static constexpr int kBlocks = kBlockN * kRowBytes / 1024;
  static constexpr int kPerWave = kBlocks / NW;
  static_assert(kBlocks % NW == 0, "tile must split evenly over waves");
  int voff[kPerWave];   // byte offset of this lane's chunk within a tile
  int lds[kPerWave];    // LDS byte offset of the wave instruction's 1 KB block

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int b = i * NW + wave;
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

  __device__ __forceinline__ void init(const uint16_t* Qb, int qrow, int Nq, int lane) {
    constexpr int kRowBytes = D * 2;
    const int half = lane >> 5, r32 = lane & 31;
    // Q rows of this lane: chunk (2s + half) of the row, clamped for rows past Nq.
    const i16x8* src = (const i16x8*)(Qb + (size_t)min(qrow, Nq - 1) * D);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = src[2 * s + half];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    m2 = -__builtin_inff();
    lrun = 0.f;
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

// S^T = K Q^T for the 64 keys of one tile: two 32x32 accumulators.  With
// BIAS the accumulators start from their current contents (a 0 / -inf mask
// bias, see score_bias) instead of zero.
template <int D, int DT, bool BIAS = false>
__device__ __forceinline__ void tile_scores(const WaveState<D>& st, const lds_t* Ks, f32x16& s0, f32x16& s1) {
  constexpr int kRowBytes = D * 2;
  constexpr int kKOff = WaveState<D>::kKOff;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const int o = st.koff[s % kKOff] + (s / kKOff) * 256;
    const i16x8 a0 = *(const lds_i16x8*)(Ks + o);
    const i16x8 a1 = *(const lds_i16x8*)(Ks + o + 32 * kRowBytes);
    s0 = Elt<DT>::mma(a0, st.qf[s], (s == 0 && !BIAS) ? f32x16{} : s0);
    s1 = Elt<DT>::mma(a1, st.qf[s], (s == 0 && !BIAS) ? f32x16{} : s1);
  }
}

// O^T += V^T P^T for one tile, V from LDS through transpose reads.
template <int D, int DT>
__device__ __forceinline__ void pv_tile(WaveState<D>& st, const i16x8 (&pf)[4], const lds_t* Vs) {
  constexpr int kRowBytes = D * 2;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const lds_t* base = Vs + (db >> 2) * 256 + 16 * ks * kRowBytes;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + st.voff[db & 3][0]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + st.voff[db & 3][1]));
      const i16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      st.oacc[db] = Elt<DT>::mma(a, pf[ks], st.oacc[db]);
    }
  }
}

// Rows may hold p = exp2(s*c - m2) up to 2^kLazy before the reference max
// m2 is raised and O, l rescaled: the final O / l and m2 + log2 l do not
// depend on which reference was used, only the rounding does.
constexpr float kLazy = 8.0f;

// Mask bias of a tile: rem = last visible key of this lane's row minus the
// lane's first key (key0 + 4*half); element r of s0 sits 8*(r>>2) + (r&3)
// keys later, of s1 another 32.
__device__ __forceinline__ void mask_bias(f32x16& s0, f32x16& s1, int rem) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int o = 8 * (r >> 2) + (r & 3);
    s0[r] = o > rem ? -__builtin_inff() : 0.f;
    s1[r] = o + 32 > rem ? -__builtin_inff() : 0.f;
  }
}

// Row max of one tile over this lane's 32 scores (two v_max3 chains) and the
// other half of the row, times c.
__device__ __forceinline__ float tile_max2(const f32x16& s0, const f32x16& s1, float c) {
  float ma = fmaxf(s0[0], s1[0]), mb = fmaxf(s0[1], s1[1]);
#pragma unroll
  for (int r = 2; r < 16; r += 2) {
    ma = fmaxf(fmaxf(ma, s0[r]), s1[r]);
    mb = fmaxf(fmaxf(mb, s0[r + 1]), s1[r + 1]);
  }
  return swap_halves_max(fmaxf(ma, mb)) * c;
}

template <int DT>
__device__ __forceinline__ i16x8 pack8(const f32x16& p, int base) {
  return __builtin_bit_cast(i16x8, u32x4{Elt<DT>::pack(p[base + 0], p[base + 1]),
                                         Elt<DT>::pack(p[base + 2], p[base + 3]),
                                         Elt<DT>::pack(p[base + 4], p[base + 5]),
                                         Elt<DT>::pack(p[base + 6], p[base + 7])});
}

// Per-wave constants of the key loop.
struct LoopCtx {
  int qw0, qrow, diag, Nk, half, wave_kend, nt;
  float c;
  // Causal: a tile is visible to the wave iff it starts at or before the
  // wave's last visible key (visibility only decreases along the loop).
  __device__ __forceinline__ bool visible(int t) const { return t < nt && t * kBlockN <= wave_kend; }
  // Tile t needs masking (ragged end, or the causal diagonal crosses it).
  template <bool CAUSAL>
  __device__ __forceinline__ bool needs_mask(int t) const {
    const int key0 = t * kBlockN;
    return (key0 + kBlockN > Nk) || (CAUSAL && key0 + kBlockN - 1 > qw0 + diag);
  }
  template <bool CAUSAL>
  __device__ __forceinline__ int mask_rem(int t) const {
    const int lim = CAUSAL ? min(qrow + diag, Nk - 1) : Nk - 1;
    return lim - t * kBlockN - 4 * half;
  }
};

// Initial accumulators of tile t's scores, so that the score MFMAs apply the
// mask themselves: 0 for visible keys, -inf for keys past Nk or above the
// causal diagonal, and -inf everywhere for a tile the wave does not see (its
// softmax then gives P = 0 and leaves m, l and O alone).  Returns false when
// no element is masked (the MFMAs may then start from zero).
template <bool CAUSAL>
__device__ __forceinline__ bool score_bias(const LoopCtx& cx, int t, f32x16& s0, f32x16& s1) {
  const bool vis = cx.visible(t);
  if (vis && !cx.needs_mask<CAUSAL>(t)) return false;
  mask_bias(s0, s1, vis ? cx.mask_rem<CAUSAL>(t) : -(1 << 30));
  return true;
}

// Scores of tile t (K from Ks) into (s0, s1), masked through the bias.
template <int D, int DT, bool CAUSAL>
__device__ __forceinline__ void masked_scores(const WaveState<D>& st, const LoopCtx& cx, int t, const lds_t* Ks,
                                              f32x16& s0, f32x16& s1) {
  if (score_bias<CAUSAL>(cx, t, s0, s1)) tile_scores<D, DT, true>(st, Ks, s0, s1);
  else tile_scores<D, DT, false>(st, Ks, s0, s1);
}

// Reference update from a tile's row max (in units of scale*log2(e)):
// raise m2 only when some row's max exceeds it by more than kLazy.  Returns
// the factor O and l must be multiplied by, 1 when nothing changed.
__device__ __forceinline__ float update_reference(float& m2, float m2t, bool& rescale) {
  rescale = __any(m2t > m2 + kLazy);  // wave-uniform
  const float m2new = rescale ? fmaxf(m2, m2t) : m2;
  const float alpha = (m2new == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(m2 - m2new);
  m2 = m2new;
  return alpha;
}

// One step of the key loop for tile j, as two MFMA blocks with the softmax
// VALU work spread over both (about 5 VALU instructions per MFMA, which a
// wave issues while its MFMAs run):
//   phase A: S_{j+1} = K_{j+1} Q^T (Kn; into n0, n1)  | p_j = exp2(s_j*c - m2),
//                                                         P_j = round(p_j)
//   phase B: O^T += V_j^T P_j^T (Vs)                  | l += sum(p_j),
//                                                         row max of S_{j+1},
//                                                         reference update
// then, rarely, O and l are rescaled to the new reference.  s0, s1 hold S_j
// on entry (and p_j after phase A).
template <int D, int DT, bool CAUSAL>
__device__ __forceinline__ void step(WaveState<D>& st, const LoopCtx& cx, int j, f32x16& s0, f32x16& s1,
                                     f32x16& n0, f32x16& n1, const lds_t* Kn, const lds_t* Vs) {
  // Phase A
  masked_scores<D, DT, CAUSAL>(st, cx, j + 1, Kn, n0, n1);
  const float mref = (st.m2 == -__builtin_inff()) ? 0.f : st.m2;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], cx.c, -mref));
    s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], cx.c, -mref));
  }
  i16x8 pf[4];
  pf[0] = pack8<DT>(s0, 0);
  pf[1] = pack8<DT>(s0, 8);
  pf[2] = pack8<DT>(s1, 0);
  pf[3] = pack8<DT>(s1, 8);
  __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // Phase B
  pv_tile<D, DT>(st, pf, Vs);
  float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    ls0 += s0[r];
    ls1 += s1[r];
  }
  st.lrun += ls0 + ls1;
  bool rescale;
  const float alpha = update_reference(st.m2, tile_max2(n0, n1, cx.c), rescale);
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (rescale) {
    st.lrun *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) st.oacc[i] *= alpha;
  }
}

// Output: O = O^T / l (rounded to the element type), LSE = ln2 * (m2 + log2 l).
template <int D, int DT>
__device__ __forceinline__ void store_output(const Params& p, const WaveState<D>& st, int bh, int qrow,
                                             int half) {
  const float ltot = swap_halves_sum(st.lrun);
  const bool has_key = ltot > 0.f;
  const float inv = has_key ? 1.0f / ltot : 0.f;
  if (qrow < p.Nq) {
    const size_t row = (size_t)bh * p.Nq + qrow;
    if (half == 0) p.lse[row] = has_key ? (st.m2 + __builtin_amdgcn_logf(ltot)) * kLn2 : -__builtin_inff();
    uint16_t* orow = p.o + row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
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

constexpr int kWaves = 4;
constexpr int kBlockM = kWaves * kRowsPerWave;  // query rows per workgroup

template <int D, int DT, bool CAUSAL>
__global__ void __launch_bounds__(64 * kWaves) attn_fwd_kernel(Params p) {
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kBlockN * kRowBytes;
  // K and V rings of two stages each, as four separate LDS objects.  K runs
  // one tile ahead of V: step j reads K_{j+1} (scores of the next tile) and
  // V_j while K_{j+2} and V_{j+1} stream in.  With every stage a distinct
  // object and the loop unrolled by two, each LDS read names its stage
  // statically, so the compiler can prove it never aliases the in-flight
  // direct-to-LDS loads into another stage and does not wait on them.
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

  int bh, qt;
  schedule(p, blockIdx.x, CAUSAL, bh, qt);
  const int q0 = qt * kBlockM;
  LoopCtx cx;
  cx.qw0 = q0 + wave * kRowsPerWave;
  cx.qrow = cx.qw0 + (lane & 31);
  cx.diag = p.Nk - p.Nq;  // key j visible to row i iff j <= i + diag
  cx.Nk = p.Nk;
  cx.half = lane >> 5;
  cx.c = p.c;
  cx.wave_kend = CAUSAL ? cx.qw0 + kRowsPerWave - 1 + cx.diag : p.Nk;
  int kend = p.Nk;
  if (CAUSAL) kend = min(p.Nk, q0 + kBlockM + cx.diag);
  const int nt = kend > 0 ? (kend + kBlockN - 1) / kBlockN : 0;
  cx.nt = nt;

  const uint32_t head_bytes = (uint32_t)p.Nk * kRowBytes;
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc(p.k + (size_t)bh * p.Nk * D, head_bytes);
  const __amdgpu_buffer_rsrc_t Vr = make_rsrc(p.v + (size_t)bh * p.Nk * D, head_bytes);

  TileLoader<D, kWaves> ld;
  ld.init(wave, lane);
  WaveState<D> st;
  st.init(p.q + (size_t)bh * p.Nq * D, cx.qrow, p.Nq, lane);

  // Scores (then probabilities) of even tiles live in (a0, a1), of odd
  // tiles in (b0, b1).
  f32x16 a0, a1, b0, b1;
  if (nt > 0) {
    // K_1 is loaded even when there is no tile 1: its rows then fail the
    // range check and arrive as zeros, so every K stage a step reads holds
    // finite data (scores of tiles past the end are -inf, never NaN).
    ld.load(K0, Kr, 0);
    ld.load(V0, Vr, 0);
    ld.load(K1, Kr, kBlockN);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    masked_scores<D, DT, CAUSAL>(st, cx, 0, K0, a0, a1);
    bool rescale;
    update_reference(st.m2, tile_max2(a0, a1, cx.c), rescale);
  }
  for (int j = 0; j < nt; j += 2) {
    // Even step: (a0, a1) = S_j; K_{j+1} in K1, V_j in V0; K_{j+2} -> K0, V_{j+1} -> V1.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 2 < nt) ld.load(K0, Kr, (j + 2) * kBlockN);
    if (j + 1 < nt) ld.load(V1, Vr, (j + 1) * kBlockN);
    step<D, DT, CAUSAL>(st, cx, j, a0, a1, b0, b1, K1, V0);
    if (j + 1 >= nt) break;
    // Odd step: (b0, b1) = S_{j+1}; K_{j+2} in K0, V_{j+1} in V1; K_{j+3} -> K1, V_{j+2} -> V0.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 3 < nt) ld.load(K1, Kr, (j + 3) * kBlockN);
    if (j + 2 < nt) ld.load(V0, Vr, (j + 2) * kBlockN);
    step<D, DT, CAUSAL>(st, cx, j + 1, b0, b1, a0, a1, K0, V1);
  }
  store_output<D, DT>(p, st, bh, cx.qrow, cx.half);
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------
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
  hipLaunchKernelGGL((attn_fwd_kernel<D, DT, CAUSAL>), dim3(p.total_tiles), dim3(64 * kWaves), 0, stream, p);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Dispatch one head dimension over dtype and causality.
template <int D>
int launch_head_dim(const Problem& p, hipStream_t s) {
  switch (p.dtype) {
    case ATTN_F16:
      return p.causal ? launch_one<D, ATTN_F16, true>(p, s) : launch_one<D, ATTN_F16, false>(p, s);
    case ATTN_BF16:
      return p.causal ? launch_one<D, ATTN_BF16, true>(p, s) : launch_one<D, ATTN_BF16, false>(p, s);
    default:
      return ATTN_ERR_DTYPE;
  }
}

}  // namespace kernels
}  // namespace attn
