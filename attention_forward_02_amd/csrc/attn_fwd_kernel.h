#pragma once
// Fused attention forward for MI355X (gfx950, CDNA4): device code, shared by
// one translation unit per head dimension and input format
// (attn_fwd_d{64,128,256}.hip, attn_fwd_d{64,128,256}_fp8.hip).
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
//     v_mfma_f32_32x32x16_{f16,bf16} (or v_mfma_f32_32x32x64_f8f6f4 for
//     E4M3): the accumulator then gives every lane 32 scores of ONE query
//     row (lanes l and l+32 share a row), so the row max and row sum are
//     in-lane work plus one v_permlane32_swap.
//   * The output is accumulated transposed too, O^T += V^T P^T: P^T is the
//     score accumulator itself after exp2 and rounding (no data movement),
//     and V^T comes from LDS through ds_read_b64_tr_b16 / ds_read_b64_tr_b8
//     transpose reads.
//   * exp is v_exp_f32 (2^x) on scores pre-multiplied by scale * log2(e);
//     LSE is converted back to natural log at the end.
//
// The four default kernels share these pieces:
//   * attn_fwd_producer_kernel (binary16 d = 128): eight consumer waves run
//     the sequential step below while a ninth, producer wave streams K and
//     V into the LDS ring;
//   * attn_fwd_kernel (bfloat16 d = 128, 16-bit d = 64, E4M3 d = 64): each step
//     overlaps the score MFMAs of the next tile with the exponentials of the
//     current one, and the P V MFMAs with the row sums and the next tile's
//     row max (the pages' two-stage overlap of matrix multiplies and
//     softmax), while the SIMD's second wave fills the matrix core from its
//     own step;
//   * attn_fwd_seq_kernel (E4M3 d = 128 with 128-key tiles, every d = 256,
//     and the block-scaled E4M3 variant): the same loop without the
//     pipelined score tile, for a step bound by softmax VALU work or by
//     registers;
//   * attn_fwd_split_kernel (16-bit d = 64, mid-size grids): two wave groups
//     walk the two halves of the key range and merge.
// Those are the defaults (launch_one).  Every kernel built for a (d,
// format) can also be requested explicitly as a tuning variant, including
// the pipelined kernel with a four-stage K/V ring, the three-stage
// pipelined kernel (attn_fwd_pipe3_kernel), the sequential kernel with 32-
// or 128-key tiles, at d = 128 attn_fwd_pingpong_kernel (the pages'
// explicit two-group pingpong) and, at 16-bit d = 128, attn_fwd_wide_kernel
// (64 query rows per wave, one wave per SIMD; attn_fwd_wide.h, its own
// translation unit).  The split-key forward across workgroups is in
// attn_fwd_splitkv.h.
// Masking is folded into the initial values of the score accumulators; the
// key loops run the unmasked steps and the masked ones (ragged end, causal
// diagonal) as two loops of one step variant each, so every step is one
// basic block under one instruction interleave.
//
// FP8 E4M3 ("Inside FlashAttention-3", section 5): Q, K, V are E4M3 codes
// with one descale per tensor.  The q and k descales are folded into the
// score scale and the v descale into the final normalisation; P is rounded
// to E4M3 (round to nearest even) for the P V product while the row sum
// uses the unrounded probabilities; O is binary16.  The block-scaled
// variant (one descale per 64 rows, the same section's block scaling) folds
// each key tile's K and V descales into that tile's exponent (TileScale).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) unsigned char lds_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i16x8 lds_i16x8;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;

struct Params {
  const unsigned char* q;
  const unsigned char* k;
  const unsigned char* v;
  uint16_t* o;
  float* lse;
  int Nq, Nk;
  int n_qtiles;     // ceil(Nq / query rows per workgroup)
  int total_tiles;  // B * H * n_qtiles
  float c;          // |scale| * log2(e): scores -> base-2 exponent units (> 0)
  // Applied to every 32-bit word of Q as it is loaded, (w & q_and) ^ q_xor:
  // the sign bits flipped for a negative scale (so that c stays positive and
  // the -inf mask bias keeps its meaning), all bits cleared for a zero scale
  // (every score is then exactly 0), else unchanged.
  uint32_t q_and, q_xor;
  float o_scale;    // multiplies P V (the v descale for E4M3, else 1)
  // Block-scaled E4M3 only: descales of 64-row blocks, [B*H][nqb] for Q and
  // [B*H][nkb] for K and V (one K/V block per key tile).
  const float* qs;
  const float* ks;
  const float* vs;
  int nqb, nkb;
  // Split-key forward only (attn_fwd_splitkv.h): partial results, splits
  // per query tile at most, key tiles per split at most.
  float* part;
  int nsplit, split_tiles;
#ifdef ATTN_TIMELINE
  // Timeline probe only (attn_timeline.hip): kTimelineSlots counters per wave.
  unsigned long long* timeline;
#endif
};

// Shader-clock trace points of the timeline probe (attn_timeline.hip, a
// library of its own).  In the attention library ATTN_TIMELINE is not
// defined and every member is an empty inline function.  Per wave, lane 0
// writes: slot 0 the clock at kernel entry, 1 after the Q load and the first
// tile loads are issued, 2 + j after step j (steps 0 .. kTimelineSteps - 1),
// and the last four slots the cycles spent waiting at the step barriers, the
// clock after the output is stored, the step count and the hardware id.
constexpr int kTimelineSlots = 64;
constexpr int kTimelineSteps = kTimelineSlots - 6;
struct Timeline {
#ifdef ATTN_TIMELINE
  unsigned long long* slot = nullptr;
  long long wait = 0, mark0 = 0;
  bool lane0 = false;
  __device__ __forceinline__ void init(const Params& p, int waves, int wave) {
    lane0 = (threadIdx.x & 63) == 0;
    slot = p.timeline + ((size_t)blockIdx.x * waves + wave) * kTimelineSlots;
    if (lane0) slot[0] = __builtin_amdgcn_s_memtime();
  }
  __device__ __forceinline__ void mark(int i) {
    if (lane0 && i < kTimelineSlots - 4) slot[i] = __builtin_amdgcn_s_memtime();
  }
  __device__ __forceinline__ void step(int j) {
    if (j < kTimelineSteps) mark(2 + j);
  }
  __device__ __forceinline__ void wait_begin() { mark0 = __builtin_amdgcn_s_memtime(); }
  __device__ __forceinline__ void wait_end() { wait += __builtin_amdgcn_s_memtime() - mark0; }
  __device__ __forceinline__ void finish(int nt) {
    unsigned hw;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    if (lane0) {
      slot[kTimelineSlots - 4] = wait;
      slot[kTimelineSlots - 3] = __builtin_amdgcn_s_memtime();
      slot[kTimelineSlots - 2] = nt;
      slot[kTimelineSlots - 1] = hw;
    }
  }
#else
  __device__ __forceinline__ void init(const Params&, int, int) {}
  __device__ __forceinline__ void mark(int) {}
  __device__ __forceinline__ void step(int) {}
  __device__ __forceinline__ void wait_begin() {}
  __device__ __forceinline__ void wait_end() {}
  __device__ __forceinline__ void finish(int) {}
#endif
};

// Input element formats: size and MFMA.
template <int DT>
struct Fmt;

template <>
struct Fmt<ATTN_F16> {
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ f32x16 mma(i16x8 a, i16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Fmt<ATTN_BF16> {
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ f32x16 mma(i16x8 a, i16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Fmt<ATTN_FP8_E4M3> {
  static constexpr int kBytes = 1;
  // v_mfma_f32_32x32x64_f8f6f4 with both operands E4M3 (format code 0) and
  // no block scales.
  static __device__ __forceinline__ f32x16 mma(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

// Float pairs -> packed 16-bit output / probability elements (RNE):
// binary16 for f16 and E4M3 inputs, bfloat16 for bf16 inputs.
template <int DT>
__device__ __forceinline__ uint32_t pack16(float x, float y) {
  if constexpr (DT == ATTN_BF16)  // v_cvt_pk_bf16_f32
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
  else  // v_cvt_pk_f16_f32
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, f16x2));
}

// Four floats -> four E4M3 bytes, in order (v_cvt_pk_fp8_f32 twice, RNE).
// Inputs here are probabilities in [0, 2^8], inside E4M3's finite range.
// The first conversion writes the low half of the word and the second the
// high half, so the word's previous contents never matter.  The builtin
// takes them as an operand (and the compiler then clears the word with a
// v_mov first); with kAsm the first conversion is written out instead,
// leaving the high half as it finds it until the second one overwrites it.
// The pipelined step keeps the builtin: its instruction interleave counts
// VALU instructions, and an asm statement is not one to the scheduler.
template <bool kAsm = true>
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int lo;
  if constexpr (kAsm) asm("v_cvt_pk_fp8_f32 %0, %1, %2" : "=v"(lo) : "v"(a), "v"(b));
  else lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// XOR swizzle f(row) of the 16-byte chunk index within an LDS row: logical
// chunk c of row r sits at chunk c ^ f(r).  The gfx950 LDS serves 256 bytes
// (64 banks x 4 B) per cycle, i.e. 16 lanes of a 128-bit read or 32 lanes of
// a 64-bit read, and each format's operand reads must fill those 256 bytes
// without two lanes meeting in one bank:
//
// 16-bit elements (row bytes 2d):
//   * K reads (ds_read_b128): 16 consecutive rows, one logical chunk;
//   * V transpose reads (ds_read_b64_tr_b16): 4 consecutive rows (a 4-aligned
//     group) x 4 consecutive chunks (a 4-aligned group).
//   Rows of >= 256 bytes: f(r) = 4*(r&3) + ((r>>2)&3) is a bijection on
//   r mod 16, and inside a 4-row group its values differ in bits [3:2].
//   Rows of 128 bytes (two rows per bank window): f(r) = 4*((r>>1)&1) +
//   ((r>>2)&3) is distinct over the even and over the odd rows of any 16,
//   and rows r, r+2 of a 4-row group differ in bit 2.
//
// E4M3 elements (row bytes d):
//   * K reads (ds_read_b128): as above;
//   * V transpose reads (ds_read_b64_tr_b8): rows {b..b+3, b+8..b+11}
//     (b = 0 or 4 mod 16) x one aligned pair of chunks {2m, 2m+1}.
//   With (r0, r1, r2, r3) the low bits of the row:
//   256-byte rows: f = (r3, r1, r0, r2) as bits [3:0] -- a bijection on
//     r mod 16, and f >> 1 = (r3, r1, r0) is distinct over the 8 rows of a
//     transpose read;
//   128-byte rows (two rows per window, r0 selects the half): f = (r3, r1,
//     r2) as bits [2:0] -- distinct over the rows of one parity, and f >> 1 =
//     (r3, r1) distinct over the 4 rows of one parity in a transpose read;
//   64-byte rows (four rows per window, r1:r0 selects the quarter): f =
//     (r3, r2) as bits [1:0] -- distinct over 4 rows of one residue, and the
//     2 rows of one residue in a transpose read differ in r3.
// Every f uses bits [3:0] of the row only, so f(r + 16k) = f(r).
template <int D, int DT>
__device__ __forceinline__ int swz(int r) {
  if constexpr (Fmt<DT>::kBytes == 2) {
    if constexpr (D >= 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return ((r & 2) << 1) | ((r >> 2) & 3);
  } else {
    const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
    if constexpr (D == 256) return (r3 << 3) | (r1 << 2) | (r0 << 1) | r2;
    else if constexpr (D == 128) return (r3 << 2) | (r1 << 1) | r2;
    else return (r3 << 1) | r2;
  }
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
template <int D, int DT, int NW, int BN = kBlockN>
struct TileLoader {
  static constexpr int kRowBytes = D * Fmt<DT>::kBytes;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kRowsPerKB = 1024 / kRowBytes;
  static constexpr int kBlocks = BN * kRowBytes / 1024;
  static constexpr int kPerWave = kBlocks / NW;
  static_assert(kBlocks % NW == 0, "tile must split evenly over waves");
  int voff[kPerWave];   // byte offset of this lane's chunk within a tile
  int lds[kPerWave];    // LDS byte offset of the wave instruction's 1 KB block

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int b = i * NW + wave;
      const int row = b * kRowsPerKB + lane / kChunks;
      voff[i] = row * kRowBytes + ((lane % kChunks) ^ swz<D, DT>(row)) * 16;
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

// Wait until at most N vector-memory loads of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit counter");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Buffer resource over `bytes` bytes at `base` (raw, stride 0; gfx9 word 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}

// Per-wave state carried across key tiles, 16-bit inputs.
//   MFMA 32x32x16: lane l holds row/column (l & 31) and k elements
//   8*(l >> 5) .. +7 of each operand.
template <int D, int DT>
struct WaveState16 {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kKOff = (D / 16 < 8) ? D / 16 : 8;
  i16x8 qf[D / 16];       // Q rows of this lane as MFMA B-operand fragments
  f32x16 oacc[D / 32];    // O^T accumulator, 32 output columns per block
  float m2;               // reference row max for exp2, in units of scale*log2(e)
  float lrun;             // running row sum over this lane's half of the keys
  int koff[kKOff];        // per-lane LDS byte offsets of K operand reads
  int voff[4][2];         // per-lane LDS byte offsets of V transpose reads

  __device__ __forceinline__ void init(const unsigned char* Qb, int qrow, int Nq, int lane, uint32_t q_and,
                                       uint32_t q_xor) {
    const int half = lane >> 5, r32 = lane & 31;
    // Q rows of this lane: chunk (2s + half) of the row, clamped for rows past Nq.
    const i16x8* src = (const i16x8*)(Qb + (size_t)min(qrow, Nq - 1) * kRowBytes);
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qf[s] = __builtin_bit_cast(i16x8, (__builtin_bit_cast(u32x4, src[2 * s + half]) & q_and) ^ q_xor);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    m2 = -__builtin_inff();
    lrun = 0.f;
    // K operand: row r32 (+32 for the second key block), chunk 2s + half.
    const int xk = swz<D, DT>(r32);
#pragma unroll
    for (int s = 0; s < kKOff; ++s) koff[s] = r32 * kRowBytes + (((2 * s + half) ^ xk) * 16);
    // V transpose reads: 16-lane group G reads rows 4*(G>>1) + t/4 (+8 for
    // the second read) and columns 16*(G&1) + 4*(t&3) of a 32-column block.
    const int G = lane >> 4, t = lane & 15;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = 4 * (G >> 1) + (t >> 2) + 8 * e;
      const int x = swz<D, DT>(row);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int chunk = (4 * db + 2 * (G & 1) + ((t & 3) >> 1)) ^ x;
        voff[db][e] = row * kRowBytes + chunk * 16 + 8 * (t & 1);
      }
    }
  }
};

// Per-wave state, E4M3 inputs.
//   MFMA 32x32x64 f8: lane l holds row/column (l & 31) and the 32
//   consecutive k elements 32*(l >> 5) .. +31 of each operand.
//   Scores: MFMA k-step s covers head-dim bytes 64s .. 64s+63.
//   P V: the 64 keys of a tile are the MFMA's k, in the order of the score
//   accumulator: the lane's 32-byte B operand holds P for keys
//   32s + 8i + 4h + j at byte 16s + 4i + j (h = lane half; i, j < 4), so the
//   A operand (V^T) is read in that key order.
template <int D>
struct WaveState8 {
  static constexpr int kRowBytes = D;
  i32x8 qf[D / 64];       // Q rows of this lane as MFMA B-operand fragments
  f32x16 oacc[D / 32];    // O^T accumulator, 32 output columns per block
  float m2;               // reference row max for exp2, in units of c
  float lrun;             // running row sum over this lane's half of the keys
  int koff[D / 32];       // K operand reads: two 16-byte chunks per k-step
  int voff[D / 32];       // V transpose reads: one offset per 32-column block

  __device__ __forceinline__ void init(const unsigned char* Qb, int qrow, int Nq, int lane, uint32_t q_and,
                                       uint32_t q_xor) {
    const int half = lane >> 5, r32 = lane & 31;
    const i32x4* src = (const i32x4*)(Qb + (size_t)min(qrow, Nq - 1) * kRowBytes);
    const int qa = (int)q_and, qx = (int)q_xor;
#pragma unroll
    for (int s = 0; s < D / 64; ++s) {
      const i32x4 lo = src[4 * s + 2 * half], hi = src[4 * s + 2 * half + 1];
      qf[s] = (__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7) & qa) ^ qx;
    }
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    m2 = -__builtin_inff();
    lrun = 0.f;
    // K operand: row r32 (+32 for the second key block), chunks 4s + 2*half + e.
    const int xk = swz<D, ATTN_FP8_E4M3>(r32);
#pragma unroll
    for (int s = 0; s < D / 64; ++s)
#pragma unroll
      for (int e = 0; e < 2; ++e) koff[2 * s + e] = r32 * kRowBytes + (((4 * s + 2 * half + e) ^ xk) * 16);
    // V transpose reads (ds_read_b64_tr_b8): in a 16-lane group G, result
    // byte t of lane i is byte (i & 7) of the 8 bytes addressed by lane
    // 2t + (i >> 3).  Read e (0..3) must give lane i the keys of bytes
    // 8e..8e+7 of the k order above -- keys 16e + 4h + 8*(t>>2) + (t&3) --
    // for head-dim column 32*db + 16*(G&1) + i.  So lane p addresses row
    // 16e + 4h + 8*(p>>3) + ((p>>1)&3), columns 32*db + 16*(G&1) + 8*(p&1) .. +7;
    // the 16e part is a constant offset of each read.
    const int G = lane >> 4, p = lane & 15;
    const int row = 4 * half + 8 * (p >> 3) + ((p >> 1) & 3);
    const int xv = swz<D, ATTN_FP8_E4M3>(row);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      voff[db] = row * kRowBytes + (((2 * db + (G & 1)) ^ xv) * 16) + 8 * (p & 1);
  }
};

template <int D, int DT>
struct StateOf {
  typedef WaveState16<D, DT> type;
};
template <int D>
struct StateOf<D, ATTN_FP8_E4M3> {
  typedef WaveState8<D> type;
};
template <int D, int DT>
using WaveState = typename StateOf<D, DT>::type;

// S^T = K Q^T for the BN (64 or 32) keys of one tile: one 32x32 accumulator
// per 32 keys (s1 unused for 32-key tiles).  With BIAS the accumulators
// start from their current contents (a 0 / -inf mask bias, see
// needs_bias) instead of zero.
template <int D, int DT, bool BIAS = false, int BN = kBlockN>
__device__ __forceinline__ void tile_scores(const WaveState16<D, DT>& st, const lds_t* Ks, f32x16& s0, f32x16& s1) {
  constexpr int kRowBytes = D * 2;
  constexpr int kKOff = WaveState16<D, DT>::kKOff;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const int o = st.koff[s % kKOff] + (s / kKOff) * 256;
    const i16x8 a0 = *(const lds_i16x8*)(Ks + o);
    s0 = Fmt<DT>::mma(a0, st.qf[s], (s == 0 && !BIAS) ? f32x16{} : s0);
    if constexpr (BN == 64) {
      const i16x8 a1 = *(const lds_i16x8*)(Ks + o + 32 * kRowBytes);
      s1 = Fmt<DT>::mma(a1, st.qf[s], (s == 0 && !BIAS) ? f32x16{} : s1);
    }
  }
}

template <int D, int DT, bool BIAS = false, int BN = kBlockN>
__device__ __forceinline__ void tile_scores(const WaveState8<D>& st, const lds_t* Ks, f32x16& s0, f32x16& s1) {
  static_assert(BN == 64, "E4M3 tiles are 64 keys (the MFMA's k)");
  constexpr int kRowBytes = D;
#pragma unroll
  for (int s = 0; s < D / 64; ++s) {
    const lds_t* k0 = Ks + st.koff[2 * s];
    const lds_t* k1 = Ks + st.koff[2 * s + 1];
    const i32x8 a0 = __builtin_shufflevector(*(const lds_i32x4*)k0, *(const lds_i32x4*)k1, 0, 1, 2, 3, 4, 5, 6, 7);
    const i32x8 a1 = __builtin_shufflevector(*(const lds_i32x4*)(k0 + 32 * kRowBytes),
                                             *(const lds_i32x4*)(k1 + 32 * kRowBytes), 0, 1, 2, 3, 4, 5, 6, 7);
    s0 = Fmt<ATTN_FP8_E4M3>::mma(a0, st.qf[s], (s == 0 && !BIAS) ? f32x16{} : s0);
    s1 = Fmt<ATTN_FP8_E4M3>::mma(a1, st.qf[s], (s == 0 && !BIAS) ? f32x16{} : s1);
  }
}

// O^T += V^T P^T for one tile, V from LDS through transpose reads.  The
// k-step loop is outermost so that consecutive MFMAs accumulate into
// different 32-column blocks of O.
template <int D, int DT, int BN = kBlockN, int NPF>
__device__ __forceinline__ void pv_tile(WaveState16<D, DT>& st, const i16x8 (&pf)[NPF], const lds_t* Vs) {
  static_assert(BN / 16 <= NPF, "one P fragment per 16 keys");
  constexpr int kRowBytes = D * 2;
#pragma unroll
  for (int ks = 0; ks < BN / 16; ++ks) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const lds_t* base = Vs + (db >> 2) * 256 + 16 * ks * kRowBytes;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + st.voff[db & 3][0]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + st.voff[db & 3][1]));
      const i16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      st.oacc[db] = Fmt<DT>::mma(a, pf[ks], st.oacc[db]);
    }
  }
}

template <int D>
__device__ __forceinline__ void pv_tile(WaveState8<D>& st, const i32x8& pf, const lds_t* Vs) {
  constexpr int kRowBytes = D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const lds_t* base = Vs + st.voff[db];
    const i32x2 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(base));
    const i32x2 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(base + 16 * kRowBytes));
    const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(base + 32 * kRowBytes));
    const i32x2 r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(base + 48 * kRowBytes));
    const i32x4 lo = __builtin_shufflevector(r0, r1, 0, 1, 2, 3);
    const i32x4 hi = __builtin_shufflevector(r2, r3, 0, 1, 2, 3);
    const i32x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    st.oacc[db] = Fmt<ATTN_FP8_E4M3>::mma(a, pf, st.oacc[db]);
  }
}

// Rows may hold p = exp2(s*c - m2) up to 2^kLazy before the reference max
// m2 is raised and O, l rescaled: the final O / l and m2 + log2 l do not
// depend on which reference was used, only the rounding does.  (2^8 also
// keeps every E4M3-rounded probability inside that format's range.)
constexpr float kLazy = 8.0f;

// Mask bias of a tile: rem = last visible key of this lane's row minus the
// lane's first key (key0 + 4*half); element r of s0 sits 8*(r>>2) + (r&3)
// keys later, of s1 (64-key tiles) another 32.
template <int BN = kBlockN>
__device__ __forceinline__ void mask_bias(f32x16& s0, f32x16& s1, int rem) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int o = 8 * (r >> 2) + (r & 3);
    s0[r] = o > rem ? -__builtin_inff() : 0.f;
    if constexpr (BN == 64) s1[r] = o + 32 > rem ? -__builtin_inff() : 0.f;
  }
}

// Row max of one tile over this lane's scores (32, or 16 for 32-key tiles;
// two v_max3 chains) and the other half of the row, times c.
template <int BN = kBlockN>
__device__ __forceinline__ float tile_max2(const f32x16& s0, const f32x16& s1, float c) {
  float ma, mb;
  if constexpr (BN == 64) {
    ma = fmaxf(s0[0], s1[0]);
    mb = fmaxf(s0[1], s1[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
      ma = fmaxf(fmaxf(ma, s0[r]), s1[r]);
      mb = fmaxf(fmaxf(mb, s0[r + 1]), s1[r + 1]);
    }
  } else {
    ma = fmaxf(s0[0], s0[1]);
    mb = fmaxf(s0[2], s0[3]);
#pragma unroll
    for (int r = 4; r < 16; r += 4) {
      ma = fmaxf(fmaxf(ma, s0[r]), s0[r + 1]);
      mb = fmaxf(fmaxf(mb, s0[r + 2]), s0[r + 3]);
    }
  }
  return swap_halves_max(fmaxf(ma, mb)) * c;
}

template <int DT>
__device__ __forceinline__ i16x8 pack8(const f32x16& p, int base) {
  return __builtin_bit_cast(i16x8, u32x4{pack16<DT>(p[base + 0], p[base + 1]), pack16<DT>(p[base + 2], p[base + 3]),
                                         pack16<DT>(p[base + 4], p[base + 5]), pack16<DT>(p[base + 6], p[base + 7])});
}

// Row sum (this lane's half) of packed binary16 P, NP 8-element fragments,
// with v_dot2_f32_f16 against (1, 1): half the instructions of fp32 adds.
// It sums P as rounded for the MFMA (relative error below 2^-11 per term, so
// |dLSE| stays below 5e-4 in the worst case), which also makes the
// normalisation consistent with the P V product.  bfloat16's coarser
// rounding could move LSE by up to 2e-3, so bf16 keeps the fp32 sum of the
// unrounded p.
template <int NP, int NPF>
__device__ __forceinline__ float row_sum_f16(const i16x8 (&pf)[NPF]) {
  static_assert(NP <= NPF, "fragments to sum");
  float l[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const u32x4 w = __builtin_bit_cast(u32x4, pf[i]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // Copy the element out first: a bit cast applied directly to a vector
      // element reads element 0.
      const uint32_t we = w[e];
      l[e] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, we), (f16x2){(_Float16)1.0f, (_Float16)1.0f}, l[e],
                                    false);
    }
  }
  return (l[0] + l[1]) + (l[2] + l[3]);
}

// The same sum added straight into acc as one v_dot2 chain: no zeroed
// partial sums to start and no adds to join them (a wave64 VALU
// instruction takes four cycles, so the chain's dependences cost nothing).
template <int NP, int NPF>
__device__ __forceinline__ float row_sum_f16_into(const i16x8 (&pf)[NPF], float acc) {
  static_assert(NP <= NPF, "fragments to sum");
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const u32x4 w = __builtin_bit_cast(u32x4, pf[i]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t we = w[e];
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, we), (f16x2){(_Float16)1.0f, (_Float16)1.0f}, acc, false);
    }
  }
  return acc;
}

// P^T as the E4M3 B operand of the P V MFMA: byte 16s + r holds element r
// of the tile's s-th score accumulator.
template <bool kAsm = true>
__device__ __forceinline__ i32x8 pack_p_fp8(const f32x16& p0, const f32x16& p1) {
  i32x8 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    r[w] = pack_fp8x4<kAsm>(p0[4 * w], p0[4 * w + 1], p0[4 * w + 2], p0[4 * w + 3]);
    r[w + 4] = pack_fp8x4<kAsm>(p1[4 * w], p1[4 * w + 1], p1[4 * w + 2], p1[4 * w + 3]);
  }
  return r;
}

// Scaling of one key tile in the block-scaled E4M3 variant.  A score s of
// codes is worth 2^(c s) in the softmax (c = scale * log2(e) times the Q and
// K block descales), and V's block descale vd multiplies the tile's values.
// Both go into the exponent: p' = 2^(c s + lv - m2) with lv = log2(vd), so
// the E4M3 P' V product accumulates the descaled values, the reference m2
// tracks the maximum of c s + lv, and the row sum takes p' / vd = 2^(c s -
// m2) (iv = 1 / vd).  O / l and m2 + log2 l then come out as with descaled
// inputs.
struct TileScale {
  float c, lv, iv;
};

// Per-wave constants of the key loop over BN-key tiles.
template <int BN>
struct LoopCtxT {
  int qw0, qrow, diag, Nk, half, wave_kend, nt;
  float c;
  // Causal: a tile is visible to the wave iff it starts at or before the
  // wave's last visible key (visibility only decreases along the loop).
  __device__ __forceinline__ bool visible(int t) const { return t < nt && t * BN <= wave_kend; }
  // Tile t needs masking (ragged end, or the causal diagonal crosses it).
  template <bool CAUSAL>
  __device__ __forceinline__ bool needs_mask(int t) const {
    const int key0 = t * BN;
    return (key0 + BN > Nk) || (CAUSAL && key0 + BN - 1 > qw0 + diag);
  }
  template <bool CAUSAL>
  __device__ __forceinline__ int mask_rem(int t) const {
    const int lim = CAUSAL ? min(qrow + diag, Nk - 1) : Nk - 1;
    return lim - t * BN - 4 * half;
  }
};
using LoopCtx = LoopCtxT<kBlockN>;

// Whether tile t's scores need a mask bias: initial accumulators of 0 for
// visible keys, -inf for keys past Nk or above the causal diagonal, and -inf
// everywhere for a tile the wave does not see (its softmax then gives P = 0
// and leaves m, l and O alone), so that the score MFMAs apply the mask
// themselves.  Wave-uniform; false for all but the last tile of a
// non-causal row and the diagonal tiles of a causal one.
template <bool CAUSAL, int BN>
__device__ __forceinline__ bool needs_bias(const LoopCtxT<BN>& cx, int t) {
  return !cx.visible(t) || cx.template needs_mask<CAUSAL>(t);
}

// The first tile for which needs_bias holds (every later tile needs one
// too): min(nt, the ragged last tile Nk / 64, and for causal the first tile
// whose last key lies past the wave's first row's diagonal).  A tile the
// wave cannot see lies past that diagonal as well.
template <bool CAUSAL, int BN>
__device__ __forceinline__ int first_bias_tile(const LoopCtxT<BN>& cx) {
  int t = min(cx.nt, cx.Nk / BN);
  if (CAUSAL) {
    const int x = cx.qw0 + cx.diag - (BN - 2);  // tile t is crossed iff BN t >= x
    t = min(t, x <= 0 ? 0 : (x + BN - 1) / BN);
  }
  return t;
}

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// Scores of tile t (K from Ks) into (s0, s1).  MASKED: the accumulators
// start from the tile's mask bias (see needs_bias); else from zero.
template <int D, int DT, bool CAUSAL, bool MASKED, int BN>
__device__ __forceinline__ void masked_scores(const WaveState<D, DT>& st, const LoopCtxT<BN>& cx, int t,
                                              const lds_t* Ks, f32x16& s0, f32x16& s1) {
  if constexpr (MASKED) {
    mask_bias<BN>(s0, s1, cx.visible(t) ? cx.template mask_rem<CAUSAL>(t) : -(1 << 30));
    tile_scores<D, DT, true, BN>(st, Ks, s0, s1);
  } else {
    tile_scores<D, DT, false, BN>(st, Ks, s0, s1);
  }
}

// Reference update from a tile's row max (in units of scale*log2(e)):
// raise m2 only when some row's max exceeds it by more than kLazy, and
// rescale O and l by 2^(old - new) then.  Only the test runs on every tile;
// the rest sits in a wave-uniform, rarely taken branch.
template <int D, int DT>
__device__ __forceinline__ void lazy_rescale(WaveState<D, DT>& st, float m2t) {
  if (__any(m2t > st.m2 + kLazy)) {
    // The empty asm keeps this block a real branch (see step).
    asm volatile("" ::: "memory");
    const float m2new = fmaxf(st.m2, m2t);
    const float alpha = (m2new == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(st.m2 - m2new);
    st.m2 = m2new;
    st.lrun *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) st.oacc[i] *= alpha;
  }
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

// Instruction interleave of one phase: after `pre` LDS reads, `n` groups of
// one MFMA, `valu` VALU or transcendental instructions (mask 0x402: v_exp_f32
// is not in the plain VALU class) and `reads` LDS reads.  Both phases of a
// step form one scheduling region, so the first V reads of phase B may be
// issued under the last MFMAs of phase A.
#define ATTN_INTERLEAVE(pre, n, valu, reads)                  \
  do {                                                        \
    __builtin_amdgcn_sched_group_barrier(0x100, pre, 0);      \
    _Pragma("unroll") for (int i_ = 0; i_ < (n); ++i_) {      \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      \
      __builtin_amdgcn_sched_group_barrier(0x402, valu, 0);   \
      __builtin_amdgcn_sched_group_barrier(0x100, reads, 0);  \
    }                                                         \
  } while (0)

// One step of the key loop for tile j, as two MFMA blocks with the softmax
// VALU work spread over both:
//   phase A: S_{j+1} = K_{j+1} Q^T (Kn; into n0, n1)  | p_j = exp2(s_j*c - m2),
//                                                         P_j = round(p_j)
//   phase B: O^T += V_j^T P_j^T (Vs)                  | l += sum(p_j),
//                                                         row max of S_{j+1},
//                                                         reference update
// then, rarely, O and l are rescaled to the new reference.  s0, s1 hold S_j
// on entry (and p_j after phase A).  The mask choice is a template
// parameter, taken by a wave-uniform branch around the whole step, so each
// phase is one basic block and its interleave holds.
template <int D, int DT, bool CAUSAL, bool MASKED>
__device__ __forceinline__ void step(WaveState<D, DT>& st, const LoopCtx& cx, int j, f32x16& s0, f32x16& s1,
                                     f32x16& n0, f32x16& n1, const lds_t* Kn, const lds_t* Vs) {
  // Phase A
  masked_scores<D, DT, CAUSAL, MASKED>(st, cx, j + 1, Kn, n0, n1);
  const float mref = (st.m2 == -__builtin_inff()) ? 0.f : st.m2;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], cx.c, -mref));
    s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], cx.c, -mref));
  }
  if constexpr (DT == ATTN_FP8_E4M3) {
    // D/32 MFMAs of 64 cycles per phase; two 16-byte K reads per MFMA.
    const i32x8 pf = pack_p_fp8<false>(s0, s1);
    if constexpr (D == 64) ATTN_INTERLEAVE(2, 2, 40, 2);
    else if constexpr (D == 128) ATTN_INTERLEAVE(2, 4, 20, 2);
    else ATTN_INTERLEAVE(2, 8, 10, 2);
    // Phase B
    pv_tile<D>(st, pf, Vs);
  } else {
    i16x8 pf[4];
    pf[0] = pack8<DT>(s0, 0);
    pf[1] = pack8<DT>(s0, 8);
    pf[2] = pack8<DT>(s1, 0);
    pf[3] = pack8<DT>(s1, 8);
    // D/8 MFMAs of 32 cycles per phase, one K read each; the 80 VALU
    // instructions of phase A (32 FMA, 32 exp2, 16 packs) spread evenly.
    constexpr int kValuA = (80 + D / 8 - 1) / (D / 8);
    ATTN_INTERLEAVE(3, D / 8, kValuA, 1);
    // Phase B
    pv_tile<D, DT>(st, pf, Vs);
    if constexpr (DT == ATTN_F16) st.lrun += row_sum_f16<4>(pf);
  }
  if constexpr (DT != ATTN_F16) {
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      ls0 += s0[r];
      ls1 += s1[r];
    }
    st.lrun += ls0 + ls1;
  }
  bool rescale;
  const float alpha = update_reference(st.m2, tile_max2(n0, n1, cx.c), rescale);
  if constexpr (DT == ATTN_FP8_E4M3) {
    // D/32 MFMAs, four 8-byte transpose reads each.
    if constexpr (D == 64) ATTN_INTERLEAVE(4, 2, 30, 4);
    else if constexpr (D == 128) ATTN_INTERLEAVE(4, 4, 15, 4);
    else ATTN_INTERLEAVE(4, 8, 8, 4);
  } else {
    // About 64 VALU instructions (32 adds, 16 max3, the reference update).
    constexpr int kValuB = ((DT == ATTN_F16 ? 48 : 64) + D / 8 - 1) / (D / 8);
    ATTN_INTERLEAVE(4, D / 8, kValuB, 2);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (rescale) {
    // The empty asm keeps this block a real (wave-uniform, rarely taken)
    // branch: without it the compiler speculates the multiplies, since on
    // 16-wide vectors they look cheap, and would scale O by alpha = 1 on
    // every tile.
    asm volatile("" ::: "memory");
    st.lrun *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) st.oacc[i] *= alpha;
  }
}

// Output: O = o_scale * O^T / l (rounded to the output type),
// LSE = ln2 * (m2 + log2 l).
template <int D, int DT>
__device__ __forceinline__ void store_output(const Params& p, const WaveState<D, DT>& st, int bh, int qrow,
                                             int half) {
  const float ltot = swap_halves_sum(st.lrun);
  const bool has_key = ltot > 0.f;
  const float inv = has_key ? p.o_scale / ltot : 0.f;
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
        w[0] = pack16<DT>(st.oacc[db][4 * g] * inv, st.oacc[db][4 * g + 1] * inv);
        w[1] = pack16<DT>(st.oacc[db][4 * g + 2] * inv, st.oacc[db][4 * g + 3] * inv);
        *(u32x2*)(orow + d0) = w;
      }
    }
  }
}

// Keys per tile of the sequential kernel: 32 for 16-bit d = 256, where O
// (128 registers) and Q (64) leave room for one 32x32 score accumulator
// within the 256 registers of a wave that shares its SIMD with another;
// 64 elsewhere (E4M3 tiles are the 64-key k of its MFMA).
template <int D, int DT>
struct TileKeys {
  static constexpr int value = (D == 256 && DT != ATTN_FP8_E4M3) ? 32 : 64;
};

// Waves per workgroup (32 query rows each).  At d = 128 and 256 one 8-wave
// workgroup per CU (two waves per SIMD, 256 query rows) shares each K/V
// tile among twice the rows of two 4-wave workgroups, halving the
// global-to-LDS loads per FLOP: measured +0.9% at d = 128 and +1.5% at
// d = 256 (causal bf16).  At d = 64, 4 waves measured faster.
template <int D, int DT>
struct Waves {
  static constexpr int value = (D == 128 || D == 256) ? 8 : 4;
};

// NS: stages of the K ring and of the V ring, 2 (the default) or 4.  With
// four, the workgroup synchronises once per two key tiles instead of once
// per tile and loads run a whole step pair ahead, for twice the LDS; on
// 16-bit d = 128 that measured 1.5% slower, so it is a tuning variant.
template <int D, int DT, bool CAUSAL, int NS = 2>
__global__ void __launch_bounds__(64 * (Waves<D, DT>::value)) attn_fwd_kernel(Params p) {
  static_assert(NS == 2 || NS == 4, "two or four ring stages");
  constexpr int kWaves = Waves<D, DT>::value;
  constexpr int kBlockM = kWaves * kRowsPerWave;  // query rows per workgroup
  constexpr int kRowBytes = D * Fmt<DT>::kBytes;
  constexpr int kTileBytes = kBlockN * kRowBytes;
  constexpr int kExtraBytes = NS == 4 ? kTileBytes : 16;
  // K and V rings of NS stages each, as separate LDS objects.  K runs one
  // tile ahead of V: step j reads K_{j+1} (scores of the next tile) and V_j.
  // With every stage a distinct object and the loop unrolled over a whole
  // turn of the ring, each LDS read names its stage statically, so the
  // compiler can prove it never aliases the in-flight direct-to-LDS loads
  // into another stage and does not wait on them.
  __shared__ __attribute__((aligned(1024))) unsigned char k_st0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k_st1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_st0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_st1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k_st2[kExtraBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k_st3[kExtraBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_st2[kExtraBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_st3[kExtraBytes];
  lds_t* const K0 = (lds_t*)k_st0;
  lds_t* const K1 = (lds_t*)k_st1;
  lds_t* const V0 = (lds_t*)v_st0;
  lds_t* const V1 = (lds_t*)v_st1;
  lds_t* const K2 = (lds_t*)k_st2;
  lds_t* const K3 = (lds_t*)k_st3;
  lds_t* const V2 = (lds_t*)v_st2;
  lds_t* const V3 = (lds_t*)v_st3;

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
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc(p.k + (size_t)bh * p.Nk * kRowBytes, head_bytes);
  const __amdgpu_buffer_rsrc_t Vr = make_rsrc(p.v + (size_t)bh * p.Nk * kRowBytes, head_bytes);

  // K/V tile loads: in the 8-wave 16-bit form (d = 128) waves 0-3 issue
  // them all, the four that get their SIMD's matrix core first and then
  // wait at the step barrier (see the sequential kernel): bfloat16 2.0%
  // faster (causal 2.2%), binary16 1%, the four-stage ring 3%; waves 4-7
  // measured no change.  Elsewhere every wave issues its share.
  constexpr bool kHalfLoad = kWaves == 8 && DT != ATTN_FP8_E4M3;
  constexpr int kLoadWaves = kHalfLoad ? 4 : kWaves;
  const bool loader = !kHalfLoad || wave < kLoadWaves;
  TileLoader<D, DT, kLoadWaves> ldr;
  ldr.init(loader ? wave : 0, lane);
  auto load = [&](lds_t* dst, __amdgpu_buffer_rsrc_t src, int key0) {
    if (loader) ldr.load(dst, src, key0);
  };
  WaveState<D, DT> st;
  st.init(p.q + (size_t)bh * p.Nq * kRowBytes, cx.qrow, p.Nq, lane, p.q_and, p.q_xor);

  // Scores (then probabilities) of even tiles live in (a0, a1), of odd
  // tiles in (b0, b1).
  f32x16 a0, a1, b0, b1;
  const int tb = first_bias_tile<CAUSAL>(cx);
  if constexpr (NS == 4) {
    // Tile t sits in stage t % 4 of each ring.  Steps run in pairs (j, j+1),
    // j even, behind one barrier: the pair reads K_{j+1}, K_{j+2}, V_j,
    // V_{j+1}, while K_{j+3}, K_{j+4}, V_{j+2}, V_{j+3} stream into the
    // stages the previous pair read.  Every K stage a step reads holds
    // finite data: the stages start with tiles 0..2 (and tile 3 when the
    // loop does not load it), rows past the end arriving as zeros through
    // the range check; later a stage past the last tile keeps an earlier
    // tile.  Scores of tiles past the end are masked to -inf.
    if (nt > 0) {
      load(K0, Kr, 0);
      load(V0, Vr, 0);
      load(K1, Kr, kBlockN);
      load(V1, Vr, kBlockN);
      load(K2, Kr, 2 * kBlockN);
      if (nt <= 3) load(K3, Kr, 3 * kBlockN);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tb > 0) masked_scores<D, DT, CAUSAL, false>(st, cx, 0, K0, a0, a1);
      else masked_scores<D, DT, CAUSAL, true>(st, cx, 0, K0, a0, a1);
      bool rescale;
      update_reference(st.m2, tile_max2(a0, a1, cx.c), rescale);
    }
    // Four steps from j (j % 4 == 0); returns false after the last step.
    auto four_steps = [&](int j, auto masked) -> bool {
      constexpr bool M = decltype(masked)::value;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (j + 3 < nt) load(K3, Kr, (j + 3) * kBlockN);
      if (j + 4 < nt) load(K0, Kr, (j + 4) * kBlockN);
      if (j + 2 < nt) load(V2, Vr, (j + 2) * kBlockN);
      if (j + 3 < nt) load(V3, Vr, (j + 3) * kBlockN);
      step<D, DT, CAUSAL, M>(st, cx, j, a0, a1, b0, b1, K1, V0);
      if (j + 1 >= nt) return false;
      step<D, DT, CAUSAL, M>(st, cx, j + 1, b0, b1, a0, a1, K2, V1);
      if (j + 2 >= nt) return false;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (j + 5 < nt) load(K1, Kr, (j + 5) * kBlockN);
      if (j + 6 < nt) load(K2, Kr, (j + 6) * kBlockN);
      if (j + 4 < nt) load(V0, Vr, (j + 4) * kBlockN);
      if (j + 5 < nt) load(V1, Vr, (j + 5) * kBlockN);
      step<D, DT, CAUSAL, M>(st, cx, j + 2, a0, a1, b0, b1, K3, V2);
      if (j + 3 >= nt) return false;
      step<D, DT, CAUSAL, M>(st, cx, j + 3, b0, b1, a0, a1, K0, V3);
      return j + 4 < nt;
    };
    // Steps j < jm (a multiple of 4) need no mask bias for the tile they
    // score (j + 1 < tb); the rest run the masked variant.
    const int jm = tb > 1 ? (tb - 1) & ~3 : 0;
    int j = 0;
    for (; j < jm; j += 4) four_steps(j, BoolTag<false>{});
    for (; j < nt; j += 4)
      if (!four_steps(j, BoolTag<true>{})) break;
    store_output<D, DT>(p, st, bh, cx.qrow, cx.half);
    return;
  }
  // Two stages.  Tiles before tb need no mask bias; step j works on the
  // scores of tile j + 1, so steps j < jm (jm even, so the second loop again
  // starts with S_j in (a0, a1)) run the unmasked step and the rest the
  // masked one.  Two loops with one step variant each keep the register
  // assignment of the unrolled pair identical on every iteration.
  const int jm = tb > 1 ? (tb - 1) & ~1 : 0;
  if (nt > 0) {
    // K_1 is loaded even when there is no tile 1: its rows then fail the
    // range check and arrive as zeros, so every K stage a step reads holds
    // finite data (scores of tiles past the end are -inf, never NaN).
    load(K0, Kr, 0);
    load(V0, Vr, 0);
    load(K1, Kr, kBlockN);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tb > 0) masked_scores<D, DT, CAUSAL, false>(st, cx, 0, K0, a0, a1);
    else masked_scores<D, DT, CAUSAL, true>(st, cx, 0, K0, a0, a1);
    bool rescale;
    update_reference(st.m2, tile_max2(a0, a1, cx.c), rescale);
  }
  // One even and one odd step; returns false after the last step.
  auto two_steps = [&](int j, auto masked) -> bool {
    constexpr bool M = decltype(masked)::value;
    // Even step: (a0, a1) = S_j; K_{j+1} in K1, V_j in V0; K_{j+2} -> K0, V_{j+1} -> V1.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 2 < nt) load(K0, Kr, (j + 2) * kBlockN);
    if (j + 1 < nt) load(V1, Vr, (j + 1) * kBlockN);
    step<D, DT, CAUSAL, M>(st, cx, j, a0, a1, b0, b1, K1, V0);
    if (j + 1 >= nt) return false;
    // Odd step: (b0, b1) = S_{j+1}; K_{j+2} in K0, V_{j+1} in V1; K_{j+3} -> K1, V_{j+2} -> V0.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 3 < nt) load(K1, Kr, (j + 3) * kBlockN);
    if (j + 2 < nt) load(V0, Vr, (j + 2) * kBlockN);
    step<D, DT, CAUSAL, M>(st, cx, j + 1, b0, b1, a0, a1, K0, V1);
    return true;
  };
  int j = 0;
  for (; j < jm; j += 2) two_steps(j, BoolTag<false>{});
  for (; j < nt; j += 2)
    if (!two_steps(j, BoolTag<true>{})) break;
  store_output<D, DT>(p, st, bh, cx.qrow, cx.half);
}

// ---------------------------------------------------------------------------
// Three-stage pipelined kernel (16-bit, d = 64 and 128; a tuning variant):
// the score MFMAs run two key tiles ahead of the P V MFMAs, so step j
// overlaps the matrix work of S_{j+2} and of O += P_j V_j with the softmax
// of tile j + 1 -- the three-stage form of the concept card's "Overlap of
// matrix multiplies and softmax inside one warpgroup".  It holds one more
// score tile and one more packed P than the two-stage kernel.
//
// References: P_{j+1} is formed against the reference m2 of its step, and a
// raise decided from the row max of S_{j+2} reaches l at once (its next
// term is P_{j+2}) but O only one step later, after P_{j+1} V_{j+1} has been
// added against the old reference (the pending factor alpha_o).
// K runs two tiles ahead of V: step j reads K_{j+2} and V_j from stage j % 2
// of each ring while K_{j+3} and V_{j+1} stream into the other stage.
// ---------------------------------------------------------------------------
template <int D, int DT, bool CAUSAL, bool MASKED>
__device__ __forceinline__ void step3(WaveState16<D, DT>& st, const LoopCtx& cx, int j, const i16x8 (&pj)[4],
                                      i16x8 (&pn)[4], f32x16& s0, f32x16& s1, f32x16& n0, f32x16& n1, float& alpha_o,
                                      bool& pend, const lds_t* Kn, const lds_t* Vs) {
  // Phase A: S_{j+2} = K_{j+2} Q^T | P_{j+1} = exp2(c S_{j+1} - m2), packed
  masked_scores<D, DT, CAUSAL, MASKED>(st, cx, j + 2, Kn, n0, n1);
  const float mref = (st.m2 == -__builtin_inff()) ? 0.f : st.m2;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], cx.c, -mref));
    s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], cx.c, -mref));
  }
  pn[0] = pack8<DT>(s0, 0);
  pn[1] = pack8<DT>(s0, 8);
  pn[2] = pack8<DT>(s1, 0);
  pn[3] = pack8<DT>(s1, 8);
  constexpr int kValuA = (80 + D / 8 - 1) / (D / 8);
  ATTN_INTERLEAVE(3, D / 8, kValuA, 1);
  // Phase B: O += P_j V_j | l += rowsum(P_{j+1}), row max of S_{j+2} and the
  // reference update
  pv_tile<D, DT>(st, pj, Vs);
  if constexpr (DT == ATTN_F16) {
    st.lrun += row_sum_f16<4>(pn);
  } else {
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      ls0 += s0[r];
      ls1 += s1[r];
    }
    st.lrun += ls0 + ls1;
  }
  bool rescale;
  const float alpha = update_reference(st.m2, tile_max2(n0, n1, cx.c), rescale);
  constexpr int kValuB = ((DT == ATTN_F16 ? 48 : 64) + D / 8 - 1) / (D / 8);
  ATTN_INTERLEAVE(4, D / 8, kValuB, 2);
  __builtin_amdgcn_sched_barrier(0);
  if (pend || rescale) {
    asm volatile("" ::: "memory");  // keep the branch (see step)
    st.lrun *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) st.oacc[i] *= alpha_o;
  }
  alpha_o = alpha;
  pend = rescale;
}

template <int D, int DT, bool CAUSAL>
__global__ void __launch_bounds__(64 * (Waves<D, DT>::value)) attn_fwd_pipe3_kernel(Params p) {
  static_assert(DT != ATTN_FP8_E4M3 && D != 256, "three-stage kernel: 16-bit, d = 64 or 128");
  constexpr int kWaves = Waves<D, DT>::value;
  constexpr int kBlockM = kWaves * kRowsPerWave;
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kBlockN * kRowBytes;
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
  cx.diag = p.Nk - p.Nq;
  cx.Nk = p.Nk;
  cx.half = lane >> 5;
  cx.c = p.c;
  cx.wave_kend = CAUSAL ? cx.qw0 + kRowsPerWave - 1 + cx.diag : p.Nk;
  int kend = p.Nk;
  if (CAUSAL) kend = min(p.Nk, q0 + kBlockM + cx.diag);
  const int nt = kend > 0 ? (kend + kBlockN - 1) / kBlockN : 0;
  cx.nt = nt;

  const uint32_t head_bytes = (uint32_t)p.Nk * kRowBytes;
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc(p.k + (size_t)bh * p.Nk * kRowBytes, head_bytes);
  const __amdgpu_buffer_rsrc_t Vr = make_rsrc(p.v + (size_t)bh * p.Nk * kRowBytes, head_bytes);
  TileLoader<D, DT, kWaves> ld;
  ld.init(wave, lane);
  WaveState16<D, DT> st;
  st.init(p.q + (size_t)bh * p.Nq * kRowBytes, cx.qrow, p.Nq, lane, p.q_and, p.q_xor);

  if (nt > 0) {
    const int tb = first_bias_tile<CAUSAL>(cx);
    // Prologue: S_0 and its reference; S_1, P_0 and the reference after
    // S_1.  K_1 is loaded even past the end (rows past Nk arrive as zeros),
    // so every K stage a step reads holds finite data: scores of tiles past
    // the end are -inf through the mask bias.
    ld.load(K0, Kr, 0);
    ld.load(V0, Vr, 0);
    ld.load(K1, Kr, kBlockN);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    f32x16 a0, a1, b0, b1;
    i16x8 pa[4], pb[4];
    bool rescale;
    if (tb > 0) masked_scores<D, DT, CAUSAL, false>(st, cx, 0, K0, a0, a1);
    else masked_scores<D, DT, CAUSAL, true>(st, cx, 0, K0, a0, a1);
    update_reference(st.m2, tile_max2(a0, a1, cx.c), rescale);
    if (tb > 1) masked_scores<D, DT, CAUSAL, false>(st, cx, 1, K1, b0, b1);
    else masked_scores<D, DT, CAUSAL, true>(st, cx, 1, K1, b0, b1);
    {
      const float mref = (st.m2 == -__builtin_inff()) ? 0.f : st.m2;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        a0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(a0[r], cx.c, -mref));
        a1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(a1[r], cx.c, -mref));
      }
      pa[0] = pack8<DT>(a0, 0);
      pa[1] = pack8<DT>(a0, 8);
      pa[2] = pack8<DT>(a1, 0);
      pa[3] = pack8<DT>(a1, 8);
      if constexpr (DT == ATTN_F16) {
        st.lrun += row_sum_f16<4>(pa);
      } else {
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) ls += a0[r] + a1[r];
        st.lrun += ls;
      }
    }
    // l (the sum of P_0) moves to the new reference at once; O receives
    // P_0 V_0, formed against the old one, in step 0 and moves after it
    float alpha_o = update_reference(st.m2, tile_max2(b0, b1, cx.c), rescale);
    st.lrun *= alpha_o;
    bool pend = rescale;
    __syncthreads();  // every wave is done with K_0's stage
    if (2 < nt) ld.load(K0, Kr, 2 * kBlockN);
    // Step j: P_j in (pa | pb), S_{j+1} in (b | a); steps j < jm score an
    // unmasked tile j + 2.
    auto two_steps = [&](int j, auto masked) -> bool {
      constexpr bool M = decltype(masked)::value;
      // even step: K_{j+2} in K0, V_j in V0; K_{j+3} -> K1, V_{j+1} -> V1
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (j + 3 < nt) ld.load(K1, Kr, (j + 3) * kBlockN);
      if (j + 1 < nt) ld.load(V1, Vr, (j + 1) * kBlockN);
      step3<D, DT, CAUSAL, M>(st, cx, j, pa, pb, b0, b1, a0, a1, alpha_o, pend, K0, V0);
      if (j + 1 >= nt) return false;
      // odd step: K_{j+3} in K1, V_{j+1} in V1; K_{j+4} -> K0, V_{j+2} -> V0
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (j + 4 < nt) ld.load(K0, Kr, (j + 4) * kBlockN);
      if (j + 2 < nt) ld.load(V0, Vr, (j + 2) * kBlockN);
      step3<D, DT, CAUSAL, M>(st, cx, j + 1, pb, pa, a0, a1, b0, b1, alpha_o, pend, K1, V1);
      return true;
    };
    const int jm = tb > 2 ? (tb - 2) & ~1 : 0;
    int j = 0;
    for (; j < jm; j += 2) two_steps(j, BoolTag<false>{});
    for (; j < nt; j += 2)
      if (!two_steps(j, BoolTag<true>{})) break;
    if (pend) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) st.oacc[i] *= alpha_o;
    }
  }
  store_output<D, DT>(p, st, bh, cx.qrow, cx.half);
}

// ---------------------------------------------------------------------------
// Pingpong kernel (d = 128, every format): the pages' two-consumer schedule
// (concept card, "Pingpong scheduling between two consumer warpgroups";
// "Inside FlashAttention-3", section 3).  The workgroup's 8 waves form two
// groups, A = waves 0-3 and B = waves 4-7, so every SIMD holds one wave of
// each.  Every wave alternates
//   * an MFMA half: O += P_j V_j and S_{j+1} = K_{j+1} Q^T, with nothing but
//     their LDS operand reads beside them, at s_setprio 1, and
//   * a softmax half: S_{j+1} -> P_{j+1} (row max and reference update, exp2,
//     rounding, row sum), with no matrix work;
// group B runs one half behind group A and every half ends at a workgroup
// barrier, so on each SIMD one wave's matrix work overlaps the other wave's
// softmax.  The softmax half consumes the score tile before the next MFMA
// half overwrites it, so a wave holds one score tile (fewer registers than
// the pipelined kernel's two).
//
// Ring: K and V in NS stages each (two built; three measured no faster).
// K_{j+NS} and V_{j+NS-1} are loaded at the start of A's MFMA half j (= B's
// softmax half j) into the stages both groups finished reading one half
// earlier; A waits for its share at the end of its softmax half before the
// MFMA half that reads them, B at the end of its MFMA half before that.
// ---------------------------------------------------------------------------
// P of one tile as the P V MFMA's B operand: four 16-key fragments at 16
// bits, one 64-key fragment for E4M3.
template <int DT>
struct PTile {
  i16x8 f[4];
};
template <>
struct PTile<ATTN_FP8_E4M3> {
  i32x8 f;
};

template <int D, int DT, bool CAUSAL, bool MASKED, bool PV>
__device__ __forceinline__ void pp_mfma_half(WaveState<D, DT>& st, const LoopCtx& cx, int j, const PTile<DT>& pt,
                                             f32x16& s0, f32x16& s1, const lds_t* Kn, const lds_t* Vc) {
  __builtin_amdgcn_s_setprio(1);
  masked_scores<D, DT, CAUSAL, MASKED>(st, cx, j + 1, Kn, s0, s1);
  if constexpr (DT == ATTN_FP8_E4M3) {
    if constexpr (PV) pv_tile<D>(st, pt.f, Vc);
    // scores: two 16-byte K reads per 64-cycle MFMA, one MFMA's worth
    // ahead; P V: the four transpose reads of the next MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 2 * D / 64; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    if constexpr (PV) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
    }
  } else {
    if constexpr (PV) pv_tile<D, DT>(st, pt.f, Vc);
    // scores: 3 K reads ahead, one per MFMA; P V: 4 V reads ahead, two per MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int i = 0; i < 2 * D / 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (PV) {
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
}

template <int D, int DT>
__device__ __forceinline__ void pp_softmax_half(WaveState<D, DT>& st, const LoopCtx& cx, f32x16& s0, f32x16& s1,
                                                PTile<DT>& pt) {
  bool rescale;
  const float alpha = update_reference(st.m2, tile_max2(s0, s1, cx.c), rescale);
  if (rescale) {
    asm volatile("" ::: "memory");  // keep the branch (see step)
    st.lrun *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) st.oacc[i] *= alpha;
  }
  const float mref = (st.m2 == -__builtin_inff()) ? 0.f : st.m2;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], cx.c, -mref));
    s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], cx.c, -mref));
  }
  if constexpr (DT == ATTN_FP8_E4M3) {
    pt.f = pack_p_fp8(s0, s1);
  } else {
    pt.f[0] = pack8<DT>(s0, 0);
    pt.f[1] = pack8<DT>(s0, 8);
    pt.f[2] = pack8<DT>(s1, 0);
    pt.f[3] = pack8<DT>(s1, 8);
  }
  if constexpr (DT == ATTN_F16) {
    st.lrun += row_sum_f16<4>(pt.f);
  } else {
    // bfloat16 and E4M3: the unrounded p
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      ls0 += s0[r];
      ls1 += s1[r];
    }
    st.lrun += ls0 + ls1;
  }
}

template <int D, int DT, bool CAUSAL, int NS = 2>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) attn_fwd_pingpong_kernel(Params p) {
  static_assert(D == 128, "pingpong kernel: d = 128");
  static_assert(NS == 2 || NS == 3, "two or three ring stages");
  constexpr int kWaves = 8;
  constexpr int kBlockM = kWaves * kRowsPerWave;
  constexpr int kRowBytes = D * Fmt<DT>::kBytes;
  constexpr int kTileBytes = kBlockN * kRowBytes;
  __shared__ __attribute__((aligned(1024))) unsigned char k_st[NS][kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_st[NS][kTileBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;  // 0: group A, 1: group B (one half behind)

  int bh, qt;
  schedule(p, blockIdx.x, CAUSAL, bh, qt);
  const int q0 = qt * kBlockM;
  LoopCtx cx;
  cx.qw0 = q0 + wave * kRowsPerWave;
  cx.qrow = cx.qw0 + (lane & 31);
  cx.diag = p.Nk - p.Nq;
  cx.Nk = p.Nk;
  cx.half = lane >> 5;
  cx.c = p.c;
  cx.wave_kend = CAUSAL ? cx.qw0 + kRowsPerWave - 1 + cx.diag : p.Nk;
  int kend = p.Nk;
  if (CAUSAL) kend = min(p.Nk, q0 + kBlockM + cx.diag);
  const int nt = kend > 0 ? (kend + kBlockN - 1) / kBlockN : 0;
  cx.nt = nt;

  const uint32_t head_bytes = (uint32_t)p.Nk * kRowBytes;
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc(p.k + (size_t)bh * p.Nk * kRowBytes, head_bytes);
  const __amdgpu_buffer_rsrc_t Vr = make_rsrc(p.v + (size_t)bh * p.Nk * kRowBytes, head_bytes);
  using Loader = TileLoader<D, DT, kWaves>;
  constexpr int kLoads = 2 * Loader::kPerWave;  // a wave's loads per batch (its share of one K and one V tile)
  Loader ld;
  ld.init(wave, lane);
  WaveState<D, DT> st;
  st.init(p.q + (size_t)bh * p.Nq * kRowBytes, cx.qrow, p.Nq, lane, p.q_and, p.q_xor);

  if (nt > 0) {
    // K_0 .. K_{NS-1} and V_0 .. V_{NS-2}, also past the last tile (zeros),
    // so that every K stage an MFMA half reads holds finite data.
#pragma unroll
    for (int s = 0; s < NS; ++s) ld.load((lds_t*)k_st[s], Kr, s * kBlockN);
#pragma unroll
    for (int s = 0; s + 1 < NS; ++s) ld.load((lds_t*)v_st[s], Vr, s * kBlockN);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    f32x16 s0, s1;
    PTile<DT> pf;
    const int tb = first_bias_tile<CAUSAL>(cx);
    if (grp == 1) __syncthreads();
    // MFMA half -1: S_0 only
    if (tb > 0) pp_mfma_half<D, DT, CAUSAL, false, false>(st, cx, -1, pf, s0, s1, (const lds_t*)k_st[0], nullptr);
    else pp_mfma_half<D, DT, CAUSAL, true, false>(st, cx, -1, pf, s0, s1, (const lds_t*)k_st[0], nullptr);
    __syncthreads();
    // Batch t (issued by group A at the start of its MFMA half t and by
    // group B at the start of its softmax half t, the same half of the
    // schedule): K_{t+NS} into the stage K_t left (scored in MFMA half
    // t - 1) and V_{t+NS-1} into the stage V_{t-1} left.  The data of MFMA
    // half t (K_{t+1}, V_t) come from batch t + 1 - NS; when it must have
    // landed, each wave has issued NS - 2 batches since, all full unless
    // the tiles ran out (then it waits for everything).
    auto issue = [&](int t, lds_t* Kd, lds_t* Vd) {
      if (t + NS < nt) ld.load(Kd, Kr, (t + NS) * kBlockN);
      if (t + NS - 1 < nt) ld.load(Vd, Vr, (t + NS - 1) * kBlockN);
    };
    auto wait_batches = [&](bool full) {
      if constexpr (NS == 3) {
        if (full) {
          wait_vmcnt<kLoads>();
          return;
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    // Softmax half t, then MFMA half t: P_t V_t (V stage t % NS) and
    // S_{t+1} (K stage (t + 1) % NS); R = t % NS.  Returns false after the
    // last MFMA half.
    auto pair = [&](int t, auto r, auto masked) -> bool {
      constexpr int R = decltype(r)::value;
      constexpr bool M = decltype(masked)::value;
      lds_t* const Kd = (lds_t*)k_st[R];
      lds_t* const Vd = (lds_t*)v_st[(R + NS - 1) % NS];
      if (grp == 1) issue(t, Kd, Vd);
      pp_softmax_half<D, DT>(st, cx, s0, s1, pf);
      if (grp == 0) wait_batches(t + NS - 1 < nt);
      __syncthreads();
      if (grp == 0) issue(t, Kd, Vd);
      pp_mfma_half<D, DT, CAUSAL, M, true>(st, cx, t, pf, s0, s1, (const lds_t*)k_st[(R + 1) % NS],
                                           (const lds_t*)v_st[R]);
      if (grp == 1) wait_batches(t + NS < nt);
      __syncthreads();
      return t + 1 < nt;
    };
    // The MFMA halves of tiles t .. t + NS - 1 score tiles t + 1 .. t + NS:
    // unmasked while all lie before the first tile that needs a mask bias.
    auto round = [&](int t, auto masked) -> bool {
      if (!pair(t, std::integral_constant<int, 0>{}, masked)) return false;
      if (!pair(t + 1, std::integral_constant<int, 1>{}, masked)) return false;
      if constexpr (NS == 3) {
        if (!pair(t + 2, std::integral_constant<int, 2>{}, masked)) return false;
      }
      return true;
    };
    int t = 0;
    for (; t + NS < tb; t += NS) round(t, BoolTag<false>{});
    for (; t < nt; t += NS)
      if (!round(t, BoolTag<true>{})) break;
    if (grp == 0) __syncthreads();
  }
  store_output<D, DT>(p, st, bh, cx.qrow, cx.half);
}

// ---------------------------------------------------------------------------
// Sequential-step kernel: the same tile loop without software pipelining of
// the scores.  Each step computes S_j, its softmax and O += P_j V_j in
// order; the overlap of matrix work and softmax comes from the other wave
// of the SIMD instead of from within the wave.  Used where the softmax VALU
// work bounds the step (E4M3 at d = 128, where one 64-cycle MFMA carries the
// softmax of 32 scores per lane) and where the pipelined kernel's registers
// would leave one wave per SIMD (d = 256).  K_j and V_j share a ring stage;
// the loads of tile j + 1 are issued at the start of step j.
// ---------------------------------------------------------------------------
// Largest half-row sum of probabilities a tile may reach against the current
// reference before the reference is raised: 2^kLazy, so every p <= 2^kLazy.
constexpr float kLazySum = 256.0f;

// SUMCHECK (the default for 16-bit inputs below d = 256): the reference is
// checked through the half-row sums, below.  Without it every tile's row
// max is taken first, as in step().  Measured against that form on the
// sequential kernel: binary16 d = 128 +3.8%, bfloat16 d = 64 causal +5%, but
// E4M3 d = 128 -19% (its row sum is 32 fp32 adds, which the check moves
// from under the P V product to before it).  The producer-wave kernel and
// d = 256 keep the max-first form too: holding the packed probabilities
// through the check does not fit their registers (168 with a producer wave
// beside two consumers per SIMD; 256 beside O and Q at d = 256).
template <int D, int DT, bool CAUSAL, bool MASKED, int BN, bool BS,
          bool SUMCHECK = (D != 256 && DT != ATTN_FP8_E4M3)>
__device__ __forceinline__ void seq_step(WaveState<D, DT>& st, const LoopCtxT<BN>& cx, int j, const lds_t* Kc,
                                         const lds_t* Vc, const TileScale& ts) {
  f32x16 s0, s1;
  masked_scores<D, DT, CAUSAL, MASKED>(st, cx, j, Kc, s0, s1);
  const float c = BS ? ts.c : cx.c;
  if constexpr (!SUMCHECK) {
    float m2t = tile_max2<BN>(s0, s1, c);
    if constexpr (BS) m2t += ts.lv;
    lazy_rescale<D, DT>(st, m2t);
    const float mref = (st.m2 == -__builtin_inff()) ? 0.f : st.m2;
    const float off = BS ? ts.lv - mref : -mref;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c, off));
      if constexpr (BN == 64) s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c, off));
    }
    if constexpr (DT == ATTN_FP8_E4M3) {
      pv_tile<D>(st, pack_p_fp8(s0, s1), Vc);
    } else {
      i16x8 pf[4];
      pf[0] = pack8<DT>(s0, 0);
      pf[1] = pack8<DT>(s0, 8);
      if constexpr (BN == 64) {
        pf[2] = pack8<DT>(s1, 0);
        pf[3] = pack8<DT>(s1, 8);
      }
      pv_tile<D, DT, BN>(st, pf, Vc);
      if constexpr (DT == ATTN_F16) {
        st.lrun = row_sum_f16_into<BN / 16>(pf, st.lrun);
        return;
      }
    }
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      ls0 += s0[r];
      ls1 += s0[r + 1];
    }
    if constexpr (BN == 64) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        ls0 += s1[r];
        ls1 += s1[r + 1];
      }
    }
    if constexpr (BS) st.lrun = __builtin_fmaf(ls0 + ls1, ts.iv, st.lrun);
    else st.lrun += ls0 + ls1;
    return;
  }
  i16x8 pf[4];
  i32x8 pf8;
  // p = 2^(c s + lv - mref) in place of the scores, packed for the P V
  // product; returns this lane's half-row sum (of the rounded binary16 P,
  // else of the unrounded p).
  auto probs = [&](float mref) -> float {
    const float off = BS ? ts.lv - mref : -mref;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c, off));
      if constexpr (BN == 64) s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c, off));
    }
    if constexpr (DT == ATTN_FP8_E4M3) {
      pf8 = pack_p_fp8(s0, s1);
    } else {
      pf[0] = pack8<DT>(s0, 0);
      pf[1] = pack8<DT>(s0, 8);
      if constexpr (BN == 64) {
        pf[2] = pack8<DT>(s1, 0);
        pf[3] = pack8<DT>(s1, 8);
      }
    }
    if constexpr (DT == ATTN_F16) {
      return row_sum_f16<BN / 16>(pf);
    } else {
      float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        ls0 += s0[r];
        ls1 += s0[r + 1];
      }
      if constexpr (BN == 64) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          ls0 += s1[r];
          ls1 += s1[r + 1];
        }
      }
      return ls0 + ls1;
    }
  };
  // The reference m2 moves only when it must (lazy rescale).  With a set
  // reference the probabilities are formed against it directly, and the
  // half-row sums show whether every p stayed within 2^kLazy; only if one
  // did not (or a row has no reference yet) is the tile scored again, its
  // row max taken, the reference raised to it, O and l rescaled by
  // 2^(old - new), and the probabilities formed again.  The result does
  // not depend on the reference, only its rounding does.
  float ls;
  bool refresh = __any(st.m2 == -__builtin_inff());  // wave-uniform
  if (!refresh) {
    ls = probs(st.m2);
    refresh = __any(!(ls <= kLazySum));
    if (refresh) {
      asm volatile("" ::: "memory");  // a real, rarely taken branch
      masked_scores<D, DT, CAUSAL, MASKED>(st, cx, j, Kc, s0, s1);
    }
  }
  if (refresh) {
    asm volatile("" ::: "memory");
    float m2t = tile_max2<BN>(s0, s1, c);
    if constexpr (BS) m2t += ts.lv;
    const float m2new = fmaxf(st.m2, m2t);
    const float alpha = m2new == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(st.m2 - m2new);
    st.m2 = m2new;
    st.lrun *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) st.oacc[i] *= alpha;
    ls = probs(m2new == -__builtin_inff() ? 0.f : m2new);
  }
  if constexpr (DT == ATTN_FP8_E4M3) pv_tile<D>(st, pf8, Vc);
  else pv_tile<D, DT, BN>(st, pf, Vc);
  if constexpr (BS) st.lrun = __builtin_fmaf(ls, ts.iv, st.lrun);
  else st.lrun += ls;
}

// The sequential step over a 128-key tile (the key-tile-size axis of the
// tuning variants): two 64-key halves share one row max, one reference
// update and one rescale check, and each barrier hands over twice the keys.
// BS: block-scaled E4M3, one K/V block (and TileScale) per half.
template <int D, int DT, bool CAUSAL, bool MASKED, bool BS = false>
__device__ __forceinline__ void seq_step128(WaveState<D, DT>& st, const LoopCtxT<128>& cx, int j, const lds_t* Kc,
                                            const lds_t* Vc, const TileScale (&ts)[2]) {
  static_assert(!BS || DT == ATTN_FP8_E4M3, "block scales are an E4M3 variant");
  // score scale and exponent offset of each half
  const float c0 = BS ? ts[0].c : cx.c, c1 = BS ? ts[1].c : cx.c;
  constexpr int kRowBytes = D * Fmt<DT>::kBytes;
  constexpr int kHalf = 64 * kRowBytes;
  // The half-row-sum check of seq_step (no row max per tile) at binary16
  // d = 64 only: 3-4% faster there at B=8 H=8 N=1024 causal and B=2 H=16
  // N=2048, 1% at B=4 H=8 N=1024 causal; bfloat16 d = 64, which sums the
  // unrounded p, measured 2-3% slower with it, and at 16-bit d = 128 the
  // check's live P fragments spill.
  constexpr bool kSumCheck = D == 64 && DT == ATTN_F16;
  f32x16 s0, s1, s2, s3;
  auto scores = [&]() {
    // A masked-loop step whose tile needs no bias (the loop starts at an
    // even tile, so it can take one fully visible tile before the first
    // that needs one) skips the per-score compare and select.
    if (MASKED && needs_bias<CAUSAL>(cx, j)) {
      const int rem = cx.visible(j) ? cx.template mask_rem<CAUSAL>(j) : -(1 << 30);
      mask_bias<64>(s0, s1, rem);
      mask_bias<64>(s2, s3, rem - 64);
      tile_scores<D, DT, true, 64>(st, Kc, s0, s1);
      tile_scores<D, DT, true, 64>(st, Kc + kHalf, s2, s3);
    } else {
      tile_scores<D, DT, false, 64>(st, Kc, s0, s1);
      tile_scores<D, DT, false, 64>(st, Kc + kHalf, s2, s3);
    }
  };
  i16x8 pf[8];
  // p in place of the scores, packed (16-bit); returns this lane's half-row
  // sum (binary16: of the rounded P; else of the unrounded p)
  auto probs = [&](float mref) -> float {
    const float off0 = BS ? ts[0].lv - mref : -mref, off1 = BS ? ts[1].lv - mref : -mref;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c0, off0));
      s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c0, off0));
      s2[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[r], c1, off1));
      s3[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s3[r], c1, off1));
    }
    if constexpr (DT != ATTN_FP8_E4M3) {
      pf[0] = pack8<DT>(s0, 0);
      pf[1] = pack8<DT>(s0, 8);
      pf[2] = pack8<DT>(s1, 0);
      pf[3] = pack8<DT>(s1, 8);
      pf[4] = pack8<DT>(s2, 0);
      pf[5] = pack8<DT>(s2, 8);
      pf[6] = pack8<DT>(s3, 0);
      pf[7] = pack8<DT>(s3, 8);
    }
    if constexpr (DT == ATTN_F16) {
      return row_sum_f16<8>(pf);
    } else if constexpr (BS) {
      // each half's p' / vd of its block
      float la = 0.f, lb = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        la += s0[r] + s1[r];
        lb += s2[r] + s3[r];
      }
      return __builtin_fmaf(la, ts[0].iv, lb * ts[1].iv);
    } else {
      float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        ls0 += s0[r] + s2[r];
        ls1 += s1[r] + s3[r];
      }
      return ls0 + ls1;
    }
  };
  // the reference, as in seq_step
  auto refresh_reference = [&]() {
    float ma = fmaxf(s0[0], s1[0]), mb = fmaxf(s2[0], s3[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      ma = fmaxf(fmaxf(ma, s0[r]), s1[r]);
      mb = fmaxf(fmaxf(mb, s2[r]), s3[r]);
    }
    const float m2t = BS ? swap_halves_max(fmaxf(__builtin_fmaf(ma, c0, ts[0].lv), __builtin_fmaf(mb, c1, ts[1].lv)))
                         : swap_halves_max(fmaxf(ma, mb)) * cx.c;
    const float m2new = fmaxf(st.m2, m2t);
    const float alpha = m2new == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(st.m2 - m2new);
    st.m2 = m2new;
    st.lrun *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) st.oacc[i] *= alpha;
  };
  scores();
  float ls;
  if constexpr (kSumCheck) {
    bool refresh = __any(st.m2 == -__builtin_inff());
    if (!refresh) {
      ls = probs(st.m2);
      refresh = __any(!(ls <= kLazySum));
      if (refresh) {
        asm volatile("" ::: "memory");  // a real, rarely taken branch
        scores();
      }
    }
    if (refresh) {
      asm volatile("" ::: "memory");
      refresh_reference();
      ls = probs(st.m2 == -__builtin_inff() ? 0.f : st.m2);
    }
  } else {
    float ma = fmaxf(s0[0], s1[0]), mb = fmaxf(s2[0], s3[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      ma = fmaxf(fmaxf(ma, s0[r]), s1[r]);
      mb = fmaxf(fmaxf(mb, s2[r]), s3[r]);
    }
    const float m2t = BS ? swap_halves_max(fmaxf(__builtin_fmaf(ma, c0, ts[0].lv), __builtin_fmaf(mb, c1, ts[1].lv)))
                         : swap_halves_max(fmaxf(ma, mb)) * cx.c;
    lazy_rescale<D, DT>(st, m2t);
    ls = probs(st.m2 == -__builtin_inff() ? 0.f : st.m2);
  }
  if constexpr (DT == ATTN_FP8_E4M3) {
    pv_tile<D>(st, pack_p_fp8(s0, s1), Vc);
    pv_tile<D>(st, pack_p_fp8(s2, s3), Vc + kHalf);
  } else {
    pv_tile<D, DT, 128>(st, pf, Vc);
  }
  st.lrun += ls;
}

// BS: block-scaled E4M3 (per-tile descales, see TileScale).  BNV: keys per
// tile, 0 for the default (TileKeys); 32 or 128 for the tile-size variants.
template <int D, int DT, bool CAUSAL, bool BS = false, int BNV = 0>
__global__ void __launch_bounds__(64 * (Waves<D, DT>::value)) __attribute__((amdgpu_waves_per_eu(2)))
attn_fwd_seq_kernel(Params p) {
  static_assert(!BS || DT == ATTN_FP8_E4M3, "block scales are an E4M3 variant");
  constexpr int kWaves = Waves<D, DT>::value;
  constexpr int kBlockM = kWaves * kRowsPerWave;
  constexpr int kRowBytes = D * Fmt<DT>::kBytes;
  constexpr int BN = BNV ? BNV : TileKeys<D, DT>::value;
  static_assert(!BS || BN == 64 || BN == 128, "block-scaled tiles are one or two 64-row blocks");
  static_assert(DT != ATTN_FP8_E4M3 || BN == 64 || BN == 128, "E4M3 tiles are multiples of the MFMA's 64 keys");
  constexpr int kTileBytes = BN * kRowBytes;
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
  Timeline tl;
  tl.init(p, kWaves, wave);
  int bh, qt;
  schedule(p, blockIdx.x, CAUSAL, bh, qt);
  const int q0 = qt * kBlockM;
  LoopCtxT<BN> cx;
  cx.qw0 = q0 + wave * kRowsPerWave;
  cx.qrow = cx.qw0 + (lane & 31);
  cx.diag = p.Nk - p.Nq;
  cx.Nk = p.Nk;
  cx.half = lane >> 5;
  cx.c = p.c;
  cx.wave_kend = CAUSAL ? cx.qw0 + kRowsPerWave - 1 + cx.diag : p.Nk;
  int kend = p.Nk;
  if (CAUSAL) kend = min(p.Nk, q0 + kBlockM + cx.diag);
  const int nt = kend > 0 ? (kend + BN - 1) / BN : 0;
  cx.nt = nt;

  const uint32_t head_bytes = (uint32_t)p.Nk * kRowBytes;
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc(p.k + (size_t)bh * p.Nk * kRowBytes, head_bytes);
  const __amdgpu_buffer_rsrc_t Vr = make_rsrc(p.v + (size_t)bh * p.Nk * kRowBytes, head_bytes);
  // Who issues the K/V tile loads: every wave its share, except in the
  // 8-wave forms at 16-bit d = 256 and at E4M3 (d = 128, 256), where four
  // waves issue them all.  Wave w shares SIMD w with wave w + 4, and one
  // wave of each pair gets the matrix core first and then waits at the step
  // barrier (the timeline probe shows it for the producer-wave kernel).
  // Which four pays was measured: at 16-bit d = 256 waves 0-3
  // (causal_d256_bf16 1.8% faster; waves 4-7 2% slower), at E4M3 waves 4-7
  // (d = 128 0.8% faster, block-scaled 1.2%, d = 256 1.5-1.7%; waves 0-3
  // 0.7-2.5% slower).
  constexpr bool kE4M3Hi = DT == ATTN_FP8_E4M3 && kWaves == 8;
  constexpr int kLoadFirst = kE4M3Hi ? 4 : 0;
  constexpr int kLoadWaves = ((D == 256 && DT != ATTN_FP8_E4M3) || kE4M3Hi) ? 4 : kWaves;
  const int lw = wave - kLoadFirst;
  const bool loader = lw >= 0 && lw < kLoadWaves;
  TileLoader<D, DT, kLoadWaves, BN> ld;
  ld.init(loader ? lw : 0, lane);
  WaveState<D, DT> st;
  st.init(p.q + (size_t)bh * p.Nq * kRowBytes, cx.qrow, p.Nq, lane, p.q_and, p.q_xor);

  if (nt > 0 && loader) {
    ld.load(K0, Kr, 0);
    ld.load(V0, Vr, 0);
  }
  // Tiles before tb need no mask bias: steps j < jm (jm even) run the
  // unmasked step, the rest the masked one (two loops, one step variant
  // each).
  const int tb = min(first_bias_tile<CAUSAL>(cx), nt);
  const int jm = tb & ~1;
  // Block scales: the wave's 32 rows lie in one 64-row Q block (rows past
  // Nq take the last block; they are not stored); K/V blocks NB j .. NB j +
  // NB - 1 are tile j (a block past the last one, whose keys are all
  // masked, takes the last block's descales).  The descales of tile j + 1
  // are read with that tile's loads, so the step's vmcnt wait covers them
  // too.  The pointers are global-address-space ones: through a generic
  // pointer the reads become flat loads, which the compiler must order
  // after the tile's direct-to-LDS loads (a flat address may be LDS), so it
  // waits for those loads right after issuing them.
  constexpr int NB = BN / 64 > 0 ? BN / 64 : 1;
  float cq = 0.f, kd[NB] = {}, vd[NB] = {};
  typedef const __attribute__((address_space(1))) float gfloat;
  gfloat* ksh = nullptr;
  gfloat* vsh = nullptr;
  auto read_scales = [&](int t) {
#pragma unroll
    for (int h = 0; h < NB; ++h) {
      const int b = min(NB * t + h, p.nkb - 1);
      kd[h] = ksh[b];
      vd[h] = vsh[b];
    }
  };
  if constexpr (BS) {
    cq = p.c * ((gfloat*)p.qs)[(size_t)bh * p.nqb + min(cx.qw0 / 64, p.nqb - 1)];
    ksh = (gfloat*)(p.ks + (size_t)bh * p.nkb);
    vsh = (gfloat*)(p.vs + (size_t)bh * p.nkb);
    if (nt > 0) read_scales(0);
  }
  tl.mark(1);
  // Step j: K_j, V_j in (Kc, Vc); tile j + 1 -> (Kl, Vl).
  auto step = [&](int j, const lds_t* Kc, const lds_t* Vc, lds_t* Kl, lds_t* Vl, auto masked) {
    constexpr bool M = decltype(masked)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    TileScale ts[NB] = {};
    if constexpr (BS) {
#pragma unroll
      for (int h = 0; h < NB; ++h) {
        ts[h].c = cq * kd[h];
        ts[h].lv = __builtin_amdgcn_logf(vd[h]);
        ts[h].iv = __builtin_amdgcn_rcpf(vd[h]);
      }
    }
    tl.wait_begin();
    __syncthreads();
    tl.wait_end();
    if (j + 1 < nt) {
      if (loader) {
        ld.load(Kl, Kr, (j + 1) * BN);
        ld.load(Vl, Vr, (j + 1) * BN);
      }
      if constexpr (BS) read_scales(j + 1);
    }
    if constexpr (BN == 128) seq_step128<D, DT, CAUSAL, M, BS>(st, cx, j, Kc, Vc, ts);
    else seq_step<D, DT, CAUSAL, M, BN, BS>(st, cx, j, Kc, Vc, ts[0]);
    tl.step(j);
  };
  int j = 0;
  for (; j < jm; j += 2) {
    step(j, K0, V0, K1, V1, BoolTag<false>{});
    step(j + 1, K1, V1, K0, V0, BoolTag<false>{});
  }
  for (; j < nt; j += 2) {
    step(j, K0, V0, K1, V1, BoolTag<true>{});
    if (j + 1 >= nt) break;
    step(j + 1, K1, V1, K0, V0, BoolTag<true>{});
  }
  store_output<D, DT>(p, st, bh, cx.qrow, cx.half);
  tl.finish(nt);
}

// ---------------------------------------------------------------------------
// Producer-wave kernel (16-bit, d = 128): the pages' producer / consumer
// split ("Producer and consumer roles", concept card; "GPU producer-consumer
// kernel pattern").  Eight consumer waves run the sequential step and never
// touch global memory after loading Q; NP more waves only stream K and V
// tiles into an NS-stage ring.  Per step one workgroup barrier hands a stage
// over: before barrier j the producers have waited for their loads of tile j
// (vmcnt, loads retire in order), and every consumer has finished step j - 1;
// after it the producers refill the stage that step j - 1 read with tile
// j + NS - 1.  The consumers need at most 168 VGPRs, so three waves share a
// SIMD and the extra waves fit beside the eight.
// ---------------------------------------------------------------------------

template <int D, int DT, bool CAUSAL, int NS, int NP>
__global__ void __launch_bounds__(64 * (8 + NP)) attn_fwd_producer_kernel(Params p) {
  static_assert(D == 128, "producer-wave kernel: d = 128");
  constexpr int kConsumers = Waves<D, DT>::value;
  constexpr int kBlockM = kConsumers * kRowsPerWave;
  constexpr int kRowBytes = D * Fmt<DT>::kBytes;
  constexpr int BN = TileKeys<D, DT>::value;
  constexpr int kTileBytes = BN * kRowBytes;
  using Loader = TileLoader<D, DT, NP, BN>;
  constexpr int kLoads = 2 * Loader::kPerWave;  // a producer wave's loads per K/V tile
  // At most NS - 1 tiles are in flight per producer wave.
  static_assert((NS - 1) * kLoads <= 63, "in-flight loads must fit the vmcnt counter");
  __shared__ __attribute__((aligned(1024))) unsigned char k_st[NS][kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_st[NS][kTileBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Timeline tl;
  tl.init(p, kConsumers + NP, wave);
  int bh, qt;
  schedule(p, blockIdx.x, CAUSAL, bh, qt);
  const int q0 = qt * kBlockM;
  int kend = p.Nk;
  if (CAUSAL) kend = min(p.Nk, q0 + kBlockM + (p.Nk - p.Nq));
  const int nt = kend > 0 ? (kend + BN - 1) / BN : 0;

  if (wave >= kConsumers) {
    const uint32_t head_bytes = (uint32_t)p.Nk * kRowBytes;
    const __amdgpu_buffer_rsrc_t Kr = make_rsrc(p.k + (size_t)bh * p.Nk * kRowBytes, head_bytes);
    const __amdgpu_buffer_rsrc_t Vr = make_rsrc(p.v + (size_t)bh * p.Nk * kRowBytes, head_bytes);
    Loader ld;
    ld.init(wave - kConsumers, lane);
    auto issue = [&](int t) {
      const int s = t % NS;
      ld.load((lds_t*)k_st[s], Kr, t * BN);
      ld.load((lds_t*)v_st[s], Vr, t * BN);
    };
    for (int t = 0; t < NS - 1 && t < nt; ++t) issue(t);
    tl.mark(1);
    for (int j = 0; j < nt; ++j) {
      // Issued so far: tiles 0 .. min(j + NS - 2, nt - 1); tile j must land.
      if (j + NS - 2 < nt) wait_vmcnt<(NS - 2) * kLoads>();
      else wait_vmcnt<0>();
      tl.wait_begin();
      __syncthreads();
      tl.wait_end();
      if (j + NS - 1 < nt) issue(j + NS - 1);
    }
    tl.finish(nt);
    return;  // the consumers' last barrier is the producers' last one
  }

  LoopCtxT<BN> cx;
  cx.qw0 = q0 + wave * kRowsPerWave;
  cx.qrow = cx.qw0 + (lane & 31);
  cx.diag = p.Nk - p.Nq;
  cx.Nk = p.Nk;
  cx.half = lane >> 5;
  cx.c = p.c;
  cx.wave_kend = CAUSAL ? cx.qw0 + kRowsPerWave - 1 + cx.diag : p.Nk;
  cx.nt = nt;
  WaveState<D, DT> st;
  st.init(p.q + (size_t)bh * p.Nq * kRowBytes, cx.qrow, p.Nq, lane, p.q_and, p.q_xor);
  const int tb = min(first_bias_tile<CAUSAL>(cx), nt);
  const TileScale ts{};
  tl.mark(1);
  // One barrier per step, nt in all, as on the producer side.
  auto step = [&](int j, int s, auto masked) {
    constexpr bool M = decltype(masked)::value;
    tl.wait_begin();
    __syncthreads();
    tl.wait_end();
    seq_step<D, DT, CAUSAL, M, BN, false, false>(st, cx, j, (const lds_t*)k_st[s], (const lds_t*)v_st[s], ts);
    tl.step(j);
  };
  // Steps run in groups of NS so that each one's stage is a constant.
  const int jm = tb - tb % NS;
  int j = 0;
  for (; j < jm; j += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) step(j + s, s, BoolTag<false>{});
  }
  for (; j < nt; j += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (j + s >= nt) break;
      step(j + s, s, BoolTag<true>{});
    }
  }
  store_output<D, DT>(p, st, bh, cx.qrow, cx.half);
  tl.finish(nt);
}

// ---------------------------------------------------------------------------
// Split-key kernel for small grids (16-bit, d = 64): each 128-row query tile
// gets an 8-wave workgroup whose two 4-wave groups walk the two halves of the
// tile's key range at the same time, each through its own K/V ring, and
// merge at the end -- group B hands (m, l, O) to group A through LDS, which
// rescales both partial results to the larger maximum and adds them (the
// online-softmax rescale of the concept card's sketch, applied once across
// the split).  Halves the sequential key loop of the longest query tiles,
// which is the critical path when there are about as many query tiles as
// CUs.
// ---------------------------------------------------------------------------
template <int D, int DT, bool CAUSAL>
__global__ void __launch_bounds__(512) attn_fwd_split_kernel(Params p) {
  static_assert(D == 64 && DT != ATTN_FP8_E4M3, "split-key kernel: 16-bit, d = 64");
  constexpr int kGroupWaves = 4;
  constexpr int kBlockM = kGroupWaves * kRowsPerWave;  // 128 query rows
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kBlockN * kRowBytes;
  constexpr int kAcc = D / 32 * 16;  // O accumulator floats per lane
  // Two rings (group A, group B), each with two K and two V stages.
  __shared__ __attribute__((aligned(1024))) unsigned char ka0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char ka1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char va0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char va1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char kb0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char kb1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vb0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vb1[kTileBytes];
  // Group B's partial results, [row block][m, l, O...][lane].
  __shared__ float xch[kGroupWaves][kAcc + 2][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = wave & 3, grp = wave >> 2;

  int bh, qt;
  schedule(p, blockIdx.x, CAUSAL, bh, qt);
  const int q0 = qt * kBlockM;
  int kend = p.Nk;
  if (CAUSAL) kend = min(p.Nk, q0 + kBlockM + (p.Nk - p.Nq));
  const int nt = kend > 0 ? (kend + kBlockN - 1) / kBlockN : 0;
  const int mid = (nt + 1) / 2;                 // group A: tiles [0, mid)
  const int j0 = grp ? mid : 0, j1 = grp ? nt : mid;  // this group's tiles
  LoopCtx cx;
  cx.qw0 = q0 + rb * kRowsPerWave;
  cx.qrow = cx.qw0 + (lane & 31);
  cx.diag = p.Nk - p.Nq;
  cx.Nk = p.Nk;
  cx.half = lane >> 5;
  cx.c = p.c;
  cx.wave_kend = CAUSAL ? cx.qw0 + kRowsPerWave - 1 + cx.diag : p.Nk;
  cx.nt = j1;  // tiles from j1 on belong to the other group (or do not exist)

  const uint32_t head_bytes = (uint32_t)p.Nk * kRowBytes;
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc(p.k + (size_t)bh * p.Nk * kRowBytes, head_bytes);
  const __amdgpu_buffer_rsrc_t Vr = make_rsrc(p.v + (size_t)bh * p.Nk * kRowBytes, head_bytes);
  TileLoader<D, DT, kGroupWaves> ld;
  ld.init(rb, lane);
  WaveState<D, DT> st;
  st.init(p.q + (size_t)bh * p.Nq * kRowBytes, cx.qrow, p.Nq, lane, p.q_and, p.q_xor);

  // The key loop of one group over tiles [j0, j1), as in attn_fwd_kernel.
  // Every group executes the same number of barriers: 1 + (mid + 1) / 2
  // loop pairs, steps past its range being barrier-only.
  const int pairs = (mid + 1) / 2;
  auto run = [&](lds_t* K0, lds_t* K1, lds_t* V0, lds_t* V1) {
    f32x16 a0, a1, b0, b1;
    const int len = j1 - j0;
    if (len > 0) {
      ld.load(K0, Kr, j0 * kBlockN);
      ld.load(V0, Vr, j0 * kBlockN);
      ld.load(K1, Kr, (j0 + 1) * kBlockN);  // zeros or finite data when past the range
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int tb = first_bias_tile<CAUSAL>(cx);
    if (len > 0) {
      if (tb > j0) masked_scores<D, DT, CAUSAL, false>(st, cx, j0, K0, a0, a1);
      else masked_scores<D, DT, CAUSAL, true>(st, cx, j0, K0, a0, a1);
      bool rescale;
      update_reference(st.m2, tile_max2(a0, a1, cx.c), rescale);
    }
    auto two_steps = [&](int j, auto masked) {
      constexpr bool M = decltype(masked)::value;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (j < j1) {
        if (j + 2 < j1) ld.load(K0, Kr, (j + 2) * kBlockN);
        if (j + 1 < j1) ld.load(V1, Vr, (j + 1) * kBlockN);
        step<D, DT, CAUSAL, M>(st, cx, j, a0, a1, b0, b1, K1, V0);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (j + 1 < j1) {
        if (j + 3 < j1) ld.load(K1, Kr, (j + 3) * kBlockN);
        if (j + 2 < j1) ld.load(V0, Vr, (j + 2) * kBlockN);
        step<D, DT, CAUSAL, M>(st, cx, j + 1, b0, b1, a0, a1, K0, V1);
      }
    };
    // Unmasked pairs while tile j + 2 needs no bias, then masked pairs.
    int i = 0;
    for (; i < pairs && j0 + 2 * i + 2 < tb; ++i) two_steps(j0 + 2 * i, BoolTag<false>{});
    for (; i < pairs; ++i) two_steps(j0 + 2 * i, BoolTag<true>{});
  };
  if (grp == 0) run((lds_t*)ka0, (lds_t*)ka1, (lds_t*)va0, (lds_t*)va1);
  else run((lds_t*)kb0, (lds_t*)kb1, (lds_t*)vb0, (lds_t*)vb1);

  // Merge: group B publishes, group A combines and stores.
  if (grp == 1) {
    xch[rb][0][lane] = st.m2;
    xch[rb][1][lane] = st.lrun;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[rb][2 + 16 * i + r][lane] = st.oacc[i][r];
  }
  __syncthreads();
  if (grp == 0) {
    const float mb = xch[rb][0][lane];
    const float m = fmaxf(st.m2, mb);
    const float wa = (st.m2 == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(st.m2 - m);
    const float wb = (mb == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(mb - m);
    st.m2 = m;
    st.lrun = wa * st.lrun + wb * xch[rb][1][lane];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[i][r] = wa * st.oacc[i][r] + wb * xch[rb][2 + 16 * i + r][lane];
    store_output<D, DT>(p, st, bh, cx.qrow, cx.half);
  }
}

// 16-bit d = 64 on grids of kSplitMinGrid to kSplitMaxGrid 128-row query
// tiles (a grid of a few tiles is bound by launch and load latency, a grid
// of more than two rounds of the 256 CUs by throughput): the split-key
// kernel where the longest key loops are the critical path -- up to one
// round of tiles with at least kSplitMinKeys keys, or causal with at least
// kSplitMinKeysCausal keys on up to two rounds -- and the sequential kernel
// with 128-key tiles (two 4-wave workgroups per CU) otherwise.  Tuner runs
// over 20 shapes in this range put each choice ahead of the other by 1-35%,
// except at 64 tiles with 1,024 keys, where the two are within 2%.
template <int D, int DT>
struct UseSplit {
  static constexpr bool value = (D == 64 && DT != ATTN_FP8_E4M3);
};
constexpr long long kSplitMinGrid = 64;
constexpr long long kSplitMaxGrid = 512;
constexpr int kSplitMinKeys = 2048;
constexpr int kSplitMinKeysCausal = 4096;
constexpr int kSmallGridSeqKeys = 256;  // below kSplitMinGrid: 64-key kernel up to this many keys, non-causal
__host__ inline bool split_wins(long long grid128, int Nk, bool causal) {
  if (grid128 <= 256) return Nk >= kSplitMinKeys;
  return causal && Nk >= kSplitMinKeysCausal;
}

// Which loop a (head dim, format) uses: the sequential-step kernel for
// E4M3 at d = 128 and for d = 256 (where dropping the pipelined score tile,
// and for 16-bit inputs halving the key tile, lets two workgroups share a
// CU, so every SIMD runs two waves: 887 -> 1,145 TFLOP/s on causal bf16),
// and for 16-bit d = 64 (its half-row-sum check keeps it at three waves per
// SIMD: 3% faster than the pipelined kernel at B=2 H=16 N=8192, fp16 and
// causal bf16); the pipelined one elsewhere.
template <int D, int DT>
struct Sequential {
  static constexpr bool value = (D == 128 && DT == ATTN_FP8_E4M3) || D == 256 || (D == 64 && DT != ATTN_FP8_E4M3);
};

// binary16 at d = 128 takes the producer-wave kernel: 1.8-3.5% faster than
// the pipelined one on every binary16 shape measured (8K and 2K keys, causal
// or not).  bfloat16 (0.5-3% slower) and E4M3 (1% slower) keep theirs.
template <int D, int DT>
struct UseProducer {
  static constexpr bool value = D == 128 && DT == ATTN_F16;
};

// E4M3 at d = 128 takes the sequential kernel with 128-key tiles: its step
// is bound by softmax VALU work, and one row max, reference update and
// barrier per 128 keys instead of per 64 measured 5% faster than 64-key
// tiles on B=2 H=16 N=8192 with outliers (0.557 vs 0.585 ms).  (At d = 64
// it is 5% faster than the pipelined kernel too, 0.388 vs 0.409 ms, but it
// misses the E4M3 gate on a one-row edge case the pipelined kernel meets,
// so d = 64 keeps that one.)
template <int D, int DT>
struct UseBC128 {
  static constexpr bool value = D == 128 && DT == ATTN_FP8_E4M3;
};

// Kernel choices a caller can make (include/attn.h, attn_fwd_variant):
// the pipelined kernel with a two- or four-stage ring (not at d = 256, whose
// pipelined registers leave one wave per SIMD), the sequential kernel, the
// split-key kernel (16-bit d = 64), the pingpong kernel (d = 128), the
// producer-wave kernel (d = 128), the wide-wave kernel (16-bit d = 128), the
// sequential kernel with 32- or 128-key tiles and the three-stage pipelined
// kernel.  ATTN_VARIANT_AUTO takes the measured defaults above.
template <int D, int DT>
struct Variants {
  static constexpr bool pipelined = D != 256;
  static constexpr bool split = UseSplit<D, DT>::value;
  static constexpr bool pingpong = D == 128;
  static constexpr bool producer = D == 128;
  static constexpr bool wide = D == 128 && DT != ATTN_FP8_E4M3;
  // key-tile-size axis of the sequential kernel: 32 keys (16-bit d = 64,
  // 128; 16-bit d = 256 already runs 32) and 128 keys (d = 64, 128; at
  // d = 256 the four score accumulators do not fit beside O and Q)
  static constexpr bool bc32 = DT != ATTN_FP8_E4M3 && D != 256;
  static constexpr bool bc128 = D != 256;
  static constexpr bool pipe3 = DT != ATTN_FP8_E4M3 && D != 256;
};

// The wide-wave kernels (attn_fwd_wide.h) live in a translation unit of
// their own, built with the compiler's default MFMA register form.
int launch_wide_d128(const Params& p, int dtype, bool causal, hipStream_t stream);
// The 16-bit d = 128 tile-size variants likewise (attn_fwd_d128_bc.hip).
int launch_seq_bc_d128(const Params& p, int dtype, bool causal, int bn, hipStream_t stream);

// Score scaling of a launch.  The kernels need c = scale * log2(e) > 0: the
// -inf mask bias must stay -inf after the multiply, and the row max must be
// the max of c * s.  A negative scale is folded into Q instead (its sign
// bits flipped as Q is loaded: (-Q) K^T is exactly -(Q K^T)), and a zero one
// (or one whose c underflows to 0) clears Q, so every score is exactly 0 and
// any c > 0 gives the uniform softmax over the visible keys.
__host__ inline void set_scale(Params& p, float scale, int dtype) {
  const uint32_t sign = dtype == ATTN_FP8_E4M3 ? 0x80808080u : 0x80008000u;
  p.c = fabsf(scale) * kLog2e;
  p.q_and = 0xffffffffu;
  p.q_xor = 0u;
  if (!(p.c > 0.f)) {
    p.c = 1.f;
    p.q_and = 0u;
  } else if (scale < 0.f) {
    p.q_xor = sign;
  }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------
template <int D, int DT, bool CAUSAL>
int launch_one(const Problem& pr, hipStream_t stream) {
  Params p;
  p.q = (const unsigned char*)pr.q;
  p.k = (const unsigned char*)pr.k;
  p.v = (const unsigned char*)pr.v;
  p.o = (uint16_t*)pr.o;
  p.lse = pr.lse;
  p.Nq = pr.Nq;
  p.Nk = pr.Nk;
  constexpr int kWaves = Waves<D, DT>::value;
  constexpr int kBlockM = kWaves * kRowsPerWave;
  p.n_qtiles = (pr.Nq + kBlockM - 1) / kBlockM;
  const long long total = (long long)pr.B * pr.H * p.n_qtiles;
  if (total > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  p.total_tiles = (int)total;
  set_scale(p, pr.scale, DT);
  p.o_scale = pr.v_descale;
  p.qs = p.ks = p.vs = nullptr;
  p.nqb = p.nkb = 0;
  const int n128 = (pr.Nq + 127) / 128;
  const long long grid128 = (long long)pr.B * pr.H * n128;
  int variant = pr.variant;
  if (variant == ATTN_VARIANT_AUTO) {
    variant = Sequential<D, DT>::value ? ATTN_VARIANT_SEQUENTIAL : ATTN_VARIANT_PIPELINED;
    if (UseProducer<D, DT>::value) variant = ATTN_VARIANT_PRODUCER;
    if (UseBC128<D, DT>::value) variant = ATTN_VARIANT_SEQUENTIAL_BC128;
    // Mid-size 16-bit d = 64 grids: split-key or 128-key sequential kernel.
    if (UseSplit<D, DT>::value && grid128 >= kSplitMinGrid && grid128 <= kSplitMaxGrid)
      variant = split_wins(grid128, pr.Nk, CAUSAL) ? ATTN_VARIANT_SPLIT : ATTN_VARIANT_SEQUENTIAL_BC128;
    // Smaller ones the same way, but for short non-causal key ranges, where
    // the 64-key kernel is as fast or 3% faster (one 128-key step against
    // two 64-key ones; graph-replayed: the split kernel 10-15% ahead from
    // 2,048 keys on, the 128-key kernel 3-10% ahead below them).
    if (UseSplit<D, DT>::value && grid128 < kSplitMinGrid) {
      if (split_wins(grid128, pr.Nk, CAUSAL)) variant = ATTN_VARIANT_SPLIT;
      else if (CAUSAL || pr.Nk > kSmallGridSeqKeys) variant = ATTN_VARIANT_SEQUENTIAL_BC128;
    }
  }
  const dim3 block(64 * kWaves);
  switch (variant) {
    case ATTN_VARIANT_SPLIT:
      if constexpr (Variants<D, DT>::split) {
        if (grid128 > 0x7fffffffLL) return ATTN_ERR_SHAPE;
        p.n_qtiles = n128;
        p.total_tiles = (int)grid128;
        hipLaunchKernelGGL((attn_fwd_split_kernel<D, DT, CAUSAL>), dim3(p.total_tiles), dim3(512), 0, stream, p);
        break;
      }
      return ATTN_ERR_VARIANT;
    case ATTN_VARIANT_SEQUENTIAL:
      hipLaunchKernelGGL((attn_fwd_seq_kernel<D, DT, CAUSAL>), dim3(p.total_tiles), block, 0, stream, p);
      break;
    case ATTN_VARIANT_PIPELINED:
      if constexpr (Variants<D, DT>::pipelined) {
        hipLaunchKernelGGL((attn_fwd_kernel<D, DT, CAUSAL, 2>), dim3(p.total_tiles), block, 0, stream, p);
        break;
      }
      return ATTN_ERR_VARIANT;
    case ATTN_VARIANT_PIPELINED_4STAGE:
      if constexpr (Variants<D, DT>::pipelined) {
        hipLaunchKernelGGL((attn_fwd_kernel<D, DT, CAUSAL, 4>), dim3(p.total_tiles), block, 0, stream, p);
        break;
      }
      return ATTN_ERR_VARIANT;
    case ATTN_VARIANT_PINGPONG:
      if constexpr (Variants<D, DT>::pingpong) {
        hipLaunchKernelGGL((attn_fwd_pingpong_kernel<D, DT, CAUSAL>), dim3(p.total_tiles), block, 0, stream, p);
        break;
      }
      return ATTN_ERR_VARIANT;
    case ATTN_VARIANT_PRODUCER:
      if constexpr (Variants<D, DT>::producer) {
        hipLaunchKernelGGL((attn_fwd_producer_kernel<D, DT, CAUSAL, 2, 1>), dim3(p.total_tiles), dim3(64 * 9), 0,
                           stream, p);
        break;
      }
      return ATTN_ERR_VARIANT;
    case ATTN_VARIANT_WIDE:
      if constexpr (Variants<D, DT>::wide) return launch_wide_d128(p, DT, CAUSAL, stream);
      return ATTN_ERR_VARIANT;
    case ATTN_VARIANT_PIPELINED_3STAGE:
      if constexpr (Variants<D, DT>::pipe3) {
        hipLaunchKernelGGL((attn_fwd_pipe3_kernel<D, DT, CAUSAL>), dim3(p.total_tiles), block, 0, stream, p);
        break;
      }
      return ATTN_ERR_VARIANT;
    case ATTN_VARIANT_SEQUENTIAL_BC32:
      if constexpr (Variants<D, DT>::bc32) {
        if constexpr (D == 128) return launch_seq_bc_d128(p, DT, CAUSAL, 32, stream);
        else hipLaunchKernelGGL((attn_fwd_seq_kernel<D, DT, CAUSAL, false, 32>), dim3(p.total_tiles), block, 0, stream, p);
        break;
      }
      return ATTN_ERR_VARIANT;
    case ATTN_VARIANT_SEQUENTIAL_BC128:
      if constexpr (Variants<D, DT>::bc128) {
        if constexpr (D == 128 && DT != ATTN_FP8_E4M3) return launch_seq_bc_d128(p, DT, CAUSAL, 128, stream);
        else hipLaunchKernelGGL((attn_fwd_seq_kernel<D, DT, CAUSAL, false, 128>), dim3(p.total_tiles), block, 0, stream,
                                p);
        break;
      }
      return ATTN_ERR_VARIANT;
    default:
      return ATTN_ERR_VARIANT;
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Dispatch one head dimension over the 16-bit dtypes and causality.
template <int D>
int launch_16bit(const Problem& p, hipStream_t s) {
  switch (p.dtype) {
    case ATTN_F16:
      return p.causal ? launch_one<D, ATTN_F16, true>(p, s) : launch_one<D, ATTN_F16, false>(p, s);
    case ATTN_BF16:
      return p.causal ? launch_one<D, ATTN_BF16, true>(p, s) : launch_one<D, ATTN_BF16, false>(p, s);
    default:
      return ATTN_ERR_DTYPE;
  }
}

// Block-scaled E4M3: always the sequential kernel, whose steps take one
// key tile (= one K/V block) at a time.
template <int D, bool CAUSAL>
int launch_blockscaled(const Problem& pr, hipStream_t stream) {
  constexpr int kWaves = Waves<D, ATTN_FP8_E4M3>::value;
  constexpr int kBlockM = kWaves * kRowsPerWave;
  static_assert(TileKeys<D, ATTN_FP8_E4M3>::value == ATTN_FP8_BLOCK_ROWS, "one K/V block per key tile");
  Params p;
  p.q = (const unsigned char*)pr.q;
  p.k = (const unsigned char*)pr.k;
  p.v = (const unsigned char*)pr.v;
  p.o = (uint16_t*)pr.o;
  p.lse = pr.lse;
  p.Nq = pr.Nq;
  p.Nk = pr.Nk;
  p.n_qtiles = (pr.Nq + kBlockM - 1) / kBlockM;
  const long long total = (long long)pr.B * pr.H * p.n_qtiles;
  if (total > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  p.total_tiles = (int)total;
  set_scale(p, pr.scale, ATTN_FP8_E4M3);
  p.o_scale = 1.f;
  p.qs = pr.q_descales;
  p.ks = pr.k_descales;
  p.vs = pr.v_descales;
  p.nqb = (pr.Nq + ATTN_FP8_BLOCK_ROWS - 1) / ATTN_FP8_BLOCK_ROWS;
  p.nkb = (pr.Nk + ATTN_FP8_BLOCK_ROWS - 1) / ATTN_FP8_BLOCK_ROWS;
  // d = 64, 128: 128-key tiles (two blocks per tile), as the per-tensor default
  if constexpr (D != 256)
    hipLaunchKernelGGL((attn_fwd_seq_kernel<D, ATTN_FP8_E4M3, CAUSAL, true, 128>), dim3(p.total_tiles),
                       dim3(64 * kWaves), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_seq_kernel<D, ATTN_FP8_E4M3, CAUSAL, true>), dim3(p.total_tiles), dim3(64 * kWaves),
                       0, stream, p);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// E4M3, one head dimension.
template <int D>
int launch_fp8(const Problem& p, hipStream_t s) {
  if (p.dtype != ATTN_FP8_E4M3) return ATTN_ERR_DTYPE;
  if (p.q_descales)
    return p.causal ? launch_blockscaled<D, true>(p, s) : launch_blockscaled<D, false>(p, s);
  return p.causal ? launch_one<D, ATTN_FP8_E4M3, true>(p, s) : launch_one<D, ATTN_FP8_E4M3, false>(p, s);
}

}  // namespace kernels
}  // namespace attn
