#pragma once
// Wide-wave kernel (16-bit inputs, d = 128): every wave owns 64 query rows,
// as two 32-row blocks, instead of 32.  Each K operand fragment read from
// LDS then feeds two score MFMAs and each V^T fragment two P V MFMAs, which
// halves the LDS operand bytes per FLOP.  A wave holds Q (64 registers), O
// (128) and two score tiles (64 each), more than the 256 registers of a wave
// that shares its SIMD, so the workgroup runs four waves, one per SIMD, with
// up to 512 registers each (the MFMA accumulators in AGPRs), and all overlap
// of matrix work and softmax comes from within the wave: the two-stage
// pipelined step of the concept card ("Overlap of matrix multiplies and
// softmax inside one warpgroup"), phase A issuing the scores of tile j + 1
// under the exponentials of tile j, phase B O += P_j V_j under the row sums
// and the next row maxima.
//
// Included by its own translation unit only (attn_fwd_d128_wide.hip), which
// is built without the VGPR-form MFMA option.
#include "attn_fwd_kernel.h"

namespace attn {
namespace kernels {

constexpr int kWideWaves = 4;
constexpr int kWideRows = 2 * kRowsPerWave;  // query rows per wave

// Score accumulators of one BN-key tile: s[h] (keys 32h .. 32h + 31) of
// block x, s[NB + h] of block y, NB = BN / 32.
template <int BN>
struct WideTile {
  static constexpr int NB = BN / 32;
  f32x16 s[2 * NB];
};

// S^T = K Q^T of one tile for both row blocks.  Each K fragment read feeds
// one MFMA per block.
template <int D, int DT, bool BIAS, int BN>
__device__ __forceinline__ void wide_scores(const WaveState16<D, DT>& x, const WaveState16<D, DT>& y,
                                            const lds_t* Ks, WideTile<BN>& t) {
  constexpr int kRowBytes = D * 2;
  constexpr int kKOff = WaveState16<D, DT>::kKOff;
  constexpr int NB = WideTile<BN>::NB;
#pragma unroll
  for (int k = 0; k < D / 16; ++k) {
    const int o = x.koff[k % kKOff] + (k / kKOff) * 256;
    const bool zero = k == 0 && !BIAS;
#pragma unroll
    for (int h = 0; h < NB; ++h) {
      const i16x8 a = *(const lds_i16x8*)(Ks + o + h * 32 * kRowBytes);
      t.s[h] = Fmt<DT>::mma(a, x.qf[k], zero ? f32x16{} : t.s[h]);
      t.s[NB + h] = Fmt<DT>::mma(a, y.qf[k], zero ? f32x16{} : t.s[NB + h]);
    }
  }
}

// O^T += V^T P^T for both row blocks over the 16-key steps KS0 ..
// KS0 + NKS - 1 of the tile; each V^T fragment (two transpose reads) feeds
// one MFMA per block.
template <int D, int DT, int KS0, int NKS>
__device__ __forceinline__ void wide_pv(WaveState16<D, DT>& x, WaveState16<D, DT>& y, const i16x8 (&px)[4],
                                        const i16x8 (&py)[4], const lds_t* Vs) {
  constexpr int kRowBytes = D * 2;
#pragma unroll
  for (int ks = KS0; ks < KS0 + NKS; ++ks) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const lds_t* base = Vs + (db >> 2) * 256 + 16 * ks * kRowBytes;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + x.voff[db & 3][0]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + x.voff[db & 3][1]));
      const i16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      x.oacc[db] = Fmt<DT>::mma(a, px[ks], x.oacc[db]);
      y.oacc[db] = Fmt<DT>::mma(a, py[ks], y.oacc[db]);
    }
  }
}

// Scores of tile t for both blocks; MASKED starts each block's accumulators
// from its own mask bias (see needs_bias).
template <int D, int DT, bool CAUSAL, bool MASKED, int BN>
__device__ __forceinline__ void wide_masked_scores(const WaveState16<D, DT>& x, const WaveState16<D, DT>& y,
                                                   const LoopCtxT<BN>& cx, const LoopCtxT<BN>& cy, int t,
                                                   const lds_t* Ks, WideTile<BN>& w) {
  constexpr int NB = WideTile<BN>::NB;
  if constexpr (MASKED) {
    const int rx = cx.visible(t) ? cx.template mask_rem<CAUSAL>(t) : -(1 << 30);
    const int ry = cy.visible(t) ? cy.template mask_rem<CAUSAL>(t) : -(1 << 30);
    mask_bias<BN>(w.s[0], w.s[NB - 1], rx);
    mask_bias<BN>(w.s[NB], w.s[2 * NB - 1], ry);
  }
  wide_scores<D, DT, MASKED, BN>(x, y, Ks, w);
}

// p = exp2(s c - m2) for one block's NB score accumulators, then packed to
// the 16-bit P fragments of the P V product (2 NB of them).
template <int DT, int NB>
__device__ __forceinline__ void wide_probs(f32x16* s, float m2, float c, i16x8 (&pf)[4]) {
  const float mref = (m2 == -__builtin_inff()) ? 0.f : m2;
#pragma unroll
  for (int h = 0; h < NB; ++h) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[h][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[h][r], c, -mref));
    pf[2 * h] = pack8<DT>(s[h], 0);
    pf[2 * h + 1] = pack8<DT>(s[h], 8);
  }
}

template <int DT, int NB>
__device__ __forceinline__ float wide_row_sum(const f32x16* s, const i16x8 (&pf)[4]) {
  if constexpr (DT == ATTN_F16) {
    return row_sum_f16<2 * NB>(pf);
  } else {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int h = 0; h < NB; ++h)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        a += s[h][r];
        b += s[h][r + 1];
      }
    return a + b;
  }
}

// Instruction interleave of np MFMA pairs: after `pre` LDS reads, pairs of
// MFMAs with `valu` VALU or transcendental instructions after each and
// `reads` LDS reads after the first (mask 0x402: v_exp_f32 is not in the
// plain VALU class); then the end of the scheduling region.
#define ATTN_WIDE_INTERLEAVE(np, pre, valu, reads)           \
  do {                                                       \
    __builtin_amdgcn_sched_group_barrier(0x100, pre, 0);     \
    _Pragma("unroll") for (int i_ = 0; i_ < (np); ++i_) {    \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     \
      __builtin_amdgcn_sched_group_barrier(0x402, valu, 0);  \
      __builtin_amdgcn_sched_group_barrier(0x100, reads, 0); \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     \
      __builtin_amdgcn_sched_group_barrier(0x402, valu, 0);  \
    }                                                        \
    __builtin_amdgcn_sched_barrier(0);                       \
  } while (0)

// One pipelined step for tile j (s = S_j of both blocks on entry; n gets
// S_{j+1}):
//   phase A: S_{j+1} MFMAs              | exp2 and packing of P_j, both blocks
//   phase B: O += P_j V_j MFMAs         | row sums of P_j, row maxima of
//                                         S_{j+1}, reference updates
// then, rarely, a block's O and l are rescaled to its new reference.  A
// single wave per SIMD issues in order, so the VALU work has to sit between
// the MFMAs; each part is a scheduling region of at most 32 MFMAs (16 in
// phase B), which keeps the interleave.  The accumulators of S_{j+1} are
// read out of the AGPRs by the row-max code.
template <int D, int DT, bool CAUSAL, bool MASKED, int BN>
__device__ __forceinline__ void wide_step(WaveState16<D, DT>& x, WaveState16<D, DT>& y, const LoopCtxT<BN>& cx,
                                          const LoopCtxT<BN>& cy, int j, WideTile<BN>& s, WideTile<BN>& n,
                                          const lds_t* Kn, const lds_t* Vs) {
  constexpr int NB = WideTile<BN>::NB;
  static_assert(NB == 2, "64-key tiles");
  // Phase A: 16 NB MFMAs, one K read per MFMA pair; 80 NB VALU and
  // transcendental instructions (FMA, exp2, packs).
  wide_masked_scores<D, DT, CAUSAL, MASKED, BN>(x, y, cx, cy, j + 1, Kn, n);
  i16x8 px[4], py[4];
  wide_probs<DT, NB>(s.s, x.m2, cx.c, px);
  wide_probs<DT, NB>(s.s + NB, y.m2, cx.c, py);
  ATTN_WIDE_INTERLEAVE(8 * NB, 2 * NB, 5, 1);
  // Phase B in two halves of 16 MFMAs: keys 0-31 under the row sums and
  // block x's row max, keys 32-63 under block y's.
  bool rx, ry;
  wide_pv<D, DT, 0, 2>(x, y, px, py, Vs);
  x.lrun += wide_row_sum<DT, NB>(s.s, px);
  y.lrun += wide_row_sum<DT, NB>(s.s + NB, py);
  const float ax = update_reference(x.m2, tile_max2<BN>(n.s[0], n.s[1], cx.c), rx);
  ATTN_WIDE_INTERLEAVE(8, 4, 5, 2);
  wide_pv<D, DT, 2, 2>(x, y, px, py, Vs);
  const float ay = update_reference(y.m2, tile_max2<BN>(n.s[2], n.s[3], cx.c), ry);
  ATTN_WIDE_INTERLEAVE(8, 4, 4, 2);
  if (rx) {
    asm volatile("" ::: "memory");  // a real, rarely taken branch (see step)
    x.lrun *= ax;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) x.oacc[i] *= ax;
  }
  if (ry) {
    asm volatile("" ::: "memory");
    y.lrun *= ay;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) y.oacc[i] *= ay;
  }
}

template <int D, int DT, bool CAUSAL>
__global__ void __launch_bounds__(64 * kWideWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_fwd_wide_kernel(Params p) {
  static_assert(D == 128 && DT != ATTN_FP8_E4M3, "wide-wave kernel: 16-bit, d = 128");
  constexpr int BN = kBlockN;
  constexpr int kBlockM = kWideWaves * kWideRows;  // 256 query rows per workgroup
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = BN * kRowBytes;
  // Two-stage K and V rings; K runs one tile ahead of V (as in
  // attn_fwd_kernel).
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
  int kend = p.Nk;
  if (CAUSAL) kend = min(p.Nk, q0 + kBlockM + (p.Nk - p.Nq));
  const int nt = kend > 0 ? (kend + BN - 1) / BN : 0;
  // Block x: rows q0 + 64 wave + 0..31; block y: the next 32.
  LoopCtxT<BN> cx, cy;
  cx.qw0 = q0 + wave * kWideRows;
  cx.qrow = cx.qw0 + (lane & 31);
  cx.diag = p.Nk - p.Nq;
  cx.Nk = p.Nk;
  cx.half = lane >> 5;
  cx.c = p.c;
  cx.wave_kend = CAUSAL ? cx.qw0 + kRowsPerWave - 1 + cx.diag : p.Nk;
  cx.nt = nt;
  cy = cx;
  cy.qw0 = cx.qw0 + kRowsPerWave;
  cy.qrow = cx.qrow + kRowsPerWave;
  cy.wave_kend = CAUSAL ? cy.qw0 + kRowsPerWave - 1 + cy.diag : p.Nk;

  const uint32_t head_bytes = (uint32_t)p.Nk * kRowBytes;
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc(p.k + (size_t)bh * p.Nk * kRowBytes, head_bytes);
  const __amdgpu_buffer_rsrc_t Vr = make_rsrc(p.v + (size_t)bh * p.Nk * kRowBytes, head_bytes);
  TileLoader<D, DT, kWideWaves, BN> ld;
  ld.init(wave, lane);
  WaveState16<D, DT> x, y;
  const unsigned char* Qh = p.q + (size_t)bh * p.Nq * kRowBytes;
  x.init(Qh, cx.qrow, p.Nq, lane, p.q_and, p.q_xor);
  y.init(Qh, cy.qrow, p.Nq, lane, p.q_and, p.q_xor);

  WideTile<BN> a, b;
  // Block x's rows come first, so its first masked tile is the wave's.
  // Step j scores tile j + 1: steps j < jm (jm even) run unmasked.
  const int tb = first_bias_tile<CAUSAL>(cx);
  const int jm = tb > 1 ? (tb - 1) & ~1 : 0;
  if (nt > 0) {
    // K_1 is loaded even when there is no tile 1 (rows past Nk arrive as
    // zeros), so every K stage a step reads holds finite data.
    ld.load(K0, Kr, 0);
    ld.load(V0, Vr, 0);
    ld.load(K1, Kr, BN);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tb > 0) wide_masked_scores<D, DT, CAUSAL, false, BN>(x, y, cx, cy, 0, K0, a);
    else wide_masked_scores<D, DT, CAUSAL, true, BN>(x, y, cx, cy, 0, K0, a);
    constexpr int NB = WideTile<BN>::NB;
    bool r;
    update_reference(x.m2, tile_max2<BN>(a.s[0], a.s[NB - 1], cx.c), r);
    update_reference(y.m2, tile_max2<BN>(a.s[NB], a.s[2 * NB - 1], cx.c), r);
  }
  auto two_steps = [&](int j, auto masked) -> bool {
    constexpr bool M = decltype(masked)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 2 < nt) ld.load(K0, Kr, (j + 2) * BN);
    if (j + 1 < nt) ld.load(V1, Vr, (j + 1) * BN);
    wide_step<D, DT, CAUSAL, M, BN>(x, y, cx, cy, j, a, b, K1, V0);
    if (j + 1 >= nt) return false;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 3 < nt) ld.load(K1, Kr, (j + 3) * BN);
    if (j + 2 < nt) ld.load(V0, Vr, (j + 2) * BN);
    wide_step<D, DT, CAUSAL, M, BN>(x, y, cx, cy, j + 1, b, a, K0, V1);
    return true;
  };
  int j = 0;
  for (; j < jm; j += 2) two_steps(j, BoolTag<false>{});
  for (; j < nt; j += 2)
    if (!two_steps(j, BoolTag<true>{})) break;
  store_output<D, DT>(p, x, bh, cx.qrow, cx.half);
  store_output<D, DT>(p, y, bh, cy.qrow, cy.half);
}

}  // namespace kernels
}  // namespace attn
