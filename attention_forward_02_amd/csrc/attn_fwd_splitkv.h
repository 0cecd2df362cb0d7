#pragma once
// Split-key forward: the key range of every query tile is cut into up to S
// splits, each run by its own workgroup, so a grid of few query tiles (or a
// causal grid whose heaviest tiles dominate) spreads its key loops over the
// chip.  Each split walks its key tiles with the sequential step of
// attn_fwd_kernel.h and ends with a partial result (O, m, l): the unnormalised
// output, the base-2 reference max and the row sum over its keys.  Partials
// combine exactly as consecutive key tiles do in the online softmax of the
// concept card's implementation sketch: with m = max_r m_r and weights
// w_r = 2^(m_r - m),
//   O = sum_r w_r O_r,  l = sum_r w_r l_r,  output O / l,  LSE = m + log2 l
// (natural log after the ln 2 conversion); the log-sum-exp the sketch
// returns is what makes this merge possible.
//
// Two launches, in stream order.  The split kernel runs every (query tile,
// split) workgroup; a query tile whose key range fits one split stores O and
// LSE directly, the others write their partial to the workspace.  The merge
// kernel then reads the partials of each split query tile, combines them in
// split order (so results are bitwise reproducible) and stores O and LSE.
// The kernel boundary makes the partials visible to the merge, so the split
// kernel needs no device-wide fences: on this chip a device-scope release
// writes back a whole L2 (measured: a 2-way split of one 128-row tile cost
// 3.9 us of fences and atomics, a 4-way split of B=4 H=8 N=1024 d=64 causal
// 100 us, against 2-3 us for the second launch).
//
// Workspace layout: partials per (query tile, split, wave), PartWords x 64
// floats each: the O^T accumulators as [32-column block][group of 4][lane]
// float4 (a wave's 64 lanes access 1 KB contiguously), then m2 and l as
// [lane] floats.  Nothing in it needs initialising.
#include "attn_fwd_kernel.h"

namespace attn {
namespace kernels {

// Floats per lane of one wave's partial: O^T accumulators, m2, l.
template <int D>
struct PartWords {
  static constexpr int value = D / 32 * 16 + 2;
};

// Workgroups of 4-wave kernels that share a CU (d = 64: up to four), used
// to decide how far to split.
template <int D, int DT>
struct SplitSlotsPerCU {
  static constexpr int value = Waves<D, DT>::value == 4 ? 4 : 1;
};

constexpr int kSplitMaxSplits = 32;
constexpr int kSplitMinTiles = 2;  // key tiles per split at least (auto choice)
constexpr int kSplitTwoMinKeys = 2048;  // keys a two-way split needs (auto choice)
constexpr int kCUs = 256;

// How a shape is split.  items = B * H * query tiles; nsplit = splits per
// query tile at most; tiles = key tiles per split at most.
struct SplitPlan {
  long long items;
  int nsplit, tiles;
  size_t bytes;  // workspace bytes
};

__host__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int D, int DT>
__host__ inline SplitPlan split_plan(int B, int H, int Nq, int Nk, bool causal, int num_splits) {
  constexpr int kRows = Waves<D, DT>::value * kRowsPerWave;
  constexpr int BN = TileKeys<D, DT>::value;
  SplitPlan sp;
  sp.items = (long long)B * H * ((Nq + kRows - 1) / kRows);
  const int nt_max = (Nk + BN - 1) / BN;
  int s = num_splits;
  if (s <= 0) {
    // auto: split only grids of fewer query tiles than CUs.  Without causal
    // masking, into as many workgroups as fit every CU's slots in one round
    // (more would run a second round of equal-length loops: two splits of
    // 192 tiles measured up to 1.5x slower); with it, into enough to fill
    // them (the diagonal tiles' long loops dominate: three splits of 96
    // causal tiles measured 13-29% faster than two).  At least
    // kSplitMinTiles key tiles per split.  (A grid with a tile per CU is not
    // helped: at B=4 H=8 N=1024 d=64 causal, four splits measured 17.8 us
    // in the split kernel alone against 17.5 us unsplit -- the per-split Q
    // and K/V loads and partial writes cost what the shorter key loops
    // save.)
    const long long slots = (long long)kCUs * SplitSlotsPerCU<D, DT>::value;
    if (sp.items >= kCUs) s = 1;
    else if (causal) s = (int)((slots + sp.items - 1) / sp.items);
    else s = (int)(slots / sp.items);
    const int most = nt_max / kSplitMinTiles > 1 ? nt_max / kSplitMinTiles : 1;
    if (s > most) s = most;
    // A two-way split of equal-length key loops pays for its merge only on
    // long key ranges.
    if (!causal && s == 2 && Nk < kSplitTwoMinKeys) s = 1;
  }
  if (s > kSplitMaxSplits) s = kSplitMaxSplits;
  if (s > nt_max) s = nt_max;
  if (s < 1) s = 1;
  sp.tiles = (nt_max + s - 1) / s;
  sp.nsplit = (nt_max + sp.tiles - 1) / sp.tiles;
  sp.bytes = 0;
  if (sp.nsplit > 1)
    sp.bytes = (size_t)sp.items * sp.nsplit * Waves<D, DT>::value * PartWords<D>::value * 64 * sizeof(float);
  return sp;
}

template <int D, int DT, bool CAUSAL>
__global__ void __launch_bounds__(64 * (Waves<D, DT>::value)) __attribute__((amdgpu_waves_per_eu(2)))
attn_fwd_splitkv_kernel(Params p) {
  constexpr int kWaves = Waves<D, DT>::value;
  constexpr int kBlockM = kWaves * kRowsPerWave;
  constexpr int kRowBytes = D * Fmt<DT>::kBytes;
  constexpr int BN = TileKeys<D, DT>::value;
  constexpr int kTileBytes = BN * kRowBytes;
  constexpr int kPart = PartWords<D>::value;
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

  // Workgroup -> (query tile item, split).  Workgroups reach the 8 XCDs
  // round-robin; all splits of an item go to one XCD (the item's partials
  // then meet in that XCD's L2), and the items of an XCD are those of the
  // heads congruent to it mod 8, heaviest query tiles first.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int m8 = slot / p.nsplit, s = slot - m8 * p.nsplit;
  const int item = xcd + 8 * m8;
  if (item >= p.total_tiles) return;
  const int BH = p.total_tiles / p.n_qtiles;
  const int bh = item % BH;
  int qt = item / BH;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;
  const int q0 = qt * kBlockM;
  int kend = p.Nk;
  if (CAUSAL) kend = min(p.Nk, q0 + kBlockM + (p.Nk - p.Nq));
  const int nt = kend > 0 ? (kend + BN - 1) / BN : 0;
  const int ns = max(1, (nt + p.split_tiles - 1) / p.split_tiles);  // splits of this item
  if (s >= ns) return;
  const int t0 = (int)((long long)s * nt / ns), t1 = (int)((long long)(s + 1) * nt / ns);

  LoopCtxT<BN> cx;
  cx.qw0 = q0 + wave * kRowsPerWave;
  cx.qrow = cx.qw0 + (lane & 31);
  cx.diag = p.Nk - p.Nq;
  cx.Nk = p.Nk;
  cx.half = lane >> 5;
  cx.c = p.c;
  cx.wave_kend = CAUSAL ? cx.qw0 + kRowsPerWave - 1 + cx.diag : p.Nk;
  cx.nt = nt;

  const uint32_t head_bytes = (uint32_t)p.Nk * kRowBytes;
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc(p.k + (size_t)bh * p.Nk * kRowBytes, head_bytes);
  const __amdgpu_buffer_rsrc_t Vr = make_rsrc(p.v + (size_t)bh * p.Nk * kRowBytes, head_bytes);
  TileLoader<D, DT, kWaves, BN> ld;
  ld.init(wave, lane);
  WaveState<D, DT> st;
  st.init(p.q + (size_t)bh * p.Nq * kRowBytes, cx.qrow, p.Nq, lane, p.q_and, p.q_xor);

  if (t1 > t0) {
    ld.load(K0, Kr, t0 * BN);
    ld.load(V0, Vr, t0 * BN);
  }
  // Tiles before tb need no mask bias: pairs of unmasked steps while both
  // tiles lie before tb, then masked steps (one step variant per loop).
  const int tb = min(first_bias_tile<CAUSAL>(cx), nt);
  const TileScale ts{};
  auto step = [&](int j, const lds_t* Kc, const lds_t* Vc, lds_t* Kl, lds_t* Vl, auto masked) {
    constexpr bool M = decltype(masked)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < t1) {
      ld.load(Kl, Kr, (j + 1) * BN);
      ld.load(Vl, Vr, (j + 1) * BN);
    }
    seq_step<D, DT, CAUSAL, M, BN, false>(st, cx, j, Kc, Vc, ts);
  };
  const int jm = t0 + (max(min(tb, t1) - t0, 0) & ~1);
  int j = t0;
  for (; j < jm; j += 2) {
    step(j, K0, V0, K1, V1, BoolTag<false>{});
    step(j + 1, K1, V1, K0, V0, BoolTag<false>{});
  }
  for (; j < t1; j += 2) {
    step(j, K0, V0, K1, V1, BoolTag<true>{});
    if (j + 1 >= t1) break;
    step(j + 1, K1, V1, K0, V0, BoolTag<true>{});
  }
  if (ns == 1) {
    store_output<D, DT>(p, st, bh, cx.qrow, cx.half);
    return;
  }

  // Partial of this split: (item, s, wave).
  const size_t wave_words = (size_t)kPart * 64;
  float* const mine = p.part + (((size_t)item * p.nsplit + s) * kWaves + wave) * wave_words;
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(f32x4*)(mine + ((4 * i + g) * 64 + lane) * 4) =
          f32x4{st.oacc[i][4 * g], st.oacc[i][4 * g + 1], st.oacc[i][4 * g + 2], st.oacc[i][4 * g + 3]};
  mine[(kPart - 2) * 64 + lane] = st.m2;
  mine[(kPart - 1) * 64 + lane] = st.lrun;
}

// Merge of the split query tiles: one single-wave workgroup per (query tile
// item, wave of the split kernel's workgroup, 32-column block of O), i.e.
// per 32 query rows x 32 columns, so that the merge of a few long query
// tiles still spreads over the chip.
template <int D, int DT, bool CAUSAL>
__global__ void __launch_bounds__(64) attn_splitkv_merge_kernel(Params p) {
  constexpr int kWaves = Waves<D, DT>::value;
  constexpr int kBlockM = kWaves * kRowsPerWave;
  constexpr int BN = TileKeys<D, DT>::value;
  constexpr int kPart = PartWords<D>::value;
  constexpr int NB = D / 32;
  const int lane = threadIdx.x;
  const int blk = blockIdx.x % NB, iw = blockIdx.x / NB;
  const int item = iw / kWaves, wave = iw - item * kWaves;
  const int BH = p.total_tiles / p.n_qtiles;
  const int bh = item % BH;
  int qt = item / BH;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;
  const int q0 = qt * kBlockM;
  int kend = p.Nk;
  if (CAUSAL) kend = min(p.Nk, q0 + kBlockM + (p.Nk - p.Nq));
  const int nt = kend > 0 ? (kend + BN - 1) / BN : 0;
  const int ns = max(1, (nt + p.split_tiles - 1) / p.split_tiles);
  if (ns == 1) return;  // stored by the split kernel
  const int qrow = q0 + wave * kRowsPerWave + (lane & 31), half = lane >> 5;

  const size_t split_words = (size_t)kWaves * kPart * 64;
  const float* const base = p.part + ((size_t)item * p.nsplit * kWaves + wave) * kPart * 64;
  // In split order: the common reference, the row sum, then this block of O.
  float m = -__builtin_inff();
#pragma unroll 4
  for (int r = 0; r < ns; ++r) m = fmaxf(m, base[r * split_words + (kPart - 2) * 64 + lane]);
  auto weight = [&](int r) {
    const float mr = base[r * split_words + (kPart - 2) * 64 + lane];
    return mr == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mr - m);
  };
  float l = 0.f;
  f32x4 acc[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};
#pragma unroll 2
  for (int r = 0; r < ns; ++r) {
    const float w = weight(r);
    const float* pr = base + r * split_words;
    l = __builtin_fmaf(w, pr[(kPart - 1) * 64 + lane], l);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 x = *(const f32x4*)(pr + ((4 * blk + g) * 64 + lane) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[g][e] = __builtin_fmaf(w, x[e], acc[g][e]);
    }
  }
  const float ltot = swap_halves_sum(l);
  const bool has_key = ltot > 0.f;
  const float inv = has_key ? p.o_scale / ltot : 0.f;
  if (qrow >= p.Nq) return;
  const size_t row = (size_t)bh * p.Nq + qrow;
  if (half == 0 && blk == 0) p.lse[row] = has_key ? (m + __builtin_amdgcn_logf(ltot)) * kLn2 : -__builtin_inff();
  uint16_t* orow = p.o + row * D;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    u32x2 o2;
    o2[0] = pack16<DT>(acc[g][0] * inv, acc[g][1] * inv);
    o2[1] = pack16<DT>(acc[g][2] * inv, acc[g][3] * inv);
    *(u32x2*)(orow + 32 * blk + 8 * g + 4 * half) = o2;
  }
}

template <int D, int DT, bool CAUSAL>
int launch_splitkv_one(const Problem& pr, hipStream_t stream) {
  constexpr int kWaves = Waves<D, DT>::value;
  constexpr int kBlockM = kWaves * kRowsPerWave;
  const SplitPlan sp = split_plan<D, DT>(pr.B, pr.H, pr.Nq, pr.Nk, pr.causal != 0, pr.num_splits);
  if (sp.bytes > pr.workspace_bytes || (sp.bytes > 0 && !pr.workspace)) return ATTN_ERR_WORKSPACE;
  const long long grid = 8LL * ((sp.items + 7) / 8) * sp.nsplit;
  if (sp.items > 0x7fffffffLL || grid > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  Params p;
  p.q = (const unsigned char*)pr.q;
  p.k = (const unsigned char*)pr.k;
  p.v = (const unsigned char*)pr.v;
  p.o = (uint16_t*)pr.o;
  p.lse = pr.lse;
  p.Nq = pr.Nq;
  p.Nk = pr.Nk;
  p.n_qtiles = (pr.Nq + kBlockM - 1) / kBlockM;
  p.total_tiles = (int)sp.items;
  set_scale(p, pr.scale, DT);
  p.o_scale = pr.v_descale;
  p.qs = p.ks = p.vs = nullptr;
  p.nqb = p.nkb = 0;
  p.part = (float*)pr.workspace;
  p.nsplit = sp.nsplit;
  p.split_tiles = sp.tiles;
  hipLaunchKernelGGL((attn_fwd_splitkv_kernel<D, DT, CAUSAL>), dim3((unsigned)grid), dim3(64 * kWaves), 0, stream,
                     p);
  if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
  if (sp.nsplit > 1) {
    const long long mgrid = sp.items * kWaves * (D / 32);
    if (mgrid > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    hipLaunchKernelGGL((attn_splitkv_merge_kernel<D, DT, CAUSAL>), dim3((unsigned)mgrid), dim3(64), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

}  // namespace kernels
}  // namespace attn
