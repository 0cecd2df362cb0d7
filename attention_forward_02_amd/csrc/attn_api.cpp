// C ABI of the fused attention forward library: argument validation and
// dispatch.  Declarations and the full contract are in include/attn.h.
#include <math.h>
#include <stdint.h>

#include "attn.h"
#include "attn_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Half-open byte ranges [a, a+na) and [b, b+nb) overlap.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool positive_finite(float x) { return isfinite(x) && x > 0.f; }

int validate(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
             int Nq, int Nk, int d, int dtype) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_HEADDIM;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3) return ATTN_ERR_DTYPE;
  const long long nq = (long long)B * H * Nq * d, nk = (long long)B * H * Nk * d;
  if (nq >= (1LL << 31) || nk >= (1LL << 31)) return ATTN_ERR_SHAPE;
  // The kernels address one head's K or V block through a buffer resource
  // with 32-bit byte offsets.
  const long long head_kv_bytes = (long long)Nk * d * (dtype == ATTN_FP8_E4M3 ? 1 : 2);
  if (head_kv_bytes >= (1LL << 31)) return ATTN_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return ATTN_ERR_ALIGN;
  const size_t in_elt = dtype == ATTN_FP8_E4M3 ? 1 : 2;
  const size_t qb = (size_t)nq * in_elt, kb = (size_t)nk * in_elt;
  const size_t ob = (size_t)nq * 2, lb = (size_t)B * H * Nq * sizeof(float);
  if (overlap(o, ob, q, qb) || overlap(o, ob, k, kb) || overlap(o, ob, v, kb) || overlap(o, ob, lse, lb) ||
      overlap(lse, lb, q, qb) || overlap(lse, lb, k, kb) || overlap(lse, lb, v, kb))
    return ATTN_ERR_ALIAS;
  return ATTN_OK;
}

bool variant_available(int d, int dtype, int variant) {
  const bool d_ok = d == 64 || d == 128 || d == 256;
  const bool t_ok = dtype == ATTN_F16 || dtype == ATTN_BF16 || dtype == ATTN_FP8_E4M3;
  if (!d_ok || !t_ok) return false;
  switch (variant) {
    case ATTN_VARIANT_AUTO:
    case ATTN_VARIANT_SEQUENTIAL:
      return true;
    case ATTN_VARIANT_PIPELINED:
    case ATTN_VARIANT_PIPELINED_4STAGE:
      return d != 256;
    case ATTN_VARIANT_SPLIT:
      return d == 64 && dtype != ATTN_FP8_E4M3;
    case ATTN_VARIANT_PINGPONG:
      return d == 128;
    case ATTN_VARIANT_PRODUCER:
      return d == 128;
    case ATTN_VARIANT_WIDE:
      return d == 128 && dtype != ATTN_FP8_E4M3;
    case ATTN_VARIANT_SEQUENTIAL_BC32:
      return dtype != ATTN_FP8_E4M3 && d != 256;
    case ATTN_VARIANT_SEQUENTIAL_BC128:
      return d != 256;
    case ATTN_VARIANT_PIPELINED_3STAGE:
      return dtype != ATTN_FP8_E4M3 && d != 256;
    default:
      return false;
  }
}

// Scale and descales of a per-tensor call: the scale any finite value, the
// descales finite and > 0, their product finite.
int check_scales(float scale, float q_ds, float k_ds, float v_ds) {
  if (!isfinite(scale) || !positive_finite(q_ds) || !positive_finite(k_ds) || !positive_finite(v_ds))
    return ATTN_ERR_SCALE;
  if (!isfinite(scale * q_ds * k_ds)) return ATTN_ERR_SCALE;
  return ATTN_OK;
}

attn::Problem make_problem(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                           int Nk, int d, int causal, float scale, int dtype, float q_ds, float k_ds, float v_ds,
                           int variant) {
  attn::Problem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.d = d;
  p.causal = causal != 0;
  p.dtype = dtype;
  p.scale = scale * q_ds * k_ds;
  p.v_descale = v_ds;
  p.q_descales = p.k_descales = p.v_descales = nullptr;
  p.variant = variant;
  p.num_splits = 0;
  p.workspace = nullptr;
  p.workspace_bytes = 0;
  return p;
}

int run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int d,
        int causal, float scale, int dtype, float q_ds, float k_ds, float v_ds, int variant, ihipStream_t* stream) {
  int st = validate(q, k, v, o, lse, B, H, Nq, Nk, d, dtype);
  if (st != ATTN_OK) return st;
  if (!variant_available(d, dtype, variant)) return ATTN_ERR_VARIANT;
  st = check_scales(scale, q_ds, k_ds, v_ds);
  if (st != ATTN_OK) return st;
  const attn::Problem p = make_problem(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, q_ds, k_ds, v_ds,
                                       variant);
  return attn::launch_forward(p, (hipStream_t)stream);
}

bool splitkv_args_ok(int B, int H, int Nq, int Nk, int d, int dtype, int num_splits) {
  return B >= 1 && H >= 1 && Nq >= 1 && Nk >= 1 && num_splits >= 0 && (d == 64 || d == 128 || d == 256) &&
         (dtype == ATTN_F16 || dtype == ATTN_BF16 || dtype == ATTN_FP8_E4M3);
}

// The split-key forward on a caller's workspace (attn_fwd_splitkv).
int run_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                int d, int causal, float scale, int dtype, float q_ds, float k_ds, float v_ds, int num_splits,
                void* ws, size_t ws_bytes, ihipStream_t* stream) {
  int st = validate(q, k, v, o, lse, B, H, Nq, Nk, d, dtype);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_FP8_E4M3) q_ds = k_ds = v_ds = 1.f;
  st = check_scales(scale, q_ds, k_ds, v_ds);
  if (st != ATTN_OK) return st;
  if (num_splits < 0) return ATTN_ERR_SHAPE;
  const size_t need = attn::splitkv_workspace_bytes(B, H, Nq, Nk, d, causal, dtype, num_splits);
  if (need > 0) {
    if (!ws || !aligned(ws, 256) || ws_bytes < need) return ATTN_ERR_WORKSPACE;
    const size_t in_elt = dtype == ATTN_FP8_E4M3 ? 1 : 2;
    const size_t qb = (size_t)B * H * Nq * d * in_elt, kb = (size_t)B * H * Nk * d * in_elt;
    const size_t ob = (size_t)B * H * Nq * d * 2, lb = (size_t)B * H * Nq * sizeof(float);
    if (overlap(ws, need, q, qb) || overlap(ws, need, k, kb) || overlap(ws, need, v, kb) ||
        overlap(ws, need, o, ob) || overlap(ws, need, lse, lb))
      return ATTN_ERR_WORKSPACE;
  }
  attn::Problem p = make_problem(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, q_ds, k_ds, v_ds,
                                 ATTN_VARIANT_AUTO);
  p.num_splits = num_splits;
  p.workspace = ws;
  p.workspace_bytes = ws_bytes;
  return attn::launch_splitkv(p, (hipStream_t)stream);
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
             int d, int causal, float scale, int dtype, ihipStream_t* stream) {
  return run(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, 1.f, 1.f, 1.f, ATTN_VARIANT_AUTO, stream);
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                 int Nk, int d, int causal, float scale, float q_descale, float k_descale, float v_descale,
                 ihipStream_t* stream) {
  return run(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, ATTN_FP8_E4M3, q_descale, k_descale, v_descale,
             ATTN_VARIANT_AUTO, stream);
}

int attn_variant_available(int d, int dtype, int variant) { return variant_available(d, dtype, variant) ? 1 : 0; }

int attn_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                     int d, int causal, float scale, int dtype, float q_descale, float k_descale, float v_descale,
                     int variant, ihipStream_t* stream) {
  if (dtype != ATTN_FP8_E4M3) q_descale = k_descale = v_descale = 1.f;
  return run(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, q_descale, k_descale, v_descale, variant,
             stream);
}

int attn_quantize_fp8(const void* x, int dtype, void* codes, float* descales, int B, int H, int N, int d,
                      int hadamard, ihipStream_t* stream) {
  if (!x || !codes || !descales) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_HEADDIM;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  const long long n = (long long)B * H * N * d;
  if (n >= (1LL << 31)) return ATTN_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(descales, 4)) return ATTN_ERR_ALIGN;
  const size_t xb = (size_t)n * 2, cb = (size_t)n;
  const size_t db = (size_t)B * H * ((N + ATTN_FP8_BLOCK_ROWS - 1) / ATTN_FP8_BLOCK_ROWS) * sizeof(float);
  if (overlap(codes, cb, x, xb) || overlap(descales, db, x, xb) || overlap(descales, db, codes, cb))
    return ATTN_ERR_ALIAS;
  attn::QuantProblem p;
  p.x = x;
  p.codes = codes;
  p.descales = descales;
  p.B = B;
  p.H = H;
  p.N = N;
  p.d = d;
  p.dtype = dtype;
  p.hadamard = hadamard != 0;
  return attn::launch_quantize(p, (hipStream_t)stream);
}

int attn_fwd_fp8_blockscaled(const void* q, const void* k, const void* v, const float* q_descales,
                             const float* k_descales, const float* v_descales, void* o, float* lse, int B, int H,
                             int Nq, int Nk, int d, int causal, float scale, ihipStream_t* stream) {
  int st = validate(q, k, v, o, lse, B, H, Nq, Nk, d, ATTN_FP8_E4M3);
  if (st != ATTN_OK) return st;
  if (!q_descales || !k_descales || !v_descales) return ATTN_ERR_NULL;
  if (!aligned(q_descales, 4) || !aligned(k_descales, 4) || !aligned(v_descales, 4)) return ATTN_ERR_ALIGN;
  const size_t ob = (size_t)B * H * Nq * d * 2, lb = (size_t)B * H * Nq * sizeof(float);
  const size_t qdb = (size_t)B * H * ((Nq + ATTN_FP8_BLOCK_ROWS - 1) / ATTN_FP8_BLOCK_ROWS) * sizeof(float);
  const size_t kdb = (size_t)B * H * ((Nk + ATTN_FP8_BLOCK_ROWS - 1) / ATTN_FP8_BLOCK_ROWS) * sizeof(float);
  const void* ds[3] = {q_descales, k_descales, v_descales};
  const size_t dsb[3] = {qdb, kdb, kdb};
  for (int i = 0; i < 3; ++i)
    if (overlap(o, ob, ds[i], dsb[i]) || overlap(lse, lb, ds[i], dsb[i])) return ATTN_ERR_ALIAS;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  attn::Problem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.d = d;
  p.causal = causal != 0;
  p.dtype = ATTN_FP8_E4M3;
  p.scale = scale;
  p.v_descale = 1.f;
  p.q_descales = q_descales;
  p.k_descales = k_descales;
  p.v_descales = v_descales;
  p.variant = ATTN_VARIANT_AUTO;
  p.num_splits = 0;
  p.workspace = nullptr;
  p.workspace_bytes = 0;
  return attn::launch_forward(p, (hipStream_t)stream);
}

unsigned long long attn_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int causal, int dtype,
                                                    int num_splits) {
  if (!splitkv_args_ok(B, H, Nq, Nk, d, dtype, num_splits)) return 0;
  return attn::splitkv_workspace_bytes(B, H, Nq, Nk, d, causal, dtype, num_splits);
}

int attn_fwd_splitkv_num_splits(int B, int H, int Nq, int Nk, int d, int causal, int dtype, int num_splits) {
  if (!splitkv_args_ok(B, H, Nq, Nk, d, dtype, num_splits)) return 0;
  return attn::splitkv_splits(B, H, Nq, Nk, d, causal, dtype, num_splits);
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                     int d, int causal, float scale, int dtype, float q_descale, float k_descale, float v_descale,
                     int num_splits, void* workspace, unsigned long long workspace_bytes, ihipStream_t* stream) {
  return run_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, q_descale, k_descale, v_descale,
                     num_splits, workspace, (size_t)workspace_bytes, stream);
}

int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                             int Nk, int d, int causal, float scale, int dtype, float q_descale, float k_descale,
                             float v_descale, int num_splits, ihipStream_t* stream) {
  int st = validate(q, k, v, o, lse, B, H, Nq, Nk, d, dtype);
  if (st != ATTN_OK) return st;
  if (num_splits < 0) return ATTN_ERR_SHAPE;
  const size_t need = attn::splitkv_workspace_bytes(B, H, Nq, Nk, d, causal, dtype, num_splits);
  if (need > (size_t)ATTN_SPLITKV_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    st = attn::splitkv_scratch(&ws);
    if (st != ATTN_OK) return st;
  }
  return run_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, q_descale, k_descale, v_descale,
                     num_splits, ws, (size_t)ATTN_SPLITKV_SCRATCH_BYTES, stream);
}

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE:
      return "B, H, Nq and Nk must be >= 1, each tensor < 2^31 elements and one head's K or V < 2^31 bytes";
    case ATTN_ERR_HEADDIM: return "head dimension must be 64, 128 or 256";
    case ATTN_ERR_DTYPE: return "unknown dtype";
    case ATTN_ERR_ALIGN:
      return "q, k, v, o (x, codes) must be 16-byte aligned and lse (descales) 4-byte aligned";
    case ATTN_ERR_SCALE: return "scale must be finite, and descales finite and > 0";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_ALIAS: return "an output overlaps an input or another output";
    case ATTN_ERR_VARIANT: return "unknown kernel variant, or not built for this head dim and dtype";
    case ATTN_ERR_SCRATCH:
      return "the shape needs more than ATTN_SPLITKV_SCRATCH_BYTES of static split-key scratch (use fewer "
             "splits), or the scratch's device address could not be found";
    case ATTN_ERR_WORKSPACE:
      return "split-key workspace is NULL, smaller than the shape needs, not 256-byte aligned or overlapping "
             "an input or output";
    default: return "unknown status";
  }
}

}  // extern "C"
