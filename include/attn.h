/*
 * attn.h -- C ABI of the MI355X (gfx950) fused attention forward library.
 *
 * The operation is the attention forward pass with per-row log-sum-exp,
 * computed block by block with a running row max and row sum so that the
 * Nq x Nk score matrix never reaches device memory:
 *
 *   S   = scale * Q K^T                       (per batch b and head h)
 *   P   = softmax(S) over keys, row by row    (causal: only allowed keys)
 *   O   = P V
 *   LSE = m + ln(sum_j exp(S_ij - m)),  m = max_j S_ij   (natural log)
 *
 * Source: "Warp specialization" concept card (wikillm), "Implementation
 * sketch": a block of queries with keys and values streamed from global
 * memory yields the output block and one log-sum-exp per row, returned as
 * (output / row_sum, row_max + log(row_sum)).  The FP8 E4M3 variant with
 * per-tensor scaling is section 5 of "Inside FlashAttention-3 &
 * Warp-Specialized CUDA Kernels" (tekromancy.com), and so is the
 * block-scaled variant with 16x16 Walsh-Hadamard smoothing of Q and K
 * (attn_quantize_fp8 + attn_fwd_fp8_blockscaled).  The pages describe one
 * key/value tile stream per (batch, head) of a (B, H, N, D) tensor.
 *
 * Layout (all tensors dense, row-major, innermost dimension contiguous):
 *   q   [B][H][Nq][d]     element type per `dtype`
 *   k   [B][H][Nk][d]     same type as q
 *   v   [B][H][Nk][d]     same type as q
 *   o   [B][H][Nq][d]     f16 for ATTN_F16 and ATTN_FP8_E4M3, bf16 for ATTN_BF16
 *   lse [B][H][Nq]        float32
 *
 * Causal masking keeps key j for query i iff j <= i + (Nk - Nq)
 * (bottom-right alignment; identical to j <= i when Nq == Nk).  A query row
 * that sees no key (causal with Nq > Nk) gets O = 0 and LSE = -inf.
 *
 * Ownership: every pointer is a DEVICE pointer allocated and owned by the
 * caller.  The library allocates nothing, keeps no mutable global state, and
 * is safe to call from several host threads.  o and lse must not overlap the
 * inputs or each other.
 *
 * Stream: the call validates its arguments on the host, enqueues the work on
 * `stream` (NULL = the default stream) and returns without synchronising.
 *
 * Errors: validation happens before anything touches the device; a rejected
 * call returns a negative ATTN_ERR_* code and enqueues nothing.  A failed
 * launch returns ATTN_ERR_LAUNCH.  Faults during execution surface on the
 * stream when the caller synchronises.  The library never aborts or prints.
 */
#ifndef ATTN_MI355X_ATTN_H
#define ATTN_MI355X_ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t. */
struct ihipStream_t;

/* Rows per quantisation block of the block-scaled FP8 variant: each
 * (batch, head) of a tensor is cut into blocks of this many consecutive rows
 * (the last one may be shorter), each with its own float32 descale. */
#define ATTN_FP8_BLOCK_ROWS 64

typedef enum {
  ATTN_F16 = 0,       /* IEEE binary16 in, binary16 out */
  ATTN_BF16 = 1,      /* bfloat16 in, bfloat16 out */
  ATTN_FP8_E4M3 = 2   /* OCP FP8 E4M3 ("fn") in, binary16 out */
} attn_dtype;

enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,     /* a required pointer is NULL */
  ATTN_ERR_SHAPE = -2,    /* B, H, Nq or Nk < 1, a tensor has >= 2^31 elements, or one
                             head's K (or V) block, Nk * d * element size, is >= 2^31 bytes */
  ATTN_ERR_HEADDIM = -3,  /* d not in {64, 128, 256} */
  ATTN_ERR_DTYPE = -4,    /* unknown dtype code */
  ATTN_ERR_ALIGN = -5,    /* q, k, v, o (x, codes) not 16-byte aligned, or lse (descales)
                             not 4-byte aligned */
  ATTN_ERR_SCALE = -6,    /* scale is not finite, or a descale is not finite and > 0 */
  ATTN_ERR_LAUNCH = -7,   /* the kernel launch failed */
  ATTN_ERR_ALIAS = -8,    /* an output overlaps an input or another output */
  ATTN_ERR_VARIANT = -9,  /* unknown kernel variant, or not built for this d and dtype */
  ATTN_ERR_WORKSPACE = -10, /* split-key workspace NULL, smaller than the shape needs, not
                              256-byte aligned, or overlapping an input or output */
  ATTN_ERR_SCRATCH = -11   /* the shape needs more than ATTN_SPLITKV_SCRATCH_BYTES of static
                              scratch, or the scratch's device address could not be found */
};

/* Size of the static device scratch of attn_fwd_splitkv_noalloc (one copy on
 * every device the library runs on, held until the process ends). */
#define ATTN_SPLITKV_SCRATCH_BYTES (64u << 20)

/* Kernel variants (attn_fwd_variant).  All compute the same result; they
 * differ in schedule, so their speed depends on the shape:
 *   AUTO               the library's measured default for the (d, dtype,
 *                      shape) -- what attn_fwd and attn_fwd_fp8 run
 *   PIPELINED          scores of the next key tile computed under the
 *                      softmax of the current one, 2-stage K/V ring
 *                      (d = 64, 128)
 *   PIPELINED_4STAGE   the same with a 4-stage ring and one workgroup
 *                      barrier per two key tiles (d = 64, 128)
 *   SEQUENTIAL         one key tile per step, no score pipelining (all d)
 *   SPLIT              two wave groups over the two halves of the key range,
 *                      merged at the end (16-bit d = 64)
 *   PINGPONG           two wave groups alternating matrix-only and
 *                      softmax-only halves of each step behind workgroup
 *                      barriers, so that one group's softmax runs under the
 *                      other's MFMAs (d = 128)
 *   PRODUCER           a ninth, producer wave streams K and V into a
 *                      2-stage ring; the eight consumer waves run the
 *                      sequential step on tiles already in LDS (d = 128)
 *   WIDE               64 query rows per wave (two 32-row blocks sharing
 *                      every K and V operand read), one wave per SIMD with
 *                      the output accumulators in AGPRs, pipelined steps
 *                      (16-bit d = 128)
 *   SEQUENTIAL_BC32    SEQUENTIAL with 32-key tiles (16-bit d = 64, 128)
 *   SEQUENTIAL_BC128   SEQUENTIAL with 128-key tiles: one row max,
 *                      reference update and barrier per 128 keys (d = 64,
 *                      128)
 *   PIPELINED_3STAGE   scores two key tiles ahead of P V, so each step
 *                      overlaps both matrix products with the softmax of
 *                      the tile between them (16-bit d = 64, 128) */
enum {
  ATTN_VARIANT_AUTO = 0,
  ATTN_VARIANT_PIPELINED = 1,
  ATTN_VARIANT_PIPELINED_4STAGE = 2,
  ATTN_VARIANT_SEQUENTIAL = 3,
  ATTN_VARIANT_SPLIT = 4,
  ATTN_VARIANT_PINGPONG = 5,
  ATTN_VARIANT_PRODUCER = 6,
  ATTN_VARIANT_WIDE = 7,
  ATTN_VARIANT_SEQUENTIAL_BC32 = 8,
  ATTN_VARIANT_SEQUENTIAL_BC128 = 9,
  ATTN_VARIANT_PIPELINED_3STAGE = 10
};

/*
 * attn_fwd: one fused attention forward over all B*H (batch, head) pairs.
 *
 * q, k, v  device inputs, layout above, element type `dtype`
 * o, lse   device outputs, layout above (every element is written)
 * B, H     batch size and heads (>= 1)
 * Nq, Nk   query and key counts (>= 1; need not be multiples of any tile;
 *          Nk * d * element size < 2^31 bytes)
 * d        head dimension: 64, 128 or 256
 * causal   0 = full attention, nonzero = bottom-right causal mask
 * scale    multiplies Q K^T before the softmax, e.g. 1/sqrt(d); any finite
 *          value: 0 gives the uniform average of the visible values, a
 *          negative scale favours the least similar keys
 * dtype    an attn_dtype; ATTN_FP8_E4M3 here means unit descales
 * stream   HIP stream to enqueue on (NULL = default stream)
 *
 * Returns ATTN_OK or a negative ATTN_ERR_* code.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Nq, int Nk, int d, int causal, float scale,
             int dtype, struct ihipStream_t* stream);

/*
 * attn_fwd_fp8: the FP8 E4M3 forward with per-tensor scaling ("Inside
 * FlashAttention-3", section 5).  The real value of each input element is
 * its E4M3 code times that tensor's descale.  Scores accumulate in fp32;
 * the probabilities are rounded to E4M3 for the P V product; O is binary16.
 * Arguments as attn_fwd, plus q_descale, k_descale, v_descale (finite, > 0);
 * scale * q_descale * k_descale must be finite.
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Nq, int Nk, int d, int causal, float scale,
                 float q_descale, float k_descale, float v_descale,
                 struct ihipStream_t* stream);

/*
 * attn_variant_available: 1 if `variant` is built for head dimension d and
 * `dtype` (an attn_dtype), else 0.  Host-only; touches no device.
 */
int attn_variant_available(int d, int dtype, int variant);

/*
 * attn_fwd_variant: attn_fwd / attn_fwd_fp8 with an explicit kernel
 * variant, for measuring which one suits a shape (tile and stage tuning).
 * Arguments as attn_fwd_fp8 (the descales are used only for ATTN_FP8_E4M3;
 * pass 1 otherwise), plus `variant` (an ATTN_VARIANT_* code).  Returns
 * ATTN_ERR_VARIANT, before touching the device, for a variant that
 * attn_variant_available rejects.
 */
int attn_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int Nq, int Nk, int d, int causal, float scale,
                     int dtype, float q_descale, float k_descale, float v_descale,
                     int variant, struct ihipStream_t* stream);

/*
 * attn_quantize_fp8: block-scaled FP8 E4M3 quantisation of one attention
 * input, optionally after a 16x16 Walsh-Hadamard transform ("Inside
 * FlashAttention-3", section 5, block scaling with Hadamard outlier
 * smoothing).  With `hadamard` nonzero every group of 16 consecutive
 * channels of a row is multiplied by H/4, H the Sylvester-ordered 16x16
 * Walsh-Hadamard matrix (entry (i, j) = (-1)^popcount(i & j)); H/4 is
 * orthogonal, so applying it to both Q and K leaves Q K^T unchanged.  Use
 * it for Q and K, never for V.
 *
 * Per block of ATTN_FP8_BLOCK_ROWS rows of one (batch, head), with y the
 * (transformed) values rounded once to float32:
 *   descale = amax|y| / 448 in IEEE float32 (1 if the block is all zero)
 *   code    = E4M3 round-to-nearest-even of (y / descale), float32 division
 * so that code * descale approximates y.
 *
 * x         device input [B][H][N][d], binary16 (ATTN_F16) or bfloat16
 *           (ATTN_BF16), finite values, 16-byte aligned
 * dtype     ATTN_F16 or ATTN_BF16
 * codes     device output [B][H][N][d] E4M3 codes, 16-byte aligned
 * descales  device output [B][H][ceil(N / ATTN_FP8_BLOCK_ROWS)] float32,
 *           4-byte aligned
 * B, H, N   >= 1; d is 64, 128 or 256; B*H*N*d < 2^31
 * hadamard  nonzero: transform before quantising
 * stream    HIP stream to enqueue on (NULL = default stream)
 *
 * codes and descales must not overlap x or each other (ATTN_ERR_ALIAS).
 * Returns ATTN_OK or a negative ATTN_ERR_* code, as attn_fwd.
 */
int attn_quantize_fp8(const void* x, int dtype, void* codes, float* descales,
                      int B, int H, int N, int d, int hadamard,
                      struct ihipStream_t* stream);

/*
 * attn_fwd_fp8_blockscaled: the FP8 E4M3 forward with one descale per block
 * of ATTN_FP8_BLOCK_ROWS rows, as attn_quantize_fp8 produces them.  The real
 * value of an element of q (k, v) in row r of head (b, h) is its code times
 * q_descales[(b*H + h)*nq + r / ATTN_FP8_BLOCK_ROWS] with nq = ceil(Nq /
 * ATTN_FP8_BLOCK_ROWS) (nk = ceil(Nk / ATTN_FP8_BLOCK_ROWS) for k and v).
 * If q and k were quantised after the Walsh-Hadamard transform, the scores,
 * and so O and LSE, are those of the untransformed inputs up to rounding.
 *
 * q, k, v          device E4M3 codes, layout above, 16-byte aligned
 * q_descales       device float32 [B][H][nq]; k_descales, v_descales
 *                  [B][H][nk]; 4-byte aligned; every value finite and > 0
 *                  (not checked: they live in device memory)
 * o, lse, B, H, Nq, Nk, d, causal, scale, stream: as attn_fwd; o is binary16
 *
 * o and lse must not overlap any input, descale array or each other.
 * Returns ATTN_OK or a negative ATTN_ERR_* code.
 */
int attn_fwd_fp8_blockscaled(const void* q, const void* k, const void* v,
                             const float* q_descales, const float* k_descales,
                             const float* v_descales, void* o, float* lse,
                             int B, int H, int Nq, int Nk, int d, int causal,
                             float scale, struct ihipStream_t* stream);

/*
 * attn_fwd_splitkv_workspace_bytes: device workspace, in bytes, that
 * attn_fwd_splitkv needs for this shape, causal flag and num_splits (0 =
 * the library's choice, which depends on causal): 0 when the shape is not
 * split, and 0 for invalid arguments (use attn_fwd_splitkv_num_splits to
 * tell them apart).  Host-only.
 */
unsigned long long attn_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int causal,
                                                    int dtype, int num_splits);

/*
 * attn_fwd_splitkv_num_splits: the number of key splits per query tile at
 * most that attn_fwd_splitkv uses for this shape, causal flag and
 * num_splits request (1 = no split), or 0 if d or dtype is not supported.
 * Host-only.
 */
int attn_fwd_splitkv_num_splits(int B, int H, int Nq, int Nk, int d, int causal, int dtype,
                                int num_splits);

/*
 * attn_fwd_splitkv: the same forward with the key range of each query tile
 * split over several workgroups, for grids that would not fill the GPU
 * (few query tiles, long key ranges, the heavy diagonal tiles of a causal
 * grid).  Each split produces a partial (unnormalised O, row max, row sum)
 * over its keys, and a second launch on the same stream merges the partials
 * of a query tile with the online-softmax rescale -- the row max and row sum
 * the concept card's implementation sketch returns ("Warp specialization",
 * implementation sketch: output / row_sum and row_max + log(row_sum)) are
 * exactly what two partial results need to combine.  The merge takes the
 * splits in a fixed order, so results are bitwise reproducible.
 *
 * Arguments as attn_fwd_variant without `variant`, plus:
 * num_splits       key splits per query tile at most; 0 = the library's
 *                  choice (grids of fewer query tiles than CUs only; as
 *                  many workgroups as fit the CUs in one round, or, with
 *                  causal masking, enough to fill them; at least two key
 *                  tiles per split); 1 = no split (one launch)
 * workspace        device memory of at least
 *                  attn_fwd_splitkv_workspace_bytes(...) bytes (0 when the
 *                  shape is not split; then it may be NULL), 256-byte
 *                  aligned, owned by the caller, no initial contents needed.
 *                  Calls that share one workspace must not overlap in time
 *                  (same stream, or synchronised).
 * workspace_bytes  its size
 *
 * Returns ATTN_ERR_WORKSPACE (before touching the device) for a missing,
 * misaligned, too small or overlapping workspace, else as attn_fwd.
 */
int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int Nq, int Nk, int d, int causal, float scale,
                     int dtype, float q_descale, float k_descale, float v_descale,
                     int num_splits, void* workspace, unsigned long long workspace_bytes,
                     struct ihipStream_t* stream);

/*
 * attn_fwd_splitkv_noalloc: attn_fwd_splitkv without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The partials live
 * in a static device array of ATTN_SPLITKV_SCRATCH_BYTES per device; the
 * call allocates nothing.  Same split plan, kernels and results (bitwise)
 * as attn_fwd_splitkv with the same num_splits.
 *
 * Arguments as attn_fwd_splitkv without workspace and workspace_bytes.  The
 * current device must be the one `stream` belongs to.
 *
 * Every call on one device shares that device's scratch: calls that overlap
 * in time on one device (different streams, or host threads) race and give
 * wrong results; serialise them.  Nothing in the scratch needs clearing.
 * Returns ATTN_ERR_SCRATCH, before touching the device, when the shape needs
 * more than ATTN_SPLITKV_SCRATCH_BYTES (attn_fwd_splitkv_workspace_bytes
 * gives the need; a smaller num_splits needs less), else as attn_fwd_splitkv.
 */
int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int Nq, int Nk, int d, int causal, float scale,
                             int dtype, float q_descale, float k_descale, float v_descale,
                             int num_splits, struct ihipStream_t* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* attn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_ATTN_H */
