/*
 * bfz.h -- C ABI of the block-wise FP8 ZeRO-1 shard step on MI355X (gfx950).
 *
 * One data-parallel rank owns a contiguous run of whole 128x128 weight tiles
 * (the block-wise split of "A ZeRO Optimizer Design for Blockwise FP8
 * Quantization", section "Block-wise split").  Per optimizer step it
 *   1. folds its row-major FP32 gradients into tile-major order (pack_shard;
 *      the fold of section "Parameter layout transform"),
 *   2. runs AdamW on the FP32 master weights and moments of those tiles and
 *      re-quantizes every updated tile to E4M3 with one scale per tile,
 *      scale_inv = amax / 448 (adamw_fp8_step; the update and quantization
 *      steps of section "Summary", the AdamW of section 4.3 of the lpnh.cn
 *      optimizer-state quantization essay, the per-tile scale and quantizer
 *      of "FP8-Flow-MoE", section 3.1),
 *   3. unfolds the codes and scales back to row-major FP8 weights and the
 *      row-major scale grid (unpack_fp8; the unfold of "Parameter layout
 *      transform" and "Summary").
 * fold_adamw_fp8_step does 1 and 2 in one pass, reading the gradients
 * straight from their row-major weights; fold_adamw_fp8_step_unpack does
 * 1, 2 and 3 in one pass.
 *
 * Conventions shared by every call:
 *   - A tile is 16384 contiguous elements: 128 rows of 128, row-major.
 *     A shard is q tiles back to back (q = bfz_plan_shard_tiles), except
 *     the FP32 optimizer state (master, m, v), whose tiles may sit a stride
 *     apart (bfz_step_options.state_stride; e.g. one [master | m | v] block
 *     per tile) -- same values, same order, other addresses.
 *   - Device pointers are caller-owned (the library never frees them); the
 *     library allocates only the plan's small device table, in
 *     bfz_plan_create (or bfz_plan_upload), freed by bfz_plan_destroy.
 *   - pack_shard(_strided), adamw_fp8_step, fold_adamw_fp8_step,
 *     fold_adamw_fp8_step_unpack and unpack_fp8 are asynchronous on the HIP
 *     stream passed as `stream` (NULL = the null stream): they only enqueue
 *     kernels, never allocate, never synchronize.
 *   - Return value: 0 on success, else a negative BFZ_E* code; the message
 *     for the calling thread's last failure is bfz_last_error().
 *   - Non-finite inputs (NaN, Inf) give unspecified results.
 */
#ifndef BFZ_H
#define BFZ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BFZ_TILE_DIM 128
#define BFZ_TILE_ELEMS 16384
/* The interleaved state layout's tile stride, in floats (see
 * bfz_step_options.state_stride): one [master | m | v] block per tile
 * (49152 floats) and a 1024-float (4 KiB) gap after it. */
#define BFZ_STATE_STRIDE_INTERLEAVED 50176

#define BFZ_OK 0
#define BFZ_EINVAL (-1) /* null pointer, bad size or shape, bad hyper-parameter */
#define BFZ_EALIGN (-2) /* a pointer lacks its required alignment */
#define BFZ_EHIP (-3)   /* a HIP runtime call or kernel launch failed */
#define BFZ_ESTATE (-4) /* plan has no device table, or its table is on another device than the current one */

/* The block-wise split of one rank: the lookup table of its tiles. */
typedef struct bfz_plan bfz_plan;

/* AdamW hyper-parameters of one step (the update of section 4.3 of the
 * lpnh.cn optimizer-state quantization essay).  step is the counter t >= 1
 * of the step being taken (the first step is t = 1).  Requires lr and
 * weight_decay finite, eps finite and > 0 (eps is the denominator's floor:
 * with eps = 0 an all-zero slot would compute 0 / 0), 0 <= beta1 < 1,
 * 0 <= beta2 < 1.  48 bytes; every step call reads exactly this struct. */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    int64_t step;
} bfz_adamw;

/* Options of a step beyond the hyper-parameters, taken by the _ex and fold
 * entry points (a NULL pointer means every field 0, the defaults).
 * scale_pow2 = 0: scale_inv = amax / 448.  scale_pow2 != 0: scale_inv is
 * the smallest power of two 2^T with 448 * 2^T >= amax (T >= -149), so
 * every quotient p / scale_inv is exact and codes can later be moved
 * between scales by exponent edits alone ("FP8-Flow-MoE", section 3.1;
 * see bfz_transpose_pow2).
 * state_stride: floats from tile s to tile s + 1 in each of master, m and
 * v (the FP32 state of the shard).  0 means 16384: three separate
 * tile-major arrays.  Otherwise a multiple of 4 in [16384, 2^26]; the
 * three arrays' tiles must not overlap one another.  With m = master +
 * 16384 and v = master + 32768 the state is interleaved: one contiguous
 * 192 KiB block [master | m | v] per tile, so each tile's updated state
 * leaves as a single write stream (on MI355X the one-kernel step is
 * 2.5% faster than with three separate arrays).  Strides above 49152
 * leave gaps between the blocks, which are never read or written; a
 * 4 KiB gap (BFZ_STATE_STRIDE_INTERLEAVED = 50176) staggers the blocks'
 * start addresses and measured another 0.8-1.5% faster than blocks back
 * to back (49152).  The gradient, codes and scale_inv keep their
 * tile-major layout whatever this value.
 * reserved must be 0 (BFZ_EINVAL otherwise). */
typedef struct {
    int32_t scale_pow2;
    int32_t reserved;
    int64_t state_stride;
} bfz_step_options;

/*
 * Build rank `rank`'s block-wise split of n_params weights.
 * dims: host array of n_params triples {E, H, W}: weight p is a row-major
 * FP32 tensor of E experts of H x W (E = 1 for a plain matrix), all >= 1.
 * Every weight is cut into ceil(H/128) x ceil(W/128) tiles per expert, the
 * last row / column of tiles zero-padded.  Tiles are numbered through all
 * weights in the order given, and within a weight by (expert, tile row,
 * tile column) -- the fold order.  With T tiles in all, every rank gets the
 * same quota q = ceil(T / D) and rank r owns global tiles
 * [r q, min((r + 1) q, T)); a shorter shard ends in all-zero padding slots
 * so that every shard is q tiles (section "Block-wise split" pads buckets to
 * the largest one; the contiguous equal quota is this library's reading of
 * how the page deals tiles to ranks).
 * The table is built on the host and, when the process sees a HIP device,
 * copied to the current device (about 28 bytes per tile, allocated here and
 * freed by bfz_plan_destroy; synchronous).  Every call that takes the plan
 * then needs that device to be current.  On a host with no HIP device the
 * plan is host-only: the queries below work, the device calls return
 * BFZ_ESTATE.
 * On success *out receives a new plan.  Errors: BFZ_EINVAL for null
 * pointers, n_params < 1, D < 1, rank outside [0, D), a dimension < 1,
 * H, W > 2^31 - 1, a weight of more than 2^31 - 1 tiles, a quota q of more
 * than 2^31 - 1 tiles, or too little host memory for the table (80 bytes
 * per slot); BFZ_EHIP if the device copy fails.
 */
int bfz_plan_create(const int64_t* dims, int32_t n_params, int32_t D, int32_t rank,
                    bfz_plan** out);

/* Copy the plan's tile table to the current HIP device if it has no device
 * copy yet (a plan created while no device was visible).  A plan whose table
 * is already on the current device is left as it is (bfz_plan_create has
 * usually done the upload); one whose table is on another device gives
 * BFZ_EINVAL.  Errors: BFZ_EINVAL, BFZ_EHIP. */
int bfz_plan_upload(bfz_plan* plan);

/* Free the plan and its device table.  NULL is accepted. */
void bfz_plan_destroy(bfz_plan* plan);

/* q: slots in the shard (owned tiles plus padding slots). */
int64_t bfz_plan_shard_tiles(const bfz_plan* plan);
/* Tiles the rank actually owns (<= q); slots [owned, q) are padding. */
int64_t bfz_plan_owned_tiles(const bfz_plan* plan);
/* T: tiles of all weights, over all ranks. */
int64_t bfz_plan_total_tiles(const bfz_plan* plan);

/* Host copy of the lookup table: out receives q rows of
 * {param, expert, tile_row, tile_col, valid_rows, valid_cols}; a padding
 * slot reads {-1, 0, 0, 0, 0, 0}.  bfz_plan_tile reads one slot.
 * Errors: BFZ_EINVAL (null, slot outside [0, q)). */
int bfz_plan_table(const bfz_plan* plan, int64_t* out);
int bfz_plan_tile(const bfz_plan* plan, int64_t slot, int64_t out[6]);

/*
 * The param-wise split of "A ZeRO Optimizer Design for Blockwise FP8
 * Quantization", section "Param-wise split" -- the alternative the page
 * replaces with the block-wise split, provided to compare their padding:
 * each weight stays whole on one rank; weights are taken largest first
 * (E H W elements; equal sizes in declared order) and each goes to the
 * bucket holding the fewest elements so far (the lower index on ties);
 * every bucket is then padded to the largest.  Host only.
 * dims as in bfz_plan_create.  Out: bucket_of_param[n_params] in [0, D),
 * bucket_elems[D] the elements per bucket (padded shard = their maximum).
 * Errors: BFZ_EINVAL (null pointers, n_params < 1, D < 1, a dimension < 1,
 * H, W > 2^31, more than 2^62 elements in all, too little host memory).
 */
int bfz_paramwise_split(const int64_t* dims, int32_t n_params, int32_t D,
                        int32_t* bucket_of_param, int64_t* bucket_elems);

/*
 * Fold: dst[s][a][b] = src[p][e][128 i + a][128 j + b] for the weight p,
 * expert e and tile (i, j) of slot s, and +0.0 outside the weight's edge
 * and in padding slots.
 * src: host array of n_params device pointers (the plan's weight order); an
 *      entry may be NULL when the rank owns none of that weight's tiles.
 *      Each weight is read, never written; 4-byte alignment is enough (a
 *      16-byte aligned weight whose W is a multiple of 4 takes the
 *      vector path).
 * dst: device buffer of q * 16384 floats, 16-byte aligned, written whole.
 * Errors: BFZ_EINVAL (null plan / dst, NULL src entry of an owned weight),
 *         BFZ_EALIGN, BFZ_ESTATE, BFZ_EHIP.
 */
int pack_shard(const bfz_plan* plan, const float* const* src, float* dst, void* stream);

/*
 * pack_shard into tiles dst_stride floats apart: slot s is written at
 * dst + s * dst_stride (pack_shard is dst_stride = 16384).  Folds master,
 * m or v into a strided state layout (bfz_step_options.state_stride), e.g. the
 * interleaved one, where master, m and v are dst = state, state + 16384
 * and state + 32768 with dst_stride = 49152.  dst_stride: a multiple of 4
 * in [16384, 2^26]; only the 16384 floats of each slot are written.
 * Errors: as pack_shard, and BFZ_EINVAL for a bad dst_stride.
 */
int pack_shard_strided(const bfz_plan* plan, const float* const* src, float* dst,
                       int64_t dst_stride, void* stream);

/*
 * One fused optimizer step over n_tiles whole tiles (n_tiles * 16384
 * elements per array), all device buffers:
 *   per element, FP32:  m = b1 m + (1 - b1) g
 *                       v = b2 v + (1 - b2) g^2
 *                       p = p - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps)
 *                       p = p - lr wd p          (when wd != 0; on the updated p)
 *   per tile:           amax = max |p|;  scale_inv = amax / 448 (or its power-of-two
 *                       form, see bfz_step_options.scale_pow2), or 1 when amax == 0, or
 *                       2^-149 when amax / 448 rounds to zero in FP32
 *                       (0 < amax <= 224 * 2^-149: subnormal tiles)
 *   per element:        code = E4M3(p / scale_inv), 0 in an all-zero tile,
 * where E4M3 is round-to-nearest (ties to even) onto the OCP E4M3FN values,
 * saturating at +-448, keeping the sign (tiny negatives give 0x80).
 * The per-step scalars (1 - b1, lr / (1 - b1^t), sqrt(1 - b2^t), lr wd, ...)
 * are formed in double on the host and rounded once to FP32; every element
 * operation is a single IEEE binary32 operation (no fused multiply-add,
 * correctly rounded sqrt and divide).
 * master, m, v: three tile-major arrays of n_tiles * 16384 floats, read
 * and overwritten in place (16-byte aligned).
 * grad: read only (16-byte aligned).  codes: n_tiles * 16384 bytes written
 * (16-byte aligned).  scale_inv: n_tiles floats written (4-byte aligned).
 * hp: the 48-byte bfz_adamw, read during the call only.
 * n_tiles = 0 is a no-op; at most 4,194,303 tiles per call (one 1024-thread
 * workgroup per tile, and a launch counts its work-items in 32 bits).
 * Padding tiles (all zero) stay zero and give scale_inv 1 and codes 0.
 * Errors: BFZ_EINVAL (null pointer, n_tiles < 0, bad hyper-parameters),
 *         BFZ_EALIGN, BFZ_EHIP.
 */
int adamw_fp8_step(float* master, const float* grad, float* m, float* v, uint8_t* codes,
                   float* scale_inv, int64_t n_tiles, const bfz_adamw* hp, void* stream);

/*
 * adamw_fp8_step with options (opts NULL: the defaults, which is exactly
 * adamw_fp8_step): power-of-two tile scales, and master / m / v tiles
 * opts->state_stride floats apart (tile s of each at s * stride).
 * Errors: as adamw_fp8_step, and BFZ_EINVAL for bad options.
 */
int adamw_fp8_step_ex(float* master, const float* grad, float* m, float* v, uint8_t* codes,
                      float* scale_inv, int64_t n_tiles, const bfz_adamw* hp,
                      const bfz_step_options* opts, void* stream);

/*
 * pack_shard of the gradients and adamw_fp8_step in one pass: the same
 * result, bit for bit, as
 *     pack_shard(plan, grad, tmp, stream);
 *     adamw_fp8_step(master, tmp, m, v, codes, scale_inv, q, hp, stream);
 * but each gradient element is read once from its row-major weight and the
 * folded copy is never written (the fold of the reduced gradients,
 * "Parameter layout transform" and "Summary", done inside the update).
 * grad: host array of n_params device pointers to the row-major FP32
 * gradients (NULL allowed for weights the rank does not touch; 4-byte
 * alignment is enough, a 16-byte aligned weight whose W is a multiple of 4
 * takes the vector path).  master, m, v: q tiles in the shard layout
 * (tile s at s * opts->state_stride floats, 16384 when 0 or opts is
 * NULL), updated in place; codes: q * 16384 bytes; scale_inv: q floats.
 * opts: as in adamw_fp8_step_ex (NULL: defaults).
 * Padding slots must hold zero state; their gradient is taken as zero.
 * Errors: BFZ_EINVAL, BFZ_EALIGN, BFZ_ESTATE, BFZ_EHIP.
 */
int fold_adamw_fp8_step(const bfz_plan* plan, const float* const* grad, float* master, float* m,
                        float* v, uint8_t* codes, float* scale_inv, const bfz_adamw* hp,
                        const bfz_step_options* opts, void* stream);

/*
 * fold_adamw_fp8_step and unpack_fp8 in one pass: the same results, bit for
 * bit, as
 *     fold_adamw_fp8_step(plan, grad, master, m, v, codes, scale_inv, hp, opts, stream);
 *     unpack_fp8(plan, codes, scale_inv, dst_fp8, dst_scale, stream);
 * with each tile's codes and scale written straight into the row-major FP8
 * weight and scale grid from the registers that produced them (the unfold
 * of "Parameter layout transform" / "Summary" done inside the update; the
 * rank's own tiles need no second pass).  codes and scale_inv may both be
 * NULL when no tile-major copy is wanted (e.g. a single rank, D = 1, with
 * nothing to all-gather); otherwise both are written as in adamw_fp8_step.
 * dst_fp8 / dst_scale: as in unpack_fp8 (entries of weights the rank does
 * not touch may be NULL; 4-byte aligned rows whose W is a multiple of 4
 * take 32-bit stores).  Other arguments as in fold_adamw_fp8_step.
 * Errors: BFZ_EINVAL (incl. exactly one of codes / scale_inv NULL),
 *         BFZ_EALIGN, BFZ_ESTATE, BFZ_EHIP.
 */
int fold_adamw_fp8_step_unpack(const bfz_plan* plan, const float* const* grad, float* master,
                               float* m, float* v, uint8_t* codes, float* scale_inv,
                               uint8_t* const* dst_fp8, float* const* dst_scale,
                               const bfz_adamw* hp, const bfz_step_options* opts, void* stream);

/*
 * fold_adamw_fp8_step_unpack with power-of-two scales, plus the transposed
 * copy of bfz_transpose_pow2, in one pass: the same results, bit for bit, as
 *     fold_adamw_fp8_step_unpack(plan, grad, master, m, v, codes, scale_inv,
 *                                dst_fp8, dst_scale, hp, opts, stream);
 *     bfz_transpose_pow2(plan, codes, scale_inv, dst_t, dst_t_scale, stream);
 * with W^T built from the step's codes in LDS instead of read back ("FP8-Flow-
 * MoE", section 3.1: the column-wise copy the backward pass reads, made by
 * exponent edits only).  opts->scale_pow2 must be set (BFZ_EINVAL
 * otherwise, NULL opts included).
 * dst_t / dst_t_scale: as in bfz_transpose_pow2.  codes and scale_inv may
 * both be NULL (no tile-major copy).  Other arguments as in
 * fold_adamw_fp8_step_unpack.
 * Errors: BFZ_EINVAL, BFZ_EALIGN, BFZ_ESTATE, BFZ_EHIP.
 */
int fold_adamw_fp8_step_unpack_t(const bfz_plan* plan, const float* const* grad, float* master,
                                 float* m, float* v, uint8_t* codes, float* scale_inv,
                                 uint8_t* const* dst_fp8, float* const* dst_scale,
                                 uint8_t* const* dst_t, float* const* dst_t_scale,
                                 const bfz_adamw* hp, const bfz_step_options* opts,
                                 void* stream);

/*
 * Unfold of the rank's owned slots: dst_fp8[p][e][128 i + a][128 j + b] =
 * codes[s][a][b] inside the weight's edge, and dst_scale[p][(e hb + i) wb + j]
 * = scale_inv[s] (hb = ceil(H/128), wb = ceil(W/128): the row-major scale
 * grid [E, hb, wb]).  Elements of tiles other ranks own are not touched.
 * codes: q * 16384 bytes (16-byte aligned); scale_inv: q floats.
 * dst_fp8 / dst_scale: host arrays of n_params device pointers; entries of
 * weights the rank does not touch may be NULL.  Any alignment is accepted:
 * rows take 16-byte stores where they start on a 16-byte boundary, aligned
 * 32-bit words otherwise (bytes only at the ends of rows that start off a
 * 4-byte boundary).
 * Errors: BFZ_EINVAL, BFZ_EALIGN, BFZ_ESTATE, BFZ_EHIP.
 */
int unpack_fp8(const bfz_plan* plan, const uint8_t* codes, const float* scale_inv,
               uint8_t* const* dst_fp8, float* const* dst_scale, void* stream);

/*
 * Scaling-aware transpose ("FP8-Flow-MoE", section 3.1, direct transpose):
 * the transposed copy W^T of the rank's tiles, re-quantized by exponent
 * edits only.  Input: codes and scales of a step run with
 * bfz_step_options.scale_pow2 (every
 * scale_inv a power of two; other scales give unspecified results).
 * Output, for every owned tile (i, j) of weight p, expert e:
 *   dst_t[p][e][128 j + c][128 i + r]   (W^T, row-major [E, W, H])
 *     = code of the tile's value at (r, c), re-expressed on the scale
 *   dst_t_scale[p][e][128 j + c][i]     ([E, W, ceil(H/128)])
 * which is the smallest power of two holding that 128-element group of the
 * W^T row (the tile rule applied to the group; >= 2^-149).  The group scale
 * never exceeds the tile's, so the edits only raise exponents: every value
 * is reproduced exactly, with none of the extra rounding a dequantize ->
 * transpose -> quantize pass with arbitrary scales would add.  An all-zero
 * group gets scale 1 and codes 0.  codes: q * 16384 bytes (16-byte
 * aligned); scale_inv: q floats; dst_t / dst_t_scale: host arrays of
 * n_params device pointers (NULL allowed for weights the rank does not
 * touch; any alignment for dst_t, 4 bytes for dst_t_scale).  Asynchronous
 * on `stream`; no allocation.
 * Errors: BFZ_EINVAL, BFZ_EALIGN, BFZ_ESTATE, BFZ_EHIP.
 */
int bfz_transpose_pow2(const bfz_plan* plan, const uint8_t* codes, const float* scale_inv,
                       uint8_t* const* dst_t, float* const* dst_t_scale, void* stream);

/*
 * The E4M3 rounding adamw_fp8_step applies to p / scale_inv, exposed on
 * its own so it can be checked over every fp32 bit pattern:
 * out[k] = E4M3(in[k]) for k < n.  Device buffers, any alignment.
 * Errors: BFZ_EINVAL (null, n < 0), BFZ_EHIP.
 */
int bfz_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream);

/* Message of the calling thread's last failed call ("" if none). */
const char* bfz_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BFZ_H */
