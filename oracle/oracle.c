/*
 * Plain CPU oracle for the block-wise FP8 ZeRO-1 shard step.
 * TEST INFRASTRUCTURE ONLY -- see oracle.h for who may use it and for the
 * full titles of the pages cited below.
 *
 * Built with:  gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math
 * so every float expression below is evaluated as written, one IEEE-754
 * binary32 rounding per operation.
 */
#include "oracle.h"

#include <math.h>
#include <stddef.h>
#include <string.h>

/* ===================================================================== *
 * E4M3 (OCP E4M3FN)                                                      *
 * ===================================================================== */

/*
 * Value of a code, straight from the encoding in [FP8-Flow, §3.1]:
 * sign S, 4 exponent bits E with bias 7, 3 mantissa bits M, so a normal
 * value is (-1)^S 2^(E-7) (1 + M/8).  Codes with E = 0 are the
 * subnormals (-1)^S 2^(-6) (M/8).  The all-ones pattern S.1111.111 is NaN,
 * which leaves 448 = 2^8 * 1.75 as the largest finite value, the E4M3
 * maximum both [FP8-Flow, §3.1] and [FP8-Scale, §1] name.
 * Parity: pinned by tests/test_oracle_e4m3.py (hand-derived golden values
 * and the exhaustive comparison against torch's float8_e4m3fn cast).
 */
double ora_e4m3_decode(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* The 127 non-negative finite values, ascending: codes 0x00 .. 0x7E.
 * Filled once when the library is loaded, before any caller thread runs. */
static double g_pos[127];

__attribute__((constructor)) static void pos_table_init(void) {
    for (int c = 0; c < 127; ++c) g_pos[c] = ora_e4m3_decode((uint8_t)c);
}

/* Largest k in [0, 126] with g_pos[k] <= a (a >= 0), by bisection over the
 * ascending table. */
static int bracket(double a) {
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (g_pos[mid] <= a) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/*
 * Encoding of a real y: [FP8-Scale, §1.1] clamps to the representable range
 * and [FP8-Flow, §3.1] maps to the nearest representable value.  Reading
 * taken: saturate |y| to 448, pick the nearest of the 127 non-negative
 * values, break an exact tie toward the code with an even last bit (round
 * half to even, which the pages leave unstated), and keep y's sign bit (so
 * a negative value that rounds to zero encodes as 0x80).
 * Every double below is exact: y has 24 significant bits and the table
 * values 4, within the exponent range of a double.
 */
uint8_t ora_e4m3_encode(float y) {
    double a = fabs((double)y);
    if (a > 448.0) a = 448.0;
    int k = bracket(a);
    int c = k;
    if (k < 126) {
        double below = a - g_pos[k], above = g_pos[k + 1] - a;
        if (above < below) c = k + 1;
        else if (above == below) c = (k % 2 == 0) ? k : k + 1;
    }
    return (uint8_t)(signbit(y) ? (c | 0x80) : c);
}

int ora_e4m3_near_midpoint(float y, double rel) {
    double a = fabs((double)y);
    if (a >= 448.0) return 0;
    int k = bracket(a);
    double mid = 0.5 * (g_pos[k] + g_pos[k + 1]);
    return fabs(a - mid) <= rel * mid;
}

void ora_e4m3_encode_array(const float* y, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = ora_e4m3_encode(y[i]);
}

/* ===================================================================== *
 * Block-wise split                                                       *
 * ===================================================================== */

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t ora_total_tiles(const int64_t* dims, int32_t n_params) {
    int64_t t = 0;
    for (int32_t p = 0; p < n_params; ++p)
        t += dims[3 * p] * ceil_div(dims[3 * p + 1], ORA_TILE_DIM) *
             ceil_div(dims[3 * p + 2], ORA_TILE_DIM);
    return t;
}

/*
 * [ZeRO-FP8, "Block-wise split"]: every quantized dimension is padded up to
 * a multiple of 128 and the flattened buffer is cut at 128x128 units, with
 * a lookup table recording each unit's parameter and its real extent.
 * [ZeRO-FP8, "Parameter layout transform"]: units follow the fold order --
 * expert, tile row, tile column.  The page does not spell out how units are
 * dealt to ranks; the reading taken is a contiguous fill in declared
 * parameter order with an equal quota q = ceil(T/D) per rank (rank r owns
 * global units [r q, min((r+1) q, T))), the shorter shards padded to q like
 * the page's param-wise buckets are padded to the largest one
 * ["Param-wise split"].
 * Parity: the rule itself is a reading (parity unpinned); the properties
 * (exactly-once ownership, contiguity, counts) are pinned by brute force in
 * tests/test_oracle_plan.py.
 */
int ora_plan(const int64_t* dims, int32_t n_params, int32_t D, int32_t rank,
             int64_t* q_out, int64_t* owned_out, int64_t* table) {
    if (n_params < 0 || D < 1 || rank < 0 || rank >= D) return -1;
    for (int32_t p = 0; p < n_params; ++p)
        if (dims[3 * p] < 1 || dims[3 * p + 1] < 1 || dims[3 * p + 2] < 1)
            return -1;
    int64_t T = ora_total_tiles(dims, n_params);
    int64_t q = ceil_div(T, D);
    int64_t first = (int64_t)rank * q;
    int64_t last = first + q < T ? first + q : T;
    int64_t owned = last > first ? last - first : 0;
    *q_out = q;
    *owned_out = owned;
    if (!table) return 0;
    for (int64_t s = 0; s < q; ++s) {
        int64_t* row = table + 6 * s;
        row[0] = -1; row[1] = row[2] = row[3] = row[4] = row[5] = 0;
    }
    int64_t g = 0;
    for (int32_t p = 0; p < n_params; ++p) {
        int64_t E = dims[3 * p], H = dims[3 * p + 1], W = dims[3 * p + 2];
        int64_t hb = ceil_div(H, ORA_TILE_DIM), wb = ceil_div(W, ORA_TILE_DIM);
        for (int64_t e = 0; e < E; ++e)
            for (int64_t i = 0; i < hb; ++i)
                for (int64_t j = 0; j < wb; ++j, ++g) {
                    if (g < first || g >= last) continue;
                    int64_t* row = table + 6 * (g - first);
                    row[0] = p; row[1] = e; row[2] = i; row[3] = j;
                    row[4] = (H - ORA_TILE_DIM * i) < ORA_TILE_DIM ? H - ORA_TILE_DIM * i : ORA_TILE_DIM;
                    row[5] = (W - ORA_TILE_DIM * j) < ORA_TILE_DIM ? W - ORA_TILE_DIM * j : ORA_TILE_DIM;
                }
    }
    return 0;
}

/*
 * [ZeRO-FP8, "Param-wise split"]: the weights are sorted by size and dealt
 * greedily so that the D buckets come out as even as possible; every bucket
 * is then padded to the largest one.  Reading of "greedy": largest weight
 * first, each into the bucket holding the fewest elements so far (ties: the
 * lower bucket; equal sizes: declared order) -- the longest-processing-time
 * rule.  A weight is its whole E x H x W tensor; no 128-padding is needed,
 * since each weight stays whole on one rank.
 * Parity: the tie-breaking is a reading (parity unpinned); the rule is
 * pinned by brute-force optima against Graham's LPT bound in
 * tests/test_oracle_plan.py.
 */
int ora_paramwise_split(const int64_t* dims, int32_t n_params, int32_t D,
                        int32_t* bucket_of_param, int64_t* bucket_elems) {
    if (n_params < 0 || D < 1) return -1;
    for (int32_t b = 0; b < D; ++b) bucket_elems[b] = 0;
    for (int32_t p = 0; p < n_params; ++p) {
        if (dims[3 * p] < 1 || dims[3 * p + 1] < 1 || dims[3 * p + 2] < 1) return -1;
        bucket_of_param[p] = -1;
    }
    for (int32_t done = 0; done < n_params; ++done) {
        /* the largest weight not yet placed (first in declared order on ties) */
        int32_t pick = -1;
        int64_t pick_size = -1;
        for (int32_t p = 0; p < n_params; ++p) {
            if (bucket_of_param[p] >= 0) continue;
            int64_t size = dims[3 * p] * dims[3 * p + 1] * dims[3 * p + 2];
            if (size > pick_size) { pick = p; pick_size = size; }
        }
        /* the emptiest bucket (lowest index on ties) */
        int32_t best = 0;
        for (int32_t b = 1; b < D; ++b)
            if (bucket_elems[b] < bucket_elems[best]) best = b;
        bucket_of_param[pick] = best;
        bucket_elems[best] += pick_size;
    }
    return 0;
}

/* ===================================================================== *
 * Fold / unfold                                                          *
 * ===================================================================== */

/*
 * [ZeRO-FP8, "Parameter layout transform"]: fold rewrites a row-major
 * [E,H,W] weight so that each 128x128 unit is contiguous, units ordered by
 * expert, tile row, tile column; inside a unit the rows stay in row-major
 * order.  [ZeRO-FP8, "Block-wise split"] pads each dimension to a multiple
 * of 128; the pad value is unstated -- zero is taken.
 * Parity: pinned against torch's im2col (F.unfold) in tests/test_oracle_layout.py.
 */
void ora_fold_tile(const float* src, int64_t H, int64_t W, int64_t e,
                   int64_t i, int64_t j, float* tile) {
    for (int64_t a = 0; a < ORA_TILE_DIM; ++a)
        for (int64_t b = 0; b < ORA_TILE_DIM; ++b) {
            int64_t r = ORA_TILE_DIM * i + a, c = ORA_TILE_DIM * j + b;
            tile[a * ORA_TILE_DIM + b] =
                (r < H && c < W) ? src[(e * H + r) * W + c] : 0.0f;
        }
}

void ora_pack(const int64_t* dims, int32_t n_params, const float* const* src,
              const int64_t* table, int64_t q, float* shard) {
    (void)n_params;
    for (int64_t s = 0; s < q; ++s) {
        const int64_t* row = table + 6 * s;
        float* tile = shard + s * ORA_TILE_ELEMS;
        if (row[0] < 0) {
            for (int64_t k = 0; k < ORA_TILE_ELEMS; ++k) tile[k] = 0.0f;
            continue;
        }
        const int64_t* d = dims + 3 * row[0];
        ora_fold_tile(src[row[0]], d[1], d[2], row[1], row[2], row[3], tile);
    }
}

/*
 * [ZeRO-FP8, "Parameter layout transform" and "Summary"]: unfold is the
 * inverse of fold, applied to the FP8 weights and to their scales after
 * the update.  The scales of one weight form the grid
 * [E, ceil(H/128), ceil(W/128)], row-major, one value per unit.
 * Parity: pinned against torch's col2im (F.fold) in tests/test_oracle_layout.py.
 */
void ora_unpack(const int64_t* dims, int32_t n_params, const uint8_t* codes,
                const float* scale_inv, const int64_t* table, int64_t q,
                uint8_t* const* dst_codes, float* const* dst_scale) {
    (void)n_params;
    for (int64_t s = 0; s < q; ++s) {
        const int64_t* row = table + 6 * s;
        if (row[0] < 0) continue;
        int64_t p = row[0], e = row[1], i = row[2], j = row[3];
        int64_t vr = row[4], vc = row[5];
        int64_t H = dims[3 * p + 1], W = dims[3 * p + 2];
        int64_t hb = ceil_div(H, ORA_TILE_DIM), wb = ceil_div(W, ORA_TILE_DIM);
        const uint8_t* tile = codes + s * ORA_TILE_ELEMS;
        for (int64_t a = 0; a < vr; ++a)
            for (int64_t b = 0; b < vc; ++b)
                dst_codes[p][(e * H + ORA_TILE_DIM * i + a) * W + ORA_TILE_DIM * j + b] =
                    tile[a * ORA_TILE_DIM + b];
        dst_scale[p][(e * hb + i) * wb + j] = scale_inv[s];
    }
}

/*
 * [FP8-Flow, §3.1, direct transpose]: with power-of-two scales a tensor
 * quantized in one grouping can be re-expressed in another by exponent
 * edits, so the transposed copy the backward pass needs carries no second
 * rounding.  What it computes, written as the naive route (dequantize,
 * transpose, quantize again): the tile's values v = dec(code) * 2^T; each
 * 128-element group of a W^T row -- one column of the tile, its valid
 * rows -- gets the power-of-two scale of its own amax (ora_pow2_scale, the
 * tile rule; an all-zero group gets 1 and codes +0) and its values are
 * encoded again.  Everything here is exact in double; the claim that the
 * result equals the codes moved by exponent edits is what the GPU kernel
 * is checked against.
 * Parity: pinned in tests/test_oracle_transpose.py (lossless values,
 * torch's own dequantize/transpose/quantize route, tight group scales).
 */
static double pow2_scale_d(double amax) {
    int T = -149;
    while (ldexp(448.0, T) < amax) ++T;
    return ldexp(1.0, T);
}

void ora_transpose_pow2(const int64_t* dims, int32_t n_params, const uint8_t* codes,
                        const float* scale_inv, const int64_t* table, int64_t q,
                        uint8_t* const* dst_t, float* const* dst_t_scale) {
    (void)n_params;
    for (int64_t s = 0; s < q; ++s) {
        const int64_t* row = table + 6 * s;
        if (row[0] < 0) continue;
        int64_t p = row[0], e = row[1], i = row[2], j = row[3], vr = row[4], vc = row[5];
        int64_t H = dims[3 * p + 1], W = dims[3 * p + 2];
        int64_t hb = ceil_div(H, ORA_TILE_DIM);
        const uint8_t* tile = codes + s * ORA_TILE_ELEMS;
        double tile_scale = (double)scale_inv[s];
        for (int64_t c = 0; c < vc; ++c) {
            double amax = 0.0;
            for (int64_t r = 0; r < vr; ++r) {
                double v = fabs(ora_e4m3_decode(tile[r * ORA_TILE_DIM + c]) * tile_scale);
                if (v > amax) amax = v;
            }
            int64_t out_row = e * W + ORA_TILE_DIM * j + c;  /* row of W^T */
            double g = amax == 0.0 ? 1.0 : pow2_scale_d(amax);
            dst_t_scale[p][out_row * hb + i] = (float)g;
            for (int64_t r = 0; r < vr; ++r) {
                double v = ora_e4m3_decode(tile[r * ORA_TILE_DIM + c]) * tile_scale;
                uint8_t code = amax == 0.0 ? 0 : ora_e4m3_encode((float)(v / g));
                dst_t[p][out_row * H + ORA_TILE_DIM * i + r] = code;
            }
        }
    }
}

/* ===================================================================== *
 * AdamW                                                                  *
 * ===================================================================== */

/*
 * [Int8AdamW, §4.3]: per element, in this order,
 *   m <- beta1 m + (1 - beta1) g
 *   v <- beta2 v + (1 - beta2) g^2
 *   denom = sqrt(v) / sqrt(1 - beta2^t) + eps
 *   p <- p - (lr / (1 - beta1^t)) m / denom
 *   if weight_decay != 0:  p <- p - lr * weight_decay * p   (on the updated p)
 * The step counter is incremented before use, so the first step is t = 1.
 * [ZeRO-FP8, "ZeRO-1 optimizer"] keeps master params, grads and both
 * moments in FP32, so the arithmetic is binary32.  The per-step scalars are
 * computed once in double (the page computes them from Python floats) and
 * rounded to binary32 once each.
 * Parity: pinned by closed forms (t = 1 from zero state; warm state at any
 * t), by torch.optim.AdamW (weight_decay = 0) and by the exact weight-decay
 * placement difference, in tests/test_oracle_adamw.py.
 */
typedef struct {
    float b1, c1, b2, c2, step_size, sbc2, eps, decay;
    int has_decay;
} ora_scalars;

static ora_scalars make_scalars(const ora_hparams* hp) {
    ora_scalars s;
    double t = (double)hp->step;
    s.b1 = (float)hp->beta1;
    s.c1 = (float)(1.0 - hp->beta1);
    s.b2 = (float)hp->beta2;
    s.c2 = (float)(1.0 - hp->beta2);
    s.step_size = (float)(hp->lr / (1.0 - pow(hp->beta1, t)));
    s.sbc2 = (float)sqrt(1.0 - pow(hp->beta2, t));
    s.eps = (float)hp->eps;
    s.decay = (float)(hp->lr * hp->weight_decay);
    s.has_decay = hp->weight_decay != 0.0;
    return s;
}

static void adamw_one(float* p, float g, float* m, float* v, const ora_scalars* s) {
    float mm = s->b1 * *m + s->c1 * g;
    float vv = s->b2 * *v + s->c2 * (g * g);
    float denom = sqrtf(vv) / s->sbc2 + s->eps;
    float pp = *p - s->step_size * (mm / denom);
    if (s->has_decay) pp = pp - s->decay * pp;
    *m = mm;
    *v = vv;
    *p = pp;
}

void ora_adamw(float* p, const float* g, float* m, float* v, int64_t n,
               const ora_hparams* hp) {
    ora_scalars s = make_scalars(hp);
    for (int64_t k = 0; k < n; ++k) adamw_one(p + k, g[k], m + k, v + k, &s);
}

/* ===================================================================== *
 * Per-tile quantization                                                  *
 * ===================================================================== */

/*
 * [FP8-Flow, §3.1]: one scale per tile, s = max|x| / 448, and the code is
 * x/s mapped to the nearest E4M3 value; dequantization multiplies back by
 * s.  The scale stored is s itself (the "scale_inv" of the weight: the
 * factor that turns codes back into values); quantization divides by it.
 * A tile that is all zero would give s = 0 and a division by zero;
 * [Int8AdamW, §4.2 and §5.1] guard that case by using a scale of 1, which
 * is taken here (test: amax == 0 exactly), and all its codes are +0.
 * A tile whose amax is positive but at most 224 * 2^-149 makes amax / 448
 * round to zero in binary32 -- the same division by zero for a nonzero
 * tile, which the pages do not address.  Reading: its scale is 2^-149, the
 * smallest positive binary32 (the floor the power-of-two rule below also
 * stops at); then x / s = x * 2^149 is exact and at most 224 in magnitude,
 * so every code is finite.
 * [ZeRO-FP8, "Summary"]: the new FP8 weights and scales come from the
 * updated FP32 master, one tile at a time.
 * Parity: pinned by invariants (max code = 448, error bound, idempotence,
 * zero tiles) and hand-built tiles in tests/test_oracle_quant.py.
 */
/*
 * [FP8-Flow, §3.1]: when every scale is a power of two, moving codes from
 * one scale to another is a change of exponent bits only.  The power-of-two
 * tile scale taken here is the smallest 2^T that still holds the tile:
 * 448 * 2^T >= amax (a reading: rounding the scale up keeps every quotient
 * within +-448, so nothing saturates).  T stops at -149, the smallest
 * binary32 power of two.
 * Parity: pinned in tests/test_oracle_quant.py (power of two, tight,
 * max code in (224, 448], exact-grid tiles).
 */
float ora_pow2_scale(float amax) {
    int T = -149;
    while (ldexp(448.0, T) < (double)amax) ++T;
    return (float)ldexp(1.0, T);
}

void ora_quant_tiles_mode(const float* p, int64_t n_tiles, uint8_t* codes,
                          float* scale_inv, uint8_t* near_mid, double rel, int pow2) {
    for (int64_t t = 0; t < n_tiles; ++t) {
        const float* x = p + t * ORA_TILE_ELEMS;
        uint8_t* c = codes + t * ORA_TILE_ELEMS;
        uint8_t* nm = near_mid ? near_mid + t * ORA_TILE_ELEMS : NULL;
        float amax = 0.0f;
        for (int64_t k = 0; k < ORA_TILE_ELEMS; ++k)
            if (fabsf(x[k]) > amax) amax = fabsf(x[k]);
        if (amax == 0.0f) {
            scale_inv[t] = 1.0f;
            for (int64_t k = 0; k < ORA_TILE_ELEMS; ++k) {
                c[k] = 0;
                if (nm) nm[k] = 0;
            }
            continue;
        }
        float s = pow2 ? ora_pow2_scale(amax) : amax / 448.0f;
        if (s == 0.0f) s = (float)ldexp(1.0, -149);  /* amax / 448 underflowed */
        scale_inv[t] = s;
        for (int64_t k = 0; k < ORA_TILE_ELEMS; ++k) {
            float y = x[k] / s;
            c[k] = ora_e4m3_encode(y);
            if (nm) nm[k] = (uint8_t)ora_e4m3_near_midpoint(y, rel);
        }
    }
}

void ora_quant_tiles(const float* p, int64_t n_tiles, uint8_t* codes,
                     float* scale_inv, uint8_t* near_mid, double rel) {
    ora_quant_tiles_mode(p, n_tiles, codes, scale_inv, near_mid, rel, 0);
}

/* [ZeRO-FP8, "Summary"]: the element-wise update of the rank's slice, then
 * the new FP8 weights and scales from the updated FP32 master. */
void ora_step_mode(float* p, const float* g, float* m, float* v, int64_t n_tiles,
                   const ora_hparams* hp, uint8_t* codes, float* scale_inv,
                   uint8_t* near_mid, double rel, int pow2) {
    ora_adamw(p, g, m, v, n_tiles * ORA_TILE_ELEMS, hp);
    ora_quant_tiles_mode(p, n_tiles, codes, scale_inv, near_mid, rel, pow2);
}

void ora_step(float* p, const float* g, float* m, float* v, int64_t n_tiles,
              const ora_hparams* hp, uint8_t* codes, float* scale_inv,
              uint8_t* near_mid, double rel) {
    ora_step_mode(p, g, m, v, n_tiles, hp, codes, scale_inv, near_mid, rel, 0);
}
