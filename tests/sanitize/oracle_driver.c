/*
 * The C oracle under AddressSanitizer / UndefinedBehaviorSanitizer (CPU,
 * test infrastructure): every oracle entry point runs on small seeded
 * inputs held in buffers of exactly the documented sizes, over ragged
 * weights, several experts, every rank of several splits and both scale
 * modes, including subnormal and all-zero tiles.  Functional checks are
 * kept to what the layout fixes (fold then unfold gives back every owned
 * element's code, the transposed copy decodes to the tile's values, every
 * tile owned once); the numerical pins live in the Python tests.
 * Exit status 0 when every check passes.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static int failures = 0;
#define CHECK(cond, msg)                                            \
    do {                                                            \
        if (!(cond)) {                                              \
            fprintf(stderr, "CHECK failed at line %d: %s\n", __LINE__, msg); \
            ++failures;                                             \
        }                                                           \
    } while (0)

static uint64_t rng = 0x2545F4914F6CDD1Dull;
static uint64_t next_u64(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return rng;
}
static int64_t uniform(int64_t lo, int64_t hi) { return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1)); }
static double gauss(void) {
    const double u1 = ((double)(next_u64() >> 11) + 1.0) / 9007199254740993.0;
    const double u2 = (double)(next_u64() >> 11) / 9007199254740992.0;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}
static void* exact(size_t n, size_t size) { return malloc(n ? n * size : 1); }

static void run_case(const int64_t* dims, int32_t n, int32_t D, int pow2) {
    const int64_t T = ora_total_tiles(dims, n);
    float** w = (float**)exact((size_t)n, sizeof(float*));
    for (int32_t p = 0; p < n; ++p) {
        const int64_t E = dims[3 * p], H = dims[3 * p + 1], W = dims[3 * p + 2];
        w[p] = (float*)exact((size_t)(E * H * W), sizeof(float));
        const int kind = (int)(p % 3);  /* normal, subnormal, all zero */
        for (int64_t k = 0; k < E * H * W; ++k)
            w[p][k] = kind == 0 ? (float)(0.02 * gauss()) : kind == 1 ? (float)(uniform(-300, 300) * ldexp(1.0, -149)) : 0.0f;
    }
    int64_t seen = 0;
    for (int32_t rank = 0; rank < D; ++rank) {
        int64_t q = 0, owned = 0;
        CHECK(ora_plan(dims, n, D, rank, &q, &owned, NULL) == 0, "plan size");
        CHECK(q * D >= T && (q - 1) * D < T && owned <= q, "quota");
        int64_t* table = (int64_t*)exact((size_t)(6 * q), sizeof(int64_t));
        CHECK(ora_plan(dims, n, D, rank, &q, &owned, table) == 0, "plan");
        seen += owned;
        const int64_t ne = q * ORA_TILE_ELEMS;
        float* p = (float*)exact((size_t)ne, sizeof(float));
        float* g = (float*)exact((size_t)ne, sizeof(float));
        float* m = (float*)exact((size_t)ne, sizeof(float));
        float* v = (float*)exact((size_t)ne, sizeof(float));
        uint8_t* codes = (uint8_t*)exact((size_t)ne, 1);
        uint8_t* near = (uint8_t*)exact((size_t)ne, 1);
        float* sc = (float*)exact((size_t)q, sizeof(float));
        ora_pack(dims, n, (const float* const*)w, table, q, p);
        for (int64_t k = 0; k < ne; ++k) {
            g[k] = (float)(1e-3 * gauss());
            m[k] = 0.0f;
            v[k] = 0.0f;
        }
        /* one tile's worth through the single-tile fold, against the shard */
        if (owned > 0) {
            const int64_t* r = table;
            float* tile = (float*)exact(ORA_TILE_ELEMS, sizeof(float));
            ora_fold_tile(w[r[0]], dims[3 * r[0] + 1], dims[3 * r[0] + 2], r[1], r[2], r[3], tile);
            CHECK(memcmp(tile, p, ORA_TILE_ELEMS * sizeof(float)) == 0, "fold_tile vs pack");
            free(tile);
        }
        ora_hparams hp = {1e-4, 0.9, 0.95, 1e-8, 0.1, 3};
        ora_step_mode(p, g, m, v, q, &hp, codes, sc, near, 1e-6, pow2);
        ora_quant_tiles_mode(p, q, codes, sc, NULL, 1e-6, pow2);
        /* unfold, then check every owned element's code landed */
        uint8_t** d8 = (uint8_t**)exact((size_t)n, sizeof(uint8_t*));
        float** dg = (float**)exact((size_t)n, sizeof(float*));
        uint8_t** dt = (uint8_t**)exact((size_t)n, sizeof(uint8_t*));
        float** dts = (float**)exact((size_t)n, sizeof(float*));
        for (int32_t k = 0; k < n; ++k) {
            const int64_t E = dims[3 * k], H = dims[3 * k + 1], W = dims[3 * k + 2];
            const int64_t hb = (H + 127) / 128, wb = (W + 127) / 128;
            d8[k] = (uint8_t*)exact((size_t)(E * H * W), 1);
            dg[k] = (float*)exact((size_t)(E * hb * wb), sizeof(float));
            dt[k] = (uint8_t*)exact((size_t)(E * W * H), 1);
            dts[k] = (float*)exact((size_t)(E * W * hb), sizeof(float));
        }
        ora_unpack(dims, n, codes, sc, table, q, d8, dg);
        for (int64_t s = 0; s < owned; ++s) {
            const int64_t* r = table + 6 * s;
            const int64_t H = dims[3 * r[0] + 1], W = dims[3 * r[0] + 2];
            for (int64_t a = 0; a < r[4]; ++a)
                for (int64_t b = 0; b < r[5]; ++b)
                    CHECK(d8[r[0]][(r[1] * H + 128 * r[2] + a) * W + 128 * r[3] + b] ==
                              codes[s * ORA_TILE_ELEMS + a * 128 + b],
                          "unfold");
        }
        if (pow2) {
            /* the transposed copy decodes to the tile's values */
            ora_transpose_pow2(dims, n, codes, sc, table, q, dt, dts);
            for (int64_t s = 0; s < owned; ++s) {
                const int64_t* r = table + 6 * s;
                const int64_t H = dims[3 * r[0] + 1], W = dims[3 * r[0] + 2];
                const int64_t hb = (H + 127) / 128;
                for (int64_t b = 0; b < r[5]; ++b) {
                    const int64_t out_row = r[1] * W + 128 * r[3] + b;
                    const double gs = dts[r[0]][out_row * hb + r[2]];
                    for (int64_t a = 0; a < r[4]; ++a)
                        CHECK(ora_e4m3_decode(dt[r[0]][out_row * H + 128 * r[2] + a]) * gs ==
                                  ora_e4m3_decode(codes[s * ORA_TILE_ELEMS + a * 128 + b]) * (double)sc[s],
                              "transposed value");
                }
            }
        }
        for (int32_t k = 0; k < n; ++k) {
            free(d8[k]);
            free(dg[k]);
            free(dt[k]);
            free(dts[k]);
        }
        free(d8);
        free(dg);
        free(dt);
        free(dts);
        free(p);
        free(g);
        free(m);
        free(v);
        free(codes);
        free(near);
        free(sc);
        free(table);
    }
    CHECK(seen == T, "every tile owned once");
    int32_t* bop = (int32_t*)exact((size_t)n, sizeof(int32_t));
    int64_t* be = (int64_t*)exact((size_t)D, sizeof(int64_t));
    CHECK(ora_paramwise_split(dims, n, D, bop, be) == 0, "paramwise");
    int64_t sum = 0, want = 0;
    for (int32_t b = 0; b < D; ++b) sum += be[b];
    for (int32_t k = 0; k < n; ++k) want += dims[3 * k] * dims[3 * k + 1] * dims[3 * k + 2];
    CHECK(sum == want, "paramwise total");
    free(bop);
    free(be);
    for (int32_t p = 0; p < n; ++p) free(w[p]);
    free(w);
}

int main(void) {
    /* E4M3 helpers over every code and a sweep of values */
    for (int c = 0; c < 256; ++c)
        if ((c & 0x7F) != 0x7F) CHECK(ora_e4m3_encode((float)ora_e4m3_decode((uint8_t)c)) == c, "decode/encode");
    float ys[4096];
    uint8_t cs[4096];
    for (int k = 0; k < 4096; ++k) ys[k] = (float)ldexp(gauss(), (int)uniform(-20, 10));
    ora_e4m3_encode_array(ys, cs, 4096);
    for (int k = 0; k < 4096; ++k) (void)ora_e4m3_near_midpoint(ys[k], 1e-6);
    CHECK(ora_pow2_scale(448.0f) == 1.0f, "pow2 scale");
    /* bad arguments */
    int64_t q, owned;
    const int64_t one[3] = {1, 10, 10};
    CHECK(ora_plan(one, 1, 0, 0, &q, &owned, NULL) != 0, "D = 0");
    CHECK(ora_plan(one, 1, 2, 2, &q, &owned, NULL) != 0, "rank = D");
    for (int trial = 0; trial < 10; ++trial) {
        const int32_t n = (int32_t)uniform(1, 5);
        int64_t* dims = (int64_t*)exact((size_t)(3 * n), sizeof(int64_t));
        for (int32_t p = 0; p < n; ++p) {
            dims[3 * p] = uniform(1, 3);
            dims[3 * p + 1] = uniform(1, 300);
            dims[3 * p + 2] = uniform(1, 300);
        }
        run_case(dims, n, (int32_t)uniform(1, 7), trial & 1);
        free(dims);
    }
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
