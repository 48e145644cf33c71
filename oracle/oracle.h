/*
 * Plain CPU oracle for the block-wise FP8 ZeRO-1 shard step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code: only the tests, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no source with the HIP
 * library; the two meet only through the seeded input generator.
 *
 * Everything here is deliberately slow and literal: one element at a time,
 * IEEE-754 binary32 arithmetic with no fused multiply-add (built with
 * -ffp-contract=off), correctly rounded sqrtf and division, no blocking,
 * no threads, no vector code.
 *
 * Sources (web pages, cited by title and section):
 *  [ZeRO-FP8]  "A ZeRO Optimizer Design for Blockwise FP8 Quantization"
 *              (beipo.top, 2025): sections "Block-wise split",
 *              "Parameter layout transform" (fold / unfold) and "Summary"
 *              (the block-wise ZeRO-1 update flow).
 *  [Int8AdamW] lpnh.cn essay on optimizer-state quantization ("Model-
 *              Optimizer"): section 4.3, the AdamW step of its Int8AdamW,
 *              and sections 4.2 / 5.1 (zero-scale guard).
 *  [FP8-Flow]  "FP8-Flow-MoE: A Casting-Free FP8 Recipe without Double
 *              Quantization Error" (papercache summary): section 3.1, the
 *              per-tile scale s = amax/448, the quantizer Q(x)=round(x/s),
 *              the dequantizer, same-layout idempotence and the E4M3
 *              encoding (-1)^S 2^(E-7) (1+M/8).
 *  [FP8-Scale] "FP8 training: core scaling strategies" (mhpn.cn): section
 *              1.1 (clamp(round(x/scale)) abstraction, E4M3 range +-448)
 *              and section 3.2 (128x128 block quantization).
 *
 * Parity status of each function is stated at its definition.
 */
#ifndef BFZ_ORACLE_H
#define BFZ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORA_TILE_DIM 128
#define ORA_TILE_ELEMS (128 * 128)

/* AdamW hyper-parameters, as the optimizer's caller supplies them. */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    int64_t step; /* t >= 1: the step counter after its increment */
} ora_hparams;

/* ---- E4M3 (OCP E4M3FN) -------------------------------------------- */
double  ora_e4m3_decode(uint8_t code);
uint8_t ora_e4m3_encode(float y);
/* 1 when |y| (clamped to 448) lies within rel*mid of a rounding midpoint
 * between two neighbouring E4M3 values. */
int     ora_e4m3_near_midpoint(float y, double rel);
void    ora_e4m3_encode_array(const float* y, uint8_t* out, int64_t n);

/* ---- Block-wise partition (lookup table) -------------------------- */
/* dims: n_params triples {E, H, W} (E = experts, 1 for a plain matrix). */
int64_t ora_total_tiles(const int64_t* dims, int32_t n_params);
/* Writes q (slots per rank) and owned (<= q) and, if table != NULL,
 * q rows of {param, e, i, j, valid_rows, valid_cols}; slots past `owned`
 * are written as {-1, 0, 0, 0, 0, 0}.  Returns 0, or -1 on bad input. */
int ora_plan(const int64_t* dims, int32_t n_params, int32_t D, int32_t rank,
             int64_t* q, int64_t* owned, int64_t* table);

/* The param-wise split (compared against, not used by, the block-wise
 * split): bucket_of_param[p] in [0, D) for each weight, bucket_elems[D] the
 * elements per bucket.  Returns 0, or -1 on bad input. */
int ora_paramwise_split(const int64_t* dims, int32_t n_params, int32_t D,
                        int32_t* bucket_of_param, int64_t* bucket_elems);

/* ---- Fold / unfold ------------------------------------------------ */
/* One tile of a row-major [E,H,W] fp32 tensor into 128x128 row-major tile
 * storage, zero beyond the tensor's edge. */
void ora_fold_tile(const float* src, int64_t H, int64_t W, int64_t e,
                   int64_t i, int64_t j, float* tile);
/* Whole shard: src[p] is param p's row-major tensor (may be NULL for
 * params owning no slot).  Padding slots are all zero. */
void ora_pack(const int64_t* dims, int32_t n_params, const float* const* src,
              const int64_t* table, int64_t q, float* shard);
/* Codes and scales of every owned slot back to row-major FP8 codes and
 * the row-major scale grid [E, ceil(H/128), ceil(W/128)] of each param. */
void ora_unpack(const int64_t* dims, int32_t n_params, const uint8_t* codes,
                const float* scale_inv, const int64_t* table, int64_t q,
                uint8_t* const* dst_codes, float* const* dst_scale);

/* Transposed copy of power-of-two-quantized tiles: for every owned slot,
 * W^T[e][128 j + c][128 i + r] = code of the value at (r, c) of the tile,
 * requantized with one power-of-two scale per 128-element group of a W^T
 * row (a column segment of the tile).  dst_t[p]: uint8 [E, W, H];
 * dst_t_scale[p]: float [E, W, ceil(H/128)]. */
void ora_transpose_pow2(const int64_t* dims, int32_t n_params, const uint8_t* codes,
                        const float* scale_inv, const int64_t* table, int64_t q,
                        uint8_t* const* dst_t, float* const* dst_t_scale);

/* ---- AdamW (element-wise, fp32) ----------------------------------- */
void ora_adamw(float* p, const float* g, float* m, float* v, int64_t n,
               const ora_hparams* hp);

/* ---- Per-tile E4M3 quantization ----------------------------------- */
/* Smallest power of two 2^T with 448 * 2^T >= amax (amax > 0), T >= -149. */
float ora_pow2_scale(float amax);
/* n_tiles tiles of 16384 contiguous values.  near_mid (nullable) gets a 1
 * for every element whose quotient p/scale_inv is within rel of an E4M3
 * rounding midpoint.  pow2 != 0: power-of-two scales (ora_pow2_scale). */
void ora_quant_tiles(const float* p, int64_t n_tiles, uint8_t* codes,
                     float* scale_inv, uint8_t* near_mid, double rel);
void ora_quant_tiles_mode(const float* p, int64_t n_tiles, uint8_t* codes,
                          float* scale_inv, uint8_t* near_mid, double rel, int pow2);

/* ---- The fused step: AdamW then per-tile requantization ----------- */
void ora_step(float* p, const float* g, float* m, float* v, int64_t n_tiles,
              const ora_hparams* hp, uint8_t* codes, float* scale_inv,
              uint8_t* near_mid, double rel);
void ora_step_mode(float* p, const float* g, float* m, float* v, int64_t n_tiles,
                   const ora_hparams* hp, uint8_t* codes, float* scale_inv,
                   uint8_t* near_mid, double rel, int pow2);

#ifdef __cplusplus
}
#endif
#endif
