/*
 * coli_ref.h — CPU oracle of one routed Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY. This library is the plain, slow definition that the
 * GPU library is checked against. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; no product code path calls it.
 * It shares no code, header, table or constant with the GPU library.
 *
 * What it computes, and where the pages state it:
 *   - Q8_0-style int8 activations, 32-element blocks, scale = max|x| / 127
 *     (colibri-strix README, "What's implemented", integer-dot kernels item).
 *   - int8 / packed int4 / packed int2 weights with one fp32 scale per output
 *     row, dequantised on use; packing must round-trip bit-identically
 *     (colibri-strix README, "What's implemented", quantization kernels item).
 *   - DeepSeek-V3-style sigmoid router, noaux_tc with routed_scaling_factor, and
 *     a shared expert (colibri-strix README, "What's implemented", router item).
 *   - Batch-union grouping: every distinct expert of the batch is applied to all
 *     positions routed to it (colibri-strix README, "What's implemented",
 *     batch-union item; JustVugg/colibri README, "Never wait for the disk twice").
 *     The union changes which weights are read once, never the result, so the
 *     layer oracle evaluates pair by pair.
 *
 * Every floating-point step is carried in double except where a stored format
 * fixes fp32: the activation x and h fed to Q8_0 are fp32, the Q8_0 scale d is
 * fp32, the router weights handed out are fp32, and the layer output is fp32.
 *
 * All pointers are host pointers owned by the caller. Functions return 0 on
 * success and a negative value when an argument is invalid; nothing is written
 * in that case.
 */
#ifndef COLI_REF_H
#define COLI_REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t hidden;       /* H, multiple of 32 */
  int32_t ffn;          /* F, multiple of 32 */
  int32_t n_experts;    /* E routed experts */
  int32_t top_k;        /* k */
  int32_t n_group;      /* G, divides E */
  int32_t topk_group;   /* Gk, 1 <= Gk <= G */
  float   rsf;          /* routed_scaling_factor */
  int32_t has_shared;   /* 0/1: shared expert stored after the routed ones */
  int32_t wbits;        /* 2, 4, 8, or COLI_REF_W_MXFP4 */
  int32_t scale_group;  /* 0: one fp32 scale per row; 64: one per 64 consecutive inputs of a row;
                           32 (and only 32) with COLI_REF_W_MXFP4: one E8M0 byte per block */
  float   topp;         /* 0: plain top-k; 0 < topp <= 1: adaptive expert top-p (see coli_ref_moe_route) */
} coli_ref_cfg;

/* MXFP4 weights (the Kimi K3 / DeepSeek V4 expert format named on the JustVugg/colibri
 * README, "Other supported models"; the pages name it only, so the element and scale
 * encodings are the OCP Microscaling (MX) v1.0 ones): blocks of 32 E2M1 codes sharing
 * one E8M0 scale byte. A code c = s e1 e0 m (bit 3 .. bit 0) is (-1)^s * 2^(e - 1) *
 * (1 + m / 2) for e > 0 and (-1)^s * m / 2 for e = 0; a scale byte u is 2^(u - 127),
 * and u = 255 is NaN. Packed as int4 (code j in the low nibble of byte j, code j + 16 in
 * the high nibble, per block); scales per expert: gate [F][H/32] | up [F][H/32] |
 * down [H][F/32] bytes. */
#define COLI_REF_W_MXFP4 40

/* Value of one E2M1 code (0..15) and of one E8M0 byte. */
double coli_ref_e2m1(uint32_t code);
double coli_ref_e8m0(uint32_t u);

/* E2M1 values of n packed codes (n % 32 == 0), in value order. */
int coli_ref_mxfp4_decode(const uint8_t *in, int64_t n, double *v);

/* Q8_0 of rows x cols fp32 values (cols % 32 == 0): q int8 [rows, cols], d fp32 [rows, cols/32]. */
int coli_ref_quantize_q8_0(const float *x, int64_t rows, int32_t cols, int8_t *q, float *d);

/* Packed row layout. n values (n % 32 == 0), grouped in 32-value blocks.
 * int8: one byte per value. int4: 16 bytes per block, byte j holds value j in
 * its low nibble and value j+16 in its high nibble (two's complement).
 * int2: 8 bytes per block, byte j holds value j+8m in bits 2m..2m+1, m=0..3. */
int coli_ref_pack(int32_t wbits, const int8_t *q, int64_t n, uint8_t *out);
int coli_ref_unpack(int32_t wbits, const uint8_t *in, int64_t n, int8_t *q);

/* Router for T tokens: topk_idx int32 [T, k], topk_w fp32 [T, k]. With topp > 0 (adaptive
 * expert top-p, the --topp knob of the colibri-strix README, "Experimental resident CUDA backend",
 * useful-knobs paragraph) only the shortest prefix of the
 * k slots whose summed scores reach topp of the k slots' sum is kept (at least one slot); the
 * kept weights are renormalised over the kept slots and the dropped slots hold index -1 and
 * weight 0. The grouping and the FFN skip index -1. */
int coli_ref_moe_route(const coli_ref_cfg *cfg, const float *router_w, const float *router_bias,
                       const float *x, int32_t T, int32_t *topk_idx, float *topk_w);

/* Same as coli_ref_moe_route, and also the fp64 scores s = sigmoid(z) [T, E]. */
int coli_ref_moe_route_scores(const coli_ref_cfg *cfg, const float *router_w, const float *router_bias,
                              const float *x, int32_t T, int32_t *topk_idx, float *topk_w,
                              double *scores);

/* Batch-union grouping of the T*k pairs (pair id p = t*k + j). */
int coli_ref_moe_group(const coli_ref_cfg *cfg, const int32_t *topk_idx, int32_t T,
                       int32_t *expert_cnt /*[E]*/, int32_t *expert_off /*[E+1]*/,
                       int32_t *pair_perm /*[T*k]*/, int32_t *active /*[E]*/, int32_t *n_active);

/* One expert applied to one Q8_0 activation row, with every intermediate.
 * blob: gate[F] | up[F] | down[H] packed rows. scales (fp32): with scale_group 0,
 * [2F + H] one per row (gate rows, up rows, down rows); with scale_group 64, one
 * per 64 inputs of a row, gate [F][H/64] | up [F][H/64] | down [H][F/64]; with
 * MXFP4 weights, E8M0 bytes, one per 32 inputs of a row in the same order.
 * Outputs (any may be NULL): g, u double [F]; h fp32 [F]; hq int8 [F];
 * hd fp32 [F/32]; y double [H]. */
int coli_ref_expert_ffn(int32_t hidden, int32_t ffn, int32_t wbits, int32_t scale_group, const uint8_t *blob,
                        const void *scales, const int8_t *xq, const float *xd,
                        double *g, double *u, float *h, int8_t *hq, float *hd, double *y);

/* Expert FFNs and combine for given routing. experts: (E + has_shared) blobs of
 * blob stride bytes; scales: (E + has_shared) x (scales of one expert, as above; fp32,
 * or bytes for MXFP4). out fp32 [T, H]. */
int coli_ref_moe_ffn(const coli_ref_cfg *cfg, const uint8_t *experts, const void *scales,
                     const float *x, int32_t T, const int32_t *topk_idx, const float *topk_w,
                     float *out);

/* Whole layer: route, then FFN and combine. */
int coli_ref_moe_layer(const coli_ref_cfg *cfg, const uint8_t *experts, const void *scales,
                       const float *router_w, const float *router_bias, const float *x, int32_t T,
                       float *out, int32_t *topk_idx_opt, float *topk_w_opt);

/* Bytes of one packed row of n values, and of one expert blob. */
int64_t coli_ref_row_bytes(int32_t wbits, int32_t n);
int64_t coli_ref_blob_bytes(int32_t hidden, int32_t ffn, int32_t wbits);

/* Threads the OpenMP build may use (1 when built without OpenMP); set_threads(0) keeps the default. */
int coli_ref_threads(void);
void coli_ref_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
