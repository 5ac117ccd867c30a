/*
 * coli_moe_taps.h — test-only entry points of libcolimoe_taps.so, the same HIP
 * sources as libcolimoe.so compiled with COLI_TAPS. The product library does not
 * export these symbols and its kernels contain no tap code.
 *
 * Why: the integer-dot kernels item of the colibri-strix README ("What's
 * implemented") multiplies Q8_0 activations with the quantised weights by integer
 * block dots. The gate and up values of a row are g = s * sum_b d_b * I_b and
 * u likewise, with I_b the exact int32 dot of block b. The layer output only sees
 * them through SiLU and an 8-bit requantisation of h, which hides small errors in
 * one I_b. The taps expose g and u themselves, before SiLU, exactly as the
 * epilogue of every gate/up kernel (GEMV or grouped GEMM) computes them, so that a
 * test can pin each block dot bit for bit: with one non-zero Q8_0 block in a
 * token's activations (block scale exactly 1) and unit weight scales, g = I_b.
 *
 * tap_gu: DEVICE fp32 [P + has_shared * T][2F], caller-owned, P = T * top_k. Row p
 * (pair p = t * top_k + j) holds g[0..F) then u[0..F) of that token's j-th routed
 * expert; row P + t those of the shared expert for token t. Rows of empty slots
 * (adaptive top-p) are not written. Everything else (arguments, validation, status
 * codes, results) is as for coli_moe_layer / coli_moe_ffn in coli_moe.h;
 * COLI_E_INVALID also when tap_gu is NULL or not 4-byte aligned.
 */
#ifndef COLI_MOE_TAPS_H
#define COLI_MOE_TAPS_H

#include "coli_moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* coli_moe_layer, recording the pre-SiLU gate and up values of every output row. */
int coli_moe_layer_taps(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T, float *out,
                        int32_t *topk_idx_opt, float *topk_w_opt, float *tap_gu, void *workspace, size_t ws_bytes,
                        void *stream);

/* coli_moe_ffn, recording the pre-SiLU gate and up values of every output row. */
int coli_moe_ffn_taps(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T,
                      const int32_t *topk_idx, const float *topk_w, const int32_t *expert_off, const int32_t *pair_perm,
                      const int32_t *active, const int32_t *n_active, float *out, float *tap_gu, void *workspace,
                      size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif
