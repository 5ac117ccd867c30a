/*
 * coli_ref.c — CPU oracle of one routed MoE layer (plain C, slow, obvious).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path. Shares nothing with
 * the GPU library. Built with -O2 -ffp-contract=off -fno-fast-math so that every
 * floating-point operation below is the single IEEE operation it reads as.
 *
 * The pages describe the method in prose only. Each function names the passage
 * it follows; where the pages leave a step open the comment states the reading
 * taken. Parity pins for every function live in the test suite.
 */
#include "coli_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QK 32 /* Q8_0 block length, fixed by the workload statement (32-element blocks) */

int coli_ref_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void coli_ref_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int64_t coli_ref_row_bytes(int32_t wbits, int32_t n) {
  if (n <= 0 || n % QK) return -1;
  if (wbits == COLI_REF_W_MXFP4) return (int64_t)n / 2; /* 4-bit codes; the scales are stored apart */
  if (wbits != 2 && wbits != 4 && wbits != 8) return -1;
  return (int64_t)n * wbits / 8;
}

int64_t coli_ref_blob_bytes(int32_t hidden, int32_t ffn, int32_t wbits) {
  int64_t rh = coli_ref_row_bytes(wbits, hidden), rf = coli_ref_row_bytes(wbits, ffn);
  if (rh < 0 || rf < 0) return -1;
  return 2 * (int64_t)ffn * rh + (int64_t)hidden * rf;
}

/* ---------------------------------------------------------------- Q8_0 --
 * colibri-strix README, "What's implemented", integer-dot kernels item:
 * activations become Q8_0-style int8. Per 32-value block: d = max|x| / 127 as
 * one fp32 division; q = round-half-away-from-zero(x / d) clamped to [-127, 127];
 * an all-zero block has d = 0 and q = 0. (Reading: d kept in fp32 rather than
 * fp16, and a true division rather than a reciprocal, so that one correctly
 * rounded operation defines every code.) */
static void q8_0_block(const float *x, int8_t *q, float *d) {
  float amax = 0.0f;
  for (int i = 0; i < QK; i++) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float dd = amax / 127.0f;
  *d = dd;
  for (int i = 0; i < QK; i++) {
    if (dd == 0.0f) {
      q[i] = 0;
      continue;
    }
    float v = roundf(x[i] / dd);
    if (v > 127.0f) v = 127.0f;
    if (v < -127.0f) v = -127.0f;
    q[i] = (int8_t)v;
  }
}

int coli_ref_quantize_q8_0(const float *x, int64_t rows, int32_t cols, int8_t *q, float *d) {
  if (!x || !q || !d || rows < 0 || cols <= 0 || cols % QK) return -1;
  int32_t nb = cols / QK;
  for (int64_t r = 0; r < rows; r++)
    for (int32_t b = 0; b < nb; b++)
      q8_0_block(x + r * cols + (int64_t)b * QK, q + r * cols + (int64_t)b * QK, d + r * nb + b);
  return 0;
}

/* ------------------------------------------------------------ pack/unpack --
 * colibri-strix README, "What's implemented", quantization kernels item: int8,
 * packed int4 and packed int2 weights with per-row scales; packing must
 * reproduce the int8 values bit-identically. The pages do not print the bit
 * layout; the one used here (two's-complement fields, value j with j+16 for
 * int4, value j with j+8, j+16, j+24 for int2, per 32-value block) is this
 * build's own container format. */
int coli_ref_pack(int32_t wbits, const int8_t *q, int64_t n, uint8_t *out) {
  if (!q || !out || n < 0 || n % QK) return -1;
  for (int64_t b = 0; b < n / QK; b++) {
    const int8_t *v = q + b * QK;
    if (wbits == 8) {
      for (int i = 0; i < QK; i++) out[b * QK + i] = (uint8_t)v[i];
    } else if (wbits == 4) {
      for (int i = 0; i < QK; i++)
        if (v[i] < -8 || v[i] > 7) return -2;
      for (int j = 0; j < 16; j++)
        out[b * 16 + j] = (uint8_t)(((unsigned)v[j] & 0xFu) | (((unsigned)v[j + 16] & 0xFu) << 4));
    } else if (wbits == 2) {
      for (int i = 0; i < QK; i++)
        if (v[i] < -2 || v[i] > 1) return -2;
      for (int j = 0; j < 8; j++) {
        unsigned byte = 0;
        for (int m = 0; m < 4; m++) byte |= ((unsigned)v[j + 8 * m] & 3u) << (2 * m);
        out[b * 8 + j] = (uint8_t)byte;
      }
    } else {
      return -1;
    }
  }
  return 0;
}

/* sign-extend the low `bits` bits of v */
static int8_t sext(unsigned v, int bits) {
  int x = (int)(v & ((1u << bits) - 1u));
  if (x >= (1 << (bits - 1))) x -= (1 << bits);
  return (int8_t)x;
}

int coli_ref_unpack(int32_t wbits, const uint8_t *in, int64_t n, int8_t *q) {
  if (!in || !q || n < 0 || n % QK) return -1;
  for (int64_t b = 0; b < n / QK; b++) {
    int8_t *v = q + b * QK;
    if (wbits == 8) {
      for (int i = 0; i < QK; i++) v[i] = (int8_t)in[b * QK + i];
    } else if (wbits == 4) {
      for (int j = 0; j < 16; j++) {
        unsigned byte = in[b * 16 + j];
        v[j] = sext(byte, 4);
        v[j + 16] = sext(byte >> 4, 4);
      }
    } else if (wbits == 2) {
      for (int j = 0; j < 8; j++) {
        unsigned byte = in[b * 8 + j];
        for (int m = 0; m < 4; m++) v[j + 8 * m] = sext(byte >> (2 * m), 2);
      }
    } else {
      return -1;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ MXFP4 --
 * The element and scale encodings of the OCP MX formats (the pages name MXFP4
 * experts without spelling the format out): E2M1 has one sign bit, two exponent
 * bits of bias 1 and one mantissa bit; exponent field 0 holds the subnormals 0 and
 * 1/2. E8M0 is a bare biased exponent, 2^(u - 127), with u = 255 reserved for NaN. */
double coli_ref_e2m1(uint32_t code) {
  const uint32_t sgn = (code >> 3) & 1u, ex = (code >> 1) & 3u, man = code & 1u;
  const double mag = ex == 0 ? 0.5 * man : ldexp(1.0 + 0.5 * man, (int)ex - 1);
  return sgn ? -mag : mag;
}

double coli_ref_e8m0(uint32_t u) {
  if (u > 255) return NAN;
  return u == 255 ? NAN : ldexp(1.0, (int)u - 127);
}

int coli_ref_mxfp4_decode(const uint8_t *in, int64_t n, double *v) {
  if (!in || !v || n < 0 || n % QK) return -1;
  for (int64_t b = 0; b < n / QK; b++)
    for (int j = 0; j < 16; j++) {
      const unsigned byte = in[b * 16 + j];
      v[b * QK + j] = coli_ref_e2m1(byte & 0xFu);
      v[b * QK + j + 16] = coli_ref_e2m1(byte >> 4);
    }
  return 0;
}

/* ------------------------------------------------------------------ router --
 * colibri-strix README, "What's implemented", router item: DeepSeek-V3-style
 * sigmoid router, noaux_tc, routed_scaling_factor. The pages name the scheme
 * without spelling it out; the reading taken is the DeepSeek-V3 convention:
 *   z_e = x . W_e (fp64), s_e = 1 / (1 + exp(-z_e)), c_e = s_e + bias_e;
 *   experts form G contiguous groups; a group's score is the sum of its two
 *   largest c (its single c when a group has one expert);
 *   the Gk best groups are kept (score descending, lower index first on ties);
 *   the k best experts by c inside the kept groups are the route, in that order
 *   (lower index first on ties); experts outside the kept groups are excluded;
 *   the bias steers selection only: w_j = s_{e_j} / sum_j s_{e_j} * rsf. */
static int cfg_ok(const coli_ref_cfg *c) {
  if (!c) return 0;
  if (c->hidden <= 0 || c->hidden % QK || c->ffn <= 0 || c->ffn % QK) return 0;
  if (c->n_experts <= 0 || c->n_group <= 0 || c->n_experts % c->n_group) return 0;
  if (c->topk_group < 1 || c->topk_group > c->n_group) return 0;
  if (c->top_k < 1 || c->top_k > c->topk_group * (c->n_experts / c->n_group)) return 0;
  if (c->wbits != 2 && c->wbits != 4 && c->wbits != 8 && c->wbits != COLI_REF_W_MXFP4) return 0;
  if (c->has_shared != 0 && c->has_shared != 1) return 0;
  if (c->wbits == COLI_REF_W_MXFP4 ? c->scale_group != 32 : (c->scale_group != 0 && c->scale_group != 64)) return 0;
  if (c->scale_group && (c->hidden % c->scale_group || c->ffn % c->scale_group)) return 0;
  if (!(c->topp >= 0.0f && c->topp <= 1.0f)) return 0;
  return 1;
}

static void route_token(const coli_ref_cfg *cfg, const float *W, const float *bias, const float *x,
                        double *s, double *c, double *gscore, char *gpick, char *taken,
                        int32_t *idx, float *w) {
  const int E = cfg->n_experts, H = cfg->hidden, G = cfg->n_group, m = E / G;
  for (int e = 0; e < E; e++) {
    double z = 0.0;
    for (int h = 0; h < H; h++) z += (double)x[h] * (double)W[(int64_t)e * H + h];
    s[e] = 1.0 / (1.0 + exp(-z));
    c[e] = s[e] + (double)bias[e];
  }
  for (int g = 0; g < G; g++) {
    const double *cg = c + (int64_t)g * m;
    if (m == 1) {
      gscore[g] = cg[0];
      continue;
    }
    int a = 0; /* position of the largest (lowest index on ties) */
    for (int i = 1; i < m; i++)
      if (cg[i] > cg[a]) a = i;
    int b = -1; /* largest of the rest */
    for (int i = 0; i < m; i++)
      if (i != a && (b < 0 || cg[i] > cg[b])) b = i;
    gscore[g] = cg[a] + cg[b];
  }
  memset(gpick, 0, (size_t)G);
  for (int r = 0; r < cfg->topk_group; r++) {
    int best = -1;
    for (int g = 0; g < G; g++)
      if (!gpick[g] && (best < 0 || gscore[g] > gscore[best])) best = g;
    gpick[best] = 1;
  }
  memset(taken, 0, (size_t)E);
  for (int j = 0; j < cfg->top_k; j++) {
    int best = -1;
    for (int e = 0; e < E; e++) {
      if (!gpick[e / m] || taken[e]) continue;
      if (best < 0 || c[e] > c[best]) best = e;
    }
    taken[best] = 1;
    idx[j] = best;
  }
  double S = 0.0;
  for (int j = 0; j < cfg->top_k; j++) S += s[idx[j]];
  int kept = cfg->top_k;
  if (cfg->topp > 0.0f) {
    /* adaptive top-p: the shortest prefix of the slots (descending c) whose summed
     * scores reach topp * S; its sum, in the same order, renormalises the weights */
    const double target = (double)cfg->topp * S;
    double cum = 0.0;
    for (int j = 0; j < cfg->top_k; j++) {
      cum += s[idx[j]];
      if (cum >= target) {
        kept = j + 1;
        break;
      }
    }
    S = cum;
  }
  for (int j = 0; j < cfg->top_k; j++) {
    if (j < kept) {
      w[j] = (float)((s[idx[j]] / S) * (double)cfg->rsf);
    } else {
      idx[j] = -1;
      w[j] = 0.0f;
    }
  }
}

int coli_ref_moe_route_scores(const coli_ref_cfg *cfg, const float *router_w, const float *router_bias,
                              const float *x, int32_t T, int32_t *topk_idx, float *topk_w,
                              double *scores) {
  if (!cfg_ok(cfg) || !router_w || !router_bias || T < 0 || (T > 0 && (!x || !topk_idx || !topk_w)))
    return -1;
  const int E = cfg->n_experts, G = cfg->n_group, k = cfg->top_k;
  int bad = 0;
#pragma omp parallel
  {
    double *s = malloc(sizeof(double) * E), *c = malloc(sizeof(double) * E),
           *gs = malloc(sizeof(double) * G);
    char *gp = malloc((size_t)G), *tk = malloc((size_t)E);
    if (!s || !c || !gs || !gp || !tk) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(static)
      for (int32_t t = 0; t < T; t++) {
        route_token(cfg, router_w, router_bias, x + (int64_t)t * cfg->hidden, s, c, gs, gp, tk,
                    topk_idx + (int64_t)t * k, topk_w + (int64_t)t * k);
        if (scores) memcpy(scores + (int64_t)t * E, s, sizeof(double) * E);
      }
    }
    free(s); free(c); free(gs); free(gp); free(tk);
  }
  return bad ? -3 : 0;
}

int coli_ref_moe_route(const coli_ref_cfg *cfg, const float *router_w, const float *router_bias,
                       const float *x, int32_t T, int32_t *topk_idx, float *topk_w) {
  return coli_ref_moe_route_scores(cfg, router_w, router_bias, x, T, topk_idx, topk_w, NULL);
}

/* ------------------------------------------------------------------- group --
 * colibri-strix README, "What's implemented", batch-union item: the weights of an
 * expert are fetched a single time per batch, however many tokens chose it.
 * The grouping lists, per expert, its pairs p = t*k + j in ascending p (a stable
 * counting sort by expert), the exclusive offsets into that list, and the
 * experts that received at least one pair, ascending. */
int coli_ref_moe_group(const coli_ref_cfg *cfg, const int32_t *topk_idx, int32_t T,
                       int32_t *expert_cnt, int32_t *expert_off, int32_t *pair_perm,
                       int32_t *active, int32_t *n_active) {
  if (!cfg_ok(cfg) || T < 0 || !expert_cnt || !expert_off || !active || !n_active) return -1;
  const int E = cfg->n_experts;
  const int64_t P = (int64_t)T * cfg->top_k;
  if (P > 0 && (!topk_idx || !pair_perm)) return -1;
  /* index -1 is an empty slot (adaptive top-p): part of no expert */
  for (int64_t p = 0; p < P; p++)
    if (topk_idx[p] < -1 || topk_idx[p] >= E) return -2;
  for (int e = 0; e < E; e++) expert_cnt[e] = 0;
  for (int64_t p = 0; p < P; p++)
    if (topk_idx[p] >= 0) expert_cnt[topk_idx[p]]++;
  expert_off[0] = 0;
  for (int e = 0; e < E; e++) expert_off[e + 1] = expert_off[e] + expert_cnt[e];
  int32_t *fill = malloc(sizeof(int32_t) * (size_t)E);
  if (!fill) return -3;
  for (int e = 0; e < E; e++) fill[e] = expert_off[e];
  for (int64_t p = 0; p < P; p++)
    if (topk_idx[p] >= 0) pair_perm[fill[topk_idx[p]]++] = (int32_t)p;
  free(fill);
  int32_t u = 0;
  for (int e = 0; e < E; e++)
    if (expert_cnt[e] > 0) active[u++] = e;
  *n_active = u;
  return 0;
}

/* -------------------------------------------------------------- expert FFN --
 * One expert on one activation row. The expert is the usual gated FFN of this
 * model family (SiLU(gate) * up, then down); the weights are dequantised on use
 * (colibri-strix README, "What's implemented", quantization kernels item) and
 * multiplied with Q8_0 activations by integer dots (integer-dot kernels item):
 *   I_b(row) = sum over the 32 values of block b of xq * wq    (exact int32)
 *   g_f = s_gate[f] * sum_b xd_b * I_b(gate row f)           (double)
 *   u_f = s_up[f]   * sum_b xd_b * I_b(up row f)             (double)
 *   h_f = g_f / (1 + exp(-g_f)) * u_f, stored as fp32 (the input of Q8_0)
 *   hq, hd = Q8_0(h)
 *   y_r = s_down[r] * sum_b hd_b * I_b(down row r)           (double)
 * With group scales (one per 64 inputs of a row; JustVugg/colibri README, "2. Get
 * the model": the gs64 int4 container) the dequantised weight is s_row,grp * q, so
 * a row's dot is sum over groups s_grp * sum_{b in grp} d_b * I_b: a 32-value
 * block lies inside one group. */
static int64_t block_dot(const int8_t *a, const int8_t *b) {
  int64_t acc = 0;
  for (int i = 0; i < QK; i++) acc += (int64_t)a[i] * (int64_t)b[i];
  return acc;
}

static double row_dot(const int8_t *wrow, const int8_t *aq, const float *ad, int32_t n) {
  double acc = 0.0;
  for (int32_t b = 0; b < n / QK; b++)
    acc += (double)ad[b] * (double)block_dot(aq + (int64_t)b * QK, wrow + (int64_t)b * QK);
  return acc;
}

/* MXFP4 row: the weight is e2m1(code) * 2^(u_b - 127) with one scale byte u_b per
 * 32-value block, so a row's dot is sum_b d_b * 2^(u_b - 127) * J_b, J_b = sum over the
 * block of xq * e2m1 (a multiple of 1/2, exact in double). */
static double mx_row_dot(const uint8_t *row, const uint8_t *u, const int8_t *aq, const float *ad, int32_t n) {
  double acc = 0.0;
  for (int32_t b = 0; b < n / QK; b++) {
    double j = 0.0;
    for (int i = 0; i < 16; i++) {
      const unsigned byte = row[(int64_t)b * 16 + i];
      j += (double)aq[(int64_t)b * QK + i] * coli_ref_e2m1(byte & 0xFu);
      j += (double)aq[(int64_t)b * QK + i + 16] * coli_ref_e2m1(byte >> 4);
    }
    acc += (double)ad[b] * coli_ref_e8m0(u[b]) * j;
  }
  return acc;
}

/* The scaled dot of one row: s[0] * row_dot with one scale per row (gs = 0), else
 * sum over the n / gs groups of s[grp] * (the row_dot of that group's inputs). */
static double scaled_row_dot(const int8_t *wrow, const int8_t *aq, const float *ad, int32_t n, int32_t gs,
                             const float *s) {
  if (gs == 0) return (double)s[0] * row_dot(wrow, aq, ad, n);
  double acc = 0.0;
  for (int32_t grp = 0; grp < n / gs; grp++)
    acc += (double)s[grp] * row_dot(wrow + (int64_t)grp * gs, aq + (int64_t)grp * gs, ad + grp * (gs / QK), gs);
  return acc;
}

int coli_ref_expert_ffn(int32_t hidden, int32_t ffn, int32_t wbits, int32_t scale_group, const uint8_t *blob,
                        const void *scales, const int8_t *xq, const float *xd,
                        double *g_out, double *u_out, float *h_out, int8_t *hq_out, float *hd_out,
                        double *y_out) {
  const int64_t rh = coli_ref_row_bytes(wbits, hidden), rf = coli_ref_row_bytes(wbits, ffn);
  if (rh < 0 || rf < 0 || !blob || !scales || !xq || !xd) return -1;
  const int mx = wbits == COLI_REF_W_MXFP4;
  if (mx ? scale_group != 32 : (scale_group != 0 && (scale_group != 64 || hidden % 64 || ffn % 64))) return -1;
  const int32_t H = hidden, F = ffn, gs = scale_group;
  /* scales of one row of each matrix: per-row index, or [row][group] */
  const int64_t sgh = gs ? H / gs : 1, sgf = gs ? F / gs : 1;
  const float *sg = scales, *su = sg + (int64_t)F * sgh, *sd = sg + 2 * (int64_t)F * sgh;
  const uint8_t *ug = scales, *uu = ug + (int64_t)F * sgh, *ud = ug + 2 * (int64_t)F * sgh; /* MXFP4 */
  int8_t *wrow = malloc((size_t)(H > F ? H : F));
  float *h = malloc(sizeof(float) * (size_t)F);
  int8_t *hq = malloc((size_t)F);
  float *hd = malloc(sizeof(float) * (size_t)(F / QK));
  if (!wrow || !h || !hq || !hd) {
    free(wrow); free(h); free(hq); free(hd);
    return -3;
  }
  const uint8_t *gate = blob, *up = blob + (int64_t)F * rh, *down = blob + 2 * (int64_t)F * rh;
  for (int32_t f = 0; f < F; f++) {
    double g, u;
    if (mx) {
      g = mx_row_dot(gate + (int64_t)f * rh, ug + f * sgh, xq, xd, H);
      u = mx_row_dot(up + (int64_t)f * rh, uu + f * sgh, xq, xd, H);
    } else {
      coli_ref_unpack(wbits, gate + (int64_t)f * rh, H, wrow);
      g = scaled_row_dot(wrow, xq, xd, H, gs, sg + f * sgh);
      coli_ref_unpack(wbits, up + (int64_t)f * rh, H, wrow);
      u = scaled_row_dot(wrow, xq, xd, H, gs, su + f * sgh);
    }
    h[f] = (float)(g / (1.0 + exp(-g)) * u);
    if (g_out) g_out[f] = g;
    if (u_out) u_out[f] = u;
  }
  coli_ref_quantize_q8_0(h, 1, F, hq, hd);
  if (y_out)
    for (int32_t r = 0; r < H; r++) {
      if (mx) {
        y_out[r] = mx_row_dot(down + (int64_t)r * rf, ud + r * sgf, hq, hd, F);
      } else {
        coli_ref_unpack(wbits, down + (int64_t)r * rf, F, wrow);
        y_out[r] = scaled_row_dot(wrow, hq, hd, F, gs, sd + r * sgf);
      }
    }
  if (h_out) memcpy(h_out, h, sizeof(float) * (size_t)F);
  if (hq_out) memcpy(hq_out, hq, (size_t)F);
  if (hd_out) memcpy(hd_out, hd, sizeof(float) * (size_t)(F / QK));
  free(wrow); free(h); free(hq); free(hd);
  return 0;
}

/* -------------------------------------------------------------- FFN + combine --
 * Per token t: out_t = sum_j w_tj * y_{e_tj}(x_t) + y_shared(x_t), summed in
 * double in slot order j = 0..k-1 with the shared expert last (weight 1), then
 * rounded once to fp32. The shared expert is always applied (colibri-strix
 * README, "What's implemented", router item; "The idea": shared experts are part
 * of the dense, always-resident set). */
int coli_ref_moe_ffn(const coli_ref_cfg *cfg, const uint8_t *experts, const void *scales,
                     const float *x, int32_t T, const int32_t *topk_idx, const float *topk_w,
                     float *out) {
  if (!cfg_ok(cfg) || T < 0 || !experts || !scales) return -1;
  if (T == 0) return 0;
  if (!x || !topk_idx || !topk_w || !out) return -1;
  const int32_t H = cfg->hidden, F = cfg->ffn, k = cfg->top_k, E = cfg->n_experts;
  const int64_t blob = coli_ref_blob_bytes(H, F, cfg->wbits);
  const int32_t gs = cfg->scale_group;
  const int64_t srow = gs ? 3 * (int64_t)F * (H / gs) : 2 * (int64_t)F + H;  /* scales per expert */
  const int64_t sbytes = srow * (cfg->wbits == COLI_REF_W_MXFP4 ? 1 : (int64_t)sizeof(float));
  for (int64_t p = 0; p < (int64_t)T * k; p++)
    if (topk_idx[p] < -1 || topk_idx[p] >= E) return -2;  /* -1: empty slot (adaptive top-p) */
  const int nslot = k + (cfg->has_shared ? 1 : 0);
  int bad = 0;
#pragma omp parallel
  {
    int8_t *xq = malloc((size_t)H);
    float *xd = malloc(sizeof(float) * (size_t)(H / QK));
    double *y = malloc(sizeof(double) * (size_t)H * (size_t)nslot);
    if (!xq || !xd || !y) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int32_t t = 0; t < T; t++) {
        coli_ref_quantize_q8_0(x + (int64_t)t * H, 1, H, xq, xd);
        for (int j = 0; j < nslot; j++) {
          int64_t e = j < k ? topk_idx[(int64_t)t * k + j] : E; /* shared expert stored after the routed ones */
          if (e < 0) continue;                                  /* empty slot: weight 0, never read */
          coli_ref_expert_ffn(H, F, cfg->wbits, gs, experts + e * blob, (const uint8_t *)scales + e * sbytes, xq, xd,
                              NULL, NULL, NULL, NULL, NULL, y + (int64_t)j * H);
        }
        for (int32_t r = 0; r < H; r++) {
          double acc = 0.0;
          for (int j = 0; j < k; j++)
            if (topk_idx[(int64_t)t * k + j] >= 0) acc += (double)topk_w[(int64_t)t * k + j] * y[(int64_t)j * H + r];
          if (cfg->has_shared) acc += y[(int64_t)k * H + r];
          out[(int64_t)t * H + r] = (float)acc;
        }
      }
    }
    free(xq); free(xd); free(y);
  }
  return bad ? -3 : 0;
}

int coli_ref_moe_layer(const coli_ref_cfg *cfg, const uint8_t *experts, const void *scales,
                       const float *router_w, const float *router_bias, const float *x, int32_t T,
                       float *out, int32_t *topk_idx_opt, float *topk_w_opt) {
  if (!cfg_ok(cfg) || T < 0) return -1;
  if (T == 0) return 0;
  const int64_t P = (int64_t)T * cfg->top_k;
  int32_t *idx = topk_idx_opt ? topk_idx_opt : malloc(sizeof(int32_t) * (size_t)P);
  float *w = topk_w_opt ? topk_w_opt : malloc(sizeof(float) * (size_t)P);
  int rc = (!idx || !w) ? -3 : coli_ref_moe_route(cfg, router_w, router_bias, x, T, idx, w);
  if (rc == 0) rc = coli_ref_moe_ffn(cfg, experts, scales, x, T, idx, w, out);
  if (!topk_idx_opt) free(idx);
  if (!topk_w_opt) free(w);
  return rc;
}
