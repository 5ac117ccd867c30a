/*
 * coli_moe.h — C ABI of libcolimoe.so: one routed Mixture-of-Experts layer on
 * an AMD Instinct MI355X (gfx950), in hand-written HIP kernels.
 *
 * The layer, as the Colibri pages state it:
 *   - router: DeepSeek-V3-style sigmoid router, noaux_tc, routed_scaling_factor,
 *     plus a shared expert (colibri-strix README, "What's implemented", router item);
 *   - batch-union: the weights of an expert are fetched a single time per batch,
 *     however many tokens chose it (colibri-strix README, "What's implemented",
 *     batch-union item; JustVugg/colibri README, "Never wait for the disk twice");
 *   - quantised experts: int8 / packed int4 / packed int2 weights with per-row
 *     scales, dequantised on use (colibri-strix README, "What's implemented",
 *     quantization kernels item), multiplied with Q8_0-style int8 activations by
 *     integer dots (same section, integer-dot kernels item).
 * The pages leave the router's group rule, the bit layouts and the rounding
 * rules open; the readings this library implements are spelled out below.
 *
 * Conventions for every entry point (the expert tier's host-side calls, at the end of
 * this header, state their own exceptions):
 *   - All array pointers are DEVICE pointers, allocated and owned by the caller.
 *     The library allocates no device memory and keeps no state between calls
 *     (coli_moe_layer_noalloc runs on a scratch array the library holds, see there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is
 *     enqueued asynchronously; no call synchronises the stream or copies device
 *     data to the host.
 *   - Arguments are validated on the host before anything is enqueued. On any
 *     negative status nothing has been enqueued and no output was touched.
 *   - T = 0 is a no-op that returns COLI_OK.
 *   - Faults inside kernels surface as HIP errors at the caller's next
 *     synchronisation, as with any HIP launch.
 *
 * Data layout (row-major throughout):
 *   x            fp32 [T][H]
 *   experts      (E + has_shared) expert blobs, blob i at experts + i * blob_bytes;
 *                a blob is gate[F rows] | up[F rows] | down[H rows] of packed rows;
 *                gate and up rows have H inputs, down rows have F inputs.
 *                The shared expert, when present, is blob E.
 *   scales       fp32, per expert (scale_group 0) [2F + H]: one per row, gate rows,
 *                up rows, down rows; or (scale_group 64) [3 F H / 64]: one per 64
 *                consecutive inputs of a row, gate [F][H/64] | up [F][H/64] |
 *                down [H][F/64]. Expert i's scales start at i * coli_moe_scales_per_expert.
 *                (Group scales: JustVugg/colibri README, "2. Get the model", the gs64
 *                int4 container; the pages fix neither the scale type nor the layout,
 *                this library reads them as fp32 in that order.)
 *                MXFP4 (wfmt COLI_W_MXFP4, scale_group 32): bytes, not fp32: one E8M0
 *                code u per 32 inputs of a row, gate [F][H/32] | up [F][H/32] |
 *                down [H][F/32]; expert i's bytes start at i * coli_moe_scales_per_expert.
 *   router_w     fp32 [E][H];  router_bias fp32 [E] (noaux_tc correction bias).
 *   Packed row of n inputs = n/32 blocks of 32 values, two's complement:
 *     int8 (wfmt 8): 32 bytes/block, byte i = value i;
 *     int4 (wfmt 4): 16 bytes/block, byte j = value j | value (j+16) << 4;
 *     int2 (wfmt 2):  8 bytes/block, byte j = sum_m value (j+8m) << 2m, m = 0..3;
 *     MXFP4 (wfmt COLI_W_MXFP4): 16 bytes/block of 4-bit E2M1 codes, byte j = code j |
 *       code (j+16) << 4.
 *   Dequantised weight = scale[row] * value, or scale[row][input / 64] * value; MXFP4:
 *   e2m1(code) * 2^(u - 127) with the block's scale byte u (u = 255 is NaN).
 *   (MXFP4: the Kimi K3 / DeepSeek V4 expert format of JustVugg/colibri README, "Other
 *   supported models"; the pages name it only, so the encodings are OCP MX v1.0's:
 *   E2M1 = sign, two exponent bits of bias 1, one mantissa bit; E8M0 = 2^(u - 127).)
 *
 * Numerics (the readings):
 *   Q8_0: per 32-value block d = max|x| / 127 (one fp32 division, stored fp32),
 *     q = round-half-away-from-zero(x / d) clamped to [-127, 127]; d = 0 gives q = 0.
 *   Router: z = x . W_e accumulated in fp64 from exact fp32 products,
 *     s = 1 / (1 + exp(-z)) and c = s + bias in fp64; G contiguous groups of E/G
 *     experts scored by the sum of their two largest c (their c when E/G = 1);
 *     the Gk best groups kept; the k best c inside them are the route, in
 *     descending order; every tie goes to the lower index;
 *     w_j = (float)(s_j / sum_j s_j * rsf), the sum taken in slot order.
 *   Expert (SwiGLU): g = s_gate * sum_b xd_b * I_b (group scales: sum_b s_gate,b/2 *
 *     xd_b * I_b, a 32-value block lying inside one group; MXFP4: sum_b 2^(u_b - 127) *
 *     xd_b * J_b with J_b the exact block dot of the codes with their E2M1 values, a
 *     multiple of 1/2), u likewise with the up rows,
 *     where I_b is the exact int32 dot of block b; h = silu(g) * u in fp32;
 *     hq, hd = Q8_0(h); y = s_down * sum_b hd_b * I_b(hq, down row).
 *   Combine: out_t = sum_j w_tj * y_{e_tj} (j = 0..k-1 in order) + y_shared, fp32,
 *     no atomics: results are bitwise reproducible run to run.
 */
#ifndef COLI_MOE_H
#define COLI_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  COLI_OK = 0,
  COLI_E_INVALID = -1,     /* a config value or argument is invalid (NULL, negative size, bad enum) */
  COLI_E_UNSUPPORTED = -2, /* valid but outside this library's limits (see coli_moe_cfg) */
  COLI_E_WORKSPACE = -3,   /* workspace NULL or smaller than coli_moe_workspace_bytes(cfg, T) */
  COLI_E_ALIGN = -4,       /* a pointer is not aligned as documented */
  COLI_E_DEVICE = -5,      /* the HIP runtime rejected a launch */
  COLI_E_SCRATCH = -6      /* coli_moe_layer_noalloc: the batch needs more than coli_moe_scratch_bytes() */
} coli_status;

typedef enum { COLI_W_INT2 = 2, COLI_W_INT4 = 4, COLI_W_INT8 = 8, COLI_W_MXFP4 = 40 } coli_wfmt;

/* Layer shape. Limits: hidden and ffn multiples of 128; 1 <= n_experts <= 1024;
 * n_experts % n_group == 0; 1 <= topk_group <= n_group <= 64;
 * 1 <= top_k <= min(64, topk_group * n_experts / n_group); has_shared 0 or 1;
 * wfmt 2, 4, 8 (scale_group 0 or 64) or COLI_W_MXFP4 (scale_group 32); 0 <= topp <= 1. */
typedef struct {
  int32_t hidden;               /* H */
  int32_t ffn;                  /* F, width of every expert (shared included) */
  int32_t n_experts;            /* E routed experts */
  int32_t top_k;                /* k */
  int32_t n_group;              /* G */
  int32_t topk_group;           /* Gk */
  float routed_scaling_factor;  /* rsf */
  int32_t has_shared;           /* 1: blob E is a shared expert applied to every token */
  int32_t wfmt;                 /* coli_wfmt, one format for all experts of the layer */
  int32_t scale_group;          /* 0: one scale per weight row; 64: one per 64 inputs of a row;
                                   32: MXFP4's E8M0 byte per 32 inputs (MXFP4 only) */
  float topp;                   /* 0: plain top-k; 0 < topp <= 1: adaptive expert top-p (see the router) */
} coli_moe_cfg;

/* Device weights of one layer. experts: 16-byte aligned; router_w: 16-byte aligned;
 * scales, router_bias: 4-byte aligned. scales holds fp32 values, or E8M0 bytes for
 * MXFP4 (then passed as this pointer type). */
typedef struct {
  const void *experts;
  const float *scales;
  const float *router_w;
  const float *router_bias;
} coli_moe_weights;

/* Bytes of one packed expert blob (0 if cfg is invalid). */
size_t coli_moe_blob_bytes(const coli_moe_cfg *cfg);

/* Scales of one expert: 2F + H fp32 (scale_group 0), 3 F H / 64 fp32 (scale_group 64),
 * or 3 F H / 32 E8M0 bytes (MXFP4); 0 if cfg is invalid. */
size_t coli_moe_scales_per_expert(const coli_moe_cfg *cfg);

/* Workspace bytes that coli_moe_route / coli_moe_ffn / coli_moe_layer need for
 * up to T_max tokens (0 if cfg is invalid or T_max out of range). T_max * top_k
 * must not exceed 65535. The workspace must be 256-byte aligned. */
size_t coli_moe_workspace_bytes(const coli_moe_cfg *cfg, int32_t T_max);

/* Q8_0 quantisation of rows x cols fp32 values (cols % 32 == 0, x 16-byte aligned):
 * q int8 [rows][cols] (4-byte aligned), d fp32 [rows][cols/32].
 * Follows colibri-strix README, "What's implemented", integer-dot kernels item. */
int coli_moe_quantize_q8_0(const float *x, int64_t rows, int32_t cols, int8_t *q, float *d, void *stream);

/* Sigmoid noaux_tc router for T tokens: topk_idx int32 [T][k] (expert ids, slot
 * order), topk_w fp32 [T][k]. Uses the workspace for fp64 logits.
 * Follows colibri-strix README, "What's implemented", router item.
 * With cfg->topp > 0 (adaptive expert top-p, the --topp knob of the colibri-strix README,
 * "Experimental resident CUDA backend", useful-knobs paragraph; opt-in, it changes the router's result): only the shortest prefix of the k
 * slots whose scores s sum (fp64, slot order) to at least topp times the k slots' sum
 * is kept, at least one slot; the kept weights are s_j / (that prefix sum) * rsf, and
 * every dropped slot holds index -1 and weight 0. */
int coli_moe_route(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T,
                   int32_t *topk_idx, float *topk_w, void *workspace, size_t ws_bytes, void *stream);

/* Batch-union grouping of the T*k pairs p = t*k + j (no workspace):
 *   expert_cnt int32 [E]: pairs per expert;
 *   expert_off int32 [E+1]: exclusive prefix sum, expert_off[E] = T*k;
 *   pair_perm int32 [T*k]: pair ids sorted by (expert, p) ascending;
 *   active int32 [E]: experts with cnt > 0, ascending, in the first *n_active entries;
 *   n_active int32 [1].
 * topk_idx values must lie in [0, E) or be -1, an empty slot (adaptive top-p) that
 * belongs to no expert; other values are counted nowhere and leave n_active = -1
 * (checked by the kernel). expert_off[E] is then the number of non-empty pairs.
 * Follows colibri-strix README, "What's implemented", batch-union item. */
int coli_moe_group(const coli_moe_cfg *cfg, const int32_t *topk_idx, int32_t T, int32_t *expert_cnt,
                   int32_t *expert_off, int32_t *pair_perm, int32_t *active, int32_t *n_active,
                   void *stream);

/* Expert FFNs over the batch union and the combine, given a route and its
 * grouping (the outputs of coli_moe_route and coli_moe_group for the same T):
 * quantises x (Q8_0), runs gate/up with fused SiLU*up and Q8_0 requantisation,
 * runs down, then out fp32 [T][H] = slot-order weighted sum + shared expert.
 * Follows the router, batch-union, quantization-kernel and integer-dot items of
 * colibri-strix README, "What's implemented". */
int coli_moe_ffn(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T,
                 const int32_t *topk_idx, const float *topk_w, const int32_t *expert_off,
                 const int32_t *pair_perm, const int32_t *active, const int32_t *n_active, float *out,
                 void *workspace, size_t ws_bytes, void *stream);

/* The whole layer on one stream: route, group, FFN, combine. topk_idx_opt and
 * topk_w_opt ([T][k]) receive the route when non-NULL. For one token (T = 1, hidden a
 * multiple of 256, n_experts <= 512) the route's selection runs inside the gate/up
 * kernel instead of a kernel of its own; the route and the output are the same bit for
 * bit as coli_moe_route followed by coli_moe_group and coli_moe_ffn. */
int coli_moe_layer(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T, float *out,
                   int32_t *topk_idx_opt, float *topk_w_opt, void *workspace, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): coli_moe_layer without a workspace
 * argument. The work runs on a fixed scratch array that the library holds in device
 * memory, one per GPU (coli_moe_scratch_bytes() = 32 MiB each, allocated when the library's
 * code is loaded on that GPU and kept until the process ends); this call allocates
 * nothing and calls no allocating routine. The scratch belongs to the current device
 * (hipGetDevice), which must be the device of `stream` and of every pointer argument.
 * Every call on one GPU uses that GPU's single scratch array: calls that overlap on one
 * GPU (concurrent streams, or several host threads) race and corrupt each other's
 * results; serialise them, e.g. on one stream. Nothing in the scratch needs to start at
 * zero, and the contents left by the previous call are never read.
 * Returns COLI_E_SCRATCH, with nothing enqueued, when the batch needs more scratch than
 * that (coli_moe_workspace_bytes(cfg, T) > coli_moe_scratch_bytes(): GLM-5.2-scale decode
 * fits up to T = 112, OLMoE-scale up to T = 412); otherwise arguments, results and
 * statuses are those of coli_moe_layer, bit for bit. */
size_t coli_moe_scratch_bytes(void);
int coli_moe_layer_noalloc(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T, float *out,
                           int32_t *topk_idx_opt, float *topk_w_opt, void *stream);

/* Measurement variant of coli_moe_layer: events[i] (hipEvent_t passed as void*,
 * created by the caller) is recorded on `stream` just before stage i and
 * events[n_stages] after the last stage; n_events must be coli_moe_num_stages()+1.
 * A stage run inside another stage's kernel is empty (its two events back to back:
 * "group" below 513 (token, expert) pairs, "quantize_x" always (x is quantised by
 * the logits or the selection kernel), "route_select" for one token, whose selection
 * is timed in "ffn_gate_up"). Results are identical to coli_moe_layer. */
int coli_moe_layer_profiled(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T,
                            float *out, void *workspace, size_t ws_bytes, void *stream, void **events,
                            int32_t n_events);
int coli_moe_num_stages(void);
const char *coli_moe_stage_name(int32_t stage);

/* Static text for a status code. */
const char *coli_moe_strerror(int status);

/* ---- Expert residency tier: host RAM -> a pool of expert slots in HBM ----
 * JustVugg/colibri README, "Never wait for the disk twice" and the I/O items: a per-layer
 * LRU of experts with pinned ("hot") experts, missing experts loaded on demand, each expert
 * of the batch union read once. Here the slow tier is host RAM and the fast tier a pool of
 * `slots` expert blobs (+ scales) in HBM; the shared expert, when present, always lives in
 * slot `slots` (the pool has slots + has_shared entries). The group/FFN entry points run on
 * the pool unchanged, with cfg.n_experts = slots, the pool as coli_moe_weights.experts /
 * .scales, and the route remapped to slot ids: the expert arithmetic, the pair order and
 * the combine order are those of the resident layer, so the output is bit-identical to it.
 * The router lookahead (coli_moe_tier_prefetch) stages a layer's predicted union ahead.
 * Unlike the entry points above, coli_moe_layer_tiered and coli_moe_tier_prefetch read the
 * route on the host (each waits once for the device) and keep, per calling host thread, a
 * pinned host buffer for it and, in coli_moe_layer_tiered, one event per device. */

/* Host-side state of one layer's pool. All arrays are caller-owned host memory:
 * slot_of [n_experts], expert_in [slots], last_use [slots], pinned [n_experts]. */
typedef struct {
  int32_t n_experts;  /* E */
  int32_t slots;      /* HBM slots for routed experts, 1 <= slots <= E */
  int32_t *slot_of;   /* slot holding expert e, or -1 */
  int32_t *expert_in; /* expert held by slot s, or -1 */
  uint64_t *last_use; /* LRU clock of the last batch that used slot s */
  const uint8_t *pinned; /* 1: once loaded, never evicted (the pinned hot store); may be NULL */
  uint64_t clock;     /* batches planned so far */
} coli_tier;

/* Empties the pool: slot_of = -1, expert_in = -1, last_use = 0, clock = 0.
 * COLI_E_INVALID on NULL arrays or sizes out of range. */
int coli_tier_init(coli_tier *t);

/* Plans one batch. topk_idx (host, [T][k], expert ids or -1 for an empty slot) is the
 * route; its distinct experts are the union. Experts of the union already in the pool are
 * hits; each miss, in ascending expert order, takes an empty slot (lowest first) or evicts
 * the least recently used slot whose expert is neither pinned nor in this union (lowest
 * slot on ties). Outputs (host): slot_idx [T][k] = the route in slot ids (-1 kept);
 * load_expert / load_slot [*n_load] = the misses and their slots (capacity: slots).
 * COLI_E_INVALID for ids outside [-1, E) or an inconsistent state (slot_of and expert_in
 * not inverse to each other); COLI_E_UNSUPPORTED when the union does not fit
 * (more distinct experts than slots that can be freed). On error the state is unchanged. */
int coli_tier_plan(coli_tier *t, const int32_t *topk_idx, int32_t T, int32_t k, int32_t *slot_idx,
                   int32_t *load_expert, int32_t *load_slot, int32_t *n_load);

/* Enqueues the host->HBM copies of a plan on `stream`: for each i, blob load_expert[i] of
 * host_experts -> slot load_slot[i] of slot_experts, and its scales (coli_moe_scales_per_expert
 * elements: fp32, or bytes for MXFP4) of host_scales -> slot_scales. load_expert may be E,
 * the shared expert, with load_slot = slots. host_experts / host_scales should be pinned host
 * memory (hipHostMalloc) for the copies to be asynchronous; they must stay valid until the
 * stream has run them. slots: the pool's routed slot count. */
int coli_moe_tier_stage(const coli_moe_cfg *cfg, int32_t slots, const void *host_experts, const void *host_scales,
                        const int32_t *load_expert, const int32_t *load_slot, int32_t n_load, void *slot_experts,
                        void *slot_scales, void *stream);

/* Workspace bytes of coli_moe_layer_tiered for up to T_max tokens on a pool of `slots`
 * slots (0 if invalid). 256-byte aligned, like every workspace. */
size_t coli_moe_tier_workspace_bytes(const coli_moe_cfg *cfg, int32_t slots, int32_t T_max);

/* One layer through the tier, on `stream`, with the misses' loads overlapping the resident
 * experts' compute (JustVugg/colibri README: missing experts load while resident ones
 * compute):
 *   1. route (w: router_w / router_bias; experts and scales unused);
 *   2. on the device, the route in slot ids of the experts the pool holds when the call
 *      starts (a kernel that takes that expert -> slot map as an argument; the pairs of
 *      experts not in the pool get -1), and the route into pinned host memory;
 *   3. the FFN of those resident pairs, the shared expert among them, is enqueued at once;
 *   4. the call waits for the route (an event recorded after step 2, its only wait for the
 *      device; the FFN of step 3 keeps running) and runs coli_tier_plan on *tier;
 *   5. the misses are copied host->HBM on `copy_stream` (a second stream of the same device,
 *      default priority) and `copy_event` is recorded after them; `stream` waits for it,
 *      then the FFN of the missing pairs and the combine over every slot of every token run
 *      (with no misses, the combine alone).
 * The output is bit-identical to coli_moe_layer on the resident weights. The pool
 * (pool_experts / pool_scales: slots + has_shared entries) must already hold the shared
 * expert in slot `slots` (coli_moe_tier_stage with load_expert = E). host_experts /
 * host_scales: all E + has_shared experts in pinned host memory. topk_idx_opt / topk_w_opt
 * (device, [T][k]) receive the route (expert ids) when non-NULL. COLI_E_UNSUPPORTED when the
 * union does not fit: nothing is copied, `out` is not written and *tier is unchanged (the
 * resident pairs' FFN of step 3 has run into the workspace). After COLI_E_DEVICE the tier
 * may list experts whose copies did not run: reset it with coli_tier_init. The tier's
 * arrays and the host experts must stay valid until `stream` and `copy_stream` have run the
 * call. The library keeps one pinned host buffer for the route and one event per device for
 * each calling host thread; calls from one thread are sequential. */
int coli_moe_layer_tiered(const coli_moe_cfg *cfg, const coli_moe_weights *w, coli_tier *tier,
                          const void *host_experts, const void *host_scales, void *pool_experts, void *pool_scales,
                          const float *x, int32_t T, float *out, int32_t *topk_idx_opt, float *topk_w_opt,
                          void *workspace, size_t ws_bytes, void *stream, void *copy_stream, void *copy_event);

/* Router lookahead (JustVugg/colibri README: a router-lookahead thread prefetches the next
 * layer's experts; routing is largely predictable one layer ahead): routes x with the router
 * of another layer (w: its router_w / router_bias; typically layer l+1's, applied to layer
 * l's input), plans that union on that layer's *tier and enqueues the misses' copies into
 * that layer's pool on copy_stream, then returns. The layer's next coli_moe_layer_tiered
 * call on the same copy_stream waits for these copies before it reads the pool. Waits for
 * `stream` after the route. workspace: coli_moe_tier_workspace_bytes(cfg, tier->slots, T).
 * Ordering: the copies overwrite least recently used slots of that pool, so every earlier
 * call that reads the pool must have finished, or be ordered before copy_stream's next
 * work, when this is called. A coli_moe_layer_tiered call of a later layer, made on the
 * same stream as the pool's last tiered call, guarantees it (its route waits for that
 * stream); otherwise make copy_stream wait for an event recorded after the pool's last
 * call.
 * *n_loaded_opt receives the number of experts copied. COLI_E_UNSUPPORTED when the
 * predicted union does not fit (nothing copied, *tier unchanged); after COLI_E_DEVICE reset
 * the tier with coli_tier_init. */
int coli_moe_tier_prefetch(const coli_moe_cfg *cfg, const coli_moe_weights *w, coli_tier *tier,
                           const void *host_experts, const void *host_scales, void *pool_experts, void *pool_scales,
                           const float *x, int32_t T, void *workspace, size_t ws_bytes, void *stream,
                           void *copy_stream, int32_t *n_loaded_opt);

#ifdef __cplusplus
}
#endif
#endif
