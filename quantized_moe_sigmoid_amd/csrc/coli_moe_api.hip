// coli_moe_api.hip — the C ABI of libcolimoe: host-side validation, workspace
// layout and the launch sequence of the routed MoE layer (one stream, no host
// synchronisation, no device allocation).
#include <limits.h>

#include <mutex>

#include "coli_internal.h"
#ifdef COLI_TAPS
#include "../../include/coli_moe_taps.h"
#endif

namespace coli {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(const coli_moe_cfg &c, int32_t T, int32_t ksplit) {
  const size_t H = c.hidden, F = c.ffn, E = c.n_experts, k = c.top_k;
  const size_t P = (size_t)T * k, R = P + (size_t)T * c.has_shared;  // pair rows (+ shared rows)
  WsLayout L{};
  size_t o = 0;
  L.xq = o;     o = align256(o + (size_t)T * H);
  L.xd = o;     o = align256(o + (size_t)T * (H / QK) * sizeof(float));
  L.hq = o;     o = align256(o + R * F);
  L.hd = o;     o = align256(o + R * (F / QK) * sizeof(float));
  L.ypair = o;  o = align256(o + R * H * sizeof(float));
  L.logits = o; o = align256(o + (size_t)ksplit * T * E * sizeof(double));
  L.idx = o;    o = align256(o + P * sizeof(int32_t));
  L.w = o;      o = align256(o + P * sizeof(float));
  L.cnt = o;    o = align256(o + E * sizeof(int32_t));
  L.off = o;    o = align256(o + (E + 1) * sizeof(int32_t));
  L.perm = o;   o = align256(o + P * sizeof(int32_t));
  L.active = o; o = align256(o + E * sizeof(int32_t));
  L.nact = o;   o = align256(o + sizeof(int32_t));
  L.tiles = o;  o = align256(o + (size_t)mfma_gmax(T, c.top_k, c.n_experts, c.has_shared) * sizeof(int4));
  L.ntiles = o; o = align256(o + sizeof(int32_t));
  L.redo = o;   o = align256(o + (size_t)mfma_redo_words(c, T) * sizeof(int32_t));
  L.total = o;
  return L;
}

static constexpr size_t GEMV_LDS_LIMIT = 64 * 1024;

static size_t gemv_lds(int K) {
  return (size_t)GEMV_NT * K + (size_t)GEMV_NT * (K / QK) * sizeof(float) + (size_t)GEMV_NT * GEMV_ROWS * sizeof(float) +
         2 * GEMV_NT * sizeof(int);
}

static int check_cfg(const coli_moe_cfg *c) {
  if (!c) return COLI_E_INVALID;
  if (c->hidden <= 0 || c->ffn <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->n_group <= 0 ||
      c->topk_group <= 0)
    return COLI_E_INVALID;
  if (c->wfmt != 2 && c->wfmt != 4 && c->wfmt != 8 && c->wfmt != COLI_W_MXFP4) return COLI_E_INVALID;
  if (c->has_shared != 0 && c->has_shared != 1) return COLI_E_INVALID;
  if (c->n_experts % c->n_group || c->topk_group > c->n_group) return COLI_E_INVALID;
  if (c->top_k > c->topk_group * (c->n_experts / c->n_group)) return COLI_E_INVALID;
  if (!(c->routed_scaling_factor == c->routed_scaling_factor)) return COLI_E_INVALID;  // NaN
  // MXFP4 carries one E8M0 scale per 32 inputs; the integer formats one per row or per 64
  if (c->wfmt == COLI_W_MXFP4 ? c->scale_group != 32 : (c->scale_group != 0 && c->scale_group != 64))
    return COLI_E_INVALID;
  if (!(c->topp >= 0.0f && c->topp <= 1.0f)) return COLI_E_INVALID;  // NaN included
  if (c->hidden % 128 || c->ffn % 128) return COLI_E_UNSUPPORTED;
  if (c->n_experts > 1024 || c->n_group > 64 || c->top_k > 64) return COLI_E_UNSUPPORTED;
  if (gemv_lds(c->hidden) > GEMV_LDS_LIMIT || gemv_lds(c->ffn) > GEMV_LDS_LIMIT) return COLI_E_UNSUPPORTED;
  if ((int64_t)c->hidden * c->ffn > ((int64_t)1 << 40)) return COLI_E_UNSUPPORTED;
  return COLI_OK;
}

static int check_T(const coli_moe_cfg *c, int32_t T) {
  if (T < 0) return COLI_E_INVALID;
  if ((int64_t)T * c->top_k > 65535) return COLI_E_UNSUPPORTED;
  if (T > 0 && !group_supported(T * c->top_k, c->n_experts)) return COLI_E_UNSUPPORTED;
  return COLI_OK;
}

static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

static int check_weights(const coli_moe_weights *w, bool need_experts, bool need_router) {
  if (!w) return COLI_E_INVALID;
  if (need_experts) {
    if (!w->experts || !w->scales) return COLI_E_INVALID;
    if (!aligned(w->experts, 16) || !aligned(w->scales, 4)) return COLI_E_ALIGN;
  }
  if (need_router) {
    if (!w->router_w || !w->router_bias) return COLI_E_INVALID;
    if (!aligned(w->router_w, 16) || !aligned(w->router_bias, 4)) return COLI_E_ALIGN;
  }
  return COLI_OK;
}

static int dev(hipError_t e) { return e == hipSuccess ? COLI_OK : COLI_E_DEVICE; }

template <typename Tp>
static Tp *at(void *ws, size_t off) {
  return reinterpret_cast<Tp *>(static_cast<char *>(ws) + off);
}

// Expert FFNs and combine. With quantize_x the standalone Q8_0 kernel runs first;
// otherwise x was quantised by the routing kernel (or by an earlier phase). Without
// shared the shared expert's rows are left as they are (an earlier phase computed
// them); without combine the pair rows are only computed (a later phase combines).
static int ffn_enqueue(const coli_moe_cfg &c, const coli_moe_weights &w, const float *x, int32_t T,
                       const float *topk_w, const int32_t *off, const int32_t *perm, const int32_t *active,
                       const int32_t *nact, const int32_t *local_idx, float *out, void *ws, const WsLayout &L,
                       hipStream_t s, hipEvent_t *ev, bool quantize_x, float *tap = nullptr, bool shared = true,
                       bool combine = true, const SelectArgs *fsel = nullptr) {
  int st;
  if (ev && (st = dev(hipEventRecord(ev[0], s)))) return st;
  if (quantize_x && (st = dev(launch_q8_0(x, T, c.hidden, at<int8_t>(ws, L.xq), at<float>(ws, L.xd), s))))
    return st;
  FfnArgs a{};
  a.experts = static_cast<const uint8_t *>(w.experts);
  a.scales = w.scales;
  a.blob_bytes = coli_moe_blob_bytes(&c);
  a.scale_stride = coli_moe_scales_per_expert(&c);
  a.gs = c.scale_group;
  a.H = c.hidden;
  a.F = c.ffn;
  a.E = c.n_experts;
  a.k = c.top_k;
  a.T = T;
  a.has_shared = shared ? c.has_shared : 0;
  a.off = off;
  a.perm = perm;
  a.active = active;
  a.nact = nact;
  a.idx = local_idx;
  a.xq = at<int8_t>(ws, L.xq);
  a.xd = at<float>(ws, L.xd);
  a.hq = at<int8_t>(ws, L.hq);
  a.hd = at<float>(ws, L.hd);
  a.ypair = at<float>(ws, L.ypair);
  a.tap = tap;
  a.redo = at<int32_t>(ws, L.redo);
  // Batches past the decode size run the expert FFNs as grouped GEMMs on the
  // matrix cores; a tile plan of the union comes first.
  const bool gemm = local_idx == nullptr && (int64_t)T * c.top_k > LOCAL_GROUP_MAX_P;
  const int32_t gmax = mfma_gmax(T, c.top_k, c.n_experts, c.has_shared);
  int4 *tiles = at<int4>(ws, L.tiles);
  int32_t *ntiles = at<int32_t>(ws, L.ntiles);
  if (gemm && (st = dev(launch_plan(a, tiles, ntiles, gmax, s)))) return st;
  if (ev && (st = dev(hipEventRecord(ev[1], s)))) return st;
  if (fsel && !gemm) a.sel = *fsel;  // the gate/up GEMV selects the route (local_idx is its output)
  if ((st = dev(gemm ? launch_mfma_gateup(c.wfmt, a, tiles, ntiles, gmax, s) : launch_gateup(c.wfmt, a, s)))) return st;
  a.sel = SelectArgs{};
  if (ev && (st = dev(hipEventRecord(ev[2], s)))) return st;
  if ((st = dev(gemm ? launch_mfma_down(c.wfmt, a, tiles, ntiles, gmax, s) : launch_down(c.wfmt, a, s)))) return st;
  if (ev && (st = dev(hipEventRecord(ev[3], s)))) return st;
  if (combine && (st = dev(launch_combine(a.ypair, topk_w, T, c.top_k, c.hidden, c.has_shared, out, s)))) return st;
  if (ev && (st = dev(hipEventRecord(ev[4], s)))) return st;
  return COLI_OK;
}

int ffn_phase(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T, const int32_t *topk_idx,
              const float *topk_w, const int32_t *expert_off, const int32_t *pair_perm, const int32_t *active,
              const int32_t *n_active, float *out, void *workspace, size_t ws_bytes, hipStream_t s, bool quantize_x,
              bool shared, bool combine) {
  int st;
  if ((st = check_cfg(cfg))) return st;
  if ((st = check_T(cfg, T))) return st;
  if (T == 0) return COLI_OK;
  if ((st = check_weights(w, true, false))) return st;
  if (!x || !topk_idx || !topk_w || (combine && !out)) return COLI_E_INVALID;
  const bool local = (int64_t)T * cfg->top_k <= LOCAL_GROUP_MAX_P;
  if (!local && (!expert_off || !pair_perm || !active || !n_active)) return COLI_E_INVALID;
  const WsLayout L = ws_layout(*cfg, T, route_ksplit(*cfg, T));
  if (!workspace || ws_bytes < L.total) return COLI_E_WORKSPACE;
  return ffn_enqueue(*cfg, *w, x, T, topk_w, expert_off, pair_perm, active, n_active, local ? topk_idx : nullptr, out,
                     workspace, L, s, nullptr, quantize_x, nullptr, shared, combine);
}

int combine_phase(const coli_moe_cfg *cfg, int32_t T, const float *topk_w, float *out, void *workspace,
                  size_t ws_bytes, hipStream_t s) {
  int st;
  if ((st = check_cfg(cfg))) return st;
  if ((st = check_T(cfg, T))) return st;
  if (T == 0) return COLI_OK;
  if (!topk_w || !out) return COLI_E_INVALID;
  const WsLayout L = ws_layout(*cfg, T, route_ksplit(*cfg, T));
  if (!workspace || ws_bytes < L.total) return COLI_E_WORKSPACE;
  return dev(launch_combine(at<float>(workspace, L.ypair), topk_w, T, cfg->top_k, cfg->hidden, cfg->has_shared, out,
                            s));
}

int route_phase(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T, int32_t *topk_idx,
                float *topk_w, void *workspace, size_t ws_bytes, int8_t *xq, float *xd, hipStream_t s) {
  int st;
  if ((st = check_cfg(cfg))) return st;
  if ((st = check_T(cfg, T))) return st;
  if (T == 0) return COLI_OK;
  if ((st = check_weights(w, false, true))) return st;
  if (!x || !topk_idx || !topk_w || !xq || !xd) return COLI_E_INVALID;
  if (!aligned(x, 16)) return COLI_E_ALIGN;
  const int32_t ks = route_ksplit(*cfg, T);
  const WsLayout L = ws_layout(*cfg, T, ks);
  if (!workspace || ws_bytes < L.total) return COLI_E_WORKSPACE;
  RouteLaunch r{};
  r.cfg = cfg;
  r.x = x;
  r.T = T;
  r.W = w->router_w;
  r.bias = w->router_bias;
  r.logits = at<double>(workspace, L.logits);
  r.ksplit = ks;
  r.idx = topk_idx;
  r.w = topk_w;
  r.xq = xq;
  r.xd = xd;
  return dev(launch_route(r, s, nullptr));
}

int8_t *ws_xq(const coli_moe_cfg &c, int32_t T, void *ws) { return at<int8_t>(ws, ws_layout(c, T, 1).xq); }
float *ws_xd(const coli_moe_cfg &c, int32_t T, void *ws) { return at<float>(ws, ws_layout(c, T, 1).xd); }

// stage order of coli_moe_layer_profiled; a stage fused into the previous kernel is empty
static const char *const kStages[] = {"route_logits", "route_select", "group", "quantize_x",
                                      "ffn_gate_up", "ffn_down", "combine"};
static constexpr int kNumStages = 7;

static int layer_impl(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T, float *out,
                      int32_t *idx_opt, float *w_opt, void *ws, size_t ws_bytes, void *stream, hipEvent_t *ev,
                      float *tap = nullptr) {
  int st;
  if ((st = check_cfg(cfg))) return st;
  if ((st = check_T(cfg, T))) return st;
  if (T == 0) return COLI_OK;
  if ((st = check_weights(w, true, true))) return st;
  if (!x || !out) return COLI_E_INVALID;
  if (!aligned(x, 16) || !aligned(out, 16)) return COLI_E_ALIGN;
  if ((idx_opt && !aligned(idx_opt, 4)) || (w_opt && !aligned(w_opt, 4))) return COLI_E_ALIGN;
  const int32_t ks = route_ksplit(*cfg, T);
  const WsLayout L = ws_layout(*cfg, T, ks);
  if (!ws || ws_bytes < L.total) return COLI_E_WORKSPACE;
  if (!aligned(ws, 256)) return COLI_E_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t *idx = idx_opt ? idx_opt : at<int32_t>(ws, L.idx);
  float *tw = w_opt ? w_opt : at<float>(ws, L.w);
  int32_t *off = at<int32_t>(ws, L.off), *perm = at<int32_t>(ws, L.perm), *act = at<int32_t>(ws, L.active),
          *nact = at<int32_t>(ws, L.nact), *cnt = at<int32_t>(ws, L.cnt);
  RouteLaunch r{};
  r.cfg = cfg;
  r.x = x;
  r.T = T;
  r.W = w->router_w;
  r.bias = w->router_bias;
  r.logits = at<double>(ws, L.logits);
  r.ksplit = ks;
  r.idx = idx;
  r.w = tw;
  r.xq = at<int8_t>(ws, L.xq);
  r.xd = at<float>(ws, L.xd);
  // decode-sized batches: every GEMV workgroup groups the route itself
  const bool local = (int64_t)T * cfg->top_k <= LOCAL_GROUP_MAX_P;
  // small decode batches: the gate/up GEMV selects the route itself (fsel.part set)
  SelectArgs fsel{};
  if (ev && (st = dev(hipEventRecord(ev[0], s)))) return st;
  if ((st = dev(launch_route(r, s, ev ? ev[1] : nullptr, local ? &fsel : nullptr)))) return st;
  if (ev && (st = dev(hipEventRecord(ev[2], s)))) return st;
  if (!local && (st = dev(launch_group(*cfg, idx, T, cnt, off, perm, act, nact, s)))) return st;
  return ffn_enqueue(*cfg, *w, x, T, tw, off, perm, act, nact, local ? idx : nullptr, out, ws, L, s,
                     ev ? ev + 3 : nullptr, false, tap, true, true, fsel.part ? &fsel : nullptr);
}

// ---- fixed device scratch of the allocation-free entry point --------------------
// coli_moe_layer_noalloc runs the same launch sequence as coli_moe_layer on this
// library-owned array instead of a caller's workspace. It is a file-scope device
// array (one copy per GPU, allocated when the code object is loaded on that GPU and
// held until the process ends). In host code `scratch` only names the symbol: its
// device address is looked up once per device with hipGetSymbolAddress, with that
// device current, and only that address is ever passed to kernels.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device

static int scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return COLI_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return COLI_E_DEVICE;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return COLI_OK;
}

}  // namespace coli

using namespace coli;

extern "C" {

size_t coli_moe_blob_bytes(const coli_moe_cfg *cfg) {
  if (check_cfg(cfg) != COLI_OK) return 0;
  return (size_t)(2 * (int64_t)cfg->ffn * row_bytes(cfg->wfmt, cfg->hidden) +
                  (int64_t)cfg->hidden * row_bytes(cfg->wfmt, cfg->ffn));
}

size_t coli_moe_scales_per_expert(const coli_moe_cfg *cfg) {
  if (check_cfg(cfg) != COLI_OK) return 0;
  const int64_t H = cfg->hidden, F = cfg->ffn;
  return (size_t)(cfg->scale_group ? 3 * F * (H / cfg->scale_group) : 2 * F + H);
}

size_t coli_moe_workspace_bytes(const coli_moe_cfg *cfg, int32_t T_max) {
  if (check_cfg(cfg) != COLI_OK || check_T(cfg, T_max) != COLI_OK) return 0;
  // A call with T tokens needs ws_layout(T, K split of T). Every region grows with T and
  // with the K split, but the K split shrinks as T grows, so size for T_max tokens with
  // the largest K split of any T <= T_max: that covers every call up to T_max.
  int32_t ks = 1;
  for (int32_t T = 1; T <= T_max; T++) {
    const int32_t k = route_ksplit(*cfg, T);
    if (k > ks) ks = k;
  }
  return ws_layout(*cfg, T_max, ks).total;
}

int coli_moe_quantize_q8_0(const float *x, int64_t rows, int32_t cols, int8_t *q, float *d, void *stream) {
  if (rows < 0 || cols <= 0) return COLI_E_INVALID;
  if (cols % QK) return COLI_E_UNSUPPORTED;
  if (rows == 0) return COLI_OK;
  if (!x || !q || !d) return COLI_E_INVALID;
  if (!aligned(x, 16) || !aligned(q, 4) || !aligned(d, 4)) return COLI_E_ALIGN;
  return dev(launch_q8_0(x, rows, cols, q, d, static_cast<hipStream_t>(stream)));
}

int coli_moe_route(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T,
                   int32_t *topk_idx, float *topk_w, void *workspace, size_t ws_bytes, void *stream) {
  int st;
  if ((st = check_cfg(cfg))) return st;
  if ((st = check_T(cfg, T))) return st;
  if (T == 0) return COLI_OK;
  if ((st = check_weights(w, false, true))) return st;
  if (!x || !topk_idx || !topk_w) return COLI_E_INVALID;
  if (!aligned(x, 16) || !aligned(topk_idx, 4) || !aligned(topk_w, 4)) return COLI_E_ALIGN;
  const int32_t ks = route_ksplit(*cfg, T);
  const WsLayout L = ws_layout(*cfg, T, ks);
  if (!workspace || ws_bytes < L.total) return COLI_E_WORKSPACE;
  if (!aligned(workspace, 256)) return COLI_E_ALIGN;
  RouteLaunch r{};
  r.cfg = cfg;
  r.x = x;
  r.T = T;
  r.W = w->router_w;
  r.bias = w->router_bias;
  r.logits = at<double>(workspace, L.logits);
  r.ksplit = ks;
  r.idx = topk_idx;
  r.w = topk_w;
  return dev(launch_route(r, static_cast<hipStream_t>(stream), nullptr));
}

int coli_moe_group(const coli_moe_cfg *cfg, const int32_t *topk_idx, int32_t T, int32_t *expert_cnt,
                   int32_t *expert_off, int32_t *pair_perm, int32_t *active, int32_t *n_active, void *stream) {
  int st;
  if ((st = check_cfg(cfg))) return st;
  if ((st = check_T(cfg, T))) return st;
  if (T == 0) return COLI_OK;
  if (!topk_idx || !expert_cnt || !expert_off || !pair_perm || !active || !n_active) return COLI_E_INVALID;
  if (!aligned(topk_idx, 4) || !aligned(expert_cnt, 4) || !aligned(expert_off, 4) || !aligned(pair_perm, 4) ||
      !aligned(active, 4) || !aligned(n_active, 4))
    return COLI_E_ALIGN;
  return dev(launch_group(*cfg, topk_idx, T, expert_cnt, expert_off, pair_perm, active, n_active,
                          static_cast<hipStream_t>(stream)));
}

static int ffn_impl(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T,
                    const int32_t *topk_idx, const float *topk_w, const int32_t *expert_off, const int32_t *pair_perm,
                    const int32_t *active, const int32_t *n_active, float *out, void *workspace, size_t ws_bytes,
                    void *stream, float *tap) {
  int st;
  if ((st = check_cfg(cfg))) return st;
  if ((st = check_T(cfg, T))) return st;
  if (T == 0) return COLI_OK;
  if ((st = check_weights(w, true, false))) return st;
  if (!x || !topk_idx || !topk_w || !expert_off || !pair_perm || !active || !n_active || !out)
    return COLI_E_INVALID;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(topk_w, 4) || !aligned(expert_off, 4) ||
      !aligned(pair_perm, 4) || !aligned(active, 4) || !aligned(n_active, 4))
    return COLI_E_ALIGN;
  const WsLayout L = ws_layout(*cfg, T, route_ksplit(*cfg, T));
  if (!workspace || ws_bytes < L.total) return COLI_E_WORKSPACE;
  if (!aligned(workspace, 256)) return COLI_E_ALIGN;
  return ffn_enqueue(*cfg, *w, x, T, topk_w, expert_off, pair_perm, active, n_active, nullptr, out, workspace, L,
                     static_cast<hipStream_t>(stream), nullptr, true, tap);
}

int coli_moe_ffn(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T,
                 const int32_t *topk_idx, const float *topk_w, const int32_t *expert_off, const int32_t *pair_perm,
                 const int32_t *active, const int32_t *n_active, float *out, void *workspace, size_t ws_bytes,
                 void *stream) {
  return ffn_impl(cfg, w, x, T, topk_idx, topk_w, expert_off, pair_perm, active, n_active, out, workspace, ws_bytes,
                  stream, nullptr);
}

int coli_moe_layer(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T, float *out,
                   int32_t *topk_idx_opt, float *topk_w_opt, void *workspace, size_t ws_bytes, void *stream) {
  return layer_impl(cfg, w, x, T, out, topk_idx_opt, topk_w_opt, workspace, ws_bytes, stream, nullptr);
}

size_t coli_moe_scratch_bytes(void) { return kScratchBytes; }

int coli_moe_layer_noalloc(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T, float *out,
                           int32_t *topk_idx_opt, float *topk_w_opt, void *stream) {
  int st;
  if ((st = check_cfg(cfg))) return st;
  if ((st = check_T(cfg, T))) return st;
  if (T == 0) return COLI_OK;
  // the batch must fit the fixed scratch: rejected before anything is enqueued
  if (coli_moe_workspace_bytes(cfg, T) > kScratchBytes) return COLI_E_SCRATCH;
  void *ws = nullptr;
  if ((st = scratch_of_current_device(&ws))) return st;
  return layer_impl(cfg, w, x, T, out, topk_idx_opt, topk_w_opt, ws, kScratchBytes, stream, nullptr);
}

int coli_moe_layer_profiled(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T,
                            float *out, void *workspace, size_t ws_bytes, void *stream, void **events,
                            int32_t n_events) {
  if (!events || n_events != kNumStages + 1) return COLI_E_INVALID;
  for (int i = 0; i < n_events; i++)
    if (!events[i]) return COLI_E_INVALID;
  return layer_impl(cfg, w, x, T, out, nullptr, nullptr, workspace, ws_bytes, stream,
                    reinterpret_cast<hipEvent_t *>(events));
}

#ifdef COLI_TAPS
int coli_moe_layer_taps(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T, float *out,
                        int32_t *topk_idx_opt, float *topk_w_opt, float *tap_gu, void *workspace, size_t ws_bytes,
                        void *stream) {
  if (!tap_gu || !aligned(tap_gu, 4)) return COLI_E_INVALID;
  return layer_impl(cfg, w, x, T, out, topk_idx_opt, topk_w_opt, workspace, ws_bytes, stream, nullptr, tap_gu);
}

int coli_moe_ffn_taps(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T,
                      const int32_t *topk_idx, const float *topk_w, const int32_t *expert_off, const int32_t *pair_perm,
                      const int32_t *active, const int32_t *n_active, float *out, float *tap_gu, void *workspace,
                      size_t ws_bytes, void *stream) {
  if (!tap_gu || !aligned(tap_gu, 4)) return COLI_E_INVALID;
  return ffn_impl(cfg, w, x, T, topk_idx, topk_w, expert_off, pair_perm, active, n_active, out, workspace, ws_bytes,
                  stream, tap_gu);
}
#endif

int coli_moe_num_stages(void) { return kNumStages; }

const char *coli_moe_stage_name(int32_t stage) {
  return (stage >= 0 && stage < kNumStages) ? kStages[stage] : "";
}

const char *coli_moe_strerror(int status) {
  switch (status) {
    case COLI_OK: return "ok";
    case COLI_E_INVALID: return "invalid argument or configuration";
    case COLI_E_UNSUPPORTED: return "configuration outside the library's limits";
    case COLI_E_WORKSPACE: return "workspace missing or too small";
    case COLI_E_ALIGN: return "pointer not aligned as required";
    case COLI_E_DEVICE: return "HIP runtime rejected a launch";
    case COLI_E_SCRATCH: return "batch needs more than the fixed scratch of coli_moe_layer_noalloc";
  }
  return "unknown status";
}

}  // extern "C"
