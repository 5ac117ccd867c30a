// tier.hip — the expert residency tier: host RAM -> a pool of expert slots in HBM.
//
// JustVugg/colibri README, "Never wait for the disk twice" and its I/O items: a
// per-layer LRU of experts with a pinned hot store, missing experts loaded on demand,
// every expert of the batch union read once. The planner is host code over
// caller-owned state; the copies are host->device DMA on the caller's stream. The
// FFN kernels are not involved: they run on the pool with the route in slot ids.
#include <vector>

#include "coli_internal.h"

namespace {

// Expert -> slot map of one phase of a tiered call, passed by value as a kernel argument
// (the runtime copies arguments at launch, so the host map needs no lifetime beyond the
// call): slot of expert e, -1 when e is not served by the phase. E <= 1024, slots <= E.
struct TierMap {
  int16_t slot[1024];
};

// The route in slot ids of one phase: out[p] = slot of expert idx[p] in `map` (-1 when the
// map has none, or for an empty slot of the route). host_idx (device-mapped pinned host
// memory, when not null) receives the route itself.
__global__ __launch_bounds__(256) void tier_remap_kernel(const int32_t *__restrict__ idx, int32_t P, TierMap map,
                                                         int32_t *__restrict__ out, int32_t *__restrict__ host_idx) {
  for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < P; p += gridDim.x * blockDim.x) {
    const int e = idx[p];
    out[p] = (e >= 0 && e < 1024) ? (int)map.slot[e] : -1;
    if (host_idx) host_idx[p] = e;
  }
}

// The route's way to the host: pinned, device-mapped host memory that the remap kernel
// writes, and an event recorded after it, per host thread (a tiered call waits for its
// own event before it returns, so the thread's next call finds the buffer free). A
// buffer that grows is replaced and the old one kept: nothing frees memory that a kernel
// may have written.
struct HostRoute {
  int32_t *h = nullptr;
  size_t cap = 0;
  hipEvent_t ev[64] = {};
};
thread_local HostRoute t_route;

int32_t *host_route(size_t n) {
  if (n > t_route.cap) {
    size_t cap = t_route.cap ? 2 * t_route.cap : 4096;
    while (cap < n) cap *= 2;
    void *p = nullptr;
    if (hipHostMalloc(&p, cap * sizeof(int32_t), hipHostMallocMapped | hipHostMallocPortable | hipHostMallocCoherent) !=
        hipSuccess)
      return nullptr;
    t_route.h = static_cast<int32_t *>(p);
    t_route.cap = cap;
  }
  return t_route.h;
}

hipEvent_t route_event(hipStream_t s) {
  int dev = 0;
  if (hipStreamGetDevice(s, &dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (!t_route.ev[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    hipEvent_t e = nullptr;
    const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (cur != dev) (void)hipSetDevice(cur);
    if (r != hipSuccess) return nullptr;
    t_route.ev[dev] = e;
  }
  return t_route.ev[dev];
}

// The pool state is caller-owned memory: every slot and expert index must be in range
// and the two maps must agree before any of it is used.
bool tier_state_ok(const coli_tier &t) {
  const int32_t E = t.n_experts, S = t.slots;
  if (!t.slot_of || !t.expert_in || !t.last_use || E <= 0 || E > 1024 || S <= 0 || S > E) return false;
  for (int32_t s = 0; s < S; s++) {
    const int32_t e = t.expert_in[s];
    if (e < -1 || e >= E || (e >= 0 && t.slot_of[e] != s)) return false;
  }
  for (int32_t e = 0; e < E; e++) {
    const int32_t s = t.slot_of[e];
    if (s < -1 || s >= S || (s >= 0 && t.expert_in[s] != e)) return false;
  }
  return true;
}

}  // namespace

extern "C" {

int coli_tier_init(coli_tier *t) {
  if (!t || !t->slot_of || !t->expert_in || !t->last_use) return COLI_E_INVALID;
  if (t->n_experts <= 0 || t->n_experts > 1024 || t->slots <= 0 || t->slots > t->n_experts) return COLI_E_INVALID;
  for (int32_t e = 0; e < t->n_experts; e++) t->slot_of[e] = -1;
  for (int32_t s = 0; s < t->slots; s++) {
    t->expert_in[s] = -1;
    t->last_use[s] = 0;
  }
  t->clock = 0;
  return COLI_OK;
}

int coli_tier_plan(coli_tier *t, const int32_t *topk_idx, int32_t T, int32_t k, int32_t *slot_idx,
                   int32_t *load_expert, int32_t *load_slot, int32_t *n_load) {
  if (!t || !t->slot_of || !t->expert_in || !t->last_use || !n_load || T < 0 || k <= 0) return COLI_E_INVALID;
  const int32_t E = t->n_experts, S = t->slots;
  if (E <= 0 || E > 1024 || S <= 0 || S > E) return COLI_E_INVALID;
  const int64_t P = (int64_t)T * k;
  if (P > 0 && (!topk_idx || !slot_idx || !load_expert || !load_slot)) return COLI_E_INVALID;
  // the union (ascending) and validation, before any state changes
  std::vector<uint8_t> in_union(E, 0);
  for (int64_t p = 0; p < P; p++) {
    const int32_t e = topk_idx[p];
    if (e < -1 || e >= E) return COLI_E_INVALID;
    if (e >= 0) in_union[e] = 1;
  }
  // the state must be consistent (caller-owned memory): every index stays in range below
  if (!tier_state_ok(*t)) return COLI_E_INVALID;
  std::vector<int32_t> misses;
  for (int32_t e = 0; e < E; e++)
    if (in_union[e] && t->slot_of[e] < 0) misses.push_back(e);
  // victims: empty slots first (lowest index), then the least recently used slots whose
  // expert is neither pinned nor in this union (lowest index on equal clocks)
  std::vector<int32_t> victims;
  for (int32_t s = 0; s < S && victims.size() < misses.size(); s++)
    if (t->expert_in[s] < 0) victims.push_back(s);
  if (victims.size() < misses.size()) {
    std::vector<int32_t> cand;
    for (int32_t s = 0; s < S; s++) {
      const int32_t e = t->expert_in[s];
      if (e >= 0 && !in_union[e] && !(t->pinned && t->pinned[e])) cand.push_back(s);
    }
    // stable selection by (last_use, slot)
    std::vector<uint8_t> taken(cand.size(), 0);
    while (victims.size() < misses.size()) {
      int best = -1;
      for (size_t i = 0; i < cand.size(); i++)
        if (!taken[i] && (best < 0 || t->last_use[cand[i]] < t->last_use[cand[best]])) best = (int)i;
      if (best < 0) return COLI_E_UNSUPPORTED;  // the union does not fit; nothing changed
      taken[best] = 1;
      victims.push_back(cand[best]);
    }
  }
  // commit
  t->clock++;
  for (size_t i = 0; i < misses.size(); i++) {
    const int32_t e = misses[i], s = victims[i];
    const int32_t old = t->expert_in[s];
    if (old >= 0) t->slot_of[old] = -1;
    t->expert_in[s] = e;
    t->slot_of[e] = s;
    load_expert[i] = e;
    load_slot[i] = s;
  }
  *n_load = (int32_t)misses.size();
  for (int32_t e = 0; e < E; e++)
    if (in_union[e]) t->last_use[t->slot_of[e]] = t->clock;
  for (int64_t p = 0; p < P; p++) slot_idx[p] = topk_idx[p] < 0 ? -1 : t->slot_of[topk_idx[p]];
  return COLI_OK;
}

int coli_moe_tier_stage(const coli_moe_cfg *cfg, int32_t slots, const void *host_experts, const void *host_scales,
                        const int32_t *load_expert, const int32_t *load_slot, int32_t n_load, void *slot_experts,
                        void *slot_scales, void *stream) {
  const size_t blob = coli_moe_blob_bytes(cfg);
  const size_t nsc = coli_moe_scales_per_expert(cfg);
  if (blob == 0 || nsc == 0) return COLI_E_INVALID;
  if (n_load < 0 || slots <= 0 || slots > cfg->n_experts) return COLI_E_INVALID;
  if (n_load == 0) return COLI_OK;
  if (!host_experts || !host_scales || !load_expert || !load_slot || !slot_experts || !slot_scales)
    return COLI_E_INVALID;
  const size_t scb = nsc * (cfg->wfmt == COLI_W_MXFP4 ? 1 : sizeof(float));
  for (int32_t i = 0; i < n_load; i++) {  // validate all before enqueueing any
    const int32_t e = load_expert[i], s = load_slot[i];
    const bool shared = cfg->has_shared && e == cfg->n_experts;
    if (e < 0 || (e >= cfg->n_experts && !shared)) return COLI_E_INVALID;
    if (shared ? s != slots : (s < 0 || s >= slots)) return COLI_E_INVALID;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int32_t i = 0; i < n_load; i++) {
    const int64_t e = load_expert[i], s = load_slot[i];
    if (hipMemcpyAsync(static_cast<uint8_t *>(slot_experts) + s * blob,
                       static_cast<const uint8_t *>(host_experts) + e * blob, blob, hipMemcpyHostToDevice,
                       st) != hipSuccess)
      return COLI_E_DEVICE;
    if (hipMemcpyAsync(static_cast<uint8_t *>(slot_scales) + s * scb,
                       static_cast<const uint8_t *>(host_scales) + e * scb, scb, hipMemcpyHostToDevice,
                       st) != hipSuccess)
      return COLI_E_DEVICE;
  }
  return COLI_OK;
}

static coli_moe_cfg pool_cfg(const coli_moe_cfg &c, int32_t slots) {
  coli_moe_cfg p = c;  // the FFN's view: `slots` experts, the router fields unused
  p.n_experts = slots;
  p.n_group = 1;
  p.topk_group = 1;
  p.topp = 0.0f;
  return p;
}

static size_t a256(size_t n) { return (n + 255) & ~(size_t)255; }

namespace {
struct TierWs {  // byte offsets of coli_moe_layer_tiered's workspace
  size_t route, ffn, idx, w, sidx[2], cnt[2], off[2], perm[2], act[2], nact[2], total;
};
}  // namespace

static bool tier_ws(const coli_moe_cfg *cfg, int32_t slots, int32_t T, TierWs &L) {
  if (!cfg || slots <= 0 || slots > cfg->n_experts || cfg->top_k > slots) return false;
  const coli_moe_cfg pc = pool_cfg(*cfg, slots);
  const size_t a = coli_moe_workspace_bytes(cfg, T), b = coli_moe_workspace_bytes(&pc, T);
  if (a == 0 || b == 0) return false;
  const size_t P = (size_t)T * cfg->top_k, S = (size_t)slots;
  size_t o = 0;
  L.route = o;  o += a256(a);
  L.ffn = o;    o += a256(b);
  L.idx = o;    o += a256(P * 4);
  L.w = o;      o += a256(P * 4);
  for (int h = 0; h < 2; h++) {
    L.sidx[h] = o; o += a256(P * 4);
    L.cnt[h] = o;  o += a256(S * 4);
    L.off[h] = o;  o += a256((S + 1) * 4);
    L.perm[h] = o; o += a256(P * 4);
    L.act[h] = o;  o += a256(S * 4);
    L.nact[h] = o; o += 256;
  }
  L.total = o;
  return true;
}

size_t coli_moe_tier_workspace_bytes(const coli_moe_cfg *cfg, int32_t slots, int32_t T_max) {
  TierWs L;
  if (T_max < 1 || !tier_ws(cfg, slots, T_max, L)) return 0;
  return L.total;
}

int coli_moe_layer_tiered(const coli_moe_cfg *cfg, const coli_moe_weights *w, coli_tier *tier,
                          const void *host_experts, const void *host_scales, void *pool_experts, void *pool_scales,
                          const float *x, int32_t T, float *out, int32_t *topk_idx_opt, float *topk_w_opt,
                          void *workspace, size_t ws_bytes, void *stream, void *copy_stream, void *copy_event) {
  if (!cfg || !w || !tier || T < 0) return COLI_E_INVALID;
  if (T == 0) return COLI_OK;
  if (tier->n_experts != cfg->n_experts) return COLI_E_INVALID;
  const int32_t slots = tier->slots, k = cfg->top_k;
  TierWs L;
  if (!tier_ws(cfg, slots, T, L)) return COLI_E_INVALID;
  if (!workspace || ws_bytes < L.total) return COLI_E_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return COLI_E_ALIGN;
  if (!host_experts || !host_scales || !pool_experts || !pool_scales || !copy_stream || !copy_event)
    return COLI_E_INVALID;
  if (!tier_state_ok(*tier)) return COLI_E_INVALID;
  const coli_moe_cfg pc = pool_cfg(*cfg, slots);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  auto at = [&](size_t off) { return static_cast<void *>(ws + off); };
  int32_t *idx = static_cast<int32_t *>(at(L.idx));
  float *wt = static_cast<float *>(at(L.w));
  hipStream_t s = static_cast<hipStream_t>(stream), cs = static_cast<hipStream_t>(copy_stream);
  hipEvent_t cev = static_cast<hipEvent_t>(copy_event);
  const size_t P = (size_t)T * k;
  const size_t a_bytes = L.ffn - L.route, b_bytes = L.idx - L.ffn;
  const bool local = (int64_t)T * k <= coli::LOCAL_GROUP_MAX_P;
  int32_t *hidx = host_route(P), *hidx_d = nullptr;
  hipEvent_t rev = route_event(s);
  if (!hidx || !rev || hipHostGetDevicePointer(reinterpret_cast<void **>(&hidx_d), hidx, 0) != hipSuccess)
    return COLI_E_DEVICE;
  const unsigned rgrid = (unsigned)((P + 255) / 256);
  // one phase of the FFN on the pool: the pairs whose slot in sidx is set
  auto phase = [&](int h, bool shared, bool combine) -> int {
    const int32_t *si = static_cast<const int32_t *>(at(L.sidx[h]));
    int32_t *cnt = static_cast<int32_t *>(at(L.cnt[h])), *off = static_cast<int32_t *>(at(L.off[h]));
    int32_t *perm = static_cast<int32_t *>(at(L.perm[h])), *act = static_cast<int32_t *>(at(L.act[h]));
    int32_t *nact = static_cast<int32_t *>(at(L.nact[h]));
    int r;
    // batches past the decode size are grouped explicitly; smaller ones group inside the
    // GEMV workgroups
    if (!local && (r = coli_moe_group(&pc, si, T, cnt, off, perm, act, nact, stream))) return r;
    const coli_moe_weights pw{pool_experts, static_cast<const float *>(pool_scales), w->router_w, w->router_bias};
    return coli::ffn_phase(&pc, &pw, x, T, si, wt, off, perm, act, nact, out, at(L.ffn), b_bytes, s, false, shared,
                           combine);
  };
  int st;
  // 1. route (quantising x into the FFN workspace)
  if ((st = coli::route_phase(cfg, w, x, T, idx, wt, at(L.route), a_bytes, coli::ws_xq(pc, T, at(L.ffn)),
                              coli::ws_xd(pc, T, at(L.ffn)), s)))
    return st;
  // 2. the route in slot ids of the experts the pool holds now (every pair of a miss is -1
  // here), and the route itself into pinned host memory
  TierMap map;
  for (int32_t e = 0; e < 1024; e++) map.slot[e] = (e < cfg->n_experts) ? (int16_t)tier->slot_of[e] : (int16_t)-1;
  hipLaunchKernelGGL(tier_remap_kernel, dim3(rgrid), dim3(256), 0, s, idx, (int32_t)P, map,
                     static_cast<int32_t *>(at(L.sidx[0])), hidx_d);
  if (hipGetLastError() != hipSuccess || hipEventRecord(rev, s) != hipSuccess) return COLI_E_DEVICE;
  // 3. the resident pairs' FFN, the shared expert among them, is enqueued before the host
  // plans. Copies already enqueued on the copy stream (a lookahead prefetch into this pool:
  // its experts count as resident) are waited for first. Past this point the call waits
  // for its route event before it returns, also on an error.
  if (hipEventRecord(cev, cs) != hipSuccess || hipStreamWaitEvent(s, cev, 0) != hipSuccess) {
    (void)hipEventSynchronize(rev);
    return COLI_E_DEVICE;
  }
  if ((st = phase(0, true, false))) {
    (void)hipEventSynchronize(rev);
    return st;
  }
  // 4. the plan, on the host, from the route (the call's one wait for the device)
  if (hipEventSynchronize(rev) != hipSuccess) return COLI_E_DEVICE;
  std::vector<int32_t> hs(P), le(slots), ls(slots);
  int32_t nl = 0;
  if ((st = coli_tier_plan(tier, hidx, T, k, hs.data(), le.data(), ls.data(), &nl))) return st;
  if (nl > 0) {
    // 5. the misses are copied on the copy stream; their pairs wait for the copies, then
    // run with the combine over every slot of every token (the weights of the whole
    // route, in slot order, over the pair rows both phases wrote)
    if ((st = coli_moe_tier_stage(cfg, slots, host_experts, host_scales, le.data(), ls.data(), nl, pool_experts,
                                  pool_scales, copy_stream)))
      return st;
    if (hipEventRecord(cev, cs) != hipSuccess) return COLI_E_DEVICE;
    TierMap miss;
    for (int32_t e = 0; e < 1024; e++) miss.slot[e] = -1;
    for (int32_t i = 0; i < nl; i++) miss.slot[le[i]] = (int16_t)ls[i];
    hipLaunchKernelGGL(tier_remap_kernel, dim3(rgrid), dim3(256), 0, s, idx, (int32_t)P, miss,
                       static_cast<int32_t *>(at(L.sidx[1])), static_cast<int32_t *>(nullptr));
    if (hipGetLastError() != hipSuccess || hipStreamWaitEvent(s, cev, 0) != hipSuccess) return COLI_E_DEVICE;
    if ((st = phase(1, false, true))) return st;
  } else if ((st = coli::combine_phase(&pc, T, wt, out, at(L.ffn), b_bytes, s))) {
    return st;
  }
  if (topk_idx_opt && hipMemcpyAsync(topk_idx_opt, idx, P * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return COLI_E_DEVICE;
  if (topk_w_opt && hipMemcpyAsync(topk_w_opt, wt, P * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return COLI_E_DEVICE;
  return COLI_OK;
}

int coli_moe_tier_prefetch(const coli_moe_cfg *cfg, const coli_moe_weights *w, coli_tier *tier,
                           const void *host_experts, const void *host_scales, void *pool_experts, void *pool_scales,
                           const float *x, int32_t T, void *workspace, size_t ws_bytes, void *stream,
                           void *copy_stream, int32_t *n_loaded_opt) {
  if (n_loaded_opt) *n_loaded_opt = 0;
  if (!cfg || !w || !tier || T < 0) return COLI_E_INVALID;
  if (T == 0) return COLI_OK;
  if (tier->n_experts != cfg->n_experts) return COLI_E_INVALID;
  const int32_t slots = tier->slots, k = cfg->top_k;
  TierWs L;
  if (!tier_ws(cfg, slots, T, L)) return COLI_E_INVALID;
  if (!workspace || ws_bytes < L.total) return COLI_E_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return COLI_E_ALIGN;
  if (!host_experts || !host_scales || !pool_experts || !pool_scales || !copy_stream) return COLI_E_INVALID;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  int32_t *idx = reinterpret_cast<int32_t *>(ws + L.idx);
  float *wt = reinterpret_cast<float *>(ws + L.w);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t P = (size_t)T * k;
  int st;
  int32_t *hidx = host_route(P);
  if (!hidx) return COLI_E_DEVICE;
  if ((st = coli_moe_route(cfg, w, x, T, idx, wt, ws + L.route, L.ffn - L.route, stream))) return st;
  if (hipMemcpyAsync(hidx, idx, P * 4, hipMemcpyDeviceToHost, s) != hipSuccess) return COLI_E_DEVICE;
  if (hipStreamSynchronize(s) != hipSuccess) return COLI_E_DEVICE;
  std::vector<int32_t> hs(P), le(slots), ls(slots);
  int32_t nl = 0;
  if ((st = coli_tier_plan(tier, hidx, T, k, hs.data(), le.data(), ls.data(), &nl))) return st;
  if (nl > 0 && (st = coli_moe_tier_stage(cfg, slots, host_experts, host_scales, le.data(), ls.data(), nl,
                                          pool_experts, pool_scales, copy_stream)))
    return st;
  if (n_loaded_opt) *n_loaded_opt = nl;
  return COLI_OK;
}

}  // extern "C"
