// tier.hip — the expert residency tier: host RAM -> a pool of expert slots in HBM.
//
// JustVugg/colibri README, "Never wait for the disk twice" and its I/O items: a
// per-layer LRU of experts with a pinned hot store, missing experts loaded on demand,
// every expert of the batch union read once. The planner is host code over
// caller-owned state; the copies are host->device DMA on the caller's stream. The
// FFN kernels are not involved: they run on the pool with the route in slot ids.
#include <vector>

#include "coli_internal.h"

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

}  // extern "C"
