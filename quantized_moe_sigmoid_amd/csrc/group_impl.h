// group_impl.h — batch-union grouping as a workgroup-level device routine, shared
// by the standalone grouping kernel (1024 threads) and the fused tail of the
// routing kernel (256 threads).
//
// colibri-strix README, "What's implemented", batch-union item: the weights of an
// expert are fetched a single time per batch, however many tokens chose it.
// The route (pair p = t*k + j -> expert) becomes per-expert segments: counts,
// exclusive offsets, the pair ids of each expert in ascending p (a stable counting
// sort), and the list of experts with work, ascending.
//
// LDS only, no atomics, so the result is identical run to run. Pairs are cut into
// chunks of 64*Q consecutive ids; a wavefront ranks the pairs of a chunk that
// share an expert with ballots over the bits of the expert id (a 64-lane match),
// so the rank of a pair is the number of earlier pairs of its chunk with the same
// expert. Per-chunk counts go to an LDS histogram [chunk][expert]; one scan along
// chunks and one along experts give every pair its slot.
#pragma once

#include "coli_internal.h"

namespace coli {

constexpr int GROUP_HIST_BYTES = 48 * 1024;
constexpr int GROUP_ID_BITS = 11;  // expert ids 0..1023 are matched as id + 1 (0 = no pair)

__device__ __forceinline__ uint64_t group_match_mask(int v, int mine) {
  uint64_t m = ~0ull;
#pragma unroll
  for (int b = 0; b < GROUP_ID_BITS; b++) {
    const uint64_t bb = __ballot((v >> b) & 1);
    m &= ((mine >> b) & 1) ? bb : ~bb;
  }
  return m;
}

// For each of the Q pairs a lane owns in chunk c: expert (or -1), rank in the chunk,
// and the number of pairs of the chunk with the same expert.
template <int Q>
__device__ __forceinline__ void group_rank_chunk(const int32_t *__restrict__ idx, int P, int E, int c, int lane,
                                                 int (&ev)[Q], int (&rank)[Q], int (&tot)[Q], int &bad) {
#pragma unroll
  for (int q = 0; q < Q; q++) {
    const int p = c * 64 * Q + q * 64 + lane;
    int e = -1;
    if (p < P) {
      e = idx[p];
      if (e < 0 || e >= E) {
        if (e != -1) bad = 1;  // -1: an empty slot (adaptive top-p), part of no expert
        e = -1;
      }
    }
    ev[q] = e;
    rank[q] = 0;
    tot[q] = 0;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int qq = 0; qq < Q; qq++) {
    const int vq = ev[qq] + 1;
#pragma unroll
    for (int q = 0; q < Q; q++) {
      const uint64_t mm = group_match_mask(vq, ev[q] + 1);
      const int n = __popcll(mm);
      tot[q] += n;
      if (qq < q) rank[q] += n;
      if (qq == q) rank[q] += __popcll(mm & below);
    }
  }
}

// Pairs per lane (Q) and chunk count (C) so that the uint16 histogram fits in LDS.
__host__ __device__ inline bool group_shape(int P, int E, int &Q, int &C) {
  const int cmax = GROUP_HIST_BYTES / (2 * E);
  for (Q = 1; Q <= 16; Q <<= 1) {
    C = (P + 64 * Q - 1) / (64 * Q);
    if (C < 1) C = 1;
    if (C <= cmax) return true;
  }
  return false;
}

// LDS the routine needs besides the histogram.
template <int NT>
struct GroupLds {
  int32_t off_s[1024];
  int32_t wsum[NT / 64];
  int32_t wsum2[NT / 64];
  int bad;
};

// The whole workgroup (NT threads) groups the P pairs of idx. hist: C*E uint16 in LDS.
template <int NT, int Q>
__device__ void group_body(const int32_t *__restrict__ idx, int P, int E, int C, const GroupOut &o,
                           uint16_t *hist, GroupLds<NT> &L) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) L.bad = 0;
  for (int i = tid; i < C * E; i += NT) hist[i] = 0;
  __syncthreads();

  int bad = 0;
  for (int c = wv; c < C; c += NW) {
    int ev[Q], rank[Q], tot[Q];
    group_rank_chunk<Q>(idx, P, E, c, lane, ev, rank, tot, bad);
#pragma unroll
    for (int q = 0; q < Q; q++)
      if (ev[q] >= 0 && rank[q] == tot[q] - 1) hist[c * E + ev[q]] = (uint16_t)tot[q];
  }
  if (bad) L.bad = 1;
  __syncthreads();

  // experts [e_beg, e_end) of this thread: exclusive prefix over chunks (in place) and counts
  const int ept = (E + NT - 1) / NT;
  const int e_beg = min(E, tid * ept), e_end = min(E, e_beg + ept);
  int my_cnt = 0, my_flag = 0;
  for (int e = e_beg; e < e_end; e++) {
    int run = 0;
    for (int c = 0; c < C; c++) {
      const int h = hist[c * E + e];
      hist[c * E + e] = (uint16_t)run;
      run += h;
    }
    o.cnt[e] = run;
    L.off_s[e] = run;  // count for now; replaced by the offset below
    my_cnt += run;
    my_flag += run > 0 ? 1 : 0;
  }
  int incl = my_cnt, fincl = my_flag;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int a = __shfl_up(incl, s), b = __shfl_up(fincl, s);
    if (lane >= s) {
      incl += a;
      fincl += b;
    }
  }
  if (lane == 63) {
    L.wsum[wv] = incl;
    L.wsum2[wv] = fincl;
  }
  __syncthreads();
  int base = 0, fbase = 0;
  for (int i = 0; i < wv; i++) {
    base += L.wsum[i];
    fbase += L.wsum2[i];
  }
  int run = base + incl - my_cnt, frun = fbase + fincl - my_flag;
  for (int e = e_beg; e < e_end; e++) {
    const int n = L.off_s[e];
    o.off[e] = run;
    L.off_s[e] = run;
    if (n > 0) o.active[frun++] = e;
    run += n;
  }
  if (e_beg < e_end && e_end == E) {
    o.off[E] = run;
    *o.nact = L.bad ? -1 : frun;
  }
  __syncthreads();

  for (int c = wv; c < C; c += NW) {
    int ev[Q], rank[Q], tot[Q];
    int dummy = 0;
    group_rank_chunk<Q>(idx, P, E, c, lane, ev, rank, tot, dummy);
#pragma unroll
    for (int q = 0; q < Q; q++)
      if (ev[q] >= 0) o.perm[L.off_s[ev[q]] + hist[c * E + ev[q]] + rank[q]] = c * 64 * Q + q * 64 + lane;
  }
}

}  // namespace coli
