// group.hip — batch-union grouping on gfx950.
//
// colibri-strix README, "What's implemented", batch-union item: each distinct
// expert of the batch is read once and applied to every position routed to it.
// This kernel turns the route (pair p = t*k + j -> expert) into per-expert
// segments: counts, exclusive offsets, the pair ids of each expert in ascending
// p (a stable counting sort), and the list of experts with work, ascending.
//
// One workgroup of 1024 threads, LDS only, no atomics (results are identical
// run to run). Pairs are cut into chunks of 64*Q consecutive ids; a wavefront
// ranks the pairs of a chunk that share an expert with ballots over the bits of
// the expert id (a 64-lane "match"), so the rank of a pair is the number of
// earlier pairs of its chunk with the same expert. Per-chunk counts go to an
// LDS histogram [chunk][expert]; one scan along chunks and one along experts
// give every pair its final slot.
#include "coli_internal.h"

namespace coli {

constexpr int GROUP_THREADS = 1024;
constexpr int GROUP_HIST_BYTES = 48 * 1024;
constexpr int ID_BITS = 11;  // expert ids 0..1023 are stored as id + 1 (0 = no pair)

// Mask of the lanes whose value v' (in the wave) equals v, from the ballots of v's bits.
__device__ __forceinline__ uint64_t match_mask(int v, int mine) {
  uint64_t m = ~0ull;
#pragma unroll
  for (int b = 0; b < ID_BITS; b++) {
    const uint64_t bb = __ballot((v >> b) & 1);
    m &= ((mine >> b) & 1) ? bb : ~bb;
  }
  return m;
}

// For each of the Q pairs a lane owns in chunk c: expert (or -1) and rank in chunk;
// tot = number of pairs in the chunk with the same expert.
template <int Q>
__device__ __forceinline__ void rank_chunk(const int32_t *__restrict__ idx, int P, int E, int c, int lane,
                                           int (&ev)[Q], int (&rank)[Q], int (&tot)[Q], int &bad) {
#pragma unroll
  for (int q = 0; q < Q; q++) {
    const int p = c * 64 * Q + q * 64 + lane;
    int e = -1;
    if (p < P) {
      e = idx[p];
      if (e < 0 || e >= E) {
        bad = 1;
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
      const uint64_t mm = match_mask(vq, ev[q] + 1);
      const int n = __popcll(mm);
      tot[q] += n;
      if (qq < q) rank[q] += n;
      if (qq == q) rank[q] += __popcll(mm & below);
    }
  }
}

template <int Q>
__global__ __launch_bounds__(GROUP_THREADS) void group_kernel(const int32_t *__restrict__ idx, int P, int E,
                                                              int C, int32_t *__restrict__ cnt,
                                                              int32_t *__restrict__ off,
                                                              int32_t *__restrict__ perm,
                                                              int32_t *__restrict__ active,
                                                              int32_t *__restrict__ nact) {
  extern __shared__ uint16_t hist[];  // [C][E]
  __shared__ int32_t off_s[1024];
  __shared__ int32_t wsum[16];
  __shared__ int32_t wsum2[16];
  __shared__ int bad_s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) bad_s = 0;
  for (int i = tid; i < C * E; i += GROUP_THREADS) hist[i] = 0;
  __syncthreads();

  int bad = 0;
  for (int c = wv; c < C; c += GROUP_THREADS / 64) {
    int ev[Q], rank[Q], tot[Q];
    rank_chunk<Q>(idx, P, E, c, lane, ev, rank, tot, bad);
#pragma unroll
    for (int q = 0; q < Q; q++)
      if (ev[q] >= 0 && rank[q] == tot[q] - 1) hist[c * E + ev[q]] = (uint16_t)tot[q];
  }
  if (bad) bad_s = 1;
  __syncthreads();

  // per expert: exclusive prefix over chunks (in place) and total count
  int my_cnt = 0;
  if (tid < E) {
    int run = 0;
    for (int c = 0; c < C; c++) {
      const int h = hist[c * E + tid];
      hist[c * E + tid] = (uint16_t)run;
      run += h;
    }
    my_cnt = run;
    cnt[tid] = run;
  }
  // block-wide exclusive scans of the counts and of the "has work" flags
  const int flag = (tid < E && my_cnt > 0) ? 1 : 0;
  int incl = my_cnt, fincl = flag;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(incl, o), b = __shfl_up(fincl, o);
    if (lane >= o) {
      incl += a;
      fincl += b;
    }
  }
  if (lane == 63) {
    wsum[wv] = incl;
    wsum2[wv] = fincl;
  }
  __syncthreads();
  int base = 0, fbase = 0;
  for (int i = 0; i < wv; i++) {
    base += wsum[i];
    fbase += wsum2[i];
  }
  const int excl = base + incl - my_cnt, fexcl = fbase + fincl - flag;
  if (tid < E) {
    off[tid] = excl;
    off_s[tid] = excl;
    if (flag) active[fexcl] = tid;
  }
  if (tid == E - 1) {
    off[E] = excl + my_cnt;
    *nact = bad_s ? -1 : fexcl + flag;
  }
  __syncthreads();

  for (int c = wv; c < C; c += GROUP_THREADS / 64) {
    int ev[Q], rank[Q], tot[Q];
    int dummy = 0;
    rank_chunk<Q>(idx, P, E, c, lane, ev, rank, tot, dummy);
#pragma unroll
    for (int q = 0; q < Q; q++)
      if (ev[q] >= 0) perm[off_s[ev[q]] + hist[c * E + ev[q]] + rank[q]] = c * 64 * Q + q * 64 + lane;
  }
}

// Pairs per lane (Q) and chunk count (C) so that the histogram fits in LDS.
static bool group_shape(int P, int E, int &Q, int &C) {
  const int cmax = GROUP_HIST_BYTES / (2 * E);
  for (Q = 1; Q <= 16; Q <<= 1) {
    C = (P + 64 * Q - 1) / (64 * Q);
    if (C <= cmax) return true;
  }
  return false;
}

bool group_supported(int P, int E) {
  int Q, C;
  return P <= 65535 && E <= 1024 && group_shape(P, E, Q, C);
}

hipError_t launch_group(const coli_moe_cfg &c, const int32_t *idx, int32_t T, int32_t *cnt, int32_t *off,
                        int32_t *perm, int32_t *active, int32_t *nact, hipStream_t s) {
  const int E = c.n_experts, P = T * c.top_k;
  int Q, C;
  if (!group_shape(P, E, Q, C)) return hipErrorInvalidValue;
  if (C < 1) C = 1;
  const size_t lds = (size_t)C * E * sizeof(uint16_t);
  switch (Q) {
    case 1: hipLaunchKernelGGL(group_kernel<1>, dim3(1), dim3(GROUP_THREADS), lds, s, idx, P, E, C, cnt, off, perm, active, nact); break;
    case 2: hipLaunchKernelGGL(group_kernel<2>, dim3(1), dim3(GROUP_THREADS), lds, s, idx, P, E, C, cnt, off, perm, active, nact); break;
    case 4: hipLaunchKernelGGL(group_kernel<4>, dim3(1), dim3(GROUP_THREADS), lds, s, idx, P, E, C, cnt, off, perm, active, nact); break;
    case 8: hipLaunchKernelGGL(group_kernel<8>, dim3(1), dim3(GROUP_THREADS), lds, s, idx, P, E, C, cnt, off, perm, active, nact); break;
    default: hipLaunchKernelGGL(group_kernel<16>, dim3(1), dim3(GROUP_THREADS), lds, s, idx, P, E, C, cnt, off, perm, active, nact); break;
  }
  return hipGetLastError();
}

}  // namespace coli
