// select_impl.h — the expert selection of the sigmoid noaux_tc router as device code,
// shared by the selection kernel (router.hip) and by the decode gate/up GEMVs that
// select a one-token route themselves (ffn_gemv_impl.h), so that both give the same ids
// and weights bit for bit.
//
// colibri-strix README, "What's implemented", router item (DeepSeek-V3-style sigmoid
// noaux_tc router with routed_scaling_factor). From the fp64 logits z_e (summed from
// K-split partials in split order):
//   s_e = 1 / (1 + exp(-z_e)), c_e = s_e + bias_e;
//   group score = sum of the two largest c of a group of E/G contiguous experts (its
//   single c when E/G = 1); keep the Gk best groups; the k best c inside them,
//   descending, lower index first on every tie;
//   w_j = (float)(s_j / sum_j s_j * rsf), summed in slot order; with topp > 0 only the
//   shortest prefix of the slots whose scores reach topp of their sum is kept and
//   renormalised by the prefix's sum.
#pragma once

#include "coli_internal.h"

namespace coli {

constexpr int SEL_NT = 256;  // threads per token (selection kernels, fused route)

// lane j's value (j wave-uniform), through scalar registers
__device__ __forceinline__ double lane_d(double v, int j) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, j);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), j);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// (v, i) ranks before (v2, i2): larger value first, then lower index
__device__ __forceinline__ bool before(double v2, int i2, double v, int i) { return v2 > v || (v2 == v && i2 < i); }

// The K-split logit partials of expert e (clamped: every load is valid, values past
// E or ksplit are never used), first PK of them into registers
template <int PK>
__device__ __forceinline__ void load_partials(const SelectArgs &a, int t, int e, double (&pv)[PK]) {
  const int ec = min(e, a.E - 1);
#pragma unroll
  for (int j = 0; j < PK; j++) pv[j] = a.part[((int64_t)min(j, a.ksplit - 1) * a.T + t) * a.E + ec];
}

// z of expert e: the partials summed in split order (the first PK from registers, the
// rest loaded eight at a time)
template <int PK>
__device__ __forceinline__ double sum_partials(const SelectArgs &a, int t, int e, const double (&pv)[PK]) {
  double z = 0.0;
#pragma unroll
  for (int j = 0; j < PK; j++)
    if (j < a.ksplit) z += pv[j];
  const double *pp = a.part + (int64_t)t * a.E + e;
  const int64_t stride = (int64_t)a.T * a.E;
  for (int k0 = PK; k0 < a.ksplit; k0 += 8) {
    double v[8];
#pragma unroll
    for (int j = 0; j < 8; j++) v[j] = (k0 + j < a.ksplit) ? pp[(k0 + j) * stride] : 0.0;
#pragma unroll
    for (int j = 0; j < 8; j++)
      if (k0 + j < a.ksplit) z += v[j];
  }
  return z;
}

// s and c of expert e of token t from its partials (pv: the first PK, loaded ahead)
template <int PK>
__device__ __forceinline__ void sel_score(const SelectArgs &a, int t, int e, const double (&pv)[PK], double &s,
                                          double &c) {
  const double z = sum_partials(a, t, e, pv);
  s = 1.0 / (1.0 + exp(-z));
  c = s + (double)a.bias[e];
}

// ---- the rank-based selection of one token by a whole workgroup ------------------
// Every step is a count of ranks over LDS, the comparisons of a step independent of
// each other and spread over the workgroup's threads (no chain of lane exchanges):
//   - the rank of each expert inside its group (c desc, lower index first), P threads
//     per expert splitting the group's entries when E < SEL_NT;
//   - one group: the in-group rank is the slot;
//   - else the two best c of a group (in-group ranks 0 and 1) sum to its score, and a
//     group is kept when fewer than Gk group scores rank before it (lower group index
//     first on ties). An expert with k or more better experts in its own group cannot
//     be among the k best, so the candidates are the kk = min(k, m) best of each kept
//     group, placed at (rank of the group among the kept ones) * kk + in-group rank;
//     the rank of a candidate among the candidates is its rank among all kept experts
//     (every expert ranked before a selected one is a candidate), hence its slot when
//     below k.
// Ranks are exact (the index breaks every tie), so the result is that of the
// definition.
template <int EPT>
struct SelBlockLds {
  double cand_c[SEL_NT * EPT];
  double cand_s[SEL_NT * EPT];
  int cand_e[SEL_NT * EPT];
  double gtop[64][2];
  int gpos[64];  // rank of a kept group among the kept groups, else -1
  int sel_e[64];
  double sel_s[64];
};

// entries j in [first, first + n) of (val[j], id(j)) that rank before (c, e); n is the
// same in every lane of the wavefront
template <typename IdOf>
__device__ __forceinline__ int count_before_n(const double *val, int first, int n, double c, int e, IdOf id) {
  int r = 0;
#pragma unroll 4
  for (int j = 0; j < n; j++) r += before(val[first + j], id(first + j), c, e) ? 1 : 0;
  return r;
}

// sum of v over each aligned group of P consecutive lanes (P a power of two <= 64),
// in every lane of the group: a butterfly over the DPP partners l ^ 1, l ^ 2 (quad
// permutes), l ^ 7, l ^ 15 (half-row and row mirrors), which pair the halves of groups
// of 2, 4, 8 and 16 lanes, then lane shuffles for 32 and 64
__device__ __forceinline__ int sum_lanes(int v, int P) {
  if (P > 1) v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  if (P > 2) v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  if (P > 4) v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  if (P > 8) v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  if (P > 16) v += __shfl_xor(v, 16);
  if (P > 32) v += __shfl_xor(v, 32);
  return v;
}

// threads per item when SEL_NT threads share n items of `len` entries each: the
// largest power of two P <= 64 with n * P <= SEL_NT that divides len
__host__ __device__ inline int sel_split(int n, int len) {
  int P = 1;
  while (P < 64 && n * (2 * P) <= SEL_NT && len % (2 * P) == 0) P *= 2;
  return P;
}

// The selection's shape for E experts in G groups, k slots, Gk kept groups (host side,
// once per launch; the kernels read it from the arguments instead of dividing)
inline void sel_plan(SelectArgs &a) {
  const int m = a.E / a.G;
  a.m = m;
  a.gshift = (m & (m - 1)) ? -1 : __builtin_ctz(m);
  a.P = (a.E <= SEL_NT) ? sel_split(a.E, m) : 1;
  a.n1 = m / a.P;
  a.kk = a.k < m ? a.k : m;
  a.nc = a.Gk * a.kk;
  a.P2 = (a.nc <= SEL_NT) ? sel_split(a.nc, a.nc) : 1;
  a.n2 = a.nc / a.P2;
}

// group of expert e
__device__ __forceinline__ int sel_group(const SelectArgs &a, int e) { return a.gshift >= 0 ? e >> a.gshift : e / a.m; }

// cs, ss: c and s of the token's E <= SEL_NT * EPT experts in LDS, visible to every
// thread. Every thread of the workgroup calls it; thread j < k returns slot j's expert
// (-1 when dropped by top-p) and weight. L may be reused once every thread has
// returned and passed a barrier.
template <int EPT>
__device__ __forceinline__ void sel_block(const SelectArgs &a, const double *cs, const double *ss,
                                          SelBlockLds<EPT> &L, int &e_out, float &w_out) {
  const int tid = threadIdx.x;
  const int E = a.E, G = a.G, k = a.k, m = a.m;
  auto self = [](int j) { return j; };
  if (tid < 64) L.sel_e[tid] = -1;
  // in-group ranks: expert tid / P, part tid % P of its group's m entries (P = 1 when
  // a thread holds several experts)
  const int P = (EPT == 1) ? a.P : 1, n1 = (EPT == 1) ? a.n1 : m;
  const int p = tid & (P - 1), lp = __builtin_ctz(P);
  int ex[EPT], rin[EPT], gx[EPT];
  double cx[EPT];
#pragma unroll
  for (int i = 0; i < EPT; i++) {
    ex[i] = (EPT == 1) ? tid >> lp : tid + SEL_NT * i;
    gx[i] = sel_group(a, ex[i]);
    rin[i] = 0;
    cx[i] = 0.0;
    if (ex[i] < E) {
      cx[i] = cs[ex[i]];
      rin[i] = count_before_n(cs, gx[i] * m + p * n1, n1, cx[i], ex[i], self);
    }
    rin[i] = sum_lanes(rin[i], P);
  }
  const bool lead = p == 0;
  if (G == 1) {
    __syncthreads();  // sel_e initialised
#pragma unroll
    for (int i = 0; i < EPT; i++)
      if (lead && ex[i] < E && rin[i] < k) {
        L.sel_e[rin[i]] = ex[i];
        L.sel_s[rin[i]] = ss[ex[i]];
      }
  } else {
#pragma unroll
    for (int i = 0; i < EPT; i++)
      if (lead && ex[i] < E && rin[i] < 2) L.gtop[gx[i]][rin[i]] = cx[i];
    __syncthreads();
    // group scores and their ranks (lane g of wavefront 0 for group g)
    if (tid < 64) {
      const int g = tid;
      double sc = -INFINITY;
      if (g < G) sc = (m > 1) ? L.gtop[g][0] + L.gtop[g][1] : L.gtop[g][0];
      int r = 0;
      for (int j = 0; j < G; j++) r += before(lane_d(sc, j), j, sc, g) ? 1 : 0;
      if (g < G) L.gpos[g] = (r < a.Gk) ? r : -1;
    }
    __syncthreads();
    const int kk = a.kk;
#pragma unroll
    for (int i = 0; i < EPT; i++)
      if (lead && ex[i] < E && rin[i] < kk) {
        const int gp = L.gpos[gx[i]];
        if (gp >= 0) {
          const int q = gp * kk + rin[i];
          L.cand_c[q] = cx[i];
          L.cand_s[q] = ss[ex[i]];
          L.cand_e[q] = ex[i];
        }
      }
    __syncthreads();
    // rank of each candidate among the nc candidates, P2 threads per candidate
    const int nc = a.nc;
    auto cid = [&](int j) { return L.cand_e[j]; };
    if (nc <= SEL_NT) {
      const int P2 = a.P2, n2 = a.n2;
      const int q = tid >> __builtin_ctz(P2), p2 = tid & (P2 - 1);
      int r = 0;
      double cq = 0.0;
      int eq = 0;
      if (q < nc) {
        cq = L.cand_c[q];
        eq = L.cand_e[q];
        r = count_before_n(L.cand_c, p2 * n2, n2, cq, eq, cid);
      }
      r = sum_lanes(r, P2);
      if (q < nc && p2 == 0 && r < k) {
        L.sel_e[r] = eq;
        L.sel_s[r] = L.cand_s[q];
      }
    } else {
      for (int q = tid; q < nc; q += SEL_NT) {
        const double cq = L.cand_c[q];
        const int eq = L.cand_e[q];
        const int r = count_before_n(L.cand_c, 0, nc, cq, eq, cid);
        if (r < k) {
          L.sel_e[r] = eq;
          L.sel_s[r] = L.cand_s[q];
        }
      }
    }
  }
  __syncthreads();
  e_out = -1;
  w_out = 0.0f;
  if (tid < k) {
    double S = 0.0;
    for (int j = 0; j < k; j++) S += L.sel_s[j];
    int kept = k;
    if (a.topp > 0.0f) {
      // adaptive top-p: the shortest prefix of the slots whose scores reach topp * S;
      // its sum (same order) renormalises the kept weights
      const double target = (double)a.topp * S;
      double cum = 0.0;
      for (int j = 0; j < k; j++) {
        cum += L.sel_s[j];
        if (cum >= target) {
          kept = j + 1;
          break;
        }
      }
      S = cum;
    }
    const int e = L.sel_e[tid];
    if (tid < kept && e >= 0) {
      e_out = e;
      w_out = (float)((L.sel_s[tid] / S) * (double)a.rsf);
    }
  }
}

// ---- the route selected inside a decode gate/up GEMV workgroup --------------------
// The whole workgroup (SEL_NT threads) sums the partials of the T * E (token, expert)
// items into s and c in LDS, NB items per thread in flight with their first PK
// partials in registers (sel_score, as select_kernel); then it selects the tokens one
// after another (sel_block) and writes the ids to route[t * k + j] (LDS); the writer
// workgroup also stores ids and weights to a.idx / a.w for the kernels that follow.
// Every thread of the workgroup calls it; it returns after a workgroup barrier. The
// arithmetic is select_kernel's, so ids and weights are the same bit for bit.
template <int NB, int PK>
__device__ __forceinline__ void fused_scores(const SelectArgs &a, double *cs, double *ss) {
  const int tid = threadIdx.x, E = a.E, n = a.T * E;
  for (int q0 = 0; q0 < n; q0 += NB * SEL_NT) {
    double pv[NB][PK];
#pragma unroll
    for (int i = 0; i < NB; i++) {
      const int q = min(q0 + tid + SEL_NT * i, n - 1);  // clamped: every load is valid
      load_partials(a, q / E, q % E, pv[i]);
    }
#pragma unroll
    for (int i = 0; i < NB; i++) {
      const int q = q0 + tid + SEL_NT * i;
      if (q < n) sel_score(a, q / E, q % E, pv[i], ss[q], cs[q]);
    }
  }
}

// The selection of the T tokens one after another by the whole workgroup (sel_block);
// sl: its LDS (E <= SEL_NT * EPT).
template <int EPT>
__device__ __forceinline__ void fused_select(const SelectArgs &a, const double *cs, const double *ss, int *route,
                                             bool writer, SelBlockLds<EPT> &sl) {
  const int tid = threadIdx.x, k = a.k, E = a.E;
  for (int t = 0; t < a.T; t++) {
    int e;
    float wt;
    sel_block<EPT>(a, cs + t * E, ss + t * E, sl, e, wt);
    if (tid < k) {
      route[t * k + tid] = e;
      if (writer) {
        a.idx[(int64_t)t * k + tid] = e;
        a.w[(int64_t)t * k + tid] = wt;
      }
    }
    __syncthreads();  // sl reused by the next token; route visible
  }
}

// dyn: dynamic LDS of fused_lds_bytes (c and s of the T * E items, the selection's LDS)
__device__ __forceinline__ void fused_route(const SelectArgs &a, char *dyn, int *route, bool writer) {
  double *cs = reinterpret_cast<double *>(dyn);
  double *ss = cs + a.T * a.E;
  char *sl = reinterpret_cast<char *>(ss + a.T * a.E);
  if (a.ksplit > 16)
    fused_scores<1, 24>(a, cs, ss);
  else if (a.ksplit > 8)
    fused_scores<1, 16>(a, cs, ss);
  else
    fused_scores<1, 8>(a, cs, ss);
  __syncthreads();
  if (a.E <= SEL_NT)
    fused_select<1>(a, cs, ss, route, writer, *reinterpret_cast<SelBlockLds<1> *>(sl));
  else
    fused_select<2>(a, cs, ss, route, writer, *reinterpret_cast<SelBlockLds<2> *>(sl));
}

// dynamic LDS of fused_route: c and s of T * E items and the selection's LDS
__host__ __device__ inline size_t fused_route_lds(int T, int E) {
  const size_t sl = E <= SEL_NT ? sizeof(SelBlockLds<1>) : sizeof(SelBlockLds<2>);
  return (size_t)2 * T * E * sizeof(double) + sl;
}

}  // namespace coli
