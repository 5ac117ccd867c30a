// router.hip — sigmoid noaux_tc router on gfx950, fused with the Q8_0
// quantisation of x.
//
// colibri-strix README, "What's implemented", router item: DeepSeek-V3-style
// sigmoid router (noaux_tc, routed_scaling_factor). Reading implemented here:
//   z_e = x . W_e in fp64 (each fp32*fp32 product is exact in fp64),
//   s_e = 1 / (1 + exp(-z_e)), c_e = s_e + bias_e (fp64);
//   group score = sum of the two largest c of a group of E/G contiguous experts
//   (its single c when E/G = 1); keep the Gk best groups; route the k best c
//   inside them, descending; lower index first on every tie;
//   w_j = (float)(s_j / sum_j s_j * rsf), summed in slot order.
// fp64 comparisons make the selection independent of summation order except for
// logits closer than fp64 rounding, and identical router rows give identical
// logits here, so ties resolve exactly as the definition says.
//
// Kernels:
//   logits_decode_kernel (T <= 16): 8 experts per workgroup and one K-chunk of
//     x staged in LDS for 1, 4 or 8 tokens; every lane issues all its weight loads
//     before the barrier; the 2 x TT fp64 partial sums of a wavefront are folded with
//     a reduce-scatter.
//   logits_mfma_kernel (T > 16): fp64 MFMA GEMM, K-split; logits_kernel (T <= 16
//     with H not a multiple of 256): LDS-tiled fp64 vector GEMM, K-split.
//   select_kernel: one workgroup per token quantises the token's x (Q8_0) unless
//     the logits kernel did, sums the K-split partials in a fixed order
//     (deterministic) and performs the group-limited top-k as rank counts over
//     LDS spread over the workgroup (sel_block, select_impl.h). For one decode
//     token the gate/up GEMV runs the same selection itself instead
//     (route_fusable).
#include "q8_0_impl.h"
#include "select_impl.h"

namespace coli {

// ------------------------------------------------------------------ logits, T <= 16
constexpr int LD_TT = 16;   // token capacity
constexpr int LD_EPW = 2;   // experts per wavefront

// fp64 lane exchanges without LDS traffic, one 32-bit half at a time. Within an
// aligned group of 2*O lanes the step for O pairs every lane of the lower half
// with one of the upper half: O = 32 and 16 by the permlane swaps (the upper 32
// lanes of one register with the lower 32 of another; odd 16-lane rows with even
// ones), O = 8 and 4 by the DPP row mirrors (partner l ^ 15, l ^ 7), O = 2 and 1
// by DPP quad permutes (l ^ 2, l ^ 1).
template <int O>
__device__ __forceinline__ double dpp_partner_d(double v) {
  constexpr int ctrl = (O == 8) ? 0x140 : (O == 4) ? 0x141 : (O == 2) ? 0x4E : 0xB1;
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, ctrl, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), ctrl, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// lower-half lanes get lo + partner's lo, upper-half lanes hi + partner's hi
template <int O>
__device__ __forceinline__ double pair_sum_d(double lo, double hi, bool up) {
  if constexpr (O == 32 || O == 16) {
    const uint64_t l = (uint64_t)__double_as_longlong(lo), h = (uint64_t)__double_as_longlong(hi);
    const auto r0 = (O == 32) ? __builtin_amdgcn_permlane32_swap((uint32_t)l, (uint32_t)h, false, false)
                              : __builtin_amdgcn_permlane16_swap((uint32_t)l, (uint32_t)h, false, false);
    const auto r1 = (O == 32) ? __builtin_amdgcn_permlane32_swap((uint32_t)(l >> 32), (uint32_t)(h >> 32), false, false)
                              : __builtin_amdgcn_permlane16_swap((uint32_t)(l >> 32), (uint32_t)(h >> 32), false, false);
    const double a = __longlong_as_double((long long)(((uint64_t)r1[0] << 32) | r0[0]));
    const double b = __longlong_as_double((long long)(((uint64_t)r1[1] << 32) | r0[1]));
    return a + b;
  } else {
    const double send = up ? lo : hi;
    const double keep = up ? hi : lo;
    return keep + dpp_partner_d<O>(send);
  }
}

template <int V, int O>
__device__ __forceinline__ void reduce_scatter_d(double *a, int lane, int &base) {
  if constexpr (O >= 1) {
    const bool up = (lane & O) != 0;
    if constexpr (V > 1) {
#pragma unroll
      for (int i = 0; i < V / 2; i++) a[i] = pair_sum_d<O>(a[i], a[i + V / 2], up);
      if (up) base += V / 2;
      reduce_scatter_d<V / 2, O / 2>(a, lane, base);
    } else {
      a[0] = pair_sum_d<O>(a[0], a[0], up);
      reduce_scatter_d<1, O / 2>(a, lane, base);
    }
  }
}

// When xq is set, the workgroups of each K chunk also quantise that chunk of x
// (Q8_0, 32-value blocks, eight lanes per block) from the copy staged in LDS, 32
// blocks per workgroup, so the selection kernel has no x work left.
// TT tokens per workgroup (tokens TT z .. TT z + TT - 1 of blockIdx.z): the 2 TT sums of
// a wavefront are folded with one reduce-scatter, so a one-token batch folds 2 sums,
// not 32, and 16 tokens run as two slices of 8 over twice the workgroups.
template <int NI, int TT>  // float4 per lane per row: kc = 256 * NI
__global__ __launch_bounds__(256) void logits_decode_kernel(const float *__restrict__ x, const float *__restrict__ W,
                                                            int T, int E, int H, double *__restrict__ part,
                                                            int8_t *__restrict__ xq, float *__restrict__ xd) {
  constexpr int KC = 256 * NI;
  constexpr int V = LD_EPW * TT;  // sums per lane
  static_assert(V <= 64 && (V & (V - 1)) == 0, "sums per wavefront fold to lanes");
  __shared__ float4 xs[TT * KC / 4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ks = blockIdx.y, k0 = ks * KC;
  const int t0 = blockIdx.z * TT, nt = min(TT, T - t0);  // this workgroup's tokens
  const int e0 = blockIdx.x * (4 * LD_EPW) + wv * LD_EPW;
  // weight loads first (independent of the LDS staging)
  float4 w[LD_EPW][NI];
#pragma unroll
  for (int j = 0; j < LD_EPW; j++) {
    const int e = min(e0 + j, E - 1);
#pragma unroll
    for (int i = 0; i < NI; i++)
      w[j][i] = reinterpret_cast<const float4 *>(W + (int64_t)e * H + k0)[i * 64 + lane];
  }
  for (int i = tid; i < nt * (KC / 4); i += 256) {
    const int t = i / (KC / 4), c = i % (KC / 4);
    xs[i] = reinterpret_cast<const float4 *>(x + (int64_t)(t0 + t) * H + k0)[c];
  }
  __syncthreads();
  if (xq) {
    constexpr int BPT = KC / QK;  // blocks per token in this chunk
    const int nq = nt * BPT, sub = tid & 7;
    for (int q0 = blockIdx.x * 32; q0 < nq; q0 += gridDim.x * 32) {
      const int q = q0 + (tid >> 3);
      if (q < nq) {  // uniform over the eight lanes of a block
        const int t = q / BPT, b = q % BPT;
        uint32_t packed;
        const float d = q8_0_block8(xs[t * (KC / 4) + b * 8 + sub], packed);
        reinterpret_cast<uint32_t *>(xq + (int64_t)(t0 + t) * H + k0)[b * 8 + sub] = packed;
        if (sub == 0) xd[(int64_t)(t0 + t) * (H / QK) + k0 / QK + b] = d;
      }
    }
  }
  double acc[V];
#pragma unroll
  for (int i = 0; i < V; i++) acc[i] = 0.0;
#pragma unroll
  for (int t = 0; t < TT; t++) {
    if (t < nt) {
#pragma unroll
      for (int i = 0; i < NI; i++) {
        const float4 xv = xs[t * (KC / 4) + i * 64 + lane];
#pragma unroll
        for (int j = 0; j < LD_EPW; j++) {
          double a = acc[j * TT + t];
          a = fma((double)xv.x, (double)w[j][i].x, a);
          a = fma((double)xv.y, (double)w[j][i].y, a);
          a = fma((double)xv.z, (double)w[j][i].z, a);
          a = fma((double)xv.w, (double)w[j][i].w, a);
          acc[j * TT + t] = a;
        }
      }
    }
  }
  int base = 0;
  reduce_scatter_d<V, 32>(acc, lane, base);
  if ((lane & (64 / V - 1)) == 0) {  // each sum is held by 64 / V lanes
    const int j = base / TT, t = base % TT, e = e0 + j;
    if (t < nt && e < E) part[((int64_t)ks * T + t0 + t) * E + e] = acc[0];
  }
}

// ------------------------------------------------------------------ logits, any T
// partial[ks][t][e] = sum over h in K-chunk ks of x[t][h] * W[e][h]
template <int TT, int TE, int RT, int RE>
__global__ __launch_bounds__(256) void logits_kernel(const float *__restrict__ x, const float *__restrict__ W,
                                                     int T, int E, int H, int kc, double *__restrict__ part) {
  constexpr int KB = 32;
  constexpr int NTX = TE / RE;  // threads along experts
  static_assert((TT / RT) * (TE / RE) == 256, "256 threads");
  __shared__ double xs[KB][TT + 1];
  __shared__ double ws[KB][TE + 1];
  const int tid = threadIdx.x;
  const int tx = tid % NTX, ty = tid / NTX;
  const int e0 = blockIdx.x * TE, t0 = blockIdx.y * TT, ks = blockIdx.z;
  const int hbeg = ks * kc;
  double acc[RT][RE];
#pragma unroll
  for (int i = 0; i < RT; i++)
#pragma unroll
    for (int j = 0; j < RE; j++) acc[i][j] = 0.0;

  for (int k0 = hbeg; k0 < hbeg + kc; k0 += KB) {
    for (int i = tid; i < TT * KB; i += 256) {
      const int tt = i / KB, kk = i % KB, t = t0 + tt;
      xs[kk][tt] = (t < T) ? (double)x[(int64_t)t * H + k0 + kk] : 0.0;
    }
    for (int i = tid; i < TE * KB; i += 256) {
      const int ee = i / KB, kk = i % KB, e = e0 + ee;
      ws[kk][ee] = (e < E) ? (double)W[(int64_t)e * H + k0 + kk] : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < KB; kk++) {
      double a[RT], b[RE];
#pragma unroll
      for (int i = 0; i < RT; i++) a[i] = xs[kk][ty * RT + i];
#pragma unroll
      for (int j = 0; j < RE; j++) b[j] = ws[kk][tx * RE + j];
#pragma unroll
      for (int i = 0; i < RT; i++)
#pragma unroll
        for (int j = 0; j < RE; j++) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < RT; i++) {
    const int t = t0 + ty * RT + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < RE; j++) {
      const int e = e0 + tx * RE + j;
      if (e < E) part[((int64_t)ks * T + t) * E + e] = acc[i][j];
    }
  }
}

// ------------------------------------------------------------------ logits, T > 16
// fp64 matrix cores (v_mfma_f64_16x16x4f64): a workgroup owns 64 tokens x 64
// experts of one K split, a wavefront 32 x 32 as 2 x 2 MFMA tiles. x and W stay
// fp32 in LDS (staged 32 K at a time, double-buffered) and are widened to fp64
// as operands, so every product is exact and only the fp64 summation order
// differs from any other evaluation. Lane l, result r of a 16 x 16 tile holds
// row (token) l / 16 + 4 r and column (expert) l % 16.
typedef double v4d __attribute__((ext_vector_type(4)));
constexpr int LM_T = 64, LM_E = 64, LM_KB = 32;

__global__ __launch_bounds__(256) void logits_mfma_kernel(const float *__restrict__ x, const float *__restrict__ W,
                                                          int T, int E, int H, int kc, double *__restrict__ part) {
  __shared__ float xs[2][LM_T][LM_KB + 1];
  __shared__ float ws[2][LM_E][LM_KB + 1];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;
  const int t0 = blockIdx.y * LM_T, e0 = blockIdx.x * LM_E, ks = blockIdx.z;
  const int k0 = ks * kc, nst = kc / LM_KB;

  // staging: 2 float4 of x and 2 of W per thread and stage
  float4 rx[2], rw[2];
  auto gload = [&](int st) {
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int q = tid + 256 * j, row = q >> 3, c4 = q & 7;
      const int t = t0 + row, e = e0 + row;
      const int64_t k = k0 + (int64_t)st * LM_KB + 4 * c4;
      rx[j] = (t < T) ? *reinterpret_cast<const float4 *>(x + (int64_t)t * H + k) : make_float4(0.f, 0.f, 0.f, 0.f);
      rw[j] = (e < E) ? *reinterpret_cast<const float4 *>(W + (int64_t)e * H + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int q = tid + 256 * j, row = q >> 3, c = 4 * (q & 7);
      xs[buf][row][c] = rx[j].x;
      xs[buf][row][c + 1] = rx[j].y;
      xs[buf][row][c + 2] = rx[j].z;
      xs[buf][row][c + 3] = rx[j].w;
      ws[buf][row][c] = rw[j].x;
      ws[buf][row][c + 1] = rw[j].y;
      ws[buf][row][c + 2] = rw[j].z;
      ws[buf][row][c + 3] = rw[j].w;
    }
  };

  v4d acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; a++)
#pragma unroll
    for (int b = 0; b < 2; b++) acc[a][b] = (v4d){0.0, 0.0, 0.0, 0.0};

  const int ri = lane & 15, rk = lane >> 4;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int st = 0; st < nst; st++) {
    const int buf = st & 1;
    const bool more = st + 1 < nst;
    if (more) gload(st + 1);
#pragma unroll
    for (int kk = 0; kk < LM_KB; kk += 4) {
      double av[2], bv[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; s2++) {
        av[s2] = (double)xs[buf][wm * 32 + s2 * 16 + ri][kk + rk];
        bv[s2] = (double)ws[buf][wn * 32 + s2 * 16 + ri][kk + rk];
      }
#pragma unroll
      for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 2; b++) acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; a++)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int t = t0 + wm * 32 + a * 16 + rk + 4 * r;
        const int e = e0 + wn * 32 + b * 16 + ri;
        if (t < T && e < E) part[((int64_t)ks * T + t) * E + e] = acc[a][b][r];
      }
}

// ------------------------------------------------------------------ selection
// One workgroup per token: the token's row of x is quantised (Q8_0) first when the
// logits kernel has not done it, the K-split partials are summed in a fixed order
// (deterministic) into s and c in LDS, and the whole workgroup selects (sel_block:
// group-limited top-k as rank counts over LDS).
template <int EPT>
__global__ __launch_bounds__(SEL_NT) void select_kernel(SelectArgs a) {
  __shared__ double cs[SEL_NT * EPT], ss[SEL_NT * EPT];
  __shared__ SelBlockLds<EPT> L;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int E = a.E;

  // the K-split partials of this thread's experts, loaded before the x work so
  // that both round trips overlap (up to PK splits in registers, the rest later)
  // (clamped indices: every load is valid and unconditional, so all of them go
  // out before the first wait; values past E or ksplit are never used)
  constexpr int PK = (EPT == 1) ? 24 : 8;
  double pv[EPT][PK];
#pragma unroll
  for (int i = 0; i < EPT; i++) load_partials(a, t, tid + SEL_NT * i, pv[i]);

  if (a.xq) {  // eight lanes per 32-value block; XQ blocks per thread loaded at once
    constexpr int XQ = 8;
    const int nblk = a.H / QK;
    const float *xr = a.x + (int64_t)t * a.H;
    const int sub = tid & 7;
    auto chunk = [&](int b0) {
      float4 v[XQ];
#pragma unroll
      for (int i = 0; i < XQ; i++) {  // clamped: blocks past nblk are quantised but not stored
        const int blk = min(b0 + i * (SEL_NT / 8) + (tid >> 3), nblk - 1);
        v[i] = reinterpret_cast<const float4 *>(xr)[blk * 8 + sub];
      }
#pragma unroll
      for (int i = 0; i < XQ; i++) {
        if (b0 + i * (SEL_NT / 8) < nblk) {  // uniform: whole groups of eight lanes
          const int blk = b0 + i * (SEL_NT / 8) + (tid >> 3);
          uint32_t packed;
          const float d = q8_0_block8(v[i], packed);
          if (blk < nblk) {
            reinterpret_cast<uint32_t *>(a.xq + (int64_t)t * a.H)[blk * 8 + sub] = packed;
            if (sub == 0) a.xd[(int64_t)t * nblk + blk] = d;
          }
        }
      }
    };
    chunk(0);  // outside the loop: its loads need not wait for the partials
    for (int b0 = XQ * (SEL_NT / 8); b0 < nblk; b0 += XQ * (SEL_NT / 8)) chunk(b0);
  }

#pragma unroll
  for (int i = 0; i < EPT; i++) {
    const int e = tid + SEL_NT * i;
    if (e < E) sel_score(a, t, e, pv[i], ss[e], cs[e]);
  }
  __syncthreads();
  int e;
  float wt;
  sel_block<EPT>(a, cs, ss, L, e, wt);
  if (tid < a.k) {
    a.idx[(int64_t)t * a.k + tid] = e;
    a.w[(int64_t)t * a.k + tid] = wt;
  }
}

// ------------------------------------------------------------------ host side
int32_t route_ksplit(const coli_moe_cfg &c, int32_t T) {
  // decode sizes: 256-wide K chunks give enough workgroups; one token takes 512-wide
  // chunks, half the partials for the selection inside the gate/up GEMV to sum
  // (measured: GLM-scale T = 1 45.8 -> 44.5 us per layer)
  if (T == 1 && c.hidden % 512 == 0) return c.hidden / 512;
  if (T <= LD_TT && c.hidden % 256 == 0) return c.hidden / 256;
  // larger T: enough K splits for about 512 workgroups of 64 x 64 (tokens x experts)
  const int nkb = c.hidden / 32;
  const int64_t tiles = (int64_t)((c.n_experts + LM_E - 1) / LM_E) * ((T + LM_T - 1) / LM_T);
  const int64_t want = (512 + tiles - 1) / tiles;
  const int cand[6] = {8, 6, 4, 3, 2, 1};
  for (int i = 0; i < 6; i++)
    if (cand[i] <= want && nkb % cand[i] == 0) return cand[i];
  return 1;
}

// Whether the decode gate/up GEMVs select this batch's route themselves: one token
// (every workgroup repeats the selection, about 2 us at E = 64 and 4.5 us at E = 256
// in a workgroup's timeline, against about 3 us that the selection launch and its
// boundary cost; two tokens would double the repeated work), the decode logits kernel
// runs (x quantised there), E <= 512, and the partials every workgroup reads (E *
// ksplit doubles) stay small.
constexpr int64_t FUSE_PART_BYTES = 64 << 10;
bool route_fusable(const coli_moe_cfg &c, int32_t T, int32_t ks) {
  if (T != 1 || c.hidden % 256 || c.top_k > LOCAL_GROUP_MAX_P || c.n_experts > 2 * SEL_NT) return false;
  return (int64_t)c.n_experts * ks * 8 <= FUSE_PART_BYTES;
}

hipError_t launch_route(const RouteLaunch &r, hipStream_t s, hipEvent_t mid, SelectArgs *fused) {
  const coli_moe_cfg &c = *r.cfg;
  const int E = c.n_experts, H = c.hidden, T = r.T;
  const int ks = r.ksplit;
  bool x_done = false;  // x quantised by the logits kernel
  if (T <= LD_TT && H % 256 == 0) {
    // route_ksplit gives 256-wide K chunks here (one float4 per lane and row), or
    // 512-wide ones (two) for one token
    if (H / ks != 256 && !(T == 1 && H / ks == 512)) return hipErrorInvalidValue;
    const int gx = (E + 4 * LD_EPW - 1) / (4 * LD_EPW);
    if (H / ks == 512)
      hipLaunchKernelGGL((logits_decode_kernel<2, 1>), dim3(gx, ks, 1), dim3(256), 0, s, r.x, r.W, T, E, H, r.logits,
                         r.xq, r.xd);
    else if (T == 1)
      hipLaunchKernelGGL((logits_decode_kernel<1, 1>), dim3(gx, ks, 1), dim3(256), 0, s, r.x, r.W, T, E, H, r.logits,
                         r.xq, r.xd);
    else if (T <= 4)
      hipLaunchKernelGGL((logits_decode_kernel<1, 4>), dim3(gx, ks, 1), dim3(256), 0, s, r.x, r.W, T, E, H, r.logits,
                         r.xq, r.xd);
    else
      hipLaunchKernelGGL((logits_decode_kernel<1, 8>), dim3(gx, ks, (T + 7) / 8), dim3(256), 0, s, r.x, r.W, T, E, H,
                         r.logits, r.xq, r.xd);
    x_done = true;
  } else if (T <= LD_TT) {
    dim3 grid((E + 15) / 16, 1, ks);
    hipLaunchKernelGGL((logits_kernel<16, 16, 1, 1>), grid, dim3(256), 0, s, r.x, r.W, T, E, H, H / ks, r.logits);
  } else {
    dim3 grid((E + LM_E - 1) / LM_E, (T + LM_T - 1) / LM_T, ks);
    hipLaunchKernelGGL(logits_mfma_kernel, grid, dim3(256), 0, s, r.x, r.W, T, E, H, H / ks, r.logits);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid && (err = hipEventRecord(mid, s)) != hipSuccess) return err;

  SelectArgs a{};
  a.part = r.logits;
  a.ksplit = ks;
  a.T = T;
  a.E = E;
  a.G = c.n_group;
  a.Gk = c.topk_group;
  a.k = c.top_k;
  a.rsf = c.routed_scaling_factor;
  a.topp = c.topp;
  a.bias = r.bias;
  a.idx = r.idx;
  a.w = r.w;
  a.x = r.x;
  a.H = H;
  a.xq = x_done ? nullptr : r.xq;
  a.xd = r.xd;
  sel_plan(a);
  if (fused) {
    *fused = SelectArgs{};
    if (x_done && route_fusable(c, T, ks)) {  // the selection runs in the gate/up GEMV
      *fused = a;
      return hipSuccess;
    }
  }
  if (T == 0) return hipSuccess;
  if (E <= SEL_NT)
    hipLaunchKernelGGL(select_kernel<1>, dim3(T), dim3(SEL_NT), 0, s, a);
  else if (E <= 2 * SEL_NT)
    hipLaunchKernelGGL(select_kernel<2>, dim3(T), dim3(SEL_NT), 0, s, a);
  else
    hipLaunchKernelGGL(select_kernel<4>, dim3(T), dim3(SEL_NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace coli
