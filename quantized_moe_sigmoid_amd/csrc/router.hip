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
//     x staged in LDS; every lane issues all its weight loads before the barrier;
//     the 2 x T fp64 partial sums of a wavefront are folded with a reduce-scatter.
//   logits_kernel (larger T): LDS-tiled fp64 GEMM, K-split.
//   select_kernel: one wavefront per token sums the K-split partials in a fixed
//     order (deterministic), quantises the token's x, and performs the
//     group-limited top-k with shuffles.
#include "q8_0_impl.h"

namespace coli {

// ------------------------------------------------------------------ logits, T <= 16
constexpr int LD_TT = 16;   // token capacity
constexpr int LD_EPW = 2;   // experts per wavefront

template <int V, int O>
__device__ __forceinline__ void reduce_scatter_d(double *a, int lane, int &base) {
  if constexpr (O >= 1) {
    if constexpr (V > 1) {
      const bool up = (lane & O) != 0;
#pragma unroll
      for (int i = 0; i < V / 2; i++) {
        const double send = up ? a[i] : a[i + V / 2];
        const double keep = up ? a[i + V / 2] : a[i];
        a[i] = keep + __shfl_xor(send, O);
      }
      if (up) base += V / 2;
      reduce_scatter_d<V / 2, O / 2>(a, lane, base);
    } else {
      a[0] += __shfl_xor(a[0], O);
      reduce_scatter_d<1, O / 2>(a, lane, base);
    }
  }
}

template <int NI>  // float4 per lane per row: kc = 256 * NI
__global__ __launch_bounds__(256) void logits_decode_kernel(const float *__restrict__ x, const float *__restrict__ W,
                                                            int T, int E, int H, double *__restrict__ part) {
  constexpr int KC = 256 * NI;
  __shared__ float4 xs[LD_TT * KC / 4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ks = blockIdx.y, k0 = ks * KC;
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
  for (int i = tid; i < T * (KC / 4); i += 256) {
    const int t = i / (KC / 4), c = i % (KC / 4);
    xs[i] = reinterpret_cast<const float4 *>(x + (int64_t)t * H + k0)[c];
  }
  __syncthreads();
  double acc[LD_EPW * LD_TT];
#pragma unroll
  for (int i = 0; i < LD_EPW * LD_TT; i++) acc[i] = 0.0;
#pragma unroll
  for (int t = 0; t < LD_TT; t++) {
    if (t < T) {
#pragma unroll
      for (int i = 0; i < NI; i++) {
        const float4 xv = xs[t * (KC / 4) + i * 64 + lane];
#pragma unroll
        for (int j = 0; j < LD_EPW; j++) {
          double a = acc[j * LD_TT + t];
          a = fma((double)xv.x, (double)w[j][i].x, a);
          a = fma((double)xv.y, (double)w[j][i].y, a);
          a = fma((double)xv.z, (double)w[j][i].z, a);
          a = fma((double)xv.w, (double)w[j][i].w, a);
          acc[j * LD_TT + t] = a;
        }
      }
    }
  }
  int base = 0;
  reduce_scatter_d<LD_EPW * LD_TT, 32>(acc, lane, base);
  if ((lane & 1) == 0) {
    const int j = base / LD_TT, t = base % LD_TT, e = e0 + j;
    if (t < T && e < E) part[((int64_t)ks * T + t) * E + e] = acc[0];
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

// ------------------------------------------------------------------ selection
// Arg-max over the wavefront of (v, i), larger v first, then lower i; carries s.
__device__ __forceinline__ void wave_argmax(double &v, int &i, double &s) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const double ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(i, o);
    const double os = __shfl_xor(s, o);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
      s = os;
    }
  }
}

struct SelectArgs {
  const double *part;
  int ksplit, T, E, G, Gk, k;
  float rsf;
  const float *bias;
  int32_t *idx;
  float *w;
  const float *x;  // quantised into xq/xds when xq != nullptr
  int H;
  int8_t *xq;
  int2 *xds;
};

template <int EPL>
__device__ __forceinline__ void select_token(const SelectArgs &a, int t, int lane) {
  const int E = a.E, G = a.G, k = a.k;
  const int m = E / G;
  const double NEG = -INFINITY;
  double s[EPL], c[EPL];
#pragma unroll
  for (int i = 0; i < EPL; i++) {
    s[i] = 0.0;
    c[i] = NEG;
    const int e = lane * EPL + i;
    if (e < E) {
      double z = 0.0;
#pragma unroll 8
      for (int ks = 0; ks < a.ksplit; ks++) z += a.part[((int64_t)ks * a.T + t) * E + e];
      s[i] = 1.0 / (1.0 + exp(-z));
      c[i] = s[i] + (double)a.bias[e];
    }
  }
  // group scores; lane g keeps the score of group g
  double my_gs = NEG;
  for (int g = 0; g < G; g++) {
    const int lo = g * m, hi = lo + m;
    double v1 = NEG, dummy = 0.0;
    int i1 = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPL; i++) {
      const int e = lane * EPL + i;
      if (e >= lo && e < hi && (c[i] > v1 || (c[i] == v1 && e < i1))) {
        v1 = c[i];
        i1 = e;
      }
    }
    wave_argmax(v1, i1, dummy);
    double gs = v1;
    if (m > 1) {
      double v2 = NEG;
      int i2 = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < EPL; i++) {
        const int e = lane * EPL + i;
        if (e >= lo && e < hi && e != i1 && (c[i] > v2 || (c[i] == v2 && e < i2))) {
          v2 = c[i];
          i2 = e;
        }
      }
      wave_argmax(v2, i2, dummy);
      gs = v1 + v2;
    }
    if (lane == g) my_gs = gs;
  }
  uint64_t kept = 0;
  for (int r = 0; r < a.Gk; r++) {
    const bool cand = lane < G && !((kept >> lane) & 1ull);
    double v = cand ? my_gs : NEG, dummy = 0.0;
    int gi = cand ? lane : 0x7fffffff;
    wave_argmax(v, gi, dummy);
    kept |= 1ull << gi;
  }
  uint32_t taken = 0;
  double my_s = 0.0;
  int my_e = 0;
  for (int j = 0; j < k; j++) {
    double v = NEG, sv = 0.0;
    int ei = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPL; i++) {
      const int e = lane * EPL + i;
      if (e < E && ((kept >> (e / m)) & 1ull) && !((taken >> i) & 1u) && (c[i] > v || (c[i] == v && e < ei))) {
        v = c[i];
        ei = e;
        sv = s[i];
      }
    }
    wave_argmax(v, ei, sv);
    if (ei / EPL == lane) taken |= 1u << (ei - lane * EPL);
    if (lane == j) {
      my_s = sv;
      my_e = ei;
    }
  }
  double S = 0.0;
  for (int j = 0; j < k; j++) S += __shfl(my_s, j);
  if (lane < k) {
    a.idx[(int64_t)t * k + lane] = my_e;
    a.w[(int64_t)t * k + lane] = (float)((my_s / S) * (double)a.rsf);
  }
}

// One wavefront per token, four tokens per workgroup.
template <int EPL>
__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  if (a.xq) q8_0_row_wave(a.x + (int64_t)t * a.H, a.H, a.xq + (int64_t)t * a.H, a.xds + (int64_t)t * (a.H / QK), lane);
  select_token<EPL>(a, t, lane);
}

// ------------------------------------------------------------------ host side
int32_t route_ksplit(const coli_moe_cfg &c, int32_t T) {
  if (T <= LD_TT && c.hidden % 256 == 0) return (c.hidden % 512 == 0) ? c.hidden / 512 : c.hidden / 256;
  const int nkb = c.hidden / 32;
  for (int d = 2; d >= 1; d--)
    if (nkb % d == 0) return d;
  return 1;
}

hipError_t launch_route(const RouteLaunch &r, hipStream_t s, hipEvent_t mid) {
  const coli_moe_cfg &c = *r.cfg;
  const int E = c.n_experts, H = c.hidden, T = r.T;
  const int ks = r.ksplit;
  if (T <= LD_TT && H % 256 == 0) {
    dim3 grid((E + 4 * LD_EPW - 1) / (4 * LD_EPW), ks);
    if (H / ks == 512)
      hipLaunchKernelGGL(logits_decode_kernel<2>, grid, dim3(256), 0, s, r.x, r.W, T, E, H, r.logits);
    else
      hipLaunchKernelGGL(logits_decode_kernel<1>, grid, dim3(256), 0, s, r.x, r.W, T, E, H, r.logits);
  } else if (T <= LD_TT) {
    dim3 grid((E + 15) / 16, 1, ks);
    hipLaunchKernelGGL((logits_kernel<16, 16, 1, 1>), grid, dim3(256), 0, s, r.x, r.W, T, E, H, H / ks, r.logits);
  } else {
    dim3 grid((E + 63) / 64, (T + 63) / 64, ks);
    hipLaunchKernelGGL((logits_kernel<64, 64, 4, 4>), grid, dim3(256), 0, s, r.x, r.W, T, E, H, H / ks, r.logits);
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
  a.bias = r.bias;
  a.idx = r.idx;
  a.w = r.w;
  a.x = r.x;
  a.H = H;
  a.xq = r.xq;
  a.xds = r.xds;
  const int epl = (E + 63) / 64;
#define COLI_SEL(EPLV) hipLaunchKernelGGL((select_kernel<EPLV>), dim3((T + 3) / 4), dim3(256), 0, s, a)
#define COLI_SEL_Q(EPLV) COLI_SEL(EPLV);
  if (epl <= 1) {
    COLI_SEL_Q(1)
  } else if (epl <= 2) {
    COLI_SEL_Q(2)
  } else if (epl <= 4) {
    COLI_SEL_Q(4)
  } else if (epl <= 8) {
    COLI_SEL_Q(8)
  } else {
    COLI_SEL_Q(16)
  }
#undef COLI_SEL_Q
#undef COLI_SEL
  return hipGetLastError();
}

}  // namespace coli
