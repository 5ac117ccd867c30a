// router.hip — sigmoid noaux_tc router on gfx950.
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
// Two kernels: a tiled fp64 logits kernel writing K-split partial sums, and a
// one-wavefront-per-token selection kernel that adds the partials in a fixed
// order (deterministic) and performs the group-limited top-k with shuffles.
#include "coli_internal.h"

namespace coli {

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
    // stage x[t0..t0+TT)[k0..k0+KB) and W[e0..e0+TE)[k0..k0+KB) as fp64
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

constexpr int TOPK_EPL = 16;  // experts per lane, E <= 1024

__global__ __launch_bounds__(256) void topk_kernel(const double *__restrict__ part, int ksplit, int T, int E,
                                                   int G, int Gk, int k, float rsf,
                                                   const float *__restrict__ bias, int32_t *__restrict__ idx,
                                                   float *__restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefront leaves together
  const int epl = (E + 63) / 64;
  const int m = E / G;
  const double NEG = -INFINITY;
  double s[TOPK_EPL], c[TOPK_EPL];
#pragma unroll
  for (int i = 0; i < TOPK_EPL; i++) {
    s[i] = 0.0;
    c[i] = NEG;
    const int e = lane * epl + i;
    if (i < epl && e < E) {
      double z = 0.0;
      for (int ks = 0; ks < ksplit; ks++) z += part[((int64_t)ks * T + t) * E + e];
      s[i] = 1.0 / (1.0 + exp(-z));
      c[i] = s[i] + (double)bias[e];
    }
  }
  // group scores; lane g keeps the score of group g
  double my_gs = NEG;
  for (int g = 0; g < G; g++) {
    const int lo = g * m, hi = lo + m;
    double v1 = NEG, dummy = 0.0;
    int i1 = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < TOPK_EPL; i++) {
      const int e = lane * epl + i;
      if (i < epl && e >= lo && e < hi && (c[i] > v1 || (c[i] == v1 && e < i1))) {
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
      for (int i = 0; i < TOPK_EPL; i++) {
        const int e = lane * epl + i;
        if (i < epl && e >= lo && e < hi && e != i1 && (c[i] > v2 || (c[i] == v2 && e < i2))) {
          v2 = c[i];
          i2 = e;
        }
      }
      wave_argmax(v2, i2, dummy);
      gs = v1 + v2;
    }
    if (lane == g) my_gs = gs;
  }
  // keep the Gk best groups
  uint64_t kept = 0;
  for (int r = 0; r < Gk; r++) {
    double v = (lane < G && !((kept >> lane) & 1ull)) ? my_gs : NEG;
    int gi = (lane < G && !((kept >> lane) & 1ull)) ? lane : 0x7fffffff;
    double dummy = 0.0;
    wave_argmax(v, gi, dummy);
    kept |= 1ull << gi;
  }
  // route the k best experts of the kept groups
  uint32_t taken = 0;
  double my_s = 0.0;
  int my_e = 0;
  for (int j = 0; j < k; j++) {
    double v = NEG, sv = 0.0;
    int ei = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < TOPK_EPL; i++) {
      const int e = lane * epl + i;
      if (i < epl && e < E && ((kept >> (e / m)) & 1ull) && !((taken >> i) & 1u) &&
          (c[i] > v || (c[i] == v && e < ei))) {
        v = c[i];
        ei = e;
        sv = s[i];
      }
    }
    wave_argmax(v, ei, sv);
    if (ei / epl == lane) taken |= 1u << (ei - lane * epl);
    if (lane == j) {
      my_s = sv;
      my_e = ei;
    }
  }
  double S = 0.0;
  for (int j = 0; j < k; j++) S += __shfl(my_s, j);
  if (lane < k) {
    idx[(int64_t)t * k + lane] = my_e;
    w[(int64_t)t * k + lane] = (float)((my_s / S) * (double)rsf);
  }
}

hipError_t launch_route(const coli_moe_cfg &c, const float *x, int32_t T, const float *W, const float *bias,
                        double *logits, int32_t ksplit, int32_t *idx, float *w, hipStream_t s, hipEvent_t mid) {
  const int E = c.n_experts, H = c.hidden;
  const int kc = H / ksplit;
  if (T <= 16) {
    dim3 grid((E + 15) / 16, 1, ksplit);
    hipLaunchKernelGGL((logits_kernel<16, 16, 1, 1>), grid, dim3(256), 0, s, x, W, T, E, H, kc, logits);
  } else {
    dim3 grid((E + 63) / 64, (T + 63) / 64, ksplit);
    hipLaunchKernelGGL((logits_kernel<64, 64, 4, 4>), grid, dim3(256), 0, s, x, W, T, E, H, kc, logits);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid) {
    err = hipEventRecord(mid, s);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, ksplit, T, E, c.n_group,
                     c.topk_group, c.top_k, c.routed_scaling_factor, bias, idx, w);
  return hipGetLastError();
}

int32_t route_ksplit(const coli_moe_cfg &c, int32_t T) {
  // K chunks of at least ROUTE_KC inputs for decode-sized T (more workgroups), two for larger T
  const int nkb = c.hidden / 32;
  int target = (T <= 16) ? c.hidden / ROUTE_KC : 2;
  if (target < 1) target = 1;
  for (int d = target; d >= 1; d--)
    if (nkb % d == 0) return d;
  return 1;
}

}  // namespace coli
