// ffn_gemv.hip — dispatch of the quantised expert GEMVs by weight format, and the
// deterministic weighted combine. The GEMV kernels are templates in ffn_gemv_impl.h,
// instantiated one weight format per source file (ffn_gemv_w4/w8/w2/mx.hip).
#include "coli_internal.h"

namespace coli {

static hipError_t launch_fmt(int mode, int wfmt, const FfnArgs &a, hipStream_t s) {
  // MXFP4 always has its E8M0 scale per 32 inputs; the integer formats one per row or per 64
  if (wfmt == W_MX) return a.gs == 32 ? launch_gemv_mx(mode, a, s) : hipErrorInvalidValue;
  if (a.gs != 0 && a.gs != 64) return hipErrorInvalidValue;
  const bool gs = a.gs != 0;
  switch (wfmt) {
    case 4: return launch_gemv_w4(mode, gs, a, s);
    case 8: return launch_gemv_w8(mode, gs, a, s);
    case 2: return launch_gemv_w2(mode, gs, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gateup(int wfmt, const FfnArgs &a, hipStream_t s) { return launch_fmt(0, wfmt, a, s); }

hipError_t launch_down(int wfmt, const FfnArgs &a, hipStream_t s) { return launch_fmt(1, wfmt, a, s); }

// out[t] = sum_j w[t][j] * ypair[t*k + j] (j ascending) + ypair[P + t] (shared).
// The slots are loaded eight at a time (independent loads in flight together) and
// added in ascending order, so the result does not depend on the batching. A slot
// of weight 0 is an empty slot (adaptive top-p: its pair row was never written) and
// is not added; a kept slot's weight is never 0 (sigmoid scores are positive).
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ ypair, const float *__restrict__ w,
                                                      int T, int k, int H, int has_shared,
                                                      float *__restrict__ out) {
  constexpr int JB = 8;
  const int t = blockIdx.y;
  const int c4 = blockIdx.x * 256 + threadIdx.x;  // float4 column
  if (c4 * 4 >= H) return;
  const int64_t stride = H / 4;
  const float4 *yp = reinterpret_cast<const float4 *>(ypair + (int64_t)t * k * H) + c4;
  const float *wt = w + (int64_t)t * k;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += JB) {
    float4 y[JB];
    float wj[JB];
#pragma unroll
    for (int j = 0; j < JB; j++) {  // clamped: slots past k repeat the last one and are not added
      const int jj = min(j0 + j, k - 1);
      y[j] = yp[jj * stride];
      wj[j] = wt[jj];
    }
#pragma unroll
    for (int j = 0; j < JB; j++) {
      if (j0 + j < k && wj[j] != 0.0f) {
        acc.x += wj[j] * y[j].x;
        acc.y += wj[j] * y[j].y;
        acc.z += wj[j] * y[j].z;
        acc.w += wj[j] * y[j].w;
      }
    }
  }
  if (has_shared) {
    const float4 y = reinterpret_cast<const float4 *>(ypair + ((int64_t)T * k + t) * H)[c4];
    acc.x += y.x;
    acc.y += y.y;
    acc.z += y.z;
    acc.w += y.w;
  }
  reinterpret_cast<float4 *>(out + (int64_t)t * H)[c4] = acc;
}

hipError_t launch_combine(const float *ypair, const float *w, int32_t T, int32_t k, int32_t H, int32_t has_shared,
                          float *out, hipStream_t s) {
  dim3 grid((H / 4 + 255) / 256, T);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, ypair, w, T, k, H, has_shared, out);
  return hipGetLastError();
}

}  // namespace coli
