// q8_0.hip — Q8_0 activation quantisation on gfx950.
//
// Per 32-value block (colibri-strix README, "What's implemented", integer-dot
// kernels item; the workload fixes 32-value blocks and scale = max|x| / 127):
// d = max|x| / 127 as one correctly rounded fp32 division, q = round-half-away
// (x / d) clamped to [-127, 127], q = 0 when d = 0.
//
// Eight lanes own one block (one float4 each), so a wavefront covers 8 blocks
// with fully coalesced 16-byte loads and 4-byte stores. Besides q and d the
// kernel can emit {d, sum q} pairs, which the expert GEMV kernels use for the
// offset-binary weight trick (sum_i x_i w_i = sum_i x_i (w_i + 8) - 8 sum_i x_i).
#include "coli_internal.h"

namespace coli {

__device__ __forceinline__ int q8_code(float v, float d) {
  if (d == 0.0f) return 0;
  float r = roundf(v / d);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

__global__ __launch_bounds__(256) void q8_0_kernel(const float *__restrict__ x, int64_t nblk,
                                                   int8_t *__restrict__ q, float *__restrict__ d,
                                                   int2 *__restrict__ ds) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = gid >> 3;
  const int sub = threadIdx.x & 7;
  const bool valid = blk < nblk;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (valid) v = *reinterpret_cast<const float4 *>(x + blk * QK + sub * 4);
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  a = fmaxf(a, __shfl_xor(a, 1, 8));
  a = fmaxf(a, __shfl_xor(a, 2, 8));
  a = fmaxf(a, __shfl_xor(a, 4, 8));
  const float dd = a / 127.0f;
  const int c0 = q8_code(v.x, dd), c1 = q8_code(v.y, dd), c2 = q8_code(v.z, dd), c3 = q8_code(v.w, dd);
  int sum = c0 + c1 + c2 + c3;
  sum += __shfl_xor(sum, 1, 8);
  sum += __shfl_xor(sum, 2, 8);
  sum += __shfl_xor(sum, 4, 8);
  if (!valid) return;
  const uint32_t packed = (uint32_t)(c0 & 0xFF) | ((uint32_t)(c1 & 0xFF) << 8) | ((uint32_t)(c2 & 0xFF) << 16) |
                          ((uint32_t)(c3 & 0xFF) << 24);
  *reinterpret_cast<uint32_t *>(q + blk * QK + sub * 4) = packed;
  if (sub == 0) {
    if (d) d[blk] = dd;
    if (ds) ds[blk] = make_int2(__float_as_int(dd), sum);
  }
}

hipError_t launch_q8_0(const float *x, int64_t rows, int32_t cols, int8_t *q, float *d, int2 *ds,
                       hipStream_t s) {
  const int64_t nblk = rows * (int64_t)(cols / QK);
  if (nblk == 0) return hipSuccess;
  const int64_t grid = (nblk * 8 + 255) / 256;
  hipLaunchKernelGGL(q8_0_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, nblk, q, d, ds);
  return hipGetLastError();
}

}  // namespace coli
