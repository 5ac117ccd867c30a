// q8_0.hip — standalone Q8_0 activation quantisation (rule in q8_0_impl.h).
//
// Eight lanes own one block (one float4 each): fully coalesced 16-byte loads and
// 4-byte stores.
#include "q8_0_impl.h"

namespace coli {

__global__ __launch_bounds__(256) void q8_0_kernel(const float *__restrict__ x, int64_t nblk,
                                                   int8_t *__restrict__ q, float *__restrict__ d) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = gid >> 3;
  const int sub = threadIdx.x & 7;
  const bool valid = blk < nblk;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (valid) v = *reinterpret_cast<const float4 *>(x + blk * QK + sub * 4);
  uint32_t packed;
  const float dd = q8_0_block8(v, packed);
  if (!valid) return;
  *reinterpret_cast<uint32_t *>(q + blk * QK + sub * 4) = packed;
  if (sub == 0) d[blk] = dd;
}

hipError_t launch_q8_0(const float *x, int64_t rows, int32_t cols, int8_t *q, float *d, hipStream_t s) {
  const int64_t nblk = rows * (int64_t)(cols / QK);
  if (nblk == 0) return hipSuccess;
  const int64_t grid = (nblk * 8 + 255) / 256;
  hipLaunchKernelGGL(q8_0_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, nblk, q, d);
  return hipGetLastError();
}

}  // namespace coli
