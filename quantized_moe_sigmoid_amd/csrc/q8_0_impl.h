// q8_0_impl.h — the Q8_0 rule as device code, shared by the quantisation kernels.
//
// Per 32-value block (colibri-strix README, "What's implemented", integer-dot
// kernels item; the workload fixes 32-value blocks and scale = max|x| / 127):
// d = max|x| / 127 as one correctly rounded fp32 division (the library is built
// with correctly rounded fp32 division), q = round-half-away(x / d) clamped to
// [-127, 127], q = 0 when d = 0.
#pragma once

#include "coli_internal.h"

namespace coli {

__device__ __forceinline__ int q8_code(float v, float d) {
  if (d == 0.0f) return 0;
  float r = roundf(v / d);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

// One block per 8 consecutive lanes, 4 values per lane (v). Returns d; writes the
// lane's 4 codes (packed).
__device__ __forceinline__ float q8_0_block8(const float4 v, uint32_t &packed) {
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  a = fmaxf(a, __shfl_xor(a, 1, 8));
  a = fmaxf(a, __shfl_xor(a, 2, 8));
  a = fmaxf(a, __shfl_xor(a, 4, 8));
  const float d = a / 127.0f;
  const int c0 = q8_code(v.x, d), c1 = q8_code(v.y, d), c2 = q8_code(v.z, d), c3 = q8_code(v.w, d);
  packed = (uint32_t)(c0 & 0xFF) | ((uint32_t)(c1 & 0xFF) << 8) | ((uint32_t)(c2 & 0xFF) << 16) |
           ((uint32_t)(c3 & 0xFF) << 24);
  return d;
}

// A whole wavefront quantises one row of n values (n % 32 == 0): q [n], d [n/32].
__device__ __forceinline__ void q8_0_row_wave(const float *__restrict__ x, int n, int8_t *__restrict__ q,
                                              float *__restrict__ dout, int lane) {
  const int nblk = n / QK;
  const int sub = lane & 7;
#pragma unroll 4
  for (int b0 = 0; b0 < nblk; b0 += 8) {
    const int blk = b0 + (lane >> 3);
    const bool valid = blk < nblk;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) v = reinterpret_cast<const float4 *>(x)[blk * 8 + sub];
    uint32_t packed;
    const float d = q8_0_block8(v, packed);
    if (valid) {
      reinterpret_cast<uint32_t *>(q)[blk * 8 + sub] = packed;
      if (sub == 0) dout[blk] = d;
    }
  }
}

}  // namespace coli
