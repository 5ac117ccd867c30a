// gen_device.hip — device-side twin of synth.expert_blob(): fills packed expert
// blobs with the SplitMix64 stream of each expert's key. Integer arithmetic only,
// so the bytes equal the host generator's bit for bit. Not part of the MoE
// library: it produces synthetic inputs, plus the reference kernels that the
// benchmark times beside the library's (a copy and a streaming read of known
// traffic, and an exactly scaled int8 matrix-core loop).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// byte b -> ((b * 255) >> 8) - 127 in each of the 8 bytes of v
__device__ __forceinline__ uint64_t to_int8_weights(uint64_t v) {
  uint64_t r = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t b = (uint32_t)(v >> (8 * i)) & 0xFFu;
    const int32_t q = (int32_t)((b * 255u) >> 8) - 127;
    r |= (uint64_t)(uint8_t)(int8_t)q << (8 * i);
  }
  return r;
}

__global__ void fill_blobs_kernel(uint64_t *__restrict__ out, const uint64_t *__restrict__ keys, int64_t words_per_blob,
                                  int32_t n_blobs, int32_t int8_map) {
  const int64_t total = words_per_blob * n_blobs;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = g / words_per_blob, i = g % words_per_blob;
    uint64_t v = mix64(keys[e] + (uint64_t)(i + 1) * kGolden);
    if (int8_map) v = to_int8_weights(v);
    out[g] = v;
  }
}

// Plain streaming copy of n16 16-byte words: a kernel whose HBM traffic is known
// exactly (n16 * 16 bytes read, the same written), run beside the MoE kernels so
// that hardware byte counters can be scaled to bytes.
__global__ void copy_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst, int64_t n16) {
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n16; g += (int64_t)gridDim.x * blockDim.x)
    dst[g] = src[g];
}

// Streaming read of n16 16-byte words: the measured read-bandwidth ceiling beside the
// HBM specification. Each workgroup reads contiguous chunks of 8 x 256 words (eight
// 16-byte loads in flight per thread, nontemporal: the data is used once), and each
// wavefront folds what it read into one word of `sink` ([gridDim.x * 4]) so that the
// loads are not elided. Words past the last whole chunk are read by a tail loop.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_kernel(const uint4 *__restrict__ src, int64_t n16,
                                                   uint32_t *__restrict__ sink) {
  constexpr int U = 8;
  const u32x4 *s = reinterpret_cast<const u32x4 *>(src);
  const int64_t chunk = (int64_t)U * 256;
  uint32_t acc = 0;
  int64_t base = (int64_t)blockIdx.x * chunk;
  for (; base + chunk <= n16; base += (int64_t)gridDim.x * chunk) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; u++) v[u] = __builtin_nontemporal_load(s + base + u * 256 + threadIdx.x);
#pragma unroll
    for (int u = 0; u < U; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // the tail (fewer than gridDim.x * chunk words are left at most; base >= the tail start)
  for (int64_t g = (n16 / chunk) * chunk + (int64_t)blockIdx.x * 256 + threadIdx.x; g < n16;
       g += (int64_t)gridDim.x * 256) {
    const u32x4 v = s[g];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

// Throughput of int8 matrix-core work that scales every block dot exactly: a loop of
// v_mfma_i32_32x32x32_i8 (32 rows x 32 columns x one 32-value block) whose 16 int32
// results per lane are each converted to fp32 and multiply-added into an fp32
// accumulator with a per-lane factor, with no memory traffic in the loop. That is the
// arithmetic a grouped GEMM over Q8_0 blocks performs per block when it keeps each
// block dot exact and applies the block's scale to it, so the measured rate is that
// GEMM's ceiling on the device, beside the 5.0 POP/s int8 specification (which
// counts the matrix cores alone). Two independent chains per wavefront; the operands
// change every iteration, so nothing is loop-invariant.
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef int v16i_t __attribute__((ext_vector_type(16)));

constexpr int kMfGrid = 2048;  // 8 workgroups of 4 wavefronts per CU on 256 CUs

__global__ __launch_bounds__(256) void scaled_mfma_kernel(float *__restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  v4i_t a = {lane, 3 * lane + 1, 5, 7}, b = {11 - lane, 13, 2 * lane + 17, 19};
  const float d0 = 1.0e-3f * (float)(lane + 1), d1 = 2.0e-3f * (float)(lane + 2);
  float acc0[16], acc1[16];
#pragma unroll
  for (int r = 0; r < 16; r++) {
    acc0[r] = 0.0f;
    acc1[r] = 0.0f;
  }
  for (int i = 0; i < iters; i++) {
    const v16i_t z = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const v16i_t I0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, z, 0, 0, 0);
    const v16i_t I1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, z, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; r++) {
      acc0[r] = fmaf(d0, (float)I0[r], acc0[r]);
      acc1[r] = fmaf(d1, (float)I1[r], acc1[r]);
    }
    a.x += 1;
    b.z += 1;
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r++) s += acc0[r] + acc1[r];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

constexpr int kReadGrid = 4096;

extern "C" int coli_synth_read_sink_words(void) { return kReadGrid * 4; }

extern "C" int coli_synth_read(const void *src, int64_t bytes, void *sink, void *stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16) return -1;
  if (((uintptr_t)src % 16) != 0 || ((uintptr_t)sink % 4) != 0) return -4;
  hipLaunchKernelGGL(read_kernel, dim3(kReadGrid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4 *>(src), bytes / 16, static_cast<uint32_t *>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int coli_synth_copy(const void *src, void *dst, int64_t bytes, void *stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16) return -1;
  if (((uintptr_t)src % 16) != 0 || ((uintptr_t)dst % 16) != 0) return -4;
  hipLaunchKernelGGL(copy_kernel, dim3(2048), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int coli_synth_fill_blobs(void *out, const void *keys_dev, int64_t blob_bytes, int32_t n_blobs,
                                     int32_t wbits, void *stream) {
  if (!out || !keys_dev || blob_bytes <= 0 || blob_bytes % 8 || n_blobs <= 0) return -1;
  if (((uintptr_t)out % 8) != 0) return -4;
  const int64_t words = blob_bytes / 8;
  hipLaunchKernelGGL(fill_blobs_kernel, dim3(4096), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint64_t *>(out), static_cast<const uint64_t *>(keys_dev), words, n_blobs,
                     wbits == 8 ? 1 : 0);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int coli_synth_scaled_mfma_out_words(void) { return kMfGrid * 256; }

// int8 operations (2 per multiply-add) of one coli_synth_scaled_mfma launch
extern "C" double coli_synth_scaled_mfma_ops(int32_t iters) {
  return 2.0 * 32 * 32 * 32 * 2 /* MFMAs per iteration */ * (double)iters * 4 /* wavefronts */ * kMfGrid;
}

extern "C" int coli_synth_scaled_mfma(void *out, int32_t iters, void *stream) {
  if (!out || iters <= 0) return -1;
  if (((uintptr_t)out % 4) != 0) return -4;
  hipLaunchKernelGGL(scaled_mfma_kernel, dim3(kMfGrid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<float *>(out), iters);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
