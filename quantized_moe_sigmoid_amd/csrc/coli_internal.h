// coli_internal.h — shared declarations of the HIP side of libcolimoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/coli_moe.h"

namespace coli {

constexpr int QK = 32;              // Q8_0 block length
constexpr int WAVE = 64;            // CDNA wavefront
constexpr int GEMV_ROWS = 32;       // rows per workgroup tile of the GEMV kernels (= one Q8_0 block of h)
constexpr int GEMV_NT = 8;          // tokens handled per pass of the GEMV kernels
constexpr int ROUTE_KC = 256;       // K chunk of the router logits kernel (decode tiling)

constexpr int W_MX = COLI_W_MXFP4;  // MXFP4 weights: 4-bit E2M1 codes, one E8M0 byte per 32 inputs

// Packed bytes of one row of n inputs.
__host__ __device__ inline int64_t row_bytes(int wfmt, int n) {
  return wfmt == W_MX ? (int64_t)n / 2 : (int64_t)n * wfmt / 8;
}

// Group scales (one per GSZ<WB> inputs of a row): fp32, or E8M0 bytes for MXFP4.
// gs_base gives element `elem` of the layer's scale array; gs_load reads element i
// from there as fp32. E8M0 byte u is 2^(u - 127), u = 255 is NaN (OCP MX v1.0).
template <int WB>
constexpr int GSZ = (WB == W_MX) ? 32 : 64;

template <int WB>
__device__ __forceinline__ const void *gs_base(const float *scales, int64_t elem) {
  if constexpr (WB == W_MX) return reinterpret_cast<const uint8_t *>(scales) + elem;
  else return scales + elem;
}

__device__ __forceinline__ float e8m0_f32(uint32_t u) {
  return __uint_as_float(u == 0 ? 0x00400000u : (u == 255 ? 0x7fc00000u : u << 23));
}

template <int WB>
__device__ __forceinline__ float gs_load(const void *base, int64_t i) {
  if constexpr (WB == W_MX) return e8m0_f32(static_cast<const uint8_t *>(base)[i]);
  else return static_cast<const float *>(base)[i];
}

// Four E2M1 codes, one in the low nibble of each byte of n (high nibbles ignored),
// to four int8 bytes holding twice their values (integers in [-12, 12], so block dots
// stay exact int32). Byte permutes do the lookups: one returns 2|v| for the magnitude
// bits, one -2|v|, and a third builds the per-byte select mask from the sign bit
// (permute selectors 5 and 7 read a zero source byte, 13 and 15 give 0xFF).
__device__ __forceinline__ uint32_t e2m1x4_to_i8x4(uint32_t n) {
  const uint32_t mag = n & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, mag);  // 0 1 2 3 | 4 6 8 12
  const uint32_t neg = __builtin_amdgcn_perm(0xF4F8FAFCu, 0xFDFEFF00u, mag);  // negated
  const uint32_t msk = __builtin_amdgcn_perm(0u, 0u, (n & 0x08080808u) | 0x05050505u);
  return (neg & msk) | (pos & ~msk);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// 32 Q8_0 codes of a block (x[i] = codes 4 i .. 4 i + 3) -> 16 fp16 pairs (q_j, q_j+16):
// a byte permute places q_j and q_j+16 over zero bytes, an XOR turns each half into
// 0x64 : (q + 128), the fp16 number 1024 + q + 128, and one packed fp16 subtraction of
// 1152 leaves q exactly.
__device__ __forceinline__ void q8_to_f16_pairs(const int (&x)[8], uint32_t (&h)[16]) {
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const uint32_t sel = (uint32_t)b | 0x0C00u | ((uint32_t)(4 + b) << 16) | 0x0C000000u;
      const uint32_t t = __builtin_amdgcn_perm((uint32_t)x[4 + i], (uint32_t)x[i], sel) ^ 0x64806480u;
      h[4 * i + b] = as_u32(as_f16x2(t) - f16x2{(_Float16)1152.0f, (_Float16)1152.0f});
    }
}

struct WsLayout {
  // byte offsets into the workspace (all 256-byte aligned)
  size_t xq, xd, hq, hd, ypair, logits, idx, w, cnt, off, perm, active, nact, tiles, ntiles, redo, total;
};

// Workspace layout for T tokens (valid cfg assumed).
WsLayout ws_layout(const coli_moe_cfg &c, int32_t T, int32_t ksplit);

// number of K splits of the router logits for T tokens
int32_t route_ksplit(const coli_moe_cfg &c, int32_t T);

struct GroupOut {
  int32_t *cnt, *off, *perm, *active, *nact;
};

constexpr int LOCAL_GROUP_MAX_P = 512;  // pairs a GEMV workgroup groups by itself (decode-sized batches)

// ---- launchers (host side, one per kernel family); return hipError_t
hipError_t launch_q8_0(const float *x, int64_t rows, int32_t cols, int8_t *q, float *d, hipStream_t s);

// The router's selection step: partials in, route out (router.hip select kernels;
// with part set in FfnArgs::sel, the decode gate/up GEMVs select the route themselves)
struct SelectArgs {
  const double *part;  // K-split logit partials [ksplit][T][E]
  int ksplit, T, E, G, Gk, k;
  float rsf;
  float topp;  // 0: plain top-k; else adaptive expert top-p
  const float *bias;
  int32_t *idx;    // [T][k] out
  float *w;        // [T][k] out
  const float *x;  // quantised into xq/xd when xq != nullptr (select_kernel only)
  int H;
  int8_t *xq;
  float *xd;
  // the selection's shape, worked out on the host (sel_plan): m = E / G experts per
  // group (gshift = log2 m when m is a power of two, else -1); P threads per expert
  // splitting its group's m entries into n1 each; kk = min(k, m) candidates per kept
  // group, nc = Gk * kk in all; P2 threads per candidate, n2 candidates each
  int m, gshift, P, n1, kk, nc, P2, n2;
};

struct RouteLaunch {
  const coli_moe_cfg *cfg;
  const float *x;
  int32_t T;
  const float *W, *bias;
  double *logits;
  int32_t ksplit;
  int32_t *idx;
  float *w;
  int8_t *xq;        // quantise x into xq/xd in the selection kernel when non-null
  float *xd;
};
// Logits, then the selection; with `fused` set and route_fusable, the selection is
// left to the gate/up GEMV: *fused receives its arguments (else part = nullptr).
hipError_t launch_route(const RouteLaunch &r, hipStream_t s, hipEvent_t mid, SelectArgs *fused = nullptr);
bool route_fusable(const coli_moe_cfg &c, int32_t T, int32_t ks);
hipError_t launch_group(const coli_moe_cfg &c, const int32_t *idx, int32_t T, int32_t *cnt, int32_t *off,
                        int32_t *perm, int32_t *active, int32_t *nact, hipStream_t s);
bool group_supported(int P, int E);

struct FfnArgs {
  const uint8_t *experts;
  const float *scales;
  int64_t blob_bytes;
  int64_t scale_stride;  // fp32 scales per expert
  int32_t gs;            // 0: one scale per row; 64: one per 64 inputs of a row
  int32_t H, F, E, k, T, has_shared;
  const int32_t *off, *perm, *active, *nact;  // grouping arrays (read when idx == nullptr)
  const int32_t *idx;  // route [T][k]: each workgroup groups locally when set (T*k <= LOCAL_GROUP_MAX_P)
  const int8_t *xq;   // [T][H]
  const float *xd;    // [T][H/32] Q8_0 block scales
  int8_t *hq;         // [P+T][F]
  float *hd;          // [P+T][F/32]
  float *ypair;       // [P+T][H]
  float *tap;         // test builds (COLI_TAPS) only: [P+T][2F] pre-SiLU g | u per output row
  int32_t *redo;      // MXFP4 grouped GEMM: per work item, 1 = its scales need the integer path
  // gate/up GEMVs only: with sel.part set, every workgroup selects the route from the
  // logit partials itself (idx is then sel.idx, written by one workgroup)
  SelectArgs sel;
};

// Test builds (compiled with COLI_TAPS) record the gate and up values of every output
// row before SiLU (row scale applied, fp32, exactly as the epilogue uses them). Product
// builds compile this to nothing.
#ifdef COLI_TAPS
#define COLI_TAP_GU(a, row, f, gv, uv)                                    \
  do {                                                                   \
    if ((a).tap) {                                                       \
      (a).tap[(int64_t)(row) * 2 * (a).F + (f)] = (gv);                  \
      (a).tap[(int64_t)(row) * 2 * (a).F + (a).F + (f)] = (uv);          \
    }                                                                    \
  } while (0)
#else
#define COLI_TAP_GU(a, row, f, gv, uv) \
  do {                                 \
  } while (0)
#endif
hipError_t launch_gateup(int wfmt, const FfnArgs &a, hipStream_t s);
hipError_t launch_down(int wfmt, const FfnArgs &a, hipStream_t s);
// per-format GEMV launchers (ffn_gemv_w4/w8/w2/mx.hip); mode 0 = gate/up, 1 = down;
// gs: group-scale path (MXFP4 always takes it)
hipError_t launch_gemv_w4(int mode, bool gs, const FfnArgs &a, hipStream_t s);
hipError_t launch_gemv_w8(int mode, bool gs, const FfnArgs &a, hipStream_t s);
hipError_t launch_gemv_w2(int mode, bool gs, const FfnArgs &a, hipStream_t s);
hipError_t launch_gemv_mx(int mode, const FfnArgs &a, hipStream_t s);
// grouped-GEMM (MFMA) path for batches whose experts see many tokens
int32_t mfma_gmax(int32_t T, int32_t k, int32_t E, int32_t has_shared);  // token-tile capacity
int64_t mfma_redo_words(const coli_moe_cfg &c, int32_t T);  // redo flags of an MXFP4 batch (0 otherwise)
hipError_t launch_plan(const FfnArgs &a, int4 *tiles, int32_t *ntiles, int32_t gmax, hipStream_t s);
hipError_t launch_mfma_gateup(int wfmt, const FfnArgs &a, const int4 *tiles, const int32_t *ntiles, int32_t gmax,
                              hipStream_t s);
hipError_t launch_mfma_down(int wfmt, const FfnArgs &a, const int4 *tiles, const int32_t *ntiles, int32_t gmax,
                            hipStream_t s);
// One phase of coli_moe_ffn for the expert tier (validation as coli_moe_ffn): the Q8_0
// of x only with quantize_x, the shared expert only with shared, the combine only with
// combine; the workspace layout is that of cfg. Decode-sized batches group inside the
// GEMV workgroups from topk_idx (the grouping arrays may then be null).
int ffn_phase(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T, const int32_t *topk_idx,
              const float *topk_w, const int32_t *expert_off, const int32_t *pair_perm, const int32_t *active,
              const int32_t *n_active, float *out, void *workspace, size_t ws_bytes, hipStream_t s, bool quantize_x,
              bool shared, bool combine);
// The combine of ffn_phase alone (the pair rows of earlier phases, workspace layout of cfg).
int combine_phase(const coli_moe_cfg *cfg, int32_t T, const float *topk_w, float *out, void *workspace,
                  size_t ws_bytes, hipStream_t s);
// coli_moe_route that also quantises x (Q8_0) into xq [T][H] / xd [T][H/32].
int route_phase(const coli_moe_cfg *cfg, const coli_moe_weights *w, const float *x, int32_t T, int32_t *topk_idx,
                float *topk_w, void *workspace, size_t ws_bytes, int8_t *xq, float *xd, hipStream_t s);
// Where a workspace for T tokens holds the Q8_0 of x (the same for every cfg of hidden H).
int8_t *ws_xq(const coli_moe_cfg &c, int32_t T, void *ws);
float *ws_xd(const coli_moe_cfg &c, int32_t T, void *ws);

hipError_t launch_combine(const float *ypair, const float *w, int32_t T, int32_t k, int32_t H,
                          int32_t has_shared, float *out, hipStream_t s);

}  // namespace coli
