// ffn_gemv_impl.h — quantised expert GEMV kernels over the batch union (gfx950),
// as templates over the weight format; each ffn_gemv_w*.hip instantiates one format.
//
//
// One expert of the union is one grid row (blockIdx.y = slot); a workgroup owns
// 32 consecutive output rows of that expert and streams their packed weights
// exactly once, applying them to every token routed to the expert (batch-union:
// colibri-strix README, "What's implemented", batch-union item). Weights stay
// packed in HBM and are dequantised on use (same section, quantization kernels
// item); the products are integer dots against Q8_0 activations (integer-dot
// kernels item):
//   I_b = sum over block b of xq * wq         (v_dot4_i32_i8, exact int32)
//   acc = sum_b d_b * I_b                     (fp32)
//   out = s_row * acc
// Packed int4 / int2 fields are two's complement. A shift and a mask move each
// field into the top bits of its own byte, where the byte reads as S * w (S = 16
// for int4, 64 for int2) with no sign fix-up, so the signed dot4 gives S * I_b
// exactly (|S * I_b| < 2^24, so its fp32 conversion is exact too). Every fp32
// step below then carries the factor S, a power of two that commutes with
// rounding, and the row scale absorbs it: (s_row / S) * (S * acc) is the same
// fp32 number as s_row * acc.
//
// Lane mapping: the 16-byte "chunk" of a packed row is one Q8_0 block for int4,
// half of one for int8 (the two halves go to one lane as a 32-byte chunk) and
// two blocks for int2. LPR lanes share one row (each loads every LPR-th chunk),
// so one load instruction of a wavefront covers 64 consecutive chunks of one
// row (LPR = 64) or of 64/LPR rows: fully coalesced 128-bit weight loads.
// Activations of up to GEMV_NT tokens are staged in LDS once per workgroup.
//
// Gate/up epilogue (fused): h = silu(g) * u in fp32, then Q8_0 of the 32 rows of
// the tile (one block of h per token): hq int8 and hd fp32.
// Down epilogue: y fp32 rows, written per token as 32 consecutive floats.
#pragma once

#include <algorithm>
#include <type_traits>

#include "coli_internal.h"
#include "select_impl.h"

namespace coli {

template <int WB>
struct Fmt;
template <>
struct Fmt<4> {
  static constexpr int CHUNK = 16;         // bytes per lane chunk
  static constexpr int BPC = 1;            // Q8_0 blocks per chunk
  static constexpr float INV = 0.0625f;    // 1 / S: the top-bit bytes read 16 * w
};
template <>
struct Fmt<8> {
  static constexpr int CHUNK = 32;
  static constexpr int BPC = 1;
  static constexpr float INV = 1.0f;
};
template <>
struct Fmt<2> {
  static constexpr int CHUNK = 16;
  static constexpr int BPC = 2;
  static constexpr float INV = 0.015625f;  // the top-bit bytes read 64 * w
};
template <>
struct Fmt<W_MX> {
  static constexpr int CHUNK = 16;         // one block of 32 E2M1 codes, int4 nibble order
  static constexpr int BPC = 1;
  static constexpr float INV = 0.5f;       // the table bytes read 2 * e2m1
};


__device__ __forceinline__ int dot4(int a, int b, int c) { return __builtin_amdgcn_sdot4(a, b, c, false); }

// Integer dot of one weight chunk with the activation block(s) it covers, times
// the activation block scale(s); returns the fp32 contribution.
template <int WB>
__device__ __forceinline__ float chunk_dot(const uint32_t (&wq)[Fmt<WB>::CHUNK / 4], const int8_t *xa,
                                           const float *xd);

template <>
__device__ __forceinline__ float chunk_dot<4>(const uint32_t (&wq)[4], const int8_t *xa, const float *xd) {
  const int4 xl = *reinterpret_cast<const int4 *>(xa);
  const int4 xh = *reinterpret_cast<const int4 *>(xa + 16);
  const int xv[8] = {xl.x, xl.y, xl.z, xl.w, xh.x, xh.y, xh.z, xh.w};
  int acc = 0;  // 16 * I_b
#pragma unroll
  for (int i = 0; i < 4; i++) {
    acc = dot4((int)((wq[i] << 4) & 0xF0F0F0F0u), xv[i], acc);
    acc = dot4((int)(wq[i] & 0xF0F0F0F0u), xv[4 + i], acc);
  }
  return xd[0] * (float)acc;
}

template <>
__device__ __forceinline__ float chunk_dot<W_MX>(const uint32_t (&wq)[4], const int8_t *xa, const float *xd) {
  const int4 xl = *reinterpret_cast<const int4 *>(xa);
  const int4 xh = *reinterpret_cast<const int4 *>(xa + 16);
  const int xv[8] = {xl.x, xl.y, xl.z, xl.w, xh.x, xh.y, xh.z, xh.w};
  int acc = 0;  // 2 * J_b
#pragma unroll
  for (int i = 0; i < 4; i++) {
    acc = dot4((int)e2m1x4_to_i8x4(wq[i]), xv[i], acc);
    acc = dot4((int)e2m1x4_to_i8x4(wq[i] >> 4), xv[4 + i], acc);
  }
  return xd[0] * (float)acc;
}

template <>
__device__ __forceinline__ float chunk_dot<8>(const uint32_t (&wq)[8], const int8_t *xa, const float *xd) {
  const int4 xl = *reinterpret_cast<const int4 *>(xa);
  const int4 xh = *reinterpret_cast<const int4 *>(xa + 16);
  const int xv[8] = {xl.x, xl.y, xl.z, xl.w, xh.x, xh.y, xh.z, xh.w};
  int acc = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) acc = dot4((int)wq[i], xv[i], acc);
  return xd[0] * (float)acc;
}

template <>
__device__ __forceinline__ float chunk_dot<2>(const uint32_t (&wq)[4], const int8_t *xa, const float *xd) {
  float r = 0.0f;
#pragma unroll
  for (int blk = 0; blk < 2; blk++) {
    const int4 xl = *reinterpret_cast<const int4 *>(xa + 32 * blk);
    const int4 xh = *reinterpret_cast<const int4 *>(xa + 32 * blk + 16);
    const int xv[8] = {xl.x, xl.y, xl.z, xl.w, xh.x, xh.y, xh.z, xh.w};
    int acc = 0;  // 64 * I_b
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const uint32_t t = wq[2 * blk + h];
#pragma unroll
      for (int m = 0; m < 4; m++) acc = dot4((int)((t << (6 - 2 * m)) & 0xC0C0C0C0u), xv[2 * m + h], acc);
    }
    r += xd[blk] * (float)acc;
  }
  return r;
}

// Weight chunks are loaded with the nontemporal hint: each expert row is streamed once
// per launch, and nontemporal loads stream from HBM faster than cached ones (a plain
// read of 4 GiB: 7.0 TB/s against 6.3 TB/s; the GLM-scale gate/up GEMV at T = 16: 6.25
// against 5.85 TB/s).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// KEEP: an ordinary (L2-allocating) load, for rows that are read again by later token
// passes of the same workgroup.
template <int WB, bool KEEP = false>
__device__ __forceinline__ void load_chunk(const uint8_t *p, uint32_t (&wq)[Fmt<WB>::CHUNK / 4]) {
  const u32x4 a = KEEP ? *reinterpret_cast<const u32x4 *>(p) : __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  wq[0] = a.x;
  wq[1] = a.y;
  wq[2] = a.z;
  wq[3] = a.w;
  if constexpr (Fmt<WB>::CHUNK == 32) {
    const u32x4 b = KEEP ? *reinterpret_cast<const u32x4 *>(p + 16)
                         : __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + 16));
    wq[4] = b.x;
    wq[5] = b.y;
    wq[6] = b.z;
    wq[7] = b.w;
  }
}

// Split form of chunk_dot for the batched kernels: the unpacked weight bytes of a
// chunk (top-bit S * w, or raw int8) and the activation registers of one token are
// kept separately so that one unpack serves every token.
template <int WB>
struct Unp {
  // dwords of unpacked weights per chunk (MXFP4: 16 dwords of fp16 pairs)
  static constexpr int N = (WB == 2 || WB == W_MX) ? 16 : 8;
};

// MXFP4 in the batched and pipelined GEMVs: the E2M1 codes are converted to fp16 by
// the hardware (v_cvt_scalef32_pk_f16_fp4, scale 1: byte b of a dword gives the pair
// (low nibble, high nibble) = (K_j, K_j+16), j = 4 i + b in dword i of the chunk), the
// Q8_0 codes to fp16 pairs (q_j, q_j+16) once per token and chunk, and v_dot2_f32_f16
// sums the products. Every E2M1 value (0 .. 6 in halves) and every code (|q| <= 127) is
// exact in fp16, each product is exact in fp32 and every partial sum of a block is a
// multiple of 1/2 below 2^15, so the fp32 sum is the block's exact J_b = sum e2m1 * q,
// the same number as the integer path's 2 * J_b / 2.
template <int WB>
__device__ __forceinline__ void unpack_chunk(const uint32_t (&wq)[Fmt<WB>::CHUNK / 4], int (&u)[Unp<WB>::N]) {
  if constexpr (WB == 4) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      u[i] = (int)((wq[i] << 4) & 0xF0F0F0F0u);
      u[4 + i] = (int)(wq[i] & 0xF0F0F0F0u);
    }
  } else if constexpr (WB == 8) {
#pragma unroll
    for (int i = 0; i < 8; i++) u[i] = (int)wq[i];
  } else if constexpr (WB == W_MX) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      u[4 * i] = (int)as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wq[i], 1.0f, 0));
      u[4 * i + 1] = (int)as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wq[i], 1.0f, 1));
      u[4 * i + 2] = (int)as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wq[i], 1.0f, 2));
      u[4 * i + 3] = (int)as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wq[i], 1.0f, 3));
    }
  } else {
    // block blk, element dword d (elements 4d..4d+3) = field m of source dword h, d = 2m + h
#pragma unroll
    for (int blk = 0; blk < 2; blk++)
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const uint32_t t = wq[2 * blk + h];
#pragma unroll
        for (int m = 0; m < 4; m++) u[8 * blk + 2 * m + h] = (int)((t << (6 - 2 * m)) & 0xC0C0C0C0u);
      }
  }
}

// activation registers of one chunk for one token: Q8_0 bytes (MXFP4: fp16 pairs) and
// d per block
template <int WB>
struct Act {
  int x[Unp<WB>::N];
  float d[Fmt<WB>::BPC];
};

template <int WB>
__device__ __forceinline__ void load_act(const int8_t *xa, const float *xd, Act<WB> &a) {
  if constexpr (WB == W_MX) {
    int q[8];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int4 v = *reinterpret_cast<const int4 *>(xa + 16 * i);
      q[4 * i] = v.x;
      q[4 * i + 1] = v.y;
      q[4 * i + 2] = v.z;
      q[4 * i + 3] = v.w;
    }
    uint32_t h[16];
    q8_to_f16_pairs(q, h);
#pragma unroll
    for (int j = 0; j < 16; j++) a.x[j] = (int)h[j];
  } else {
#pragma unroll
    for (int i = 0; i < Unp<WB>::N / 4; i++) {
      const int4 v = *reinterpret_cast<const int4 *>(xa + 16 * i);
      a.x[4 * i] = v.x;
      a.x[4 * i + 1] = v.y;
      a.x[4 * i + 2] = v.z;
      a.x[4 * i + 3] = v.w;
    }
  }
#pragma unroll
  for (int b = 0; b < Fmt<WB>::BPC; b++) a.d[b] = xd[b];
}

template <int WB>
__device__ __forceinline__ float dot_unpacked(const int (&u)[Unp<WB>::N], const Act<WB> &a) {
  if constexpr (WB == W_MX) {
    float j = 0.0f;  // J_b, exact
#pragma unroll
    for (int i = 0; i < 16; i++) j = __builtin_amdgcn_fdot2(as_f16x2((uint32_t)u[i]), as_f16x2((uint32_t)a.x[i]), j, false);
    return a.d[0] * (2.0f * j);  // 2 J_b, as the integer path (INV = 1/2 at the end)
  }
  float r = 0.0f;
#pragma unroll
  for (int b = 0; b < Fmt<WB>::BPC; b++) {
    int acc = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) acc = dot4(u[8 * b + i], a.x[8 * b + i], acc);
    if (b == 0)
      r = a.d[b] * (float)acc;
    else
      r += a.d[b] * (float)acc;
  }
  return r;
}

enum { MODE_GATEUP = 0, MODE_DOWN = 1 };

// Resolve a grid slot to its expert and its pairs. Slot 0 is the shared expert
// when there is one (every token, output rows P + t); routed slot u is the u-th
// expert, ascending, with at least one pair. With a.idx set (decode-sized batches,
// P <= LOCAL_GROUP_MAX_P) the workgroup derives this from the route itself: one
// wavefront loads the P expert ids, marks them in an LDS bitmap, picks the u-th
// set bit and lists the expert's pair ids in ascending order with ballots. This
// replaces the grouping kernel and the chain of dependent loads (active -> offsets
// -> perm) with one load. Otherwise the grouping arrays are read.
struct SlotLds {
  int e, n;
  uint32_t bits[32];  // E <= 1024
  int pairs[LOCAL_GROUP_MAX_P];
};

//
// FUSE (gate/up kernels): with a.sel.part set, the workgroup first selects the route
// itself from the logit partials (fused_route; its LDS and the route in the dynamic
// LDS `dyn`, sized by fused_lds_bytes); the workgroup of the first routed slot's first
// tile stores it to a.sel.idx / a.sel.w. The shared expert's workgroups need no route.
template <bool FUSE = false>
__device__ __forceinline__ bool resolve_slot(const FfnArgs &a, int slot, SlotLds &L, int &e, int &n, int &beg,
                                             bool &shared, char *dyn = nullptr) {
  if (a.has_shared && slot == 0) {
    e = a.E;
    n = a.T;
    beg = 0;
    shared = true;
    return n > 0;
  }
  shared = false;
  const int u = slot - a.has_shared;
  if (a.idx == nullptr) {
    const int na = *a.nact;
    if (u >= na) return false;
    e = a.active[u];
    beg = a.off[e];
    n = a.off[e + 1] - beg;
    return n > 0;
  }
  beg = 0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int P = a.T * a.k;
  const int *rt = nullptr;  // route selected in this workgroup (LDS)
  if constexpr (FUSE) {
    if (a.sel.part != nullptr) {
      int *r = reinterpret_cast<int *>(dyn + fused_route_lds(a.T, a.E));
      fused_route(a.sel, dyn, r, blockIdx.x == 0 && slot == a.has_shared);
      rt = r;
    }
  }
  if (tid < 64) {
    constexpr int QD = LOCAL_GROUP_MAX_P / 64;
    int ev[QD];
#pragma unroll
    for (int i = 0; i < QD; i++) {
      const int p = lane + 64 * i;
      ev[i] = -1;
      if (p < P) {
        const int v = (FUSE && rt) ? rt[p] : a.idx[p];
        ev[i] = ((unsigned)v < (unsigned)a.E) ? v : -1;
      }
    }
    if (lane < 32) L.bits[lane] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < QD; i++)
      if (ev[i] >= 0) atomicOr(&L.bits[ev[i] >> 5], 1u << (ev[i] & 31));
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    __builtin_amdgcn_wave_barrier();
    const uint32_t word = (lane < 32) ? L.bits[lane] : 0u;
    const int c = __popc(word);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    const int excl = incl - c;
    const int total = __shfl(incl, 63);
    int me = -1;
    if (excl <= u && u < incl) {
      uint32_t w = word;
      for (int i = 0; i < u - excl; i++) w &= w - 1;
      me = lane * 32 + __ffs((int)w) - 1;
    }
    // broadcast the owner's expert (exactly one lane has it when u < total)
    const uint64_t own = __ballot(me >= 0);
    const int ex = (u < total && own) ? __shfl(me, __ffsll((long long)own) - 1) : -1;
    int cnt = 0;
    if (ex >= 0) {
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
      for (int i = 0; i < QD; i++) {
        const bool m = ev[i] == ex;
        const uint64_t b = __ballot(m);
        if (m) L.pairs[cnt + __popcll(b & below)] = lane + 64 * i;
        cnt += __popcll(b);
      }
    }
    if (lane == 0) {
      L.e = ex;
      L.n = cnt;
    }
  }
  __syncthreads();
  e = L.e;
  n = L.n;
  return e >= 0 && n > 0;
}

// pair id (row of hq / ypair) of the i-th token of a resolved slot
__device__ __forceinline__ int slot_pair(const FfnArgs &a, const SlotLds &L, bool shared, int beg, int i) {
  if (shared) return a.T * a.k + i;
  return a.idx ? L.pairs[i] : a.perm[beg + i];
}

// Cross-lane exchanges without LDS traffic. Within an aligned group of 2*O lanes
// the step for O pairs every lane of the lower half with one of the upper half:
// O = 32 and 16 by the permlane swaps (v_permlane32_swap exchanges the upper 32
// lanes of one register with the lower 32 of another, v_permlane16_swap the odd
// 16-lane rows with the even ones), O = 8 and 4 by the DPP row mirrors (partner
// lane l ^ 15 and l ^ 7), O = 2 and 1 by DPP quad permutes (l ^ 2, l ^ 1).
template <int O>
__device__ __forceinline__ float dpp_partner(float v) {
  static_assert(O == 8 || O == 4 || O == 2 || O == 1, "DPP partner within a 16-lane row");
  constexpr int ctrl = (O == 8) ? 0x140 : (O == 4) ? 0x141 : (O == 2) ? 0x4E : 0xB1;
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}

// lo, hi of every lane -> lower-half lanes get lo + partner's lo, upper-half lanes
// hi + partner's hi
template <int O>
__device__ __forceinline__ float pair_sum(float lo, float hi, bool up) {
  if constexpr (O == 32 || O == 16) {
    const auto r = (O == 32) ? __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false)
                             : __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const float send = up ? lo : hi;
    const float keep = up ? hi : lo;
    return keep + dpp_partner<O>(send);
  }
}

// Sum a[0..V) over the lanes of an aligned group of 2*O lanes. Scatter steps keep
// half of the values per lane; once one value is left the remaining steps are a
// butterfly. On return a[0..kept) hold full sums of original indices
// base .. base + kept - 1, the same in every lane of a group of LPR >> log2(V).
template <int V, int O>
__device__ __forceinline__ void reduce_scatter(float *a, int lane, int &base) {
  if constexpr (O >= 1) {
    const bool up = (lane & O) != 0;
    if constexpr (V > 1) {
#pragma unroll
      for (int i = 0; i < V / 2; i++) a[i] = pair_sum<O>(a[i], a[i + V / 2], up);
      if (up) base += V / 2;
      reduce_scatter<V / 2, O / 2>(a, lane, base);
    } else {
      a[0] = pair_sum<O>(a[0], a[0], up);
      reduce_scatter<1, O / 2>(a, lane, base);
    }
  }
}

// max over aligned groups of 32 lanes (exact in any order)
__device__ __forceinline__ float max32(float v) {
  v = fmaxf(v, dpp_partner<8>(v));
  v = fmaxf(v, dpp_partner<4>(v));
  v = fmaxf(v, dpp_partner<2>(v));
  v = fmaxf(v, dpp_partner<1>(v));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}


// GS: one scale per 64 inputs of a row (the scale of a chunk's group multiplies the
// chunk's contribution; a chunk never straddles two groups) instead of one per row.
template <int WB, int LPR, int MODE, bool GS = false>
__global__ __launch_bounds__(256) void gemv_kernel(FfnArgs a) {
  constexpr int NT = GEMV_NT;
  constexpr int RPI = WAVE / LPR;        // rows per wave iteration
  constexpr int WROWS = GEMV_ROWS / 4;   // rows per wave
  constexpr int NMAT = (MODE == MODE_GATEUP) ? 2 : 1;
  constexpr int CW = Fmt<WB>::CHUNK / 4;
  constexpr int BPC = Fmt<WB>::BPC;

  __shared__ SlotLds SL;
  extern __shared__ __align__(16) char smem[];
  int e, n, beg;
  bool shared;
  if (!resolve_slot<MODE == MODE_GATEUP>(a, blockIdx.y, SL, e, n, beg, shared, smem)) return;

  const int K = (MODE == MODE_GATEUP) ? a.H : a.F;       // inputs per row
  const int NROWS = (MODE == MODE_GATEUP) ? a.F : a.H;   // output rows per matrix
  const int nkb = K / QK;
  const int nchunk = nkb / BPC;
  const int cpl = nchunk / LPR;
  const int64_t rb = row_bytes(WB, K);
  const int P = a.T * a.k;

  const uint8_t *blob = a.experts + (int64_t)e * a.blob_bytes;
  const int64_t rbh = row_bytes(WB, a.H);
  const uint8_t *mat0 = (MODE == MODE_GATEUP) ? blob : blob + 2 * (int64_t)a.F * rbh;
  const uint8_t *mat1 = blob + (int64_t)a.F * rbh;  // up (gate/up mode only)
  const float *sc = a.scales + (int64_t)e * a.scale_stride;
  const float *sc0 = (MODE == MODE_GATEUP) ? sc : sc + 2 * a.F;
  const float *sc1 = sc + a.F;
  // group scales (G = GSZ inputs): gate [F][H/G] | up [F][H/G] | down [H][F/G]
  constexpr int G = GSZ<WB>;
  const int64_t ngh = (int64_t)a.F * (a.H / G);
  const int64_t se = (int64_t)e * a.scale_stride;
  const void *gsc0 = gs_base<WB>(a.scales, (MODE == MODE_GATEUP) ? se : se + 2 * ngh);
  const void *gsc1 = gs_base<WB>(a.scales, se + ngh);

  int8_t *xs = reinterpret_cast<int8_t *>(smem);                      // [NT][K]
  float *xds = reinterpret_cast<float *>(smem + NT * K);              // [NT][nkb]
  float *obuf = reinterpret_cast<float *>(xds + NT * nkb);            // [NT][32]
  int *orow = reinterpret_cast<int *>(obuf + NT * GEMV_ROWS);         // [NT]

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int rs = lane / LPR, sub = lane % LPR;
  const int r0 = blockIdx.x * GEMV_ROWS;

  for (int tc = 0; tc < n; tc += NT) {
    const int nt = min(NT, n - tc);
    // token -> activation row and output row
    if (tid < NT) {
      int out = -1, act = 0;
      if (tid < nt) {
        const int i = tc + tid;
        out = slot_pair(a, SL, shared, beg, i);
        act = (MODE == MODE_GATEUP) ? (shared ? i : out / a.k) : out;
      }
      orow[tid] = out;
      orow[NT + tid] = act;
    }
    __syncthreads();
    // stage activations (16 bytes per thread per step) and their block scales
    const int8_t *asrc = (MODE == MODE_GATEUP) ? a.xq : a.hq;
    const float *dsrc = (MODE == MODE_GATEUP) ? a.xd : a.hd;
    const int v16 = K / 16;
    for (int i = tid; i < nt * v16; i += 256) {
      const int t = i / v16, c = i % v16;
      const int act = orow[NT + t];
      *reinterpret_cast<int4 *>(xs + t * K + c * 16) =
          *reinterpret_cast<const int4 *>(asrc + (int64_t)act * K + c * 16);
    }
    for (int i = tid; i < nt * nkb; i += 256) {
      const int t = i / nkb, b = i % nkb;
      xds[t * nkb + b] = dsrc[(int64_t)orow[NT + t] * nkb + b];
    }
    __syncthreads();

    for (int it = 0; it < WROWS; it += RPI) {
      const int rl = it + rs;  // row within this wave's WROWS
      const bool rv = rl < WROWS;
      const int r = r0 + wv * WROWS + (rv ? rl : 0);
      const uint8_t *p0 = mat0 + (int64_t)r * rb;
      const uint8_t *p1 = mat1 + (int64_t)r * rb;
      float acc0[NT], acc1[NT];
#pragma unroll
      for (int t = 0; t < NT; t++) {
        acc0[t] = 0.0f;
        acc1[t] = 0.0f;
      }
      for (int ci = 0; ci < cpl; ci++) {
        const int c = sub + ci * LPR;
        uint32_t w0[CW], w1[CW];
        load_chunk<WB>(p0 + (int64_t)c * Fmt<WB>::CHUNK, w0);
        if constexpr (NMAT == 2) load_chunk<WB>(p1 + (int64_t)c * Fmt<WB>::CHUNK, w1);
        const int kx = c * BPC * QK;  // first input of this chunk
        float g0 = 1.0f, g1 = 1.0f;
        if constexpr (GS) {
          const int64_t gi = (int64_t)r * (K / G) + kx / G;
          g0 = gs_load<WB>(gsc0, gi);
          if constexpr (NMAT == 2) g1 = gs_load<WB>(gsc1, gi);
        }
#pragma unroll
        for (int t = 0; t < NT; t++) {
          if (t < nt) {
            const int8_t *xa = xs + t * K + kx;
            const float *xd = xds + t * nkb + c * BPC;
            if constexpr (GS) {
              acc0[t] = fmaf(g0, chunk_dot<WB>(w0, xa, xd), acc0[t]);
              if constexpr (NMAT == 2) acc1[t] = fmaf(g1, chunk_dot<WB>(w1, xa, xd), acc1[t]);
            } else {
              acc0[t] += chunk_dot<WB>(w0, xa, xd);
              if constexpr (NMAT == 2) acc1[t] += chunk_dot<WB>(w1, xa, xd);
            }
          }
        }
      }
      // reduce across the LPR lanes of the row
#pragma unroll
      for (int t = 0; t < NT; t++) {
        int b0 = 0;
        reduce_scatter<1, LPR / 2>(&acc0[t], lane, b0);
        if constexpr (NMAT == 2) reduce_scatter<1, LPR / 2>(&acc1[t], lane, b0);
      }
      if (rv && sub == 0) {
        const int rloc = wv * WROWS + rl;
        const float s0 = (GS ? 1.0f : sc0[r]) * Fmt<WB>::INV;
#pragma unroll
        for (int t = 0; t < NT; t++) {
          if (t < nt) {
            float v;
            if constexpr (MODE == MODE_GATEUP) {
              const float g = s0 * acc0[t];
              const float u = ((GS ? 1.0f : sc1[r]) * Fmt<WB>::INV) * acc1[t];
              COLI_TAP_GU(a, orow[t], r, g, u);
              v = (g / (1.0f + expf(-g))) * u;
            } else {
              v = s0 * acc0[t];
            }
            obuf[t * GEMV_ROWS + rloc] = v;
          }
        }
      }
    }
    __syncthreads();

    // epilogue: 32 rows x nt tokens; half a wavefront per token
    {
      const int t = tid >> 5, i = tid & 31;
      if (t < nt) {
        const float v = obuf[t * GEMV_ROWS + i];
        const int out = orow[t];
        if constexpr (MODE == MODE_GATEUP) {
          float am = fabsf(v);
          am = max32(am);
          const float d = am / 127.0f;
          int q = 0;
          if (d != 0.0f) q = (int)fminf(fmaxf(roundf(v / d), -127.0f), 127.0f);
          a.hq[(int64_t)out * a.F + r0 + i] = (int8_t)q;
          if (i == 0) a.hd[(int64_t)out * (a.F / QK) + r0 / QK] = d;
        } else {
          a.ypair[(int64_t)out * a.H + r0 + i] = v;
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Batched GEMV (the hot path for the common shapes). Same arithmetic and the same
// per-(row, token) summation tree as gemv_kernel; what changes is the schedule:
// each lane issues all weight loads of a batch of rows at once (up to 16 chunk
// loads, i.e. 16 KB in flight per wavefront), then computes every (row, token)
// partial sum of the batch, then reduces them across the LPR lanes of a row with
// a reduce-scatter (each shuffle step halves the values a lane carries), so the
// cross-lane cost is about one shuffle per value instead of log2(LPR).
template <int A, int B>
struct cmin {
  static constexpr int v = A < B ? A : B;
};

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

struct FastCtx {
  const uint8_t *mat0, *mat1;
  int64_t rb;        // packed bytes per row
  int K, nkb;
  const int8_t *xs;  // LDS activations [ntmax][K]
  const float *xds;  // LDS block scales [ntmax][nkb]
  float *obuf;       // LDS results [NMAT][8][TILE]
  int r0;            // first row of the tile
  const void *gs0, *gs1;  // group scales [rows][K/G] of the two matrices (GS only; see gs_base)
};

template <int WB, int NMAT, int LPR, int CPL, int WR, int NTC, bool GS, bool KEEP = false>
__device__ __forceinline__ void fast_pass(const FastCtx &c, int nt, int lane, int wv) {
  constexpr int RPI = WAVE / LPR;
  constexpr int CW = Fmt<WB>::CHUNK / 4;
  constexpr int BPC = Fmt<WB>::BPC;
  constexpr int LPC = Fmt<WB>::CHUNK / 16;
  constexpr int TILE = 4 * WR;
  // rows per lane and step: up to 16 chunk loads in flight, at most 32 accumulators
  constexpr int BR_LOAD = cmin<8, (16 / (NMAT * LPC) > 0 ? 16 / (NMAT * LPC) : 1)>::v;
  constexpr int BR_ACC = (32 / (NMAT * NTC) > 0) ? 32 / (NMAT * NTC) : 1;
  constexpr int BR_ROWS = (WR / RPI > 0) ? WR / RPI : 1;
  constexpr int BR = cmin<cmin<BR_LOAD, BR_ACC>::v, BR_ROWS>::v;
  constexpr int RPB = BR * RPI;  // rows of the wave per batch
  constexpr int V = BR * NMAT * NTC;
  constexpr int SCAT = cmin<ilog2(V), ilog2(LPR)>::v;
  constexpr int KEPT = V >> SCAT;
  constexpr int WMASK = (LPR >> SCAT) - 1;
  const int rs = lane / LPR, sub = lane % LPR;

  for (int b0 = 0; b0 < WR; b0 += RPB) {
    int64_t roff[BR];
    int64_t goff[BR];  // group-scale offset of the row (GS)
#pragma unroll
    for (int j = 0; j < BR; j++) {
      int rw = b0 + j * RPI + rs;
      rw = rw < WR ? rw : WR - 1;
      roff[j] = (int64_t)(c.r0 + wv * WR + rw) * c.rb;
      goff[j] = (int64_t)(c.r0 + wv * WR + rw) * (c.K / GSZ<WB>);
    }
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; i++) acc[i] = 0.0f;
#pragma unroll 1
    for (int ci = 0; ci < CPL; ci++) {
      const int ch = sub + ci * LPR;
      uint32_t w[BR][NMAT][CW];
#pragma unroll
      for (int j = 0; j < BR; j++)
#pragma unroll
        for (int m = 0; m < NMAT; m++)
          load_chunk<WB, KEEP>((m == 0 ? c.mat0 : c.mat1) + roff[j] + (int64_t)ch * Fmt<WB>::CHUNK, w[j][m]);
      float gsr[BR][NMAT];  // the chunk's group scale per row (a chunk lies in one group)
      if constexpr (GS) {
#pragma unroll
        for (int j = 0; j < BR; j++)
#pragma unroll
          for (int m = 0; m < NMAT; m++)
            gsr[j][m] = gs_load<WB>(m == 0 ? c.gs0 : c.gs1, goff[j] + ch * BPC * QK / GSZ<WB>);
      }
      Act<WB> act[NTC];
#pragma unroll
      for (int t = 0; t < NTC; t++)
        if (t < nt) load_act<WB>(c.xs + t * c.K + ch * BPC * QK, c.xds + t * c.nkb + ch * BPC, act[t]);
#pragma unroll
      for (int j = 0; j < BR; j++)
#pragma unroll
        for (int m = 0; m < NMAT; m++) {
          int u[Unp<WB>::N];
          unpack_chunk<WB>(w[j][m], u);
#pragma unroll
          for (int t = 0; t < NTC; t++) {
            if (t < nt) {
              if constexpr (GS)
                acc[(j * NMAT + m) * NTC + t] = fmaf(gsr[j][m], dot_unpacked<WB>(u, act[t]), acc[(j * NMAT + m) * NTC + t]);
              else
                acc[(j * NMAT + m) * NTC + t] += dot_unpacked<WB>(u, act[t]);
            }
          }
        }
    }
    int base = 0;
    reduce_scatter<V, LPR / 2>(acc, lane, base);
    if ((lane & WMASK) == 0) {
#pragma unroll
      for (int i = 0; i < KEPT; i++) {
        const int o = base + i;
        const int t = o % NTC, m = (o / NTC) % NMAT, j = o / (NTC * NMAT);
        const int rw = b0 + j * RPI + rs;
        if (t < nt && rw < WR) c.obuf[(m * 8 + t) * TILE + wv * WR + rw] = acc[i];
      }
    }
  }
}

// Software-pipelined form of fast_pass: the wavefront's rows are cut into steps of
// BR rows x one chunk per lane (8 loads per lane), and the loads of step s + 1 are
// issued before step s is computed, into a second register set. A wavefront thus
// keeps its next loads in flight while it computes, instead of waiting one memory
// round trip per chunk round; the registers held are those of fast_pass (two sets of
// half the rows). Same products, the same per-lane order of chunks and the same
// reduce-scatter as fast_pass, so the results are bit-identical.
template <int WB, int NMAT, int LPR, int CPL, int WR, int NTC, bool GS, bool KEEP = false>
__device__ __forceinline__ void fast_pass_pl(const FastCtx &c, int nt, int lane, int wv) {
  constexpr int RPI = WAVE / LPR;
  constexpr int CW = Fmt<WB>::CHUNK / 4;
  constexpr int BPC = Fmt<WB>::BPC;
  constexpr int LPC = Fmt<WB>::CHUNK / 16;
  constexpr int TILE = 4 * WR;
  // MXFP4 steps take two rows: its converted codes and fp16 activation pairs need twice
  // the registers of the integer formats
  constexpr int BR_LOAD = cmin<(WB == W_MX ? 2 : 4), (8 / (NMAT * LPC) > 0 ? 8 / (NMAT * LPC) : 1)>::v;
  constexpr int BR_ACC = (32 / (NMAT * NTC) > 0) ? 32 / (NMAT * NTC) : 1;
  constexpr int BR_ROWS = (WR / RPI > 0) ? WR / RPI : 1;
  constexpr int BR = cmin<cmin<BR_LOAD, BR_ACC>::v, BR_ROWS>::v;
  constexpr int RPB = BR * RPI;  // rows of the wave per batch
  constexpr int NB = (WR + RPB - 1) / RPB;
  constexpr int NS = NB * CPL;   // steps: (batch, chunk round)
  constexpr int V = BR * NMAT * NTC;
  constexpr int SCAT = cmin<ilog2(V), ilog2(LPR)>::v;
  constexpr int KEPT = V >> SCAT;
  constexpr int WMASK = (LPR >> SCAT) - 1;
  const int rs = lane / LPR, sub = lane % LPR;

  uint32_t w[2][BR][NMAT][CW];
  float gsr[2][BR][NMAT];  // the chunk's group scale per row (GS)
  auto row_of = [&](int b, int j) {
    const int rw = b * RPB + j * RPI + rs;
    return c.r0 + wv * WR + (rw < WR ? rw : WR - 1);
  };
  auto issue = [&](int st, int buf) __attribute__((always_inline)) {
    const int b = st / CPL, ch = sub + (st % CPL) * LPR;
#pragma unroll
    for (int j = 0; j < BR; j++) {
      const int64_t roff = (int64_t)row_of(b, j) * c.rb + (int64_t)ch * Fmt<WB>::CHUNK;
#pragma unroll
      for (int m = 0; m < NMAT; m++) load_chunk<WB, KEEP>((m == 0 ? c.mat0 : c.mat1) + roff, w[buf][j][m]);
      if constexpr (GS) {
        const int64_t goff = (int64_t)row_of(b, j) * (c.K / GSZ<WB>) + ch * BPC * QK / GSZ<WB>;
#pragma unroll
        for (int m = 0; m < NMAT; m++) gsr[buf][j][m] = gs_load<WB>(m == 0 ? c.gs0 : c.gs1, goff);
      }
    }
  };

  float acc[V];
  issue(0, 0);
#pragma unroll
  for (int st = 0; st < NS; st++) {
    const int buf = st & 1, b = st / CPL, ci = st % CPL;
    if (st + 1 < NS) {
      // the next step's loads go out before this step's products (kept in this order)
#pragma unroll
      for (int j = 0; j < BR; j++)
#pragma unroll
        for (int m = 0; m < NMAT; m++)
#pragma unroll
          for (int q = 0; q < CW; q++) asm volatile("" : "+v"(w[buf][j][m][q]));
      issue(st + 1, buf ^ 1);
    }
    if (ci == 0) {
#pragma unroll
      for (int i = 0; i < V; i++) acc[i] = 0.0f;
    }
    const int ch = sub + ci * LPR;
    Act<WB> act[NTC];
#pragma unroll
    for (int t = 0; t < NTC; t++)
      if (t < nt) load_act<WB>(c.xs + t * c.K + ch * BPC * QK, c.xds + t * c.nkb + ch * BPC, act[t]);
#pragma unroll
    for (int j = 0; j < BR; j++)
#pragma unroll
      for (int m = 0; m < NMAT; m++) {
        int u[Unp<WB>::N];
        unpack_chunk<WB>(w[buf][j][m], u);
#pragma unroll
        for (int t = 0; t < NTC; t++) {
          if (t < nt) {
            if constexpr (GS)
              acc[(j * NMAT + m) * NTC + t] = fmaf(gsr[buf][j][m], dot_unpacked<WB>(u, act[t]), acc[(j * NMAT + m) * NTC + t]);
            else
              acc[(j * NMAT + m) * NTC + t] += dot_unpacked<WB>(u, act[t]);
          }
        }
      }
    if (ci == CPL - 1) {
      int base = 0;
      reduce_scatter<V, LPR / 2>(acc, lane, base);
      if ((lane & WMASK) == 0) {
#pragma unroll
        for (int i = 0; i < KEPT; i++) {
          const int o = base + i;
          const int t = o % NTC, m = (o / NTC) % NMAT, j = o / (NTC * NMAT);
          const int rw = b * RPB + j * RPI + rs;
          if (t < nt && rw < WR) c.obuf[(m * 8 + t) * TILE + wv * WR + rw] = acc[i];
        }
      }
    }
  }
}

// The pipelined pass where it measured faster and fits three wavefronts per SIMD
// without spilling: int4 gate/up rows of three chunks per lane with one scale per row
// (GLM-scale experts). Elsewhere its second register set spills or costs occupancy.
// MXFP4 gate/up rows of three chunks take it for one-token batches only (`one`; two
// wavefronts per SIMD, as the plain pass): GLM-scale T = 1 gate/up 38.0 -> 34.9 us,
// while at T = 4 and 16 it measured slower (84.4 -> 90.1 us, 288.3 -> 305.4 us).
template <int WB, int CPL, int MODE, bool GS>
struct FastPl {
  static constexpr bool on = WB == 4 && CPL == 3 && MODE == MODE_GATEUP && !GS;
  static constexpr bool one = WB == W_MX && CPL == 3 && MODE == MODE_GATEUP;
};

// GS: one scale per 64 inputs of a row, applied per chunk (see gemv_kernel).
// PL: every pass takes the pipelined form (fast_pass_pl), bit-identical to fast_pass.
template <int WB, int LPR, int CPL, int MODE, int WR, bool GS = false, bool PL = FastPl<WB, CPL, MODE, GS>::on>
__global__ __launch_bounds__(256, (PL ? (WB == 4 ? 3 : 2) : 1)) void gemv_fast_kernel(FfnArgs a, int ntmax) {
  constexpr int NMAT = (MODE == MODE_GATEUP) ? 2 : 1;
  constexpr int TILE = 4 * WR;
  static_assert(MODE == MODE_DOWN || TILE % QK == 0, "gate/up tiles hold whole Q8_0 blocks of h");

  __shared__ SlotLds SL;
  extern __shared__ __align__(16) char smem[];
  int e, n, beg;
  bool shared;
  if (!resolve_slot<MODE == MODE_GATEUP>(a, blockIdx.y, SL, e, n, beg, shared, smem)) return;

  const int K = (MODE == MODE_GATEUP) ? a.H : a.F;
  const int nkb = K / QK;
  const uint8_t *blob = a.experts + (int64_t)e * a.blob_bytes;
  const int64_t rbh = row_bytes(WB, a.H);
  const float *sc = a.scales + (int64_t)e * a.scale_stride;

  FastCtx c;
  c.mat0 = (MODE == MODE_GATEUP) ? blob : blob + 2 * (int64_t)a.F * rbh;
  c.mat1 = blob + (int64_t)a.F * rbh;
  c.rb = row_bytes(WB, K);
  c.K = K;
  c.nkb = nkb;
  int8_t *xs = reinterpret_cast<int8_t *>(smem);
  float *xds = reinterpret_cast<float *>(smem + (size_t)ntmax * K);
  float *obuf = reinterpret_cast<float *>(xds + (size_t)ntmax * nkb);
  int *orow = reinterpret_cast<int *>(obuf + NMAT * 8 * TILE);
  c.xs = xs;
  c.xds = xds;
  c.obuf = obuf;
  c.r0 = blockIdx.x * TILE;
  {
    const int64_t ngh = (int64_t)a.F * (a.H / GSZ<WB>);
    const int64_t se = (int64_t)e * a.scale_stride;
    c.gs0 = gs_base<WB>(a.scales, (MODE == MODE_GATEUP) ? se : se + 2 * ngh);
    c.gs1 = gs_base<WB>(a.scales, se + ngh);
  }

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int8_t *asrc = (MODE == MODE_GATEUP) ? a.xq : a.hq;
  const float *dsrc = (MODE == MODE_GATEUP) ? a.xd : a.hd;

  for (int tc = 0; tc < n; tc += ntmax) {
    const int nt = min(ntmax, n - tc);
    if (tid < 8) {
      int out = -1, act = 0;
      if (tid < nt) {
        const int i = tc + tid;
        out = slot_pair(a, SL, shared, beg, i);
        act = (MODE == MODE_GATEUP) ? (shared ? i : out / a.k) : out;
      }
      orow[tid] = out;
      orow[8 + tid] = act;
    }
    __syncthreads();
    const int v16 = K / 16;
    for (int i = tid; i < nt * v16; i += 256) {
      const int t = i / v16, ch = i % v16;
      *reinterpret_cast<int4 *>(xs + t * K + ch * 16) =
          *reinterpret_cast<const int4 *>(asrc + (int64_t)orow[8 + t] * K + ch * 16);
    }
    for (int i = tid; i < nt * nkb; i += 256) {
      const int t = i / nkb, b = i % nkb;
      xds[t * nkb + b] = dsrc[(int64_t)orow[8 + t] * nkb + b];
    }
    __syncthreads();
    // a slot with more tokens than one pass takes re-reads its rows on every pass: those
    // loads allocate in L2 so that the later passes find them there
    const bool keep = n > ntmax;
    if constexpr (PL) {
      if (keep)
        fast_pass_pl<WB, NMAT, LPR, CPL, WR, 2, GS, true>(c, nt, lane, wv);
      else if (nt <= 1)
        fast_pass_pl<WB, NMAT, LPR, CPL, WR, 1, GS>(c, nt, lane, wv);
      else
        fast_pass_pl<WB, NMAT, LPR, CPL, WR, 2, GS>(c, nt, lane, wv);
    } else {
      if (keep)
        fast_pass<WB, NMAT, LPR, CPL, WR, 2, GS, true>(c, nt, lane, wv);
      else if (nt <= 1)
        fast_pass<WB, NMAT, LPR, CPL, WR, 1, GS>(c, nt, lane, wv);
      else
        fast_pass<WB, NMAT, LPR, CPL, WR, 2, GS>(c, nt, lane, wv);
    }
    __syncthreads();
    // epilogue over the tile's rows x nt tokens
    if constexpr (MODE == MODE_GATEUP) {
      const float *sg = sc, *su = sc + a.F;
      for (int p = tid; p < nt * TILE; p += 256) {  // one Q8_0 block of h per 32 consecutive lanes
        const int t = p / TILE, i = p % TILE, r = c.r0 + i;
        const float g = ((GS ? 1.0f : sg[r]) * Fmt<WB>::INV) * obuf[(0 * 8 + t) * TILE + i];
        const float u = ((GS ? 1.0f : su[r]) * Fmt<WB>::INV) * obuf[(1 * 8 + t) * TILE + i];
        COLI_TAP_GU(a, orow[t], r, g, u);
        const float v = (g / (1.0f + expf(-g))) * u;
        float am = fabsf(v);
        am = max32(am);
        const float d = am / 127.0f;
        int q = 0;
        if (d != 0.0f) q = (int)fminf(fmaxf(roundf(v / d), -127.0f), 127.0f);
        const int out = orow[t];
        a.hq[(int64_t)out * a.F + r] = (int8_t)q;
        if ((i & 31) == 0) a.hd[(int64_t)out * (a.F / QK) + r / QK] = d;
      }
    } else {
      const float *sd = sc + 2 * a.F;
      for (int p = tid; p < nt * TILE; p += 256) {
        const int t = p / TILE, i = p % TILE, r = c.r0 + i;
        a.ypair[(int64_t)orow[t] * a.H + r] = ((GS ? 1.0f : sd[r]) * Fmt<WB>::INV) * obuf[t * TILE + i];
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Register-resident GEMV: the shapes whose row is one chunk per lane (CPL = 1) and
// whose tile fits in registers. Every lane loads all of its tile's weight chunks
// once, right after the slot is known, and keeps them across the token passes, so
// the weights of an expert are read from memory exactly once whatever its token
// count. Activations (Q8_0 rows, L2-resident) are read per pass straight into
// registers, without LDS staging. Same arithmetic and summation tree as
// gemv_fast_kernel.
// Barrier for LDS hand-offs only: wait for this wavefront's LDS accesses
// (lgkmcnt = 0), then s_barrier. __syncthreads() also waits for every outstanding
// global load and store (vmcnt = 0), i.e. for the epilogue's stores to reach
// memory, which under full HBM load costs microseconds per pass.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0 (gfx9 encoding)
  __builtin_amdgcn_s_barrier();
}

template <int WB, int LPR, int MODE, int WR, int NTC>
__global__ __launch_bounds__(256) void gemv_reg_kernel(FfnArgs a) {
  constexpr int NMAT = (MODE == MODE_GATEUP) ? 2 : 1;
  constexpr int RPI = WAVE / LPR;
  constexpr int R = WR / RPI;  // rows per lane
  constexpr int CW = Fmt<WB>::CHUNK / 4;
  constexpr int BPC = Fmt<WB>::BPC;
  constexpr int TILE = 4 * WR;
  constexpr int V = R * NMAT * NTC;
  constexpr int SCAT = cmin<ilog2(V), ilog2(LPR)>::v;
  constexpr int KEPT = V >> SCAT;
  constexpr int WMASK = (LPR >> SCAT) - 1;
  static_assert(R * RPI == WR && R * NMAT * CW <= 64, "tile weights fit in 64 registers per lane");
  static_assert(MODE == MODE_DOWN || TILE % QK == 0, "gate/up tiles hold whole Q8_0 blocks of h");
  static_assert(NTC * TILE <= 256, "one epilogue value per thread and pass");

  __shared__ SlotLds SL;
  __shared__ float obuf[NMAT][NTC][TILE];
  extern __shared__ __align__(16) char smem[];  // fused route only
  int e, n = 0, beg = 0;
  bool shared;
  if (!resolve_slot<MODE == MODE_GATEUP>(a, blockIdx.y, SL, e, n, beg, shared, smem)) return;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int rs = lane / LPR, sub = lane % LPR;
  const int K = (MODE == MODE_GATEUP) ? a.H : a.F;
  const int nkb = K / QK;
  const int64_t rb = row_bytes(WB, K);
  const int64_t rbh = row_bytes(WB, a.H);
  const uint8_t *blob = a.experts + (int64_t)e * a.blob_bytes;
  const uint8_t *mat0 = (MODE == MODE_GATEUP) ? blob : blob + 2 * (int64_t)a.F * rbh;
  const uint8_t *mat1 = blob + (int64_t)a.F * rbh;
  const int r0 = blockIdx.x * TILE;

  // epilogue value of this thread: token pt, row r0 + pi of the tile; its raw row
  // scales are loaded first (1/S is applied at use, so nothing waits for them early)
  const int pt = tid / TILE, pi = tid % TILE;
  const float *sc = a.scales + (int64_t)e * a.scale_stride;
  float s0 = 0.0f, s1 = 0.0f;
  if (pt < NTC) {
    if constexpr (MODE == MODE_GATEUP) {
      s0 = sc[r0 + pi];
      s1 = sc[a.F + r0 + pi];
    } else {
      s0 = sc[2 * a.F + r0 + pi];
    }
  }
  uint32_t w[R][NMAT][CW];
#pragma unroll
  for (int j = 0; j < R; j++) {
    const int64_t roff = (int64_t)(r0 + wv * WR + j * RPI + rs) * rb + (int64_t)sub * Fmt<WB>::CHUNK;
#pragma unroll
    for (int m = 0; m < NMAT; m++) load_chunk<WB>((m == 0 ? mat0 : mat1) + roff, w[j][m]);
  }
  const int8_t *asrc = (MODE == MODE_GATEUP) ? a.xq : a.hq;
  const float *dsrc = (MODE == MODE_GATEUP) ? a.xd : a.hd;

  for (int tc = 0; tc < n; tc += NTC) {
    const int nt = min(NTC, n - tc);
    int orow[NTC];
    Act<WB> act[NTC];
#pragma unroll
    for (int t = 0; t < NTC; t++) {
      const int i = tc + min(t, nt - 1);  // past nt: repeat the last token, write nothing
      const int p = slot_pair(a, SL, shared, beg, i);
      orow[t] = p;
      const int64_t arow = (MODE == MODE_GATEUP) ? (shared ? i : p / a.k) : p;
      load_act<WB>(asrc + arow * K + sub * BPC * QK, dsrc + arow * nkb + sub * BPC, act[t]);
    }
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; i++) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < R; j++)
#pragma unroll
      for (int m = 0; m < NMAT; m++) {
        // unpack per pass: kept out of the pass loop the unpacked tile would need
        // twice the registers (the empty asm makes the packed words opaque)
#pragma unroll
        for (int q = 0; q < CW; q++) asm volatile("" : "+v"(w[j][m][q]));
        int u[Unp<WB>::N];
        unpack_chunk<WB>(w[j][m], u);
#pragma unroll
        for (int t = 0; t < NTC; t++) acc[(j * NMAT + m) * NTC + t] += dot_unpacked<WB>(u, act[t]);
      }
    int base = 0;
    reduce_scatter<V, LPR / 2>(acc, lane, base);
    if ((lane & WMASK) == 0) {
#pragma unroll
      for (int i = 0; i < KEPT; i++) {
        const int o = base + i;
        const int t = o % NTC, m = (o / NTC) % NMAT, j = o / (NTC * NMAT);
        obuf[m][t][wv * WR + j * RPI + rs] = acc[i];
      }
    }
    lds_barrier();
    if (pt < NTC) {
      const int r = r0 + pi;
      const bool live = pt < nt;
      int out = orow[0];
#pragma unroll
      for (int t = 1; t < NTC; t++)
        if (pt == t) out = orow[t];
      if constexpr (MODE == MODE_GATEUP) {
        // a Q8_0 block of h = 32 consecutive rows = 32 consecutive threads of one token
        const float g = s0 * (obuf[0][pt][pi] * Fmt<WB>::INV);
        const float u = s1 * (obuf[NMAT - 1][pt][pi] * Fmt<WB>::INV);
        if (live) COLI_TAP_GU(a, out, r, g, u);
        const float v = (g / (1.0f + expf(-g))) * u;
        float am = fabsf(v);
        am = max32(am);
        const float d = am / 127.0f;
        int q = 0;
        if (d != 0.0f) q = (int)fminf(fmaxf(roundf(v / d), -127.0f), 127.0f);
        if (live) {
          a.hq[(int64_t)out * a.F + r] = (int8_t)q;
          if ((pi & 31) == 0) a.hd[(int64_t)out * (a.F / QK) + r / QK] = d;
        }
      } else {
        if (live) a.ypair[(int64_t)out * a.H + r] = s0 * (obuf[0][pt][pi] * Fmt<WB>::INV);
      }
    }
    lds_barrier();
  }
}

// ---------------------------------------------------------------------------
// Pipelined register GEMV (decode-sized batches: the route is at hand and
// P <= LOCAL_GROUP_MAX_P). The work is cut into units, one unit being one
// TILE-row tile of one slot (the shared expert, or a hit expert). A grid of G
// workgroups, about as many as are resident on the chip at once, walks them:
// workgroup b takes units b, b + G, b + 2G, ... (a shared work counter was
// measured slower: thousands of same-address atomics per launch serialise).
// A workgroup lists the hit experts from the route once. Per unit:
//  - one wavefront lists the next unit's pairs (ascending) at the top;
//  - the next unit's weights are loaded into the tile registers as soon as the
//    last token pass has consumed them (per half of the rows), so they are in
//    flight during that pass's cross-lane reduction and epilogue and HBM keeps
//    streaming while the SIMDs compute;
//  - the activations of the next unit's first token pass are loaded during the
//    last epilogue, so a unit's first products wait only for its weights.
// Token passes take two tokens, the last one a single token when the count is
// odd; no pass computes a token twice. Same arithmetic and summation tree as
// gemv_reg_kernel. Unit i is tile i % NT of slot i / NT of the slot list
// [shared expert] + hit experts (ascending). (Loading the first units' weights
// before the route is read, numbering them over every expert, was measured no
// faster: the loads of experts without tokens are wasted.)
struct PipeLds {
  int route[LOCAL_GROUP_MAX_P];     // expert id of pair p (-1 past P or out of range)
  int live[1024];                   // hit experts, ascending (E <= 1024)
  int pairs[2][LOCAL_GROUP_MAX_P];  // pair ids of the current / next unit's expert
  int npairs[2];
  int nlive;                        // hit experts
  uint32_t bits[32];
};

// pairs of expert e in ascending order (one wavefront)
__device__ __forceinline__ void pipe_list_pairs(const PipeLds &L, int e, int P, int *out, int *nout, int lane) {
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < LOCAL_GROUP_MAX_P / 64; i++) {
    if (64 * i < P) {
      const bool m = L.route[lane + 64 * i] == e;
      const uint64_t b = __ballot(m);
      if (m) out[cnt + __popcll(b & below)] = lane + 64 * i;
      cnt += __popcll(b);
    }
  }
  if (lane == 0) *nout = cnt;
}

// GS: one scale per 64 inputs of a row; the lane's chunk lies in one group, whose
// scale per tile row is loaded with the row's weights and multiplies the chunk's
// products (the row scales of the epilogue are then 1).
template <int WB, int LPR, int MODE, int WR, bool GS = false>
__global__ __launch_bounds__(256) void gemv_pipe_kernel(FfnArgs a) {
  constexpr int NMAT = (MODE == MODE_GATEUP) ? 2 : 1;
  constexpr int RPI = WAVE / LPR;
  constexpr int R = WR / RPI;  // rows per lane
  constexpr int CW = Fmt<WB>::CHUNK / 4;
  constexpr int BPC = Fmt<WB>::BPC;
  constexpr int TILE = 4 * WR;
  constexpr int QD = LOCAL_GROUP_MAX_P / 64;
  constexpr int RH = (R % 2 == 0) ? R / 2 : R;  // rows per half
  static_assert(R * RPI == WR && R * NMAT * CW <= 64, "tile weights fit in 64 registers per lane");
  static_assert(MODE == MODE_DOWN || TILE % QK == 0, "gate/up tiles hold whole Q8_0 blocks of h");
  static_assert(2 * TILE <= 192, "epilogue of two tokens on wavefronts 0..2; wavefront 3 lists pairs");

  __shared__ PipeLds L;
  __shared__ float obuf[NMAT][2][TILE];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int rs = lane / LPR, sub = lane % LPR;
  const int K = (MODE == MODE_GATEUP) ? a.H : a.F;
  const int NROWS = (MODE == MODE_GATEUP) ? a.F : a.H;
  const int NT = NROWS / TILE;  // tiles per slot
  const int nkb = K / QK;
  const int64_t rb = row_bytes(WB, K);
  const int64_t rbh = row_bytes(WB, a.H);
  const int P = a.T * a.k;
  const int hs = a.has_shared;
  const int G = (int)gridDim.x, b = (int)blockIdx.x;

  // Load addresses are a wave-uniform base (scalar registers) plus one per-lane
  // 32-bit offset, so a reload in mid-flight costs no extra vector registers.
  // Epilogue thread tid: token pt, row pi of the tile.
  const int pt = tid / TILE, pi = tid % TILE;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const uint32_t lane_w = (uint32_t)(rs * rb + sub * Fmt<WB>::CHUNK);
  const uint32_t lane_x = (uint32_t)(sub * BPC * QK);
  uint32_t w[R][NMAT][CW];
  float gsr[R][NMAT];  // group scales of the lane's chunk per tile row (GS)
  // weights of expert e (a.E: the shared expert), tile rows r0..: rows
  // h * RH .. h * RH + RH - 1 of the lane's tile rows (h < 0: all rows), preceded
  // by the row scales when h <= 0 (raw: 1/S is applied at use, so nothing waits
  // for these loads before the epilogue)
  auto issue = [&](int e, int r0, int h, float &t0, float &t1) {
    if (GS) {
      t0 = 1.0f;
      t1 = 1.0f;
    } else if (h <= 0 && pt < 2) {
      const float *sc = a.scales + (int64_t)e * a.scale_stride;
      if constexpr (MODE == MODE_GATEUP) {
        t0 = sc[r0 + pi];
        t1 = sc[a.F + r0 + pi];
      } else {
        t0 = sc[2 * a.F + r0 + pi];
      }
    }
    int64_t eoff = (int64_t)e * a.blob_bytes;
    asm volatile("" : "+s"(eoff));  // the loads stay after whatever precedes the call
    const uint8_t *blob = a.experts + eoff;
    const uint8_t *mat0 = (MODE == MODE_GATEUP) ? blob : blob + 2 * (int64_t)a.F * rbh;
    const uint8_t *mat1 = blob + (int64_t)a.F * rbh;
#pragma unroll
    for (int j = 0; j < R; j++) {
      if (h >= 0 && j / RH != h) continue;
      const int64_t roff = (int64_t)(r0 + wvu * WR + j * RPI) * rb;
#pragma unroll
      for (int m = 0; m < NMAT; m++) load_chunk<WB>((m == 0 ? mat0 : mat1) + roff + lane_w, w[j][m]);
    }
    if constexpr (GS) {
      // group scales (G = GSZ inputs): gate [F][H/G] | up [F][H/G] | down [H][F/G]
      constexpr int G = GSZ<WB>;
      const int64_t ngh = (int64_t)a.F * (a.H / G);
      const void *gsc = gs_base<WB>(a.scales, (int64_t)e * a.scale_stride + ((MODE == MODE_GATEUP) ? 0 : 2 * ngh));
#pragma unroll
      for (int j = 0; j < R; j++) {
        if (h >= 0 && j / RH != h) continue;
        const int64_t goff = (int64_t)(r0 + wvu * WR + j * RPI + rs) * (K / G) + lane_x / G;
#pragma unroll
        for (int m = 0; m < NMAT; m++) gsr[j][m] = gs_load<WB>(gsc, m * ngh + goff);
      }
    }
  };

  float s0 = 0.0f, s1 = 0.0f, s0n = 0.0f, s1n = 0.0f;

  // the route: selected here from the logit partials (gate/up with a.sel.part set;
  // the first workgroup stores it for the kernels that follow), else loaded
  bool fused = false;
  if constexpr (MODE == MODE_GATEUP) {
    if (a.sel.part != nullptr) {
      extern __shared__ __align__(16) char smem[];
      fused_route(a.sel, smem, L.route, b == 0);
      fused = true;
    }
  }
  // the hit experts, ascending (wavefront 0); the route loads go out together
  if (wv == 0) {
    int ev[QD];
#pragma unroll
    for (int i = 0; i < QD; i++) {
      const int p = lane + 64 * i;
      ev[i] = (p < P) ? (fused ? L.route[p] : a.idx[p]) : -1;
    }
#pragma unroll
    for (int i = 0; i < QD; i++) {
      ev[i] = ((unsigned)ev[i] < (unsigned)a.E) ? ev[i] : -1;
      L.route[lane + 64 * i] = ev[i];
    }
    if (lane < 32) L.bits[lane] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < QD; i++)
      if (ev[i] >= 0) atomicOr(&L.bits[ev[i] >> 5], 1u << (ev[i] & 31));
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    __builtin_amdgcn_wave_barrier();
    uint32_t word = (lane < 32) ? L.bits[lane] : 0u;
    const int c = __popc(word);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    int o = incl - c;
    while (word) {
      L.live[o++] = lane * 32 + __ffs((int)word) - 1;
      word &= word - 1;
    }
    if (lane == 63) L.nlive = incl;
  }
  __syncthreads();
  const int nlive = __builtin_amdgcn_readfirstlane(L.nlive);
  const int total = (hs + nlive) * NT;
  if (b >= total) return;
  // expert of unit i (a.E: shared) and its first tile row; both wave-uniform
  // (scalar registers, so the load addresses stay scalar bases)
  auto unit = [&](int i, int &r0) -> int {
    const int sl = i / NT;
    r0 = __builtin_amdgcn_readfirstlane((i % NT) * TILE);
    return __builtin_amdgcn_readfirstlane((sl < hs) ? a.E : L.live[sl - hs]);
  };
  auto list = [&](int e, int bb) {
    if (e >= 0 && e < a.E) pipe_list_pairs(L, e, P, L.pairs[bb], &L.npairs[bb], lane);
  };

  int cur = b, nxt = G + b;
  int r0c = 0;
  int ec = unit(cur, r0c);
  issue(ec, r0c, -1, s0, s1);
  if (wv == 3) list(ec, 0);
  lds_barrier();
  const int8_t *asrc = (MODE == MODE_GATEUP) ? a.xq : a.hq;
  const float *dsrc = (MODE == MODE_GATEUP) ? a.xd : a.hd;
  // activations (and output rows) of tokens tc, tc + 1 of expert e, pair list bb
  Act<WB> act[2];
  int orow[2];
  auto load_acts = [&](int e, int bb, int tc, int cnt) {
    const bool sh = e == a.E;
#pragma unroll
    for (int t = 0; t < 2; t++) {
      if (t < cnt) {
        const int i = tc + t;
        const int p = sh ? P + i : __builtin_amdgcn_readfirstlane(L.pairs[bb][i]);
        orow[t] = p;
        const int64_t arow = (MODE == MODE_GATEUP) ? (sh ? i : p / a.k) : p;
        load_act<WB>(asrc + arow * K + lane_x, dsrc + arow * nkb + sub * BPC, act[t]);
      }
    }
  };
  // first token pass of a unit, loaded a unit ahead
  auto load_first = [&](int e, int bb) {
    if (e < 0) return;
    const int n = (e == a.E) ? a.T : __builtin_amdgcn_readfirstlane(L.npairs[bb]);
    load_acts(e, bb, 0, n < 2 ? n : 2);
  };
  load_first(ec, 0);
  int buf = 0;
  for (;;) {
    const bool has_next = nxt < total;
    int r0n = 0;
    const int en = has_next ? unit(nxt, r0n) : -1;
    if (wv == 3) list(en, buf ^ 1);  // visible after this unit's first barrier
    {
      const bool shared = ec == a.E;
      const int n = shared ? a.T : __builtin_amdgcn_readfirstlane(L.npairs[buf]);
      auto pass = [&](auto ntc_tag, int tc) {
        constexpr int NTC = decltype(ntc_tag)::value;
        constexpr int V = RH * NMAT * NTC;  // accumulators of one half
        constexpr int SCAT = cmin<ilog2(V), ilog2(LPR)>::v;
        constexpr int KEPT = V >> SCAT;
        constexpr int WMASK = (LPR >> SCAT) - 1;
        const bool last = tc + NTC >= n;
        if (tc > 0) load_acts(ec, buf, tc, NTC);
        // two halves of the tile rows: products, then (last pass) the next unit's
        // loads into the freed registers, then the half's reduction
#pragma unroll
        for (int h = 0; h < R / RH; h++) {
          float acc[V];
#pragma unroll
          for (int i = 0; i < V; i++) acc[i] = 0.0f;
#pragma unroll
          for (int jj = 0; jj < RH; jj++)
#pragma unroll
            for (int m = 0; m < NMAT; m++) {
              const int j = h * RH + jj;
#pragma unroll
              for (int q = 0; q < CW; q++) asm volatile("" : "+v"(w[j][m][q]));
              int uq[Unp<WB>::N];
              unpack_chunk<WB>(w[j][m], uq);
#pragma unroll
              for (int t = 0; t < NTC; t++) {
                if constexpr (GS)
                  acc[(jj * NMAT + m) * NTC + t] = fmaf(gsr[j][m], dot_unpacked<WB>(uq, act[t]), acc[(jj * NMAT + m) * NTC + t]);
                else
                  acc[(jj * NMAT + m) * NTC + t] += dot_unpacked<WB>(uq, act[t]);
              }
            }
          if (last && en >= 0) {
            // ordered after the products: hoisted above them the loads would need
            // a second set of tile registers
#pragma unroll
            for (int i = 0; i < V; i++) asm volatile("" : "+v"(acc[i]));
            issue(en, r0n, h, s0n, s1n);
          }
          int base = 0;
          reduce_scatter<V, LPR / 2>(acc, lane, base);
          if ((lane & WMASK) == 0) {
#pragma unroll
            for (int i = 0; i < KEPT; i++) {
              const int o = base + i;
              const int t = o % NTC, m = (o / NTC) % NMAT, jj = o / (NTC * NMAT);
              obuf[m][t][wv * WR + (h * RH + jj) * RPI + rs] = acc[i];
            }
          }
        }
        lds_barrier();
        int out = orow[0];
#pragma unroll
        for (int t = 1; t < NTC; t++)
          if (pt == t) out = orow[t];
        if (last) load_first(en, buf ^ 1);  // the next unit's first pass, during the epilogue
        if (pt < NTC) {
          const int r = r0c + pi;
          if constexpr (MODE == MODE_GATEUP) {
            // a Q8_0 block of h = 32 consecutive rows = 32 consecutive threads of one
            // token (obuf * 1/S is exact: s * (obuf / S) is the one rounding of s * acc)
            const float g = s0 * (obuf[0][pt][pi] * Fmt<WB>::INV);
            const float uv = s1 * (obuf[NMAT - 1][pt][pi] * Fmt<WB>::INV);
            COLI_TAP_GU(a, out, r, g, uv);
            const float v = (g / (1.0f + expf(-g))) * uv;
            const float am = max32(fabsf(v));
            const float d = am / 127.0f;
            int q = 0;
            if (d != 0.0f) q = (int)fminf(fmaxf(roundf(v / d), -127.0f), 127.0f);
            a.hq[(int64_t)out * a.F + r] = (int8_t)q;
            if ((pi & 31) == 0) a.hd[(int64_t)out * (a.F / QK) + r / QK] = d;
          } else {
            a.ypair[(int64_t)out * a.H + r] = s0 * (obuf[0][pt][pi] * Fmt<WB>::INV);
          }
        }
        lds_barrier();
      };
      int tc = 0;
      for (; tc + 2 <= n; tc += 2) pass(std::integral_constant<int, 2>{}, tc);
      if (tc < n) pass(std::integral_constant<int, 1>{}, tc);
    }
    if (!has_next) break;
    cur = nxt;
    nxt += G;
    ec = en;
    r0c = r0n;
    buf ^= 1;
    s0 = s0n;
    s1 = s1n;
  }
}

// dynamic LDS of a gate/up launch that selects the route itself: fused_route's, and
// (with_route) the route of the batch
static size_t fused_lds_bytes(const FfnArgs &a, bool with_route) {
  if (a.sel.part == nullptr) return 0;
  return fused_route_lds(a.T, a.E) + (with_route ? (size_t)a.T * a.k * sizeof(int) : 0);
}

// resident workgroups of a kernel on the current device (cached per device)
template <typename Kern>
static int resident_groups(Kern k, int threads) {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k, threads, 0) != hipSuccess) return 0;
  const int g = (per > 0 ? per : 1) * cus;
  if (dev < 64) cache[dev] = g;
  return g;
}

template <int WB, int LPR, int MODE, bool GS>
static hipError_t launch_pipe(const FfnArgs &a, int nrows, hipStream_t s) {
  constexpr int WRMAX = 64 * (WAVE / LPR) / (Fmt<WB>::CHUNK / 4);
  // rows per wavefront: 8, or 16 for down rows of at most 32 lanes (a row of 64 lanes is
  // 16 KB of loads per wavefront at 16 rows; 8 measured faster there: GLM-scale down at
  // T = 16 104.8 -> 102.9 us, T = 1 14.9 -> 13.3 us, while OLMoE-scale down, 32 lanes
  // per row, lost 1.7 us at 8)
  constexpr int WR = (MODE == MODE_DOWN && LPR < 64) ? (WRMAX < 16 ? WRMAX : 16) : 8;
  constexpr int TILE = 4 * WR;
  if (nrows % TILE) return hipErrorNotSupported;
  auto kern = gemv_pipe_kernel<WB, LPR, MODE, WR, GS>;
  const int res = resident_groups(kern, 256);
  if (res <= 0) return hipErrorNotSupported;
  const int64_t units = (int64_t)(a.has_shared + min(a.E, a.T * a.k)) * (nrows / TILE);
  const int grid = (int)(units < res ? units : res);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), fused_lds_bytes(a, false), s, a);
  return hipGetLastError();
}

template <int WB, int LPR, int MODE>
static hipError_t launch_reg(const FfnArgs &a, int nrows, int slots, hipStream_t s) {
  // rows per wavefront: gate/up 8 (two matrices, 32-row tiles = one Q8_0 block of h),
  // down 16 (64-row tiles; measured best for both 32 and 64 lanes per row)
  constexpr int WRMAX = 64 * (WAVE / LPR) / (Fmt<WB>::CHUNK / 4);  // 64 registers of weights
  constexpr int WR = (MODE == MODE_DOWN) ? (WRMAX < 16 ? WRMAX : 16) : 8;
  constexpr int TILE = 4 * WR;
  if (nrows % TILE) return hipErrorNotSupported;
  // token passes: two tokens when the experts average two or more (gate/up), else one
  // (fewer accumulators, one more wave per SIMD; measured faster for down and for
  // small batches)
  const bool dense = (int64_t)a.T * a.k >= 2 * (int64_t)a.E;  // most experts hit (about 86% or more)
  const dim3 grid(nrows / TILE, slots);
  const size_t lds = fused_lds_bytes(a, true);
  if (MODE == MODE_GATEUP && dense)
    hipLaunchKernelGGL((gemv_reg_kernel<WB, LPR, MODE, WR, 2>), grid, dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL((gemv_reg_kernel<WB, LPR, MODE, WR, 1>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

// lanes per row: largest power of two <= 64 dividing the chunks per row
static int pick_lpr(int nchunk) {
  int l = 64;
  while (l > 1 && nchunk % l) l >>= 1;
  return l;
}

template <int WB, int LPR, int CPL, int MODE, bool GS>
static hipError_t launch_fast(const FfnArgs &a, dim3 slots_grid, int nrows, int K, hipStream_t s) {
  constexpr int WR = (MODE == MODE_DOWN && LPR < 64) ? 16 : 8;
  constexpr int TILE = 4 * WR;
  constexpr int NMAT = (MODE == MODE_GATEUP) ? 2 : 1;
  if (nrows % TILE) return hipErrorNotSupported;
  // two tokens per pass: the accumulators of larger passes cost occupancy (2 -> 3 waves
  // per SIMD for the int4 gate/up instantiation), which matters more than reloading a
  // tile's weights from L2 for the rare expert with more than two tokens
  const int ntmax = min(2, a.T);
  const size_t lds = std::max((size_t)ntmax * K + (size_t)ntmax * (K / QK) * sizeof(float) +
                                  (size_t)NMAT * 8 * TILE * sizeof(float) + 16 * sizeof(int),
                              fused_lds_bytes(a, true));
  dim3 grid(nrows / TILE, slots_grid.y);
  if constexpr (FastPl<WB, CPL, MODE, GS>::one) {
    if (a.T == 1) {
      hipLaunchKernelGGL((gemv_fast_kernel<WB, LPR, CPL, MODE, WR, GS, true>), grid, dim3(256), lds, s, a, ntmax);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemv_fast_kernel<WB, LPR, CPL, MODE, WR, GS>), grid, dim3(256), lds, s, a, ntmax);
  return hipGetLastError();
}

template <int WB, int MODE, bool GS>
static hipError_t launch_mode(const FfnArgs &a, hipStream_t s) {
  const int K = (MODE == MODE_GATEUP) ? a.H : a.F;
  const int NROWS = (MODE == MODE_GATEUP) ? a.F : a.H;
  const int nkb = K / QK;
  const int nchunk = nkb / Fmt<WB>::BPC;
  const int lpr = pick_lpr(nchunk);
  const int cpl = nchunk / lpr;
  const int slots = a.has_shared + min(a.E, a.T * a.k);
  // one chunk per lane and row, and the tile fits in registers: weights stay resident
  constexpr int NMATC = (MODE == MODE_GATEUP) ? 2 : 1;
  if constexpr (WB != 2 && (Fmt<WB>::CHUNK / 4) * NMATC * 8 <= 64) {
    if (cpl == 1 && (lpr == 64 || lpr == 32)) {
      hipError_t r = hipErrorNotSupported;
      if (a.idx != nullptr)
        r = (lpr == 64) ? launch_pipe<WB, 64, MODE, GS>(a, NROWS, s) : launch_pipe<WB, 32, MODE, GS>(a, NROWS, s);
      // the register-resident kernel keeps one scale per row
      if constexpr (!GS)
        if (r == hipErrorNotSupported)
          r = (lpr == 64) ? launch_reg<WB, 64, MODE>(a, NROWS, slots, s) : launch_reg<WB, 32, MODE>(a, NROWS, slots, s);
      if (r != hipErrorNotSupported) return r;
    }
  }
  // the batched kernel for the shapes it is instantiated for
  if (lpr == 64 || lpr == 32) {
    hipError_t r = hipErrorNotSupported;
    const dim3 sg(1, slots);
    if (lpr == 64 && cpl == 1) r = launch_fast<WB, 64, 1, MODE, GS>(a, sg, NROWS, K, s);
    else if (lpr == 64 && cpl == 2) r = launch_fast<WB, 64, 2, MODE, GS>(a, sg, NROWS, K, s);
    else if (lpr == 64 && cpl == 3) r = launch_fast<WB, 64, 3, MODE, GS>(a, sg, NROWS, K, s);
    else if (lpr == 32 && cpl == 1) r = launch_fast<WB, 32, 1, MODE, GS>(a, sg, NROWS, K, s);
    else if (lpr == 32 && cpl == 3) r = launch_fast<WB, 32, 3, MODE, GS>(a, sg, NROWS, K, s);
    if (r != hipErrorNotSupported) return r;
  }
  dim3 grid(NROWS / GEMV_ROWS, slots);
  const size_t lds = std::max((size_t)GEMV_NT * K + (size_t)GEMV_NT * nkb * sizeof(float) +
                                  (size_t)GEMV_NT * GEMV_ROWS * sizeof(float) + 2 * GEMV_NT * sizeof(int),
                              fused_lds_bytes(a, true));
  switch (lpr) {
#define COLI_LPR_CASE(L) \
  case L: hipLaunchKernelGGL((gemv_kernel<WB, L, MODE, GS>), grid, dim3(256), lds, s, a); break;
    COLI_LPR_CASE(64)
    COLI_LPR_CASE(32)
    COLI_LPR_CASE(16)
    COLI_LPR_CASE(8)
    COLI_LPR_CASE(4)
    COLI_LPR_CASE(2)
    COLI_LPR_CASE(1)
#undef COLI_LPR_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace coli
