// ffn_mfma.hip — expert FFNs of large batches (prefill, long verify) as grouped
// GEMMs on the int8 matrix cores of gfx950 (v_mfma_i32_32x32x32_i8).
//
// Batch-union (colibri-strix README, "What's implemented", batch-union item): each
// expert of the union is one GEMM of its weight rows against the Q8_0 rows of the
// tokens routed to it, the weights dequantised on use (same section, quantization
// kernels item) and multiplied with integer dots (integer-dot kernels item).
//
// One MFMA of 32 x 32 x 32 covers exactly one Q8_0 block along K, so its int32
// results are the exact block dots I_b of 32 weight rows x 32 tokens. Each lane's
// outputs belong to one token (the MFMA column), so scaling by that token's block
// scale is one fp32 multiply-add per result: acc += d_b * I_b. The K order inside
// a block is free (the block is reduced whole), which is what makes the packed
// layouts cheap to feed: lanes 0-31 take the first 16 values of a block, lanes
// 32-63 the last 16, i.e. the low resp. high nibbles of an int4 block.
//
// Work: a workgroup (4 wavefronts) owns 64 weight rows x 32 tokens of one expert;
// wavefront (wm, wk) computes rows 32 wm .. 32 wm + 31 for all 32 tokens over the
// blocks kb = wk mod 2 of every K stage (gate and up together in the gate/up
// pass); the two K halves are added through LDS at the end. 32-token tiles keep
// the padding of each expert's last tile small (the union's token counts are
// uneven). Token tiles of the union are listed by plan_kernel; the 1-D grid is
// remapped so that the token tiles of one (expert, row tile) land on one XCD in
// consecutive order and share its L2 copy of the weight rows.
#include "coli_internal.h"

namespace coli {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int MF_ROWS = 64;  // weight rows per workgroup
constexpr int MF_TOK = 32;   // tokens per workgroup (one token tile)
constexpr int MF_KC = 4;     // Q8_0 blocks per K stage staged through LDS

// ------------------------------------------------------------------ plan
// Token tiles of the union, in slot order (shared expert first, then the experts of
// `active`): tiles[g] = {expert, first perm index (-1: shared expert), tokens of the
// expert, tile index}. *ntiles = number of tiles.
__global__ __launch_bounds__(1024) void plan_kernel(FfnArgs a, int4 *__restrict__ tiles, int32_t *__restrict__ ntiles,
                                                    int gmax) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hs = a.has_shared;
  const int na = max(0, min(*a.nact, a.E));
  const int ns = hs + na;
  // two slots per thread: u0 = 2 * tid, u0 + 1
  int e[2], beg[2], n[2], nt[2];
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const int u = 2 * tid + q;
    e[q] = 0;
    beg[q] = 0;
    n[q] = 0;
    if (u < ns) {
      if (hs && u == 0) {
        e[q] = a.E;
        beg[q] = -1;
        n[q] = a.T;
      } else {
        const int ex = a.active[u - hs];
        e[q] = ex;
        beg[q] = a.off[ex];
        n[q] = a.off[ex + 1] - beg[q];
      }
    }
    nt[q] = (n[q] + MF_TOK - 1) / MF_TOK;
  }
  const int mine = nt[0] + nt[1];
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int i = 0; i < 16; i++) {
    if (i < wv) base += wsum[i];
    total += wsum[i];
  }
  int g = base + incl - mine;
#pragma unroll
  for (int q = 0; q < 2; q++)
    for (int t = 0; t < nt[q]; t++, g++)
      if (g < gmax) tiles[g] = make_int4(e[q], beg[q], n[q], t);
  if (tid == 0) *ntiles = min(total, gmax);
}

// ------------------------------------------------------------------ staging
// Packed weights enter the MFMA as int8 with the field in the top bits of its
// byte: an int4 field w becomes the byte 16 w, an int2 field 64 w (two's
// complement keeps the sign). One AND (and a shift) per four values, and the block
// dots come out as exact multiples SCALE * I_b; the accumulated sums are divided
// by SCALE at the end, exactly (a power of two).
// MXFP4 codes go through a byte table instead: the byte holds 2 * e2m1 (SCALE 2).
template <int WB>
struct Top {
  static constexpr int scale = (WB == 4) ? 16 : (WB == 2) ? 64 : (WB == W_MX) ? 2 : 1;
  static constexpr int block_bytes = (WB == W_MX) ? 16 : QK * WB / 8;  // packed bytes per block
};


// LDS tiles of one K stage of KC blocks, int8 in natural K order; rows padded by
// 16 bytes against bank conflicts.
template <int NMAT, int KC, int G>
struct MfLds {
  static constexpr int ROWB = KC * QK + 16;  // bytes per row (and per token)
  int8_t a[2][NMAT][MF_ROWS][ROWB];
  int8_t b[2][MF_TOK][ROWB];
  float d[2][MF_TOK][KC];  // block scale of each token
  __attribute__((aligned(16))) float gs[2][NMAT][KC * QK / G][MF_ROWS];  // group scales of the stage's rows
};

enum { MF_GATEUP = 0, MF_DOWN = 1 };

// Global -> register part of one stage: the lane's share of the packed weight
// rows, of the token rows and of the block scales.
template <int WB, int NMAT, int KC>
struct MfRegs {
  // weight bytes per (matrix, row) and stage: KC blocks; 16-byte pieces per row
  static constexpr int APIECES = KC * Top<WB>::block_bytes / 16;
  static constexpr int ATOTAL = NMAT * MF_ROWS * APIECES;
  static constexpr int ALOADS = (ATOTAL + 255) / 256;  // per thread (the last may be partial)
  static constexpr int BLOADS = (MF_TOK * KC * QK / 16 + 255) / 256;
  uint4 a[ALOADS];
  uint4 b[BLOADS];
  float d;
  float gs;      // group scale (fp32 formats)
  uint32_t gsx;  // MXFP4: the stage's KC = 4 E8M0 bytes of one row
};

// ------------------------------------------------------------------ GEMM
// GS: one scale per 64 inputs of a row (group scales): each block's scale is then
// d_b * s(row, group of b), applied per result; otherwise one scale per row, applied
// in the epilogue.
template <int WB, int MODE, int KC, bool GS>
__global__ __launch_bounds__(256, 2) void mfma_kernel(FfnArgs a, const int4 *__restrict__ tiles,
                                                   const int32_t *__restrict__ ntiles, int gmax, int nf) {
  constexpr int NMAT = (MODE == MF_GATEUP) ? 2 : 1;
  using Lds = MfLds<NMAT, KC, GSZ<WB>>;
  using Regs = MfRegs<WB, NMAT, KC>;
  constexpr int ROWB = Lds::ROWB;
  constexpr int APIECES = Regs::APIECES;
  constexpr int ATOTAL = Regs::ATOTAL;
  static_assert(ATOTAL % 64 == 0, "weight pieces: whole wavefronts");
  static_assert(MF_TOK * KC * 2 == 256, "one 16-byte token piece per thread and stage");
  static_assert(MF_TOK * KC <= 256, "at most one block scale per thread and stage");
  static_assert(KC % 2 == 0, "the two K halves take alternate blocks");
  __shared__ Lds L;
  __shared__ int act_rows[MF_TOK];

  // XCD-aware order: hardware workgroup i runs on XCD i % 8; give each XCD one
  // contiguous range of work (token tiles fastest), so the tiles of one (expert,
  // row tile) run on one XCD one after the other and share its L2
  const int nwork = nf * gmax;  // a multiple of 8
  const int bid = blockIdx.x;
  const int w = (bid & 7) * (nwork >> 3) + (bid >> 3);
  const int ft = w / gmax, g = w % gmax;
  if (g >= *ntiles) return;
  const int4 ti = tiles[g];  // expert, first perm index (-1: shared), tokens, tile

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wv & 1, wk = wv >> 1;
  const int grp = lane >> 5, li = lane & 31;
  const int K = (MODE == MF_GATEUP) ? a.H : a.F;
  const int nkb = K / QK;
  const int P = a.T * a.k;
  const int64_t rb = row_bytes(WB, K);
  const int64_t rbh = row_bytes(WB, a.H);
  const uint8_t *blob = a.experts + (int64_t)ti.x * a.blob_bytes;
  const uint8_t *mat0 = (MODE == MF_GATEUP) ? blob : blob + 2 * (int64_t)a.F * rbh;
  const uint8_t *mat1 = blob + (int64_t)a.F * rbh;
  const int r0 = ft * MF_ROWS;

  // token rows of the tile: activation row and output row; past the expert's
  // tokens the tile repeats its first token and writes nothing
  if (tid < MF_TOK) {
    const int i = ti.w * MF_TOK + tid;
    const int ic = i < ti.z ? i : ti.w * MF_TOK;
    int act;
    if (ti.y < 0) act = (MODE == MF_GATEUP) ? ic : P + ic;
    else {
      const int p = a.perm[ti.y + ic];
      act = (MODE == MF_GATEUP) ? p / a.k : p;
    }
    act_rows[tid] = act;
  }
  __syncthreads();
  const int8_t *asrc = (MODE == MF_GATEUP) ? a.xq : a.hq;
  const float *dsrc = (MODE == MF_GATEUP) ? a.xd : a.hd;
  // this thread's token pieces: piece q -> token q / (2 KC), 16-byte part q % (2 KC)
  int64_t boff[Regs::BLOADS];
#pragma unroll
  for (int j = 0; j < Regs::BLOADS; j++) {
    const int q = tid + 256 * j;
    boff[j] = (int64_t)act_rows[q / (2 * KC)] * K + (q % (2 * KC)) * 16;
  }
  const bool dthread = tid < MF_TOK * KC;
  const int64_t doff = (int64_t)act_rows[dthread ? tid / KC : 0] * nkb + tid % KC;
  // group scales of a stage: NMAT x NG groups x 64 rows. fp32 (groups of 64): one per
  // thread, thread q -> matrix q / (NG * 64), group (q / 64) % NG, row q % 64.
  // MXFP4 (groups of 32): the row's KC = 4 E8M0 bytes as one 32-bit load per thread,
  // thread q -> matrix q / 64, row q % 64 (K / 32 is a multiple of 4: aligned).
  constexpr int G = GSZ<WB>;
  constexpr int NG = KC * QK / G;
  constexpr bool MXS = WB == W_MX;
  static_assert(!MXS || KC == 4, "one 32-bit load holds a stage's four E8M0 bytes");
  const bool gthread = GS && tid < NMAT * (MXS ? 1 : NG) * MF_ROWS;
  const void *gsrc = nullptr;
  if constexpr (GS) {
    const int sc_m = tid / ((MXS ? 1 : NG) * MF_ROWS), sc_row = r0 + tid % MF_ROWS;
    const int64_t ngh = (int64_t)a.F * (a.H / G);
    const int64_t se = (int64_t)ti.x * a.scale_stride + ((MODE == MF_GATEUP) ? (sc_m == 1 ? ngh : 0) : 2 * ngh);
    gsrc = gs_base<WB>(a.scales, se + (int64_t)sc_row * (K / G) + (MXS ? 0 : (tid / MF_ROWS) % NG));
  }

  auto gload = [&](int s, Regs &r) {
    const int kb0 = s * KC;  // first block of the stage
#pragma unroll
    for (int j = 0; j < Regs::ALOADS; j++) {
      const int q = tid + 256 * j;
      if (ATOTAL % 256 != 0 && q >= ATOTAL) break;
      const int m = q / (MF_ROWS * APIECES), row = (q / APIECES) % MF_ROWS, pc = q % APIECES;
      const uint8_t *base = (NMAT == 2 && m == 1) ? mat1 : mat0;
      r.a[j] = *reinterpret_cast<const uint4 *>(base + (int64_t)(r0 + row) * rb + (int64_t)kb0 * Top<WB>::block_bytes +
                                                pc * 16);
    }
#pragma unroll
    for (int j = 0; j < Regs::BLOADS; j++)
      r.b[j] = *reinterpret_cast<const uint4 *>(asrc + boff[j] + (int64_t)kb0 * QK);
    if (dthread) r.d = dsrc[doff + kb0];
    if constexpr (MXS) {
      if (gthread) r.gsx = *reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(gsrc) + s * KC);
    } else {
      if (gthread) r.gs = gs_load<WB>(gsrc, s * NG);
    }
  };

  auto lstore = [&](int buf, const Regs &r) {
#pragma unroll
    for (int j = 0; j < Regs::ALOADS; j++) {
      const int q = tid + 256 * j;
      if (ATOTAL % 256 != 0 && q >= ATOTAL) break;
      const int m = q / (MF_ROWS * APIECES), row = (q / APIECES) % MF_ROWS, pc = q % APIECES;
      int8_t *dst = &L.a[buf][m][row][0];
      const uint4 v = r.a[j];
      if constexpr (WB == 8) {
        *reinterpret_cast<uint4 *>(dst + pc * 16) = v;
      } else if constexpr (WB == W_MX) {
        // one block of 32 codes: 0..15 in the low nibbles, 16..31 in the high ones
        uint4 lo, hi;
        lo.x = e2m1x4_to_i8x4(v.x);
        lo.y = e2m1x4_to_i8x4(v.y);
        lo.z = e2m1x4_to_i8x4(v.z);
        lo.w = e2m1x4_to_i8x4(v.w);
        hi.x = e2m1x4_to_i8x4(v.x >> 4);
        hi.y = e2m1x4_to_i8x4(v.y >> 4);
        hi.z = e2m1x4_to_i8x4(v.z >> 4);
        hi.w = e2m1x4_to_i8x4(v.w >> 4);
        *reinterpret_cast<uint4 *>(dst + pc * 32) = lo;
        *reinterpret_cast<uint4 *>(dst + pc * 32 + 16) = hi;
      } else if constexpr (WB == 4) {
        // one 16-byte block: values 0..15 in the low nibbles, 16..31 in the high ones
        uint4 lo, hi;
        lo.x = (v.x << 4) & 0xF0F0F0F0u;
        lo.y = (v.y << 4) & 0xF0F0F0F0u;
        lo.z = (v.z << 4) & 0xF0F0F0F0u;
        lo.w = (v.w << 4) & 0xF0F0F0F0u;
        hi.x = v.x & 0xF0F0F0F0u;
        hi.y = v.y & 0xF0F0F0F0u;
        hi.z = v.z & 0xF0F0F0F0u;
        hi.w = v.w & 0xF0F0F0F0u;
        *reinterpret_cast<uint4 *>(dst + pc * 32) = lo;
        *reinterpret_cast<uint4 *>(dst + pc * 32 + 16) = hi;
      } else {
        // two 8-byte blocks; byte j holds values j + 8m in bits 2m (m = 0..3)
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const uint32_t w0 = h ? v.z : v.x, w1 = h ? v.w : v.y;
          uint4 o0, o1;
          o0.x = (w0 << 6) & 0xC0C0C0C0u;
          o0.y = (w1 << 6) & 0xC0C0C0C0u;
          o0.z = (w0 << 4) & 0xC0C0C0C0u;
          o0.w = (w1 << 4) & 0xC0C0C0C0u;
          o1.x = (w0 << 2) & 0xC0C0C0C0u;
          o1.y = (w1 << 2) & 0xC0C0C0C0u;
          o1.z = w0 & 0xC0C0C0C0u;
          o1.w = w1 & 0xC0C0C0C0u;
          *reinterpret_cast<uint4 *>(dst + pc * 64 + h * 32) = o0;
          *reinterpret_cast<uint4 *>(dst + pc * 64 + h * 32 + 16) = o1;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < Regs::BLOADS; j++) {
      const int q = tid + 256 * j;
      *reinterpret_cast<uint4 *>(&L.b[buf][q / (2 * KC)][(q % (2 * KC)) * 16]) = r.b[j];
    }
    if (dthread) L.d[buf][tid / KC][tid % KC] = r.d;
    if constexpr (MXS) {
      if (gthread) {
#pragma unroll
        for (int kb = 0; kb < KC; kb++) L.gs[buf][tid / MF_ROWS][kb][tid % MF_ROWS] = e8m0_f32((r.gsx >> (8 * kb)) & 0xFFu);
      }
    } else {
      if (gthread) L.gs[buf][tid / (NG * MF_ROWS)][(tid / MF_ROWS) % NG][tid % MF_ROWS] = r.gs;
    }
  };

  float acc[NMAT][16];
#pragma unroll
  for (int m = 0; m < NMAT; m++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[m][r] = 0.0f;

  // one stage from LDS: per block, an exact int32 block dot by MFMA, then the scale
  auto compute = [&](int buf) {
    const int8_t *arow0 = &L.a[buf][0][wm * 32 + li][16 * grp];
    const int8_t *brow = &L.b[buf][li][16 * grp];
    for (int kb = wk; kb < KC; kb += 2) {
      const v4i bv = *reinterpret_cast<const v4i *>(brow + kb * QK);
      const float d = L.d[buf][li][kb];
#pragma unroll
      for (int m = 0; m < NMAT; m++) {
        const v4i av = *reinterpret_cast<const v4i *>(arow0 + m * (MF_ROWS * ROWB) + kb * QK);
        const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        const v16i I = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, zero, 0, 0, 0);
        if constexpr (GS) {
          // rows wm * 32 + 8 q + 4 grp + (0..3) of the tile: four float4 reads
          const float *gr = &L.gs[buf][m][kb * QK / G][wm * 32 + 4 * grp];
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const float4 g4 = *reinterpret_cast<const float4 *>(gr + 8 * q);
            acc[m][4 * q] = fmaf(d * g4.x, (float)I[4 * q], acc[m][4 * q]);
            acc[m][4 * q + 1] = fmaf(d * g4.y, (float)I[4 * q + 1], acc[m][4 * q + 1]);
            acc[m][4 * q + 2] = fmaf(d * g4.z, (float)I[4 * q + 2], acc[m][4 * q + 2]);
            acc[m][4 * q + 3] = fmaf(d * g4.w, (float)I[4 * q + 3], acc[m][4 * q + 3]);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; r++) acc[m][r] += d * (float)I[r];
        }
      }
    }
  };

  // stage s: the next stage's global loads go out before this stage's compute and
  // land in the other LDS buffer afterwards (one barrier per stage)
  const int ns = nkb / KC;
  {
    Regs r;
    gload(0, r);
    lstore(0, r);
  }
  __syncthreads();
  for (int s = 0; s < ns; s++) {
    Regs r;
    const bool more = s + 1 < ns;
    if (more) gload(s + 1, r);
    compute(s & 1);
    if (more) lstore((s + 1) & 1, r);
    __syncthreads();
  }
  if constexpr (Top<WB>::scale != 1) {
    constexpr float inv = 1.0f / Top<WB>::scale;
#pragma unroll
    for (int m = 0; m < NMAT; m++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[m][r] *= inv;
  }

  // add the K half of wavefronts wk = 1 to that of wk = 0 (the stage buffers are free)
  float *red = reinterpret_cast<float *>(&L.a[0][0][0][0]);
  static_assert(sizeof(L.a) >= 2 * 64 * NMAT * 16 * sizeof(float), "reduction buffer");
  if (wk == 1) {
#pragma unroll
    for (int m = 0; m < NMAT; m++)
#pragma unroll
      for (int r = 0; r < 16; r++) red[((wm * NMAT + m) * 16 + r) * 64 + lane] = acc[m][r];
  }
  __syncthreads();
  if (wk == 1) return;
#pragma unroll
  for (int m = 0; m < NMAT; m++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[m][r] += red[((wm * NMAT + m) * 16 + r) * 64 + lane];

  // epilogue. Result r of this lane: row r0 + 32 wm + 8 (r / 4) + 4 grp + r % 4,
  // token li of the tile.
  const int i = ti.w * MF_TOK + li;
  const bool valid = i < ti.z;
  int out_row = 0;
  if (valid) out_row = (ti.y < 0) ? P + i : a.perm[ti.y + i];
  const int rbase = r0 + wm * 32;
  const float *sc = a.scales + (int64_t)ti.x * a.scale_stride;
  if constexpr (MODE == MF_GATEUP) {
    float h[16];
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int f = rbase + 8 * (r >> 2) + 4 * grp + (r & 3);
      const float gv = (GS ? 1.0f : sc[f]) * acc[0][r];
      const float uv = (GS ? 1.0f : sc[a.F + f]) * acc[1][r];
      if (valid) COLI_TAP_GU(a, out_row, f, gv, uv);
      h[r] = (gv / (1.0f + expf(-gv))) * uv;
      amax = fmaxf(amax, fabsf(h[r]));
    }
    // the 32 rows of this Q8_0 block of h sit in lanes li and li + 32
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float d = amax / 127.0f;
    uint32_t packed[4];
#pragma unroll
    for (int rr = 0; rr < 4; rr++) {
      uint32_t pk = 0;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        int q = 0;
        if (d != 0.0f) q = (int)fminf(fmaxf(roundf(h[4 * rr + j] / d), -127.0f), 127.0f);
        pk |= (uint32_t)(q & 0xFF) << (8 * j);
      }
      packed[rr] = pk;
    }
    if (valid) {
      int8_t *hrow = a.hq + (int64_t)out_row * a.F + rbase + 4 * grp;
#pragma unroll
      for (int rr = 0; rr < 4; rr++) *reinterpret_cast<uint32_t *>(hrow + 8 * rr) = packed[rr];
      if (grp == 0) a.hd[(int64_t)out_row * (a.F / QK) + rbase / QK] = d;
    }
  } else {
    if (valid) {
      const float *sd = sc + 2 * a.F;
      float *yrow = a.ypair + (int64_t)out_row * a.H + rbase + 4 * grp;
#pragma unroll
      for (int rr = 0; rr < 4; rr++) {
        const int f = rbase + 8 * rr + 4 * grp;
        float4 v;
        v.x = (GS ? 1.0f : sd[f]) * acc[0][4 * rr];
        v.y = (GS ? 1.0f : sd[f + 1]) * acc[0][4 * rr + 1];
        v.z = (GS ? 1.0f : sd[f + 2]) * acc[0][4 * rr + 2];
        v.w = (GS ? 1.0f : sd[f + 3]) * acc[0][4 * rr + 3];
        *reinterpret_cast<float4 *>(yrow + 8 * rr) = v;
      }
    }
  }
}

// ------------------------------------------------------------------ host side
int32_t mfma_gmax(int32_t T, int32_t k, int32_t E, int32_t has_shared) {
  const int64_t rows = (int64_t)T * k + (int64_t)has_shared * T;
  const int64_t g = (rows + MF_TOK - 1) / MF_TOK + E + has_shared;
  return (int32_t)((g + 7) / 8 * 8);
}

hipError_t launch_plan(const FfnArgs &a, int4 *tiles, int32_t *ntiles, int32_t gmax, hipStream_t s) {
  if (a.E + a.has_shared > 2048) return hipErrorInvalidValue;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, a, tiles, ntiles, gmax);
  return hipGetLastError();
}

template <int WB, int MODE>
static hipError_t launch_mf(const FfnArgs &a, const int4 *tiles, const int32_t *ntiles, int32_t gmax, hipStream_t s) {
  const int rows = (MODE == MF_GATEUP) ? a.F : a.H;
  const int K = (MODE == MF_GATEUP) ? a.H : a.F;
  if (rows % MF_ROWS || K % (MF_KC * QK) || gmax % 8) return hipErrorInvalidValue;
  // MXFP4 always has its E8M0 scale per 32 inputs; the integer formats one per row or per 64
  if (WB == W_MX ? a.gs != 32 : (a.gs != 0 && a.gs != 64)) return hipErrorInvalidValue;
  const int nf = rows / MF_ROWS;
  const int64_t nwork = (int64_t)nf * gmax;
  if (nwork > 0x7fffffff) return hipErrorInvalidValue;
  if (WB == W_MX || a.gs)  // MXFP4 always takes the group-scale path (a.gs == 32 checked above)
    hipLaunchKernelGGL((mfma_kernel<WB, MODE, MF_KC, true>), dim3((unsigned)nwork), dim3(256), 0, s, a, tiles, ntiles,
                       gmax, nf);
  else if constexpr (WB != W_MX)
    hipLaunchKernelGGL((mfma_kernel<WB, MODE, MF_KC, false>), dim3((unsigned)nwork), dim3(256), 0, s, a, tiles, ntiles,
                       gmax, nf);
  return hipGetLastError();
}

hipError_t launch_mfma_gateup(int wfmt, const FfnArgs &a, const int4 *tiles, const int32_t *ntiles, int32_t gmax,
                              hipStream_t s) {
  switch (wfmt) {
    case 4: return launch_mf<4, MF_GATEUP>(a, tiles, ntiles, gmax, s);
    case 8: return launch_mf<8, MF_GATEUP>(a, tiles, ntiles, gmax, s);
    case 2: return launch_mf<2, MF_GATEUP>(a, tiles, ntiles, gmax, s);
    case W_MX: return launch_mf<W_MX, MF_GATEUP>(a, tiles, ntiles, gmax, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mfma_down(int wfmt, const FfnArgs &a, const int4 *tiles, const int32_t *ntiles, int32_t gmax,
                            hipStream_t s) {
  switch (wfmt) {
    case 4: return launch_mf<4, MF_DOWN>(a, tiles, ntiles, gmax, s);
    case 8: return launch_mf<8, MF_DOWN>(a, tiles, ntiles, gmax, s);
    case 2: return launch_mf<2, MF_DOWN>(a, tiles, ntiles, gmax, s);
    case W_MX: return launch_mf<W_MX, MF_DOWN>(a, tiles, ntiles, gmax, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace coli
