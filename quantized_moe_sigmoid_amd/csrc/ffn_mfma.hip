// ffn_mfma.hip — expert FFNs of large batches (prefill, long verify) as grouped
// GEMMs on the int8 matrix cores of gfx950 (v_mfma_i32_32x32x32_i8); MXFP4 weights on
// the fp16 matrix cores instead (mfma_mx_kernel, further down).
//
// Batch-union (colibri-strix README, "What's implemented", batch-union item): each
// expert of the union is one GEMM of its weight rows against the Q8_0 rows of the
// tokens routed to it, the weights dequantised on use (same section, quantization
// kernels item) and multiplied with integer dots (integer-dot kernels item).
//
// One MFMA of 32 x 32 x 32 covers exactly one Q8_0 block along K, so its int32
// results are the exact block dots I_b of 32 weight rows x 32 tokens. Each lane's
// outputs belong to one token (the MFMA column), so scaling by that token's block
// scale is one fp32 multiply-add per result: acc += d_b * I_b.
//
// Work: a workgroup (4 wavefronts) owns 128 weight rows of one expert (32 per
// wavefront; gate and up rows together in the gate/up pass) and a chunk of up to
// 64 of the expert's tokens (two 32-token tiles). The weights are the stream that
// matters (the union's experts are read once per token chunk; most experts have one
// chunk), the tokens' Q8_0 rows are small and shared by every row tile:
//   - weights go from global memory straight into the MFMA's A registers. A lane
//     loads 16 packed bytes of its row; the two halves of the wavefront load
//     neighbouring blocks, and one v_permlane32_swap per register hands each half
//     the part of both blocks it needs (the MFMA takes K values 0-15 of a block in
//     lanes 0-31 and 16-31 in lanes 32-63: for int4 that is the low resp. high
//     nibbles of the same 16 bytes). Each A register then feeds one MFMA per
//     token tile;
//   - the tokens' Q8_0 rows of a stage of four blocks are staged in LDS (double
//     buffered, rows padded against bank conflicts) and read as B operands.
// Token chunks are listed by plan_kernel; the 1-D grid is remapped so that each XCD
// takes one contiguous range of (row tile, chunk) work, chunks fastest: the chunks
// of one heavy expert and row tile run on one XCD side by side and share its L2
// copy of the weight rows. mfma_item is the work of one (row tile, chunk) item;
// mfma_kernel runs one item per workgroup.
#include <type_traits>

#include "coli_internal.h"

namespace coli {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Tiles per workgroup: two (a chunk of 64 tokens) keeps the gate/up kernel at 167
// registers, three wavefronts per SIMD; four tiles (128 tokens, weights re-read half
// as often) need 243 and leave two, which measured slower: the kernel is bound by
// the per-result scaling on the vector ALUs, and a third wavefront hides the MFMA ->
// VALU latency of the other two.
constexpr int GM_ROWS = 128;              // weight rows per workgroup (4 wavefronts x 32)
constexpr int GM_TILES = 2;               // 32-token tiles per workgroup
constexpr int GM_TOK = 32 * GM_TILES;     // tokens per chunk
constexpr int GM_KB = 4;                  // Q8_0 blocks per K stage
constexpr int GM_XROW = GM_KB * QK + 16;  // LDS bytes per token row of a stage (16 of padding)

// ------------------------------------------------------------------ plan
// Token chunks of the union, in slot order (shared expert first, then the experts of
// `active`): chunks[g] = {expert, first perm index of the expert (-1: shared expert),
// tokens in the chunk (1..GM_TOK), index of the chunk's first token within the
// expert}. *nchunks = number of chunks.
__global__ __launch_bounds__(1024) void plan_kernel(FfnArgs a, int4 *__restrict__ chunks, int32_t *__restrict__ nchunks,
                                                    int gmax) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hs = a.has_shared;
  const int na = max(0, min(*a.nact, a.E));
  const int ns = hs + na;
  // two slots per thread: u0 = 2 * tid, u0 + 1
  int e[2], beg[2], n[2], nc[2];
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
    nc[q] = (n[q] + GM_TOK - 1) / GM_TOK;
  }
  const int mine = nc[0] + nc[1];
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
    for (int c = 0; c < nc[q]; c++, g++)
      if (g < gmax) chunks[g] = make_int4(e[q], beg[q], min(GM_TOK, n[q] - c * GM_TOK), c * GM_TOK);
  if (tid == 0) *nchunks = min(total, gmax);
}

// ------------------------------------------------------------------ weights -> A
// Packed weights enter the MFMA as int8 with the field in the top bits of its
// byte: an int4 field w becomes the byte 16 w, an int2 field 64 w (two's
// complement keeps the sign). One AND (and a shift) per four values, and the block
// dots come out as exact multiples SCALE * I_b; the sums are divided by SCALE in
// the epilogue, exactly (a power of two). MXFP4 codes go through a byte table
// instead: the byte holds 2 * e2m1 (SCALE 2).
template <int WB>
struct Top {
  static constexpr int scale = (WB == 4) ? 16 : (WB == 2) ? 64 : (WB == W_MX) ? 2 : 1;
  static constexpr int block_bytes = (WB == W_MX) ? 16 : QK * WB / 8;  // packed bytes per block
  // 16-byte loads per lane, matrix and stage of GM_KB blocks (32 rows per wavefront)
  static constexpr int loads = GM_KB * block_bytes * 32 / (64 * 16);
};

// Lane (row r, half h) of a wavefront, stage s: the 16-byte pieces of its row.
//   int8:  load j = block 4s + j, bytes 16h .. 16h + 15 (the half the MFMA takes);
//   int4 / MXFP4: load j = the whole block 4s + 2j + h;
//   int2:  the two blocks 4s + 2h, 4s + 2h + 1.
template <int WB>
__device__ __forceinline__ int64_t a_piece(int s, int j, int h) {
  if constexpr (WB == 8) return (int64_t)(GM_KB * s + j) * 32 + 16 * h;
  else if constexpr (WB == 2) return (int64_t)(GM_KB * s + 2 * h) * 8;
  else return (int64_t)(GM_KB * s + 2 * j + h) * 16;
}

__device__ __forceinline__ void swap32(uint32_t &lo, uint32_t &hi) {
  // lo := [lo of lanes 0-31 | hi of lanes 0-31], hi := [lo of lanes 32-63 | hi of lanes 32-63]
  const auto r = __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
  lo = r[0];
  hi = r[1];
}

// Blocks of a stage whose A operands come out of the same registers: pair jp holds
// blocks pair_block<WB>(jp, 0) and pair_block<WB>(jp, 1). int2 pairs blocks 4s + c and
// 4s + 2 + c (lanes 0-31 load blocks 4s, 4s + 1 and lanes 32-63 blocks 4s + 2, 4s + 3).
template <int WB>
__device__ __forceinline__ constexpr int pair_block(int jp, int i) {
  return (WB == 2) ? jp + 2 * i : 2 * jp + i;
}

// A operands of the two blocks of pair jp of one matrix, from the lane's raw pieces.
template <int WB>
__device__ __forceinline__ void a_pair(const uint4 (&raw)[Top<WB>::loads], int jp, v4i (&A)[2]) {
  if constexpr (WB == 8) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const uint4 v = raw[2 * jp + i];
      A[i] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
    }
  } else if constexpr (WB == 4 || WB == W_MX) {
    // load jp: lanes 0-31 hold block 4s + 2 jp, lanes 32-63 block 4s + 2 jp + 1. The
    // low nibbles are K values 0-15 of a block, the high nibbles 16-31.
    const uint32_t w[4] = {raw[jp].x, raw[jp].y, raw[jp].z, raw[jp].w};
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if constexpr (WB == 4) {
        lo[i] = (w[i] << 4) & 0xF0F0F0F0u;
        hi[i] = w[i] & 0xF0F0F0F0u;
      } else {
        lo[i] = e2m1x4_to_i8x4(w[i]);
        hi[i] = e2m1x4_to_i8x4(w[i] >> 4);
      }
      swap32(lo[i], hi[i]);
    }
    A[0] = v4i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]};
    A[1] = v4i{(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  } else {
    // int2, 8 bytes (two dwords w0 w1) per block; field m of byte j is value j + 8m, so
    // K values 0-15 are fields 0 and 1, and 16-31 fields 2 and 3. jp = c selects the
    // lane's block 4s + c resp. 4s + 2 + c.
    const uint32_t w0 = (jp == 0) ? raw[0].x : raw[0].z, w1 = (jp == 0) ? raw[0].y : raw[0].w;
    uint32_t lo[4] = {(w0 << 6) & 0xC0C0C0C0u, (w1 << 6) & 0xC0C0C0C0u, (w0 << 4) & 0xC0C0C0C0u,
                      (w1 << 4) & 0xC0C0C0C0u};
    uint32_t hi[4] = {(w0 << 2) & 0xC0C0C0C0u, (w1 << 2) & 0xC0C0C0C0u, w0 & 0xC0C0C0C0u, w1 & 0xC0C0C0C0u};
#pragma unroll
    for (int i = 0; i < 4; i++) swap32(lo[i], hi[i]);
    A[0] = v4i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]};
    A[1] = v4i{(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
}

// ------------------------------------------------------------------ LDS
template <int NMAT, int NGS>
struct GmLds {
  int8_t x[2][GM_TOK][GM_XROW];  // Q8_0 rows of the chunk's tokens, one stage
  float d[2][GM_TOK][GM_KB];     // their block scales
  __attribute__((aligned(16))) float gs[2][NMAT][NGS][GM_ROWS];  // group scales of the stage (GS)
  float rs[NMAT][GM_ROWS];       // row scales (one per row)
  int act[GM_TOK];               // activation row of each token slot
  int outr[GM_TOK];              // output row of each token slot (-1: past the chunk)
};

enum { MF_GATEUP = 0, MF_DOWN = 1 };

// ------------------------------------------------------------------ GEMM
// GS: one scale per group of G = GSZ<WB> inputs of a row (group scales; MXFP4's E8M0
// per block): each block's scale is then d_b * s(row, group of b), applied per result;
// otherwise one scale per row, applied in the epilogue.
// One work item wk = (row tile, chunk) of the grouped GEMM; the kernels below map
// workgroups to work items.
template <int WB, int MODE, bool GS>
__device__ __forceinline__ void mfma_item(const FfnArgs &a, const int4 *__restrict__ chunks,
                                          const int32_t *__restrict__ nchunks, int gmax, int wk) {
  constexpr int NMAT = (MODE == MF_GATEUP) ? 2 : 1;
  constexpr int G = GSZ<WB>;
  constexpr int NGS = GM_KB * QK / G;  // groups per stage: 2 (G = 64) or 4 (MXFP4)
  constexpr int NL = Top<WB>::loads;
  using Lds = GmLds<NMAT, NGS>;
  __shared__ Lds L;

  const int rt = wk / gmax, g = wk % gmax;
  if (g >= *nchunks) return;
  const int4 ch = chunks[g];  // expert, first perm index (-1: shared), tokens, first token
  const int n = ch.z;
  const int nt = __builtin_amdgcn_readfirstlane((n + 31) >> 5);  // token tiles (1..4)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int K = (MODE == MF_GATEUP) ? a.H : a.F;
  const int nkb = K / QK;
  const int ns = nkb / GM_KB;
  const int P = a.T * a.k;
  const int64_t rb = row_bytes(WB, K);
  const int64_t rbh = row_bytes(WB, a.H);
  const int r0 = rt * GM_ROWS;
  const uint8_t *blob = a.experts + (int64_t)ch.x * a.blob_bytes;
  const uint8_t *mat0 = (MODE == MF_GATEUP) ? blob : blob + 2 * (int64_t)a.F * rbh;
  const uint8_t *mat1 = blob + (int64_t)a.F * rbh;
  // this lane's weight row (the MFMA's A row li of this wavefront's 32 rows)
  const int64_t arow = (int64_t)(r0 + 32 * wv + li) * rb;

  // token slots: activation and output rows; past the chunk's tokens a slot repeats
  // the chunk's first token and writes nothing
  if (tid < GM_TOK) {
    const int i = ch.w + (tid < n ? tid : 0);
    int act, outr;
    if (ch.y < 0) {
      outr = P + i;
      act = (MODE == MF_GATEUP) ? i : P + i;
    } else {
      const int p = a.perm[ch.y + i];
      outr = p;
      act = (MODE == MF_GATEUP) ? p / a.k : p;
    }
    L.act[tid] = act;
    L.outr[tid] = tid < n ? outr : -1;
  }
  const float *sc = a.scales + (int64_t)ch.x * a.scale_stride;
  if constexpr (!GS) {
    if (tid < NMAT * GM_ROWS) {
      const int m = tid / GM_ROWS, row = tid % GM_ROWS;
      L.rs[m][row] = sc[((MODE == MF_GATEUP) ? m * a.F : 2 * a.F) + r0 + row];
    }
  }
  __syncthreads();

  const int8_t *asrc = (MODE == MF_GATEUP) ? a.xq : a.hq;
  const float *dsrc = (MODE == MF_GATEUP) ? a.xd : a.hd;
  // activation staging: piece j of this thread = token 32 j + tid / 8, 16-byte part
  // tid % 8 of the stage (a wavefront's pieces belong to one token tile: j)
  int64_t xoff[GM_TILES];
#pragma unroll
  for (int j = 0; j < GM_TILES; j++) xoff[j] = (int64_t)L.act[32 * j + (tid >> 3)] * K + (tid & 7) * 16;
  // block scales: two per thread, f = tid + 256 j -> token f / 4, block f % 4
  int64_t doff[2];
#pragma unroll
  for (int j = 0; j < 2; j++) doff[j] = (int64_t)L.act[(tid + 256 * j) >> 2] * nkb + ((tid + 256 * j) & 3);
  // group scales of a stage (GS): NMAT x NGS x GM_ROWS values. fp32 groups of 64:
  // thread q -> value q, q + 256 (matrix, group, row); MXFP4: thread q < NMAT * 128
  // loads its row's four E8M0 bytes of the stage as one 32-bit word.
  constexpr bool MXS = WB == W_MX;
  constexpr int GVALS = MXS ? NMAT * GM_ROWS : NMAT * NGS * GM_ROWS;
  const void *gsrc[2] = {nullptr, nullptr};
  if constexpr (GS) {
    const int64_t ngh = (int64_t)a.F * (a.H / G);
    const int64_t se = (int64_t)ch.x * a.scale_stride;
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int q = tid + 256 * j;
      const int m = MXS ? q / GM_ROWS : q / (NGS * GM_ROWS);
      const int grp = MXS ? 0 : (q / GM_ROWS) % NGS;
      const int row = q % GM_ROWS;
      const int64_t mbase = (MODE == MF_GATEUP) ? m * ngh : 2 * ngh;
      gsrc[j] = gs_base<WB>(a.scales, se + mbase + (int64_t)(r0 + row) * (K / G) + grp);
    }
  }

  // the lane's packed weights of one stage: two register sets (the one computed, the
  // next one in flight)
  uint4 w0[NMAT][NL], w1[NMAT][NL];
  auto wload = [&](int s, uint4 (&wr)[NMAT][NL]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NMAT; m++)
#pragma unroll
      for (int j = 0; j < NL; j++)
        wr[m][j] = *reinterpret_cast<const uint4 *>((m == 0 ? mat0 : mat1) + arow + a_piece<WB>(s, j, h));
  };
  // the activations, block scales and group scales of one stage, in flight to LDS
  uint32_t xr[GM_TILES][4];
  float dr[2], gr[2];
  uint32_t gxr = 0;
  auto gload = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < GM_TILES; j++)
      if (j < nt) {
        const uint4 v = *reinterpret_cast<const uint4 *>(asrc + xoff[j] + (int64_t)s * (GM_KB * QK));
        xr[j][0] = v.x;
        xr[j][1] = v.y;
        xr[j][2] = v.z;
        xr[j][3] = v.w;
      }
#pragma unroll
    for (int j = 0; j < 2; j++)
      if (((tid + 256 * j) >> 7) < nt) dr[j] = dsrc[doff[j] + s * GM_KB];
    if constexpr (GS) {
      if constexpr (MXS) {
        if (tid < GVALS) gxr = *reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(gsrc[0]) + s * GM_KB);
      } else {
#pragma unroll
        for (int j = 0; j < 2; j++)
          if (tid + 256 * j < GVALS) gr[j] = gs_load<WB>(gsrc[j], (int64_t)s * NGS);
      }
    }
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < GM_TILES; j++)
      if (j < nt)
        *reinterpret_cast<uint4 *>(&L.x[buf][32 * j + (tid >> 3)][(tid & 7) * 16]) =
            make_uint4(xr[j][0], xr[j][1], xr[j][2], xr[j][3]);
#pragma unroll
    for (int j = 0; j < 2; j++)
      if (((tid + 256 * j) >> 7) < nt) L.d[buf][(tid + 256 * j) >> 2][(tid + 256 * j) & 3] = dr[j];
    if constexpr (GS) {
      if constexpr (MXS) {
        if (tid < GVALS) {
#pragma unroll
          for (int kb = 0; kb < GM_KB; kb++)
            L.gs[buf][tid / GM_ROWS][kb][tid % GM_ROWS] = e8m0_f32((gxr >> (8 * kb)) & 0xFFu);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; j++) {
          const int q = tid + 256 * j;
          if (q < GVALS) L.gs[buf][q / (NGS * GM_ROWS)][(q / GM_ROWS) % NGS][q % GM_ROWS] = gr[j];
        }
      }
    }
  };

  float acc[NMAT][GM_TILES][16];
#pragma unroll
  for (int m = 0; m < NMAT; m++)
#pragma unroll
    for (int t = 0; t < GM_TILES; t++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[m][t][r] = 0.0f;

  // one stage: the A operands of the four blocks from the raw weights, then per block
  // and token tile one MFMA per matrix and its scaling
  auto compute = [&](int buf, const uint4 (&st)[NMAT][NL]) __attribute__((always_inline)) {
#pragma unroll
    for (int jp = 0; jp < 2; jp++) {
      v4i A[NMAT][2];
#pragma unroll
      for (int m = 0; m < NMAT; m++) a_pair<WB>(st[m], jp, A[m]);
      if constexpr (GS && G == 2 * QK && WB != 2) {
        // 64-input groups: the pair's blocks 2 jp and 2 jp + 1 share group jp's scale, so
        // each result takes g * (d0 * I0 + d1 * I1), the group sum of the definition
        // (five VALU operations per two blocks instead of six)
#pragma unroll
        for (int t = 0; t < GM_TILES; t++) {
          if (t >= nt) continue;
          const v4i bv0 = *reinterpret_cast<const v4i *>(&L.x[buf][32 * t + li][2 * jp * QK + 16 * h]);
          const v4i bv1 = *reinterpret_cast<const v4i *>(&L.x[buf][32 * t + li][(2 * jp + 1) * QK + 16 * h]);
          const float d0 = L.d[buf][32 * t + li][2 * jp], d1 = L.d[buf][32 * t + li][2 * jp + 1];
#pragma unroll
          for (int m = 0; m < NMAT; m++) {
            const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
            const v16i I0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[m][0], bv0, zero, 0, 0, 0);
            const v16i I1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[m][1], bv1, zero, 0, 0, 0);
            const float *gr = &L.gs[buf][m][jp][32 * wv + 4 * h];
#pragma unroll
            for (int q = 0; q < 4; q++) {
              const float4 g4 = *reinterpret_cast<const float4 *>(gr + 8 * q);
              const float gq[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
              for (int c = 0; c < 4; c++) {
                const int r = 4 * q + c;
                const float sum = fmaf(d1, (float)I1[r], d0 * (float)I0[r]);
                acc[m][t][r] = fmaf(gq[c], sum, acc[m][t][r]);
              }
            }
          }
        }
        continue;
      }
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const int kb = pair_block<WB>(jp, i);
#pragma unroll
        for (int t = 0; t < GM_TILES; t++) {
          if (t >= nt) continue;
          const v4i bv = *reinterpret_cast<const v4i *>(&L.x[buf][32 * t + li][kb * QK + 16 * h]);
          const float d = L.d[buf][32 * t + li][kb];
#pragma unroll
          for (int m = 0; m < NMAT; m++) {
            const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
            const v16i I = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[m][i], bv, zero, 0, 0, 0);
            if constexpr (GS) {
              // rows 32 wv + 8 q + 4 h + (0..3) of the workgroup's rows: four float4 reads
              const float *gr = &L.gs[buf][m][kb * QK / G][32 * wv + 4 * h];
#pragma unroll
              for (int q = 0; q < 4; q++) {
                const float4 g4 = *reinterpret_cast<const float4 *>(gr + 8 * q);
                acc[m][t][4 * q] = fmaf(d * g4.x, (float)I[4 * q], acc[m][t][4 * q]);
                acc[m][t][4 * q + 1] = fmaf(d * g4.y, (float)I[4 * q + 1], acc[m][t][4 * q + 1]);
                acc[m][t][4 * q + 2] = fmaf(d * g4.z, (float)I[4 * q + 2], acc[m][t][4 * q + 2]);
                acc[m][t][4 * q + 3] = fmaf(d * g4.w, (float)I[4 * q + 3], acc[m][t][4 * q + 3]);
              }
            } else {
#pragma unroll
              for (int r = 0; r < 16; r++) acc[m][t][r] = fmaf(d, (float)I[r], acc[m][t][r]);
            }
          }
        }
      }
    }
  };

  // Pipeline: at stage s the activations of stage s + 1 (to LDS, the other buffer)
  // and the weights of stage s + 1 (to registers, the other set) go out before stage s
  // is computed. Activation loads are issued first, so storing them into LDS at the end
  // of the stage waits for them only; the barrier waits for LDS traffic alone
  // (__syncthreads would also wait for every outstanding global load).
  auto lds_barrier = []() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0 (gfx9 encoding)
    __builtin_amdgcn_s_barrier();
  };
  gload(0);
  lstore(0);
  wload(0, w0);
  lds_barrier();
  auto body = [&](int s, const uint4 (&wc)[NMAT][NL], uint4 (&wn)[NMAT][NL]) __attribute__((always_inline)) {
    if (s + 1 < ns) gload(s + 1);
    if (s + 1 < ns) wload(s + 1, wn);
    compute(s & 1, wc);
    if (s + 1 < ns) lstore((s + 1) & 1);
    lds_barrier();
  };
  for (int s = 0; s < ns; s += 2) {
    body(s, w0, w1);
    if (s + 1 < ns) body(s + 1, w1, w0);
  }

  // epilogue. Result r of this lane in tile t: row r0 + 32 wv + 8 (r / 4) + 4 h + r % 4,
  // token slot 32 t + li.
  constexpr float inv = 1.0f / Top<WB>::scale;
  const int rw = 32 * wv + 4 * h;  // the lane's first row within the workgroup's rows
#pragma unroll
  for (int t = 0; t < GM_TILES; t++) {
    if (t >= nt) continue;
    const int out_row = L.outr[32 * t + li];
    const bool valid = out_row >= 0;
    if constexpr (MODE == MF_GATEUP) {
      float hv[16];
      float amax = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int rl = rw + 8 * (r >> 2) + (r & 3);
        const float gv = (GS ? inv : L.rs[0][rl] * inv) * acc[0][t][r];
        const float uv = (GS ? inv : L.rs[1][rl] * inv) * acc[1][t][r];
        if (valid) COLI_TAP_GU(a, out_row, r0 + rl, gv, uv);
        hv[r] = (gv / (1.0f + expf(-gv))) * uv;
        amax = fmaxf(amax, fabsf(hv[r]));
      }
      // the 32 rows of this Q8_0 block of h sit in lanes li and li + 32
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const float d = amax / 127.0f;
      uint32_t packed[4];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        uint32_t pk = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          int c = 0;
          if (d != 0.0f) c = (int)fminf(fmaxf(roundf(hv[4 * q + j] / d), -127.0f), 127.0f);
          pk |= (uint32_t)(c & 0xFF) << (8 * j);
        }
        packed[q] = pk;
      }
      if (valid) {
        int8_t *hrow = a.hq + (int64_t)out_row * a.F + r0 + rw;
#pragma unroll
        for (int q = 0; q < 4; q++) *reinterpret_cast<uint32_t *>(hrow + 8 * q) = packed[q];
        if (h == 0) a.hd[(int64_t)out_row * (a.F / QK) + (r0 + 32 * wv) / QK] = d;
      }
    } else {
      if (valid) {
        float *yrow = a.ypair + (int64_t)out_row * a.H + r0 + rw;
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int rl = rw + 8 * q;
          float4 v;
          v.x = (GS ? inv : L.rs[0][rl] * inv) * acc[0][t][4 * q];
          v.y = (GS ? inv : L.rs[0][rl + 1] * inv) * acc[0][t][4 * q + 1];
          v.z = (GS ? inv : L.rs[0][rl + 2] * inv) * acc[0][t][4 * q + 2];
          v.w = (GS ? inv : L.rs[0][rl + 3] * inv) * acc[0][t][4 * q + 3];
          *reinterpret_cast<float4 *>(yrow + 8 * q) = v;
        }
      }
    }
  }
}

// XCD-aware order: hardware workgroup i runs on XCD i % 8; each XCD takes one contiguous
// range of work items (chunks fastest), so the chunks of one heavy expert and row tile
// run side by side on one XCD
__device__ __forceinline__ int xcd_item(int bid, int nwork) { return (bid & 7) * (nwork >> 3) + (bid >> 3); }

template <int WB, int MODE, bool GS>
__global__ __launch_bounds__(256, 2) void mfma_kernel(FfnArgs a, const int4 *__restrict__ chunks,
                                                   const int32_t *__restrict__ nchunks, int gmax, int nrt) {
  mfma_item<WB, MODE, GS>(a, chunks, nchunks, gmax, xcd_item((int)blockIdx.x, nrt * gmax));
}

// The MXFP4 work items that mfma_mx_kernel flagged (a scale byte it cannot fold into the
// fp16 convert), through the integer path. A small grid reads the flags 256 at a time and
// computes the flagged items; with none flagged it costs one load per thread.
template <int MODE>
__global__ __launch_bounds__(256, 2) void mfma_redo_kernel(FfnArgs a, const int4 *__restrict__ chunks,
                                                           const int32_t *__restrict__ nchunks, int gmax, int nrt) {
  __shared__ int list[256];
  __shared__ int cnt;
  const int nwork = nrt * gmax, nch = *nchunks;
  for (int base = (int)blockIdx.x * 256; base < nwork; base += (int)gridDim.x * 256) {
    const int wk = base + (int)threadIdx.x;
    const bool set = wk < nwork && wk % gmax < nch && a.redo[wk] != 0;
    if (threadIdx.x == 0) cnt = 0;
    __syncthreads();
    if (set) list[atomicAdd(&cnt, 1)] = wk;
    __syncthreads();
    const int n = cnt;
    for (int i = 0; i < n; i++) {
      mfma_item<W_MX, MODE, true>(a, chunks, nchunks, gmax, list[i]);
      __syncthreads();  // the next item reuses the item's LDS
    }
  }
}

// ------------------------------------------------------------------ MXFP4 on the fp16 matrix cores
// MXFP4 weights take the fp16 MFMA (v_mfma_f32_32x32x16_f16, two per Q8_0 block) instead
// of widening the codes to int8:
//   - the hardware fp4 -> fp16 convert (v_cvt_scalef32_pk_f16_fp4) multiplies by the
//     block's E8M0 scale s = 2^(u - 127) on the way; e2m1 * s is exact and a normal fp16
//     number for every code when 114 <= u <= 140 (0.5 s >= 2^-14, 6 s <= 65504);
//   - the tokens' Q8_0 codes are staged in LDS as fp16 (exact, |q| <= 127);
//   - each product (e2m1 s) q is exact in fp32, and every partial sum of a block is a
//     multiple of s / 2 with fewer than 2^24 such units, so the MFMAs return s J_b exactly
//     (J_b = sum e2m1 q, the block dot of the definition);
//   - the scaling is one multiply-add per result, acc += d_b (s J_b): the single rounding
//     of d_b s J_b + acc, the same number the integer path forms as (d_b s) * J_b.
// A workgroup that meets a scale byte outside that range writes nothing and flags its work
// item; a second launch (mfma_redo_kernel) runs the flagged items only through the integer
// path (mfma_item<W_MX, MODE, true>), with the same sums. Keeping that path out of this
// kernel keeps its registers and code small (gate/up 2030 against 2374 us at the GLM-scale
// prefill with it inline).
// K order: the convert of byte j of a block gives the pair (K_j, K_j+16), and both
// operands take their fp16 pairs in that order (A: the pair of byte j; B: (q_j, q_j+16)).
// Lane half hl covers bytes 8 hl .. 8 hl + 7 of each block, the first MFMA bytes
// 8 hl + 0..3 and the second 8 hl + 4..7; an MFMA multiplies A and B slot by slot, so
// any K order shared by both operands gives the same sums.
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int MX_XROW = GM_KB * 16 + 4;  // LDS dwords per token row of a stage: 4 blocks x 16 pairs + padding
constexpr uint32_t MX_FOLD_LO = 114, MX_FOLD_HI = 140;

struct MxLds {
  // fp16 pairs (q_j, q_j+16) of the stage's blocks; 16-byte aligned so that a lane's
  // eight fp16 of a B operand are one ds_read_b128
  __attribute__((aligned(16))) uint32_t x[2][GM_TOK][MX_XROW];
  float d[2][GM_TOK][GM_KB];       // their block scales
  int bad[4];                      // per wavefront: a scale byte outside the folding range
  int act[GM_TOK];
  int outr[GM_TOK];
};

__device__ __forceinline__ bool mx_foldable(uint32_t w) {  // every scale byte of w in range
  bool ok = true;
#pragma unroll
  for (int b = 0; b < 4; b++) ok = ok && (((w >> (8 * b)) & 0xFFu) - MX_FOLD_LO) <= (MX_FOLD_HI - MX_FOLD_LO);
  return ok;
}

// A operands of one block: eight fp16 pairs from two dwords of codes, times `s`.
__device__ __forceinline__ void mx_a(uint32_t w_lo, uint32_t w_hi, float s, v8h &a_lo, v8h &a_hi) {
  a_lo = __builtin_bit_cast(v8h, make_uint4(as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w_lo, s, 0)),
                                             as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w_lo, s, 1)),
                                             as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w_lo, s, 2)),
                                             as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w_lo, s, 3))));
  a_hi = __builtin_bit_cast(v8h, make_uint4(as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w_hi, s, 0)),
                                             as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w_hi, s, 1)),
                                             as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w_hi, s, 2)),
                                             as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w_hi, s, 3))));
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void mfma_mx_kernel(FfnArgs a, const int4 *__restrict__ chunks,
                                                         const int32_t *__restrict__ nchunks, int gmax, int nrt) {
  constexpr int NMAT = (MODE == MF_GATEUP) ? 2 : 1;
  constexpr int NL = Top<W_MX>::loads;  // two 16-byte pieces per matrix and stage
  __shared__ MxLds L;

  // work item, chunk and token slots: as mfma_item
  const int wk = xcd_item((int)blockIdx.x, nrt * gmax);
  const int rt = wk / gmax, g = wk % gmax;
  if (g >= *nchunks) return;
  const int4 ch = chunks[g];
  const int n = ch.z;
  const int nt = __builtin_amdgcn_readfirstlane((n + 31) >> 5);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int K = (MODE == MF_GATEUP) ? a.H : a.F;
  const int nkb = K / QK;
  const int ns = nkb / GM_KB;
  const int P = a.T * a.k;
  const int64_t rb = row_bytes(W_MX, K);
  const int64_t rbh = row_bytes(W_MX, a.H);
  const int r0 = rt * GM_ROWS;
  const uint8_t *blob = a.experts + (int64_t)ch.x * a.blob_bytes;
  const uint8_t *mat0 = (MODE == MF_GATEUP) ? blob : blob + 2 * (int64_t)a.F * rbh;
  const uint8_t *mat1 = blob + (int64_t)a.F * rbh;
  const int row = r0 + 32 * wv + li;  // this lane's weight row
  const int64_t arow = (int64_t)row * rb;
  // E8M0 bytes of the lane's row (gate [F][H/32] | up [F][H/32] | down [H][F/32]): the
  // four of a stage are one dword
  const uint8_t *sbase = reinterpret_cast<const uint8_t *>(a.scales) + (int64_t)ch.x * a.scale_stride;
  const int64_t ngh = (int64_t)a.F * (a.H / QK);
  const uint8_t *srow0 = sbase + ((MODE == MF_GATEUP) ? 0 : 2 * ngh) + (int64_t)row * nkb;
  const uint8_t *srow1 = sbase + ngh + (int64_t)row * nkb;

  if (tid < GM_TOK) {
    const int i = ch.w + (tid < n ? tid : 0);
    int act, outr;
    if (ch.y < 0) {
      outr = P + i;
      act = (MODE == MF_GATEUP) ? i : P + i;
    } else {
      const int p = a.perm[ch.y + i];
      outr = p;
      act = (MODE == MF_GATEUP) ? p / a.k : p;
    }
    L.act[tid] = act;
    L.outr[tid] = tid < n ? outr : -1;
  }
  __syncthreads();

  const int8_t *asrc = (MODE == MF_GATEUP) ? a.xq : a.hq;
  const float *dsrc = (MODE == MF_GATEUP) ? a.xd : a.hd;
  // activation staging: thread tid takes block tid % 4 of the stage for token slot tid / 4
  const int st_tok = tid >> 2, st_kb = tid & 3;
  const bool st_on = st_tok < 32 * nt;
  const int64_t xoff = (int64_t)L.act[st_tok] * K + st_kb * QK;
  const int64_t doff = (int64_t)L.act[st_tok] * nkb + st_kb;

  uint4 w0[NMAT][NL], w1[NMAT][NL];
  uint32_t u0[NMAT], u1[NMAT];  // the stage's scale bytes of the lane's row
  auto wload = [&](int s, uint4 (&wr)[NMAT][NL], uint32_t (&ur)[NMAT]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NMAT; m++) {
#pragma unroll
      for (int j = 0; j < NL; j++)
        wr[m][j] = *reinterpret_cast<const uint4 *>((m == 0 ? mat0 : mat1) + arow + a_piece<W_MX>(s, j, h));
      ur[m] = *reinterpret_cast<const uint32_t *>((m == 0 ? srow0 : srow1) + s * GM_KB);
    }
  };
  uint4 xr0 = make_uint4(0, 0, 0, 0), xr1 = make_uint4(0, 0, 0, 0);
  float dr = 0.0f;
  auto gload = [&](int s) __attribute__((always_inline)) {
    if (st_on) {
      const int8_t *p = asrc + xoff + (int64_t)s * (GM_KB * QK);
      xr0 = *reinterpret_cast<const uint4 *>(p);
      xr1 = *reinterpret_cast<const uint4 *>(p + 16);
      dr = dsrc[doff + s * GM_KB];
    }
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
    if (st_on) {
      const int x[8] = {(int)xr0.x, (int)xr0.y, (int)xr0.z, (int)xr0.w, (int)xr1.x, (int)xr1.y, (int)xr1.z, (int)xr1.w};
      uint32_t hp[16];
      q8_to_f16_pairs(x, hp);
      uint4 *dst = reinterpret_cast<uint4 *>(&L.x[buf][st_tok][16 * st_kb]);
#pragma unroll
      for (int q = 0; q < 4; q++) dst[q] = make_uint4(hp[4 * q], hp[4 * q + 1], hp[4 * q + 2], hp[4 * q + 3]);
      L.d[buf][st_tok][st_kb] = dr;
    }
  };

  float acc[NMAT][GM_TILES][16];
#pragma unroll
  for (int m = 0; m < NMAT; m++)
#pragma unroll
    for (int t = 0; t < GM_TILES; t++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[m][t][r] = 0.0f;

  // one stage: s rides in the convert (lanes whose row has a byte out of range compute
  // garbage and mark the work item for the integer path)
  bool bad = false;
  auto compute = [&](int buf, const uint4 (&wc)[NMAT][NL], const uint32_t (&uc)[NMAT]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NMAT; m++) bad = bad || !mx_foldable(uc[m]);
#pragma unroll
    for (int jp = 0; jp < 2; jp++) {
      // lanes 0-31 hold block 4s + 2 jp, lanes 32-63 block 4s + 2 jp + 1; after the swaps
      // each lane holds bytes 8 h .. 8 h + 7 of both: wd[m][i][0..1] for block 2 jp + i
      uint32_t wd[NMAT][2][2];
#pragma unroll
      for (int m = 0; m < NMAT; m++) {
        uint32_t x0 = wc[m][jp].x, z0 = wc[m][jp].z, y0 = wc[m][jp].y, w0_ = wc[m][jp].w;
        swap32(x0, z0);
        swap32(y0, w0_);
        wd[m][0][0] = x0;
        wd[m][0][1] = y0;
        wd[m][1][0] = z0;
        wd[m][1][1] = w0_;
      }
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const int kb = 2 * jp + i;
        v8h alo[NMAT], ahi[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; m++)
          mx_a(wd[m][i][0], wd[m][i][1], __uint_as_float(((uc[m] >> (8 * kb)) & 0xFFu) << 23), alo[m], ahi[m]);
#pragma unroll
        for (int t = 0; t < GM_TILES; t++) {
          if (t >= nt) continue;
          const v8h blo = *reinterpret_cast<const v8h *>(&L.x[buf][32 * t + li][16 * kb + 8 * h]);
          const v8h bhi = *reinterpret_cast<const v8h *>(&L.x[buf][32 * t + li][16 * kb + 8 * h + 4]);
          const float d = L.d[buf][32 * t + li][kb];
#pragma unroll
          for (int m = 0; m < NMAT; m++) {
            const v16f zero = {};
            v16f D = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[m], blo, zero, 0, 0, 0);
            D = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[m], bhi, D, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; r++) acc[m][t][r] = fmaf(d, D[r], acc[m][t][r]);
          }
        }
      }
    }
  };

  auto lds_barrier = []() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0 (gfx9 encoding)
    __builtin_amdgcn_s_barrier();
  };
  gload(0);
  lstore(0);
  wload(0, w0, u0);
  lds_barrier();
  auto body = [&](int s, const uint4 (&wc)[NMAT][NL], const uint32_t (&uc)[NMAT], uint4 (&wn)[NMAT][NL],
                  uint32_t (&un)[NMAT]) __attribute__((always_inline)) {
    if (s + 1 < ns) gload(s + 1);
    if (s + 1 < ns) wload(s + 1, wn, un);
    compute(s & 1, wc, uc);
    if (s + 1 < ns) lstore((s + 1) & 1);
    lds_barrier();
  };
  for (int s = 0; s < ns; s += 2) {
    body(s, w0, u0, w1, u1);
    if (s + 1 < ns) body(s + 1, w1, u1, w0, u0);
  }

  // a work item with any scale byte out of range is left to the integer kernel
  if (lane == 0) L.bad[wv] = __any(bad) ? 1 : 0;
  __syncthreads();
  const int redo = L.bad[0] | L.bad[1] | L.bad[2] | L.bad[3];
  if (tid == 0) a.redo[wk] = redo;
  if (redo) return;

  // epilogue: result r of this lane in tile t is row r0 + 32 wv + 8 (r / 4) + 4 h + r % 4,
  // token slot 32 t + li; the sums carry every scale (no row scales with MXFP4)
  const int rw = 32 * wv + 4 * h;
#pragma unroll
  for (int t = 0; t < GM_TILES; t++) {
    if (t >= nt) continue;
    const int out_row = L.outr[32 * t + li];
    const bool valid = out_row >= 0;
    if constexpr (MODE == MF_GATEUP) {
      float hv[16];
      float amax = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int rl = rw + 8 * (r >> 2) + (r & 3);
        const float gv = acc[0][t][r], uv = acc[1][t][r];
        if (valid) COLI_TAP_GU(a, out_row, r0 + rl, gv, uv);
        hv[r] = (gv / (1.0f + expf(-gv))) * uv;
        amax = fmaxf(amax, fabsf(hv[r]));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const float d = amax / 127.0f;
      uint32_t packed[4];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        uint32_t pk = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          int c = 0;
          if (d != 0.0f) c = (int)fminf(fmaxf(roundf(hv[4 * q + j] / d), -127.0f), 127.0f);
          pk |= (uint32_t)(c & 0xFF) << (8 * j);
        }
        packed[q] = pk;
      }
      if (valid) {
        int8_t *hrow = a.hq + (int64_t)out_row * a.F + r0 + rw;
#pragma unroll
        for (int q = 0; q < 4; q++) *reinterpret_cast<uint32_t *>(hrow + 8 * q) = packed[q];
        if (h == 0) a.hd[(int64_t)out_row * (a.F / QK) + (r0 + 32 * wv) / QK] = d;
      }
    } else {
      if (valid) {
        float *yrow = a.ypair + (int64_t)out_row * a.H + r0 + rw;
#pragma unroll
        for (int q = 0; q < 4; q++)
          *reinterpret_cast<float4 *>(yrow + 8 * q) =
              make_float4(acc[0][t][4 * q], acc[0][t][4 * q + 1], acc[0][t][4 * q + 2], acc[0][t][4 * q + 3]);
      }
    }
  }
}

// ------------------------------------------------------------------ host side
int32_t mfma_gmax(int32_t T, int32_t k, int32_t E, int32_t has_shared) {
  const int64_t rows = (int64_t)T * k + (int64_t)has_shared * T;
  const int64_t g = (rows + GM_TOK - 1) / GM_TOK + E + has_shared;
  return (int32_t)((g + 7) / 8 * 8);
}

int64_t mfma_redo_words(const coli_moe_cfg &c, int32_t T) {
  if (c.wfmt != W_MX || (int64_t)T * c.top_k <= LOCAL_GROUP_MAX_P) return 0;
  return (int64_t)mfma_gmax(T, c.top_k, c.n_experts, c.has_shared) * (max(c.hidden, c.ffn) / GM_ROWS);
}

hipError_t launch_plan(const FfnArgs &a, int4 *chunks, int32_t *nchunks, int32_t gmax, hipStream_t s) {
  if (a.E + a.has_shared > 2048) return hipErrorInvalidValue;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, a, chunks, nchunks, gmax);
  return hipGetLastError();
}

template <int WB, int MODE>
static hipError_t launch_mf(const FfnArgs &a, const int4 *chunks, const int32_t *nchunks, int32_t gmax,
                            hipStream_t s) {
  const int rows = (MODE == MF_GATEUP) ? a.F : a.H;
  const int K = (MODE == MF_GATEUP) ? a.H : a.F;
  if (rows % GM_ROWS || K % (GM_KB * QK) || gmax % 8) return hipErrorInvalidValue;
  // MXFP4 always has its E8M0 scale per 32 inputs; the integer formats one per row or per 64
  if (WB == W_MX ? a.gs != 32 : (a.gs != 0 && a.gs != 64)) return hipErrorInvalidValue;
  const int nrt = rows / GM_ROWS;
  const int64_t nwork = (int64_t)nrt * gmax;
  if (nwork > 0x7fffffff) return hipErrorInvalidValue;
  if constexpr (WB == W_MX) {
    // the fp16 kernel, then the integer kernel for the work items it flagged
    hipLaunchKernelGGL((mfma_mx_kernel<MODE>), dim3((unsigned)nwork), dim3(256), 0, s, a, chunks, nchunks, gmax, nrt);
    const int64_t rg = (nwork + 255) / 256;
    hipLaunchKernelGGL((mfma_redo_kernel<MODE>), dim3((unsigned)(rg < 256 ? rg : 256)), dim3(256), 0, s, a, chunks,
                       nchunks, gmax, nrt);
  } else if (a.gs)
    hipLaunchKernelGGL((mfma_kernel<WB, MODE, true>), dim3((unsigned)nwork), dim3(256), 0, s, a, chunks, nchunks,
                       gmax, nrt);
  else
    hipLaunchKernelGGL((mfma_kernel<WB, MODE, false>), dim3((unsigned)nwork), dim3(256), 0, s, a, chunks, nchunks,
                       gmax, nrt);
  return hipGetLastError();
}

hipError_t launch_mfma_gateup(int wfmt, const FfnArgs &a, const int4 *chunks, const int32_t *nchunks, int32_t gmax,
                              hipStream_t s) {
  switch (wfmt) {
    case 4: return launch_mf<4, MF_GATEUP>(a, chunks, nchunks, gmax, s);
    case 8: return launch_mf<8, MF_GATEUP>(a, chunks, nchunks, gmax, s);
    case 2: return launch_mf<2, MF_GATEUP>(a, chunks, nchunks, gmax, s);
    case W_MX: return launch_mf<W_MX, MF_GATEUP>(a, chunks, nchunks, gmax, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mfma_down(int wfmt, const FfnArgs &a, const int4 *chunks, const int32_t *nchunks, int32_t gmax,
                            hipStream_t s) {
  switch (wfmt) {
    case 4: return launch_mf<4, MF_DOWN>(a, chunks, nchunks, gmax, s);
    case 8: return launch_mf<8, MF_DOWN>(a, chunks, nchunks, gmax, s);
    case 2: return launch_mf<2, MF_DOWN>(a, chunks, nchunks, gmax, s);
    case W_MX: return launch_mf<W_MX, MF_DOWN>(a, chunks, nchunks, gmax, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace coli
