// Ragged grouped GEMMs on gfx950 fp8 MFMA (OCP e4m3, v_mfma_scale_f32_32x32x64_f8f6f4 with unit
// block exponents) with fp32 block scales: activations carry one scale per row per 128 values
// of K, weights one per 128x128 block.  Blockwise FP8 is one of the data types of the fused MoE
// backward on the Prime Mega MoE page ("Prime Mega MoE: tanításra is jó a DeepSeek MoE
// kernele", section "Mit csinált a Prime Intellect?"); quantisation adds work on top of the
// 16-bit master weights (TE MoE page "NVIDIA מציגה דרך יעילה לאמן מודלי MoE בביולוגיה",
// section "צמצום הזיכרון ותקורות הכימות").
//
// One K stage is exactly one 128-wide scale block: the stage's two 64-deep MFMAs accumulate
// into a temporary, which is then promoted into the fp32 accumulator with s_a(row) * s_b(block).
// Tiles are 256 x 256 x 128 with 8 waves (2 x 4), each owning 128 x 64.  Operands reach LDS by
// DMA; K-contiguous tiles are read with ds_read_b128, N-contiguous weight tiles with the 8-bit
// LDS transpose read.  The row scales of each stage arrive by DMA as well; they are stored by
// k block in the experts' sorted order, so those of 32 rows are one contiguous run.
//
// Epilogues: UP writes H (bf16, kept for the backward), As = w * silu(g) * u in bf16 (for the
// weight gradient) and requantised to e4m3 with one scale per row per 128 columns (the next
// GEMM's K); DACT writes dH in bf16 and requantised the same way, plus the routing-weight
// partials; DOWN and DX write bf16 rows in slot order.
#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace moe {

enum Fp8Mode { F_UP = 0, F_DOWN = 1, F_DACT = 2, F_DX = 3 };

// Row tiles per group of the tile order (grouped_tile): the large weight panels of the fp8
// shapes are reused across this many row tiles while they sit in L2.
#ifndef FP8_GM
#define FP8_GM 8
#endif

struct Fp8Args {
  const uint8_t* A;        // fp8 rows, K contiguous
  int64_t lda;             // bytes
  const float* A_scale;    // by k step: the scale of sorted row pos for k block t at t * as_kstride + pos
  int as_kstride;          // floats from one k block's scales to the next (rows of the buffer)
  const uint8_t* B;        // fp8 weights of all experts
  int64_t ldb, b_estride;  // bytes
  const float* B_scale;    // per expert [rows/128, cols/128] of B as stored
  int64_t bs_estride;
  int bs_ld;
  int N, K, kslots, f;
  const int32_t* offsets;
  const int32_t* perm;
  const int2* tiles;
  const int32_t* ntiles;
  int gatherA;
  const float* topk_w;
  uint16_t* C0;
  int64_t ldc0;
  uint16_t* C1;
  int64_t ldc1;
  uint8_t* Q;  // requantised output (UP: As, DACT: dH)
  int64_t ldq;
  float* QS;  // their scales by k step, as A_scale
  int64_t qs_kstride;
  const uint16_t* Hs;
  int64_t ldh;
  float* dwp;  // d_topk_w partials, part-major: dwp[part * dwp_stride + pos]
  int64_t dwp_stride;
};

// Quantise 8 values of a 128-wide block held by 16 consecutive lanes: scale = amax / 448 of the
// block (1 when all are zero); returns the 8 codes and sets *scale.
__device__ __forceinline__ u32x2 quant8_group16(const float (&v)[8], float* scale) {
  float m = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(v[t]));
#pragma unroll
  for (int s = 8; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  const float sc = m > 0.0f ? m / 448.0f : 1.0f;
  const float inv = m > 0.0f ? 448.0f / m : 1.0f;
  *scale = sc;
  u32x2 q;
  q.x = pack_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  q.y = pack_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  return q;
}

template <int MODE>
__global__ __launch_bounds__(512, 1) void grouped_gemm_fp8_kernel(const Fp8Args g) {
  constexpr int BM = kFp8BM, BN = 256, BK = 128, S = 2, WM = 2, WN = 4, NW = 8, NTH = 512;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr bool B_KN = (MODE == F_UP || MODE == F_DOWN);
  constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK, SC_BYTES = NW * 256;
  constexpr int STAGE = A_BYTES + B_BYTES + SC_BYTES;
  constexpr int QA = A_BYTES / (1024 * NW), QB = B_BYTES / (1024 * NW);
  constexpr int CPAD = BN + 4;
  constexpr int PH = 2;  // row fragments per epilogue phase: the band holds 64 * PH rows
  constexpr int CBAND_BYTES = 2 * 32 * PH * CPAD * 4;
  constexpr int ARENA = S * STAGE > CBAND_BYTES ? S * STAGE : CBAND_BYTES;
  static_assert(BM == 256 && QA == 4 && QB == 4, "DMA split");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[ARENA];
  float* cband = reinterpret_cast<float*>(smem);
  __shared__ float s_w[BM];
  __shared__ int s_slot[BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr_of(smem));

  // ------------------------------------------------------------------ tile coordinates
  const int nN = (MODE == F_UP) ? g.f / (BN / 2) : g.N / BN;
  const int G_valid = *(const CONST_AS int32_t*)g.ntiles * nN;
  if ((int)blockIdx.x >= G_valid) return;
  const int lid = xcd_remap(blockIdx.x, G_valid);
  const int2 rc = grouped_tile(lid, G_valid / nN, nN, FP8_GM);
  const int nt = rc.y;
  const int2 te = g.tiles[rc.x];
  const int e = te.x;
  const int m0 = g.offsets[e] + te.y * BM;
  const int mrows = min(BM, g.offsets[e + 1] - m0);
  const int n0 = (MODE == F_UP) ? nt * (BN / 2) : nt * BN;
  for (int r = tid; r < BM; r += NTH) {
    int p = -1;
    float wv = 0.0f;
    if (r < mrows) {
      p = g.perm[m0 + r];
      if (MODE == F_UP || MODE == F_DACT) wv = g.topk_w[p];
    }
    s_slot[r] = p;
    s_w[r] = wv;
  }
  const uint8_t* Bexp = g.B + (int64_t)e * g.b_estride;

  // ------------------------------------------------------------------ DMA sources
  // A (KM, 256 rows x 128 bytes): block gi = 4*wave + q holds rows 8*gi..8*gi+7.
  const uint8_t* a_src[QA];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int row = 8 * (wave * QA + q) + lane / 8;
    const int c = (lane % 8) ^ ((row >> 1) & 7);
    const int pos = m0 + (row < mrows ? row : 0);  // rows past the expert feed unstored outputs
    const int64_t src = g.gatherA ? (int64_t)(g.perm[pos] / g.kslots) : (int64_t)pos;
    a_src[q] = g.A + src * g.lda + 16 * c;
  }
  // Scales of a K stage, one 4-byte DMA per wave into its 256-byte slot: lanes 0..31 bring the
  // row scales of rows 32w..32w+31 (128 contiguous bytes: the row scales are stored by k step
  // in the sorted order), lanes 32 and 33 the weight-block scales of the wave's two B fragments
  // (lanes past 33 repeat lane 32).  Each lane's source advances by sc_step floats per stage.  With no scalar load in the K loop the stage's LDS reads retire in order, so each
  // MFMA waits only for its own fragments.
  const float* sc_src;
  int sc_step;
  if (lane < 32) {
    const int row = 32 * wave + lane;
    sc_src = g.A_scale + (m0 + (row < mrows ? row : 0));
    sc_step = g.as_kstride;
  } else {
    const int j = lane == 33 ? 1 : 0;
    int nb;  // 128-column block of the weight matrix holding B fragment j
    if constexpr (MODE == F_UP) nb = j == 0 ? nt : g.f / 128 + nt;  // gate / up columns of the tile
    else nb = (n0 + wn * (BN / WN) + j * 32) / 128;
    sc_src = g.B_scale + (int64_t)e * g.bs_estride + (B_KN ? (int64_t)nb : (int64_t)nb * g.bs_ld);
    sc_step = B_KN ? g.bs_ld : 1;
  }
  const uint8_t* b_src[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    if constexpr (B_KN) {
      // k rows 4*gi + lane/16 (256 bytes each), chunk lane%16 holds logical chunk c
      const int kr = 4 * (wave * QB + q) + lane / 16;
      const int c = (lane % 16) ^ (2 * (kr & 7));
      int col;
      if constexpr (MODE == F_UP) col = c < 8 ? n0 + 16 * c : g.f + n0 + 16 * (c - 8);
      else col = n0 + 16 * c;
      b_src[q] = Bexp + (int64_t)kr * g.ldb + col;
    } else {
      const int row = 8 * (wave * QB + q) + lane / 8;
      const int c = (lane % 8) ^ ((row >> 1) & 7);
      b_src[q] = Bexp + (int64_t)(n0 + row) * g.ldb + 16 * c;
    }
  }
  auto issue = [&](int t, int st) __attribute__((always_inline)) {
    const int k0 = t * BK;
    const uint32_t abase = lds0 + st * STAGE, bbase = abase + A_BYTES, sbase = bbase + B_BYTES;
#pragma unroll
    for (int q = 0; q < QA; ++q) dma16(a_src[q] + k0, abase + (wave * QA + q) * 1024);
#pragma unroll
    for (int q = 0; q < QB; ++q)
      dma16(B_KN ? b_src[q] + (int64_t)k0 * g.ldb : b_src[q] + k0, bbase + (wave * QB + q) * 1024);
    dma4(sc_src + (int64_t)t * sc_step, sbase + wave * 256);
  };

  // LDS column of the wave's j-th 32-column B fragment (UP: gate fragments, then up fragments)
  auto b_row = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (MODE == F_UP)
      return j < FN / 2 ? wn * (TN / 2) + j * 32 : BN / 2 + wn * (TN / 2) + (j - FN / 2) * 32;
    else
      return wn * TN + j * 32;
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // One K stage = one 128-wide scale block: per 32-row fragment i, two 64-deep MFMAs per B
  // fragment into a temporary, then acc += temp * s_a(row) * s_b(block).  The MFMAs take the B
  // fragment as their first operand, so each 32x32 block is held transposed: lane l holds row
  // l % 32 of the fragment (one row scale per lane) and 16 of its columns, all in one 128-column
  // weight block, so a block's promotion is one scale product and 16 fmas per lane.
  // In an expert's last row tile, a wave whose rows all lie past the expert's end skips its
  // fragment reads and MFMAs (uniform: mrows and wm are); it still issues its DMA share.
  const bool busy = __builtin_amdgcn_readfirstlane(wm * TM < mrows);
  auto compute = [&](int st) __attribute__((always_inline)) {
    const uint32_t abase = lds0 + st * STAGE, bbase = abase + A_BYTES, sbase = bbase + B_BYTES;
    auto arow = [&](int i) __attribute__((always_inline)) { return wm * TM + i * 32 + (lane & 31); };
    // LDS reads in the order of first use: the first k half's B fragments and A fragment, then
    // the second half's, then the scales
    i32x8 bv[2][FN];
    i32x8 a0, a1;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (B_KN) bv[kk][j] = read_kn8(bbase, b_row(j), kk, lane);
        else bv[kk][j] = read_km8(bbase, b_row(j) + (lane & 31), kk, lane);
      }
      if (kk == 0) a0 = read_km8(abase, arow(0), 0, lane);
      else a1 = read_km8(abase, arow(0), 1, lane);
    }
    // the scale of the lane's row in each row fragment (rows 32w.. of the stage sit at 256 * w)
    // and the wave's two weight-block scales (words 32, 33 of its own slot)
    float sa[FM], sb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
      sa[i] = *(const LDS_AS float*)(uintptr_t)(sbase + (wm * FM + i) * 256 + (lane & 31) * 4);
#pragma unroll
    for (int j = 0; j < FN; ++j) sb[j] = *(const LDS_AS float*)(uintptr_t)(sbase + wave * 256 + (32 + j) * 4);
    __builtin_amdgcn_sched_barrier(0);
    // Software pipeline over the row fragments, in a fixed order (scheduling fences): the
    // promotion of block (i, 0) runs under the MFMA of (i, 1) and that of (i, 1) under the first
    // MFMA of (i + 1, 0), each temporary being rewritten only after its promotion has read it;
    // the next row fragment's k halves are read from LDS as soon as the current ones have been
    // consumed.  Same registers as a plain loop: two temporaries, two A fragments.
    static_assert(FN == 2, "pipeline written for two column fragments per wave");
    auto mfma = [&](const i32x8& b, const i32x8& a, const f32x16_t& c) __attribute__((always_inline)) {
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 0, 0, 0, 127, 0, 127);
    };
    auto promote = [&](int i, int j, const f32x16_t& t) __attribute__((always_inline)) {
      const float s2 = sa[i] * sb[j];
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(t[r], s2, acc[i][j][r]);
    };
    const f32x16_t z = {};
    f32x16_t t0 = mfma(bv[0][0], a0, z), t1 = mfma(bv[0][1], a0, z);
    __builtin_amdgcn_sched_barrier(0);
    if (FM > 1) a0 = read_km8(abase, arow(1), 0, lane);
    __builtin_amdgcn_sched_barrier(0);
    t0 = mfma(bv[1][0], a1, t0);
    t1 = mfma(bv[1][1], a1, t1);
    __builtin_amdgcn_sched_barrier(0);
    if (FM > 1) a1 = read_km8(abase, arow(1), 1, lane);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      promote(i, 0, t0);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < FM) t0 = mfma(bv[0][0], a0, z);
      __builtin_amdgcn_sched_barrier(0);
      promote(i, 1, t1);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < FM) {
        t1 = mfma(bv[0][1], a0, z);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 2 < FM) a0 = read_km8(abase, arow(i + 2), 0, lane);
        __builtin_amdgcn_sched_barrier(0);
        t0 = mfma(bv[1][0], a1, t0);
        t1 = mfma(bv[1][1], a1, t1);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 2 < FM) a1 = read_km8(abase, arow(i + 2), 1, lane);
      }
    }
  };

  // ------------------------------------------------------------------ main loop (2 stages)
  const int nk = g.K / BK;
  __syncthreads();
  issue(0, 0);
  for (int it = 0; it < nk; ++it) {
    vm_lgkm_wait_barrier<0>();
    if (it + 1 < nk) issue(it + 1, (it + 1) % S);
    if (busy) compute(it % S);
  }
  __syncthreads();

  // ------------------------------------------------------------------ epilogues (LDS band)
  const int lcol = lane & 31;
  constexpr int CH = BN / 8;
  // DACT: 32 threads per row, 8 columns each, ITEMS rows per thread and phase
  constexpr int BR = 64 * PH, ITEMS = BR * CH / NTH;  // band rows, dA items per thread
  static_assert(FM % PH == 0 && (MODE != F_DACT || ITEMS * NTH == BR * CH), "epilogue band");
#pragma unroll
  for (int ph = 0; ph < FM / PH; ++ph) {
    // band row q: wave row q / (32*PH), row fragment PH*ph + (q % (32*PH)) / 32, row q % 32
    auto tile_row = [&](int q) __attribute__((always_inline)) {
      return (q / (32 * PH)) * TM + 32 * (PH * ph + (q % (32 * PH)) / 32) + (q & 31);
    };
    // DACT: the phase's H loads go out before the band is written, so their latency hides
    // behind the band writes and the barrier
    uint4 hgv[ITEMS], huv[ITEMS];
    if constexpr (MODE == F_DACT) {
#pragma unroll
      for (int it = 0; it < ITEMS; ++it) {
        const int id = tid + it * NTH, q = id / CH, cc = id % CH;
        const int lr = tile_row(q);
        const int64_t pos = m0 + (lr < mrows ? lr : 0);  // rows past the expert's end read row m0
        hgv[it] = *(const uint4*)&g.Hs[pos * g.ldh + n0 + cc * 8];
        huv[it] = *(const uint4*)&g.Hs[pos * g.ldh + g.f + n0 + cc * 8];
      }
    }
#pragma unroll
    for (int ii = 0; ii < PH; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        // transposed block: lane l holds band row 32*PH*wm + 32*ii + l%32, columns
        // 8*(r/4) + 4*(l/32) + r%4
        const int i = PH * ph + ii, q = 32 * PH * wm + 32 * ii + lcol;
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const int c = b_row(j) + 8 * (r >> 2) + 4 * (lane >> 5);
          *(float4*)&cband[q * CPAD + c] = make_float4(acc[i][j][r], acc[i][j][r + 1], acc[i][j][r + 2], acc[i][j][r + 3]);
        }
      }
    __syncthreads();
    if constexpr (MODE == F_UP) {
      // 16 lanes per row: 8 gate + 8 up columns each; As's 128 columns of the tile form one block
      for (int id = tid; id < BR * (CH / 2); id += NTH) {
        const int q = id / (CH / 2), cc = id % (CH / 2);
        const int lr = tile_row(q);
        const bool ok = lr < mrows;
        const float* gp = &cband[q * CPAD + cc * 8];
        const float* up = &cband[q * CPAD + BN / 2 + cc * 8];
        const float w = s_w[lr];
        float as[8];
        uint32_t hg[4], hu[4], ab[4];
#pragma unroll
        for (int t2 = 0; t2 < 4; ++t2) {
          const float g0 = gp[2 * t2], g1 = gp[2 * t2 + 1], u0 = up[2 * t2], u1 = up[2 * t2 + 1];
          hg[t2] = pack_bf16x2(g0, g1);
          hu[t2] = pack_bf16x2(u0, u1);
          as[2 * t2] = w * g0 * sigmoidf_fast(g0) * u0;
          as[2 * t2 + 1] = w * g1 * sigmoidf_fast(g1) * u1;
          ab[t2] = pack_bf16x2(as[2 * t2], as[2 * t2 + 1]);
        }
        float sc;
        const u32x2 qv = quant8_group16(as, &sc);
        if (ok) {
          const int64_t pos = m0 + lr;
          const int col = n0 + cc * 8;
          *(uint4*)&g.C0[pos * g.ldc0 + col] = make_uint4(hg[0], hg[1], hg[2], hg[3]);
          *(uint4*)&g.C0[pos * g.ldc0 + g.f + col] = make_uint4(hu[0], hu[1], hu[2], hu[3]);
          *(uint4*)&g.C1[pos * g.ldc1 + col] = make_uint4(ab[0], ab[1], ab[2], ab[3]);
          *(u32x2*)&g.Q[pos * g.ldq + col] = qv;
          if (cc == 0) g.QS[nt * g.qs_kstride + pos] = sc;
        }
      }
    } else if constexpr (MODE == F_DACT) {
      // 32 lanes per row (8 columns each): dSwiGLU, routing-weight partial, dH in bf16 and e4m3
#pragma unroll
      for (int it = 0; it < ITEMS; ++it) {
        const int id = tid + it * NTH, q = id / CH, cc = id % CH;
        const int lr = tile_row(q);
        const bool ok = lr < mrows;
        const int64_t pos = m0 + (ok ? lr : 0);
        const int col = n0 + cc * 8;
        const float* Gp = &cband[q * CPAD + cc * 8];
        const float w = s_w[lr];
        float part = 0.0f, dg[8], du[8];
#pragma unroll
        for (int t2 = 0; t2 < 4; ++t2) {
          const uint32_t wg = word_of(hgv[it], t2), wu = word_of(huv[it], t2);
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const float gv = hh ? hi_bf16(wg) : lo_bf16(wg), uv = hh ? hi_bf16(wu) : lo_bf16(wu);
            const float G = Gp[2 * t2 + hh];
            const float sg = sigmoidf_fast(gv), sl = gv * sg, da = w * G;
            part += G * (sl * uv);
            dg[2 * t2 + hh] = da * uv * sg * (1.0f + gv * (1.0f - sg));
            du[2 * t2 + hh] = da * sl;
          }
        }
        float sg_, su_;
        const u32x2 qg = quant8_group16(dg, &sg_);
        const u32x2 qu = quant8_group16(du, &su_);
#pragma unroll
        for (int m = CH / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
        if (ok) {
          *(uint4*)&g.C0[pos * g.ldc0 + col] = make_uint4(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]),
                                                          pack_bf16x2(dg[4], dg[5]), pack_bf16x2(dg[6], dg[7]));
          *(uint4*)&g.C0[pos * g.ldc0 + g.f + col] = make_uint4(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]),
                                                                pack_bf16x2(du[4], du[5]), pack_bf16x2(du[6], du[7]));
          *(u32x2*)&g.Q[pos * g.ldq + col] = qg;
          *(u32x2*)&g.Q[pos * g.ldq + g.f + col] = qu;
          if ((cc & 15) == 0) {
            g.QS[(col / 128) * g.qs_kstride + pos] = sg_;
            g.QS[((g.f + col) / 128) * g.qs_kstride + pos] = su_;
          }
          if (cc == 0) g.dwp[nt * g.dwp_stride + pos] = part;
        }
      }
    } else {
      for (int id = tid; id < BR * CH; id += NTH) {
        const int q = id / CH, cc = id % CH;
        const int lr = tile_row(q);
        if (lr < mrows) {
          const float* cp = &cband[q * CPAD + cc * 8];
          const uint4 o = make_uint4(pack_bf16x2(cp[0], cp[1]), pack_bf16x2(cp[2], cp[3]),
                                     pack_bf16x2(cp[4], cp[5]), pack_bf16x2(cp[6], cp[7]));
          *(uint4*)&g.C0[(int64_t)s_slot[lr] * g.ldc0 + n0 + cc * 8] = o;
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------- host launchers
namespace {
template <int MODE>
hipError_t run_fp8(const Fp8Args& g, int64_t A, int E, int nN, hipStream_t st) {
  const int64_t blocks = (int64_t)max_row_tiles(A, E, kFp8BM) * nN;
  if (blocks == 0) return hipSuccess;
  grouped_gemm_fp8_kernel<MODE><<<(unsigned)blocks, 512, 0, st>>>(g);
  return hipGetLastError();
}
Fp8Args fp8_base(const MoeShape& s, const int32_t* offsets, const int32_t* perm, const int2* tiles,
                 const int32_t* ntiles) {
  Fp8Args g{};
  g.kslots = s.k;
  g.f = s.f;
  g.offsets = offsets;
  g.perm = perm;
  g.tiles = tiles;
  g.ntiles = ntiles;
  return g;
}
}  // namespace

hipError_t launch_fp8_up(const MoeShape& s, const uint8_t* x, const float* xs, const uint8_t* W1, const float* W1s,
                         const float* topk_w, const int32_t* offsets, const int32_t* perm, const int2* tiles,
                         const int32_t* ntiles, uint16_t* H, uint16_t* As, uint8_t* Asq, float* Ass, hipStream_t st) {
  Fp8Args g = fp8_base(s, offsets, perm, tiles, ntiles);
  g.A = x;
  g.lda = s.d;
  g.A_scale = xs;  // sorted by launch_kstep_sort
  g.as_kstride = (int)(s.T * s.k);
  g.gatherA = 1;
  g.B = W1;
  g.ldb = 2 * (int64_t)s.f;
  g.b_estride = (int64_t)s.d * 2 * s.f;
  g.B_scale = W1s;
  g.bs_estride = (int64_t)(s.d / 128) * (2 * s.f / 128);
  g.bs_ld = 2 * s.f / 128;
  g.N = 2 * s.f;
  g.K = s.d;
  g.topk_w = topk_w;
  g.C0 = H;
  g.ldc0 = 2 * (int64_t)s.f;
  g.C1 = As;
  g.ldc1 = s.f;
  g.Q = Asq;
  g.ldq = s.f;
  g.QS = Ass;
  g.qs_kstride = s.T * s.k;
  return run_fp8<F_UP>(g, (int64_t)s.T * s.k, s.E, s.f / 128, st);
}

hipError_t launch_fp8_down(const MoeShape& s, const uint8_t* Asq, const float* Ass, const uint8_t* W2,
                           const float* W2s, const int32_t* offsets, const int32_t* perm, const int2* tiles,
                           const int32_t* ntiles, uint16_t* Op, hipStream_t st) {
  Fp8Args g = fp8_base(s, offsets, perm, tiles, ntiles);
  g.A = Asq;
  g.lda = s.f;
  g.A_scale = Ass;
  g.as_kstride = (int)(s.T * s.k);
  g.B = W2;
  g.ldb = s.d;
  g.b_estride = (int64_t)s.f * s.d;
  g.B_scale = W2s;
  g.bs_estride = (int64_t)(s.f / 128) * (s.d / 128);
  g.bs_ld = s.d / 128;
  g.N = s.d;
  g.K = s.f;
  g.C0 = Op;
  g.ldc0 = s.d;
  return run_fp8<F_DOWN>(g, (int64_t)s.T * s.k, s.E, s.d / 256, st);
}

hipError_t launch_fp8_dact(const MoeShape& s, const uint8_t* dyq, const float* dys, const uint8_t* W2,
                           const float* W2s, const uint16_t* H, const float* topk_w, const int32_t* offsets,
                           const int32_t* perm, const int2* tiles, const int32_t* ntiles, uint16_t* dH, uint8_t* dHq,
                           float* dHs, float* dwp, hipStream_t st) {
  Fp8Args g = fp8_base(s, offsets, perm, tiles, ntiles);
  g.A = dyq;
  g.lda = s.d;
  g.A_scale = dys;  // sorted by launch_kstep_sort
  g.as_kstride = (int)(s.T * s.k);
  g.gatherA = 1;
  g.B = W2;  // row n of W2[e] ([f, d]) is column n of W2[e]^T, contiguous in K = d
  g.ldb = s.d;
  g.b_estride = (int64_t)s.f * s.d;
  g.B_scale = W2s;
  g.bs_estride = (int64_t)(s.f / 128) * (s.d / 128);
  g.bs_ld = s.d / 128;
  g.N = s.f;
  g.K = s.d;
  g.topk_w = topk_w;
  g.Hs = H;
  g.ldh = 2 * (int64_t)s.f;
  g.C0 = dH;
  g.ldc0 = 2 * (int64_t)s.f;
  g.Q = dHq;
  g.ldq = 2 * (int64_t)s.f;
  g.QS = dHs;
  g.qs_kstride = s.T * s.k;
  g.dwp = dwp;
  g.dwp_stride = (int64_t)s.T * s.k;  // one partial per 256-column N tile
  return run_fp8<F_DACT>(g, (int64_t)s.T * s.k, s.E, s.f / 256, st);
}

hipError_t launch_fp8_dx(const MoeShape& s, const uint8_t* dHq, const float* dHs, const uint8_t* W1, const float* W1s,
                         const int32_t* offsets, const int32_t* perm, const int2* tiles, const int32_t* ntiles,
                         uint16_t* dXp, hipStream_t st) {
  Fp8Args g = fp8_base(s, offsets, perm, tiles, ntiles);
  g.A = dHq;
  g.lda = 2 * (int64_t)s.f;
  g.A_scale = dHs;
  g.as_kstride = (int)(s.T * s.k);
  g.B = W1;  // row n of W1[e] ([d, 2f]) is column n of W1[e]^T, contiguous in K = 2f
  g.ldb = 2 * (int64_t)s.f;
  g.b_estride = (int64_t)s.d * 2 * s.f;
  g.B_scale = W1s;
  g.bs_estride = (int64_t)(s.d / 128) * (2 * s.f / 128);
  g.bs_ld = 2 * s.f / 128;
  g.N = s.d;
  g.K = 2 * s.f;
  g.C0 = dXp;
  g.ldc0 = s.d;
  return run_fp8<F_DX>(g, (int64_t)s.T * s.k, s.E, s.d / 256, st);
}

// ------------------------------------------------------------------ fp8 data movement
// dy (bf16) -> e4m3 with one scale per row per 128 values; 16 threads per block of 128.
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ src, int64_t n8, int cols,
                                                         uint8_t* __restrict__ q, float* __restrict__ qs) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one 8-value group per thread
  const bool ok = i < n8;
  const int64_t ii = ok ? i : 0;
  const uint4 v = load_once16(src + ii * 8);
  float f[8] = {lo_bf16(v.x), hi_bf16(v.x), lo_bf16(v.y), hi_bf16(v.y),
                lo_bf16(v.z), hi_bf16(v.z), lo_bf16(v.w), hi_bf16(v.w)};
  float sc;
  const u32x2 qv = quant8_group16(f, &sc);
  if (ok) {
    *(u32x2*)(q + ii * 8) = qv;
    if ((ii & 15) == 0) {
      const int64_t row = (ii * 8) / cols, blk = ((ii * 8) % cols) / 128;
      qs[row * (cols / 128) + blk] = sc;
    }
  }
}

hipError_t launch_quant_rows(const uint16_t* src, int64_t rows, int cols, uint8_t* q, float* qs, hipStream_t st) {
  const int64_t n8 = rows * cols / 8;
  if (n8 == 0) return hipSuccess;
  quant_rows_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(src, n8, cols, q, qs);
  return hipGetLastError();
}

// e4m3 codes with one fp32 scale per row per 128 values -> bf16 (code * scale in fp32, one RNE
// rounding).  One thread per 8 values: an 8-byte load, a 16-byte store.
__global__ __launch_bounds__(256) void dequant_rows_kernel(const uint8_t* __restrict__ q, const float* __restrict__ qs,
                                                           int64_t n8, int cols, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const int64_t e0 = i * 8, row = e0 / cols;
  const float sc = qs[row * (cols / 128) + (e0 % cols) / 128];  // the 8 values share one 128-block
  const u32x2 w = *(const u32x2*)(q + e0);
  uint32_t o[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t word = h ? w.y : w.x;
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
    o[2 * h] = pack_bf16x2(a[0] * sc, a[1] * sc);
    o[2 * h + 1] = pack_bf16x2(b[0] * sc, b[1] * sc);
  }
  *(uint4*)(out + e0) = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_dequant_rows(const uint8_t* q, const float* qs, int64_t rows, int cols, uint16_t* out,
                               hipStream_t st) {
  const int64_t n8 = rows * cols / 8;
  if (n8 == 0) return hipSuccess;
  dequant_rows_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(q, qs, n8, cols, out);
  return hipGetLastError();
}

}  // namespace moe
