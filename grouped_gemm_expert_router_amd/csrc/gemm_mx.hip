// MXFP8 ragged grouped GEMMs and quantisers for gfx950.  MXFP8 (named on the JAX MoE page,
// "Az NVIDIA szerint tízszer gyorsabb lett a dropless MoE tanítása JAX-ban", section
// "Csoportosított mátrixszorzás és összevont adatmozgatás", and on the TE MoE page,
// "NVIDIA מציגה דרך יעילה לאמן מודלי MoE בביולוגיה", section "צמצום הזיכרון ותקורות הכימות")
// shares one power-of-two scale per 32 consecutive values.  Here the blocks run along each
// GEMM's K, so the E8M0 exponents go straight into the per-lane scale operands of
// v_mfma_scale_f32_32x32x64_f8f6f4: in a 32x32x64 step lane l gives the exponent of row
// (column) l % 32 for k block l / 32 of the step, and its 32 operand bytes are two 16-byte
// halves, one from each block (read_k*8_mx).  No software promotion is needed.
//
// Inputs stay 16-bit (the master weights): the quantisers below produce, per call, x and dy in
// row blocks (K = d), W1 and W2 in column blocks for the forward (K = d and f) and in row blocks
// for the data gradients (K = 2f and d).  The epilogues requantise As (K = f of the down
// projection) and dH (K = 2f of dX) the same way.  The block exponent is the smallest power of
// two that brings the block's maximum magnitude within 448, so no element is clipped.  The
// exponents of a row-blocked operand are kept as 32-bit words by k step (see MxArgs), so a
// stage's DMA reads those of 32 rows as one contiguous run.
//
// Tiles are 256 x 256 x 128 (four scale blocks per stage) with 8 waves (2 x 4) of 128 x 64.
#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace moe {

enum MxMode { X_UP = 0, X_DOWN = 1, X_DACT = 2, X_DX = 3 };

#ifndef MX_GM
#define MX_GM 8
#endif

// Exponents of a row-blocked (KM) operand are kept by k step: the 32-bit word (t, r) at
// byte 4 * (t * R + r) holds the E8M0 bytes of k blocks 4t .. 4t+3 of row r (R rows, K/128
// steps).  A 128-deep step of a tile then takes its rows' exponents from one contiguous run
// (128 bytes per 32 rows) instead of one cache line per row.
struct MxArgs {
  const uint8_t* A;   // e4m3 rows, K contiguous
  int64_t lda;        // bytes
  const uint8_t* Ae;  // E8M0 words by k step, rows in the experts' sorted order
  int64_t ae_kstride;  // bytes from one k step's words to the next (4 * rows of the buffer)
  const uint8_t* B;   // e4m3 weights of all experts
  int64_t ldb, b_estride;
  const uint8_t* Be;  // E8M0 per expert: KN weights [K/32, N] bytes, KM weights words by k step
  int64_t lde_b, be_estride;  // KN: bytes per exponent row; KM: bytes per k step (4 N)
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
  uint8_t* Q;   // requantised output codes (UP: As, DACT: dH)
  int64_t ldq;
  uint8_t* Qe;  // their E8M0 exponents, one per 32 columns, words by k step as Ae
  int64_t qe_kstride;
  const uint16_t* Hs;
  int64_t ldh;
  float* dwp;  // d_topk_w partials, part-major: dwp[part * dwp_stride + pos]
  int64_t dwp_stride;
};

// Shared exponent s of a block with maximum magnitude amax: the smallest s with
// amax <= 448 * 2^s, limited to [-127, 127]; 0 for an all-zero block.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int ex;
  (void)frexpf(amax, &ex);  // amax = m 2^ex, m in [0.5, 1)
  int s = ex - 9;           // 2^(s+8) <= amax < 2^(s+9)
  if (amax > ldexpf(448.0f, s)) ++s;
  return min(max(s, -127), 127);
}

// Quantise 8 values of a 32-value block held by 4 consecutive lanes: returns the 8 e4m3 codes
// and sets *e to the block's E8M0 byte.
__device__ __forceinline__ u32x2 mx_quant8_group4(const float (&v)[8], uint32_t* e) {
  float m = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(v[t]));
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  const int s = mx_exponent(m);
  const float inv = ldexpf(1.0f, -s);  // exact: a power of two
  *e = (uint32_t)(s + 127);
  u32x2 q;
  q.x = pack_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  q.y = pack_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  return q;
}

template <int MODE>
__global__ __launch_bounds__(512, 1) void grouped_gemm_mx_kernel(const MxArgs g) {
  constexpr int BM = kFp8BM, BN = 256, BK = 128, S = 2, WM = 2, WN = 4, NW = 8, NTH = 512;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr bool B_KN = (MODE == X_UP || MODE == X_DOWN);
  constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK, AE_BYTES = NW * 256, BE_BYTES = B_KN ? 4 * 256 : NW * 256;
  constexpr int STAGE = A_BYTES + B_BYTES + AE_BYTES + BE_BYTES;
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
  const int nN = (MODE == X_UP) ? g.f / (BN / 2) : g.N / BN;
  const int G_valid = *(const CONST_AS int32_t*)g.ntiles * nN;
  if ((int)blockIdx.x >= G_valid) return;
  const int lid = xcd_remap(blockIdx.x, G_valid);
  const int2 rc = grouped_tile(lid, G_valid / nN, nN, nN < 8 ? 1 : MX_GM);
  const int nt = rc.y;
  const int2 te = g.tiles[rc.x];
  const int e = te.x;
  const int m0 = g.offsets[e] + te.y * BM;
  const int mrows = min(BM, g.offsets[e + 1] - m0);
  const int n0 = (MODE == X_UP) ? nt * (BN / 2) : nt * BN;
  for (int r = tid; r < BM; r += NTH) {
    int p = -1;
    float wv = 0.0f;
    if (r < mrows) {
      p = g.perm[m0 + r];
      if (MODE == X_UP || MODE == X_DACT) wv = g.topk_w[p];
    }
    s_slot[r] = p;
    s_w[r] = wv;
  }
  const uint8_t* Bexp = g.B + (int64_t)e * g.b_estride;
  const uint8_t* Beexp = g.Be + (int64_t)e * g.be_estride;

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
  // A exponents: wave w brings the word (k blocks of the stage) of rows 32w..32w+31, 128
  // contiguous bytes of the sorted order; lanes past 31 repeat row 32w + 31.
  const uint8_t* ae_src;
  {
    const int row = 32 * wave + min(lane, 31);
    ae_src = g.Ae + (int64_t)(m0 + (row < mrows ? row : 0)) * 4;
  }
  const uint8_t* b_src[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    if constexpr (B_KN) {
      const int kr = 4 * (wave * QB + q) + lane / 16;
      const int c = (lane % 16) ^ (2 * (kr & 7));
      int col;
      if constexpr (MODE == X_UP) col = c < 8 ? n0 + 16 * c : g.f + n0 + 16 * (c - 8);
      else col = n0 + 16 * c;
      b_src[q] = Bexp + (int64_t)kr * g.ldb + col;
    } else {
      const int row = 8 * (wave * QB + q) + lane / 8;
      const int c = (lane % 8) ^ ((row >> 1) & 7);
      b_src[q] = Bexp + (int64_t)(n0 + row) * g.ldb + 16 * c;
    }
  }
  // B exponents.  KN: rows kb = 4t..4t+3 of [K/32, N], 256 tile columns each; wave w < 4 brings
  // row w, lane l columns 4l..4l+3 (UP: lanes < 32 gate, others up).  KM: like A, the words of
  // W's rows n0 + 32w ..
  const uint8_t* be_src;
  if constexpr (B_KN) {
    int col;
    if constexpr (MODE == X_UP) col = lane < 32 ? n0 + 4 * lane : g.f + n0 + 4 * (lane - 32);
    else col = n0 + 4 * lane;
    be_src = Beexp + (int64_t)(wave & 3) * g.lde_b + col;
  } else {
    be_src = Beexp + (int64_t)(n0 + 32 * wave + min(lane, 31)) * 4;
  }
  auto issue = [&](int t, int st) __attribute__((always_inline)) {
    const int k0 = t * BK;
    const uint32_t abase = lds0 + st * STAGE, bbase = abase + A_BYTES, aebase = bbase + B_BYTES,
                   bebase = aebase + AE_BYTES;
#pragma unroll
    for (int q = 0; q < QA; ++q) dma16(a_src[q] + k0, abase + (wave * QA + q) * 1024);
#pragma unroll
    for (int q = 0; q < QB; ++q)
      dma16(B_KN ? b_src[q] + (int64_t)k0 * g.ldb : b_src[q] + k0, bbase + (wave * QB + q) * 1024);
    dma4(ae_src + (int64_t)t * g.ae_kstride, aebase + wave * 256);
    if constexpr (B_KN) {
      if (wave < 4) dma4(be_src + (int64_t)(4 * t) * g.lde_b, bebase + wave * 256);
    } else {
      dma4(be_src + (int64_t)t * g.lde_b, bebase + wave * 256);
    }
  };

  auto b_row = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (MODE == X_UP)
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

  // Lane l of a 64-deep step kk gives the exponent of k block 2*kk + l/32 of the stage for its
  // row (column); the fragments are read in the matching k order (read_k*8_mx).
  const int kbsel = lane >> 5;
  auto compute = [&](int st) __attribute__((always_inline)) {
    const uint32_t abase = lds0 + st * STAGE, bbase = abase + A_BYTES, aebase = bbase + B_BYTES,
                   bebase = aebase + AE_BYTES;
    i32x8 bv[2][FN];
    uint32_t sbw[2][FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = b_row(j) + (lane & 31);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if constexpr (B_KN) bv[kk][j] = read_kn8_mx(bbase, b_row(j), kk, lane);
        else bv[kk][j] = read_km8_mx(bbase, col, kk, lane);
      }
      if constexpr (B_KN) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          sbw[kk][j] = *(const LDS_AS uint8_t*)(uintptr_t)(bebase + (2 * kk + kbsel) * 256 + col);
      } else {
        const uint32_t dw = *(const LDS_AS uint32_t*)(uintptr_t)(bebase + (col >> 5) * 256 + (col & 31) * 4);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) sbw[kk][j] = (dw >> (8 * (2 * kk + kbsel))) & 0xFFu;
      }
    }
    // A fragments one (row fragment, k half) step ahead: the LDS read of step q + 1 is in
    // flight while the MFMAs of step q run (reads retire in order, so each MFMA waits for its own
    // fragment only)
    auto arow = [&](int i) __attribute__((always_inline)) { return wm * TM + i * 32 + (lane & 31); };
    auto a_exp = [&](int i) __attribute__((always_inline)) {
      return *(const LDS_AS uint32_t*)(uintptr_t)(aebase + (arow(i) >> 5) * 256 + (arow(i) & 31) * 4);
    };
    i32x8 af = read_km8_mx(abase, arow(0), 0, lane);
    uint32_t adw = a_exp(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 2 * FM; ++q) {
      const int i = q >> 1, kk = q & 1;
      i32x8 af_next;
      uint32_t adw_next = adw;
      if (q + 1 < 2 * FM) {
        af_next = read_km8_mx(abase, arow((q + 1) >> 1), (q + 1) & 1, lane);
        if (kk == 1) adw_next = a_exp(i + 1);
      }
      const int sa = (int)((adw >> (8 * (2 * kk + kbsel))) & 0xFFu);
      __builtin_amdgcn_sched_barrier(0);  // keep the next step's reads ahead of these MFMAs
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bv[kk][j], acc[i][j], 0, 0, 0, sa, 0,
                                                                    (int)sbw[kk][j]);
      __builtin_amdgcn_sched_barrier(0);
      if (q + 1 < 2 * FM) {
        af = af_next;
        adw = adw_next;
      }
    }
  };

  // ------------------------------------------------------------------ main loop (2 stages)
  const int nk = g.K / BK;
  // In an expert's last row tile, a wave whose rows all lie past the expert's end skips its
  // fragment reads and MFMAs (uniform: mrows and wm are); it still issues its DMA share.
  const bool busy = __builtin_amdgcn_readfirstlane(wm * TM < mrows);
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
  static_assert(FM % PH == 0 && (MODE != X_DACT || ITEMS * NTH == BR * CH), "epilogue band");
#pragma unroll
  for (int ph = 0; ph < FM / PH; ++ph) {
    // band row q: wave row q / (32*PH), row fragment PH*ph + (q % (32*PH)) / 32, row q % 32
    auto tile_row = [&](int q) __attribute__((always_inline)) {
      return (q / (32 * PH)) * TM + 32 * (PH * ph + (q % (32 * PH)) / 32) + (q & 31);
    };
    // DACT: the phase's H loads go out before the band is written, so their latency hides
    // behind the band writes and the barrier
    uint4 hgv[ITEMS], huv[ITEMS];
    if constexpr (MODE == X_DACT) {
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
        const int i = PH * ph + ii, c = b_row(j) + lcol;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = 32 * PH * wm + 32 * ii + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          cband[q * CPAD + c] = acc[i][j][r];
        }
      }
    __syncthreads();
    if constexpr (MODE == X_UP) {
      // 16 lanes per row, 8 gate + 8 up columns each; 4 lanes form one 32-column block of As
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
        uint32_t ex;
        const u32x2 qv = mx_quant8_group4(as, &ex);
        if (ok) {
          const int64_t pos = m0 + lr;
          const int col = n0 + cc * 8;
          *(uint4*)&g.C0[pos * g.ldc0 + col] = make_uint4(hg[0], hg[1], hg[2], hg[3]);
          *(uint4*)&g.C0[pos * g.ldc0 + g.f + col] = make_uint4(hu[0], hu[1], hu[2], hu[3]);
          *(uint4*)&g.C1[pos * g.ldc1 + col] = make_uint4(ab[0], ab[1], ab[2], ab[3]);
          *(u32x2*)&g.Q[pos * g.ldq + col] = qv;
          if ((cc & 3) == 0) g.Qe[(col >> 7) * g.qe_kstride + pos * 4 + ((col >> 5) & 3)] = (uint8_t)ex;
        }
      }
    } else if constexpr (MODE == X_DACT) {
      // 32 lanes per row (8 columns each): dSwiGLU, routing-weight partial, dH in bf16 and MXFP8
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
        uint32_t eg, eu;
        const u32x2 qg = mx_quant8_group4(dg, &eg);
        const u32x2 qu = mx_quant8_group4(du, &eu);
#pragma unroll
        for (int m = CH / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
        if (ok) {
          *(uint4*)&g.C0[pos * g.ldc0 + col] = make_uint4(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]),
                                                          pack_bf16x2(dg[4], dg[5]), pack_bf16x2(dg[6], dg[7]));
          *(uint4*)&g.C0[pos * g.ldc0 + g.f + col] = make_uint4(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]),
                                                                pack_bf16x2(du[4], du[5]), pack_bf16x2(du[6], du[7]));
          *(u32x2*)&g.Q[pos * g.ldq + col] = qg;
          *(u32x2*)&g.Q[pos * g.ldq + g.f + col] = qu;
          if ((cc & 3) == 0) {
            const int cu = g.f + col;
            g.Qe[(col >> 7) * g.qe_kstride + pos * 4 + ((col >> 5) & 3)] = (uint8_t)eg;
            g.Qe[(cu >> 7) * g.qe_kstride + pos * 4 + ((cu >> 5) & 3)] = (uint8_t)eu;
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

// ---------------------------------------------------------------------- quantisers
// Row blocks: src bf16 [rows, cols] -> codes [rows, cols], exponents [rows, cols/32]; four
// threads per 32-value block, eight values each.
__global__ __launch_bounds__(256) void mx_quant_rows_kernel(const uint16_t* __restrict__ src, int64_t n8, int cols,
                                                            uint8_t* __restrict__ q, uint8_t* __restrict__ qe) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool ok = i < n8;
  const int64_t ii = ok ? i : 0;
  const uint4 v = load_once16(src + ii * 8);
  float f[8] = {lo_bf16(v.x), hi_bf16(v.x), lo_bf16(v.y), hi_bf16(v.y),
                lo_bf16(v.z), hi_bf16(v.z), lo_bf16(v.w), hi_bf16(v.w)};
  uint32_t ex;
  const u32x2 qv = mx_quant8_group4(f, &ex);
  if (ok) {
    *(u32x2*)(q + ii * 8) = qv;
    if ((ii & 3) == 0) qe[(ii * 8) / 32] = (uint8_t)ex;  // cols % 32 == 0: blocks never straddle rows
  }
}

// Column blocks within each matrix of a batch: src bf16 [batch, rows, cols] -> codes of the same
// shape, exponents [batch, rows/32, cols].  One thread per 32 rows x 8 columns.
__global__ __launch_bounds__(256) void mx_quant_cols_kernel(const uint16_t* __restrict__ src, int64_t nunits,
                                                            int rows, int cols, uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ qe) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= nunits) return;
  const int c8 = cols / 8;
  const int64_t per_mat = (int64_t)(rows / 32) * c8;
  const int64_t b = u / per_mat;
  const int64_t rem = u % per_mat;
  const int rb = (int)(rem / c8), cc = (int)(rem % c8);
  const int64_t base = (b * rows + (int64_t)rb * 32) * cols + cc * 8;
  float amax[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = 0; r < 32; ++r) {
    const uint4 v = *(const uint4*)(src + base + (int64_t)r * cols);
    const float f[8] = {lo_bf16(v.x), hi_bf16(v.x), lo_bf16(v.y), hi_bf16(v.y),
                        lo_bf16(v.z), hi_bf16(v.z), lo_bf16(v.w), hi_bf16(v.w)};
#pragma unroll
    for (int t = 0; t < 8; ++t) amax[t] = fmaxf(amax[t], fabsf(f[t]));
  }
  int s[8];
  float inv[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    s[t] = mx_exponent(amax[t]);
    inv[t] = ldexpf(1.0f, -s[t]);
  }
  for (int r = 0; r < 32; ++r) {
    const uint4 v = *(const uint4*)(src + base + (int64_t)r * cols);
    const float f[8] = {lo_bf16(v.x), hi_bf16(v.x), lo_bf16(v.y), hi_bf16(v.y),
                        lo_bf16(v.z), hi_bf16(v.z), lo_bf16(v.w), hi_bf16(v.w)};
    u32x2 o;
    o.x = pack_e4m3x4(f[0] * inv[0], f[1] * inv[1], f[2] * inv[2], f[3] * inv[3]);
    o.y = pack_e4m3x4(f[4] * inv[4], f[5] * inv[5], f[6] * inv[6], f[7] * inv[7]);
    *(u32x2*)(q + base + (int64_t)r * cols) = o;
  }
  uint8_t* eo = qe + (b * (rows / 32) + rb) * (int64_t)cols + cc * 8;
  u32x2 ev;
  ev.x = (uint32_t)(s[0] + 127) | ((uint32_t)(s[1] + 127) << 8) | ((uint32_t)(s[2] + 127) << 16) |
         ((uint32_t)(s[3] + 127) << 24);
  ev.y = (uint32_t)(s[4] + 127) | ((uint32_t)(s[5] + 127) << 8) | ((uint32_t)(s[6] + 127) << 16) |
         ((uint32_t)(s[7] + 127) << 24);
  *(u32x2*)eo = ev;
}

// Both orientations in one pass (a weight matrix read once): src bf16 [batch, rows, cols] ->
// qc/qce in column blocks (exponents [batch, rows/32, cols]) and qr/qre in row blocks
// (exponents as words by k step, [batch, cols/128, rows] words).  One block of 256 threads per 32 x 256 tile: thread t owns
// 4 rows (group t / 32) x 8 columns (chunk t % 32).  Row blocks: 4 neighbouring lanes.  Column
// blocks: the 8 row groups' maxima meet in LDS.
__global__ __launch_bounds__(256) void mx_quant_dual_kernel(const uint16_t* __restrict__ src, int rows, int cols,
                                                            uint8_t* __restrict__ qc, uint8_t* __restrict__ qce,
                                                            uint8_t* __restrict__ qr, uint8_t* __restrict__ qre) {
  __shared__ float s_amax[8][256];
  __shared__ uint8_t s_rex[32][8];  // row-block exponents of the tile: [row][block]
  const int t = threadIdx.x, cc = t & 31, rg = t >> 5;
  const int tiles_c = cols / 256, tiles_r = rows / 32;
  const int64_t b = blockIdx.x / (tiles_r * tiles_c);
  const int rem = blockIdx.x % (tiles_r * tiles_c);
  const int r0 = (rem / tiles_c) * 32, c0 = (rem % tiles_c) * 256 + cc * 8;
  const int64_t mat = b * (int64_t)rows * cols;
  float v[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = *(const uint4*)(src + mat + (int64_t)(r0 + 4 * rg + i) * cols + c0);
    v[i][0] = lo_bf16(w.x); v[i][1] = hi_bf16(w.x); v[i][2] = lo_bf16(w.y); v[i][3] = hi_bf16(w.y);
    v[i][4] = lo_bf16(w.z); v[i][5] = hi_bf16(w.z); v[i][6] = lo_bf16(w.w); v[i][7] = hi_bf16(w.w);
  }
  // row blocks (32 columns = 4 lanes); their exponents meet in LDS and leave below as two runs
  // of 32 words (one per k step of the tile's 256 columns)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t ex;
    const u32x2 q = mx_quant8_group4(v[i], &ex);
    const int64_t row = r0 + 4 * rg + i;
    *(u32x2*)(qr + mat + row * cols + c0) = q;
    if ((cc & 3) == 0) s_rex[4 * rg + i][cc >> 2] = (uint8_t)ex;
  }
  // column blocks (32 rows = 8 row groups)
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(v[i][c]));
    s_amax[rg][cc * 8 + c] = m;
  }
  __syncthreads();
  if (t < 64) {
    const int h = t >> 5, r = t & 31;
    const int64_t kstep = (int64_t)(rem % tiles_c) * 2 + h;
    *(uint32_t*)(qre + ((b * (cols / 128) + kstep) * rows + r0 + r) * 4) = *(const uint32_t*)&s_rex[r][4 * h];
  }
  float inv[8];
  int sx[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float m = 0.0f;
#pragma unroll
    for (int g = 0; g < 8; ++g) m = fmaxf(m, s_amax[g][cc * 8 + c]);
    sx[c] = mx_exponent(m);
    inv[c] = ldexpf(1.0f, -sx[c]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x2 o;
    o.x = pack_e4m3x4(v[i][0] * inv[0], v[i][1] * inv[1], v[i][2] * inv[2], v[i][3] * inv[3]);
    o.y = pack_e4m3x4(v[i][4] * inv[4], v[i][5] * inv[5], v[i][6] * inv[6], v[i][7] * inv[7]);
    *(u32x2*)(qc + mat + (int64_t)(r0 + 4 * rg + i) * cols + c0) = o;
  }
  if (rg == 0) {
    u32x2 ev;
    ev.x = (uint32_t)(sx[0] + 127) | ((uint32_t)(sx[1] + 127) << 8) | ((uint32_t)(sx[2] + 127) << 16) |
           ((uint32_t)(sx[3] + 127) << 24);
    ev.y = (uint32_t)(sx[4] + 127) | ((uint32_t)(sx[5] + 127) << 8) | ((uint32_t)(sx[6] + 127) << 16) |
           ((uint32_t)(sx[7] + 127) << 24);
    *(u32x2*)(qce + (b * (rows / 32) + r0 / 32) * (int64_t)cols + c0) = ev;
  }
}

// The same for cols % 512 == 0 with 32 x 512 tiles: thread t owns 4 rows (group t / 32) x 16
// columns (chunk t % 32), so every code store is 16 bytes.  Row blocks: 2 neighbouring lanes.
// Column blocks: the 8 row groups' maxima meet in LDS; thread t reduces columns 2t and 2t+1.
__global__ __launch_bounds__(256) void mx_quant_dual16_kernel(const uint16_t* __restrict__ src, int rows, int cols,
                                                              uint8_t* __restrict__ qc, uint8_t* __restrict__ qce,
                                                              uint8_t* __restrict__ qr, uint8_t* __restrict__ qre) {
  __shared__ float s_amax[8][512];
  __shared__ int s_cex[512];         // column-block exponents s of the tile's 512 columns
  __shared__ uint8_t s_rex[32][16];  // row-block exponent bytes: [row][block]
  const int t = threadIdx.x, cc = t & 31, rg = t >> 5;
  const int tiles_c = cols / 512, tiles_r = rows / 32;
  const int64_t b = blockIdx.x / (tiles_r * tiles_c);
  const int rem = blockIdx.x % (tiles_r * tiles_c);
  const int r0 = (rem / tiles_c) * 32, tc = rem % tiles_c, c0 = tc * 512 + cc * 16;
  const int64_t mat = b * (int64_t)rows * cols;
  float v[4][16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t* p = src + mat + (int64_t)(r0 + 4 * rg + i) * cols + c0;
    const uint4 w0 = *(const uint4*)p, w1 = *(const uint4*)(p + 8);
    const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      v[i][2 * q] = lo_bf16(w[q]);
      v[i][2 * q + 1] = hi_bf16(w[q]);
    }
  }
  // row blocks: 32 columns = lanes cc and cc ^ 1
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) m = fmaxf(m, fabsf(v[i][c]));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    const int sx = mx_exponent(m);
    const float inv = ldexpf(1.0f, -sx);  // exact: a power of two
    uint4 o;
    o.x = pack_e4m3x4(v[i][0] * inv, v[i][1] * inv, v[i][2] * inv, v[i][3] * inv);
    o.y = pack_e4m3x4(v[i][4] * inv, v[i][5] * inv, v[i][6] * inv, v[i][7] * inv);
    o.z = pack_e4m3x4(v[i][8] * inv, v[i][9] * inv, v[i][10] * inv, v[i][11] * inv);
    o.w = pack_e4m3x4(v[i][12] * inv, v[i][13] * inv, v[i][14] * inv, v[i][15] * inv);
    *(uint4*)(qr + mat + (int64_t)(r0 + 4 * rg + i) * cols + c0) = o;
    if ((cc & 1) == 0) s_rex[4 * rg + i][cc >> 1] = (uint8_t)(sx + 127);
  }
  // column blocks: this thread's maxima over its 4 rows, then over the 8 row groups
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(v[i][c]));
    s_amax[rg][cc * 16 + c] = m;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int col = 2 * t + h;
    float m = 0.0f;
#pragma unroll
    for (int g = 0; g < 8; ++g) m = fmaxf(m, s_amax[g][col]);
    s_cex[col] = mx_exponent(m);
  }
  if (t < 128) {  // row-block exponent words: 4 k steps of 128 columns x 32 rows
    const int h = t >> 5, r = t & 31;
    const int64_t kstep = (int64_t)tc * 4 + h;
    *(uint32_t*)(qre + ((b * (cols / 128) + kstep) * rows + r0 + r) * 4) = *(const uint32_t*)&s_rex[r][4 * h];
  }
  __syncthreads();
  float inv[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) inv[c] = ldexpf(1.0f, -s_cex[cc * 16 + c]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 o;
    o.x = pack_e4m3x4(v[i][0] * inv[0], v[i][1] * inv[1], v[i][2] * inv[2], v[i][3] * inv[3]);
    o.y = pack_e4m3x4(v[i][4] * inv[4], v[i][5] * inv[5], v[i][6] * inv[6], v[i][7] * inv[7]);
    o.z = pack_e4m3x4(v[i][8] * inv[8], v[i][9] * inv[9], v[i][10] * inv[10], v[i][11] * inv[11]);
    o.w = pack_e4m3x4(v[i][12] * inv[12], v[i][13] * inv[13], v[i][14] * inv[14], v[i][15] * inv[15]);
    *(uint4*)(qc + mat + (int64_t)(r0 + 4 * rg + i) * cols + c0) = o;
  }
  if (t < 128) {  // column-block exponents: 4 bytes per thread
    uint32_t ev = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) ev |= (uint32_t)(s_cex[4 * t + j] + 127) << (8 * j);
    *(uint32_t*)(qce + (b * (rows / 32) + r0 / 32) * (int64_t)cols + tc * 512 + 4 * t) = ev;
  }
}

hipError_t launch_mx_quant_dual(const uint16_t* src, int64_t batch, int rows, int cols, uint8_t* qc, uint8_t* qce,
                                uint8_t* qr, uint8_t* qre, hipStream_t st) {
  if (cols % 512 == 0) {
    const int64_t blocks = batch * (rows / 32) * (cols / 512);
    if (blocks == 0) return hipSuccess;
    mx_quant_dual16_kernel<<<(unsigned)blocks, 256, 0, st>>>(src, rows, cols, qc, qce, qr, qre);
    return hipGetLastError();
  }
  const int64_t blocks = batch * (rows / 32) * (cols / 256);
  if (blocks == 0) return hipSuccess;
  mx_quant_dual_kernel<<<(unsigned)blocks, 256, 0, st>>>(src, rows, cols, qc, qce, qr, qre);
  return hipGetLastError();
}

hipError_t launch_mx_quant(const uint16_t* src, int64_t batch, int rows, int cols, int along_rows, uint8_t* q,
                           uint8_t* qe, hipStream_t st) {
  if (batch * rows * cols == 0) return hipSuccess;
  if (!along_rows) {  // blocks of 32 consecutive values of a row
    const int64_t n8 = batch * rows * (int64_t)cols / 8;
    mx_quant_rows_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(src, n8, cols, q, qe);
  } else {            // blocks of 32 consecutive rows of a column
    const int64_t nunits = batch * (int64_t)(rows / 32) * (cols / 8);
    mx_quant_cols_kernel<<<(unsigned)((nunits + 255) / 256), 256, 0, st>>>(src, nunits, rows, cols, q, qe);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------- GEMM launchers
namespace {
template <int MODE>
hipError_t run_mx(const MxArgs& g, int64_t A, int E, int nN, hipStream_t st) {
  const int64_t blocks = (int64_t)max_row_tiles(A, E, kFp8BM) * nN;
  if (blocks == 0) return hipSuccess;
  grouped_gemm_mx_kernel<MODE><<<(unsigned)blocks, 512, 0, st>>>(g);
  return hipGetLastError();
}
MxArgs mx_base(const MoeShape& s, const int32_t* offsets, const int32_t* perm, const int2* tiles,
               const int32_t* ntiles) {
  MxArgs g{};
  g.kslots = s.k;
  g.f = s.f;
  g.offsets = offsets;
  g.perm = perm;
  g.tiles = tiles;
  g.ntiles = ntiles;
  return g;
}
}  // namespace

hipError_t launch_mx_up(const MoeShape& s, const uint8_t* xq, const uint8_t* xe, const uint8_t* W1q,
                        const uint8_t* W1e, const float* topk_w, const int32_t* offsets, const int32_t* perm,
                        const int2* tiles, const int32_t* ntiles, uint16_t* H, uint16_t* As, uint8_t* Asq,
                        uint8_t* Ase, hipStream_t st) {
  MxArgs g = mx_base(s, offsets, perm, tiles, ntiles);
  g.A = xq;
  g.lda = s.d;
  g.Ae = xe;  // sorted by launch_kstep_sort
  g.ae_kstride = 4 * (int64_t)s.T * s.k;
  g.gatherA = 1;
  g.B = W1q;  // [E, d, 2f], column blocks: exponents [E, d/32, 2f]
  g.ldb = 2 * (int64_t)s.f;
  g.b_estride = (int64_t)s.d * 2 * s.f;
  g.Be = W1e;
  g.lde_b = 2 * (int64_t)s.f;
  g.be_estride = (int64_t)(s.d / 32) * 2 * s.f;
  g.N = 2 * s.f;
  g.K = s.d;
  g.topk_w = topk_w;
  g.C0 = H;
  g.ldc0 = 2 * (int64_t)s.f;
  g.C1 = As;
  g.ldc1 = s.f;
  g.Q = Asq;
  g.ldq = s.f;
  g.Qe = Ase;
  g.qe_kstride = 4 * (int64_t)s.T * s.k;
  return run_mx<X_UP>(g, (int64_t)s.T * s.k, s.E, s.f / 128, st);
}

hipError_t launch_mx_down(const MoeShape& s, const uint8_t* Asq, const uint8_t* Ase, const uint8_t* W2q,
                          const uint8_t* W2e, const int32_t* offsets, const int32_t* perm, const int2* tiles,
                          const int32_t* ntiles, uint16_t* Op, hipStream_t st) {
  MxArgs g = mx_base(s, offsets, perm, tiles, ntiles);
  g.A = Asq;
  g.lda = s.f;
  g.Ae = Ase;
  g.ae_kstride = 4 * (int64_t)s.T * s.k;
  g.B = W2q;  // [E, f, d], column blocks: exponents [E, f/32, d]
  g.ldb = s.d;
  g.b_estride = (int64_t)s.f * s.d;
  g.Be = W2e;
  g.lde_b = s.d;
  g.be_estride = (int64_t)(s.f / 32) * s.d;
  g.N = s.d;
  g.K = s.f;
  g.C0 = Op;
  g.ldc0 = s.d;
  return run_mx<X_DOWN>(g, (int64_t)s.T * s.k, s.E, s.d / 256, st);
}

hipError_t launch_mx_dact(const MoeShape& s, const uint8_t* dyq, const uint8_t* dye, const uint8_t* W2q,
                          const uint8_t* W2e, const uint16_t* H, const float* topk_w, const int32_t* offsets,
                          const int32_t* perm, const int2* tiles, const int32_t* ntiles, uint16_t* dH, uint8_t* dHq,
                          uint8_t* dHe, float* dwp, hipStream_t st) {
  MxArgs g = mx_base(s, offsets, perm, tiles, ntiles);
  g.A = dyq;
  g.lda = s.d;
  g.Ae = dye;  // sorted by launch_kstep_sort
  g.ae_kstride = 4 * (int64_t)s.T * s.k;
  g.gatherA = 1;
  g.B = W2q;  // [E, f, d], row blocks (K = d): exponent words [E, d/128, f]
  g.ldb = s.d;
  g.b_estride = (int64_t)s.f * s.d;
  g.Be = W2e;
  g.lde_b = 4 * (int64_t)s.f;
  g.be_estride = (int64_t)s.f * (s.d / 32);
  g.N = s.f;
  g.K = s.d;
  g.topk_w = topk_w;
  g.Hs = H;
  g.ldh = 2 * (int64_t)s.f;
  g.C0 = dH;
  g.ldc0 = 2 * (int64_t)s.f;
  g.Q = dHq;
  g.ldq = 2 * (int64_t)s.f;
  g.Qe = dHe;
  g.qe_kstride = 4 * (int64_t)s.T * s.k;
  g.dwp = dwp;
  g.dwp_stride = (int64_t)s.T * s.k;  // one partial per 256-column N tile
  return run_mx<X_DACT>(g, (int64_t)s.T * s.k, s.E, s.f / 256, st);
}

hipError_t launch_mx_dx(const MoeShape& s, const uint8_t* dHq, const uint8_t* dHe, const uint8_t* W1q,
                        const uint8_t* W1e, const int32_t* offsets, const int32_t* perm, const int2* tiles,
                        const int32_t* ntiles, uint16_t* dXp, hipStream_t st) {
  MxArgs g = mx_base(s, offsets, perm, tiles, ntiles);
  g.A = dHq;
  g.lda = 2 * (int64_t)s.f;
  g.Ae = dHe;
  g.ae_kstride = 4 * (int64_t)s.T * s.k;
  g.B = W1q;  // [E, d, 2f], row blocks (K = 2f): exponent words [E, 2f/128, d]
  g.ldb = 2 * (int64_t)s.f;
  g.b_estride = (int64_t)s.d * 2 * s.f;
  g.Be = W1e;
  g.lde_b = 4 * (int64_t)s.d;
  g.be_estride = (int64_t)s.d * (2 * s.f / 32);
  g.N = s.d;
  g.K = 2 * s.f;
  g.C0 = dXp;
  g.ldc0 = s.d;
  return run_mx<X_DX>(g, (int64_t)s.T * s.k, s.E, s.d / 256, st);
}


// ---------------------------------------------------------------------- weight gradients
// dW2[e] = As_e^T dy_e and dW1[e] = x_e^T dH_e, with K = the expert's rows (ragged K).  Both
// operands are quantised along that K in blocks of 32 rows that stay inside one expert (the
// pages' MXFP8 with group-aware quantisation: JAX MoE page, section "Csoportosított
// mátrixszorzás és összevont adatmozgatás").  Each expert's rows go to a segment of a padded
// buffer that starts at poff[e], a multiple of 128, and is completed with zero rows: a zero row
// leaves a block's maximum unchanged and adds nothing to a product, and no 128-deep K step of
// the GEMM below ever mixes two experts.

// poff[e] = sum over e' < e of count(e') rounded up to 128; poff[E] = the padded total.
__global__ __launch_bounds__(1024) void mx_pad_offsets_kernel(const int32_t* __restrict__ offsets, int E,
                                                             int32_t* __restrict__ poff) {
  __shared__ int sh[64];
  const int e = threadIdx.x;
  const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
  int ex;
  const int tot = block_excl_scan_1024((c + 127) & ~127, sh, &ex);
  if (e < E) poff[e] = ex;
  if (e == 0) poff[E] = tot;
}

// Rows of a source [*, C] in the experts' sorted order -- row perm[pos] / kslots of a
// token-major source when gather, else row pos -- are quantised along the rows into the padded
// segments: codes [P, C], exponents [P / 32, C] (mx_quant_tokens_kernel below).  The source is
// bf16; rows past an expert's count are zero.
// Source row of each of the 32 padded positions pp0.. (-1 for the zero rows that pad an expert's
// segment to a multiple of 128): threads 0..31 fill s_row, then the block synchronises.
__device__ __forceinline__ void token_block_rows(int pp0, int gather, int kslots, const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ perm, const int32_t* __restrict__ poff,
                                                 int E, int64_t* s_row) {
  if (threadIdx.x < 32) {
    // the expert whose segment holds pp0: poff[lo] <= pp0 < poff[hi] throughout
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (poff[mid] <= pp0) lo = mid;
      else hi = mid;
    }
    const int local = pp0 - poff[lo] + (int)threadIdx.x;
    int64_t row = -1;
    if (local < offsets[lo + 1] - offsets[lo]) {
      const int pos = offsets[lo] + local;
      row = gather ? (int64_t)(perm[pos] / kslots) : (int64_t)pos;
    }
    s_row[threadIdx.x] = row;
  }
  __syncthreads();
}

struct MxWgArgs {
  const uint8_t* A;   // codes [P, Mo]: the product's left operand, k-major (row = padded position)
  const uint8_t* Ae;  // exponents [P / 32, Mo]
  const uint8_t* B;   // codes [P, N]
  const uint8_t* Be;  // exponents [P / 32, N]
  int Mo, N;
  const int32_t* poff;
  const int2* units;     // (expert, chunk) work units, largest first
  const int32_t* meta;   // [0] units, [1] chunk rows KC, [2] 1 = bucketed XCD order
  const int32_t* pslot;  // first fp32 partial of a split expert, -1 if not split
  float* partial;
  uint16_t* dW;          // [E, Mo, N] bf16
};

// dW[e] tile (m0, n0) of 256 x 256 over one unit's K range, 128 per stage (four exponent rows
// per operand).  8 waves of 128 x 64; the unit order and XCD bucketing follow the bf16
// weight-gradient kernel.  WHICH only names the launch (0: dW2, 1: dW1) in kernel traces.
template <int WHICH>
__global__ __launch_bounds__(512, 1) void grouped_gemm_mx_wg_kernel(const MxWgArgs g) {
  constexpr int BM = 256, BN = 256, BK = 128, S = 2, WN = 4, NW = 8;
  constexpr int TM = 128, TN = 64, FM = 4, FN = 2;
  constexpr int A_BYTES = BK * BM, B_BYTES = BK * BN, E_BYTES = 4 * 256;
  constexpr int STAGE = A_BYTES + B_BYTES + 2 * E_BYTES;
  constexpr int QA = A_BYTES / (1024 * NW), QB = B_BYTES / (1024 * NW);
  static_assert(QA == 4 && QB == 4, "DMA split");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr_of(smem));

  // ------------------------------------------------------------------ unit and tile
  const int nN = g.N / BN, nM = g.Mo / BM, per_u = nM * nN;
  const CONST_AS int32_t* meta = (const CONST_AS int32_t*)g.meta;
  const int U = meta[0];
  const int G_valid = U * per_u;
  if ((int)blockIdx.x >= G_valid) return;
  int pos = blockIdx.x, u;
  if (meta[2]) {
    // deal the units (largest first) to 8 buckets round-robin; XCD b takes bucket b's tiles
    pos = xcd_remap(blockIdx.x, G_valid);
    const int j = pos / per_u;
    const int q = U / 8, r = U % 8;
    int b, jb;
    if (j < r * (q + 1)) {
      b = j / (q + 1);
      jb = j % (q + 1);
    } else {
      b = r + (j - r * (q + 1)) / q;
      jb = (j - r * (q + 1)) % q;
    }
    u = b + 8 * jb;
  } else {
    u = pos / per_u;
  }
  const CONST_AS int32_t* up = (const CONST_AS int32_t*)g.units;
  const int e = up[2 * u], kchunk = up[2 * u + 1];
  const int t = pos % per_u;
  int m0, nt;
  // Within a unit, the tile index walks the dimension with fewer tiles first, so the tiles that
  // run together cover all of it and share the other operand's rows in L2 (measured: qwen3 dW1
  // and dW2 -2 %, Mixtral dW2 -5 % against walking by tile-count divisibility).
  if (nM <= nN) {
    m0 = (t % nM) * BM;
    nt = t / nM;
  } else {
    nt = t % nN;
    m0 = (t / nN) * BM;
  }
  const int n0 = nt * BN;
  const CONST_AS int32_t* pf = (const CONST_AS int32_t*)g.poff;
  const int KC = meta[1];
  const int kbeg = pf[e] + kchunk * KC;
  const int kend = min(pf[e + 1], kbeg + KC);
  const int pslot = ((const CONST_AS int32_t*)g.pslot)[e];
  const int nk = (kend - kbeg) / BK;  // segments and chunks are multiples of 128 rows

  // ------------------------------------------------------------------ DMA sources
  // Operand instruction q of wave w: k rows 4*(4w+q) .. +3 of the stage, 16 lanes per row;
  // lane l fills physical chunk l % 16 of its row from logical chunk (l % 16) ^ (2 * (row & 7)).
  const uint8_t* a_src[QA];
  const uint8_t* b_src[QB];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int kr = 4 * (wave * QA + q) + lane / 16;
    const int c = (lane % 16) ^ (2 * (kr & 7));
    a_src[q] = g.A + (int64_t)(kbeg + kr) * g.Mo + m0 + 16 * c;
    b_src[q] = g.B + (int64_t)(kbeg + kr) * g.N + n0 + 16 * c;
  }
  // exponent row w % 4 of the stage: waves 0..3 for A, 4..7 for B; lane l brings 4 columns
  const bool e_is_a = wave < 4;
  const uint8_t* e_src = e_is_a ? g.Ae + (int64_t)(kbeg / 32 + wave) * g.Mo + m0 + 4 * lane
                                : g.Be + (int64_t)(kbeg / 32 + wave - 4) * g.N + n0 + 4 * lane;
  const int64_t e_ld = e_is_a ? g.Mo : g.N;
  auto issue = [&](int it, int st) __attribute__((always_inline)) {
    const int k0 = it * BK;
    const uint32_t abase = lds0 + st * STAGE, bbase = abase + A_BYTES, aebase = bbase + B_BYTES,
                   bebase = aebase + E_BYTES;
#pragma unroll
    for (int q = 0; q < QA; ++q) dma16(a_src[q] + (int64_t)k0 * g.Mo, abase + (wave * QA + q) * 1024);
#pragma unroll
    for (int q = 0; q < QB; ++q) dma16(b_src[q] + (int64_t)k0 * g.N, bbase + (wave * QB + q) * 1024);
    dma4(e_src + (int64_t)(k0 / 32) * e_ld, (e_is_a ? aebase : bebase) + (wave & 3) * 256);
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Both operands are k-major: each fragment is a transpose read (read_kn8_mx), and lane l
  // gives the exponent of its row (column) l % 32 for k block 2*kk + l/32 of the stage.  The
  // B fragment is the MFMA's first operand, so the accumulators hold transposed blocks.
  const int kbsel = lane >> 5;
  auto compute = [&](int st) __attribute__((always_inline)) {
    const uint32_t abase = lds0 + st * STAGE, bbase = abase + A_BYTES, aebase = bbase + B_BYTES,
                   bebase = aebase + E_BYTES;
    i32x8 bv[2][FN];
    int sb[2][FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int col = wn * TN + 32 * j;
        bv[kk][j] = read_kn8_mx(bbase, col, kk, lane);
        sb[kk][j] = *(const LDS_AS uint8_t*)(uintptr_t)(bebase + (2 * kk + kbsel) * 256 + col + (lane & 31));
      }
    // A fragments and their exponents one (row fragment, k half) step ahead, as in the
    // ragged-M kernel
    auto a_frag = [&](int q, i32x8& af, int& sa) __attribute__((always_inline)) {
      const int row = wm * TM + 32 * (q >> 1), kk = q & 1;
      af = read_kn8_mx(abase, row, kk, lane);
      sa = *(const LDS_AS uint8_t*)(uintptr_t)(aebase + (2 * kk + kbsel) * 256 + row + (lane & 31));
    };
    i32x8 af;
    int sa;
    a_frag(0, af, sa);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 2 * FM; ++q) {
      const int i = q >> 1, kk = q & 1;
      i32x8 af_next;
      int sa_next = 0;
      if (q + 1 < 2 * FM) a_frag(q + 1, af_next, sa_next);
      __builtin_amdgcn_sched_barrier(0);  // keep the next step's reads ahead of these MFMAs
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv[kk][j], af, acc[i][j], 0, 0, 0, sb[kk][j], 0,
                                                                    sa);
      __builtin_amdgcn_sched_barrier(0);
      if (q + 1 < 2 * FM) {
        af = af_next;
        sa = sa_next;
      }
    }
  };

  // ------------------------------------------------------------------ main loop (2 stages)
  __syncthreads();
  if (nk > 0) issue(0, 0);
  for (int it = 0; it < nk; ++it) {
    vm_lgkm_wait_barrier<0>();
    if (it + 1 < nk) issue(it + 1, (it + 1) % S);
    compute(it % S);
  }

  // ------------------------------------------------------------------ epilogue (registers)
  // Lane l holds dW row m0 + wm*TM + 32*i + l%32 and, for r = 0..15, column
  // n0 + wn*TN + 32*j + 8*(r/4) + 4*(l/32) + r%4.  An empty unit (no rows) stores zeros.
  const int h = lane >> 5, lrow = lane & 31;
  if (pslot >= 0) {
    // one chunk of a split expert: fp32 partial, summed later in chunk order
    float* out = g.partial + (int64_t)(pslot + kchunk) * g.Mo * g.N;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float* orow = out + (int64_t)(m0 + wm * TM + 32 * i + lrow) * g.N + n0 + wn * TN;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(float4*)(orow + 32 * j + 8 * q + 4 * h) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      uint16_t* orow = g.dW + ((int64_t)e * g.Mo + m0 + wm * TM + 32 * i + lrow) * g.N + n0 + wn * TN;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        // bf16 pairs, then lanes l and l+32 trade halves so each holds 8 consecutive columns
        uint32_t p[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          p[q][0] = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
          p[q][1] = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
#pragma unroll
        for (int a = 0; a < 4; a += 2)
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const auto r = __builtin_amdgcn_permlane32_swap(p[a][d], p[a + 1][d], false, false);
            p[a][d] = r[0];
            p[a + 1][d] = r[1];
          }
        *(uint4*)(orow + 32 * j + 8 * h) = make_uint4(p[0][0], p[0][1], p[1][0], p[1][1]);
        *(uint4*)(orow + 32 * j + 16 + 8 * h) = make_uint4(p[2][0], p[2][1], p[3][0], p[3][1]);
      }
    }
  }
}

hipError_t launch_mx_pad_offsets(const int32_t* offsets, int E, int32_t* poff, hipStream_t st) {
  mx_pad_offsets_kernel<<<1, 1024, 0, st>>>(offsets, E, poff);
  return hipGetLastError();
}

// Token-axis quantisation: the rows of a source [*, C] in the experts' sorted order (see
// token_block_rows) into the padded segments, in blocks of 32 rows of one column.  Two threads
// share a 32 x 8 block, each loading 16 of its rows up front and keeping the raw words for both
// the column maxima and the codes (one read); thread t takes column chunk t / 2 of the block's
// 1024 columns and rows 16 (t % 2) .., and the pair's maxima meet by a lane exchange.  Against
// one thread per block holding all 32 rows this halves the registers, so twice the waves are in
// flight (qwen3: x and dy 160 -> 121 us, dH 148 -> 120 us, As 93 -> 57 us).
__global__ __launch_bounds__(256) void mx_quant_tokens_kernel(const uint16_t* __restrict__ src, int C,
                                                                   int gather, int kslots,
                                                                   const int32_t* __restrict__ offsets,
                                                                   const int32_t* __restrict__ perm,
                                                                   const int32_t* __restrict__ poff, int E,
                                                                   uint8_t* __restrict__ q,
                                                                   uint8_t* __restrict__ qe) {
  __shared__ int64_t s_row[32];
  const int pp0 = blockIdx.x * 32;
  if (pp0 >= poff[E]) return;                        // block-uniform: past the padded total
  token_block_rows(pp0, gather, kslots, offsets, perm, poff, E, s_row);
  const int half = threadIdx.x & 1;
  const int c0 = blockIdx.y * 1024 + (threadIdx.x >> 1) * 8;
  if (c0 >= C) return;                               // both threads of a pair: C is a multiple of 8
  uint4 raw[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t row = s_row[16 * half + r];
    raw[r] = make_uint4(0u, 0u, 0u, 0u);
    // a gathered token row is read again by its other experts' blocks: keep it cached then
    if (row >= 0) raw[r] = gather ? *(const uint4*)(src + row * C + c0) : load_once16(src + row * C + c0);
  }
  auto decode = [&](int r, float (&v)[8]) __attribute__((always_inline)) {
    const uint4 w = raw[r];
    v[0] = lo_bf16(w.x); v[1] = hi_bf16(w.x); v[2] = lo_bf16(w.y); v[3] = hi_bf16(w.y);
    v[4] = lo_bf16(w.z); v[5] = hi_bf16(w.z); v[6] = lo_bf16(w.w); v[7] = hi_bf16(w.w);
  };
  float amax[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float v[8];
    decode(r, v);
#pragma unroll
    for (int t = 0; t < 8; ++t) amax[t] = fmaxf(amax[t], fabsf(v[t]));
  }
  int sx[8];
  float inv[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    amax[t] = fmaxf(amax[t], __shfl_xor(amax[t], 1, 64));
    sx[t] = mx_exponent(amax[t]);
    inv[t] = ldexpf(1.0f, -sx[t]);  // exact: a power of two
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float v[8];
    decode(r, v);
    u32x2 o;
    o.x = pack_e4m3x4(v[0] * inv[0], v[1] * inv[1], v[2] * inv[2], v[3] * inv[3]);
    o.y = pack_e4m3x4(v[4] * inv[4], v[5] * inv[5], v[6] * inv[6], v[7] * inv[7]);
    *(u32x2*)(q + (int64_t)(pp0 + 16 * half + r) * C + c0) = o;
  }
  if (half == 0) {
    u32x2 ev;
    ev.x = (uint32_t)(sx[0] + 127) | ((uint32_t)(sx[1] + 127) << 8) | ((uint32_t)(sx[2] + 127) << 16) |
           ((uint32_t)(sx[3] + 127) << 24);
    ev.y = (uint32_t)(sx[4] + 127) | ((uint32_t)(sx[5] + 127) << 8) | ((uint32_t)(sx[6] + 127) << 16) |
           ((uint32_t)(sx[7] + 127) << 24);
    *(u32x2*)(qe + (int64_t)(pp0 / 32) * C + c0) = ev;
  }
}

hipError_t launch_mx_quant_tokens(const uint16_t* src, int C, int gather, const MoeShape& s, const int32_t* offsets,
                                  const int32_t* perm, const int32_t* poff, uint8_t* q, uint8_t* qe, hipStream_t st) {
  const int64_t blocks = mx_padded_rows((int64_t)s.T * s.k, s.E) / 32;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks, (unsigned)((C + 1023) / 1024));
  mx_quant_tokens_kernel<<<grid, 256, 0, st>>>(src, C, gather, s.k, offsets, perm, poff, s.E, q, qe);
  return hipGetLastError();
}

hipError_t launch_mx_wg(int which, const MoeShape& s, const uint8_t* Aq, const uint8_t* Ae, int Mo, const uint8_t* Bq,
                        const uint8_t* Be, int N, const int32_t* poff, const WgSplit& sp, uint16_t* dW,
                        hipStream_t st) {
  MxWgArgs g{};
  g.A = Aq;
  g.Ae = Ae;
  g.B = Bq;
  g.Be = Be;
  g.Mo = Mo;
  g.N = N;
  g.poff = poff;
  g.units = sp.units;
  g.meta = sp.meta;
  g.pslot = sp.pslot;
  g.partial = sp.partial;
  g.dW = dW;
  const int64_t blocks = (int64_t)(Mo / 256) * (N / 256) * (s.E + sp.max_partials);
  if (blocks == 0) return hipSuccess;
  if (which == 0) grouped_gemm_mx_wg_kernel<0><<<(unsigned)blocks, 512, 0, st>>>(g);
  else grouped_gemm_mx_wg_kernel<1><<<(unsigned)blocks, 512, 0, st>>>(g);
  return hipGetLastError();
}

}  // namespace moe
