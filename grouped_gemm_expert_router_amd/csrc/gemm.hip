// Ragged grouped GEMMs on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// All experts' matrix products run in one launch, each at its real token count, with no
// padding to a capacity (page "Az NVIDIA szerint tízszer gyorsabb lett a dropless MoE tanítása
// JAX-ban", section "Csoportosított mátrixszorzás és összevont adatmozgatás"; per-expert split
// sizes: TE MoE page "NVIDIA מציגה דרך יעילה לאמן מודלי MoE בביולוגיה", section "מומחים מקובצים
// במקום לולאת Python").  The SwiGLU and routing-weight scaling are fused into the first GEMM's
// epilogue (TE MoE page, section "צמצום הזיכרון ותקורות הכימות": GroupedLinear -> ScaledSwiGLU
// -> GroupedLinear), and the token gather into its operand loads (Mega MoE announcement,
// section "Mega MoE คืออะไร?": dispatch fused with the linear layers).
//
// One kernel template covers the six products of the layer:
//   UP    H  = x[tok] W1[e]        ragged M, A rows gathered, B = W1 [d,2f] (N contiguous)
//   DOWN  Op = As W2[e]            ragged M, B = W2 [f,d] (N contiguous); rows stored in slot order
//   DACT  G  = dy[tok] W2[e]^T     ragged M, A gathered, B = W2 rows (K contiguous); dSwiGLU epilogue
//   DX    dXp = dH W1[e]^T         ragged M, B = W1 rows (K contiguous); rows stored in slot order
//   WG    dW = P_e^T Q_e           ragged K = the expert's rows; both operands row-major over K
// Tiles are BM x BN x BK (256 x 256 x 64 where the shape allows); the waves of a WM x WN grid
// each own (BM/WM) x (BN/WN) of the tile as 32x32 MFMA blocks.  Operand tiles go from global
// memory straight into LDS (global_load_lds_dwordx4), in their global orientation, with a
// 16-byte-chunk XOR swizzle: a K-contiguous tile is read as one ds_read_b128 per MFMA operand,
// an M- or N-contiguous one with the gfx950 transpose read ds_read_b64_tr_b16.  Two LDS stages:
// the DMA of k step t+1 is in flight during step t's MFMAs.  Epilogues store from registers,
// except the dSwiGLU one, which moves H and dH through the freed operand stages as whole rows.
#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace moe {

// M_WG and M_WG1 are the same ragged-K weight-gradient kernel (dW2 and dW1), kept as two
// instantiations so the two launches carry distinct names in kernel traces.
enum GemmMode { M_UP = 0, M_DOWN = 1, M_DACT = 2, M_DX = 3, M_WG = 4, M_WG1 = 5 };

struct GemmArgs {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  int64_t b_estride;  // elements between consecutive experts' weight matrices
  int N, K;           // ragged M: output columns, reduction depth.  WG: dW columns
  int Mo;             // WG: dW rows
  int kslots, f;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* tokrow;  // ragged K: token row of each sorted position (perm[pos] / k)
  const int2* tiles;
  const int32_t* ntiles;
  const float* topk_w;
  uint16_t* C0;
  int64_t ldc0;
  uint16_t* C1;
  int64_t ldc1;
  const uint16_t* Hs;
  int64_t ldh;
  float* dwp;        // d_topk_w partials, part-major: partial q of sorted row pos at dwp[q*dwp_stride + pos]
  int64_t dwp_stride;
  // ragged K split: work unit u = (expert, chunk) of KC rows; experts split into several chunks
  // write fp32 partials (slot wg_pslot[e] + chunk) that a second kernel sums in chunk order
  const int2* wg_units;
  const int32_t* wg_meta;   // [0] units, [1] KC
  const int32_t* wg_pslot;  // first partial slot of a split expert, -1 if not split
  float* partial;
};

// Scheduling order for one k step: NM MFMAs, each followed by its share of NRD LDS reads.
template <int NM, int NRD>
__device__ __forceinline__ void sched_interleave() {
  if constexpr (NM > 0) {
    constexpr int r = (NRD + NM - 1) / NM;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // r LDS reads
    sched_interleave<NM - 1, NRD - r>();
  }
}

// 1: interleave the next k step's LDS reads with the current MFMAs by scheduling barriers.
#ifndef GEMM_SCHED
#define GEMM_SCHED 1
#endif

// Row tiles per group of the ragged-M tile order (grouped_tile).  With fewer than 8 column
// tiles a row tile's column tiles run back to back instead (a group of one row tile): measured
// -2 % for the qwen3 up and dA products, whose 6 and 3 column tiles then share their A rows.
#ifndef GEMM_GM
#define GEMM_GM 8
#endif

// One output tile: expert e, rows m0 .. m0+mrows-1 of the sorted order (ragged M) or of dW[e]
// (ragged K), column tile nt starting at n0, reduction over k rows kbeg .. kend-1; ragged K:
// chunk kchunk of the expert and its first partial slot pslot (-1: the expert is not split).
struct TileCoord {
  int e, m0, mrows, n0, nt, kbeg, kend, kchunk, pslot;
};

// LDS bytes of a tile's operand stages
template <int BM, int BN, int BK>
constexpr int tile_lds_bytes() {
  return (BK == 32 ? 4 : 2) * (BM * BK * 2 + BN * BK * 2);
}

// The tile of block blockIdx.x in a grid of one block per tile; false for blocks past the tiles
// that exist (known on the device only).  Uniform over the block.
template <int MODE, int BM, int BN>
__device__ __forceinline__ bool tile_coord(const GemmArgs& g, TileCoord& c) {
  constexpr bool RAGGED_K = (MODE == M_WG || MODE == M_WG1);
  int e, m0, mrows, n0, nt, kbeg, kend;
  int kchunk = 0, pslot = -1;
  if constexpr (RAGGED_K) {
    const int nN = g.N / BN;
    const int per_u = (g.Mo / BM) * nN;
    const CONST_AS int32_t* meta = (const CONST_AS int32_t*)g.wg_meta;
    const int U = meta[0];
    const int G_valid = U * per_u;
    if ((int)blockIdx.x >= G_valid) return false;  // uniform: the block has no work
    // Units come in decreasing size.  Deal them to 8 buckets round-robin (bucket b holds units
    // b, b+8, ...: near-equal work per bucket) and give XCD b the tiles of bucket b, so each
    // XCD streams its units' operand rows from HBM into its own L2 once instead of every XCD
    // re-reading every unit.  The logical order is bucket-major, cut into 8 equal tile ranges
    // by xcd_remap, which also spreads the tiles when there are fewer than 8 units.
    // When that leaves the buckets uneven (a few long units), the split kernel clears meta[2]
    // and blocks take the units in order instead: the round-robin dispatch then hands every
    // XCD an equal share of each unit.
    int pos = blockIdx.x, u;
    if (meta[2]) {
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
    const CONST_AS int32_t* up = (const CONST_AS int32_t*)g.wg_units;
    e = up[2 * u];
    kchunk = up[2 * u + 1];
    const int t = pos % per_u, nM = g.Mo / BM;
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
    mrows = BM;
    n0 = nt * BN;
    const CONST_AS int32_t* off4 = (const CONST_AS int32_t*)g.offsets;
    const int KC = meta[1];
    kbeg = off4[e] + kchunk * KC;
    kend = min(off4[e + 1], kbeg + KC);
    pslot = ((const CONST_AS int32_t*)g.wg_pslot)[e];
  } else {
    const int nN = (MODE == M_UP) ? g.f / (BN / 2) : g.N / BN;
    const int G_valid = *(const CONST_AS int32_t*)g.ntiles * nN;
    if ((int)blockIdx.x >= G_valid) return false;  // uniform: the block has no work
    const int lid = xcd_remap(blockIdx.x, G_valid);
    const int2 rc = grouped_tile(lid, G_valid / nN, nN, nN < 8 ? 1 : GEMM_GM);
    nt = rc.y;
    // uniform loads through the scalar cache (the tile table and offsets are read-only here)
    const CONST_AS int32_t* tp = (const CONST_AS int32_t*)g.tiles;
    e = tp[2 * rc.x];
    const CONST_AS int32_t* off4 = (const CONST_AS int32_t*)g.offsets;
    m0 = off4[e] + tp[2 * rc.x + 1] * BM;
    mrows = min(BM, off4[e + 1] - m0);
    n0 = (MODE == M_UP) ? nt * (BN / 2) : nt * BN;
    kbeg = 0;
    kend = g.K;
  }
  c = TileCoord{e, m0, mrows, n0, nt, kbeg, kend, kchunk, pslot};
  return true;
}

// One BM x BN output tile, computed by the block's NW = 2*WN waves.  smem holds the operand
// stages (tile_lds_bytes), s_w and s_slot the routing weight and pair of each tile row (ragged
// M), s_part the dA epilogue's per-wave-column partials ([WN][BM]).  The arena must be free when
// the tile starts: no wave of the block may still read it.
template <int MODE, int BM, int BN, int WN, int BK>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, const TileCoord& tc, uint8_t* smem, float* s_w,
                                          int* s_slot, float* s_part) {
  constexpr int S = BK == 32 ? 4 : 2, WM = 2, NW = WM * WN, NTH = 64 * NW;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr bool RAGGED_K = (MODE == M_WG || MODE == M_WG1);
  constexpr bool A_KN = RAGGED_K;                              // A stored [k][m]
  constexpr bool B_KN = !(MODE == M_DACT || MODE == M_DX);     // B stored [k][n]
  // operand rows that come from token perm[pos] / k instead of sorted position pos: x (UP, dW1)
  // and dy (dA, dW2)
  constexpr bool GA = (MODE == M_UP || MODE == M_DACT || MODE == M_WG1), GB = (MODE == M_WG);
  static_assert(MODE != M_UP || (FN % 2 == 0), "gate/up pairing needs an even fragment count");
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
  constexpr int QA = BM * BK / (512 * NW), QB = BN * BK / (512 * NW);  // DMA instrs per thread per tile
  constexpr int KRW = BK / NW;                                 // ragged K: k rows per wave's DMA
  static_assert(QA >= 1 && QB >= 1 && (!RAGGED_K || KRW == 4 || KRW == 8), "tile / wave split");
  constexpr int DPT = QA + QB;
  static_assert(DPT * (S - 2) <= 63 && (BK == 32 || BK == 64), "vmcnt range");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr_of(smem));
  const int e = tc.e, m0 = tc.m0, mrows = tc.mrows, n0 = tc.n0, nt = tc.nt, kbeg = tc.kbeg, kend = tc.kend;
  const int kchunk = tc.kchunk, pslot = tc.pslot;
  (void)kchunk;
  (void)pslot;
  const uint16_t* Bexp = g.B + (RAGGED_K ? 0 : (int64_t)e * g.b_estride);

  // ------------------------------------------------------------------ DMA source pointers
  // KM operand, instruction q: LDS block gi = wave*(R/64) + q holds rows 16*gi..16*gi+15; lane
  // L fills physical chunk L%4 of row 16*gi + L/4 from logical chunk (L%4) ^ ((row >> 2) & 3).
  // KN operand (C columns), instruction q: block gi = wave*(C/64) + q holds k rows
  // (512/C)*gi ..; lane L fills physical chunk L % (C/8) of k row (512/C)*gi + L/(C/8).
  const uint16_t* a_src[QA];
  const uint16_t* b_src[QB];
  int a_kr[QA], b_kr[QB];  // KN: k row within the tile; KM: unused
  int a_col[QA], b_col[QB];  // KN: global column offset of the lane's chunk
  if constexpr (!A_KN) {
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      constexpr int CPR = BK / 8;  // 16-byte chunks per row
      const int row = (64 / CPR) * (wave * QA + q) + lane / CPR;
      const int c = (lane % CPR) ^ (BK == 32 ? ((row >> 2) & 3) : ((row >> 1) & 7));
      // rows past the expert's end read row m0: they only feed accumulator rows the epilogue
      // never stores (an output row depends on its own A row only)
      const int pos = m0 + (row < mrows ? row : 0);
      const int64_t src = GA ? (int64_t)(g.perm[pos] / g.kslots) : (int64_t)pos;
      a_src[q] = g.A + src * g.lda + 8 * c;
    }
  } else {
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      constexpr int CH = BM / 8;
      a_kr[q] = (512 / BM) * (wave * QA + q) + lane / CH;
      const int c = (lane % CH) ^ (4 * (a_kr[q] & 3));
      a_col[q] = m0 + 8 * c;
    }
  }
  if constexpr (!B_KN) {
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      constexpr int CPR = BK / 8;
      const int row = (64 / CPR) * (wave * QB + q) + lane / CPR;
      const int c = (lane % CPR) ^ (BK == 32 ? ((row >> 2) & 3) : ((row >> 1) & 7));
      b_src[q] = Bexp + (int64_t)(n0 + row) * g.ldb + 8 * c;
    }
  } else {
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      constexpr int CH = BN / 8;
      b_kr[q] = (512 / BN) * (wave * QB + q) + lane / CH;
      const int c = (lane % CH) ^ (4 * (b_kr[q] & 3));
      int col;
      if constexpr (MODE == M_UP) col = c < CH / 2 ? n0 + 8 * c : g.f + n0 + 8 * (c - CH / 2);
      else col = n0 + 8 * c;
      b_col[q] = col;
      if constexpr (!RAGGED_K) b_src[q] = Bexp + (int64_t)b_kr[q] * g.ldb + col;
    }
  }

  // Ragged K: a wave's DMA covers the KRW consecutive k rows KRW*wave.. of the tile.  Their
  // token rows come from one scalar load (tokrow[pos] = perm[pos] / k); rows past kend read the
  // expert's first row and their A values are zeroed in LDS before use.
  const int klen = kend - kbeg;
  int tok_first = 0;
  if constexpr (RAGGED_K)
    if (klen > 0 && (GA || GB)) tok_first = ((const CONST_AS int32_t*)g.tokrow)[kbeg];
  // Ragged K: the tokens of the wave's KRW k rows of step t, one scalar load.
  auto load_tk = [&](int t) __attribute__((always_inline)) -> i32x8 {
    i32x8 tk = {0, 0, 0, 0, 0, 0, 0, 0};
    if (RAGGED_K && (GA || GB)) {
      if constexpr (KRW == 8) {
        tk = *(const CONST_AS i32x8*)(g.tokrow + kbeg + t * BK + KRW * wave);
      } else {
        const i32x4 v = *(const CONST_AS i32x4*)(g.tokrow + kbeg + t * BK + KRW * wave);
        tk = i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
      }
    }
    return tk;
  };
  auto issue = [&](int t, int st, const i32x8& tk) __attribute__((always_inline)) {
    const int k0 = t * BK;
    const uint32_t abase = lds0 + st * STAGE, bbase = abase + A_BYTES;
    if constexpr (!RAGGED_K) {
#pragma unroll
      for (int q = 0; q < QA; ++q) dma16(a_src[q] + k0, abase + (wave * QA + q) * 1024);
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const uint16_t* src = B_KN ? b_src[q] + (int64_t)k0 * g.ldb : b_src[q] + k0;
        dma16(src, bbase + (wave * QB + q) * 1024);
      }
    } else {
      // Instruction q of an operand with C columns covers k rows KRW*wave + R*q + r, where
      // R = 512/C rows per instruction and r = lane / (C/8): the lane's token is one of R
      // elements at fixed positions (a two-way select for C = 256).  Selecting with fixed
      // indices keeps the values in registers; a select on a computed index (k row - KRW*wave)
      // is turned by the compiler into an indexed array in LDS, one LDS round trip per DMA.
      auto tok_sel = [&](int q, int R, int CHL) __attribute__((always_inline)) -> int {
        int t = tk[R * q];
        const int r = lane / CHL;
#pragma unroll
        for (int z = 1; z < 4; ++z)
          if (z < R) t = (r == z) ? tk[R * q + z] : t;
        return t;
      };
      auto row_of = [&](int kr, int t, bool gather) __attribute__((always_inline)) -> int64_t {
        const bool ok = k0 + kr < klen;
        if (!gather) return ok ? (int64_t)(kbeg + k0 + kr) : (int64_t)kbeg;
        return ok ? (int64_t)t : (int64_t)tok_first;
      };
#pragma unroll
      for (int q = 0; q < QA; ++q)
        dma16(g.A + row_of(a_kr[q], tok_sel(q, 512 / BM, BM / 8), GA) * g.lda + a_col[q],
              abase + (wave * QA + q) * 1024);
#pragma unroll
      for (int q = 0; q < QB; ++q)
        dma16(g.B + row_of(b_kr[q], tok_sel(q, 512 / BN, BN / 8), GB) * g.ldb + b_col[q],
              bbase + (wave * QB + q) * 1024);
    }
  };

  // LDS column of the wave's j-th 32-column B fragment
  auto b_row = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (MODE == M_UP)
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

  auto load_frags = [&](uint32_t abase, uint32_t bbase, int kk, bf16x8_t (&af)[FM], bf16x8_t (&bv)[FN])
      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if constexpr (A_KN) af[i] = read_kn<BM>(abase, wm * TM + i * 32, kk, lane);
      else af[i] = read_km<BK>(abase, wm * TM + i * 32 + (lane & 31), 2 * kk + (lane >> 5));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (B_KN) bv[j] = read_kn<BN>(bbase, b_row(j), kk, lane);
      else bv[j] = read_km<BK>(bbase, b_row(j) + (lane & 31), 2 * kk + (lane >> 5));
    }
  };
  // The fragments of k step kk+1 are read from LDS while the MFMAs of step kk run (two register
  // sets); the scheduling barriers keep each read next to an MFMA instead of just before its use.
  auto compute = [&](int st) __attribute__((always_inline)) {
    const uint32_t abase = lds0 + st * STAGE, bbase = abase + A_BYTES;
    constexpr int KS = BK / 16;
    bf16x8_t af[2][FM], bv[2][FN];
    // first k step: the first MFMA's operands (A fragment 0, B fragment 0) are read first, so
    // the MFMAs can start before the whole step's fragments have arrived
    auto read_a = [&](int i, int kk) __attribute__((always_inline)) {
      if constexpr (A_KN) return read_kn<BM>(abase, wm * TM + i * 32, kk, lane);
      else return read_km<BK>(abase, wm * TM + i * 32 + (lane & 31), 2 * kk + (lane >> 5));
    };
    auto read_b = [&](int j, int kk) __attribute__((always_inline)) {
      if constexpr (B_KN) return read_kn<BN>(bbase, b_row(j), kk, lane);
      else return read_km<BK>(bbase, b_row(j) + (lane & 31), 2 * kk + (lane >> 5));
    };
    af[0][0] = read_a(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      bv[0][j] = read_b(j, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 1; i < FM; ++i) {
      af[0][i] = read_a(i, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Raised wave priority while the MFMAs issue: with two waves per SIMD, the arbiter then
    // favours the wave that feeds the matrix pipe over one issuing its DMA.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < KS) load_frags(abase, bbase, kk + 1, af[cur ^ 1], bv[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[cur][j], af[cur][i], acc[i][j], 0, 0, 0);
#if GEMM_SCHED
      // LDS read instructions of one step: b128 per KM fragment, two transpose reads per KN one
      if (kk + 1 < KS) sched_interleave<FM * FN, FM * (A_KN ? 2 : 1) + FN * (B_KN ? 2 : 1)>();
#endif
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // dA epilogue staging.  Row block i (32 rows) of wave (wm, wn) keeps its saved H, and then
  // its dH in place, in a slot of LDS: stage i % 2, offset EP_SLOT * wave.  The slot holds the
  // wave's TN gate columns of the 32 rows (KM layout of a TN-deep tile: rows of EP_RB bytes,
  // 16-byte chunks XOR-swizzled), then their TN up columns.  A DMA or store instruction moves
  // EP_RPI whole rows of one half; a row of the wave's 64 gate (or up) columns is one whole
  // 128-byte line of H or dH (TN = 64), or half of one (TN = 32).
  constexpr int EP_RB = TN * 2, EP_HALF = 32 * EP_RB, EP_SLOT = 2 * EP_HALF;
  constexpr int EP_CPR = TN / 8, EP_RPI = 64 / EP_CPR, EP_QH = 32 / EP_RPI, EP_Q = 2 * EP_QH;
  static_assert(MODE != M_DACT || ((TN == 64 || TN == 32) && TM == 128 && NW * EP_SLOT <= STAGE),
                "dA epilogue slots");
  // H rows of row block i into stage st; a row past the expert's end reads row m0
  auto dact_h_dma = [&](int i, int st) __attribute__((always_inline)) {
    if constexpr (MODE == M_DACT) {
      const uint32_t slot = lds0 + st * STAGE + wave * EP_SLOT;
      const int rl = lane / EP_CPR, pc = lane % EP_CPR;
#pragma unroll
      for (int q = 0; q < EP_Q; ++q) {
        const int half = q / EP_QH, r = EP_RPI * (q % EP_QH) + rl;
        const int lr = wm * TM + 32 * i + r;
        const int64_t pos = m0 + (lr < mrows ? lr : 0);
        const int c = pc ^ km_swz<TN>(r);  // the logical chunk that physical chunk pc holds
        dma16(g.Hs + pos * g.ldh + half * g.f + n0 + wn * TN + 8 * c, slot + half * EP_HALF + (q % EP_QH) * 1024);
      }
    }
  };

  // ------------------------------------------------------------------ main loop
  // Stage t%S holds tile t.  Iteration t: wait until tile t's DMA has landed (tiles t+1..t+S-2
  // may stay in flight) and all waves are past tile t-1, refill tile t-1's stage with tile
  // t+S-1, then run tile t's MFMAs.
  const int nk = (klen + BK - 1) / BK;
  // In an expert's last row tile, a wave whose rows all lie past the expert's end skips its
  // fragment reads and MFMAs (uniform: mrows and wm are); it still issues its DMA share.
  const bool busy = __builtin_amdgcn_readfirstlane(wm * TM < mrows);
  // The first stages' DMA goes out before anything else waits on memory (the arena of a new
  // block is free); the epilogue's per-row slot and routing weight are fetched under it.
#pragma unroll
  for (int t = 0; t < S - 1; ++t)
    if (t < nk) issue(t, t, load_tk(t));
  if constexpr (!RAGGED_K) {
    for (int r = tid; r < BM; r += NTH) {
      int p = -1;
      float wv = 0.0f;
      if (r < mrows) {
        p = g.perm[m0 + r];
        if (MODE == M_UP || MODE == M_DACT) wv = g.topk_w[p];
      }
      s_slot[r] = p;
      s_w[r] = wv;
    }
  }
  __syncthreads();  // s_slot / s_w visible
  for (int it = 0; it < nk; ++it) {
    // the tokens of the step refilled below are loaded before the wait, so the scalar load's
    // latency overlaps the DMA wait and the barrier
    const bool refill = it + S - 1 < nk;
    i32x8 tk = {0, 0, 0, 0, 0, 0, 0, 0};
    if (RAGGED_K && refill) tk = load_tk(it + S - 1);
    const int pend = min(S - 2, nk - 1 - it);
    if (S >= 4 && pend >= 2) vm_wait_barrier<(S >= 4 ? 2 : 0) * DPT>();
    else if (S >= 3 && pend == 1) vm_wait_barrier<(S >= 3 ? 1 : 0) * DPT>();
    else vm_wait_barrier<0>();
    if constexpr (RAGGED_K) {
      const int kvalid = klen - it * BK;
      if (kvalid < BK) {  // last tile of the expert: zero A's k rows past kend
        uint8_t* a = smem + (it % S) * STAGE;
        for (int z = kvalid * 2 * BM + tid * 16; z < A_BYTES; z += NTH * 16)
          *(u32x4*)(a + z) = u32x4{0u, 0u, 0u, 0u};
        lds_barrier();
      }
    }
    if (refill) issue(it + S - 1, (it + S - 1) % S, tk);
    // dA: the H lines of the epilogue's first row block land in the stage the last k step
    // does not read, under that step's MFMAs
    if constexpr (MODE == M_DACT)
      if (it == nk - 1 && busy) dact_h_dma(0, (it + 1) % S);
    // Ragged K: the token scalar load may still be outstanding here on the path without a
    // refill; retiring it now (visibly to the compiler's wait-count tracking) lets the step's
    // first MFMAs wait for their own LDS reads only instead of for every outstanding one.
    if constexpr (RAGGED_K) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    if (busy) compute(it % S);
  }

  // ------------------------------------------------------------------ epilogues
  // The MFMAs take the B fragment as their first operand, so each 32x32 accumulator block is
  // held transposed: lane l holds tile row wm*TM + 32*i + l%32 and, for r = 0..15, the column
  // b_row(j) + 8*(r/4) + 4*(l/32) + r%4.  Exchanging half-waves (v_permlane32_swap) turns the
  // four 4-column groups of lanes l and l+32 into two runs of 8 consecutive columns each, at
  // 8h and 16 + 8h (h = l/32), which are stored as 16-byte chunks straight from registers.
  const int h = lane >> 5, lrow = lane & 31;
  auto pack_rows = [&](const f32x16_t& v, uint4& lo, uint4& hi) __attribute__((always_inline)) {
    pack_rows_bf16(v, lo, hi);
  };

  if constexpr (MODE == M_UP) {
    // gate block j and up block j + FN/2 hold the same columns of the same rows
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int lr = wm * TM + 32 * i + lrow;
      const bool ok = lr < mrows;
      const float w = s_w[lr];
      const int64_t pos = m0 + lr;
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
        const f32x16_t& G = acc[i][j];
        const f32x16_t& U = acc[i][j + FN / 2];
        f32x16_t a;
#pragma unroll
        for (int r = 0; r < 16; ++r) a[r] = w * G[r] * sigmoidf_fast(G[r]) * U[r];
        uint4 glo, ghi, ulo, uhi, alo, ahi;
        pack_rows(G, glo, ghi);
        pack_rows(U, ulo, uhi);
        pack_rows(a, alo, ahi);
        if (ok) {
          const int col = n0 + wn * (TN / 2) + 32 * j + 8 * h;
          uint16_t* hrow = g.C0 + pos * g.ldc0;
          uint16_t* arow = g.C1 + pos * g.ldc1;
          *(uint4*)(hrow + col) = glo;
          *(uint4*)(hrow + col + 16) = ghi;
          *(uint4*)(hrow + g.f + col) = ulo;
          *(uint4*)(hrow + g.f + col + 16) = uhi;
          *(uint4*)(arow + col) = alo;
          *(uint4*)(arow + col + 16) = ahi;
        }
      }
    }
  } else if constexpr (MODE == M_DACT) {
    static_assert(WN == 4, "the d_topk_w part count assumes 4 waves across N");
    // G = dL/dAs.  a = silu(g) u from the saved H; da = w G; dH = [da u sig(g) (1 + g (1 - sig(g))),
    // da silu(g)]; the d_topk_w partial <G, a> of a row over the tile's columns is summed over the
    // WN wave columns in LDS (in wave-column order) and stored once per row as part nt, rows
    // consecutive.
    // H and dH move through the LDS slots as whole rows (dact_h_dma above): row block i's H
    // arrives while block i-1 is computed and stored, and dH leaves by buffer stores whose
    // bounds (the tile's valid rows) drop the rows past the expert's end.  Every wave that has
    // rows issues EP_Q DMA and EP_Q store instructions per block, so the waits below count
    // exactly the vector-memory instructions issued after the awaited DMA.
    // Every wave is past the last k step's LDS reads: the stage it read is free.
    asm volatile("s_barrier" ::: "memory");
    const __amdgpu_buffer_rsrc_t dst =
        __builtin_amdgcn_make_buffer_rsrc(g.C0 + (int64_t)m0 * g.ldc0, 0, (int)(mrows * g.ldc0 * 2), 0x00020000);
    if (busy) dact_h_dma(1, (nk + 1) % S);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (!busy) break;  // uniform
      const uint32_t slot = lds0 + ((nk + i) % S) * STAGE + wave * EP_SLOT;
      if (i == 0) vm_wait<EP_Q>();             // then: block 1's DMA
      else if (i < FM - 1) vm_wait<2 * EP_Q>();  // then: block i-1's stores, block i+1's DMA
      else vm_wait<EP_Q>();                     // then: block i-1's stores
      const int lr = wm * TM + 32 * i + lrow;
      const float w = s_w[lr];
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        // fp32 half-wave exchange (in place: the block is dead afterwards): then G[8c + e] is
        // column 16c + 8h + e
        f32x16_t& G = acc[i][j];
#pragma unroll
        for (int a = 0; a < 16; a += 8)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(G[a + t]), __float_as_uint(G[a + 4 + t]),
                                                             false, false);
            G[a + t] = __uint_as_float(r[0]);
            G[a + 4 + t] = __uint_as_float(r[1]);
          }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          // the lane's 8 columns: chunk 4j + 2c + h of the wave's TN gate (up) columns
          const uint32_t ag = slot + km_off<TN>(lrow, 4 * j + 2 * c + h), au = ag + EP_HALF;
          const u32x4 hgv = *(const LDS_AS u32x4*)(uintptr_t)ag, huv = *(const LDS_AS u32x4*)(uintptr_t)au;
          u32x4 dg, du;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t wg = hgv[t], wu = huv[t];
            float r0, r1, s0, s1;
            {
              const float gv = lo_bf16(wg), uv = lo_bf16(wu), Gv = G[8 * c + 2 * t];
              const float sg = sigmoidf_fast(gv), sl = gv * sg, da = w * Gv;
              part += Gv * (sl * uv);
              r0 = da * uv * sg * (1.0f + gv * (1.0f - sg));
              s0 = da * sl;
            }
            {
              const float gv = hi_bf16(wg), uv = hi_bf16(wu), Gv = G[8 * c + 2 * t + 1];
              const float sg = sigmoidf_fast(gv), sl = gv * sg, da = w * Gv;
              part += Gv * (sl * uv);
              r1 = da * uv * sg * (1.0f + gv * (1.0f - sg));
              s1 = da * sl;
            }
            dg[t] = pack_bf16x2(r0, r1);
            du[t] = pack_bf16x2(s0, s1);
          }
          // dH in place of the H it came from (the wave's LDS operations run in order)
          *(LDS_AS u32x4*)(uintptr_t)ag = dg;
          *(LDS_AS u32x4*)(uintptr_t)au = du;
        }
      }
      part += __shfl_xor(part, 32, 64);  // lanes l and l+32 hold the same row
      if (h == 0) s_part[wn * BM + lr] = part;
      // the block's dH rows, whole lines per instruction
      {
        const int rl = lane / EP_CPR, cc = lane % EP_CPR;
#pragma unroll
        for (int q = 0; q < EP_Q; ++q) {
          const int half = q / EP_QH, r = EP_RPI * (q % EP_QH) + rl;
          const u32x4 v = *(const LDS_AS u32x4*)(uintptr_t)(slot + half * EP_HALF + km_off<TN>(r, cc));
          const int lr2 = wm * TM + 32 * i + r;
          const int col = half * g.f + n0 + wn * TN + 8 * cc;
          __builtin_amdgcn_raw_buffer_store_b128(v, dst, (int)((lr2 * g.ldc0 + col) * 2), 0, 0);
        }
      }
      if (i + 2 < FM) {
        lds_wait();  // the slot's reads are done before the DMA refills it
        dact_h_dma(i + 2, (nk + i) % S);
      }
    }
    __syncthreads();
    for (int r = tid; r < BM; r += NTH) {
      float sum = s_part[r];
#pragma unroll
      for (int c = 1; c < WN; ++c) sum += s_part[c * BM + r];
      if (r < mrows) g.dwp[(int64_t)nt * g.dwp_stride + m0 + r] = sum;
    }
  } else if (RAGGED_K && pslot >= 0) {
    // one chunk of a split expert: fp32 partial, summed later in chunk order; each 4-column
    // group is one 16-byte store
    float* out = g.partial + (int64_t)(pslot + kchunk) * g.Mo * g.N;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float* orow = out + (int64_t)(m0 + wm * TM + 32 * i + lrow) * g.N + n0;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(float4*)(orow + b_row(j) + 8 * q + 4 * h) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    }
  } else {
    // plain bf16 store: DOWN/DX rows go to the pair's slot, weight-gradient rows to dW[e]
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int lr = wm * TM + 32 * i + lrow;
      bool ok;
      int64_t orow;
      if constexpr (RAGGED_K) {
        ok = true;
        orow = (int64_t)e * g.Mo + m0 + lr;
      } else {
        ok = lr < mrows;
        orow = s_slot[lr];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        uint4 lo, hi;
        pack_rows(acc[i][j], lo, hi);
        if (ok) {
          uint16_t* dst = g.C0 + orow * g.ldc0 + n0 + b_row(j) + 8 * h;
          *(uint4*)dst = lo;
          *(uint4*)(dst + 16) = hi;
        }
      }
    }
  }
}

// One block per tile; the grid is sized for the worst case and only the first G_valid blocks
// (known on the device) have work.  They are spread round-robin over the XCDs, so remapping
// within G_valid keeps every XCD equally busy.
template <int MODE, int BM, int BN, int WN, int OCC, int BK>
__global__ __launch_bounds__(128 * WN, OCC) void grouped_gemm_kernel(const GemmArgs g) {
  constexpr bool RAGGED_K = (MODE == M_WG || MODE == M_WG1);
  // the operand stages of the K loop (reused by the dA epilogue for H and dH)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[tile_lds_bytes<BM, BN, BK>()];
  __shared__ float s_w[RAGGED_K ? 1 : BM];
  __shared__ int s_slot[RAGGED_K ? 1 : BM];
  __shared__ float s_part[MODE == M_DACT ? WN * BM : 1];
  TileCoord tc;
  if (!tile_coord<MODE, BM, BN>(g, tc)) return;
  gemm_tile<MODE, BM, BN, WN, BK>(g, tc, smem, s_w, s_slot, s_part);
}

// ---------------------------------------------------------------------- single-launch forward
// The forward's gather, up product with its scaled-SwiGLU epilogue and down product in one
// persistent launch with a device work queue (the one-kernel MoE forward of the Mega MoE
// announcement, section "Mega MoE คืออะไร?", here without the communication it overlaps).
//
// A work item is one row tile: 256 sorted rows of one expert.  Its block runs the up product
// over all f/128 column tiles (H and As written as in the two-launch forward), waits for its own
// stores, and then the down product over all of d for the same rows, reading As back through
// its compute unit's path to L2.  No block ever waits for another: the only shared state is one
// counter per queue, advanced by an atomic add per take.
//
// Queue layout (fwd_queue_kernel): expert e's row tiles go to queue e % 8, full tiles first in
// expert order, then the partial last tiles, most rows first.  Block b drains queue b % 8 first
// (the hardware deals blocks to the 8 XCDs round-robin, so that is one XCD's queue and the
// tiles of one expert share its weights in that XCD's L2), then the other queues in turn.
constexpr int kFqTotal = 0, kFqBeg = 16, kFqCnt = 32;  // qinfo words: total, 9 queue starts, 8 counters

__global__ __launch_bounds__(1024) void fwd_queue_kernel(const int32_t* __restrict__ offsets, int E,
                                                         int2* __restrict__ items, int32_t* __restrict__ qinfo) {
  constexpr int BM = 256;
  __shared__ int s_full[1024], s_rem[1024];
  __shared__ int s_qbeg[9], s_qfull[8];
  const int e = threadIdx.x;
  const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
  const int full = c / BM, rem = c % BM;
  s_full[e] = full;
  s_rem[e] = rem;
  __syncthreads();
  if (e < 8) {
    int nf = 0, np = 0;
    for (int j = e; j < E; j += 8) {
      nf += s_full[j];
      np += s_rem[j] > 0;
    }
    s_qfull[e] = nf;
    s_qbeg[e + 1] = nf + np;
  }
  __syncthreads();
  if (e == 0) {
    s_qbeg[0] = 0;
    for (int q = 1; q <= 8; ++q) s_qbeg[q] += s_qbeg[q - 1];
  }
  __syncthreads();
  if (e < E) {
    const int q = e % 8;
    int pos = s_qbeg[q];
    for (int j = q; j < e; j += 8) pos += s_full[j];
    for (int r = 0; r < full; ++r) items[pos + r] = make_int2(e, r);
    if (rem > 0) {
      int rank = 0;
      for (int j = q; j < E; j += 8) {
        const int rj = s_rem[j];
        rank += (rj > rem) || (rj == rem && j < e);
      }
      items[s_qbeg[q] + s_qfull[q] + rank] = make_int2(e, full);
    }
  }
  if (e <= 8) qinfo[kFqBeg + e] = s_qbeg[e];
  if (e < 8) qinfo[kFqCnt + e] = 0;
  if (e == 0) qinfo[kFqTotal] = s_qbeg[8];
}

// gu: the up product's arguments, gd: the down product's; BND: the down product's tile width.
template <int BND>
__global__ __launch_bounds__(512, 1) void fused_forward_kernel(const GemmArgs gu, const GemmArgs gd,
                                                               const int2* __restrict__ items,
                                                               int32_t* __restrict__ qinfo) {
  constexpr int BM = 256;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[tile_lds_bytes<BM, 256, 64>()];
  __shared__ float s_w[BM];
  __shared__ int s_slot[BM];
  __shared__ int s_item;
  const int q0 = blockIdx.x % 8;
  int tries = 0;  // thread 0: queues found empty so far, in the order q0, q0 + 1, ...
  for (;;) {
    __syncthreads();  // every wave is past the previous item (LDS arena, s_item)
    if (threadIdx.x == 0) {
      int it = -1;
      for (; tries < 8; ++tries) {
        const int q = (q0 + tries) & 7;
        const int beg = qinfo[kFqBeg + q], n = qinfo[kFqBeg + q + 1] - beg;
        const int i = atomicAdd(&qinfo[kFqCnt + q], 1);
        if (i < n) {
          it = beg + i;
          break;
        }
      }
      s_item = it;
    }
    __syncthreads();
    const int item = s_item;
    if (item < 0) break;  // uniform: every queue is drained
    const int2 te = items[item];
    TileCoord tc;
    tc.e = te.x;
    tc.m0 = gu.offsets[te.x] + te.y * BM;
    tc.mrows = min(BM, gu.offsets[te.x + 1] - tc.m0);
    tc.kbeg = 0;
    tc.kchunk = 0;
    tc.pslot = -1;
    tc.kend = gu.K;
    for (int nt = 0; nt < gu.f / 128; ++nt) {
      if (nt > 0) __syncthreads();  // the previous tile's waves are out of the arena
      tc.nt = nt;
      tc.n0 = nt * 128;
      gemm_tile<M_UP, BM, 256, 4, 64>(gu, tc, smem, s_w, s_slot, nullptr);
    }
    // The down product reads the As rows this block just stored: all of them complete first.
    vm_wait<0>();
    tc.kend = gd.K;
    for (int nt = 0; nt < gd.N / BND; ++nt) {
      __syncthreads();
      tc.nt = nt;
      tc.n0 = nt * BND;
      gemm_tile<M_DOWN, BM, BND, 4, 64>(gd, tc, smem, s_w, s_slot, nullptr);
    }
  }
}

// ---------------------------------------------------------------------- host launchers
namespace {

// Launch MODE with a BM x BN tile: 256x256 (waves own 128x128, one block per CU) where the
// output width allows, else 256x128 / 128x256 / 128x128.
// Tile configs: 256x256 and 256x128 run 8 waves (2 per SIMD, each owning 128x64 or 128x32)
// so one wave's MFMAs cover the other's LDS and barrier waits; 128x128 runs 4 waves.  K step
// per LDS stage: BK = 32 with 4 stages or BK = 64 with 2 stages (GEMM_BK below).
#ifndef GEMM_BK
#define GEMM_BK 64
#endif
template <int MODE>
hipError_t run(const GemmArgs& g, int bm, int bn, dim3 grid, hipStream_t st) {
  constexpr int BKC = GEMM_BK;
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  if (bm == 256 && bn == 256)
    grouped_gemm_kernel<MODE, 256, 256, 4, 1, BKC><<<grid, 512, 0, st>>>(g);
  else if (bm == 256 && bn == 128)
    grouped_gemm_kernel<MODE, 256, 128, (MODE == M_UP ? 2 : 4), 1, BKC><<<grid, (MODE == M_UP ? 256 : 512), 0, st>>>(g);
  else if ((MODE == M_WG || MODE == M_WG1) && bm == 128 && bn == 256)
    grouped_gemm_kernel<(MODE == M_WG || MODE == M_WG1) ? MODE : M_WG, 128, 256, 4, 1, BKC><<<grid, 512, 0, st>>>(g);
  else if (MODE != M_DACT && bm == 128 && bn == 128)
    grouped_gemm_kernel<MODE == M_DACT ? M_DOWN : MODE, 128, 128, 2, 2, 32><<<grid, 256, 0, st>>>(g);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

int pick_bn(int n) { return n % 256 == 0 ? 256 : 128; }

GemmArgs base_args(const MoeShape& s, const int32_t* offsets, const int32_t* perm, const int2* tiles,
                   const int32_t* ntiles) {
  GemmArgs g{};
  g.kslots = s.k;
  g.f = s.f;
  g.offsets = offsets;
  g.perm = perm;
  g.tiles = tiles;
  g.ntiles = ntiles;
  return g;
}
}  // namespace

int dact_bn(int f) { return pick_bn(f); }
// d_topk_w partials per pair: one per N tile of the activation-gradient GEMM
int dact_parts_bf16(int f) { return f / dact_bn(f); }

int max_row_tiles(int64_t A, int E, int bm) {
  const int64_t t = (A + bm - 1) / bm + (A < E ? A : E);
  return (int)t;
}

namespace {
GemmArgs up_args(const MoeShape& s, const uint16_t* x, const uint16_t* W1, const float* topk_w,
                 const int32_t* offsets, const int32_t* perm, const int2* tiles, const int32_t* ntiles, uint16_t* H,
                 uint16_t* As) {
  GemmArgs g = base_args(s, offsets, perm, tiles, ntiles);
  g.A = x;
  g.lda = s.d;
  g.B = W1;
  g.ldb = 2 * (int64_t)s.f;
  g.b_estride = (int64_t)s.d * 2 * s.f;
  g.N = 2 * s.f;
  g.K = s.d;
  g.topk_w = topk_w;
  g.C0 = H;
  g.ldc0 = 2 * (int64_t)s.f;
  g.C1 = As;
  g.ldc1 = s.f;
  return g;
}

GemmArgs down_args(const MoeShape& s, const uint16_t* As, const uint16_t* W2, const int32_t* offsets,
                   const int32_t* perm, const int2* tiles, const int32_t* ntiles, uint16_t* Op) {
  GemmArgs g = base_args(s, offsets, perm, tiles, ntiles);
  g.A = As;
  g.lda = s.f;
  g.B = W2;
  g.ldb = s.d;
  g.b_estride = (int64_t)s.f * s.d;
  g.N = s.d;
  g.K = s.f;
  g.C0 = Op;
  g.ldc0 = s.d;
  return g;
}
}  // namespace

hipError_t launch_gemm_up(const MoeShape& s, const uint16_t* x, const uint16_t* W1, const float* topk_w,
                          const int32_t* offsets, const int32_t* perm, const int2* tiles, const int32_t* ntiles,
                          uint16_t* H, uint16_t* As, hipStream_t st) {
  const GemmArgs g = up_args(s, x, W1, topk_w, offsets, perm, tiles, ntiles, H, As);
  const int64_t A = (int64_t)s.T * s.k;
  const int bn = 256;  // 128 gate + 128 up columns (f is a multiple of 128)
  dim3 grid((unsigned)(max_row_tiles(A, s.E, kGemmBM) * (s.f / (bn / 2))));
  return run<M_UP>(g, kGemmBM, bn, grid, st);
}

hipError_t launch_gemm_down(const MoeShape& s, const uint16_t* As, const uint16_t* W2, const int32_t* offsets,
                            const int32_t* perm, const int2* tiles, const int32_t* ntiles, uint16_t* Op,
                            hipStream_t st) {
  const GemmArgs g = down_args(s, As, W2, offsets, perm, tiles, ntiles, Op);
  const int64_t A = (int64_t)s.T * s.k;
  const int bn = pick_bn(s.d);
  dim3 grid((unsigned)(max_row_tiles(A, s.E, kGemmBM) * (s.d / bn)));
  return run<M_DOWN>(g, kGemmBM, bn, grid, st);
}

hipError_t launch_fwd_queue(const MoeShape& s, const int32_t* offsets, int2* items, int32_t* qinfo, hipStream_t st) {
  fwd_queue_kernel<<<1, 1024, 0, st>>>(offsets, s.E, items, qinfo);
  return hipGetLastError();
}

hipError_t launch_fused_forward(const MoeShape& s, const uint16_t* x, const uint16_t* W1, const uint16_t* W2,
                                const float* topk_w, const int32_t* offsets, const int32_t* perm, const int2* items,
                                int32_t* qinfo, uint16_t* H, uint16_t* As, uint16_t* Op, hipStream_t st) {
  int dev = 0, ncu = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  if (ncu < 1) return hipErrorInvalidValue;
  // one block per compute unit; the tile tables are not used (the queue replaces them)
  const GemmArgs gu = up_args(s, x, W1, topk_w, offsets, perm, nullptr, nullptr, H, As);
  const GemmArgs gd = down_args(s, As, W2, offsets, perm, nullptr, nullptr, Op);
  if (s.d % 256 == 0)
    fused_forward_kernel<256><<<ncu, 512, 0, st>>>(gu, gd, items, qinfo);
  else
    fused_forward_kernel<128><<<ncu, 512, 0, st>>>(gu, gd, items, qinfo);
  return hipGetLastError();
}

hipError_t launch_gemm_dact(const MoeShape& s, const uint16_t* dy, const uint16_t* W2, const uint16_t* H,
                            const float* topk_w, const int32_t* offsets, const int32_t* perm, const int2* tiles,
                            const int32_t* ntiles, uint16_t* dH, float* dwp, hipStream_t st) {
  GemmArgs g = base_args(s, offsets, perm, tiles, ntiles);
  g.A = dy;
  g.lda = s.d;
  g.B = W2;  // row n of W2[e] ([f, d]) is column n of W2[e]^T, contiguous in K = d
  g.ldb = s.d;
  g.b_estride = (int64_t)s.f * s.d;
  g.N = s.f;
  g.K = s.d;
  g.topk_w = topk_w;
  g.Hs = H;
  g.ldh = 2 * (int64_t)s.f;
  g.C0 = dH;
  g.ldc0 = 2 * (int64_t)s.f;
  g.dwp = dwp;
  g.dwp_stride = (int64_t)s.T * s.k;
  const int bn = dact_bn(s.f);
  const int64_t A = (int64_t)s.T * s.k;
  dim3 grid((unsigned)(max_row_tiles(A, s.E, kGemmBM) * (s.f / bn)));
  return run<M_DACT>(g, kGemmBM, bn, grid, st);
}

hipError_t launch_gemm_dx(const MoeShape& s, const uint16_t* dH, const uint16_t* W1, const int32_t* offsets,
                          const int32_t* perm, const int2* tiles, const int32_t* ntiles, uint16_t* dXp,
                          hipStream_t st) {
  GemmArgs g = base_args(s, offsets, perm, tiles, ntiles);
  g.A = dH;
  g.lda = 2 * (int64_t)s.f;
  g.B = W1;  // row n of W1[e] ([d, 2f]) is column n of W1[e]^T, contiguous in K = 2f
  g.ldb = 2 * (int64_t)s.f;
  g.b_estride = (int64_t)s.d * 2 * s.f;
  g.N = s.d;
  g.K = 2 * s.f;
  g.C0 = dXp;
  g.ldc0 = s.d;
  const int64_t A = (int64_t)s.T * s.k;
  const int bn = pick_bn(s.d);
  dim3 grid((unsigned)(max_row_tiles(A, s.E, kGemmBM) * (s.d / bn)));
  return run<M_DX>(g, kGemmBM, bn, grid, st);
}

// ------------------------------------------------------------------ weight-gradient split
// One block: per expert e with c rows, nchunks = ceil(c / KC) if c > KC else 1 (an empty expert
// still gets one unit, which writes its zero gradient).  KC starts at kWgChunk and doubles until
// the split experts' chunks fit the max_partials fp32 slots.
__global__ __launch_bounds__(1024) void wg_split_kernel(const int32_t* __restrict__ offsets, int E, int kc_min,
                                                        int max_partials, int2* __restrict__ units,
                                                        int32_t* __restrict__ meta, int32_t* __restrict__ pslot) {
  __shared__ int sh[64];
  __shared__ int s_flag;
  const int e = threadIdx.x;
  const int c = (e < E) ? offsets[e + 1] - offsets[e] : 0;
  int KC = kc_min;
  if (max_partials < 2) KC = 0x40000000;  // no room for partials: never split
  for (;;) {
    const int need = (max_partials >= 2 && e < E && c > KC) ? (c + KC - 1) / KC : 0;
    int ex;
    const int tot = block_excl_scan_1024(need, sh, &ex);
    if (tot <= max_partials || KC >= 0x40000000) break;
    KC *= 2;
  }
  const bool split = max_partials >= 2 && e < E && c > KC;
  const int nch = (e < E) ? (split ? (c + KC - 1) / KC : 1) : 0;
  int pbase, ubase;
  block_excl_scan_1024(split ? nch : 0, sh, &pbase);
  const int total = block_excl_scan_1024(nch, sh, &ubase);
  // Unit list in expert order, with each unit's row count, staged in LDS; then written out
  // largest first (ties by position), so the long units start first and the hardware's
  // round-robin over XCDs spreads them evenly.
  __shared__ int2 s_unit[2048];
  __shared__ int s_rows[2048];
  __shared__ int s_sorted[2048];  // rows of the unit at each position of the written order
  if (e < E) {
    pslot[e] = split ? pbase : -1;
    for (int ch = 0; ch < nch; ++ch) {
      s_unit[ubase + ch] = make_int2(e, ch);
      s_rows[ubase + ch] = min(KC, c - ch * KC);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < total; i += 1024) {
    const int ri = s_rows[i];
    int rank = 0;
    for (int j = 0; j < total; ++j) {
      const int rj = s_rows[j];
      rank += (rj > ri) || (rj == ri && j < i);
    }
    units[rank] = s_unit[i];
    s_sorted[rank] = ri;
  }
  // Rows per XCD bucket (units b, b+8, ... in the order just written); the bucketed tile order
  // is used only when the fullest bucket is within 1/32 of the mean.
  __syncthreads();
  __shared__ int s_bucket[8];
  if (threadIdx.x < 8) {
    int rows = 0;
    for (int i = threadIdx.x; i < total; i += 8) rows += s_sorted[i];
    s_bucket[threadIdx.x] = rows;
  }
  __syncthreads();
  if (e == 0) {
    int mx = 0, sum = 0;
    for (int b = 0; b < 8; ++b) {
      mx = max(mx, s_bucket[b]);
      sum += s_bucket[b];
    }
    meta[0] = total;
    meta[1] = KC;
    meta[2] = (int64_t)mx * 8 * 32 <= (int64_t)sum * 33 ? 1 : 0;
  }
  (void)s_flag;
}

// dW[e] = bf16(sum over chunks, in chunk order, of the fp32 partials) for split experts.
__global__ __launch_bounds__(256) void wg_reduce_kernel(const float* __restrict__ partial,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ meta,
                                                        const int32_t* __restrict__ pslot, int64_t per_e,
                                                        uint16_t* __restrict__ dW) {
  const int e = blockIdx.y;
  const int ps = pslot[e];
  if (ps < 0) return;
  const int KC = meta[1];
  const int c = offsets[e + 1] - offsets[e];
  const int nch = (c + KC - 1) / KC;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i < per_e; i += (int64_t)gridDim.x * 256 * 8) {
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int ch = 0; ch < nch; ++ch) {
      const float* p = partial + (int64_t)(ps + ch) * per_e + i;
      const float4 u = *(const float4*)p, v = *(const float4*)(p + 4);
      a[0] += u.x; a[1] += u.y; a[2] += u.z; a[3] += u.w;
      a[4] += v.x; a[5] += v.y; a[6] += v.z; a[7] += v.w;
    }
    *(uint4*)&dW[(int64_t)e * per_e + i] = make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                                      pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7]));
  }
}

int wg_max_partials(const MoeShape& s) {
  const int64_t per = (int64_t)s.d * 2 * s.f * 4;  // the larger of dW1 / dW2, in fp32
  int64_t p = kWgPartialBudget / per;
  if (p > kWgMaxPartials) p = kWgMaxPartials;
  return p < 2 ? 0 : (int)p;
}

hipError_t launch_wg_split(const MoeShape& s, const int32_t* offsets, const WgSplit& sp, hipStream_t st) {
  wg_split_kernel<<<1, 1024, 0, st>>>(offsets, s.E, kWgChunk, sp.max_partials, sp.units, sp.meta, sp.pslot);
  return hipGetLastError();
}

hipError_t launch_wg_reduce(const MoeShape& s, const WgSplit& sp, int64_t per_e, uint16_t* dW, hipStream_t st) {
  if (sp.max_partials == 0) return hipSuccess;
  dim3 grid(64, s.E);
  wg_reduce_kernel<<<grid, 256, 0, st>>>(sp.partial, sp.offsets, sp.meta, sp.pslot, per_e, dW);
  return hipGetLastError();
}

hipError_t launch_gemm_dw2(const MoeShape& s, const uint16_t* As, const uint16_t* dy, const int32_t* offsets,
                           const int32_t* perm, const int32_t* tokrow, const WgSplit& sp, uint16_t* dW2, hipStream_t st) {
  GemmArgs g = base_args(s, offsets, perm, nullptr, nullptr);
  g.tokrow = tokrow;
  g.wg_units = sp.units;
  g.wg_meta = sp.meta;
  g.wg_pslot = sp.pslot;
  g.partial = sp.partial;
  g.A = As;
  g.lda = s.f;
  g.B = dy;
  g.ldb = s.d;
  g.Mo = s.f;
  g.N = s.d;
  g.C0 = dW2;
  g.ldc0 = s.d;
  const int bm = pick_bn(s.f), bn = pick_bn(s.d);
  dim3 grid((unsigned)((s.f / bm) * (s.d / bn) * (s.E + sp.max_partials)));
  return run<M_WG>(g, bm, bn, grid, st);
}

hipError_t launch_gemm_dw1(const MoeShape& s, const uint16_t* x, const uint16_t* dH, const int32_t* offsets,
                           const int32_t* perm, const int32_t* tokrow, const WgSplit& sp, uint16_t* dW1, hipStream_t st) {
  GemmArgs g = base_args(s, offsets, perm, nullptr, nullptr);
  g.tokrow = tokrow;
  g.wg_units = sp.units;
  g.wg_meta = sp.meta;
  g.wg_pslot = sp.pslot;
  g.partial = sp.partial;
  g.A = x;
  g.lda = s.d;
  g.B = dH;
  g.ldb = 2 * (int64_t)s.f;
  g.Mo = s.d;
  g.N = 2 * s.f;
  g.C0 = dW1;
  g.ldc0 = 2 * (int64_t)s.f;
  const int bm = pick_bn(s.d), bn = pick_bn(2 * s.f);
  dim3 grid((unsigned)((s.d / bm) * (2 * s.f / bn) * (s.E + sp.max_partials)));
  return run<M_WG1>(g, bm, bn, grid, st);
}

}  // namespace moe
