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
// Tiles are BM x BN x BK; 4 waves in a WM x WN grid each own (BM/WM) x (BN/WN) of the tile as
// 32x32 MFMA blocks.  Both operand tiles live in LDS K-contiguous per row with a 16-byte-chunk
// XOR swizzle (chunk ^ row%8), so every MFMA operand is one ds_read_b128.  Operands whose
// global layout is not K-contiguous are transposed in registers (4x8 blocks of bf16) on their
// way into LDS.  Two LDS stages: global loads for tile k+1 are in flight during tile k's MFMAs.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

enum GemmMode { M_UP = 0, M_DOWN = 1, M_DACT = 2, M_DX = 3, M_WG = 4 };

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
  const int2* tiles;
  const int32_t* ntiles;
  int gatherA, gatherB;  // operand rows come from token perm[pos] / k instead of position pos
  const float* topk_w;
  uint16_t* C0;
  int64_t ldc0;
  uint16_t* C1;
  int64_t ldc1;
  const uint16_t* Hs;
  int64_t ldh;
  float* dwp;
  int nparts;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// v if ok else 0
__device__ __forceinline__ u32x4 keep_if(u32x4 v, bool ok) {
  const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
  return v & m;
}

// Write a 4(k) x 8(n) block, loaded as 4 rows of 8 consecutive n, into the K-contiguous LDS
// tile: LDS row n gets 4 consecutive k (8 bytes) at k offset 4*kb.
template <int BK>
__device__ __forceinline__ void store_transposed(uint16_t* lds, int n_base, int kb, u32x4 v0, u32x4 v1, u32x4 v2,
                                                 u32x4 v3) {
  constexpr int KCH = BK / 8;
  const int chunk = kb >> 1, half = kb & 1;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t r0 = v0[w], r1 = v1[w], r2 = v2[w], r3 = v3[w];
    u32x2 ce, co;
    ce.x = (r0 & 0xFFFFu) | (r1 << 16);
    ce.y = (r2 & 0xFFFFu) | (r3 << 16);
    co.x = (r0 >> 16) | (r1 & 0xFFFF0000u);
    co.y = (r2 >> 16) | (r3 & 0xFFFF0000u);
    int n = n_base + 2 * w;
    *(u32x2*)&lds[n * BK + ((chunk ^ (n % KCH)) * 8) + half * 4] = ce;
    n += 1;
    *(u32x2*)&lds[n * BK + ((chunk ^ (n % KCH)) * 8) + half * 4] = co;
  }
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).  Renumber them so
// XCD j runs a contiguous range of logical tiles: neighbouring tiles share an expert's weights
// and a block of token rows, and now share one L2.
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  constexpr int NX = 8;
  const int q = G / NX, r = G % NX;
  const int x = bid % NX, i = bid / NX;
  return x * q + min(x, r) + i;
}

template <int MODE, int BM, int BN, int BK, int WM, int WN, int OCC>
__global__ __launch_bounds__(256, OCC) void grouped_gemm_kernel(const GemmArgs g) {
  constexpr int NTH = 256;
  static_assert(WM * WN == 4, "four waves");
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr int KCH = BK / 8;
  constexpr bool RAGGED_K = (MODE == M_WG);
  constexpr bool B_KC = (MODE == M_DACT || MODE == M_DX);
  static_assert(MODE != M_UP || (FN % 2 == 0), "gate/up pairing needs an even fragment count");

  // One LDS arena: two operand stages during the K loop, then the fp32 staging band of the
  // epilogue (64 rows x BN columns, rows padded by 4 floats against bank conflicts).
  constexpr int CPAD = BN + 4;
  constexpr int STAGE_BYTES = 2 * (BM + BN) * BK * 2;
  constexpr int CBAND_BYTES = 2 * 32 * CPAD * 4;
  static_assert(WM == 2, "the epilogue band holds one 32-row fragment block of each of 2 wave rows");
  __shared__ __attribute__((aligned(16))) uint8_t smem[STAGE_BYTES > CBAND_BYTES ? STAGE_BYTES : CBAND_BYTES];
  uint16_t (*sA)[BM * BK] = reinterpret_cast<uint16_t (*)[BM * BK]>(smem);
  uint16_t (*sB)[BN * BK] = reinterpret_cast<uint16_t (*)[BN * BK]>(smem + 2 * BM * BK * 2);
  float* cband = reinterpret_cast<float*>(smem);
  __shared__ float s_w[RAGGED_K ? 1 : BM];
  __shared__ int s_slot[RAGGED_K ? 1 : BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ------------------------------------------------------------------ tile coordinates
  int e, m0, mrows, n0, nt, kbeg, kend;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  if constexpr (RAGGED_K) {
    const int nN = g.N / BN;
    const int per_e = (g.Mo / BM) * nN;
    e = lid / per_e;
    nt = (lid % per_e) % nN;
    m0 = ((lid % per_e) / nN) * BM;
    mrows = BM;
    n0 = nt * BN;
    kbeg = g.offsets[e];
    kend = g.offsets[e + 1];
  } else {
    const int nN = (MODE == M_UP) ? g.f / (BN / 2) : g.N / BN;
    nt = lid % nN;
    const int tile = lid / nN;
    if (tile >= *g.ntiles) return;  // uniform: the block has no work
    const int2 te = g.tiles[tile];
    e = te.x;
    m0 = g.offsets[e] + te.y * BM;
    mrows = min(BM, g.offsets[e + 1] - m0);
    n0 = (MODE == M_UP) ? nt * (BN / 2) : nt * BN;
    kbeg = 0;
    kend = g.K;
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

  // ------------------------------------------------------------------ operand loaders
  // K-contiguous rows: thread owns 16-byte chunk c of rows tid/KCH + i*(NTH/KCH).
  constexpr int A_PER = RAGGED_K ? 1 : BM * KCH / NTH;
  constexpr int B_PER = B_KC ? BN * KCH / NTH : 1;
  // K-strided 4x8 units: thread owns k rows 4*kb..4*kb+3 and 8 columns of unit u.
  constexpr int UK = BK / 4;
  constexpr int A_UNITS = RAGGED_K ? (UK * (BM / 8)) / NTH : 1;
  constexpr int B_UNITS = B_KC ? 1 : (UK * (BN / 8)) / NTH;
  const int kc = tid % KCH;
  const int kb = tid % UK;

  const uint16_t* a_ptr[A_PER];
  bool a_ok[A_PER];
  const uint16_t* Bexp = g.B + (RAGGED_K ? 0 : (int64_t)e * g.b_estride);
  if constexpr (!RAGGED_K) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int r = tid / KCH + i * (NTH / KCH);
      a_ok[i] = r < mrows;
      const int pos = m0 + (a_ok[i] ? r : 0);  // rows past the expert's end read row m0, then mask
      const int64_t src = g.gatherA ? (int64_t)(g.perm[pos] / g.kslots) : (int64_t)pos;
      a_ptr[i] = g.A + src * g.lda + kc * 8;
    }
  }
  // K-contiguous B rows n0 + tid/KCH + i*(NTH/KCH): one base pointer and a fixed row step
  const uint16_t* b_base = Bexp + (int64_t)(n0 + tid / KCH) * g.ldb + kc * 8;
  const int64_t b_step = (int64_t)(NTH / KCH) * g.ldb;
  // global column of LDS row n for the K-strided B operand (UP pairs gate and up columns)
  auto b_col = [&](int n) __attribute__((always_inline)) -> int {
    if constexpr (MODE == M_UP) return n < BN / 2 ? n0 + n : g.f + n0 + (n - BN / 2);
    else return n0 + n;
  };

  constexpr int NA = RAGGED_K ? 4 * A_UNITS : A_PER;
  constexpr int NB = B_KC ? B_PER : 4 * B_UNITS;
  u32x4 a_buf[NA];
  u32x4 b_buf[NB];

  auto load_tiles = [&](int k0) __attribute__((always_inline)) {
    if constexpr (!RAGGED_K) {
#pragma unroll
      for (int i = 0; i < A_PER; ++i) {
        a_buf[i] = keep_if(*(const u32x4*)(a_ptr[i] + k0), a_ok[i]);
      }
      if constexpr (B_KC) {
#pragma unroll
        for (int i = 0; i < B_PER; ++i) b_buf[i] = *(const u32x4*)(b_base + i * b_step + k0);
      } else {
#pragma unroll
        for (int u = 0; u < B_UNITS; ++u) {
          const int cb = tid / UK + u * (NTH / UK);
          const uint16_t* base = Bexp + (int64_t)(k0 + 4 * kb) * g.ldb + b_col(cb * 8);
#pragma unroll
          for (int r = 0; r < 4; ++r) b_buf[4 * u + r] = *(const u32x4*)(base + (int64_t)r * g.ldb);
        }
      }
    } else {
      // ragged K: rows pos = k0 + 4*kb + r of this expert, masked past kend
      // rows past kend read the expert's first row (kbeg < kend whenever a tile is loaded), then mask
      const uint16_t* arow[4];
      const uint16_t* brow[4];
      bool ok[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p0 = k0 + 4 * kb + r;
        ok[r] = p0 < kend;
        const int pos = ok[r] ? p0 : kbeg;
        const int tok = g.perm[pos] / g.kslots;
        arow[r] = g.A + (int64_t)(g.gatherA ? tok : pos) * g.lda;
        brow[r] = g.B + (int64_t)(g.gatherB ? tok : pos) * g.ldb;
      }
#pragma unroll
      for (int u = 0; u < A_UNITS; ++u) {
        const int cb = tid / UK + u * (NTH / UK);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a_buf[4 * u + r] = keep_if(*(const u32x4*)(arow[r] + m0 + cb * 8), ok[r]);
        }
      }
#pragma unroll
      for (int u = 0; u < B_UNITS; ++u) {
        const int cb = tid / UK + u * (NTH / UK);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          b_buf[4 * u + r] = keep_if(*(const u32x4*)(brow[r] + n0 + cb * 8), ok[r]);
        }
      }
    }
  };

  auto store_tiles = [&](int buf) __attribute__((always_inline)) {
    uint16_t* la = sA[buf];
    uint16_t* lb = sB[buf];
    if constexpr (!RAGGED_K) {
#pragma unroll
      for (int i = 0; i < A_PER; ++i) {
        const int r = tid / KCH + i * (NTH / KCH);
        *(u32x4*)&la[r * BK + ((kc ^ (r % KCH)) * 8)] = a_buf[i];
      }
    } else {
#pragma unroll
      for (int u = 0; u < A_UNITS; ++u)
        store_transposed<BK>(la, (tid / UK + u * (NTH / UK)) * 8, kb, a_buf[4 * u], a_buf[4 * u + 1], a_buf[4 * u + 2],
                             a_buf[4 * u + 3]);
    }
    if constexpr (B_KC) {
#pragma unroll
      for (int i = 0; i < B_PER; ++i) {
        const int r = tid / KCH + i * (NTH / KCH);
        *(u32x4*)&lb[r * BK + ((kc ^ (r % KCH)) * 8)] = b_buf[i];
      }
    } else {
#pragma unroll
      for (int u = 0; u < B_UNITS; ++u)
        store_transposed<BK>(lb, (tid / UK + u * (NTH / UK)) * 8, kb, b_buf[4 * u], b_buf[4 * u + 1], b_buf[4 * u + 2],
                             b_buf[4 * u + 3]);
    }
  };

  // LDS row of the wave's j-th 32-column B fragment
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

  auto compute = [&](int buf) __attribute__((always_inline)) {
    const uint16_t* la = sA[buf];
    const uint16_t* lb = sB[buf];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      bf16x8_t af[FM], bv[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * TM + i * 32 + (lane & 31);
        af[i] = *(const bf16x8_t*)&la[r * BK + ((ch ^ (r % KCH)) * 8)];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = b_row(j) + (lane & 31);
        bv[j] = *(const bf16x8_t*)&lb[r * BK + ((ch ^ (r % KCH)) * 8)];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bv[j], acc[i][j], 0, 0, 0);
    }
  };

  // ------------------------------------------------------------------ main loop
  const int nk = (kend - kbeg + BK - 1) / BK;
  if (nk > 0) {
    load_tiles(kbeg);
    store_tiles(0);
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
      const int cur = it & 1;
      const bool more = it + 1 < nk;
      if (more) load_tiles(kbeg + (it + 1) * BK);
      compute(cur);
      if (more) store_tiles(cur ^ 1);
      __syncthreads();
    }
  }
  __syncthreads();

  // ------------------------------------------------------------------ epilogues
  // Pass i stages fragment row-block i of both wave rows: band row q = 32*wm + (row in block),
  // tile row = wm*TM + 32*i + (q % 32); band column = the LDS B row of the value (for UP:
  // gate columns [0, BN/2), up columns [BN/2, BN)).  32x32 accumulator layout: lane holds
  // column lane%32 and rows 8*(r/4) + 4*(lane/32) + r%4, r = 0..15.
  const int lcol = lane & 31;
  constexpr int CH = BN / 8;             // 8-column chunks per band row
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int c = b_row(j) + lcol;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = 32 * wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        cband[q * CPAD + c] = acc[i][j][r];
      }
    }
    __syncthreads();
    auto tile_row = [&](int q) __attribute__((always_inline)) { return (q >> 5) * TM + 32 * i + (q & 31); };
    if constexpr (MODE == M_UP) {
      // chunk = 8 gate columns + the matching 8 up columns of one row
      for (int id = tid; id < 64 * (CH / 2); id += NTH) {
        const int q = id / (CH / 2), cc = id % (CH / 2);
        const int lr = tile_row(q);
        if (lr < mrows) {
          const float* gp = &cband[q * CPAD + cc * 8];
          const float* up = &cband[q * CPAD + BN / 2 + cc * 8];
          const float w = s_w[lr];
          uint32_t hg[4], hu[4], as[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float g0 = gp[2 * t], g1 = gp[2 * t + 1], u0 = up[2 * t], u1 = up[2 * t + 1];
            hg[t] = pack_bf16x2(g0, g1);
            hu[t] = pack_bf16x2(u0, u1);
            as[t] = pack_bf16x2(w * g0 * sigmoidf_fast(g0) * u0, w * g1 * sigmoidf_fast(g1) * u1);
          }
          const int64_t pos = m0 + lr;
          const int col = n0 + cc * 8;
          *(uint4*)&g.C0[pos * g.ldc0 + col] = make_uint4(hg[0], hg[1], hg[2], hg[3]);
          *(uint4*)&g.C0[pos * g.ldc0 + g.f + col] = make_uint4(hu[0], hu[1], hu[2], hu[3]);
          *(uint4*)&g.C1[pos * g.ldc1 + col] = make_uint4(as[0], as[1], as[2], as[3]);
        }
      }
    } else if constexpr (MODE == M_DACT) {
      // G = dL/dAs.  a = silu(g) u from the saved H; d_topk_w partial = <G, a> over this
      // tile's columns; da = w G; dH = [da u sig(g) (1 + g (1 - sig(g))), da silu(g)].
      // A row's CH chunks sit in CH consecutive lanes (CH = 32 or 16), summed by a fixed
      // butterfly; chunk 0's lane writes the row's partial.
      static_assert(CH == 32 || CH == 16, "row chunks must map onto one half-wave");
      for (int id = tid; id < 64 * CH; id += NTH) {
        const int q = id / CH, cc = id % CH;
        const int lr = tile_row(q);
        const bool ok = lr < mrows;
        float part = 0.0f;
        if (ok) {
          const int64_t pos = m0 + lr;
          const int col = n0 + cc * 8;
          const uint4 hg = *(const uint4*)&g.Hs[pos * g.ldh + col];
          const uint4 hu = *(const uint4*)&g.Hs[pos * g.ldh + g.f + col];
          const float* Gp = &cband[q * CPAD + cc * 8];
          const float w = s_w[lr];
          uint32_t dg[4], du[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t wg = word_of(hg, t), wu = word_of(hu, t);
            float r0, r1, s0, s1;
            {
              const float gv = lo_bf16(wg), uv = lo_bf16(wu), G = Gp[2 * t];
              const float sg = sigmoidf_fast(gv), sl = gv * sg, da = w * G;
              part += G * (sl * uv);
              r0 = da * uv * sg * (1.0f + gv * (1.0f - sg));
              s0 = da * sl;
            }
            {
              const float gv = hi_bf16(wg), uv = hi_bf16(wu), G = Gp[2 * t + 1];
              const float sg = sigmoidf_fast(gv), sl = gv * sg, da = w * G;
              part += G * (sl * uv);
              r1 = da * uv * sg * (1.0f + gv * (1.0f - sg));
              s1 = da * sl;
            }
            dg[t] = pack_bf16x2(r0, r1);
            du[t] = pack_bf16x2(s0, s1);
          }
          *(uint4*)&g.C0[pos * g.ldc0 + col] = make_uint4(dg[0], dg[1], dg[2], dg[3]);
          *(uint4*)&g.C0[pos * g.ldc0 + g.f + col] = make_uint4(du[0], du[1], du[2], du[3]);
        }
#pragma unroll
        for (int m = CH / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
        if (ok && cc == 0) g.dwp[(int64_t)(m0 + lr) * g.nparts + nt] = part;
      }
    } else {
      // plain bf16 store: DOWN/DX rows go to the pair's slot, WG rows to dW[e]
      for (int id = tid; id < 64 * CH; id += NTH) {
        const int q = id / CH, cc = id % CH;
        const int lr = tile_row(q);
        if (lr < mrows) {
          const float* cp = &cband[q * CPAD + cc * 8];
          const uint4 o = make_uint4(pack_bf16x2(cp[0], cp[1]), pack_bf16x2(cp[2], cp[3]),
                                     pack_bf16x2(cp[4], cp[5]), pack_bf16x2(cp[6], cp[7]));
          int64_t orow;
          if constexpr (MODE == M_WG) orow = (int64_t)e * g.Mo + m0 + lr;
          else orow = s_slot[lr];
          *(uint4*)&g.C0[orow * g.ldc0 + n0 + cc * 8] = o;
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------- host launchers
namespace {
constexpr int BK = 64;

// Launch MODE with a BM x BN tile: 256x256 (waves own 128x128, one block per CU) where the
// output width allows, else 256x128 / 128x256 / 128x128.
template <int MODE>
hipError_t run(const GemmArgs& g, int bm, int bn, dim3 grid, hipStream_t st) {
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  if (bm == 256 && bn == 256)
    grouped_gemm_kernel<MODE, 256, 256, BK, 2, 2, 1><<<grid, 256, 0, st>>>(g);
  else if (bm == 256 && bn == 128)
    grouped_gemm_kernel<MODE, 256, 128, BK, 2, 2, 1><<<grid, 256, 0, st>>>(g);
  else if (MODE == M_WG && bm == 128 && bn == 256)
    grouped_gemm_kernel<MODE, 128, 256, BK, 2, 2, 1><<<grid, 256, 0, st>>>(g);
  else if (bm == 128 && bn == 128)
    grouped_gemm_kernel<MODE, 128, 128, BK, 2, 2, 2><<<grid, 256, 0, st>>>(g);
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

int max_row_tiles(int64_t A, int E, int bm) {
  const int64_t t = (A + bm - 1) / bm + (A < E ? A : E);
  return (int)t;
}

hipError_t launch_gemm_up(const MoeShape& s, const uint16_t* x, const uint16_t* W1, const float* topk_w,
                          const int32_t* offsets, const int32_t* perm, const int2* tiles, const int32_t* ntiles,
                          uint16_t* H, uint16_t* As, hipStream_t st) {
  GemmArgs g = base_args(s, offsets, perm, tiles, ntiles);
  g.A = x;
  g.lda = s.d;
  g.gatherA = 1;
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
  const int64_t A = (int64_t)s.T * s.k;
  const int bn = 256;  // 128 gate + 128 up columns (f is a multiple of 128)
  dim3 grid((unsigned)(max_row_tiles(A, s.E, kGemmBM) * (s.f / (bn / 2))));
  return run<M_UP>(g, kGemmBM, bn, grid, st);
}

hipError_t launch_gemm_down(const MoeShape& s, const uint16_t* As, const uint16_t* W2, const int32_t* offsets,
                            const int32_t* perm, const int2* tiles, const int32_t* ntiles, uint16_t* Op,
                            hipStream_t st) {
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
  const int64_t A = (int64_t)s.T * s.k;
  const int bn = pick_bn(s.d);
  dim3 grid((unsigned)(max_row_tiles(A, s.E, kGemmBM) * (s.d / bn)));
  return run<M_DOWN>(g, kGemmBM, bn, grid, st);
}

hipError_t launch_gemm_dact(const MoeShape& s, const uint16_t* dy, const uint16_t* W2, const uint16_t* H,
                            const float* topk_w, const int32_t* offsets, const int32_t* perm, const int2* tiles,
                            const int32_t* ntiles, uint16_t* dH, float* dwp, hipStream_t st) {
  GemmArgs g = base_args(s, offsets, perm, tiles, ntiles);
  g.A = dy;
  g.lda = s.d;
  g.gatherA = 1;
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
  const int bn = dact_bn(s.f);
  g.nparts = s.f / bn;
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

hipError_t launch_gemm_dw2(const MoeShape& s, const uint16_t* As, const uint16_t* dy, const int32_t* offsets,
                           const int32_t* perm, uint16_t* dW2, hipStream_t st) {
  GemmArgs g = base_args(s, offsets, perm, nullptr, nullptr);
  g.A = As;
  g.lda = s.f;
  g.gatherA = 0;
  g.B = dy;
  g.ldb = s.d;
  g.gatherB = 1;
  g.Mo = s.f;
  g.N = s.d;
  g.C0 = dW2;
  g.ldc0 = s.d;
  const int bm = pick_bn(s.f), bn = pick_bn(s.d);
  dim3 grid((unsigned)((s.f / bm) * (s.d / bn) * s.E));
  return run<M_WG>(g, bm, bn, grid, st);
}

hipError_t launch_gemm_dw1(const MoeShape& s, const uint16_t* x, const uint16_t* dH, const int32_t* offsets,
                           const int32_t* perm, uint16_t* dW1, hipStream_t st) {
  GemmArgs g = base_args(s, offsets, perm, nullptr, nullptr);
  g.A = x;
  g.lda = s.d;
  g.gatherA = 1;
  g.B = dH;
  g.ldb = 2 * (int64_t)s.f;
  g.gatherB = 0;
  g.Mo = s.d;
  g.N = 2 * s.f;
  g.C0 = dW1;
  g.ldc0 = 2 * (int64_t)s.f;
  const int bm = pick_bn(s.d), bn = pick_bn(2 * s.f);
  dim3 grid((unsigned)((s.d / bm) * (2 * s.f / bn) * s.E));
  return run<M_WG>(g, bm, bn, grid, st);
}

}  // namespace moe
