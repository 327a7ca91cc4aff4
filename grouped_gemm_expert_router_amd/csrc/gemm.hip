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

__device__ __forceinline__ uint32_t word_of(const uint4& v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

// Write a 4(k) x 8(n) block, loaded as 4 rows of 8 consecutive n, into the K-contiguous LDS
// tile: LDS row n gets 4 consecutive k (8 bytes) at k offset 4*kb.
template <int BK>
__device__ __forceinline__ void store_transposed(uint16_t* lds, int n_base, int kb, const uint4 (&v)[4]) {
  constexpr int KCH = BK / 8;
  const int chunk = kb >> 1, half = kb & 1;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t r0 = word_of(v[0], w), r1 = word_of(v[1], w), r2 = word_of(v[2], w), r3 = word_of(v[3], w);
    const uint2 ce = make_uint2((r0 & 0xFFFFu) | (r1 << 16), (r2 & 0xFFFFu) | (r3 << 16));
    const uint2 co = make_uint2((r0 >> 16) | (r1 & 0xFFFF0000u), (r2 >> 16) | (r3 & 0xFFFF0000u));
    int n = n_base + 2 * w;
    *(uint2*)&lds[n * BK + ((chunk ^ (n % KCH)) * 8) + half * 4] = ce;
    n += 1;
    *(uint2*)&lds[n * BK + ((chunk ^ (n % KCH)) * 8) + half * 4] = co;
  }
}

template <int MODE, int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(const GemmArgs g) {
  constexpr int NTH = 256;
  static_assert(WM * WN == 4, "four waves");
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr int KCH = BK / 8;
  constexpr bool RAGGED_K = (MODE == M_WG);
  constexpr bool B_KC = (MODE == M_DACT || MODE == M_DX);
  static_assert(MODE != M_UP || (FN % 2 == 0), "gate/up pairing needs an even fragment count");

  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];
  __shared__ float s_w[RAGGED_K ? 1 : BM];
  __shared__ int s_slot[RAGGED_K ? 1 : BM];
  __shared__ float s_red[MODE == M_DACT ? WN : 1][MODE == M_DACT ? BM : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ------------------------------------------------------------------ tile coordinates
  int e, m0, mrows, n0, nt, kbeg, kend;
  if constexpr (RAGGED_K) {
    const int nN = g.N / BN;
    nt = blockIdx.x % nN;
    e = blockIdx.y;
    m0 = (blockIdx.x / nN) * BM;
    mrows = BM;
    n0 = nt * BN;
    kbeg = g.offsets[e];
    kend = g.offsets[e + 1];
  } else {
    const int nN = (MODE == M_UP) ? g.f / (BN / 2) : g.N / BN;
    nt = blockIdx.x % nN;
    const int tile = blockIdx.x / nN;
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
  const uint16_t* b_ptr[B_PER];
  const uint16_t* Bexp = g.B + (RAGGED_K ? 0 : (int64_t)e * g.b_estride);
  if constexpr (!RAGGED_K) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int r = tid / KCH + i * (NTH / KCH);
      const uint16_t* p = nullptr;
      if (r < mrows) {
        const int pos = m0 + r;
        const int64_t src = g.gatherA ? (int64_t)(g.perm[pos] / g.kslots) : (int64_t)pos;
        p = g.A + src * g.lda + kc * 8;
      }
      a_ptr[i] = p;
    }
  }
  if constexpr (B_KC) {
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int r = tid / KCH + i * (NTH / KCH);
      b_ptr[i] = Bexp + (int64_t)(n0 + r) * g.ldb + kc * 8;
    }
  }
  // global column of LDS row n for the K-strided B operand (UP pairs gate and up columns)
  auto b_col = [&](int n) -> int {
    if constexpr (MODE == M_UP) return n < BN / 2 ? n0 + n : g.f + n0 + (n - BN / 2);
    else return n0 + n;
  };

  uint4 a_buf[RAGGED_K ? A_UNITS : A_PER][RAGGED_K ? 4 : 1];
  uint4 b_buf[B_KC ? B_PER : B_UNITS][B_KC ? 1 : 4];
  const uint4 zero4 = make_uint4(0, 0, 0, 0);

  auto load_tiles = [&](int k0) {
    if constexpr (!RAGGED_K) {
#pragma unroll
      for (int i = 0; i < A_PER; ++i) a_buf[i][0] = a_ptr[i] ? *(const uint4*)(a_ptr[i] + k0) : zero4;
      if constexpr (B_KC) {
#pragma unroll
        for (int i = 0; i < B_PER; ++i) b_buf[i][0] = *(const uint4*)(b_ptr[i] + k0);
      } else {
#pragma unroll
        for (int u = 0; u < B_UNITS; ++u) {
          const int cb = tid / UK + u * (NTH / UK);
          const uint16_t* base = Bexp + (int64_t)(k0 + 4 * kb) * g.ldb + b_col(cb * 8);
#pragma unroll
          for (int r = 0; r < 4; ++r) b_buf[u][r] = *(const uint4*)(base + (int64_t)r * g.ldb);
        }
      }
    } else {
      // ragged K: rows pos = k0 + 4*kb + r of this expert, masked past kend
      const uint16_t* arow[4];
      const uint16_t* brow[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = k0 + 4 * kb + r;
        arow[r] = nullptr;
        brow[r] = nullptr;
        if (pos < kend) {
          const int tok = g.perm[pos] / g.kslots;
          arow[r] = g.A + (int64_t)(g.gatherA ? tok : pos) * g.lda;
          brow[r] = g.B + (int64_t)(g.gatherB ? tok : pos) * g.ldb;
        }
      }
#pragma unroll
      for (int u = 0; u < A_UNITS; ++u) {
        const int cb = tid / UK + u * (NTH / UK);
#pragma unroll
        for (int r = 0; r < 4; ++r) a_buf[u][r] = arow[r] ? *(const uint4*)(arow[r] + m0 + cb * 8) : zero4;
      }
#pragma unroll
      for (int u = 0; u < B_UNITS; ++u) {
        const int cb = tid / UK + u * (NTH / UK);
#pragma unroll
        for (int r = 0; r < 4; ++r) b_buf[u][r] = brow[r] ? *(const uint4*)(brow[r] + n0 + cb * 8) : zero4;
      }
    }
  };

  auto store_tiles = [&](int buf) {
    uint16_t* la = sA[buf];
    uint16_t* lb = sB[buf];
    if constexpr (!RAGGED_K) {
#pragma unroll
      for (int i = 0; i < A_PER; ++i) {
        const int r = tid / KCH + i * (NTH / KCH);
        *(uint4*)&la[r * BK + ((kc ^ (r % KCH)) * 8)] = a_buf[i][0];
      }
    } else {
#pragma unroll
      for (int u = 0; u < A_UNITS; ++u) store_transposed<BK>(la, (tid / UK + u * (NTH / UK)) * 8, kb, a_buf[u]);
    }
    if constexpr (B_KC) {
#pragma unroll
      for (int i = 0; i < B_PER; ++i) {
        const int r = tid / KCH + i * (NTH / KCH);
        *(uint4*)&lb[r * BK + ((kc ^ (r % KCH)) * 8)] = b_buf[i][0];
      }
    } else {
#pragma unroll
      for (int u = 0; u < B_UNITS; ++u) store_transposed<BK>(lb, (tid / UK + u * (NTH / UK)) * 8, kb, b_buf[u]);
    }
  };

  // LDS row of the wave's j-th 32-column B fragment
  auto b_row = [&](int j) -> int {
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

  auto compute = [&](int buf) {
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
  // 32x32 fp32 accumulator layout: lane holds column lane%32 and rows
  // 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15.
  const int lcol = lane & 31;
  auto lrow = [&](int i, int r) { return wm * TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); };

  if constexpr (MODE == M_UP) {
    // H[pos] = [g | u] (bf16), As[pos] = w * silu(g) * u (bf16)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
        const int col = n0 + wn * (TN / 2) + j * 32 + lcol;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = lrow(i, r);
          if (lr < mrows) {
            const int64_t pos = m0 + lr;
            const float gv = acc[i][j][r], uv = acc[i][j + FN / 2][r];
            g.C0[pos * g.ldc0 + col] = f32_to_bf16(gv);
            g.C0[pos * g.ldc0 + g.f + col] = f32_to_bf16(uv);
            g.C1[pos * g.ldc1 + col] = f32_to_bf16(s_w[lr] * gv * sigmoidf_fast(gv) * uv);
          }
        }
      }
  } else if constexpr (MODE == M_DOWN || MODE == M_DX) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * TN + j * 32 + lcol;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = lrow(i, r);
          if (lr < mrows) g.C0[(int64_t)s_slot[lr] * g.ldc0 + col] = f32_to_bf16(acc[i][j][r]);
        }
      }
  } else if constexpr (MODE == M_DACT) {
    // G = dL/dAs.  a = silu(g) u from the saved H; d_topk_w partial = <G, a> over this tile's
    // columns; da = w G; dH = [da u sig(g) (1 + g (1 - sig(g))), da silu(g)].
    float part[FM][16];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[i][r] = 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * TN + j * 32 + lcol;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = lrow(i, r);
          if (lr < mrows) {
            const int64_t pos = m0 + lr;
            const float gv = bf16_to_f32(g.Hs[pos * g.ldh + col]);
            const float uv = bf16_to_f32(g.Hs[pos * g.ldh + g.f + col]);
            const float G = acc[i][j][r];
            const float sg = sigmoidf_fast(gv);
            const float sl = gv * sg;
            part[i][r] += G * (sl * uv);
            const float da = s_w[lr] * G;
            g.C0[pos * g.ldc0 + col] = f32_to_bf16(da * uv * sg * (1.0f + gv * (1.0f - sg)));
            g.C0[pos * g.ldc0 + g.f + col] = f32_to_bf16(da * sl);
          }
        }
      }
    // row sums across the 32 columns a half-wave holds (fixed butterfly order)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = part[i][r];
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
        if (lcol == 0) s_red[wn][lrow(i, r)] = v;
      }
    __syncthreads();
    for (int r = tid; r < mrows; r += NTH) {
      float v = 0.0f;
#pragma unroll
      for (int q = 0; q < WN; ++q) v += s_red[q][r];
      g.dwp[(int64_t)(m0 + r) * g.nparts + nt] = v;
    }
  } else {  // M_WG
    uint16_t* out = g.C0 + (int64_t)e * g.Mo * g.N;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * TN + j * 32 + lcol;
#pragma unroll
        for (int r = 0; r < 16; ++r) out[(int64_t)(m0 + lrow(i, r)) * g.N + col] = f32_to_bf16(acc[i][j][r]);
      }
  }
}

// ---------------------------------------------------------------------- host launchers
namespace {
constexpr int BM = kGemmBM, BN = 128, BK = 64;

template <int MODE>
hipError_t run(const GemmArgs& g, dim3 grid, hipStream_t st) {
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  grouped_gemm_kernel<MODE, BM, BN, BK, 2, 2><<<grid, 256, 0, st>>>(g);
  return hipGetLastError();
}

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
  dim3 grid((unsigned)(max_row_tiles(A, s.E, BM) * (s.f / (BN / 2))));
  return run<M_UP>(g, grid, st);
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
  dim3 grid((unsigned)(max_row_tiles(A, s.E, BM) * (s.d / BN)));
  return run<M_DOWN>(g, grid, st);
}

hipError_t launch_gemm_dact(const MoeShape& s, const uint16_t* dy, const uint16_t* W2, const uint16_t* H,
                            const float* topk_w, const int32_t* offsets, const int32_t* perm, const int2* tiles,
                            const int32_t* ntiles, uint16_t* dH, float* dwp, hipStream_t st) {
  static_assert(kDactBN == BN, "partial count follows the DACT tile width");
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
  g.nparts = s.f / BN;
  const int64_t A = (int64_t)s.T * s.k;
  dim3 grid((unsigned)(max_row_tiles(A, s.E, BM) * (s.f / BN)));
  return run<M_DACT>(g, grid, st);
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
  dim3 grid((unsigned)(max_row_tiles(A, s.E, BM) * (s.d / BN)));
  return run<M_DX>(g, grid, st);
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
  dim3 grid((unsigned)((s.f / BM) * (s.d / BN)), (unsigned)s.E);
  return run<M_WG>(g, grid, st);
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
  dim3 grid((unsigned)((s.d / BM) * (2 * s.f / BN)), (unsigned)s.E);
  return run<M_WG>(g, grid, st);
}

}  // namespace moe
