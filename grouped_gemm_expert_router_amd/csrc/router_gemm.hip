// The router's dense products on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// A learned router scores every token against every expert before the top-k choice (page "Az
// NVIDIA szerint tízszer gyorsabb lett a dropless MoE tanítása JAX-ban", section "A dropless MoE
// minden tokent feldolgoz").  With the gate weight Wg [d, E]:
//   LOGITS  logits[T, E] = x[T, d] . Wg            fp32 out
//   DX      dx[T, d]    += d_logits[T, E] . Wg^T   added in fp32 to the bf16 dx, one rounding
//   DWG     dWg[d, E]    = x^T . d_logits          K = tokens, cut into slices whose fp32 partials
//                                                  are summed in slice order (deterministic)
// fp32 operands (d_logits) are rounded to bf16 when staged.  These products are small next to the
// expert GEMMs (2*T*d*E flop each), so the kernel is a plain 64x64x32 tile: 4 waves of one 32x32
// MFMA block each, operands loaded into registers one k step ahead and staged through two LDS
// buffers with K contiguous (rows padded to 80 bytes, so the 16-byte fragment reads of 16 lanes
// hit 16 distinct bank groups).  Every load and store is bounds-checked: T, d and E are arbitrary
// within the layer's limits (E need not be a multiple of anything).
#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace moe {

enum RouterMode { R_LOGITS = 0, R_DX = 1, R_DWG = 2 };

struct RouterArgs {
  const void* A;  // element (m, k) at A[m*lda + k], or A[k*lda + m] when A_KM
  int64_t lda;
  const void* B;  // element (k, n) at B[k*ldb + n], or B[n*ldb + k] when B_NK
  int64_t ldb;
  int M, N, K;
  int kslice;      // K rows per slice (DWG); the grid's third coordinate is the slice
  int mt, nt;      // tiles along M and N
  int64_t ntotal;  // mt * nt * slices
  int vecA, vecB;  // 1: rows are 16-byte aligned, so 8 in-bounds values load as vectors
  void* C;
  int64_t ldc;
  float* partial;  // DWG with several slices: [slices, M, N]
};

constexpr int kRBM = 64, kRBN = 64, kRBK = 32, kRLd = 40;  // LDS row: 32 k values + 8 padding

template <bool F32>
__device__ __forceinline__ uint16_t to_bf16(const void* p, int64_t i) {
  if constexpr (F32) return f32_to_bf16(((const float*)p)[i]);
  else return ((const uint16_t*)p)[i];
}

// 8 consecutive values of one source row (bounds lo..lim along that row) -> 8 bf16.
template <bool F32>
__device__ __forceinline__ void load8(const void* base, int64_t row_off, int c0, int lim, bool vec, uint16_t (&v)[8]) {
  if (vec && c0 + 8 <= lim) {
    if constexpr (F32) {
      const float4* p = (const float4*)((const float*)base + row_off + c0);
      const float4 a = p[0], b = p[1];
      v[0] = f32_to_bf16(a.x); v[1] = f32_to_bf16(a.y); v[2] = f32_to_bf16(a.z); v[3] = f32_to_bf16(a.w);
      v[4] = f32_to_bf16(b.x); v[5] = f32_to_bf16(b.y); v[6] = f32_to_bf16(b.z); v[7] = f32_to_bf16(b.w);
    } else {
      const uint4 w = *(const uint4*)((const uint16_t*)base + row_off + c0);
      const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = (uint16_t)(q[i] & 0xFFFFu);
        v[2 * i + 1] = (uint16_t)(q[i] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (c0 + i < lim) ? to_bf16<F32>(base, row_off + c0 + i) : (uint16_t)0;
  }
}

template <int MODE, bool A_KM, bool A_F32, bool B_NK, bool B_F32>
__global__ __launch_bounds__(256) void router_gemm_kernel(const RouterArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][kRBM * kRLd];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][kRBN * kRLd];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // one (M tile, N tile, slice) per iteration; the grid strides over all of them
  for (int64_t bid = blockIdx.x; bid < g.ntotal; bid += gridDim.x) {
    const int tn = (int)(bid % g.nt), tm = (int)((bid / g.nt) % g.mt), slice = (int)(bid / ((int64_t)g.nt * g.mt));
    const int m0 = tm * kRBM, n0 = tn * kRBN;
    const int kbeg = slice * g.kslice, kend = min(g.K, kbeg + g.kslice);

    // Operand tile of 64 rows (m or n) x 32 k.  K-contiguous source: thread -> row tid/4, k chunk
    // tid%4 (8 values, one 16-byte LDS write).  M/N-contiguous source: thread -> k row tid/8,
    // 8 consecutive m (n) from 8*(tid%8), written transposed.
    auto load_tile = [&](const void* src, int64_t ld, bool vec, bool kmajor_src, bool f32, int r0, int rlim, int k0,
                         uint16_t (&v)[8]) __attribute__((always_inline)) {
      if (!kmajor_src) {  // src[r*ld + k]
        const int r = r0 + (tid >> 2), kc = k0 + 8 * (tid & 3);
        if (r < rlim) {
          if (f32) load8<true>(src, (int64_t)r * ld, kc, kend, vec, v);
          else load8<false>(src, (int64_t)r * ld, kc, kend, vec, v);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = 0;
        }
      } else {  // src[k*ld + r]
        const int k = k0 + (tid >> 3), rc = r0 + 8 * (tid & 7);
        if (k < kend) {
          if (f32) load8<true>(src, (int64_t)k * ld, rc, rlim, vec, v);
          else load8<false>(src, (int64_t)k * ld, rc, rlim, vec, v);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = 0;
        }
      }
    };
    auto store_tile = [&](uint16_t* s, bool kmajor_src, const uint16_t (&v)[8]) __attribute__((always_inline)) {
      if (!kmajor_src) {
        const int r = tid >> 2, c = 8 * (tid & 3);
        *(uint4*)(s + r * kRLd + c) = make_uint4(v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                                                 v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16));
      } else {
        const int k = tid >> 3, r = 8 * (tid & 7);
#pragma unroll
        for (int i = 0; i < 8; ++i) s[(r + i) * kRLd + k] = v[i];
      }
    };

    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    uint16_t va[8], vb[8];
    const int nk = kend > kbeg ? (kend - kbeg + kRBK - 1) / kRBK : 0;
    if (nk > 0) {
      load_tile(g.A, g.lda, g.vecA, A_KM, A_F32, m0, g.M, kbeg, va);
      load_tile(g.B, g.ldb, g.vecB, !B_NK, B_F32, n0, g.N, kbeg, vb);
    }
    for (int t = 0; t < nk; ++t) {
      const int st = t & 1;
      store_tile(sa[st], A_KM, va);
      store_tile(sb[st], !B_NK, vb);
      __syncthreads();
      if (t + 1 < nk) {  // the next step's loads are in flight during this step's MFMAs
        load_tile(g.A, g.lda, g.vecA, A_KM, A_F32, m0, g.M, kbeg + (t + 1) * kRBK, va);
        load_tile(g.B, g.ldb, g.vecB, !B_NK, B_F32, n0, g.N, kbeg + (t + 1) * kRBK, vb);
      }
      // lane l: row (column) 32*w + l%32, k = 16*kk + 8*(l/32) .. +7
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8_t af = *(const bf16x8_t*)(sa[st] + (wm * 32 + (lane & 31)) * kRLd + 16 * kk + 8 * (lane >> 5));
        const bf16x8_t bf = *(const bf16x8_t*)(sb[st] + (wn * 32 + (lane & 31)) * kRLd + 16 * kk + 8 * (lane >> 5));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
      }
    }

    // lane l holds column n = l%32 of the wave's block and rows 8*(r/4) + 4*(l/32) + r%4
    const int n = n0 + wn * 32 + (lane & 31);
    if (n < g.N) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m >= g.M) continue;
        const int64_t o = (int64_t)m * g.ldc + n;
        if constexpr (MODE == R_LOGITS) {
          ((float*)g.C)[o] = acc[r];
        } else if constexpr (MODE == R_DX) {
          uint16_t* c = (uint16_t*)g.C;
          c[o] = f32_to_bf16(bf16_to_f32(c[o]) + acc[r]);
        } else {
          if (g.partial) g.partial[((int64_t)slice * g.M + m) * g.N + n] = acc[r];
          else ((uint16_t*)g.C)[o] = f32_to_bf16(acc[r]);
        }
      }
    }
    __syncthreads();  // every wave is done with both LDS buffers before the next tile refills them
  }
}

// ---------------------------------------------------------------- E = 128 or 256
// With the gate's row a whole number of 16-byte chunks and E at most 256, each block owns whole
// rows of the output along E and its operands reach LDS by DMA (global_load_lds_dwordx4) in the
// layouts of the grouped GEMMs: K-contiguous tiles read with ds_read_b128 (KM), N- or
// M-contiguous ones with the transpose read (KN).  These products are bound by HBM (x, dx) and
// L2 (the gate and d_logits, re-read by every block), so the tiles favour bytes in flight over
// MFMA efficiency.  4 waves, 2 x 2.

// logits[T, E] = x . Wg: 64 token rows x all E columns per block, 3 stages of BK (128, or 64 for
// E = 256) along d.  Stage: x rows as BK/64 KM sub-tiles of 64 x 64, then Wg's BK rows (KN, E wide).
template <int EP>
__global__ __launch_bounds__(256, 1) void router_logits_fast_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ Wg, int T, int d,
                                                                   float* __restrict__ logits) {
  constexpr int BM = 64, BK = EP == 256 ? 64 : 128, S = 3;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * EP * 2, STAGE = A_BYTES + B_BYTES;
  constexpr int QA = A_BYTES / 4096, QB = B_BYTES / 4096, DPT = QA + QB;  // 1 KiB DMAs per wave
  constexpr int FN = EP / 64, RB = 512 / EP, CHB = EP / 8;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr_of(smem));
  const int m0 = blockIdx.x * BM;

  const uint16_t* a_src[QA];
  const uint16_t* b_src[QB];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int gi = wave * QA + q, h = gi / 8, row = 8 * (gi % 8) + lane / 8;
    const int c = (lane % 8) ^ km_swz<64>(row);
    a_src[q] = x + (int64_t)min(m0 + row, T - 1) * d + 64 * h + 8 * c;  // rows past T feed unstored outputs
  }
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int gi = wave * QB + q, kr = RB * gi + lane / CHB;
    const int c = (lane % CHB) ^ (4 * (kr & 3));
    b_src[q] = Wg + (int64_t)kr * EP + 8 * c;
  }
  auto issue = [&](int t, int st) __attribute__((always_inline)) {
    const uint32_t abase = lds0 + st * STAGE, bbase = abase + A_BYTES;
#pragma unroll
    for (int q = 0; q < QA; ++q) dma16(a_src[q] + t * BK, abase + (wave * QA + q) * 1024);
#pragma unroll
    for (int q = 0; q < QB; ++q) dma16(b_src[q] + (int64_t)t * BK * EP, bbase + (wave * QB + q) * 1024);
  };
  f32x16_t acc[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;

  const int nk = d / BK;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  for (int it = 0; it < nk; ++it) {
    if (it + 1 < nk) vm_wait_barrier<DPT>();
    else vm_wait_barrier<0>();
    if (it + 2 < nk) issue(it + 2, (it + 2) % S);
    const uint32_t abase = lds0 + (it % S) * STAGE, bbase = abase + A_BYTES;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const bf16x8_t af = read_km<64>(abase + (kk / 4) * 8192, wm * 32 + (lane & 31), 2 * (kk % 4) + (lane >> 5));
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const bf16x8_t bv = read_kn<EP>(bbase, wn * (EP / 2) + 32 * j, kk, lane);
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, af, acc[j], 0, 0, 0);
      }
    }
  }
  // lane l holds token row l % 32 of the wave's rows and, per block j, columns 8 (r / 4) +
  // 4 (l / 32) + r % 4
  const int row = m0 + wm * 32 + (lane & 31);
  if (row < T) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = wn * (EP / 2) + 32 * j + 8 * q + 4 * (lane >> 5);
        *(float4*)(logits + (int64_t)row * EP + col) =
            make_float4(acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]);
      }
  }
}

// dx[T, d] += d_logits[T, E] . Wg^T.  A block owns 128 columns of d: the gate's rows n0 ..
// n0 + BN - 1 (K-contiguous: row i holds its E values) arrive once by DMA as KM sub-tiles of
// BN x 64 and stay in LDS while the block walks its 64-row token tiles (every rgroups-th tile).
// Per tile, d_logits rows are rounded to bf16 through registers (loaded one tile ahead) into KM
// sub-tiles of 64 x 64, the product takes the whole K = E at once, and the sum with dx (whose
// rows are loaded before the MFMAs) is taken in fp32 and rounded once.
template <int EP>
__global__ __launch_bounds__(256, EP == 128 ? 2 : 1) void router_dx_fast_kernel(const float* __restrict__ dl,
                                                                               const uint16_t* __restrict__ Wg,
                                                                               int T, int d, int rgroups,
                                                                               uint16_t* __restrict__ dx) {
  constexpr int BM = 64, BN = 128, KS = EP / 64;
  constexpr int A_SUB = BM * 128, B_SUB = BN * 128;  // bytes of one 64-deep sub-tile
  constexpr int A_BYTES = KS * A_SUB, QB = KS * B_SUB / 4096;
  constexpr int FN = BN / 64, NV = BM * EP / 4 / 256;  // float4 of d_logits per thread per tile
  __shared__ __attribute__((aligned(1024))) uint8_t smem[KS * B_SUB + 2 * A_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr_of(smem));
  const uint32_t bbase = lds0, abase0 = lds0 + KS * B_SUB;
  const int nblk = d / BN;
  const int n0 = (blockIdx.x % nblk) * BN, rg = blockIdx.x / nblk;
  const int ntile = (T + BM - 1) / BM;
  // the gate's rows by DMA: instruction gi covers sub-tile gi / (B_SUB / 1024), rows
  // 8 (gi % (B_SUB / 1024)) + lane / 8
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int gi = wave * QB + q, h = gi / (B_SUB / 1024), row = 8 * (gi % (B_SUB / 1024)) + lane / 8;
    const int c = (lane % 8) ^ km_swz<64>(row);
    dma16(Wg + (int64_t)(n0 + row) * EP + 64 * h + 8 * c, bbase + gi * 1024);
  }
  // d_logits of token tile rt: float4 u of thread tid is element 4 (256 u + tid) of the 64 x E
  // tile, row-major; rows past T are zero
  auto load_dl = [&](int rt, float4 (&v)[NV]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int e4 = u * 256 + tid, row = e4 / (EP / 4), col = 4 * (e4 % (EP / 4));
      const int t = rt * BM + row;
      v[u] = t < T ? *(const float4*)(dl + (int64_t)t * EP + col) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_dl = [&](uint32_t ab, const float4 (&v)[NV]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int e4 = u * 256 + tid, row = e4 / (EP / 4), col = 4 * (e4 % (EP / 4));
      const uint32_t a = ab + (col / 64) * A_SUB + km_off<64>(row, (col % 64) / 8) + 2 * (col % 8);
      *(LDS_AS u32x2*)(uintptr_t)a = u32x2{pack_bf16x2(v[u].x, v[u].y), pack_bf16x2(v[u].z, v[u].w)};
    }
  };
  const int h = lane >> 5;
  float4 v[NV];
  if (rg < ntile) load_dl(rg, v);
  for (int rt = rg, i = 0; rt < ntile; rt += rgroups, ++i) {
    const uint32_t ab = abase0 + (i & 1) * A_BYTES;
    store_dl(ab, v);
    if (i == 0) vm_wait<0>();  // this wave's DMA of the gate
    lds_barrier();             // the tile (and the gate) visible to every wave
    if (rt + rgroups < ntile) load_dl(rt + rgroups, v);  // next tile, under this one's work
    // this lane's dx values: block j, half c: row t, columns 16c + 8h .. + 7 of the block
    const int t = rt * BM + wm * 32 + (lane & 31);
    uint4 o[FN][2];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        o[j][c] = t < T ? *(const uint4*)(dx + (int64_t)t * d + n0 + wn * (BN / 2) + 32 * j + 16 * c + 8 * h)
                        : make_uint4(0u, 0u, 0u, 0u);
    f32x16_t acc[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < EP / 16; ++kk) {
      const bf16x8_t af = read_km<64>(ab + (kk / 4) * A_SUB, wm * 32 + (lane & 31), 2 * (kk % 4) + (lane >> 5));
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const bf16x8_t bv =
            read_km<64>(bbase + (kk / 4) * B_SUB, wn * (BN / 2) + 32 * j + (lane & 31), 2 * (kk % 4) + (lane >> 5));
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, af, acc[j], 0, 0, 0);
      }
    }
    // half-wave exchange: then acc[j][8c + e] is column 16c + 8h + e of block j
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      f32x16_t& G = acc[j];
#pragma unroll
      for (int a = 0; a < 16; a += 8)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(G[a + u]), __float_as_uint(G[a + 4 + u]),
                                                           false, false);
          G[a + u] = __uint_as_float(r[0]);
          G[a + 4 + u] = __uint_as_float(r[1]);
        }
      if (t < T) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint32_t ow[4] = {o[j][c].x, o[j][c].y, o[j][c].z, o[j][c].w};
          uint32_t nw[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            nw[u] = pack_bf16x2(lo_bf16(ow[u]) + G[8 * c + 2 * u], hi_bf16(ow[u]) + G[8 * c + 2 * u + 1]);
          *(uint4*)(dx + (int64_t)t * d + n0 + wn * (BN / 2) + 32 * j + 16 * c + 8 * h) =
              make_uint4(nw[0], nw[1], nw[2], nw[3]);
        }
      }
    }
  }
  vm_wait<0>();  // a block with no token tile still waits for its DMA before it ends
}

// dWg[d, E] = x^T . d_logits over one slice of the token axis: 128 rows of d x all E columns per
// block, 64 tokens per step, 2 stages.  x's token rows (128 columns each, M-contiguous) arrive by
// DMA as a KN tile; d_logits rows are rounded to bf16 through registers, one step ahead, into a
// KN tile.  Tokens past the slice (or T) get zero d_logits.  fp32 partials per slice, or dWg in
// bf16 directly when there is one slice.
template <int EP>
__global__ __launch_bounds__(256, 1) void router_dwg_fast_kernel(const uint16_t* __restrict__ x,
                                                                const float* __restrict__ dl, int T, int d, int kslice,
                                                                float* __restrict__ partial,
                                                                uint16_t* __restrict__ dWg) {
  constexpr int BM = 128, BK = 64, S = 2;
  constexpr int A_BYTES = BK * BM * 2, B_BYTES = BK * EP * 2, STAGE = A_BYTES + B_BYTES;
  constexpr int QA = A_BYTES / 4096;
  constexpr int FM = 2, FN = EP / 64;
  constexpr int BV = BK * EP / 256 / 4;  // float4 loads of d_logits per thread per step
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr_of(smem));
  const int nblk = d / BM;
  const int i0 = (blockIdx.x % nblk) * BM, slice = blockIdx.x / nblk;
  const int kbeg = slice * kslice, kend = min(T, kbeg + kslice);
  const int nk = (kend - kbeg + BK - 1) / BK;
  // x: instruction gi covers token rows 4 gi .. 4 gi + 3 (256-byte rows of 16 chunks)
  auto issue_a = [&](int t, int st) __attribute__((always_inline)) {
    const uint32_t abase = lds0 + st * STAGE;
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int gi = wave * QA + q, kr = 4 * gi + lane / 16;
      const int c = (lane % 16) ^ (4 * (kr & 3));
      const int tok = min(kbeg + t * BK + kr, T - 1);  // past the slice: zero d_logits rows
      dma16(x + (int64_t)tok * d + i0 + 8 * c, abase + gi * 1024);
    }
  };
  // d_logits: float4 u of thread tid is element 4 (256 u + tid) of the 64 x E tile, row-major
  auto load_b = [&](int t, float4 (&v)[BV]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < BV; ++u) {
      const int e4 = u * 256 + tid;  // float4 index within the 64 x EP tile
      const int kr = e4 / (EP / 4), col = 4 * (e4 % (EP / 4));
      const int tok = kbeg + t * BK + kr;
      v[u] = tok < kend ? *(const float4*)(dl + (int64_t)tok * EP + col) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_b = [&](int st, const float4 (&v)[BV]) __attribute__((always_inline)) {
    const uint32_t bbase = lds0 + st * STAGE + A_BYTES;
#pragma unroll
    for (int u = 0; u < BV; ++u) {
      const int e4 = u * 256 + tid;
      const int kr = e4 / (EP / 4), col = 4 * (e4 % (EP / 4));
      *(LDS_AS u32x2*)(uintptr_t)(bbase + kn_off<EP>(kr, col)) =
          u32x2{pack_bf16x2(v[u].x, v[u].y), pack_bf16x2(v[u].z, v[u].w)};
    }
  };
  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  float4 bvv[BV];
  if (nk > 0) {
    issue_a(0, 0);
    load_b(0, bvv);
  }
  for (int it = 0; it < nk; ++it) {
    const int st = it % S;
    store_b(st, bvv);
    vm_wait_barrier<0>();
    lds_barrier();
    if (it + 1 < nk) {  // the next step's operands are in flight during this step's MFMAs
      issue_a(it + 1, (it + 1) % S);
      load_b(it + 1, bvv);
    }
    const uint32_t abase = lds0 + st * STAGE, bbase = abase + A_BYTES;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[FM], bv[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = read_kn<BM>(abase, wm * 64 + 32 * i, kk, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) bv[j] = read_kn<EP>(bbase, wn * (EP / 2) + 32 * j, kk, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[j], af[i], acc[i][j], 0, 0, 0);
    }
    lds_barrier();  // every wave is done with this stage before the next refill
  }
  // lane l holds row i0 + wm 64 + 32 i + l % 32 of dWg and, per block j, columns 8 (r / 4) +
  // 4 (l / 32) + r % 4
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = i0 + wm * 64 + 32 * i + (lane & 31);
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = wn * (EP / 2) + 32 * j + 8 * q + 4 * (lane >> 5);
        if (partial) {
          *(float4*)(partial + ((int64_t)slice * d + row) * EP + col) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        } else {
          *(u32x2*)(dWg + (int64_t)row * EP + col) =
              u32x2{pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]), pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
        }
      }
  }
}

// dWg = bf16(sum over slices, in slice order, of the fp32 partials).
__global__ __launch_bounds__(256) void router_dwg_reduce_kernel(const float* __restrict__ partial, int64_t n,
                                                                int slices, uint16_t* __restrict__ dWg) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float a = 0.0f;
  for (int s = 0; s < slices; ++s) a += partial[(int64_t)s * n + i];
  dWg[i] = f32_to_bf16(a);
}

namespace {
bool aligned16(const void* p, int64_t ld, int esize) { return ((uintptr_t)p & 15u) == 0 && (ld * esize) % 16 == 0; }

template <int MODE, bool A_KM, bool A_F32, bool B_NK, bool B_F32>
hipError_t run_router(RouterArgs g, int slices, hipStream_t st) {
  g.mt = (g.M + kRBM - 1) / kRBM;
  g.nt = (g.N + kRBN - 1) / kRBN;
  g.ntotal = (int64_t)g.mt * g.nt * slices;
  if (g.ntotal == 0) return hipSuccess;
  const int64_t blocks = g.ntotal < (1 << 20) ? g.ntotal : (1 << 20);
  router_gemm_kernel<MODE, A_KM, A_F32, B_NK, B_F32><<<(unsigned)blocks, 256, 0, st>>>(g);
  return hipGetLastError();
}
}  // namespace

// Slices of the token axis for dWg: enough blocks to fill the chip, at least 256 tokens each.
void router_dwg_split(int64_t T, int d, int E, int* slices, int* kslice) {
  const int64_t tiles = (int64_t)((d + kRBM - 1) / kRBM) * ((E + kRBN - 1) / kRBN);
  int64_t s = (1024 + tiles - 1) / tiles;
  s = s < 1 ? 1 : (s > 64 ? 64 : s);
  const int64_t by_rows = (T + 255) / 256;
  if (s > by_rows) s = by_rows;
  if (s < 1) s = 1;
  int64_t ks = (T + s - 1) / s;
  ks = (ks + kRBK - 1) / kRBK * kRBK;
  if (ks < kRBK) ks = kRBK;
  *kslice = (int)ks;
  *slices = (int)((T + ks - 1) / ks);
  if (*slices < 1) *slices = 1;
}

size_t router_ws_bytes(int64_t T, int d, int E) {
  int s, ks;
  router_dwg_split(T, d, E, &s, &ks);
  return s > 1 ? (size_t)s * d * E * sizeof(float) : 0;
}

// The E = 128 / 256 kernels' shape rules (d is a multiple of 128 for every layer; 16-byte
// alignment of x, Wg, d_logits and dx is checked at the boundary).
static bool router_fast(int E) { return E == 128 || E == 256; }

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* Wg, int T, int d, int E, float* logits,
                                hipStream_t st) {
  if (router_fast(E) && T > 0) {
    const unsigned grid = (unsigned)((T + 63) / 64);
    if (E == 128) router_logits_fast_kernel<128><<<grid, 256, 0, st>>>(x, Wg, T, d, logits);
    else router_logits_fast_kernel<256><<<grid, 256, 0, st>>>(x, Wg, T, d, logits);
    return hipGetLastError();
  }
  RouterArgs g{};
  g.A = x;
  g.lda = d;
  g.B = Wg;
  g.ldb = E;
  g.M = T;
  g.N = E;
  g.K = d;
  g.kslice = d;
  g.vecA = aligned16(x, d, 2);
  g.vecB = aligned16(Wg, E, 2);
  g.C = logits;
  g.ldc = E;
  return run_router<R_LOGITS, false, false, false, false>(g, 1, st);
}

hipError_t launch_router_dx(const float* d_logits, const uint16_t* Wg, int T, int d, int E, uint16_t* dx,
                            hipStream_t st) {
  const int bn = 128;
  if (router_fast(E) && T > 0 && d % bn == 0) {
    // two blocks per compute unit (E = 128) or one: each column slice of d takes rgroups
    // interleaved groups of token tiles
    const int nblk = d / bn, ntile = (T + 63) / 64;
    const int want = E == 128 ? 512 : 256;
    int rgroups = (want + nblk - 1) / nblk;
    if (rgroups > ntile) rgroups = ntile;
    const unsigned grid = (unsigned)(nblk * rgroups);
    if (E == 128) router_dx_fast_kernel<128><<<grid, 256, 0, st>>>(d_logits, Wg, T, d, rgroups, dx);
    else router_dx_fast_kernel<256><<<grid, 256, 0, st>>>(d_logits, Wg, T, d, rgroups, dx);
    return hipGetLastError();
  }
  RouterArgs g{};
  g.A = d_logits;  // [T, E]: (m = t, k = e)
  g.lda = E;
  g.B = Wg;        // (k = e, n = i) at Wg[i*E + e]
  g.ldb = E;
  g.M = T;
  g.N = d;
  g.K = E;
  g.kslice = E;
  g.vecA = aligned16(d_logits, E, 4);
  g.vecB = aligned16(Wg, E, 2);
  g.C = dx;
  g.ldc = d;
  return run_router<R_DX, false, true, true, false>(g, 1, st);
}

hipError_t launch_router_dwg(const uint16_t* x, const float* d_logits, int T, int d, int E, uint16_t* dWg,
                             float* partial, hipStream_t st) {
  int slices, kslice;
  router_dwg_split(T, d, E, &slices, &kslice);
  if (router_fast(E) && T > 0) {
    float* part = slices > 1 ? partial : nullptr;
    const unsigned grid = (unsigned)((d / 128) * slices);
    if (E == 128) router_dwg_fast_kernel<128><<<grid, 256, 0, st>>>(x, d_logits, T, d, kslice, part, dWg);
    else router_dwg_fast_kernel<256><<<grid, 256, 0, st>>>(x, d_logits, T, d, kslice, part, dWg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || slices == 1) return e;
    const int64_t n = (int64_t)d * E;
    router_dwg_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(partial, n, slices, dWg);
    return hipGetLastError();
  }
  RouterArgs g{};
  g.A = x;         // (m = i, k = t) at x[t*d + i]
  g.lda = d;
  g.B = d_logits;  // (k = t, n = e) at d_logits[t*E + e]
  g.ldb = E;
  g.M = d;
  g.N = E;
  g.K = T;
  g.kslice = kslice;
  g.vecA = aligned16(x, d, 2);
  g.vecB = aligned16(d_logits, E, 4);
  g.C = dWg;
  g.ldc = E;
  g.partial = slices > 1 ? partial : nullptr;
  hipError_t e = run_router<R_DWG, true, false, false, true>(g, slices, st);
  if (e != hipSuccess || slices == 1) return e;
  const int64_t n = (int64_t)d * E;
  router_dwg_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(partial, n, slices, dWg);
  return hipGetLastError();
}

}  // namespace moe
