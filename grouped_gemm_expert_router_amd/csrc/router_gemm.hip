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

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* Wg, int T, int d, int E, float* logits,
                                hipStream_t st) {
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
