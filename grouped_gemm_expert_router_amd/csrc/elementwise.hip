// Bandwidth-bound steps: dispatch gather, fixed-order combine, router backward.
//
// Dispatch and combine move tokens to their experts and bring the results back in token order
// (page "Az NVIDIA szerint tízszer gyorsabb lett a dropless MoE tanítása JAX-ban", sections
// "Az egyenetlen terhelés lassítja a tanítást" and "Csoportosított mátrixszorzás és összevont
// adatmozgatás").  The combine adds a token's k per-pair rows in fp32 in ascending slot order
// and rounds once, so it is bitwise reproducible.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// xp[pos] = x[perm[pos] / k] for pos < *total.  One block per row, 16-byte vectors.
// Token-major: block t reads x[t] once and writes it to the sorted position of each of its
// routed slots (inv_perm[t*k+j] >= 0), so x is read once and each copy written once.
__global__ __launch_bounds__(256) void permute_kernel(const uint16_t* __restrict__ x,
                                                      const int32_t* __restrict__ inv_perm, int d, int k,
                                                      uint16_t* __restrict__ xp) {
  const int t = blockIdx.x;
  const int64_t p0 = (int64_t)t * k;
  const uint4* src = (const uint4*)(x + (size_t)t * d);
  for (int c = threadIdx.x; c < d / 8; c += blockDim.x) {
    const uint4 v = src[c];
    for (int j = 0; j < k; ++j) {
      const int pos = inv_perm[p0 + j];
      if (pos >= 0) store_once16((uint4*)(xp + (size_t)pos * d) + c, v);  // non-temporal: 5.0 -> 5.8 TB/s
    }
  }
}

hipError_t launch_permute(const uint16_t* x, const int32_t* inv_perm, int T, int d, int k, uint16_t* xp,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  permute_kernel<<<(unsigned)T, 256, 0, st>>>(x, inv_perm, d, k, xp);
  return hipGetLastError();
}

// Per-row words of token rows, one per 128-wide k step (MXFP8 exponent words, fp8 row scales),
// into the experts' sorted order, k-step-major: out[t * rows_cap + pos] = src[token * nk + t]
// with token = perm[pos] / kslots, for every sorted position pos < offsets[E].  A GEMM tile's
// k step then finds the words of its rows in one contiguous run instead of one line per row.
// One thread per (sorted position, four k steps blockIdx.y): one 16-byte load of the token's
// words when nk % 4 == 0 (rows then stay 16-byte aligned), else up to four word loads.
__global__ __launch_bounds__(256) void kstep_sort_kernel(const uint32_t* __restrict__ src, int nk,
                                                         const int32_t* __restrict__ perm, int kslots,
                                                         const int32_t* __restrict__ offsets, int E,
                                                         int64_t rows_cap, uint32_t* __restrict__ out) {
  const int64_t pos = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (pos >= offsets[E]) return;
  const int t0 = 4 * blockIdx.y;
  const uint32_t* row = src + (int64_t)(perm[pos] / kslots) * nk;
  uint32_t w[4];
  if (nk % 4 == 0) {
    const uint4 v = *(const uint4*)(row + t0);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = t0 + j < nk ? row[t0 + j] : 0u;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (t0 + j < nk) out[(t0 + j) * rows_cap + pos] = w[j];
}

hipError_t launch_kstep_sort(const void* src, int nk, const int32_t* perm, int kslots, const int32_t* offsets, int E,
                             int64_t rows_cap, void* out, hipStream_t st) {
  if (rows_cap == 0 || nk == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows_cap + 255) / 256), (unsigned)((nk + 3) / 4));
  kstep_sort_kernel<<<grid, 256, 0, st>>>((const uint32_t*)src, nk, perm, kslots, offsets, E, rows_cap,
                                          (uint32_t*)out);
  return hipGetLastError();
}

// y[t] = bf16( sum_{j=0..k-1, inv_perm[t*k+j] >= 0} op[t*k+j] ) with an fp32 running sum.
// The slots are taken 4 at a time: their row loads are all issued before the first add, and
// the adds then run in slot order.  The per-pair rows are read once (non-temporal loads).
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ op,
                                                      const int32_t* __restrict__ inv_perm, int d, int k,
                                                      uint16_t* __restrict__ y) {
  const int t = blockIdx.x;
  const int64_t p0 = (int64_t)t * k;
  for (int c = threadIdx.x; c < d / 8; c += blockDim.x) {
    float a[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += 4) {
      uint4 v[4];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u;
        ok[u] = j < k && inv_perm[p0 + j] >= 0;
        v[u] = make_uint4(0u, 0u, 0u, 0u);
        if (ok[u]) {
          v[u] = load_once16((const uint4*)(op + (p0 + j) * d) + c);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (!ok[u]) continue;
        a[0] += lo_bf16(v[u].x);
        a[1] += hi_bf16(v[u].x);
        a[2] += lo_bf16(v[u].y);
        a[3] += hi_bf16(v[u].y);
        a[4] += lo_bf16(v[u].z);
        a[5] += hi_bf16(v[u].z);
        a[6] += lo_bf16(v[u].w);
        a[7] += hi_bf16(v[u].w);
      }
    }
    uint4 o;
    o.x = pack_bf16x2(a[0], a[1]);
    o.y = pack_bf16x2(a[2], a[3]);
    o.z = pack_bf16x2(a[4], a[5]);
    o.w = pack_bf16x2(a[6], a[7]);
    ((uint4*)(y + (int64_t)t * d))[c] = o;
  }
}

hipError_t launch_combine(const uint16_t* op, const int32_t* inv_perm, int T, int d, int k, uint16_t* y,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  combine_kernel<<<T, 256, 0, st>>>(op, inv_perm, d, k, y);
  return hipGetLastError();
}

// Router backward, one wave per token.  d_topk_w[p] = sum over column tiles of the partial
// inner products <dL/dAs, a> (fixed order; partial q of sorted row pos at dwp[q*stride + pos]);
// d_logits[t, ids[t,j]] =
// w_j (d_topk_w_j - sum_i w_i d_topk_w_i), zero for experts outside the token's top-k.
__global__ __launch_bounds__(256) void dlogits_kernel(const float* __restrict__ dwp, int nparts, int64_t stride,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const int32_t* __restrict__ ids,
                                                      const float* __restrict__ topk_w, int T, int E, int k,
                                                      float* __restrict__ d_topk_w, float* __restrict__ d_logits) {
  extern __shared__ float sh_row[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  const bool active = t < T;
  float dw = 0.0f, wj = 0.0f;
  int e = -1;
  if (active && lane < k) {
    const int64_t p = (int64_t)t * k + lane;
    const int pos = inv_perm[p];
    if (pos >= 0) {
      // partials summed in part order; loaded 4 at a time so the loads overlap
      const float* src = dwp + pos;
      for (int q0 = 0; q0 < nparts; q0 += 4) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = q0 + u < nparts ? src[(int64_t)(q0 + u) * stride] : 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (q0 + u < nparts) dw += v[u];
      }
      wj = topk_w[p];
      if (ids) e = ids[p];
    }
    d_topk_w[p] = dw;
  }
  if (d_logits == nullptr) return;  // uniform across the block
  float inner = wj * dw;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) inner += __shfl_xor(inner, m, 64);
  float* row = sh_row + wv * E;
  if (active)
    for (int c = lane; c < E; c += 64) row[c] = 0.0f;
  __syncthreads();
  if (active && lane < k && e >= 0 && e < E) row[e] = wj * (dw - inner);
  __syncthreads();
  if (active)
    for (int c = lane; c < E; c += 64) d_logits[(int64_t)t * E + c] = row[c];
}

hipError_t launch_dlogits(const float* dwp, int nparts, const int32_t* inv_perm, const int32_t* ids,
                          const float* topk_w, int T, int E, int k, float* d_topk_w, float* d_logits, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const size_t lds = d_logits ? 4 * (size_t)E * sizeof(float) : 0;
  const int64_t stride = (int64_t)T * k;  // partials are part-major over the T*k sorted positions
  dlogits_kernel<<<(T + 3) / 4, 256, lds, st>>>(dwp, nparts, stride, inv_perm, ids, topk_w, T, E, k, d_topk_w,
                                                 d_logits);
  return hipGetLastError();
}

}  // namespace moe
