// Router (top-k + softmax over the kept logits) and the expert plan (histogram -> scan ->
// stable scatter), plus the per-GEMM tile table built from the plan's offsets.
//
// Routing: a learned router activates only each token's top-K experts (page "Az NVIDIA szerint
// tízszer gyorsabb lett a dropless MoE tanítása JAX-ban", section "A dropless MoE minden
// tokent feldolgoz").  Ragged per-expert groups (same page, "Az egyenetlen terhelés lassítja a
// tanítást") are described by counts/offsets and a permutation, the per-expert split sizes of
// the TE MoE page ("NVIDIA מציגה דרך יעילה לאמן מודלי MoE בביולוגיה", section "מומחים מקובצים
// במקום לולאת Python").
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------------------------- router
// One wave per token.  Lane l holds logits e = l, l+64, ...; k rounds of a wave arg-max on
// the key (value descending, expert id ascending) select the slots in order.  Slot j's
// (value, id) stays in lane j; the softmax over the k kept values is then one wave reduction.
template <int EPL>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                          int k, int32_t* __restrict__ ids,
                                                          float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = logits + (size_t)t * E;
  float v[EPL];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      v[i] = row[e];
    } else {
      v[i] = 0.0f;
      taken |= 1u << i;
    }
  }
  float sel_v = 0.0f;
  int sel_e = -1;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (!((taken >> i) & 1u)) {
        const int e = lane + 64 * i;
        if (be == 0x7FFFFFFF || v[i] > bv || (v[i] == bv && e < be)) {
          bv = v[i];
          be = e;
        }
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const int oe = __shfl_xor(be, m, 64);
      // an empty candidate carries id 0x7FFFFFFF and loses to any real one
      const bool take = (oe != 0x7FFFFFFF) && (be == 0x7FFFFFFF || ov > bv || (ov == bv && oe < be));
      if (take) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      sel_v = bv;
      sel_e = be;
    }
  }
  const float vmax = __shfl(sel_v, 0, 64);
  float z = (lane < k) ? expf(sel_v - vmax) : 0.0f;
  float s = z;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if (lane < k) {
    ids[(size_t)t * k + lane] = sel_e;
    w[(size_t)t * k + lane] = z / s;
  }
}

// G lanes per token (64/G tokens per wave), for k <= G.  Lane g holds logits g*EPL .. g*EPL+EPL-1
// (one contiguous load).  Each of the k rounds takes the lane's best remaining (value, id), then
// a butterfly over the G lanes on the same key (value descending, id ascending); every lane of
// the group ends with the winner, lane j keeps slot j.  exp(v_j - v_0) is formed per round and
// summed in slot order.
template <int G, int EPL>
__global__ __launch_bounds__(256) void router_topk_group_kernel(const float* __restrict__ logits, int T, int E,
                                                                int k, int32_t* __restrict__ ids,
                                                                float* __restrict__ w) {
  const int gl = threadIdx.x % G;
  const int t = (blockIdx.x * 256 + threadIdx.x) / G;
  if (t >= T) return;  // uniform per group; a butterfly never leaves its group
  const float* row = logits + (size_t)t * E;
  float v[EPL];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = gl * EPL + i;
    v[i] = e < E ? row[e] : 0.0f;
    if (e < E) avail |= 1u << i;
  }
  float vmax = 0.0f, ssum = 0.0f, myz = 0.0f;
  int mye = -1;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      // ids rise with i, so a tie keeps the earlier (lower) id
      if (((avail >> i) & 1u) && (be == 0x7FFFFFFF || v[i] > bv)) {
        bv = v[i];
        be = gl * EPL + i;
      }
    }
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const int oe = __shfl_xor(be, m, 64);
      // an empty candidate carries id 0x7FFFFFFF and loses to any real one
      const bool take = (oe != 0x7FFFFFFF) && (be == 0x7FFFFFFF || ov > bv || (ov == bv && oe < be));
      if (take) {
        bv = ov;
        be = oe;
      }
    }
    if (be / EPL == gl) avail &= ~(1u << (be % EPL));
    if (j == 0) vmax = bv;
    const float z = expf(bv - vmax);
    ssum += z;
    if (gl == j) {
      myz = z;
      mye = be;
    }
  }
  if (gl < k) {
    ids[(size_t)t * k + gl] = mye;
    w[(size_t)t * k + gl] = myz / ssum;
  }
}

hipError_t launch_router(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t st) {
  if (T == 0) return hipSuccess;
  // group kernel: G lanes per token with EPL = 8 logits each, when k fits in the group
  const unsigned gg16 = (unsigned)(((int64_t)T * 16 + 255) / 256);
  if (E <= 64 && k <= 8) {
    router_topk_group_kernel<8, 8><<<(unsigned)(((int64_t)T * 8 + 255) / 256), 256, 0, st>>>(logits, T, E, k, ids, w);
    return hipGetLastError();
  }
  if (E <= 128 && k <= 16) {
    router_topk_group_kernel<16, 8><<<gg16, 256, 0, st>>>(logits, T, E, k, ids, w);
    return hipGetLastError();
  }
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    router_topk_kernel<1><<<grid, block, 0, st>>>(logits, T, E, k, ids, w);
  else if (E <= 128)
    router_topk_kernel<2><<<grid, block, 0, st>>>(logits, T, E, k, ids, w);
  else if (E <= 256)
    router_topk_kernel<4><<<grid, block, 0, st>>>(logits, T, E, k, ids, w);
  else if (E <= 512)
    router_topk_kernel<8><<<grid, block, 0, st>>>(logits, T, E, k, ids, w);
  else
    router_topk_kernel<16><<<grid, block, 0, st>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------ plan
// Pairs are cut into S contiguous segments of `seg` pairs, one wave per segment.
//   hist:    segcnt[e*S + s] = pairs of segment s routed to expert e
//   scan:    segbase = exclusive scan of segcnt in (expert, segment) order; counts, offsets
//   scatter: each wave walks its segment in 64-pair steps in ascending pair order; a pair's
//            position is segbase[e*S+s] + (pairs of e earlier in the segment).  Lanes with the
//            same expert are found with one ballot per id bit, so the rank within a step is a
//            popcount.  No atomics decide positions, so the result is the unique stable order.

void plan_geometry(int64_t A, int* seg, int* S) {
  int64_t sg = 1024;
  int64_t need = (A + 511) / 512;
  if (need > sg) sg = (need + 63) / 64 * 64;
  *seg = (int)sg;
  *S = (int)((A + sg - 1) / sg);
}

__global__ __launch_bounds__(256) void plan_hist_kernel(const int32_t* __restrict__ ids, int A, int E,
                                                        int seg, int S, int32_t* __restrict__ segcnt) {
  extern __shared__ int sh_cnt[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int s = blockIdx.x * 4 + wv;
  int* cnt = sh_cnt + wv * E;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  __syncthreads();
  if (s < S) {
    const int lo = s * seg, hi = min(A, lo + seg);
    for (int p = lo + lane; p < hi; p += 64) {
      const int e = ids[p];
      if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  if (s < S)
    for (int e = lane; e < E; e += 64) segcnt[(size_t)e * S + s] = cnt[e];
}

// One block.  Thread t owns the contiguous (expert, segment) entries [t*per, (t+1)*per).  When the
// table fits, it is moved through LDS with coalesced loads and stores (one CU issuing a scattered
// 4-byte access per entry is limited by its request rate, not by latency); the LDS copy is padded
// by one word per 16 so the threads' strided chunk walks hit distinct banks.
constexpr int kScanLdsCap = 24576;
__device__ __forceinline__ int scan_pad(int i) { return i + (i >> 4); }

__global__ __launch_bounds__(1024) void plan_scan_kernel(const int32_t* __restrict__ segcnt, int E, int S,
                                                         int32_t* __restrict__ segbase,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets) {
  __shared__ int sh[64];
  __shared__ int first[1025];
  __shared__ int buf[kScanLdsCap + kScanLdsCap / 16];
  const int n = E * S;
  const int per = (n + 1023) / 1024;
  const int lo = threadIdx.x * per, hi = min(n, lo + per);
  const bool in_lds = n <= kScanLdsCap;
  if (in_lds) {
    for (int i = threadIdx.x; i < n; i += 1024) buf[scan_pad(i)] = segcnt[i];
    __syncthreads();
  }
  // out of LDS: the thread's entries are read in groups of 8 independent loads
  constexpr int G = 8;
  int sum = 0;
  for (int i0 = lo; i0 < hi; i0 += G) {
    int v[G];
#pragma unroll
    for (int u = 0; u < G; ++u) v[u] = i0 + u < hi ? (in_lds ? buf[scan_pad(i0 + u)] : segcnt[i0 + u]) : 0;
#pragma unroll
    for (int u = 0; u < G; ++u) sum += v[u];
  }
  int run;
  const int total = block_excl_scan_1024(sum, sh, &run);
  // (expert, segment) of entry lo, then stepped along without a division per entry
  int ce = S > 0 ? lo / S : 0, cs = S > 0 ? lo - ce * S : 0;
  for (int i0 = lo; i0 < hi; i0 += G) {
    int v[G];
#pragma unroll
    for (int u = 0; u < G; ++u) v[u] = i0 + u < hi ? (in_lds ? buf[scan_pad(i0 + u)] : segcnt[i0 + u]) : 0;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int i = i0 + u;
      if (i < hi) {
        if (cs == 0) first[ce] = run;
        if (in_lds) buf[scan_pad(i)] = run;  // the thread's own entry: read above, no other reader
        else segbase[i] = run;
        run += v[u];
        if (++cs == S) {
          cs = 0;
          ++ce;
        }
      }
    }
  }
  if (S == 0)
    for (int e = threadIdx.x; e < E; e += 1024) first[e] = 0;
  if (threadIdx.x == 0) first[E] = total;
  __syncthreads();
  if (in_lds)
    for (int i = threadIdx.x; i < n; i += 1024) segbase[i] = buf[scan_pad(i)];
  for (int e = threadIdx.x; e < E; e += 1024) {
    offsets[e] = first[e];
    counts[e] = first[e + 1] - first[e];
  }
  if (threadIdx.x == 0) offsets[E] = total;
}

__global__ __launch_bounds__(256) void plan_scatter_kernel(const int32_t* __restrict__ ids, int A, int E,
                                                           int seg, int S, const int32_t* __restrict__ segbase,
                                                           int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ inv_perm) {
  extern __shared__ int sh_run[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int s = blockIdx.x * 4 + wv;
  int* run = sh_run + wv * E;
  if (s < S)
    for (int e = lane; e < E; e += 64) run[e] = segbase[(size_t)e * S + s];
  __syncthreads();
  if (s >= S) return;
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const int lo = s * seg, hi = min(A, lo + seg);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = lo; base < hi; base += 64) {
    const int p = base + lane;
    const bool in = p < hi;
    const int e = in ? ids[p] : -1;
    const bool valid = in && e >= 0 && e < E;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    int rank = 0, pos = 0;
    if (valid) {
      rank = __popcll(m & below);
      pos = run[e] + rank;
      perm[pos] = p;
      inv_perm[p] = pos;
    } else if (in) {
      inv_perm[p] = -1;
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && rank == 0) run[e] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
}

size_t plan_ws_bytes(int64_t A, int64_t E) {
  int seg, S;
  plan_geometry(A, &seg, &S);
  return 2 * (size_t)E * (size_t)S * sizeof(int32_t);
}

hipError_t launch_plan(const int32_t* ids, int64_t A, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv_perm, void* ws, hipStream_t st) {
  int seg, S;
  plan_geometry(A, &seg, &S);
  int32_t* segcnt = (int32_t*)ws;
  int32_t* segbase = segcnt + (size_t)E * S;
  const size_t lds = 4 * (size_t)E * sizeof(int);
  if (S > 0) plan_hist_kernel<<<(S + 3) / 4, 256, lds, st>>>(ids, (int)A, E, seg, S, segcnt);
  plan_scan_kernel<<<1, 1024, 0, st>>>(segcnt, E, S, segbase, counts, offsets);
  if (S > 0) plan_scatter_kernel<<<(S + 3) / 4, 256, lds, st>>>(ids, (int)A, E, seg, S, segbase, perm, inv_perm);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ tile table
// For a grouped GEMM with BM-row tiles over ragged experts: tiles[t] = (expert, m-tile) for
// t < ntiles, experts in order, empty experts contributing no tile.
__global__ __launch_bounds__(1024) void tile_map_kernel(const int32_t* __restrict__ offsets, int E, int BM,
                                                        int2* __restrict__ tiles, int32_t* __restrict__ ntiles) {
  __shared__ int sh[64];
  __shared__ int start[1025];
  const int e = threadIdx.x;
  const int c = (e < E) ? offsets[e + 1] - offsets[e] : 0;
  const int nt = (c + BM - 1) / BM;
  int ex;
  const int total = block_excl_scan_1024(nt, sh, &ex);
  if (e < E) start[e] = ex;
  __syncthreads();
  for (int t = threadIdx.x; t < total; t += 1024) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (start[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    tiles[t] = make_int2(lo, t - start[lo]);
  }
  if (threadIdx.x == 0) *ntiles = total;
}

hipError_t launch_tile_map(const int32_t* offsets, int E, int BM, int2* tiles, int32_t* ntiles, hipStream_t st) {
  tile_map_kernel<<<1, 1024, 0, st>>>(offsets, E, BM, tiles, ntiles);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ token rows
// tokrow[pos] = perm[pos] / k for routed positions; every other entry (unrouted tail and the
// padding the weight-gradient GEMMs may read past an expert's last row) is 0, a valid row.
__global__ __launch_bounds__(256) void tokrow_kernel(const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ total, int64_t n, int k,
                                                     int32_t* __restrict__ tokrow) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  tokrow[i] = (i < *total) ? perm[i] / k : 0;
}

hipError_t launch_tokrow(const int32_t* perm, const int32_t* offsets, int E, int64_t A, int k, int32_t* tokrow,
                         hipStream_t st) {
  const int64_t n = A + kTokrowPad;
  tokrow_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(perm, offsets + E, n, k, tokrow);
  return hipGetLastError();
}

}  // namespace moe
