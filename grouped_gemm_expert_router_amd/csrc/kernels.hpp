// Host-side launchers of the MoE kernels (stream-ordered, no host synchronisation).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// routing and plan
hipError_t launch_router(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t st);
void plan_geometry(int64_t A, int* seg, int* S);
size_t plan_ws_bytes(int64_t A, int64_t E);
hipError_t launch_plan(const int32_t* ids, int64_t A, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv_perm, void* ws, hipStream_t st);
hipError_t launch_tile_map(const int32_t* offsets, int E, int BM, int2* tiles, int32_t* ntiles, hipStream_t st);

// grouped GEMMs (bf16 operands, fp32 accumulation)
struct MoeShape {
  int T, d, f, E, k;
};

// Row-tile height of the ragged-M grouped GEMMs (the tile table is built for it).
constexpr int kGemmBM = 256;
// Column-tile width of the activation-gradient GEMM for expert FFN dim f; f / dact_bn(f)
// partial sums of d_topk_w are written per routed pair.
int dact_bn(int f);
int dact_parts_bf16(int f);

int max_row_tiles(int64_t A, int E, int BM);

// GEMM1: H = x[perm/k] . W1[e] (gate|up), As = w * silu(gate) * up.
hipError_t launch_gemm_up(const MoeShape& s, const uint16_t* x, const uint16_t* W1, const float* topk_w,
                          const int32_t* offsets, const int32_t* perm, const int2* tiles, const int32_t* ntiles,
                          uint16_t* H, uint16_t* As, hipStream_t st);
// GEMM2: Op[perm[pos]] = As[pos] . W2[e]  (per-pair output in slot order).
hipError_t launch_gemm_down(const MoeShape& s, const uint16_t* As, const uint16_t* W2, const int32_t* offsets,
                            const int32_t* perm, const int2* tiles, const int32_t* ntiles, uint16_t* Op,
                            hipStream_t st);
// Single-launch forward: the work queue of row tiles (items: up to max_row_tiles(A, E, 256)
// entries; qinfo: 40 words), then GEMM1 and GEMM2 of every row tile in one persistent launch.
hipError_t launch_fwd_queue(const MoeShape& s, const int32_t* offsets, int2* items, int32_t* qinfo, hipStream_t st);
hipError_t launch_fused_forward(const MoeShape& s, const uint16_t* x, const uint16_t* W1, const uint16_t* W2,
                                const float* topk_w, const int32_t* offsets, const int32_t* perm, const int2* items,
                                int32_t* qinfo, uint16_t* H, uint16_t* As, uint16_t* Op, hipStream_t st);
// dA: G = dy[perm/k] . W2[e]^T; epilogue -> dH (dSwiGLU) and d_topk_w partials.
hipError_t launch_gemm_dact(const MoeShape& s, const uint16_t* dy, const uint16_t* W2, const uint16_t* H,
                            const float* topk_w, const int32_t* offsets, const int32_t* perm, const int2* tiles,
                            const int32_t* ntiles, uint16_t* dH, float* dwp, hipStream_t st);
// dX: dXp[perm[pos]] = dH[pos] . W1[e]^T.
hipError_t launch_gemm_dx(const MoeShape& s, const uint16_t* dH, const uint16_t* W1, const int32_t* offsets,
                          const int32_t* perm, const int2* tiles, const int32_t* ntiles, uint16_t* dXp,
                          hipStream_t st);
// Weight gradients (ragged K = the expert's rows):
//   dW2[e] = As_e^T . dy[perm/k]_e     dW1[e] = x[perm/k]_e^T . dH_e
//   tokrow[pos] = perm[pos] / k for pos < offsets[E], padded by kTokrowPad readable entries.
// Experts with more than KC rows (KC >= kWgChunk, chosen on the device) are split into chunks
// whose fp32 partials (at most max_partials slots) are summed in chunk order by launch_wg_reduce.
constexpr int kWgChunk = 2048;
constexpr int kWgMaxPartials = 32;
constexpr int64_t kWgPartialBudget = (int64_t)512 << 20;
struct WgSplit {
  int2* units;       // [E + max_partials]
  int32_t* meta;     // [3]: unit count, chunk rows KC, 1 = bucketed XCD tile order
  int32_t* pslot;    // [E]
  float* partial;    // [max_partials, max(d*2f, f*d)]
  const int32_t* offsets;
  int max_partials;
};
int wg_max_partials(const MoeShape& s);
hipError_t launch_wg_split(const MoeShape& s, const int32_t* offsets, const WgSplit& sp, hipStream_t st);
hipError_t launch_wg_reduce(const MoeShape& s, const WgSplit& sp, int64_t per_e, uint16_t* dW, hipStream_t st);
hipError_t launch_gemm_dw2(const MoeShape& s, const uint16_t* As, const uint16_t* dy, const int32_t* offsets,
                           const int32_t* perm, const int32_t* tokrow, const WgSplit& sp, uint16_t* dW2,
                           hipStream_t st);
hipError_t launch_gemm_dw1(const MoeShape& s, const uint16_t* x, const uint16_t* dH, const int32_t* offsets,
                           const int32_t* perm, const int32_t* tokrow, const WgSplit& sp, uint16_t* dW1,
                           hipStream_t st);
constexpr int kTokrowPad = 64;
hipError_t launch_tokrow(const int32_t* perm, const int32_t* offsets, int E, int64_t A, int k, int32_t* tokrow,
                         hipStream_t st);

// fp8 (OCP e4m3) grouped GEMMs with fp32 block scales: activations [rows, K/128] (one scale per
// row per 128 values), weights [E, rows/128, cols/128] of each matrix as stored.  Row tiles are
// kFp8BM high; d and f must be multiples of 256.
constexpr int kFp8BM = 256;
// H = x[perm/k] . W1[e]; As = w * silu(gate) * up in bf16 and as e4m3 + scales [A, f/128].
hipError_t launch_fp8_up(const MoeShape& s, const uint8_t* x, const float* xs, const uint8_t* W1, const float* W1s,
                         const float* topk_w, const int32_t* offsets, const int32_t* perm, const int2* tiles,
                         const int32_t* ntiles, uint16_t* H, uint16_t* As, uint8_t* Asq, float* Ass, hipStream_t st);
// Op[perm[pos]] = As[pos] . W2[e] from the e4m3 As.
hipError_t launch_fp8_down(const MoeShape& s, const uint8_t* Asq, const float* Ass, const uint8_t* W2,
                           const float* W2s, const int32_t* offsets, const int32_t* perm, const int2* tiles,
                           const int32_t* ntiles, uint16_t* Op, hipStream_t st);
// G = dy_q[perm/k] . W2[e]^T; dH in bf16 and e4m3 + scales [A, 2f/128]; f/256 d_topk_w partials.
hipError_t launch_fp8_dact(const MoeShape& s, const uint8_t* dyq, const float* dys, const uint8_t* W2,
                           const float* W2s, const uint16_t* H, const float* topk_w, const int32_t* offsets,
                           const int32_t* perm, const int2* tiles, const int32_t* ntiles, uint16_t* dH, uint8_t* dHq,
                           float* dHs, float* dwp, hipStream_t st);
// dXp[perm[pos]] = dH_q[pos] . W1[e]^T.
hipError_t launch_fp8_dx(const MoeShape& s, const uint8_t* dHq, const float* dHs, const uint8_t* W1, const float* W1s,
                         const int32_t* offsets, const int32_t* perm, const int2* tiles, const int32_t* ntiles,
                         uint16_t* dXp, hipStream_t st);
// bf16 rows -> e4m3 + one scale per row per 128 values (cols % 128 == 0), and back to bf16.
hipError_t launch_quant_rows(const uint16_t* src, int64_t rows, int cols, uint8_t* q, float* qs, hipStream_t st);
hipError_t launch_dequant_rows(const uint8_t* q, const float* qs, int64_t rows, int cols, uint16_t* out,
                               hipStream_t st);
// MXFP8: e4m3 codes with one E8M0 exponent byte per 32 values along each GEMM's K.
// along_rows = 0: blocks of 32 consecutive values of a row -> exponents [batch, rows, cols/32];
// along_rows = 1: blocks of 32 consecutive rows of a column -> exponents [batch, rows/32, cols].
hipError_t launch_mx_quant(const uint16_t* src, int64_t batch, int rows, int cols, int along_rows, uint8_t* q,
                           uint8_t* qe, hipStream_t st);
// Both orientations of [batch, rows, cols] in one pass (rows % 32 == 0, cols % 256 == 0):
// column blocks into qc/qce, row blocks into qr with their exponents as 32-bit words by k step
// in qre ([batch, cols/128, rows] words: word (t, r) = the exponents of blocks 4t..4t+3 of row r).
// MXFP8 weight gradients: each expert's rows padded to a multiple of 128 (see gemm_mx.hip).
inline int64_t mx_padded_rows(int64_t A, int E) { return (A + 127 * (int64_t)E + 127) / 128 * 128; }
hipError_t launch_mx_pad_offsets(const int32_t* offsets, int E, int32_t* poff, hipStream_t st);
// bf16 rows (token rows perm[pos] / k when gather is set, else sorted rows pos) -> e4m3 codes in
// blocks of 32 consecutive sorted rows of one expert, with E8M0 exponents
hipError_t launch_mx_quant_tokens(const uint16_t* src, int C, int gather, const MoeShape& s, const int32_t* offsets,
                                  const int32_t* perm, const int32_t* poff, uint8_t* q, uint8_t* qe, hipStream_t st);
hipError_t launch_mx_wg(int which, const MoeShape& s, const uint8_t* Aq, const uint8_t* Ae, int Mo, const uint8_t* Bq,
                        const uint8_t* Be, int N, const int32_t* poff, const WgSplit& sp, uint16_t* dW,
                        hipStream_t st);
hipError_t launch_mx_quant_dual(const uint16_t* src, int64_t batch, int rows, int cols, uint8_t* qc, uint8_t* qce,
                                uint8_t* qr, uint8_t* qre, hipStream_t st);
// The MX GEMMs take every row-blocked operand's exponents as words by k step: x and dy sorted
// by launch_kstep_sort, As and dH as the epilogues write them, W1/W2 as launch_mx_quant_dual's
// row-block output.
hipError_t launch_mx_up(const MoeShape& s, const uint8_t* xq, const uint8_t* xe, const uint8_t* W1q,
                        const uint8_t* W1e, const float* topk_w, const int32_t* offsets, const int32_t* perm,
                        const int2* tiles, const int32_t* ntiles, uint16_t* H, uint16_t* As, uint8_t* Asq,
                        uint8_t* Ase, hipStream_t st);
hipError_t launch_mx_down(const MoeShape& s, const uint8_t* Asq, const uint8_t* Ase, const uint8_t* W2q,
                          const uint8_t* W2e, const int32_t* offsets, const int32_t* perm, const int2* tiles,
                          const int32_t* ntiles, uint16_t* Op, hipStream_t st);
hipError_t launch_mx_dact(const MoeShape& s, const uint8_t* dyq, const uint8_t* dye, const uint8_t* W2q,
                          const uint8_t* W2e, const uint16_t* H, const float* topk_w, const int32_t* offsets,
                          const int32_t* perm, const int2* tiles, const int32_t* ntiles, uint16_t* dH, uint8_t* dHq,
                          uint8_t* dHe, float* dwp, hipStream_t st);
hipError_t launch_mx_dx(const MoeShape& s, const uint8_t* dHq, const uint8_t* dHe, const uint8_t* W1q,
                        const uint8_t* W1e, const int32_t* offsets, const int32_t* perm, const int2* tiles,
                        const int32_t* ntiles, uint16_t* dXp, hipStream_t st);

// router front end (dense gate products, bf16 MFMA): logits = x Wg; dx += d_logits Wg^T;
// dWg = x^T d_logits with the token axis cut into slices whose fp32 partials (router_ws_bytes) are
// summed in slice order
void router_dwg_split(int64_t T, int d, int E, int* slices, int* kslice);
size_t router_ws_bytes(int64_t T, int d, int E);
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* Wg, int T, int d, int E, float* logits,
                                hipStream_t st);
hipError_t launch_router_dx(const float* d_logits, const uint16_t* Wg, int T, int d, int E, uint16_t* dx,
                            hipStream_t st);
hipError_t launch_router_dwg(const uint16_t* x, const float* d_logits, int T, int d, int E, uint16_t* dWg,
                             float* partial, hipStream_t st);

// data movement and router backward
// Per-row words of token rows ([T, nk] 32-bit words, one per 128-wide k step) into the sorted
// order by k step: out word (t, pos) at out + t * rows_cap + pos, from token perm[pos] / kslots,
// for pos < offsets[E].
hipError_t launch_kstep_sort(const void* src, int nk, const int32_t* perm, int kslots, const int32_t* offsets, int E,
                             int64_t rows_cap, void* out, hipStream_t st);
hipError_t launch_permute(const uint16_t* x, const int32_t* inv_perm, int T, int d, int k, uint16_t* xp,
                          hipStream_t st);
hipError_t launch_combine(const uint16_t* op, const int32_t* inv_perm, int T, int d, int k, uint16_t* y,
                          hipStream_t st);
hipError_t launch_dlogits(const float* dwp, int nparts, const int32_t* inv_perm, const int32_t* ids,
                          const float* topk_w, int T, int E, int k, float* d_topk_w, float* d_logits, hipStream_t st);

}  // namespace moe
