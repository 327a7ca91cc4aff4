// Device building blocks shared by the bf16 and fp8 grouped GEMMs (gfx950): LDS DMA with
// explicit wait counts, XCD-aware block numbering, swizzled LDS operand layouts and the MFMA
// operand reads (ds_read_b128 for K-contiguous tiles, LDS transpose reads for N-contiguous ones).
#pragma once
#include "common.hpp"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// Logical tile lid of a grid of nrows row tiles x nN column tiles -> (row tile, column tile),
// in groups of GM row tiles: consecutive lids walk the rows of a group first and then move to
// the next column tile, so the tiles an XCD runs together share GM row panels and a few column
// panels in its L2 instead of streaming every column panel once per row tile.
__device__ __forceinline__ int2 grouped_tile(int lid, int nrows, int nN, int GM) {
  const int grp = lid / (GM * nN);
  const int r0 = grp * GM;
  const int gsz = min(GM, nrows - r0);
  const int idx = lid - grp * GM * nN;
  return make_int2(r0 + idx % gsz, idx / gsz);
}

// ---------------------------------------------------------------- LDS DMA and barriers
// global_load_lds_dwordx4 copies each lane's 16 bytes to LDS at m0 + 16*lane.  It is issued
// through inline asm so the compiler's wait-count pass does not make every LDS read wait for
// all DMA in flight; the kernel waits explicitly (vm_wait_barrier) before the barrier that
// publishes a stage.  One wait state separates the m0 write from the DMA.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_byte_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_byte_addr)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
}

// Same, also waiting for this wave's LDS reads (and scalar loads) before the barrier, so a
// stage another wave refills right after it can have no read of this wave still pending.
template <int N>
__device__ __forceinline__ void vm_lgkm_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory"); }

// This wave's vector-memory instructions (loads, LDS DMA and stores, retired in issue order)
// down to at most N outstanding; no barrier.
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// This wave's LDS operations (and scalar loads) complete; no barrier.
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const LDS_AS void*)p;
}

// Operand tiles in LDS (16-byte chunks, XOR-swizzled so the 16 lanes an LDS cycle serves hit
// 16 distinct 16-byte bank groups of the 64-bank LDS):
//   KM: [row][BK] for K-contiguous sources.  BK = 32: row = 64 bytes = 4 chunks, chunk c of
//       row r lives at chunk c ^ ((r >> 2) & 3); BK = 64: row = 128 bytes = 8 chunks, chunk c
//       at c ^ ((r >> 1) & 7).  MFMA operand = one ds_read_b128.
//   KN: [k][C] for sources contiguous along M or N; k row = 2C bytes; chunk c of k row r lives
//       at chunk c ^ (4 * (r & 3)).  MFMA operand = two ds_read_b64_tr_b16: within a 16-lane
//       group, lane s supplies the address of (k = k0 + s/4, col = c0 + 4*(s%4)) and lane i
//       receives the 4 values (k0..k0+3, c0 + i).
template <int BK>
__device__ __forceinline__ int km_swz(int row) {
  if constexpr (BK == 32) return (row >> 2) & 3;
  else return (row >> 1) & 7;
}
template <int BK>
__device__ __forceinline__ uint32_t km_off(int row, int c) {
  return row * (2 * BK) + ((c ^ km_swz<BK>(row)) << 4);
}
template <int C>
__device__ __forceinline__ uint32_t kn_off(int kr, int col) {
  return kr * (2 * C) + ((((col >> 3) ^ (4 * (kr & 3)))) << 4) + ((col & 7) << 1);
}

template <int BK>
__device__ __forceinline__ bf16x8_t read_km(uint32_t base, int row, int c) {
  return *(const LDS_AS bf16x8_t*)(uintptr_t)(base + km_off<BK>(row, c));
}
// 32-column fragment at column cbase, k16 step kk: lane holds column cbase + lane%32 and
// k = 16*kk + 8*(lane/32) + 0..7.
template <int C>
__device__ __forceinline__ bf16x8_t read_kn(uint32_t base, int cbase, int kk, int lane) {
  const int grp = lane >> 4, i16 = lane & 15;
  const int col = cbase + 16 * (grp & 1) + 4 * (i16 & 3);
  const int kr0 = 16 * kk + 8 * (grp >> 1) + (i16 >> 2);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(uintptr_t)(base + kn_off<C>(kr0, col)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(uintptr_t)(base + kn_off<C>(kr0 + 4, col)));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  const u32x4 v = {l2.x, l2.y, h2.x, h2.y};
  return __builtin_bit_cast(bf16x8_t, v);
}

// LDS DMA of one dword per lane (to m0 + 4*lane).
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_byte_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gptr), "s"(lds_byte_addr)
               : "memory", "m0");
}

// ---------------------------------------------------------------- fp8 (OCP e4m3) operand tiles
typedef int i32x2v __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// KN fp8 layout: [k][256 bytes]; chunk c (16 columns) of k row r lives at chunk c ^ (2 * (r & 7)).
__device__ __forceinline__ uint32_t kn8_off(int kr, int col) {
  return kr * 256 + ((((col >> 4) ^ (2 * (kr & 7)))) << 4) + (col & 15);
}

// 32-column fragment at column cbase, 64-deep step kk: lane holds column cbase + lane%32 and
// k = 64*kk + 32*(lane/32) + 0..31.  Within a 16-lane group, lane s supplies the address of
// (k = k0 + s/2, col = c0 + 8*(s%2)) and lane i receives the 8 bytes (k0..k0+7, c0 + i).
__device__ __forceinline__ i32x8 read_kn8(uint32_t base, int cbase, int kk, int lane) {
  const int grp = lane >> 4, i16 = lane & 15;
  const int col = cbase + 16 * (grp & 1) + 8 * (i16 & 1);
  const int krb = 64 * kk + 32 * (grp >> 1) + (i16 >> 1);
  i32x8 v;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const i32x2v t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2v*)(uintptr_t)(base + kn8_off(krb + 8 * h, col)));
    v[2 * h] = t.x;
    v[2 * h + 1] = t.y;
  }
  return v;
}

// KM fp8 layout: [row][128 bytes], chunk c of row r at chunk c ^ ((r >> 1) & 7); 32 bytes per
// lane = two chunks.
__device__ __forceinline__ i32x8 read_km8(uint32_t base, int row, int kk, int lane) {
  const int c = 4 * kk + 2 * (lane >> 5);
  const u32x4 lo = *(const LDS_AS u32x4*)(uintptr_t)(base + km_off<64>(row, c));
  const u32x4 hi = *(const LDS_AS u32x4*)(uintptr_t)(base + km_off<64>(row, c + 1));
  i32x8 v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

// The same fragments in the k order the block-scaled MFMA assigns to its two 32-value scale
// blocks: bytes 0..15 of lane l hold k = 64*kk + 16*(l/32) + 0..15 and bytes 16..31 hold
// k = 64*kk + 32 + 16*(l/32) + 0..15, so scale block b of the step (lane l's exponent for
// b = l/32) covers k = 64*kk + 32*b + 0..31.  (An unscaled product only needs A and B in the same
// order; per-block exponents need this one.)
__device__ __forceinline__ i32x8 read_kn8_mx(uint32_t base, int cbase, int kk, int lane) {
  const int grp = lane >> 4, i16 = lane & 15, half = grp >> 1;
  const int col = cbase + 16 * (grp & 1) + 8 * (i16 & 1);
  i32x8 v;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int k0 = 64 * kk + (h < 2 ? 16 * half + 8 * h : 32 + 16 * half + 8 * (h - 2));
    const i32x2v t =
        __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2v*)(uintptr_t)(base + kn8_off(k0 + (i16 >> 1), col)));
    v[2 * h] = t.x;
    v[2 * h + 1] = t.y;
  }
  return v;
}
__device__ __forceinline__ i32x8 read_km8_mx(uint32_t base, int row, int kk, int lane) {
  const int half = lane >> 5;
  const u32x4 lo = *(const LDS_AS u32x4*)(uintptr_t)(base + km_off<64>(row, 4 * kk + half));
  const u32x4 hi = *(const LDS_AS u32x4*)(uintptr_t)(base + km_off<64>(row, 4 * kk + 2 + half));
  i32x8 v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

// A transposed 32x32 accumulator block (lane l holds row l % 32; element r is column
// 8*(r/4) + 4*(l/32) + r%4) as bf16 runs of 8 consecutive columns: v_permlane32_swap trades
// halves between lanes l and l+32, leaving lo = columns 8h..8h+7 and hi = columns 16+8h..23+8h
// (h = l/32), each one 16-byte store.
__device__ __forceinline__ void pack_rows_bf16(const f32x16_t& v, uint4& lo, uint4& hi) {
  uint32_t p[4][2];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    p[q][0] = pack_bf16x2(v[4 * q], v[4 * q + 1]);
    p[q][1] = pack_bf16x2(v[4 * q + 2], v[4 * q + 3]);
  }
#pragma unroll
  for (int a = 0; a < 4; a += 2)
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const auto r = __builtin_amdgcn_permlane32_swap(p[a][d], p[a + 1][d], false, false);
      p[a][d] = r[0];
      p[a + 1][d] = r[1];
    }
  lo = make_uint4(p[0][0], p[0][1], p[1][0], p[1][1]);
  hi = make_uint4(p[2][0], p[2][1], p[3][0], p[3][1]);
}

// e4m3 with round to nearest even, saturating at +-448.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  auto sat = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), w, true);
  return (uint32_t)w;
}

}  // namespace moe
