// Shared device helpers for the gfx950 MoE kernels (wave64, CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 converts two values in one
// instruction (bit-identical to rounding the fp32 pattern by hand for finite inputs, including
// ties and subnormals; checked on the GPU against the integer form).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// 16-byte load of data read once, whose 128-byte lines one wave instruction reads whole:
// non-temporal, so it does not displace lines that are reused (the combine: 5.0 -> 6.2 TB/s).
// Loads that take a line in several pieces from several instructions stay cached: the dA
// epilogue's H loads ran 11 % slower non-temporal.
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_once16(const void* p) {
  const u32x4_nt w = __builtin_nontemporal_load((const u32x4_nt*)p);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ void store_once16(void* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4_nt{v.x, v.y, v.z, v.w}, (u32x4_nt*)p);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Logistic sigmoid with the hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32: about 1 ulp
// each) instead of an IEEE division, whose scale/fixup sequence cost ten VALU instructions per
// element in the SwiGLU epilogues.  z -> -inf gives 1/inf = 0.
__device__ __forceinline__ float sigmoidf_fast(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

// Exclusive scan of one int per thread over a 1024-thread block; returns the block total.
__device__ __forceinline__ int block_excl_scan_1024(int v, int* sh, int* excl) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wv] = x;
  __syncthreads();
  if (wv == 0) {
    int t = (lane < 16) ? sh[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(t, o, 64);
      if (lane >= o) t += y;
    }
    if (lane < 16) sh[16 + lane] = t;  // inclusive wave totals
  }
  __syncthreads();
  const int before = (wv == 0) ? 0 : sh[16 + wv - 1];
  *excl = before + x - v;
  const int total = sh[16 + 15];
  __syncthreads();
  return total;
}

}  // namespace moe
