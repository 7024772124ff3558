// Internal device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = PA_BLOCK_SIZE;  // tokens per KV block
constexpr int kWave = 64;              // CDNA wavefront width

// 16x16 output tile, K = 32: lane l supplies A[l%16][8 k-values] and
// B[8 k-values][l%16]; lane l receives C[4*(l/16) + j][l%16], j < 4.
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Same tile with K = 16: each lane supplies 4 k-values of A and of B, k-index
// 4*(l/16) + j.
__device__ __forceinline__ f32x4 mfma16x16x16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Reductions over the 4 lanes l, l^16, l^32, l^48 (the four 16-lane rows
// of a column), with the gfx950 row-swap instructions instead of an LDS
// permute: permlane16_swap(v, v) yields, in every lane, its own value and
// the one 16 lanes away (in some order); permlane32_swap(v, v) likewise for
// 32 lanes.  Both results are the same in all 4 lanes.
__device__ __forceinline__ float wave_max_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Element offsets of (slot s, dim c) inside a (block, kv head) tile of the
// pools (layout documented in include/pa.h): K as [D/8][16][8], V as
// [D/32][4][16][2][4], so that 16-byte-per-lane loads of MFMA operands read
// 1 KiB per wavefront with consecutive lanes on consecutive bytes.
__host__ __device__ __forceinline__ int k_tile_off(int s, int c) {
  return (c >> 3) * 128 + s * 8 + (c & 7);
}
__host__ __device__ __forceinline__ int v_tile_off(int s, int c) {
  return (c >> 5) * 512 + (s >> 2) * 128 + (c & 15) * 8 + ((c >> 4) & 1) * 4 + (s & 3);
}

// Byte offsets of (slot s, dim c) inside a tile of the FP8 pools: the same
// operands, one byte per value, ordered so that a 16-byte-per-lane load
// brings two K steps (K as [D/64][4][16][2][8]) or two V pairs (V as
// [D/64][4][16][2][2][4]) of the fp16 order above.
__host__ __device__ __forceinline__ int k8_tile_off(int s, int c) {
  return (c >> 6) * 1024 + ((c >> 3) & 3) * 256 + s * 16 + ((c >> 5) & 1) * 8 + (c & 7);
}
__host__ __device__ __forceinline__ int v8_tile_off(int s, int c) {
  return (c >> 6) * 1024 + (s >> 2) * 256 + (c & 15) * 16 + ((c >> 5) & 1) * 8 +
         ((c >> 4) & 1) * 4 + (s & 3);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Read a wave-uniform int32 through the scalar cache (s_load): it is counted
// by lgkmcnt, so using it right away does not wait for the wave's in-flight
// vector loads.  Only for memory no kernel writes while the reader runs.
__device__ __forceinline__ int32_t scalar_load(const int32_t* p, int64_t i) {
  typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;
  return ((const_i32_ptr)p)[i];
}

inline pa_status launch_status() {
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Softmax scale accepted by the attention entry points: positive and finite
// (the kernels take max(s * c) = c * max(s), which needs c > 0).
inline bool scale_ok(float scale) { return scale > 0.0f && scale <= 3.4028234e38f; }

}  // namespace pa
