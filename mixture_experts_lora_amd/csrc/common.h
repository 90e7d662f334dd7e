// Shared device helpers for the gfx950 MoE-LoRA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// The element type of activations, weights and LoRA factors is bf16, or fp16
// when MOE_F16 is defined: every kernel source that converts elements or
// multiplies them is compiled once per type, into moe::el_bf16 or
// moe::el_f16 (an inline namespace, so code inside one build names its own
// helpers and kernels unqualified).
#ifndef MOE_EL
#ifdef MOE_F16
#define MOE_EL el_f16
#else
#define MOE_EL el_bf16
#endif
#endif

namespace moe {

typedef uint16_t bf16_t;  // raw bits of one 16-bit element (bf16, or fp16 in the fp16 build)
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

inline namespace MOE_EL {

#ifdef MOE_F16
typedef _Float16 e16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf2f(bf16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// float -> fp16 bits, round to nearest even.
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (_Float16)f); }

// One 32x32x16 fp16 MFMA, fp32 accumulate.
__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(e16x8, a),
                                                __builtin_bit_cast(e16x8, b), c, 0, 0, 0);
}
#else
typedef __bf16 e16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// One 32x32x16 bf16 MFMA, fp32 accumulate.
__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(e16x8, a),
                                                 __builtin_bit_cast(e16x8, b), c, 0, 0, 0);
}
#endif

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

}  // inline namespace MOE_EL

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }
__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + __expf(-x)); }


// Exclusive scan of one int per thread over a 256-thread block (all threads
// must call).  `sh` is 4 ints of shared memory; `total` gets the block sum.
__device__ inline int block_excl_scan256(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wid] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int s = sh[w];
    if (w < wid) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
