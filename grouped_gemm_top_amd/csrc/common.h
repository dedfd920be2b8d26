// Shared device/host helpers for the MoE-LoRA library (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bfloat16 bits

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

__host__ __device__ inline float bf16_to_f32(bf16_t v) {
  union { uint32_t u; float f; } x;
  x.u = ((uint32_t)v) << 16;
  return x.f;
}

// round to nearest even; NaN stays a quiet NaN
__host__ __device__ inline bf16_t f32_to_bf16(float f) {
  union { uint32_t u; float f; } x;
  x.f = f;
  if ((x.u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((x.u >> 16) | 0x40);
  uint32_t r = x.u + 0x7fffu + ((x.u >> 16) & 1u);
  return (bf16_t)(r >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static inline float load(const float* p) { return *p; }
  __device__ static inline float to_f(float v) { return v; }
  __device__ static inline float from_f(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  __device__ static inline float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static inline float to_f(bf16_t v) { return bf16_to_f32(v); }
  __device__ static inline bf16_t from_f(float v) { return f32_to_bf16(v); }
};

__device__ inline float to_f(float v) { return v; }
__device__ inline float to_f(bf16_t v) { return bf16_to_f32(v); }
template <typename T> __device__ inline T from_f(float v);
template <> __device__ inline float from_f<float>(float v) { return v; }
template <> __device__ inline bf16_t from_f<bf16_t>(float v) { return f32_to_bf16(v); }

__device__ inline float sigmoidf_(float v) { return 1.0f / (1.0f + __expf(-v)); }

// wave64 reductions through cross-lane shuffles
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace moe
