// Device helpers shared by the HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// ---- bfloat16 <-> float -----------------------------------------------------------------------
// bf16 is carried as its 16-bit pattern.  Widening is exact (shift into the high half).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round-to-nearest-even narrowing (inputs here are finite; NaN is kept a NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Two floats -> packed pair of bf16 (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return uint32_t(f32_to_bf16(a)) | (uint32_t(f32_to_bf16(b)) << 16);
}

// Element access for the two storage types used by the plain kernels.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float *p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// ---- wavefront reductions (64 lanes) -----------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block-wide reductions for blocks of up to 1024 threads; `red` must hold 16 floats.
__device__ __forceinline__ float block_max(float v, float *red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float r = -INFINITY;
  for (int i = 0; i < nw; ++i) r = fmaxf(r, red[i]);
  return r;
}
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < nw; ++i) r += red[i];
  return r;
}

}  // namespace mla
