// Device-side helpers: storage conversions, RoPE angles, wave reductions,
// the status word. gfx950 only.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_internal.hpp"

namespace mla {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFp8Max = 448.0f;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// OCP E4M3FN byte -> f32 (v_cvt_f32_fp8; gfx950 uses the OCP encoding).
__device__ __forceinline__ float fp8_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(byte & 0xFFu), 0);
}

// f32 -> OCP E4M3FN byte, round to nearest even, saturated to +-448 first so
// out-of-range inputs never become NaN.
__device__ __forceinline__ uint8_t f32_to_fp8(float f) {
  f = fminf(fmaxf(f, -kFp8Max), kFp8Max);
  return static_cast<uint8_t>(__builtin_amdgcn_cvt_pk_fp8_f32(f, 0.0f, 0, false) & 0xFF);
}

// Load element i of an array of the given dtype as f32 (generic path).
__device__ __forceinline__ float load_elem(const void *p, int64_t i, mla_dtype t) {
  switch (t) {
    case MLA_F32: return static_cast<const float *>(p)[i];
    case MLA_BF16: return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    default: return fp8_to_f32(static_cast<const uint8_t *>(p)[i]);
  }
}

__device__ __forceinline__ int elem_bytes(mla_dtype t) {
  return t == MLA_F32 ? 4 : (t == MLA_BF16 ? 2 : 1);
}

// RoPE angle pos * base^(-2j/d) and its cosine/sine, formed in fp64 so large
// positions (131071 and beyond) keep full fp32 accuracy.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, int j, int d, float base, float *c, float *s) {
  double theta = pow(static_cast<double>(base), -2.0 * j / d);
  double a = static_cast<double>(pos) * theta;
  double sd, cd;
  sincos(a, &sd, &cd);
  *c = static_cast<float>(cd);
  *s = static_cast<float>(sd);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide reductions for blockDim.x == 256 (4 waves); `red` is 4 floats of LDS.
__device__ __forceinline__ float block_sum_256(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__device__ __forceinline__ float block_max_256(float v, float *red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// First error wins.
__device__ __forceinline__ void set_status(int32_t *status, int32_t code) {
  atomicCAS(status, 0, code);
}

}  // namespace mla
