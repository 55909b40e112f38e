// Device-side helpers: storage conversions, RoPE angles, wave reductions,
// the status word. gfx950 only.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_internal.hpp"

namespace mla {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFp8Max = 448.0f;
// Largest finite fp16 magnitude: the matrix-core path carries cached values
// (bf16, or fp8 codes times their scale) and the absorbed query in fp16.
constexpr float kF16Max = 65504.0f;

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
// positions (131071 and beyond) keep full fp32 accuracy. The angle is first
// reduced to [-pi, pi] by a - k 2 pi with 2 pi split into two doubles (the
// fused multiply-add keeps k * hi exact; accurate to ~1e-15 for |k| < 2^30),
// so the sine and cosine only ever see a small argument.

// The rotation frequency of RoPE pair j of d dimensions, base^(-2j/d).
__device__ __forceinline__ double rope_theta(int j, int d, float base) {
  return pow(static_cast<double>(base), -2.0 * j / d);
}
// cos and sin of the angle pos * theta, reduced by 2 pi in fp64.
__device__ __forceinline__ void rope_cos_sin_theta(int64_t pos, double theta, float *c, float *s) {
  const double a = static_cast<double>(pos) * theta;
  const double k = rint(a * 0.15915494309189535);  // 1 / (2 pi)
  double r = fma(-k, 6.283185307179586, a);          // 2 pi, high part
  r = fma(-k, 2.4492935982947064e-16, r);            // 2 pi, low part
  double sd, cd;
  sincos(r, &sd, &cd);
  *c = static_cast<float>(cd);
  *s = static_cast<float>(sd);
}
__device__ __forceinline__ void rope_cos_sin(int64_t pos, int j, int d, float base, float *c, float *s) {
  rope_cos_sin_theta(pos, rope_theta(j, d, base), c, s);
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
__device__ __forceinline__ void set_status(int32_t *status, int32_t code);

// Finish one appended row from its fp32 projections outv[0 .. d_c + d_rope)
// (already in LDS, k_rope part rotated): round to the storage dtypes and
// store it at `row`. fp8 latents get the per-token scale amax / 448 (1 for a
// zero row). A bf16 or fp8 row (the dtypes the matrix-core decode widens to
// fp16) with a magnitude of 65504 or more is stored as it is and reported
// (MLA_ERR_RANGE). Called by all 256 threads of the block; `red` is 4 floats
// of LDS.
__device__ __forceinline__ void store_appended_row(const mla_dims &d, const mla_cache &c, int64_t row,
                                                   const float *outv, float *red, int32_t *status) {
  const int tid = threadIdx.x;
  char *rowp = static_cast<char *>(c.rows) + row * c.row_stride;
  if (c.latent_dtype != MLA_F32) {
    float am = 0.0f;
    for (int k = tid; k < d.d_c + d.d_rope; k += 256) am = fmaxf(am, fabsf(outv[k]));
    am = block_max_256(am, red);
    if (tid == 0 && !(am < kF16Max)) set_status(status, MLA_ERR_RANGE);
  }
  if (c.latent_dtype == MLA_FP8_E4M3) {
    float am = 0.0f;
    for (int k = tid; k < d.d_c; k += 256) am = fmaxf(am, fabsf(outv[k]));
    am = block_max_256(am, red);
    const float s = am > 0.0f ? am / kFp8Max : 1.0f;
    for (int k = tid; k < d.d_c; k += 256) reinterpret_cast<uint8_t *>(rowp)[k] = f32_to_fp8(outv[k] / s);
    if (tid == 0) c.scale[row] = s;
  } else if (c.latent_dtype == MLA_BF16) {
    for (int k = tid; k < d.d_c; k += 256) reinterpret_cast<uint16_t *>(rowp)[k] = f32_to_bf16_bits(outv[k]);
  } else {
    for (int k = tid; k < d.d_c; k += 256) reinterpret_cast<float *>(rowp)[k] = outv[k];
  }
  char *rp = rowp + static_cast<int64_t>(d.d_c) * elem_bytes(c.latent_dtype);
  if (c.rope_dtype == MLA_BF16) {
    for (int k = tid; k < d.d_rope; k += 256) reinterpret_cast<uint16_t *>(rp)[k] = f32_to_bf16_bits(outv[d.d_c + k]);
  } else {
    for (int k = tid; k < d.d_rope; k += 256) reinterpret_cast<float *>(rp)[k] = outv[d.d_c + k];
  }
}

// First error wins.
__device__ __forceinline__ void set_status(int32_t *status, int32_t code) {
  atomicCAS(status, 0, code);
}

// Run by every thread of one workgroup of the first kernel of a decode: the
// checksum of the workspace's plan copy against the plan's; on a mismatch
// the copy is fetched again from the plan's pinned host block (the kernels
// that read the copy run after this one, in stream order).
__device__ __forceinline__ void plan_verify(const PlanRef &p) {
  typedef uint32_t u32x4_ __attribute__((ext_vector_type(4)));
  __shared__ unsigned long long sum;
  if (threadIdx.x == 0) sum = 0;
  __syncthreads();
  const u32x4_ *dev = static_cast<const u32x4_ *>(p.dev);
  uint64_t h = 0;
  for (int x = threadIdx.x; x < p.nchunks; x += blockDim.x) {
    const u32x4_ v = dev[x];
    h += plan_chunk_hash(static_cast<uint32_t>(x), v[0], v[1], v[2], v[3]);
  }
  // the wave's sum first (one LDS atomic per wave, not per thread)
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(h), off), hi = __shfl_xor(static_cast<uint32_t>(h >> 32), off);
    h += (static_cast<uint64_t>(hi) << 32) | lo;
  }
  if ((threadIdx.x & 63) == 0) atomicAdd(&sum, static_cast<unsigned long long>(h));
  __syncthreads();
  if (sum != p.hash) {
    const u32x4_ *host = static_cast<const u32x4_ *>(p.host);
    for (int x = threadIdx.x; x < p.nchunks; x += blockDim.x) const_cast<u32x4_ *>(dev)[x] = host[x];
  }
}

// Token range [0, t1) of sequence b lies in the cache: within its reserved
// tokens, and (contiguous) within the rows or (paged) within its block
// table row.
__device__ __forceinline__ bool seq_range_ok(const mla_cache &c, int b, int64_t t1) {
  if (t1 > c.seq_cap[b]) return false;
  if (c.block_table == nullptr)
    return static_cast<int64_t>(c.seq_start[b]) >= 0 && static_cast<int64_t>(c.seq_start[b]) + t1 <= c.n_rows;
  return t1 <= static_cast<int64_t>(c.max_blocks) * c.block_tokens;
}

// Whether n_new >= 1 tokens can be appended to sequence b at its current
// length len: the range [0, len + n_new) passes seq_range_ok and, in a
// paged cache, every block the new tokens fall in is inside the cache.
// MLA_OK, MLA_ERR_CAPACITY or MLA_ERR_PLAN (a block id outside the cache).
// The append kernels write a sequence's rows, and advance_len_kernel adds
// n_new to its length, only when this gives MLA_OK: a refused sequence is
// left untouched.
__device__ __forceinline__ int32_t append_check(const mla_cache &c, int b, int32_t len, int32_t n_new) {
  if (len < 0 || !seq_range_ok(c, b, static_cast<int64_t>(len) + n_new)) return MLA_ERR_CAPACITY;
  if (c.block_table != nullptr) {
    const int64_t bt = c.block_tokens;
    const int64_t last = (static_cast<int64_t>(len) + n_new - 1) / bt;
    for (int64_t x = len / bt; x <= last; ++x) {
      const int64_t blk = c.block_table[static_cast<int64_t>(b) * c.max_blocks + x];
      if (blk < 0 || (blk + 1) * bt > c.n_rows) return MLA_ERR_PLAN;
    }
  }
  return MLA_OK;
}

// Row of token t of sequence b (t inside a range seq_range_ok accepted):
// seq_start[b] + t, or through the block table. A block id outside the cache
// sets bad and reads block 0 instead.
__device__ __forceinline__ int64_t cache_row(const mla_cache &c, int b, int64_t t, bool &bad) {
  if (c.block_table == nullptr) return static_cast<int64_t>(c.seq_start[b]) + t;
  const int64_t bt = c.block_tokens;
  int64_t blk = c.block_table[static_cast<int64_t>(b) * c.max_blocks + t / bt];
  if (blk < 0 || (blk + 1) * bt > c.n_rows) {
    bad = true;
    blk = 0;
  }
  return blk * bt + t % bt;
}

}  // namespace mla
