// Checksum of a plan's work list, computed on the host when the plan is made
// and on the device by the first kernel of every decode, which compares it
// with the copy the workspace holds: a copy that differs (a fresh workspace,
// one the caller reused for other data, or one an append's partial products
// overwrote) is fetched again from the plan's pinned host block before any
// kernel reads it. The library keeps no record of which workspace holds
// which plan: the workspace is checked, every call.
//
// The block is hashed as 16-byte chunks: chunk i with 32-bit words w0..w3
// contributes mix(mix(lo ^ i * phi) ^ hi) (lo = w1:w0, hi = w3:w2), summed
// modulo 2^64. mix is the 64-bit finaliser of Steele, Lea and Flood's
// SplitMix64 generator; phi is the 64-bit golden-ratio constant it uses as
// its increment.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mla {

__host__ __device__ inline uint64_t plan_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t plan_chunk_hash(uint32_t i, uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  const uint64_t lo = (static_cast<uint64_t>(w1) << 32) | w0;
  const uint64_t hi = (static_cast<uint64_t>(w3) << 32) | w2;
  return plan_mix64(plan_mix64(lo ^ (static_cast<uint64_t>(i) * 0x9e3779b97f4a7c15ull)) ^ hi);
}

// Where a decode finds its plan: the pinned host block (device-readable),
// the workspace copy the kernels read, its size in 16-byte chunks, and the
// checksum the copy must have.
struct PlanRef {
  const void *host;
  void *dev;
  int32_t nchunks;
  uint64_t hash;
};

}  // namespace mla
