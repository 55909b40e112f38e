// Internal declarations shared by the host library (mla_api.cpp) and the HIP
// kernel sources. Not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/mla.h"
#include "plan_hash.hpp"

namespace mla {

// Tokens per tile of the matrix-core split-K kernels; work-item boundaries
// are multiples of it so every tile except a sequence's last is full.
constexpr int kTile = 32;

// Most new query tokens per sequence one mla_decode_multi call takes.
constexpr int kMaxQueryTokens = 16;

// Kernel ids for the optional event-based profiler.
enum KernelId : int {
  K_INIT = 0,
  K_APPEND_GENERIC,
  K_APPEND_GEMM,
  K_APPEND_FINISH,
  K_ABSORB_GENERIC,
  K_ABSORB_FAST,
  K_DECODE_GENERIC,
  K_DECODE_BF16,
  K_DECODE_FP8,
  K_COMBINE_GENERIC,
  K_COMBINE_FAST,
  K_COPY,
  K_READ,
  K_MERGE_GEMM,
  K_ABSORB_MERGED,
  K_OUT_MERGED,
  K_COMBINE_EMIT,
  K_COUNT
};

// One decode work item: sequence b, tokens [t0, t1). Its partial result goes
// to slot k (its index in the item list).
struct alignas(16) WorkItem {
  int32_t b, t0, t1, pad;
};

// Per-sequence plan data: items [item_begin, item_begin + item_count), and
// the length the plan was made for.
struct alignas(16) SeqInfo {
  int32_t item_begin, item_count, len, pad;
};

}  // namespace mla

// The plan is host-owned; items and seq info live in one pinned host block
// (device-readable). The first kernel of each decode checks the workspace's
// copy of it against the block's checksum and fetches the block again when
// they differ.
struct mla_plan {
  int32_t batch = 0;
  int32_t n_items = 0;
  int32_t n_ranges = 0;            // workgroup ranges: range j runs items ranges[j] .. ranges[j + 1] - 1
  int32_t n_workers = 0;
  // [n_items WorkItem][batch SeqInfo][n_ranges + 1 int32, padded to 16
  // bytes], pinned when a device is there
  void *host_block = nullptr;
  const void *host_dev = nullptr;  // the same block's device address (nullptr: not pinned)
  bool pinned = false;
  size_t host_block_bytes = 0;
  uint64_t hash = 0;               // plan_chunk_hash sum over the block
  std::vector<int32_t> lens;
  const mla::WorkItem *items() const { return static_cast<const mla::WorkItem *>(host_block); }
  const mla::SeqInfo *seqs() const {
    return reinterpret_cast<const mla::SeqInfo *>(static_cast<const char *>(host_block) +
                                                   sizeof(mla::WorkItem) * n_items);
  }
};

namespace mla {

// Workspace layout for decode (byte offsets from ws). The plan copy comes
// last, past the region an append's partial products use whenever the
// decode arrays are larger than those (so a decode step's append leaves it
// intact; if it does not, the copy is fetched again).
struct DecodeWs {
  size_t status = 0;  // int32 status word (256 bytes reserved)
  size_t q = 0;       // absorbed query [batch, H, d_c + d_rope]: fp16 (matrix-core path) or f32
  size_t opart = 0;   // normalised split partials [n_items, H, d_c]: fp16 (matrix-core path) or f32
  size_t lse = 0;     // f32 [n_items, H]
  size_t items = 0;   // WorkItem[n_items]
  size_t seqs = 0;    // SeqInfo[batch]
  size_t ranges = 0;  // int32[n_ranges + 1] (items, seqs, ranges: one copy of the plan's block)
  size_t total = 0;
};
// q_len new query tokens per sequence multiply every per-head array; fast
// selects the matrix-core path's 2-byte query and partials.
DecodeWs decode_ws_layout(const mla_dims &d, const mla_plan &plan, int32_t q_len, bool fast);
// Bytes of a plan's block: its items, sequence records and range starts.
size_t plan_block_bytes(int32_t n_items, int32_t batch, int32_t n_ranges);

struct AppendWs {
  size_t status = 0;
  size_t partial = 0;  // f32 [ksplit, tokens, d_c + d_rope] (fast path only)
  size_t total = 0;
  int ksplit = 0;
};
AppendWs append_ws_layout(const mla_dims &d, int32_t batch, int32_t n_new);

// Which decode implementation handles these arguments.
bool decode_fast_path(const mla_dims &d, const mla_cache &c, mla_dtype q_w_dtype);
bool append_fast_path(const mla_dims &d, int32_t tokens, mla_dtype act_w_dtype);
// The shapes the matrix-core append handles (the workspace is sized for it
// whenever the shape qualifies, whatever the dtype or environment).
bool append_fast_shape(const mla_dims &d, int32_t tokens);
// K-splits of the matrix-core append's down-projection (d_model inputs per
// split fixed by the kernel), when append_fast_shape holds.
int append_fast_ksplit(const mla_dims &d);

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error. All take the stream first.

hipError_t launch_init(hipStream_t s, int32_t *status);

hipError_t launch_append_generic(hipStream_t s, const mla_dims &d, const mla_cache &c,
                                 const void *h, int32_t n_new, const void *w_dkv,
                                 const void *w_kr, mla_dtype act, int32_t *status);
hipError_t launch_append_fast(hipStream_t s, const mla_dims &d, const mla_cache &c,
                              const void *h, int32_t n_new, const void *w_dkv, const void *w_kr,
                              float *partial, int ksplit, int32_t *status);
hipError_t launch_append_finish(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t n_new,
                                const float *partial, int ksplit, int32_t *status);
hipError_t launch_advance_len(hipStream_t s, const mla_cache &c, int32_t n_new);

// The absorb kernels, the first of every decode, also check the
// workspace's plan copy (one workgroup, see PlanRef); the matrix-core one
// reports MLA_ERR_RANGE in the status word when a query value leaves fp16's
// range. They take the query position from the cache's seq_len (equal to
// the plan's length, or the split-K kernel reports MLA_ERR_PLAN and zeroes
// the output).
hipError_t launch_absorb_generic(hipStream_t s, const mla_dims &d, int32_t batch,
                                 const void *q_nope, const void *q_rope, const int32_t *q_pos,
                                 const void *w_uk, mla_dtype qw, const int32_t *seq_len, float *q_out,
                                 const PlanRef &plan, int32_t *status);
// The matrix-core launchers take q_len new query tokens per sequence (1 for
// a plain decode): heads become (token, head) pairs, token-major.
hipError_t launch_absorb_fast(hipStream_t s, const mla_dims &d, int32_t batch, int32_t q_len,
                              const void *q_nope, const void *q_rope, const int32_t *q_pos,
                              const void *w_uk, const int32_t *seq_len, uint16_t *q_out, const PlanRef &plan,
                              int32_t *status);

hipError_t launch_decode_generic(hipStream_t s, const mla_dims &d, const mla_cache &c,
                                 int32_t n_items, const WorkItem *items, const SeqInfo *seqs,
                                 const float *q, float *opart, float *lse, int32_t *status);
// fp8 latents on the fp8 matrix cores (k_splitk8.hip); launch_decode_fast
// sends fp8 caches there.
// The matrix-core split-K kernels run one workgroup per (range, head block
// of 128): it walks the range's items one after the other.
hipError_t launch_decode_fast8(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t q_len, int32_t n_items,
                               int32_t n_ranges, const int32_t *ranges, const WorkItem *items, const SeqInfo *seqs,
                               const uint16_t *q, uint16_t *opart, float *lse, int32_t *status);
hipError_t launch_decode_fast(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t q_len,
                              int32_t n_items, int32_t n_ranges, const int32_t *ranges, const WorkItem *items,
                              const SeqInfo *seqs, const uint16_t *q, uint16_t *opart, float *lse, int32_t *status);

hipError_t launch_combine_generic(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t n_items,
                                  const SeqInfo *seqs, const float *opart, const float *lse,
                                  const void *w_uv, mla_dtype qw, void *o, mla_dtype od, int32_t *status);
hipError_t launch_combine_fast(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t q_len, int32_t n_items,
                               const SeqInfo *seqs, const uint16_t *opart, const float *lse, const uint16_t *w_uv,
                               void *o, int o_bf16, int32_t *status);

// Decode from precomputed absorbed weights (k_merged.hip). The combine
// kernels, given ohat, write o^ instead of applying W_UV: fp32 [B, H d_c] on
// the generic path, bf16 hi and lo planes [B, H 512] on the matrix-core path.
namespace merged {
constexpr int DC = 512;
// K splits of the matrix-core output product (each a multiple of 256 wide)
inline int out_splits(int64_t K) { return K % (16 * 256) == 0 ? 16 : 1; }
// Layout of a merged weight [R rows x K columns]: when R % 32 == 0 and
// K % 64 == 0, fragment-tiled, so that every load of the weight-streaming
// kernel reads 1 KB contiguous: tile (r / 32, k / 64) of 2048 elements at
// ((r / 32) (K / 64) + k / 64) 2048, and inside it element (r, k) at
// ((k % 32) / 8) 512 + (r % 32 + 32 ((k % 64) / 32)) 8 + k % 8 (the order
// in which the lanes of a wave take the A operand of four 32x32x16
// products). Otherwise row-major, r K + k.
__host__ __device__ inline bool tiled(int64_t R, int64_t K) { return R % 32 == 0 && K % 64 == 0; }
__host__ __device__ inline int64_t weight_off(int64_t r, int64_t k, int64_t K, bool tl) {
  if (!tl) return r * K + k;
  return ((r >> 5) * (K >> 6) + (k >> 6)) * 2048 + ((k & 31) >> 3) * 512 + ((r & 31) + 32 * ((k & 63) >> 5)) * 8 +
         (k & 7);
}
}  // namespace merged
// C[t] = P[t]^T Q[t]; element (t, m, n) goes to the row-major offset
// t sCt + m sCm + n sCn, or, with tileK > 0, to that offset's place in the
// fragment-tiled layout of a weight whose rows are tileK long.
hipError_t launch_merge_gemm(hipStream_t s, int T, int M, int N, int K, const void *P, int64_t sPt, int64_t sPk,
                             int64_t sPm, const void *Q, int64_t sQt, int64_t sQk, int64_t sQn, mla_dtype in, void *C,
                             int64_t sCt, int64_t sCm, int64_t sCn, mla_dtype out, int64_t tileK);
hipError_t launch_absorb_merged_fast(hipStream_t s, const mla_dims &d, int32_t batch, int32_t d_x, const void *x,
                                     const void *q_rope, const int32_t *q_pos, const void *a,
                                     const int32_t *seq_len, uint16_t *q_out, const PlanRef &plan, int32_t *status);
hipError_t launch_out_merged_fast(hipStream_t s, int32_t batch, int32_t d_out, int64_t K, const void *bm,
                                  const uint16_t *ohat_hi, const uint16_t *ohat_lo, float *part, void *y, int y_bf16);
hipError_t launch_absorb_merged_generic(hipStream_t s, const mla_dims &d, int32_t batch, int32_t d_x, const void *x,
                                        const void *q_rope, const int32_t *q_pos, const void *a, mla_dtype wt,
                                        const int32_t *seq_len, float *q_out, const PlanRef &plan);
hipError_t launch_out_merged_generic(hipStream_t s, int32_t batch, int32_t d_out, int64_t K, const void *bm,
                                     mla_dtype wt, const float *ohat, void *y, mla_dtype yt);
hipError_t launch_combine_generic_emit(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t n_items,
                                       const SeqInfo *seqs, const float *opart, const float *lse, float *ohat,
                                       int32_t *status);
hipError_t launch_combine_fast_emit(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t n_items,
                                    const SeqInfo *seqs, const uint16_t *opart, const float *lse, uint16_t *ohat_hi,
                                    uint16_t *ohat_lo, int32_t *status);

hipError_t launch_copy(hipStream_t s, void *dst, const void *src, size_t n16);
// *dst = *src for one int32 (a one-thread kernel: capturable, no memcpy node)
hipError_t launch_status_copy(hipStream_t s, const int32_t *src, int32_t *dst);

// The decode entry points' shared steps (mla_api.cpp). decode_launch runs
// absorb, split-K and combine with the workspace at ws; compact lays the
// workspace out for the path that runs (2-byte query and partials on the
// matrix-core path; decode_compact_bytes gives that size) instead of the
// size the workspace queries report; clear_status zeroes the status word
// first (a one-thread kernel).
mla_status decode_check_args(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan,
                             const void *q_nope, const void *q_rope, const void *w_uk, const void *w_uv,
                             mla_dtype qw, const void *o, mla_dtype od, const void *ws, size_t ws_bytes,
                             int32_t q_len);
size_t decode_compact_bytes(const mla_dims &d, const mla_cache &c, const mla_plan &plan, mla_dtype qw);
// softmax_scale 0 in mla_dims stands for the default (d_nope + d_rope)^(-1/2),
// computed in double and rounded once to float.
inline mla_dims with_default_scale(const mla_dims &d) {
  mla_dims r = d;
  if (r.softmax_scale == 0.0f) r.softmax_scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d.d_nope + d.d_rope)));
  return r;
}
mla_status decode_launch(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan, const void *q_nope,
                         const void *q_rope, const int32_t *q_pos, const void *w_uk, const void *w_uv, mla_dtype qw,
                         void *o, mla_dtype od, void *ws, hipStream_t s, int32_t q_len, bool compact,
                         bool clear_status);
hipError_t launch_read(hipStream_t s, const void *src, size_t n16, uint32_t *sink);

// Profiling hooks used by the launch wrappers in mla_api.cpp. While a
// profiled call is pending, prof_take() hands its start/stop events to the
// first kernel launched through launch_kernel(), which has the dispatch
// itself record them (kernel-precise, like a kernel trace).
void prof_before(hipStream_t s, int kernel_id);
void prof_after(hipStream_t s, int kernel_id);
bool prof_take(hipEvent_t *start, hipEvent_t *stop);

template <class T> struct same_type { using type = T; };

// Every kernel of the library is launched through this (arguments are
// converted to the kernel's own parameter types first).
template <typename... KArgs>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shm, hipStream_t s,
                                typename same_type<KArgs>::type... args) {
  hipEvent_t a = nullptr, b = nullptr;
  if (prof_take(&a, &b)) {
    hipExtLaunchKernelGGL(kernel, grid, block, shm, s, a, b, 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shm, s, args...);
  }
  return hipGetLastError();
}

}  // namespace mla
