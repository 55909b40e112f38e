// Internal declarations shared by the host library (mla_api.cpp) and the HIP
// kernel sources. Not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/mla.h"

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
// that each decode call copies into the workspace.
struct mla_plan {
  int32_t batch = 0;
  int32_t n_items = 0;
  int32_t chunk = 0;
  int32_t n_workers = 0;
  uint64_t id = 0;             // unique per plan made in this process
  void *host_block = nullptr;  // pinned: [n_items WorkItem][batch SeqInfo]
  size_t host_block_bytes = 0;
  bool pinned = false;
  std::vector<int32_t> lens;
  const mla::WorkItem *items() const { return static_cast<const mla::WorkItem *>(host_block); }
  const mla::SeqInfo *seqs() const {
    return reinterpret_cast<const mla::SeqInfo *>(static_cast<const char *>(host_block) +
                                                   sizeof(mla::WorkItem) * n_items);
  }
};

namespace mla {

// Workspace layout for decode (byte offsets from ws).
struct DecodeWs {
  size_t status = 0;  // int32 status word (256 bytes reserved)
  size_t items = 0;   // WorkItem[n_items]
  size_t seqs = 0;    // SeqInfo[batch]
  size_t q = 0;       // absorbed query [batch, H, d_c + d_rope]: bf16 (fast) or f32
  size_t opart = 0;   // normalised split partials [n_items, H, d_c]: f32, or fp16 on the matrix-core path
  size_t lse = 0;     // f32 [n_items, H]
  size_t total = 0;
};
// q_len new query tokens per sequence multiply every per-head array.
DecodeWs decode_ws_layout(const mla_dims &d, int32_t batch, int32_t n_items, int32_t q_len = 1);

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

hipError_t launch_absorb_generic(hipStream_t s, const mla_dims &d, int32_t batch,
                                 const void *q_nope, const void *q_rope, const int32_t *q_pos,
                                 const void *w_uk, mla_dtype qw, const SeqInfo *seqs, float *q_out);
// The matrix-core launchers take q_len new query tokens per sequence (1 for
// a plain decode): heads become (token, head) pairs, token-major.
hipError_t launch_absorb_fast(hipStream_t s, const mla_dims &d, int32_t batch, int32_t q_len,
                              const void *q_nope, const void *q_rope, const int32_t *q_pos,
                              const void *w_uk, const SeqInfo *seqs, uint16_t *q_out);

hipError_t launch_decode_generic(hipStream_t s, const mla_dims &d, const mla_cache &c,
                                 int32_t n_items, const WorkItem *items, const SeqInfo *seqs,
                                 const float *q, float *opart, float *lse, int32_t *status);
hipError_t launch_decode_fast(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t q_len,
                              int32_t n_items, const WorkItem *items, const SeqInfo *seqs,
                              const uint16_t *q, uint16_t *opart, float *lse, int32_t *status);

hipError_t launch_combine_generic(hipStream_t s, const mla_dims &d, const mla_cache &c,
                                  const SeqInfo *seqs, const float *opart, const float *lse,
                                  const void *w_uv, mla_dtype qw, void *o, mla_dtype od);
hipError_t launch_combine_fast(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t q_len, const SeqInfo *seqs,
                               const uint16_t *opart, const float *lse, const uint16_t *w_uv, void *o, int o_bf16);

hipError_t launch_copy(hipStream_t s, void *dst, const void *src, size_t n16);
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
