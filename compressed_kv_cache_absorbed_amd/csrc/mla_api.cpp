// libmla host library: the C ABI of include/mla.h. Argument validation, the
// split planner, workspace layout, kernel dispatch, the device status word
// and the optional event profiler. Every validation runs before any HIP call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "mla_internal.hpp"

using namespace mla;

namespace {

constexpr size_t kStatusBytes = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int dtype_bytes(mla_dtype t) { return t == MLA_F32 ? 4 : (t == MLA_BF16 ? 2 : 1); }

bool is_dtype(mla_dtype t) { return t == MLA_F32 || t == MLA_BF16 || t == MLA_FP8_E4M3; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mla_status check_dims(const mla_dims *d, bool need_model, bool need_heads) {
  if (!d) return MLA_ERR_INVALID_ARG;
  if (d->d_c < 1 || d->d_rope < 2 || (d->d_rope & 1)) return MLA_ERR_INVALID_ARG;
  if (need_heads && (d->n_heads < 1 || d->d_nope < 1 || d->d_v < 1)) return MLA_ERR_INVALID_ARG;
  if (need_model && d->d_model < 1) return MLA_ERR_INVALID_ARG;
  if (!(d->rope_base > 0.0f)) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

mla_status check_cache(const mla_dims &d, const mla_cache *c) {
  if (!c || !c->rows || !c->seq_cap || !c->seq_len) return MLA_ERR_INVALID_ARG;
  if (c->block_table) {
    // paged: blocks of a multiple of 32 rows (one split-K tile never spans two)
    if (c->block_tokens < kTile || c->block_tokens % kTile || c->max_blocks < 1 || c->n_rows < c->block_tokens)
      return MLA_ERR_INVALID_ARG;
  } else if (!c->seq_start) {
    return MLA_ERR_INVALID_ARG;
  }
  if (c->batch < 1 || c->n_rows < 1) return MLA_ERR_INVALID_ARG;
  if (!is_dtype(c->latent_dtype) || (c->rope_dtype != MLA_F32 && c->rope_dtype != MLA_BF16))
    return MLA_ERR_INVALID_ARG;
  if ((c->latent_dtype == MLA_FP8_E4M3) != (c->scale != nullptr)) return MLA_ERR_INVALID_ARG;
  if (c->row_stride < 16 || (c->row_stride & 15) || !aligned16(c->rows)) return MLA_ERR_INVALID_ARG;
  const int64_t lat = static_cast<int64_t>(d.d_c) * dtype_bytes(c->latent_dtype);
  const int64_t rope = static_cast<int64_t>(d.d_rope) * dtype_bytes(c->rope_dtype);
  if (lat + rope > c->row_stride) return MLA_ERR_INVALID_ARG;
  if (lat % 4) return MLA_ERR_INVALID_ARG;  // keeps the k_rope part element-aligned
  return MLA_OK;
}

// ------------------------------------------------------------- profiler
struct ProfRecord {
  int kernel;
  hipEvent_t a, b;
};
struct Profiler {
  std::mutex mu;
  bool on = false;
  int max_records = 0;
  std::vector<ProfRecord> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  hipEvent_t pending_a = nullptr, pending_b = nullptr;
  int pending_kernel = -1;
  bool taken = false;
};
Profiler &prof() {
  static Profiler *p = new Profiler();
  return *p;
}

const char *kKernelNames[K_COUNT] = {
    "init",           "append_generic", "append_gemm",    "append_finish",
    "absorb_generic", "absorb_fast",    "decode_generic", "decode_bf16",
    "decode_fp8",     "combine_generic", "combine_fast",  "copy",
    "read"};

#define MLA_LAUNCH(stream, kid, call)          \
  do {                                         \
    prof_before((stream), (kid));              \
    hipError_t e_ = (call);                    \
    prof_after((stream), (kid));               \
    if (e_ != hipSuccess) return MLA_ERR_HIP;  \
  } while (0)

}  // namespace

namespace mla {

void prof_before(hipStream_t, int kernel_id) {
  Profiler &p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.on || static_cast<int>(p.recs.size()) >= p.max_records) return;
  hipEvent_t a = p.get();
  hipEvent_t b = a ? p.get() : nullptr;
  if (!b) {
    if (a) p.pool.push_back(a);
    return;
  }
  p.pending_a = a;
  p.pending_b = b;
  p.pending_kernel = kernel_id;
  p.taken = false;
}

bool prof_take(hipEvent_t *start, hipEvent_t *stop) {
  Profiler &p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.on || !p.pending_a || p.taken) return false;
  *start = p.pending_a;
  *stop = p.pending_b;
  p.taken = true;
  return true;
}

// A call that launched nothing (or whose launch failed) leaves no record; a
// call that launched several kernels is timed over its first one.
void prof_after(hipStream_t, int kernel_id) {
  Profiler &p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.pending_a || p.pending_kernel != kernel_id) return;
  if (p.taken && p.on) {
    p.recs.push_back({kernel_id, p.pending_a, p.pending_b});
  } else {
    p.pool.push_back(p.pending_a);
    p.pool.push_back(p.pending_b);
  }
  p.pending_a = p.pending_b = nullptr;
  p.pending_kernel = -1;
  p.taken = false;
}

DecodeWs decode_ws_layout(const mla_dims &d, int32_t batch, int32_t n_items, int32_t q_len) {
  DecodeWs w;
  size_t off = kStatusBytes;
  // items and seq info are contiguous: one copy of the plan's host block
  w.items = off;
  w.seqs = off + sizeof(WorkItem) * n_items;
  off = align_up(w.seqs + sizeof(SeqInfo) * batch, 256);
  w.q = off;
  const size_t hq = static_cast<size_t>(d.n_heads) * std::max(q_len, 1);
  off = align_up(off + sizeof(float) * batch * hq * (d.d_c + d.d_rope), 256);
  w.opart = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(std::max(n_items, 1)) * hq * d.d_c, 256);
  w.lse = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(std::max(n_items, 1)) * hq, 256);
  w.total = off;
  return w;
}

AppendWs append_ws_layout(const mla_dims &d, int32_t batch, int32_t n_new) {
  AppendWs w;
  size_t off = kStatusBytes;
  w.partial = off;
  const int64_t tokens = static_cast<int64_t>(batch) * n_new;
  if (append_fast_shape(d, static_cast<int32_t>(std::min<int64_t>(tokens, INT32_MAX)))) {
    w.ksplit = std::max(1, d.d_model / 512);
    off = align_up(off + sizeof(float) * w.ksplit * tokens * (d.d_c + d.d_rope), 256);
  }
  w.total = off;
  return w;
}

}  // namespace mla

// ======================================================================= ABI
extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

const char *mla_status_str(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_CAPACITY: return "MLA_ERR_CAPACITY";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_PLAN: return "MLA_ERR_PLAN";
  }
  return "MLA_ERR_UNKNOWN";
}

// ------------------------------------------------------------------ plan
mla_status mla_plan_create(const mla_dims *dims, const int32_t *host_lens, int32_t batch,
                           int32_t n_workers, mla_plan **out) {
  if (!out) return MLA_ERR_INVALID_ARG;
  *out = nullptr;
  if (!dims || !host_lens || batch < 1 || n_workers < 0) return MLA_ERR_INVALID_ARG;
  int64_t total = 0, maxlen = 0;
  int32_t nonempty = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (host_lens[b] < 0) return MLA_ERR_INVALID_ARG;
    total += host_lens[b];
    maxlen = std::max<int64_t>(maxlen, host_lens[b]);
    nonempty += host_lens[b] > 0;
  }
  int64_t min_tiles = 1;
  if (n_workers == 0) {
    min_tiles = 2;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return MLA_ERR_HIP;
    n_workers = cus;
  }

  // Smallest chunk C (a multiple of the tile) whose item count fits the
  // workers; with more non-empty sequences than workers, aim for whole waves.
  const int64_t T = kTile;
  auto count = [&](int64_t C) {
    int64_t n = 0;
    for (int32_t b = 0; b < batch; ++b) n += (host_lens[b] + C - 1) / C;
    return n;
  };
  int64_t target = n_workers;
  if (nonempty > target) target = (nonempty + n_workers - 1) / n_workers * n_workers;
  int64_t C = T;
  if (total > 0) {
    int64_t lo = 1, hi = (maxlen + T - 1) / T;  // in tiles
    while (lo < hi) {
      const int64_t mid = (lo + hi) / 2;
      if (count(mid * T) <= target) hi = mid; else lo = mid + 1;
    }
    C = std::max(lo, min_tiles) * T;
  }

  std::vector<WorkItem> items;
  std::vector<SeqInfo> seqs(batch);
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = host_lens[b];
    const int64_t n = (L + C - 1) / C;
    seqs[b].item_begin = static_cast<int32_t>(items.size());
    seqs[b].item_count = static_cast<int32_t>(n);
    seqs[b].len = static_cast<int32_t>(L);
    seqs[b].pad = 0;
    if (n == 0) continue;
    // n nearly equal chunks, boundaries on tile multiples
    const int64_t per = ((L + n - 1) / n + T - 1) / T * T;
    for (int64_t k = 0, t0 = 0; k < n; ++k) {
      const int64_t t1 = (k == n - 1) ? L : std::min(L, t0 + per);
      items.push_back({b, static_cast<int32_t>(t0), static_cast<int32_t>(t1), 0});
      t0 = t1;
    }
  }
  // Dropping trailing empty chunks can happen when per * n > L; remove them.
  std::vector<WorkItem> kept;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t begin = static_cast<int32_t>(kept.size());
    for (int32_t k = 0; k < seqs[b].item_count; ++k) {
      const WorkItem &it = items[seqs[b].item_begin + k];
      if (it.t1 > it.t0) kept.push_back(it);
    }
    seqs[b].item_begin = begin;
    seqs[b].item_count = static_cast<int32_t>(kept.size()) - begin;
  }

  mla_plan *p = new (std::nothrow) mla_plan();
  if (!p) return MLA_ERR_INVALID_ARG;
  p->batch = batch;
  p->n_items = static_cast<int32_t>(kept.size());
  p->chunk = static_cast<int32_t>(C);
  p->n_workers = n_workers;
  p->lens.assign(host_lens, host_lens + batch);
  static std::atomic<uint64_t> next_id{1};
  p->id = next_id.fetch_add(1);
  p->host_block_bytes = sizeof(WorkItem) * kept.size() + sizeof(SeqInfo) * batch;
  void *blk = nullptr;
  if (hipHostMalloc(&blk, p->host_block_bytes, hipHostMallocDefault) == hipSuccess && blk) {
    p->pinned = true;
  } else {
    (void)hipGetLastError();
    blk = std::malloc(p->host_block_bytes);
    p->pinned = false;
  }
  if (!blk) {
    delete p;
    return MLA_ERR_INVALID_ARG;
  }
  p->host_block = blk;
  std::memcpy(blk, kept.data(), sizeof(WorkItem) * kept.size());
  std::memcpy(static_cast<char *>(blk) + sizeof(WorkItem) * kept.size(), seqs.data(),
              sizeof(SeqInfo) * batch);
  *out = p;
  return MLA_OK;
}

void mla_plan_destroy(mla_plan *plan) {
  if (!plan) return;
  if (plan->host_block) {
    if (plan->pinned) (void)hipHostFree(plan->host_block); else std::free(plan->host_block);
  }
  delete plan;
}

int32_t mla_plan_num_items(const mla_plan *plan) { return plan ? plan->n_items : -1; }

mla_status mla_plan_item(const mla_plan *plan, int32_t k, int32_t *b, int32_t *t0, int32_t *t1) {
  if (!plan || !b || !t0 || !t1 || k < 0 || k >= plan->n_items) return MLA_ERR_INVALID_ARG;
  const WorkItem &it = plan->items()[k];
  *b = it.b;
  *t0 = it.t0;
  *t1 = it.t1;
  return MLA_OK;
}

// ------------------------------------------------------------- workspace
size_t mla_append_workspace_bytes(const mla_dims *dims, int32_t batch, int32_t n_new) {
  if (check_dims(dims, true, false) != MLA_OK || batch < 1 || n_new < 0) return 0;
  return append_ws_layout(*dims, batch, n_new).total;
}

size_t mla_decode_workspace_bytes(const mla_dims *dims, const mla_plan *plan) {
  if (check_dims(dims, false, true) != MLA_OK || !plan) return 0;
  return decode_ws_layout(*dims, plan->batch, plan->n_items).total;
}

size_t mla_workspace_bytes(const mla_dims *dims, const mla_plan *plan) {
  const size_t dec = mla_decode_workspace_bytes(dims, plan);
  if (dec == 0 || dims->d_model < 1) return dec;
  const size_t app = mla_append_workspace_bytes(dims, plan->batch, 1);
  return app > dec ? app : dec;
}

size_t mla_decode_multi_workspace_bytes(const mla_dims *dims, const mla_plan *plan, int32_t q_len) {
  if (check_dims(dims, false, true) != MLA_OK || !plan || q_len < 1 || q_len > kMaxQueryTokens) return 0;
  return decode_ws_layout(*dims, plan->batch, plan->n_items, q_len).total;
}

}  // extern "C"

// The device copy of a plan's work list lives in the workspace. A decode
// whose workspace already holds the copy of the same plan (made by an
// earlier call on it, and not overwritten since) skips the upload: one fewer
// copy per step. mla_workspace_init and the matrix-core append (whose
// partial products share that region) forget the workspace's entry.
namespace {
struct PlanCopies {
  std::mutex mu;
  std::unordered_map<const void *, uint64_t> last;
};
PlanCopies &plan_copies() {
  static PlanCopies *p = new PlanCopies();
  return *p;
}
}  // namespace

static bool plan_copy_current(const void *ws, uint64_t id) {
  PlanCopies &c = plan_copies();
  std::lock_guard<std::mutex> g(c.mu);
  auto it = c.last.find(ws);
  return it != c.last.end() && it->second == id;
}
static void plan_copy_record(const void *ws, uint64_t id) {
  PlanCopies &c = plan_copies();
  std::lock_guard<std::mutex> g(c.mu);
  c.last[ws] = id;
}
static void plan_copy_forget(const void *ws) {
  PlanCopies &c = plan_copies();
  std::lock_guard<std::mutex> g(c.mu);
  c.last.erase(ws);
}

extern "C" {

mla_status mla_workspace_init(void *ws, size_t ws_bytes, void *stream) {
  if (!ws || ws_bytes < kStatusBytes || !aligned16(ws)) return MLA_ERR_INVALID_ARG;
  plan_copy_forget(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  MLA_LAUNCH(s, K_INIT, launch_init(s, static_cast<int32_t *>(ws)));
  return MLA_OK;
}

mla_status mla_device_error(void *ws, void *stream, int32_t *code, int32_t reset) {
  if (!ws || !code || !aligned16(ws)) return MLA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  if (hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess) return MLA_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return MLA_ERR_HIP;
  *code = v;
  if (reset) {
    if (launch_init(s, static_cast<int32_t *>(ws)) != hipSuccess) return MLA_ERR_HIP;
  }
  return MLA_OK;
}

// ---------------------------------------------------------------- append
static mla_status validate_append(const mla_dims *dims, const mla_cache *cache, const void *h,
                                  int32_t n_new, const void *w_dkv, const void *w_kr,
                                  mla_dtype act, void *ws, size_t ws_bytes) {
  mla_status st = check_dims(dims, true, false);
  if (st != MLA_OK) return st;
  st = check_cache(*dims, cache);
  if (st != MLA_OK) return st;
  if (n_new < 0 || !h || !w_dkv || !w_kr || !ws || !aligned16(ws)) return MLA_ERR_INVALID_ARG;
  if (act != MLA_F32 && act != MLA_BF16) return MLA_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w_dkv) || !aligned16(w_kr)) return MLA_ERR_INVALID_ARG;
  if (ws_bytes < append_ws_layout(*dims, cache->batch, n_new).total) return MLA_ERR_WORKSPACE;
  // generic kernel keeps h and the output row in LDS
  const size_t shm = sizeof(float) * (static_cast<size_t>(dims->d_model) + dims->d_c + dims->d_rope + 4);
  if (!append_fast_path(*dims, cache->batch * n_new, act) && shm > 64 * 1024) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

static mla_status do_append(const mla_dims *dims, const mla_cache *cache, const void *h, int32_t n_new,
                            const void *w_dkv, const void *w_kr, mla_dtype act, void *ws,
                            hipStream_t s) {
  if (n_new == 0) return MLA_OK;
  int32_t *status = static_cast<int32_t *>(ws);
  if (append_fast_path(*dims, cache->batch * n_new, act)) {
    const AppendWs w = append_ws_layout(*dims, cache->batch, n_new);
    float *partial = reinterpret_cast<float *>(static_cast<char *>(ws) + w.partial);
    plan_copy_forget(ws);  // the partial products overwrite the plan's copy
    MLA_LAUNCH(s, K_APPEND_GEMM,
               launch_append_fast(s, *dims, *cache, h, n_new, w_dkv, w_kr, partial, w.ksplit, status));
    MLA_LAUNCH(s, K_APPEND_FINISH, launch_append_finish(s, *dims, *cache, n_new, partial, w.ksplit, status));
  } else {
    MLA_LAUNCH(s, K_APPEND_GENERIC,
               launch_append_generic(s, *dims, *cache, h, n_new, w_dkv, w_kr, act, status));
  }
  return MLA_OK;
}

mla_status mla_append(const mla_dims *dims, const mla_cache *cache, const void *h, int32_t n_new,
                      const void *w_dkv, const void *w_kr, mla_dtype act_w_dtype, void *ws,
                      size_t ws_bytes, void *stream) {
  mla_status st = validate_append(dims, cache, h, n_new, w_dkv, w_kr, act_w_dtype, ws, ws_bytes);
  if (st != MLA_OK) return st;
  return do_append(dims, cache, h, n_new, w_dkv, w_kr, act_w_dtype, ws, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- decode
static mla_status validate_decode(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan,
                                  const void *q_nope, const void *q_rope, const void *w_uk,
                                  const void *w_uv, mla_dtype qw, const void *o, mla_dtype od,
                                  void *ws, size_t ws_bytes, int32_t q_len = 1) {
  mla_status st = check_dims(dims, false, true);
  if (st != MLA_OK) return st;
  st = check_cache(*dims, cache);
  if (st != MLA_OK) return st;
  if (!plan || plan->batch != cache->batch) return MLA_ERR_INVALID_ARG;
  if (!q_nope || !q_rope || !w_uk || !w_uv || !o || !ws) return MLA_ERR_INVALID_ARG;
  if (qw != MLA_F32 && qw != MLA_BF16) return MLA_ERR_INVALID_ARG;
  if (od != MLA_F32 && od != MLA_BF16) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(w_uk) || !aligned16(w_uv) ||
      !aligned16(o) || !aligned16(ws))
    return MLA_ERR_INVALID_ARG;
  if (q_len < 1 || q_len > kMaxQueryTokens) return MLA_ERR_INVALID_ARG;
  if (ws_bytes < decode_ws_layout(*dims, plan->batch, plan->n_items, q_len).total) return MLA_ERR_WORKSPACE;
  if (!decode_fast_path(*dims, *cache, qw)) {
    if (q_len > 1) return MLA_ERR_UNSUPPORTED;
    if (dims->d_c > 1024) return MLA_ERR_UNSUPPORTED;
    if (sizeof(float) * (static_cast<size_t>(dims->d_c) + dims->d_rope + 260) > 64 * 1024 ||
        sizeof(float) * static_cast<size_t>(dims->d_nope) > 64 * 1024)
      return MLA_ERR_UNSUPPORTED;
  }
  return MLA_OK;
}

static mla_status do_decode(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan,
                            const void *q_nope, const void *q_rope, const int32_t *q_pos,
                            const void *w_uk, const void *w_uv, mla_dtype qw, void *o, mla_dtype od,
                            void *ws, hipStream_t s, int32_t q_len = 1) {
  const DecodeWs w = decode_ws_layout(*dims, plan->batch, plan->n_items, q_len);
  char *base = static_cast<char *>(ws);
  int32_t *status = reinterpret_cast<int32_t *>(base + w.status);
  WorkItem *items = reinterpret_cast<WorkItem *>(base + w.items);
  SeqInfo *seqs = reinterpret_cast<SeqInfo *>(base + w.seqs);
  if (!plan_copy_current(ws, plan->id)) {
    if (hipMemcpyAsync(items, plan->host_block, plan->host_block_bytes, hipMemcpyHostToDevice, s) != hipSuccess)
      return MLA_ERR_HIP;
    plan_copy_record(ws, plan->id);
  }
  float *opart = reinterpret_cast<float *>(base + w.opart);
  uint16_t *opart16 = reinterpret_cast<uint16_t *>(base + w.opart);
  float *lse = reinterpret_cast<float *>(base + w.lse);
  if (decode_fast_path(*dims, *cache, qw)) {
    uint16_t *q = reinterpret_cast<uint16_t *>(base + w.q);
    MLA_LAUNCH(s, K_ABSORB_FAST,
               launch_absorb_fast(s, *dims, plan->batch, q_len, q_nope, q_rope, q_pos, w_uk, seqs, q));
    MLA_LAUNCH(s, cache->latent_dtype == MLA_FP8_E4M3 ? K_DECODE_FP8 : K_DECODE_BF16,
               launch_decode_fast(s, *dims, *cache, q_len, plan->n_items, items, seqs, q, opart16, lse, status));
    MLA_LAUNCH(s, K_COMBINE_FAST,
               launch_combine_fast(s, *dims, *cache, q_len, seqs, opart16, lse, static_cast<const uint16_t *>(w_uv),
                                   o, od));
  } else {
    float *q = reinterpret_cast<float *>(base + w.q);
    MLA_LAUNCH(s, K_ABSORB_GENERIC,
               launch_absorb_generic(s, *dims, plan->batch, q_nope, q_rope, q_pos, w_uk, qw, seqs, q));
    MLA_LAUNCH(s, K_DECODE_GENERIC,
               launch_decode_generic(s, *dims, *cache, plan->n_items, items, seqs, q, opart, lse, status));
    MLA_LAUNCH(s, K_COMBINE_GENERIC,
               launch_combine_generic(s, *dims, *cache, seqs, opart, lse, w_uv, qw, o, od));
  }
  return MLA_OK;
}

mla_status mla_decode(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan,
                      const void *q_nope, const void *q_rope, const int32_t *q_pos, const void *w_uk,
                      const void *w_uv, mla_dtype q_w_dtype, void *o, mla_dtype o_dtype, void *ws,
                      size_t ws_bytes, void *stream) {
  mla_status st = validate_decode(dims, cache, plan, q_nope, q_rope, w_uk, w_uv, q_w_dtype, o, o_dtype,
                                  ws, ws_bytes);
  if (st != MLA_OK) return st;
  return do_decode(dims, cache, plan, q_nope, q_rope, q_pos, w_uk, w_uv, q_w_dtype, o, o_dtype, ws,
                   static_cast<hipStream_t>(stream));
}

mla_status mla_decode_multi(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan, int32_t q_len,
                            const void *q_nope, const void *q_rope, const int32_t *q_pos, const void *w_uk,
                            const void *w_uv, mla_dtype q_w_dtype, void *o, mla_dtype o_dtype, void *ws,
                            size_t ws_bytes, void *stream) {
  mla_status st = validate_decode(dims, cache, plan, q_nope, q_rope, w_uk, w_uv, q_w_dtype, o, o_dtype,
                                  ws, ws_bytes, q_len);
  if (st != MLA_OK) return st;
  return do_decode(dims, cache, plan, q_nope, q_rope, q_pos, w_uk, w_uv, q_w_dtype, o, o_dtype, ws,
                   static_cast<hipStream_t>(stream), q_len);
}

mla_status mla_append_decode(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan,
                             const void *h, int32_t n_new, const void *w_dkv, const void *w_kr,
                             const void *q_nope, const void *q_rope, const int32_t *q_pos,
                             const void *w_uk, const void *w_uv, mla_dtype act_w_dtype, void *o,
                             mla_dtype o_dtype, void *ws, size_t ws_bytes, void *stream) {
  mla_status st = validate_append(dims, cache, h, n_new, w_dkv, w_kr, act_w_dtype, ws, ws_bytes);
  if (st != MLA_OK) return st;
  st = validate_decode(dims, cache, plan, q_nope, q_rope, w_uk, w_uv, act_w_dtype, o, o_dtype, ws,
                       ws_bytes);
  if (st != MLA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = do_append(dims, cache, h, n_new, w_dkv, w_kr, act_w_dtype, ws, s);
  if (st != MLA_OK) return st;
  return do_decode(dims, cache, plan, q_nope, q_rope, q_pos, w_uk, w_uv, act_w_dtype, o, o_dtype, ws, s);
}

// ------------------------------------------------------------- profiling
mla_status mla_prof_begin(int32_t max_records) {
  if (max_records < 1) return MLA_ERR_INVALID_ARG;
  Profiler &p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  for (auto &r : p.recs) {
    p.pool.push_back(r.a);
    p.pool.push_back(r.b);
  }
  p.recs.clear();
  p.max_records = max_records;
  p.on = true;
  return MLA_OK;
}

mla_status mla_prof_end(double *ms, int32_t *count, int32_t n) {
  Profiler &p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.on = false;
  if (ms && count) {
    for (int32_t k = 0; k < n; ++k) {
      ms[k] = 0.0;
      count[k] = 0;
    }
  }
  mla_status st = MLA_OK;
  for (auto &r : p.recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) st = MLA_ERR_HIP;
    float t = 0.0f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) st = MLA_ERR_HIP;
    if (ms && count && r.kernel < n) {
      ms[r.kernel] += t;
      count[r.kernel] += 1;
    }
    p.pool.push_back(r.a);
    p.pool.push_back(r.b);
  }
  p.recs.clear();
  return st;
}

const char *mla_prof_kernel_name(int32_t id) {
  return (id >= 0 && id < K_COUNT) ? kKernelNames[id] : "unknown";
}

int32_t mla_prof_num_kernels(void) { return K_COUNT; }

mla_status mla_calib_copy(void *dst, const void *src, size_t n_bytes, void *stream) {
  if (!dst || !src || (n_bytes & 15) || !aligned16(dst) || !aligned16(src)) return MLA_ERR_INVALID_ARG;
  if (n_bytes == 0) return MLA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  MLA_LAUNCH(s, K_COPY, launch_copy(s, dst, src, n_bytes / 16));
  return MLA_OK;
}

mla_status mla_calib_read(const void *src, size_t n_bytes, uint32_t *sink, void *stream) {
  if (!src || !sink || (n_bytes & 15) || !aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3))
    return MLA_ERR_INVALID_ARG;
  if (n_bytes == 0) return MLA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  MLA_LAUNCH(s, K_READ, launch_read(s, src, n_bytes / 16, sink));
  return MLA_OK;
}

}  // extern "C"
