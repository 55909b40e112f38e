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
    "read",           "merge_gemm",     "absorb_merged",  "out_merged",
    "combine_emit"};

#define MLA_LAUNCH(stream, kid, call)          \
  do {                                         \
    prof_before((stream), (kid));              \
    hipError_t e_ = (call);                    \
    prof_after((stream), (kid));               \
    if (e_ != hipSuccess) return MLA_ERR_HIP;  \
  } while (0)

}  // namespace

namespace mla {

void prof_before(hipStream_t s, int kernel_id) {
  Profiler &p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.on || static_cast<int>(p.recs.size()) >= p.max_records) return;
  // start each recorded kernel on an idle stream: a dispatch queued behind
  // running work can take its start time before that work has ended
  (void)hipStreamSynchronize(s);
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

DecodeWs decode_ws_layout(const mla_dims &d, const mla_plan &plan, int32_t q_len, bool fast) {
  DecodeWs w;
  const int32_t batch = plan.batch, n_items = plan.n_items;
  const size_t eb = fast ? 2 : sizeof(float);  // query and partial element size
  const size_t hq = static_cast<size_t>(d.n_heads) * std::max(q_len, 1);
  const size_t ni = static_cast<size_t>(std::max(n_items, 1));
  size_t off = kStatusBytes;
  w.q = off;
  off = align_up(off + eb * batch * hq * (d.d_c + d.d_rope), 256);
  w.opart = off;
  off = align_up(off + eb * ni * hq * d.d_c, 256);
  w.lse = off;
  off = align_up(off + sizeof(float) * ni * hq, 256);
  w.items = off;
  w.seqs = off + sizeof(WorkItem) * n_items;
  w.ranges = w.seqs + sizeof(SeqInfo) * batch;
  off = align_up(off + plan.host_block_bytes, 256);
  w.total = off;
  return w;
}

AppendWs append_ws_layout(const mla_dims &d, int32_t batch, int32_t n_new) {
  AppendWs w;
  size_t off = kStatusBytes;
  w.partial = off;
  const int64_t tokens = static_cast<int64_t>(batch) * n_new;
  if (append_fast_shape(d, static_cast<int32_t>(std::min<int64_t>(tokens, INT32_MAX)))) {
    w.ksplit = append_fast_ksplit(d);
    off = align_up(off + sizeof(float) * w.ksplit * tokens * (d.d_c + d.d_rope), 256);
  }
  w.total = off;
  return w;
}

// ------------------------------------------------------------- planning
// A workgroup walks a range of consecutive items; its time is about its
// tiles plus a fixed cost per item, counted here in tiles: at an item's
// start its first copies arrive before any product can start, and at its
// end the last tiles' products run with no copy under them, then the 128 KB
// partial is written. Measured per workgroup on MI355X (the time of every
// workgroup against its tiles and items, least squares): 2.4 us per tile
// and 11.5 us per item with a bf16 cache, 2.3 and 13.3 with an fp8 one,
// about five to six tiles.
constexpr int64_t kItemCostTiles = 6;

struct Cut {
  std::vector<WorkItem> items;
  std::vector<int32_t> ranges;  // the first item of every range
};

// Walks the sequences' tiles in order and fills each range up to cost cap
// (tiles + kItemCostTiles per item); a piece has at least min_piece tiles
// unless its sequence has fewer left. Returns the number of ranges, or
// stops early once it passes limit; with out, records the items and the
// first item of every range.
int64_t cut_ranges(const int32_t *lens, int32_t batch, int64_t cap, int64_t min_piece, int64_t limit, Cut *out) {
  const int64_t T = kTile;
  int64_t n = 0, rem = 0;  // ranges so far, cost left in the current one
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t tiles = (static_cast<int64_t>(lens[b]) + T - 1) / T;
    for (int64_t t = 0; t < tiles;) {
      const int64_t left = tiles - t;
      int64_t take = std::min(left, rem - kItemCostTiles);
      if (take < std::min(left, min_piece)) {
        // a new range (cap >= kItemCostTiles + min_piece: take >= 1)
        if (++n > limit && !out) return n;
        if (out) out->ranges.push_back(static_cast<int32_t>(out->items.size()));
        rem = cap;
        take = std::min(left, rem - kItemCostTiles);
      }
      if (out)
        out->items.push_back({b, static_cast<int32_t>(t * T),
                              static_cast<int32_t>(std::min<int64_t>((t + take) * T, lens[b])), 0});
      rem -= kItemCostTiles + take;
      t += take;
    }
  }
  return n;
}

size_t plan_block_bytes(int32_t n_items, int32_t batch, int32_t n_ranges) {
  return sizeof(WorkItem) * n_items + sizeof(SeqInfo) * batch + align_up(sizeof(int32_t) * (n_ranges + 1), 16);
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
    case MLA_ERR_RANGE: return "MLA_ERR_RANGE";
  }
  return "MLA_ERR_UNKNOWN";
}

// ------------------------------------------------------------------ plan
mla_status mla_plan_create(const mla_dims *dims, const int32_t *host_lens, int32_t batch,
                           int32_t n_workers, mla_plan **out) {
  return mla_plan_create_multi(dims, host_lens, batch, 1, n_workers, out);
}

mla_status mla_plan_create_multi(const mla_dims *dims, const int32_t *host_lens, int32_t batch, int32_t q_len,
                                 int32_t n_workers, mla_plan **out) {
  if (!out) return MLA_ERR_INVALID_ARG;
  *out = nullptr;
  if (!dims || !host_lens || batch < 1 || n_workers < 0) return MLA_ERR_INVALID_ARG;
  if (q_len < 1 || q_len > kMaxQueryTokens || dims->n_heads < 1) return MLA_ERR_INVALID_ARG;
  // each range runs as one workgroup per 128 of the q_len * H (token, head)
  // pairs (the matrix-core kernels' head blocks)
  const int32_t blocks = static_cast<int32_t>((static_cast<int64_t>(q_len) * dims->n_heads + 127) / 128);
  int64_t total = 0, maxlen = 0;
  int32_t nonempty = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (host_lens[b] < 0) return MLA_ERR_INVALID_ARG;
    total += host_lens[b];
    maxlen = std::max<int64_t>(maxlen, host_lens[b]);
    nonempty += host_lens[b] > 0;
  }
  int64_t min_piece = 1;
  if (n_workers == 0) {
    min_piece = 2;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return MLA_ERR_HIP;
    n_workers = cus;
  }
  (void)maxlen;
  n_workers = std::max(1, n_workers / blocks);

  // The smallest range cost whose cut needs at most n_workers ranges (the
  // cut is monotone in the cost: a larger one never needs more ranges).
  Cut cut;
  if (total > 0) {
    const int64_t T = kTile;
    int64_t lo = kItemCostTiles + min_piece;
    int64_t hi = (total + T * nonempty) / T + kItemCostTiles * nonempty + min_piece;  // one range holds it all
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (cut_ranges(host_lens, batch, mid, min_piece, n_workers, nullptr) <= n_workers) hi = mid; else lo = mid + 1;
    }
    cut_ranges(host_lens, batch, lo, min_piece, n_workers, &cut);
  }
  cut.ranges.push_back(static_cast<int32_t>(cut.items.size()));  // the end of the last range
  const int32_t n_ranges = static_cast<int32_t>(cut.ranges.size()) - 1;

  std::vector<SeqInfo> seqs(batch);
  for (int32_t b = 0; b < batch; ++b) seqs[b] = {0, 0, host_lens[b], 0};
  for (size_t k = 0; k < cut.items.size(); ++k) {
    SeqInfo &si = seqs[cut.items[k].b];
    if (si.item_count++ == 0) si.item_begin = static_cast<int32_t>(k);
  }

  mla_plan *p = new (std::nothrow) mla_plan();
  if (!p) return MLA_ERR_INVALID_ARG;
  p->batch = batch;
  p->n_items = static_cast<int32_t>(cut.items.size());
  p->n_ranges = n_ranges;
  p->n_workers = n_workers;
  p->lens.assign(host_lens, host_lens + batch);
  p->host_block_bytes = plan_block_bytes(p->n_items, batch, n_ranges);
  // pinned and mapped: the first kernel of a decode reads it directly when
  // the workspace's copy does not match. Without a device (host-side
  // planning, inspection) the block is ordinary memory and decodes refuse
  // the plan.
  void *blk = nullptr, *dev = nullptr;
  if (hipHostMalloc(&blk, p->host_block_bytes, hipHostMallocMapped) == hipSuccess && blk) {
    p->pinned = true;
    if (hipHostGetDevicePointer(&dev, blk, 0) != hipSuccess) dev = nullptr;
  } else {
    blk = std::malloc(p->host_block_bytes);
  }
  (void)hipGetLastError();
  if (!blk) {
    delete p;
    return MLA_ERR_INVALID_ARG;
  }
  p->host_block = blk;
  p->host_dev = dev;
  std::memset(blk, 0, p->host_block_bytes);
  std::memcpy(blk, cut.items.data(), sizeof(WorkItem) * cut.items.size());
  std::memcpy(static_cast<char *>(blk) + sizeof(WorkItem) * cut.items.size(), seqs.data(), sizeof(SeqInfo) * batch);
  std::memcpy(static_cast<char *>(blk) + sizeof(WorkItem) * cut.items.size() + sizeof(SeqInfo) * batch,
              cut.ranges.data(), sizeof(int32_t) * (n_ranges + 1));
  const uint32_t *words = static_cast<const uint32_t *>(blk);
  uint64_t h = 0;
  for (size_t i = 0; i < p->host_block_bytes / 16; ++i)
    h += plan_chunk_hash(static_cast<uint32_t>(i), words[4 * i], words[4 * i + 1], words[4 * i + 2], words[4 * i + 3]);
  p->hash = h;
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

int32_t mla_plan_num_ranges(const mla_plan *plan) { return plan ? plan->n_ranges : -1; }

mla_status mla_plan_range(const mla_plan *plan, int32_t j, int32_t *item_begin, int32_t *item_end) {
  if (!plan || !item_begin || !item_end || j < 0 || j >= plan->n_ranges) return MLA_ERR_INVALID_ARG;
  const int32_t *r = reinterpret_cast<const int32_t *>(plan->seqs() + plan->batch);
  *item_begin = r[j];
  *item_end = r[j + 1];
  return MLA_OK;
}

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
  // sized for the generic path's fp32 arrays, so one size serves either path
  return decode_ws_layout(*dims, *plan, 1, false).total;
}

size_t mla_workspace_bytes(const mla_dims *dims, const mla_plan *plan) {
  const size_t dec = mla_decode_workspace_bytes(dims, plan);
  if (dec == 0 || dims->d_model < 1) return dec;
  const size_t app = mla_append_workspace_bytes(dims, plan->batch, 1);
  return app > dec ? app : dec;
}

size_t mla_decode_multi_workspace_bytes(const mla_dims *dims, const mla_plan *plan, int32_t q_len) {
  if (check_dims(dims, false, true) != MLA_OK || !plan || q_len < 1 || q_len > kMaxQueryTokens) return 0;
  return decode_ws_layout(*dims, *plan, q_len, false).total;
}

}  // extern "C"

extern "C" {

mla_status mla_workspace_init(void *ws, size_t ws_bytes, void *stream) {
  if (!ws || ws_bytes < kStatusBytes || !aligned16(ws)) return MLA_ERR_INVALID_ARG;
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
}  // extern "C"

namespace mla {

mla_status decode_check_args(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan,
                             const void *q_nope, const void *q_rope, const void *w_uk, const void *w_uv,
                             mla_dtype qw, const void *o, mla_dtype od, const void *ws, size_t ws_bytes,
                             int32_t q_len) {
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
  if (ws_bytes < decode_ws_layout(*dims, *plan, q_len, false).total) return MLA_ERR_WORKSPACE;
  if (!decode_fast_path(*dims, *cache, qw)) {
    if (q_len > 1) return MLA_ERR_UNSUPPORTED;
    if (dims->d_c > 1024) return MLA_ERR_UNSUPPORTED;
    if (sizeof(float) * (static_cast<size_t>(dims->d_c) + dims->d_rope + 260) > 64 * 1024 ||
        sizeof(float) * static_cast<size_t>(dims->d_nope) > 64 * 1024)
      return MLA_ERR_UNSUPPORTED;
  }
  if (!plan->host_dev) return MLA_ERR_HIP;  // made where no pinned, device-mapped memory was available
  return MLA_OK;
}

size_t decode_compact_bytes(const mla_dims &d, const mla_cache &c, const mla_plan &plan, mla_dtype qw) {
  return decode_ws_layout(d, plan, 1, decode_fast_path(d, c, qw)).total;
}

mla_status decode_launch(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan, const void *q_nope,
                         const void *q_rope, const int32_t *q_pos, const void *w_uk, const void *w_uv, mla_dtype qw,
                         void *o, mla_dtype od, void *ws, hipStream_t s, int32_t q_len, bool compact,
                         bool clear_status) {
  const mla_dims dd = with_default_scale(*dims);
  dims = &dd;
  const bool fast = decode_fast_path(*dims, *cache, qw);
  const DecodeWs w = decode_ws_layout(*dims, *plan, q_len, compact && fast);
  char *base = static_cast<char *>(ws);
  int32_t *status = reinterpret_cast<int32_t *>(base + w.status);
  WorkItem *items = reinterpret_cast<WorkItem *>(base + w.items);
  SeqInfo *seqs = reinterpret_cast<SeqInfo *>(base + w.seqs);
  const int32_t *ranges = reinterpret_cast<const int32_t *>(base + w.ranges);
  // the absorb kernel checks this copy against the plan (and refetches it)
  // before the kernels after it read it
  const PlanRef pr{plan->host_dev, items, static_cast<int32_t>(plan->host_block_bytes / 16), plan->hash};
  float *opart = reinterpret_cast<float *>(base + w.opart);
  uint16_t *opart16 = reinterpret_cast<uint16_t *>(base + w.opart);
  float *lse = reinterpret_cast<float *>(base + w.lse);
  if (clear_status) MLA_LAUNCH(s, K_INIT, launch_init(s, status));
  if (fast) {
    uint16_t *q = reinterpret_cast<uint16_t *>(base + w.q);
    MLA_LAUNCH(s, K_ABSORB_FAST,
               launch_absorb_fast(s, *dims, plan->batch, q_len, q_nope, q_rope, q_pos, w_uk, cache->seq_len, q, pr,
                                  status));
    MLA_LAUNCH(s, cache->latent_dtype == MLA_FP8_E4M3 ? K_DECODE_FP8 : K_DECODE_BF16,
               launch_decode_fast(s, *dims, *cache, q_len, plan->n_items, plan->n_ranges, ranges, items, seqs, q, opart16, lse,
                                  status));
    MLA_LAUNCH(s, K_COMBINE_FAST,
               launch_combine_fast(s, *dims, *cache, q_len, plan->n_items, seqs, opart16, lse,
                                   static_cast<const uint16_t *>(w_uv), o, od, status));
  } else {
    float *q = reinterpret_cast<float *>(base + w.q);
    MLA_LAUNCH(s, K_ABSORB_GENERIC,
               launch_absorb_generic(s, *dims, plan->batch, q_nope, q_rope, q_pos, w_uk, qw, cache->seq_len, q, pr,
                                     status));
    MLA_LAUNCH(s, K_DECODE_GENERIC,
               launch_decode_generic(s, *dims, *cache, plan->n_items, items, seqs, q, opart, lse, status));
    MLA_LAUNCH(s, K_COMBINE_GENERIC,
               launch_combine_generic(s, *dims, *cache, plan->n_items, seqs, opart, lse, w_uv, qw, o, od, status));
  }
  return MLA_OK;
}

}  // namespace mla

extern "C" {

mla_status mla_decode(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan,
                      const void *q_nope, const void *q_rope, const int32_t *q_pos, const void *w_uk,
                      const void *w_uv, mla_dtype q_w_dtype, void *o, mla_dtype o_dtype, void *ws,
                      size_t ws_bytes, void *stream) {
  mla_status st = decode_check_args(dims, cache, plan, q_nope, q_rope, w_uk, w_uv, q_w_dtype, o, o_dtype, ws,
                                    ws_bytes, 1);
  if (st != MLA_OK) return st;
  return decode_launch(dims, cache, plan, q_nope, q_rope, q_pos, w_uk, w_uv, q_w_dtype, o, o_dtype, ws,
                       static_cast<hipStream_t>(stream), 1, false, false);
}

mla_status mla_decode_multi(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan, int32_t q_len,
                            const void *q_nope, const void *q_rope, const int32_t *q_pos, const void *w_uk,
                            const void *w_uv, mla_dtype q_w_dtype, void *o, mla_dtype o_dtype, void *ws,
                            size_t ws_bytes, void *stream) {
  mla_status st = decode_check_args(dims, cache, plan, q_nope, q_rope, w_uk, w_uv, q_w_dtype, o, o_dtype, ws,
                                    ws_bytes, q_len);
  if (st != MLA_OK) return st;
  return decode_launch(dims, cache, plan, q_nope, q_rope, q_pos, w_uk, w_uv, q_w_dtype, o, o_dtype, ws,
                       static_cast<hipStream_t>(stream), q_len, false, false);
}

mla_status mla_append_decode(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan,
                             const void *h, int32_t n_new, const void *w_dkv, const void *w_kr,
                             const void *q_nope, const void *q_rope, const int32_t *q_pos,
                             const void *w_uk, const void *w_uv, mla_dtype act_w_dtype, void *o,
                             mla_dtype o_dtype, void *ws, size_t ws_bytes, void *stream) {
  mla_status st = validate_append(dims, cache, h, n_new, w_dkv, w_kr, act_w_dtype, ws, ws_bytes);
  if (st != MLA_OK) return st;
  st = decode_check_args(dims, cache, plan, q_nope, q_rope, w_uk, w_uv, act_w_dtype, o, o_dtype, ws, ws_bytes, 1);
  if (st != MLA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = do_append(dims, cache, h, n_new, w_dkv, w_kr, act_w_dtype, ws, s);
  if (st != MLA_OK) return st;
  return decode_launch(dims, cache, plan, q_nope, q_rope, q_pos, w_uk, w_uv, act_w_dtype, o, o_dtype, ws, s, 1, false,
                       false);
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

// ------------------------------------------- precomputed absorbed weights

namespace {

struct MergedWs {
  mla::DecodeWs dec;
  size_t ohat = 0, part = 0, total = 0;
};

// The decode workspace, then o^ (fp32 [B, H d_c], or bf16 hi and lo planes
// of the same total size), then the K-split partials of the output product.
MergedWs merged_ws_layout(const mla_dims &d, const mla_plan &plan, int32_t d_out) {
  MergedWs w;
  const int32_t batch = plan.batch;
  w.dec = mla::decode_ws_layout(d, plan, 1, false);
  const int64_t K = static_cast<int64_t>(d.n_heads) * d.d_c;
  size_t off = w.dec.total;
  w.ohat = off;
  off = align_up(off + sizeof(float) * batch * K, 256);
  w.part = off;
  off = align_up(off + sizeof(float) * mla::merged::out_splits(K) * batch * d_out, 256);
  w.total = off;
  return w;
}

bool merged_fast_path(const mla_dims &d, const mla_cache &c, mla_dtype wt, int32_t d_x, int32_t d_out) {
  // (each of the query product's four waves takes d_x / 4 inputs, an even
  // number of 64-wide steps)
  return mla::decode_fast_path(d, c, wt) && d_x % 512 == 0 && d_out % 128 == 0;
}

mla_status check_weight_args(const mla_dims *dims, int32_t n, const void *p0, const void *p1, mla_dtype wt,
                             const void *out) {
  mla_status st = check_dims(dims, false, true);
  if (st != MLA_OK) return st;
  if (n < 1 || !p0 || !p1 || !out) return MLA_ERR_INVALID_ARG;
  if (wt != MLA_F32 && wt != MLA_BF16) return MLA_ERR_INVALID_ARG;
  if (!aligned16(p0) || !aligned16(p1) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_merge_query_weight(const mla_dims *dims, int32_t d_x, const void *w_q, const void *w_uk,
                                  mla_dtype w_dtype, void *a, void *stream) {
  mla_status st = check_weight_args(dims, d_x, w_q, w_uk, w_dtype, a);
  if (st != MLA_OK) return st;
  const mla_dims &d = *dims;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // per head: A[c][x] = sum_n W_UK[n][c] W_Q[n][x] (A as a weight of H d_c
  // rows and d_x columns: fragment-tiled when the shape allows)
  const int64_t dn = d.d_nope, dc = d.d_c, dx = d_x;
  const int64_t tk = merged::tiled(static_cast<int64_t>(d.n_heads) * dc, dx) ? dx : 0;
  MLA_LAUNCH(s, K_MERGE_GEMM,
             launch_merge_gemm(s, d.n_heads, d.d_c, d_x, d.d_nope, w_uk, dn * dc, dc, 1, w_q, dn * dx, dx, 1, w_dtype,
                               a, dc * dx, dx, 1, w_dtype, tk));
  return MLA_OK;
}

mla_status mla_merge_output_weight(const mla_dims *dims, int32_t d_out, const void *w_o, const void *w_uv,
                                   mla_dtype w_dtype, void *bm, void *stream) {
  mla_status st = check_weight_args(dims, d_out, w_o, w_uv, w_dtype, bm);
  if (st != MLA_OK) return st;
  const mla_dims &d = *dims;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // per head i: Bm[o][i d_c + c] = sum_v W_O[o][i d_v + v] W_UV[i][v][c]
  // (fragment-tiled when the shape allows)
  const int64_t H = d.n_heads, dv = d.d_v, dc = d.d_c;
  const int64_t tk = merged::tiled(d_out, H * dc) ? H * dc : 0;
  MLA_LAUNCH(s, K_MERGE_GEMM,
             launch_merge_gemm(s, d.n_heads, d_out, d.d_c, d.d_v, w_o, dv, 1, H * dv, w_uv, dv * dc, dc, 1, w_dtype,
                               bm, dc, H * dc, 1, w_dtype, tk));
  return MLA_OK;
}

size_t mla_decode_merged_workspace_bytes(const mla_dims *dims, const mla_plan *plan, int32_t d_out) {
  if (check_dims(dims, false, true) != MLA_OK || !plan || d_out < 1) return 0;
  return merged_ws_layout(*dims, *plan, d_out).total;
}

mla_status mla_decode_merged(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan, int32_t d_x,
                             const void *x, const void *q_rope, const int32_t *q_pos, const void *a, int32_t d_out,
                             const void *bm, mla_dtype w_dtype, void *y, mla_dtype y_dtype, void *ws,
                             size_t ws_bytes, void *stream) {
  mla_status st = check_dims(dims, false, true);
  if (st != MLA_OK) return st;
  st = check_cache(*dims, cache);
  if (st != MLA_OK) return st;
  if (!plan || plan->batch != cache->batch) return MLA_ERR_INVALID_ARG;
  if (!x || !q_rope || !a || !bm || !y || !ws || d_x < 1 || d_out < 1) return MLA_ERR_INVALID_ARG;
  if (w_dtype != MLA_F32 && w_dtype != MLA_BF16) return MLA_ERR_INVALID_ARG;
  if (y_dtype != MLA_F32 && y_dtype != MLA_BF16) return MLA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(q_rope) || !aligned16(a) || !aligned16(bm) || !aligned16(y) || !aligned16(ws))
    return MLA_ERR_INVALID_ARG;
  const mla_dims d = with_default_scale(*dims);
  const MergedWs w = merged_ws_layout(d, *plan, d_out);
  if (ws_bytes < w.total) return MLA_ERR_WORKSPACE;
  const bool fast = merged_fast_path(d, *cache, w_dtype, d_x, d_out);
  if (!fast) {
    if (d.d_c > 1024 || sizeof(float) * (static_cast<size_t>(d.d_c) + d.d_rope + 260) > 64 * 1024 ||
        sizeof(float) * static_cast<size_t>(d_x) > 64 * 1024)
      return MLA_ERR_UNSUPPORTED;
  }
  if (!plan->host_dev) return MLA_ERR_HIP;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char *base = static_cast<char *>(ws);
  int32_t *status = reinterpret_cast<int32_t *>(base + w.dec.status);
  WorkItem *items = reinterpret_cast<WorkItem *>(base + w.dec.items);
  SeqInfo *seqs = reinterpret_cast<SeqInfo *>(base + w.dec.seqs);
  const int32_t *ranges = reinterpret_cast<const int32_t *>(base + w.dec.ranges);
  const PlanRef pr{plan->host_dev, items, static_cast<int32_t>(plan->host_block_bytes / 16), plan->hash};
  float *lse = reinterpret_cast<float *>(base + w.dec.lse);
  const int64_t K = static_cast<int64_t>(d.n_heads) * d.d_c;
  if (fast) {
    uint16_t *q = reinterpret_cast<uint16_t *>(base + w.dec.q);
    uint16_t *opart = reinterpret_cast<uint16_t *>(base + w.dec.opart);
    uint16_t *ohat_hi = reinterpret_cast<uint16_t *>(base + w.ohat);
    uint16_t *ohat_lo = ohat_hi + static_cast<size_t>(plan->batch) * K;
    float *part = reinterpret_cast<float *>(base + w.part);
    MLA_LAUNCH(s, K_ABSORB_MERGED,
               launch_absorb_merged_fast(s, d, plan->batch, d_x, x, q_rope, q_pos, a, cache->seq_len, q, pr, status));
    MLA_LAUNCH(s, cache->latent_dtype == MLA_FP8_E4M3 ? K_DECODE_FP8 : K_DECODE_BF16,
               launch_decode_fast(s, d, *cache, 1, plan->n_items, plan->n_ranges, ranges, items, seqs, q, opart, lse, status));
    MLA_LAUNCH(s, K_COMBINE_EMIT,
               launch_combine_fast_emit(s, d, *cache, plan->n_items, seqs, opart, lse, ohat_hi, ohat_lo, status));
    MLA_LAUNCH(s, K_OUT_MERGED,
               launch_out_merged_fast(s, plan->batch, d_out, K, bm, ohat_hi, ohat_lo, part, y, y_dtype == MLA_BF16));
  } else {
    float *q = reinterpret_cast<float *>(base + w.dec.q);
    float *opart = reinterpret_cast<float *>(base + w.dec.opart);
    float *ohat = reinterpret_cast<float *>(base + w.ohat);
    MLA_LAUNCH(s, K_ABSORB_MERGED,
               launch_absorb_merged_generic(s, d, plan->batch, d_x, x, q_rope, q_pos, a, w_dtype, cache->seq_len, q,
                                            pr));
    MLA_LAUNCH(s, K_DECODE_GENERIC,
               launch_decode_generic(s, d, *cache, plan->n_items, items, seqs, q, opart, lse, status));
    MLA_LAUNCH(s, K_COMBINE_EMIT,
               launch_combine_generic_emit(s, d, *cache, plan->n_items, seqs, opart, lse, ohat, status));
    MLA_LAUNCH(s, K_OUT_MERGED, launch_out_merged_generic(s, plan->batch, d_out, K, bm, w_dtype, ohat, y, y_dtype));
  }
  return MLA_OK;
}

}  // extern "C"
