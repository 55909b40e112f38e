/*
 * mla.h — C ABI of libmla: Multi-head Latent Attention (MLA) decode with
 * weight absorption, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources cited by page title and section):
 *
 *  - The cache holds, per token, only a compressed latent c_t = W_DKV h_t
 *    (width d_c) and a small decoupled rotary key k^R_t (width d_rope),
 *    shared by all heads; per-head keys and values are the up-projections
 *    W_UK c_t and W_UV c_t.  ("02 — Multi-Latent Attention (MLA)", sections
 *    "La compresión de MLA" and "Truco de codificación posicional";
 *    "Multi-head Latent Attention (MLA) și arhitectura DeepSeekMoE", opening
 *    paragraph: (d_c + d_hR) elements per token and layer.)
 *  - The score of a cached token is a content term plus a positional term
 *    ("DeepSeek MLA" card, section on the problem RoPE causes).
 *  - Weight absorption: the up-projections fold into the query side (W_UK)
 *    and the output side (W_UV), so attention runs directly on the latent
 *    and full per-head K/V are never formed ("02 — Multi-Latent Attention
 *    (MLA)", "Coste de cómputo"; "Atención latente de múltiples cabezas",
 *    "Información técnica").
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless the comment says "host".
 *  - Every call is asynchronous on the given stream; MLA_OK means the work
 *    was validated and launched. The caller keeps all buffers alive until
 *    the stream has completed the work.
 *  - Arguments are validated on the host before any HIP call; a rejected
 *    call launches nothing and returns its status synchronously.
 *  - Errors that only the device can see (an append past a sequence's
 *    capacity, a seq_len that differs from the plan) are recorded, first
 *    error wins, in a status word at the start of the workspace; read it with
 *    mla_device_error(). The offending sequence's rows are not written and
 *    its output is set to zero.
 *  - The library never allocates device memory. The caller owns the cache,
 *    weights, activations, outputs and workspace; the library owns only the
 *    host-side plan (pinned host memory) between mla_plan_create() and
 *    mla_plan_destroy().
 *  - No C++ exception crosses this boundary.
 *  - Calls on different streams may run concurrently if they use different
 *    workspaces.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 1

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null pointer, bad size or dtype, misalignment */
  MLA_ERR_UNSUPPORTED = 2, /* a valid combination no kernel implements      */
  MLA_ERR_CAPACITY = 3,    /* device: append would pass seq_cap             */
  MLA_ERR_HIP = 4,         /* a HIP runtime call or launch failed           */
  MLA_ERR_WORKSPACE = 5,   /* ws_bytes below the required size              */
  MLA_ERR_PLAN = 6         /* device: seq_len differs from the plan         */
} mla_status;

typedef enum {
  MLA_F32 = 0,
  MLA_BF16 = 1,
  MLA_FP8_E4M3 = 2 /* OCP E4M3FN: bias 7, max 448, no inf, NaN 0x7F/0xFF */
} mla_dtype;

/* Shapes of one MLA layer. softmax_scale multiplies the whole
 * (d_nope + d_rope)-wide score; rope_base is the RoPE base (10000 in the
 * workloads). RoPE pairs are interleaved, (2j, 2j+1), at frequency
 * rope_base^(-2j/d_rope), positions absolute from 0. d_model is used only by
 * mla_append. d_rope must be even. */
typedef struct {
  int32_t n_heads, d_c, d_rope, d_nope, d_v, d_model;
  float softmax_scale, rope_base;
} mla_dims;

/* A ragged latent cache, contiguous per sequence or paged.
 * Row r is rows + r * row_stride: [c_kv: d_c elements of latent_dtype |
 * k_rope: d_rope elements of rope_dtype], packed from byte 0; the rest of
 * the stride is padding the library never reads or writes. k_rope is stored
 * already rotated at its own position. For MLA_FP8_E4M3 latents, scale[r]
 * (fp32) multiplies row r's latent codes; scale is NULL otherwise.
 * Contiguous (block_table NULL): sequence b's token t is row seq_start[b] + t,
 * for t < seq_cap[b].
 * Paged (block_table not NULL): the rows form blocks of block_tokens rows
 * (a multiple of 32); sequence b's token t is row
 *     block_table[b * max_blocks + t / block_tokens] * block_tokens
 *         + t % block_tokens,
 * for t < seq_cap[b] <= max_blocks * block_tokens; seq_start is not read and
 * may be NULL. A block id outside [0, n_rows / block_tokens) is a device
 * error (MLA_ERR_PLAN): the access is clamped to block 0 and the status word
 * set. (Block tables are not on the pages: the layout serving engines use,
 * orthogonal to what MLA stores per token.)
 * Either way the first seq_len[b] tokens are valid. */
typedef struct {
  mla_dtype latent_dtype; /* F32, BF16 or FP8_E4M3 */
  mla_dtype rope_dtype;   /* F32 or BF16 */
  void *rows;             /* [n_rows, row_stride] bytes, 16-byte aligned */
  int64_t row_stride;     /* bytes, multiple of 16                      */
  float *scale;           /* [n_rows] for FP8 latents, else NULL         */
  int64_t n_rows;
  int32_t batch;
  const int32_t *seq_start; /* [batch] first row of each sequence (contiguous) */
  const int32_t *seq_cap;   /* [batch] tokens reserved per sequence             */
  int32_t *seq_len;         /* [batch] valid tokens; mla_append adds            */
  const int32_t *block_table; /* NULL, or [batch, max_blocks] block ids (paged) */
  int32_t block_tokens;       /* rows per block, multiple of 32 (paged), else 0 */
  int32_t max_blocks;         /* entries per sequence in block_table            */
} mla_cache;

/* Host-side split plan for decode (opaque). */
typedef struct mla_plan mla_plan;

/* ------------------------------------------------------------------ append
 * mla_append — down-project n_new new tokens per sequence into the cache.
 * For sequence b and new token j (0 <= j < n_new), at position
 * p = seq_len[b] + j:
 *     c   = W_DKV h[b, j]                 (d_c values)
 *     k_r = RoPE(W_KR h[b, j], p)         (d_rope values)
 * written to row seq_start[b] + p in the cache's dtypes (round to nearest
 * even; FP8 latents: s = max|c| / 448 in fp32, codes = RNE(c / s) clamped
 * to +-448, scale[row] = s, s = 1 for an all-zero row); then
 * seq_len[b] += n_new. Accumulation is fp32.
 * ("02 — Multi-Latent Attention (MLA)", "La compresión de MLA": c_t = W_DKV
 *  h_t is what is cached; "Truco de codificación posicional": the rotary key
 *  part is cached as it is.)
 *   h       [batch, n_new, d_model], act_w_dtype (F32 or BF16)
 *   w_dkv   [d_c, d_model], act_w_dtype
 *   w_kr    [d_rope, d_model], act_w_dtype
 *   ws      workspace of at least mla_append_workspace_bytes() bytes; its
 *           first 256 bytes hold the device status word (see
 *           mla_workspace_init).
 * A sequence with seq_len[b] + n_new > seq_cap[b] is left untouched and
 * MLA_ERR_CAPACITY is recorded in the status word. */
size_t mla_append_workspace_bytes(const mla_dims *dims, int32_t batch, int32_t n_new);
mla_status mla_append(const mla_dims *dims, const mla_cache *cache, const void *h,
                      int32_t n_new, const void *w_dkv, const void *w_kr,
                      mla_dtype act_w_dtype, void *ws, size_t ws_bytes,
                      void *stream /* hipStream_t */);

/* -------------------------------------------------------------------- plan
 * mla_plan_create — split the decode work of a batch with cached lengths
 * host_lens[batch] (host) into work items (b, t0, t1) of about equal token
 * counts, so that one launch fills the GPU even for a few long sequences.
 * Split-K over the sequence is not on the pages; it is exact by the
 * log-sum-exp identity (the combine step). n_workers is the number of
 * concurrent work items to aim for; 0 means "derive from the current HIP
 * device" (one per compute unit), and then no item is made shorter than
 * 64 tokens unless its sequence is (an item's fixed cost, its first copies
 * and its partial result, outweighs a one-tile item's work; a 4K-token
 * sequence alone runs fastest in 64 items of two tiles).
 * With an explicit n_workers the chunks are as short as that count needs
 * (one 32-token tile at the least). The plan is deterministic in its inputs
 * and reusable across layers and calls with the same lengths. Returns
 * MLA_ERR_INVALID_ARG for batch < 1, a negative length or a null pointer. */
mla_status mla_plan_create(const mla_dims *dims, const int32_t *host_lens, int32_t batch,
                           int32_t n_workers, mla_plan **out);
void mla_plan_destroy(mla_plan *plan);
/* Plan inspection (host): number of work items, and item k's
 * (sequence, first token, end token). */
int32_t mla_plan_num_items(const mla_plan *plan);
mla_status mla_plan_item(const mla_plan *plan, int32_t k, int32_t *b, int32_t *t0, int32_t *t1);

/* ------------------------------------------------------------------ decode
 * mla_decode — one query token per sequence attends over its cached rows.
 * For sequence b (L = the plan's length for b, P = q_pos[b] if q_pos is not
 * NULL, else L - 1) and head i:
 *     q~   = W_UK,i^T q_nope[b,i]                        (absorbed, d_c)
 *     q_r  = RoPE(q_rope[b,i], P)
 *     s_t  = softmax_scale * (q~ . c_t + q_r . k_rope_t),  t = 0 .. L-1
 *     o^   = sum_t softmax(s)_t c_t                      (latent space, d_c)
 *     o[b,i] = W_UV,i o^                                 (d_v)
 * which equals standard softmax attention with K = [W_UK c | k_rope] and
 * V = W_UV c in exact arithmetic. L = 0 gives o = 0.
 * ("02 — Multi-Latent Attention (MLA)", "Coste de cómputo" and "Lo que MLA no
 *  es"; "Atención latente de múltiples cabezas", "Información técnica";
 *  "DeepSeek MLA", content + positional score.)
 *   q_nope  [batch, n_heads, d_nope], q_w_dtype (F32 or BF16)
 *   q_rope  [batch, n_heads, d_rope], q_w_dtype, unrotated
 *   q_pos   [batch] int32 or NULL
 *   w_uk    [n_heads, d_nope, d_c], q_w_dtype
 *   w_uv    [n_heads, d_v, d_c], q_w_dtype
 *   o       [batch, n_heads, d_v], o_dtype (F32 or BF16)
 *   ws      at least mla_decode_workspace_bytes(dims, plan) bytes
 * The device checks seq_len[b] against the plan (MLA_ERR_PLAN). Arithmetic:
 * fp32 accumulation throughout. The matrix-core path (d_c = 512,
 * d_rope = 64, d_nope = d_v = 128, n_heads a multiple of 128, bf16 q and
 * weights, bf16 or fp8 latents, bf16 k_rope) rounds q~ and the softmax
 * weights to fp16 and widens the cached values to fp16 (exact for every e4m3
 * value and for bf16 values up to 65504 in magnitude) for the matrix cores;
 * the merged latent output enters the W_UV product as a bf16 hi + lo pair.
 * Every other shape runs fp32 kernels. */
size_t mla_decode_workspace_bytes(const mla_dims *dims, const mla_plan *plan);
/* mla_workspace_bytes — one size that serves every call on this plan with at
 * most one new token per sequence: mla_decode, and, when dims->d_model > 0,
 * mla_append and mla_append_decode with n_new = 1 (the append a decode step
 * makes): the larger of mla_decode_workspace_bytes(dims, plan) and
 * mla_append_workspace_bytes(dims, plan's batch, 1). Longer appends and
 * several query tokens size theirs with the specific functions. 0 for
 * invalid dims or a NULL plan. */
size_t mla_workspace_bytes(const mla_dims *dims, const mla_plan *plan);
mla_status mla_decode(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan,
                      const void *q_nope, const void *q_rope, const int32_t *q_pos,
                      const void *w_uk, const void *w_uv, mla_dtype q_w_dtype, void *o,
                      mla_dtype o_dtype, void *ws, size_t ws_bytes, void *stream);

/* mla_decode_multi — q_len new query tokens per sequence (multi-token
 * prediction, speculative verification: "Multi-head Latent Attention (MLA)
 * și arhitectura DeepSeekMoE", "Concepte cheie și caracteristici"), causal
 * among themselves. The q_len new tokens are the last q_len cached rows of
 * each sequence (appended first). Query j (0 .. q_len-1) of sequence b sits
 * at position P - (q_len - 1 - j), P = q_pos[b] if q_pos is not NULL, else
 * L - 1, and attends over rows 0 .. L - 1 - (q_len - 1 - j) exactly as
 * mla_decode does over 0 .. L - 1; a query that sees no row gives o = 0.
 *   q_nope  [batch, q_len, n_heads, d_nope], bf16
 *   q_rope  [batch, q_len, n_heads, d_rope], bf16, unrotated
 *   o       [batch, q_len, n_heads, d_v], o_dtype (F32 or BF16)
 *   ws      at least mla_decode_multi_workspace_bytes(dims, plan, q_len)
 * 1 <= q_len <= 16 (MLA_ERR_INVALID_ARG otherwise). Matrix-core path only:
 * arguments the fast path does not take (see mla_decode) return
 * MLA_ERR_UNSUPPORTED when q_len > 1. q_len = 1 is mla_decode, bit for bit.
 * The cache is read once for all q_len queries: the work per cached byte
 * grows q_len times. */
mla_status mla_decode_multi(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan, int32_t q_len,
                            const void *q_nope, const void *q_rope, const int32_t *q_pos, const void *w_uk,
                            const void *w_uv, mla_dtype q_w_dtype, void *o, mla_dtype o_dtype, void *ws,
                            size_t ws_bytes, void *stream);
size_t mla_decode_multi_workspace_bytes(const mla_dims *dims, const mla_plan *plan, int32_t q_len);

/* mla_append_decode — mla_append of n_new tokens followed, in stream order,
 * by mla_decode. The plan must have been made from the lengths after the
 * append (old lengths + n_new). ws must satisfy both workspace sizes. */
mla_status mla_append_decode(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan,
                             const void *h, int32_t n_new, const void *w_dkv, const void *w_kr,
                             const void *q_nope, const void *q_rope, const int32_t *q_pos,
                             const void *w_uk, const void *w_uv, mla_dtype act_w_dtype, void *o,
                             mla_dtype o_dtype, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ status
 * mla_workspace_init — clear the device status word at the start of ws
 * (a one-thread kernel, no memset, so it can sit in a captured graph).
 * mla_device_error — synchronise the stream, read the status word into
 * *code (an mla_status value), and clear it if reset != 0. */
mla_status mla_workspace_init(void *ws, size_t ws_bytes, void *stream);
mla_status mla_device_error(void *ws, void *stream, int32_t *code, int32_t reset);

const char *mla_status_str(mla_status s);
int32_t mla_abi_version(void);

/* ------------------------------------------------------------- profiling
 * Optional per-kernel timing with HIP events recorded around each kernel
 * this library launches (kernel ids: see mla_prof_kernel_name).
 * mla_prof_begin enables recording of up to max_records launches;
 * mla_prof_end synchronises the recorded events, writes the summed
 * milliseconds and launch counts per kernel id into ms[n] / count[n] and
 * disables recording. */
mla_status mla_prof_begin(int32_t max_records);
mla_status mla_prof_end(double *ms, int32_t *count, int32_t n);
const char *mla_prof_kernel_name(int32_t id);
int32_t mla_prof_num_kernels(void);

/* ------------------------------------------------------------ calibration
 * mla_calib_copy — a plain device copy (16-byte vector loads and stores) of
 * n_bytes (multiple of 16) from src to dst. Not part of the method: it gives
 * hardware counters a kernel of known traffic to calibrate against. */
mla_status mla_calib_copy(void *dst, const void *src, size_t n_bytes, void *stream);
/* mla_calib_read — reads n_bytes (multiple of 16) of device memory at src
 * (16-byte aligned) once, in 16-byte vector loads with several in flight per
 * thread, and XORs all the 32-bit words read into the device word *sink
 * (caller-owned, 4-byte aligned; atomic, one update per workgroup, so two
 * calls on the same data restore it). Not part of the method: timed over a
 * buffer larger than the on-package cache it is the achievable HBM read
 * rate, the ceiling a read-bound kernel is compared with beside the vendor
 * peak. Asynchronous on stream; MLA_ERR_INVALID_ARG for a null or misaligned
 * pointer or a size not a multiple of 16. */
mla_status mla_calib_read(const void *src, size_t n_bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
