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
 *    host-side plan (pinned, device-mapped host memory) between
 *    mla_plan_create() and mla_plan_destroy().
 *  - A workspace carries nothing a later call depends on except its status
 *    word: between calls the caller may reuse it for other data, or pass it
 *    to calls on other plans. (Each decode keeps a copy of its plan's work
 *    list in the workspace; the first kernel of every decode checks that
 *    copy against the plan's checksum and fetches the plan again from its
 *    pinned host block when they differ. The library keeps no record of
 *    which workspace holds which plan.)
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
  MLA_ERR_PLAN = 6,        /* device: seq_len differs from the plan         */
  MLA_ERR_RANGE = 7        /* device: a value the matrix-core path carries
                              in fp16 is beyond fp16's range (see mla_decode) */
} mla_status;

typedef enum {
  MLA_F32 = 0,
  MLA_BF16 = 1,
  MLA_FP8_E4M3 = 2 /* OCP E4M3FN: bias 7, max 448, no inf, NaN 0x7F/0xFF */
} mla_dtype;

/* Shapes of one MLA layer. softmax_scale multiplies the whole
 * (d_nope + d_rope)-wide score; 0 selects (d_nope + d_rope)^(-1/2), the
 * scale of the workloads (computed in double, rounded once to float); rope_base is the RoPE base (10000 in the
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
 * A sequence whose new tokens do not fit is left untouched (no row
 * written, seq_len unchanged) and its error recorded in the status word:
 * MLA_ERR_CAPACITY when seq_len[b] + n_new > seq_cap[b], or (contiguous)
 * seq_start[b] + seq_len[b] + n_new > n_rows, or (paged) the new tokens
 * pass max_blocks * block_tokens; MLA_ERR_PLAN when a block a new token
 * falls in has an id outside the cache. The other sequences append. */
size_t mla_append_workspace_bytes(const mla_dims *dims, int32_t batch, int32_t n_new);
mla_status mla_append(const mla_dims *dims, const mla_cache *cache, const void *h,
                      int32_t n_new, const void *w_dkv, const void *w_kr,
                      mla_dtype act_w_dtype, void *ws, size_t ws_bytes,
                      void *stream /* hipStream_t */);

/* -------------------------------------------------------------------- plan
 * mla_plan_create — split the decode work of a batch with cached lengths
 * host_lens[batch] (host) into work items (b, t0, t1), pieces of one
 * sequence on 32-token tile boundaries, listed in sequence order, and cut
 * that list into at most n_workers ranges of consecutive items, one
 * workgroup (per 128 heads) each, so that one launch fills the GPU and its
 * workgroups finish together whatever the mix of lengths. The ranges are
 * balanced on tiles plus a fixed cost of six tiles per item (an item's
 * pipeline fill and drain and its 128 KB partial result): the concatenated
 * tiles of all sequences are cut at about equal cost, so a range may end
 * one sequence and begin the next. Split-K over the sequence is not on the
 * pages; it is exact by the log-sum-exp identity (the combine step).
 * n_workers 0 means "derive from the current HIP device" (one range per
 * compute unit), and then no item is made shorter than 64 tokens unless its
 * sequence (or what a range leaves of it) is; with an explicit n_workers
 * items may be a single 32-token tile. The plan is deterministic in its inputs
 * and reusable across layers and calls with the same lengths. Its work list
 * lives in pinned host memory mapped for the current device, which the
 * decode's first kernel reads when a workspace's copy of it does not match;
 * where no such memory can be had (no device), the plan is made in ordinary
 * memory for inspection and decodes refuse it (MLA_ERR_HIP). Returns
 * MLA_ERR_INVALID_ARG for batch < 1, a negative length or a null pointer. */
mla_status mla_plan_create(const mla_dims *dims, const int32_t *host_lens, int32_t batch,
                           int32_t n_workers, mla_plan **out);
/* mla_plan_create_multi — the same for mla_decode_multi with q_len new
 * query tokens per sequence ("Multi-head Latent Attention (MLA) și
 * arhitectura DeepSeekMoE", "Concepte cheie și caracteristici": several
 * tokens per step for speculative decoding). Each range then runs as
 * ceil(q_len * n_heads / 128) workgroups, one per head block of the
 * (token, head) pairs, so the ranges are cut for n_workers divided by that
 * count (at least one): every compute unit still gets one workgroup, and an
 * item's fixed cost is paid once per compute unit rather than once per head
 * block. n_workers 0 means the compute units of the current HIP device.
 * mla_plan_create(...) is mla_plan_create_multi(..., q_len = 1, ...); a plan
 * from either serves every decode call with the same lengths.
 * MLA_ERR_INVALID_ARG as mla_plan_create, and for q_len outside 1..16. */
mla_status mla_plan_create_multi(const mla_dims *dims, const int32_t *host_lens, int32_t batch, int32_t q_len,
                                 int32_t n_workers, mla_plan **out);
void mla_plan_destroy(mla_plan *plan);
/* Plan inspection (host): number of work items, and item k's
 * (sequence, first token, end token); number of workgroup ranges, and range
 * j's items [item_begin, item_end). MLA_ERR_INVALID_ARG for an index out
 * of range or a null pointer (the counts return -1 for a null plan). */
int32_t mla_plan_num_items(const mla_plan *plan);
mla_status mla_plan_item(const mla_plan *plan, int32_t k, int32_t *b, int32_t *t0, int32_t *t1);
int32_t mla_plan_num_ranges(const mla_plan *plan);
mla_status mla_plan_range(const mla_plan *plan, int32_t j, int32_t *item_begin, int32_t *item_end);

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
 * weights, bf16 or fp8 latents, bf16 k_rope) rounds q~ (times softmax_scale
 * * log2 e) and the softmax weights to fp16 and widens the cached values
 * (bf16, or e4m3 codes times their scale) to fp16 for the matrix cores; the
 * merged latent output enters the W_UV product as a bf16 hi + lo pair.
 * Every other shape runs fp32 kernels.
 * Numeric domain of the matrix-core path: a widened cached value is exact
 * when its magnitude lies in [2^-14, 65504) (every bf16 value there has a
 * significand fp16 holds; e4m3 codes times a scale are rounded once to
 * fp16's 11 bits); below 2^-14 it becomes an fp16 subnormal (absolute
 * precision 2^-24: the relative error grows as the value shrinks), below
 * 2^-24 it reads as zero (bf16 values are converted rounding toward zero);
 * at 65504 and above a bf16 value saturates to +-65504. q~ obeys the same
 * range (rounded to nearest; beyond 65504 it is reported). The scores' relative
 * precision does not matter for tiny values (they are tiny in absolute
 * terms); the value product's does: a cache whose rows are uniformly below
 * 2^-14, or that reach 65504, is outside the domain and belongs on the fp32
 * path. The decode reports a query value beyond fp16's range, and
 * mla_append a row it writes beyond it, as MLA_ERR_RANGE (the row is
 * stored as it is); rows the caller writes itself are not checked.
 * Accuracy inside that range: the absorbed query (times softmax_scale and
 * log2 e) is rounded to fp16, relative 2^-11, so a score's error grows with
 * the score's own size. With s the scores in log2 units, the output's max
 * error over its rms stays within 2e-2 while max|s| <= 64, and within
 * 2e-2 + 2^-13 max|s| beyond (measured and emulated: near 0.12 at
 * max|s| = 1800). A bf16 query would carry 8 significand bits, not 11. */
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
 * Each range of the plan runs as one workgroup per 128 (token, head) pairs;
 * the workgroups of one range sit on one XCD, so the cache comes from HBM
 * about once for all q_len queries while the work per cached byte grows
 * q_len times. A plan from mla_plan_create_multi with the same q_len keeps
 * one workgroup per compute unit (any plan for these lengths is valid). */
mla_status mla_decode_multi(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan, int32_t q_len,
                            const void *q_nope, const void *q_rope, const int32_t *q_pos, const void *w_uk,
                            const void *w_uv, mla_dtype q_w_dtype, void *o, mla_dtype o_dtype, void *ws,
                            size_t ws_bytes, void *stream);
size_t mla_decode_multi_workspace_bytes(const mla_dims *dims, const mla_plan *plan, int32_t q_len);

/* Precomputed absorbed weights. The up-projections can be folded into the
 * query and output projections ahead of time, so the decode never forms
 * per-head keys or values ("02 — Multi-Latent Attention (MLA)", "Coste de
 * cómputo": attention rearranged with some matrix products precomputed;
 * "Atención latente de múltiples cabezas", "Información técnica": the
 * up-projection weights absorbed into the query and output projections;
 * "Multi-head Latent Attention (MLA) și arhitectura DeepSeekMoE", opening
 * paragraph). The rotary query cannot be folded (same sections: the
 * decoupled key path exists for that) and stays an input.
 * Layouts: W_Q [n_heads, d_nope, d_x] (head i's no-RoPE query is
 * W_Q,i x, x the token's query input: its hidden state, or a query latent
 * where the model compresses queries); W_O [d_out, n_heads d_v] (the layer
 * output is W_O applied to the heads' outputs concatenated in head order).
 *
 * mla_merge_query_weight — a [n_heads, d_c, d_x] = W_UK,i^T W_Q,i per head,
 * as a weight of R = n_heads d_c rows and K = d_x columns (row h d_c + c).
 * mla_merge_output_weight — bm [d_out, n_heads d_c], column block i =
 * W_O[:, i d_v .. (i+1) d_v) W_UV,i: R = d_out rows, K = n_heads d_c.
 * Storage of such a weight: when R % 32 == 0 and K % 64 == 0,
 * fragment-tiled, so that the decode streams it in contiguous 1 KB loads:
 * element (r, k) at ((r / 32) (K / 64) + k / 64) 2048 + ((k % 32) / 8) 512 +
 * (r % 32 + 32 ((k % 64) / 32)) 8 + k % 8; otherwise row-major, r K + k.
 * The buffers are meant for mla_decode_merged with the same dims, d_x and
 * d_out (which reads them in that storage).
 * One-time weight preparation (fp32 accumulation, stored in w_dtype, F32 or
 * BF16 with round-to-nearest-even); the inputs keep their W_UK and W_UV
 * layouts of mla_decode. All pointers are device memory the caller owns,
 * 16-byte aligned; asynchronous on the stream. MLA_ERR_INVALID_ARG for
 * invalid dims, d_x or d_out < 1, NULL or misaligned pointers, other dtypes.
 * Sizes: a holds n_heads d_c d_x elements, bm d_out n_heads d_c; at the
 * DeepSeek-V3 shape with a 1536-wide query latent and d_out = 7168 that is
 * 201 MB and 940 MB in bf16, against 16.8 MB each for W_UK and W_UV. */
mla_status mla_merge_query_weight(const mla_dims *dims, int32_t d_x, const void *w_q, const void *w_uk,
                                  mla_dtype w_dtype, void *a, void *stream);
mla_status mla_merge_output_weight(const mla_dims *dims, int32_t d_out, const void *w_o, const void *w_uv,
                                   mla_dtype w_dtype, void *bm, void *stream);

/* mla_decode_merged — mla_decode from the merged weights, emitting the
 * post-W_O output: per sequence b and head i, q~_i = A_i x_b, the same
 * scores, softmax and latent-space output o^_i as mla_decode, and
 * y_b = bm [o^_1; ..; o^_n_heads].
 *   x       [batch, d_x], w_dtype
 *   q_rope  [batch, n_heads, d_rope], w_dtype, unrotated; q_pos as mla_decode
 *   a, bm   from the merge calls, w_dtype (F32 or BF16)
 *   y       [batch, d_out], y_dtype (F32 or BF16)
 *   ws      at least mla_decode_merged_workspace_bytes(dims, plan, d_out)
 * One query token per sequence. Matrix-core path when mla_decode's fast
 * path applies (w_dtype BF16) and d_x % 512 == 0 and d_out % 128 == 0; else
 * the fp32 kernels (d_x up to 16384). Errors, status word and numeric domain
 * as mla_decode (o^ enters the output product as bf16 hi + lo, about 16
 * significant bits). */
mla_status mla_decode_merged(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan, int32_t d_x,
                             const void *x, const void *q_rope, const int32_t *q_pos, const void *a, int32_t d_out,
                             const void *bm, mla_dtype w_dtype, void *y, mla_dtype y_dtype, void *ws,
                             size_t ws_bytes, void *stream);
size_t mla_decode_merged_workspace_bytes(const mla_dims *dims, const mla_plan *plan, int32_t d_out);

/* mla_append_decode — mla_append of n_new tokens followed, in stream order,
 * by mla_decode. The plan must have been made from the lengths after the
 * append (old lengths + n_new). ws must satisfy both workspace sizes. */
mla_status mla_append_decode(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan,
                             const void *h, int32_t n_new, const void *w_dkv, const void *w_kr,
                             const void *q_nope, const void *q_rope, const int32_t *q_pos,
                             const void *w_uk, const void *w_uv, mla_dtype act_w_dtype, void *o,
                             mla_dtype o_dtype, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------- no workspace
 * mla_decode_noalloc — mla_decode for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments and results as mla_decode (one
 * query token per sequence), with no workspace argument. Its workspace is a
 * fixed array of MLA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * held from the library's first use on that GPU until the process ends;
 * the call allocates nothing (no hipMalloc, no allocating library call).
 *   dev_status  NULL, or a device int32 (4-byte aligned) that receives the
 *               call's device status word (an mla_status value: MLA_ERR_PLAN
 *               for lengths that differ from the plan) once the call's
 *               kernels have run. The word is cleared at the start of every
 *               call.
 * Returns MLA_ERR_WORKSPACE when the plan needs more than the array holds:
 * on the matrix-core path 2 * (batch * n_heads * (d_c + d_rope) + n_items *
 * n_heads * d_c) bytes plus small per-item and per-sequence arrays (batch
 * 32 with 256 work items: about 38 MB; the default plan of 128 sequences:
 * about 53 MB); the fp32 path needs twice that. Every call on one GPU uses
 * that GPU's one array, which keeps the last call's contents: calls that
 * overlap on one GPU (several streams, several host threads) race and must
 * be ordered by the caller. */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
mla_status mla_decode_noalloc(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan,
                              const void *q_nope, const void *q_rope, const int32_t *q_pos, const void *w_uk,
                              const void *w_uv, mla_dtype q_w_dtype, void *o, mla_dtype o_dtype,
                              int32_t *dev_status, void *stream);

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
 * this library launches (kernel ids: see mla_prof_kernel_name). While
 * recording, every call synchronises its stream before each kernel it
 * launches, so each recorded kernel starts on an idle stream (its time is
 * its own, not the wait for earlier work); calls are therefore slower.
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
