// Generic MLA kernels: any head count and widths, fp32 arithmetic on the
// vector ALUs. They run the fp32 workloads and every shape the matrix-core
// path does not cover, and serve as a differential reference for it.
//
// Steps (see mla.h for the definitions and their sources):
//   append_generic_kernel   c = W_DKV h, k_r = RoPE(W_KR h, p), round, store
//   advance_len_kernel      seq_len[b] += n_new where the append fitted
//   absorb_generic_kernel   Q = [W_UK^T q_nope ; RoPE(q_rope, P)] * scale * log2(e)
//   decode_generic_kernel   split-K partial: online softmax over one work item
//   combine_generic_kernel  log-sum-exp merge of the splits, then o = W_UV o^
#include <cfloat>
#include <cmath>

#include "device_util.hpp"

namespace mla {
namespace {

__global__ void init_kernel(int32_t *status) {
  if (threadIdx.x == 0 && blockIdx.x == 0) status[0] = 0;
}

__global__ void status_copy_kernel(const int32_t *src, int32_t *dst) {
  if (threadIdx.x == 0 && blockIdx.x == 0) dst[0] = src[0];
}

__global__ __launch_bounds__(256) void append_generic_kernel(mla_dims d, mla_cache c, const void *h,
                                                            int32_t n_new, const void *w_dkv,
                                                            const void *w_kr, mla_dtype act,
                                                            int32_t *status) {
  extern __shared__ float smem[];
  const int b = blockIdx.x, j = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = d.d_c + d.d_rope;
  float *hs = smem;              // [d_model]
  float *outv = hs + d.d_model;  // [d_c + d_rope]
  float *red = outv + R;         // [4]

  const int32_t len = c.seq_len[b];
  const int64_t pos = static_cast<int64_t>(len) + j;
  const int32_t chk = append_check(c, b, len, n_new);
  if (chk != MLA_OK) {
    if (tid == 0 && j == 0) set_status(status, chk);
    return;
  }
  bool bad = false;
  const int64_t row = cache_row(c, b, pos, bad);  // (every block was checked)

  const int64_t hoff = (static_cast<int64_t>(b) * n_new + j) * d.d_model;
  for (int k = tid; k < d.d_model; k += 256) hs[k] = load_elem(h, hoff + k, act);
  __syncthreads();

  // One wave per output row; lanes split the d_model sum (coalesced weight rows).
  for (int r = wave; r < R; r += 4) {
    const void *W = r < d.d_c ? w_dkv : w_kr;
    const int64_t wrow = static_cast<int64_t>(r < d.d_c ? r : r - d.d_c) * d.d_model;
    float acc = 0.0f;
    for (int k = lane; k < d.d_model; k += 64) acc = fmaf(load_elem(W, wrow + k, act), hs[k], acc);
    acc = wave_sum(acc);
    if (lane == 0) outv[r] = acc;
  }
  __syncthreads();

  for (int p = tid; p < d.d_rope / 2; p += 256) {
    float cs, sn;
    rope_cos_sin(pos, p, d.d_rope, d.rope_base, &cs, &sn);
    const float x0 = outv[d.d_c + 2 * p], x1 = outv[d.d_c + 2 * p + 1];
    outv[d.d_c + 2 * p] = x0 * cs - x1 * sn;
    outv[d.d_c + 2 * p + 1] = x0 * sn + x1 * cs;
  }
  __syncthreads();

  store_appended_row(d, c, row, outv, red, status);
}

__global__ void advance_len_kernel(mla_cache c, int32_t n_new) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= c.batch) return;
  const int32_t len = c.seq_len[b];
  if (append_check(c, b, len, n_new) == MLA_OK) c.seq_len[b] = len + n_new;
}

__global__ __launch_bounds__(256) void absorb_generic_kernel(mla_dims d, const void *q_nope,
                                                            const void *q_rope, const int32_t *q_pos,
                                                            const void *w_uk, mla_dtype qw,
                                                            const int32_t *dev_len, float *q_out, PlanRef plan) {
  extern __shared__ float qn[];  // [d_nope]
  const int b = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
  const int H = d.n_heads, D = d.d_c + d.d_rope;
  const int64_t bi = static_cast<int64_t>(b) * H + i;
  for (int n = tid; n < d.d_nope; n += 256) qn[n] = load_elem(q_nope, bi * d.d_nope + n, qw);
  __syncthreads();
  const float qs = d.softmax_scale * kLog2e;
  float *out = q_out + bi * D;
  for (int cc = tid; cc < d.d_c; cc += 256) {
    float acc = 0.0f;
    for (int n = 0; n < d.d_nope; ++n)
      acc = fmaf(load_elem(w_uk, (static_cast<int64_t>(i) * d.d_nope + n) * d.d_c + cc, qw), qn[n], acc);
    out[cc] = acc * qs;
  }
  const int64_t P = q_pos ? q_pos[b] : static_cast<int64_t>(dev_len[b]) - 1;
  for (int p = tid; p < d.d_rope / 2; p += 256) {
    float cs, sn;
    rope_cos_sin(P, p, d.d_rope, d.rope_base, &cs, &sn);
    const float x0 = load_elem(q_rope, bi * d.d_rope + 2 * p, qw);
    const float x1 = load_elem(q_rope, bi * d.d_rope + 2 * p + 1, qw);
    out[d.d_c + 2 * p] = (x0 * cs - x1 * sn) * qs;
    out[d.d_c + 2 * p + 1] = (x0 * sn + x1 * cs) * qs;
  }
  // the plan copy the decode and combine kernels read
  if (blockIdx.x == 0 && blockIdx.y == 0) plan_verify(plan);
}

// True when the item names a sequence of the batch, the device length agrees
// with the plan and the item's rows lie in the sequence's reserved range and
// in the cache.
__device__ __forceinline__ bool item_ok(const mla_cache &c, const WorkItem &it, const SeqInfo *seqs) {
  if (it.b < 0 || it.b >= c.batch) return false;
  return c.seq_len[it.b] == seqs[it.b].len && it.t0 >= 0 && it.t0 < it.t1 && seq_range_ok(c, it.b, it.t1);
}

__global__ __launch_bounds__(256) void decode_generic_kernel(mla_dims d, mla_cache c,
                                                            const WorkItem *items, const SeqInfo *seqs,
                                                            const float *q, float *opart, float *lse,
                                                            int32_t *status) {
  extern __shared__ float smem[];
  const int k = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
  const int H = d.n_heads, D = d.d_c + d.d_rope;
  const WorkItem it = items[k];
  float *qs = smem;     // [D]
  float *ps = qs + D;   // [256]
  float *red = ps + 256;
  float *op = opart + (static_cast<int64_t>(k) * H + i) * d.d_c;

  if (!item_ok(c, it, seqs)) {
    if (tid == 0 && i == 0) set_status(status, MLA_ERR_PLAN);
    for (int cc = tid; cc < d.d_c; cc += 256) op[cc] = 0.0f;
    if (tid == 0) lse[static_cast<int64_t>(k) * H + i] = -INFINITY;
    return;
  }
  const float *qrow = q + (static_cast<int64_t>(it.b) * H + i) * D;
  for (int x = tid; x < D; x += 256) qs[x] = qrow[x];
  __syncthreads();

  bool bad = false;
  const int lat_b = elem_bytes(c.latent_dtype);
  const bool fp8 = c.latent_dtype == MLA_FP8_E4M3;
  float m = -INFINITY, l = 0.0f;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // latent columns tid + 256 r; d_c <= 1024

  for (int t0 = it.t0; t0 < it.t1; t0 += 256) {
    const int t = t0 + tid;
    float s = -INFINITY;
    if (t < it.t1) {
      const int64_t row = cache_row(c, it.b, t, bad);
      const char *rowp = static_cast<const char *>(c.rows) + row * c.row_stride;
      float dot = 0.0f;
      for (int x = 0; x < d.d_c; ++x) dot = fmaf(qs[x], load_elem(rowp, x, c.latent_dtype), dot);
      if (fp8) dot *= c.scale[row];
      const char *rp = rowp + static_cast<int64_t>(d.d_c) * lat_b;
      for (int x = 0; x < d.d_rope; ++x) dot = fmaf(qs[d.d_c + x], load_elem(rp, x, c.rope_dtype), dot);
      s = dot;
    }
    const float m_new = fmaxf(m, block_max_256(s, red));
    const float p = t < it.t1 ? exp2f(s - m_new) : 0.0f;
    ps[tid] = p;
    const float psum = block_sum_256(p, red);
    const float alpha = exp2f(m - m_new);
    l = l * alpha + psum;
    m = m_new;
    const int nt = min(256, it.t1 - t0);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] *= alpha;
    for (int tt = 0; tt < nt; ++tt) {
      const int64_t row = cache_row(c, it.b, t0 + tt, bad);
      const char *rowp = static_cast<const char *>(c.rows) + row * c.row_stride;
      const float pt = fp8 ? ps[tt] * c.scale[row] : ps[tt];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int cc = tid + 256 * r;
        if (cc < d.d_c) acc[r] = fmaf(pt, load_elem(rowp, cc, c.latent_dtype), acc[r]);
      }
    }
    __syncthreads();
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int cc = tid + 256 * r;
    if (cc < d.d_c) op[cc] = acc[r] * inv;
  }
  if (tid == 0) lse[static_cast<int64_t>(k) * H + i] = m + log2f(l);
  if (bad && tid == 0) set_status(status, MLA_ERR_PLAN);  // a block id outside the cache: block 0 was read
}

// With ohat set, o^ is written there ([B, H, d_c] fp32) and W_UV is not
// applied (the precomputed-weights decode applies W_O W_UV itself).
__global__ __launch_bounds__(256) void combine_generic_kernel(mla_dims d, mla_cache c, int n_items,
                                                             const SeqInfo *seqs, const float *opart,
                                                             const float *lse, const void *w_uv,
                                                             mla_dtype qw, void *o, mla_dtype od, float *ohat,
                                                             int32_t *status) {
  extern __shared__ float oh[];  // [d_c]
  const int b = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int H = d.n_heads;
  const SeqInfo si = seqs[b];
  const bool in_list = si.item_begin >= 0 && si.item_count >= 0 && si.item_begin <= n_items - si.item_count;
  if (!in_list && tid == 0 && i == 0) set_status(status, MLA_ERR_PLAN);
  const bool ok = in_list && si.item_count > 0 && c.seq_len[b] == si.len;
  if (ok) {
    float M = -INFINITY;
    for (int s = 0; s < si.item_count; ++s) M = fmaxf(M, lse[static_cast<int64_t>(si.item_begin + s) * H + i]);
    float den = 0.0f;
    for (int s = 0; s < si.item_count; ++s) den += exp2f(lse[static_cast<int64_t>(si.item_begin + s) * H + i] - M);
    const float inv = 1.0f / den;
    for (int cc = tid; cc < d.d_c; cc += 256) {
      float num = 0.0f;
      for (int s = 0; s < si.item_count; ++s) {
        const int64_t slot = static_cast<int64_t>(si.item_begin + s) * H + i;
        num = fmaf(exp2f(lse[slot] - M), opart[slot * d.d_c + cc], num);
      }
      oh[cc] = num * inv;
    }
  } else {
    for (int cc = tid; cc < d.d_c; cc += 256) oh[cc] = 0.0f;
  }
  __syncthreads();
  if (ohat) {
    float *dst = ohat + (static_cast<int64_t>(b) * H + i) * d.d_c;
    for (int cc = tid; cc < d.d_c; cc += 256) dst[cc] = oh[cc];
    return;
  }
  const int64_t obase = (static_cast<int64_t>(b) * H + i) * d.d_v;
  for (int v = wave; v < d.d_v; v += 4) {
    const int64_t wrow = (static_cast<int64_t>(i) * d.d_v + v) * d.d_c;
    float acc = 0.0f;
    for (int cc = lane; cc < d.d_c; cc += 64) acc = fmaf(load_elem(w_uv, wrow + cc, qw), oh[cc], acc);
    acc = wave_sum(acc);
    if (lane == 0) {
      if (od == MLA_BF16)
        static_cast<uint16_t *>(o)[obase + v] = f32_to_bf16_bits(acc);
      else
        static_cast<float *>(o)[obase + v] = acc;
    }
  }
}

__global__ __launch_bounds__(256) void copy_kernel(uint4 *__restrict__ dst, const uint4 *__restrict__ src, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t x = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; x < n16; x += stride)
    dst[x] = src[x];
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Stream read: every 16-byte chunk read once, eight non-temporal loads in
// flight per thread (streamed data is not kept in the caches: about 5 %
// more than plain loads on a 4 GiB buffer); the XOR of all 32-bit words read is folded per wave (shuffles),
// per workgroup (LDS) and into *sink with one atomic per workgroup, so the
// loads cannot be dropped and the kernel writes next to nothing.
__global__ __launch_bounds__(256) void read_kernel(const uint4 *__restrict__ src, size_t n16, uint32_t *__restrict__ sink) {
  constexpr int U = 8;
  __shared__ uint32_t red[4];
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  size_t x = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint4 acc = {0, 0, 0, 0};
  for (; x + (U - 1) * stride < n16; x += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src) + x + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc.x ^= v[u].x;
      acc.y ^= v[u].y;
      acc.z ^= v[u].z;
      acc.w ^= v[u].w;
    }
  }
  for (; x < n16; x += stride) {
    const uint4 v = src[x];
    acc.x ^= v.x;
    acc.y ^= v.y;
    acc.z ^= v.z;
    acc.w ^= v.w;
  }
  uint32_t h = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) h ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(h), off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = h;
  __syncthreads();
  if (threadIdx.x == 0) atomicXor(sink, red[0] ^ red[1] ^ red[2] ^ red[3]);
}

}  // namespace

hipError_t launch_init(hipStream_t s, int32_t *status) {
  return launch_kernel(init_kernel, 1, 64, 0, s, status);
}

hipError_t launch_status_copy(hipStream_t s, const int32_t *src, int32_t *dst) {
  return launch_kernel(status_copy_kernel, 1, 64, 0, s, src, dst);
}

hipError_t launch_advance_len(hipStream_t s, const mla_cache &c, int32_t n_new) {
  return launch_kernel(advance_len_kernel, (c.batch + 255) / 256, 256, 0, s, c, n_new);
}

hipError_t launch_append_generic(hipStream_t s, const mla_dims &d, const mla_cache &c, const void *h,
                                 int32_t n_new, const void *w_dkv, const void *w_kr, mla_dtype act,
                                 int32_t *status) {
  const size_t shm = sizeof(float) * (d.d_model + d.d_c + d.d_rope + 4);
  hipError_t e = launch_kernel(append_generic_kernel, dim3(c.batch, n_new), 256, shm, s, d, c, h, n_new, w_dkv,
                               w_kr, act, status);
  if (e != hipSuccess) return e;
  return launch_advance_len(s, c, n_new);
}

hipError_t launch_absorb_generic(hipStream_t s, const mla_dims &d, int32_t batch, const void *q_nope,
                                 const void *q_rope, const int32_t *q_pos, const void *w_uk,
                                 mla_dtype qw, const int32_t *seq_len, float *q_out, const PlanRef &plan,
                                 int32_t *) {
  return launch_kernel(absorb_generic_kernel, dim3(batch, d.n_heads), 256, sizeof(float) * d.d_nope, s, d, q_nope,
                       q_rope, q_pos, w_uk, qw, seq_len, q_out, plan);
}

hipError_t launch_decode_generic(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t n_items,
                                 const WorkItem *items, const SeqInfo *seqs, const float *q,
                                 float *opart, float *lse, int32_t *status) {
  if (n_items == 0) return hipSuccess;
  const size_t shm = sizeof(float) * (d.d_c + d.d_rope + 256 + 4);
  return launch_kernel(decode_generic_kernel, dim3(n_items, d.n_heads), 256, shm, s, d, c, items, seqs, q, opart,
                       lse, status);
}

hipError_t launch_combine_generic(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t n_items,
                                  const SeqInfo *seqs, const float *opart, const float *lse,
                                  const void *w_uv, mla_dtype qw, void *o, mla_dtype od, int32_t *status) {
  return launch_kernel(combine_generic_kernel, dim3(c.batch, d.n_heads), 256, sizeof(float) * d.d_c, s, d, c, n_items,
                       seqs, opart, lse, w_uv, qw, o, od, nullptr, status);
}

hipError_t launch_combine_generic_emit(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t n_items,
                                       const SeqInfo *seqs, const float *opart, const float *lse, float *ohat,
                                       int32_t *status) {
  return launch_kernel(combine_generic_kernel, dim3(c.batch, d.n_heads), 256, sizeof(float) * d.d_c, s, d, c, n_items,
                       seqs, opart, lse, nullptr, MLA_F32, nullptr, MLA_F32, ohat, status);
}

hipError_t launch_copy(hipStream_t s, void *dst, const void *src, size_t n16) {
  return launch_kernel(copy_kernel, 2048, 256, 0, s, static_cast<uint4 *>(dst), static_cast<const uint4 *>(src), n16);
}

hipError_t launch_read(hipStream_t s, const void *src, size_t n16, uint32_t *sink) {
  return launch_kernel(read_kernel, 4096, 256, 0, s, static_cast<const uint4 *>(src), n16, sink);
}

}  // namespace mla
