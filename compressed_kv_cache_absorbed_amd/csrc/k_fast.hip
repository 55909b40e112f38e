// Matrix-core (MFMA) fast path for the DeepSeek-V3 shape: latent width 512,
// RoPE key width 64, heads a multiple of 128, bf16 activations and weights,
// bf16 or fp8-e4m3 latents with a bf16 RoPE key.
//
//   absorb_fast_kernel   Q[b,i] = fp16([W_UK,i^T q_nope[b,i] ; RoPE(q_rope[b,i], P_b)]
//                                      * softmax_scale * log2 e)
//                        (fp16, not bf16: the score's sensitivity to the
//                        rounding of q~ is what limits accuracy on peaked rows)
//   (the split-K kernel between them lives in k_splitk.hip)
//   append_gemm_kernel   [c ; k_r] = [W_DKV ; W_KR] h for the new tokens (K-split)
//   append_finish_kernel sum of the splits, RoPE, rounding / fp8 scale, row store
//   merge_fast_kernel    log-sum-exp merge of the split partials into o^
//   project_fast_kernel  o = W_UV o^ (the output-side absorption)
//
// Weight absorption ("02 — Multi-Latent Attention (MLA)", "Coste de cómputo";
// "Atención latente de múltiples cabezas", "Información técnica"): W_UK is
// applied to the query once per sequence and W_UV to the latent-space output,
// so the loop over cached tokens touches only [c_kv | k_rope] rows, each one
// reused by all heads.
//
// MFMA lane layouts used (v_mfma_f32_32x32x16_bf16, wave64, checked on the
// hardware): A[32 x 16]: lane l holds row l%32, k = 8(l/32) .. +7;
// B[16 x 32]: lane l holds column l%32, k = 8(l/32) .. +7; D[32 x 32]: lane l,
// register r holds row 8(r/4) + 4(l/32) + r%4, column l%32. The k order inside
// one product is free as long as A and B agree, which the value product uses
// to take P straight from the score registers.
// ds_read_b64_tr_b16: in each 16-lane group, source lane j supplies the
// address of 4 consecutive 16-bit elements; lane i receives element i%4 of
// source lanes i/4 + 4e, e = 0..3 (a 4x16 -> 16x4 transpose).
#include <cmath>
#include <cstdlib>

#include "device_util.hpp"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

namespace fast {
constexpr int DC = 512;        // latent width
constexpr int DR = 64;         // RoPE key width
constexpr int D = DC + DR;     // 576: score width
constexpr int DNOPE = 128;     // query no-RoPE width
constexpr int DV = 128;        // value head width
constexpr int HPW = 32;        // heads per wave of the split-K kernel
constexpr int WAVES = 4;       // its waves: 128 heads per workgroup
constexpr int APPEND_KS = 512;     // d_model inputs per K-split of the append GEMM
constexpr int APPEND_NMAX = 1024;  // largest d_c + d_rope the append finish holds in LDS
}  // namespace fast

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// MLA_FORCE_GENERIC=1 in the environment routes every call to the generic
// kernels (for differential testing of the two paths on the same inputs).
static bool force_generic() {
  const char *e = std::getenv("MLA_FORCE_GENERIC");
  return e && e[0] == '1';
}

bool decode_fast_path(const mla_dims &d, const mla_cache &c, mla_dtype q_w_dtype) {
  return !force_generic() && d.d_c == fast::DC && d.d_rope == fast::DR && d.d_nope == fast::DNOPE && d.d_v == fast::DV &&
         d.n_heads % (fast::HPW * fast::WAVES) == 0 && q_w_dtype == MLA_BF16 &&
         (c.latent_dtype == MLA_BF16 || c.latent_dtype == MLA_FP8_E4M3) && c.rope_dtype == MLA_BF16 &&
         c.row_stride <= (int64_t{1} << 26);  // the split-K copies use 32-bit offsets within a tile
}

namespace {

// ----------------------------------------------------------------- absorb
// Grid (H, 4, ceil(B/32)), 256 threads: head i, latent quarter cq (columns
// 128 cq .. +127), 32 sequences. The quarter of W_UK,i [128 n x 128 c] is
// staged in LDS with a 288-byte row stride (rows 32 bytes apart in the banks,
// so the transposed reads below are conflict-free) and read transposed as the
// A operand of q~^T = W_UK,i^T q_nope^T; wave w owns columns 32 w of the
// quarter. The quarter also rotates RoPE pairs 8 cq .. 8 cq + 7 of q_rope.
__global__ __launch_bounds__(256) void absorb_fast_kernel(int B, int H, float qscale, float rope_base,
                                                          const uint16_t *__restrict__ q_nope,
                                                          const uint16_t *__restrict__ q_rope,
                                                          const int32_t *__restrict__ q_pos,
                                                          const uint16_t *__restrict__ w_uk,
                                                          const SeqInfo *__restrict__ seqs,
                                                          uint16_t *__restrict__ Q) {
  using namespace fast;
  constexpr int WROW = 288;  // LDS bytes per W row (128 columns = 256 bytes + 32)
  __shared__ __attribute__((aligned(16))) char smem[DNOPE * WROW];
  const int i = blockIdx.x, cq = blockIdx.y, b0 = blockIdx.z * 32;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint16_t *W = w_uk + static_cast<size_t>(i) * DNOPE * DC + 128 * cq;
  // 32 KB of weights: 128 rows x 16 chunks of 16 bytes, 8 per thread
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const int q = tid + 256 * x, n = q >> 4, ch = q & 15;
    *reinterpret_cast<u32x4 *>(smem + n * WROW + 16 * ch) = *reinterpret_cast<const u32x4 *>(W + n * DC + 8 * ch);
  }

  // RoPE: thread (sequence b0 + tid / 8, pair 8 cq + tid % 8)
  {
    const int bb = b0 + (tid >> 3), p = 8 * cq + (tid & 7);
    if (bb < B) {
      const size_t bi = static_cast<size_t>(bb) * H + i;
      const int64_t P = q_pos ? q_pos[bb] : static_cast<int64_t>(seqs[bb].len) - 1;
      float cs, sn;
      rope_cos_sin(P, p, DR, rope_base, &cs, &sn);
      const uint32_t xr = *reinterpret_cast<const uint32_t *>(q_rope + bi * DR + 2 * p);
      const float x0 = bf16_bits_to_f32(static_cast<uint16_t>(xr & 0xffffu));
      const float x1 = bf16_bits_to_f32(static_cast<uint16_t>(xr >> 16));
      f16x2 r;
      r[0] = static_cast<_Float16>((x0 * cs - x1 * sn) * qscale);
      r[1] = static_cast<_Float16>((x0 * sn + x1 * cs) * qscale);
      *reinterpret_cast<f16x2 *>(Q + bi * D + DC + 2 * p) = r;
    }
  }

  // B operand: q_nope^T [16 n x 32 b]: lane holds sequence b0 + l%32, n = 16 kk + 8(l/32) .. +7
  const int bb = b0 + (lane & 31);
  bf16x8 qb[DNOPE / 16];
#pragma unroll
  for (int kk = 0; kk < DNOPE / 16; ++kk) {
    if (bb < B) {
      qb[kk] = *reinterpret_cast<const bf16x8 *>(q_nope + (static_cast<size_t>(bb) * H + i) * DNOPE +
                                                 16 * kk + 8 * (lane >> 5));
    } else {
      qb[kk] = bf16x8{};
    }
  }
  __syncthreads();
  // A operand: W^T [32 c x 16 n] via transposed LDS reads of W [n][c], with
  // the same contiguous k order as the B operand: in 16-lane group g the
  // lanes take c = c0 + 16(g%2) + i and n = 16 kk + 8(g/2) + e, e = 0..3 from
  // the first read and 4..7 from the second; source lane j points at
  // W[16 kk + 8(g/2) + j/4 (+4)][c0 + 16(g%2) + 4(j%4)].
  const int g = (lane >> 4) & 3, j = lane & 15;
  const int c0 = 32 * w;
  f32x16 acc = {};
#pragma unroll
  for (int kk = 0; kk < DNOPE / 16; ++kk) {
    const int n0 = 16 * kk + 8 * (g >> 1) + (j >> 2);
    const int cc = c0 + 16 * (g & 1) + 4 * (j & 3);
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, smem + n0 * WROW + cc * 2));
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, smem + (n0 + 4) * WROW + cc * 2));
    bf16x8 a;
    a.lo = __builtin_bit_cast(bf16x4, lo);
    a.hi = __builtin_bit_cast(bf16x4, hi);
    acc = mfma32(a, qb[kk], acc);
  }
  // D [32 c x 32 b]: lane holds sequence b0 + l%32, c = c0 + 8(r/4) + 4(l/32) + r%4
  if (bb < B) {
    uint16_t *dst = Q + (static_cast<size_t>(bb) * H + i) * D + 128 * cq + c0 + 4 * (lane >> 5);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      f16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = static_cast<_Float16>(acc[4 * g4 + r] * qscale);
      *reinterpret_cast<f16x4 *>(dst + 8 * g4) = v;
    }
  }
}

// ------------------------------------------------------------------ merge
// Grid (batch, H/32, d_c/32), 256 threads: sequence b, head block hb,
// latent block db (32 columns). Log-sum-exp merge of the sequence's split
// partials (base 2): o^ = sum_s 2^(lse_s - M) o^_s / sum_s 2^(lse_s - M).
// First the 32 heads' M and denominator, in one pass: thread (head h,
// part p = tid / 32) runs an online max-and-sum over splits p, p + 8, ..
// (loads issued four at a time), and the 8 parts are combined through LDS.
// Then the weighted sum: in the fragment order of the (fp16) partials the
// (hb, db) block is 2 KB contiguous per split; thread (g = tid / 64, lane)
// owns the four values at 256 g + 4 lane of it (head hl = lane % 32,
// columns 8 g + 4 (lane / 32) ..) and keeps 16 splits' loads (and their
// lse) in flight (4 for a sequence of at most 4 splits). The result goes out as bf16 hi and lo planes
// (lo = bf16(o^ - hi), about 16 significant bits), laid out
// [head][sequence][column] for the W_UV product, through an LDS transpose.
__device__ __forceinline__ void lse_combine(float &m, float &d, float m2, float d2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  d = d * exp2f(m - mn) + d2 * exp2f(m2 - mn);
  m = mn;
}
// Weighted sum over a sequence's S splits, SB loads (and their lse) in
// flight per batch; the last batch re-reads split S - 1 for its tail (in
// bounds, weight 0), so short sequences take the small batch.
template <int SB>
__device__ __forceinline__ void merge_accumulate(float4 &acc, int S, const uint16_t *src, size_t stride,
                                                 const float *lrow, int H, float M, float inv) {
  for (int s0 = 0; s0 < S; s0 += SB) {
    f16x4 x[SB];
    float l[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int s = min(s0 + u, S - 1);
      l[u] = lrow[static_cast<size_t>(s) * H];
      x[u] = *reinterpret_cast<const f16x4 *>(src + s * stride);
    }
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const float wt = s0 + u < S ? exp2f(l[u] - M) * inv : 0.0f;
      acc.x = fmaf(wt, static_cast<float>(x[u][0]), acc.x);
      acc.y = fmaf(wt, static_cast<float>(x[u][1]), acc.y);
      acc.z = fmaf(wt, static_cast<float>(x[u][2]), acc.z);
      acc.w = fmaf(wt, static_cast<float>(x[u][3]), acc.w);
    }
  }
}
__global__ __launch_bounds__(256) void merge_fast_kernel(int B, int H, const SeqInfo *__restrict__ seqs,
                                                         const int32_t *__restrict__ dev_len,
                                                         const uint16_t *__restrict__ opart,
                                                         const float *__restrict__ lse, uint16_t *__restrict__ ohat) {
  using namespace fast;
  __shared__ float tile[32 * 33];
  __shared__ float part_m[8][32], part_d[8][32];
  const int b = blockIdx.x, hb = blockIdx.y, db = blockIdx.z;
  const int tid = threadIdx.x, g = tid >> 6, lane = tid & 63, hl = lane & 31, half = lane >> 5;
  const int head = 32 * hb + hl;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const SeqInfo si = seqs[b];
  const bool live = si.item_count > 0 && dev_len[b] == si.len;  // uniform over the workgroup
  if (live) {
    const int S = si.item_count;
    const float *lcol = lse + static_cast<size_t>(si.item_begin) * H + 32 * hb;
    {
      const int h = tid & 31, p = tid >> 5;
      float m = -INFINITY, d = 0.0f;
      for (int s0 = p; s0 < S; s0 += 32) {
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int s = s0 + 8 * u;
          x[u] = s < S ? lcol[static_cast<size_t>(s) * H + h] : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) lse_combine(m, d, x[u], 1.0f);  // -inf past S adds nothing
      }
      part_m[p][h] = m;
      part_d[p][h] = d;
    }
    __syncthreads();
    float M = part_m[0][hl], den = part_d[0][hl];
#pragma unroll
    for (int p = 1; p < 8; ++p) lse_combine(M, den, part_m[p][hl], part_d[p][hl]);
    if (M != -INFINITY) {
      const float inv = 1.0f / den;
      const float *lrow = lcol + hl;
      const size_t stride = static_cast<size_t>(H / 32) * 16 * 1024;  // elements per item
      const uint16_t *src = opart + (static_cast<size_t>(si.item_begin) * (H / 32) + hb) * (16 * 1024) + 1024 * db +
                            256 * g + 4 * lane;
      if (S <= 4) merge_accumulate<4>(acc, S, src, stride, lrow, H, M, inv);
      else merge_accumulate<16>(acc, S, src, stride, lrow, H, M, inv);
    }
  }
  float *trow = tile + hl * 33 + 8 * g + 4 * half;
  trow[0] = acc.x;
  trow[1] = acc.y;
  trow[2] = acc.z;
  trow[3] = acc.w;
  __syncthreads();
  if (tid < 128) {  // head hh, 8 columns from c0
    const int hh = tid >> 2, c0 = 8 * (tid & 3);
    bf16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = tile[hh * 33 + c0 + e];
      const __bf16 h = static_cast<__bf16>(v);
      hi[e] = h;
      lo[e] = static_cast<__bf16>(v - static_cast<float>(h));
    }
    uint16_t *dh = ohat + (static_cast<size_t>(32 * hb + hh) * B + b) * DC + 32 * db + c0;
    *reinterpret_cast<bf16x8 *>(dh) = hi;
    *reinterpret_cast<bf16x8 *>(dh + static_cast<size_t>(H) * B * DC) = lo;
  }
}

// ---------------------------------------------------------------- project
// Grid (H, d_v/32, ceil(B/32)), one wave: o[b, i, v] = W_UV,i[v, :] o^[b, i, :]
// for 32 values v and 32 sequences, as D^T [32 v x 32 b] = W_UV rows (A,
// straight from global memory) times o^^T (B: the hi and lo planes, two
// products per k-step).
__global__ __launch_bounds__(64) void project_fast_kernel(int B, int H, const uint16_t *__restrict__ ohat,
                                                          const uint16_t *__restrict__ w_uv, void *o, int o_bf16) {
  using namespace fast;
  const int i = blockIdx.x, vb = blockIdx.y, b0 = blockIdx.z * 32;
  const int lane = threadIdx.x, hl = lane & 31, half = lane >> 5;
  const int b = b0 + hl;
  const uint16_t *wrow = w_uv + (static_cast<size_t>(i) * DV + 32 * vb + hl) * DC + 8 * half;
  const uint16_t *hrow = ohat + (static_cast<size_t>(i) * B + min(b, B - 1)) * DC + 8 * half;
  const uint16_t *lrow = hrow + static_cast<size_t>(H) * B * DC;
  // two batches of 16 k-steps, every load of a batch issued before its
  // products (a lone wave per output tile: the loads' latency, not the
  // matrix core, bounds the kernel)
  f32x16 acc = {};
#pragma unroll
  for (int k0 = 0; k0 < DC / 16; k0 += 16) {
    bf16x8 a[16], bh[16], bl[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      a[u] = *reinterpret_cast<const bf16x8 *>(wrow + 16 * (k0 + u));
      bh[u] = *reinterpret_cast<const bf16x8 *>(hrow + 16 * (k0 + u));
      bl[u] = *reinterpret_cast<const bf16x8 *>(lrow + 16 * (k0 + u));
    }
    __builtin_amdgcn_sched_barrier(0);  // keep all 48 loads ahead of the products
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      acc = mfma32(a[u], bh[u], acc);
      acc = mfma32(a[u], bl[u], acc);
    }
  }
  // D: lane holds sequence b0 + l%32, v = 32 vb + 8(r/4) + 4(l/32) + r%4
  if (b < B) {
    const size_t base = (static_cast<size_t>(b) * H + i) * DV + 32 * vb + 4 * half;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      if (o_bf16) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = static_cast<__bf16>(acc[4 * g4 + r]);
        *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(o) + base + 8 * g4) = v;
      } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(o) + base + 8 * g4) =
            make_float4(acc[4 * g4], acc[4 * g4 + 1], acc[4 * g4 + 2], acc[4 * g4 + 3]);
      }
    }
  }
}

// ----------------------------------------------------------------- append
// The down-projection of the new tokens, [c ; k_r] = [W_DKV ; W_KR] h ("02 —
// Multi-Latent Attention (MLA)", "La compresión de MLA"; the RoPE key
// projection, "Truco de codificación posicional"), as a K-split GEMM on the
// matrix cores. Grid (N/32, ceil(T/32), d_model/512), one wave: a 32 token x
// 32 output tile over 512 of the d_model inputs, D = h W^T with A = h rows
// (token m0 + l%32, k = 16 kk + 8(l/32) ..) and B = weight rows (output
// n0 + l%32, same k), both read straight from global memory. The fp32 tile
// goes to partial[ks][token][output]; append_finish_kernel sums the splits.
__global__ __launch_bounds__(64) void append_gemm_kernel(int T, int d_c, int d_model, const uint16_t *__restrict__ h,
                                                         const uint16_t *__restrict__ w_dkv,
                                                         const uint16_t *__restrict__ w_kr,
                                                         float *__restrict__ partial) {
  using namespace fast;
  const int nt = blockIdx.x, mt = blockIdx.y, ks = blockIdx.z;
  const int N = gridDim.x * 32;
  const int lane = threadIdx.x, l32 = lane & 31, half = lane >> 5;
  const int m = min(mt * 32 + l32, T - 1);
  const int n = nt * 32 + l32;
  const size_t k0 = static_cast<size_t>(ks) * APPEND_KS + 8 * half;
  const uint16_t *arow = h + static_cast<size_t>(m) * d_model + k0;
  const uint16_t *brow = (n < d_c ? w_dkv + static_cast<size_t>(n) * d_model
                                  : w_kr + static_cast<size_t>(n - d_c) * d_model) + k0;
  f32x16 acc = {};
#pragma unroll 8
  for (int kk = 0; kk < APPEND_KS / 16; ++kk) {
    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(arow + 16 * kk);
    const bf16x8 b = *reinterpret_cast<const bf16x8 *>(brow + 16 * kk);
    acc = mfma32(a, b, acc);
  }
  // D: lane l, register r holds token m0 + 8(r/4) + 4(l/32) + r%4, output n
  float *out = partial + static_cast<size_t>(ks) * T * N;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int mm = mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
    if (mm < T) out[static_cast<size_t>(mm) * N + n] = acc[r];
  }
}

// Grid (batch * n_new), 256 threads: token t = b n_new + j goes to row
// seq_start[b] + seq_len[b] + j at position seq_len[b] + j. Sums the K-split
// partials, rotates the k_r part at that position, rounds to the storage
// dtypes and writes the row; a sequence without room for all n_new tokens
// is left untouched and reported (MLA_ERR_CAPACITY), as on the generic path.
__global__ __launch_bounds__(256) void append_finish_kernel(mla_dims d, mla_cache c, int32_t n_new, int ksplit,
                                                            const float *__restrict__ partial,
                                                            int32_t *__restrict__ status) {
  using namespace fast;
  __shared__ float outv[APPEND_NMAX];
  __shared__ float red[4];
  const int t = blockIdx.x, T = gridDim.x;
  const int b = t / n_new, j = t - b * n_new;
  const int tid = threadIdx.x;
  const int N = d.d_c + d.d_rope;
  const int32_t len = c.seq_len[b];
  const int64_t pos = static_cast<int64_t>(len) + j;
  const int64_t row = static_cast<int64_t>(c.seq_start[b]) + pos;
  if (len < 0 || static_cast<int64_t>(len) + n_new > c.seq_cap[b] || row < 0 || row >= c.n_rows) {
    if (tid == 0 && j == 0) set_status(status, MLA_ERR_CAPACITY);
    return;
  }
  for (int n = tid; n < N; n += 256) {
    float acc = 0.0f;
    for (int ks = 0; ks < ksplit; ++ks) acc += partial[(static_cast<size_t>(ks) * T + t) * N + n];
    outv[n] = acc;
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
  store_appended_row(d, c, row, outv, red);
}

}  // namespace

bool append_fast_shape(const mla_dims &d, int32_t tokens) {
  const int n = d.d_c + d.d_rope;
  return tokens > 0 && n % 32 == 0 && n <= fast::APPEND_NMAX && d.d_model >= fast::APPEND_KS &&
         d.d_model % fast::APPEND_KS == 0;
}

bool append_fast_path(const mla_dims &d, int32_t tokens, mla_dtype act) {
  return !force_generic() && act == MLA_BF16 && append_fast_shape(d, tokens);
}

hipError_t launch_append_fast(hipStream_t s, const mla_dims &d, const mla_cache &c, const void *h, int32_t n_new,
                              const void *w_dkv, const void *w_kr, float *partial, int ksplit, int32_t *) {
  const int T = c.batch * n_new, N = d.d_c + d.d_rope;
  if (ksplit * fast::APPEND_KS != d.d_model) return hipErrorInvalidValue;
  return launch_kernel(append_gemm_kernel, dim3(N / 32, (T + 31) / 32, ksplit), 64, 0, s, T, d.d_c, d.d_model,
                       static_cast<const uint16_t *>(h), static_cast<const uint16_t *>(w_dkv),
                       static_cast<const uint16_t *>(w_kr), partial);
}

hipError_t launch_append_finish(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t n_new,
                                const float *partial, int ksplit, int32_t *status) {
  hipError_t e = launch_kernel(append_finish_kernel, c.batch * n_new, 256, 0, s, d, c, n_new, ksplit, partial, status);
  if (e != hipSuccess) return e;
  return launch_advance_len(s, c, n_new);
}

hipError_t launch_absorb_fast(hipStream_t s, const mla_dims &d, int32_t batch, const void *q_nope,
                              const void *q_rope, const int32_t *q_pos, const void *w_uk,
                              const SeqInfo *seqs, uint16_t *q_out) {
  return launch_kernel(absorb_fast_kernel, dim3(d.n_heads, fast::DC / 128, (batch + 31) / 32), 256, 0, s, batch,
                       d.n_heads, d.softmax_scale * kLog2e, d.rope_base, static_cast<const uint16_t *>(q_nope),
                       static_cast<const uint16_t *>(q_rope), q_pos, static_cast<const uint16_t *>(w_uk), seqs, q_out);
}

hipError_t launch_merge_fast(hipStream_t s, const mla_dims &d, const mla_cache &c, const SeqInfo *seqs,
                             const uint16_t *opart, const float *lse, uint16_t *ohat) {
  return launch_kernel(merge_fast_kernel, dim3(c.batch, d.n_heads / 32, fast::DC / 32), 256, 0, s, c.batch,
                       d.n_heads, seqs, c.seq_len, opart, lse, ohat);
}

hipError_t launch_project_fast(hipStream_t s, const mla_dims &d, int32_t batch, const uint16_t *ohat,
                               const void *w_uv, void *o, mla_dtype od) {
  return launch_kernel(project_fast_kernel, dim3(d.n_heads, fast::DV / 32, (batch + 31) / 32), 64, 0, s, batch,
                       d.n_heads, ohat, static_cast<const uint16_t *>(w_uv), o, od == MLA_BF16 ? 1 : 0);
}

}  // namespace mla
