// Decode from precomputed absorbed weights. The up-projections are folded
// into the query and output projections ahead of time ("02 — Multi-Latent
// Attention (MLA)", "Coste de cómputo": some matrix products precomputed so
// attention works from the latent directly; "Atención latente de múltiples
// cabezas", "Información técnica": the up-projection weights absorbed into
// the query and output projections; "Multi-head Latent Attention (MLA) și
// arhitectura DeepSeekMoE", opening paragraph). The rotary query part cannot
// be folded and stays an input.
//
//   A_i = W_UK,i^T W_Q,i   [H, d_c, d_x]      q~_i = A_i x
//   Bm  = [W_O,i W_UV,i]_i [d_out, H d_c]     y = Bm [o^_1; ..; o^_H]
//
// Kernels:
//   merge_gemm_kernel      C[t] = P[t]^T Q[t] for strided operands, fp32
//                          accumulation: the one-time products A and Bm
//   wstream_kernel         Y = W X^T for a bf16 weight W [rows x K] and up to
//                          32 activation columns on the matrix cores; the
//                          weight streams from HBM once. Epilogues: the
//                          absorbed query (fp16, the split-K kernel's layout,
//                          with the rotary part) or fp32 K-split partials
//   wsum_kernel            y = sum of the K-split partials
//   absorb_merged_generic_kernel, out_generic_kernel   fp32 forms, any shape
// The split-K decode between them is the one every decode uses; the combine
// kernels emit o^ instead of applying W_UV.
#include "device_util.hpp"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

// ------------------------------------------------------------ merge GEMM
// Grid (ceil(N/64), ceil(M/64), T), 256 threads: a 64 x 64 tile of C[t],
// k in steps of 16 through LDS; thread (ty, tx) = (tid / 16, tid % 16) owns
// rows 4 ty .. +3 and columns 4 tx .. +3.
__global__ __launch_bounds__(256) void merge_gemm_kernel(int M, int N, int K, const void *P, int64_t sPt, int64_t sPk,
                                                         int64_t sPm, const void *Q, int64_t sQt, int64_t sQk,
                                                         int64_t sQn, mla_dtype in, void *C, int64_t sCt,
                                                         int64_t sCm, int64_t sCn, mla_dtype out, int64_t tileK) {
  __shared__ float ps[16][65], qs[16][65];
  const int t = blockIdx.z, m0 = 64 * blockIdx.y, n0 = 64 * blockIdx.x;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = tid; e < 16 * 64; e += 256) {
      const int kk = e >> 6, mm = e & 63, k = k0 + kk;
      ps[kk][mm] = (k < K && m0 + mm < M) ? load_elem(P, t * sPt + k * sPk + (m0 + mm) * sPm, in) : 0.0f;
      qs[kk][mm] = (k < K && n0 + mm < N) ? load_elem(Q, t * sQt + k * sQk + (n0 + mm) * sQn, in) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ps[kk][4 * ty + i], qs[kk][4 * tx + j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * ty + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 4 * tx + j;
      if (n >= N) continue;
      int64_t off = t * sCt + m * sCm + n * sCn;
      if (tileK > 0) off = merged::weight_off(off / tileK, off % tileK, tileK, true);
      if (out == MLA_BF16)
        static_cast<uint16_t *>(C)[off] = f32_to_bf16_bits(acc[i][j]);
      else
        static_cast<float *>(C)[off] = acc[i][j];
    }
  }
}

// ------------------------------------------------------- weight stream
// Y[b][r] = sum_k W[r][k] X[b][k] on v_mfma_f32_32x32x16_bf16 (A: lane l
// holds row l%32, 8 k; B: lane l holds column l%32, the same 8 k; D: lane
// l, register j holds row 8(j/4) + 4(l/32) + j%4, column l%32). The k order
// inside a product is free as long as A and B agree: in a step of 64 k the
// lanes of half h = l/32 read 32 consecutive k (64 contiguous bytes of a
// weight row), and product f of the step takes k = 32 h + 8 f .. +7 from
// both operands.
//
// 1-D grid of NRG * KS * NBB workgroups of 4 waves: row group rg (32 NR
// rows), K split ks (kchunk columns), batch block bb (32 columns of X).
// With KS a multiple of 8 every workgroup of one split runs on the same XCD
// (workgroup L on XCD L % 8), so that split's slice of X stays in one L2.
// Wave w takes k = ks kchunk + w kchunk/4 .. +kchunk/4 for all NR row
// blocks; the four waves' sums meet in LDS and wave w finishes row block w.
// X is given as bf16 planes: hi, and with LO also lo = the rounding rest of
// an fp32 activation (two products per step).
enum Epi : int { EPI_QUERY = 0, EPI_PARTIAL = 1 };

struct QueryEpi {  // the absorbed query in the split-K kernel's layout
  int H;
  float qscale, rope_base;
  const uint16_t *q_rope;  // [B, H, 64] bf16, unrotated
  const int32_t *q_pos;    // [B] or null: seq_len - 1
  const int32_t *seq_len;
  uint16_t *Q;             // [B, H, 576] fp16
  PlanRef plan;
  int32_t *status;
};
struct PartialEpi {
  float *part;  // [KS, B, rows] fp32
};

template <int NR, bool LO, int EPI>
__global__ __launch_bounds__(256) void wstream_kernel(int R, int K, int B, int kchunk, int NRG, int KS,
                                                      const uint16_t *__restrict__ W,
                                                      const uint16_t *__restrict__ Xhi,
                                                      const uint16_t *__restrict__ Xlo, QueryEpi qe,
                                                      PartialEpi pe) {
  static_assert(NR == 4, "wave w finishes row block w");
  __shared__ __attribute__((aligned(16))) float red[4][NR][16][64];  // [wave][block][register][lane]
  const int L = blockIdx.x;
  int ks, rest;
  if (KS % 8 == 0) {
    const int slot = L >> 3;
    ks = (L & 7) + 8 * (slot % (KS / 8));
    rest = slot / (KS / 8);
  } else {
    ks = L % KS;
    rest = L / KS;
  }
  const int rg = rest % NRG, bb = rest / NRG;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5;
  const int row0 = 32 * NR * rg, b0 = 32 * bb;
  const int bcol = b0 + (lane & 31);
  const bool bval = bcol < B;
  const int kw = kchunk / 4, kbeg = ks * kchunk + w * kw;

  // the weight is fragment-tiled (merged::weight_off): row block r, step s
  // is 2048 contiguous elements, product f of it 512, this lane's 8 at 8 lane
  const uint16_t *wp[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r)
    wp[r] = W + (static_cast<size_t>(row0 / 32 + r) * (K / 64) + kbeg / 64) * 2048 + 8 * lane;
  // columns past B read column b0's data (in bounds) and are zeroed by a select
  const size_t xrow = static_cast<size_t>(bval ? bcol : b0) * K + kbeg + 32 * h;
  const uint16_t *xh = Xhi + xrow;
  const uint16_t *xl = LO ? Xlo + xrow : nullptr;
  constexpr int NX = LO ? 8 : 4;

  f32x16 acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = f32x16{};
  // two named register stages, so the next step's loads are in flight while
  // this step's products run
  u32x4 a0[NR][4], a1[NR][4], x0[NX], x1[NX];
  auto load = [&](u32x4(&a)[NR][4], u32x4(&xv)[NX], int s) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int f = 0; f < 4; ++f) a[r][f] = *reinterpret_cast<const u32x4 *>(wp[r] + 2048 * s + 512 * f);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      xv[f] = *reinterpret_cast<const u32x4 *>(xh + 64 * s + 8 * f);
      if (LO) xv[4 + f] = *reinterpret_cast<const u32x4 *>(xl + 64 * s + 8 * f);
    }
  };
  auto compute = [&](const u32x4(&a)[NR][4], const u32x4(&xv)[NX]) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const bf16x8 bh = __builtin_bit_cast(bf16x8, bval ? xv[f] : u32x4{0, 0, 0, 0});
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, a[r][f]);
        acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bh, acc[r], 0, 0, 0);
        if (LO) {
          const bf16x8 bl = __builtin_bit_cast(bf16x8, bval ? xv[4 + f] : u32x4{0, 0, 0, 0});
          acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bl, acc[r], 0, 0, 0);
        }
      }
    }
  };
  // kw is a multiple of 128 (an even number of steps), so the loop body has
  // no branch and the waits stay counted: a stage's data is waited for with
  // the other stage's loads still in flight (past the end the prefetch
  // re-reads the last step, from L2); scheduling barriers keep the four
  // phases in this order
  const int nsteps = kw / 64;
  load(a0, x0, 0);
  for (int s = 0; s < nsteps; s += 2) {
    load(a1, x1, s + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(a0, x0);
    __builtin_amdgcn_sched_barrier(0);
    load(a0, x0, min(s + 2, nsteps - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(a1, x1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the four waves' partial sums: wave w finishes row block w
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int j = 0; j < 16; ++j) red[w][r][j][lane] = acc[r][j];
  __syncthreads();
  float v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = red[0][w][j][lane] + red[1][w][j][lane] + red[2][w][j][lane] + red[3][w][j][lane];
  const int rb = row0 + 32 * w;  // this wave's row block

  if constexpr (EPI == EPI_PARTIAL) {
    if (bval) {
      float *dst = pe.part + (static_cast<size_t>(ks) * B + bcol) * R + rb + 4 * h;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4 *>(dst + 8 * g4) = make_float4(v[4 * g4], v[4 * g4 + 1], v[4 * g4 + 2], v[4 * g4 + 3]);
    }
  } else {
    constexpr int DC = 512, DR = 64, D = DC + DR;
    const int i = rb / DC, c0 = rb % DC;
    if (bval) {
      uint16_t *dst = qe.Q + (static_cast<size_t>(bcol) * qe.H + i) * D + c0 + 4 * h;
      float amax = 0.0f;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f16x4 q;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = v[4 * g4 + e] * qe.qscale;
          amax = fmaxf(amax, fabsf(x));
          q[e] = static_cast<_Float16>(x);
        }
        *reinterpret_cast<f16x4 *>(dst + 8 * g4) = q;
      }
      if (!(amax < kF16Max)) set_status(qe.status, MLA_ERR_RANGE);
    }
    // the rotary part: the first row group of each head rotates its 32
    // pairs for the batch block's sequences (4 per thread)
    if (row0 % DC == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = tid + 256 * u, b = b0 + (e >> 5), p = e & 31;
        if (b >= B) continue;
        const int64_t P = qe.q_pos ? qe.q_pos[b] : static_cast<int64_t>(qe.seq_len[b]) - 1;
        const uint32_t xr =
            *reinterpret_cast<const uint32_t *>(qe.q_rope + (static_cast<size_t>(b) * qe.H + i) * DR + 2 * p);
        float cs, sn;
        rope_cos_sin(P, p, DR, qe.rope_base, &cs, &sn);
        const float x0 = bf16_bits_to_f32(static_cast<uint16_t>(xr & 0xffffu));
        const float x1 = bf16_bits_to_f32(static_cast<uint16_t>(xr >> 16));
        const float r0 = (x0 * cs - x1 * sn) * qe.qscale, r1 = (x0 * sn + x1 * cs) * qe.qscale;
        if (!(fmaxf(fabsf(r0), fabsf(r1)) < kF16Max)) set_status(qe.status, MLA_ERR_RANGE);
        f16x2 q;
        q[0] = static_cast<_Float16>(r0);
        q[1] = static_cast<_Float16>(r1);
        *reinterpret_cast<f16x2 *>(qe.Q + (static_cast<size_t>(b) * qe.H + i) * D + DC + 2 * p) = q;
      }
    }
    // the plan copy the split-K and combine kernels read
    if (L == 0) plan_verify(qe.plan);
  }
}

// y[b][r] = sum over the KS splits of part[ks][b][r]; n4 = B * rows / 4.
__global__ __launch_bounds__(256) void wsum_kernel(const float *__restrict__ part, int KS, size_t n4, void *y,
                                                   int y_bf16) {
  for (size_t e = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; e < n4; e += static_cast<size_t>(gridDim.x) * 256) {
    float4 s = reinterpret_cast<const float4 *>(part)[e];
    for (int k = 1; k < KS; ++k) {
      const float4 t = reinterpret_cast<const float4 *>(part)[k * n4 + e];
      s.x += t.x;
      s.y += t.y;
      s.z += t.z;
      s.w += t.w;
    }
    if (y_bf16) {
      uint16_t *o = static_cast<uint16_t *>(y) + 4 * e;
      o[0] = f32_to_bf16_bits(s.x);
      o[1] = f32_to_bf16_bits(s.y);
      o[2] = f32_to_bf16_bits(s.z);
      o[3] = f32_to_bf16_bits(s.w);
    } else {
      reinterpret_cast<float4 *>(y)[e] = s;
    }
  }
}

// ------------------------------------------------------- generic (fp32)
// Grid (B, H), 256 threads: q~ = A_i x_b (one wave per latent column, lanes
// over d_x, x staged in LDS), the rotary part, all times softmax_scale log2 e.
__global__ __launch_bounds__(256) void absorb_merged_generic_kernel(mla_dims d, int d_x, const void *x,
                                                                    const void *q_rope, const int32_t *q_pos,
                                                                    const void *a, mla_dtype wt,
                                                                    const int32_t *seq_len, float *q_out,
                                                                    PlanRef plan) {
  extern __shared__ float xs[];  // [d_x]
  const int b = blockIdx.x, i = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = d.n_heads, D = d.d_c + d.d_rope;
  for (int k = tid; k < d_x; k += 256) xs[k] = load_elem(x, static_cast<int64_t>(b) * d_x + k, wt);
  __syncthreads();
  const float qs = d.softmax_scale * kLog2e;
  float *out = q_out + (static_cast<int64_t>(b) * H + i) * D;
  const bool tl = merged::tiled(static_cast<int64_t>(H) * d.d_c, d_x);
  for (int c = wave; c < d.d_c; c += 4) {
    const int64_t row = static_cast<int64_t>(i) * d.d_c + c;
    float acc = 0.0f;
    for (int k = lane; k < d_x; k += 64) acc = fmaf(load_elem(a, merged::weight_off(row, k, d_x, tl), wt), xs[k], acc);
    acc = wave_sum(acc);
    if (lane == 0) out[c] = acc * qs;
  }
  const int64_t bi = static_cast<int64_t>(b) * H + i;
  const int64_t P = q_pos ? q_pos[b] : static_cast<int64_t>(seq_len[b]) - 1;
  for (int p = tid; p < d.d_rope / 2; p += 256) {
    float cs, sn;
    rope_cos_sin(P, p, d.d_rope, d.rope_base, &cs, &sn);
    const float x0 = load_elem(q_rope, bi * d.d_rope + 2 * p, wt);
    const float x1 = load_elem(q_rope, bi * d.d_rope + 2 * p + 1, wt);
    out[d.d_c + 2 * p] = (x0 * cs - x1 * sn) * qs;
    out[d.d_c + 2 * p + 1] = (x0 * sn + x1 * cs) * qs;
  }
  if (blockIdx.x == 0 && blockIdx.y == 0) plan_verify(plan);
}

// Grid (ceil(d_out / 4), B), 256 threads: one wave per output row,
// y[b][r] = Bm[r] . o^[b] over K = H d_c.
__global__ __launch_bounds__(256) void out_generic_kernel(int d_out, int64_t K, const void *bm, mla_dtype wt,
                                                          const float *ohat, void *y, mla_dtype yt) {
  const int b = blockIdx.y, r = 4 * blockIdx.x + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= d_out) return;
  const float *o = ohat + static_cast<int64_t>(b) * K;
  const bool tl = merged::tiled(d_out, K);
  float acc = 0.0f;
  for (int64_t k = lane; k < K; k += 64) acc = fmaf(load_elem(bm, merged::weight_off(r, k, K, tl), wt), o[k], acc);
  acc = wave_sum(acc);
  if (lane == 0) {
    const int64_t off = static_cast<int64_t>(b) * d_out + r;
    if (yt == MLA_BF16)
      static_cast<uint16_t *>(y)[off] = f32_to_bf16_bits(acc);
    else
      static_cast<float *>(y)[off] = acc;
  }
}

}  // namespace

// ---------------------------------------------------------------- launchers

hipError_t launch_merge_gemm(hipStream_t s, int T, int M, int N, int K, const void *P, int64_t sPt, int64_t sPk,
                             int64_t sPm, const void *Q, int64_t sQt, int64_t sQk, int64_t sQn, mla_dtype in, void *C,
                             int64_t sCt, int64_t sCm, int64_t sCn, mla_dtype out, int64_t tileK) {
  if (T == 0 || M == 0 || N == 0) return hipSuccess;
  return launch_kernel(merge_gemm_kernel, dim3((N + 63) / 64, (M + 63) / 64, T), 256, 0, s, M, N, K, P, sPt, sPk, sPm,
                       Q, sQt, sQk, sQn, in, C, sCt, sCm, sCn, out, tileK);
}

hipError_t launch_absorb_merged_fast(hipStream_t s, const mla_dims &d, int32_t batch, int32_t d_x, const void *x,
                                     const void *q_rope, const int32_t *q_pos, const void *a,
                                     const int32_t *seq_len, uint16_t *q_out, const PlanRef &plan, int32_t *status) {
  if (batch == 0) return hipSuccess;
  const int R = d.n_heads * merged::DC, NRG = R / 128, NBB = (batch + 31) / 32;
  QueryEpi qe{d.n_heads, d.softmax_scale * kLog2e, d.rope_base, static_cast<const uint16_t *>(q_rope), q_pos,
              seq_len, q_out, plan, status};
  return launch_kernel(wstream_kernel<4, false, EPI_QUERY>, dim3(NRG * NBB), 256, 0, s, R, d_x, batch, d_x, NRG, 1,
                       static_cast<const uint16_t *>(a), static_cast<const uint16_t *>(x), nullptr, qe,
                       PartialEpi{nullptr});
}

hipError_t launch_out_merged_fast(hipStream_t s, int32_t batch, int32_t d_out, int64_t K, const void *bm,
                                  const uint16_t *ohat_hi, const uint16_t *ohat_lo, float *part, void *y, int y_bf16) {
  if (batch == 0) return hipSuccess;
  const int KS = merged::out_splits(K), NRG = d_out / 128, NBB = (batch + 31) / 32;
  const int kchunk = static_cast<int>(K / KS);
  QueryEpi qe{};
  hipError_t e = launch_kernel(wstream_kernel<4, true, EPI_PARTIAL>, dim3(NRG * KS * NBB), 256, 0, s, d_out,
                               static_cast<int>(K), batch, kchunk, NRG, KS, static_cast<const uint16_t *>(bm), ohat_hi,
                               ohat_lo, qe, PartialEpi{part});
  if (e != hipSuccess) return e;
  const size_t n4 = static_cast<size_t>(batch) * d_out / 4;
  const int grid = static_cast<int>(std::min<size_t>((n4 + 255) / 256, 2048));
  return launch_kernel(wsum_kernel, grid, 256, 0, s, part, KS, n4, y, y_bf16);
}

hipError_t launch_absorb_merged_generic(hipStream_t s, const mla_dims &d, int32_t batch, int32_t d_x, const void *x,
                                        const void *q_rope, const int32_t *q_pos, const void *a, mla_dtype wt,
                                        const int32_t *seq_len, float *q_out, const PlanRef &plan) {
  if (batch == 0) return hipSuccess;
  return launch_kernel(absorb_merged_generic_kernel, dim3(batch, d.n_heads), 256, sizeof(float) * d_x, s, d, d_x, x,
                       q_rope, q_pos, a, wt, seq_len, q_out, plan);
}

hipError_t launch_out_merged_generic(hipStream_t s, int32_t batch, int32_t d_out, int64_t K, const void *bm,
                                     mla_dtype wt, const float *ohat, void *y, mla_dtype yt) {
  if (batch == 0 || d_out == 0) return hipSuccess;
  return launch_kernel(out_generic_kernel, dim3((d_out + 3) / 4, batch), 256, 0, s, d_out, K, bm, wt, ohat, y, yt);
}

}  // namespace mla
