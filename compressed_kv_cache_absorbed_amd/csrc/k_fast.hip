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
//   combine_fast_kernel  log-sum-exp merge of the split partials and
//                        o = W_UV o^ (the output-side absorption)
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
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
// Grid (Hr, 4), 256 threads: weight head iw, latent quarter cq (columns
// 128 cq .. +127). The quarter of W_UK,iw [128 n x 128 c] is staged in LDS
// once, with a 288-byte row stride (rows 32 bytes apart in the banks, so the
// transposed reads below are conflict-free), and serves every unit that uses
// it: the q_len query heads i = j Hr + iw (new token j) times the blocks of
// 32 sequences. Per unit it is read transposed as the A operand of
// q~^T = W_UK,iw^T q_nope^T; wave w owns columns 32 w of the quarter. The
// unit also rotates RoPE pairs 8 cq .. 8 cq + 7 of q_rope. A unit's inputs
// are loaded while the previous unit runs, and its RoPE is computed from
// them then. (One workgroup per unit instead made 2048 workgroups at 128
// sequences or four query tokens, each loading its 32 KB quarter again.)
struct AbsorbIn {
  int64_t P;     // RoPE position of this thread's pair
  uint32_t xr;   // its two q_rope values (bf16)
  bf16x8 qb[fast::DNOPE / 16];  // B operand: q_nope^T [16 n x 32 b], lane holds sequence b0 + l%32
};
__device__ __forceinline__ void absorb_load(AbsorbIn &in, int B, int H, int Hr, int q_len, int u, int nzb, int iw,
                                            int cq, int tid, const uint16_t *__restrict__ q_nope,
                                            const uint16_t *__restrict__ q_rope, const int32_t *__restrict__ q_pos,
                                            const int32_t *__restrict__ dev_len) {
  using namespace fast;
  const int j = u / nzb, b0 = (u - j * nzb) * 32;
  const int i = j * Hr + iw, back = q_len - 1 - j;
  const int lane = tid & 63;
  const int rb = b0 + (tid >> 3), rp = 8 * cq + (tid & 7);  // RoPE: sequence, pair
  in.P = 0;
  in.xr = 0;
  if (rb < B) {
    in.P = (q_pos ? q_pos[rb] : static_cast<int64_t>(dev_len[rb]) - 1) - back;
    in.xr = *reinterpret_cast<const uint32_t *>(q_rope + (static_cast<size_t>(rb) * H + i) * DR + 2 * rp);
  }
  const int bb = b0 + (lane & 31);
#pragma unroll
  for (int kk = 0; kk < DNOPE / 16; ++kk) {
    if (bb < B) {
      in.qb[kk] = *reinterpret_cast<const bf16x8 *>(q_nope + (static_cast<size_t>(bb) * H + i) * DNOPE +
                                                    16 * kk + 8 * (lane >> 5));
    } else {
      in.qb[kk] = bf16x8{};
    }
  }
}
// RoPE of pair rp = 8 cq + tid % 8 of sequence b0 + tid / 8 for query head i
// of a unit, from its loaded inputs and the pair's frequency theta.
__device__ __forceinline__ void absorb_rope(const AbsorbIn &in, int B, int H, int i, int b0, int cq, int tid,
                                            double theta, float qscale, uint16_t *__restrict__ Q,
                                            int32_t *__restrict__ status) {
  using namespace fast;
  const int rb = b0 + (tid >> 3), rp = 8 * cq + (tid & 7);
  if (rb < B) {
    float cs, sn;
    rope_cos_sin_theta(in.P, theta, &cs, &sn);
    const float x0 = bf16_bits_to_f32(static_cast<uint16_t>(in.xr & 0xffffu));
    const float x1 = bf16_bits_to_f32(static_cast<uint16_t>(in.xr >> 16));
    f16x2 r;
    const float r0 = (x0 * cs - x1 * sn) * qscale, r1 = (x0 * sn + x1 * cs) * qscale;
    if (!(fmaxf(fabsf(r0), fabsf(r1)) < kF16Max)) set_status(status, MLA_ERR_RANGE);
    r[0] = static_cast<_Float16>(r0);
    r[1] = static_cast<_Float16>(r1);
    *reinterpret_cast<f16x2 *>(Q + (static_cast<size_t>(rb) * H + i) * D + DC + 2 * rp) = r;
  }
}
__global__ __launch_bounds__(256) void absorb_fast_kernel(int B, int H, int Hr, int q_len, float qscale, float rope_base,
                                                          const uint16_t *__restrict__ q_nope,
                                                          const uint16_t *__restrict__ q_rope,
                                                          const int32_t *__restrict__ q_pos,
                                                          const uint16_t *__restrict__ w_uk,
                                                          const int32_t *__restrict__ dev_len,
                                                          uint16_t *__restrict__ Q, PlanRef plan,
                                                          int32_t *__restrict__ status) {
  using namespace fast;
  constexpr int WROW = 288;  // LDS bytes per W row (128 columns = 256 bytes + 32)
  __shared__ __attribute__((aligned(16))) char smem[DNOPE * WROW];
  const int iw = blockIdx.x, cq = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nzb = (B + 31) / 32, units = q_len * nzb;
  // the first unit's inputs, then the weight quarter (32 KB: 128 rows x 16
  // chunks of 16 bytes, 8 per thread)
  AbsorbIn in;
  absorb_load(in, B, H, Hr, q_len, 0, nzb, iw, cq, tid, q_nope, q_rope, q_pos, dev_len);
  const uint16_t *W = w_uk + static_cast<size_t>(iw) * DNOPE * DC + 128 * cq;
  u32x4 wv[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const int q = tid + 256 * x, n = q >> 4, ch = q & 15;
    wv[x] = *reinterpret_cast<const u32x4 *>(W + n * DC + 8 * ch);
  }
  // the plan copy the split-K and combine kernels read, checked while this
  // workgroup's loads are in flight (after its own work it lengthened the
  // launch by its full latency)
  if (blockIdx.x == 0 && blockIdx.y == 0) plan_verify(plan);
  // the first unit's RoPE while the weights land (this thread's pair, hence
  // its frequency, is the same in every unit)
  const double theta = rope_theta(8 * cq + (tid & 7), DR, rope_base);
  absorb_rope(in, B, H, iw, 0, cq, tid, theta, qscale, Q, status);
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const int q = tid + 256 * x, n = q >> 4, ch = q & 15;
    *reinterpret_cast<u32x4 *>(smem + n * WROW + 16 * ch) = wv[x];
  }
  __syncthreads();

  // A operand: W^T [32 c x 16 n] via transposed LDS reads of W [n][c], with
  // the same contiguous k order as the B operand: in 16-lane group g the
  // lanes take c = c0 + 16(g%2) + i and n = 16 kk + 8(g/2) + e, e = 0..3 from
  // the first read and 4..7 from the second; source lane j points at
  // W[16 kk + 8(g/2) + j/4 (+4)][c0 + 16(g%2) + 4(j%4)].
  const int g = (lane >> 4) & 3, jl = lane & 15;
  const int c0 = 32 * w;
  for (int u = 0; u < units; ++u) {
    const AbsorbIn cur = in;
    if (u + 1 < units) absorb_load(in, B, H, Hr, q_len, u + 1, nzb, iw, cq, tid, q_nope, q_rope, q_pos, dev_len);
    const int j = u / nzb, b0 = (u - j * nzb) * 32;
    const int i = j * Hr + iw;
    // (from inputs loaded one unit earlier; the first unit's ran above)
    if (u > 0) absorb_rope(cur, B, H, i, b0, cq, tid, theta, qscale, Q, status);
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < DNOPE / 16; ++kk) {
      const int n0 = 16 * kk + 8 * (g >> 1) + (jl >> 2);
      const int cc = c0 + 16 * (g & 1) + 4 * (jl & 3);
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, smem + n0 * WROW + cc * 2));
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, smem + (n0 + 4) * WROW + cc * 2));
      bf16x8 a;
      a.lo = __builtin_bit_cast(bf16x4, lo);
      a.hi = __builtin_bit_cast(bf16x4, hi);
      acc = mfma32(a, cur.qb[kk], acc);
    }
    // D [32 c x 32 b]: lane holds sequence b0 + l%32, c = c0 + 8(r/4) + 4(l/32) + r%4
    const int bb = b0 + (lane & 31);
    if (bb < B) {
      uint16_t *dst = Q + (static_cast<size_t>(bb) * H + i) * D + 128 * cq + c0 + 4 * (lane >> 5);
      float amax = 0.0f;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = acc[4 * g4 + r] * qscale;
          amax = fmaxf(amax, fabsf(x));
          v[r] = static_cast<_Float16>(x);
        }
        *reinterpret_cast<f16x4 *>(dst + 8 * g4) = v;
      }
      if (!(amax < kF16Max)) set_status(status, MLA_ERR_RANGE);
    }
  }
}

// ---------------------------------------------------------------- combine
// The log-sum-exp merge of the split partials (base 2) and the W_UV product
// ("02 — Multi-Latent Attention (MLA)", "Coste de cómputo": W_UV is applied
// to the latent-space output) in one kernel. 1-D grid of H GW workgroups,
// 512 threads (8 waves); the G = ceil(B / NB) groups of NB sequences of a
// head are dealt to its GW workgroups, each of which loads its W_UV rows once
// and then runs steps 1-3 below for each of its groups in turn (GW is set so
// that every workgroup of the launch is resident at once: with one
// workgroup per group, 128 sequences gave 1024 workgroups, four rounds of
// one per compute unit, each loading its head's weight rows again).
// Workgroup L runs on XCD L % 8 and all workgroups of one head get the same
// L % 8, so W_UV,i is fetched from HBM once and from that XCD's L2 by the
// others. The partial rows arrive whole (1 KB per load instruction), the
// W_UV rows as 64-byte pieces of 16 rows.
//   1. For each sequence b of the group: M_b = max_s lse_s and
//      den_b = sum_s 2^(lse_s - M_b), by an online max-and-sum of its
//      TPB = 512 / NB threads over splits p, p + TPB, .., combined by
//      shuffles (and across waves in LDS, in a fixed order).
//   2. o^[b] = sum_s 2^(lse_s - M_b) / den_b o^_s[b]: the partial rows are
//      512 fp16 per (item, head); each of the TPB threads of a sequence owns
//      512 / TPB columns (TPB >= 64: 8 columns, and R = TPB / 64 interleaved
//      subsets of the splits whose sums meet in LDS in a fixed order), with
//      12 or 16 splits' rows in flight, the first of them issued before
//      step 1. o^ goes to LDS as bf16 hi and lo planes
//      (lo = bf16(o^ - hi): about 16 significant bits).
//   3. o[b, i, :] = W_UV,i o^[b] as D [16 v x 16 b] = W_UV rows (A) x o^^T
//      (B, from LDS; hi and lo, two products per k-step) on
//      v_mfma_f32_16x16x32_bf16 (A: lane l holds row l%16, k = 8(l/16) ..
//      +7; B: column l%16, same k; D: lane l, register r holds row
//      4(l/16) + r, column l%16). Wave w owns values 16 w .. 16 w + 15; it
//      loads their rows straight into the A layout at the start (staging
//      them through LDS instead took 3.6 us of a 12 us workgroup).
// A sequence with no splits, or whose length no longer matches the plan,
// gets o = 0.
__device__ __forceinline__ void lse_combine(float &m, float &d, float m2, float d2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  d = d * exp2f(m - mn) + d2 * exp2f(m2 - mn);
  m = mn;
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// One batch of the weighted sum over a sequence's splits: the rows of
// splits s0, s0 + R, .. (SBX of them, NL 16-byte loads each) and their lse.
// Past the last split the batch re-reads split S - 1 (in bounds, weight 0).
template <int NL, int SBX, int R>
struct RowBatch {
  u32x4 x[SBX][NL];
  float l[SBX];
  __device__ __forceinline__ void issue(int s0, int S, const uint16_t *src, size_t stride, const float *lcol, int H) {
#pragma unroll
    for (int u = 0; u < SBX; ++u) {
      const int s = min(s0 + R * u, S - 1);
      l[u] = lcol[static_cast<size_t>(s) * H];
#pragma unroll
      for (int n = 0; n < NL; ++n) x[u][n] = *reinterpret_cast<const u32x4 *>(src + s * stride + 8 * n);
    }
  }
  __device__ __forceinline__ void consume(float (&acc)[8 * NL], int s0, int S, float M, float inv) const {
#pragma unroll
    for (int u = 0; u < SBX; ++u) {
      const float wt = s0 + R * u < S ? exp2f(l[u] - M) * inv : 0.0f;
#pragma unroll
      for (int n = 0; n < NL; ++n) {
        const f16x8 v = __builtin_bit_cast(f16x8, x[u][n]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[8 * n + e] = fmaf(wt, static_cast<float>(v[e]), acc[8 * n + e]);
      }
    }
  }
};
// EMIT: no W_UV product; o^ goes to ohat as bf16 hi and lo planes
// [B, H 512] (the precomputed-weights decode applies W_O W_UV itself).
template <int NB, bool EMIT>
__global__ __launch_bounds__(512) void combine_fast_kernel(int B, int H, int Hr, int G, int GW, int VH, int n_items,
                                                           const SeqInfo *__restrict__ seqs,
                                                           const int32_t *__restrict__ dev_len,
                                                           const uint16_t *__restrict__ opart,
                                                           const float *__restrict__ lse,
                                                           const uint16_t *__restrict__ w_uv, void *o, int o_bf16,
                                                           uint16_t *__restrict__ ohat_hi,
                                                           uint16_t *__restrict__ ohat_lo,
                                                           int32_t *__restrict__ status) {
  using namespace fast;
  constexpr int NW = 8;                            // waves
  constexpr int TPB = 64 * NW / NB;                // threads per sequence
  constexpr int R = TPB >= 64 ? TPB / 64 : 1;      // split subsets per sequence
  constexpr int CPT = TPB >= 64 ? 8 : DC / TPB;    // columns per thread: 8 or 16
  constexpr int NL = CPT / 8;                      // 16-byte loads per split
  constexpr int SB = NL == 1 ? 16 : 12;            // splits per batch (rows in flight per thread)
  constexpr int OROW = 1040;                       // LDS bytes per o^ row (conflict-free B reads)
  __shared__ __attribute__((aligned(16))) char so[2 * 16 * OROW];
  __shared__ float red_m[NW], red_d[NW];
  __shared__ __attribute__((aligned(16))) float red_acc[R > 1 ? NW : 1][DC];
  // workgroup L: head i (on XCD L % 8, with every workgroup of that head),
  // groups gs, gs + GW, .. < G of NB sequences each, output rows
  // vh * DV / VH .. +DV / VH - 1 (VH = 2 only when a workgroup per head and
  // group leaves compute units idle: the weight rows are then split between
  // two workgroups, and wave w < 8 / VH takes rows 16 w .. 16 w + 15 of that
  // half). The weight rows are loaded once for all of the workgroup's groups.
  const int L = blockIdx.x, slot = L >> 3, per_head = GW * VH;
  const int i = (L & 7) + 8 * (slot / per_head), gs = (slot % per_head) / VH, vh = slot % VH;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool wact = !EMIT && 16 * w < DV / VH;  // this wave has weight rows
  const int vrow = vh * (DV / VH) + 16 * w;
  const int bl = tid / TPB, q = tid % TPB;

  // rows vrow .. vrow + 15 of W_UV,i straight into the A layout of the
  // products: k-step kk, lane l takes row l % 16, columns 32 kk + 8 (l / 16)
  // .. +7 (each load reads 64 contiguous bytes of 16 rows; two consecutive
  // k-steps cover a 128-byte line)
  bf16x8 wa[DC / 32];
  if (wact) {
    const uint16_t *wrow = w_uv + (static_cast<size_t>(i % Hr) * DV + vrow + (lane & 15)) * DC + 8 * (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < DC / 32; ++kk) wa[kk] = *reinterpret_cast<const bf16x8 *>(wrow + 32 * kk);
  }
  // rows NB .. 15 of the B operand are zero (no group writes them)
  if (NB < 16) {
    constexpr int ZR = NB < 16 ? 16 - NB : 1;
    for (int x = tid; x < 2 * ZR * 64; x += 64 * NW) {
      const int pl = x / (ZR * 64), row = NB + (x / 64) % ZR;
      *reinterpret_cast<u32x4 *>(so + (pl * 16 + row) * OROW + 16 * (x % 64)) = u32x4{0, 0, 0, 0};
    }
  }

  const int r = TPB >= 64 ? q / 64 : 0;
  const int c0 = TPB >= 64 ? 8 * (q % 64) : CPT * q;
  const size_t stride = static_cast<size_t>(H) * DC;
  // Group g's sequence for this thread: its plan entry and device length
  // (loaded from an index clamped into the batch), then its split count S
  // and first item ib (S = 0 past the batch, or when the entry is unusable).
  struct GroupSeq {
    SeqInfo si;
    int32_t len;
  };
  auto group_seq = [&](int g) {
    const int bc = min(g * NB + bl, B - 1);
    return GroupSeq{seqs[bc], dev_len[bc]};
  };
  auto group_splits = [&](int g, const GroupSeq &x, int &S, int &ib) {
    S = 0;
    ib = 0;
    if (g * NB + bl < B) {
      // (a sequence's items must lie in the item list; the plan copy was
      // checked, so this only guards the reads below)
      const SeqInfo &si = x.si;
      const bool in_list = si.item_begin >= 0 && si.item_count >= 0 && si.item_begin <= n_items - si.item_count;
      if (!in_list && q == 0 && i == 0) set_status(status, MLA_ERR_PLAN);
      if (in_list && si.item_count > 0 && x.len == si.len) {
        S = si.item_count;
        ib = si.item_begin;
      }
    }
  };
  // a group's first loads, in the order they are needed: this thread's first
  // lse for step 1, then the first batch of partial rows for step 2
  RowBatch<NL, SB, R> rb;
  auto group_issue = [&](int S, int ib, float &l0) {
    const float *lcol = lse + static_cast<size_t>(ib) * H + i;
    l0 = q < S ? lcol[static_cast<size_t>(q) * H] : -INFINITY;
    if (r < S) rb.issue(r, S, opart + (static_cast<size_t>(ib) * H + i) * DC + c0, stride, lcol, H);
  };
  int S, ib;
  float l0;
  group_splits(gs, group_seq(gs), S, ib);
  group_issue(S, ib, l0);

  for (int g = gs; g < G; g += GW) {
    // every wave's products of the previous group have read o^ out of LDS
    if (g != gs) __syncthreads();
    const int b0 = g * NB;
    const int b = b0 + bl;
    // the next group's sequence, read now and used once this group's rows
    // are summed, when its first loads go out under this group's products
    const int gn = g + GW;
    GroupSeq nx;
    if (gn < G) nx = group_seq(gn);
    const float *lcol = lse + static_cast<size_t>(ib) * H + i;
    const uint16_t *src = opart + (static_cast<size_t>(ib) * H + i) * DC + c0;

    // 1. M_b and den_b
    float M = -INFINITY, den = 0.0f;
    lse_combine(M, den, l0, 1.0f);
    for (int s = q + TPB; s < S; s += TPB) lse_combine(M, den, lcol[static_cast<size_t>(s) * H], 1.0f);
#pragma unroll
    for (int off = 1; off < (TPB < 64 ? TPB : 64); off <<= 1) {
      const float m2 = __shfl_xor(M, off), d2 = __shfl_xor(den, off);
      lse_combine(M, den, m2, d2);  // symmetric: every lane ends with the same value
    }
    if (TPB > 64) {
      if (lane == 0) {
        red_m[w] = M;
        red_d[w] = den;
      }
      __syncthreads();
      M = red_m[bl * R];
      den = red_d[bl * R];
#pragma unroll
      for (int x = 1; x < R; ++x) lse_combine(M, den, red_m[bl * R + x], red_d[bl * R + x]);
    }

    // 2. o^[b]
    float acc[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) acc[e] = 0.0f;
    if (M != -INFINITY && r < S) {
      const float inv = 1.0f / den;
      rb.consume(acc, r, S, M, inv);
      for (int s0 = r + R * SB; s0 < S; s0 += R * SB) {
        rb.issue(s0, S, src, stride, lcol, H);
        rb.consume(acc, s0, S, M, inv);
      }
    }
    // (S, ib and l0 are not read again for this group)
    if (gn < G) {
      group_splits(gn, nx, S, ib);
      group_issue(S, ib, l0);
    }

    if (R > 1) {
      if (r > 0) {
#pragma unroll
        for (int e = 0; e < CPT; e += 4)
          *reinterpret_cast<float4 *>(&red_acc[w][c0 + e]) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
      }
      __syncthreads();
      if (r == 0) {
#pragma unroll
        for (int x = 1; x < R; ++x) {
#pragma unroll
          for (int e = 0; e < CPT; ++e) acc[e] += red_acc[w + x][c0 + e];
        }
      }
    }
    if (r == 0) {
#pragma unroll
      for (int e0 = 0; e0 < CPT; e0 += 8) {
        bf16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const __bf16 hv = static_cast<__bf16>(acc[e0 + e]);
          hi[e] = hv;
          lo[e] = static_cast<__bf16>(acc[e0 + e] - static_cast<float>(hv));
        }
        if constexpr (EMIT) {
          if (b < B) {
            const size_t off = (static_cast<size_t>(b) * H + i) * DC + c0 + e0;
            *reinterpret_cast<bf16x8 *>(ohat_hi + off) = hi;
            *reinterpret_cast<bf16x8 *>(ohat_lo + off) = lo;
          }
        } else {
          char *row = so + bl * OROW + 2 * (c0 + e0);
          *reinterpret_cast<bf16x8 *>(row) = hi;
          *reinterpret_cast<bf16x8 *>(row + 16 * OROW) = lo;
        }
      }
    }
    if constexpr (EMIT) continue;
    __syncthreads();

    // 3. o = W_UV,i o^
    f32x4 d = {};
    if (wact) {
      const char *bp = so + (lane & 15) * OROW + 16 * (lane >> 4);
#pragma unroll
      for (int kk = 0; kk < DC / 32; ++kk) {
        d = mfma16(wa[kk], *reinterpret_cast<const bf16x8 *>(bp + 64 * kk), d);
        d = mfma16(wa[kk], *reinterpret_cast<const bf16x8 *>(bp + 64 * kk + 16 * OROW), d);
      }
    }
    const int bo = b0 + (lane & 15);
    if (wact && (lane & 15) < NB && bo < B) {
      const size_t base = (static_cast<size_t>(bo) * H + i) * DV + vrow + 4 * (lane >> 4);
      if (o_bf16) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<__bf16>(d[e]);
        *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(o) + base) = v;
      } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(o) + base) = make_float4(d[0], d[1], d[2], d[3]);
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
  // two batches of 16 k-steps, every load of a batch issued before its
  // products (a lone wave per tile: the loads' latency, not the matrix core,
  // bounds it)
  f32x16 acc = {};
#pragma unroll
  for (int k0 = 0; k0 < APPEND_KS / 16; k0 += 16) {
    bf16x8 a[16], b[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      a[u] = *reinterpret_cast<const bf16x8 *>(arow + 16 * (k0 + u));
      b[u] = *reinterpret_cast<const bf16x8 *>(brow + 16 * (k0 + u));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 16; ++u) acc = mfma32(a[u], b[u], acc);
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
// With one new token per sequence (advance) the sequence's only workgroup
// also adds it to seq_len once the row is written (no other workgroup reads
// that length); with several, advance_len_kernel does it afterwards.
__global__ __launch_bounds__(256) void append_finish_kernel(mla_dims d, mla_cache c, int32_t n_new, int ksplit, bool advance,
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
  const int32_t chk = append_check(c, b, len, n_new);
  if (chk != MLA_OK) {
    if (tid == 0 && j == 0) set_status(status, chk);
    return;
  }
  bool bad = false;
  const int64_t row = cache_row(c, b, pos, bad);  // (every block was checked)
  // the K-split partials, up to 16 loads in flight per output
  for (int n = tid; n < N; n += 256) {
    float acc = 0.0f;
    for (int k0 = 0; k0 < ksplit; k0 += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        v[u] = k0 + u < ksplit ? partial[(static_cast<size_t>(k0 + u) * T + t) * N + n] : 0.0f;
#pragma unroll
      for (int u = 0; u < 16; ++u) acc += v[u];
    }
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
  store_appended_row(d, c, row, outv, red, status);
  if (advance && tid == 0) c.seq_len[b] = len + 1;
}

}  // namespace

bool append_fast_shape(const mla_dims &d, int32_t tokens) {
  const int n = d.d_c + d.d_rope;
  return tokens > 0 && n % 32 == 0 && n <= fast::APPEND_NMAX && d.d_model >= fast::APPEND_KS &&
         d.d_model % fast::APPEND_KS == 0;
}

int append_fast_ksplit(const mla_dims &d) { return d.d_model / fast::APPEND_KS; }

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
  const bool advance = n_new == 1;
  hipError_t e =
      launch_kernel(append_finish_kernel, c.batch * n_new, 256, 0, s, d, c, n_new, ksplit, advance, partial, status);
  if (e != hipSuccess || advance) return e;
  return launch_advance_len(s, c, n_new);
}

hipError_t launch_absorb_fast(hipStream_t s, const mla_dims &d, int32_t batch, int32_t q_len, const void *q_nope,
                              const void *q_rope, const int32_t *q_pos, const void *w_uk,
                              const int32_t *seq_len, uint16_t *q_out, const PlanRef &plan,
                              int32_t *status) {
  const int H = d.n_heads * q_len;
  return launch_kernel(absorb_fast_kernel, dim3(d.n_heads, fast::DC / 128), 256, 0, s, batch, H,
                       d.n_heads, q_len, d.softmax_scale * kLog2e, d.rope_base, static_cast<const uint16_t *>(q_nope),
                       static_cast<const uint16_t *>(q_rope), q_pos, static_cast<const uint16_t *>(w_uk), seq_len, q_out, plan, status);
}

// Workgroups per head (and weight half) of the combine: G groups dealt to at
// most one workgroup per compute unit over the launch (its 8 waves of ~250
// registers fill a unit), so that all of them are resident at once.
static int combine_workgroups_per_head(int heads, int G) {
  constexpr int kSlots = 256;
  const int per_head = kSlots / heads > 1 ? kSlots / heads : 1;
  return G < per_head ? G : per_head;
}

hipError_t launch_combine_fast(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t q_len, int32_t n_items,
                               const SeqInfo *seqs, const uint16_t *opart, const float *lse, const uint16_t *w_uv,
                               void *o, int o_bf16, int32_t *status) {
  const int B = c.batch, H = d.n_heads * q_len;
  if (B == 0) return hipSuccess;
  // the largest group (up to the 16 columns of one product) that still
  // gives a workgroup to every compute unit
  int nb = 1;
  while (nb < 16 && static_cast<int64_t>(H) * ((B + 2 * nb - 1) / (2 * nb)) >= 256) nb *= 2;
  const int G = (B + nb - 1) / nb;
  // still fewer workgroups than compute units (one sequence): split each
  // head's weight rows over two workgroups
  const int VH = static_cast<int64_t>(H) * G < 256 ? 2 : 1;
  const int GW = combine_workgroups_per_head(H * VH, G);
  const dim3 grid(H * GW * VH);
#define MLA_COMBINE(NBV)                                                                                          \
  case NBV:                                                                                                      \
    return launch_kernel(combine_fast_kernel<NBV, false>, grid, 512, 0, s, B, H, d.n_heads, G, GW, VH, n_items, \
                         seqs, c.seq_len, opart, lse, w_uv, o, o_bf16, nullptr, nullptr, status)
  switch (nb) {
    MLA_COMBINE(1);
    MLA_COMBINE(2);
    MLA_COMBINE(4);
    MLA_COMBINE(8);
    default:
      MLA_COMBINE(16);
  }
#undef MLA_COMBINE
}

hipError_t launch_combine_fast_emit(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t n_items,
                                    const SeqInfo *seqs, const uint16_t *opart, const float *lse, uint16_t *ohat_hi,
                                    uint16_t *ohat_lo, int32_t *status) {
  const int B = c.batch, H = d.n_heads;
  if (B == 0) return hipSuccess;
  int nb = 1;
  while (nb < 16 && static_cast<int64_t>(H) * ((B + 2 * nb - 1) / (2 * nb)) >= 256) nb *= 2;
  const int G = (B + nb - 1) / nb;
  const int GW = combine_workgroups_per_head(H, G);
  const dim3 grid(H * GW);
#define MLA_COMBINE(NBV)                                                                                          \
  case NBV:                                                                                                      \
    return launch_kernel(combine_fast_kernel<NBV, true>, grid, 512, 0, s, B, H, d.n_heads, G, GW, 1, n_items,   \
                         seqs, c.seq_len, opart, lse, nullptr, nullptr, 0, ohat_hi, ohat_lo, status)
  switch (nb) {
    MLA_COMBINE(1);
    MLA_COMBINE(2);
    MLA_COMBINE(4);
    MLA_COMBINE(8);
    default:
      MLA_COMBINE(16);
  }
#undef MLA_COMBINE
}

}  // namespace mla
