// Split-K flash-decode over an fp8 (e4m3) latent cache on the fp8 matrix
// cores ("Multi-head Latent Attention (MLA) și arhitectura DeepSeekMoE",
// "Exemplul 1": the cache stored in fp8). Same decomposition as the bf16
// kernel with the value product split by heads: one workgroup per range of
// work items and 128 heads (the items one after the other), wave w owns
// heads 32 w .. 32 w + 31. Per tile of 32 tokens
//   S^T [32 tok x 32 heads]   = scale_t (codes [32 x 512] q~^T) + k_rope q_r^T
//   online softmax per head, base 2
//   O^T [512 x 32 heads]     += codes^T [512 x 32 tok] (P scale_t)^T
// with the cached e4m3 codes read straight from the copied rows: no
// widening pass.
//
// Arithmetic (v_mfma_scale_f32_32x32x64_f8f6f4: e4m3 operands, fp32
// accumulation, one E8M0 power-of-two scale per operand row or column and
// 32-wide block of k):
// * q~ (fp16 in the workspace) becomes a pair of e4m3 values per element,
//   hi = e4m3(q~ 2^-E) and lo = e4m3(16 (q~ 2^-E - hi)), with E the least
//   power of two that brings the head's largest |q~| to 448 or below; the
//   score takes two products, scaled 2^E and 2^(E-4) (about 8 significant
//   bits together).
// * A token's scale s_t = m_t 2^e_t (m_t in [1, 2)): 2^e_t is the codes'
//   block scale, the k_rope operand is divided by m_t, and the fp32 sum of
//   both products is multiplied by m_t.
// * P s_t of each head over a tile becomes a hi + lo pair the same way (one
//   power of two per head and tile), hi in the first 32-wide k block and lo
//   in the second, each against the same codes: one product per 32 latent
//   columns.
// Matrix-core time equals the fp16 products' (twice the rate, twice the
// products); the operand bytes read from LDS halve and the widening pass
// goes. Errors against the oracle stay well inside the fp8 tolerance (the
// emulation of exactly this arithmetic, and the GPU tests).
//
// Operand layouts (measured on the hardware): lane l holds row / column
// l % 32 and 32 bytes of k; bytes 0..15 of lanes l and l + 32 form k-block 0
// of that row, bytes 16..31 k-block 1; lane l + 32 b supplies the scale of
// row l % 32, block b. D as for the fp16 products: lane l, register r holds
// row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
// ds_read_b64_tr_b8: in each 16-lane group, lane i receives byte i % 8 of
// the 8-byte rows addressed by source lanes 2 e + i / 8, e = 0..7.
//
// LDS: four raw tiles (32 rows of 640 bytes: 512 codes and 64 bf16 k_rope,
// the 16-byte chunks of row t permuted by rsw8(t) so that every fragment
// read is free of bank conflicts) and per-wave copies of each tile's 32
// scales. Pipeline per step i: score products of tile i+1 with the softmax
// of tile i woven between them, then the value products of tile i with the
// copies of tile i+3 issued under them (the wave mostly waits on the matrix
// cores there: a step takes about 6600 cycles, against 7400 with the copies
// under the score products), then one barrier.
#include <cmath>

#include "device_util.hpp"
#include "splitk_addr.hpp"
#include "splitk_common.hpp"

namespace mla {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

namespace s8 {
constexpr int DC = 512, D = 576;
constexpr int T = kTile;              // 32 tokens per tile
constexpr int ROWB = 640;             // raw row: 512 codes + 128 bytes of k_rope
constexpr int TILE = T * ROWB;        // 20480
constexpr int NBUF = 4;
constexpr int SLACK = 8;              // running max kept unless exceeded by 2^8
constexpr int VPF = 4;                // value fragments read ahead of their product
constexpr int VBLK = 15;              // the output block kept in VGPRs (its AGPRs hold the scores)
constexpr int OROW = 1040;            // partial row stride of the closing transpose (bytes)
constexpr int raw(int b) { return TILE * b; }
constexpr int scl(int b, int w) { return TILE * NBUF + 1024 * b + 256 * w; }
constexpr int DATA_END = scl(NBUF, 0);
constexpr int LDS_BYTES = 4 * 32 * OROW > DATA_END ? 4 * 32 * OROW : DATA_END;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert(ROWB == sa::RAW_ROWB && T == sa::T, "tile geometry shared with the copy addresses");
}  // namespace s8

__shared__ __attribute__((aligned(1024))) char g_lds8[s8::LDS_BYTES];

namespace {

using sa::Item;
using sa::RawSrc;
using sa::raw_src;
using sa::rsw8;
using sa::tile_src;

__device__ __forceinline__ f32x16 mma8(i32x8 a, i32x8 b, f32x16 c, int sa_, int sb_) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa_, 0, sb_);
}
// The same product accumulating in AGPRs (the builtin keeps its accumulator
// in VGPRs, and the output blocks live in AGPRs). The compiler does not see
// into the asm, so the s_nop covers vector-ALU writes of the operands just
// before it (the weights, the duplicated value fragment, the rescaled
// accumulator); reads of the accumulators after the last product are covered
// where the partials are written.
__device__ __forceinline__ void mma8_acc(f32x16 &c, i32x8 a, i32x8 b, int sa_, int sb_) {
  asm volatile("s_nop 4\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4"
               : "+a"(c)
               : "v"(a), "v"(b), "v"(sa_), "v"(sb_));
}
// The output block kept in VGPRs (its AGPRs hold the scores).
__device__ __forceinline__ void mma8_acc_v(f32x16 &c, i32x8 a, i32x8 b, int sa_, int sb_) {
  asm volatile("s_nop 4\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4"
               : "+v"(c)
               : "v"(a), "v"(b), "v"(sa_), "v"(sb_));
}
// The chain's first product, from a zero accumulator.
__device__ __forceinline__ void mma8_first(f32x16 &c, i32x8 a, i32x8 b, int sa_, int sb_) {
  c = f32x16{};
  asm volatile("" : "+a"(c));
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4"
               : "+a"(c)
               : "v"(a), "v"(b), "v"(sa_), "v"(sb_));
}
// A score product in the AGPR chain: its operands are the query registers
// (set when the item starts), LDS reads (waited for by the compiler) and
// the token's block scale (computed before the chain's first four
// products), so no vector-ALU write precedes it closely.
__device__ __forceinline__ void mma8_chain(f32x16 &c, i32x8 a, i32x8 b, int sa_, int sb_) {
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4"
               : "+a"(c)
               : "v"(a), "v"(b), "v"(sa_), "v"(sb_));
}
__device__ __forceinline__ f32x16 mma16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// A positive float as s = m 2^e: the E8M0 code of 2^e (its biased exponent)
// and m in [1, 2). (Cache scales are positive normals.)
__device__ __forceinline__ int e8m0_of(float s) { return static_cast<int>((__float_as_uint(s) >> 23) & 0xffu); }
__device__ __forceinline__ float mant_of(float s) { return __uint_as_float((__float_as_uint(s) & 0x007fffffu) | 0x3f800000u); }

// The least E with amax 2^-E <= 448 (amax >= 0; 0 gives -9).
__device__ __forceinline__ int pow2_for_448(float amax) {
  int e;
  const float f = frexpf(amax, &e);  // amax = f 2^e, f in [0.5, 1)
  return f <= 0.875f ? e - 9 : e - 8;
}

// Four values x (already scaled into [-448, 448]) to e4m3 hi and
// lo = e4m3(16 (x - hi)), packed four to a dword.
__device__ __forceinline__ void hilo4(float x0, float x1, float x2, float x3, uint32_t &hi, uint32_t &lo) {
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, hi, true);
  const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (x0 - h01[0]), 16.0f * (x1 - h01[1]), 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (x2 - h23[0]), 16.0f * (x3 - h23[1]), lo, true);
}

// Raw tile copy, 6 loads per wave: x < 5 copies 1 KB of wave w's rows into
// the permuted layout (slot P = 64 (5 w + x) + lane), x = 5 the tile's 32
// scales into wave w's own copy (lanes 32..63 repeat lanes 0..31).
template <int R>
__device__ __forceinline__ void dma8_piece(const RawSrc &rs, int w, int lane, int x) {
  const uint32_t lds0 = LDS_OFF(g_lds8);
  const int ln = opaque(lane);
  if (x < sa::RAW_DMA_PER_WAVE) {
    const int q = sa::RAW_DMA_PER_WAVE * w + x;
    lds_dma16(rs.base, sa::raw_piece_off_sw(rs, w, ln, x), __builtin_amdgcn_readfirstlane(lds0 + s8::raw(R) + 1024u * q));
  } else {
    lds_dma4(rs.sbase, sa::raw_scale_off(rs, ln), __builtin_amdgcn_readfirstlane(lds0 + s8::scl(R, 0) + 256u * w));
  }
}
// The same copy with the per-lane constants of the item (sa::RawLane),
// offset from the tile's first row tbase: the form the steps issue.
template <int R>
__device__ __forceinline__ void dma8_piece_lane(const RawSrc &rs, const char *tbase, const sa::RawLane &rl, int w,
                                                int lane, int x) {
  if (x < sa::RAW_DMA_PER_WAVE) {
    const int q = sa::RAW_DMA_PER_WAVE * w + x;
    lds_dma16(tbase, sa::raw_piece_off_lane(rl, x, rs.tmax, rs.stride),
              __builtin_amdgcn_readfirstlane(LDS_OFF(g_lds8) + s8::raw(R) + 1024u * q));
  } else {
    dma8_piece<R>(rs, w, lane, x);
  }
}
template <int R>
__device__ __forceinline__ void dma8(const Item &it, int tile, int w, int lane) {
  const RawSrc rs = raw_src(tile_src(it, tile), w);
#pragma unroll
  for (int x = 0; x <= sa::RAW_DMA_PER_WAVE; ++x) dma8_piece<R>(rs, w, lane, x);
}

// Per-lane state: q~ as e4m3 hi / lo (the B operand of the score products:
// head l % 32, latent column 64 mm + 32 h + j in byte j of qh[mm], h = l /
// 32) and their E8M0 scales, the rotated q_rope in fp16, the output
// accumulator O^T [512 x 32 heads] as 16 column blocks, and the running max
// and denominator of the lane's head.
struct State8 {
  sa::RawLane rl;  // this lane's copy constants for the item's row stride
  i32x8 qh[8], ql[8];
  f16x8 qr[4];
  int sq_hi, sq_lo;
  f32x16 O[s8::DC / 32];
  float m, l;
  int w, lane;
};

// (Score A fragments for token t = lane % 32: latent chunk pair mm, columns
// 64 mm + 32 h .. +31, two 16-byte chunks of the permuted row; k_rope step
// kk, dims 16 kk + 8 h .. +7, bf16 divided by m_t and rounded to fp16.)

// Online softmax of one tile (this lane's head: 16 tokens here, 16 in lane ^
// 32), cut into pieces run between the score products of the next tile;
// piece n runs after product n. Sv holds the scores already multiplied by
// the token scales' mantissas; the probabilities p_r replace them.
//   0..3   partial maxima of 4 rows each
//   4      max exchange with lane ^ 32
//   5      row max
//   6      new running max (kept unless exceeded by SLACK), alpha
//   7..22  p_r = exp2(s_r - m), summed
//   23     sum exchange
//   24     l and m updated
// soft8_weights then turns p_r s_t into e4m3 hi / lo in Pb (bytes 0..15 hi,
// 16..31 lo, token order of the rows) with this lane's block scale sp, once
// the score chain's registers are free.
struct Soft8 {
  float m4[4], mx, m_new, m_sub, alpha, psum;
  uint32_t xs[2];
  i32x8 Pb;
  int sp;
};
__device__ __forceinline__ void soft8_piece(State8 &st, Soft8 &sm, f32x16 &Sv, int n) {
  using namespace s8;
  if (n < 4) {
    sm.m4[n] = fmaxf(fmaxf(Sv[4 * n], Sv[4 * n + 1]), fmaxf(Sv[4 * n + 2], Sv[4 * n + 3]));
  } else if (n == 4) {
    const float t = fmaxf(fmaxf(sm.m4[0], sm.m4[1]), fmaxf(sm.m4[2], sm.m4[3]));
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    sm.xs[0] = r[0];
    sm.xs[1] = r[1];
  } else if (n == 5) {
    sm.mx = fmaxf(__uint_as_float(sm.xs[0]), __uint_as_float(sm.xs[1]));
  } else if (n == 6) {
    // (a head whose tokens are all masked so far keeps m = -inf: alpha 1 and
    // exponents taken against 0, so every p is exactly 0)
    sm.m_new = sm.mx > st.m + SLACK ? sm.mx : st.m;
    sm.alpha = sm.m_new == st.m ? 1.0f : __builtin_amdgcn_exp2f(st.m - sm.m_new);
    sm.m_sub = sm.m_new == -INFINITY ? 0.0f : sm.m_new;
    sm.psum = 0.0f;
  } else if (n < 23) {
    const int r = n - 7;
    const float p = __builtin_amdgcn_exp2f(Sv[r] - sm.m_sub);
    sm.psum += p;
    Sv[r] = p;
  } else if (n == 23) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(sm.psum), __float_as_uint(sm.psum), false, false);
    sm.xs[0] = r[0];
    sm.xs[1] = r[1];
  } else if (n == 24) {
    st.l = fmaf(st.l, sm.alpha, __uint_as_float(sm.xs[0]) + __uint_as_float(sm.xs[1]));
    st.m = sm.m_new;
  }
}
template <int B>
__device__ __forceinline__ void soft8_weights(const State8 &st, Soft8 &sm, f32x16 &Sv) {
  const float *sp = reinterpret_cast<const float *>(g_lds8 + s8::scl(B, st.w)) + 4 * (st.lane >> 5);
  float wmax = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 sc = *reinterpret_cast<const f32x4 *>(sp + 8 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Sv[4 * q + e] *= sc[e];
      wmax = fmaxf(wmax, Sv[4 * q + e]);
    }
  }
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(wmax), __float_as_uint(wmax), false, false);
  const int ep = pow2_for_448(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
  // block 0 (hi) scale from lanes 0..31, block 1 (lo) from lanes 32..63
  sm.sp = 127 + ep - 4 * (st.lane >> 5);
  const float k = __builtin_ldexpf(1.0f, -ep);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint32_t hi, lo;
    hilo4(Sv[4 * g] * k, Sv[4 * g + 1] * k, Sv[4 * g + 2] * k, Sv[4 * g + 3] * k, hi, lo);
    sm.Pb[g] = static_cast<int>(hi);
    sm.Pb[4 + g] = static_cast<int>(lo);
  }
}

// Score products of tile buffer B: 4 fp16 k_rope products and 16 scaled
// e4m3 products (hi and lo per 64 latent columns) in one AGPR chain, with
// the softmax pieces of the previous tile (Sv) and the copies woven in.
struct NoHide8 {
  __device__ __forceinline__ void step(int) {}
};
// Where a step issues its six copies: under the value products (the wave
// mostly waits on the matrix cores there), value products 1..6, or under
// the score products 0..5.
constexpr bool kCopiesUnderValues = true;
template <int DMA_RAW>
struct Hide8 {
  RawSrc rs;
  const char *tbase;  // the tile's first row
  const sa::RawLane *rl;
  int w, lane;
  __device__ __forceinline__ void step(int n) {
    if (!kCopiesUnderValues && n <= sa::RAW_DMA_PER_WAVE) dma8_piece_lane<DMA_RAW>(rs, tbase, *rl, w, lane, n);
  }
  __device__ __forceinline__ void value_step(int cb) {
    if (kCopiesUnderValues && cb >= 1 && cb - 1 <= sa::RAW_DMA_PER_WAVE)
      dma8_piece_lane<DMA_RAW>(rs, tbase, *rl, w, lane, cb - 1);
  }
};
template <int B, bool SOFTMAX, class Hide>
__device__ __forceinline__ void score_chain8(State8 &st, f32x16 &S, f32x16 &Sv, Soft8 &sm, Hide &hide) {
  const int ln = opaque(st.lane), t = ln & 31, h = ln >> 5, sig = rsw8(t);
  const int row = s8::raw(B) + s8::ROWB * t;
  // this token's scale: the codes' block scale and the k_rope divisor
  const float s_t = reinterpret_cast<const float *>(g_lds8 + s8::scl(B, st.w))[t];
  const int sa_ = e8m0_of(s_t);
  const float inv_m = 1.0f / mant_of(s_t);
  // chunk 4 mm + 2 h + p of the row sits at 8 (mm / 2) + ((4 (mm % 2) + 2 h + p) ^ sig): four bases, the
  // rest an immediate offset
  int fb[2][2];
#pragma unroll
  for (int o = 0; o < 2; ++o)
#pragma unroll
    for (int p = 0; p < 2; ++p) fb[o][p] = row + 16 * ((4 * o + 2 * h + p) ^ sig);
  auto frag = [&](int mm) {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(g_lds8 + fb[mm & 1][0] + 128 * (mm >> 1));
    const u32x4 b = *reinterpret_cast<const u32x4 *>(g_lds8 + fb[mm & 1][1] + 128 * (mm >> 1));
    return i32x8{static_cast<int>(a[0]), static_cast<int>(a[1]), static_cast<int>(a[2]), static_cast<int>(a[3]),
                 static_cast<int>(b[0]), static_cast<int>(b[1]), static_cast<int>(b[2]), static_cast<int>(b[3])};
  };
  // latent products first, each fragment read two products ahead (at the
  // top of the previous pair); the k_rope products last, their rows read
  // during the last two pairs
  int n = 0;
  i32x8 af = frag(0);
  u32x4 rr[4];
  const char *rrow = g_lds8 + row;
#pragma unroll
  for (int mm = 0; mm < 8; ++mm) {
    const i32x8 a = af;
    if (mm + 1 < 8) af = frag(mm + 1);
    if (mm >= 6) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int kk = 2 * (mm - 6) + q;
        rr[kk] = *reinterpret_cast<const u32x4 *>(rrow + 16 * (32 + ((2 * kk + h) ^ sig)));
      }
    }
    // (the reads stay here: the products are asm the compiler would
    // otherwise sink them past)
    __builtin_amdgcn_sched_barrier(0);
    if (mm == 0) mma8_first(S, a, st.qh[mm], sa_, st.sq_hi);
    else mma8_chain(S, a, st.qh[mm], sa_, st.sq_hi);
    hide.step(n);
    if (SOFTMAX) soft8_piece(st, sm, Sv, n);
    ++n;
    __builtin_amdgcn_sched_barrier(0);
    mma8_chain(S, a, st.ql[mm], sa_, st.sq_lo);
    hide.step(n);
    if (SOFTMAX) soft8_piece(st, sm, Sv, n);
    ++n;
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    f16x8 ar;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ar[2 * e] = static_cast<_Float16>(__uint_as_float(rr[kk][e] << 16) * inv_m);
      ar[2 * e + 1] = static_cast<_Float16>(__uint_as_float(rr[kk][e] & 0xffff0000u) * inv_m);
    }
    S = mma16(ar, st.qr[kk], S);
    asm volatile("" : "+a"(S));
    hide.step(n);
    if (SOFTMAX) soft8_piece(st, sm, Sv, n);
    ++n;
    __builtin_amdgcn_sched_barrier(0);
  }
  if (SOFTMAX) {
#pragma unroll
    for (int k = 20; k < 25; ++k) soft8_piece(st, sm, Sv, k);
  }
}

// Value A fragment of column block cb (transposed 8-bit reads): 16-lane
// group G = l / 16 (token half h = G / 2, column half ch = G % 2), lane j in
// it points at token 8 (e / 4) + 4 h + e % 4 (e = j / 2; + 16 for the
// second read), logical chunk 2 cb + ch, bytes 8 (j % 2) ..; lane l then
// holds latent column 32 cb + l % 32 for the 16 tokens of its half, in the
// order of the softmax weights, duplicated into bytes 16..31 (the lo block).
// Chunk 2 cb + ch sits at 8 (cb / 4) + ((2 (cb % 4) + ch) ^ rsw8(token)) of
// the row (rsw8(token + 16) = rsw8(token)): four bases per lane, the rest
// an immediate offset.
typedef int i32x4 __attribute__((ext_vector_type(4)));
struct VBase {
  int b[4];
};
template <int B>
__device__ __forceinline__ VBase value_bases8(int lane_) {
  const int ln = opaque(lane_);
  const int G = ln >> 4, j = ln & 15, h = G >> 1, ch = G & 1, e = j >> 1;
  const int tok = 8 * (e >> 2) + 4 * h + (e & 3);
  const int row = s8::raw(B) + s8::ROWB * tok + 8 * (j & 1), sig = rsw8(tok);
  VBase v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v.b[q] = row + 16 * ((2 * q + ch) ^ sig);
  return v;
}
__device__ __forceinline__ i32x4 value_frag8(const VBase &vb, int cb) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  const char *p = g_lds8 + vb.b[cb & 3] + 128 * (cb >> 2);
  const i32x2 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(p));
  const i32x2 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(p + 16 * s8::ROWB));
  return i32x4{r0[0], r0[1], r1[0], r1[1]};
}
// The same fragment read twice, straight into both halves of the 64-wide
// operand (the lo block of P multiplies the same codes): two more LDS reads
// instead of four register copies, and no vector-ALU write before the product.
// (vb2 holds the same bases as vb in other registers, so the compiler cannot
// merge the two reads back into one and copy its result)
__device__ __forceinline__ i32x8 value_frag8x2(const VBase &vb, const VBase &vb2, int cb) {
  const i32x4 a = value_frag8(vb, cb), b = value_frag8(vb2, cb);
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
constexpr int VPF2 = 2;  // doubled fragments read ahead of their product

// Value products of tile buffer B for this wave's heads, after the rescale
// (if the running max moved): O^T block cb += codes^T P^T with P as hi / lo
// in one product.
template <int B, class Hide>
__device__ __forceinline__ void pv8(State8 &st, const Soft8 &sm, bool fresh, Hide &hide) {
  using namespace s8;
  const VBase vb = value_bases8<B>(st.lane);
  VBase vb2;
#pragma unroll
  for (int q = 0; q < 4; ++q) vb2.b[q] = opaque(vb.b[q]);
  i32x8 va[VPF2 + 1];
#pragma unroll
  for (int n = 0; n < VPF2; ++n) va[n] = value_frag8x2(vb, vb2, n);
  if (!fresh && __any(sm.alpha != 1.0f)) {
#pragma unroll
    for (int x = 0; x < DC / 32; ++x) {
      f32x16 t = st.O[x];
      asm volatile("" : "+v"(t));
      t *= sm.alpha;
      st.O[x] = t;
      if (x == VBLK) asm volatile("" : "+v"(st.O[x]));
      else asm volatile("" : "+a"(st.O[x]));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int cb = 0; cb < DC / 32; ++cb) {
    if (cb + VPF2 < DC / 32) va[(cb + VPF2) % (VPF2 + 1)] = value_frag8x2(vb, vb2, cb + VPF2);
    __builtin_amdgcn_sched_barrier(0);
    if (cb == VBLK) mma8_acc_v(st.O[cb], va[cb % (VPF2 + 1)], sm.Pb, 127, sm.sp);
    else mma8_acc(st.O[cb], va[cb % (VPF2 + 1)], sm.Pb, 127, sm.sp);
    hide.value_step(cb);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One pipeline step (I = i mod 4): S holds tile i's scores on entry. The
// scores of tile i+1 with the softmax of tile i and the copies of tile i+3,
// then the weights and value products of tile i, then this wave's copies of
// tile i+2 waited for and one barrier. An item's last step runs the softmax
// alone.
template <int I>
__device__ __forceinline__ void step8(State8 &st, f32x16 &S, const Item &it, int i, int w, int lane) {
  using namespace s8;
  Hide8<(I + 3) % NBUF> hd;
  {
    const sa::TileSrc src = tile_src(it, i + 3);
    hd.rs = raw_src(src, w);
    hd.tbase = src.base;
  }
  hd.rl = &st.rl;
  hd.w = w;
  hd.lane = lane;
  // (the last score product is asm: cover its result latency before the
  // vector ALU reads it)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+a"(S));
  f32x16 Sv = S;
  asm volatile("" : "+v"(Sv));
  {
    // the scores times the mantissas of their tokens' scales (rows 8 q + 4 h ..)
    const float *sp = reinterpret_cast<const float *>(g_lds8 + scl(I % NBUF, st.w)) + 4 * (st.lane >> 5);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 sc = *reinterpret_cast<const f32x4 *>(sp + 8 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) Sv[4 * q + e] *= mant_of(sc[e]);
    }
  }
  const int valid = min(T, it.tvis - (it.t0 + i * T));
  if (valid < T) {
    asm volatile("; tail mask");
    const int lim = valid - 4 * (opaque(st.lane) >> 5);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + (r & 3) >= lim) Sv[r] = -INFINITY;
  }
  Soft8 sm;
  if (i + 1 < it.ntiles) {
    score_chain8<(I + 1) % NBUF, true>(st, S, Sv, sm, hd);
  } else {
#pragma unroll
    for (int k = 0; k < 25; ++k) soft8_piece(st, sm, Sv, k);
  }
  soft8_weights<I % NBUF>(st, sm, Sv);
  pv8<I % NBUF>(st, sm, i == 0, hd);
  wait_vm<sa::RAW_DMA_PER_WAVE + 1>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Item k of the plan, head block y (of H / 128), by one workgroup.
__device__ __forceinline__ void splitk8_item(const mla_cache &c, int H, int Hr, int q_len, int k, int y,
                                             const WorkItem *__restrict__ items, const SeqInfo *__restrict__ seqs,
                                             const uint16_t *__restrict__ Q, uint16_t *__restrict__ opart,
                                             float *__restrict__ lse, int32_t *__restrict__ status) {
  using namespace s8;
  // (through opaque(): the lane-derived addresses are then made per item, not
  // hoisted out of the item loop and kept live across it)
  const int tid = opaque(static_cast<int>(threadIdx.x)), lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int head = y * 128 + 32 * w + (lane & 31);
  const int jq = (y * 128 + 32 * w) / Hr;
  const WorkItem wi = items[k];
  uint16_t *ob = opart + (static_cast<size_t>(k) * H + y * 128) * DC;

  const ItemSeq sq = item_seq(c, seqs, wi);
  if (!sq.ok) {
    if (tid == 0 && y == 0) set_status(status, MLA_ERR_PLAN);
    for (int x = tid; x < 128 * DC / 8; x += 256) reinterpret_cast<u32x4 *>(ob)[x] = u32x4{0, 0, 0, 0};
    if (half == 0) lse[static_cast<size_t>(k) * H + head] = -INFINITY;
    return;
  }
  Item it;
  it.rows = static_cast<const char *>(c.rows);
  it.scale = c.scale;
  it.stride = c.row_stride;
  it.row0 = sq.row0;
  it.blocks = c.block_table == nullptr ? nullptr : c.block_table + static_cast<int64_t>(wi.b) * c.max_blocks;
  it.block_tokens = c.block_tokens;
  it.n_blocks = c.block_table == nullptr ? 0 : static_cast<int>(c.n_rows / c.block_tokens);
  if (it.blocks != nullptr && w == 0) {
    const int nb = (wi.t1 - 1) / c.block_tokens - wi.t0 / c.block_tokens + 1;
    for (int x = lane; x < nb; x += 64) {
      const int blk = it.blocks[wi.t0 / c.block_tokens + x];
      if (blk < 0 || blk >= it.n_blocks) set_status(status, MLA_ERR_PLAN);
    }
  }
  it.t0 = wi.t0;
  it.t1 = wi.t1;
  it.ntiles = (wi.t1 - wi.t0 + T - 1) / T;
  it.tvis = min(wi.t1, sq.len - (q_len - 1 - jq));

  dma8<0>(it, 0, w, lane);
  dma8<1>(it, 1, w, lane);
  dma8<2>(it, 2, w, lane);

  // q~ of this lane's head to e4m3 hi / lo: the head's largest |q~| (this
  // lane's 256 values and lane ^ 32's), then the pairs; the rotated q_rope
  // stays fp16
  State8 st;
  st.w = w;
  st.lane = lane;
  st.rl = sa::raw_lane(w, opaque(lane), it.stride);
  {
    const uint16_t *qrow = Q + (static_cast<size_t>(wi.b) * H + head) * D;
    float amax = 0.0f;
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16x8 v = *reinterpret_cast<const f16x8 *>(qrow + 64 * mm + 32 * half + 8 * q);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(static_cast<float>(v[e])));
      }
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const int E = pow2_for_448(amax);
    const float k2 = __builtin_ldexpf(1.0f, -E);
    st.sq_hi = 127 + E;
    st.sq_lo = 127 + E - 4;
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16x8 v = *reinterpret_cast<const f16x8 *>(qrow + 64 * mm + 32 * half + 8 * q);
        uint32_t h0, l0, h1, l1;
        hilo4(static_cast<float>(v[0]) * k2, static_cast<float>(v[1]) * k2, static_cast<float>(v[2]) * k2,
              static_cast<float>(v[3]) * k2, h0, l0);
        hilo4(static_cast<float>(v[4]) * k2, static_cast<float>(v[5]) * k2, static_cast<float>(v[6]) * k2,
              static_cast<float>(v[7]) * k2, h1, l1);
        st.qh[mm][2 * q] = static_cast<int>(h0);
        st.qh[mm][2 * q + 1] = static_cast<int>(h1);
        st.ql[mm][2 * q] = static_cast<int>(l0);
        st.ql[mm][2 * q + 1] = static_cast<int>(l1);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) st.qr[kk] = *reinterpret_cast<const f16x8 *>(qrow + DC + 16 * kk + 8 * half);
  }
#pragma unroll
  for (int db = 0; db < DC / 32; ++db) {
    st.O[db] = f32x16{};
    if (db == VBLK) asm volatile("" : "+v"(st.O[db]));
    else asm volatile("" : "+a"(st.O[db]));
  }
  st.m = -INFINITY;
  st.l = 0.0f;

  // tiles 0..2 landed (every wave's copies: the barrier), then the scores
  // of tile 0 alone
  wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  f32x16 S;
  {
    NoHide8 nh;
    Soft8 sm;
    f32x16 dummy = {};
    score_chain8<0, false>(st, S, dummy, sm, nh);
  }
  for (int i = 0; i < it.ntiles; i += 4) {
    step8<0>(st, S, it, i, w, lane);
    if (i + 1 < it.ntiles) step8<1>(st, S, it, i + 1, w, lane);
    if (i + 2 < it.ntiles) step8<2>(st, S, it, i + 2, w, lane);
    if (i + 3 < it.ntiles) step8<3>(st, S, it, i + 3, w, lane);
  }

  wait_vm<0>();  // no copy may still be landing in LDS when the workgroup ends
  // the value products are asm: cover their result latency before the
  // vector ALU reads the accumulators
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  // ---- normalised partials and log-sum-exp (base 2), head by head (one
  // 1 KB row of 512 fp16 per head), turned around in LDS: every wave is past
  // its last tile read once all have reached the barrier
  __builtin_amdgcn_s_barrier();
  if (half == 0) lse[static_cast<size_t>(k) * H + head] = st.l > 0.0f ? st.m + log2f(st.l) : -INFINITY;
  const float inv = st.l > 0.0f ? 1.0f / st.l : 0.0f;
  char *tb = g_lds8 + w * 32 * OROW;
#pragma unroll
  for (int cb = 0; cb < DC / 32; ++cb) {
    f32x16 o = st.O[cb];
    if (cb != VBLK) asm volatile("" : "+v"(o));
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      f16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = static_cast<_Float16>(o[4 * g4 + e] * inv);
      // head lane % 32, columns 32 cb + 8 g4 + 4 half .. +3
      *reinterpret_cast<f16x4 *>(tb + (lane & 31) * OROW + 64 * cb + 16 * g4 + 8 * half) = v;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // the rows come from other lanes
  uint16_t *orow = ob + static_cast<size_t>(32 * w) * DC + 8 * lane;
#pragma unroll
  for (int h = 0; h < 32; ++h)
    *reinterpret_cast<u32x4 *>(orow + h * DC) = *reinterpret_cast<const u32x4 *>(tb + h * OROW + 16 * lane);
}

// One workgroup per (range, head block): range j's items one after the other.
__global__ __launch_bounds__(256, 1) void splitk8_kernel(SplitArgs args) {
  int j, y;
  range_of(static_cast<int>(blockIdx.x), args.n_ranges, args.H >> 7, j, y);
  const int kb = args.ranges[j], ke = args.ranges[j + 1];
  if (kb < 0 || kb > ke || ke > args.n_items) {
    if (threadIdx.x == 0) set_status(args.status, MLA_ERR_PLAN);
    return;
  }
  for (int k = kb; k < ke; ++k) {
    // every wave has read its turned-around rows of the last item out of
    // LDS before the next item's first copies land there
    if (k > kb) __syncthreads();
    const KernArgs a = kernel_args();
    splitk8_item(cache_of(a), a->H, a->Hr, a->q_len, k, y, a->items, a->seqs, a->Q, a->opart, a->lse, a->status);
  }
}

}  // namespace

hipError_t launch_decode_fast8(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t q_len, int32_t n_items,
                               int32_t n_ranges, const int32_t *ranges, const WorkItem *items, const SeqInfo *seqs,
                               const uint16_t *q, uint16_t *opart, float *lse, int32_t *status) {
  if (n_items == 0 || n_ranges == 0) return hipSuccess;
  const int H = d.n_heads * q_len;
  const SplitArgs args{c, H, d.n_heads, q_len, n_items, n_ranges, ranges, items, seqs, q, opart, lse, status};
  return launch_kernel(splitk8_kernel, dim3(n_ranges * (H / 128)), 256, 0, s, args);
}

}  // namespace mla
