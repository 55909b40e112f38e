// Split-K flash-decode over the latent cache (the hot loop of MLA decode).
//
// One workgroup per range of work items (each a sequence b and its tokens
// [t0, t1), run one after the other) and 128 heads, four waves; wave w
// computes the scores and softmax of heads 32 w .. 32 w +
// 31. For every tile of 32 cached tokens
//   S^T [32 tok x 32 heads]  = K [32 x 576] Q^T [576 x 32 heads]
//   online softmax per head, base 2 (Q is pre-scaled by scale * log2 e)
//   O^T [512 x 128 heads]   += C^T [512 x 32 tok] P^T [32 tok x 128 heads]
// where K = [c_kv | k_rope] rows and C = the c_kv part of the same rows: the
// score is the content term plus the positional term ("DeepSeek MLA" card),
// and both products read the one tile, shared by all 128 heads, because W_UK
// is already folded into Q and W_UV is applied after the loop ("02 —
// Multi-Latent Attention (MLA)", "Coste de cómputo"). The value product is
// split between the waves by latent columns for bf16 latents (wave w: columns
// 128 w .. +127 of every head; the softmax weights of all heads pass through
// LDS) and by heads for fp8 latents (wave w: its own 32 heads, the weights
// straight from its registers).
//
// Arithmetic: both products take fp16 operands with fp32 accumulation. The
// absorbed query arrives in fp16; cached values are widened to fp16 in LDS
// (bf16: exactly, below 65504 in magnitude; e4m3: times the token's scale,
// rounded once to fp16).
//
// Pipeline, per step i (the loop is unrolled so every buffer index is a
// compile-time constant and every LDS address a per-lane base plus a
// constant):
//   score products of tile i+1, with the softmax of tile i woven between
//   them and the copies of tile i+3 (global_load_lds_dwordx4: straight into
//   LDS, no registers) issued under them; then the value products of tile
//   i, with this wave's rows of tile i+2 widened under them (bf16; fp8
//   widens under the score products); one barrier (bf16: two, the first
//   before the value products read the exchanged weights).
// Each wave widens exactly the rows it copied, so it waits for its own
// copies only; the barrier makes the widened tile visible to all.
//
// LDS tile layout (16-bit elements), chosen so that both fragment reads are
// free of bank conflicts and every copy is a plain row copy:
//   latent: token t at 1072 t (1024 bytes of data + 48 of padding; the odd
//           stride of 67 chunks of 16 bytes spreads tokens over the banks),
//   k_rope: token t at 128 t in a region of its own, chunk c of the row at
//           position c ^ ((t >> 1) & 7).
// bf16 latents are copied into that layout and widened in place (four
// buffers); fp8 rows [512 e4m3 codes | 64 bf16 k_rope] (640 bytes) land in a
// raw buffer with their scales and are widened into it (three fp16 buffers,
// two raw ones).
#include <cmath>
#include <cstdlib>

#include "device_util.hpp"
#include "splitk_addr.hpp"
#include "splitk_common.hpp"

namespace mla {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_S16X4(p) ((__attribute__((address_space(3))) s16x4 *)(p))

namespace sk {
constexpr int DC = 512, D = 576;
constexpr int T = kTile;             // 32 tokens per tile
constexpr int LROW = 1072;           // latent row stride in LDS (bytes)
constexpr int LTILE = T * LROW;      // 34304
constexpr int RTILE = T * 128;       // 4096: k_rope rows
constexpr int RAW_ROWB = 640;        // fp8 row: 512 codes + 128 bytes k_rope
constexpr int RAW_TILE = T * RAW_ROWB;                 // 20480
constexpr int RAW_DMA_PER_WAVE = RAW_TILE / 1024 / 4;  // 5: 8 rows of 640 bytes
constexpr int SLACK = 8;             // running max is kept unless exceeded by 2^8
constexpr int SPF = 3;               // score fragments read ahead of their product
constexpr int VPF = 4;               // value fragments read ahead of their product
constexpr int VBLK = 15;             // the output block kept in VGPRs (its AGPRs hold the scores)
constexpr int OROW = 1040;           // partial row stride of the closing transpose in LDS (bytes), fp8
constexpr int OROWQ = 272;           // the same for the bf16 kernel's quarter rows (128 columns + 16 bytes)

// LDS map. bf16 latents: four fp16 tiles (copied and widened in place).
// fp8 latents: three fp16 tiles, two raw tiles and their per-token scales,
// one copy per wave (256 bytes each), so that a wave reads only what it
// loaded itself. NSTEP: the loop unroll, a multiple of every buffer count.
template <bool FP8> struct Map {
  static constexpr int NBUF = FP8 ? 3 : 4;
  static constexpr int NSTEP = FP8 ? 6 : 4;
  static constexpr int lat(int b) { return LTILE * b; }
  static constexpr int rope(int b) { return LTILE * NBUF + RTILE * b; }
  static constexpr int raw(int r) { return LTILE * NBUF + RTILE * NBUF + RAW_TILE * r; }
  static constexpr int scl(int r, int w) { return raw(2) + 1024 * r + 256 * w; }
  // bf16 only: one tile's softmax weights of all 128 heads in the value
  // products' operand layout ([head block][k-step][lane] x 16 bytes), and a
  // per-head float for each head block ([head % 32][head block]: alpha
  // during the loop, the softmax denominator at the end)
  static constexpr int pex() { return rope(NBUF); }
  static constexpr int aex() { return pex() + 8192; }
  static constexpr int end() { return FP8 ? raw(2) + 2048 : aex() + 512; }
};
constexpr int LDS_BYTES = Map<false>::end() > Map<true>::end() ? Map<false>::end() : Map<true>::end();
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert(4 * 32 * OROW <= Map<true>::end() && 4 * 128 * OROWQ <= Map<false>::pex(), "transpose area");
}  // namespace sk

__shared__ __attribute__((aligned(1024))) char g_lds[sk::LDS_BYTES];

namespace {

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// Value products with the accumulator's register file fixed (every output
// block in AGPRs but one, whose AGPRs hold the scores), so the compiler never
// moves a block between files. Operands come from LDS reads (waited for by
// lgkmcnt) or from the rescale, which runs long before; the leading s_nop
// covers a vector-ALU write of the VGPR-form accumulator.
__device__ __forceinline__ void mfma_acc_a(f32x16 &c, f16x8 a, f16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc_v(f32x16 &c, f16x8 a, f16x8 b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}


// k_rope chunk swizzle: chunk c of token t's row sits at c ^ rsw(t) (the
// copies' source chunks use the same function).
using sa::rsw;
static_assert(sk::T == sa::T && sk::RAW_DMA_PER_WAVE == sa::RAW_DMA_PER_WAVE && sk::RAW_ROWB == sa::RAW_ROWB,
              "tile geometry shared with the copy addresses");




using sa::Item;
using sa::RawSrc;
using sa::RopeSrc;
using sa::TileSrc;
using sa::raw_src;
using sa::tile_src;

// bf16 tile copy, 9 loads per wave (w uniform): x < 8 copies the 1024 latent
// bytes of token 8 w + x into its LDS row (lane i: bytes 16 i .. 16 i + 15);
// x = 8 copies the k_rope parts of tokens 8 w .. 8 w + 7 (lane i: token
// 8 w + i / 8, physical chunk i % 8, which holds chunk (i % 8) ^ rsw(token)).
template <int B>
__device__ __forceinline__ void dma_bf16_piece(const TileSrc &src, int w, int lane, int x) {
  using M = sk::Map<false>;
  const uint32_t lds0 = LDS_OFF(g_lds);
  if (x < 8) {
    lds_dma16(sa::latent_row(src, w, x), static_cast<uint32_t>(16 * lane), lds0 + M::lat(B) + sk::LROW * (8 * w + x));
  } else {
    const RopeSrc r = sa::rope_src(src, w, opaque(lane));
    lds_dma16(r.base, r.voff, lds0 + M::rope(B) + 1024 * w);
  }
}
template <int B>
__device__ __forceinline__ void dma_bf16(const Item &it, int tile, int w, int lane) {
  const TileSrc src = tile_src(it, tile);
#pragma unroll
  for (int x = 0; x < 9; ++x) dma_bf16_piece<B>(src, w, lane, x);
}

// Raw fp8 tile copy, 6 loads per wave: x < 5 copies 1 KB of wave w's rows
// (the raw tile is the rows back to back, 40 chunks of 16 bytes each:
// chunk P = 64 (5 w + x) + lane holds token P / 40, bytes 16 (P % 40)), x = 5
// the tile's 32 per-token scales into wave w's own copy (lanes 32..63 repeat
// lanes 0..31), so a wave needs only its own copies.
template <int R>
__device__ __forceinline__ void dma_raw_piece(const RawSrc &rs, int w, int lane, int x) {
  using M = sk::Map<true>;
  const uint32_t lds0 = LDS_OFF(g_lds);
  const int ln = opaque(lane);
  if (x < sk::RAW_DMA_PER_WAVE) {
    const int q = sk::RAW_DMA_PER_WAVE * w + x;
    lds_dma16(rs.base, sa::raw_piece_off(rs, w, ln, x), __builtin_amdgcn_readfirstlane(lds0 + M::raw(R) + 1024u * q));
  } else {
    lds_dma4(rs.sbase, sa::raw_scale_off(rs, ln), __builtin_amdgcn_readfirstlane(lds0 + M::scl(R, 0) + 256u * w));
  }
}
template <int R>
__device__ __forceinline__ void dma_raw(const Item &it, int tile, int w, int lane) {
  const RawSrc rs = raw_src(tile_src(it, tile), w);
#pragma unroll
  for (int x = 0; x <= sk::RAW_DMA_PER_WAVE; ++x) dma_raw_piece<R>(rs, w, lane, x);
}

// Widening a bf16 tile to fp16 in place, 9 chunks of 16 bytes per thread,
// exactly the bytes the thread's wave copied (dma_bf16_piece), so a wave
// needs to wait for its own copies only: x < 8: latent token 8 w + x, bytes
// 16 lane ..; x = 8: chunk tid of the k_rope region (wave w's 1 KB). Split
// into load and convert-store so the two can be spread over a matrix-core
// loop.
template <int B>
__device__ __forceinline__ char *widen_bf16_addr(int tid, int x) {
  using M = sk::Map<false>;
  return x < 8 ? g_lds + M::lat(B) + sk::LROW * (8 * (tid >> 6) + x) + 16 * (tid & 63)
               : g_lds + M::rope(B) + 16 * tid;
}
template <int B>
__device__ __forceinline__ u32x4 widen_bf16_load(int tid, int x) {
  return *reinterpret_cast<const u32x4 *>(widen_bf16_addr<B>(tid, x));
}
template <int B>
__device__ __forceinline__ void widen_bf16_store(int tid, int x, u32x4 v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = bf16x2_to_f16x2(v[k]);
  *reinterpret_cast<u32x4 *>(widen_bf16_addr<B>(tid, x)) = v;
}
template <int B>
__device__ __forceinline__ void widen_bf16_inplace(int tid_) {
  const int tid = opaque(tid_);
#pragma unroll
  for (int x = 0; x < 9; ++x) widen_bf16_store<B>(tid, x, widen_bf16_load<B>(tid, x));
}

// Widening this wave's rows of a raw fp8 tile (raw buffer R) into fp16
// buffer B, 5 chunks of 16 bytes per thread with no divergence: x < 4 takes
// code chunk c = 64 x + lane (token 8 w + c / 32, codes 16 (c % 32) ..), 16
// codes to 32 bytes of fp16 times the token's scale; x = 4 takes k_rope chunk
// lane (token 8 w + lane / 8, chunk lane % 8), bf16 to fp16. The scale
// s = m 2^e splits into the power of two, applied by the conversion itself
// (which uses only the exponent of its scale operand), and the mantissa
// m in [1, 2), applied by an fp16 multiply: one rounding of a short product.
template <int R>
__device__ __forceinline__ const char *widen_fp8_src(int tid, int x) {
  using M = sk::Map<true>;
  const int w = tid >> 6, lane = tid & 63;
  if (x < 4) {
    const int c = 64 * x + lane;
    return g_lds + M::raw(R) + sk::RAW_ROWB * (8 * w + (c >> 5)) + 16 * (c & 31);
  }
  return g_lds + M::raw(R) + sk::RAW_ROWB * (8 * w + (lane >> 3)) + 512 + 16 * (lane & 7);
}
template <int R>
__device__ __forceinline__ u32x4 widen_fp8_load(int tid, int x) {
  return *reinterpret_cast<const u32x4 *>(widen_fp8_src<R>(tid, x));
}
template <int R, int B>
__device__ __forceinline__ void widen_fp8_store(int tid, int x, u32x4 v) {
  using M = sk::Map<true>;
  const int w = tid >> 6, lane = tid & 63;
  if (x < 4) {
    const int c = 64 * x + lane, t = 8 * w + (c >> 5);
    const uint32_t sb = __float_as_uint(reinterpret_cast<const float *>(g_lds + M::scl(R, 0) + 256 * w)[t]);
    const float pow2 = __uint_as_float(sb & 0x7f800000u);
    const _Float16 mh = static_cast<_Float16>(__uint_as_float((sb & 0x807fffffu) | 0x3f800000u));
    const f16x2 m2 = {mh, mh};
    u32x4 lo, hi;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      lo[2 * k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[k], pow2, false) * m2);
      lo[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[k], pow2, true) * m2);
      hi[2 * k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[k + 2], pow2, false) * m2);
      hi[2 * k + 1] =
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[k + 2], pow2, true) * m2);
    }
    char *row = g_lds + M::lat(B) + sk::LROW * t + 32 * (c & 31);
    *reinterpret_cast<u32x4 *>(row) = lo;
    *reinterpret_cast<u32x4 *>(row + 16) = hi;
  } else {
    const int t = 8 * w + (lane >> 3);
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = bf16x2_to_f16x2(v[k]);
    *reinterpret_cast<u32x4 *>(g_lds + M::rope(B) + 128 * t + 16 * ((lane & 7) ^ rsw(t))) = r;
  }
}
template <int R, int B>
__device__ __forceinline__ void widen_fp8(int tid_) {
  const int tid = opaque(tid_);
#pragma unroll
  for (int x = 0; x < 5; ++x) widen_fp8_store<R, B>(tid, x, widen_fp8_load<R>(tid, x));
}

// Per-lane state of one wave: the absorbed query of its 32 heads (fp16, the
// B operand of the score products), the output accumulator O^T [512 x 32
// heads] as 16 column blocks (O[cb]: latent columns 32 cb ..), and the
// running max and denominator of its lane's head.
struct WaveState {
  f16x8 qf[sk::D / 16];
  f32x16 O[sk::DC / 32];
  float m, l;
  int w, lane;
};

// Fragment base addresses, recomputed from the lane index at the start of
// each phase (from an opaque copy, so they are not hoisted into registers
// kept live across the whole loop). Buffers 2 and 3 lie beyond the 16-bit
// offset range of LDS reads and get their own base.
struct ScoreBase {
  int sl;  // latent A fragment, k-step 0: token hl, chunk half of the row
  int sr;  // k_rope A fragment of k-step 32; k-step 32 + j is at sr ^ 32 j
};
template <bool FP8, int B>
__device__ __forceinline__ ScoreBase score_base(int lane_) {
  using M = sk::Map<FP8>;
  const int ln = opaque(lane_), hl = ln & 31, half = ln >> 5;
  ScoreBase b;
  b.sl = sk::LROW * hl + 16 * half + (B < 2 ? 0 : M::lat(2));
  // chunk (2 j + half) ^ rsw(hl) of the k_rope row: the XOR with 2 j only
  // touches bits 5 and 6 of the byte offset, which the region base (a
  // multiple of 128) and the row offset leave clear
  static_assert(M::rope(0) % 128 == 0, "k_rope region alignment");
  b.sr = M::rope(0) + 128 * hl + 16 * (half ^ rsw(hl));
  return b;
}
// Score A fragment kk: token hl, dims 16 kk + 8 half .. +7 (one 16-byte
// read; latent for kk < 32, k_rope after).
template <bool FP8, int B>
__device__ __forceinline__ f16x8 score_frag(const ScoreBase &sb, int kk) {
  using M = sk::Map<FP8>;
  const char *p = kk < 32 ? g_lds + sb.sl + (B < 2 ? M::lat(B) : M::lat(B) - M::lat(2)) + 32 * kk
                          : g_lds + (sb.sr ^ (32 * (kk - 32))) + (M::rope(B) - M::rope(0));
  return *reinterpret_cast<const f16x8 *>(p);
}

// Online softmax of one tile's scores (this lane's head: 16 tokens here, 16
// in lane ^ 32), cut into pieces that run between the score products of the
// next tile: piece kk runs after product kk. The wave issues in order, so a
// piece never waits on a result produced in the same piece (a stalled vector
// op would hold back the next matrix-core op): the cross-lane exchanges and
// each exp2 are consumed one piece later. Scores are in log2 units; exp2 of
// a value below -126 may flush to zero, below the fp16 resolution of P.
//   0..3   partial maxima of 4 rows each
//   4      max of this lane's 16 rows, exchange with lane ^ 32
//   5      row max mx
//   6      new running max (kept unless exceeded by SLACK), alpha
//   7..22  p_r = exp2(s_r - m) for r = kk - 7; p_{r-1} summed and packed
//   23     last p summed and packed, sum exchange
//   24     l = alpha l + sum, m updated
// P stays in registers (fp16 pairs, rows 2 j and 2 j + 1 in P[j]) for the
// value products of the same wave.
struct Softmax {
  float m4[4], mx, m_new, m_sub, alpha, psum, pe, prev;
  uint32_t xs[2];
  uint32_t P[8];
};
__device__ __forceinline__ void softmax_consume(Softmax &sm, int r) {
  // p_r (in sm.prev) into the sum and the packed rows
  sm.psum += sm.prev;
  if (r % 2 == 0) {
    sm.pe = sm.prev;
  } else {
    f16x2 h;
    h[0] = static_cast<_Float16>(sm.pe);
    h[1] = static_cast<_Float16>(sm.prev);
    sm.P[r >> 1] = __builtin_bit_cast(uint32_t, h);
  }
}
__device__ __forceinline__ void softmax_piece(WaveState &st, Softmax &sm, const f32x16 &S, int kk) {
  using namespace sk;
  if (kk < 4) {
    sm.m4[kk] = fmaxf(fmaxf(S[4 * kk], S[4 * kk + 1]), fmaxf(S[4 * kk + 2], S[4 * kk + 3]));
  } else if (kk == 4) {
    const float t = fmaxf(fmaxf(sm.m4[0], sm.m4[1]), fmaxf(sm.m4[2], sm.m4[3]));
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    sm.xs[0] = r[0];
    sm.xs[1] = r[1];
  } else if (kk == 5) {
    sm.mx = fmaxf(__uint_as_float(sm.xs[0]), __uint_as_float(sm.xs[1]));
  } else if (kk == 6) {
    // (a row whose tokens are all masked so far keeps m = -inf: alpha 1 and
    // exponents taken against 0, so every p is exactly 0)
    sm.m_new = sm.mx > st.m + SLACK ? sm.mx : st.m;
    sm.alpha = sm.m_new == st.m ? 1.0f : __builtin_amdgcn_exp2f(st.m - sm.m_new);
    sm.m_sub = sm.m_new == -INFINITY ? 0.0f : sm.m_new;
    sm.psum = 0.0f;
  } else if (kk < 23) {
    const int r = kk - 7;
    const float p = __builtin_amdgcn_exp2f(S[r] - sm.m_sub);
    if (r > 0) softmax_consume(sm, r - 1);
    sm.prev = p;
  } else if (kk == 23) {
    softmax_consume(sm, 15);
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(sm.psum), __float_as_uint(sm.psum), false, false);
    sm.xs[0] = r[0];
    sm.xs[1] = r[1];
  } else if (kk == 24) {
    st.l = fmaf(st.l, sm.alpha, __uint_as_float(sm.xs[0]) + __uint_as_float(sm.xs[1]));
    st.m = sm.m_new;
  }
}

// Score products of one tile (fp16 buffer B): one chain over the 36
// k-steps, accumulating in AGPRs (S), with the softmax of the previous
// tile's scores (Sv, a VGPR copy) woven in when SOFTMAX is set. An AGPR-form
// chain leaves the VGPR file's ports to the vector ALU, and the compiler's
// own hazard handling needs no blanket wait before each product, so the
// softmax's vector work runs in the products' shadow (with a VGPR-form
// chain, or an s_nop before each product, it mostly serialises).
__device__ __forceinline__ void px_write_part(const WaveState &st, const Softmax &sm, int part);
template <bool FP8, int B, bool SOFTMAX, class Hide>
__device__ __forceinline__ void score_chain(WaveState &st, f32x16 &S, const f32x16 &Sv, Softmax &sm, Hide &hide) {
  using namespace sk;
  const ScoreBase sb = score_base<FP8, B>(st.lane);
  f16x8 af[SPF + 1];
#pragma unroll
  for (int j = 0; j < SPF; ++j) af[j] = score_frag<FP8, B>(sb, j);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (kk + SPF < D / 16) af[(kk + SPF) % (SPF + 1)] = score_frag<FP8, B>(sb, kk + SPF);
    const f16x8 a = af[kk % (SPF + 1)];
    S = mfma32(a, st.qf[kk], kk == 0 ? f32x16{} : S);
    asm volatile("" : "+a"(S));
    hide.score_step(kk);
    if (SOFTMAX) softmax_piece(st, sm, Sv, kk);
    if (SOFTMAX && !FP8 && (kk == 7 || kk == 16 || kk == 24)) px_write_part(st, sm, kk == 7 ? 0 : (kk == 16 ? 1 : 2));
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Value A fragment (transposed read): 16-lane group g, lane j in it points
// at token 16 kb + 8 h + tt (tt = 4 (g/2) + j/4), latent column 32 cb + dd
// (dd = 16 (g%2) + 4 (j%4)); the base includes the offset of buffers 2 and
// up, beyond the 16-bit range of LDS read offsets.
template <bool FP8, int B>
__device__ __forceinline__ int value_base(int lane_) {
  using M = sk::Map<FP8>;
  const int ln = opaque(lane_);
  const int g = (ln >> 4) & 3, j = ln & 15;
  const int tt = 4 * (g >> 1) + (j >> 2);
  const int dd = 16 * (g & 1) + 4 * (j & 3);
  return sk::LROW * tt + 2 * dd + (B < 2 ? 0 : M::lat(2));
}
template <bool FP8, int B>
__device__ __forceinline__ f16x8 value_frag(int vl, int cb, int kb) {
  using M = sk::Map<FP8>;
  const char *p0 = g_lds + vl + (B < 2 ? M::lat(B) : M::lat(B) - M::lat(2)) + sk::LROW * 16 * kb + 64 * cb;
  const char *p1 = p0 + sk::LROW * 8;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_S16X4(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_S16X4(p1));
  f16x8 a;
  a.lo = __builtin_bit_cast(f16x4, lo);
  a.hi = __builtin_bit_cast(f16x4, hi);
  return a;
}

// Value products of one tile (fp16 buffer B) for this wave's heads:
// O^T [512 x 32 heads] += C^T [512 x 32 tok] P^T [32 tok x 32 heads], 16
// column blocks x 2 k-steps, value fragments read VPF products ahead. P is
// the wave's own, used in place: in k-step kb, element e of lane l stands
// for token 16 kb + 8 (e / 4) + 4 (l / 32) + e % 4 in both operands (the
// rows the softmax left in the lane, and the tokens the transposed value
// reads fetch), an order of the 16 tokens the contraction does not see.
// Every accumulator value of a lane belongs to the lane's head, so the
// rescale is a per-lane factor.
template <bool FP8, int B>
__device__ __forceinline__ void pv_rows(WaveState &st, const Softmax &sm, bool fresh) {
  using namespace sk;
  const int vl = value_base<FP8, B>(st.lane);
  f16x8 va[VPF + 1];
#pragma unroll
  for (int n = 0; n < VPF; ++n) va[n] = value_frag<FP8, B>(vl, n & 15, n >> 4);
  f16x8 pb[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
    pb[kb] = __builtin_bit_cast(f16x8, u32x4{sm.P[4 * kb], sm.P[4 * kb + 1], sm.P[4 * kb + 2], sm.P[4 * kb + 3]});
  // wait states between the vector-ALU writes of P and the asm products
  // reading it
  asm volatile("s_nop 4" : "+v"(pb[0]), "+v"(pb[1]));
  // (an item's first tile needs none: the accumulators are still zero)
  if (!fresh && __any(sm.alpha != 1.0f)) {
    // one 16-register block at a time through VGPRs, back into AGPRs (the
    // VGPR block stays there)
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
  for (int n = 0; n < 2 * (DC / 32); ++n) {
    const int kb = n >> 4, cb = n & 15;
    if (n + VPF < 2 * (DC / 32)) va[(n + VPF) % (VPF + 1)] = value_frag<FP8, B>(vl, (n + VPF) & 15, (n + VPF) >> 4);
    if (cb == VBLK) mfma_acc_v(st.O[cb], va[n % (VPF + 1)], pb[kb]);
    else mfma_acc_a(st.O[cb], va[n % (VPF + 1)], pb[kb]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// bf16 kernel: value products split by latent columns instead of heads.
// Wave w owns columns 128 w .. 128 w + 127 of all 128 heads: block
// O[4 cb + hb] is O^T [32 cols x 32 heads] for columns 128 w + 32 cb .. and
// heads 32 hb ..; per tile
//   O^T block (cb, hb) += C^T [32 cols x 16 tok] P^T [16 tok x 32 heads]
// over two k-steps: 32 products, as with the row split, but each transposed
// value fragment serves four products (8 fragments per wave and tile, a
// quarter of the row split's transposed reads), and the weights of every
// head come from LDS, where each head block's score wave left them in the
// B-operand layout (the P registers of lane l of wave hb are the B operand
// lane l of any wave needs for head block hb; same token order as the
// transposed reads deliver). Each lane's alpha for its head in every head
// block comes from LDS too.
// The exchange writes of this wave's softmax results, each issued as soon as
// the softmax piece that completes it has run (the previous tile's readers
// of the exchange area are past the previous step's closing barrier): after
// piece 7 alpha, after piece 16 the weights of k-step 0, after piece 24
// those of k-step 1; px_write writes all three (an item's last tile).
__device__ __forceinline__ void px_write_part(const WaveState &st, const Softmax &sm, int part) {
  using M = sk::Map<false>;
  if (part == 0) {
    if (st.lane < 32) reinterpret_cast<float *>(g_lds + M::aex() + 16 * st.lane)[st.w] = sm.alpha;
  } else {
    const int kb = part - 1;
    *reinterpret_cast<u32x4 *>(g_lds + M::pex() + 1024 * (2 * st.w + kb) + 16 * st.lane) =
        u32x4{sm.P[4 * kb], sm.P[4 * kb + 1], sm.P[4 * kb + 2], sm.P[4 * kb + 3]};
  }
}
__device__ __forceinline__ void px_write(const WaveState &st, const Softmax &sm) {
#pragma unroll
  for (int part = 0; part < 3; ++part) px_write_part(st, sm, part);
}
// The first two value fragments come from the tile itself (complete since
// an earlier step), so they are read before the exchange barrier.
template <int B>
__device__ __forceinline__ void pv_cols_pre(const WaveState &st, f16x8 (&va)[3]) {
  const int vl = value_base<false, B>(st.lane) + 256 * st.w;
  va[0] = value_frag<false, B>(vl, 0, 0);
  va[1] = value_frag<false, B>(vl, 1, 0);
}
template <int B, class Hide>
__device__ __forceinline__ void pv_cols(WaveState &st, bool fresh, Hide &hide, f16x8 (&va)[3]) {
  using namespace sk;
  using M = Map<false>;
  const int vl = value_base<false, B>(st.lane) + 256 * st.w;  // this wave's 128 columns
  const int ln = opaque(st.lane);
  // alpha first: the rescale test waits for it alone, the fragments keep flying
  const f32x4 a4 = *reinterpret_cast<const f32x4 *>(g_lds + M::aex() + 16 * (ln & 31));
  f16x8 pf[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
    pf[hb] = *reinterpret_cast<const f16x8 *>(g_lds + M::pex() + 1024 * (2 * hb) + 16 * ln);
  // (an item's first tile needs none: the accumulators are still zero)
  if (!fresh && __any(a4[0] != 1.0f || a4[1] != 1.0f || a4[2] != 1.0f || a4[3] != 1.0f)) {
#pragma unroll
    for (int x = 0; x < DC / 32; ++x) {
      f32x16 t = st.O[x];
      asm volatile("" : "+v"(t));
      t *= a4[x & 3];
      st.O[x] = t;
      if (x == VBLK) asm volatile("" : "+v"(st.O[x]));
      else asm volatile("" : "+a"(st.O[x]));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int cb = n & 3;
    if (n == 4) {
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        pf[hb] = *reinterpret_cast<const f16x8 *>(g_lds + M::pex() + 1024 * (2 * hb + 1) + 16 * ln);
    }
    if (n + 2 < 8) va[(n + 2) % 3] = value_frag<false, B>(vl, (n + 2) & 3, (n + 2) >> 2);
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int x = 4 * cb + hb;
      if (x == VBLK) mfma_acc_v(st.O[x], va[n % 3], pf[hb]);
      else mfma_acc_a(st.O[x], va[n % 3], pf[hb]);
      hide.value_step(4 * n + hb);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Work a step hides under its score products: score_step(kk) runs after
// score product kk and issues at most one copy, one load or one
// convert-and-store. Copies of a tile past the item's end re-read the item's
// last tile (in bounds, cached) into a buffer nobody reads any more, and
// widening such a tile rewrites that dead buffer: branch-free steps let the
// compiler count outstanding LDS operations exactly, so no wait drains the
// fragment prefetch.
//
// bf16 latents: the 9 copies of tile i+3 under the score products (one
// every fourth product, the k_rope part at product 32), and the widening of
// this wave's rows of tile i+2, in place, under the value products (which,
// split by columns, leave the LDS and the issue slots room for it): 9 chunks
// of 16 bytes per thread, chunk x loaded after value product 3 x, once this
// wave's copies of tile i+2 have landed (only this step's 9 copies of tile
// i+3 may still fly), and converted and stored two products later. The
// latent copy's source row pointer advances by the stride per row (no
// multiply), and stops at the item's last row.
// (kBf16CopiesUnderValues: the copies of tile i+3 go under the value
// products instead, after value products 1, 4, .., 22 and the k_rope part
// after 25, once every earlier copy has landed.)
constexpr bool kBf16CopiesUnderValues = true;
template <int DMA_BUF, int WIDEN_BUF>
struct HideBf16 {
  const char *row;        // latent source of the next copy
  const char *rope_base;  // the k_rope copy's base row (rope_src)
  int64_t stride;
  int lim;                // rows 8 w + x with x <= lim exist; later ones repeat the last
  uint32_t rope_voff;     // this lane's k_rope source offset from rope_base
  int w, lane, tid;
  u32x4 v[2];
  __device__ __forceinline__ void copy(int x) {
    using M = sk::Map<false>;
    if (x < 8) {
      lds_dma16(row, static_cast<uint32_t>(16 * lane), LDS_OFF(g_lds) + M::lat(DMA_BUF) + sk::LROW * (8 * w + x));
      row = sa::latent_row_next(row, stride, lim, x);
    } else {
      lds_dma16(rope_base, rope_voff, LDS_OFF(g_lds) + M::rope(DMA_BUF) + 1024 * w);
    }
  }
  __device__ __forceinline__ void score_step(int kk) {
    if (kBf16CopiesUnderValues) return;
    if (kk % 4 == 0 && kk / 4 < 8) copy(kk / 4);
    if (kk == 32) copy(8);
  }
  // after value product m (0 .. 31)
  __device__ __forceinline__ void value_step(int m) {
    if (m == 0) {
      if (kBf16CopiesUnderValues) wait_vm<0>();
      else wait_vm<9>();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kBf16CopiesUnderValues && m % 3 == 1 && m / 3 < 9) copy(m / 3);
    if (m % 3 == 2 && (m - 2) / 3 < 9) {
      const int x = (m - 2) / 3;
      widen_bf16_store<WIDEN_BUF>(tid, x, v[x & 1]);
    }
    if (m % 3 == 0 && m / 3 < 9) {
      const int x = m / 3;
      v[x & 1] = widen_bf16_load<WIDEN_BUF>(tid, x);
    }
  }
};

// fp8 latents: the 6 copies of raw tile i+3 (products 0..5) into the raw
// buffer tile i+1 used, and the widening of this wave's rows of raw tile i+2
// into fp16 buffer (i+2) % 3: chunk x loaded after product 8 + 4 x, once this
// wave's copies of tile i+2 have landed (waited for at product 8: only this
// step's 6 may still fly), converted and stored three products later.
template <int DMA_RAW, int WIDEN_RAW, int WIDEN_BUF>
struct HideFp8 {
  RawSrc rs;
  int w, lane, tid;
  u32x4 v;
  __device__ __forceinline__ void score_step(int kk) {
    if (kk <= sk::RAW_DMA_PER_WAVE) dma_raw_piece<DMA_RAW>(rs, w, lane, kk);
    if (kk == 8) {
      wait_vm<sk::RAW_DMA_PER_WAVE + 1>();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kk >= 11 && (kk - 11) % 4 == 0 && (kk - 11) / 4 < 5) widen_fp8_store<WIDEN_RAW, WIDEN_BUF>(tid, (kk - 11) / 4, v);
    if (kk >= 8 && (kk - 8) % 4 == 0 && (kk - 8) / 4 < 5) v = widen_fp8_load<WIDEN_RAW>(tid, (kk - 8) / 4);
  }
};

struct NoHide {
  __device__ __forceinline__ void score_step(int) {}
};

template <bool FP8, int I> struct StepHide;
template <int I> struct StepHide<false, I> {
  using type = HideBf16<(I + 3) % 4, (I + 2) % 4>;
  __device__ __forceinline__ static void init(type &h, const TileSrc &src, int w, int lane, int tid) {
    h.stride = src.stride;
    h.lim = src.tmax - 8 * w;
    h.row = sa::latent_row_first(src, w);
    const RopeSrc r = sa::rope_src(src, w, opaque(lane));
    h.rope_base = r.base;
    h.rope_voff = r.voff;
    h.w = w;
    h.lane = lane;
    h.tid = opaque(tid);
  }
};
template <int I> struct StepHide<true, I> {
  using type = HideFp8<(I + 3) % 2, (I + 2) % 2, (I + 2) % 3>;
  __device__ __forceinline__ static void init(type &h, const TileSrc &src, int w, int lane, int tid) {
    h.rs = raw_src(src, w);
    h.w = w;
    h.lane = lane;
    h.tid = opaque(tid);
  }
};

// One pipeline step (I = i mod NSTEP), software-pipelined by one tile. On
// entry tile i+1 is widened and visible and S (AGPRs) holds tile i's scores;
// they are copied to VGPRs first. The step runs the score products of tile
// i+1 with the softmax of tile i, the copies of tile i+3 and the widening of
// this wave's rows of tile i+2 woven in, then the value products of tile i,
// then one barrier: tile i+2 is ready for the next step's scores, and tile
// i's buffer (and, fp8, the raw buffer tile i+2 came from) is free for the
// next step's copies. An item's last step runs the softmax alone.
template <bool FP8, int I>
__device__ __forceinline__ void step(WaveState &st, f32x16 &S, const Item &it, int i, int w, int lane, int tid) {
  constexpr int NB = sk::Map<FP8>::NBUF;
  typename StepHide<FP8, I>::type h;
  StepHide<FP8, I>::init(h, tile_src(it, i + 3), w, lane, tid);
  f32x16 Sv = S;
  asm volatile("" : "+v"(Sv));
  const int valid = min(sk::T, it.tvis - (it.t0 + i * sk::T));
  if (valid < sk::T) {  // the last tile(s) only (a real branch: the asm cannot be speculated)
    asm volatile("; tail mask");
    const int lim = valid - 4 * (opaque(st.lane) >> 5);  // one register, not 16 hoisted row indices
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + (r & 3) >= lim) Sv[r] = -INFINITY;
  }
  Softmax sm;
  if (i + 1 < it.ntiles) {
    score_chain<FP8, (I + 1) % NB, true>(st, S, Sv, sm, h);
  } else {
    // the item's last tile: no next tile to score and nothing left to copy
    // or widen, only this tile's softmax
#pragma unroll
    for (int kk = 0; kk <= 24; ++kk) softmax_piece(st, sm, Sv, kk);
  }
  if constexpr (FP8) {
    pv_rows<FP8, I % NB>(st, sm, i == 0);
  } else {
    // every head's weights and alpha in LDS (written by the score chain as
    // the softmax produced them; an item's last tile writes them here)
    // before any wave's value products read them
    if (i + 1 >= it.ntiles) px_write(st, sm);
    f16x8 va[3];
    pv_cols_pre<I % NB>(st, va);
    wait_lds();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    pv_cols<I % NB>(st, i == 0, h, va);
  }
  wait_lds();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Item k of the plan, head block y (of H / 128), by one workgroup.
template <bool FP8>
__device__ __forceinline__ void splitk_item(const mla_cache &c, int H, int Hr, int q_len, int k, int y,
                                            const WorkItem *__restrict__ items, const SeqInfo *__restrict__ seqs,
                                            const uint16_t *__restrict__ Q, uint16_t *__restrict__ opart,
                                            float *__restrict__ lse, int32_t *__restrict__ status) {
  using namespace sk;
  // (through opaque(): the lane-derived addresses are then made per item, not
  // hoisted out of the item loop and kept live across it)
  const int tid = opaque(static_cast<int>(threadIdx.x)), lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int head = y * 128 + 32 * w + (lane & 31);
  // with several new query tokens per sequence the heads are (token j,
  // head) pairs, token-major: this wave's 32 all belong to token
  // jq = (y * 128 + 32 w) / Hr, which sees the rows before len - (q_len - 1 - jq)
  const int jq = (y * 128 + 32 * w) / Hr;
  const WorkItem wi = items[k];
  // this workgroup's 128 heads of item k: 128 rows of 512 fp16 partials
  uint16_t *ob = opart + (static_cast<size_t>(k) * H + y * 128) * DC;

  // (the item must name a sequence of the batch before anything is indexed by it)
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
    // the item's block ids, checked once (one per lane)
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

  // prologue copies first, so they overlap the Q fetch (tiles past the end
  // re-read the item's last tile, like the steps)
  if (FP8) {
    dma_raw<0>(it, 0, w, lane);
    dma_raw<1>(it, 1, w, lane);
  } else {
    dma_bf16<0>(it, 0, w, lane);
  }

  WaveState st;
  st.w = w;
  st.lane = lane;
  {
    const uint16_t *qrow = Q + (static_cast<size_t>(wi.b) * H + head) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) st.qf[kk] = *reinterpret_cast<const f16x8 *>(qrow + 16 * kk);
  }
  // bf16: tiles 1 and 2 only once tile 0 and Q have landed (below): with
  // every workgroup loading at once, a workgroup's tile 0 otherwise queues
  // behind the others' tiles 1 and 2
#pragma unroll
  for (int db = 0; db < DC / 32; ++db) {
    st.O[db] = f32x16{};
    if (db == VBLK) asm volatile("" : "+v"(st.O[db]));
    else asm volatile("" : "+a"(st.O[db]));
  }
  st.m = -INFINITY;
  st.l = 0.0f;

  // fp8: this wave's rows of tiles 0 and 1 landed and widened, then raw
  // buffer 0 takes tile 2 (only this wave's rows, which only it read); bf16:
  // tile 0 widened. Then the scores of tile 0 alone (bf16: and tile 1
  // widened after them)
  if (FP8) {
    wait_vm<0>();
    __builtin_amdgcn_sched_barrier(0);
    widen_fp8<0, 0>(tid);
    widen_fp8<1, 1>(tid);
    wait_lds();
    dma_raw<0>(it, 2, w, lane);
  } else {
    wait_vm<0>();  // tile 0 and Q landed
    __builtin_amdgcn_sched_barrier(0);
    dma_bf16<1>(it, 1, w, lane);
    dma_bf16<2>(it, 2, w, lane);
    widen_bf16_inplace<0>(tid);
    wait_lds();
  }
  __builtin_amdgcn_s_barrier();
  f32x16 S;
  {
    NoHide nh;
    Softmax sm;
    score_chain<FP8, 0, false>(st, S, S, sm, nh);
  }
  if (!FP8) {
    // tile 1 (this wave's rows) landed while tile 0 was scored
    wait_vm<9>();
    __builtin_amdgcn_sched_barrier(0);
    widen_bf16_inplace<1>(tid);
    wait_lds();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (FP8) {
    for (int i = 0; i < it.ntiles; i += 6) {
      step<true, 0>(st, S, it, i, w, lane, tid);
      if (i + 1 < it.ntiles) step<true, 1>(st, S, it, i + 1, w, lane, tid);
      if (i + 2 < it.ntiles) step<true, 2>(st, S, it, i + 2, w, lane, tid);
      if (i + 3 < it.ntiles) step<true, 3>(st, S, it, i + 3, w, lane, tid);
      if (i + 4 < it.ntiles) step<true, 4>(st, S, it, i + 4, w, lane, tid);
      if (i + 5 < it.ntiles) step<true, 5>(st, S, it, i + 5, w, lane, tid);
    }
  } else {
    for (int i = 0; i < it.ntiles; i += 4) {
      step<false, 0>(st, S, it, i, w, lane, tid);
      if (i + 1 < it.ntiles) step<false, 1>(st, S, it, i + 1, w, lane, tid);
      if (i + 2 < it.ntiles) step<false, 2>(st, S, it, i + 2, w, lane, tid);
      if (i + 3 < it.ntiles) step<false, 3>(st, S, it, i + 3, w, lane, tid);
    }
  }

  wait_vm<0>();  // no copy may still be landing in LDS when the workgroup ends
  // the value products are asm: cover their result latency before the
  // vector ALU reads the accumulators
#pragma unroll
  for (int x = 0; x < DC / 32; ++x) {
    if (x == VBLK) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(st.O[x]));
    else asm volatile("" : "+a"(st.O[x]));
  }
  // ---- normalised partials and log-sum-exp (base 2) of this wave's heads,
  // written head by head (one 1 KB row of 512 fp16 per head). The
  // accumulator holds a head per lane, so the wave turns it around in LDS:
  // every wave's copies have landed and every wave is past its last tile
  // read once all have reached the barrier, so the tile buffers are free.
  __builtin_amdgcn_s_barrier();
  // (a row that saw no token, possible with several new tokens, has l = 0:
  // partial 0, log-sum-exp -inf)
  if (half == 0) lse[static_cast<size_t>(k) * H + head] = st.l > 0.0f ? st.m + log2f(st.l) : -INFINITY;
  if (FP8) {
    const float inv = st.l > 0.0f ? 1.0f / st.l : 0.0f;
    char *tb = g_lds + w * 32 * OROW;
#pragma unroll
    for (int cb = 0; cb < DC / 32; ++cb) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<_Float16>(st.O[cb][4 * g4 + e] * inv);
        // head lane%32, columns 32 cb + 8 g4 + 4 half .. +3
        *reinterpret_cast<f16x4 *>(tb + (lane & 31) * OROW + 64 * cb + 16 * g4 + 8 * half) = v;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // the rows come from other lanes
    uint16_t *orow = ob + static_cast<size_t>(32 * w) * DC + 8 * lane;
#pragma unroll
    for (int h = 0; h < 32; ++h)
      *reinterpret_cast<u32x4 *>(orow + h * DC) = *reinterpret_cast<const u32x4 *>(tb + h * OROW + 16 * lane);
  } else {
    // this wave holds columns 128 w .. of every head: every head's softmax
    // denominator through LDS, then each head's 128 columns (256 bytes) as
    // one quarter row in LDS, stored as 16-byte pieces of the head's row
    using M = Map<false>;
    if (lane < 32) reinterpret_cast<float *>(g_lds + M::aex() + 16 * lane)[w] = st.l;
    wait_lds();
    __builtin_amdgcn_s_barrier();
    const f32x4 l4 = *reinterpret_cast<const f32x4 *>(g_lds + M::aex() + 16 * (lane & 31));
    f32x4 inv4;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) inv4[hb] = l4[hb] > 0.0f ? 1.0f / l4[hb] : 0.0f;
    // one head block at a time, so the stores of a block's rows start while
    // the next block is converted (with every workgroup writing its partial
    // at once, the stores are bound by the write bandwidth)
    char *tb = g_lds + w * 128 * OROWQ;
    uint16_t *orow = ob + 128 * w + 8 * (lane & 15);
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int x = 4 * cb + hb;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = static_cast<_Float16>(st.O[x][4 * g4 + e] * inv4[hb]);
          // head 32 hb + lane%32, columns 32 cb + 8 g4 + 4 half .. +3 of this wave's 128
          *reinterpret_cast<f16x4 *>(tb + (32 * hb + (lane & 31)) * OROWQ + 64 * cb + 16 * g4 + 8 * half) = v;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // the rows come from other lanes
#pragma unroll
      for (int x = 8 * hb; x < 8 * hb + 8; ++x) {
        const int h = 4 * x + (lane >> 4);
        *reinterpret_cast<u32x4 *>(orow + static_cast<size_t>(h) * DC) =
            *reinterpret_cast<const u32x4 *>(tb + h * OROWQ + 16 * (lane & 15));
      }
    }
  }
}

// One workgroup per (range, head block): range j's items one after the other.
template <bool FP8>
__global__ __launch_bounds__(256, 1) void splitk_kernel(SplitArgs args) {
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
    splitk_item<FP8>(cache_of(a), a->H, a->Hr, a->q_len, k, y, a->items, a->seqs, a->Q, a->opart, a->lse, a->status);
  }
}

}  // namespace

// MLA_FP8_WIDEN=1 in the environment runs fp8 caches through the widening
// kernel (fp16 products) instead of the fp8 matrix-core one, for comparing
// the two on the same inputs.
static bool fp8_widen() {
  const char *e = std::getenv("MLA_FP8_WIDEN");
  return e && e[0] == '1';
}

hipError_t launch_decode_fast(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t q_len, int32_t n_items,
                              int32_t n_ranges, const int32_t *ranges, const WorkItem *items, const SeqInfo *seqs,
                              const uint16_t *q, uint16_t *opart, float *lse, int32_t *status) {
  if (n_items == 0 || n_ranges == 0) return hipSuccess;
  const int H = d.n_heads * q_len;
  const dim3 grid(n_ranges * (H / 128));
  const SplitArgs args{c, H, d.n_heads, q_len, n_items, n_ranges, ranges, items, seqs, q, opart, lse, status};
  if (c.latent_dtype == MLA_FP8_E4M3) {
    if (!fp8_widen())
      return launch_decode_fast8(s, d, c, q_len, n_items, n_ranges, ranges, items, seqs, q, opart, lse, status);
    return launch_kernel(splitk_kernel<true>, grid, 256, 0, s, args);
  }
  return launch_kernel(splitk_kernel<false>, grid, 256, 0, s, args);
}

}  // namespace mla
