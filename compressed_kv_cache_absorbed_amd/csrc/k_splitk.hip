// Split-K flash-decode over the latent cache (the hot loop of MLA decode).
//
// One workgroup per work item (sequence b, tokens [t0, t1)) and 128 heads,
// four waves. For every tile of 32 cached tokens
//   S^T [32 tok x 32 heads] = K [32 x 576] Q^T [576 x 32]   wave w: heads 32 w ..
//   online softmax per head, base 2 (Q is pre-scaled by scale * log2 e)
//   O^T [128 x 128 heads]  += C^T [128 x 32 tok] P^T [32 tok x 128]
//                                                     wave w: latent columns 128 w ..
// where K = [c_kv | k_rope] rows and C = the c_kv part of the same rows: the
// score is the content term plus the positional term ("DeepSeek MLA" card),
// and both products read the one tile, reused by all 128 heads, because W_UK
// is already folded into Q and W_UV is applied after the loop ("02 —
// Multi-Latent Attention (MLA)", "Coste de cómputo"). Each wave scores its
// own 32 heads, then hands P (fp16) and the rescale factors to every wave
// through LDS, and accumulates its quarter of the latent columns for all
// heads: each value fragment is read once and used by four products.
//
// Arithmetic: both products take fp16 operands with fp32 accumulation. The
// absorbed query arrives in fp16; cached bf16 (or e4m3) values are widened to
// fp16 exactly (any bf16 value below 65504 in magnitude, every e4m3 value).
//
// Memory pipeline: each tile is copied global -> LDS with direct-to-LDS loads
// (global_load_lds_dwordx4, no registers), issued three tiles ahead and
// spread over the score products; the widening of the next tile is spread
// over both products. A bare s_barrier plus explicit waits separates
// the steps. The tile loop is unrolled by the buffer count so every LDS
// address is a per-lane base plus a constant.
//
// LDS tile layout (16-bit elements), chosen so that both fragment reads are
// free of bank conflicts and every copy is a plain row copy:
//   latent: token t at 1072 t (1024 bytes of data + 48 of padding; the odd
//           stride of 67 chunks of 16 bytes spreads tokens over the banks),
//   k_rope: token t at 128 t in a region of its own, chunk c of the row at
//           position c ^ ((t >> 1) & 7).
//
// fp8 latents: raw rows [512 e4m3 codes | 64 bf16 k_rope] (640 bytes) are
// loaded into a raw buffer and widened into the tile layout above; the
// per-token scale multiplies the content score and P.
#include <cmath>

#include "device_util.hpp"

namespace mla {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_S16X4(p) ((__attribute__((address_space(3))) s16x4 *)(p))
// LDS byte offset of a __shared__ array (a link-time constant when applied
// to the array itself).
#define LDS_OFF(arr) static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char *)(arr)))

namespace sk {
constexpr int DC = 512, D = 576;
constexpr int T = kTile;             // 32 tokens per tile
constexpr int LROW = 1072;           // latent row stride in LDS (bytes)
constexpr int LTILE = T * LROW;      // 34304
constexpr int RTILE = T * 128;       // 4096: k_rope rows
constexpr int RAW_ROWB = 640;        // fp8 row: 512 codes + 128 bytes k_rope
constexpr int RAW_TILE = T * RAW_ROWB;                 // 20480
constexpr int RAW_DMA_PER_WAVE = RAW_TILE / 1024 / 4;  // 5
constexpr int SLACK = 8;             // running max is kept unless exceeded by 2^8
constexpr int SPF = 3;               // score fragments read ahead of their product
constexpr int VBLK = 15;             // bf16 path: the output block kept in VGPRs (its AGPRs hold the scores)

// LDS map. bf16 latents: four fp16 tiles. fp8 latents: two fp16 tiles, three
// raw tiles and their per-token scales. Both: the P exchange (8 KB), the
// per-head rescale factors and the final denominators.
template <bool FP8> struct Map {
  static constexpr int NBUF = FP8 ? 2 : 4;
  static constexpr int lat(int b) { return LTILE * b; }
  static constexpr int rope(int b) { return LTILE * NBUF + RTILE * b; }
  static constexpr int raw(int r) { return LTILE * NBUF + RTILE * NBUF + RAW_TILE * r; }
  static constexpr int scl(int r) { return raw(3) + 256 * r; }
  static constexpr int sclbf(int b) { return scl(3) + 128 * b; }
  static constexpr int px() { return FP8 ? sclbf(2) : rope(NBUF); }
  static constexpr int alpha() { return px() + 8192; }
  static constexpr int stat() { return alpha() + 512; }
  static constexpr int end() { return stat() + 512; }
};
constexpr int LDS_BYTES = Map<false>::end() > Map<true>::end() ? Map<false>::end() : Map<true>::end();
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
}  // namespace sk

__shared__ __attribute__((aligned(1024))) char g_lds[sk::LDS_BYTES];

namespace {

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// Value products with the accumulator's register file fixed (bf16 path:
// every output block in AGPRs but one, whose AGPRs hold the scores), so the
// compiler never moves a block between files. Operands come from LDS reads
// (waited for by lgkmcnt) or from the rescale, which runs long before; the
// leading s_nop covers a vector-ALU write of the VGPR-form accumulator.
__device__ __forceinline__ void mfma_acc_a(f32x16 &c, f16x8 a, f16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc_v(f32x16 &c, f16x8 a, f16x8 b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}

// Score products (fp16 x fp16 -> fp32) in VGPR form, issued as inline asm: the compiler would
// otherwise give every matrix-core accumulator of the kernel the AGPR form, and
// the 256 output registers already fill the AGPR file. srcC is the destination
// itself (exact overlap, same opcode: back-to-back accumulation is allowed);
// the first product of a chain uses the inline constant 0 as srcC. Its result
// is read by the vector ALU only after mfma_vgpr_drain().
// The leading s_nop gives the wait states a matrix-core read of a register
// needs after a vector-ALU write of it (the compiler may move operands with
// VALU instructions just before); it does not know this asm is a matrix-core
// op and would not insert them.
__device__ __forceinline__ f32x16 mfma_vgpr_first(f16x8 a, f16x8 b) {
  f32x16 d;
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma_vgpr_acc(f32x16 &c, f16x8 a, f16x8 b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}

// Wait states between the last score product and any vector-ALU read of its
// result (the hardware does not interlock this; 32 covers the 16-pass case).
// Tied to both accumulators so no read can be scheduled above it.
__device__ __forceinline__ void mfma_vgpr_drain(f32x16 &x, f32x16 &y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void mfma_vgpr_drain(f32x16 &x) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x));
}


// 2 bf16 (one dword) -> 2 fp16, exact for |x| < 65504 (a bf16 significand
// fits in fp16's); round-toward-zero saturates larger magnitudes to +-65504.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// k_rope chunk swizzle: chunk c of token t's row sits at c ^ rsw(t).
__device__ __forceinline__ int rsw(int t) { return (t >> 1) & 7; }

// A copy of a thread index the compiler cannot see through, so per-tile
// address arithmetic is recomputed in place instead of hoisted into live
// registers.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// vmcnt(n) with expcnt / lgkmcnt left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// vmcnt(n) and lgkmcnt(0): this wave's copies into the tile the next step
// widens have landed, and its own LDS writes are done, before the barrier.
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Direct-to-LDS loads (global_load_lds_dword / _dwordx4, SGPR base + 32-bit
// lane offset): lane i's 4 / 16 bytes from base + voff land at LDS byte
// lds_addr + 4 i / 16 i. Issued as inline asm so the compiler's own LDS-DMA
// tracking (which, lacking alias-scope information, would wait for every
// outstanding copy before any LDS read) stays out of the way; the kernel waits
// for its copies explicitly with wait_vm<>(). The instructions have no
// register results, and VMEM operations the compiler does not see can only
// make its own vmcnt waits stricter, never too weak.
__device__ __forceinline__ void lds_dma16(const char *base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const char *base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}

struct Item {
  const char *rows;
  const float *scale;
  int64_t stride, row0;
  int t0, t1, ntiles;
};

// Where tile `tile` of an item starts in global memory, and its last valid
// token (tokens past it repeat that row: finite data, masked out of the
// softmax).
struct TileSrc {
  const char *base;   // row of the tile's first token
  const char *sbase;  // fp8 scales
  int64_t stride;
  int tmax;
};
__device__ __forceinline__ TileSrc tile_src(const Item &it, int tile) {
  const int ts = it.t0 + tile * sk::T;
  TileSrc r;
  r.base = it.rows + (it.row0 + ts) * it.stride;
  r.sbase = reinterpret_cast<const char *>(it.scale + it.row0 + ts);
  r.stride = it.stride;
  r.tmax = it.t1 - 1 - ts;
  return r;
}

// Source of the k_rope copy of wave w: lane i reads chunk (i % 8) ^ rsw(t)
// of token t = 8 w + i / 8, clamped to the item's last token. The base is
// the wave's first (clamped) row, so the lane offset stays within 8 rows and
// never goes negative, also for a tile past the item's end (tmax < 0).
struct RopeSrc {
  const char *base;
  uint32_t voff;
};
__device__ __forceinline__ RopeSrc rope_src(const TileSrc &src, int w, int lane) {
  const int ln = opaque(lane);
  const int t = 8 * w + (ln >> 3);
  const int t0 = min(8 * w, src.tmax);
  RopeSrc r;
  r.base = src.base + static_cast<int64_t>(t0) * src.stride;
  r.voff = static_cast<uint32_t>(min(t, src.tmax) - t0) * static_cast<uint32_t>(src.stride) + 1024u +
           16u * static_cast<uint32_t>((ln & 7) ^ rsw(t));
  return r;
}

// bf16 tile copy, 9 loads per wave (w uniform): x < 8 copies the 1024 latent
// bytes of token 8 w + x into its LDS row (lane i: bytes 16 i .. 16 i + 15);
// x = 8 copies the k_rope parts of tokens 8 w .. 8 w + 7 (lane i: token
// 8 w + i / 8, physical chunk i % 8, which holds chunk (i % 8) ^ rsw(token)).
template <int B>
__device__ __forceinline__ void dma_bf16_piece(const TileSrc &src, int w, int lane, int x) {
  using M = sk::Map<false>;
  const uint32_t lds0 = LDS_OFF(g_lds);
  if (x < 8) {
    const int t = 8 * w + x;
    const char *row = src.base + static_cast<int64_t>(min(t, src.tmax)) * src.stride;
    lds_dma16(row, static_cast<uint32_t>(16 * lane), lds0 + M::lat(B) + sk::LROW * t);
  } else {
    const RopeSrc r = rope_src(src, w, lane);
    lds_dma16(r.base, r.voff, lds0 + M::rope(B) + 1024 * w);
  }
}
template <int B>
__device__ __forceinline__ void dma_bf16(const Item &it, int tile, int w, int lane) {
  const TileSrc src = tile_src(it, tile);
#pragma unroll
  for (int x = 0; x < 9; ++x) dma_bf16_piece<B>(src, w, lane, x);
}

// Raw fp8 tile copy, 6 loads per wave: x < 5 copies rows (640 bytes each,
// unswizzled, 40 chunks of 16 bytes), x = 5 the per-token scales (every wave
// loads them, into the same place, so that every wave issues the same number
// of loads).
template <int R>
__device__ __forceinline__ void dma_raw_piece(const TileSrc &src, int w, int lane, int x) {
  using M = sk::Map<true>;
  const uint32_t lds0 = LDS_OFF(g_lds);
  const int ln = opaque(lane);
  if (x < sk::RAW_DMA_PER_WAVE) {
    const int q = sk::RAW_DMA_PER_WAVE * w + x;
    const int P = 64 * q + ln;
    const int t = P / 40;
    const int ch = P - 40 * t;
    const uint32_t voff = static_cast<uint32_t>(min(t, src.tmax) * static_cast<int>(src.stride) + ch * 16);
    lds_dma16(src.base, voff, __builtin_amdgcn_readfirstlane(lds0 + M::raw(R) + 1024u * q));
  } else {
    lds_dma4(src.sbase, static_cast<uint32_t>(min(ln & 31, src.tmax) * 4), lds0 + M::scl(R));
  }
}
template <int R>
__device__ __forceinline__ void dma_raw(const Item &it, int tile, int w, int lane) {
  const TileSrc src = tile_src(it, tile);
#pragma unroll
  for (int x = 0; x <= sk::RAW_DMA_PER_WAVE; ++x) dma_raw_piece<R>(src, w, lane, x);
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

// Widening a raw fp8 tile into an fp16 tile: 1280 raw chunks, 5 per thread
// (chunk q = tid + 256 x: token q / 40, chunk q % 40 of the row); a code
// chunk becomes two latent fp16 chunks, a k_rope chunk one.
template <int R>
__device__ __forceinline__ u32x4 widen_fp8_load(int tid, int x) {
  return *reinterpret_cast<const u32x4 *>(g_lds + sk::Map<true>::raw(R) + (tid + 256 * x) * 16);
}
template <int B>
__device__ __forceinline__ void widen_fp8_store(int tid, int x, u32x4 v) {
  using M = sk::Map<true>;
  const int q = tid + 256 * x;
  const int t = q / 40, ch = q - 40 * t;
  if (ch < 32) {
    u32x4 lo, hi;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      lo[2 * k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[k], 1.0f, false));
      lo[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[k], 1.0f, true));
      hi[2 * k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[k + 2], 1.0f, false));
      hi[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[k + 2], 1.0f, true));
    }
    char *row = g_lds + M::lat(B) + sk::LROW * t + 32 * ch;
    *reinterpret_cast<u32x4 *>(row) = lo;
    *reinterpret_cast<u32x4 *>(row + 16) = hi;
  } else {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = bf16x2_to_f16x2(v[k]);
    *reinterpret_cast<u32x4 *>(g_lds + M::rope(B) + 128 * t + 16 * ((ch - 32) ^ rsw(t))) = r;
  }
}
template <int R, int B>
__device__ __forceinline__ void widen_fp8(int tid_) {
  using M = sk::Map<true>;
  const int tid = opaque(tid_);
  if (tid < sk::T)
    reinterpret_cast<float *>(g_lds + M::sclbf(B))[tid] = reinterpret_cast<const float *>(g_lds + M::scl(R))[tid];
#pragma unroll
  for (int x = 0; x < sk::RAW_TILE / 16 / 256; ++x) widen_fp8_store<B>(tid, x, widen_fp8_load<R>(tid, x));
}

// Per-lane state of one wave. Wave w scores heads 32 w .. 32 w + 31 (its
// Q fragments and softmax statistics) and accumulates latent columns
// 128 w .. 128 w + 127 of the output for all 128 heads: O[4 j + hb] holds
// columns 128 w + 32 j .. +31 of head block hb.
struct WaveState {
  f16x8 qf[sk::D / 16];   // absorbed query (fp16), B operand of the scores
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
// Value A fragment (transposed read): 16-lane group g, lane j in it points
// at token 16 kb + 8 h + tt (tt = 4 (g/2) + j/4), latent column
// 128 w + 32 jb + dd (dd = 16 (g%2) + 4 (j%4)). The P fragments follow the
// lane index directly.
struct ValueBase {
  int vl, pl;
};
template <bool FP8, int B>
__device__ __forceinline__ ValueBase value_base(int lane_, int w) {
  using M = sk::Map<FP8>;
  const int ln = opaque(lane_);
  const int g = (ln >> 4) & 3, j = ln & 15;
  const int tt = 4 * (g >> 1) + (j >> 2);
  const int dd = 16 * (g & 1) + 4 * (j & 3);
  ValueBase b;
  b.vl = sk::LROW * tt + 2 * (128 * w + dd) + (B < 2 ? 0 : M::lat(2));
  b.pl = M::px() + 16 * ln;
  return b;
}

// Fragment reads. Score A fragment kk: token hl, dims 16 kk + 8 half .. +7
// (one 16-byte read; latent for kk < 32, k_rope after). Value A fragment
// (j, kb): latent columns 128 w + 32 j + .., tokens 16 kb + 4 (g/2) + e and
// + 8 (two transposed 8-byte reads). Value B fragment (hb, kb): P of head
// block hb, k-step kb, as the scoring wave held it.
template <bool FP8, int B>
__device__ __forceinline__ f16x8 score_frag(const ScoreBase &sb, int kk) {
  using M = sk::Map<FP8>;
  const char *p = kk < 32 ? g_lds + sb.sl + (B < 2 ? M::lat(B) : M::lat(B) - M::lat(2)) + 32 * kk
                          : g_lds + (sb.sr ^ (32 * (kk - 32))) + (M::rope(B) - M::rope(0));
  return *reinterpret_cast<const f16x8 *>(p);
}
__device__ __forceinline__ f16x8 p_frag(const ValueBase &vb, int hb, int kb) {
  return *reinterpret_cast<const f16x8 *>(g_lds + vb.pl + 1024 * (2 * hb + kb));
}
template <bool FP8, int B>
__device__ __forceinline__ f16x8 value_frag(const ValueBase &vb, int j, int kb) {
  using M = sk::Map<FP8>;
  const char *p0 = g_lds + vb.vl + (B < 2 ? M::lat(B) : M::lat(B) - M::lat(2)) + sk::LROW * 16 * kb + 64 * j;
  const char *p1 = p0 + sk::LROW * 8;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_S16X4(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_S16X4(p1));
  f16x8 a;
  a.lo = __builtin_bit_cast(f16x4, lo);
  a.hi = __builtin_bit_cast(f16x4, hi);
  return a;
}

// Work a step hides under its matrix-core loops: score_step(kk) runs after
// score product kk, value_step(n) after value product n; each issues at most
// one load or one convert-and-store.
//
// bf16 latents: the 9 direct loads of tile i+3 go out under the score
// products (one every fourth product, the k_rope part at product 32), and so
// does the widening of this wave's rows of tile i+2, 9 chunks of 16 bytes per
// thread: the score products leave LDS bandwidth to spare, the value
// products (transposed reads of the whole tile by every wave) do not. Chunk
// x is loaded after product 16 + 2 x, once this wave's copies of tile i+2
// have landed (waited for at product 16: only this step's first 5 copies
// may still fly), and converted and stored two products later.
//
// Both run unconditionally, also in an item's last steps: a copy of a tile
// past the item's end re-reads its last row (in bounds, cached) into a
// buffer nobody reads any more, and the widening of such a tile rewrites
// that dead buffer. Branch-free steps let the compiler count outstanding
// LDS operations exactly, so no wait drains the fragment prefetch. The
// latent copy's source row pointer advances by the stride per row (no
// multiply), and stops at the item's last row.
template <int DMA_BUF, int WIDEN_BUF>
struct HideBf16 {
  const char *row;        // latent source of the next copy
  const char *rope_base;  // the k_rope copy's base row (rope_src)
  int64_t stride;
  int lim;                // rows 8 w + x with x <= lim exist; later ones repeat the last
  uint32_t rope_voff;     // this lane's k_rope source offset from rope_base
  int w, lane, tid;
  u32x4 v[2];
  __device__ __forceinline__ void score_step(int kk) {
    using M = sk::Map<false>;
    if (kk % 4 == 0 && kk / 4 < 8) {
      const int x = kk / 4;
      lds_dma16(row, static_cast<uint32_t>(16 * lane), LDS_OFF(g_lds) + M::lat(DMA_BUF) + sk::LROW * (8 * w + x));
      row += x + 1 <= lim ? stride : 0;
    }
    if (kk == 32) lds_dma16(rope_base, rope_voff, LDS_OFF(g_lds) + M::rope(DMA_BUF) + 1024 * w);
    if (kk == 16) {
      wait_vm<5>();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kk >= 18 && kk % 2 == 0 && (kk - 18) / 2 < 9) {
      const int x = (kk - 18) / 2;
      widen_bf16_store<WIDEN_BUF>(tid, x, v[x & 1]);
    }
    if (kk >= 16 && kk % 2 == 0 && (kk - 16) / 2 < 9) {
      const int x = (kk - 16) / 2;
      v[x & 1] = widen_bf16_load<WIDEN_BUF>(tid, x);
    }
  }
  __device__ __forceinline__ void value_step(int) {}
};

struct NoHide {
  __device__ __forceinline__ void score_step(int) {}
  __device__ __forceinline__ void value_step(int) {}
};

// fp8 latents: the 6 direct loads of raw tile i+3 (one every sixth score
// product) and the widening of raw tile i+1 into fp16 buffer (i+1) % 2 (one
// raw chunk every sixth value product, converted three products later; the
// scales move with the last one).
template <int DMA_RAW, int WIDEN_RAW, int WIDEN_BUF>
struct HideFp8 {
  TileSrc src;
  int w, lane, tid;
  bool dma_on, widen_on;
  u32x4 v;
  __device__ __forceinline__ void score_step(int kk) {
    if (kk % 6 == 0 && kk / 6 <= sk::RAW_DMA_PER_WAVE && dma_on) dma_raw_piece<DMA_RAW>(src, w, lane, kk / 6);
  }
  __device__ __forceinline__ void value_step(int n) {
    using M = sk::Map<true>;
    constexpr int NX = sk::RAW_TILE / 16 / 256;
    const int x = n / 6;
    if (x < NX && widen_on) {
      if (n % 6 == 0) v = widen_fp8_load<WIDEN_RAW>(tid, x);
      if (n % 6 == 3) widen_fp8_store<WIDEN_BUF>(tid, x, v);
    }
    if (n == 2 * (sk::DC / 32) - 1 && widen_on && tid < sk::T)
      reinterpret_cast<float *>(g_lds + M::sclbf(WIDEN_BUF))[tid] =
          reinterpret_cast<const float *>(g_lds + M::scl(WIDEN_RAW))[tid];
  }
};

// Value products of one tile (fp16 buffer B), after the P exchange:
// O^T += C^T P^T over this wave's 128 latent columns, all heads, with the
// rescale of the accumulators first when any head's running max moved.
template <bool FP8, int B, class Hide>
__device__ __forceinline__ void pv_phase(WaveState &st, Hide &hide, bool fresh) {
  using namespace sk;
  using M = Map<FP8>;
  // k-step kb, column block j, head block hb. The P fragments of the
  // second k-step are read during the second half of the first, its value
  // fragments two to six products ahead of their first use.
  const ValueBase vb = value_base<FP8, B>(st.lane, st.w);
  f16x8 fa[2][4], fb[2][4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) fb[0][hb] = p_frag(vb, hb, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) fa[0][j] = value_frag<FP8, B>(vb, j, 0);
  float al[4];
  const int hl = opaque(st.lane) & 31;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) al[hb] = reinterpret_cast<const float *>(g_lds + M::alpha())[32 * hb + hl];
  // (an item's first tile needs none: the accumulators are still zero)
  if (!fresh && __any(al[0] != 1.0f || al[1] != 1.0f || al[2] != 1.0f || al[3] != 1.0f)) {
    // one 16-register block at a time through VGPRs, back into AGPRs
#pragma unroll
    for (int x = 0; x < DC / 32; ++x) {
      f32x16 t = st.O[x];
      asm volatile("" : "+v"(t));
      t *= al[x & 3];
      st.O[x] = t;
      asm volatile("" : "+a"(st.O[x]));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      const int j = idx >> 2, hb = idx & 3;
      if (kb == 0 && idx >= 8 && idx < 12) fb[1][idx - 8] = p_frag(vb, idx - 8, 1);
      if ((kb == 0 && (idx == 12 || idx == 14)) || (kb == 1 && (idx == 2 || idx == 6))) {
        const int jn = kb == 0 ? (idx - 12) / 2 : 2 + (idx - 2) / 4;
        fa[1][jn] = value_frag<FP8, B>(vb, jn, 1);
      }
      st.O[4 * j + hb] = mfma32(fa[kb][j], fb[kb][hb], st.O[4 * j + hb]);
      hide.value_step(16 * kb + idx);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}


// One tile (fp16 buffer B): both contractions are software-pipelined by hand
// (fragment reads run ahead of the matrix-core op that consumes them) and
// each step is fenced with a scheduling barrier, so the compiler keeps the
// order and the register footprint small instead of hoisting every read. The
// hidden work of the step sits after each product, where it runs while the
// matrix core is busy.
template <bool FP8, int B, class Hide>
__device__ __forceinline__ void compute_tile(WaveState &st, int valid, bool fresh, Hide &hide) {
  using namespace sk;
  using M = Map<FP8>;
  const int half = opaque(st.lane) >> 5;
  const ScoreBase sb = score_base<FP8, B>(st.lane);
  const float *tscl = reinterpret_cast<const float *>(g_lds + M::sclbf(B));
  // ---- S^T = K Q^T. bf16: one chain over all 36 k-steps (back-to-back
  // accumulation into the same registers runs at the full matrix-core rate).
  // fp8: Sa accumulates the 32 latent k-steps, Sb the 4 RoPE k-steps;
  // s = scale Sa + Sb.
  f32x16 Sa, Sb;
  {
    f16x8 af[SPF + 1];
#pragma unroll
    for (int j = 0; j < SPF; ++j) af[j] = score_frag<FP8, B>(sb, j);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (kk + SPF < D / 16) af[(kk + SPF) % (SPF + 1)] = score_frag<FP8, B>(sb, kk + SPF);
      const f16x8 a = af[kk % (SPF + 1)];
      if (FP8) {
        if (kk < DC / 16) {
          if (kk == 0) Sa = mfma_vgpr_first(a, st.qf[kk]);
          else mfma_vgpr_acc(Sa, a, st.qf[kk]);
        } else {
          if (kk == DC / 16) Sb = mfma_vgpr_first(a, st.qf[kk]);
          else mfma_vgpr_acc(Sb, a, st.qf[kk]);
        }
      } else {
        if (kk == 0) Sa = mfma_vgpr_first(a, st.qf[kk]);
        else mfma_vgpr_acc(Sa, a, st.qf[kk]);
      }
      hide.score_step(kk);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (FP8) mfma_vgpr_drain(Sa, Sb);
    else mfma_vgpr_drain(Sa);
  }
  float S[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) S[r] = FP8 ? fmaf(Sa[r], tscl[8 * (r >> 2) + 4 * half + (r & 3)], Sb[r]) : Sa[r];
  if (valid < T) {  // the item's last tile only (a real branch: the asm cannot be speculated)
    asm volatile("; tail mask");
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + 4 * half + (r & 3) >= valid) S[r] = -INFINITY;
  }
  // ---- online softmax (this lane's head: 16 tokens here, 16 in lane ^ 32).
  // Scores are in log2 units; exp2 of a value below -126 may flush to zero,
  // which is below the fp16 resolution of P anyway.
  float mx = fmaxf(S[0], S[1]);
#pragma unroll
  for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(S[r], S[r + 1]));
  mx = pair_max(mx);
  const float m_new = mx > st.m + SLACK ? mx : st.m;
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  float psum = 0.0f;
  f16x8 P[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float p = __builtin_amdgcn_exp2f(S[r] - m_new);
    psum += p;
    if (FP8) p *= tscl[8 * (r >> 2) + 4 * half + (r & 3)];
    P[r >> 3][r & 7] = static_cast<_Float16>(p);
  }
  st.l = fmaf(st.l, alpha, pair_sum(psum));
  st.m = m_new;
  // ---- hand P and alpha of this wave's heads to every wave
  const int ln = opaque(st.lane);
  char *px = g_lds + M::px() + 16 * ln + 2048 * st.w;
  *reinterpret_cast<f16x8 *>(px) = P[0];
  *reinterpret_cast<f16x8 *>(px + 1024) = P[1];
  if (half == 0) reinterpret_cast<float *>(g_lds + M::alpha())[32 * st.w + (ln & 31)] = alpha;
  wait_lds();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  pv_phase<FP8, B>(st, hide, fresh);
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
  float m4[4], mx, m_new, alpha, psum, pe, prev;
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
    sm.m_new = sm.mx > st.m + SLACK ? sm.mx : st.m;
    sm.alpha = __builtin_amdgcn_exp2f(st.m - sm.m_new);
    sm.psum = 0.0f;
  } else if (kk < 23) {
    const int r = kk - 7;
    const float p = __builtin_amdgcn_exp2f(S[r] - sm.m_new);
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

// Score products of one bf16-path tile (fp16 buffer B): one chain over the
// 36 k-steps, accumulating in AGPRs (S), with the softmax of the previous
// tile's scores (Sv, a VGPR copy) woven in when SOFTMAX is set. An AGPR-form
// chain leaves the VGPR file's ports to the vector ALU, and the compiler's
// own hazard handling needs no blanket wait before each product, so the
// softmax's vector work runs in the products' shadow (with a VGPR-form
// chain, or an s_nop before each product, it mostly serialises).
template <int B, bool SOFTMAX, class Hide>
__device__ __forceinline__ void score_chain_bf16(WaveState &st, f32x16 &S, const f32x16 &Sv, Softmax &sm,
                                                 Hide &hide) {
  using namespace sk;
  const ScoreBase sb = score_base<false, B>(st.lane);
  f16x8 af[SPF + 1];
#pragma unroll
  for (int j = 0; j < SPF; ++j) af[j] = score_frag<false, B>(sb, j);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (kk + SPF < D / 16) af[(kk + SPF) % (SPF + 1)] = score_frag<false, B>(sb, kk + SPF);
    const f16x8 a = af[kk % (SPF + 1)];
    S = mfma32(a, st.qf[kk], kk == 0 ? f32x16{} : S);
    asm volatile("" : "+a"(S));
    hide.score_step(kk);
    if (SOFTMAX) softmax_piece(st, sm, Sv, kk);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Value A fragment of the bf16 path (transposed read): 16-lane group g,
// lane j in it points at token 16 kb + 8 h + tt (tt = 4 (g/2) + j/4), latent
// column 32 cb + dd (dd = 16 (g%2) + 4 (j%4)); the base includes the offset
// of buffers 2 and 3, beyond the 16-bit range of LDS read offsets.
template <int B>
__device__ __forceinline__ int row_value_base(int lane_) {
  using M = sk::Map<false>;
  const int ln = opaque(lane_);
  const int g = (ln >> 4) & 3, j = ln & 15;
  const int tt = 4 * (g >> 1) + (j >> 2);
  const int dd = 16 * (g & 1) + 4 * (j & 3);
  return sk::LROW * tt + 2 * dd + (B < 2 ? 0 : M::lat(2));
}
template <int B>
__device__ __forceinline__ f16x8 row_value_frag(int vl, int cb, int kb) {
  using M = sk::Map<false>;
  const char *p0 = g_lds + vl + (B < 2 ? M::lat(B) : M::lat(B) - M::lat(2)) + sk::LROW * 16 * kb + 64 * cb;
  const char *p1 = p0 + sk::LROW * 8;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_S16X4(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_S16X4(p1));
  f16x8 a;
  a.lo = __builtin_bit_cast(f16x4, lo);
  a.hi = __builtin_bit_cast(f16x4, hi);
  return a;
}

// Value products of one bf16-path tile (buffer B) for this wave's heads:
// O^T [512 x 32 heads] += C^T [512 x 32 tok] P^T [32 tok x 32 heads], 16
// column blocks x 2 k-steps, value fragments read VPF products ahead. P is
// the wave's own, used in place: in k-step kb, element e of lane l stands
// for token 16 kb + 8 (e / 4) + 4 (l / 32) + e % 4 in both operands (the
// rows the softmax left in the lane, and the tokens the transposed value
// reads fetch), an order of the 16 tokens the contraction does not see.
// Every accumulator value of a lane belongs to the lane's head, so the
// rescale is a per-lane factor.
constexpr int VPF = 4;
template <int B, class Hide>
__device__ __forceinline__ void pv_rows(WaveState &st, const Softmax &sm, Hide &hide, bool fresh) {
  using namespace sk;
  const int vl = row_value_base<B>(st.lane);
  f16x8 va[VPF + 1];
#pragma unroll
  for (int n = 0; n < VPF; ++n) va[n] = row_value_frag<B>(vl, n & 15, n >> 4);
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
    if (n + VPF < 2 * (DC / 32)) va[(n + VPF) % (VPF + 1)] = row_value_frag<B>(vl, (n + VPF) & 15, (n + VPF) >> 4);
    if (cb == VBLK) mfma_acc_v(st.O[cb], va[n % (VPF + 1)], pb[kb]);
    else mfma_acc_a(st.O[cb], va[n % (VPF + 1)], pb[kb]);
    hide.value_step(n);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One pipeline step for bf16 latents (B = i % 4), software-pipelined by one
// tile. On entry tile i+1 is widened and visible and S (AGPRs) holds tile
// i's scores; they are copied to VGPRs first. The step
//   1. runs the score products of tile i+1 (buffer B+1) into S, with the
//      softmax of tile i woven in, the copies of tile i+3 (into buffer
//      B+3, which tile i-1 used) issued under them
//      and the widening of its rows of tile i+2 (buffer B+2) after them
//      (no other wave's copies are needed: each wave widens the rows it
//      copied);
//   2. runs the value products of tile i (buffer B);
//   3. barrier: tile i+2 is ready for the next step's scores and buffer B is
//      free for the next step's copies.
// In an item's last step the scores of the tile past its end are computed
// on the finite rows that buffer holds and dropped.
template <int B>
__device__ __forceinline__ void step_bf16(WaveState &st, f32x16 &S, const Item &it, int i, int w, int lane,
                                          int tid) {
  HideBf16<(B + 3) % 4, (B + 2) % 4> h;
  const TileSrc src = tile_src(it, i + 3);
  h.stride = src.stride;
  h.lim = src.tmax - 8 * w;
  h.row = src.base + static_cast<int64_t>(min(8 * w, src.tmax)) * src.stride;
  {
    const RopeSrc r = rope_src(src, w, lane);
    h.rope_base = r.base;
    h.rope_voff = r.voff;
  }
  h.w = w;
  h.lane = lane;
  h.tid = opaque(tid);
  f32x16 Sv = S;
  asm volatile("" : "+v"(Sv));
  const int valid = min(sk::T, it.t1 - (it.t0 + i * sk::T));
  if (valid < sk::T) {  // the item's last tile only (a real branch: the asm cannot be speculated)
    asm volatile("; tail mask");
    const int lim = valid - 4 * (opaque(st.lane) >> 5);  // one register, not 16 hoisted row indices
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + (r & 3) >= lim) Sv[r] = -INFINITY;
  }
  Softmax sm;
  score_chain_bf16<(B + 1) % 4, true>(st, S, Sv, sm, h);
  pv_rows<B>(st, sm, h, i == 0);
  wait_lds();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// One pipeline step for fp8 latents (B3 = i % 3, B2 = i % 2): computes tile
// i (fp16 buffer B2) while widening raw tile i+1 into fp16 buffer (i+1) % 2
// and fetching raw tile i+3 into the raw buffer tile i came from.
template <int B3, int B2>
__device__ __forceinline__ void step_fp8(WaveState &st, const Item &it, int i, int w, int lane, int tid) {
  constexpr int N3 = (B3 + 1) % 3, N2 = (B2 + 1) % 2;
  constexpr int PER = sk::RAW_DMA_PER_WAVE + 1;
  if (i + 2 < it.ntiles) wait_vm_lds<PER>(); else wait_vm_lds<0>();
  __builtin_amdgcn_s_barrier();
  HideFp8<B3, N3, N2> h;
  h.src = tile_src(it, i + 3);
  h.w = w;
  h.lane = lane;
  h.tid = opaque(tid);
  h.dma_on = i + 3 < it.ntiles;
  h.widen_on = i + 1 < it.ntiles;
  compute_tile<true, B2>(st, min(sk::T, it.t1 - (it.t0 + i * sk::T)), i == 0, h);
}

template <bool FP8>
__global__ __launch_bounds__(256, 1) void splitk_kernel(mla_cache c, int H,
                                                        const WorkItem *__restrict__ items,
                                                        const SeqInfo *__restrict__ seqs,
                                                        const uint16_t *__restrict__ Q,
                                                        uint16_t *__restrict__ opart,
                                                        float *__restrict__ lse,
                                                        int32_t *__restrict__ status) {
  using namespace sk;
  using M = Map<FP8>;
  const int k = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane & 31, half = lane >> 5;
  const int head = blockIdx.y * 128 + 32 * w + hl;
  const WorkItem wi = items[k];
  // this workgroup's 128 heads of item k: 4 head blocks of 32 KB in the
  // fragment order of the (fp16) partials
  uint16_t *ob = opart + (static_cast<size_t>(k) * (H / 32) + blockIdx.y * 4) * (16 * 1024);

  const bool ok = c.seq_len[wi.b] == seqs[wi.b].len && wi.t0 >= 0 && wi.t0 < wi.t1 &&
                  wi.t1 <= c.seq_cap[wi.b] && static_cast<int64_t>(c.seq_start[wi.b]) >= 0 &&
                  static_cast<int64_t>(c.seq_start[wi.b]) + wi.t1 <= c.n_rows;
  if (!ok) {
    if (tid == 0 && blockIdx.y == 0) set_status(status, MLA_ERR_PLAN);
    for (int x = tid; x < 4 * 16 * 256 / 2; x += 256) reinterpret_cast<u32x4 *>(ob)[x] = u32x4{0, 0, 0, 0};
    if (half == 0) lse[static_cast<size_t>(k) * H + head] = -INFINITY;
    return;
  }
  Item it;
  it.rows = static_cast<const char *>(c.rows);
  it.scale = c.scale;
  it.stride = c.row_stride;
  it.row0 = c.seq_start[wi.b];
  it.t0 = wi.t0;
  it.t1 = wi.t1;
  it.ntiles = (wi.t1 - wi.t0 + T - 1) / T;

  // prologue loads first, so they overlap the Q fetch
  if (FP8) {
    dma_raw<0>(it, 0, w, lane);
    if (it.ntiles > 1) dma_raw<1>(it, 1, w, lane);
    if (it.ntiles > 2) dma_raw<2>(it, 2, w, lane);
  } else {
    dma_bf16<0>(it, 0, w, lane);  // tiles past the end re-read the last row, like the steps
    dma_bf16<1>(it, 1, w, lane);
    dma_bf16<2>(it, 2, w, lane);
  }

  WaveState st;
  st.w = w;
  st.lane = lane;
  {
    const uint16_t *qrow = Q + (static_cast<size_t>(wi.b) * H + head) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) st.qf[kk] = *reinterpret_cast<const f16x8 *>(qrow + 16 * kk);
  }
#pragma unroll
  for (int db = 0; db < DC / 32; ++db) {
    st.O[db] = f32x16{};
    if (!FP8 && db == VBLK) asm volatile("" : "+v"(st.O[db]));
    else asm volatile("" : "+a"(st.O[db]));
  }
  st.m = -INFINITY;
  st.l = 0.0f;

  if (FP8) {
    // widen tile 0 before the loop; each step then widens one tile ahead
    constexpr int PER = RAW_DMA_PER_WAVE + 1;
    if (it.ntiles > 2) wait_vm<2 * PER>(); else if (it.ntiles > 1) wait_vm<PER>(); else wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    widen_fp8<0, 0>(tid);
    for (int i = 0; i < it.ntiles; i += 6) {
      step_fp8<0, 0>(st, it, i, w, lane, tid);
      if (i + 1 < it.ntiles) step_fp8<1, 1>(st, it, i + 1, w, lane, tid);
      if (i + 2 < it.ntiles) step_fp8<2, 0>(st, it, i + 2, w, lane, tid);
      if (i + 3 < it.ntiles) step_fp8<0, 1>(st, it, i + 3, w, lane, tid);
      if (i + 4 < it.ntiles) step_fp8<1, 0>(st, it, i + 4, w, lane, tid);
      if (i + 5 < it.ntiles) step_fp8<2, 1>(st, it, i + 5, w, lane, tid);
    }
  } else {
    // this wave's rows of tiles 0 and 1 landed (only Q's loads, issued
    // last, may still fly) and widened; then the scores of tile 0 alone
    wait_vm<9>();
    __builtin_amdgcn_sched_barrier(0);
    widen_bf16_inplace<0>(tid);
    widen_bf16_inplace<1>(tid);
    wait_lds();
    __builtin_amdgcn_s_barrier();
    f32x16 S;
    {
      NoHide nh;
      Softmax sm;
      score_chain_bf16<0, false>(st, S, S, sm, nh);
    }
    for (int i = 0; i < it.ntiles; i += 4) {
      step_bf16<0>(st, S, it, i, w, lane, tid);
      if (i + 1 < it.ntiles) step_bf16<1>(st, S, it, i + 1, w, lane, tid);
      if (i + 2 < it.ntiles) step_bf16<2>(st, S, it, i + 2, w, lane, tid);
      if (i + 3 < it.ntiles) step_bf16<3>(st, S, it, i + 3, w, lane, tid);
    }
  }

  wait_vm<0>();  // no copy may still be landing in LDS when the workgroup ends
  if (!FP8) {
    // the value products are asm on the bf16 path: cover their result
    // latency before the vector ALU reads the accumulators
#pragma unroll
    for (int x = 0; x < DC / 32; ++x) {
      if (x == VBLK) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(st.O[x]));
      else asm volatile("" : "+a"(st.O[x]));
    }
    // ---- normalised partials and log-sum-exp (base 2) of this wave's
    // heads: register group g4 of column block cb is one 512-byte run of
    // head block w
    const float inv = 1.0f / st.l;
    if (half == 0) lse[static_cast<size_t>(k) * H + head] = st.m + log2f(st.l);
#pragma unroll
    for (int cb = 0; cb < DC / 32; ++cb) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<_Float16>(st.O[cb][4 * g4 + e] * inv);
        *reinterpret_cast<f16x4 *>(ob + ((w * 16 + cb) * 4 + g4) * 256 + 4 * lane) = v;
      }
    }
    return;
  }
  // ---- normalised partials and log-sum-exp (base 2), fp8 path: each wave
  // writes its 128 latent columns of all 128 heads, dividing by the
  // denominators the scoring waves hand over
  float *gstat = reinterpret_cast<float *>(g_lds + M::stat());
  if (half == 0) {
    gstat[32 * w + hl] = st.l;
    lse[static_cast<size_t>(k) * H + head] = st.m + log2f(st.l);
  }
  wait_lds();
  __builtin_amdgcn_s_barrier();
  // register group g4 of accumulator (j, hb) is one 512-byte run: head
  // block hb, latent block 4 w + j
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const float inv = 1.0f / gstat[32 * hb + hl];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x16 &x = st.O[4 * j + hb];
        f16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<_Float16>(x[4 * g4 + e] * inv);
        *reinterpret_cast<f16x4 *>(ob + ((hb * 16 + 4 * w + j) * 4 + g4) * 256 + 4 * lane) = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_fast(hipStream_t s, const mla_dims &d, const mla_cache &c, int32_t n_items,
                              const WorkItem *items, const SeqInfo *seqs, const uint16_t *q, uint16_t *opart,
                              float *lse, int32_t *status) {
  if (n_items == 0) return hipSuccess;
  const dim3 grid(n_items, d.n_heads / 128);
  if (c.latent_dtype == MLA_FP8_E4M3)
    return launch_kernel(splitk_kernel<true>, grid, 256, 0, s, c, d.n_heads, items, seqs, q, opart, lse, status);
  return launch_kernel(splitk_kernel<false>, grid, 256, 0, s, c, d.n_heads, items, seqs, q, opart, lse, status);
}

}  // namespace mla
