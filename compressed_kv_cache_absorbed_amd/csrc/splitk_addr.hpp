// Source addresses of the split-K kernel's tile copies (HBM -> LDS), as
// plain integer and pointer arithmetic that compiles for the host as well,
// so a CPU test can enumerate every copy of every tile of an item, past its
// end included, and check each byte read lies in the item's own rows.
//
// The invariant they keep: every lane offset is taken from a base row that
// is itself clamped to the item's last token, so offsets are never negative
// and never reach past the item's last row, also for tiles past the item's
// end (which re-read its last tile into a buffer nobody scores).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mla {
namespace sa {

constexpr int T = 32;               // tokens per tile
constexpr int RAW_ROWB = 640;       // fp8 row as copied: 512 codes + 64 bf16 k_rope
constexpr int RAW_DMA_PER_WAVE = 5; // 1 KB copies per wave per raw tile (8 rows of 640 bytes)

__host__ __device__ inline int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ inline int imax(int a, int b) { return a > b ? a : b; }

// k_rope chunk swizzle in LDS: chunk c of token t's row sits at c ^ rsw(t).
__host__ __device__ inline int rsw(int t) { return (t >> 1) & 7; }

struct Item {
  const char *rows;
  const float *scale;
  const int32_t *blocks;  // paged cache: this sequence's block table row, else nullptr
  int64_t stride, row0;
  int block_tokens, n_blocks;  // paged: rows per block, blocks in the cache
  int t0, t1, ntiles;
  int tvis;  // this wave's queries see tokens < tvis (t1, or less for an earlier one of several new tokens)
};

// Where tile `tile` of an item starts in global memory, and its last valid
// token (tokens past it repeat that row: finite data, masked out of the
// softmax). A tile past the item's end reads the item's last tile instead
// (its data is never scored), so tmax >= 0 always. Tiles start at multiples
// of 32 tokens, so a tile never straddles two blocks of a paged cache: one
// lookup per tile.
struct TileSrc {
  const char *base;   // row of the tile's first token
  const char *sbase;  // fp8 scales
  int64_t stride;
  int tmax;
};
__host__ __device__ inline TileSrc tile_src(const Item &it, int tile) {
  const int ts = it.t0 + imin(tile, it.ntiles - 1) * T;
  int64_t row = it.row0 + ts;
  if (it.blocks != nullptr) {
    // (ids outside the cache were reported when the item started; clamped here)
    const int blk = imin(imax(it.blocks[ts / it.block_tokens], 0), it.n_blocks - 1);
    row = static_cast<int64_t>(blk) * it.block_tokens + ts % it.block_tokens;
  }
  TileSrc r;
  r.base = it.rows + row * it.stride;
  r.sbase = reinterpret_cast<const char *>(it.scale + row);
  r.stride = it.stride;
  r.tmax = it.t1 - 1 - ts;
  return r;
}

// bf16 latent copy x (< 8) of wave w: the 1024 latent bytes of token
// 8 w + x, clamped to the tile's last valid token; lane i reads bytes
// 16 i .. 16 i + 15 of that row.
__host__ __device__ inline const char *latent_row(const TileSrc &src, int w, int x) {
  return src.base + static_cast<int64_t>(imin(8 * w + x, src.tmax)) * src.stride;
}

// The same rows walked incrementally (as the pipelined steps do): start at
// the wave's first clamped row, and after copy x advance one stride only
// while row 8 w + x + 1 exists (lim = tmax - 8 w).
__host__ __device__ inline const char *latent_row_first(const TileSrc &src, int w) {
  return src.base + static_cast<int64_t>(imin(8 * w, src.tmax)) * src.stride;
}
__host__ __device__ inline const char *latent_row_next(const char *row, int64_t stride, int lim, int x) {
  return row + (x + 1 <= lim ? stride : 0);
}

// Source of the k_rope copy of wave w: lane i reads chunk (i % 8) ^ rsw(t)
// of token t = 8 w + i / 8, clamped to the tile's last valid token. The base
// is the wave's first (clamped) row, so the lane offset stays within 8 rows
// and never goes negative.
struct RopeSrc {
  const char *base;
  uint32_t voff;
};
__host__ __device__ inline RopeSrc rope_src(const TileSrc &src, int w, int ln) {
  const int t = 8 * w + (ln >> 3);
  const int t0 = imin(8 * w, src.tmax);
  RopeSrc r;
  r.base = src.base + static_cast<int64_t>(t0) * src.stride;
  r.voff = static_cast<uint32_t>(imin(t, src.tmax) - t0) * static_cast<uint32_t>(src.stride) + 1024u +
           16u * static_cast<uint32_t>((ln & 7) ^ rsw(t));
  return r;
}

// Source of wave w's part of a raw fp8 tile copy: its 8 rows (tokens
// 8 w .. 8 w + 7; 5 copies of 1 KB cover them) and the tile's 32 scales,
// each clamped to the tile's last valid token; the bases are the first
// clamped row and scale.
struct RawSrc {
  const char *base, *sbase;
  int64_t stride;
  int tmax, t0, s0;
};
__host__ __device__ inline RawSrc raw_src(const TileSrc &src, int w) {
  RawSrc r;
  r.t0 = imin(8 * w, src.tmax);
  r.s0 = imin(0, src.tmax);
  r.base = src.base + static_cast<int64_t>(r.t0) * src.stride;
  r.sbase = src.sbase + 4 * static_cast<int64_t>(r.s0);
  r.stride = src.stride;
  r.tmax = src.tmax;
  return r;
}
// Raw copy x (< 5) of wave w, lane ln: the raw tile is the rows back to back,
// 40 chunks of 16 bytes each; chunk P = 64 (5 w + x) + ln holds token P / 40,
// bytes 16 (P % 40). Offset from rs.base.
__host__ __device__ inline uint32_t raw_piece_off(const RawSrc &rs, int w, int ln, int x) {
  const int q = RAW_DMA_PER_WAVE * w + x;
  const int P = 64 * q + ln;
  const int t = P / 40;
  const int ch = P - 40 * t;
  return static_cast<uint32_t>(imin(t, rs.tmax) - rs.t0) * static_cast<uint32_t>(rs.stride) +
         static_cast<uint32_t>(16 * ch);
}
// The fp8 matrix-core kernel keeps the raw rows at the same 640-byte stride
// but permutes each row's 16-byte chunks: slot p of token t's row holds
// chunk p ^ rsw8(t) (an XOR of the low three bits: a chunk stays in its
// aligned group of eight, so the 32 code chunks and the 8 k_rope chunks keep
// their places). The permutation spreads the rows over the LDS banks both
// for reads of two chunks of one row per lane and for the transposed 8-byte
// reads of 8 rows at once.
__host__ __device__ inline int rsw8(int t) { return ((t >> 2) & 1) | (((t >> 1) & 1) << 1) | (((t >> 3) & 1) << 2); }
// Raw copy x (< 5) of wave w, lane ln, into that permuted layout: slot
// P = 64 (5 w + x) + ln of the tile (token P / 40, slot P % 40) receives
// chunk (P % 40) ^ rsw8(token) of the token's row. Offset from rs.base.
// (P / 40 as (P 1639) >> 16, exact for the tile's 1280 slots: it keeps the
// division off the copies' issue path)
__host__ __device__ inline uint32_t raw_piece_off_sw(const RawSrc &rs, int w, int ln, int x) {
  const int q = RAW_DMA_PER_WAVE * w + x;
  const uint32_t P = static_cast<uint32_t>(64 * q + ln);
  const int t = static_cast<int>((P * 1639u) >> 16);
  const int ch = (static_cast<int>(P) - 40 * t) ^ rsw8(t);
  return static_cast<uint32_t>(imin(t, rs.tmax) - rs.t0) * static_cast<uint32_t>(rs.stride) +
         static_cast<uint32_t>(16 * ch);
}
// The same copies with their per-lane constants made once per item: copy x
// of wave w, lane ln fills slot P = 64 (5 w + x) + ln, which holds token
// t[x] = P / 40 and, when no token is clamped, reads t[x] stride + 16 chunk
// bytes past the tile's first row (off[x]). A tile whose last valid token
// is tmax < t[x] reads row tmax instead: off[x] - (t[x] - tmax) stride. The
// result equals rs.base + raw_piece_off_sw(rs, w, ln, x) as an address
// (tests/c/splitk_addr_check.cpp checks every case); three instructions per
// copy instead of the division and the multiplies.
struct RawLane {
  int t[RAW_DMA_PER_WAVE];
  uint32_t off[RAW_DMA_PER_WAVE];
};
__host__ __device__ inline RawLane raw_lane(int w, int ln, int64_t stride) {
  RawLane r;
  for (int x = 0; x < RAW_DMA_PER_WAVE; ++x) {
    const int P = 64 * (RAW_DMA_PER_WAVE * w + x) + ln;
    const int t = P / 40;
    r.t[x] = t;
    r.off[x] = static_cast<uint32_t>(t) * static_cast<uint32_t>(stride) + static_cast<uint32_t>(16 * ((P - 40 * t) ^ rsw8(t)));
  }
  return r;
}
// Offset of copy x from the tile's first row (TileSrc::base).
__host__ __device__ inline uint32_t raw_piece_off_lane(const RawLane &rl, int x, int tmax, int64_t stride) {
  const int d = rl.t[x] - tmax;
  return rl.off[x] - static_cast<uint32_t>(d > 0 ? d : 0) * static_cast<uint32_t>(stride);
}
// The scale copy: lane ln reads the scale of token ln % 32 (clamped), as an
// offset from rs.sbase.
__host__ __device__ inline uint32_t raw_scale_off(const RawSrc &rs, int ln) {
  return static_cast<uint32_t>(imin(ln & 31, rs.tmax) - rs.s0) * 4u;
}

// Workgroup L of a split-K launch over R ranges and Y head blocks of 128:
// range j, head block y. Workgroup L runs on XCD L % 8, so each XCD takes a
// contiguous block of ranges: a sequence's items are consecutive, and the
// splits of a sequence then share its absorbed query in that XCD's L2; the
// head blocks of one range, next to each other there, share its cache tiles.
__host__ __device__ __forceinline__ void range_of(int L, int R, int Y, int &j, int &y) {
  const int nfull = R & ~7, lfull = nfull * Y;
  if (L < lfull) {
    const int sl = L >> 3;
    j = (L & 7) * (nfull >> 3) + sl / Y;
    y = sl - (sl / Y) * Y;
  } else {
    const int r = L - lfull;
    j = nfull + r / Y;
    y = r - (r / Y) * Y;
  }
}

}  // namespace sa
}  // namespace mla
