// CPU check of the split-K kernel's tile-copy source addresses
// (compressed_kv_cache_absorbed_amd/csrc/splitk_addr.hpp, the same functions
// the kernel calls). For items of 1..5 tiles with every tail length, at
// several starting tiles, in contiguous and paged caches with padded and
// unpadded row strides, every copy of every tile the kernel issues (tiles
// past the item's end included, which re-read its last tile) is checked:
//   * each 16-byte latent or k_rope piece and each 4-byte scale lies inside
//     a row of a token the item covers, inside that row's used bytes;
//   * for a tile inside the item, the piece is the one of the token and
//     chunk the LDS layout expects (the last valid token repeats past the
//     tile's end);
//   * the incremental row walk of the pipelined steps gives the same rows as
//     the direct form;
//   * range_of maps a launch's workgroups onto every (range, head block)
//     exactly once, each XCD taking a contiguous block of ranges.
// Built host-only by __graft_entry__.build(); prints "ok <checks>" and exits
// 0, or prints the first failure and exits 1.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "splitk_addr.hpp"

using namespace mla::sa;

namespace {

long long g_checks = 0;

[[noreturn]] void fail(const char *what, int n, int t0, int tile, int w, int lane, int x) {
  std::printf("FAIL %s: item tokens [%d, %d) tile %d wave %d lane %d piece %d\n", what, t0, t0 + n, tile, w, lane, x);
  std::exit(1);
}

struct Layout {
  std::vector<char> rows;       // the cache rows (never read, only addressed)
  std::vector<float> scale;     // one per row
  std::vector<int32_t> table;   // paged: block ids of the sequence, else empty
  int64_t stride = 0;
  int64_t seq_start = 0;        // contiguous
  int bt = 0;                   // paged block tokens
  int n_blocks = 0;
  std::vector<int> tok;         // token of each row, -1 for rows of no token of the sequence
  // row of token t of the sequence
  int64_t row_of(int t) const {
    if (table.empty()) return seq_start + t;
    return static_cast<int64_t>(table[t / bt]) * bt + t % bt;
  }
  // token of row r, or -1 if the row holds no token of the sequence
  int token_of(int64_t r) const { return r >= 0 && r < static_cast<int64_t>(tok.size()) ? tok[r] : -1; }
};

Layout make_layout(int cap, int64_t stride, int bt, unsigned seed) {
  Layout L;
  L.stride = stride;
  if (bt == 0) {
    L.seq_start = 5;  // rows of another sequence before and after
    L.rows.resize(static_cast<size_t>((L.seq_start + cap + 7) * stride));
    L.scale.resize(static_cast<size_t>(L.seq_start + cap + 7));
  } else {
    L.bt = bt;
    const int nb = (cap + bt - 1) / bt;
    L.n_blocks = nb + 3;
    std::vector<int32_t> ids(L.n_blocks);
    for (int i = 0; i < L.n_blocks; ++i) ids[i] = i;
    for (int i = L.n_blocks - 1; i > 0; --i) {  // deterministic shuffle
      seed = seed * 1103515245u + 12345u;
      const int j = static_cast<int>((seed >> 8) % static_cast<unsigned>(i + 1));
      std::swap(ids[i], ids[j]);
    }
    L.table.assign(ids.begin(), ids.begin() + nb);
    L.rows.resize(static_cast<size_t>(L.n_blocks) * bt * stride);
    L.scale.resize(static_cast<size_t>(L.n_blocks) * bt);
  }
  L.tok.assign(L.scale.size(), -1);
  for (int t = 0; t < cap; ++t) L.tok[L.row_of(t)] = t;
  return L;
}

// Every copy of tile `tile` of the item [t0, t0 + n) of this layout.
void check_tile(const Layout &L, int cap, int t0, int n, int tile, bool fp8) {
  Item it{};
  it.rows = L.rows.data();
  it.scale = L.scale.data();
  it.blocks = L.table.empty() ? nullptr : L.table.data();
  it.stride = L.stride;
  it.row0 = L.table.empty() ? L.seq_start : 0;
  it.block_tokens = L.bt;
  it.n_blocks = L.n_blocks;
  it.t0 = t0;
  it.t1 = t0 + n;
  it.ntiles = (n + T - 1) / T;
  it.tvis = it.t1;
  const TileSrc src = tile_src(it, tile);
  const int eff = imin(tile, it.ntiles - 1);  // the tile whose data is read
  const int ts = t0 + eff * T;
  if (src.tmax < 0) fail("negative tmax", n, t0, tile, 0, 0, 0);
  const int used = fp8 ? RAW_ROWB : 1152;
  // byte range [off, off + len) of the rows buffer: returns the token and
  // the byte within its row, or fails
  auto locate = [&](const char *p, int len, const char *what, int w, int lane, int x, int *tok, int *byte) {
    const int64_t off = p - L.rows.data();
    if (off < 0 || off + len > static_cast<int64_t>(L.rows.size())) fail(what, n, t0, tile, w, lane, x);
    const int64_t r = off / L.stride;
    const int b = static_cast<int>(off - r * L.stride);
    const int t = L.token_of(r);
    if (t < it.t0 || t >= it.t1) fail(what, n, t0, tile, w, lane, x);
    if (b + len > used) fail(what, n, t0, tile, w, lane, x);
    *tok = t;
    *byte = b;
    ++g_checks;
  };
  for (int w = 0; w < 4; ++w) {
    if (!fp8) {
      // latent rows, direct and incremental
      const char *inc = latent_row_first(src, w);
      const int lim = src.tmax - 8 * w;
      for (int x = 0; x < 8; ++x) {
        const char *row = latent_row(src, w, x);
        if (row != inc) fail("incremental latent row", n, t0, tile, w, 0, x);
        inc = latent_row_next(inc, src.stride, lim, x);
        for (int lane = 0; lane < 64; ++lane) {
          int tok, byte;
          locate(row + 16 * lane, 16, "latent piece out of the item", w, lane, x, &tok, &byte);
          if (tok != ts + imin(8 * w + x, src.tmax) || byte != 16 * lane)
            fail("latent piece of the wrong token or chunk", n, t0, tile, w, lane, x);
        }
      }
      for (int lane = 0; lane < 64; ++lane) {
        const RopeSrc r = rope_src(src, w, lane);
        int tok, byte;
        locate(r.base + r.voff, 16, "k_rope piece out of the item", w, lane, 8, &tok, &byte);
        const int t = 8 * w + (lane >> 3);
        if (tok != ts + imin(t, src.tmax) || byte != 1024 + 16 * ((lane & 7) ^ rsw(t)))
          fail("k_rope piece of the wrong token or chunk", n, t0, tile, w, lane, 8);
      }
    } else {
      const RawSrc rs = raw_src(src, w);
      for (int x = 0; x < RAW_DMA_PER_WAVE; ++x) {
        for (int lane = 0; lane < 64; ++lane) {
          int tok, byte;
          locate(rs.base + raw_piece_off(rs, w, lane, x), 16, "raw piece out of the item", w, lane, x, &tok, &byte);
          const int P = 64 * (RAW_DMA_PER_WAVE * w + x) + lane;
          if (tok != ts + imin(P / 40, src.tmax) || byte != 16 * (P % 40))
            fail("raw piece of the wrong token or chunk", n, t0, tile, w, lane, x);
          // the permuted layout of the fp8 matrix-core kernel: the same
          // token, chunk (P % 40) ^ rsw8(P / 40), still one of the row's 40
          locate(rs.base + raw_piece_off_sw(rs, w, lane, x), 16, "permuted raw piece out of the item", w, lane, x,
                 &tok, &byte);
          if (tok != ts + imin(P / 40, src.tmax) || byte != 16 * ((P % 40) ^ rsw8(P / 40)) || byte + 16 > 640)
            fail("permuted raw piece of the wrong token or chunk", n, t0, tile, w, lane, x);
          // the same address from the per-lane constants, offset from the
          // tile's first row
          const RawLane rl = raw_lane(w, lane, src.stride);
          if (src.base + raw_piece_off_lane(rl, x, src.tmax, src.stride) != rs.base + raw_piece_off_sw(rs, w, lane, x))
            fail("per-lane raw piece address", n, t0, tile, w, lane, x);
        }
      }
      // the multiply that stands for the division by 40 is exact on every slot
      for (int P = 0; P < 32 * 40; ++P)
        if (static_cast<int>((static_cast<uint32_t>(P) * 1639u) >> 16) != P / 40) fail("slot row", n, t0, tile, w, 0, P);
      // the permutation is one within every row: each of a token's 40 slots
      // receives a different chunk
      for (int t = 8 * w; t < 8 * w + 8; ++t) {
        bool seen[40] = {};
        for (int p = 0; p < 40; ++p) {
          const int c = p ^ rsw8(t);
          if (c < 0 || c >= 40 || seen[c]) fail("raw chunk permutation", n, t0, tile, w, 0, t);
          seen[c] = true;
        }
      }
      for (int lane = 0; lane < 64; ++lane) {
        const int64_t off = (rs.sbase + raw_scale_off(rs, lane)) - reinterpret_cast<const char *>(L.scale.data());
        if (off < 0 || off % 4 || off + 4 > static_cast<int64_t>(L.scale.size() * 4))
          fail("scale out of the array", n, t0, tile, w, lane, 5);
        const int t = L.token_of(off / 4);
        if (t != ts + imin(lane & 31, src.tmax)) fail("scale of the wrong token", n, t0, tile, w, lane, 5);
        ++g_checks;
      }
    }
  }
}

}  // namespace

int main() {
  const int caps_extra = 40;  // reserved tokens past the item
  for (int fp8 = 0; fp8 < 2; ++fp8) {
    const int64_t strides[2] = {fp8 ? 640 : 1152, fp8 ? 768 : 1280};
    for (int64_t stride : strides) {
      for (int bt : {0, 32, 64}) {
        for (int start_tile : {0, 1, 3}) {
          for (int n = 1; n <= 5 * T; ++n) {
            const int t0 = start_tile * T;
            const int cap = t0 + n + caps_extra;
            const Layout L = make_layout(cap, stride, bt, static_cast<unsigned>(n * 7 + bt + start_tile));
            const int ntiles = (n + T - 1) / T;
            for (int tile = 0; tile < ntiles + 4; ++tile) check_tile(L, cap, t0, n, tile, fp8 != 0);
          }
        }
      }
    }
  }
  // range_of: the R Y workgroups of a launch take every (range, head block)
  // exactly once, and XCD x (workgroups L % 8 == x) takes a contiguous block
  // of the first R - R % 8 ranges, the last R % 8 spread over all XCDs
  for (int Y = 1; Y <= 4; ++Y) {
    for (int R = 0; R <= 300; ++R) {
      std::vector<int> seen(static_cast<size_t>(R) * Y, 0);
      const int nfull = R & ~7;
      for (int L = 0; L < R * Y; ++L) {
        int j = -1, y = -1;
        range_of(L, R, Y, j, y);
        ++g_checks;
        if (j < 0 || j >= R || y < 0 || y >= Y || seen[static_cast<size_t>(j) * Y + y]++ != 0) {
          std::printf("FAIL range_of: L %d of R %d Y %d gives range %d block %d\n", L, R, Y, j, y);
          return 1;
        }
        if (L < nfull * Y && (j < (L % 8) * (nfull / 8) || j >= (L % 8 + 1) * (nfull / 8))) {
          std::printf("FAIL range_of: L %d of R %d Y %d gives range %d outside its XCD's block\n", L, R, Y, j);
          return 1;
        }
      }
    }
  }
  std::printf("ok %lld\n", g_checks);
  return 0;
}
