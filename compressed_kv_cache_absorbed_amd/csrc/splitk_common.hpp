// Helpers shared by the split-K kernels (bf16 / fp16-widened and fp8
// matrix-core forms): bf16 -> fp16 conversion, wait counters, direct-to-LDS
// copies.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

// LDS byte offset of a __shared__ array (a link-time constant when applied
// to the array itself).
#define LDS_OFF(arr) static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char *)(arr)))

namespace mla {
namespace {

// 2 bf16 (one dword) -> 2 fp16, exact for |x| < 65504 (a bf16 significand
// fits in fp16's); round-toward-zero saturates larger magnitudes to +-65504.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
  return __builtin_bit_cast(uint32_t, h);
}

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

// A split-K launch's arguments, passed as the kernel's only argument.
struct SplitArgs {
  mla_cache c;
  int H, Hr, q_len, n_items, n_ranges;
  const int32_t *ranges;
  const WorkItem *items;
  const SeqInfo *seqs;
  const uint16_t *Q;
  uint16_t *opart;
  float *lse;
  int32_t *status;
};
static_assert(sizeof(SplitArgs) % 4 == 0, "SplitArgs is read as 32-bit words");

typedef const __attribute__((address_space(4))) SplitArgs *KernArgs;

// The arguments, read again from the kernel-argument segment (scalar loads
// through an address the compiler cannot follow, each where it is used): a
// workgroup that walks several items reads them afresh for each, so none of
// them stays live in registers across the item loop.
__device__ __forceinline__ KernArgs kernel_args() {
  KernArgs p = (KernArgs)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return p;
}
// (field by field: a struct in that address space does not bind to a
// reference)
__device__ __forceinline__ mla_cache cache_of(KernArgs a) {
  mla_cache c;
  c.latent_dtype = a->c.latent_dtype;
  c.rope_dtype = a->c.rope_dtype;
  c.rows = a->c.rows;
  c.row_stride = a->c.row_stride;
  c.scale = a->c.scale;
  c.n_rows = a->c.n_rows;
  c.batch = a->c.batch;
  c.seq_start = a->c.seq_start;
  c.seq_cap = a->c.seq_cap;
  c.seq_len = a->c.seq_len;
  c.block_table = a->c.block_table;
  c.block_tokens = a->c.block_tokens;
  c.max_blocks = a->c.max_blocks;
  return c;
}

// An item's sequence checked and its data read, every load issued at once:
// the sequence index is checked first (nothing is indexed by an index
// outside the batch), then the device length, the plan's length, the
// reserved tokens and the start row are read together and the checks are
// combined without short-circuit evaluation, which would chain the loads one
// memory round trip after another (eight of them stood before an item's
// first copy). ok: the item's tokens lie in its sequence's range, the
// device length equals the plan's, and the item is non-empty.
struct ItemSeq {
  bool ok;
  int len;       // the plan's length of the sequence
  int64_t row0;  // the sequence's first row (contiguous cache), else 0
};
__device__ __forceinline__ ItemSeq item_seq(const mla_cache &c, const SeqInfo *seqs, const WorkItem &wi) {
  const bool b_ok = (wi.b >= 0) & (wi.b < c.batch);
  const int b = b_ok ? wi.b : 0;
  const bool paged = c.block_table != nullptr;
  const int dev_len = c.seq_len[b];
  const int plan_len = seqs[b].len;
  const int64_t cap = c.seq_cap[b];
  // (a pointer chosen without a branch, so this load issues with the others:
  // a paged cache may have no seq_start, and reads seq_len there instead)
  const int32_t *sp = paged ? c.seq_len : c.seq_start;
  const int64_t start = paged ? 0 : static_cast<int64_t>(sp[b]);
  const int64_t t1 = wi.t1;
  const bool in_rows = paged ? t1 <= static_cast<int64_t>(c.max_blocks) * c.block_tokens
                             : (start >= 0) & (start + t1 <= c.n_rows);
  ItemSeq r;
  r.ok = b_ok & (dev_len == plan_len) & (wi.t0 >= 0) & (wi.t0 < wi.t1) & (t1 <= cap) & in_rows;
  r.len = plan_len;
  r.row0 = start;
  return r;
}

// (range_of, the workgroup -> (range, head block) map, sits with the copy
// addresses in splitk_addr.hpp, where a CPU test checks it)
using sa::range_of;

}  // namespace
}  // namespace mla
