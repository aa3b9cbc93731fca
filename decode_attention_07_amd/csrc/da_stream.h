// da_stream.h -- pieces shared by the streaming decode kernels (bf16 and
// 8-bit KV): global->LDS loads, vmcnt waits and the page-table lookup.
#pragma once

#include "da_device.h"

namespace da {

// 16 bytes per lane from base + voff straight into LDS at lds + 16 * lane
// (global_load_lds_dwordx4, scalar base + 32-bit vector offset).  The cache is
// streamed through once, so the loads carry the non-temporal hint (nt): on
// this chip that alone moves the stream from about 5.5 to about 6.2 TB/s.
// Written as inline asm so that the compiler does not wait for it before
// unrelated LDS reads; completion is tracked with explicit vmcnt waits.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// vmcnt(PER * min(after, MAXA) + EXTRA) for a wave-uniform `after`.
template <int PER, int EXTRA, int MAXA>
__device__ __forceinline__ void wait_after(int after) {
  if constexpr (MAXA == 0) {
    wait_vm<EXTRA>();
  } else {
    if (after >= MAXA)
      wait_vm<PER * MAXA + EXTRA>();
    else
      wait_after<PER, EXTRA, MAXA - 1>(after);
  }
}

// First cache row of the tile starting at key j0 (a tile never straddles a page).  The
// page table is read through the scalar cache: the index is uniform and the
// table is constant during the call.
__device__ __forceinline__ size_t stream_row0(const DecodeParams& p, int b, int j0) {
  if (p.page_table) {
    const __attribute__((address_space(4))) uint32_t* pt =
        (const __attribute__((address_space(4))) uint32_t*)p.page_table;
    const uint32_t phys = pt[(size_t)b * p.max_pages + (j0 >> p.page_shift)];
    return ((size_t)phys << p.page_shift) + (size_t)(j0 & ((1 << p.page_shift) - 1));
  }
  return seq_kv_row0(p, b) + j0;
}

// Block-uniform key range of a work item: [k_lo, hmin) is visible to every row of
// its fold, [k_lo, hmax) to some.  The item's rows are rb * 16 + 0 .. 2^rps - 1 of
// the token-major fold (each head slot repeats them), valid below nrows.  A row's
// visible keys grow with its token, so the first row sets hmin and the last valid
// one hmax: two scalar reads, where a reduction across the rows' lanes took eight
// dependent lane swaps.  With no valid row both are k_lo (and nothing is streamed).
__device__ __forceinline__ void item_key_range(const DecodeParams& p, int b, int rb, int rps,
                                               int nrows, int k_lo, int& hmin, int& hmax) {
  const int first = rb * 16;
  const int last = min(nrows, first + (1 << rps)) - 1;
  int lo = k_lo, hi = k_lo;
  if (first <= last) {
    const int k_hi = k_lo + p.keys_per_partition;
    lo = max(k_lo, min(k_hi, visible_keys(p, b, first / p.group)));
    hi = max(k_lo, min(k_hi, visible_keys(p, b, last / p.group)));
  }
  hmin = __builtin_amdgcn_readfirstlane(lo);
  hmax = __builtin_amdgcn_readfirstlane(hi);
}

// A split item whose partition holds no visible key of any of its rows (a
// partition past the end of a short sequence): its partial rows are the empty
// ones, O = 0, m = -inf, l = 0, exactly what the whole item would store, without
// its Q loads and its merge of the waves through LDS.  Rows numbered as in the
// items' epilogues.  Called by all threads of the block.
template <int D>
__device__ __forceinline__ void stream_store_empty(const DecodeParams& p, int b, int g,
                                                   int pidx, int rb) {
  const int rps = 4 - p.hb_shift;  // log2 of the rows per head slot
  const int nrows = seq_tokens(p, b) * p.group;
  const size_t row0q = seq_row0(p, b);
  for (int idx = threadIdx.x; idx < 16 * D; idx += blockDim.x) {
    const int r = idx / D;
    const int d = idx % D;
    const int rrow = rb * 16 + (r & ((1 << rps) - 1));
    if (rrow >= nrows) continue;
    const int h = (g + (r >> rps)) * p.group + rrow % p.group;
    const size_t row = (row0q + rrow / p.group) * p.num_q_heads + h;
    const size_t prow = (size_t)pidx * (size_t)p.rows_total + row;
    p.part_o[prow * D + d] = 0.f;
    if (d == 0) {
      p.part_m[prow] = kNegInf;
      p.part_l[prow] = 0.f;
    }
  }
}

}  // namespace da
