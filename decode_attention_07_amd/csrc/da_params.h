// da_params.h -- launch parameters shared by the host layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

// Everything a partition-pass kernel needs.  Passed by value (kernarg segment).
struct DecodeParams {
  const void* q;                // [B, T, H, D]
  const void* k;                // dense [B, S, KVH, D] or pool [pages, ps, KVH, D]
  const void* v;                // same layout with Dv; unused by MLA (V = K[..., :Dv])
  const uint32_t* page_table;   // [B, max_pages] or nullptr
  const uint32_t* valid_length; // [B] or nullptr
  const float* sink;            // [H] or nullptr (used only when P == 1)
  void* out;                    // [B, T, H, Dv] (P == 1)
  float* lse;                   // [B, T, H] or nullptr (P == 1)
  float* part_o;                // [P, rows, Dv] (P > 1)
  float* part_m;                // [P, rows]
  float* part_l;                // [P, rows]
  int batch, q_len, num_q_heads, num_kv_heads, group, depth, depth_v, max_seq_len;
  int page_shift;               // log2(page_size) when paged
  int max_pages;
  int causal;
  int num_partitions;
  int keys_per_partition;       // C: partition p covers keys [p*C, (p+1)*C)
  int row_blocks;               // row tiles per (batch, KV head)
  // bf16 GQA stream kernel: a block folds 2^hb_shift KV heads (their query rows,
  // 16 >> hb_shift per head, share the block's 16 rows) and reads them as one
  // contiguous piece of each key row; 0 elsewhere.
  int hb_shift;
  int write_partials;           // 1: write part_*; 0: write out / lse directly
  // 1: mixed partial rows: partition 0's fp32 at part_o[row * Dv] (as with
  // fp32 partials), partition p >= 1's bf16 at ((uint16_t*)part_o)[((p + 1) *
  // rows + row) * Dv] (after partition 0's fp32 rows; the section is sized for
  // P fp32 rows per row).  Set only for the internal split of the MLA kernels with
  // long partitions, whose merge pass reads them back; partials handed to the
  // caller stay fp32.  Partition 0 stays fp32 because a short sequence's keys all
  // fall there: its partial row is then the whole result, of a few keys, and a
  // bf16 rounding of it would add to the output's own rounding.
  int part_bf16;
  float scale_log2;             // scale * log2(e) (times k_scale for an 8-bit KV cache)
  float v_scale;                // 8-bit KV cache: real value = v_scale * stored value
  // Work queue of the bf16 GQA kernel (ragged split calls; nullptr otherwise):
  // one 64-bit word in the workspace, low half = next work item, high half =
  // blocks done; zero between calls.
  unsigned long long* queue;
  int queue_blocks;             // persistent blocks launched when queue is set
  // Ragged q: the q_len_b tokens of sequence b are q / out rows q_offsets[b] ..
  // q_offsets[b+1] (q_len is then an upper bound of q_len_b); nullptr: q_len
  // tokens per sequence.
  const uint32_t* q_offsets;
  int rows_total;               // q / out rows (tokens x heads): one partition's partial rows
  // Sparse top-k (MLA): key i of sequence b is row indices[b * max_seq_len + i] of
  // the pool k [pool_rows, 1, D], for i < valid_length[b] (the top-k counts);
  // nullptr: keys from the contiguous or paged cache.
  const int32_t* indices;
  uint32_t pool_rows;
  // Ragged KV layout: key j of sequence b is row kv_row_offsets[b] + j of one
  // cache [rows, KVH, D] holding every sequence (instead of row b * max_seq_len
  // + j of the dense layout); nullptr otherwise.  Never set with a page table.
  const uint32_t* kv_row_offsets;
};

// Row-block geometry of a (batch, KV head): T*group rows (token-major:
// row = t*group + i is query head kv*group + i of token t).
__host__ __device__ inline int fold_rows(const DecodeParams& p) { return p.q_len * p.group; }

// Query tokens of sequence b (at most q_len) and the q / out row of its first
// token.  The offsets are read through the scalar cache: b is uniform and the
// table is constant during the call.
__device__ inline int seq_tokens(const DecodeParams& p, int b) {
  if (!p.q_offsets) return p.q_len;
  const __attribute__((address_space(4))) uint32_t* qo =
      (const __attribute__((address_space(4))) uint32_t*)p.q_offsets;
  const int n = (int)(qo[b + 1] - qo[b]);
  return n < p.q_len ? n : p.q_len;
}
__device__ inline size_t seq_row0(const DecodeParams& p, int b) {
  if (!p.q_offsets) return (size_t)b * p.q_len;
  const __attribute__((address_space(4))) uint32_t* qo =
      (const __attribute__((address_space(4))) uint32_t*)p.q_offsets;
  return (size_t)qo[b];
}

}  // namespace da
