/*
 * decode_attention.h -- C ABI of the MI355X (gfx950) split-K decode-attention
 * library.
 *
 * The operation (description of "mha_decoding_single_batch_pipelined"; Args of
 * "mha_sm100_dispatch" and "flare_mla_decoding_dispatch"): for every query row
 * (batch b, query token t, query head h)
 *
 *     out[b,t,h,:] = softmax_j( scale * <q[b,t,h,:], k_j> + mask_j ) . V
 *
 * over the keys j of sequence b that the row may see, computed as FA2 online
 * softmax per key partition ("split-K": each partition is a contiguous slice of
 * the key axis that writes a partial output with its running max and exp-sum)
 * followed by a log-sum-exp merge of the partials (the "mha_splitk_reduce" /
 * "mla_splitk_reduce" pass).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or synchronises, and never reads device memory on
 *    the host, so calls may be captured into a HIP graph.  All work is enqueued
 *    on `stream` (a hipStream_t; NULL = the default stream) in order.
 *  - Layouts are dense, row-major, with the last index fastest:
 *      q            [batch, q_len, num_q_heads, depth]
 *      k, v (dense) [batch, max_seq_len, num_kv_heads, depth]
 *      k, v (paged) [num_pages, page_size, num_kv_heads, depth]  (page pools)
 *      page_table   [batch, max_pages_per_seq] uint32: logical page i of
 *                   sequence b lives in pool page page_table[b * max_pages_per_seq + i]
 *      valid_length [batch] uint32: keys of sequence b (the current tokens
 *                   included); NULL means every sequence has max_seq_len keys
 *      out          [batch, q_len, num_q_heads, depth_v] in the input dtype
 *      lse          [batch, q_len, num_q_heads] fp32, natural log of the
 *                   softmax denominator (sink included); may be NULL
 *      sink_weights [num_q_heads] fp32 logits or NULL
 *  - Query head h reads KV head h / group (group = query heads per KV head).
 *  - Causal mask (q_len > 1): token t of T sees key j iff j <= N_b - T + t
 *    (the T query tokens are the last T positions of the sequence).
 *  - Sink: sigma_h joins the softmax denominator once per row, as a virtual
 *    key of score sigma_h (not multiplied by scale) whose value row is zero.
 *  - A row with no visible key and no sink yields out = 0 and lse = -inf.
 *  - Keys at or past a sequence's length (valid_length[b], else max_seq_len)
 *    are never read into the result, whatever they hold (NaN included).
 *    Keys and values inside it are expected to be finite: a row's score
 *    against a key it may not see is masked before the softmax, but the
 *    value rows a block loads are multiplied by weights that may be zero, so
 *    a non-finite value can reach other rows of the same sequence (other
 *    tokens under the causal mask; the paired KV head where a GQA block folds
 *    two KV heads).
 *  - Every argument check runs before anything is enqueued; on error nothing
 *    is enqueued and a negative status is returned.  Launch failures map to
 *    DA_ERR_HIP.  Calls are thread-safe.
 */
#ifndef DECODE_ATTENTION_H
#define DECODE_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define DA_OK 0
#define DA_ERR_INVALID_ARG (-1) /* null pointer, bad size, inconsistent shape   */
#define DA_ERR_UNSUPPORTED (-2) /* valid but not built: depth, dtype, page size */
#define DA_ERR_WORKSPACE (-3)   /* workspace missing or smaller than required   */
#define DA_ERR_HIP (-4)         /* a HIP runtime call or launch failed          */

/* Element types of q / k / v / out (the output dtype matches q:
 * "flare_mla_decoding_dispatch", Args `output`). */
#define DA_F32 0
#define DA_BF16 1

/* Masks applied to the scores ("mha_sm100_dispatch", Parameters `MaskType`). */
#define DA_MASK_NONE 0
#define DA_MASK_CAUSAL 1

/* Largest partition count accepted (bounded by the workspace layout). */
#define DA_MAX_PARTITIONS 1024

/* Human-readable text for a status code (static storage). */
const char* decode_attention_status_string(int status);

/*
 * Partition-count heuristic ("mha_sm100_dispatch", Args
 * `num_partitions_override`: 0 selects the automatic ladder;
 * "flare_mla_decoding_dispatch", Args `num_partitions`: None selects via
 * heuristic).  Picks P >= 1 so that the grid of (batch x KV head x row block x
 * partition) blocks fills `num_cus` compute units (one resident block per CU
 * for the bf16 kernels) while each partition keeps enough keys to amortise its
 * prologue and its partial write-back.  ragged != 0 (a valid_length array will
 * be passed) asks for more, smaller pieces instead (about 16 work items per CU
 * for GQA, taken from a work queue; about 8 blocks per CU for MLA), so that
 * the long sequences of a mixed batch are spread over many CUs.  A dense
 * split call (ragged = 0, P > 1) at depth 128 whose q_len x group is at most 8
 * and whose KV head count is even gets twice the partitions (at most one per
 * 256 keys): the bf16 and 8-bit streaming kernels then fold two KV heads into
 * each block, and the grid keeps its size.  num_cus <= 0 queries
 * the current device.  MLA calls pass num_kv_heads = 1, depth = 576,
 * depth_v = 512.  decode_attention() / mla_decode() with num_partitions = 0 use
 * this with ragged = (valid_length != NULL).  Returns P, or a negative status.
 */
int decode_num_partitions(int batch, int q_len, int num_q_heads, int num_kv_heads, int depth,
                          int depth_v, int max_seq_len, int ragged, int num_cus);

/*
 * Bytes of the split-K workspace for `num_partitions` partitions.  A
 * decode_attention() / mla_decode() call that runs with one partition does not
 * touch the workspace (it may be NULL); the *_partials() passes always write it.
 * Workspace layout (each section 256-byte aligned):
 *   queue    256 bytes                at offset 0: the uint64 work-queue word of ragged
 *                                     calls, then 62 uint32 merge counts (below)
 *   part_o   fp32 [P, rows, depth_v]  partial outputs, each normalised by its exp-sum
 *   part_max fp32 [P, rows]           partial max, natural-log units (-inf if empty)
 *   part_sum fp32 [P, rows]           partial exp-sum relative to part_max (0 if empty)
 * with rows = batch * q_len * num_q_heads.  Returns 0 for invalid arguments.
 * The *_partials() passes leave their partials in this layout.  A full split call
 * uses part_o as its own scratch: an MLA call over partitions of at least 512
 * keys stores partition 0's rows there in fp32 and the others' in bf16, which its
 * merge reads back; its contents are not part of the interface.
 *
 * Work queue.  A bf16 decode_attention() / decode_attention_partials() call
 * (or its 8-bit KV form) with valid_length, more than one partition and at most 16 query rows per KV
 * head runs a fixed set of blocks that take their (partition, sequence, KV
 * head) items from the queue word with device-scope atomics, so that blocks
 * whose items are short, or which run on faster parts of the chip, take more.
 * The word must be zero when such a call starts: fill a new workspace with zero
 * bytes once (hipMemset) before its first use; every completed call leaves it
 * zero again.  Its place does not depend on the partition count, so one
 * workspace sized for the largest P serves calls with any P.  Calls that share a
 * workspace must not run concurrently.
 *
 * Merge counts.  An fp32 decode_attention() / decode_attention_ragged() call with
 * 2..8 partitions and at most 62 row groups (batch x KV heads x blocks of up to 8
 * folded query rows) merges its partitions inside the partition pass: each row
 * group counts its finished partitions in a word of the queue section, and the
 * block that completes the count merges the group's rows, so the call is one
 * launch (the same results as the merge pass, bit for bit).  Like the queue
 * word, the counts must be zero when such a call starts (the same one-time zero
 * fill covers them) and every completed call leaves them zero.
 */
size_t decode_workspace_size(int num_partitions, int batch, int q_len, int num_q_heads,
                             int depth_v);

/* Byte offsets of part_o, part_max and part_sum inside that workspace. */
size_t decode_workspace_o_offset(int num_partitions, int batch, int q_len, int num_q_heads,
                                 int depth_v);
size_t decode_workspace_max_offset(int num_partitions, int batch, int q_len, int num_q_heads,
                                   int depth_v);
size_t decode_workspace_sum_offset(int num_partitions, int batch, int q_len, int num_q_heads,
                                   int depth_v);

/*
 * Decode attention over a dense or paged KV cache (MHA / GQA).
 *   q, k, v         see the layouts above; dtype DA_F32 or DA_BF16 for all of
 *                   q, k, v and out.
 *   page_table      NULL for a dense cache; otherwise page_size must be a power
 *                   of two >= 32 and max_pages_per_seq >= ceil(max_seq_len / page_size).
 *   valid_length    per-sequence key counts or NULL ("mha_sm100_dispatch", Args
 *                   `valid_length`); values above max_seq_len count as max_seq_len
 *                   (compared as unsigned 32-bit numbers: 0xFFFFFFFF counts as
 *                   max_seq_len, too).
 *   group           query heads per KV head; num_q_heads % group == 0.
 *   depth           64 or 128 (the value depth equals depth).
 *   max_seq_len     host upper bound of the key count ("mha_sm100_dispatch",
 *                   Args `max_cache_valid_length_arg`); also the dense cache's
 *                   sequence stride.
 *   scale           multiplies q.k before the softmax.
 *   num_partitions  0 = decode_num_partitions(..., ragged = valid_length != NULL, 0);
 *                   > 0 is used verbatim.
 *   mask            DA_MASK_NONE or DA_MASK_CAUSAL.
 *   workspace       >= decode_workspace_size(P, ...) bytes when P > 1 (may be
 *                   NULL when P == 1); its queue word zero (see
 *                   decode_workspace_size).
 */
int decode_attention(const void* q, const void* k, const void* v, const uint32_t* page_table,
                     int page_size, int max_pages_per_seq, const uint32_t* valid_length,
                     int batch, int q_len, int num_q_heads, int group, int depth,
                     int max_seq_len, float scale, int num_partitions,
                     const float* sink_weights, int mask, int dtype, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * decode_attention() for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments without workspace, and the same results.  The split-K workspace
 * is a static device array of DA_NO_ALLOC_SCRATCH_BYTES bytes inside the library,
 * one per device, held until the process ends (its address is looked up once per
 * device, on the first call there).  The call allocates nothing; q, k, v, out and
 * lse are the caller's as before (out is required).
 *   - A call whose workspace, decode_workspace_size(P, batch, q_len, num_q_heads,
 *     depth), exceeds DA_NO_ALLOC_SCRATCH_BYTES returns DA_ERR_WORKSPACE before
 *     anything is enqueued (with P resolved as for decode_attention(); a call
 *     with one partition uses no scratch and is never refused for its size).
 *   - Every call on a device shares that device's array, which keeps the last
 *     call's contents: calls that overlap on one device (other streams, other
 *     threads) race on it and must be serialised by the caller.  The work-queue
 *     word and the merge counts are cleared by a small kernel at the start of
 *     each call that uses them.
 */
#define DA_NO_ALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int decode_attention_no_alloc(const void* q, const void* k, const void* v,
                              const uint32_t* page_table, int page_size, int max_pages_per_seq,
                              const uint32_t* valid_length, int batch, int q_len,
                              int num_q_heads, int group, int depth, int max_seq_len,
                              float scale, int num_partitions, const float* sink_weights,
                              int mask, int dtype, void* out, float* lse, void* stream);

/*
 * The partition pass of decode_attention() alone: writes the split-K partials
 * of every row into `workspace` (layout above) for a later splitk_reduce()
 * (e.g. after the partials of several devices have been gathered).  Takes the
 * arguments of decode_attention() without sink / out / lse; num_partitions
 * must be >= 1 (used verbatim; 1 gives a single partial per row).
 */
int decode_attention_partials(const void* q, const void* k, const void* v,
                              const uint32_t* page_table, int page_size, int max_pages_per_seq,
                              const uint32_t* valid_length, int batch, int q_len,
                              int num_q_heads, int group, int depth, int max_seq_len,
                              float scale, int num_partitions, int mask, int dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention with a ragged q ("flare_mla_decoding_dispatch", Parameters
 * `ragged` and Args `valid_length`: a rank-3 q whose rows are located by
 * cumulative per-sequence offsets): q is [total_q_tokens, num_q_heads, depth]
 * and the q_len_b tokens of sequence b are its rows q_offsets[b] ..
 * q_offsets[b+1] (device uint32 [batch + 1], non-decreasing, q_offsets[batch] =
 * total_q_tokens, every q_len_b <= max_q_len; tokens past max_q_len are not
 * computed).  out is [total_q_tokens, num_q_heads, depth] and lse
 * [total_q_tokens, num_q_heads].  valid_length keeps its meaning (keys of
 * sequence b, its current tokens included); with DA_MASK_CAUSAL token t of
 * sequence b sees keys j <= N_b - q_len_b + t.  The split-K workspace is sized
 * for rows = total_q_tokens * num_q_heads: decode_workspace_size(P, 1,
 * total_q_tokens, num_q_heads, depth_v).  Other arguments as for
 * decode_attention(); num_partitions = 0 uses decode_num_partitions() with
 * q_len = max_q_len.
 */
int decode_attention_ragged(const void* q, const uint32_t* q_offsets, int total_q_tokens,
                            int max_q_len, const void* k, const void* v,
                            const uint32_t* page_table, int page_size, int max_pages_per_seq,
                            const uint32_t* valid_length, int batch, int num_q_heads, int group,
                            int depth, int max_seq_len, float scale, int num_partitions,
                            const float* sink_weights, int mask, int dtype, void* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* MLA decode with a ragged q (layouts as for decode_attention_ragged(), depth 576
 * in, 512 out; other arguments as for mla_decode()). */
int mla_decode_ragged(const void* q, const uint32_t* q_offsets, int total_q_tokens,
                      int max_q_len, const void* kv, const uint32_t* page_table, int page_size,
                      int max_pages_per_seq, const uint32_t* valid_length, int batch,
                      int num_q_heads, int max_seq_len, float scale, int num_partitions,
                      const float* sink_weights, int mask, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention over a ragged KV layout ("mha_sm100_dispatch", Args
 * `kv_input_row_offsets`: per-batch row offsets into a ragged KV layout).  The
 * caches of all sequences are concatenated into one cache
 *     k, v  [kv_rows, num_kv_heads, depth]
 * and key j of sequence b is its row kv_row_offsets[b] + j.
 *   kv_row_offsets  device uint32 [batch] (required when batch > 0).  The
 *                   caller keeps kv_row_offsets[b] + N_b <= kv_rows for every
 *                   sequence, N_b being its key count below; the kernels do
 *                   not check it.  Sequences may share rows.
 *   valid_length    key counts N_b (values above max_seq_len count as
 *                   max_seq_len), or NULL: every sequence has max_seq_len keys.
 *   max_seq_len     bound of every N_b (no stride: there is no dense layout).
 * q, out, lse, the mask, the sinks, the partitions and the workspace are as for
 * decode_attention(); there is no page table.
 */
int decode_attention_ragged_kv(const void* q, const void* k, const void* v,
                               const uint32_t* kv_row_offsets, const uint32_t* valid_length,
                               int batch, int q_len, int num_q_heads, int group, int depth,
                               int max_seq_len, float scale, int num_partitions,
                               const float* sink_weights, int mask, int dtype, void* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               void* stream);

/* MLA over a ragged KV layout ("flare_mla_decoding_dispatch", Args
 * `kv_input_row_offsets`): kv is one cache [kv_rows, 1, 576] and key j of
 * sequence b is its row kv_row_offsets[b] + j (V = the first 512 columns of the
 * same rows).  kv_row_offsets, valid_length and max_seq_len as for
 * decode_attention_ragged_kv(); every other argument as for mla_decode(). */
int mla_decode_ragged_kv(const void* q, const void* kv, const uint32_t* kv_row_offsets,
                         const uint32_t* valid_length, int batch, int q_len, int num_q_heads,
                         int max_seq_len, float scale, int num_partitions,
                         const float* sink_weights, int mask, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention with an 8-bit KV cache: q bf16, k and v one byte per element
 * in the e4m3 format (the OCP FP8 E4M3 encoding: bias 7, subnormals, no
 * infinity, S.1111.111 is NaN), out bf16.  The pages admit float8_e4m3fn
 * elements with a bf16 output and fold a scale into the softmax
 * ("flare_mla_decoding_dispatch", Parameters `dtype`, Args `output` and
 * `q_scale_ptr`) but give no scale convention for the cache; the reading taken
 * here is one fp32 scale per tensor: the real key is k_scale * (stored key),
 * the real value v_scale * (stored value).
 * Arguments, layouts (with 1-byte elements), workspace and status codes are
 * those of decode_attention(); depth must be 128 (else DA_ERR_UNSUPPORTED), and
 * k_scale, v_scale and scale * k_scale must be finite.
 */
int decode_attention_fp8kv(const void* q, const void* k, const void* v, float k_scale,
                           float v_scale, const uint32_t* page_table, int page_size,
                           int max_pages_per_seq, const uint32_t* valid_length, int batch,
                           int q_len, int num_q_heads, int group, int depth, int max_seq_len,
                           float scale, int num_partitions, const float* sink_weights, int mask,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/* The partition pass of decode_attention_fp8kv() alone (partials as for
 * decode_attention_partials(); the partial outputs include v_scale). */
int decode_attention_fp8kv_partials(const void* q, const void* k, const void* v, float k_scale,
                                    float v_scale, const uint32_t* page_table, int page_size,
                                    int max_pages_per_seq, const uint32_t* valid_length,
                                    int batch, int q_len, int num_q_heads, int group, int depth,
                                    int max_seq_len, float scale, int num_partitions, int mask,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * MLA decode ("flare_mla_decoding_dispatch", Args `k` and `kv_num_heads`): a
 * single KV head, depth 576, and no separate V operand: V is the first 512
 * columns of each K row, taken from the same cache rows.
 *   q    bf16 [batch, q_len, num_q_heads, 576]; the q_len tokens of a sequence
 *        are folded into one block of rows (the MTP token fold).
 *   kv   bf16 dense [batch, max_seq_len, 1, 576] or pool [num_pages, page_size, 1, 576]
 *   out  bf16 [batch, q_len, num_q_heads, 512]; lse fp32 [batch, q_len, num_q_heads] or NULL
 * Other arguments as for decode_attention().
 */
int mla_decode(const void* q, const void* kv, const uint32_t* page_table, int page_size,
               int max_pages_per_seq, const uint32_t* valid_length, int batch, int q_len,
               int num_q_heads, int max_seq_len, float scale, int num_partitions,
               const float* sink_weights, int mask, void* out, float* lse, void* workspace,
               size_t workspace_bytes, void* stream);

/* The partition pass of mla_decode() alone (see decode_attention_partials()). */
int mla_decode_partials(const void* q, const void* kv, const uint32_t* page_table,
                        int page_size, int max_pages_per_seq, const uint32_t* valid_length,
                        int batch, int q_len, int num_q_heads, int max_seq_len, float scale,
                        int num_partitions, int mask, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * MLA over an 8-bit cache ("flare_mla_decoding_dispatch", Parameters `dtype`: q
 * of a half type or float8_e4m3fn; Args `output`: a bfloat16 output when the
 * inputs are 8-bit).  Reading of the pages: bf16 q over an e4m3 cache (OCP FP8
 * E4M3, the elements of float8_e4m3fn) with one fp32 scale for the tensor: the
 * real cache element is k_scale x stored, for the keys and for their value
 * slice alike (V is the first 512 columns of the same stored rows).
 *   kv  uint8 e4m3 bit patterns, dense [batch, max_seq_len, 1, 576] or pool
 *       [num_pages, page_size, 1, 576]
 *   q, out, lse and every other argument as for mla_decode().
 * k_scale and scale * k_scale must be finite (else DA_ERR_INVALID_ARG).
 */
int mla_decode_fp8kv(const void* q, const void* kv, float k_scale, const uint32_t* page_table,
                     int page_size, int max_pages_per_seq, const uint32_t* valid_length,
                     int batch, int q_len, int num_q_heads, int max_seq_len, float scale,
                     int num_partitions, const float* sink_weights, int mask, void* out,
                     float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* The partition pass of mla_decode_fp8kv() alone (see decode_attention_partials()). */
int mla_decode_fp8kv_partials(const void* q, const void* kv, float k_scale,
                              const uint32_t* page_table, int page_size, int max_pages_per_seq,
                              const uint32_t* valid_length, int batch, int q_len,
                              int num_q_heads, int max_seq_len, float scale, int num_partitions,
                              int mask, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse top-k MLA ("flare_mla_decoding_dispatch", Parameters `sparse`; Args
 * `d_indices`, `indices_stride`, `topk_lengths`): the keys of sequence b are
 * not a prefix of its cache but a list of rows of a shared pool, a gather at
 * page size 1.  Every query token and head of sequence b attends to the rows
 *     indices[b * indices_stride + i],   0 <= i < topk_lengths[b]
 * of the pool, with no mask (the list is the selection; a row index carries no
 * position).  Reading of the pages: one list per sequence, shared by its
 * q_len tokens; the counts play the part of valid_length and indices_stride
 * (the allocation stride, the largest top-k) that of max_seq_len.
 *   q             bf16 [batch, q_len, num_q_heads, 576] (the MTP token fold as
 *                 for mla_decode())
 *   kv            bf16 pool [pool_rows, 1, 576]; V = the first 512 columns
 *   pool_rows     1 .. 3728270 (the pool is at most 4 GiB: rows are addressed
 *                 by 32-bit byte offsets); larger pools are DA_ERR_UNSUPPORTED
 *   indices       int32 [batch, indices_stride], indices_stride 0 .. 2^28
 *                 (larger is DA_ERR_UNSUPPORTED); entries at or past a
 *                 sequence's count are never read (NULL allowed when
 *                 indices_stride is 0)
 *   topk_lengths  int32 [batch]; a count below 0 is 0, above indices_stride is
 *                 indices_stride
 *   out           bf16 [batch, q_len, num_q_heads, 512]; lse fp32 [batch, q_len,
 *                 num_q_heads] or NULL; sink_weights as for decode_attention()
 * The caller keeps every counted index inside [0, pool_rows).  The kernel
 * clamps each one into that range before the load, so that a call with a bad
 * index still reads only the pool (the value of such a row is then that of
 * row min(index as unsigned, pool_rows - 1)).  Partition p covers list
 * positions [p*C, (p+1)*C).  num_partitions = 0 selects
 * mla_sparse_num_partitions(); the workspace is sized as for mla_decode() with
 * the same batch, q_len and num_q_heads.
 */
int mla_decode_sparse(const void* q, const void* kv, long long pool_rows, const int32_t* indices,
                      int indices_stride, const int32_t* topk_lengths, int batch, int q_len,
                      int num_q_heads, float scale, int num_partitions,
                      const float* sink_weights, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);

/* The partition pass of mla_decode_sparse() alone (see decode_attention_partials()). */
int mla_decode_sparse_partials(const void* q, const void* kv, long long pool_rows,
                               const int32_t* indices, int indices_stride,
                               const int32_t* topk_lengths, int batch, int q_len,
                               int num_q_heads, float scale, int num_partitions, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Partition count of mla_decode_sparse() with num_partitions = 0: enough
 * (batch x row block x partition) blocks for one per compute unit, each
 * partition keeping at least 512 list positions.  num_cus <= 0 queries the
 * current device.  Returns P >= 1, or a negative status.
 */
int mla_sparse_num_partitions(int batch, int q_len, int num_q_heads, int topk, int num_cus);

/*
 * Log-sum-exp merge of split-K partials ("mha_splitk_reduce"; "mla_splitk_reduce").
 *   part_o    fp32 [num_partitions, rows, depth_v]  normalised partial outputs
 *   part_max  fp32 [num_partitions, rows]           natural-log partial max
 *   part_sum  fp32 [num_partitions, rows]           partial exp-sum (0 = empty)
 *   sink_weights  [num_q_heads] or NULL; row r uses head r % num_q_heads
 *   out       [rows, depth_v] in out_dtype (DA_F32 or DA_BF16, rounded to nearest even)
 *   lse       [rows] fp32 or NULL
 * Per row: M = max(max_p part_max, sigma); w_p = part_sum_p * exp(part_max_p - M);
 * L = sum_p w_p + exp(sigma - M); out = sum_p w_p * part_o_p / L; lse = M + ln L.
 * depth_v must be one of 64, 128, 256, 512, 1024; 1 <= num_partitions <= DA_MAX_PARTITIONS.
 */
int splitk_reduce(const float* part_o, const float* part_max, const float* part_sum,
                  int num_partitions, int rows, int num_q_heads, int depth_v,
                  const float* sink_weights, void* out, int out_dtype, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTENTION_H */
