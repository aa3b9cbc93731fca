// api.cpp -- the C ABI (include/decode_attention.h): argument checks, the
// partition-count heuristic, workspace layout and kernel dispatch.
//
// Host dispatch follows the role of "mha_sm100_dispatch" / "flare_mla_decoding_dispatch"
// (descriptions): choose the kernel configuration and the split count, thread
// the optional valid-length / page-table / sink arguments through, enqueue on
// the caller's stream.  Nothing here reads device memory or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>

// The library is built with hidden visibility: the declarations of the C ABI are
// the only exported symbols.
#pragma GCC visibility push(default)
#include "../../include/decode_attention.h"
#pragma GCC visibility pop
#include "da_params.h"

namespace da {
hipError_t launch_decode_valu(const DecodeParams& p, unsigned* merge_count, hipStream_t s);
int valu_step_keys(int rows_per_block);
int valu_rows_per_block(int fold);
hipError_t launch_decode_stream(const DecodeParams& p, hipStream_t s);
int stream_step_keys();
int stream_rows_per_block();
hipError_t launch_decode_stream_fp8(const DecodeParams& p, hipStream_t s);
int stream_fp8_step_keys();
hipError_t launch_mla_sparse(const DecodeParams& p, hipStream_t s);
hipError_t launch_mla_wave8(const DecodeParams& p, hipStream_t s);
hipError_t launch_mla_wave8_fp8(const DecodeParams& p, hipStream_t s);
int mla_step_keys(int q_len);
int mla_rows_per_block(int q_len, int num_q_heads);
bool splitk_reduce_supported(int depth_v, int P);
hipError_t launch_splitk_reduce_bf16_partials(const uint16_t* po, const float* pm,
                                              const float* pl, int P, int rows, int H,
                                              const float* sink, void* out, float* lse,
                                              int batch, int seq_rows, hipStream_t s);
hipError_t launch_splitk_reduce(const float* po, const float* pm, const float* pl, int P,
                                int rows, int H, int depth_v, const float* sink, void* out,
                                bool bf16, float* lse, hipStream_t s);
}  // namespace da

namespace {

constexpr int kMlaDepth = 576;
constexpr int kMlaDepthV = 512;
// Shortest partition (keys, or list positions of a sparse call) whose MLA partial
// rows go to the merge in bf16.
constexpr int kMlaBf16PartialKeys = 512;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("DECODE_ATTN_LOG");
    return e && e[0] && e[0] != '0';
  }();
  return on;
}

// Compute-unit count of the current device, cached per device.
int device_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    hipDeviceProp_t prop;
    cache[dev] = (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
                     ? prop.multiProcessorCount
                     : 256;
  }
  return cache[dev];
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

// Which partition kernel runs, and its tiling.
enum Variant { kValu = 0, kStream = 1, kMla = 2, kStreamFp8 = 3, kMlaFp8 = 4 };

struct Plan {
  Variant variant;
  int rows_per_block;
  int row_blocks;
  int step;  // keys per block iteration; partitions are multiples of it
};

Plan plan_mha(int q_len, int group, bool bf16) {
  const int fold = q_len * group;
  Plan pl;
  if (bf16) {  // streaming matrix-core kernel; fp32 runs on the vector ALUs
    pl.variant = kStream;
    pl.rows_per_block = da::stream_rows_per_block();
    pl.step = da::stream_step_keys();
  } else {
    pl.variant = kValu;
    pl.rows_per_block = da::valu_rows_per_block(fold < 8 ? fold : 8);
    pl.step = da::valu_step_keys(pl.rows_per_block);
  }
  pl.row_blocks = (fold + pl.rows_per_block - 1) / pl.rows_per_block;
  return pl;
}

// bf16 q with an 8-bit e4m3 KV cache: the streaming kernel's 8-bit form.
Plan plan_fp8(int q_len, int group) {
  Plan pl;
  pl.variant = kStreamFp8;
  pl.rows_per_block = da::stream_rows_per_block();
  pl.step = da::stream_fp8_step_keys();
  pl.row_blocks = (q_len * group + pl.rows_per_block - 1) / pl.rows_per_block;
  return pl;
}

Plan plan_mla(int q_len, int num_q_heads) {
  Plan pl;
  pl.variant = kMla;
  pl.rows_per_block = da::mla_rows_per_block(q_len, num_q_heads);
  pl.row_blocks = (q_len * num_q_heads + pl.rows_per_block - 1) / pl.rows_per_block;
  pl.step = da::mla_step_keys(q_len);
  return pl;
}

constexpr int kMhaMinKeys = 256;  // keys per partition at least (MHA / GQA heuristic)

int heuristic_partitions(int base_blocks, int max_seq_len, int num_cus, int blocks_per_cu,
                         int min_keys) {
  if (base_blocks < 1) base_blocks = 1;
  const long target = (long)num_cus * blocks_per_cu;
  long P = (target + base_blocks - 1) / base_blocks;
  const long by_len = (max_seq_len + min_keys - 1) / min_keys;
  if (P > by_len) P = by_len;
  if (P < 1) P = 1;
  if (P > DA_MAX_PARTITIONS) P = DA_MAX_PARTITIONS;
  return (int)P;
}

// Two KV heads fit one 16-row block of the streaming GQA kernels.
bool fold_allows_two_heads(int q_len, int group, int num_kv_heads) {
  return 2 * q_len * group <= 16 && num_kv_heads % 2 == 0;
}

int keys_per_partition(int max_seq_len, int P, int step) {
  long c = ((long)max_seq_len + P - 1) / P;
  c = (c + step - 1) / step * step;
  if (c < step) c = step;
  return (int)c;
}

struct Common {
  const uint32_t* page_table;
  int page_size, max_pages;
  const uint32_t* valid_length;
  int batch, q_len, num_q_heads, max_seq_len, mask;
  float scale;
  // Ragged q: cumulative token offsets [batch + 1] (q_len bounds every
  // sequence's tokens) and the total token count; nullptr / 0 otherwise.
  const uint32_t* q_offsets = nullptr;
  int total_q_tokens = 0;
  // Ragged KV layout: per-sequence row offsets into one cache; nullptr otherwise.
  const uint32_t* kv_row_offsets = nullptr;
};

// q / out rows of a call (tokens x heads).
size_t call_rows(const Common& c) {
  const size_t tokens = c.q_offsets ? (size_t)c.total_q_tokens : (size_t)c.batch * c.q_len;
  return tokens * c.num_q_heads;
}

int check_common(const Common& c) {
  if (c.batch < 0 || c.q_len < 1 || c.num_q_heads < 1 || c.max_seq_len < 0)
    return DA_ERR_INVALID_ARG;
  if (c.total_q_tokens < 0) return DA_ERR_INVALID_ARG;
  if (c.mask != DA_MASK_NONE && c.mask != DA_MASK_CAUSAL) return DA_ERR_INVALID_ARG;
  if (!std::isfinite(c.scale)) return DA_ERR_INVALID_ARG;
  if (c.kv_row_offsets && c.page_table) return DA_ERR_INVALID_ARG;
  if (c.page_table) {
    if (c.page_size < 1 || c.max_pages < 1) return DA_ERR_INVALID_ARG;
    if (!is_pow2(c.page_size) || c.page_size < 32) return DA_ERR_UNSUPPORTED;
    if ((long)c.max_pages * c.page_size < (long)c.max_seq_len) return DA_ERR_INVALID_ARG;
  }
  return DA_OK;
}

da::DecodeParams base_params(const Common& c, const void* q, const void* k, const void* v,
                             int kv_heads, int group, int depth, int depth_v) {
  da::DecodeParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.page_table = c.page_table;
  p.valid_length = c.valid_length;
  p.batch = c.batch;
  p.q_len = c.q_len;
  p.num_q_heads = c.num_q_heads;
  p.num_kv_heads = kv_heads;
  p.group = group;
  p.depth = depth;
  p.depth_v = depth_v;
  p.max_seq_len = c.max_seq_len;
  p.page_shift = c.page_table ? log2i(c.page_size) : 0;
  p.max_pages = c.page_table ? c.max_pages : 0;
  p.causal = c.mask == DA_MASK_CAUSAL;
  p.scale_log2 = c.scale * 1.4426950408889634f;
  p.v_scale = 1.f;
  p.q_offsets = c.q_offsets;
  p.rows_total = (int)call_rows(c);
  p.kv_row_offsets = c.kv_row_offsets;
  return p;
}

// Workspace sections: the work-queue word (its own 256 bytes, at offset 0 so
// that its place does not depend on P), part_o, part_max, part_sum.  The words of
// the queue section after the 64-bit queue word are the merge counts of small fp32
// split calls (kValuMergeGroups of them).
constexpr size_t kQueueBytes = 256;
constexpr long kValuMergeGroups = (long)(kQueueBytes - 8) / 4;

void ws_sections(void* ws, int P, size_t rows, int depth_v, float** po, float** pm, float** pl,
                 unsigned long long** queue) {
  char* base = (char*)ws;
  const size_t o_bytes = align_up((size_t)P * rows * depth_v * sizeof(float));
  const size_t m_bytes = align_up((size_t)P * rows * sizeof(float));
  *queue = (unsigned long long*)base;
  *po = (float*)(base + kQueueBytes);
  *pm = (float*)(base + kQueueBytes + o_bytes);
  *pl = (float*)(base + kQueueBytes + o_bytes + m_bytes);
}

// ---- scratch of decode_attention_no_alloc() ------------------------------------
// The split-K workspace of callers that cannot allocate (graph capture, serving
// loops): one file-scope device array, a copy per device, held until the process
// ends.  Host code never uses the array's name as an address: the device address
// comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static_assert(kNoAllocScratchBytes == DA_NO_ALLOC_SCRATCH_BYTES, "header and library agree");
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The current device's address of `scratch`, or nullptr if it cannot be had.
void* scratch_address() {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    addr[dev] = ptr;
  }
  return addr[dev];
}

// Zeroes the 256-byte work-queue section at the start of a workspace (a kernel, not
// a memset: the call may be captured into a graph).  Each lane stores its own word.
__global__ void clear_queue_section(unsigned long long* q) { q[threadIdx.x] = 0ull; }

// The MLA problem over the contiguous, paged or ragged-KV cache (bf16 or 8-bit)
// runs on the two-waves-per-SIMD matrix-core kernel; the sparse form on the
// one-wave kernel.
bool uses_mla_wave8(const da::DecodeParams& p, Variant v) {
  return (v == kMla || v == kMlaFp8) && !p.indices;
}

hipError_t launch_partition_pass(const da::DecodeParams& p, Variant v, bool bf16,
                                 unsigned* merge_count, hipStream_t s) {
  switch (v) {
    case kValu: return da::launch_decode_valu(p, merge_count, s);
    case kStream: return da::launch_decode_stream(p, s);
    case kStreamFp8: return da::launch_decode_stream_fp8(p, s);
    case kMlaFp8: return da::launch_mla_wave8_fp8(p, s);
    default:
      if (uses_mla_wave8(p, v)) return da::launch_mla_wave8(p, s);
      return da::launch_mla_sparse(p, s);
  }
}

const char* variant_name(Variant v) {
  switch (v) {
    case kValu: return "valu";
    case kStream: return "stream";
    case kStreamFp8: return "stream_fp8";
    case kMlaFp8: return "mla_fp8";
    default: return "mla";
  }
}

// Shared driver of decode_attention / mla_decode (and their partial passes).
int run(const Common& c, da::DecodeParams p, const Plan& plan, bool bf16, int num_partitions,
        bool partials_only, const float* sink, void* out, float* lse, void* workspace,
        size_t workspace_bytes, void* stream, bool clear_queue = false) {
  const size_t rows = call_rows(c);
  if (rows == 0) return DA_OK;  // empty batch: nothing to enqueue
  if (rows > (size_t)INT32_MAX) return DA_ERR_INVALID_ARG;
  int P = num_partitions;
  if (P == 0) {
    P = decode_num_partitions(c.batch, c.q_len, c.num_q_heads, p.num_kv_heads, p.depth,
                              p.depth_v, c.max_seq_len, c.valid_length != nullptr, 0);
    if (P < 1) return P;
  }
  if (P < 1 || P > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  if (P > 1 && !da::splitk_reduce_supported(p.depth_v, P)) return DA_ERR_UNSUPPORTED;
  const bool split = partials_only || P > 1;
  if (split) {
    const size_t need = decode_workspace_size(P, 1, (int)(rows / c.num_q_heads), c.num_q_heads,
                                              p.depth_v);
    if (!workspace || workspace_bytes < need) return DA_ERR_WORKSPACE;
  }

  p.num_partitions = P;
  p.keys_per_partition = keys_per_partition(c.max_seq_len, P, plan.step);
  p.row_blocks = plan.row_blocks;
  p.sink = sink;
  p.out = out;
  p.lse = lse;
  p.write_partials = split ? 1 : 0;
  // An MLA call's own split over partitions of at least kMlaBf16PartialKeys keys
  // hands its merge bf16 partial rows, as the pages' partition kernel writes its
  // partial output in the output type: half the bytes of the write-back and of the
  // merge's read.  Such a partial row averages values over many keys and its
  // rounding adds at most one bf16 rounding of the same size to the output; short
  // partitions keep fp32 rows.
  p.part_bf16 = (split && !partials_only && (plan.variant == kMla || plan.variant == kMlaFp8) &&
                 p.keys_per_partition >= kMlaBf16PartialKeys)
                    ? 1
                    : 0;
  float *po = nullptr, *pm = nullptr, *pl = nullptr;
  unsigned long long* queue = nullptr;
  if (split) ws_sections(workspace, P, rows, p.depth_v, &po, &pm, &pl, &queue);
  p.part_o = po;
  p.part_m = pm;
  p.part_l = pl;
  // Ragged batches on the streaming GQA kernels take their work items from a
  // queue (blocks that finish early take more): one resident block per CU for
  // bf16 (its queue form has a 96 KB ring), two for the 8-bit cache.
  p.queue = nullptr;
  p.queue_blocks = 0;
  if (split && (plan.variant == kStream || plan.variant == kStreamFp8) && c.valid_length &&
      plan.row_blocks == 1) {
    p.queue = queue;
    p.queue_blocks = (plan.variant == kStream ? 1 : 2) * device_cus();
  }
  // A split call of the streaming GQA kernels (static mapping) whose fold leaves
  // room in the 16 rows of a block folds two KV heads into one block, which then
  // reads one contiguous piece of each key row instead of one head's: measured
  // faster on this chip (long-context batch 1: kernel 86 -> 81 us).  Only while
  // the blocks still cover the CUs; work-queue calls measured slower with it.
  p.hb_shift = 0;
  if (split && !p.queue && (plan.variant == kStream || plan.variant == kStreamFp8) &&
      plan.row_blocks == 1 && fold_allows_two_heads(c.q_len, p.group, p.num_kv_heads) &&
      (long)P * c.batch * (p.num_kv_heads / 2) * plan.row_blocks >= device_cus())
    p.hb_shift = 1;

  // A small fp32 split call (at most kValuMergeGroups row groups, at most 8
  // partitions, whose rows the merging block requests all at once) merges inside
  // its partition pass: the last block of each row group merges the group's rows
  // with the merge pass's operations, so the call is one launch instead of two
  // (such calls are bound by launch latency).  Its count words are the spare words
  // of the queue section, which no fp32 call uses for a queue.
  unsigned* merge_count = nullptr;
  if (plan.variant == kValu && split && !partials_only && P <= 8 &&
      (long)c.batch * p.num_kv_heads * plan.row_blocks <= kValuMergeGroups)
    merge_count = (unsigned*)queue + 2;
  hipStream_t s = (hipStream_t)stream;
  if (log_enabled())
    std::fprintf(stderr,
                 "[decode_attention] variant=%s B=%d T=%d H=%d KVH=%d D=%d Dv=%d S=%d P=%d C=%d "
                 "rows/block=%d row_blocks=%d grid=%d paged=%d merge=%s queue=%d heads/block=%d\n",
                 variant_name(plan.variant), c.batch, c.q_len, c.num_q_heads, p.num_kv_heads,
                 p.depth, p.depth_v, c.max_seq_len, P, p.keys_per_partition,
                 plan.rows_per_block, plan.row_blocks,
                 P * c.batch * (p.num_kv_heads >> p.hb_shift) * plan.row_blocks, c.page_table != nullptr,
                 (partials_only || P == 1) ? "none" : (merge_count ? "in-pass" : "launch"),
                 p.queue != nullptr, 1 << p.hb_shift);
  if (clear_queue && (p.queue || merge_count)) {  // the whole section: queue word and counts
    hipLaunchKernelGGL(clear_queue_section, dim3(1), dim3(kQueueBytes / 8), 0, s,
                       (unsigned long long*)queue);
    if (hipGetLastError() != hipSuccess) return DA_ERR_HIP;
  }
  if (launch_partition_pass(p, plan.variant, bf16, merge_count, s) != hipSuccess)
    return DA_ERR_HIP;
  if (!partials_only && P > 1 && !merge_count) {
    const hipError_t e =
        p.part_bf16 ? da::launch_splitk_reduce_bf16_partials(
                          (const uint16_t*)po, pm, pl, P, (int)rows, c.num_q_heads, sink, out, lse,
                          c.batch, c.q_offsets ? 0 : c.q_len * c.num_q_heads, s)
                    : da::launch_splitk_reduce(po, pm, pl, P, (int)rows, c.num_q_heads,
                                               p.depth_v, sink, out, bf16, lse, s);
    if (e != hipSuccess) return DA_ERR_HIP;
  }
  return DA_OK;
}

int check_mha(const Common& c, const void* q, const void* k, const void* v, int group,
              int depth, int dtype) {
  if (!q || !k || !v) return DA_ERR_INVALID_ARG;
  int rc = check_common(c);
  if (rc) return rc;
  if (group < 1 || c.num_q_heads % group != 0) return DA_ERR_INVALID_ARG;
  if (dtype != DA_F32 && dtype != DA_BF16) return DA_ERR_UNSUPPORTED;
  if (depth != 64 && depth != 128) return DA_ERR_UNSUPPORTED;
  return DA_OK;
}

int check_fp8kv(const Common& c, const void* q, const void* k, const void* v, int group,
                int depth, float k_scale, float v_scale) {
  if (!q || !k || !v) return DA_ERR_INVALID_ARG;
  int rc = check_common(c);
  if (rc) return rc;
  if (group < 1 || c.num_q_heads % group != 0) return DA_ERR_INVALID_ARG;
  if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || !std::isfinite(c.scale * k_scale))
    return DA_ERR_INVALID_ARG;
  if (depth != 128) return DA_ERR_UNSUPPORTED;
  return DA_OK;
}

// The partition pass and, for P > 1, the merge of bf16 q over an 8-bit KV
// cache: k_scale joins the softmax scale and v_scale the output factor.
int run_fp8kv(const Common& c, const void* q, const void* k, const void* v, float k_scale,
              float v_scale, int group, int depth, int num_partitions, bool partials_only,
              const float* sink, void* out, float* lse, void* workspace, size_t workspace_bytes,
              void* stream) {
  const int kv_heads = c.num_q_heads / group;
  da::DecodeParams p = base_params(c, q, k, v, kv_heads, group, depth, depth);
  p.scale_log2 = c.scale * k_scale * 1.4426950408889634f;
  p.v_scale = v_scale;
  return run(c, p, plan_fp8(c.q_len, group), true, num_partitions, partials_only, sink, out, lse,
             workspace, workspace_bytes, stream);
}

int check_mla(const Common& c, const void* q, const void* kv) {
  if (!q || !kv) return DA_ERR_INVALID_ARG;
  return check_common(c);
}

// MLA over an 8-bit e4m3 cache: k_scale joins the softmax scale, and the value
// slice (the same stored numbers) is scaled by it in the output.
int check_mla_fp8(const Common& c, const void* q, const void* kv, float k_scale) {
  int rc = check_mla(c, q, kv);
  if (rc) return rc;
  if (!std::isfinite(k_scale) || !std::isfinite(c.scale * k_scale)) return DA_ERR_INVALID_ARG;
  return DA_OK;
}

int run_mla_fp8(const Common& c, const void* q, const void* kv, float k_scale,
                int num_partitions, bool partials_only, const float* sink, void* out, float* lse,
                void* workspace, size_t workspace_bytes, void* stream) {
  da::DecodeParams p = base_params(c, q, kv, kv, 1, c.num_q_heads, kMlaDepth, kMlaDepthV);
  p.scale_log2 = c.scale * k_scale * 1.4426950408889634f;
  p.v_scale = k_scale;
  Plan pl = plan_mla(c.q_len, c.num_q_heads);
  pl.variant = kMlaFp8;
  return run(c, p, pl, true, num_partitions, partials_only, sink, out, lse, workspace,
             workspace_bytes, stream);
}

// Sparse top-k MLA: the kernel addresses a row by a 32-bit byte offset from
// the pool base, and a list entry by a 32-bit byte offset from its list.
constexpr long long kMaxSparsePoolRows = (1ll << 32) / (kMlaDepth * 2);
constexpr int kMaxTopk = 1 << 28;

// The list's keys per partition: long enough that a block's partial write-back
// (128 rows x 2 KB) stays below its share of the gathered rows, short enough
// that a batch of a few dozen sequences fills the chip.
constexpr int kSparseMinKeys = 512;

int sparse_partitions(int batch, int q_len, int num_q_heads, int topk, int num_cus) {
  if (num_cus <= 0) num_cus = device_cus();
  const Plan pl = plan_mla(q_len, num_q_heads);
  return heuristic_partitions(batch * pl.row_blocks, topk, num_cus, 1, kSparseMinKeys);
}

int check_sparse(const void* q, const void* kv, long long pool_rows, const int32_t* indices,
                 int indices_stride, const int32_t* topk_lengths, int batch, int q_len,
                 int num_q_heads, float scale) {
  if (!q || !kv || !topk_lengths) return DA_ERR_INVALID_ARG;
  if (!indices && indices_stride > 0) return DA_ERR_INVALID_ARG;  // stride 0: nothing is read
  if (batch < 0 || q_len < 1 || num_q_heads < 1 || indices_stride < 0 || pool_rows < 1)
    return DA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return DA_ERR_INVALID_ARG;
  if (pool_rows > kMaxSparsePoolRows || indices_stride > kMaxTopk) return DA_ERR_UNSUPPORTED;
  return DA_OK;
}

// The partition pass and, for P > 1, the merge over the listed pool rows: the
// counts take the place of the valid lengths and the list stride that of the
// cache length.
int run_sparse(const void* q, const void* kv, long long pool_rows, const int32_t* indices,
               int indices_stride, const int32_t* topk_lengths, int batch, int q_len,
               int num_q_heads, float scale, int num_partitions, bool partials_only,
               const float* sink, void* out, float* lse, void* workspace,
               size_t workspace_bytes, void* stream) {
  const Common c{nullptr,        0,     0,           (const uint32_t*)topk_lengths,
                 batch,          q_len, num_q_heads, indices_stride,
                 DA_MASK_NONE,   scale};
  int P = num_partitions;
  if (P == 0) {
    if (batch == 0) return DA_OK;
    P = sparse_partitions(batch, q_len, num_q_heads, indices_stride, 0);
  }
  da::DecodeParams p = base_params(c, q, kv, kv, 1, num_q_heads, kMlaDepth, kMlaDepthV);
  p.indices = indices;
  p.pool_rows = (uint32_t)pool_rows;
  return run(c, p, plan_mla(q_len, num_q_heads), true, P, partials_only, sink, out, lse,
             workspace, workspace_bytes, stream);
}

}  // namespace

extern "C" {

const char* decode_attention_status_string(int status) {
  switch (status) {
    case DA_OK: return "ok";
    case DA_ERR_INVALID_ARG: return "invalid argument";
    case DA_ERR_UNSUPPORTED: return "unsupported configuration";
    case DA_ERR_WORKSPACE: return "workspace missing or too small";
    case DA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int decode_num_partitions(int batch, int q_len, int num_q_heads, int num_kv_heads, int depth,
                          int depth_v, int max_seq_len, int ragged, int num_cus) {
  if (batch < 1 || q_len < 1 || num_q_heads < 1 || num_kv_heads < 1 || depth < 1 ||
      depth_v < 1 || max_seq_len < 0 || num_q_heads % num_kv_heads != 0)
    return DA_ERR_INVALID_ARG;
  if (num_cus <= 0) num_cus = device_cus();
  // A dense batch wants about one block per CU.  A ragged one wants smaller
  // partitions so that its long sequences spread out: the GQA kernel takes
  // them from a work queue (about 16 items per CU), MLA from its grid.
  const bool mla = depth == kMlaDepth && num_kv_heads == 1;
  const int per_cu = ragged ? (mla ? 8 : 16) : 1;
  if (mla) {
    const Plan pl = plan_mla(q_len, num_q_heads);
    // MLA partials are 512 wide per row: keep partitions long so the partial
    // write-back stays a small fraction of the cache read.
    return heuristic_partitions(batch * pl.row_blocks, max_seq_len, num_cus, per_cu, 1024);
  }
  const Plan pl = plan_mha(q_len, num_q_heads / num_kv_heads, true);
  long P = heuristic_partitions(batch * num_kv_heads * pl.row_blocks, max_seq_len, num_cus,
                                per_cu, kMhaMinKeys);
  // A dense split call at depth 128 with room for two KV heads per block runs
  // them folded (bf16 and 8-bit caches): twice the partitions keep the grid full.
  if (!ragged && P > 1 && depth == 128 &&
      fold_allows_two_heads(q_len, num_q_heads / num_kv_heads, num_kv_heads)) {
    const long by_len = ((long)max_seq_len + kMhaMinKeys - 1) / kMhaMinKeys;
    P = std::min(std::min(2 * P, by_len), (long)DA_MAX_PARTITIONS);
  }
  return (int)P;
}

size_t decode_workspace_size(int num_partitions, int batch, int q_len, int num_q_heads,
                             int depth_v) {
  if (num_partitions < 1 || batch < 0 || q_len < 1 || num_q_heads < 1 || depth_v < 1) return 0;
  const size_t rows = (size_t)batch * q_len * num_q_heads;
  return kQueueBytes + align_up((size_t)num_partitions * rows * depth_v * sizeof(float)) +
         2 * align_up((size_t)num_partitions * rows * sizeof(float));
}

size_t decode_workspace_o_offset(int, int, int, int, int) { return kQueueBytes; }

size_t decode_workspace_max_offset(int num_partitions, int batch, int q_len, int num_q_heads,
                                   int depth_v) {
  const size_t rows = (size_t)batch * q_len * num_q_heads;
  return kQueueBytes + align_up((size_t)num_partitions * rows * depth_v * sizeof(float));
}

size_t decode_workspace_sum_offset(int num_partitions, int batch, int q_len, int num_q_heads,
                                   int depth_v) {
  const size_t rows = (size_t)batch * q_len * num_q_heads;
  return decode_workspace_max_offset(num_partitions, batch, q_len, num_q_heads, depth_v) +
         align_up((size_t)num_partitions * rows * sizeof(float));
}

int decode_attention(const void* q, const void* k, const void* v, const uint32_t* page_table,
                     int page_size, int max_pages_per_seq, const uint32_t* valid_length,
                     int batch, int q_len, int num_q_heads, int group, int depth,
                     int max_seq_len, float scale, int num_partitions,
                     const float* sink_weights, int mask, int dtype, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream) {
  const Common c{page_table, page_size, max_pages_per_seq, valid_length, batch,
                 q_len,      num_q_heads, max_seq_len, mask, scale};
  int rc = check_mha(c, q, k, v, group, depth, dtype);
  if (rc) return rc;
  if (!out) return DA_ERR_INVALID_ARG;
  if (num_partitions < 0 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  const bool bf16 = dtype == DA_BF16;
  const int kv_heads = num_q_heads / group;
  const da::DecodeParams p = base_params(c, q, k, v, kv_heads, group, depth, depth);
  return run(c, p, plan_mha(q_len, group, bf16), bf16, num_partitions, false, sink_weights, out,
             lse, workspace, workspace_bytes, stream);
}

int decode_attention_no_alloc(const void* q, const void* k, const void* v,
                              const uint32_t* page_table, int page_size, int max_pages_per_seq,
                              const uint32_t* valid_length, int batch, int q_len,
                              int num_q_heads, int group, int depth, int max_seq_len,
                              float scale, int num_partitions, const float* sink_weights,
                              int mask, int dtype, void* out, float* lse, void* stream) {
  const Common c{page_table, page_size, max_pages_per_seq, valid_length, batch,
                 q_len,      num_q_heads, max_seq_len, mask, scale};
  int rc = check_mha(c, q, k, v, group, depth, dtype);
  if (rc) return rc;
  if (!out) return DA_ERR_INVALID_ARG;
  if (num_partitions < 0 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  if (call_rows(c) == 0) return DA_OK;
  int P = num_partitions;
  if (P == 0) {
    P = decode_num_partitions(batch, q_len, num_q_heads, num_q_heads / group, depth, depth,
                              max_seq_len, valid_length != nullptr, 0);
    if (P < 1) return P;
  }
  // The scratch must hold this call's workspace (checked before anything is enqueued).
  if (P > 1 && decode_workspace_size(P, batch, q_len, num_q_heads, depth) > kNoAllocScratchBytes)
    return DA_ERR_WORKSPACE;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (P > 1) {
    ws = scratch_address();
    if (!ws) return DA_ERR_HIP;
    ws_bytes = kNoAllocScratchBytes;
  }
  const bool bf16 = dtype == DA_BF16;
  const da::DecodeParams p = base_params(c, q, k, v, num_q_heads / group, group, depth, depth);
  return run(c, p, plan_mha(q_len, group, bf16), bf16, P, false, sink_weights, out, lse, ws,
             ws_bytes, stream, /*clear_queue=*/true);
}

int decode_attention_partials(const void* q, const void* k, const void* v,
                              const uint32_t* page_table, int page_size, int max_pages_per_seq,
                              const uint32_t* valid_length, int batch, int q_len,
                              int num_q_heads, int group, int depth, int max_seq_len,
                              float scale, int num_partitions, int mask, int dtype,
                              void* workspace, size_t workspace_bytes, void* stream) {
  const Common c{page_table, page_size, max_pages_per_seq, valid_length, batch,
                 q_len,      num_q_heads, max_seq_len, mask, scale};
  int rc = check_mha(c, q, k, v, group, depth, dtype);
  if (rc) return rc;
  if (num_partitions < 1 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  const bool bf16 = dtype == DA_BF16;
  const int kv_heads = num_q_heads / group;
  const da::DecodeParams p = base_params(c, q, k, v, kv_heads, group, depth, depth);
  return run(c, p, plan_mha(q_len, group, bf16), bf16, num_partitions, true, nullptr, nullptr,
             nullptr, workspace, workspace_bytes, stream);
}

int decode_attention_ragged(const void* q, const uint32_t* q_offsets, int total_q_tokens,
                            int max_q_len, const void* k, const void* v,
                            const uint32_t* page_table, int page_size, int max_pages_per_seq,
                            const uint32_t* valid_length, int batch, int num_q_heads, int group,
                            int depth, int max_seq_len, float scale, int num_partitions,
                            const float* sink_weights, int mask, int dtype, void* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  Common c{page_table, page_size, max_pages_per_seq, valid_length, batch,
           max_q_len,  num_q_heads, max_seq_len, mask, scale};
  c.q_offsets = q_offsets;
  c.total_q_tokens = total_q_tokens;
  if (!q_offsets) return DA_ERR_INVALID_ARG;
  int rc = check_mha(c, q, k, v, group, depth, dtype);
  if (rc) return rc;
  if (!out) return DA_ERR_INVALID_ARG;
  if (num_partitions < 0 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  const bool bf16 = dtype == DA_BF16;
  const int kv_heads = num_q_heads / group;
  const da::DecodeParams p = base_params(c, q, k, v, kv_heads, group, depth, depth);
  return run(c, p, plan_mha(max_q_len, group, bf16), bf16, num_partitions, false, sink_weights,
             out, lse, workspace, workspace_bytes, stream);
}

int mla_decode_ragged(const void* q, const uint32_t* q_offsets, int total_q_tokens,
                      int max_q_len, const void* kv, const uint32_t* page_table, int page_size,
                      int max_pages_per_seq, const uint32_t* valid_length, int batch,
                      int num_q_heads, int max_seq_len, float scale, int num_partitions,
                      const float* sink_weights, int mask, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream) {
  Common c{page_table, page_size, max_pages_per_seq, valid_length, batch,
           max_q_len,  num_q_heads, max_seq_len, mask, scale};
  c.q_offsets = q_offsets;
  c.total_q_tokens = total_q_tokens;
  if (!q_offsets) return DA_ERR_INVALID_ARG;
  int rc = check_mla(c, q, kv);
  if (rc) return rc;
  if (!out) return DA_ERR_INVALID_ARG;
  if (num_partitions < 0 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  const da::DecodeParams p =
      base_params(c, q, kv, kv, 1, num_q_heads, kMlaDepth, kMlaDepthV);
  return run(c, p, plan_mla(max_q_len, num_q_heads), true, num_partitions, false, sink_weights,
             out, lse, workspace, workspace_bytes, stream);
}

int decode_attention_ragged_kv(const void* q, const void* k, const void* v,
                               const uint32_t* kv_row_offsets, const uint32_t* valid_length,
                               int batch, int q_len, int num_q_heads, int group, int depth,
                               int max_seq_len, float scale, int num_partitions,
                               const float* sink_weights, int mask, int dtype, void* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               void* stream) {
  Common c{nullptr, 0,     0,           valid_length, batch,
           q_len,   num_q_heads, max_seq_len, mask, scale};
  c.kv_row_offsets = kv_row_offsets;
  if (!kv_row_offsets && batch > 0) return DA_ERR_INVALID_ARG;
  int rc = check_mha(c, q, k, v, group, depth, dtype);
  if (rc) return rc;
  if (!out) return DA_ERR_INVALID_ARG;
  if (num_partitions < 0 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  const bool bf16 = dtype == DA_BF16;
  const int kv_heads = num_q_heads / group;
  const da::DecodeParams p = base_params(c, q, k, v, kv_heads, group, depth, depth);
  return run(c, p, plan_mha(q_len, group, bf16), bf16, num_partitions, false, sink_weights, out,
             lse, workspace, workspace_bytes, stream);
}

int mla_decode_ragged_kv(const void* q, const void* kv, const uint32_t* kv_row_offsets,
                         const uint32_t* valid_length, int batch, int q_len, int num_q_heads,
                         int max_seq_len, float scale, int num_partitions,
                         const float* sink_weights, int mask, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  Common c{nullptr, 0,     0,           valid_length, batch,
           q_len,   num_q_heads, max_seq_len, mask, scale};
  c.kv_row_offsets = kv_row_offsets;
  if (!kv_row_offsets && batch > 0) return DA_ERR_INVALID_ARG;
  int rc = check_mla(c, q, kv);
  if (rc) return rc;
  if (!out) return DA_ERR_INVALID_ARG;
  if (num_partitions < 0 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  const da::DecodeParams p = base_params(c, q, kv, kv, 1, num_q_heads, kMlaDepth, kMlaDepthV);
  return run(c, p, plan_mla(q_len, num_q_heads), true, num_partitions, false, sink_weights, out,
             lse, workspace, workspace_bytes, stream);
}

int decode_attention_fp8kv(const void* q, const void* k, const void* v, float k_scale,
                           float v_scale, const uint32_t* page_table, int page_size,
                           int max_pages_per_seq, const uint32_t* valid_length, int batch,
                           int q_len, int num_q_heads, int group, int depth, int max_seq_len,
                           float scale, int num_partitions, const float* sink_weights, int mask,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
  const Common c{page_table, page_size, max_pages_per_seq, valid_length, batch,
                 q_len,      num_q_heads, max_seq_len, mask, scale};
  int rc = check_fp8kv(c, q, k, v, group, depth, k_scale, v_scale);
  if (rc) return rc;
  if (!out) return DA_ERR_INVALID_ARG;
  if (num_partitions < 0 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  return run_fp8kv(c, q, k, v, k_scale, v_scale, group, depth, num_partitions, false,
                   sink_weights, out, lse, workspace, workspace_bytes, stream);
}

int decode_attention_fp8kv_partials(const void* q, const void* k, const void* v, float k_scale,
                                    float v_scale, const uint32_t* page_table, int page_size,
                                    int max_pages_per_seq, const uint32_t* valid_length,
                                    int batch, int q_len, int num_q_heads, int group, int depth,
                                    int max_seq_len, float scale, int num_partitions, int mask,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  const Common c{page_table, page_size, max_pages_per_seq, valid_length, batch,
                 q_len,      num_q_heads, max_seq_len, mask, scale};
  int rc = check_fp8kv(c, q, k, v, group, depth, k_scale, v_scale);
  if (rc) return rc;
  if (num_partitions < 1 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  return run_fp8kv(c, q, k, v, k_scale, v_scale, group, depth, num_partitions, true, nullptr,
                   nullptr, nullptr, workspace, workspace_bytes, stream);
}

int mla_decode(const void* q, const void* kv, const uint32_t* page_table, int page_size,
               int max_pages_per_seq, const uint32_t* valid_length, int batch, int q_len,
               int num_q_heads, int max_seq_len, float scale, int num_partitions,
               const float* sink_weights, int mask, void* out, float* lse, void* workspace,
               size_t workspace_bytes, void* stream) {
  const Common c{page_table, page_size, max_pages_per_seq, valid_length, batch,
                 q_len,      num_q_heads, max_seq_len, mask, scale};
  int rc = check_mla(c, q, kv);
  if (rc) return rc;
  if (!out) return DA_ERR_INVALID_ARG;
  if (num_partitions < 0 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  const da::DecodeParams p =
      base_params(c, q, kv, kv, 1, num_q_heads, kMlaDepth, kMlaDepthV);
  return run(c, p, plan_mla(q_len, num_q_heads), true, num_partitions, false, sink_weights, out,
             lse, workspace, workspace_bytes, stream);
}

int mla_decode_partials(const void* q, const void* kv, const uint32_t* page_table,
                        int page_size, int max_pages_per_seq, const uint32_t* valid_length,
                        int batch, int q_len, int num_q_heads, int max_seq_len, float scale,
                        int num_partitions, int mask, void* workspace, size_t workspace_bytes,
                        void* stream) {
  const Common c{page_table, page_size, max_pages_per_seq, valid_length, batch,
                 q_len,      num_q_heads, max_seq_len, mask, scale};
  int rc = check_mla(c, q, kv);
  if (rc) return rc;
  if (num_partitions < 1 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  const da::DecodeParams p =
      base_params(c, q, kv, kv, 1, num_q_heads, kMlaDepth, kMlaDepthV);
  return run(c, p, plan_mla(q_len, num_q_heads), true, num_partitions, true, nullptr, nullptr,
             nullptr, workspace, workspace_bytes, stream);
}

int mla_decode_fp8kv(const void* q, const void* kv, float k_scale, const uint32_t* page_table,
                     int page_size, int max_pages_per_seq, const uint32_t* valid_length,
                     int batch, int q_len, int num_q_heads, int max_seq_len, float scale,
                     int num_partitions, const float* sink_weights, int mask, void* out,
                     float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  const Common c{page_table, page_size, max_pages_per_seq, valid_length, batch,
                 q_len,      num_q_heads, max_seq_len, mask, scale};
  int rc = check_mla_fp8(c, q, kv, k_scale);
  if (rc) return rc;
  if (!out) return DA_ERR_INVALID_ARG;
  if (num_partitions < 0 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  return run_mla_fp8(c, q, kv, k_scale, num_partitions, false, sink_weights, out, lse,
                     workspace, workspace_bytes, stream);
}

int mla_decode_fp8kv_partials(const void* q, const void* kv, float k_scale,
                              const uint32_t* page_table, int page_size, int max_pages_per_seq,
                              const uint32_t* valid_length, int batch, int q_len,
                              int num_q_heads, int max_seq_len, float scale, int num_partitions,
                              int mask, void* workspace, size_t workspace_bytes, void* stream) {
  const Common c{page_table, page_size, max_pages_per_seq, valid_length, batch,
                 q_len,      num_q_heads, max_seq_len, mask, scale};
  int rc = check_mla_fp8(c, q, kv, k_scale);
  if (rc) return rc;
  if (num_partitions < 1 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  return run_mla_fp8(c, q, kv, k_scale, num_partitions, true, nullptr, nullptr, nullptr,
                     workspace, workspace_bytes, stream);
}

int mla_sparse_num_partitions(int batch, int q_len, int num_q_heads, int topk, int num_cus) {
  if (batch < 1 || q_len < 1 || num_q_heads < 1 || topk < 0) return DA_ERR_INVALID_ARG;
  return sparse_partitions(batch, q_len, num_q_heads, topk, num_cus);
}

int mla_decode_sparse(const void* q, const void* kv, long long pool_rows, const int32_t* indices,
                      int indices_stride, const int32_t* topk_lengths, int batch, int q_len,
                      int num_q_heads, float scale, int num_partitions,
                      const float* sink_weights, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int rc = check_sparse(q, kv, pool_rows, indices, indices_stride, topk_lengths, batch, q_len,
                        num_q_heads, scale);
  if (rc) return rc;
  if (!out) return DA_ERR_INVALID_ARG;
  if (num_partitions < 0 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  return run_sparse(q, kv, pool_rows, indices, indices_stride, topk_lengths, batch, q_len,
                    num_q_heads, scale, num_partitions, false, sink_weights, out, lse, workspace,
                    workspace_bytes, stream);
}

int mla_decode_sparse_partials(const void* q, const void* kv, long long pool_rows,
                               const int32_t* indices, int indices_stride,
                               const int32_t* topk_lengths, int batch, int q_len,
                               int num_q_heads, float scale, int num_partitions, void* workspace,
                               size_t workspace_bytes, void* stream) {
  int rc = check_sparse(q, kv, pool_rows, indices, indices_stride, topk_lengths, batch, q_len,
                        num_q_heads, scale);
  if (rc) return rc;
  if (num_partitions < 1 || num_partitions > DA_MAX_PARTITIONS) return DA_ERR_INVALID_ARG;
  return run_sparse(q, kv, pool_rows, indices, indices_stride, topk_lengths, batch, q_len,
                    num_q_heads, scale, num_partitions, true, nullptr, nullptr, nullptr,
                    workspace, workspace_bytes, stream);
}

int splitk_reduce(const float* part_o, const float* part_max, const float* part_sum,
                  int num_partitions, int rows, int num_q_heads, int depth_v,
                  const float* sink_weights, void* out, int out_dtype, float* lse,
                  void* stream) {
  if (!part_o || !part_max || !part_sum || !out) return DA_ERR_INVALID_ARG;
  if (rows < 0 || num_q_heads < 1 || num_partitions < 1) return DA_ERR_INVALID_ARG;
  if (out_dtype != DA_F32 && out_dtype != DA_BF16) return DA_ERR_UNSUPPORTED;
  if (!da::splitk_reduce_supported(depth_v, num_partitions)) return DA_ERR_UNSUPPORTED;
  if (rows == 0) return DA_OK;
  if (da::launch_splitk_reduce(part_o, part_max, part_sum, num_partitions, rows, num_q_heads,
                               depth_v, sink_weights, out, out_dtype == DA_BF16, lse,
                               (hipStream_t)stream) != hipSuccess)
    return DA_ERR_HIP;
  return DA_OK;
}

}  // extern "C"
