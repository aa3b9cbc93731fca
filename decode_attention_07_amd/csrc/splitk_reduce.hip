// splitk_reduce.hip -- log-sum-exp merge of split-K decode partials (gfx950).
//
// The merge pass that follows the split-K partition pass
// ("mha_decoding_single_batch_pipelined", description; the MLA counterpart in
// "flare_mla_decoding_dispatch", description), as a launch of its own: for
// partials from decode_attention_partials() / mla_decode_partials() or any other
// source, and the second launch of every split call (decode_attention() and
// mla_decode() with P > 1 and their 8-bit, ragged and sparse forms).
//
// The merge arithmetic (one wave per row) lives in da_merge.h.
#include "da_merge.h"

namespace da {

namespace {

constexpr int kWaves = 4;          // rows per block
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxP = 1024;

template <int DV, bool BF16OUT>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_m,
    const float* __restrict__ part_l, int P, int rows, int num_heads,
    const float* __restrict__ sink, void* __restrict__ out, float* __restrict__ lse) {
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave; nothing below synchronises the block
  merge_row<DV, BF16OUT>(part_o, part_m, part_l, P, rows, row, sink, num_heads, out, lse,
                         threadIdx.x & 63);
}

template <int DV>
hipError_t launch_reduce_dv(const float* po, const float* pm, const float* pl, int P, int rows,
                            int H, const float* sink, void* out, bool bf16, float* lse,
                            hipStream_t s) {
  const int grid = (rows + kWaves - 1) / kWaves;
  if (bf16)
    hipLaunchKernelGGL((splitk_reduce_kernel<DV, true>), dim3(grid), dim3(kThreads), 0, s, po,
                       pm, pl, P, rows, H, sink, out, lse);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<DV, false>), dim3(grid), dim3(kThreads), 0, s, po,
                       pm, pl, P, rows, H, sink, out, lse);
  return hipGetLastError();
}

}  // namespace

bool splitk_reduce_supported(int depth_v, int P) {
  return (depth_v == 64 || depth_v == 128 || depth_v == 256 || depth_v == 512 ||
          depth_v == 1024) &&
         P >= 1 && P <= kMaxP;
}

hipError_t launch_splitk_reduce(const float* po, const float* pm, const float* pl, int P,
                                int rows, int H, int depth_v, const float* sink, void* out,
                                bool bf16, float* lse, hipStream_t s) {
  switch (depth_v) {
    case 64: return launch_reduce_dv<64>(po, pm, pl, P, rows, H, sink, out, bf16, lse, s);
    case 128: return launch_reduce_dv<128>(po, pm, pl, P, rows, H, sink, out, bf16, lse, s);
    case 256: return launch_reduce_dv<256>(po, pm, pl, P, rows, H, sink, out, bf16, lse, s);
    case 512: return launch_reduce_dv<512>(po, pm, pl, P, rows, H, sink, out, bf16, lse, s);
    default: return launch_reduce_dv<1024>(po, pm, pl, P, rows, H, sink, out, bf16, lse, s);
  }
}

}  // namespace da
