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

// seq_chunks > 0: the rows come in sequences of seq_chunks blocks' worth, and the
// blocks of sequence b run on XCD b mod 8 (blocks i and i + 8 share an XCD), the
// one whose L2 took that sequence's partial rows from its partition pass.
template <int DV, bool BF16OUT, typename PO, int SLOTS = 0>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(
    const PO* __restrict__ part_o, const float* __restrict__ part_m,
    const float* __restrict__ part_l, int P, int rows, int num_heads,
    const float* __restrict__ sink, void* __restrict__ out, float* __restrict__ lse,
    int seq_chunks = 0) {
  int chunk = blockIdx.x;
  if (seq_chunks > 0) {
    const int k = blockIdx.x >> 3;
    chunk = ((blockIdx.x & 7) + 8 * (k / seq_chunks)) * seq_chunks + k % seq_chunks;
  }
  const int row = chunk * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave; nothing below synchronises the block
  merge_row<DV, BF16OUT, PO, SLOTS>(part_o, part_m, part_l, P, rows, row, sink, num_heads, out,
                                    lse, threadIdx.x & 63);
}

// Rows split into 33..64 partitions at DV <= 128 (a long sequence over few
// rows): two waves per row, each merging 32 partitions with all their partial
// rows in flight, then one combine through LDS: one memory round trip per row
// instead of two.  Two rows per block of 4 waves.
template <int DV, bool BF16OUT>
__global__ __launch_bounds__(kThreads) void splitk_reduce_pair_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_m,
    const float* __restrict__ part_l, int P, int rows, int num_heads,
    const float* __restrict__ sink, void* __restrict__ out, float* __restrict__ lse) {
  constexpr int EPL = DV / 64;
  __shared__ float s_acc[2][64 * EPL];
  __shared__ float s_ml[2][2];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slot = wave >> 1, half = wave & 1;
  const int row = blockIdx.x * 2 + slot;
  const bool valid = row < rows;  // both waves of a slot agree; every wave reaches the barrier
  float acc[EPL];
  float Mh = kNegInf, lh = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  if (valid) merge_half<DV>(part_o, part_m, part_l, P, rows, row, half, lane, acc, Mh, lh);
  if (half == 1) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_acc[slot][lane * EPL + e] = acc[e];
    if (lane == 0) {
      s_ml[slot][0] = Mh;
      s_ml[slot][1] = lh;
    }
  }
  __syncthreads();
  if (half == 1 || !valid) return;
  const float M1 = s_ml[slot][0], l1 = s_ml[slot][1];
  const float sig = sink ? sink[row % num_heads] * kLog2e : kNegInf;
  const float M = fmaxf(fmaxf(Mh, M1), sig);
  const float Ms = (M == kNegInf) ? 0.f : M;
  const float f0 = fast_exp2(Mh - Ms), f1 = fast_exp2(M1 - Ms);  // 0 for an empty half
  float L = lh * f0 + l1 * f1;
  if (sink) L += fast_exp2(sig - Ms);
  const bool any = L > 0.f;
  const float inv = any ? 1.f / L : 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = (acc[e] * f0 + s_acc[slot][lane * EPL + e] * f1) * inv;
  if constexpr (BF16OUT) {
    uint16_t* dst = (uint16_t*)out + (size_t)row * DV + lane * EPL;
    if constexpr (EPL == 1)
      dst[0] = to_bf16(o[0]);
    else
      *(uint32_t*)dst = pack_bf16(o[0], o[1]);
  } else {
    float* dst = (float*)out + (size_t)row * DV + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[e] = o[e];
  }
  if (lse && lane == 0) lse[row] = any ? (M + fast_log2(L)) * kLn2 : kNegInf;
}

template <int DV, int SLOTS>
hipError_t launch_reduce_slots(const float* po, const float* pm, const float* pl, int P,
                               int rows, int H, const float* sink, void* out, bool bf16,
                               float* lse, int grid, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL((splitk_reduce_kernel<DV, true, float, SLOTS>), dim3(grid),
                       dim3(kThreads), 0, s, po, pm, pl, P, rows, H, sink, out, lse, 0);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<DV, false, float, SLOTS>), dim3(grid),
                       dim3(kThreads), 0, s, po, pm, pl, P, rows, H, sink, out, lse, 0);
  return hipGetLastError();
}

template <int DV>
hipError_t launch_reduce_dv(const float* po, const float* pm, const float* pl, int P, int rows,
                            int H, const float* sink, void* out, bool bf16, float* lse,
                            hipStream_t s) {
  if constexpr (DV <= 128) {
    if (P > 32 && P <= 64) {
      const int grid2 = (rows + 1) / 2;
      if (bf16)
        hipLaunchKernelGGL((splitk_reduce_pair_kernel<DV, true>), dim3(grid2), dim3(kThreads), 0,
                           s, po, pm, pl, P, rows, H, sink, out, lse);
      else
        hipLaunchKernelGGL((splitk_reduce_pair_kernel<DV, false>), dim3(grid2), dim3(kThreads), 0,
                           s, po, pm, pl, P, rows, H, sink, out, lse);
      return hipGetLastError();
    }
  }
  const int grid = (rows + kWaves - 1) / kWaves;
  if constexpr (DV <= 128) {
    // Partial rows requested per group: as many as the partitions need (4, 8 or 16),
    // not 32 whatever P, so that a split into a few partitions does not re-read a
    // row for every empty slot.  The same operations in the same order.
    if (P <= 16) {
      if (P <= 4) return launch_reduce_slots<DV, 4>(po, pm, pl, P, rows, H, sink, out, bf16, lse,
                                                    grid, s);
      if (P <= 8) return launch_reduce_slots<DV, 8>(po, pm, pl, P, rows, H, sink, out, bf16, lse,
                                                    grid, s);
      return launch_reduce_slots<DV, 16>(po, pm, pl, P, rows, H, sink, out, bf16, lse, grid, s);
    }
  }
  return launch_reduce_slots<DV, 0>(po, pm, pl, P, rows, H, sink, out, bf16, lse, grid, s);
}

}  // namespace

bool splitk_reduce_supported(int depth_v, int P) {
  return (depth_v == 64 || depth_v == 128 || depth_v == 256 || depth_v == 512 ||
          depth_v == 1024) &&
         P >= 1 && P <= kMaxP;
}

hipError_t launch_splitk_reduce_bf16_partials(const uint16_t* po, const float* pm,
                                              const float* pl, int P, int rows, int H,
                                              const float* sink, void* out, float* lse,
                                              int batch, int seq_rows, hipStream_t s) {
  // Mixed partial O of the 512-wide MLA rows (partition 0 fp32, the others bf16:
  // da_params.h), bf16 output.  The MLA partition pass
  // runs sequence b's blocks on XCD b mod 8 when the batch is a multiple of 8; the
  // merge of its rows is then mapped onto the same XCD (seq_rows = T * H rows per
  // sequence, 0 when they vary).
  const int grid = (rows + kWaves - 1) / kWaves;
  const bool xcd = batch > 0 && batch % 8 == 0 && seq_rows > 0 && seq_rows % kWaves == 0 &&
                   (long)batch * seq_rows == rows;
  // Partial rows requested per group: as many as the partitions (2, 4 or 8), so
  // that a short split does not re-read a row for every empty slot.
  const int sc = xcd ? seq_rows / kWaves : 0;
  if (P <= 2)
    hipLaunchKernelGGL((splitk_reduce_kernel<512, true, uint16_t, 2>), dim3(grid),
                       dim3(kThreads), 0, s, po, pm, pl, P, rows, H, sink, out, lse, sc);
  else if (P <= 4)
    hipLaunchKernelGGL((splitk_reduce_kernel<512, true, uint16_t, 4>), dim3(grid),
                       dim3(kThreads), 0, s, po, pm, pl, P, rows, H, sink, out, lse, sc);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<512, true, uint16_t, 8>), dim3(grid),
                       dim3(kThreads), 0, s, po, pm, pl, P, rows, H, sink, out, lse, sc);
  return hipGetLastError();
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
