// splitk_reduce.hip -- log-sum-exp merge of split-K decode partials (gfx950).
//
// The "subsequent mha_splitk_reduce pass" of "mha_decoding_single_batch_pipelined"
// (description) and the "mla_splitk_reduce" of "flare_mla_decoding_dispatch"
// (description).  One wave per output row: the lanes stripe the depth so every
// partial row is read with coalesced loads; the partition weights are formed
// once per row in LDS.
//
// Per row: M = max(max_p m_p, sigma), w_p = l_p * exp(m_p - M) (0 when l_p = 0),
// L = sum_p w_p + exp(sigma - M), out = sum_p w_p * O_p / L, lse = M + ln L.
#include "da_device.h"

namespace da {

constexpr int kReduceWaves = 4;
constexpr int kReduceMaxP = 1024;

template <int DV, bool BF16OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_m,
    const float* __restrict__ part_l, int P, int rows, int num_heads,
    const float* __restrict__ sink, void* __restrict__ out, float* __restrict__ lse) {
  constexpr int PER_LANE = DV / 64;
  __shared__ float sw[kReduceWaves][kReduceMaxP];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row_raw = blockIdx.x * kReduceWaves + wave;
  const bool live = row_raw < rows;           // uniform per wave
  const int row = live ? row_raw : rows - 1;  // idle waves recompute the last row, write nothing

  // Max over partitions that hold anything (natural-log units -> log2).
  float M = kNegInf;
  for (int pp = lane; pp < P; pp += 64) {
    const float lp = part_l[(size_t)pp * rows + row];
    if (lp > 0.f) M = fmaxf(M, part_m[(size_t)pp * rows + row] * kLog2e);
  }
  for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, shfl_xor(M, x));
  float sig = kNegInf;
  if (sink) {
    sig = sink[row % num_heads] * kLog2e;
    M = fmaxf(M, sig);
  }
  const float Ms = (M == kNegInf) ? 0.f : M;

  float L = 0.f;
  for (int pp = lane; pp < P; pp += 64) {
    const float lp = part_l[(size_t)pp * rows + row];
    const float w = (lp > 0.f) ? lp * fast_exp2(part_m[(size_t)pp * rows + row] * kLog2e - Ms)
                               : 0.f;
    sw[wave][pp] = w;
    L += w;
  }
  for (int x = 32; x >= 1; x >>= 1) L += shfl_xor(L, x);
  if (sink) L += fast_exp2(sig - Ms);
  __syncthreads();  // weights in LDS visible to every lane of the wave

  float acc[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) acc[i] = 0.f;
  for (int pp = 0; pp < P; ++pp) {
    const float w = sw[wave][pp];
    if (w == 0.f) continue;  // uniform across the wave
    const float* src = part_o + ((size_t)pp * rows + row) * DV;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) acc[i] = fmaf(w, src[lane + 64 * i], acc[i]);
  }
  if (!live) return;
  const bool any = L > 0.f;
  const float inv = any ? 1.f / L : 0.f;
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const float res = acc[i] * inv;
    if constexpr (BF16OUT)
      ((uint16_t*)out)[(size_t)row * DV + lane + 64 * i] = to_bf16(res);
    else
      ((float*)out)[(size_t)row * DV + lane + 64 * i] = res;
  }
  if (lse && lane == 0) lse[row] = any ? (M + fast_log2(L)) * kLn2 : kNegInf;
}

template <int DV>
static hipError_t launch_reduce_dv(const float* po, const float* pm, const float* pl, int P,
                                   int rows, int H, const float* sink, void* out, bool bf16,
                                   float* lse, hipStream_t s) {
  const int grid = (rows + kReduceWaves - 1) / kReduceWaves;
  if (bf16)
    hipLaunchKernelGGL((splitk_reduce_kernel<DV, true>), dim3(grid), dim3(64 * kReduceWaves), 0,
                       s, po, pm, pl, P, rows, H, sink, out, lse);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<DV, false>), dim3(grid), dim3(64 * kReduceWaves),
                       0, s, po, pm, pl, P, rows, H, sink, out, lse);
  return hipGetLastError();
}

bool splitk_reduce_supported(int depth_v, int P) {
  return (depth_v == 64 || depth_v == 128 || depth_v == 256 || depth_v == 512 ||
          depth_v == 1024) &&
         P >= 1 && P <= kReduceMaxP;
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
