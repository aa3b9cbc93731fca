// splitk_reduce.hip -- log-sum-exp merge of split-K decode partials (gfx950).
//
// The "subsequent mha_splitk_reduce pass" of "mha_decoding_single_batch_pipelined"
// (description) and the "mla_splitk_reduce" of "flare_mla_decoding_dispatch"
// (description).  One block of 4 waves per output row: the block first forms
// the partition weights in LDS, then each wave accumulates every 4th partition
// (lanes stripe the depth, so each partial row is one coalesced read; four
// partitions are in flight per wave), and the 4 wave sums are added through LDS.
//
// Per row: M = max(max_p m_p, sigma), w_p = l_p * exp(m_p - M) (0 when l_p = 0),
// L = sum_p w_p + exp(sigma - M), out = sum_p w_p * O_p / L, lse = M + ln L.
#include "da_device.h"

namespace da {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxP = 1024;
constexpr int kUnroll = 4;

template <int DV, bool BF16OUT>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_m,
    const float* __restrict__ part_l, int P, int rows, int num_heads,
    const float* __restrict__ sink, void* __restrict__ out, float* __restrict__ lse) {
  constexpr int PER_LANE = DV / 64;
  __shared__ float sw[kMaxP];
  __shared__ float sred[kWaves];
  __shared__ float sacc[kWaves][DV];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = blockIdx.x;

  // Block max over the partitions that hold anything (natural log -> log2).
  float M = kNegInf;
  for (int pp = tid; pp < P; pp += kThreads) {
    const float lp = part_l[(size_t)pp * rows + row];
    if (lp > 0.f) M = fmaxf(M, part_m[(size_t)pp * rows + row] * kLog2e);
  }
  for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, shfl_xor(M, x));
  if (lane == 0) sred[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(sred[0], sred[1]), fmaxf(sred[2], sred[3]));
  float sig = kNegInf;
  if (sink) {
    sig = sink[row % num_heads] * kLog2e;
    M = fmaxf(M, sig);
  }
  const float Ms = (M == kNegInf) ? 0.f : M;
  __syncthreads();  // sred is reused below

  // Weights into LDS; block sum.
  float L = 0.f;
  for (int pp = tid; pp < P; pp += kThreads) {
    const float lp = part_l[(size_t)pp * rows + row];
    const float w = (lp > 0.f) ? lp * fast_exp2(part_m[(size_t)pp * rows + row] * kLog2e - Ms)
                               : 0.f;
    sw[pp] = w;
    L += w;
  }
  for (int x = 32; x >= 1; x >>= 1) L += shfl_xor(L, x);
  if (lane == 0) sred[wave] = L;
  __syncthreads();
  L = sred[0] + sred[1] + sred[2] + sred[3];
  if (sink) L += fast_exp2(sig - Ms);

  // Wave w accumulates partitions w, w + 4, ...; kUnroll of them in flight.
  float acc[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) acc[i] = 0.f;
  const float* base = part_o + (size_t)row * DV + lane;
  const size_t pstride = (size_t)rows * DV;
  int pp = wave;
  for (; pp + (kUnroll - 1) * kWaves < P; pp += kUnroll * kWaves) {
    float v[kUnroll][PER_LANE];
    float w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      w[u] = sw[pp + u * kWaves];
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i)
        v[u][i] = base[(size_t)(pp + u * kWaves) * pstride + 64 * i];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i)
        acc[i] = fmaf(w[u], (w[u] != 0.f) ? v[u][i] : 0.f, acc[i]);  // empty partials: skip
  }
  for (; pp < P; pp += kWaves) {
    const float w = sw[pp];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const float v = base[(size_t)pp * pstride + 64 * i];
      acc[i] = fmaf(w, (w != 0.f) ? v : 0.f, acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) sacc[wave][lane + 64 * i] = acc[i];
  __syncthreads();

  const bool any = L > 0.f;
  const float inv = any ? 1.f / L : 0.f;
  for (int d = tid; d < DV; d += kThreads) {
    const float res = (sacc[0][d] + sacc[1][d] + sacc[2][d] + sacc[3][d]) * inv;
    if constexpr (BF16OUT)
      ((uint16_t*)out)[(size_t)row * DV + d] = to_bf16(res);
    else
      ((float*)out)[(size_t)row * DV + d] = res;
  }
  if (lse && tid == 0) lse[row] = any ? (M + fast_log2(L)) * kLn2 : kNegInf;
}

template <int DV>
hipError_t launch_reduce_dv(const float* po, const float* pm, const float* pl, int P, int rows,
                            int H, const float* sink, void* out, bool bf16, float* lse,
                            hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL((splitk_reduce_kernel<DV, true>), dim3(rows), dim3(kThreads), 0, s, po,
                       pm, pl, P, rows, H, sink, out, lse);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<DV, false>), dim3(rows), dim3(kThreads), 0, s, po,
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
