// splitk_reduce.hip -- log-sum-exp merge of split-K decode partials (gfx950).
//
// The "subsequent mha_splitk_reduce pass" of "mha_decoding_single_batch_pipelined"
// (description) and the "mla_splitk_reduce" of "flare_mla_decoding_dispatch"
// (description).
//
// Per row: M = max(max_p m_p, sigma), w_p = l_p * exp(m_p - M) (0 when l_p = 0),
// L = sum_p w_p + exp(sigma - M), out = sum_p w_p * O_p / L, lse = M + ln L.
//
// One wave per row, no block barriers.  Lanes take the partitions' (m_p, l_p)
// 64 at a time, so the row max and the weights need one load round trip and
// two wave reductions; the weights are then broadcast one partition at a time
// through scalar lane reads while every lane accumulates its DV/64 consecutive
// columns of O_p (one coalesced row read per partition, eight partitions in
// flight).  Empty partitions (weight 0) are skipped without loading their row.
#include "da_device.h"

namespace da {

namespace {

constexpr int kWaves = 4;          // rows per block
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxP = 1024;
constexpr int kInFlight = 8;       // partial rows requested ahead

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x = fmaxf(x, shfl_xor(x, s));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x += shfl_xor(x, s);
  return x;
}

template <int EPL>
struct Cols {
  float v[EPL];
};

template <int EPL>
__device__ __forceinline__ Cols<EPL> load_cols(const float* p) {
  Cols<EPL> c;
  if constexpr (EPL % 4 == 0) {
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i) {
      const float4 f = *(const float4*)(p + 4 * i);
      c.v[4 * i] = f.x;
      c.v[4 * i + 1] = f.y;
      c.v[4 * i + 2] = f.z;
      c.v[4 * i + 3] = f.w;
    }
  } else if constexpr (EPL == 2) {
    const float2 f = *(const float2*)p;
    c.v[0] = f.x;
    c.v[1] = f.y;
  } else {
    c.v[0] = *p;
  }
  return c;
}

template <int DV, bool BF16OUT>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_m,
    const float* __restrict__ part_l, int P, int rows, int num_heads,
    const float* __restrict__ sink, void* __restrict__ out, float* __restrict__ lse) {
  constexpr int EPL = DV / 64;  // consecutive columns per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave; nothing below synchronises the block

  // Row max over the partitions that hold anything (natural log -> log2), and
  // the sink.
  float mx = kNegInf;
  for (int pp = lane; pp < P; pp += 64) {
    const float lp = part_l[(size_t)pp * rows + row];
    if (lp > 0.f) mx = fmaxf(mx, part_m[(size_t)pp * rows + row] * kLog2e);
  }
  float M = wave_max(mx);
  float sig = kNegInf;
  if (sink) {
    sig = sink[row % num_heads] * kLog2e;
    M = fmaxf(M, sig);
  }
  const float Ms = (M == kNegInf) ? 0.f : M;

  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float lsum = 0.f;
  const float* orow = part_o + (size_t)row * DV + lane * EPL;
  const size_t pstride = (size_t)rows * DV;
  for (int base = 0; base < P; base += 64) {
    // this lane's partition of the chunk and its weight
    const int pp = base + lane;
    float w = 0.f;
    if (pp < P) {
      const float lp = part_l[(size_t)pp * rows + row];
      if (lp > 0.f) w = lp * fast_exp2(part_m[(size_t)pp * rows + row] * kLog2e - Ms);
    }
    lsum += w;
    const int n = min(64, P - base);
    int j = 0;
    for (; j + kInFlight <= n; j += kInFlight) {
      float wj[kInFlight];
      Cols<EPL> c[kInFlight];
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) {
        wj[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j + u));
        if (wj[u] != 0.f) c[u] = load_cols<EPL>(orow + (size_t)(base + j + u) * pstride);
      }
#pragma unroll
      for (int u = 0; u < kInFlight; ++u)
        if (wj[u] != 0.f)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] = fmaf(wj[u], c[u].v[e], acc[e]);
    }
    for (; j < n; ++j) {
      const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
      if (wj != 0.f) {
        const Cols<EPL> c = load_cols<EPL>(orow + (size_t)(base + j) * pstride);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(wj, c.v[e], acc[e]);
      }
    }
  }
  float L = wave_sum(lsum);
  if (sink) L += fast_exp2(sig - Ms);

  const bool any = L > 0.f;
  const float inv = any ? 1.f / L : 0.f;
  if constexpr (BF16OUT) {
    uint16_t* dst = (uint16_t*)out + (size_t)row * DV + lane * EPL;
    if constexpr (EPL == 1) {
      dst[0] = to_bf16(acc[0] * inv);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; e += 2) *(uint32_t*)(dst + e) = pack_bf16(acc[e] * inv, acc[e + 1] * inv);
    }
  } else {
    float* dst = (float*)out + (size_t)row * DV + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[e] = acc[e] * inv;
  }
  if (lse && lane == 0) lse[row] = any ? (M + fast_log2(L)) * kLn2 : kNegInf;
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
