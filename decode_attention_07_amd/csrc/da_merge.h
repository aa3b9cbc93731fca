// da_merge.h -- log-sum-exp merge of split-K partials for one row (the body of
// the splitk_reduce kernel).
//
// Per row: M = max(max_p m_p, sigma), w_p = l_p * exp(m_p - M) (0 when l_p = 0),
// L = sum_p w_p + exp(sigma - M), out = sum_p w_p * O_p / L, lse = M + ln L
// ("mha_decoding_single_batch_pipelined", description: the mha_splitk_reduce
// pass).  One wave per row: lanes take the partitions' (m_p, l_p) 64 at a time,
// so the row max and the weights need wave reductions only; the weights are then
// broadcast one partition at a time through scalar lane reads while every lane
// accumulates its DV/64 consecutive columns of O_p (one coalesced row read per
// partition, up to 32 partitions in flight).  With at most 64 partitions the
// partial rows are requested together with (m_p, l_p), since their addresses do
// not depend on the weights: one memory round trip per row.  An empty
// partition's value (weight 0) is dropped by a select, whatever its row holds.
#pragma once

#include "da_device.h"

namespace da {

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
struct MergeCols {
  float v[EPL];
};

// EPL consecutive bf16 partial values (the dense MLA kernel's own long split).
template <int EPL>
__device__ __forceinline__ MergeCols<EPL> merge_load_cols(const uint16_t* p) {
  static_assert(EPL % 8 == 0, "bf16 partial rows are read 8 values at a time");
  MergeCols<EPL> c;
#pragma unroll
  for (int i = 0; i < EPL / 8; ++i) {
    const uint4 u = *(const uint4*)(p + 8 * i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c.v[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
      c.v[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
  return c;
}

template <int EPL>
__device__ __forceinline__ MergeCols<EPL> merge_load_cols(const float* p) {
  MergeCols<EPL> c;
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

// This lane's EPL columns of partition u's partial row.  fp32 partials: row
// (u, row) of part_o [P, rows, DV].  Mixed partials (PO = uint16_t, the MLA
// kernels' own long splits): partition 0's row is fp32 at (float*)part_o + row *
// DV, partition u >= 1's is bf16 at part_o + ((u + 1) * rows + row) * DV.
template <int DV, typename PO>
__device__ __forceinline__ MergeCols<DV / 64> merge_part_cols(const PO* __restrict__ part_o,
                                                              int rows, int row, int u,
                                                              int lane) {
  constexpr int EPL = DV / 64;
  if constexpr (sizeof(PO) == 2) {
    if (u == 0)
      return merge_load_cols<EPL>((const float*)part_o + (size_t)row * DV + lane * EPL);
    return merge_load_cols<EPL>(part_o + ((size_t)(u + 1) * rows + row) * DV + lane * EPL);
  } else {
    return merge_load_cols<EPL>(part_o + ((size_t)u * rows + row) * DV + lane * EPL);
  }
}

// acc += w_u * O_u over a group of partial rows; a zero weight drops its row.
template <int EPL, int N>
__device__ __forceinline__ void merge_accumulate(float (&acc)[EPL], const float (&wj)[N],
                                                 const MergeCols<EPL> (&c)[N]) {
#pragma unroll
  for (int u = 0; u < N; ++u)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float t = fmaf(wj[u], c[u].v[e], acc[e]);
      acc[e] = (wj[u] != 0.f) ? t : acc[e];
    }
}

// Merges row `row` (of `rows` per partition) of the partial rows (fp32, or the
// mixed fp32 / bf16 layout with PO = uint16_t: merge_part_cols), part_m / part_l
// [P, rows]; writes out[row, :] (bf16 or fp32) and lse[row] (if lse).  Called by
// all 64 lanes of one wave; sink (or nullptr) is indexed by row % num_heads.
// SLOTS > 0: partial rows requested per group (at least 2 for mixed partials);
// 0: 64 values per lane, at most 32 rows.
template <int DV, bool BF16OUT, typename PO = float, int SLOTS = 0>
__device__ __forceinline__ void merge_row(const PO* __restrict__ part_o,
                                          const float* __restrict__ part_m,
                                          const float* __restrict__ part_l, int P, int rows,
                                          int row, const float* __restrict__ sink,
                                          int num_heads, void* __restrict__ out,
                                          float* __restrict__ lse, int lane) {
  constexpr int EPL = DV / 64;  // consecutive columns per lane
  // Partial rows requested ahead: 64 values per lane in flight (8 rows at
  // DV = 512, 32 at DV <= 128, where a long split of few rows is latency bound).
  constexpr int kInFlight = SLOTS > 0 ? SLOTS : ((64 / EPL) < 32 ? (64 / EPL) : 32);
  static_assert(sizeof(PO) == 4 || kInFlight >= 2, "mixed partials: slot 1 is the spare");
  // A slot past the partitions re-reads one already requested: partition 0, or for
  // mixed partials the first bf16 one (P >= 2 there), so that slot u >= 1 is bf16.
  constexpr int kSpare = sizeof(PO) == 2 ? 1 : 0;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  const float sig = sink ? sink[row % num_heads] * kLog2e : kNegInf;
  float M, lsum;

  if (P <= 64) {
    // (m_p, l_p) in lane p and the first kInFlight partial rows, requested
    // together (clamped indices, no branches around the loads)
    const int pc = lane < P ? lane : 0;
    const float lp_raw = part_l[(size_t)pc * rows + row];
    const float mp_raw = part_m[(size_t)pc * rows + row];
    MergeCols<EPL> c[kInFlight];
    c[0] = merge_part_cols<DV>(part_o, rows, row, 0, lane);
#pragma unroll
    for (int u = 1; u < kInFlight; ++u)
      c[u] = merge_part_cols<DV>(part_o, rows, row, u < P ? u : kSpare, lane);
    const float lp = lane < P ? lp_raw : 0.f;
    M = fmaxf(wave_max(lp > 0.f ? mp_raw * kLog2e : kNegInf), sig);
    const float Ms = (M == kNegInf) ? 0.f : M;
    const float w = lp > 0.f ? lp * fast_exp2(mp_raw * kLog2e - Ms) : 0.f;
    lsum = w;
    for (int j = 0; j < P; j += kInFlight) {
      if (j > 0) {  // more partitions than one group: the next group's rows
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
          c[u] = merge_part_cols<DV>(part_o, rows, row, j + u < P ? j + u : j, lane);
      }
      float wj[kInFlight];
#pragma unroll
      for (int u = 0; u < kInFlight; ++u)
        wj[u] = (j + u < P) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j + u))
                            : 0.f;
      merge_accumulate(acc, wj, c);
    }
  } else {
    // Longer splits: the row max over every chunk of 64 first, then per chunk the
    // weights and kInFlight partial rows at a time.  A slot past the end of the
    // chunk or of an empty partition re-reads the first row of its group (already
    // in flight), and its value is dropped.
    float mx = kNegInf;
    for (int pp = lane; pp < P; pp += 64) {
      const float lp = part_l[(size_t)pp * rows + row];
      if (lp > 0.f) mx = fmaxf(mx, part_m[(size_t)pp * rows + row] * kLog2e);
    }
    M = fmaxf(wave_max(mx), sig);
    const float Ms = (M == kNegInf) ? 0.f : M;
    lsum = 0.f;
    for (int base = 0; base < P; base += 64) {
      const int pp = base + lane;  // this lane's partition of the chunk and its weight
      float w = 0.f;
      if (pp < P) {
        const float lp = part_l[(size_t)pp * rows + row];
        if (lp > 0.f) w = lp * fast_exp2(part_m[(size_t)pp * rows + row] * kLog2e - Ms);
      }
      lsum += w;
      const int n = min(64, P - base);
      for (int j = 0; j < n; j += kInFlight) {
        float wj[kInFlight];
        MergeCols<EPL> c[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
          wj[u] = (j + u < n)
                      ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j + u))
                      : 0.f;
          const int src = base + j + (wj[u] != 0.f ? u : 0);
          c[u] = merge_part_cols<DV>(part_o, rows, row, src, lane);
        }
        merge_accumulate(acc, wj, c);
      }
    }
  }

  float L = wave_sum(lsum);
  const float Ms = (M == kNegInf) ? 0.f : M;
  if (sink) L += fast_exp2(sig - Ms);
  const bool any = L > 0.f;
  const float inv = any ? 1.f / L : 0.f;
  if constexpr (BF16OUT) {
    uint16_t* dst = (uint16_t*)out + (size_t)row * DV + lane * EPL;
    if constexpr (EPL == 1) {
      dst[0] = to_bf16(acc[0] * inv);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; e += 2)
        *(uint32_t*)(dst + e) = pack_bf16(acc[e] * inv, acc[e + 1] * inv);
    }
  } else {
    float* dst = (float*)out + (size_t)row * DV + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[e] = acc[e] * inv;
  }
  if (lse && lane == 0) lse[row] = any ? (M + fast_log2(L)) * kLn2 : kNegInf;
}

// Two waves per row for a row split into 33..64 partitions at DV <= 128: wave
// `half` takes partitions 32 half .. 32 half + 31, all requested at once (one
// memory round trip), and returns its own max Mh (log2 units, no sink), the sum
// of its weights lh = sum l_p 2^(m_p - Mh) and acc = sum l_p 2^(m_p - Mh) O_p
// (this lane's DV/64 columns).  An empty half returns Mh = -inf, lh = 0, acc = 0.
template <int DV>
__device__ __forceinline__ void merge_half(const float* __restrict__ part_o,
                                           const float* __restrict__ part_m,
                                           const float* __restrict__ part_l, int P, int rows,
                                           int row, int half, int lane,
                                           float (&acc)[DV / 64], float& Mh, float& lh) {
  constexpr int EPL = DV / 64;
  constexpr int N = 32;
  const int p0 = half * N;
  const int n = min(N, P - p0);  // >= 1 for both halves when 32 < P <= 64
  const float* orow = part_o + (size_t)row * DV + lane * EPL;
  const size_t pstride = (size_t)rows * DV;
  const int pc = p0 + (lane < n ? lane : 0);
  const float lp_raw = part_l[(size_t)pc * rows + row];
  const float mp_raw = part_m[(size_t)pc * rows + row];
  MergeCols<EPL> c[N];
#pragma unroll
  for (int u = 0; u < N; ++u)
    c[u] = merge_load_cols<EPL>(orow + (size_t)(p0 + (u < n ? u : 0)) * pstride);
  const float lp = lane < n ? lp_raw : 0.f;
  Mh = wave_max(lp > 0.f ? mp_raw * kLog2e : kNegInf);
  const float Ms = (Mh == kNegInf) ? 0.f : Mh;
  const float w = lp > 0.f ? lp * fast_exp2(mp_raw * kLog2e - Ms) : 0.f;
  lh = wave_sum(w);
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float wj[N];
#pragma unroll
  for (int u = 0; u < N; ++u)
    wj[u] = (u < n) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u)) : 0.f;
  merge_accumulate(acc, wj, c);
}

}  // namespace da
