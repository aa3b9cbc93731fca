// da_device.h -- small device helpers for the gfx950 decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "da_params.h"

namespace da {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---- bf16 <-> fp32 ------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---- cross-lane (DPP within rows of 16 lanes) -----------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each half row
constexpr int kDppRowRor8 = 0x128;    // lane i <- lane (i+8) mod 16 within each row

// Sum over aligned groups of 8 lanes; every lane of the group gets the total.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor(float x, int mask) { return __shfl_xor(x, mask, 64); }

// max(x, x of lane ^ 32) with v_permlane32_swap (a VALU op: no LDS round trip).
// The swap of (x, x) leaves the low half of x in both halves of one result and
// the high half in both halves of the other.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// max(x, x of lane ^ 16) with v_permlane16_swap (rows of 16 lanes swapped in pairs).
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element (i % 4) of the 8 bytes addressed by lane
// 4 j + i / 4, for j = 0..3.  So if lane s of the group addresses
// &X[k0 + s / 4][n0 + 4 (s % 4)] of a row-major bf16 matrix X, lane i receives
// the column X[k0 .. k0 + 3][n0 + i]: half of an MFMA operand whose k index runs
// down the rows of X.
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  typedef short s4_t __attribute__((ext_vector_type(4)));
  const s4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ bf16x8_t concat_bf16x8(uint2 lo, uint2 hi) {
  return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Eight e4m3 bytes (two dwords) -> eight bf16 (exact: every finite e4m3 value is a
// bf16 value; v_cvt_scalef32_pk_bf16_fp8 with scale 1).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  // whole 32-bit words only: element-wise access of the pairs is miscompiled
  return __builtin_bit_cast(bf16x8_t, make_uint4(__builtin_bit_cast(uint32_t, a),
                                                 __builtin_bit_cast(uint32_t, b),
                                                 __builtin_bit_cast(uint32_t, c),
                                                 __builtin_bit_cast(uint32_t, d)));
}

__device__ __forceinline__ int wave_id_uniform() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// A wave-uniform 64-bit value (an address or byte offset) pinned to scalar
// registers, so that a load can take it as its scalar base even where it reaches
// the load through a phi after a divergent branch.  The readfirstlane builtin
// returns int: each half goes back through uint32_t, or a low half with bit 31
// set would be sign-extended into the high half.
__device__ __forceinline__ uint64_t pin_uniform_u64(uint64_t x) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)x);
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

// Cache row of key 0 of sequence b in an unpaged cache: b * max_seq_len in the
// dense layout, kv_row_offsets[b] in the ragged KV layout.  The offset is read
// through the scalar cache (b is uniform, the offsets are constant during the
// call); its address is pinned to scalar registers first so that the read stays
// a scalar load wherever the compiler placed b.
__device__ __forceinline__ size_t seq_kv_row0(const DecodeParams& p, int b) {
  if (!p.kv_row_offsets) return (size_t)b * p.max_seq_len;
  const uint64_t a = pin_uniform_u64((uint64_t)(p.kv_row_offsets + b));
  return (size_t)*(const __attribute__((address_space(4))) uint32_t*)a;
}

// ---- online-softmax state merge (log2 domain) ----------------------------------
// Combines (mA, lA) with (mB, lB); returns the scale factors for A and B.
__device__ __forceinline__ void merge_factors(float mA, float mB, float& m, float& fa,
                                              float& fb) {
  m = fmaxf(mA, mB);
  float ms = (m == kNegInf) ? 0.f : m;
  fa = fast_exp2(mA - ms);
  fb = fast_exp2(mB - ms);
}

// ---- per-row key limits ----------------------------------------------------------
// Keys of sequence b visible to query token t.  b is uniform at every caller, and
// the count is read through the scalar cache (the array is constant during the
// call).  Read as an ordinary load inside a per-row branch it became a vector load
// whose vmcnt(0) wait also waited for the block's stores still in flight: on the
// work queue, the previous item's partial rows, at the start of every item.
__device__ __forceinline__ int visible_keys(const DecodeParams& p, int b, int t) {
  uint32_t raw = (uint32_t)p.max_seq_len;
  if (p.valid_length) {
    const uint64_t a = pin_uniform_u64((uint64_t)(p.valid_length + b));
    raw = *(const __attribute__((address_space(4))) uint32_t*)a;
  }
  int n;
  if (p.indices) {
    // sparse top-k counts (int32): a negative count is 0, one above the list
    // stride (max_seq_len here) is the stride
    const int c = (int)raw;
    n = c < 0 ? 0 : (c < p.max_seq_len ? c : p.max_seq_len);
  } else {
    // A length above max_seq_len counts as max_seq_len; compared as unsigned, so
    // that a length of 2^31 or more is a large count, not a negative one.
    n = raw < (uint32_t)p.max_seq_len ? (int)raw : p.max_seq_len;
  }
  if (p.causal) {
    int lim = n - seq_tokens(p, b) + t + 1;
    n = lim < n ? lim : n;
  }
  return n < 0 ? 0 : n;
}

// Element offset of key j's row (row width `width` elements, KV head g).
__device__ __forceinline__ size_t kv_row(const DecodeParams& p, int b, int j, int g, int width) {
  size_t row;
  if (p.page_table) {
    uint32_t phys = p.page_table[(size_t)b * p.max_pages + (j >> p.page_shift)];
    row = ((size_t)phys << p.page_shift) + (size_t)(j & ((1 << p.page_shift) - 1));
  } else {
    row = seq_kv_row0(p, b) + j;
  }
  return (row * p.num_kv_heads + g) * (size_t)width;
}

}  // namespace da
