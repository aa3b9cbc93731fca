// mla_mfma.hip -- matrix-core MLA decode for gfx950 ("flare_mla_decoding_dispatch").
//
// One KV head (kv_num_heads must be 1), depth 576 for q.K^T and V = K[..., :512]
// read from the same cache rows ("V is derived as K[:, :, :depth_v], so V is not
// loaded separately").  The q_len tokens of a sequence and its num_q_heads heads
// are folded into one set of T*H rows (the MTP token fold); a block owns 128 of
// those rows (8 waves x 16 rows) and one partition of the keys, so every cache row
// of the partition is read from HBM once per 128 rows.
//
// Per 32-key tile, shared by the block through LDS (double buffered, filled by
// all 512 threads with 16-byte loads):
//   S^T[32 keys x 16 rows] = K[32 x 576] . Q^T[576 x 16]     18 MFMAs per 16 keys
//       A = K from LDS (16-byte reads, padded rows), B = this wave's Q^T kept
//       in registers for the whole kernel.
//   online softmax on the accumulator layout (lane l owns row l % 16); the
//       running max is updated lazily: O and l are rescaled only when a row's
//       tile max exceeds the reference max by more than 2^8, which keeps every
//       exp2 argument <= 8 and the fp32 sums far from overflow.
//   O^T[512 x 16 rows] += V^T[512 x 32 keys] . P^T[32 x 16]  32 MFMAs
//       A = V^T read by column from the same LDS tile, B = P^T straight from the
//       S^T accumulators (bf16).
// With two tokens (256 rows) a sequence needs two blocks that read the same
// tiles; their block ids differ by a multiple of 8 so that both land on the same
// XCD and the second read of each tile is served by that XCD's L2.
#include "da_device.h"

namespace da {

namespace {

constexpr int kD = 576;
constexpr int kDv = 512;
constexpr int kBN = 32;
constexpr int kWaves = 8;
constexpr int kRows = 16 * kWaves;           // rows per block
constexpr int kThreads = 64 * kWaves;
constexpr int kKS = kD / 32;                 // 18 depth steps
constexpr int kDT = kDv / 16;                // 32 output depth tiles
constexpr int kRowBytes = kD * 2;            // 1152
constexpr int kPitch = kRowBytes + 16;       // LDS row pitch (bank spread)
constexpr int kTileBytes = kBN * kPitch;
constexpr int kChunksPerRow = kRowBytes / 16;   // 72
constexpr int kChunks = kBN * kChunksPerRow;    // 2304
constexpr int kLoads = (kChunks + kThreads - 1) / kThreads;  // 5
constexpr float kLazy = 8.0f;                // rescale threshold (log2 units)

struct Stage {
  uint4 v[kLoads];
};

__device__ __forceinline__ void mla_load(const DecodeParams& p, Stage& st, int b, int j0,
                                         int kend) {
  const int tid = threadIdx.x;
  if (j0 >= kend) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) st.v[i] = make_uint4(0, 0, 0, 0);
    return;
  }
  size_t row0;
  if (p.page_table) {
    const uint32_t phys = p.page_table[(size_t)b * p.max_pages + (j0 >> p.page_shift)];
    row0 = ((size_t)phys << p.page_shift) + (size_t)(j0 & ((1 << p.page_shift) - 1));
  } else {
    row0 = (size_t)b * p.max_seq_len + j0;
  }
  const char* base = (const char*)p.k + row0 * kRowBytes;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int c = tid + i * kThreads;
    const int key = c / kChunksPerRow;
    const int col = c % kChunksPerRow;
    if (c < kChunks && j0 + key < kend)
      st.v[i] = *(const uint4*)(base + (size_t)key * kRowBytes + col * 16);
    else
      st.v[i] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void mla_store(const Stage& st, char* buf) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int c = tid + i * kThreads;
    if (c < kChunks) {
      const int key = c / kChunksPerRow;
      const int col = c % kChunksPerRow;
      *(uint4*)(buf + key * kPitch + col * 16) = st.v[i];
    }
  }
}

template <bool MASKED>
__device__ __forceinline__ void mla_tile(const char* buf, const bf16x8_t (&qf)[kKS],
                                         f32x4_t (&acc)[kDT], float& m, float& lsum, int j0,
                                         int hi, float scale_log2) {
  const int lane = threadIdx.x & 63;
  const int c16 = lane & 15, g16 = lane >> 4;
  f32x4_t s[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const char* krow = buf + (kt * 16 + c16) * kPitch + g16 * 16;
#pragma unroll
    for (int st = 0; st < kKS; ++st) {
      const bf16x8_t a = *(const bf16x8_t*)(krow + st * 64);
      s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[st], s[kt], 0, 0, 0);
    }
  }
  float x[2][4];
  float mx = kNegInf;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = s[kt][j] * scale_log2;
      if (MASKED) v = (j0 + kt * 16 + g16 * 4 + j < hi) ? v : kNegInf;
      x[kt][j] = v;
      mx = fmaxf(mx, v);
    }
  mx = fmaxf(mx, shfl_xor(mx, 16));
  mx = fmaxf(mx, shfl_xor(mx, 32));
  // Lazy rescale: move the reference max only when the tile exceeds it by > kLazy.
  if (mx > m + kLazy) {
    const float mn = mx;
    const float alpha = fast_exp2(m - mn);  // m = -inf on the first tile -> 0
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) acc[dt] *= alpha;
    m = mn;
  }
  const float ms = (m == kNegInf) ? 0.f : m;
  float pr[2][4];
  float ps = 0.f;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pr[kt][j] = fast_exp2(x[kt][j] - ms);
      ps += pr[kt][j];
    }
  lsum += ps;
  const uint4 pbu = make_uint4(pack_bf16(pr[0][0], pr[0][1]), pack_bf16(pr[0][2], pr[0][3]),
                               pack_bf16(pr[1][0], pr[1][1]), pack_bf16(pr[1][2], pr[1][3]));
  const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pbu);
  // V^T operand: k-slot (g16, j) <-> key j<4 ? 4*g16+j : 16+4*g16+(j-4); column d.
  const char* r0 = buf + (4 * g16) * kPitch + c16 * 2;
  const char* r1 = buf + (16 + 4 * g16) * kPitch + c16 * 2;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      e[j] = *(const uint16_t*)(r0 + j * kPitch + dt * 32);
      e[4 + j] = *(const uint16_t*)(r1 + j * kPitch + dt * 32);
    }
    const uint4 au = make_uint4(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16),
                                e[4] | ((uint32_t)e[5] << 16), e[6] | ((uint32_t)e[7] << 16));
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, au), pb,
                                                      acc[dt], 0, 0, 0);
  }
}

__global__ __launch_bounds__(kThreads) void mla_decode_kernel(DecodeParams p, int n_mblocks,
                                                              int n_work) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kTileBytes];
  // XCD-aware decode of the block id: blocks i and i + 8 share an XCD; the
  // n_mblocks row blocks of one (partition, sequence) get ids 8 apart.
  const int id = blockIdx.x;
  const int xcd = id & 7;
  const int r = id >> 3;
  const int mb = r % n_mblocks;
  const int work = (r / n_mblocks) * 8 + xcd;
  if (work >= n_work) return;  // padding block: leaves before any barrier
  const int b = work % p.batch;
  const int pidx = work / p.batch;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c16 = lane & 15, g16 = lane >> 4;
  const int H = p.num_q_heads;
  const int nrows = p.q_len * H;

  const int rr = mb * kRows + wave * 16 + c16;
  const bool row_ok = rr < nrows;
  const int tok = row_ok ? rr / H : 0;
  const int head = row_ok ? rr % H : 0;
  const int k_lo = pidx * p.keys_per_partition;
  const int k_end = k_lo + p.keys_per_partition;
  const int hi = row_ok ? min(k_end, visible_keys(p, b, tok)) : k_lo;
  // Visibility grows with the token index: the block's extremes come from its
  // first and last token.
  const int t_first = (mb * kRows) / H;
  const int t_last = (min(nrows, (mb + 1) * kRows) - 1) / H;
  const int hmin = max(k_lo, min(k_end, visible_keys(p, b, t_first)));
  const int hmax = max(k_lo, min(k_end, visible_keys(p, b, t_last)));

  bf16x8_t qf[kKS];
  const uint16_t* qrow =
      (const uint16_t*)p.q + (((size_t)b * p.q_len + tok) * H + head) * (size_t)kD;
#pragma unroll
  for (int s = 0; s < kKS; ++s)
    qf[s] = row_ok ? *(const bf16x8_t*)(qrow + s * 32 + g16 * 8) : bf16x8_t{};

  f32x4_t acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, lsum = 0.f;

  const int n_full = (hmin - k_lo) / kBN;
  const int n_tot = (hmax - k_lo + kBN - 1) / kBN;
  if (n_tot > 0) {
    Stage st;
    mla_load(p, st, b, k_lo, hmax);
    mla_store(st, smem);
    if (n_tot > 1) mla_load(p, st, b, k_lo + kBN, hmax);
    __syncthreads();
    for (int i = 0; i < n_tot; ++i) {
      const char* cur = smem + (i & 1) * kTileBytes;
      const int j0 = k_lo + i * kBN;
      if (i < n_full)
        mla_tile<false>(cur, qf, acc, m, lsum, j0, hi, p.scale_log2);
      else
        mla_tile<true>(cur, qf, acc, m, lsum, j0, hi, p.scale_log2);
      if (i + 1 < n_tot) {
        mla_store(st, smem + ((i + 1) & 1) * kTileBytes);
        if (i + 2 < n_tot) mla_load(p, st, b, k_lo + (i + 2) * kBN, hmax);
      }
      __syncthreads();
    }
  }

  lsum += shfl_xor(lsum, 16);
  lsum += shfl_xor(lsum, 32);
  if (!row_ok) return;
  const size_t row = ((size_t)b * p.q_len + tok) * H + head;
  if (p.write_partials) {
    const size_t prow = (size_t)pidx * ((size_t)p.batch * nrows) + row;
    const bool any = lsum > 0.f;
    const float inv = any ? 1.f / lsum : 0.f;
    float* dst = p.part_o + prow * kDv;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
      *(float4*)(dst + dt * 16 + g16 * 4) =
          make_float4(acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv, acc[dt][3] * inv);
    if (g16 == 0) {
      p.part_m[prow] = any ? m * kLn2 : kNegInf;
      p.part_l[prow] = lsum;
    }
  } else {
    float M = m, L = lsum, c = 1.f;
    if (p.sink) {
      const float sig = p.sink[head] * kLog2e;
      const float M2 = fmaxf(M, sig);
      c = fast_exp2(M - M2);
      L = L * c + fast_exp2(sig - M2);
      M = M2;
    }
    const bool any = L > 0.f;
    const float inv = any ? c / L : 0.f;
    uint16_t* dst = (uint16_t*)p.out + row * kDv;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
      *(uint2*)(dst + dt * 16 + g16 * 4) =
          make_uint2(pack_bf16(acc[dt][0] * inv, acc[dt][1] * inv),
                     pack_bf16(acc[dt][2] * inv, acc[dt][3] * inv));
    if (g16 == 0 && p.lse) p.lse[row] = any ? (M + fast_log2(L)) * kLn2 : kNegInf;
  }
}

}  // namespace

int mla_rows_per_block(int, int) { return kRows; }
int mla_step_keys(int) { return kBN; }

hipError_t launch_mla(const DecodeParams& p, hipStream_t s) {
  const int n_mblocks = p.row_blocks;
  const int n_work = p.num_partitions * p.batch;
  const int grid = ((n_work + 7) / 8) * 8 * n_mblocks;
  hipLaunchKernelGGL(mla_decode_kernel, dim3(grid), dim3(kThreads), 0, s, p, n_mblocks, n_work);
  return hipGetLastError();
}

}  // namespace da
