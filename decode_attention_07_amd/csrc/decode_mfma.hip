// decode_mfma.hip -- matrix-core split-K decode attention for wide head folds (gfx950).
//
// Used for bf16 when 8 or more query rows share a KV head (GQA groups of 8+,
// or multi-token folds): the block's rows form a 16-row matrix, so q.K^T and
// P.V are dense contractions for v_mfma_f32_16x16x32_bf16.  One block of 4 waves
// handles one (partition, batch, KV head, 16-row block); each KV byte of the
// partition is read from HBM once.
//
// FA2 online softmax per wave ("mha_decoding_single_batch_pipelined",
// description; "decoding_warp_split_k" in its Parameters): the 4 waves of a block
// take interleaved 32-key tiles of the partition and keep their own running
// (m, l, O); the block merges them by log-sum-exp at the end.
//
// Per 32-key tile and wave:
//   S^T[32 keys x 16 rows] = K[32 x D] . Q^T[D x 16]        (2 x D/32 MFMAs)
//       A = K straight from HBM: lane l holds 8 depth values of key (l % 16);
//       B = Q^T held in registers for the whole kernel.
//   online softmax on the accumulator layout: lane l owns query row (l % 16) and
//       8 of the tile's keys, so max/sum need only two cross-row shuffles and
//       the rescale of O is lane-local.
//   O^T[D x 16 rows] += V^T[D x 32 keys] . P^T[32 x 16]      (D/16 MFMAs)
//       B = P^T is the S^T accumulator of this lane converted to bf16, with no
//       data movement; A = V^T needs V transposed, so the V tile goes through a
//       wave-private LDS buffer (row-major, padded) and is read back by column.
// The next tile's K and V loads are issued before the current tile is
// processed (register double buffering).
#include "da_device.h"

namespace da {

namespace {

constexpr int kTile = 32;   // keys per wave tile
constexpr int kWaves = 4;

template <int D>
struct MfmaCfg {
  static constexpr int KS = D / 32;                 // depth steps of q.K^T
  static constexpr int DT = D / 16;                 // 16-wide depth tiles of O
  static constexpr int CHUNKS = D * 2 / 16;         // 16-byte chunks per key row
  static constexpr int VLOADS = kTile * CHUNKS / 64;  // 16-byte V loads per lane per tile
  static constexpr int KEYS_PER_VLOAD = 64 / CHUNKS;
  // LDS bytes per V row: 32 bytes past a multiple of 128, so the 4 rows x 32
  // bytes that one 16-lane transposing read touches fall in different banks
  static constexpr int PITCH = D * 2 + 32;
  static constexpr int VBUF = kTile * PITCH;        // LDS bytes per wave tile
  static constexpr int MERGE = kWaves * 16 * (D + 3) * 4;
  static constexpr int SMEM = (kWaves * VBUF > MERGE) ? kWaves * VBUF : MERGE;
};

template <int D>
struct MfmaTile {
  bf16x8_t k[2][MfmaCfg<D>::KS];
  uint4 v[MfmaCfg<D>::VLOADS];
};

// First cache row of the tile starting at key j0 (32 keys inside one page).
__device__ __forceinline__ size_t tile_row0(const DecodeParams& p, int b, int j0) {
  if (p.page_table) {
    const uint32_t phys = p.page_table[(size_t)b * p.max_pages + (j0 >> p.page_shift)];
    return ((size_t)phys << p.page_shift) + (size_t)(j0 & ((1 << p.page_shift) - 1));
  }
  return (size_t)b * p.max_seq_len + j0;
}

template <int D, bool MASKED>
__device__ __forceinline__ void mfma_load(const DecodeParams& p, MfmaTile<D>& t, int b, int g,
                                          int j0, int lane, int kend) {
  using C = MfmaCfg<D>;
  const int c16 = lane & 15, g16 = lane >> 4;
  if (MASKED && j0 >= kend) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s = 0; s < C::KS; ++s) t.k[kt][s] = bf16x8_t{};
#pragma unroll
    for (int i = 0; i < C::VLOADS; ++i) t.v[i] = make_uint4(0, 0, 0, 0);
    return;
  }
  const size_t row0 = tile_row0(p, b, j0);
  const size_t stride = (size_t)p.num_kv_heads * D;  // elements between keys
  const uint16_t* kb = (const uint16_t*)p.k + (row0 * p.num_kv_heads + g) * (size_t)D;
  const uint16_t* vb = (const uint16_t*)p.v + (row0 * p.num_kv_heads + g) * (size_t)D;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = kt * 16 + c16;
    const bool ok = !MASKED || (j0 + key < kend);
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      if (ok)
        t.k[kt][s] = *(const bf16x8_t*)(kb + key * stride + s * 32 + g16 * 8);
      else
        t.k[kt][s] = bf16x8_t{};
    }
  }
#pragma unroll
  for (int i = 0; i < C::VLOADS; ++i) {
    const int key = i * C::KEYS_PER_VLOAD + lane / C::CHUNKS;
    const int chunk = lane % C::CHUNKS;
    if (!MASKED || (j0 + key < kend))
      t.v[i] = *(const uint4*)(vb + key * stride + chunk * 8);
    else
      t.v[i] = make_uint4(0, 0, 0, 0);
  }
}

template <int D, bool MASKED>
__device__ __forceinline__ void mfma_process(const MfmaTile<D>& t, const bf16x8_t (&qf)[MfmaCfg<D>::KS],
                                             f32x4_t (&acc)[MfmaCfg<D>::DT], float& m,
                                             float& lsum, float& lsr, char* vl, int j0,
                                             int lane, int hi,
                                             float scale_log2) {
  using C = MfmaCfg<D>;
  const int c16 = lane & 15, g16 = lane >> 4;
  // V tile -> wave-private LDS, row-major with padded pitch.
#pragma unroll
  for (int i = 0; i < C::VLOADS; ++i) {
    const int key = i * C::KEYS_PER_VLOAD + lane / C::CHUNKS;
    const int chunk = lane % C::CHUNKS;
    *(uint4*)(vl + key * C::PITCH + chunk * 16) = t.v[i];
  }
  // S^T = K . Q^T for the two 16-key halves.
  f32x4_t s[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < C::KS; ++st)
      s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[kt][st], qf[st], s[kt], 0, 0, 0);
  }
  // Scale to log2 units, mask, tile max of this lane's row.
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
  const float mn = fmaxf(m, mx);
  const float ms = (mn == kNegInf) ? 0.f : mn;
  const float alpha = fast_exp2(m - ms);
  m = mn;
  float pr[2][4];
  float ps = 0.f;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pr[kt][j] = fast_exp2(x[kt][j] - ms);
      ps += pr[kt][j];
    }
  lsum = lsum * alpha + ps;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) acc[dt] *= alpha;
  // P^T operand: k-slot (g16, j) holds key j<4 ? 4*g16+j : 16+4*g16+(j-4).
  // The weights enter the MFMA rounded to bf16; O is normalised by their rounded
  // sum (lsr) so that the effective weights sum to one.
  const uint32_t pb0 = pack_bf16(pr[0][0], pr[0][1]);
  const uint32_t pb1 = pack_bf16(pr[0][2], pr[0][3]);
  const uint32_t pb2 = pack_bf16(pr[1][0], pr[1][1]);
  const uint32_t pb3 = pack_bf16(pr[1][2], pr[1][3]);
  lsr = lsr * alpha + ((bf16lo(pb0) + bf16hi(pb0)) + (bf16lo(pb1) + bf16hi(pb1)) +
                       (bf16lo(pb2) + bf16hi(pb2)) + (bf16lo(pb3) + bf16hi(pb3)));
  const uint4 pbu = make_uint4(pb0, pb1, pb2, pb3);
  const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pbu);
  // O^T += V^T . P^T.  V^T operand of depth tile dt: slots 0..3 hold keys
  // 4 g16 + 0..3, slots 4..7 keys 16 + 4 g16 + 0..3 (the P^T slot order), at
  // d = 16 dt + c16.  Each half is one transposing read: lane c16 supplies
  // &V[4 g16 + c16 / 4][16 dt + 4 (c16 % 4)] (row-major tile, padded pitch).
  const char* vt = vl + (4 * g16 + (c16 >> 2)) * C::PITCH + (c16 & 3) * 8;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    const char* a = vt + dt * 32;
    const bf16x8_t av = concat_bf16x8(lds_read_tr16(a), lds_read_tr16(a + 16 * C::PITCH));
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, acc[dt], 0, 0, 0);
  }
}

template <int D>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeParams p) {
  using C = MfmaCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id_uniform();
  const int c16 = lane & 15, g16 = lane >> 4;

  int id = blockIdx.x;
  const int rb = id % p.row_blocks; id /= p.row_blocks;
  const int g = id % p.num_kv_heads; id /= p.num_kv_heads;
  const int b = id % p.batch; id /= p.batch;
  const int pidx = id;

  // This lane's query row (16 rows per block: rows of the token-major fold).
  const int nrows = fold_rows(p);
  const int rr = rb * 16 + c16;
  const bool row_ok = rr < nrows;
  const int tok = row_ok ? rr / p.group : 0;
  const int head = g * p.group + (row_ok ? rr % p.group : 0);
  const int k_lo = pidx * p.keys_per_partition;
  const int lim = row_ok ? visible_keys(p, b, tok) : 0;
  const int hi = row_ok ? min(k_lo + p.keys_per_partition, lim) : k_lo;
  // Block-uniform key range: [k_lo, hmin) unmasked, [hmin, hmax) masked.
  int hmin_l = row_ok ? hi : 0x7fffffff, hmax_l = hi;
#pragma unroll
  for (int x = 1; x < 16; x <<= 1) {
    hmin_l = min(hmin_l, __shfl_xor(hmin_l, x, 64));
    hmax_l = max(hmax_l, __shfl_xor(hmax_l, x, 64));
  }
  const int hmin = max(k_lo, __builtin_amdgcn_readfirstlane(hmin_l));
  const int hmax = max(k_lo, __builtin_amdgcn_readfirstlane(hmax_l));

  // Q^T operand, k-slot (g16, j) <-> depth 32*s + 8*g16 + j (same order as K).
  bf16x8_t qf[C::KS];
  const uint16_t* qrow =
      (const uint16_t*)p.q + (((size_t)b * p.q_len + tok) * p.num_q_heads + head) * (size_t)D;
#pragma unroll
  for (int s = 0; s < C::KS; ++s)
    qf[s] = row_ok ? *(const bf16x8_t*)(qrow + s * 32 + g16 * 8) : bf16x8_t{};

  f32x4_t acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, lsum = 0.f, lsr = 0.f;  // exact and bf16-rounded weight sums
  char* vl = smem + wave * C::VBUF;

  const int n_full = (hmin - k_lo) / kTile;
  const int n_tot = (hmax - k_lo + kTile - 1) / kTile;
  int t = wave;
  if (t < n_full) {
    MfmaTile<D> ta, tb;
    mfma_load<D, false>(p, ta, b, g, k_lo + t * kTile, lane, 0);
    for (;;) {
      const bool more = t + kWaves < n_full;
      if (more) mfma_load<D, false>(p, tb, b, g, k_lo + (t + kWaves) * kTile, lane, 0);
      mfma_process<D, false>(ta, qf, acc, m, lsum, lsr, vl, k_lo + t * kTile, lane, hi,
                             p.scale_log2);
      t += kWaves;
      if (!more) break;
      const bool more2 = t + kWaves < n_full;
      if (more2) mfma_load<D, false>(p, ta, b, g, k_lo + (t + kWaves) * kTile, lane, 0);
      mfma_process<D, false>(tb, qf, acc, m, lsum, lsr, vl, k_lo + t * kTile, lane, hi,
                             p.scale_log2);
      t += kWaves;
      if (!more2) break;
    }
  }
  for (; t < n_tot; t += kWaves) {
    MfmaTile<D> tt;
    mfma_load<D, true>(p, tt, b, g, k_lo + t * kTile, lane, hmax);
    mfma_process<D, true>(tt, qf, acc, m, lsum, lsr, vl, k_lo + t * kTile, lane, hi, p.scale_log2);
  }

  // Row exp-sum across the 4 lane groups.
  lsum += shfl_xor(lsum, 16);
  lsum += shfl_xor(lsum, 32);
  lsr += shfl_xor(lsr, 16);
  lsr += shfl_xor(lsr, 32);

  // Merge the 4 waves through LDS (reusing the V buffers).
  __syncthreads();
  float* so = (float*)smem;                       // [wave][row][D]
  float* sm = so + kWaves * 16 * D;               // [wave][row]
  float* sl = sm + kWaves * 16;                   // [wave][row]
  float* sr = sl + kWaves * 16;                   // [wave][row]
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) so[(wave * 16 + c16) * D + dt * 16 + g16 * 4 + j] = acc[dt][j];
  if (g16 == 0) {
    sm[wave * 16 + c16] = m;
    sl[wave * 16 + c16] = lsum;
    sr[wave * 16 + c16] = lsr;
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < 16 * D; idx += blockDim.x) {
    const int r = idx / D;
    const int d = idx % D;
    const int rrow = rb * 16 + r;
    if (rrow >= nrows) continue;
    const int tt_ = rrow / p.group;
    const int h = g * p.group + rrow % p.group;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm[w * 16 + r]);
    const float Ms = (M == kNegInf) ? 0.f : M;
    float L = 0.f, Lr = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(sm[w * 16 + r] - Ms);
      L += f * sl[w * 16 + r];
      Lr += f * sr[w * 16 + r];
      O += f * so[(w * 16 + r) * D + d];
    }
    const size_t row = ((size_t)b * p.q_len + tt_) * p.num_q_heads + h;
    if (p.write_partials) {
      const size_t prow = (size_t)pidx * ((size_t)p.batch * p.q_len * p.num_q_heads) + row;
      const bool any = L > 0.f;
      p.part_o[prow * D + d] = any ? O / Lr : 0.f;
      if (d == 0) {
        p.part_m[prow] = any ? M * kLn2 : kNegInf;
        p.part_l[prow] = L;
      }
    } else {
      if (p.sink) {
        const float sig = p.sink[h] * kLog2e;
        const float M2 = fmaxf(M, sig);
        const float c = fast_exp2(M - M2);
        const float e = fast_exp2(sig - M2);
        L = L * c + e;
        Lr = Lr * c + e;
        O *= c;
        M = M2;
      }
      const bool any = L > 0.f;
      ((uint16_t*)p.out)[row * D + d] = to_bf16(any ? O / Lr : 0.f);
      if (d == 0 && p.lse) p.lse[row] = any ? (M + fast_log2(L)) * kLn2 : kNegInf;
    }
  }
}

}  // namespace

int mfma_rows_per_block() { return 16; }
int mfma_step_keys() { return kTile; }

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t s) {
  const int grid = p.num_partitions * p.batch * p.num_kv_heads * p.row_blocks;
  if (p.depth == 64)
    hipLaunchKernelGGL(decode_mfma_kernel<64>, dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(decode_mfma_kernel<128>, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace da
