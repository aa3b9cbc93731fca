// decode_stream_fp8.hip -- streaming split-K decode attention for GQA with an
// 8-bit e4m3 KV cache (gfx950): q and out in bf16, K and V one byte per element
// with per-tensor fp32 scales.
//
// The structure is that of the bf16 streaming kernel: one block of 4 waves per
// (partition, sequence, KV head, 16-row block), or persistent blocks on a work
// queue for ragged batches; each wave streams its own tiles from HBM straight
// into a private LDS ring (global_load_lds with the non-temporal hint) and keeps
// its own FA2 online-softmax state ("mha_decoding_single_batch_pipelined",
// description; "decoding_warp_split_k" in its Parameters), and the 4 states are
// merged by log-sum-exp at the end.  A tile is 32 keys here, so that a stage
// holds as many bytes as a 16-key bf16 stage; under the two-head fold of split
// calls it is 16 keys x 2 KV heads.
//
// The scales need no work per element: a key's real value is k_scale times
// its stored one, so q.k picks up k_scale, which the host folds into the
// softmax scale; every value carries v_scale, a common factor of the weighted
// sum, applied once when the output is written.  The 8-bit elements become
// bf16 exactly (every e4m3 value is a bf16 value) and the contractions run on
// the bf16 matrix cores with fp32 accumulation; the softmax weights stay bf16.
//
// Per 32-key tile and wave (rows padded to 16):
//   S^T[32 keys x 16 rows] = K . Q^T as two 16-key halves, D/32
//       v_mfma_f32_16x16x32_bf16 each.  A = 8 K bytes per lane (ds_read_b64),
//       converted to bf16 (v_cvt_scalef32_pk_bf16_fp8, scale 1); B = Q^T in
//       registers for the whole kernel.  Lane l holds row l % 16 and keys
//       4 G + r (first half) and 16 + 4 G + r (second half), G = l / 16.
//   O^T[D x 16 rows] += V^T . P^T, D/16 v_mfma_f32_16x16x32_bf16.  The k slots
//       of lane group G are keys {4G..4G+3, 16+4G..16+4G+3}, exactly the keys
//       of its score lanes, so P^T is the lane's own weights.  V^T comes from
//       one ds_read_b64_tr_b8 per depth tile: in a group of 16 lanes, lane i
//       receives byte i % 8 of the 8-byte rows addressed by lanes 2b + i / 8,
//       b = 0..7 (measured on this chip); lane 2b + h points at the 8 bytes
//       of key (slot b of G) at depth 16 dt + 8 h, so lane i gets depth
//       16 dt + i of the 8 keys of its slots.
//
// LDS stage: the tile's K rows then its V rows, row-major, 128 bytes per key,
// chunk c (16 bytes) of key k stored at chunk position c ^ swz(k) with
//   swz(k) = ((k >> 1) & 3) | ((((k >> 3) ^ (k >> 4)) & 1) << 2).
// On the 64-bank LDS a half-wave of 8-byte reads is conflict-free when its 32
// lanes cover every bank once: the score reads of 16 consecutive keys and the
// transposing reads of keys {4G.., 16+4G..} both map (k & 1, swz(k)) one to
// one, and the stage is still filled by whole rows (1 KB = 8 keys per load).
#include "da_stream.h"

namespace da {

namespace {

constexpr int kTK8 = 32;  // keys per tile
constexpr int kW8 = 4;    // waves per block

struct Fp8Cfg {
  static constexpr int D = 128;
  static constexpr int ROW = D;                   // bytes per key row of one head
  static constexpr int CH = ROW / 16;             // 16-byte chunks per row
  static constexpr int HALF = kTK8 * ROW;         // K (or V) bytes per tile: 4 KB
  static constexpr int STAGE = 2 * HALF;
  static constexpr int NI = HALF / 1024;          // 1 KB load instructions per half
  static constexpr int KEYS_PER_I = 1024 / ROW;   // rows per load instruction
  static constexpr int STAGES = 2;                // 16 KB ring per wave: two blocks per CU
  static constexpr int RING = STAGES * STAGE;
  static constexpr int KS = D / 32;               // depth steps of q.K^T
  static constexpr int DT = D / 16;               // 16-wide depth tiles of O
  static constexpr int MERGE = kW8 * 16 * (D + 3 + 3) * 4;
  static constexpr int SMEM = (kW8 * RING > MERGE) ? kW8 * RING : MERGE;
  static_assert(NI * 1024 == HALF, "a tile half must split into 1 KB loads");
  static_assert(2 * NI * (STAGES - 1) + NI <= 63, "vmcnt range");
};

__device__ __forceinline__ constexpr int swz8(int k) {
  return ((k >> 1) & 3) | ((((k >> 3) ^ (k >> 4)) & 1) << 2);
}

// Key of k slot b (0..7) of lane group G in the P.V contraction.
__device__ __forceinline__ constexpr int pv_key(int G, int b) {
  return b < 4 ? 4 * G + b : 16 + 4 * G + (b - 4);
}

__device__ __forceinline__ uint2 lds_read_tr8(const void* p) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) v2i*)(uint32_t)(uintptr_t)p);
  return make_uint2((uint32_t)t.x, (uint32_t)t.y);
}

// Requests the tile of keys [j0, j0 + 32 >> hb_shift) of KV heads g, g + 1, ...
// (2^hb_shift of them) into the LDS stage at `lds`: stage row r holds key
// j0 + (r >> hb_shift) of head g + (r & (2^hb_shift - 1)).  Keys at or past
// `kend` read the same chunk of the tile's first key instead (finite data,
// masked out of the softmax), so every tile costs exactly 2 NI loads.
__device__ __forceinline__ void fp8_issue(const DecodeParams& p, int b, int g, int j0, int kend,
                                          uint32_t lds, const uint32_t (&off)[Fp8Cfg::NI],
                                          int lane) {
  using C = Fp8Cfg;
  const size_t row0 = stream_row0(p, b, j0);
  const size_t head_off0 = (row0 * p.num_kv_heads + g) * (size_t)C::ROW;
  const size_t head_off = pin_uniform_u64(head_off0);
  const char* kb = (const char*)p.k + head_off;
  const char* vb = (const char*)p.v + head_off;
  const uint32_t rs = (uint32_t)p.num_kv_heads * C::ROW;
  const int nvalid = kend - j0;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // last reads of this stage done
  uint32_t o[C::NI];
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    o[i] = off[i];
    if (nvalid < (kTK8 >> p.hb_shift)) {
      const int key = (i * C::KEYS_PER_I + lane / C::CH) >> p.hb_shift;
      if (key >= nvalid) o[i] -= (uint32_t)key * rs;
    }
  }
#pragma unroll
  for (int i = 0; i < C::NI; ++i) dma16(kb, o[i], lds + i * 1024);
#pragma unroll
  for (int i = 0; i < C::NI; ++i) dma16(vb, o[i], lds + C::HALF + i * 1024);
}

struct Fp8State {
  f32x4_t acc[Fp8Cfg::DT];
  float m, lsum, lsr;  // running max (log2 units), exact and bf16-rounded weight sums
};

// One tile from the LDS stage `st`; `after` = this wave's tiles requested after
// it (still in flight).
__device__ __forceinline__ void fp8_tile(const char* st, const bf16x8_t (&qf)[Fp8Cfg::KS],
                                         Fp8State& s, int after, int j0, bool masked, int hi,
                                         float scale_log2, uint32_t kofs, uint32_t vofs,
                                         const int (&kkey)[8]) {
  using C = Fp8Cfg;
  wait_after<2 * C::NI, C::NI, C::STAGES - 1>(after);  // K half of this tile landed
  f32x4_t sc[2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    sc[kh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < C::KS; ++k) {
      // depth 32 k + 8 G.. of key 16 kh + l % 16: chunk 2 k + G / 2, byte 8 (G % 2);
      // swz8(key + 16) = swz8(key) ^ 4, so the second half XORs 64 bytes more
      const uint2 w = *(const uint2*)(st + kh * 16 * C::ROW + (kofs ^ (32u * k) ^ (64u * kh)));
      sc[kh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(w.x, w.y), qf[k], sc[kh],
                                                       0, 0, 0);
    }
  }
  float x[8];  // slot b: stage row pv_key(g16, b)
  float mx = kNegInf;
  const int lim = hi - j0;  // this row's visible keys from the tile's first key on
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    float v = sc[b >> 2][b & 3] * scale_log2;
    if (masked) v = (kkey[b] < lim) ? v : kNegInf;
    x[b] = v;
    mx = fmaxf(mx, v);
  }
  mx = max_xor16(mx);
  mx = max_xor32(mx);
  const float mn = fmaxf(s.m, mx);
  if (__builtin_amdgcn_ballot_w64(mn > s.m) != 0) {  // some row's max grew: rescale
    const float alpha = (mn == s.m) ? 1.f : fast_exp2(s.m - mn);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) s.acc[dt] *= alpha;
    s.lsum *= alpha;
    s.lsr *= alpha;
    s.m = mn;
  }
  const float ms = (s.m == kNegInf) ? 0.f : s.m;
  uint32_t w[4];
  float ps = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float p0 = fast_exp2(x[2 * q] - ms), p1 = fast_exp2(x[2 * q + 1] - ms);
    ps += p0 + p1;
    w[q] = pack_bf16(p0, p1);
    s.lsr = dot2_bf16(w[q], 0x3f803f80u, s.lsr);  // + both rounded weights
  }
  s.lsum += ps;
  const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
  wait_after<2 * C::NI, 0, C::STAGES - 1>(after);  // V half landed
  const char* vh = st + C::HALF;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    const uint2 av = lds_read_tr8(vh + (vofs ^ (16u * dt)));
    s.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(av.x, av.y), pb, s.acc[dt],
                                                        0, 0, 0);
  }
}

// One work item: rows rb*16.. of (sequence b, KV heads g .. g + 2^hb_shift - 1)
// over partition pidx; with hb_shift > 0 (then rb = 0) the 16 rows are 2^hb_shift
// slots of 16 >> hb_shift rows, slot s holding the fold of KV head g + s, and a
// score of a row against a stage row of another head is masked out.
template <bool EMPTY_EXIT>
__device__ __forceinline__ void fp8_item(const DecodeParams& p, char* smem, int b, int g,
                                         int pidx, int rb) {
  using C = Fp8Cfg;
  constexpr int D = C::D;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id_uniform();
  const int c16 = lane & 15, g16 = lane >> 4;
  const int hbs = p.hb_shift;
  const int kpt = kTK8 >> hbs;           // keys per tile
  const int rps = 4 - hbs;               // log2 of the rows per head slot

  const int nrows = seq_tokens(p, b) * p.group;  // this sequence's fold
  const size_t row0q = seq_row0(p, b);
  const int slot = c16 >> rps;
  const int rr = rb * 16 + (c16 & ((1 << rps) - 1));
  const bool row_ok = rr < nrows;
  const int tok = row_ok ? rr / p.group : 0;
  const int head = (g + slot) * p.group + (row_ok ? rr % p.group : 0);
  const int k_lo = pidx * p.keys_per_partition;
  const int lim = row_ok ? visible_keys(p, b, tok) : 0;
  const int hi = row_ok ? min(k_lo + p.keys_per_partition, lim) : k_lo;
  // Block-uniform key range: [k_lo, hmin) unmasked, [hmin, hmax) masked.
  int hmin, hmax;
  item_key_range(p, b, rb, rps, nrows, k_lo, hmin, hmax);
  if (EMPTY_EXIT && p.write_partials && hmax == k_lo) {  // no visible key (uniform)
    stream_store_empty<D>(p, b, g, pidx, rb);
    return;
  }

  // Q^T operand: k-slot (g16, j) of depth step s <-> depth 32 s + 8 g16 + j.
  bf16x8_t qf[C::KS];
  const uint16_t* qrow =
      (const uint16_t*)p.q + ((row0q + tok) * p.num_q_heads + head) * (size_t)D;
#pragma unroll
  for (int s = 0; s < C::KS; ++s)  // rows past the fold read row (b, 0, g * group): zeroed later
    qf[s] = *(const bf16x8_t*)(qrow + s * 32 + g16 * 8);

  Fp8State s;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) s.acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  s.m = kNegInf;
  s.lsum = 0.f;
  s.lsr = 0.f;

  // Load instruction i moves stage chunk 64 i + lane: chunk position lane % CH
  // of stage row r = i * KEYS_PER_I + lane / CH, holding its chunk
  // (lane % CH) ^ swz8(r); stage row r is key r >> hbs of head slot
  // r & (2^hbs - 1) (consecutive in the cache row).
  uint32_t off[C::NI];
  const uint32_t rs = (uint32_t)p.num_kv_heads * C::ROW;
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    const int r = i * C::KEYS_PER_I + lane / C::CH;
    off[i] = (uint32_t)(r >> hbs) * rs + (uint32_t)(r & ((1 << hbs) - 1)) * C::ROW +
             16u * (uint32_t)((lane % C::CH) ^ swz8(r));
  }
  // Key (from the tile's first) of the stage row of each weight slot; rows of
  // another head slot never pass the mask.
  int kkey[8];
#pragma unroll
  for (int bq = 0; bq < 8; ++bq) {
    const int r = pv_key(g16, bq);
    kkey[bq] = ((r & ((1 << hbs) - 1)) == slot) ? (r >> hbs) : 0x7fffffff;
  }
  // Score reads: key c16 of the first half, depth step k: chunk 2 k + g16 / 2
  // at kofs ^ 32 k (the second half adds 16 rows and XORs 64, see fp8_tile).
  const uint32_t kofs =
      c16 * C::ROW + ((16u * (uint32_t)((g16 >> 1) ^ swz8(c16))) | 8u * (g16 & 1));
  // Transposing V reads: lane 2 bb + hh of the group supplies key pv_key(g16, bb)
  // at depth 16 dt + 8 hh, i.e. chunk dt (XOR-ed at the call), byte 8 hh.
  const int bb = c16 >> 1, hh = c16 & 1;
  const int vkey = pv_key(g16, bb);
  const uint32_t vofs = vkey * C::ROW + 16u * (uint32_t)swz8(vkey) + 8u * hh;

  // Tiles below n_full are whole for every row; with several heads every tile is masked.
  const int n_full = (hbs > 0) ? 0 : (hmin - k_lo) / kpt;
  const int n_tot = (hmax - k_lo + kpt - 1) / kpt;
  const int my_cnt = (n_tot > wave) ? (n_tot - wave + kW8 - 1) / kW8 : 0;
  char* ring = smem + wave * C::RING;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  if (my_cnt > 0) {
    fp8_issue(p, b, g, k_lo + wave * kpt, hmax, ring_lds, off, lane);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): Q and the first tile
    asm volatile("" ::: "memory");
#pragma unroll
    for (int s2 = 0; s2 < C::KS; ++s2) qf[s2] = row_ok ? qf[s2] : bf16x8_t{};
    const int pro = min(C::STAGES - 1, my_cnt);
    for (int i = 1; i < pro; ++i)
      fp8_issue(p, b, g, k_lo + (wave + kW8 * i) * kpt, hmax, ring_lds + i * C::STAGE, off,
                lane);
    int cur = 0;
    for (int i = 0; i < my_cnt; ++i) {
      const int nxt = i + C::STAGES - 1;
      if (nxt < my_cnt) {  // into the stage read one tile ago
        const int sn = (cur == 0) ? C::STAGES - 1 : cur - 1;
        fp8_issue(p, b, g, k_lo + (wave + kW8 * nxt) * kpt, hmax, ring_lds + sn * C::STAGE,
                  off, lane);
      }
      const int t = wave + kW8 * i;
      fp8_tile(ring + cur * C::STAGE, qf, s, my_cnt - 1 - i, k_lo + t * kpt, t >= n_full, hi,
               p.scale_log2, kofs, vofs, kkey);
      cur = (cur + 1 == C::STAGES) ? 0 : cur + 1;
    }
  }

  float lsum = s.lsum, lsr = s.lsr;
  lsum += shfl_xor(lsum, 16);
  lsum += shfl_xor(lsum, 32);
  lsr += shfl_xor(lsr, 16);
  lsr += shfl_xor(lsr, 32);

  // Merge the 4 waves through LDS (reusing the rings: every wave's loads have
  // completed, its last tile waited for vmcnt 0).
  __syncthreads();
  float* so = (float*)smem;  // [wave][row][D + 3]
  float* sm = so + kW8 * 16 * (D + 3);
  float* sl = sm + kW8 * 16;
  float* sr = sl + kW8 * 16;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      so[(wave * 16 + c16) * (D + 3) + dt * 16 + g16 * 4 + j] = s.acc[dt][j];
  if (g16 == 0) {
    sm[wave * 16 + c16] = s.m;
    sl[wave * 16 + c16] = lsum;
    sr[wave * 16 + c16] = lsr;
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < 16 * D; idx += blockDim.x) {
    const int r = idx / D;
    const int d = idx % D;
    const int rrow = rb * 16 + (r & ((1 << rps) - 1));
    if (rrow >= nrows) continue;
    const int tt = rrow / p.group;
    const int h = (g + (r >> rps)) * p.group + rrow % p.group;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kW8; ++w) M = fmaxf(M, sm[w * 16 + r]);
    const float Ms = (M == kNegInf) ? 0.f : M;
    float L = 0.f, Lr = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kW8; ++w) {
      const float f = fast_exp2(sm[w * 16 + r] - Ms);
      L += f * sl[w * 16 + r];
      Lr += f * sr[w * 16 + r];
      O += f * so[(w * 16 + r) * (D + 3) + d];
    }
    O *= p.v_scale;
    const size_t row = (row0q + tt) * p.num_q_heads + h;
    if (p.write_partials) {
      const size_t prow = (size_t)pidx * (size_t)p.rows_total + row;
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

// Static mapping or work queue, as in the bf16 streaming kernel.
__global__ __launch_bounds__(256) void decode_stream_fp8_kernel(DecodeParams p) {
  using C = Fp8Cfg;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
  __shared__ int s_next[2];
  const int n_hg = p.num_kv_heads >> p.hb_shift;  // KV head groups
  const int n_work = p.num_partitions * p.batch * n_hg;
  if (p.queue == nullptr) {
    const int id = blockIdx.x;
    const int xcd = id & 7;
    const int rq = id >> 3;
    const int rb = rq % p.row_blocks;
    int work = (rq / p.row_blocks) * 8 + xcd;
    if (work >= n_work) return;  // padding block: no barrier reached yet
    const int g = (work % n_hg) << p.hb_shift;
    work /= n_hg;
    fp8_item<false>(p, smem, work % p.batch, g, work / p.batch, rb);
    return;
  }
  for (int it = 0;; ++it) {
    if (threadIdx.x == 0) s_next[it & 1] = (int)(uint32_t)atomicAdd(p.queue, 1ull);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_next[it & 1]);
    if (item >= n_work) break;
    int w = item;
    const int g = (w % n_hg) << p.hb_shift;
    w /= n_hg;
    fp8_item<true>(p, smem, w % p.batch, g, w / p.batch, 0);
    __syncthreads();  // the LDS is free again
  }
  if (threadIdx.x == 0) {
    const unsigned long long old = atomicAdd(p.queue, 1ull << 32);
    if ((uint32_t)(old >> 32) == gridDim.x - 1) atomicExch(p.queue, 0ull);
  }
}

}  // namespace

int stream_fp8_step_keys() { return kTK8; }

hipError_t launch_decode_stream_fp8(const DecodeParams& p, hipStream_t s) {
  if (p.depth != 128) return hipErrorInvalidValue;
  if (p.hb_shift < 0 || p.hb_shift > 1 || (p.num_kv_heads & ((1 << p.hb_shift) - 1)) != 0 ||
      (p.hb_shift > 0 && (p.row_blocks != 1 || (fold_rows(p) << p.hb_shift) > 16)))
    return hipErrorInvalidValue;
  const int n_work = p.num_partitions * p.batch * (p.num_kv_heads >> p.hb_shift);
  int grid = ((n_work + 7) / 8) * 8 * p.row_blocks;
  if (p.queue) {
    if (p.row_blocks != 1 || p.queue_blocks < 1) return hipErrorInvalidValue;
    grid = n_work < p.queue_blocks ? n_work : p.queue_blocks;
  }
  hipLaunchKernelGGL(decode_stream_fp8_kernel, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace da
