// decode_stream.hip -- streaming matrix-core split-K decode attention for bf16 GQA (gfx950).
//
// Handles every bf16 head fold (one to sixteen query rows share a KV head per
// row block; wider folds take several row blocks).  Single-query decode moves
// each KV byte once and does little arithmetic on it, so the kernel is built
// to stream: each wave moves its own 16-key tiles from HBM straight into a
// private ring of LDS stages (global_load_lds with the non-temporal hint, no
// staging registers, no block barriers), the next tile in flight while it works
// on the current one.  Under the static mapping a block takes 64 KB of LDS, so
// two blocks share a CU and one block's start-up latency hides behind the other's
// stream; work-queue blocks run one per CU with a 3-stage ring (96 KB), which
// streams ragged batches faster.
//
// One block of 4 waves handles one (partition, sequence, KV head, 16-row block);
// wave w takes the partition's tiles w, w + 4, w + 8, ... and keeps its own FA2
// online-softmax state ("mha_decoding_single_batch_pipelined", description;
// "decoding_warp_split_k" in its Parameters); the 4 states are merged by
// log-sum-exp at the end, and the block writes either the finished rows or the
// normalised partial (o, m, l) of its partition for the split-K merge.
// A split call whose fold leaves room (at most 8 rows per KV head) may give a
// block two KV heads instead (the two-head fold): its 16 rows are two slots of
// 8, a 16-row stage holds 8 keys x 2 heads (512 contiguous bytes of each key
// row per load), and a row's scores against the other head's stage rows are
// masked out.
//
// Per 16-key tile and wave (rows padded to 16):
//   S^T[16 keys x 16 rows] = K[16 x D] . Q^T[D x 16]      D/32 v_mfma_f32_16x16x32_bf16
//       A = K from the LDS stage, B = Q^T held in registers for the whole kernel.
//   softmax on the accumulator layout: lane l owns row l % 16 and keys
//       4 (l / 16) + 0..3; the row max needs two lane swaps (v_permlane16/32_swap),
//       and O is rescaled only when some row's max actually grew.
//   O^T[D x 16 rows] += V^T[D x 16 keys] . P^T[16 x 16]    D/16 v_mfma_f32_16x16x16_bf16
//       B = P^T is this lane's S^T accumulator rounded to bf16 (no data movement);
//       A = V^T comes from the LDS stage through transposing reads
//       (ds_read_b64_tr_b16), so V is never transposed in registers.
//
// LDS stage: the tile's K rows then its V rows, row-major in 16-byte chunks,
// chunk c of key k stored at position c ^ swz(k) of its row.  The stage is filled
// linearly (one 1 KB load instruction = 4 or 8 whole rows of one head), the
// 16 keys x one chunk that an A-operand read of K touches fall in distinct
// bank groups, and so do the 4 keys x 32 bytes of each 16-lane transposing read
// of V.
#include "da_stream.h"

namespace da {

namespace {

constexpr int kTK = 16;  // keys per tile
constexpr int kWaves = 4;

template <int D, int NS = 2>
struct StreamCfg {
  static constexpr int ROW = D * 2;                  // bytes per key row of one head
  static constexpr int CH = ROW / 16;                // 16-byte chunks per row
  static constexpr int HALF = kTK * ROW;             // K (or V) bytes per tile
  static constexpr int STAGE = 2 * HALF;
  static constexpr int NI = HALF / 1024;             // 1 KB load instructions per half
  static constexpr int KEYS_PER_I = 1024 / ROW;      // rows per load instruction
  // LDS stages per wave.  Static mapping (NS = 2 at D = 128): a 16 KB ring per
  // wave, 64 KB per block, so two blocks fit on a CU.  Work queue (NS = 3): one
  // resident block per CU with a deeper ring.
  static constexpr int STAGES = (D == 128) ? NS : 4;
  static constexpr int RING = STAGES * STAGE;
  static constexpr int KS = D / 32;                  // depth steps of q.K^T
  static constexpr int DT = D / 16;                  // 16-wide depth tiles of O
  static constexpr int MERGE = kWaves * 16 * (D + 3 + 3) * 4;  // o rows, then m, l, lr
  static constexpr int SMEM = (kWaves * RING > MERGE) ? kWaves * RING : MERGE;
  static_assert(NI * 1024 == HALF, "a tile half must split into 1 KB loads");
  static_assert(2 * NI * (STAGES - 1) + NI <= 63, "vmcnt range");
};

// Chunk position of chunk 0 of key k's row (XOR-ed with the chunk index).
template <int D>
__device__ __forceinline__ constexpr int swz(int k) {
  return 2 * (k & 3) + ((k >> 2) & 1) + (D == 128 ? 8 * ((k >> 3) & 1) : 0);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Requests the tile of keys [j0, j0 + 16 >> hb_shift) of KV heads g, g + 1, ...
// (2^hb_shift of them) into the LDS stage at `lds`: stage row r holds key
// j0 + (r >> hb_shift) of head g + (r & (2^hb_shift - 1)).  Keys at or past
// `kend` read the same chunk of the tile's first key instead (finite data, masked
// out of the softmax), so every tile costs exactly 2 NI instructions.
template <int D>
__device__ __forceinline__ void stream_issue(const DecodeParams& p, int b, int g, int j0,
                                             int kend, uint32_t lds,
                                             const uint32_t (&off)[StreamCfg<D>::NI],
                                             int lane) {
  using C = StreamCfg<D>;
  const size_t row0 = stream_row0(p, b, j0);
  // Uniform by construction; read through readfirstlane so that the compiler
  // keeps it in scalar registers (the loads take a scalar base) even where it
  // reaches here through a phi after a divergent branch.
  const size_t head_off0 = (row0 * p.num_kv_heads + g) * (size_t)C::ROW;
  const size_t head_off = pin_uniform_u64(head_off0);
  const char* kb = (const char*)p.k + head_off;
  const char* vb = (const char*)p.v + head_off;
  const uint32_t rs = (uint32_t)p.num_kv_heads * C::ROW;  // bytes between keys of a head
  const int nvalid = kend - j0;
  // the previous reads of this stage (one tile ago) must have completed
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  uint32_t o[C::NI];
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    o[i] = off[i];
    if (nvalid < (kTK >> p.hb_shift)) {
      const int key = (i * C::KEYS_PER_I + lane / C::CH) >> p.hb_shift;
      if (key >= nvalid) o[i] -= (uint32_t)key * rs;
    }
  }
#pragma unroll
  for (int i = 0; i < C::NI; ++i) dma16(kb, o[i], lds + i * 1024);
#pragma unroll
  for (int i = 0; i < C::NI; ++i) dma16(vb, o[i], lds + C::HALF + i * 1024);
}

// The online-softmax state of one wave: rows of lane l % 16.
template <int D>
struct StreamState {
  f32x4_t acc[StreamCfg<D>::DT];
  float m, lsum, lsr;  // running max (log2 units), exact and bf16-rounded weight sums
};


// One tile from the LDS stage `st`.  `after` = tiles of this wave requested
// after this one (still in flight); the K half is waited for first, the V half
// just before the P.V contraction.
template <int D, int NS>
__device__ __forceinline__ void stream_tile(const char* st, const bf16x8_t (&qf)[StreamCfg<D>::KS],
                                            StreamState<D>& s, int after, int j0, bool masked,
                                            int hi, float scale_log2, uint32_t kofs,
                                            uint32_t vofs, const int (&kkey)[4]) {
  using C = StreamCfg<D, NS>;
  wait_after<2 * C::NI, C::NI, C::STAGES - 1>(after);  // K half of this tile landed
  f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < C::KS; ++k) {
    const bf16x8_t a = *(const bf16x8_t*)(st + (kofs ^ (64u * k)));
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[k], sc, 0, 0, 0);
  }
  float x[4];
  float mx = kNegInf;
  const int lim = hi - j0;  // this row's visible keys from the tile's first key on
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v = sc[r] * scale_log2;
    if (masked) v = (kkey[r] < lim) ? v : kNegInf;
    x[r] = v;
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
  float pr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(x[r] - ms);
  s.lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  // P^T operand: keys 4 g16 + 0..3 of row l % 16, rounded to bf16; O is
  // normalised by the rounded sum so that the effective weights sum to one.
  const uint32_t w0 = pack_bf16(pr[0], pr[1]);
  const uint32_t w1 = pack_bf16(pr[2], pr[3]);
  s.lsr += (bf16lo(w0) + bf16hi(w0)) + (bf16lo(w1) + bf16hi(w1));
  const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(w0, w1));
  wait_after<2 * C::NI, 0, C::STAGES - 1>(after);  // V half landed
  // O^T += V^T . P^T; A of depth tile dt: V[4 g16 + 0..3][16 dt + l % 16].
  const char* vh = st + C::HALF;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    const uint2 av = lds_read_tr16(vh + (vofs ^ (32u * dt)));
    s.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, av), pb,
                                                          s.acc[dt], 0, 0, 0);
  }
}

// One work item: rows rb*16.. of (sequence b, KV heads g .. g + 2^hb_shift - 1)
// over partition pidx.  With hb_shift > 0 (then rb = 0) the 16 rows are 2^hb_shift
// slots of 16 >> hb_shift rows, slot s holding the token-major fold of KV head
// g + s, and a score of a row against a stage row of another head is masked out.
template <int D, int NS, bool EMPTY_EXIT>
__device__ __forceinline__ void stream_item(const DecodeParams& p, char* smem, int b, int g,
                                            int pidx, int rb) {
  using C = StreamCfg<D, NS>;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id_uniform();
  const int c16 = lane & 15, g16 = lane >> 4;
  const int hbs = p.hb_shift;
  const int kpt = kTK >> hbs;            // keys per tile
  const int rps = 4 - hbs;               // log2 of the rows per head slot

  // This lane's query row (16 rows per block: rows of the token-major fold).
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

  StreamState<D> s;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) s.acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  s.m = kNegInf;
  s.lsum = 0.f;
  s.lsr = 0.f;

  // Per-lane load offsets: instruction i moves stage chunk 64 i + lane, i.e.
  // chunk (lane % CH) ^ swz(r) of stage row r = i * KEYS_PER_I + lane / CH, which
  // is key r >> hbs of head slot r & (2^hbs - 1) (consecutive in the cache row).
  uint32_t off[C::NI];
  const uint32_t rs = (uint32_t)p.num_kv_heads * C::ROW;
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    const int r = i * C::KEYS_PER_I + lane / C::CH;
    off[i] = (uint32_t)(r >> hbs) * rs + (uint32_t)(r & ((1 << hbs) - 1)) * C::ROW +
             16u * (uint32_t)((lane % C::CH) ^ swz<D>(r));
  }
  // Key (from the tile's first) of the stage rows 4 g16 + 0..3 this lane scores;
  // stage rows of another head slot never pass the mask.
  int kkey[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * g16 + j;
    kkey[j] = ((r & ((1 << hbs) - 1)) == slot) ? (r >> hbs) : 0x7fffffff;
  }
  // Read offsets inside a stage: K operand of depth step k at kofs ^ 64 k; the
  // V^T operand of depth tile dt at vofs ^ 32 dt (from the half's start).
  const uint32_t kofs = c16 * C::ROW + 16u * (uint32_t)(g16 ^ swz<D>(c16));
  const int vkey = 4 * g16 + (c16 >> 2);
  const uint32_t vofs = vkey * C::ROW + 16u * (uint32_t)(((c16 & 3) >> 1) ^ swz<D>(vkey)) +
                        8u * (c16 & 1);

  // Tiles below n_full are whole for every row; with several heads every tile is masked.
  const int n_full = (hbs > 0) ? 0 : (hmin - k_lo) / kpt;
  const int n_tot = (hmax - k_lo + kpt - 1) / kpt;
  const int my_cnt = (n_tot > wave) ? (n_tot - wave + kWaves - 1) / kWaves : 0;
  char* ring = smem + wave * C::RING;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  if (my_cnt > 0) {
    // The first tile is requested while the Q loads are in flight; then
    // everything so far is waited for, so that only tile loads are counted
    // below.  The builtin form lets the compiler see that the Q registers are
    // ready; the empty asm keeps memory accesses on their side of it.
    stream_issue<D>(p, b, g, k_lo + wave * kpt, hmax, ring_lds, off, lane);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int s = 0; s < C::KS; ++s) qf[s] = row_ok ? qf[s] : bf16x8_t{};
    const int pro = min(C::STAGES - 1, my_cnt);
    for (int i = 1; i < pro; ++i)
      stream_issue<D>(p, b, g, k_lo + (wave + kWaves * i) * kpt, hmax, ring_lds + i * C::STAGE,
                      off, lane);
    int cur = 0;
    for (int i = 0; i < my_cnt; ++i) {
      const int nxt = i + C::STAGES - 1;
      if (nxt < my_cnt) {  // into the stage read one tile ago
        const int sn = (cur == 0) ? C::STAGES - 1 : cur - 1;
        stream_issue<D>(p, b, g, k_lo + (wave + kWaves * nxt) * kpt, hmax,
                        ring_lds + sn * C::STAGE, off, lane);
      }
      const int t = wave + kWaves * i;
      stream_tile<D, NS>(ring + cur * C::STAGE, qf, s, my_cnt - 1 - i, k_lo + t * kpt, t >= n_full,
                     hi, p.scale_log2, kofs, vofs, kkey);
      cur = (cur + 1 == C::STAGES) ? 0 : cur + 1;
    }
  }

  // Row sums across the 4 lane groups.
  float lsum = s.lsum, lsr = s.lsr;
  lsum += shfl_xor(lsum, 16);
  lsum += shfl_xor(lsum, 32);
  lsr += shfl_xor(lsr, 16);
  lsr += shfl_xor(lsr, 32);

  // Merge the 4 waves through LDS (reusing the rings: every wave's loads have
  // completed, its last tile waited for vmcnt 0).
  __syncthreads();
  float* so = (float*)smem;          // [wave][row][D + 3]
  float* sm = so + kWaves * 16 * (D + 3);
  float* sl = sm + kWaves * 16;
  float* sr = sl + kWaves * 16;
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
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm[w * 16 + r]);
    const float Ms = (M == kNegInf) ? 0.f : M;
    float L = 0.f, Lr = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(sm[w * 16 + r] - Ms);
      L += f * sl[w * 16 + r];
      Lr += f * sr[w * 16 + r];
      O += f * so[(w * 16 + r) * (D + 3) + d];
    }
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

// Static mapping: block -> (partition, sequence, KV head or head pair, row block); the row
// blocks of one (partition, sequence, KV head) get ids 8 apart, so that they
// share an XCD and its L2 serves the second read of their tiles.
//
// Work queue (ragged batches, one row block): items (partition, sequence, KV
// head), partition-major, so that long items tend to go first.  A block takes
// its next item, (queue's low half)++, only when it has finished the last one
// (a block that reserved ahead would hold items back from blocks that run out
// first), until the items run out; blocks with shorter items, or on faster
// parts of the chip, take more.  The queue is a single 64-bit word, so relaxed
// atomics order every access to it: a block counts itself done in the high half
// after its last take, and the block that completes the count (every take is
// then behind it) sets the word back to zero for the next call.
template <int D, int NS>
__global__ __launch_bounds__(256) void decode_stream_kernel(DecodeParams p) {
  using C = StreamCfg<D, NS>;
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
    stream_item<D, NS, false>(p, smem, work % p.batch, g, work / p.batch, rb);
    return;
  }
  // s_next is double-buffered: slot it & 1 is written again two barriers after
  // every wave has read it.
  for (int it = 0;; ++it) {
    if (threadIdx.x == 0) s_next[it & 1] = (int)(uint32_t)atomicAdd(p.queue, 1ull);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_next[it & 1]);
    if (item >= n_work) break;
    int w = item;
    const int g = (w % n_hg) << p.hb_shift;
    w /= n_hg;
    stream_item<D, NS, true>(p, smem, w % p.batch, g, w / p.batch, 0);
    __syncthreads();  // the LDS is free again
  }
  if (threadIdx.x == 0) {
    const unsigned long long old = atomicAdd(p.queue, 1ull << 32);
    if ((uint32_t)(old >> 32) == gridDim.x - 1) atomicExch(p.queue, 0ull);
  }
}

}  // namespace

int stream_rows_per_block() { return 16; }
int stream_step_keys() { return kTK; }

hipError_t launch_decode_stream(const DecodeParams& p, hipStream_t s) {
  if (p.hb_shift < 0 || p.hb_shift > 1 || (p.num_kv_heads & ((1 << p.hb_shift) - 1)) != 0 ||
      (p.hb_shift > 0 && (p.row_blocks != 1 || (fold_rows(p) << p.hb_shift) > 16)))
    return hipErrorInvalidValue;
  const int n_work = p.num_partitions * p.batch * (p.num_kv_heads >> p.hb_shift);
  int grid = ((n_work + 7) / 8) * 8 * p.row_blocks;
  if (p.queue) {
    if (p.row_blocks != 1 || p.queue_blocks < 1) return hipErrorInvalidValue;
    grid = n_work < p.queue_blocks ? n_work : p.queue_blocks;
  }
  if (p.depth == 64)
    hipLaunchKernelGGL((decode_stream_kernel<64, 2>), dim3(grid), dim3(256), 0, s, p);
  else if (p.queue)
    hipLaunchKernelGGL((decode_stream_kernel<128, 3>), dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((decode_stream_kernel<128, 2>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace da
