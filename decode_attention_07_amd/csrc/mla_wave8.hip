// mla_wave8.hip -- matrix-core MLA decode for gfx950 with two waves per SIMD
// ("flare_mla_decoding_dispatch": one KV head, depth 576, V = K[..., :512]
// taken from the same cache rows, Args `k` and `kv_num_heads`).
//
// A block owns 128 of a sequence's T*H query rows (the MTP token fold) and one
// partition of its keys, so every cache row of the partition is read from HBM
// once per 128 rows.  It runs 8 waves, two per SIMD, in two groups of four: group
// g (waves 4g .. 4g+3) owns rows 64g .. 64g+63 and does both products for them.
// Two waves per SIMD leave 256 registers per wave, too few for 32 rows of Q^T
// (144) and O^T (256), so within a group the waves split the two products
// differently:
//   scores   wave (g, w) owns rows 64g + 16w .. +15 (its Q^T, 72 registers):
//              S^T[32 keys x 16 rows] = K[32 x 576] . Q^T[576 x 16]
//              36 v_mfma_f32_16x16x32_bf16 per 32-key tile, K read from LDS.
//   softmax  on the score accumulators (lane l: row l % 16, keys 4 (l / 16)
//              + 0..3 of each 16-key half); the bf16 weights go to the group's
//              half of an 8 KB LDS buffer P[128 rows][32 keys].
//   P.V      wave (g, w) owns output columns 128w .. 128w+127 of the group's rows:
//              O^T[128 x 64] += V^T[128 x 32 keys] . P^T[32 keys x 64]
//              16 v_mfma_f32_32x32x16_bf16 per tile (128 accumulator registers),
//              V^T read from the same LDS tile by transposing reads, P^T from
//              the buffer.
// The split works because the softmax keeps a fixed reference max per row (set
// by the row's first visible tile; weights up to 2^kHeadroom = 2^64, so that
// weight x value sums over a partition stay far below fp32's 2^128 for any
// realistic cache value): O is never rescaled, so a P.V wave needs no other
// wave's running max, only the rows' final normalisers at the end (through
// LDS).  A row whose scores exceed its reference by more than kHeadroom raises
// it; the accumulated O of that row is then inconsistent, and the block runs its
// partition again with the raised references (one vote at the end of the pass).
//
// The two groups run half an iteration apart (ping-pong): in every half, one
// group does the scores and softmax of a tile (K reads from LDS, 16x16x32
// MFMAs, vector work) while the other does the P.V of the tile before (32x32x16
// MFMAs, few LDS reads), and the two waves that share a SIMD swap roles at each
// block barrier.  So LDS, the matrix core and the vector ALU all have work in
// every half.  Group 0: scores of tile t in half 2t, its P.V in half 2t + 1;
// group 1 one half later.  A tile is read in halves 2t .. 2t + 2; the 4-stage
// ring keeps two tiles in flight (tile t + 4 is requested, by group 0, at the
// start of half 2t + 3, into the stage tile t left; tiles 0 and 1 before the
// loop, 2 and 3 at the start of half 1).  The 8-bit form's rings: below.
// LDS stage layout: row-major, chunk c (16 bytes) of key k at position
// (c & ~7) | ((c & 7) ^ swz(k)) of its 72-chunk row (swz below): the K reads and
// the transposing V^T reads are conflict-free, and each 1 KB load instruction
// fills whole 128-byte lines (which lets the loads carry the non-temporal hint).
#include "da_device.h"

namespace da {

namespace {

constexpr int kD = 576;
constexpr int kDv = 512;
constexpr int kBN = 32;                      // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 128;                   // query rows per block
constexpr int kGroupRows = kRows / 2;        // rows per wave group (64)
constexpr int kSRows = kGroupRows / 4;       // score rows per wave (16)
constexpr int kCols = kDv / 4;               // output columns per wave (128)
constexpr int kKS = kD / 32;                 // 18 depth steps of 32
constexpr int kRowBytes = kD * 2;            // 1152
constexpr int kTileBytes = kRowBytes * kBN;  // 36 KB
constexpr int kStages = 4;
constexpr int kDmaWaves = 4;                 // waves 0..3 issue the tile loads
constexpr int kDmaPerWave = kTileBytes / 1024 / kDmaWaves;  // 9
static_assert(kDmaPerWave * kDmaWaves * 1024 == kTileBytes, "tile splits into 1 KB loads");
constexpr int kPRowBytes = kBN * 2;          // 64: one row of bf16 weights
constexpr int kPBytes = kRows * kPRowBytes;  // 8 KB
constexpr int kTabPerLane = 12;              // uint16 load offsets (9 used), 24 bytes
constexpr float kHeadroom = 64.0f;           // largest exp2 argument (log2 units)

// 8-bit e4m3 cache ("flare_mla_decoding_dispatch", Parameters `dtype`): a cache
// row is 576 bytes.  Waves 0..3 load keys 8w .. 8w + 7 of a tile (4608
// contiguous bytes each) into a 4-slot staging ring, tile t + 3 at the start of
// half 2t + 1 as in the bf16 form.  At the end of that half (their P.V of tile
// t) they convert tile t + 1 into the bf16 stage layout above, so that the
// scores, the softmax and P.V run unchanged.  Two bf16 stages suffice: in half
// 2t + 1 tile t's stage is being read and tile t - 1's, read last in half 2t, is
// free.  A wave converts only what it loaded itself, so its own vmcnt wait orders
// the conversion after the loads, and the next block barrier publishes the stage.
constexpr int kF8Row = kD;                          // bytes per cache row
constexpr int kF8Tile = kF8Row * kBN;               // 18 KB
constexpr int kF8WaveBytes = kF8Tile / kDmaWaves;   // 4608
constexpr int kF8Wide = 4;                          // 1 KB loads per wave and tile
constexpr int kF8Narrow = 2;                        // then 256-byte loads for the last 512 bytes
constexpr int kF8Issue = kF8Wide + kF8Narrow;
constexpr int kF8Pieces = kF8WaveBytes / (64 * 8);  // 9 eight-byte pieces per lane
constexpr int kBStagesF8 = 2;
constexpr int kF8Slots = 4;
constexpr int kF8Ring0 = kBStagesF8 * kTileBytes;   // the staging ring follows the bf16 stages
static_assert(kF8Wide * 1024 + kF8Narrow * 256 == kF8WaveBytes, "a wave's keys split into loads");
static_assert(kF8Ring0 + kF8Slots * kF8Tile <= kStages * kTileBytes,
              "8-bit rings fit the stage array");
static_assert(kF8Pieces <= kTabPerLane, "conversion table fits");

// Chunk swizzle of a key row (XOR inside each 8-chunk line), from key bits 1 and
// 2.  Fitted to gfx950's LDS: a ds_read_b128 is served in four cycles of 16
// lanes (by the measured bank-conflict counts, the lanes of one cycle share lane
// bit 5 and the parity of lane bits 2..4), and with this swizzle the 16x16x32 K
// reads (16 keys x 4 chunks per 64 lanes) and the transposing V^T reads both
// meet each bank once per cycle.
__device__ __forceinline__ constexpr int swz(int key) {
  return 2 * ((key >> 1) & 1) + 4 * (((key >> 1) ^ (key >> 2)) & 1);
}

// 16 bytes per lane from base + voff into LDS at lds_base + 16 * lane
// (global_load_lds_dwordx4; the LDS address goes in through m0).  Completion is
// tracked with vmcnt waits.  NT: the non-temporal hint, for a cache read by one
// block only; where sibling row blocks read the same tiles through their XCD's
// L2 (the MTP fold), the hint costs them L2 hits and the loads go without it
// (measured: T = 1 is 1-2.5% faster with it, T = 2 1.4% faster without).
template <bool NT>
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_base) {
  if constexpr (NT)
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(base), "{m0}"(lds_base)
                 : "memory");
  else
    asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds_base)
                 : "memory");
}

// 4 bytes per lane from base + voff into LDS at lds_base + 4 * lane.  (No
// immediate offset: on these loads it would move the LDS destination too.)
template <bool NT>
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds_base) {
  if constexpr (NT)
    asm volatile("global_load_lds_dword %0, %1 nt" : : "v"(voff), "s"(base), "{m0}"(lds_base)
                 : "memory");
  else
    asm volatile("global_load_lds_dword %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds_base)
                 : "memory");
}

// s_waitcnt vmcnt(N) (lgkmcnt and expcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Load instruction n = wave + 4 i (waves 0..3) of a tile writes stage chunks
// 64 n + lane: chunk position q = (64 n + lane) % 72 of key (64 n + lane) / 72,
// which holds that key's chunk q ^ swz(key) (the XOR stays inside the 8-chunk
// line, and 72 is a multiple of 8, so q % 8 = lane % 8).  The source offset of
// each of the lane's 9 loads (below 36 KB) is kept in LDS as a uint16.
__device__ __forceinline__ uint32_t dma_chunk(int wave, int i, int lane) {
  return 64u * (uint32_t)(wave + kDmaWaves * i) + (uint32_t)lane;
}
// c / 72 (exact for c < 2304: (c / 8) * 57 / 512 = floor(c / 72) on this range)
__device__ __forceinline__ int dma_key(uint32_t c) { return (int)(((c >> 3) * 57u) >> 9); }

__device__ __forceinline__ void dma_table_init(uint16_t* tab, int wave, int lane) {
  const int l7 = lane & 7;
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const uint32_t c = dma_chunk(wave, i, lane);
    tab[i] = (uint16_t)(16u * c + 16u * (uint32_t)((l7 ^ swz(dma_key(c))) - l7));
  }
}

// First cache row of the tile at key j0 (a tile never straddles a page).  The
// page-table entry is read through the scalar cache, its address pinned to
// scalar registers first (a vector load's wait would also wait for the tile
// loads in flight).
__device__ __forceinline__ size_t mla_row0(const DecodeParams& p, int b, int j0) {
  if (p.page_table) {
    const uint64_t a = pin_uniform_u64(
        (uint64_t)(p.page_table + (size_t)b * p.max_pages + (size_t)(j0 >> p.page_shift)));
    const uint32_t phys = *(const __attribute__((address_space(4))) uint32_t*)a;
    return ((size_t)phys << p.page_shift) + (size_t)(j0 & ((1 << p.page_shift) - 1));
  }
  return seq_kv_row0(p, b) + j0;
}

// Waves 0..3: request the 32-key tile at key j0 into one stage.  Keys at or past
// `kend` fetch the tile's first key instead (finite data, masked out of the
// softmax), so every issuing wave always has kDmaPerWave loads per tile.
template <bool NT>
__device__ __forceinline__ void mla_issue(const DecodeParams& p, uint32_t stage, int b, int j0,
                                          int kend, int wave, int lane, const uint16_t* tab) {
  const size_t off = pin_uniform_u64(mla_row0(p, b, j0) * kRowBytes);
  const char* base = (const char*)p.k + off;
  const uint2 t01 = *(const uint2*)tab;
  const uint2 t23 = *(const uint2*)(tab + 4);
  const uint2 t45 = *(const uint2*)(tab + 8);
  const uint32_t w[5] = {t01.x, t01.y, t23.x, t23.y, t45.x};
  const uint32_t dst = __builtin_amdgcn_readfirstlane(stage + wave * 1024);
  const int nvalid = kend - j0;
  if (nvalid >= kBN) {  // whole tile (uniform branch)
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const uint32_t o = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xffffu);
      dma16<NT>(base, o, dst + i * kDmaWaves * 1024);
    }
  } else {
    // The chunk index passes through an empty asm so that the compiler computes
    // the keys here instead of keeping all nine (loop-invariant) live across the loop.
    uint32_t c0 = 64u * (uint32_t)wave + (uint32_t)lane;
    asm volatile("" : "+v"(c0));
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      uint32_t o = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xffffu);
      const int key = dma_key(c0 + 256u * i);
      if (key >= nvalid) o -= (uint32_t)key * kRowBytes;
      dma16<NT>(base, o, dst + i * kDmaWaves * 1024);
    }
  }
}

// Waves 0..3, 8-bit cache: request keys 8w .. 8w + 7 of the tile at key j0 into
// this wave's part of a staging slot (byte 4608 w on).  A 16-byte piece never
// straddles two keys (576 = 36 x 16); pieces of keys at or past `kend` fetch the
// tile's first key instead, so every issuing wave has kF8Issue loads per tile.
template <bool NT>
__device__ __forceinline__ void mla_issue_fp8(const DecodeParams& p, uint32_t fslot, int b,
                                              int j0, int kend, int wave, int lane) {
  const char* base = (const char*)p.k + pin_uniform_u64(mla_row0(p, b, j0) * kF8Row);
  const uint32_t dst = __builtin_amdgcn_readfirstlane(fslot + wave * kF8WaveBytes);
  const uint32_t w0 = (uint32_t)(kF8WaveBytes * wave);
  uint32_t ow = w0 + 16u * (uint32_t)lane;                // 1 KB loads
  uint32_t on = w0 + kF8Wide * 1024u + 4u * (uint32_t)lane;  // 256-byte loads
  const int nvalid = kend - j0;
  if (nvalid >= kBN) {  // whole tile (uniform branch)
#pragma unroll
    for (int i = 0; i < kF8Wide; ++i) dma16<NT>(base, ow + 1024u * i, dst + 1024u * i);
#pragma unroll
    for (int i = 0; i < kF8Narrow; ++i)
      dma4<NT>(base, on + 256u * i, dst + kF8Wide * 1024u + 256u * i);
  } else {
    // Opaque copies: the per-load offsets and keys are computed here, not kept live.
    asm volatile("" : "+v"(ow), "+v"(on));
#pragma unroll
    for (int i = 0; i < kF8Wide; ++i) {
      uint32_t o = ow + 1024u * i;
      const uint32_t key = o / (uint32_t)kF8Row;
      if ((int)key >= nvalid) o -= key * (uint32_t)kF8Row;
      dma16<NT>(base, o, dst + 1024u * i);
    }
#pragma unroll
    for (int i = 0; i < kF8Narrow; ++i) {
      uint32_t o = on + 256u * i;
      const uint32_t key = o / (uint32_t)kF8Row;
      if ((int)key >= nvalid) o -= key * (uint32_t)kF8Row;
      dma4<NT>(base, o, dst + kF8Wide * 1024u + 256u * i);
    }
  }
}

// 8-bit cache: the bf16-stage byte offset (below 36 KB) of the 8 elements that
// piece j of this lane converts, byte 512 j + 8 lane of the wave's 4608.
__device__ __forceinline__ void f8_table_init(uint16_t* tab, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < kF8Pieces; ++j) {
    const int o = 512 * j + 8 * lane;
    const int key = 8 * wave + o / kF8Row;
    const int c = (o % kF8Row) / 8;  // 16-byte chunk of the bf16 row
    tab[j] = (uint16_t)(key * kRowBytes + 16 * ((c & ~7) | ((c & 7) ^ swz(key))));
  }
}

// This wave's keys of a staged 8-bit tile -> the bf16 stage (exact conversion).
// Software-pipelined three pieces deep: the compiler cannot tell a store into the
// stage from a later read of the staging slot, so it keeps them in program
// order; piece j + 3 is read right after piece j is stored, and three reads are
// in flight at each store (all nine at once would need more registers than the
// P.V wave has left).
__device__ __forceinline__ void mla_convert_fp8(const char* fslot, char* bst, int wave, int lane,
                                                const uint16_t* tab) {
  constexpr int kDepth = 3;
  const char* src = fslot + kF8WaveBytes * wave + 8 * lane;
  const uint2 t01 = *(const uint2*)tab;
  const uint2 t23 = *(const uint2*)(tab + 4);
  const uint2 t45 = *(const uint2*)(tab + 8);
  const uint32_t w[5] = {t01.x, t01.y, t23.x, t23.y, t45.x};
  uint2 x[kDepth];
#pragma unroll
  for (int j = 0; j < kDepth; ++j) x[j] = *(const uint2*)(src + 512 * j);
#pragma unroll
  for (int j = 0; j < kF8Pieces; ++j) {
    const uint32_t e = (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu);
    *(bf16x8_t*)(bst + e) = fp8x8_to_bf16(x[j % kDepth].x, x[j % kDepth].y);
    if (j + kDepth < kF8Pieces) x[j % kDepth] = *(const uint2*)(src + 512 * (j + kDepth));
  }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Scores of one tile for this wave's 16 rows: s[kh] = S^T[16 keys (half kh) x 16
// rows].  A = K chunk 4 st + lane / 16 of key 16 kh + lane % 16, at stage byte
// (kofs ^ 64 (st & 1)) + 128 (st >> 1) + 18432 kh (the swizzle only touches
// bits 4..6); B = this wave's Q^T for depth step st.
// The K fragments come through a ring two depth steps deep; scheduling barriers
// keep the compiler from hoisting every read ahead of the MFMAs (which would need
// 144 registers).
__device__ __forceinline__ void wave_scores(const char* buf, const bf16x8_t (&qf)[kKS],
                                            uint32_t kofs, f32x4 (&s)[2]) {
  auto kfrag = [&](int kh, int st) {
    return *(const bf16x8_t*)(buf + (kofs ^ (64u * (st & 1))) + 128u * (st >> 1) +
                              16u * kRowBytes * kh);
  };
  bf16x8_t ra[2], rb[2];
  ra[0] = kfrag(0, 0);
  rb[0] = kfrag(1, 0);
  ra[1] = kfrag(0, 1);
  rb[1] = kfrag(1, 1);
#pragma unroll
  for (int st = 0; st < kKS; ++st) {
    const int slot = st & 1;
    s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[slot], qf[st], st ? s[0] : f32x4{}, 0, 0, 0);
    if (st + 2 < kKS) ra[slot] = kfrag(0, st + 2);
    s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rb[slot], qf[st], st ? s[1] : f32x4{}, 0, 0, 0);
    if (st + 2 < kKS) rb[slot] = kfrag(1, st + 2);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// P.V of one tile for this wave's 128 columns and its group's 64 rows: acc[ct][rt]
// = O^T[32 columns (tile ct) x 32 rows (tile rt)].  A = V^T[32 d x 16 keys] by two
// transposing reads (keys 16 kh + 8 (lane / 32) + 0..3 and + 4..7); B = P^T[16
// keys x 32 rows]: keys 16 kh + 8 (lane / 32) + 0..7 of row 32 rt + lane % 32 of
// the group's rows, one 16-byte read of the swizzled weight buffer.
__device__ __forceinline__ void wave_pv(const char* vbuf, const char* pbuf, uint32_t vofs0,
                                        uint32_t vofs1, uint32_t pofs, int wq,
                                        f32x16_t (&acc)[4][2]) {
  // V^T of column tile 4 wq + 2 cp + u for key half kh.
  auto vfrag = [&](int kh, int cp, int u) {
    const int dt = 4 * wq + 2 * cp + u;  // 32-column tile of the 512 value columns
    const uint32_t x = 64u * (uint32_t)(dt & 1), y = 128u * (uint32_t)(dt >> 1) +
                                                     16u * kRowBytes * kh;
    return concat_bf16x8(lds_read_tr16(vbuf + ((vofs0 ^ x) + y)),
                         lds_read_tr16(vbuf + ((vofs1 ^ x) + y)));
  };
  auto pfrag = [&](int kh, int rt) {
    return *(const bf16x8_t*)(pbuf + rt * 32 * kPRowBytes + (pofs ^ (32u * kh)));
  };
  bf16x8_t a[2] = {vfrag(0, 0, 0), vfrag(0, 0, 1)};
  bf16x8_t bq[2] = {pfrag(0, 0), pfrag(0, 1)};  // P^T of both row tiles, key half kh
#pragma unroll
  for (int step = 0; step < 4; ++step) {  // (key half, pair of column tiles)
    const int kh = step >> 1, cp = step & 1;
    // Each fragment is requested for its next use right after its last use here,
    // so that its read has the rest of this step to land.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        acc[2 * cp + u][rt] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], bq[rt], acc[2 * cp + u][rt], 0, 0, 0);
        if (step == 1 && u == 1) bq[rt] = pfrag(1, rt);
      }
      if (step + 1 < 4) a[u] = vfrag((step + 1) >> 1, (step + 1) & 1, u);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// FP8: the cache holds e4m3 elements (real value = k_scale x stored; k_scale is
// folded into scale_log2, and v_scale, the same factor for the value slice,
// multiplies the output).  NT: the tile loads carry the non-temporal hint (one
// row block per (sequence, partition); see dma16).
template <bool FP8, bool NT>
__global__ __launch_bounds__(kThreads) void mla_wave8_kernel(DecodeParams p, int n_mblocks,
                                                               int n_work) {
  constexpr int kIssue = FP8 ? kF8Issue : kDmaPerWave;  // loads per issuing wave and tile
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kTileBytes];
  __shared__ __attribute__((aligned(16))) char pbuf[kPBytes];
  __shared__ __attribute__((aligned(16))) uint16_t dma_tab[kDmaWaves * 64 * kTabPerLane];
  __shared__ __attribute__((aligned(16))) int votes[1][kWaves];

  // XCD-aware block id: blocks i and i + 8 share an XCD; the n_mblocks row blocks
  // of one (partition, sequence) get ids 8 apart, so they read the same tiles
  // through one L2.
  const int id = blockIdx.x;
  const int xcd = id & 7;
  const int r8 = id >> 3;
  const int mb = r8 % n_mblocks;
  const int work = (r8 / n_mblocks) * 8 + xcd;
  if (work >= n_work) return;  // padding block: leaves before any barrier
  const int b = work % p.batch;
  const int pidx = work / p.batch;
  const int H = p.num_q_heads;
  const int nrows = seq_tokens(p, b) * H;
  if (mb * kRows >= nrows) return;  // ragged q: none of this block's rows exist
  const size_t row0q = seq_row0(p, b);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2, wq = wave & 3;    // wave group (half of the rows), wave in group
  const int l15 = lane & 15, sg = lane >> 4;   // score layout: row, key group
  const int l31 = lane & 31, hg = lane >> 5;   // P.V layout: row in tile, key half-group

  // This lane's score row.
  const int srow = grp * kGroupRows + wq * kSRows + l15;
  const int rr = mb * kRows + srow;
  const bool row_ok = rr < nrows;
  const int tok = row_ok ? rr / H : 0;
  const int head = row_ok ? rr % H : 0;
  const int k_lo = pidx * p.keys_per_partition;
  const int k_end = k_lo + p.keys_per_partition;
  const int hi = row_ok ? min(k_end, visible_keys(p, b, tok)) : k_lo;
  // Visibility grows with the token index: the block's last token sees the most
  // keys (uniform; pinned to scalar registers).
  const int t_last = (min(nrows, (mb + 1) * kRows) - 1) / H;
  const int hmax =
      __builtin_amdgcn_readfirstlane(max(k_lo, min(k_end, visible_keys(p, b, t_last))));
  const int n_tot = (hmax - k_lo + kBN - 1) / kBN;

  // Q^T operand of depth step st: depth 32 st + 8 sg + 0..7 of row srow.
  bf16x8_t qf[kKS];
  {
    const uint16_t* qrow = (const uint16_t*)p.q + ((row0q + tok) * H + head) * (size_t)kD;
#pragma unroll
    for (int st = 0; st < kKS; ++st)  // rows past the fold read a valid row, zeroed below
      qf[st] = *(const bf16x8_t*)(qrow + st * 32 + sg * 8);
  }

  f32x16_t acc[4][2];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) acc[ct][rt] = f32x16_t{};
  float m = kNegInf, lsum = 0.f, lsr = 0.f;  // reference max (log2), exact and rounded sums
  bool need = false;                         // some row of this lane's raised its reference

  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  uint16_t* tab = dma_tab + wq * 64 * kTabPerLane + lane * kTabPerLane;  // group 0's own entries
  if (grp == 0) {
    if constexpr (FP8)
      f8_table_init(tab, wave, lane);
    else
      dma_table_init(tab, wave, lane);
  }

  // Per-lane LDS offsets of the operand reads.
  const uint32_t kofs = kRowBytes * l15 + ((16u * sg) ^ (16u * swz(l15)));
  const int i16 = lane & 15, G = lane >> 4;
  const int cl = 2 * (G & 1) + ((i16 & 3) >> 1);
  const int vkey = 8 * hg + (i16 >> 2);
  const uint32_t vofs0 = kRowBytes * vkey + ((16u * cl) ^ (16u * swz(vkey))) + 8u * (i16 & 1);
  const uint32_t vofs1 =
      kRowBytes * (vkey + 4) + ((16u * cl) ^ (16u * swz(vkey + 4))) + 8u * (i16 & 1);
  // P^T read: row 64 grp + 32 rt + l31, chunk (hg + 2 kh) ^ ((l31 >> 2) & 3) (XOR swizzle
  // of the four 16-byte chunks of a 64-byte row: conflict-free reads and writes).
  const char* pgrp = pbuf + grp * kGroupRows * kPRowBytes;
  const uint32_t pofs = kPRowBytes * l31 + 16u * ((uint32_t)hg ^ ((l31 >> 2) & 3));
  // P write of this lane's 8 weights: row srow, keys 16 kh + 4 sg + 0..3.
  const uint32_t pw_sw = (uint32_t)((srow >> 2) & 3);
  auto pwrite_ofs = [&](int kh) -> uint32_t {
    return kPRowBytes * srow + 16u * ((uint32_t)(2 * kh + (sg >> 1)) ^ pw_sw) + 8u * (sg & 1);
  };

  // bf16 stage of tile t: a 4-slot ring, or 2 slots when the 8-bit staging ring
  // takes the rest of the array.
  auto bstage = [&](int t) __attribute__((always_inline)) {
    return FP8 ? (t & (kBStagesF8 - 1)) : (t & (kStages - 1));
  };
  // Group 0 requests the tiles: into their bf16 stage, or into staging slot t % 4.
  auto issue = [&](int t) __attribute__((always_inline)) {
    if constexpr (FP8)
      mla_issue_fp8<NT>(p, lds0 + (uint32_t)(kF8Ring0 + (t & (kF8Slots - 1)) * kF8Tile), b,
                    k_lo + t * kBN, hmax, wave, lane);
    else
      mla_issue<NT>(p, lds0 + (uint32_t)((t & (kStages - 1)) * kTileBytes), b, k_lo + t * kBN,
                hmax, wave, lane, tab);
  };
  // 8-bit cache: this wave's keys of staged tile t -> bf16 stage of tile t.
  auto convert = [&](int t) __attribute__((always_inline)) {
    if constexpr (FP8)
      mla_convert_fp8(smem + kF8Ring0 + (t & (kF8Slots - 1)) * kF8Tile,
                      smem + bstage(t) * kTileBytes, wave, lane, tab);
  };
  // vmcnt for "the oldest requested tile landed" with `later` tiles requested after it.
  auto wait_tiles = [&](int later) __attribute__((always_inline)) {
    if (later >= 3)
      wait_vm<3 * kIssue>();
    else if (later == 2)
      wait_vm<2 * kIssue>();
    else if (later == 1)
      wait_vm<kIssue>();
    else
      wait_vm<0>();
  };

  const float sl = fabsf(p.scale_log2);
  const int hi4 = hi - 4 * sg;  // this lane's key limit, less its key group's offset

  // Scores and softmax of tile t for this wave's 16 rows; the bf16 weights go to
  // the P buffer.  The scale enters once per weight, p = 2^(fma(q.k, sl, -m)), the
  // row max taken over the unscaled scores (sl >= 0: a negative scale was moved
  // into Q).  The weights enter P.V rounded to bf16, and O is normalised by the sum
  // of the rounded weights (lsr); lsum, the exact sum, gives the LSE and the
  // partition's mass.
  // The scores are the longer path of each half (the P.V wave beside them on the
  // SIMD has slack), so they run at a raised wave priority: when both waves have
  // an instruction ready, the SIMD issues the score wave's first.
  auto score_tile = [&](int t) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    f32x4 sc[2];
    wave_scores(smem + bstage(t) * kTileBytes, qf, kofs, sc);
    const int lim = hi4 - (k_lo + t * kBN);  // key 16 kh + 4 sg + v visible iff 16 kh + v < lim
    float x[8];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int v = 0; v < 4; ++v) x[4 * kh + v] = sc[kh][v];
    auto vis = [&](int j) { return (16 * (j >> 2) + (j & 3)) < lim; };
    // Exponents against the current reference; a key hidden from the row gets -inf
    // (weight 0).  Every key of the tile is visible to every row of the wave on all
    // but a partition's last tiles (uniform test; 19 is the largest key offset).
    float nms = (m == kNegInf) ? 0.f : -m;
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = fmaf(x[j], sl, nms);
    if (__builtin_amdgcn_ballot_w64(lim < 20) != 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = vis(j) ? y[j] : kNegInf;
    }
    const float ymax = fmaxf(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])),
                             fmaxf(fmaxf(y[4], y[5]), fmaxf(y[6], y[7])));
    // The row max across its four lanes is needed only where the reference moves: a
    // row's first visible tile sets it, and a score above it by more than kHeadroom
    // raises it (and votes for a restart).  Otherwise the weights above stand.
    if (__builtin_amdgcn_ballot_w64(ymax > kHeadroom || (m == kNegInf && ymax != kNegInf)) !=
        0) {
      float mx = kNegInf;
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, vis(j) ? x[j] : kNegInf);
      mx = max_xor32(max_xor16(mx));
      mx = (mx == kNegInf) ? kNegInf : mx * sl;
      const bool grow = mx > m + kHeadroom;
      need = need || (grow && m != kNegInf);  // a row's first visible tile: nothing accumulated yet
      m = grow ? mx : m;
      nms = (m == kNegInf) ? 0.f : -m;
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = vis(j) ? fmaf(x[j], sl, nms) : kNegInf;
    }
    float ps = 0.f, pr = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = fast_exp2(y[j]);
      ps += x[j];
    }
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const uint32_t w0 = pack_bf16(x[4 * kh + 0], x[4 * kh + 1]);
      const uint32_t w1 = pack_bf16(x[4 * kh + 2], x[4 * kh + 3]);
      pr = dot2_bf16(w0, 0x3f803f80u, pr);  // + both rounded weights
      pr = dot2_bf16(w1, 0x3f803f80u, pr);
      *(uint2*)(pbuf + pwrite_ofs(kh)) = make_uint2(w0, w1);
    }
    lsum += ps;
    lsr += pr;
    __builtin_amdgcn_s_setprio(0);
  };

  if (n_tot > 0) {
    // Rows outside the fold get Q = 0; a negative scale flips Q's sign (exact).
    const uint32_t qx = p.scale_log2 < 0.f ? 0x80008000u : 0u;
    for (int pass = 0;; ++pass) {  // one pass over the partition; repeated after a restart
      // Tiles 0 and 1 requested; tile 0 landed (the Q loads before it, on the first
      // pass).  Every block starts at once and needs its Q and first tile before any
      // work: the fewer tile bytes in that first burst, the sooner it ends.  Tiles 2
      // and 3 follow at the start of half 1.
      // 8-bit cache: tiles 0, 1 and 2 requested (54 KB, less than two bf16 tiles),
      // and tile 0 converted; from then on one request per half 2t + 1.
      if (grp == 0) {
        constexpr int kPre = FP8 ? 3 : 2;
        for (int t = 0; t < kPre && t < n_tot; ++t) issue(t);
        wait_tiles(min(n_tot - 1, kPre - 1));
        convert(0);
      }
      if (pass == 0) {
#pragma unroll
        for (int q = 0; q < kKS; ++q) {
          uint4 u = __builtin_bit_cast(uint4, qf[q]);
          u = make_uint4(u.x ^ qx, u.y ^ qx, u.z ^ qx, u.w ^ qx);
          qf[q] = row_ok ? __builtin_bit_cast(bf16x8_t, u) : bf16x8_t{};
        }
      }
      // The Q registers pass through an empty asm: from here on the compiler sees
      // them as defined, not as loads that may still be in flight.  Otherwise it
      // re-waits for them before every score MFMA of the loop, and the hardware
      // count it waits on also holds this wave's tile loads.
#pragma unroll
      for (int q = 0; q < kKS; ++q) asm volatile("" : "+v"(qf[q]));
      __syncthreads();  // tile 0 visible
      // Half h: group 0 scores tile t in half 2t and does its P.V in half 2t + 1;
      // group 1 runs one half behind.  One block barrier per half, the same count in
      // both groups; each group's loop body is straight-line (scores, barrier, P.V,
      // barrier), so that the two roles' temporaries share registers.
      if (grp == 0) {
        for (int t = 0; t < n_tot; ++t) {
          score_tile(t);
          __syncthreads();
          // Tile t + 3 into the stage (8-bit: the staging slot) tile t - 1 left
          // (bf16: tiles 2 and 3 in half 1).
          if (FP8 || t > 0) {
            if (t + 3 < n_tot) issue(t + 3);
          } else {
            if (2 < n_tot) issue(2);
            if (3 < n_tot) issue(3);
          }
          wave_pv(smem + bstage(t) * kTileBytes, pgrp, vofs0, vofs1, pofs, wq, acc);
          if (t + 1 < n_tot) {
            wait_tiles(min(2, n_tot - 2 - t));  // tile t + 1 landed
            convert(t + 1);  // 8-bit: into the bf16 stage tile t - 1 left
          }
          __syncthreads();
        }
        __syncthreads();  // group 1's last P.V
      } else {
        __syncthreads();  // group 0's first scores
        for (int t = 0; t < n_tot; ++t) {
          score_tile(t);
          __syncthreads();
          wave_pv(smem + bstage(t) * kTileBytes, pgrp, vofs0, vofs1, pofs, wq, acc);
          __syncthreads();
        }
      }
      // One vote per pass: did some row raise its reference after its first tile?
      if (lane == 0) votes[0][wave] = __builtin_amdgcn_ballot_w64(need) != 0;
      __syncthreads();
      const int4 v0 = *(const int4*)&votes[0][0];
      const int4 v1 = *(const int4*)&votes[0][4];
      if ((v0.x | v0.y | v0.z | v0.w | v1.x | v1.y | v1.z | v1.w) == 0) break;
      // Restart with the raised reference maxima (they now bound every score of the
      // partition to within kHeadroom): drop what was accumulated.
      wait_vm<0>();
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) acc[ct][rt] = f32x16_t{};
      lsum = 0.f;
      lsr = 0.f;
      need = false;
      __syncthreads();  // every wave has read the votes before the next pass writes them
    }
  }

  // Rows' totals over the 4 key groups (lanes l, l ^ 16, l ^ 32, l ^ 48).
  lsum = sum_xor32(lsum);
  lsr = sum_xor32(lsr);
  lsum += __shfl_xor(lsum, 16, 64);
  lsr += __shfl_xor(lsr, 16, 64);
  // Per-row normaliser for the P.V waves (in the P buffer: every read of it is done).
  float* rinv = (float*)pbuf;
  __syncthreads();
  if (sg == 0) {
    float inv = 0.f;
    if (p.write_partials) {
      inv = lsum > 0.f ? 1.f / lsr : 0.f;
      if (row_ok) {
        const size_t prow = (size_t)pidx * (size_t)p.rows_total + (row0q + tok) * H + head;
        p.part_m[prow] = lsum > 0.f ? m * kLn2 : kNegInf;
        p.part_l[prow] = lsum;
      }
    } else {
      float M = m, L = lsum, Lr = lsr, c = 1.f;
      if (p.sink && row_ok) {
        const float sig = p.sink[head] * kLog2e;
        const float M2 = fmaxf(M, sig);
        c = fast_exp2(M - M2);
        const float e = fast_exp2(sig - M2);
        L = L * c + e;
        Lr = Lr * c + e;
        M = M2;
      }
      inv = L > 0.f ? c / Lr : 0.f;
      if (row_ok && p.lse)
        p.lse[(row0q + tok) * H + head] = L > 0.f ? (M + fast_log2(L)) * kLn2 : kNegInf;
    }
    if constexpr (FP8) inv *= p.v_scale;
    rinv[srow] = inv;
  }
  __syncthreads();
  // This wave's 128 columns of its group's rows: lane holds O^T[d = 128 wq + 32 ct +
  // 8 q + 4 hg + 0..3][row 64 grp + 32 rt + l31] in acc[ct][rt][4 q + 0..3].
  // fp32 partial rows: every partition's of an fp32-partial split, and partition
  // 0's of a bf16-partial one (layout in da_params.h).  They go through LDS like
  // the bf16 rows below, 32 rows at a time (32 x 528 bytes per wave of the idle
  // tile ring), so that each store writes the wave's 512 bytes of two rows instead
  // of 16 bytes of 32 rows.  A wave reads back only what it wrote; its LDS
  // operations stay in order, so the second half's writes follow the first half's
  // reads.
  if (p.write_partials && (!p.part_bf16 || pidx == 0)) {
    constexpr int kStgRowF = kCols * 4 + 16;  // 528
    static_assert(kWaves * 32 * kStgRowF <= kStages * kTileBytes, "staging fits the ring");
    char* stgf = smem + wave * (32 * kStgRowF);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const float inv = rinv[grp * kGroupRows + 32 * rt + l31];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(float4*)(stgf + l31 * kStgRowF + 4 * (32 * ct + 8 * q + 4 * hg)) =
              make_float4(acc[ct][rt][4 * q + 0] * inv, acc[ct][rt][4 * q + 1] * inv,
                          acc[ct][rt][4 * q + 2] * inv, acc[ct][rt][4 * q + 3] * inv);
#pragma unroll 4
      for (int i = 0; i < 16; ++i) {
        const int rl = 2 * i + (lane >> 5);  // row within the half
        const int r2 = mb * kRows + grp * kGroupRows + 32 * rt + rl;
        if (r2 >= nrows) continue;
        const size_t prow =
            (size_t)pidx * (size_t)p.rows_total + (row0q + r2 / H) * H + r2 % H;
        *(float4*)(p.part_o + prow * kDv + kCols * wq + 4 * (lane & 31)) =
            *(const float4*)(stgf + rl * kStgRowF + 16 * (lane & 31));
      }
    }
    return;
  }
  // bf16 rows (the output, or the partial rows of a long split) go through LDS, so
  // that each store writes whole 256-byte pieces of four rows instead of 16 bytes
  // of 32 rows.  Each wave stages its 64 rows x 128 columns in its own part of the
  // idle tile ring (no tile load is in flight and every tile read ended a barrier
  // ago), rows kStgRow bytes apart: the pad spreads the staging writes over the
  // banks.  A wave reads back only what it wrote.
  constexpr int kStgRow = kCols * 2 + 16;  // 272
  static_assert(kWaves * kGroupRows * kStgRow <= kStages * kTileBytes, "staging fits the ring");
  char* stg = smem + wave * (kGroupRows * kStgRow);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int rl = 32 * rt + l31;  // row within the group
    const float inv = rinv[grp * kGroupRows + rl];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(uint2*)(stg + rl * kStgRow + 2 * (32 * ct + 8 * q + 4 * hg)) =
            make_uint2(pack_bf16(acc[ct][rt][4 * q + 0] * inv, acc[ct][rt][4 * q + 1] * inv),
                       pack_bf16(acc[ct][rt][4 * q + 2] * inv, acc[ct][rt][4 * q + 3] * inv));
  }
  const int chunk = lane & 15;  // 16-byte piece of the wave's 256 bytes of a row
#pragma unroll 4
  for (int i = 0; i < kGroupRows / 4; ++i) {
    const int rl = 4 * i + (lane >> 4);
    const int r2 = mb * kRows + grp * kGroupRows + rl;
    if (r2 >= nrows) continue;
    const size_t orow = (row0q + r2 / H) * H + r2 % H;
    uint16_t* dst = (p.write_partials
                         ? (uint16_t*)p.part_o +
                               ((size_t)(pidx + 1) * (size_t)p.rows_total + orow) * kDv
                         : (uint16_t*)p.out + orow * kDv) +
                    kCols * wq + 8 * chunk;
    *(uint4*)dst = *(const uint4*)(stg + rl * kStgRow + 16 * chunk);
  }
}

template <bool FP8>
hipError_t launch_wave8(const DecodeParams& p, hipStream_t s) {
  const int n_mblocks = p.row_blocks;
  const int n_work = p.num_partitions * p.batch;
  const int grid = ((n_work + 7) / 8) * 8 * n_mblocks;
  if (n_mblocks == 1)
    hipLaunchKernelGGL((mla_wave8_kernel<FP8, true>), dim3(grid), dim3(kThreads), 0, s, p,
                       n_mblocks, n_work);
  else
    hipLaunchKernelGGL((mla_wave8_kernel<FP8, false>), dim3(grid), dim3(kThreads), 0, s, p,
                       n_mblocks, n_work);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mla_wave8(const DecodeParams& p, hipStream_t s) {
  return launch_wave8<false>(p, s);
}

hipError_t launch_mla_wave8_fp8(const DecodeParams& p, hipStream_t s) {
  return launch_wave8<true>(p, s);
}

}  // namespace da
