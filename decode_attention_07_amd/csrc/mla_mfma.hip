// mla_mfma.hip -- matrix-core sparse top-k MLA decode for gfx950 ("flare_mla_decoding_dispatch",
// Parameters `sparse`).
//
// One KV head, depth 576 for q.K^T, and V = K[..., :512] taken from the same
// cache rows (Args `k` and `kv_num_heads` of that page: V has no operand of its
// own).  The q_len tokens of a sequence and its num_q_heads heads
// are folded into one set of T*H rows (the MTP token fold); a block owns 128 of
// those rows (4 waves x 32 rows, one wave per SIMD) and one partition of the
// keys, so every cache row of the partition is read from HBM once per 128 rows.
//
// Per 32-key tile, shared by the block through a 4-stage LDS ring filled by
// direct global->LDS loads (no staging registers; tiles requested two ahead):
//   S^T[32 keys x 32 rows] = K[32 x 576] . Q^T[576 x 32]    36 v_mfma_f32_32x32x16_bf16
//       A = K from LDS, B = the wave's Q^T kept in registers for the whole
//       kernel (144 VGPRs).
//   softmax on the accumulator layout: lane l owns row l % 32 and 16 of the 32
//       keys, lane l ^ 32 the other 16.  Each row keeps a fixed reference max,
//       set by its first visible tile: p = 2^(s - m) may grow to 2^64 (so that a
//       weight times a value of the cache, summed over every key of a partition,
//       stays below fp32's 2^128 for |v| up to 2^40 at 2^20 keys), so O is never
//       rescaled inside the loop.  If a row ever exceeds its reference by more than that,
//       the block restarts its partition with the raised reference; each restart
//       lifts the row's reference above every score seen so far, so restarts
//       end, and for attention scores they do not occur in practice.
//   O^T[512 x 32 rows] += V^T[512 x 32 keys] . P^T[32 x 32]  32 MFMAs
//       A = V^T read by column from the same LDS tile, B = P^T taken straight
//       from the S^T accumulators (bf16); O^T lives in the 256 accumulation
//       registers.
// LDS tile layout: row-major in 16-byte chunks, chunk c of key k stored at
// position c ^ swz(k) of its 72-chunk row, swz(k) = 4 ((k / 2) % 2) + (k / 4) % 4.
// The XOR stays inside aligned groups of 8 chunks (one 128-byte line), so a
// stage is filled linearly: each 1 KB load instruction fetches 8 whole cache
// lines (which lets the loads carry the non-temporal hint).  swz() is chosen
// for gfx950's 64-bank LDS (measured with the bank-conflict counter): the K
// operand reads (16 keys x one chunk per 16 lanes) and the transposing V^T
// reads (4 keys x 64 bytes per 32 lanes) are both conflict-free.  swz(k + 16)
// = swz(k), swz(k + 8) differs.
// With two tokens (256 rows) a sequence needs two blocks that read the same
// tiles; their block ids differ by a multiple of 8 so that both land on the same
// XCD and the second read of each tile is served by that XCD's L2.
// The tile's 32 keys are gathered from a list of pool rows (their row indices
// reach LDS ahead of the tile).  The dense MLA forms (bf16 and 8-bit caches) run
// on the two-waves-per-SIMD kernel instead.
#include "da_device.h"

namespace da {

namespace {

constexpr int kD = 576;
constexpr int kDv = 512;
constexpr int kBN = 32;
constexpr int kWaves = 4;
constexpr int kWaveRows = 32;
constexpr int kRows = kWaveRows * kWaves;    // rows per block
constexpr int kThreads = 64 * kWaves;
constexpr int kKS = kD / 16;                 // 36 depth steps of 16
constexpr int kDT = kDv / 32;                // 16 output depth tiles of 32
constexpr int kRowBytes = kD * 2;            // 1152
constexpr int kCols = kRowBytes / 16;        // 72 columns of 16 bytes
constexpr int kTileBytes = kCols * kBN * 16; // 36 KB
constexpr int kDmaPerWave = kTileBytes / 1024 / kWaves;  // 9
static_assert(kDmaPerWave * kWaves * 1024 == kTileBytes, "tile must split into 1 KB pieces");
constexpr int kStages = 4;
constexpr float kHeadroom = 64.0f;           // largest exp2 argument (log2 units)

// 16 bytes per lane from base + voff straight into LDS (gfx950
// global_load_lds_dwordx4, scalar base + 32-bit vector offset): lane i of the
// wave writes lds_base + 16 * i.  The cache is streamed through once per block
// and every instruction covers whole lines: non-temporal hint (nt).  Issued
// through inline asm so that the compiler does not serialise later LDS reads of
// other stages behind it; completion is tracked with explicit vmcnt waits.  The
// LDS address goes in through an m0 operand, so the compiler computes it into m0
// directly (one scalar op per load).
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(base), "{m0}"(lds_base)
               : "memory");
}

__device__ __forceinline__ constexpr int swz(int key) { return 4 * ((key >> 1) & 1) + ((key >> 2) & 3); }

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt_hi[15:14]; expcnt left at its maximum).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Each lane's load offsets are computed once and kept in LDS (registers are all
// in use).
constexpr int kTabPerLane = 12;  // 9 used; 48 bytes per lane keeps 16-byte reads aligned

// Sparse top-k lists ("flare_mla_decoding_dispatch", Parameters `sparse`, Args
// `d_indices`, `indices_stride`, `topk_lengths`): the 32 keys of a tile are
// arbitrary pool rows, a gather at page size 1.  The stage layout stays the
// same; only the loads change.  Wave w fills keys 8w .. 8w + 7 of the tile: its
// load i (0..8) writes stage chunks 64 (9w + i) + lane, which is chunk position
// q = (64 i + lane) % 72 of key 8w + (64 i + lane) / 72.  One load spans at
// most two keys, sp_lo(i) below lane sp_split(i) and sp_lo(i) + 1 from it on;
// the byte offsets of the wave's 8 rows are uniform scalars, so a lane's
// offset is one of two scalars plus its fixed offset inside the row (in the
// table).  Offsets are 32-bit from the pool base: the pool holds at most
// 2^32 / 1152 rows, and each row index is clamped to the pool.
// The 8 row indices of a tile are copied to LDS three tile requests ahead of the
// tile's loads (lanes 0..7, 4 bytes each), into a ring of 4 slots per wave; the
// waits that let a tile's loads land cover them.
constexpr int kSpSlots = 4;

__device__ __forceinline__ constexpr int sp_lo(int i) { return (64 * i) / 72; }
__device__ __forceinline__ constexpr int sp_split(int i) { return 72 * (sp_lo(i) + 1) - 64 * i; }

__device__ __forceinline__ void dma_table_init_sparse(uint32_t* tab, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int cr = 64 * i + lane;  // chunk within the wave's 8 keys
    const int key = 8 * wave + cr / 72;
    const int q = cr % 72;
    tab[i] = 16u * (uint32_t)((q & ~7) | ((q & 7) ^ swz(key)));
  }
}

// 4 bytes per lane from base + voff into LDS at lds_base + 4 * lane
// (global_load_lds_dword).
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds_base) {
  asm volatile("global_load_lds_dword %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds_base)
               : "memory");
}

// Requests the row indices of tile t (keys k_lo + 32 t ..) of this wave into
// its slot.  Keys at or past kend take the partition's first key (a listed
// row, finite data; masked out of the softmax), so that the index reads stay
// inside the list.
__device__ __forceinline__ void sp_rows_issue(const DecodeParams& p, int b, int t, int k_lo,
                                              int kend, int wave, int lane, uint32_t slot) {
  const int key = k_lo + t * kBN + 8 * wave + (lane & 7);
  const int src = key < kend ? key : k_lo;
  // the list's base is uniform: pinned to scalar registers for the load
  const uint64_t base = pin_uniform_u64((uint64_t)(p.indices + (size_t)b * p.max_seq_len));
  if (lane < 8) dma4((const void*)base, 4u * (uint32_t)src, slot);
}

// Requests tile t of a sparse list into one LDS stage (and the indices of
// tile t + 3 into their slot): kDmaPerWave + 1 loads per wave.
__device__ __forceinline__ void mla_issue_sparse(const DecodeParams& p, uint32_t stage, int b,
                                                 int t, int k_lo, int kend, int wave, int lane,
                                                 const uint32_t* tab, const int32_t* slots,
                                                 uint32_t slots_lds) {
  const int32_t* mine = slots + ((t & (kSpSlots - 1)) * kWaves + wave) * 8;
  const int4 ra = *(const int4*)mine;
  const int4 rb = *(const int4*)(mine + 4);
  const int rw[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
  const uint32_t last = p.pool_rows - 1u;
  uint32_t off[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t r = (uint32_t)__builtin_amdgcn_readfirstlane(rw[e]);
    off[e] = (r < last ? r : last) * (uint32_t)kRowBytes;
  }
  sp_rows_issue(p, b, t + 3, k_lo, kend, wave, lane,
                slots_lds + (uint32_t)((((t + 3) & (kSpSlots - 1)) * kWaves + wave) * 32));
  const uint4 t0 = *(const uint4*)tab;
  const uint4 t1 = *(const uint4*)(tab + 4);
  const uint32_t e[kDmaPerWave] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w, tab[8]};
  const uint32_t dst = __builtin_amdgcn_readfirstlane(stage + wave * (kDmaPerWave * 1024));
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int lo = sp_lo(i);
    const uint32_t row = (lo == 7 || lane < sp_split(i)) ? off[lo] : off[lo + 1];
    dma16(p.k, row + e[i], dst + i * 1024);
  }
}

// The MFMAs are written as inline asm so that the register classes are fixed:
// the O^T accumulator in the 256 accumulation registers, Q^T and the score
// tiles in arch VGPRs (left to itself the compiler puts the score accumulators
// in AGPRs and then spills Q^T).  The compiler does not see inside the asm, so
// the hazards are covered here: a leading s_nop for a VALU write of A / B just
// before the MFMA, and mfma_settle() before any VALU or accvgpr read of a
// result.
//
// acc += A . B, acc in AGPRs.  NOP: a VALU may have written A or B just before.
template <bool NOP>
__device__ __forceinline__ void mfma_acc(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  if (NOP)
    asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                 : "+a"(acc)
                 : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Score tile s (= / +=) A . B with s in arch VGPRs (the AGPRs hold O^T).  The
// output is early-clobber: an MFMA destination may not overlap its A/B sources.
__device__ __forceinline__ void mfma_v_first(f32x16_t& s, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16_t& s, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+&v"(s) : "v"(a), "v"(b));
}

// Wait states between the last MFMA of a chain and a VALU / accvgpr read of its
// result (24; the compiler itself uses 12 for this instruction).  The results
// pass through the asm as operands, so that no read of them can be scheduled
// above the s_nops.
__device__ __forceinline__ void mfma_settle(f32x16_t& s0, f32x16_t& s1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s0), "+v"(s1));
}
__device__ __forceinline__ void mfma_settle(f32x16_t (&acc)[kDT]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) asm volatile("" : "+a"(acc[dt]));  // ordered after the nops
}

// acc = 0 without passing through arch VGPRs (0 * 0 + 0 in the matrix core).
__device__ __forceinline__ void zero_acc(f32x16_t& acc, const bf16x8_t& zero) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(zero));
}

// Key of accumulator element j (0..15) of lane half g in a 32x32 C tile.
__device__ __forceinline__ constexpr int c32_row(int j, int g) {
  return (j / 4) * 8 + g * 4 + (j % 4);
}

// Scores of one tile: S^T = K . Q^T.  The A operand of depth step st is chunk
// 2 st + g of key c32, at byte (kofs ^ 32 (st % 4)) + 128 (st / 4) of the stage
// (the swizzle only touches bits 4..6 of the offset).  Two accumulation chains
// (even / odd st); the K fragments come from a ring kPf pairs deep so that their
// LDS latency hides behind the MFMAs in flight.
template <int kPf>
__device__ __forceinline__ void mla_scores(const char* buf, const bf16x8_t (&qf)[kKS],
                                           uint32_t kofs, f32x16_t& s0, f32x16_t& s1) {
  auto kfrag = [&](int st) {
    return *(const bf16x8_t*)(buf + ((kofs ^ (32u * (st % 4))) + 128u * (st / 4)));
  };
  constexpr int kPairs = kKS / 2;
  bf16x8_t ra[kPf], rb[kPf];
#pragma unroll
  for (int q = 0; q < kPf; ++q) {
    ra[q] = kfrag(2 * q);
    rb[q] = kfrag(2 * q + 1);
  }
#pragma unroll
  for (int pq = 0; pq < kPairs; ++pq) {
    const int slot = pq % kPf;
    if (pq == 0) {
      mfma_v_first(s0, ra[slot], qf[0]);
      mfma_v_first(s1, rb[slot], qf[1]);
    } else {
      mfma_v(s0, ra[slot], qf[2 * pq]);
      mfma_v(s1, rb[slot], qf[2 * pq + 1]);
    }
    if (pq + kPf < kPairs) {
      ra[slot] = kfrag(2 * (pq + kPf));
      rb[slot] = kfrag(2 * (pq + kPf) + 1);
    }
  }
  mfma_settle(s0, s1);
}

// O^T += V^T . P^T for one tile, one fragment per call of step(f).  V^T operand
// of depth tile dt, key-half kh (fragment f: kh = f / 16, dt = f % 16, so that
// consecutive MFMAs update different accumulators): slots 0..3 hold keys
// 16 kh + 4 g + 0..3 and slots 4..7 keys 16 kh + 8 + 4 g + 0..3 (the P^T slot
// order), at d = 32 dt + (lane % 32).  Each half is one transposing read: lane i
// of 16-lane group G supplies &V[16 kh + 4 g + i / 4][32 dt + 16 (G % 2) +
// 4 (i % 4)], i.e. chunk 4 dt + cl of that key, byte 8 (i % 2), with
// cl = 2 (G % 2) + (i % 4) / 2.  swz() of a key does not change by +16, so two
// per-lane offsets (keys 4 g + i / 4 and those + 8) serve every fragment.  The V
// fragments come from a ring kPf deep.
struct MlaPV {
  static constexpr int kFrags = kDT * 2;
  static constexpr int kPf = 4;
  const char* buf;
  uint32_t vofs0, vofs1;
  uint2 vlo[kPf], vhi[kPf];

  __device__ __forceinline__ const char* frag(int f, uint32_t vofs) const {
    const int dt = f % kDT, kh = f / kDT;
    return buf + ((vofs ^ (64u * (dt % 2))) + 128u * (dt / 2) + 16u * kRowBytes * kh);
  }
  __device__ __forceinline__ void start(const char* b, uint32_t o0, uint32_t o1) {
    buf = b;
    vofs0 = o0;
    vofs1 = o1;
#pragma unroll
    for (int f = 0; f < kPf; ++f) {
      vlo[f] = lds_read_tr16(frag(f, vofs0));
      vhi[f] = lds_read_tr16(frag(f, vofs1));
    }
  }
  // NOP: the P^T operands may have been written by VALU ops just before.
  template <bool NOP>
  __device__ __forceinline__ void step(int f, f32x16_t (&acc)[kDT], const bf16x8_t (&pb)[2]) {
    const int slot = f % kPf;
    mfma_acc<NOP>(acc[f % kDT], concat_bf16x8(vlo[slot], vhi[slot]), pb[f / kDT]);
    if (f + kPf < kFrags) {
      vlo[slot] = lds_read_tr16(frag(f + kPf, vofs0));
      vhi[slot] = lds_read_tr16(frag(f + kPf, vofs1));
    }
  }
};

// Scores of the next tile, one depth step per call of step(st): two
// accumulation chains (even / odd depth steps), interleaved by the caller with
// the softmax and the P.V MFMAs of the current tile, so that no score MFMA waits
// for the one issued just before it.  The K fragments come from a ring kPf deep
// (same operand layout as mla_scores).
template <int kPf>
struct MlaQK {
  const char* buf;
  uint32_t kofs;
  bf16x8_t ring[kPf];

  __device__ __forceinline__ bf16x8_t frag(int st) const {
    return *(const bf16x8_t*)(buf + ((kofs ^ (32u * (st % 4))) + 128u * (st / 4)));
  }
  __device__ __forceinline__ void start(const char* b, uint32_t o) {
    buf = b;
    kofs = o;
#pragma unroll
    for (int q = 0; q < kPf; ++q) ring[q] = frag(q);
  }
  __device__ __forceinline__ void step(int st, f32x16_t& s0, f32x16_t& s1,
                                       const bf16x8_t (&qf)[kKS]) {
    const int slot = st % kPf;
    f32x16_t& s = (st & 1) ? s1 : s0;
    if (st < 2)
      mfma_v_first(s, ring[slot], qf[st]);
    else
      mfma_v(s, ring[slot], qf[st]);
    if (st + kPf < kKS) ring[slot] = frag(st + kPf);
  }
};

__device__ __forceinline__ void mfma_settle(f32x16_t& s) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
}

// One tile of the loop: the softmax of tile i's scores x into bf16 weights, the
// P.V contraction of tile i (V rows in vbuf) and, when NEXT, the scores of tile
// i + 1 (K rows in kbuf), which replace x.  The score MFMAs of tile i + 1 run
// beside the vector work of the softmax and between the P.V MFMAs, so the matrix
// core always has independent work queued: the scores form two chains, the P.V
// MFMAs update 16 different accumulators.
//
// Softmax on the accumulator layout: lane l owns row l % 32 and 16 of the 32
// keys, lane l ^ 32 the other 16.  Each row keeps a fixed reference max, set by
// its first visible tile: p = 2^(s - m) may grow to 2^64 (weight x value sums stay
// far below fp32's 2^128), so O is never rescaled inside the loop.
// If a row ever exceeds its reference by more than that, the block restarts its
// partition with the raised reference.  The weights enter the MFMA rounded to
// bf16; their rounded sum (lsr) is what O is normalised by, so the effective
// weights still sum to one.
//
// The scale enters once per weight, p = 2^(fma(q.k, sl, -m)) with sl = scale *
// log2(e) >= 0 (a negative scale was moved into Q by flipping its sign), and the
// row max is taken over the unscaled scores (sl >= 0 keeps their order).  Only
// tiles that reach past some row's last visible key (MASKED) compare keys:
// element j of lane half g holds key c32_row(j, g) = c32_row(j, 0) + 4 g of the
// tile, visible when c32_row(j, 0) < lim = (row's key limit) - (tile's first key)
// - 4 g.
template <bool NEXT, bool MASKED, int kPf>
__device__ __forceinline__ void mla_step(float (&x)[16], const char* kbuf, const char* vbuf,
                                         const bf16x8_t (&qf)[kKS], uint32_t kofs,
                                         uint32_t vofs0, uint32_t vofs1, f32x16_t (&acc)[kDT],
                                         float& m, float& lsum, float& lsr, int lim, float sl,
                                         bool& restart) {
  MlaQK<kPf> qk;
  f32x16_t s0, s1;
  if (NEXT) qk.start(kbuf, kofs);
  int st = 0;
  // One score MFMA of the next tile; the scheduling barrier keeps the compiler
  // from regrouping the interleaved vector and matrix work.
  auto qk_step = [&]() {
    if (NEXT && st < kKS) {
      qk.step(st, s0, s1, qf);
      ++st;
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // The running max and sums pass through an empty volatile asm at their place in
  // the interleave: volatile asm keeps its order, so the arithmetic they depend
  // on cannot be sunk below the MFMAs it is meant to run beside.
  auto pin = [](float& v) { asm volatile("" : "+v"(v)); };
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    mx = fmaxf(mx, (!MASKED || c32_row(j, 0) < lim) ? x[j] : kNegInf);
    if (j % 2 == 1) {
      pin(mx);
      qk_step();
    }
  }
  mx = max_xor32(mx);
  mx = (mx == kNegInf) ? kNegInf : mx * sl;
  pin(mx);
  qk_step();
  const bool grow = mx > m + kHeadroom;
  restart = restart || (grow && m != kNegInf);  // a row's first visible tile: acc is still 0
  m = grow ? mx : m;
  float nms = (m == kNegInf) ? 0.f : -m;
  pin(nms);
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    x[j] = fast_exp2(fmaf(x[j], sl, nms));
    if (MASKED) x[j] = (c32_row(j, 0) < lim) ? x[j] : 0.f;
    ps += x[j];
    if (j % 2 == 1) {
      pin(ps);
      qk_step();
    }
  }
  lsum += ps;
  bf16x8_t pb[2];
  float pr = 0.f;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[q] = pack_bf16(x[8 * kh + 2 * q], x[8 * kh + 2 * q + 1]);
      pr = dot2_bf16(w[q], 0x3f803f80u, pr);  // + both rounded weights (times bf16 1.0)
      pin(pr);
      qk_step();
    }
    pb[kh] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
  }
  lsr += pr;
  // P.V of this tile (its weights were just written by vector ops: the first two
  // MFMAs that read them wait), the rest of the next tile's scores in between.
  // Its V fragments are requested only now (x is dead, so their registers are
  // free); three score MFMAs cover the read latency.
  MlaPV pv;
  pv.start(vbuf, vofs0, vofs1);
  qk_step();
  qk_step();
  qk_step();
  pv.step<true>(0, acc, pb);
  qk_step();
  pv.step<true>(1, acc, pb);
  qk_step();
#pragma unroll
  for (int f = 2; f < MlaPV::kFrags; ++f) {
    pv.step<false>(f, acc, pb);
    qk_step();
  }
#pragma unroll
  for (int r = 0; r < kKS; ++r) qk_step();  // none left when the P.V slots sufficed
  if (NEXT) {
    mfma_settle(s0, s1);
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = s0[j] + s1[j];
  }
}

template <bool V>
struct BoolTag {
  static constexpr bool value = V;
};

// Keys from a top-k list of pool rows (p.indices).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_kernel(DecodeParams p, int n_mblocks, int n_work) {
  constexpr int kIssue = kDmaPerWave + 1;  // loads per wave per tile request (the tile, its indices)
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kTileBytes];
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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c32 = lane & 31, g = lane >> 5;
  const int H = p.num_q_heads;
  const int nrows = seq_tokens(p, b) * H;  // this sequence's token x head rows
  if (mb * kRows >= nrows) return;  // ragged q: none of this block's rows exist (no barrier yet)
  const size_t row0q = seq_row0(p, b);

  const int rr = mb * kRows + wave * kWaveRows + c32;
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
  // (uniform; pinned to scalar registers so that the per-tile key counts derived
  // from them stay scalar too)
  const int hmin =
      __builtin_amdgcn_readfirstlane(max(k_lo, min(k_end, visible_keys(p, b, t_first))));
  const int hmax =
      __builtin_amdgcn_readfirstlane(max(k_lo, min(k_end, visible_keys(p, b, t_last))));

  // Q^T operand: k-slot (g, j) of depth step st <-> depth 16*st + 8*g + j.
  bf16x8_t qf[kKS];
  const uint16_t* qrow =
      (const uint16_t*)p.q + ((row0q + tok) * H + head) * (size_t)kD;
#pragma unroll
  for (int s = 0; s < kKS; ++s)  // rows past the fold read row (b, 0, 0) and are zeroed later
    qf[s] = *(const bf16x8_t*)(qrow + s * 16 + g * 8);

  f32x16_t acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) acc[dt] = f32x16_t{};
  float m = kNegInf, lsum = 0.f, lsr = 0.f;  // exact and bf16-rounded weight sums

  const int n_full = (hmin - k_lo) / kBN;
  const int n_tot = (hmax - k_lo + kBN - 1) / kBN;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  // Per-lane LDS offsets of the operand reads (see mla_scores / MlaPV).
  const uint32_t kofs = kRowBytes * c32 + ((16u * g) ^ (16u * swz(c32)));
  const int G = lane >> 4, i16 = lane & 15;
  const int cl = 2 * (G & 1) + ((i16 & 3) >> 1);
  const int vkey = 4 * g + (i16 >> 2);
  const uint32_t vofs0 = kRowBytes * vkey + ((16u * cl) ^ (16u * swz(vkey))) + 8u * (i16 & 1);
  const uint32_t vofs1 =
      kRowBytes * (vkey + 8) + ((16u * cl) ^ (16u * swz(vkey + 8))) + 8u * (i16 & 1);
  // 4-stage ring, software-pipelined: the scores of tile 0 come first; then
  // iteration i takes the softmax and the P.V of tile i while the matrix core
  // also computes the scores of tile i + 1, so stages i and i + 1 are being read;
  // tile i + 3 is requested into the stage tile i - 1 left, and before each
  // barrier a wave waits until only tile i + 3's requests are outstanding (tile
  // i + 2 landed).
  // Restart votes: each wave writes its own slot for tile i (every tile, 0 or 1)
  // into buffer i & 1 before the tile's barrier; the slots of tile i - 1 are
  // read at the top of tile i, so a read and the next write of the same buffer
  // (tile i + 1) are always a barrier apart and every wave sees the same votes.
  __shared__ __attribute__((aligned(16))) int votes[2][kWaves];
  __shared__ __attribute__((aligned(16))) uint32_t dma_tab[kThreads * kTabPerLane];
  const uint32_t* tab = dma_tab + threadIdx.x * kTabPerLane;  // this lane's own entries
  dma_table_init_sparse(dma_tab + threadIdx.x * kTabPerLane, wave, lane);
  auto bstage = [&](int t) __attribute__((always_inline)) { return t & (kStages - 1); };
  // Sparse lists: row indices of tiles t, t + 1, t + 2 sit in slots t % 4 ..
  // (t + 2) % 4 when tile t is requested.
  __shared__ __attribute__((aligned(16))) int32_t sp_slots[kSpSlots * kWaves * 8];
  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t stage = lds0 + (uint32_t)((t & (kStages - 1)) * kTileBytes);
    mla_issue_sparse(p, stage, b, t, k_lo, hmax, wave, lane, tab, sp_slots,
                     (uint32_t)(uintptr_t)sp_slots);
  };
  // Sparse lists: the indices of tiles 0, 1 and 2, waited for before tile 0 is
  // requested.
  auto prime = [&]() __attribute__((always_inline)) {
    for (int t = 0; t < 3; ++t)
      sp_rows_issue(p, b, t, k_lo, hmax, wave, lane,
                    (uint32_t)(uintptr_t)sp_slots + (uint32_t)((t * kWaves + wave) * 32));
    wait_vm_lgkm0<0>();
  };
  // Start of a pass: tiles 0, 1 and 2 requested (those that exist) and tile 0
  // landed, with whatever was requested before it (the Q rows on the first pass).
  auto start_pass = [&]() __attribute__((always_inline)) {
    prime();
    issue(0);
    if (n_tot > 2) {
      issue(1);
      issue(2);
      wait_vm_lgkm0<2 * kIssue>();
    } else if (n_tot > 1) {
      issue(1);
      wait_vm_lgkm0<kIssue>();
    } else {
      wait_vm_lgkm0<0>();
    }
  };
  if (n_tot > 0) {
    // Tile 0 is requested while the Q loads are in flight; start_pass waits for
    // both.
    start_pass();
    // Rows outside the fold get Q = 0; a negative scale flips Q's sign (exact).
    const uint32_t qx = p.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
      uint4 u = __builtin_bit_cast(uint4, qf[s]);
      u = make_uint4(u.x ^ qx, u.y ^ qx, u.z ^ qx, u.w ^ qx);
      qf[s] = row_ok ? __builtin_bit_cast(bf16x8_t, u) : bf16x8_t{};
    }
    const float sl = fabsf(p.scale_log2);
    const int hi4 = hi - 4 * g;  // the row's key limit, less the lane half's key offset
    // K fragments in flight
    constexpr int kKPf = 3;
    for (;;) {  // one pass over the partition; repeated only after a restart
      __syncthreads();  // tile 0 is in LDS for every wave
      float x[16];      // scores of the tile the loop is at
      {
        f32x16_t s0, s1;
        mla_scores<kKPf>(smem + bstage(0) * kTileBytes, qf, kofs, s0, s1);
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = s0[j] + s1[j];
      }
      // tile 1 landed; tile 2 may stay in flight
      if (n_tot > 1) {
        if (n_tot > 2)
          wait_vm_lgkm0<kIssue>();
        else
          wait_vm_lgkm0<0>();
      }
      __syncthreads();
      // One tile: returns true when the votes of the tile before it ask for a
      // restart.  NEXT: the scores of tile i + 1 are computed alongside; MASKED:
      // compare keys against each row's last visible key.  The tiles every row
      // sees whole, the rest but the last, and the last are three loops, so that
      // each loop body holds a single copy of the interleave (registers are all
      // in use).
      auto tile = [&](int i, auto next_tag, auto mask_tag) __attribute__((always_inline)) {
        constexpr bool NEXT = decltype(next_tag)::value;
        constexpr bool MASKED = decltype(mask_tag)::value;
        // Votes of tile i - 1, acted upon after tile i (the load has landed by
        // then; what tile i adds is dropped with the rest on a restart).
        int4 prev = make_int4(0, 0, 0, 0);
        if (i > 0) prev = *(const int4*)votes[(i - 1) & 1];
        const bool ahead = i + 3 < n_tot;
        if (ahead) issue(i + 3);  // into the stage of tile i - 1, last read a barrier ago
        bool need = false;
        mla_step<NEXT, MASKED, kKPf>(x, smem + bstage(i + 1) * kTileBytes,
                                     smem + bstage(i) * kTileBytes, qf, kofs, vofs0, vofs1, acc,
                                     m, lsum, lsr, hi4 - (k_lo + i * kBN), sl, need);
        if (lane == 0) votes[i & 1][wave] = __builtin_amdgcn_ballot_w64(need) != 0;
        // tile i + 2 must have landed: tile i + 3 may stay in flight
        if (ahead)
          wait_vm_lgkm0<kIssue>();
        else
          wait_vm_lgkm0<0>();
        __syncthreads();
        return (prev.x | prev.y | prev.z | prev.w) != 0;  // same votes in every wave
      };
      const int n_body = min(n_full, n_tot - 1);
      bool again = false;
      int i = 0;
      for (; !again && i < n_body; ++i) again = tile(i, BoolTag<true>{}, BoolTag<false>{});
      for (; !again && i < n_tot - 1; ++i) again = tile(i, BoolTag<true>{}, BoolTag<true>{});
      if (!again) {
        again = tile(n_tot - 1, BoolTag<false>{}, BoolTag<true>{});
        if (!again) {  // the last tile's votes, written before the barrier it ended on
          const int4 last = *(const int4*)votes[(n_tot - 1) & 1];
          if (!(last.x | last.y | last.z | last.w)) break;
        }
      }
      // Restart with the raised reference maxima: drop what was accumulated.
      wait_vm_lgkm0<0>();
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) zero_acc(acc[dt], bf16x8_t{});
      lsum = 0.f;
      lsr = 0.f;
      __syncthreads();  // every wave has read the votes before the next pass writes them
      start_pass();  // tiles 0 .. 2 of the next pass
    }
  }

  mfma_settle(acc);
  lsum = sum_xor32(lsum);
  lsr = sum_xor32(lsr);
  const size_t row = (row0q + tok) * H + head;
  // Lane holds O^T[d = 32*dt + 8*(j/4) + 4*g + j%4][row]: 4 consecutive d per j/4.
  const size_t prow = (size_t)pidx * (size_t)p.rows_total + row;
  // fp32 partial rows: every partition's of an fp32-partial split, and partition
  // 0's of a bf16-partial one (layout in da_params.h)
  if (p.write_partials && (!p.part_bf16 || pidx == 0)) {
    if (!row_ok) return;
    const bool any = lsum > 0.f;
    const float inv = any ? 1.f / lsr : 0.f;
    float* dst = p.part_o + prow * kDv;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(float4*)(dst + dt * 32 + q4 * 8 + g * 4) =
            make_float4(acc[dt][4 * q4 + 0] * inv, acc[dt][4 * q4 + 1] * inv,
                        acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv);
    if (g == 0) {
      p.part_m[prow] = any ? m * kLn2 : kNegInf;
      p.part_l[prow] = lsum;
    }
    return;
  }
  // bf16 rows: the output, or the partial rows of a long split.
  float inv = 0.f;
  if (row_ok) {
    if (p.write_partials) {
      const bool any = lsum > 0.f;
      inv = any ? 1.f / lsr : 0.f;
      if (g == 0) {
        p.part_m[prow] = any ? m * kLn2 : kNegInf;
        p.part_l[prow] = lsum;
      }
    } else {
      float M = m, L = lsum, Lr = lsr, c = 1.f;
      if (p.sink) {
        const float sig = p.sink[head] * kLog2e;
        const float M2 = fmaxf(M, sig);
        c = fast_exp2(M - M2);
        const float e = fast_exp2(sig - M2);
        L = L * c + e;
        Lr = Lr * c + e;
        M = M2;
      }
      const bool any = L > 0.f;
      inv = any ? c / Lr : 0.f;
      if (g == 0 && p.lse) p.lse[row] = any ? (M + fast_log2(L)) * kLn2 : kNegInf;
    }
  }
  // The rows go through LDS, so that each store writes one whole 1 KB row instead
  // of 16 bytes of 32 rows (and a single bf16 store loop: a second one made the
  // allocator spill most of the accumulators).  Each wave stages its 32 rows in its
  // own part of the idle tile ring (no load is in flight and every tile read ended
  // a barrier ago), rows kStgRow bytes apart: the pad spreads the staging writes
  // over the banks.  A wave reads back only what it wrote.
  constexpr int kStgRow = kDv * 2 + 16;  // 1040
  static_assert(kWaves * kWaveRows * kStgRow <= kStages * kTileBytes, "staging fits the ring");
  char* stg = smem + wave * (kWaveRows * kStgRow);
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *(uint2*)(stg + c32 * kStgRow + 2 * (dt * 32 + q4 * 8 + g * 4)) =
          make_uint2(pack_bf16(acc[dt][4 * q4 + 0] * inv, acc[dt][4 * q4 + 1] * inv),
                     pack_bf16(acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv));
  for (int i = 0; i < kWaveRows; ++i) {
    const int r2 = mb * kRows + wave * kWaveRows + i;
    if (r2 >= nrows) break;  // the wave's rows are consecutive
    const size_t orow = (row0q + r2 / H) * H + r2 % H;
    uint16_t* dst = (p.write_partials
                         ? (uint16_t*)p.part_o +
                               ((size_t)(pidx + 1) * (size_t)p.rows_total + orow) * kDv
                         : (uint16_t*)p.out + orow * kDv) +
                    8 * lane;
    *(uint4*)dst = *(const uint4*)(stg + i * kStgRow + 16 * lane);
  }
}

}  // namespace

int mla_rows_per_block(int, int) { return kRows; }
int mla_step_keys(int) { return kBN; }

hipError_t launch_mla_sparse(const DecodeParams& p, hipStream_t s) {
  if (!p.indices) return hipErrorInvalidValue;
  const int n_mblocks = p.row_blocks;
  const int n_work = p.num_partitions * p.batch;
  const int grid = ((n_work + 7) / 8) * 8 * n_mblocks;
  hipLaunchKernelGGL(mla_decode_kernel, dim3(grid), dim3(kThreads), 0, s, p, n_mblocks, n_work);
  return hipGetLastError();
}

}  // namespace da
