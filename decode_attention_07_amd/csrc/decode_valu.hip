// decode_valu.hip -- split-K decode attention on the vector ALUs (gfx950).
//
// Used for fp32 inputs, which have no matrix-core path at this precision here
// (bf16 runs the streaming matrix-core kernel).  The element type stays a
// template parameter; only fp32 is instantiated.  One block
// of 4 waves handles one (partition, batch, KV head, row block): every query
// row that shares the KV head is folded into the block, so each KV byte of the
// partition is read from HBM exactly once.
//
// FA2 online softmax (description of "mha_decoding_single_batch_pipelined"):
// the block walks its contiguous key slice; a running max m, exp-sum l and
// rescaled accumulator o per row absorb each key tile; at the end the block
// either writes the finished row (one partition) or the partial (o / l, m, l)
// for the log-sum-exp merge pass.
//
// Lane layout: a key row of D elements is read by 8 consecutive lanes, 16 bytes
// per lane per load, so each load instruction of a wave covers 8 key rows and
// each 8-lane group reads whole 128-byte lines.  A wave therefore works on 8
// keys at a time ("slots"); the block on 32.  Each slot keeps its own (m, l, o)
// so the hot loop needs no cross-slot traffic: a q.k dot product is reduced
// across its 8 lanes with three DPP adds, and the value row sits in the same
// lanes that hold its score.  Slots are merged once, at the end, by
// log-sum-exp (wave shuffles, then LDS across the 4 waves).
//
// Software pipelining: the K/V rows of the next tile are requested before the
// current tile is processed, so every lane keeps 2*U key rows in flight.
#include "da_merge.h"

namespace da {

namespace {

// ---- merge inside the pass (small split calls) ----------------------------------
// The P partition blocks of a row group may run on different XCDs, whose L2 caches
// are not coherent with each other within a launch: the partial values are stored
// and read back with device-scope (agent) relaxed atomic accesses, which go past
// each XCD's L2 state, and a count word tells the last block that every other
// block's stores have completed.  No release fence (an agent-scope release writes
// back the XCD's whole L2).
typedef __attribute__((address_space(1))) float global_f32;
typedef __attribute__((address_space(1))) unsigned global_u32;
__device__ __forceinline__ void st_agent(float* a, float v) {
  __hip_atomic_store((global_f32*)a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* a) {
  return __hip_atomic_load((global_f32*)a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct ValuMergeArgs {
  const float* po;     // part_o [P, rows_total, D]
  const float* pm;     // part_m [P, rows_total]
  const float* pl;     // part_l [P, rows_total]
  const float* sink;   // [num_q_heads] or nullptr
  float* out;          // [rows_total, D]
  float* lse;          // [rows_total] or nullptr
  size_t rows_total;
  size_t row0q;        // q / out token row of the sequence's first token
  int num_q_heads, group, g, rb, R, nrows, P;
};

// After a block has stored its partial rows: every thread waits for its stores to
// complete, one thread counts the block in its row group's word (an add that wraps
// to zero on the P-th, so the word is zero again after the call), and the block
// whose add completes the count merges the group's rows, one wave per row.  The
// merge is the merge pass's one-wave row merge (at most 32 partitions here), the
// same operations in the same order ("mha_decoding_single_batch_pipelined",
// description: the mha_splitk_reduce pass): M = max(max_p m_p, sigma), w_p = l_p
// exp(m_p - M), out = sum_p w_p O_p / (sum_p w_p + exp(sigma - M)), lse = M + ln L.
// (A function of its own: inlined, its values would join the register allocation
// of the kernel's key loop.)  `flag`: one int of LDS.
// One row group's rows, one wave per row, with NP >= P slots: every slot's partial
// row is requested at once (a slot past P re-reads partition 0 and gets weight 0),
// so a row costs one memory round trip.
template <int D, int NP>
__device__ __forceinline__ void valu_merge_rows(const ValuMergeArgs& a, int wave, int lane) {
  constexpr int EPL = D / 64;
  for (int r = wave; r < a.R; r += 4) {
    const int rr = a.rb * a.R + r;
    if (rr >= a.nrows) break;  // uniform in the wave; later rows are past the fold too
    const int h = a.g * a.group + rr % a.group;
    const size_t row = (a.row0q + (size_t)(rr / a.group)) * a.num_q_heads + h;
    const int pc = lane < a.P ? lane : 0;
    const float lp_raw = ld_agent(a.pl + (size_t)pc * a.rows_total + row);
    const float mp_raw = ld_agent(a.pm + (size_t)pc * a.rows_total + row);
    float c[NP][EPL];
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const float* src =
          a.po + ((size_t)(u < a.P ? u : 0) * a.rows_total + row) * D + lane * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) c[u][e] = ld_agent(src + e);
    }
    const float sig = a.sink ? a.sink[h] * kLog2e : kNegInf;
    const float lp = lane < a.P ? lp_raw : 0.f;
    const float M = fmaxf(wave_max(lp > 0.f ? mp_raw * kLog2e : kNegInf), sig);
    const float Ms = (M == kNegInf) ? 0.f : M;
    const float w = lp > 0.f ? lp * fast_exp2(mp_raw * kLog2e - Ms) : 0.f;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const float wj =
          u < a.P ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u)) : 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float t = fmaf(wj, c[u][e], acc[e]);
        acc[e] = (wj != 0.f) ? t : acc[e];
      }
    }
    float L = wave_sum(w);
    if (a.sink) L += fast_exp2(sig - Ms);
    const bool any = L > 0.f;
    const float inv = any ? 1.f / L : 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a.out[row * D + lane * EPL + e] = acc[e] * inv;
    if (a.lse && lane == 0) a.lse[row] = any ? (M + fast_log2(L)) * kLn2 : kNegInf;
  }
}

// After a block has stored its partial rows: every thread waits for its stores to
// complete, one thread counts the block in its row group's word (an add that wraps
// to zero on the P-th, so the word is zero again after the call), and the block
// whose add completes the count merges the group's rows.  The merge is the merge
// pass's one-wave row merge (at most 8 partitions here), the same operations in
// the same order ("mha_decoding_single_batch_pipelined", description: the
// mha_splitk_reduce pass): M = max(max_p m_p, sigma), w_p = l_p exp(m_p - M), out =
// sum_p w_p O_p / (sum_p w_p + exp(sigma - M)), lse = M + ln L.  (A function of its
// own: inlined, its values would join the register allocation of the kernel's key
// loop.)  `flag`: one int of LDS.
template <int D>
__device__ __attribute__((noinline)) void valu_count_and_merge(const ValuMergeArgs a,
                                                               unsigned* cnt, int* flag,
                                                               int wave, int lane) {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t top = (uint32_t)a.P - 1u;
    *flag = __builtin_amdgcn_atomic_inc32((global_u32*)cnt, top, __ATOMIC_RELAXED, "agent") == top
                ? 1
                : 0;
  }
  __syncthreads();
  if (!*flag) return;
  if (a.P <= 4)
    valu_merge_rows<D, 4>(a, wave, lane);
  else
    valu_merge_rows<D, 8>(a, wave, lane);
}

}  // namespace

template <bool BF16, int D, int R, int U>
struct ValuCfg {
  static constexpr int ESZ = BF16 ? 2 : 4;          // bytes per element
  static constexpr int L = 8;                        // lanes per key row
  static constexpr int ROW_BYTES = D * ESZ;
  static constexpr int NV = ROW_BYTES / (L * 16);    // 16-byte loads per lane per row
  static constexpr int EPV = 16 / ESZ;               // elements per 16-byte load
  static constexpr int EPL = NV * EPV;               // elements per lane per row
  static constexpr int WAVES = 4;
  static constexpr int SLOTS = WAVES * 64 / L;        // key slots per block (32)
  static constexpr int STEP = SLOTS * U;              // keys per block iteration
  static_assert(NV >= 1 && NV * L * 16 == ROW_BYTES, "row must split into 8 lanes x 16 B");
};

// Depth index of element e held by lane `part`.
template <class C>
__device__ __forceinline__ int lane_depth(int part, int e) {
  return ((e / C::EPV) * C::L + part) * C::EPV + (e % C::EPV);
}

template <bool BF16, int D, int R, int U>
struct ValuTile {
  using C = ValuCfg<BF16, D, R, U>;
  uint4 k[U][C::NV];
  uint4 v[U][C::NV];
};

template <bool BF16, int D, int R, int U, bool MASKED>
__device__ __forceinline__ void valu_load(const DecodeParams& p, ValuTile<BF16, D, R, U>& t,
                                          int b, int g, int kb, int wave, int slot, int part,
                                          int kend) {
  using C = ValuCfg<BF16, D, R, U>;
  const char* kbase = (const char*)p.k;
  const char* vbase = (const char*)p.v;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int jbase = kb + u * C::SLOTS;  // uniform; 32-key group inside one page
    if (MASKED && jbase >= kend) {        // whole group past the limit: no address formed
#pragma unroll
      for (int vv = 0; vv < C::NV; ++vv) {
        t.k[u][vv] = make_uint4(0, 0, 0, 0);
        t.v[u][vv] = make_uint4(0, 0, 0, 0);
      }
      continue;
    }
    size_t row0;
    if (p.page_table) {
      uint32_t phys = p.page_table[(size_t)b * p.max_pages + (jbase >> p.page_shift)];
      row0 = ((size_t)phys << p.page_shift) + (size_t)(jbase & ((1 << p.page_shift) - 1));
    } else {
      row0 = seq_kv_row0(p, b) + jbase;
    }
    const int jl = wave * 8 + slot;
    const size_t elem = ((row0 + jl) * p.num_kv_heads + g) * (size_t)D;
    const bool ok = !MASKED || (jbase + jl < kend);
#pragma unroll
    for (int vv = 0; vv < C::NV; ++vv) {
      const size_t off = (elem + (size_t)(vv * C::L + part) * C::EPV) * C::ESZ;
      if (ok) {
        t.k[u][vv] = *(const uint4*)(kbase + off);
        t.v[u][vv] = *(const uint4*)(vbase + off);
      } else {
        t.k[u][vv] = make_uint4(0, 0, 0, 0);
        t.v[u][vv] = make_uint4(0, 0, 0, 0);
      }
    }
  }
}

template <bool BF16, int D, int R, int U, bool MASKED>
__device__ __forceinline__ void valu_process(const ValuTile<BF16, D, R, U>& t,
                                             const uint4 (&qv)[R][ValuCfg<BF16, D, R, U>::NV],
                                             float (&m)[R], float (&l)[R],
                                             float (&o)[R][ValuCfg<BF16, D, R, U>::EPL],
                                             const int (&hi)[R], const bool (&row_ok)[R],
                                             int kb, int jl, float scale_log2) {
  using C = ValuCfg<BF16, D, R, U>;
  float s[R][U];
  // q.k partial dot products over this lane's EPL elements.
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int vv = 0; vv < C::NV; ++vv) {
        const uint4 kk = t.k[u][vv];
        const uint4 qq = qv[r][vv];
        if constexpr (BF16) {
          acc = dot2_bf16(qq.x, kk.x, acc);
          acc = dot2_bf16(qq.y, kk.y, acc);
          acc = dot2_bf16(qq.z, kk.z, acc);
          acc = dot2_bf16(qq.w, kk.w, acc);
        } else {
          acc = fmaf(__uint_as_float(qq.x), __uint_as_float(kk.x), acc);
          acc = fmaf(__uint_as_float(qq.y), __uint_as_float(kk.y), acc);
          acc = fmaf(__uint_as_float(qq.z), __uint_as_float(kk.z), acc);
          acc = fmaf(__uint_as_float(qq.w), __uint_as_float(kk.w), acc);
        }
      }
      s[r][u] = acc;
    }
  }
  // Reduce each dot product over the 8 lanes of its key row (all 8 get it).
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x = sum8(s[r][u]) * scale_log2;
      if (MASKED) x = (kb + u * C::SLOTS + jl < hi[r]) ? x : kNegInf;
      s[r][u] = x;
    }
  // Value rows to fp32 once, shared by every query row.
  float vf[U][C::EPL];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int vv = 0; vv < C::NV; ++vv) {
      const uint4 w = t.v[u][vv];
      if constexpr (BF16) {
        vf[u][vv * 8 + 0] = bf16lo(w.x); vf[u][vv * 8 + 1] = bf16hi(w.x);
        vf[u][vv * 8 + 2] = bf16lo(w.y); vf[u][vv * 8 + 3] = bf16hi(w.y);
        vf[u][vv * 8 + 4] = bf16lo(w.z); vf[u][vv * 8 + 5] = bf16hi(w.z);
        vf[u][vv * 8 + 6] = bf16lo(w.w); vf[u][vv * 8 + 7] = bf16hi(w.w);
      } else {
        vf[u][vv * 4 + 0] = __uint_as_float(w.x); vf[u][vv * 4 + 1] = __uint_as_float(w.y);
        vf[u][vv * 4 + 2] = __uint_as_float(w.z); vf[u][vv * 4 + 3] = __uint_as_float(w.w);
      }
    }
  // Online softmax update per row.
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (!row_ok[r]) continue;
    float mx = s[r][0];
#pragma unroll
    for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[r][u]);
    const float mn = fmaxf(m[r], mx);
    const float ms = (mn == kNegInf) ? 0.f : mn;
    const float alpha = fast_exp2(m[r] - ms);
    m[r] = mn;
    float lr = l[r] * alpha;
#pragma unroll
    for (int e = 0; e < C::EPL; ++e) o[r][e] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pu = fast_exp2(s[r][u] - ms);
      lr += pu;
#pragma unroll
      for (int e = 0; e < C::EPL; ++e) o[r][e] = fmaf(pu, vf[u][e], o[r][e]);
    }
    l[r] = lr;
  }
}

// merge_count: nullptr, or the count words of a split merged inside the pass (one
// per (sequence, KV head, row block), zero between calls).
template <bool BF16, int D, int R, int U>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeParams p, unsigned* merge_count) {
  using C = ValuCfg<BF16, D, R, U>;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id_uniform();
  const int slot = lane >> 3;
  const int part = lane & 7;
  const int jl = wave * 8 + slot;

  // Block -> (partition, batch, KV head, row block); partition slowest.
  int id = blockIdx.x;
  const int rb = id % p.row_blocks; id /= p.row_blocks;
  const int g = id % p.num_kv_heads; id /= p.num_kv_heads;
  const int b = id % p.batch; id /= p.batch;
  const int pidx = id;

  const int nrows = seq_tokens(p, b) * p.group;  // this sequence's fold
  // Ragged q: a block none of whose rows exists (a sequence without tokens, or a
  // row block past a short sequence's rows) has nothing to do.  It must leave here:
  // below, its key range would start from an empty minimum over its rows.  The
  // whole block returns before any barrier; a merge inside the pass counts no
  // such block, since every partition of the row group leaves alike.
  if (rb * R >= nrows) return;
  const size_t row0q = seq_row0(p, b);
  const int k_lo = pidx * p.keys_per_partition;
  int hi[R];
  bool row_ok[R];
  int head[R], tok[R];
  int hmin = 0x7fffffff, hmax = k_lo;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rr = rb * R + r;
    row_ok[r] = rr < nrows;
    tok[r] = row_ok[r] ? rr / p.group : 0;
    head[r] = g * p.group + (row_ok[r] ? rr % p.group : 0);
    int lim = row_ok[r] ? visible_keys(p, b, tok[r]) : 0;
    int h_ = min(k_lo + p.keys_per_partition, lim);
    hi[r] = row_ok[r] ? h_ : k_lo;
    if (row_ok[r]) {
      hmin = min(hmin, hi[r]);
      hmax = max(hmax, hi[r]);
    }
  }
  hmin = max(hmin, k_lo);

  // Query rows: this lane's EPL elements of each row.
  uint4 qv[R][C::NV];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const size_t qoff = ((row0q + tok[r]) * p.num_q_heads + head[r]) * (size_t)D;
#pragma unroll
    for (int vv = 0; vv < C::NV; ++vv) {
      if (row_ok[r])
        qv[r][vv] = *(const uint4*)((const char*)p.q +
                                    (qoff + (size_t)(vv * C::L + part) * C::EPV) * C::ESZ);
      else
        qv[r][vv] = make_uint4(0, 0, 0, 0);
    }
  }

  float m[R], l[R], o[R][C::EPL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < C::EPL; ++e) o[r][e] = 0.f;
  }

  // Unmasked tiles: every key of the tile is visible to every row.
  const int full_end = k_lo + ((hmin - k_lo) / C::STEP) * C::STEP;
  if (k_lo < full_end) {
    ValuTile<BF16, D, R, U> ta, tb;
    valu_load<BF16, D, R, U, false>(p, ta, b, g, k_lo, wave, slot, part, 0);
    int kb = k_lo;
    for (;;) {
      const bool more = kb + C::STEP < full_end;
      if (more) valu_load<BF16, D, R, U, false>(p, tb, b, g, kb + C::STEP, wave, slot, part, 0);
      valu_process<BF16, D, R, U, false>(ta, qv, m, l, o, hi, row_ok, kb, jl, p.scale_log2);
      kb += C::STEP;
      if (!more) break;
      const bool more2 = kb + C::STEP < full_end;
      if (more2) valu_load<BF16, D, R, U, false>(p, ta, b, g, kb + C::STEP, wave, slot, part, 0);
      valu_process<BF16, D, R, U, false>(tb, qv, m, l, o, hi, row_ok, kb, jl, p.scale_log2);
      kb += C::STEP;
      if (!more2) break;
    }
  }
  // Masked tail tiles: keys past a row's limit get score -inf and are not loaded
  // past the largest limit.
  for (int kb = full_end; kb < hmax; kb += C::STEP) {
    ValuTile<BF16, D, R, U> tt;
    valu_load<BF16, D, R, U, true>(p, tt, b, g, kb, wave, slot, part, hmax);
    valu_process<BF16, D, R, U, true>(tt, qv, m, l, o, hi, row_ok, kb, jl, p.scale_log2);
  }

  // Merge the 8 slots of the wave (lanes with equal `part`).
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int x = 8; x < 64; x <<= 1) {
      const float m2 = shfl_xor(m[r], x);
      const float l2 = shfl_xor(l[r], x);
      float mn, fa, fb;
      merge_factors(m[r], m2, mn, fa, fb);
      m[r] = mn;
      l[r] = fa * l[r] + fb * l2;
#pragma unroll
      for (int e = 0; e < C::EPL; ++e) {
        const float o2 = shfl_xor(o[r][e], x);
        o[r][e] = fa * o[r][e] + fb * o2;
      }
    }
  }

  // Merge the 4 waves through LDS.
  __shared__ float sm_o[C::WAVES][R][D];
  __shared__ float sm_m[C::WAVES][R];
  __shared__ float sm_l[C::WAVES][R];
  if (slot == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int e = 0; e < C::EPL; ++e) sm_o[wave][r][lane_depth<C>(part, e)] = o[r][e];
      if (part == 0) {
        sm_m[wave][r] = m[r];
        sm_l[wave][r] = l[r];
      }
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < R * D; idx += blockDim.x) {
    const int r = idx / D;
    const int d = idx % D;
    const int rr = rb * R + r;
    if (rr >= nrows) continue;
    const int t = rr / p.group;
    const int h = g * p.group + rr % p.group;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) M = fmaxf(M, sm_m[w][r]);
    const float Ms = (M == kNegInf) ? 0.f : M;
    float Lsum = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) {
      const float f = fast_exp2(sm_m[w][r] - Ms);
      Lsum += f * sm_l[w][r];
      O += f * sm_o[w][r][d];
    }
    const size_t row = (row0q + t) * p.num_q_heads + h;
    if (p.write_partials) {
      const size_t prow = (size_t)pidx * (size_t)p.rows_total + row;
      const bool any = Lsum > 0.f;
      const float pm = any ? M * kLn2 : kNegInf;
      if (merge_count) {  // read back by another block of this launch
        st_agent(p.part_o + prow * D + d, any ? O / Lsum : 0.f);
        if (d == 0) {
          st_agent(p.part_m + prow, pm);
          st_agent(p.part_l + prow, Lsum);
        }
      } else {
        p.part_o[prow * D + d] = any ? O / Lsum : 0.f;
        if (d == 0) {
          p.part_m[prow] = pm;
          p.part_l[prow] = Lsum;
        }
      }
    } else {
      if (p.sink) {
        const float sig = p.sink[h] * kLog2e;
        const float M2 = fmaxf(M, sig);
        const float c = fast_exp2(M - M2);
        Lsum = Lsum * c + fast_exp2(sig - M2);
        O *= c;
        M = M2;
      }
      const bool any = Lsum > 0.f;
      const float res = any ? O / Lsum : 0.f;
      if constexpr (BF16)
        ((uint16_t*)p.out)[row * D + d] = to_bf16(res);
      else
        ((float*)p.out)[row * D + d] = res;
      if (d == 0 && p.lse) p.lse[row] = any ? (M + fast_log2(Lsum)) * kLn2 : kNegInf;
    }
  }
  if (merge_count) {
    __shared__ int sm_flag;
    valu_count_and_merge<D>(
        ValuMergeArgs{p.part_o, p.part_m, p.part_l, p.sink, (float*)p.out, p.lse,
                      (size_t)p.rows_total, row0q, p.num_q_heads, p.group, g, rb, R, nrows,
                      p.num_partitions},
        merge_count + ((size_t)b * p.num_kv_heads + g) * p.row_blocks + rb, &sm_flag, wave,
        lane);
  }
}

// Rows per block the kernel is built for (rows are padded up to these).
static int valu_rows_bucket(int fold) {
  if (fold <= 1) return 1;
  if (fold <= 2) return 2;
  if (fold <= 4) return 4;
  return 8;
}

template <bool BF16, int D, int R>
static hipError_t launch_valu_r(const DecodeParams& p, unsigned* mc, int grid, hipStream_t s) {
  constexpr int U = (R <= 4) ? 2 : 1;
  hipLaunchKernelGGL((decode_valu_kernel<BF16, D, R, U>), dim3(grid), dim3(256), 0, s, p, mc);
  return hipGetLastError();
}

template <bool BF16, int D>
static hipError_t launch_valu_d(const DecodeParams& p, unsigned* mc, int R, int grid,
                                hipStream_t s) {
  switch (R) {
    case 1: return launch_valu_r<BF16, D, 1>(p, mc, grid, s);
    case 2: return launch_valu_r<BF16, D, 2>(p, mc, grid, s);
    case 4: return launch_valu_r<BF16, D, 4>(p, mc, grid, s);
    default: return launch_valu_r<BF16, D, 8>(p, mc, grid, s);
  }
}

// Keys per block iteration for a given row bucket (partition sizes are
// multiples of it).
int valu_step_keys(int rows_per_block) { return 32 * ((rows_per_block <= 4) ? 2 : 1); }
int valu_rows_per_block(int fold) { return valu_rows_bucket(fold); }

// fp32 inputs (bf16 runs the streaming matrix-core kernel).  merge_count: see the
// kernel (the caller guarantees P <= 8 and one word per row group).
hipError_t launch_decode_valu(const DecodeParams& p, unsigned* merge_count, hipStream_t s) {
  const int R = valu_rows_bucket(fold_rows(p));
  const int grid = p.num_partitions * p.batch * p.num_kv_heads * p.row_blocks;
  if (p.depth == 64) return launch_valu_d<false, 64>(p, merge_count, R, grid, s);
  return launch_valu_d<false, 128>(p, merge_count, R, grid, s);
}

}  // namespace da
