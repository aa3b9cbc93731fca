/*
 * decode_oracle.c -- plain, slow fp64 CPU reference for single-query (decode)
 * attention over a KV cache.  TEST INFRASTRUCTURE ONLY: nothing on the product
 * path may link or call this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header or table with
 * the HIP library.
 *
 * What it computes (per query row = (batch b, token t, query head h)):
 *
 *   out[d] = sum_j softmax_j( scale * <q, k_j> ) * v_j[d]      (visible keys j)
 *
 * as stated in the description of "mha_decoding_single_batch_pipelined"
 * (FA2 decode: attention for a single query per row) and in
 * "mha_sm100_dispatch", Args `scale` (the factor on the product of Q and K
 * before the softmax).  It is written out directly, two passes over
 * the keys (max, then exp-sum and weighted sum), no online rescaling, no
 * blocking, everything accumulated in double.
 *
 * Readings taken where the pages leave a step open:
 *   - KV head of query head h is floor(h / group), `group` counting the query
 *     heads that share one KV head ("mha_sm100_dispatch", Parameters `group`).
 *   - Keys visible to row (b, t): N_b = valid_length[b] if given, else
 *     max_seq_len ("mha_sm100_dispatch", Args `valid_length`,
 *     `max_cache_valid_length_arg`: the latter bounds the former), and a
 *     length above max_seq_len counts as max_seq_len.  N_b counts the current
 *     tokens too.  With
 *     the causal mask, token t of T sees keys j <= N_b - T + t (bottom-right
 *     aligned; the MTP tokens are the last T positions).
 *   - MLA ("flare_mla_decoding_dispatch", Args `k`): V is K[..., :depth_v];
 *     the caller passes v == NULL for that case.
 *   - Sink ("flare_mla_decoding_dispatch", Args `attn_sink_ptr`;
 *     "mha_sm100_dispatch", Args `sink_weights`): one fp32 logit sigma_h per
 *     query head that joins the softmax denominator only (a virtual key with
 *     score sigma_h and a zero value row), not multiplied by `scale`.
 *   - LSE = m + ln(l) of the full denominator, sink included.
 *   - A row with no visible key and no sink: out = 0, LSE = -inf.
 *   - Sparse top-k ("flare_mla_decoding_dispatch", Parameters `sparse`; Args
 *     `d_indices`, `indices_stride`, `topk_lengths`): the keys of sequence b
 *     are the cache rows indices[b * indices_stride + i] for i <
 *     topk_lengths[b] of a pool [pool_rows, KVH, D] (a gather at page size 1).
 *     Every query token and head of the sequence attends to that one list; no
 *     mask applies (the selection is the mask, and a row index carries no
 *     position), so a causal mask together with indices is rejected.  A count
 *     outside [0, indices_stride] or a counted index outside [0, pool_rows) is
 *     an invalid call.  Partition p covers list positions [p*C, (p+1)*C).
 *   - Ragged KV layout ("mha_sm100_dispatch", Args `kv_input_row_offsets`;
 *     "flare_mla_decoding_dispatch", Args `kv_input_row_offsets`: per-batch row
 *     offsets into a ragged KV layout): the caches of all sequences are
 *     concatenated into one cache [pool_rows, KVH, D], and key j of sequence b
 *     is its row kv_offsets[b] + j.  N_b and the mask are as above.  A
 *     sequence whose N_b keys would reach past the cache is an invalid call.
 *   - Split-K ("mha_decoding_single_batch_pipelined", description: the keys
 *     are cut into consecutive ranges, one per block, whose max and exp-sum a
 *     separate merge pass combines): partition p covers
 *     keys [p*C, (p+1)*C); its partial output is normalised by its own exp-sum;
 *     the merge is by log-sum-exp.
 *
 * Element types: 0 = float32, 1 = bfloat16 given as its raw 16-bit pattern.
 * bf16 -> double is exact (the 16 bits are the top half of a float32).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1
/* Problem dtype 2: q in bf16, k and v in ORACLE_E4M3 with per-tensor scales. */
#define ORACLE_BF16_Q_E4M3_KV 2
#define ORACLE_E4M3 3

/* 8-bit float e4m3 (the OCP FP8 E4M3 format): 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6;
 * there is no infinity, and S.1111.111 is NaN. */
static double e4m3_value(uint8_t c) {
  int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* e4m3_value of every code, filled once (by the first call that needs it). */
static double e4m3_table[256];
static int e4m3_table_ready = 0;

static void fill_e4m3_table(void) {
#pragma omp critical(oracle_e4m3_table)
  if (!e4m3_table_ready) {
    for (int c = 0; c < 256; ++c) e4m3_table[c] = e4m3_value((uint8_t)c);
#pragma omp flush
    e4m3_table_ready = 1;
  }
}

static double elem(const void* base, size_t idx, int dtype) {
  if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
  if (dtype == ORACLE_E4M3) return e4m3_table[((const uint8_t*)base)[idx]];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Problem description shared by the entry points below. */
typedef struct {
  const void* q;              /* [B, T, H, D]                                   */
  const void* k;              /* contiguous [B, S, KVH, D] or pool [pages, ps, KVH, D] */
  const void* v;              /* same layout with Dv, or NULL => V = K[..., :Dv] */
  int q_dtype, kv_dtype;      /* element types of q, and of k and v             */
  double k_scale, v_scale;    /* real key = k_scale * stored element; real value
                                 = v_scale * stored element (k_scale when V is a
                                 slice of K: the same stored numbers)            */
  const uint32_t* page_table; /* [B, max_pages] or NULL (contiguous)            */
  int page_size, max_pages;
  const uint32_t* valid_length; /* [B] or NULL                                  */
  const uint32_t* kv_offsets; /* ragged KV layout: key j of sequence b is row kv_offsets[b] + j
                                 of a cache [pool_rows, KVH, D]; NULL otherwise   */
  int B, T, H, KVH, D, Dv, S;
  double scale;
  const float* sink;          /* [H] or NULL                                    */
  int causal;
  const uint32_t* q_offsets;  /* ragged q: [B+1] cumulative token offsets, the tokens of
                                 sequence b being rows q_offsets[b]..q_offsets[b+1] of a
                                 [total, H, D] q; NULL: T tokens per sequence  */
  const int32_t* indices;     /* sparse: [B, indices_stride] pool rows, or NULL       */
  int indices_stride;
  const int32_t* topk_lengths;/* sparse: [B] listed keys of each sequence           */
  int64_t pool_rows;          /* sparse or ragged KV layout: rows of the cache k (and v) */
} problem_t;

/* Query tokens of sequence b, and the q row of its first token. */
static int seq_tokens(const problem_t* p, int b) {
  return p->q_offsets ? (int)(p->q_offsets[b + 1] - p->q_offsets[b]) : p->T;
}
static size_t first_token(const problem_t* p, int b) {
  return p->q_offsets ? (size_t)p->q_offsets[b] : (size_t)b * p->T;
}
static int64_t total_tokens(const problem_t* p) {
  return p->q_offsets ? (int64_t)p->q_offsets[p->B] : (int64_t)p->B * p->T;
}
/* Sequence and token index of q row `token`. */
static void locate_token(const problem_t* p, int64_t token, int* b, int* t) {
  if (!p->q_offsets) {
    *b = (int)(token / p->T);
    *t = (int)(token % p->T);
    return;
  }
  int s = 0;
  while (s + 1 < p->B && (int64_t)p->q_offsets[s + 1] <= token) ++s;
  *b = s;
  *t = (int)(token - (int64_t)p->q_offsets[s]);
}

/* Flat element index of depth element d of key j (of sequence b, KV head g)
 * in a cache whose rows hold `width` elements. */
static size_t kv_index(const problem_t* p, int b, int j, int g, int d, int width) {
  size_t row;
  if (p->indices) {
    row = (size_t)p->indices[(size_t)b * p->indices_stride + (size_t)j];
  } else if (p->kv_offsets) {
    row = (size_t)p->kv_offsets[b] + (size_t)j;
  } else if (p->page_table) {
    uint32_t phys = p->page_table[(size_t)b * p->max_pages + (size_t)(j / p->page_size)];
    row = (size_t)phys * p->page_size + (size_t)(j % p->page_size);
  } else {
    row = (size_t)b * p->S + (size_t)j;
  }
  return (row * p->KVH + (size_t)g) * (size_t)width + (size_t)d;
}

static double key_elem(const problem_t* p, int b, int j, int g, int d) {
  return p->k_scale * elem(p->k, kv_index(p, b, j, g, d, p->D), p->kv_dtype);
}

static double value_elem(const problem_t* p, int b, int j, int g, int d) {
  if (p->v == NULL) return p->k_scale * elem(p->k, kv_index(p, b, j, g, d, p->D), p->kv_dtype);
  return p->v_scale * elem(p->v, kv_index(p, b, j, g, d, p->Dv), p->kv_dtype);
}

/* Keys of sequence b before any mask: valid_length[b], or S without it.  A
 * length above max_seq_len counts as max_seq_len (compared as unsigned: a
 * uint32 length of 2^31 or more is a large count, not a negative one). */
static int seq_keys(const problem_t* p, int b) {
  uint32_t nv = p->valid_length ? p->valid_length[b] : (uint32_t)p->S;
  return nv < (uint32_t)p->S ? (int)nv : p->S;
}

/* Number of keys visible to row (b, t). */
static int visible_keys(const problem_t* p, int b, int t) {
  if (p->indices) return p->topk_lengths[b]; /* sparse: the listed keys, no mask */
  int n = seq_keys(p, b);
  if (p->causal) {
    int lim = n - seq_tokens(p, b) + t + 1;
    if (lim < n) n = lim;
  }
  return n < 0 ? 0 : n;
}

/* Scores s_j = scale * <q_row, k_j> for keys j in [lo, hi). */
static void scores(const problem_t* p, int b, int t, int h, int lo, int hi, double* s) {
  int g = h / (p->H / p->KVH);
  size_t qbase = ((first_token(p, b) + (size_t)t) * p->H + h) * (size_t)p->D;
  for (int j = lo; j < hi; ++j) {
    double dot = 0.0;
    for (int d = 0; d < p->D; ++d)
      dot += elem(p->q, qbase + d, p->q_dtype) * key_elem(p, b, j, g, d);
    s[j - lo] = p->scale * dot;
  }
}

/* Softmax-weighted sum over keys [lo, hi) of row (b, t, h).
 * with_sink: include the row's sink logit in max and denominator.
 * Returns through out[Dv] the normalised output, *m the max, *l the exp-sum
 * (l = 0 and m = -inf when nothing contributes). */
static void attend(const problem_t* p, int b, int t, int h, int lo, int hi, int with_sink,
                   double* s, double* out, double* m_out, double* l_out) {
  int g = h / (p->H / p->KVH);
  int n = hi > lo ? hi - lo : 0;
  if (n > 0) scores(p, b, t, h, lo, hi, s);

  double m = -INFINITY;
  for (int j = 0; j < n; ++j)
    if (s[j] > m) m = s[j];
  double sigma = (with_sink && p->sink) ? (double)p->sink[h] : -INFINITY;
  if (sigma > m) m = sigma;

  for (int d = 0; d < p->Dv; ++d) out[d] = 0.0;
  if (m == -INFINITY) { /* no key and no sink */
    *m_out = -INFINITY;
    *l_out = 0.0;
    return;
  }
  double l = 0.0;
  for (int j = 0; j < n; ++j) {
    double w = exp(s[j] - m);
    l += w;
    for (int d = 0; d < p->Dv; ++d) out[d] += w * value_elem(p, b, lo + j, g, d);
  }
  if (sigma != -INFINITY) l += exp(sigma - m);
  for (int d = 0; d < p->Dv; ++d) out[d] /= l;
  *m_out = m;
  *l_out = l;
}

static problem_t make_problem(const void* q, const void* k, const void* v, int dtype,
                              float k_scale, float v_scale, const uint32_t* page_table,
                              int page_size, int max_pages, const uint32_t* valid_length, int B,
                              int T, int H, int KVH, int D, int Dv, int S, float scale,
                              const float* sink, int causal, const uint32_t* q_offsets,
                              const int32_t* indices, int indices_stride,
                              const int32_t* topk_lengths, int64_t pool_rows,
                              const uint32_t* kv_offsets) {
  problem_t p;
  p.q_offsets = q_offsets;
  p.kv_offsets = kv_offsets;
  p.indices = indices; p.indices_stride = indices_stride;
  p.topk_lengths = topk_lengths; p.pool_rows = pool_rows;
  p.q = q; p.k = k; p.v = v;
  p.q_dtype = (dtype == ORACLE_BF16_Q_E4M3_KV) ? ORACLE_BF16 : dtype;
  p.kv_dtype = (dtype == ORACLE_BF16_Q_E4M3_KV) ? ORACLE_E4M3 : dtype;
  p.k_scale = (double)k_scale; p.v_scale = (double)v_scale;
  p.page_table = page_table; p.page_size = page_size; p.max_pages = max_pages;
  p.valid_length = valid_length;
  p.B = B; p.T = T; p.H = H; p.KVH = KVH; p.D = D; p.Dv = Dv; p.S = S;
  p.scale = (double)scale; p.sink = sink; p.causal = causal;
  if (p.kv_dtype == ORACLE_E4M3) fill_e4m3_table();
  return p;
}

static int check_problem(const problem_t* p) {
  if (p->q_dtype < ORACLE_F32 || p->q_dtype > ORACLE_BF16) return -1;
  if (p->q_offsets) {
    for (int b = 0; b < p->B; ++b)
      if (p->q_offsets[b + 1] < p->q_offsets[b]) return -1;
  }
  if (p->B < 0 || p->T < 1 || p->H < 1 || p->KVH < 1 || p->D < 1 || p->Dv < 1 || p->S < 0)
    return -1;
  if (p->H % p->KVH != 0) return -1;
  if (p->v == NULL && p->Dv > p->D) return -1;
  if (p->page_table && (p->page_size < 1 || p->max_pages < 1)) return -1;
  if (p->kv_offsets) {
    if (p->page_table || p->indices || p->pool_rows < 0) return -1;
    for (int b = 0; b < p->B; ++b) {
      int64_t most = 0; /* keys of sequence b any of its rows may read */
      for (int t = 0; t < seq_tokens(p, b); ++t) {
        int n = visible_keys(p, b, t);
        if (n > most) most = n;
      }
      if ((int64_t)p->kv_offsets[b] + most > p->pool_rows) return -1;
    }
  }
  if (p->indices) {
    if (p->causal || p->page_table || !p->topk_lengths || p->indices_stride < 0) return -1;
    for (int b = 0; b < p->B; ++b) {
      int n = p->topk_lengths[b];
      if (n < 0 || n > p->indices_stride) return -1;
      for (int j = 0; j < n; ++j) {
        int32_t r = p->indices[(size_t)b * p->indices_stride + (size_t)j];
        if (r < 0 || (int64_t)r >= p->pool_rows) return -1;
      }
    }
  }
  return 0;
}

static int longest_cache(const problem_t* p) {
  int s = p->S;
  if (p->indices && p->indices_stride > s) s = p->indices_stride;
  if (!p->indices)
    for (int b = 0; b < p->B; ++b)
      if (seq_keys(p, b) > s) s = seq_keys(p, b);
  return s;
}

/*
 * Full attention for the listed rows (row id = (token)*H + h, token = b*T + t,
 * or q_offsets[b] + t for a ragged q), or for all rows when rows == NULL.
 * out: [num_rows, Dv]; lse: [num_rows].
 */
int oracle_decode_attention(const void* q, const void* k, const void* v, int dtype,
                            float k_scale, float v_scale, const uint32_t* page_table, int page_size, int max_pages,
                            const uint32_t* valid_length, int B, int T, int H, int KVH, int D,
                            int Dv, int S, float scale, const float* sink, int causal,
                            const uint32_t* q_offsets, const int32_t* indices,
                            int indices_stride, const int32_t* topk_lengths, int64_t pool_rows,
                            const uint32_t* kv_offsets, const int64_t* rows, int64_t num_rows,
                            double* out, double* lse, int num_threads) {
  problem_t p = make_problem(q, k, v, dtype, k_scale, v_scale, page_table, page_size, max_pages,
                             valid_length, B, T, H, KVH, D, Dv, S, scale, sink, causal,
                             q_offsets, indices, indices_stride, topk_lengths, pool_rows,
                             kv_offsets);
  if (check_problem(&p)) return -1;
  int64_t n_rows = rows ? num_rows : total_tokens(&p) * H;
  int smax = longest_cache(&p);
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
  int err = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(smax > 0 ? smax : 1));
    if (!s) {
#pragma omp atomic write
      err = -2;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
      if (!s) continue;
      int64_t r = rows ? rows[i] : i;
      int h = (int)(r % H);
      int b, t;
      locate_token(&p, r / H, &b, &t);
      double m, l;
      attend(&p, b, t, h, 0, visible_keys(&p, b, t), 1, s, out + (size_t)i * Dv, &m, &l);
      lse[i] = (l > 0.0) ? m + log(l) : -INFINITY;
    }
    free(s);
  }
  return err;
}

/*
 * Split-K partials: partition part covers keys [part*C, (part+1)*C) of each
 * row's visible keys.  No sink here (it joins the merge once).
 * part_o: [P, B*T*H, Dv] (normalised by its own exp-sum, zero if empty);
 * part_m: [P, B*T*H] natural-log max (-inf if empty); part_l: exp-sum (0 if empty).
 */
int oracle_decode_partials(const void* q, const void* k, const void* v, int dtype,
                           float k_scale, float v_scale, const uint32_t* page_table, int page_size, int max_pages,
                           const uint32_t* valid_length, int B, int T, int H, int KVH, int D,
                           int Dv, int S, float scale, int causal, const uint32_t* q_offsets,
                           const int32_t* indices, int indices_stride,
                           const int32_t* topk_lengths, int64_t pool_rows,
                           const uint32_t* kv_offsets, int num_partitions,
                           int keys_per_partition, double* part_o,
                           double* part_m, double* part_l, int num_threads) {
  problem_t p = make_problem(q, k, v, dtype, k_scale, v_scale, page_table, page_size, max_pages,
                             valid_length, B, T, H, KVH, D, Dv, S, scale, NULL, causal,
                             q_offsets, indices, indices_stride, topk_lengths, pool_rows,
                             kv_offsets);
  if (check_problem(&p) || num_partitions < 1 || keys_per_partition < 1) return -1;
  int64_t n_rows = total_tokens(&p) * H;
  int64_t n_items = n_rows * num_partitions;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
  int err = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)keys_per_partition);
    if (!s) {
#pragma omp atomic write
      err = -2;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_items; ++i) {
      if (!s) continue;
      int part = (int)(i / n_rows);
      int64_t r = i % n_rows;
      int h = (int)(r % H);
      int b, t;
      locate_token(&p, r / H, &b, &t);
      int n = visible_keys(&p, b, t);
      int64_t lo64 = (int64_t)part * keys_per_partition;
      int lo = lo64 < n ? (int)lo64 : n;
      int hi = lo64 + keys_per_partition < n ? (int)(lo64 + keys_per_partition) : n;
      attend(&p, b, t, h, lo, hi, 0, s, part_o + (size_t)i * Dv, &part_m[i], &part_l[i]);
    }
    free(s);
  }
  return err;
}

/*
 * Log-sum-exp merge of split-K partials (the "mha_splitk_reduce" pass).
 * Row r uses sink[r % H] when sink != NULL.  out: [rows, Dv]; lse: [rows].
 */
int oracle_splitk_merge(const double* part_o, const double* part_m, const double* part_l,
                        int num_partitions, int64_t rows, int H, int Dv, const float* sink,
                        double* out, double* lse) {
  if (num_partitions < 1 || rows < 0 || H < 1 || Dv < 1) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    double sigma = sink ? (double)sink[r % H] : -INFINITY;
    double M = sigma;
    for (int p = 0; p < num_partitions; ++p) {
      size_t i = (size_t)p * rows + r;
      if (part_l[i] > 0.0 && part_m[i] > M) M = part_m[i];
    }
    double* o = out + (size_t)r * Dv;
    for (int d = 0; d < Dv; ++d) o[d] = 0.0;
    if (M == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double L = (sigma != -INFINITY) ? exp(sigma - M) : 0.0;
    for (int p = 0; p < num_partitions; ++p) {
      size_t i = (size_t)p * rows + r;
      if (!(part_l[i] > 0.0)) continue;
      double w = part_l[i] * exp(part_m[i] - M);
      L += w;
      for (int d = 0; d < Dv; ++d) o[d] += w * part_o[i * Dv + d];
    }
    for (int d = 0; d < Dv; ++d) o[d] /= L;
    lse[r] = M + log(L);
  }
  return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
