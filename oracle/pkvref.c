/*
 * pkvref.c -- CPU oracle for attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg do.  It shares no source,
 * header, table or helper with the HIP library.
 *
 * It computes the plain definitions, slowly and in double precision:
 *
 *   - Attention(Q, K, V) = softmax(Q K^T / sqrt(d)) V  (page 2, section 2.1,
 *     the standard attention formula), one query row at a time, as two
 *     passes: all scores and their maximum first, then the exponentials,
 *     their sum and the weighted sum of V rows.  FlashAttention's tiled
 *     online softmax (page 2, section 2.2) is exact, so the tiled GPU result
 *     must equal this up to rounding.
 *   - The paged address rule: logical token t of a sequence lives in physical
 *     page table[t / P] at offset t % P (page 3, section 3.2, the page-table
 *     lookup written as page_table[token_idx // PAGE_SIZE]); pages hold P
 *     tokens and a sequence of L tokens uses ceil(L / P) of them (page 1,
 *     section 2.3).
 *   - GQA: query head h reads KV head h / G, G = H_q / H_kv, contiguous
 *     groups (page 4, section 2.2 gives the 4:1 and 8:1 ratios; the grouping
 *     is the plainest reading).
 *   - Chunked prefill (page 4, section 3.1): the chunk's C rows are the last
 *     C positions of a sequence of kv_len tokens; row i sits at position
 *     kv_len - C + i and sees keys 0 .. that position (bottom-right causal).
 *   - Merging partial results over disjoint key sets by their log-sum-exp,
 *     the same recursion that the pages' online softmax rests on.
 *   - An fp8 KV cache (page 1, section 4.1 and page 4, section 3.2 name the
 *     e4m3 and e5m2 cache types, the latter in a serving setup that also
 *     prefills in chunks; page 4, chapter 6 calls fp8 the most
 *     cost-effective saving): element = per-tensor fp32 scale times the
 *     OCP 8-bit float value; a new token is stored as the code nearest to
 *     x / scale (x / scale taken in fp32, ties to the even code), clipped to
 *     the largest finite value.
 *   - A sliding window (page 4, section 2.3: each token attends to a local
 *     window, mixed with a few global tokens): with window w > 0 the query at
 *     the last position L - 1 sees keys t >= L - w and the first `sink` keys.
 *
 * Inputs are converted to double exactly (f32 cast; f16 decoded from its
 * sign/exponent/mantissa fields, subnormals included; bf16 shifted into the
 * high half of an f32; fp8 decoded from its fields).  exp and log are the
 * host libm's.
 *
 * Cache layout: K and V pools [num_pages][H_kv][P][D] of the element type.
 * Return value: 0 on success, -1 on an invalid argument or an index out of
 * range (nothing is written past a buffer in that case).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { REF_F32 = 0, REF_F16 = 1, REF_BF16 = 2, REF_FP8_E4M3 = 3, REF_FP8_E5M2 = 4 };

static int elem_bytes(int dtype) {
  switch (dtype) {
    case REF_F32: return 4;
    case REF_F16: return 2;
    case REF_BF16: return 2;
    case REF_FP8_E4M3: return 1;
    case REF_FP8_E5M2: return 1;
    default: return 0;
  }
}

static int is_fp8(int dtype) { return dtype == REF_FP8_E4M3 || dtype == REF_FP8_E5M2; }

/* OCP 8-bit float E4M3 ("FN": no infinities): sign, 4 exponent bits with
   bias 7, 3 mantissa bits; the single pattern S.1111.111 is NaN. */
static double fp8_e4m3_to_double(uint8_t b) {
  int sign = b >> 7;
  int expo = (b >> 3) & 15;
  int mant = b & 7;
  double v;
  if (expo == 15 && mant == 7) return NAN;
  if (expo == 0) {
    v = ldexp((double)mant, -9);                 /* mant/8 * 2^(1-7) */
  } else {
    v = ldexp((double)(8 + mant), expo - 10);    /* (1 + mant/8) * 2^(expo-7) */
  }
  return sign ? -v : v;
}

/* OCP 8-bit float E5M2: sign, 5 exponent bits with bias 15, 2 mantissa bits,
   infinities and NaNs as in IEEE 754. */
static double fp8_e5m2_to_double(uint8_t b) {
  int sign = b >> 7;
  int expo = (b >> 2) & 31;
  int mant = b & 3;
  double v;
  if (expo == 31) {
    v = mant ? NAN : INFINITY;
  } else if (expo == 0) {
    v = ldexp((double)mant, -16);                /* mant/4 * 2^(1-15) */
  } else {
    v = ldexp((double)(4 + mant), expo - 17);    /* (1 + mant/4) * 2^(expo-15) */
  }
  return sign ? -v : v;
}

static double fp8_to_double(int dtype, uint8_t b) {
  return dtype == REF_FP8_E4M3 ? fp8_e4m3_to_double(b) : fp8_e5m2_to_double(b);
}

/* IEEE binary16 -> double, field by field. */
static double half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int mant = h & 0x3ff;
  double v;
  if (expo == 0) {
    v = ldexp((double)mant, -24);               /* subnormal: mant * 2^-24 */
  } else if (expo == 31) {
    v = mant ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + mant), expo - 25); /* (1 + mant/1024) * 2^(expo-15) */
  }
  return sign ? -v : v;
}

/* bfloat16 -> double: the 16 bits are the high half of a binary32. */
static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double load_elem(const void* base, int64_t idx, int dtype) {
  if (is_fp8(dtype)) return fp8_to_double(dtype, ((const uint8_t*)base)[idx]);
  if (dtype == REF_F32) {
    float f;
    memcpy(&f, (const char*)base + idx * 4, 4);
    return (double)f;
  }
  uint16_t h;
  memcpy(&h, (const char*)base + idx * 2, 2);
  return dtype == REF_F16 ? half_to_double(h) : bf16_to_double(h);
}

int pkvref_version(void) { return 1; }

/* Convert n elements of the given type to double (for test convenience). */
int pkvref_to_double(int dtype, const void* src, int64_t n, double* dst) {
  if (!elem_bytes(dtype) || n < 0 || (n > 0 && (!src || !dst))) return -1;
  for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(src, i, dtype);
  return 0;
}

/*
 * fp8 code of y: the non-negative code whose value is nearest to |y| (on a
 * tie, the even code), with the sign bit of y.  |y| at or beyond the largest
 * finite value gives that value; NaN gives 0x7F.  A search over the codes.
 */
static uint8_t fp8_encode(int dtype, float y) {
  if (y != y) return 0x7F;
  const int max_code = dtype == REF_FP8_E4M3 ? 0x7E : 0x7B;   /* 448, 57344 */
  const double a = fabs((double)y);
  int best = max_code;
  if (a < fp8_to_double(dtype, (uint8_t)max_code)) {
    double best_d = INFINITY;
    for (int c = 0; c <= max_code; ++c) {
      const double d = fabs(fp8_to_double(dtype, (uint8_t)c) - a);
      if (d < best_d || (d == best_d && (c & 1) == 0)) {
        best = c;
        best_d = d;
      }
    }
  }
  return (uint8_t)(best | (signbit(y) ? 0x80 : 0));
}

/*
 * quant_fp8: dst[i] = fp8 code of (float)x_i / scale, x_i of src_dtype
 * (exactly representable as float), the division in IEEE fp32.
 */
int pkvref_quant_fp8(int fp8_dtype, int src_dtype, const void* src, int64_t n, float scale,
                     uint8_t* dst) {
  if (!is_fp8(fp8_dtype) || !elem_bytes(src_dtype) || is_fp8(src_dtype) || n < 0) return -1;
  if (n > 0 && (!src || !dst)) return -1;
  for (int64_t i = 0; i < n; ++i) {
    const float x = (float)load_elem(src, i, src_dtype);
    const float y = x / scale;
    dst[i] = fp8_encode(fp8_dtype, y);
  }
  return 0;
}

/*
 * kv_append: for each i with slots[i] >= 0, copy token i's K and V rows for
 * every KV head into page slots[i] / P at offset slots[i] % P.  A bitwise
 * copy.  k_new, v_new: [n][H_kv][D].
 */
int pkvref_kv_append(int dtype, int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
                     int32_t head_dim, void* k_cache, void* v_cache, const void* k_new,
                     const void* v_new, const int32_t* slots, int32_t n) {
  int es = elem_bytes(dtype);
  if (!es || num_pages <= 0 || page_size <= 0 || num_kv_heads <= 0 || head_dim <= 0 || n < 0)
    return -1;
  if (n > 0 && (!k_cache || !v_cache || !k_new || !v_new || !slots)) return -1;
  int64_t total_slots = (int64_t)num_pages * page_size;
  for (int32_t i = 0; i < n; ++i)
    if (slots[i] >= total_slots) return -1;
  size_t row = (size_t)head_dim * es;
  for (int32_t i = 0; i < n; ++i) {
    int64_t s = slots[i];
    if (s < 0) continue;
    int64_t page = s / page_size;
    int64_t off = s % page_size;
    for (int32_t g = 0; g < num_kv_heads; ++g) {
      int64_t dst = ((page * num_kv_heads + g) * page_size + off) * (int64_t)row;
      int64_t src = ((int64_t)i * num_kv_heads + g) * (int64_t)row;
      memcpy((char*)k_cache + dst, (const char*)k_new + src, row);
      memcpy((char*)v_cache + dst, (const char*)v_new + src, row);
    }
  }
  return 0;
}

/* Physical page of logical token t, or -1 if the table entry is out of range. */
static int64_t page_of(const int32_t* table_row, int64_t t, int32_t page_size, int32_t num_pages) {
  int32_t page = table_row[t / page_size];
  if (page < 0 || page >= num_pages) return -1;
  return page;
}

/* Element index of K/V[token t of the sequence][kv head g][d = 0]. */
static int64_t row_index(int64_t page, int64_t t, int32_t g, int32_t page_size,
                         int32_t num_kv_heads, int32_t head_dim) {
  return ((page * num_kv_heads + g) * page_size + t % page_size) * (int64_t)head_dim;
}

/*
 * gather: copy logical tokens [0, len) of one sequence from the pools into
 * contiguous k_out, v_out [len][H_kv][D] (bitwise).
 */
int pkvref_gather(int dtype, int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
                  int32_t head_dim, const void* k_cache, const void* v_cache,
                  const int32_t* table_row, int32_t len, void* k_out, void* v_out) {
  int es = elem_bytes(dtype);
  if (!es || page_size <= 0 || num_kv_heads <= 0 || head_dim <= 0 || len < 0) return -1;
  size_t row = (size_t)head_dim * es;
  for (int64_t t = 0; t < len; ++t) {
    int64_t page = page_of(table_row, t, page_size, num_pages);
    if (page < 0) return -1;
    for (int32_t g = 0; g < num_kv_heads; ++g) {
      int64_t src = row_index(page, t, g, page_size, num_kv_heads, head_dim) * es;
      int64_t dst = (t * num_kv_heads + g) * (int64_t)row;
      memcpy((char*)k_out + dst, (const char*)k_cache + src, row);
      memcpy((char*)v_out + dst, (const char*)v_cache + src, row);
    }
  }
  return 0;
}

/* Key t of a sequence of n_keys is visible unless a window hides it:
   visible iff t >= lo or t < sink_n (lo = 0, sink_n = 0 without a window). */
static int visible(int64_t t, int64_t lo, int64_t sink_n) { return t >= lo || t < sink_n; }

/*
 * One query row against the visible keys among 0 .. n_keys-1 of one sequence
 * and KV head g.  K and V elements are k_scale (v_scale) times the cache
 * value.  q_row: D doubles.  s: scratch of n_keys doubles.  Writes out[D],
 * *lse.  No visible key: out = 0, lse = -inf (an empty sum).
 */
static int attend_row(int kv_dtype, int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
                      int32_t head_dim, const void* k_cache, const void* v_cache, double k_scale,
                      double v_scale, const int32_t* table_row, int64_t n_keys, int64_t lo,
                      int64_t sink_n, int32_t g, const double* q_row, double scale, double* s,
                      double* out, double* lse) {
  for (int32_t d = 0; d < head_dim; ++d) out[d] = 0.0;
  /* pass 1: scores of the visible keys and their maximum */
  double m = -INFINITY;
  int64_t n_vis = 0;
  for (int64_t t = 0; t < n_keys; ++t) {
    if (!visible(t, lo, sink_n)) continue;
    int64_t page = page_of(table_row, t, page_size, num_pages);
    if (page < 0) return -1;
    int64_t base = row_index(page, t, g, page_size, num_kv_heads, head_dim);
    double dot = 0.0;
    for (int32_t d = 0; d < head_dim; ++d)
      dot += q_row[d] * (k_scale * load_elem(k_cache, base + d, kv_dtype));
    s[t] = scale * dot;
    if (s[t] > m) m = s[t];
    ++n_vis;
  }
  if (n_vis == 0) {
    *lse = -INFINITY;
    return 0;
  }
  /* pass 2: exponentials, their sum, weighted sum of V rows */
  double l = 0.0;
  for (int64_t t = 0; t < n_keys; ++t) {
    if (!visible(t, lo, sink_n)) continue;
    double w = exp(s[t] - m);
    l += w;
    int64_t page = page_of(table_row, t, page_size, num_pages);
    int64_t base = row_index(page, t, g, page_size, num_kv_heads, head_dim);
    for (int32_t d = 0; d < head_dim; ++d)
      out[d] += w * (v_scale * load_elem(v_cache, base + d, kv_dtype));
  }
  for (int32_t d = 0; d < head_dim; ++d) out[d] /= l;
  *lse = m + log(l);
  return 0;
}

static void set_threads(int32_t n_threads) {
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
}

/*
 * decode_ex: one query token per sequence.  q [B][H_q][D] of q_dtype; the
 * pools hold kv_dtype (for fp8, element = k_scale or v_scale times the code's
 * value; otherwise the scales must be 1 and kv_dtype == q_dtype).
 * block_table [B][stride]; context_lens [B].  window > 0 restricts the keys
 * to t >= L - window plus the first `sink` (window 0: all keys).  rows:
 * indices r = b * H_q + h to compute, or NULL for all B * H_q rows in order.
 * out [n_rows][D], lse [n_rows] (natural log).  scale is the float32 value
 * the GPU receives, widened.
 */
int pkvref_decode_ex(int q_dtype, int kv_dtype, int32_t num_pages, int32_t page_size,
                     int32_t num_kv_heads, int32_t head_dim, const void* k_cache,
                     const void* v_cache, float k_scale, float v_scale, const void* q,
                     int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                     int32_t stride, const int32_t* context_lens, float scale, int32_t window,
                     int32_t sink, const int64_t* rows, int64_t n_rows, double* out, double* lse,
                     int32_t n_threads) {
  if (!elem_bytes(q_dtype) || is_fp8(q_dtype) || !elem_bytes(kv_dtype) || page_size <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0 || batch < 0 || num_q_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || stride <= 0 || window < 0 || sink < 0)
    return -1;
  if (!is_fp8(kv_dtype) && (kv_dtype != q_dtype || k_scale != 1.0f || v_scale != 1.0f))
    return -1;
  int64_t all = (int64_t)batch * num_q_heads;
  if (!rows) n_rows = all;
  int32_t group = num_q_heads / num_kv_heads;
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t r = rows ? rows[i] : i;
    if (r < 0 || r >= all) return -1;
    int64_t b = r / num_q_heads;
    if (context_lens[b] < 0 || context_lens[b] > (int64_t)stride * page_size) return -1;
  }
  int err = 0;
  set_threads(n_threads);
#pragma omp parallel reduction(| : err)
  {
    double* qd = (double*)malloc(sizeof(double) * head_dim);
    double* s = NULL;
    int64_t s_cap = 0;
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
      int64_t r = rows ? rows[i] : i;
      int64_t b = r / num_q_heads;
      int32_t h = (int32_t)(r % num_q_heads);
      int64_t n_keys = context_lens[b];
      int64_t lo = 0, sink_n = 0;
      if (window > 0) {
        lo = n_keys - window > 0 ? n_keys - window : 0;
        sink_n = sink < n_keys ? sink : n_keys;
      }
      if (n_keys > s_cap) {
        free(s);
        s_cap = n_keys;
        s = (double*)malloc(sizeof(double) * s_cap);
      }
      for (int32_t d = 0; d < head_dim; ++d) qd[d] = load_elem(q, r * head_dim + d, q_dtype);
      err |= attend_row(kv_dtype, num_pages, page_size, num_kv_heads, head_dim, k_cache,
                        v_cache, (double)k_scale, (double)v_scale, block_table + b * stride,
                        n_keys, lo, sink_n, h / group, qd, (double)scale, s, out + i * head_dim,
                        lse + i);
    }
    free(s);
    free(qd);
  }
  return err ? -1 : 0;
}

/* decode: decode_ex with one element type, unit scales and no window. */
int pkvref_decode(int dtype, int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
                  int32_t head_dim, const void* k_cache, const void* v_cache, const void* q,
                  int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                  int32_t stride, const int32_t* context_lens, float scale,
                  const int64_t* rows, int64_t n_rows, double* out, double* lse,
                  int32_t n_threads) {
  if (is_fp8(dtype)) return -1;
  return pkvref_decode_ex(dtype, dtype, num_pages, page_size, num_kv_heads, head_dim, k_cache,
                          v_cache, 1.0f, 1.0f, q, batch, num_q_heads, block_table, stride,
                          context_lens, scale, 0, 0, rows, n_rows, out, lse, n_threads);
}

/*
 * prefill_ex: chunked prefill, q packed [sum_b C_b][H_q][D] of q_dtype with
 * q_indptr [B+1] (host); kv_lens[b] counts history plus chunk.  The pools hold
 * kv_dtype (for fp8, element = k_scale or v_scale times the code's value;
 * otherwise the scales must be 1 and kv_dtype == q_dtype).  rows: indices
 * r = tok * H_q + h (tok indexes the packed query tokens), or NULL for all.
 * out [n_rows][D], lse [n_rows].
 */
int pkvref_prefill_ex(int q_dtype, int kv_dtype, int32_t num_pages, int32_t page_size,
                      int32_t num_kv_heads, int32_t head_dim, const void* k_cache,
                      const void* v_cache, float k_scale, float v_scale, const void* q,
                      const int32_t* q_indptr, int32_t batch, int32_t num_q_heads,
                      const int32_t* block_table, int32_t stride, const int32_t* kv_lens,
                      float scale, const int64_t* rows, int64_t n_rows, double* out, double* lse,
                      int32_t n_threads) {
  if (!elem_bytes(q_dtype) || is_fp8(q_dtype) || !elem_bytes(kv_dtype) || page_size <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0 || batch < 0 || num_q_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || stride <= 0)
    return -1;
  if (!is_fp8(kv_dtype) && (kv_dtype != q_dtype || k_scale != 1.0f || v_scale != 1.0f))
    return -1;
  if (q_indptr[0] != 0) return -1;
  for (int32_t b = 0; b < batch; ++b) {
    int64_t c = (int64_t)q_indptr[b + 1] - q_indptr[b];
    if (c < 0 || c > kv_lens[b] || kv_lens[b] > (int64_t)stride * page_size) return -1;
  }
  int64_t n_tok = q_indptr[batch];
  int64_t all = n_tok * num_q_heads;
  if (!rows) n_rows = all;
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t r = rows ? rows[i] : i;
    if (r < 0 || r >= all) return -1;
  }
  int32_t group = num_q_heads / num_kv_heads;
  int err = 0;
  set_threads(n_threads);
#pragma omp parallel reduction(| : err)
  {
    double* qd = (double*)malloc(sizeof(double) * head_dim);
    double* s = NULL;
    int64_t s_cap = 0;
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
      int64_t r = rows ? rows[i] : i;
      int64_t tok = r / num_q_heads;
      int32_t h = (int32_t)(r % num_q_heads);
      int32_t b = 0;
      while (q_indptr[b + 1] <= tok) ++b; /* sequence that owns this query token */
      int64_t c = (int64_t)q_indptr[b + 1] - q_indptr[b];
      int64_t pos = (int64_t)kv_lens[b] - c + (tok - q_indptr[b]);
      int64_t n_keys = pos + 1;                 /* keys 0 .. pos */
      if (n_keys > s_cap) {
        free(s);
        s_cap = n_keys;
        s = (double*)malloc(sizeof(double) * s_cap);
      }
      for (int32_t d = 0; d < head_dim; ++d) qd[d] = load_elem(q, r * head_dim + d, q_dtype);
      err |= attend_row(kv_dtype, num_pages, page_size, num_kv_heads, head_dim, k_cache,
                        v_cache, (double)k_scale, (double)v_scale,
                        block_table + (int64_t)b * stride, n_keys, 0, 0, h / group, qd,
                        (double)scale, s, out + i * head_dim, lse + i);
    }
    free(s);
    free(qd);
  }
  return err ? -1 : 0;
}

/* prefill chunk: prefill_ex with one element type and unit scales. */
int pkvref_prefill(int dtype, int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
                   int32_t head_dim, const void* k_cache, const void* v_cache, const void* q,
                   const int32_t* q_indptr, int32_t batch, int32_t num_q_heads,
                   const int32_t* block_table, int32_t stride, const int32_t* kv_lens,
                   float scale, const int64_t* rows, int64_t n_rows, double* out, double* lse,
                   int32_t n_threads) {
  if (is_fp8(dtype)) return -1;
  return pkvref_prefill_ex(dtype, dtype, num_pages, page_size, num_kv_heads, head_dim, k_cache,
                           v_cache, 1.0f, 1.0f, q, q_indptr, batch, num_q_heads, block_table,
                           stride, kv_lens, scale, rows, n_rows, out, lse, n_threads);
}

/*
 * merge: rows independent results, each given as n_parts partial states
 * (o_k [D], lse_k) over disjoint key sets.  M = max_k lse_k,
 * w_k = exp(lse_k - M), o = sum_k w_k o_k / sum_k w_k, lse = M + log sum_k w_k.
 * All parts empty (every lse_k = -inf): o = 0, lse = -inf.
 * o_parts [rows][n_parts][D], lse_parts [rows][n_parts].
 */
int pkvref_merge(const double* o_parts, const double* lse_parts, int64_t rows, int32_t n_parts,
                 int32_t head_dim, double* out, double* lse) {
  if (rows < 0 || n_parts <= 0 || head_dim <= 0) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    const double* lp = lse_parts + r * n_parts;
    double m = -INFINITY;
    for (int32_t k = 0; k < n_parts; ++k)
      if (lp[k] > m) m = lp[k];
    double* o = out + r * head_dim;
    for (int32_t d = 0; d < head_dim; ++d) o[d] = 0.0;
    if (m == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double wsum = 0.0;
    for (int32_t k = 0; k < n_parts; ++k) {
      if (lp[k] == -INFINITY) continue;
      double w = exp(lp[k] - m);
      wsum += w;
      const double* ok = o_parts + (r * n_parts + k) * head_dim;
      for (int32_t d = 0; d < head_dim; ++d) o[d] += w * ok[d];
    }
    for (int32_t d = 0; d < head_dim; ++d) o[d] /= wsum;
    lse[r] = m + log(wsum);
  }
  return 0;
}
