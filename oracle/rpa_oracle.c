/*
 * CPU oracle for ragged paged GQA attention — TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load or call this library. It shares no code, header or constant with
 * the HIP library; it reads the same raw input bits and computes the plain
 * definition in f64, one (token, q head) row at a time, keys in increasing
 * order, so its results are reproducible bit for bit.
 *
 * What it computes follows the ragged paged attention kernel page
 * (zml platforms/tpu/ragged_paged.zig):
 *   - `Cfg`: head counts, page geometry, sm_scale, soft_cap, k_scale/v_scale,
 *     is_causal, sliding_window;
 *   - `run`, operand list: q [T, Hq, D], kv_pages [P, page, 2*Hkv, D],
 *     kv_lens, page_indices, cu_q_lens, num_seqs;
 *   - `createKvAsyncCopyDescriptors`: key j of a sequence lives in physical
 *     page page_indices[seq, j / page_size], slot j % page_size;
 *   - `stridedLoadKv`: combined head 2h holds K of kv head h, 2h+1 holds V;
 *   - `run`, per-kv-head step: dequant x * k_scale (v_scale), q head n reads
 *     kv head n / (Hq/Hkv);
 *   - `flashAttention`: scores q.k * sm_scale, then soft-cap
 *     c*tanh(x/c), then the causal mask (query i of a sequence sits at
 *     position kv_len - q_len + i and sees keys at positions <= its own),
 *     then the sliding-window mask (key j hidden when pos - window >= j),
 *     then softmax over the visible keys and the product with V.
 * The kernel page reaches that result blockwise with an online softmax; the
 * oracle writes the plain definition out instead: max, exp, sum, weighted
 * sum of V, all over the full visible key set at once.
 *
 * Attention sinks (optional): one logit per q head that joins its rows'
 * softmax and takes no value, as the spatial-compiler page's
 * `flat_softmax_rows_at` takes its `sinks` (gpt-oss's attention sinks): the
 * row's maximum starts from it and exp(sink - max) joins the denominator. The
 * sink is compared with the final scores (after scale and soft-cap).
 *
 * Readings where the page is silent (listed with the design notes):
 *   - the log-sum-exp output, natural log of sum exp(score) over visible keys;
 *   - a row with no visible key gets out = 0 and lse = -inf (with a sink:
 *     lse = sink, the log of its own term);
 *   - e4m3fn decode is the OCP FP8 definition (bias 7, subnormals at
 *     exponent 0, S.1111.111 is NaN, no infinities), and e5m2 the OCP one
 *     with bias 15 and IEEE-style infinities and NaN; the page only names
 *     the dtypes (`Cfg` kv_dtype, f8e4m3fn and f8e5m2);
 *   - dequantised values are code*scale exactly (f64), not re-rounded to the
 *     q dtype;
 *   - q (and out) are bf16, f16 or f32 (`Cfg` q_dtype); K/V bf16, f16, e4m3fn,
 *     e5m2 or int8 (`Cfg` kv_dtype; int8 codes are signed integers times the
 *     scale), all read exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_KV_BF16 0
#define ORACLE_KV_E4M3FN 1
#define ORACLE_KV_E5M2 2
#define ORACLE_F16 3 /* IEEE binary16: q/out type, or K/V type */
#define ORACLE_KV_I8 4 /* signed 8-bit integer codes */
#define ORACLE_F32 5   /* IEEE binary32: q/out type */

typedef struct {
  int32_t num_q_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t total_num_pages;
  int32_t page_size;
  int32_t max_num_seqs;
  int32_t pages_per_seq;
  int32_t kv_dtype;       /* ORACLE_KV_BF16, ORACLE_KV_E4M3FN, ORACLE_KV_E5M2, ORACLE_F16 or ORACLE_KV_I8 */
  int32_t is_causal;      /* 0 or 1 */
  int32_t sliding_window; /* <= 0: no window */
  int32_t has_soft_cap;   /* 0 or 1 */
  double sm_scale;
  double soft_cap;
  double k_scale; /* 1.0 when absent */
  double v_scale; /* 1.0 when absent */
  const double* sinks; /* NULL, or one logit per q head [num_q_heads] */
  int32_t q_dtype;     /* 0: bf16 q (and new K/V rows of the append), ORACLE_F16: f16, ORACLE_F32: f32 */
} oracle_cfg;

/* bf16 bits are the upper half of an IEEE binary32 value. */
double oracle_bf16_to_f64(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3 ("fn": finite, one NaN pattern per sign): 1 sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits. Exponent 0 encodes subnormals
 * m/8 * 2^-6; exponent 15 with mantissa 7 is NaN; everything else is
 * (1 + m/8) * 2^(e-7). */
double oracle_e4m3fn_to_f64(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits with bias 15, 10 mantissa bits;
 * exponent 0 encodes subnormals m/1024 * 2^-14, exponent 31 the infinities
 * (mantissa 0) and NaN. */
double oracle_f16_to_f64(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int e = (bits >> 10) & 31;
  int m = bits & 1023;
  double mag;
  if (e == 31) {
    if (m != 0) return NAN;
    mag = INFINITY;
  } else if (e == 0) {
    mag = ldexp((double)m / 1024.0, -14);
  } else {
    mag = ldexp(1.0 + (double)m / 1024.0, e - 15);
  }
  return sign ? -mag : mag;
}

/* OCP FP8 E5M2: 1 sign bit, 5 exponent bits with bias 15, 2 mantissa bits
 * (the IEEE-style format: exponent 31 holds the infinities, mantissa 0, and
 * NaN). Exponent 0 encodes subnormals m/4 * 2^-14; everything else is
 * (1 + m/4) * 2^(e-15). */
double oracle_e5m2_to_f64(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 2) & 31;
  int m = code & 3;
  double mag;
  if (e == 31) {
    if (m != 0) return NAN;
    mag = INFINITY;
  } else if (e == 0) {
    mag = ldexp((double)m / 4.0, -14);
  } else {
    mag = ldexp(1.0 + (double)m / 4.0, e - 15);
  }
  return sign ? -mag : mag;
}

/* Soft-cap of the kernel page's `Cfg`/`flashAttention`: c * tanh(x / c). */
double oracle_soft_cap(double x, double c) { return c * tanh(x / c); }

/* Element idx of a q array (or of the append's new K/V rows) in the q dtype. */
static double q_elem(const oracle_cfg* c, const void* q, int64_t idx) {
  if (c->q_dtype == ORACLE_F32) return (double)((const float*)q)[idx];
  const uint16_t bits = ((const uint16_t*)q)[idx];
  return c->q_dtype == ORACLE_F16 ? oracle_f16_to_f64(bits) : oracle_bf16_to_f64(bits);
}

static double kv_elem(const oracle_cfg* c, const void* kv_pages, int64_t idx) {
  if (c->kv_dtype == ORACLE_KV_E4M3FN) return oracle_e4m3fn_to_f64(((const uint8_t*)kv_pages)[idx]);
  if (c->kv_dtype == ORACLE_KV_E5M2) return oracle_e5m2_to_f64(((const uint8_t*)kv_pages)[idx]);
  if (c->kv_dtype == ORACLE_F16) return oracle_f16_to_f64(((const uint16_t*)kv_pages)[idx]);
  if (c->kv_dtype == ORACLE_KV_I8) return (double)((const int8_t*)kv_pages)[idx];
  return oracle_bf16_to_f64(((const uint16_t*)kv_pages)[idx]);
}

/* Flat index of element d of combined head `comb` for key j of sequence s,
 * or -1 when the page table does not give a valid physical page. */
static int64_t kv_index(const oracle_cfg* c, const int32_t* page_indices, int s, int64_t j, int comb, int d) {
  int64_t logical = j / c->page_size;
  if (logical >= c->pages_per_seq) return -1;
  int32_t phys = page_indices[(int64_t)s * c->pages_per_seq + logical];
  if (phys < 0 || phys >= c->total_num_pages) return -1;
  int64_t slot = j % c->page_size;
  return (((int64_t)phys * c->page_size + slot) * (2 * c->num_kv_heads) + comb) * c->head_dim + d;
}

/* Masks of the kernel page's `flashAttention`: with is_causal a key at
 * position j is hidden from the query at position `pos` when pos < j; with a
 * window w it is also hidden when pos - w >= j. Keys at j >= kv_len are never
 * iterated. */
static int key_visible(const oracle_cfg* c, int64_t j, int64_t pos) {
  if (c->is_causal && j > pos) return 0;
  if (c->sliding_window > 0 && pos - c->sliding_window >= j) return 0;
  return 1;
}

/* One output row (token, q head n). Returns 1 if the token is a padding
 * token (no sequence owns it), 0 on success, -1 on invalid metadata (the row
 * is then filled with NaN). `scores` is caller scratch of >= kv_len doubles. */
static int oracle_row(const oracle_cfg* c, const void* q, const void* kv_pages, const int32_t* kv_lens,
                      const int32_t* page_indices, const int32_t* cu_q_lens, int32_t num_seqs, int64_t token, int n,
                      double* out_row, double* lse, double** scores, int64_t* scores_cap) {
  const int D = c->head_dim;
  const int G = c->num_q_heads / c->num_kv_heads;
  int s = -1;
  for (int i = 0; i < num_seqs; ++i) {
    if (token >= cu_q_lens[i] && token < cu_q_lens[i + 1]) {
      s = i;
      break;
    }
  }
  if (s < 0) return 1;
  const int64_t q_len = cu_q_lens[s + 1] - cu_q_lens[s];
  const int64_t i_tok = token - cu_q_lens[s];
  const int64_t kv_len = kv_lens[s];
  const int h = n / G;
  const int64_t pos = kv_len - q_len + i_tok; /* position of this query among the keys */

  if (kv_len > *scores_cap) {
    free(*scores);
    *scores = (double*)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
    *scores_cap = kv_len;
  }
  double* sc = *scores;
  const int64_t qrow = (token * c->num_q_heads + n) * (int64_t)D;

  /* scores of the visible keys */
  int64_t n_vis = 0;
  double m = -INFINITY;
  for (int64_t j = 0; j < kv_len; ++j) {
    if (!key_visible(c, j, pos)) continue;
    int64_t base = kv_index(c, page_indices, s, j, 2 * h, 0);
    if (base < 0) goto invalid;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += q_elem(c, q, qrow + d) * (kv_elem(c, kv_pages, base + d) * c->k_scale);
    double x = dot * c->sm_scale;
    if (c->has_soft_cap) x = oracle_soft_cap(x, c->soft_cap);
    sc[j] = x;
    /* NaN-propagating maximum, as the kernel page's row max */
    if (n_vis == 0 || isnan(x) || x > m) m = x;
    ++n_vis;
  }
  for (int d = 0; d < D; ++d) out_row[d] = 0.0;
  const int has_sink = c->sinks != NULL;
  const double sink = has_sink ? c->sinks[n] : -INFINITY;
  if (n_vis == 0) {
    *lse = sink; /* -inf without a sink */
    return 0;
  }
  /* the row's maximum starts from the sink */
  if (has_sink && sink > m) m = sink;
  double l = has_sink ? exp(sink - m) : 0.0;
  for (int64_t j = 0; j < kv_len; ++j) {
    if (!key_visible(c, j, pos)) continue;
    double p = exp(sc[j] - m);
    l += p;
    int64_t base = kv_index(c, page_indices, s, j, 2 * h + 1, 0);
    for (int d = 0; d < D; ++d) out_row[d] += p * (kv_elem(c, kv_pages, base + d) * c->v_scale);
  }
  for (int d = 0; d < D; ++d) out_row[d] /= l;
  *lse = m + log(l);
  return 0;

invalid:
  for (int d = 0; d < D; ++d) out_row[d] = NAN;
  *lse = NAN;
  return -1;
}

/* Rows listed by (tokens[r], heads[r]); out is [n_rows, D], lse [n_rows].
 * status[r] receives the per-row code of oracle_row. */
int oracle_rows(const oracle_cfg* c, const void* q, const void* kv_pages, const int32_t* kv_lens,
                const int32_t* page_indices, const int32_t* cu_q_lens, int32_t num_seqs, const int64_t* tokens,
                const int32_t* heads, int64_t n_rows, double* out, double* lse, int32_t* status, int nthreads) {
  if (c->num_kv_heads <= 0 || c->num_q_heads % c->num_kv_heads != 0) return -1;
  if (num_seqs < 0 || num_seqs > c->max_num_seqs) return -1;
  int bad = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1) reduction(+ : bad)
  {
    double* scores = NULL;
    int64_t cap = 0;
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
      int st = oracle_row(c, q, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs, tokens[r], heads[r],
                          out + r * (int64_t)c->head_dim, lse + r, &scores, &cap);
      status[r] = st;
      if (st < 0) bad += 1;
    }
    free(scores);
  }
  return bad ? -2 : 0;
}

/* Every row of [num_q_tokens, Hq]; rows of padding tokens are left as they
 * were in out/lse. */
int oracle_forward(const oracle_cfg* c, const void* q, const void* kv_pages, const int32_t* kv_lens,
                   const int32_t* page_indices, const int32_t* cu_q_lens, int32_t num_seqs, double* out, double* lse,
                   int nthreads) {
  if (c->num_kv_heads <= 0 || c->num_q_heads % c->num_kv_heads != 0) return -1;
  if (num_seqs < 0 || num_seqs > c->max_num_seqs) return -1;
  const int64_t n_rows = (int64_t)c->num_q_tokens * c->num_q_heads;
  int bad = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1) reduction(+ : bad)
  {
    double* scores = NULL;
    int64_t cap = 0;
    double* tmp = (double*)malloc(sizeof(double) * (size_t)c->head_dim);
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; ++r) {
      int64_t token = r / c->num_q_heads;
      int n = (int)(r % c->num_q_heads);
      double l;
      int st = oracle_row(c, q, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs, token, n, tmp, &l, &scores,
                          &cap);
      if (st == 1) continue;
      if (st < 0) bad += 1;
      memcpy(out + r * (int64_t)c->head_dim, tmp, sizeof(double) * (size_t)c->head_dim);
      lse[r] = l;
    }
    free(tmp);
    free(scores);
  }
  return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------
 * KV-cache append. Not on the pages: the ragged paged attention kernel page
 * reads caches that already hold every query token's own key. This writes
 * them, by the same placement rule the page uses for reading (`run` and
 * `flashAttention`'s row ids): query token i of sequence s sits at key
 * position kv_len - q_len + i, and key j lives in slot j % page_size of page
 * page_indices[s, j / page_size], K of kv head h in combined head 2h, V in
 * 2h+1. A stored value is the inverse of the attention's dequant: the f32
 * quotient x / scale (IEEE binary32 division, rounded to nearest), then
 * rounded to the cache type to nearest with ties to even; e4m3fn saturates
 * at +-448 (it has no infinity) and e5m2 the same way at +-57344 (its
 * largest finite value), bf16 and f16 overflow to +-inf as IEEE rounding
 * does; int8 rounds to an integer, ties to even, saturating at -128 and
 * 127. NaN inputs give a NaN code (int8: 0). The new rows come in the q
 * dtype.
 * ------------------------------------------------------------------------ */

/* v rounded to the nearest value of a binary format with `mbits` stored
 * mantissa bits whose normal exponents start at `emin` (subnormals below),
 * ties to the even mantissa; no upper limit. Exact in double for the formats
 * used here. */
static double round_to_format(double v, int mbits, int emin) {
  if (v == 0.0 || isinf(v) || isnan(v)) return v;
  int e;
  (void)frexp(fabs(v), &e); /* |v| = f * 2^e with f in [0.5, 1) */
  int ex = e - 1;           /* floor(log2 |v|) */
  if (ex < emin) ex = emin;
  const double quantum = ldexp(1.0, ex - mbits);
  const double n = nearbyint(fabs(v) / quantum); /* default mode: nearest, ties to even */
  return copysign(n * quantum, v);
}

/* f32 -> e4m3fn code, round to nearest even, saturating at +-448. */
uint8_t oracle_f32_to_e4m3fn(float x) {
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return sign | 0x7F;
  double r = fabs(round_to_format((double)x, 3, -6));
  if (r > 448.0) r = 448.0;
  if (r == 0.0) return sign;
  int e;
  (void)frexp(r, &e);
  const int ex = e - 1;
  if (ex < -6) return sign | (uint8_t)(r / ldexp(1.0, -9)); /* subnormal: m * 2^-9 */
  const int m = (int)(r / ldexp(1.0, ex - 3)) - 8;
  return sign | (uint8_t)(((ex + 7) << 3) | m);
}

/* f32 -> e5m2 code, round to nearest even, saturating at +-57344. */
uint8_t oracle_f32_to_e5m2(float x) {
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return sign | 0x7F;
  double r = fabs(round_to_format((double)x, 2, -14));
  if (r > 57344.0) r = 57344.0;
  if (r == 0.0) return sign;
  int e;
  (void)frexp(r, &e);
  const int ex = e - 1;
  if (ex < -14) return sign | (uint8_t)(r / ldexp(1.0, -16)); /* subnormal: m * 2^-16 */
  const int m = (int)(r / ldexp(1.0, ex - 2)) - 4;
  return sign | (uint8_t)(((ex + 15) << 2) | m);
}

/* f32 -> IEEE binary16 bits, round to nearest even; overflow gives +-inf. */
uint16_t oracle_f32_to_f16(float x) {
  const uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
  if (isnan(x)) return sign | 0x7E00;
  double r = fabs(round_to_format((double)x, 10, -14));
  if (r >= 65536.0) return sign | 0x7C00; /* past the largest finite value after rounding */
  if (r == 0.0) return sign;
  int e;
  (void)frexp(r, &e);
  const int ex = e - 1;
  if (ex < -14) return sign | (uint16_t)(r / ldexp(1.0, -24)); /* subnormal: m * 2^-24 */
  const int m = (int)(r / ldexp(1.0, ex - 10)) - 1024;
  return sign | (uint16_t)(((ex + 15) << 10) | m);
}

/* f32 -> int8 code: round to the nearest integer, ties to even, saturating
 * at -128 and 127; NaN stores 0 (an integer code has no NaN). */
int8_t oracle_f32_to_i8(float x) {
  if (isnan(x)) return 0;
  double r = nearbyint((double)x); /* default mode: nearest, ties to even */
  if (r < -128.0) r = -128.0;
  if (r > 127.0) r = 127.0;
  return (int8_t)r;
}

/* f32 -> bf16 bits, round to nearest even; overflow gives +-inf. */
uint16_t oracle_f32_to_bf16(float x) {
  uint32_t w;
  if (isnan(x)) {
    memcpy(&w, &x, sizeof w);
    return (uint16_t)((w >> 16) | 0x0040);
  }
  double r = round_to_format((double)x, 7, -126);
  if (fabs(r) >= ldexp(1.0, 128)) r = copysign(INFINITY, r);
  const float f = (float)r; /* exact: r is a bf16 value or an infinity */
  memcpy(&w, &f, sizeof w);
  return (uint16_t)(w >> 16);
}

/* Cache value of one new element (x in the q dtype): RN_f32(x / scale) in
 * the cache type. */
static void store_elem(const oracle_cfg* c, void* kv_pages, int64_t idx, const void* x_rows, int64_t src,
                       double scale) {
  const float x = (float)q_elem(c, x_rows, src); /* exact: bf16, f16 and f32 values are f32 values */
  const float y = x / (float)scale;
  if (c->kv_dtype == ORACLE_KV_E4M3FN)
    ((uint8_t*)kv_pages)[idx] = oracle_f32_to_e4m3fn(y);
  else if (c->kv_dtype == ORACLE_KV_E5M2)
    ((uint8_t*)kv_pages)[idx] = oracle_f32_to_e5m2(y);
  else if (c->kv_dtype == ORACLE_F16)
    ((uint16_t*)kv_pages)[idx] = oracle_f32_to_f16(y);
  else if (c->kv_dtype == ORACLE_KV_I8)
    ((int8_t*)kv_pages)[idx] = oracle_f32_to_i8(y);
  else
    ((uint16_t*)kv_pages)[idx] = oracle_f32_to_bf16(y);
}

/* Writes k_new / v_new [num_q_tokens, Hkv, D] (in the q dtype) of every query
 * token of the first num_seqs sequences into kv_pages. A token whose key
 * position or page falls outside the table (a broken precondition) is not
 * written. Returns the number of such tokens, or -1 for a bad argument. */
int64_t oracle_kv_append(const oracle_cfg* c, const void* k_new, const void* v_new, void* kv_pages,
                         const int32_t* kv_lens, const int32_t* page_indices, const int32_t* cu_q_lens,
                         int32_t num_seqs) {
  if (num_seqs < 0 || num_seqs > c->max_num_seqs || c->num_kv_heads <= 0) return -1;
  const int Hkv = c->num_kv_heads, D = c->head_dim;
  int64_t skipped = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t q0 = cu_q_lens[s], q_len = (int64_t)cu_q_lens[s + 1] - q0;
    for (int64_t i = 0; i < q_len; ++i) {
      const int64_t t = q0 + i;
      const int64_t pos = (int64_t)kv_lens[s] - q_len + i;
      if (t < 0 || t >= c->num_q_tokens || pos < 0 || pos >= (int64_t)c->pages_per_seq * c->page_size) {
        ++skipped;
        continue;
      }
      const int32_t page = page_indices[(int64_t)s * c->pages_per_seq + pos / c->page_size];
      if (page < 0 || page >= c->total_num_pages) {
        ++skipped;
        continue;
      }
      const int64_t slot = (int64_t)page * c->page_size + pos % c->page_size;
      for (int h = 0; h < Hkv; ++h)
        for (int d = 0; d < D; ++d) {
          const int64_t src = (t * Hkv + h) * D + d;
          const int64_t dst_k = (slot * 2 * Hkv + 2 * h) * D + d;
          store_elem(c, kv_pages, dst_k, k_new, src, c->k_scale);
          store_elem(c, kv_pages, dst_k + D, v_new, src, c->v_scale);
        }
    }
  }
  return skipped;
}
