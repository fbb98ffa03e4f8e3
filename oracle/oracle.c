/*
 * oracle.c -- plain, slow CPU reference for batched paged MLA decode.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only callers.  It shares no code with
 * the GPU library and the GPU library never calls it.
 *
 * What it computes (the decode call of "sglang trtllm_mla_backend.py",
 * TRTLLMMLABackend._run_decode_kernel, and "tokenspeed flashmla.py",
 * FlashMLABackend.forward_decode / forward_extend with causal=True):
 *
 *   For request b with L = seq_lens[b] cached tokens (the new tokens
 *   included), query token j < q_len and head h, the visible tokens are
 *   t < n = L - q_len + 1 + j (bottom-right causal alignment: the last query
 *   token sees all L rows).  Token t lives in pool page
 *   block_table[b][t / page_size] at slot t % page_size; its row is 576 wide:
 *   the 512-wide latent c_kv then the 64-wide rope key.
 *
 *     s_t   = scale * sum_{d<576} q[b,j,h,d] * row_t[d]
 *     lse   = ln sum_t exp(s_t)
 *     o[c]  = sum_t exp(s_t - lse) * row_t[c],   c < 512
 *
 *   scale is the softmax scale (1/sqrt(head_dim)); with an fp8 pool every
 *   stored value is dequantised as code * k_scale before use, so the bmm1
 *   scale of the pages (softmax_scale * k_scale) and the output both see the
 *   dequantised rows.  No visible token: o = 0, lse = -inf (the zero-KV row
 *   convention of sglang's backend, where such rows are fixed up to out=0 and
 *   lse=-inf).
 *
 * Everything is evaluated in double precision: the inputs are decoded
 * exactly (bf16 and e4m3fn values are exact doubles), dot products are summed
 * sequentially over d, and the softmax takes two passes (maximum, then sum).
 *
 * Planted-mistake builds: compiling with -DORACLE_MUTANT=k changes one step
 * on purpose; the test suite uses those builds to show its pins catch each
 * such mistake.  The default build has no mutant.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif
#define MUT(k) (ORACLE_MUTANT == (k))

#define ROW_DIM 576
#define LATENT_DIM 512

typedef struct {
  int32_t batch, q_len, num_heads, page_size, num_pages, bt_stride;
  int32_t kv_is_fp8;     /* 0: bf16 bit patterns (uint16), 1: OCP e4m3fn codes (uint8) */
  double softmax_scale;  /* the fp32 scale the GPU receives, widened */
  double k_scale;        /* fp8 dequantisation factor; unused for bf16 */
} oracle_dims;

int oracle_version(void) { return 1 + 1000 * ORACLE_MUTANT; }

/* Threads the OpenMP loops below run on (reported next to CPU timings). */
#ifdef _OPENMP
#include <omp.h>
int oracle_threads(void) { return omp_get_max_threads(); }
#else
int oracle_threads(void) { return 1; }
#endif

/* bf16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << (MUT(11) ? 15 : 16);
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP float8 e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal: (m/8) * 2^-6.  S.1111.111 is NaN; there is
 * no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448. */
double oracle_e4m3fn_to_double(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
  double v;
  if (e == 0xF && m == 7) return NAN;
  if (e == 0)
    v = MUT(10) ? ldexp((double)m, -6) : ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Page id of token t of request b, or -1 when the block-table entry is out of range. */
static int32_t page_of(const oracle_dims* D, const int32_t* bt, int32_t b, int32_t t) {
  int32_t idx = MUT(3) ? t % D->page_size : t / D->page_size;
  int32_t pg = bt[(int64_t)b * D->bt_stride + idx];
  if (pg < 0 || pg >= D->num_pages) return -1;
  return pg;
}

static int32_t slot_of(const oracle_dims* D, int32_t t) {
  return MUT(3) ? t / D->page_size : t % D->page_size;
}

/* Dequantised rows of the first n tokens of request b into rows[n][576].
 * Returns 0, or -1 if a block-table entry that is read is out of range. */
int oracle_gather_rows(const oracle_dims* D, const void* pool, const int32_t* bt, int32_t b, int32_t n,
                       double* rows) {
  for (int32_t t = 0; t < n; t++) {
    int32_t pg = page_of(D, bt, b, t);
    if (pg < 0) return -1;
    int64_t base = ((int64_t)pg * D->page_size + slot_of(D, t)) * ROW_DIM;
    double* r = rows + (int64_t)t * ROW_DIM;
    if (D->kv_is_fp8) {
      const uint8_t* p = (const uint8_t*)pool + base;
      double ks = MUT(7) ? 1.0 : D->k_scale;
      for (int d = 0; d < ROW_DIM; d++) r[d] = oracle_e4m3fn_to_double(p[d]) * ks;
    } else {
      const uint16_t* p = (const uint16_t*)pool + base;
      for (int d = 0; d < ROW_DIM; d++) r[d] = oracle_bf16_to_double(p[d]);
    }
  }
  return 0;
}

/* Byte copy of the stored rows of the first n tokens of request b into dst[n][576]
 * (elements of the pool's storage type).  Returns 0 or -1 on a bad page id. */
int oracle_gather_bytes(const oracle_dims* D, const void* pool, const int32_t* bt, int32_t b, int32_t n,
                        void* dst) {
  size_t esz = D->kv_is_fp8 ? 1 : 2;
  for (int32_t t = 0; t < n; t++) {
    int32_t pg = page_of(D, bt, b, t);
    if (pg < 0) return -1;
    int64_t base = ((int64_t)pg * D->page_size + slot_of(D, t)) * ROW_DIM;
    memcpy((char*)dst + (size_t)t * ROW_DIM * esz, (const char*)pool + (size_t)base * esz, ROW_DIM * esz);
  }
  return 0;
}

/* Softmax attention of one query row over tokens [t_begin, t_end) of the
 * decoded rows.  q_row: 576 bf16 bit patterns.  o[512], *lse (natural log).
 * An empty range gives o = 0, lse = -inf. */
void oracle_attend(const uint16_t* q_row, const double* rows, int32_t t_begin, int32_t t_end, double scale,
                   double* o, double* lse) {
  int32_t n = t_end - t_begin;
  if (MUT(13)) n -= 1;
  for (int c = 0; c < LATENT_DIM; c++) o[c] = 0.0;
  if (n <= 0) {
    *lse = -INFINITY;
    return;
  }
  double q[ROW_DIM];
  for (int d = 0; d < ROW_DIM; d++) q[d] = oracle_bf16_to_double(q_row[d]);
  double* s = (double*)malloc(sizeof(double) * (size_t)n);
  const int dims = MUT(1) ? LATENT_DIM : ROW_DIM;
  for (int32_t i = 0; i < n; i++) {
    const double* r = rows + (int64_t)(t_begin + i) * ROW_DIM;
    double acc = 0.0;
    for (int d = 0; d < dims; d++) acc += q[d] * r[d];
    s[i] = MUT(4) ? acc : scale * acc;
  }
  /* pass 1: maximum and normaliser */
  double m = -INFINITY;
  for (int32_t i = 0; i < n; i++)
    if (s[i] > m) m = s[i];
  double Z = 0.0;
  for (int32_t i = 0; i < n; i++) Z += exp(s[i] - m);
  *lse = MUT(5) ? m + log2(Z) : m + log(Z);
  /* pass 2: weighted sum of the latent part of each row */
  const int c0 = MUT(6) ? ROW_DIM - LATENT_DIM : 0;
  for (int32_t i = 0; i < n; i++) {
    double p = exp(s[i] - m);
    if (!MUT(12)) p /= Z;
    const double* r = rows + (int64_t)(t_begin + i) * ROW_DIM;
    for (int c = 0; c < LATENT_DIM; c++) o[c] += p * r[c0 + c];
  }
  free(s);
}

/* Number of tokens query token j of a request with L cached tokens may see. */
static int32_t visible(int32_t L, int32_t q_len, int32_t j) {
  if (L < 0) L = 0;
  int32_t n = MUT(2) ? L - q_len + j : L - q_len + 1 + j;
  return n < 0 ? 0 : n;
}

/* Whole decode call.  out[B][q_len][H][512], lse[B][q_len][H].  Returns 0, or
 * -1 when a block-table entry that must be read is out of range. */
int oracle_decode(const oracle_dims* D, const uint16_t* q, const void* pool, const int32_t* bt,
                  const int32_t* seq_lens, double* out, double* lse) {
  int status = 0;
  for (int32_t b = 0; b < D->batch && status == 0; b++) {
    int32_t L = seq_lens[b] < 0 ? 0 : seq_lens[b];
    double* rows = (double*)malloc(sizeof(double) * ROW_DIM * (size_t)(L > 0 ? L : 1));
    if (oracle_gather_rows(D, pool, bt, b, L, rows) != 0) {
      status = -1;
    } else {
      const int32_t nrows = D->q_len * D->num_heads;
#pragma omp parallel for schedule(dynamic, 4)
      for (int32_t r = 0; r < nrows; r++) {
        int32_t j = r / D->num_heads, h = r % D->num_heads;
        int64_t row_id = ((int64_t)b * D->q_len + j) * D->num_heads + h;
        oracle_attend(q + row_id * ROW_DIM, rows, 0, visible(L, D->q_len, j), D->softmax_scale,
                      out + row_id * LATENT_DIM, lse + row_id);
      }
    }
    free(rows);
  }
  return status;
}

/* Selected query rows only: sel[k] = (b, j, h).  out[n_sel][512], lse[n_sel].
 * The rows of each request are decoded once per selected row. */
int oracle_decode_rows(const oracle_dims* D, const uint16_t* q, const void* pool, const int32_t* bt,
                       const int32_t* seq_lens, int32_t n_sel, const int32_t* sel, double* out, double* lse) {
  int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t k = 0; k < n_sel; k++) {
    int32_t b = sel[3 * k], j = sel[3 * k + 1], h = sel[3 * k + 2];
    int32_t L = seq_lens[b] < 0 ? 0 : seq_lens[b];
    int32_t n = visible(L, D->q_len, j);
    double* rows = (double*)malloc(sizeof(double) * ROW_DIM * (size_t)(n > 0 ? n : 1));
    if (oracle_gather_rows(D, pool, bt, b, n, rows) != 0) {
#pragma omp atomic write
      status = -1;
    } else {
      int64_t row_id = ((int64_t)b * D->q_len + j) * D->num_heads + h;
      oracle_attend(q + row_id * ROW_DIM, rows, 0, n, D->softmax_scale, out + (int64_t)k * LATENT_DIM, lse + k);
    }
    free(rows);
  }
  return status;
}

/* Merge S partial results of one query row, each normalised over its own
 * token range, into the result over the union of the ranges:
 *   LSE = ln sum_s exp(lse_s),  o = sum_s exp(lse_s - LSE) * o_s.
 * Parts with lse = -inf carry no weight; if all do, o = 0 and LSE = -inf. */
void oracle_merge(int32_t S, int32_t width, const double* o_parts, const double* lse_parts, double* o,
                  double* lse) {
  double M = -INFINITY;
  for (int32_t s = 0; s < S; s++)
    if (lse_parts[s] > M) M = lse_parts[s];
  for (int32_t c = 0; c < width; c++) o[c] = 0.0;
  if (M == -INFINITY) {
    *lse = -INFINITY;
    return;
  }
  double Z = 0.0;
  for (int32_t s = 0; s < S; s++) Z += exp(lse_parts[s] - M);
  *lse = M + log(Z);
  for (int32_t s = 0; s < S; s++) {
    double w = MUT(9) ? 1.0 / S : exp(lse_parts[s] - *lse);
    if (lse_parts[s] == -INFINITY) w = 0.0;
    for (int32_t c = 0; c < width; c++) o[c] += w * o_parts[(int64_t)s * width + c];
  }
}
