/*
 * Paged-KV attention oracle: plain, slow, obviously correct C in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code, header
 * or table with the HIP library and must never be reached from the product
 * path.
 *
 * What it computes (sources: the page "vLLM 架构概述" §2 on the block pool and
 * per-request int32 block tables with a lookup plus address arithmetic; the
 * page "vLLM：从 KV Cache 到高吞吐推理服务", tutorial 3 on logical block,
 * physical block, offset and slot, and tutorial 1 on MHA/GQA/MQA head sharing;
 * the reading note on "Inside vLLM", core point 1 on 16-token blocks and
 * allocation, core point 2 on the flattened super-sequence with per-sequence
 * masking):
 *
 *  - addressing: token j of sequence s lives in physical block
 *    block_tables[s][j / B] at offset j % B; its slot is phys * B + offset;
 *  - a sequence of seq_lens[s] tokens whose last q_len tokens are new has
 *    c = seq_lens[s] - q_len cached tokens; new row i sits at position c + i
 *    and attends to positions 0 .. c + i of its own sequence only;
 *  - attention is the textbook softmax(scale * q k^T) v, evaluated in two
 *    passes (max, then exp-sum and weighted sum) in double precision from the
 *    exact values of the stored inputs;
 *  - q head h reads kv head h / (Hq / Hkv);
 *  - writing new K/V: cache[slot / B][slot % B][h][:] = new[t][h][:], slot < 0
 *    skipped; fp8 E4M3 stores round-to-nearest-even(fl32(x / scale)) with
 *    saturation to +-448 (OCP E4M3FN: bias 7, no infinities, S.1111.111 NaN).
 *
 * Built with gcc -O2 -ffp-contract=off -fopenmp; no fast-math.  Threads only
 * split independent (row, head) outputs; each output's arithmetic runs in the
 * order written here.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { O_F32 = 0, O_BF16 = 1, O_FP8 = 2 };

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ---- scalar decoding of stored element types --------------------------------- */

static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16; /* bf16 is the top half of an fp32 */
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits.
 * e == 0: subnormal m * 2^-9.  e in 1..15: 2^(e-7) * (1 + m/8).
 * e == 15 && m == 7: NaN.  No infinities. */
double oracle_fp8_decode(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Round a float to the nearest E4M3FN code, ties to even mantissa, finite
 * overflow (and infinity) saturating to +-448, NaN to the NaN code with the
 * input's sign. */
uint8_t oracle_fp8_encode(float x) {
  uint32_t bits;
  memcpy(&bits, &x, 4);
  uint8_t sign = (uint8_t)((bits >> 31) << 7);
  if (isnan(x)) return (uint8_t)(sign | 0x7F);
  if (isinf(x)) return (uint8_t)(sign | 0x7E);
  double a = fabs((double)x);
  if (a == 0.0) return sign;
  /* choose the binade: quantum is 2^-9 below 2^-6, else 2^(e-3) for a in [2^e, 2^(e+1)) */
  int e;
  double quantum;
  if (a < ldexp(1.0, -6)) {
    e = -6;
    quantum = ldexp(1.0, -9);
  } else {
    e = (int)floor(log2(a));
    /* guard log2 rounding at exact powers of two */
    if (ldexp(1.0, e) > a) e -= 1;
    if (ldexp(1.0, e + 1) <= a) e += 1;
    quantum = ldexp(1.0, e - 3);
  }
  if (e > 8) return (uint8_t)(sign | 0x7E);
  double q = rint(a / quantum); /* exact division by a power of two; rint is ties-to-even */
  /* q counts quanta: below 2^-6 code = q (0..8); else code = (e + 7) * 8 + (q - 8) */
  int code;
  if (a < ldexp(1.0, -6))
    code = (int)q;
  else
    code = (e + 7) * 8 + ((int)q - 8);
  if (code > 0x7E) code = 0x7E; /* saturate: 0x7F is NaN */
  return (uint8_t)(sign | code);
}

static double load_elem(const void* base, int64_t idx, int dtype) {
  switch (dtype) {
    case O_F32: return (double)((const float*)base)[idx];
    case O_BF16: return bf16_bits_to_double(((const uint16_t*)base)[idx]);
    default: return oracle_fp8_decode(((const uint8_t*)base)[idx]);
  }
}

/* ---- slot mapping -------------------------------------------------------------- */

/* slot_mapping[t] for every new token t of every sequence. */
int oracle_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables, int32_t bt_stride,
                        const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                        int32_t block_size) {
  for (int s = 0; s < num_seqs; ++s) {
    int q_len = query_start_loc[s + 1] - query_start_loc[s];
    int cached = seq_lens[s] - q_len;
    if (q_len < 0 || cached < 0) return -1;
    for (int i = 0; i < q_len; ++i) {
      int pos = cached + i;
      int logical = pos / block_size;
      int offset = pos % block_size;
      int phys = block_tables[(int64_t)s * bt_stride + logical];
      slot_mapping[query_start_loc[s] + i] = phys * block_size + offset;
    }
  }
  return 0;
}

/* ---- writing new tokens into the pool --------------------------------------- */

/* Plain byte copy: cache[slot / B][slot % B][h][:] = src[t][h][:]. Strides in elements. */
int oracle_reshape_and_cache(const void* key, const void* value, int64_t key_tok_stride,
                             int64_t value_tok_stride, void* key_cache, void* value_cache,
                             const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             int32_t elem_bytes) {
  int64_t row = (int64_t)head_dim * elem_bytes;
  for (int t = 0; t < num_tokens; ++t) {
    int slot = slot_mapping[t];
    if (slot < 0) continue;
    int blk = slot / block_size, off = slot % block_size;
    if (blk >= num_blocks) return -1;
    for (int h = 0; h < num_kv_heads; ++h) {
      int64_t dst = (((int64_t)blk * block_size + off) * num_kv_heads + h) * row;
      memcpy((char*)key_cache + dst, (const char*)key + ((int64_t)t * key_tok_stride + (int64_t)h * head_dim) * elem_bytes, row);
      memcpy((char*)value_cache + dst, (const char*)value + ((int64_t)t * value_tok_stride + (int64_t)h * head_dim) * elem_bytes, row);
    }
  }
  return 0;
}

static float src_as_float(const void* base, int64_t idx, int dtype) {
  if (dtype == O_F32) return ((const float*)base)[idx];
  uint32_t u = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Same scatter, storing E4M3 codes of fl32(x / scale). */
int oracle_reshape_and_cache_fp8(const void* key, const void* value, int64_t key_tok_stride,
                                 int64_t value_tok_stride, uint8_t* key_cache, uint8_t* value_cache,
                                 const int32_t* slot_mapping, int32_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, int32_t src_dtype, float k_scale, float v_scale) {
  for (int t = 0; t < num_tokens; ++t) {
    int slot = slot_mapping[t];
    if (slot < 0) continue;
    int blk = slot / block_size, off = slot % block_size;
    if (blk >= num_blocks) return -1;
    for (int h = 0; h < num_kv_heads; ++h) {
      int64_t dst = (((int64_t)blk * block_size + off) * num_kv_heads + h) * head_dim;
      for (int d = 0; d < head_dim; ++d) {
        float xk = src_as_float(key, (int64_t)t * key_tok_stride + (int64_t)h * head_dim + d, src_dtype);
        float xv = src_as_float(value, (int64_t)t * value_tok_stride + (int64_t)h * head_dim + d, src_dtype);
        volatile float qk = xk / k_scale; /* one fp32 division, correctly rounded */
        volatile float qv = xv / v_scale;
        key_cache[dst + d] = oracle_fp8_encode(qk);
        value_cache[dst + d] = oracle_fp8_encode(qv);
      }
    }
  }
  return 0;
}

/* ---- attention ---------------------------------------------------------------- */

/* out[r][h][d] (fp64) for the query rows listed in rows[0..n_rows) (all rows
 * 0..T-1 when rows is NULL, n_rows = T).  Returns 0, or -1 on inconsistent
 * metadata. kv values of fp8 pools are decode(code) * k_scale / v_scale. */
/* Which keys a row sees.  Sliding window (window > 0): the row at position pos sees keys
 * max(0, pos - window + 1) .. pos, a window of `window` tokens ending at its own.  Chunked
 * local attention (chunk > 0): the positions are cut into chunks of `chunk` (0 .. chunk-1,
 * chunk .. 2*chunk-1, ...) and the row sees the keys of its own chunk up to itself,
 * pos - pos % chunk .. pos.  Neither: every key 0 .. pos.  (Readings of the pages'
 * sliding-window and chunked-local attention; the pages name them but fix no boundary.) */
static int first_visible_key(int pos, int32_t window, int32_t chunk) {
  if (chunk > 0) return pos - pos % chunk;
  if (window > 0 && pos - window + 1 > 0) return pos - window + 1;
  return 0;
}

static int attention_rows(double* out, const void* query, int32_t q_dtype, const void* key_cache,
                          const void* value_cache, int32_t kv_dtype, double k_scale, double v_scale,
                          const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                          const int32_t* query_start_loc, int32_t num_seqs, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                          const int32_t* rows, int32_t n_rows, int32_t window, int32_t chunk);

int oracle_attention(double* out, const void* query, int32_t q_dtype, const void* key_cache,
                     const void* value_cache, int32_t kv_dtype, double k_scale, double v_scale,
                     const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                     const int32_t* query_start_loc, int32_t num_seqs, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                     const int32_t* rows, int32_t n_rows) {
  return attention_rows(out, query, q_dtype, key_cache, value_cache, kv_dtype, k_scale, v_scale, block_tables,
                        bt_stride, seq_lens, query_start_loc, num_seqs, num_q_heads, num_kv_heads, head_dim,
                        block_size, scale, rows, n_rows, 0, 0);
}

int oracle_attention_window(double* out, const void* query, int32_t q_dtype, const void* key_cache,
                            const void* value_cache, int32_t kv_dtype, double k_scale, double v_scale,
                            const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                            const int32_t* query_start_loc, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                            const int32_t* rows, int32_t n_rows, int32_t window) {
  if (window < 0) return -1;
  return attention_rows(out, query, q_dtype, key_cache, value_cache, kv_dtype, k_scale, v_scale, block_tables,
                        bt_stride, seq_lens, query_start_loc, num_seqs, num_q_heads, num_kv_heads, head_dim,
                        block_size, scale, rows, n_rows, window, 0);
}

int oracle_attention_local(double* out, const void* query, int32_t q_dtype, const void* key_cache,
                           const void* value_cache, int32_t kv_dtype, double k_scale, double v_scale,
                           const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                           const int32_t* query_start_loc, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                           const int32_t* rows, int32_t n_rows, int32_t chunk) {
  if (chunk < 0) return -1;
  return attention_rows(out, query, q_dtype, key_cache, value_cache, kv_dtype, k_scale, v_scale, block_tables,
                        bt_stride, seq_lens, query_start_loc, num_seqs, num_q_heads, num_kv_heads, head_dim,
                        block_size, scale, rows, n_rows, 0, chunk);
}

static int attention_rows(double* out, const void* query, int32_t q_dtype, const void* key_cache,
                          const void* value_cache, int32_t kv_dtype, double k_scale, double v_scale,
                          const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                          const int32_t* query_start_loc, int32_t num_seqs, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                          const int32_t* rows, int32_t n_rows, int32_t window, int32_t chunk) {
  if (num_q_heads % num_kv_heads) return -1;
  int group = num_q_heads / num_kv_heads;
  int T = query_start_loc[num_seqs];
  if (!rows) n_rows = T;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t job = 0; job < (int64_t)n_rows * num_q_heads; ++job) {
    int ri = (int)(job / num_q_heads), h = (int)(job % num_q_heads);
    int t = rows ? rows[ri] : ri;
    /* which sequence owns row t */
    int s = 0;
    while (s < num_seqs && query_start_loc[s + 1] <= t) ++s;
    if (s >= num_seqs) { bad = 1; continue; }
    int q_len = query_start_loc[s + 1] - query_start_loc[s];
    int cached = seq_lens[s] - q_len;
    int pos = cached + (t - query_start_loc[s]);
    int kvh = h / group;
    int j0 = first_visible_key(pos, window, chunk);
    int n_keys = pos + 1;
    double* z = (double*)malloc(sizeof(double) * n_keys);
    double* q = (double*)malloc(sizeof(double) * head_dim);
    for (int d = 0; d < head_dim; ++d)
      q[d] = load_elem(query, ((int64_t)t * num_q_heads + h) * head_dim + d, q_dtype);
    /* pass 1: scores and their max */
    double m = -INFINITY;
    for (int j = j0; j < n_keys; ++j) {
      int phys = block_tables[(int64_t)s * bt_stride + j / block_size];
      int off = j % block_size;
      int64_t base = (((int64_t)phys * block_size + off) * num_kv_heads + kvh) * head_dim;
      double acc = 0.0;
      for (int d = 0; d < head_dim; ++d) {
        double k = load_elem(key_cache, base + d, kv_dtype);
        if (kv_dtype == O_FP8) k *= k_scale;
        acc += q[d] * k;
      }
      z[j] = (double)scale * acc;
      if (z[j] > m) m = z[j];
    }
    /* pass 2: weights, their sum, and the weighted sum of values */
    double l = 0.0;
    double* o = out + ((int64_t)ri * num_q_heads + h) * head_dim;
    for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
    for (int j = j0; j < n_keys; ++j) {
      double w = exp(z[j] - m);
      l += w;
      int phys = block_tables[(int64_t)s * bt_stride + j / block_size];
      int off = j % block_size;
      int64_t base = (((int64_t)phys * block_size + off) * num_kv_heads + kvh) * head_dim;
      for (int d = 0; d < head_dim; ++d) {
        double v = load_elem(value_cache, base + d, kv_dtype);
        if (kv_dtype == O_FP8) v *= v_scale;
        o[d] += w * v;
      }
    }
    for (int d = 0; d < head_dim; ++d) o[d] /= l;
    free(z);
    free(q);
  }
  return bad ? -1 : 0;
}
