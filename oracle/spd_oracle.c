/*
 * spd_oracle.c -- plain fp64 CPU oracle for sparse decode attention over a
 * unified paged KV pool, and for the decode index builder that feeds it.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library and must never be used as a
 * fallback for it.
 *
 * Sources (page: sglang PR #28392 summary, "key source snippet" section, the
 * paged_decode.py module docstring):
 *   - unified_kv is [total_pages, D] bf16 with page_size 1; one row is both the
 *     key and the value (the pool is a single [P, D] tensor and out is
 *     [N, H, D]).
 *   - token t attends to the rows kv_indices[kv_indptr[t] : kv_indptr[t+1]];
 *     a token with kv_indptr[t+1] == kv_indptr[t] has an empty slice.
 *   - attn_sink[H] is a per-head learnable bias in the softmax denominator,
 *     merged as a virtual key.
 *   - the GPU kernel works in the log2 domain with
 *     qk_scale = softmax_scale * log2(e); exp(x) == 2^(x*log2 e) makes that the
 *     same function as the natural-log form computed here.
 *   - slots [0, swa_pages) of the pool hold sliding-window entries at
 *     state_slot * win + ring; slots [swa_pages, ...) hold compressed entries
 *     at block_id * K_PER_BLOCK + slot_in_block (offset by swa_pages).
 *   - the production index builder emits ragged-packed indices with no
 *     sentinel values.
 *
 * FP8 pool (the pages' caches have FP8 variants; on the sglang PR #25898
 * summary page, sections "comment highlights" and "risks and impact", a
 * review flags the ROCm software FP8 conversion rounding half up where
 * round-to-nearest-even is wanted): a row is stored as D OCP e4m3 codes plus
 * one fp32 scale, and its value is scale * e4m3(code); the quantiser rounds
 * to nearest even.
 *
 * Readings where the page is silent (each is listed in the design notes):
 *   - the sink is a natural-log logit in the units of the scaled score
 *     softmax_scale * q.k (it is not multiplied by softmax_scale);
 *   - an empty slice gives exactly 0 (with a -inf sink, 0/0 is defined as 0);
 *   - duplicate indices are separate keys (the slice is a multiset);
 *   - softmax_scale is an fp32 scalar; the oracle uses its exact fp32 value;
 *   - builder order: the window part first (ring slots 0..swa_len-1
 *     ascending), then the compressed part in comp_pos order with negative
 *     entries dropped.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact bf16 -> double: a bf16 value is the top 16 bits of an IEEE fp32. */
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP e4m3 (the "fn" variant: no infinities) -> double, from its definition:
 * sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
 * subnormal (m * 2^-9); S.1111.111 is NaN. */
static double e4m3_to_double(uint8_t c) {
  const int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

double spd_oracle_e4m3_value(int code) { return e4m3_to_double((uint8_t)code); }

/* A pool row decoded to fp64: bf16 bits, or (when kv8 is given) fp8 codes
 * times the row's scale. */
static void decode_row(const uint16_t* kv, const uint8_t* kv8, const float* kv_scale, int64_t r,
                       int32_t D, double* dst) {
  if (kv8) {
    const double sc = (double)kv_scale[r];
    for (int32_t d = 0; d < D; ++d) dst[d] = sc * e4m3_to_double(kv8[r * (int64_t)D + d]);
  } else {
    for (int32_t d = 0; d < D; ++d) dst[d] = bf16_bits_to_double(kv[r * (int64_t)D + d]);
  }
}

void spd_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int spd_oracle_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Attention for one token t (all heads), written out as the definition:
 *   J = kv_indices[kv_indptr[t] : kv_indptr[t+1]],  L = |J|
 *   L == 0:  out[t,h,:] = 0
 *   else:    s_j = sigma * sum_d q[t,h,d] * KV[J_j, d]
 *            M   = max(sink_h, max_j s_j)
 *            w_j = exp(s_j - M)
 *            Z   = exp(sink_h - M) + sum_j w_j
 *            out[t,h,:] = sum_j w_j * KV[J_j, :] / Z
 * Two passes over the slice per head: scores first, then weights and the
 * weighted sum.  All arithmetic in fp64.  Returns 0, or -1 when an index is
 * outside [0, num_rows) (a caller precondition on the page).
 */
static int attend_one_token(const uint16_t* q, const uint16_t* kv, const uint8_t* kv8,
                            const float* kv_scale, int64_t num_rows,
                            const int32_t* kv_indices, const int32_t* kv_indptr,
                            const float* attn_sink, double sigma, int32_t t, int32_t H,
                            int32_t D, double* out_t /* [H][D] */) {
  const int64_t begin = kv_indptr[t];
  const int64_t end = kv_indptr[t + 1];
  const int64_t L = end - begin;
  memset(out_t, 0, sizeof(double) * (size_t)H * (size_t)D);
  if (L <= 0) return L < 0 ? -1 : 0;

  /* Decode the gathered rows and this token's queries to fp64 once. */
  double* rows = (double*)malloc(sizeof(double) * (size_t)L * (size_t)D);
  double* qd = (double*)malloc(sizeof(double) * (size_t)D);
  double* s = (double*)malloc(sizeof(double) * (size_t)L);
  if (!rows || !qd || !s) {
    free(rows); free(qd); free(s);
    return -2;
  }
  for (int64_t j = 0; j < L; ++j) {
    const int64_t r = kv_indices[begin + j];
    if (r < 0 || r >= num_rows) {
      free(rows); free(qd); free(s);
      return -1;
    }
    decode_row(kv, kv8, kv_scale, r, D, rows + j * D);
  }

  for (int32_t h = 0; h < H; ++h) {
    const uint16_t* qh = q + ((int64_t)t * H + h) * D;
    for (int32_t d = 0; d < D; ++d) qd[d] = bf16_bits_to_double(qh[d]);
    const double sink = (double)attn_sink[h];

    /* pass 1: scores and their maximum together with the sink logit */
    double M = sink;
    for (int64_t j = 0; j < L; ++j) {
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d) dot += qd[d] * rows[j * D + d];
      s[j] = sigma * dot;
      if (s[j] > M) M = s[j];
    }
    /* pass 2: weights, normaliser (sink included as a virtual key), output */
    double Z = exp(sink - M); /* 0 when the sink is -inf */
    double* o = out_t + (int64_t)h * D;
    for (int64_t j = 0; j < L; ++j) {
      const double w = exp(s[j] - M);
      Z += w;
      for (int32_t d = 0; d < D; ++d) o[d] += w * rows[j * D + d];
    }
    for (int32_t d = 0; d < D; ++d) o[d] /= Z;
  }
  free(rows); free(qd); free(s);
  return 0;
}

/*
 * q[N,H,D], kv[num_rows,D]: bf16 bit patterns; kv_indices, kv_indptr[N+1]:
 * int32; attn_sink[H]: fp32; softmax_scale: fp32.
 * tokens: optional list of n_tokens token ids to evaluate (NULL = all N, in
 * order); out: fp64 [n_out][H][D] with n_out = tokens ? n_tokens : N.
 * Returns 0 on success, -1 on an out-of-range index or a decreasing indptr,
 * -2 on allocation failure, -3 on bad sizes.
 */
static int attend_all(const uint16_t* q, const uint16_t* kv, const uint8_t* kv8,
                      const float* kv_scale, int64_t num_rows, const int32_t* kv_indices,
                      const int32_t* kv_indptr, const float* attn_sink, float softmax_scale,
                      int32_t N, int32_t H, int32_t D, const int32_t* tokens, int32_t n_tokens,
                      double* out) {
  if (N < 0 || H <= 0 || D <= 0 || num_rows < 0) return -3;
  const int32_t n_out = tokens ? n_tokens : N;
  const double sigma = (double)softmax_scale;
  int status = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int32_t i = 0; i < n_out; ++i) {
    const int32_t t = tokens ? tokens[i] : i;
    int rc;
    if (t < 0 || t >= N)
      rc = -3;
    else
      rc = attend_one_token(q, kv, kv8, kv_scale, num_rows, kv_indices, kv_indptr, attn_sink,
                            sigma, t, H, D, out + (int64_t)i * H * D);
    if (rc != 0) {
#ifdef _OPENMP
#pragma omp critical
#endif
      status = rc;
    }
  }
  return status;
}

int spd_oracle_sparse_decode_attn(const uint16_t* q, const uint16_t* kv, int64_t num_rows,
                                  const int32_t* kv_indices, const int32_t* kv_indptr,
                                  const float* attn_sink, float softmax_scale, int32_t N,
                                  int32_t H, int32_t D, const int32_t* tokens,
                                  int32_t n_tokens, double* out) {
  return attend_all(q, kv, NULL, NULL, num_rows, kv_indices, kv_indptr, attn_sink, softmax_scale,
                    N, H, D, tokens, n_tokens, out);
}

/* The same definition over an FP8 pool: row r is kv_scale[r] * e4m3(kv8[r][:]). */
int spd_oracle_sparse_decode_attn_fp8(const uint16_t* q, const uint8_t* kv8,
                                      const float* kv_scale, int64_t num_rows,
                                      const int32_t* kv_indices, const int32_t* kv_indptr,
                                      const float* attn_sink, float softmax_scale, int32_t N,
                                      int32_t H, int32_t D, const int32_t* tokens,
                                      int32_t n_tokens, double* out) {
  if (!kv8 || !kv_scale) return -3;
  return attend_all(q, NULL, kv8, kv_scale, num_rows, kv_indices, kv_indptr, attn_sink,
                    softmax_scale, N, H, D, tokens, n_tokens, out);
}

/*
 * FP8 quantisation of bf16 rows (the store into an FP8 pool), in fp32
 * arithmetic step by step, so that a device implementation doing the same
 * IEEE operations gives the same codes:
 *   amax  = max_d |x_d|                       (exact)
 *   amax < 2^-64:  scale = 0, every code 0    (a zero row)
 *   else:  scale = amax / 448, inv = 448 / amax   (fp32, correctly rounded)
 *          y_d = x_d * inv (fp32), clamped to [-448, 448]
 *          code_d = |y_d| rounded to the nearest e4m3 value, ties to the even
 *                   mantissa, with the sign bit of x_d
 * 448 is the largest finite e4m3 value.  Rounding, for a = |y_d|:
 *   a < 2^-6 (subnormal range):  m = rint(a * 2^9), code = m  (m = 8 is 2^-6)
 *   else: e = floor(log2 a), q = rint(a * 2^(3-e)) in [8, 16] (16: e + 1, q = 8),
 *         code = (e + 7) << 3 | (q - 8)
 * rint rounds half to even in the default rounding mode.
 */
static uint8_t e4m3_rne(float y, int negative) {
  float a = fabsf(y);
  uint8_t code;
  if (a < 0.015625f) { /* 2^-6 */
    code = (uint8_t)rintf(a * 512.0f);
  } else {
    uint32_t bits;
    memcpy(&bits, &a, sizeof bits);
    int e = (int)((bits >> 23) & 0xff) - 127;
    float q = rintf(ldexpf(a, 3 - e));
    if (q >= 16.0f) {
      e += 1;
      q = 8.0f;
    }
    code = (uint8_t)(((e + 7) << 3) | ((int)q - 8));
  }
  return negative ? (uint8_t)(code | 0x80) : code;
}

int spd_oracle_quantize_fp8(const uint16_t* src, int32_t n, int32_t D, uint8_t* codes,
                            float* scales) {
  if (n < 0 || D <= 0) return -3;
  for (int32_t i = 0; i < n; ++i) {
    const uint16_t* x = src + (int64_t)i * D;
    float amax = 0.0f;
    for (int32_t d = 0; d < D; ++d) {
      const float v = fabsf((float)bf16_bits_to_double(x[d]));
      if (v > amax) amax = v;
    }
    uint8_t* c = codes + (int64_t)i * D;
    if (!(amax >= 5.421010862427522e-20f)) { /* 2^-64, also catches NaN */
      scales[i] = 0.0f;
      memset(c, 0, (size_t)D);
      continue;
    }
    const volatile float amax_v = amax;  /* keep each fp32 operation as written */
    const float scale = amax_v / 448.0f;
    const float inv = 448.0f / amax_v;
    scales[i] = scale;
    for (int32_t d = 0; d < D; ++d) {
      const float xv = (float)bf16_bits_to_double(x[d]);
      float y = xv * inv;
      if (y > 448.0f) y = 448.0f;
      if (y < -448.0f) y = -448.0f;
      c[d] = e4m3_rne(y, (x[d] >> 15) & 1);
    }
  }
  return 0;
}

/*
 * Decode index builder.  For each token t, in token order:
 *   window part:      state_slot[t] * win + r          for r = 0 .. swa_len[t]-1
 *   compressed part:  swa_pages + block_table[t][c / k_per_block] * k_per_block
 *                               + c % k_per_block
 *                     for each entry c of comp_pos[t][0 .. topk-1] with c >= 0,
 *                     in row order (negative entries mean "no entry")
 * kv_indptr[0] = 0 and kv_indptr[t+1] = kv_indptr[t] + (entries of token t).
 * comp_pos may be NULL (no compressed part); block_table is then unused.
 * Returns 0, or a negative code: -3 bad sizes / win <= 0 / k_per_block <= 0,
 * -4 capacity too small, -5 swa_len outside [0, win], -6 a block lookup
 * outside [0, max_blocks).
 */
int spd_oracle_build_decode_indices(const int32_t* state_slot, const int32_t* swa_len,
                                    const int32_t* comp_pos, int32_t topk,
                                    const int32_t* block_table, int32_t max_blocks, int32_t N,
                                    int32_t win, int32_t k_per_block, int32_t swa_pages,
                                    int32_t* kv_indptr, int32_t* kv_indices, int64_t capacity) {
  if (N < 0 || win <= 0 || k_per_block <= 0 || topk < 0 || swa_pages < 0) return -3;
  int64_t n = 0;
  kv_indptr[0] = 0;
  for (int32_t t = 0; t < N; ++t) {
    if (swa_len[t] < 0 || swa_len[t] > win) return -5;
    for (int32_t r = 0; r < swa_len[t]; ++r) {
      if (n >= capacity) return -4;
      kv_indices[n++] = (int32_t)((int64_t)state_slot[t] * win + r);
    }
    if (comp_pos) {
      for (int32_t c = 0; c < topk; ++c) {
        const int32_t pos = comp_pos[(int64_t)t * topk + c];
        if (pos < 0) continue;
        const int32_t blk = pos / k_per_block;
        if (blk >= max_blocks) return -6;
        if (n >= capacity) return -4;
        const int64_t block_id = block_table[(int64_t)t * max_blocks + blk];
        kv_indices[n++] = (int32_t)(swa_pages + block_id * k_per_block + pos % k_per_block);
      }
    }
    kv_indptr[t + 1] = (int32_t)n;
  }
  return 0;
}

/*
 * The builder over metadata that breaks its preconditions (the pages say
 * nothing of such input; this is the rule the library's builder and its fused
 * page transform document): a ring length outside [0, win] counts as the
 * nearest bound, and a compressed entry c >= 0 whose block c / k_per_block
 * lies outside [0, max_blocks) counts as no entry.  The inputs are mapped by
 * that rule, then built exactly as spd_oracle_build_decode_indices does.
 * Same return codes, except that -5 and -6 cannot occur; -7 when the copies
 * cannot be allocated.
 */
int spd_oracle_build_decode_indices_clamped(const int32_t* state_slot, const int32_t* swa_len,
                                            const int32_t* comp_pos, int32_t topk,
                                            const int32_t* block_table, int32_t max_blocks,
                                            int32_t N, int32_t win, int32_t k_per_block,
                                            int32_t swa_pages, int32_t* kv_indptr,
                                            int32_t* kv_indices, int64_t capacity) {
  if (N < 0 || win <= 0 || k_per_block <= 0 || topk < 0 || swa_pages < 0) return -3;
  int32_t* len = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
  int32_t* pos = comp_pos ? (int32_t*)malloc(sizeof(int32_t) * (size_t)((int64_t)N * topk + 1))
                          : NULL;
  if (!len || (comp_pos && !pos)) {
    free(len);
    free(pos);
    return -7;
  }
  for (int32_t t = 0; t < N; ++t) len[t] = swa_len[t] < 0 ? 0 : (swa_len[t] > win ? win : swa_len[t]);
  if (comp_pos) {
    for (int64_t i = 0; i < (int64_t)N * topk; ++i) {
      const int32_t c = comp_pos[i];
      pos[i] = (c >= 0 && c / k_per_block >= max_blocks) ? -1 : c;
    }
  }
  const int rc = spd_oracle_build_decode_indices(state_slot, len, pos, topk, block_table, max_blocks,
                                                 N, win, k_per_block, swa_pages, kv_indptr,
                                                 kv_indices, capacity);
  free(len);
  free(pos);
  return rc;
}

/*
 * Producer of the decode step: per-head RMSNorm of q, RMSNorm of the token's
 * new KV row, rotary embedding of both, and the ring slot the KV row is
 * stored in (sglang PR #25898 summary page, "key files": one kernel does the
 * q per-head RMSNorm, the KV RMSNorm, RoPE, the FP8 quantisation and the paged
 * sliding-window store; its helpers are a batched RMSNorm, a GPT-J rotation
 * and a batched RoPE).  Readings (the page names the steps, not their
 * formulas):
 *   RMSNorm of a row x[0, D) with weight w:  x_d * w_d / sqrt(mean_d(x_d^2) + eps)
 *   RoPE, GPT-J (interleaved) pairs on the last rope_dim entries (o = D - rope_dim):
 *     for i < rope_dim / 2, c = cos_sin[p][i], s = cos_sin[p][rope_dim/2 + i],
 *     (y[o+2i], y[o+2i+1]) <- (y[o+2i] c - y[o+2i+1] s, y[o+2i] s + y[o+2i+1] c)
 *   where p = positions[t] and cos_sin is the caller's table [max_pos][rope_dim];
 *   the KV row's ring slot: state_slot[t] * win + p mod win (the window ring
 *   holds positions p - win + 1 .. p, slot p mod win).
 * Outputs in fp64, unrounded: q_out [N][H][D], kv_out [N][D], slot_out [N].
 * A token with p < 0, or p >= max_pos when rope_dim > 0 (a position the table
 * does not hold), gets slot_out = -1 and zero rows.
 */
static void norm_rope_row(const uint16_t* x, const float* w, double eps, const float* cs,
                          int32_t rope_dim, int32_t D, double* y) {
  double ss = 0.0;
  for (int32_t d = 0; d < D; ++d) {
    const double v = bf16_bits_to_double(x[d]);
    ss += v * v;
  }
  const double inv = 1.0 / sqrt(ss / D + eps);
  for (int32_t d = 0; d < D; ++d) y[d] = bf16_bits_to_double(x[d]) * inv * (double)w[d];
  const int32_t o = D - rope_dim, half = rope_dim / 2;
  for (int32_t i = 0; i < half; ++i) {
    const double c = cs[i], s = cs[half + i];
    const double a = y[o + 2 * i], b = y[o + 2 * i + 1];
    y[o + 2 * i] = a * c - b * s;
    y[o + 2 * i + 1] = a * s + b * c;
  }
}

int spd_oracle_qk_norm_rope(const uint16_t* q, const uint16_t* kv, const float* q_weight,
                            const float* kv_weight, float eps, const int32_t* positions,
                            const float* cos_sin, int32_t max_pos, int32_t rope_dim,
                            const int32_t* state_slot, int32_t win, int32_t N, int32_t H,
                            int32_t D, double* q_out, double* kv_out, int64_t* slot_out) {
  if (N < 0 || H <= 0 || D <= 0 || rope_dim < 0 || rope_dim > D || (rope_dim & 1) || win <= 0 ||
      max_pos < 0 || !(eps >= 0.0f))
    return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t t = 0; t < N; ++t) {
    const int32_t p = positions[t];
    if (p < 0 || (rope_dim > 0 && p >= max_pos)) {
      memset(q_out + (int64_t)t * H * D, 0, sizeof(double) * (size_t)H * D);
      memset(kv_out + (int64_t)t * D, 0, sizeof(double) * (size_t)D);
      slot_out[t] = -1;
      continue;
    }
    const float* cs = cos_sin + (int64_t)p * rope_dim;
    for (int32_t h = 0; h < H; ++h)
      norm_rope_row(q + ((int64_t)t * H + h) * D, q_weight, (double)eps, cs, rope_dim, D,
                    q_out + ((int64_t)t * H + h) * D);
    norm_rope_row(kv + (int64_t)t * D, kv_weight, (double)eps, cs, rope_dim, D,
                  kv_out + (int64_t)t * D);
    slot_out[t] = (int64_t)state_slot[t] * win + p % win;
  }
  return 0;
}
