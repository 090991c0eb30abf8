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
static int attend_one_token(const uint16_t* q, const uint16_t* kv, int64_t num_rows,
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
    for (int32_t d = 0; d < D; ++d)
      rows[j * D + d] = bf16_bits_to_double(kv[r * (int64_t)D + d]);
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
int spd_oracle_sparse_decode_attn(const uint16_t* q, const uint16_t* kv, int64_t num_rows,
                                  const int32_t* kv_indices, const int32_t* kv_indptr,
                                  const float* attn_sink, float softmax_scale, int32_t N,
                                  int32_t H, int32_t D, const int32_t* tokens,
                                  int32_t n_tokens, double* out) {
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
      rc = attend_one_token(q, kv, num_rows, kv_indices, kv_indptr, attn_sink, sigma, t, H, D,
                            out + (int64_t)i * H * D);
    if (rc != 0) {
#ifdef _OPENMP
#pragma omp critical
#endif
      status = rc;
    }
  }
  return status;
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
