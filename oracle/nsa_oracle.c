/*
 * Native sparse attention forward -- CPU fp64 ORACLE.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: it exists so that tests, the smoke check and the benchmark's
 * CPU-baseline leg can compare the HIP library against a plain, slow,
 * obviously correct definition.  It shares no code, header or constant with
 * the HIP library.
 *
 * What it computes (ejKernel "native_sparse_attention" API page, description
 * of the module and of `run` / `native_sparse_attention`, "Parameters"):
 * each query token attends only to the key blocks its row of `block_indices`
 * lists, truncated to `block_counts` entries, each block being `block_size`
 * consecutive keys; scores are scaled dot products q.k, normalised with a
 * softmax, and the output is the probability-weighted sum of values.  The
 * module "uses explicit block indices" instead of a mask builder; the oracle
 * turns the indices back into the token mask they stand for and then runs
 * plain dense masked softmax attention over it (the boolean token-mask form
 * of `create_attention_mask` on the ejKernel ragged-decode page).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - block_indices is per token: [B, T, Hkv, S] int32 (type annotation of
 *    `run`); block_counts is [B, T, Hkv] int32.
 *  - n = clamp(block_counts, 0, S); only entries 0..n-1 are read; entries < 0
 *    contribute nothing; the entry set is a set (order and repeats do not
 *    matter here).
 *  - causal: key s is visible to query t iff s <= t (inclusive diagonal, the
 *    causal block rule of the ejKernel block-sparse mask page: query block i
 *    attends blocks [0, i+1)).
 *  - query head hq uses kv head hq / (Hq / Hkv) (contiguous GQA groups).
 *  - varlen (cu_seqlens given): B == 1, tokens packed; block j of a sequence
 *    starting at bos covers tokens [bos + j*bs, bos + (j+1)*bs) clipped to
 *    the sequence, and keys come only from the token's own sequence.
 *  - lse is the natural log of sum over visible keys of exp(scale * q.k);
 *    an empty key set gives out = 0 and lse = -inf.
 *
 * Parity pins (tests/test_oracle.py): dense-causal indices equal
 * torch scaled_dot_product_attention in fp64; brute force with Python sets on
 * tiny inputs; t = 0 and q = 0 closed forms; lse gradient identity; varlen ==
 * per-sequence; invariance to entry order and to entries past the count; the
 * block-level causal example of the block-sparse mask page.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* sequence bounds of packed token x */
static void seq_bounds(int64_t x, int64_t T, const int32_t* cu, int64_t num_seqs,
                       int64_t* bos, int64_t* len) {
  if (!cu) {
    int64_t b = x / T;
    *bos = b * T;
    *len = T;
    return;
  }
  int64_t lo = 0, hi = num_seqs - 1; /* find s with cu[s] <= x < cu[s+1] */
  while (lo < hi) {
    int64_t mid = (lo + hi + 1) / 2;
    if ((int64_t)cu[mid] <= x) lo = mid; else hi = mid - 1;
  }
  *bos = cu[lo];
  *len = (int64_t)cu[lo + 1] - cu[lo];
}

/*
 * Returns 0 on success, -1 on bad arguments.
 *  q [B*T, Hq, D], k/v [B*T, Hkv, D] float32 (exact input values, widened to
 *  double here); block_indices [B*T, Hkv, S]; block_counts [B*T, Hkv];
 *  cu_seqlens [num_seqs+1] or NULL; tokens: packed token ids to evaluate
 *  (NULL = all B*T, in order); out [n_tokens, Hq, D]; lse [n_tokens, Hq].
 */
int nsa_oracle_fwd(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, int64_t S,
                   int64_t block_size, const float* q, const float* k, const float* v,
                   const int32_t* block_indices, const int32_t* block_counts,
                   const int32_t* cu_seqlens, int64_t num_seqs, double scale,
                   const int64_t* tokens, int64_t n_tokens, double* out, double* lse,
                   int num_threads) {
  if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || S <= 0 || block_size <= 0) return -1;
  if (Hq % Hkv) return -1;
  if (cu_seqlens && (B != 1 || num_seqs <= 0)) return -1;
  const int64_t G = Hq / Hkv;
  const int64_t ntok = tokens ? n_tokens : B * T;
  int64_t maxlen = T;
  if (cu_seqlens) {
    maxlen = 0;
    for (int64_t s = 0; s < num_seqs; s++) {
      int64_t l = (int64_t)cu_seqlens[s + 1] - cu_seqlens[s];
      if (l < 0) return -1;
      if (l > maxlen) maxlen = l;
    }
    if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T) return -1;
  }
  for (int64_t r = 0; r < ntok; r++) {
    int64_t x = tokens ? tokens[r] : r;
    if (x < 0 || x >= B * T) return -1;
  }
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#endif

#pragma omp parallel
  {
    const int64_t nb_max = (maxlen + block_size - 1) / block_size;
    unsigned char* sel = (unsigned char*)malloc((size_t)nb_max + 1);
    unsigned char* mask = (unsigned char*)malloc((size_t)maxlen + 1);
    double* z = (double*)malloc(sizeof(double) * ((size_t)maxlen + 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t work = 0; work < ntok * Hkv; work++) {
      const int64_t r = work / Hkv, h = work % Hkv;
      const int64_t x = tokens ? tokens[r] : r;
      int64_t bos, L;
      seq_bounds(x, T, cu_seqlens, num_seqs, &bos, &L);
      const int64_t t = x - bos;                 /* position inside its sequence */
      const int64_t nb = (L + block_size - 1) / block_size;

      /* 1. which blocks the row lists (first n entries, negatives and
       *    blocks outside the sequence contribute nothing) */
      memset(sel, 0, (size_t)nb + 1);
      int64_t n = block_counts[x * Hkv + h];
      if (n < 0) n = 0;
      if (n > S) n = S;
      for (int64_t i = 0; i < n; i++) {
        int64_t idx = block_indices[(x * Hkv + h) * S + i];
        if (idx >= 0 && idx < nb) sel[idx] = 1;
      }
      /* 2. the token mask: key s visible iff its block is listed and s <= t */
      for (int64_t s = 0; s < L; s++) mask[s] = (s <= t) && sel[s / block_size];

      /* 3. dense masked softmax for each query head of the group */
      for (int64_t g = 0; g < G; g++) {
        const int64_t hq = h * G + g;
        const float* qrow = q + (x * Hq + hq) * D;
        double* orow = out + (r * Hq + hq) * D;
        double m = -INFINITY;
        int64_t nvis = 0;
        for (int64_t s = 0; s < L; s++) {
          if (!mask[s]) continue;
          const float* krow = k + ((bos + s) * Hkv + h) * D;
          double acc = 0.0;
          for (int64_t d = 0; d < D; d++) acc += (double)qrow[d] * (double)krow[d];
          z[s] = scale * acc;
          if (z[s] > m) m = z[s];
          nvis++;
        }
        if (nvis == 0) {
          for (int64_t d = 0; d < D; d++) orow[d] = 0.0;
          lse[r * Hq + hq] = -INFINITY;
          continue;
        }
        double denom = 0.0;
        for (int64_t s = 0; s < L; s++)
          if (mask[s]) denom += exp(z[s] - m);
        const double lse_v = m + log(denom);
        lse[r * Hq + hq] = lse_v;
        for (int64_t d = 0; d < D; d++) orow[d] = 0.0;
        for (int64_t s = 0; s < L; s++) {
          if (!mask[s]) continue;
          const double p = exp(z[s] - lse_v);
          const float* vrow = v + ((bos + s) * Hkv + h) * D;
          for (int64_t d = 0; d < D; d++) orow[d] += p * (double)vrow[d];
        }
      }
    }
    free(sel);
    free(mask);
    free(z);
  }
  return 0;
}

/* Number of threads OpenMP would use (for reporting the CPU baseline). */
int nsa_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
