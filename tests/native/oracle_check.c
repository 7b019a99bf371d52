/*
 * Sanitizer driver for the CPU oracle (test infrastructure).  Built with
 * -fsanitize=address,undefined and run by tests/test_sanitizers.py: it feeds
 * the oracle hostile index rows (negative entries, blocks past the token's
 * own block and past the sequence, repeats, counts outside [0, S]), packed
 * sequences with empty and one-token members and token subsets, so that any
 * out-of-bounds access or undefined arithmetic on those paths aborts.
 *
 * It also checks, independently of the oracle's mask code, that with q = 0
 * every row's exp(lse) is the number of visible keys counted key by key
 * (a key s <= t is visible iff one of the first clamp(n, 0, S) entries
 * equals s / block_size), and that empty rows give out = 0, lse = -inf.
 * Exit status 0 = all checks passed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/nsa_oracle.c"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static int64_t uniform_int(int64_t lo, int64_t hi) { /* inclusive */
  return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1));
}

static int run_case(int64_t B, const int32_t* lens, int64_t nseq, int64_t Hq, int64_t Hkv, int64_t D,
                    int64_t S, int64_t bs, int zero_q, int use_tokens) {
  int64_t T = 0;
  int32_t* cu = NULL;
  if (lens) {
    cu = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nseq + 1));
    cu[0] = 0;
    for (int64_t i = 0; i < nseq; i++) cu[i + 1] = cu[i] + lens[i];
    T = cu[nseq];
    B = 1;
  } else {
    T = 97;
  }
  const int64_t rows = B * T;
  float* q = (float*)malloc(sizeof(float) * (size_t)(rows * Hq * D));
  float* k = (float*)malloc(sizeof(float) * (size_t)(rows * Hkv * D));
  float* v = (float*)malloc(sizeof(float) * (size_t)(rows * Hkv * D));
  int32_t* bi = (int32_t*)malloc(sizeof(int32_t) * (size_t)(rows * Hkv * S));
  int32_t* bc = (int32_t*)malloc(sizeof(int32_t) * (size_t)(rows * Hkv));
  for (int64_t i = 0; i < rows * Hq * D; i++) q[i] = zero_q ? 0.f : (float)uniform_int(-8, 8) / 8.f;
  for (int64_t i = 0; i < rows * Hkv * D; i++) {
    k[i] = (float)uniform_int(-8, 8) / 8.f;
    v[i] = (float)uniform_int(-8, 8) / 8.f;
  }
  const int64_t nb_hi = (T + bs - 1) / bs + 2;
  for (int64_t i = 0; i < rows * Hkv * S; i++) bi[i] = (int32_t)uniform_int(-3, nb_hi);
  for (int64_t i = 0; i < rows * Hkv; i++) bc[i] = (int32_t)uniform_int(-2, S + 3);
  int64_t ntok = rows;
  int64_t* tokens = NULL;
  if (use_tokens) {
    ntok = rows / 3 + 1;
    tokens = (int64_t*)malloc(sizeof(int64_t) * (size_t)ntok);
    for (int64_t i = 0; i < ntok; i++) tokens[i] = uniform_int(0, rows - 1);
  }
  double* out = (double*)malloc(sizeof(double) * (size_t)(ntok * Hq * D));
  double* lse = (double*)malloc(sizeof(double) * (size_t)(ntok * Hq));
  int rc = nsa_oracle_fwd(B, T, Hq, Hkv, D, S, bs, q, k, v, bi, bc, cu, lens ? nseq : 0, 0.125, tokens, ntok,
                          out, lse, 1);
  int bad = rc != 0;
  const int64_t G = Hq / Hkv;
  for (int64_t r = 0; r < ntok && !bad; r++) {
    const int64_t x = tokens ? tokens[r] : r;
    int64_t bos = (x / T) * T, len = T;
    if (cu) {
      int64_t s = 0;
      while (!(cu[s] <= x && x < cu[s + 1])) s++;
      bos = cu[s];
      len = cu[s + 1] - cu[s];
    }
    (void)len;
    const int64_t t = x - bos;
    for (int64_t h = 0; h < Hkv; h++) {
      int64_t n = bc[x * Hkv + h];
      n = n < 0 ? 0 : (n > S ? S : n);
      int64_t visible = 0;
      for (int64_t s = 0; s <= t; s++) {
        int hit = 0;
        for (int64_t i = 0; i < n; i++) hit |= bi[(x * Hkv + h) * S + i] == s / bs;
        visible += hit;
      }
      for (int64_t g = 0; g < G; g++) {
        const int64_t hq = h * G + g;
        const double l = lse[r * Hq + hq];
        if (visible == 0) {
          bad |= !(isinf(l) && l < 0);
          for (int64_t d = 0; d < D; d++) bad |= out[(r * Hq + hq) * D + d] != 0.0;
        } else {
          bad |= !isfinite(l);
          if (zero_q) bad |= fabs(exp(l) - (double)visible) > 1e-9 * (double)visible;
          for (int64_t d = 0; d < D; d++) bad |= !(fabs(out[(r * Hq + hq) * D + d]) <= 1.0 + 1e-12);
        }
      }
    }
  }
  free(q); free(k); free(v); free(bi); free(bc); free(out); free(lse); free(cu); free(tokens);
  return bad;
}

int main(void) {
  int fails = 0;
  const int32_t lens_a[] = {0, 1, 65, 0, 130, 7};
  const int32_t lens_b[] = {1};
  const int32_t lens_c[] = {33, 0, 0, 64};
  for (int zq = 0; zq < 2; zq++) {
    fails += run_case(2, NULL, 0, 4, 2, 8, 5, 16, zq, 0);
    fails += run_case(1, NULL, 0, 6, 3, 4, 9, 32, zq, 1);
    fails += run_case(1, lens_a, 6, 4, 1, 8, 6, 16, zq, 0);
    fails += run_case(1, lens_b, 1, 2, 2, 4, 3, 64, zq, 0);
    fails += run_case(1, lens_c, 4, 8, 2, 8, 4, 32, zq, 1);
  }
  /* arguments the oracle must refuse without touching memory */
  float f = 0.f;
  int32_t i32 = 0;
  double d = 0.0;
  int32_t bad_cu[] = {0, 5, 3};   /* decreasing */
  fails += nsa_oracle_fwd(1, 3, 2, 2, 1, 1, 16, &f, &f, &f, &i32, &i32, bad_cu, 2, 1.0, NULL, 3, &d, &d, 1) != -1;
  fails += nsa_oracle_fwd(1, 3, 3, 2, 1, 1, 16, &f, &f, &f, &i32, &i32, NULL, 0, 1.0, NULL, 3, &d, &d, 1) != -1;
  int64_t tok = 7;
  fails += nsa_oracle_fwd(1, 3, 2, 2, 1, 1, 16, &f, &f, &f, &i32, &i32, NULL, 0, 1.0, &tok, 1, &d, &d, 1) != -1;
  printf("oracle sanitizer check: %s\n", fails ? "FAILED" : "ok");
  return fails ? 1 : 0;
}
