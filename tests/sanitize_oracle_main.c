/* Host sanitizer driver for the fp64 oracle (tests/test_sanitizers_cpu.py
 * builds it with -fsanitize=address,undefined and runs it; any report aborts
 * with a non-zero status). It calls every oracle function on small seeded
 * inputs, in both storage types, including the edge cases the definitions
 * name: empty and repeated selections, negative, future and out-of-range
 * indices, -inf score tails, windows wider than the context, buffer offsets,
 * sinks, grouped KV heads, all-zero FP8 rows and every ReLU mode. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_index_scores(const void *, const void *, const void *, int, int, int, int, int, int,
                         int, double, int, double *);
void oracle_e4m3_codes(const float *, int64_t, uint8_t *);
void oracle_index_quant_fp8(const uint16_t *, int64_t, int, uint8_t *, float *);
void oracle_index_scores_fp8(const uint8_t *, const float *, const uint8_t *, const float *,
                             const void *, int, int, int, int, int, int, int, double, int,
                             double *);
void oracle_indexer_prologue(const void *, const void *, const void *, const void *, const void *,
                             const void *, const void *, const float *, const float *, int, int,
                             int, int, int, int, int, int, int, double, double *, double *,
                             double *);
void oracle_topk(const float *, int64_t, int64_t, int, int32_t *);
void oracle_sparse_attn_pas(const void *, const void *, const void *, const void *, const void *,
                            int, const int32_t *, const void *, int, int, int, int, int, int, int,
                            int, int, double, int, double *);
void oracle_swa_attn_pas(const void *, const void *, const void *, const void *, const void *, int,
                         const void *, int, int, int, int, int, int, int, int, int, int, double,
                         int, double *);
void oracle_swa_attn_gqa(const void *, const void *, const void *, const void *, int, int, int,
                         int, int, int, int, int, int, int, int, double, int, double *);

static uint64_t st = 88172645463325252ull;
static uint64_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
static float unif(void) { return (float)((rnd() >> 11) * (1.0 / 9007199254740992.0)) * 2.f - 1.f; }

/* n values of storage type dt (0 fp32, 1 bf16 bits), uniform in (-a, a) */
static void *fill(int dt, size_t n, float a) {
  void *p = malloc((n ? n : 1) * (dt ? 2 : 4));
  for (size_t i = 0; i < n; ++i) {
    float f = unif() * a;
    if (dt) {
      uint32_t b;
      memcpy(&b, &f, 4);
      ((uint16_t *)p)[i] = (uint16_t)(b >> 16);
    } else {
      ((float *)p)[i] = f;
    }
  }
  return p;
}

static int check_finite(const double *x, size_t n, const char *what) {
  for (size_t i = 0; i < n; ++i)
    if (isnan(x[i])) {
      fprintf(stderr, "%s: NaN at %zu\n", what, i);
      return 1;
    }
  return 0;
}

int main(void) {
  int bad = 0;
  for (int dt = 0; dt < 2; ++dt) {
    /* indexer, every mode, with and without a past */
    int B = 2, S = 5, T = 13, HI = 3, DI = 16;
    for (int P = 0; P <= T - S; P += T - S) {
      void *q = fill(dt, (size_t)B * S * HI * DI, 1), *k = fill(dt, (size_t)B * T * DI, 1),
           *w = fill(dt, (size_t)B * S * HI, 1);
      double *o = malloc(sizeof(double) * B * S * T);
      for (int mode = 0; mode < 3; ++mode) {
        oracle_index_scores(q, k, w, dt, B, S, T, P, HI, DI, 0.25, mode, o);
        for (int i = 0; i < B * S * T; ++i)
          if (isnan(o[i])) bad |= 1;
      }
      /* top-k of those rows (with -inf tails), k below and above the row length */
      float *sc = malloc(sizeof(float) * B * S * T);
      for (int i = 0; i < B * S * T; ++i) sc[i] = (float)o[i];
      int32_t *ix = malloc(sizeof(int32_t) * B * S * (T + 4));
      oracle_topk(sc, B * S, T, 4, ix);
      oracle_topk(sc, B * S, T, T + 4, ix);
      free(sc);
      free(ix);
      free(q), free(k), free(w), free(o);
    }
    /* sparse attention with sinks and junk / repeated / empty selections */
    {
      int B = 2, S = 4, T = 11, P = 7, H = 3, Dqk = 24, Dv = 8, K = 6;
      void *q = fill(dt, (size_t)B * S * H * Dqk, 1), *kc = fill(dt, (size_t)B * T * H * Dqk, 1),
           *vc = fill(dt, (size_t)B * T * H * Dv, 1), *g = fill(dt, (size_t)B * S * H * Dv, 4);
      void *sk = fill(dt, (size_t)2 * H * Dqk, 1), *sv = fill(dt, (size_t)2 * H * Dv, 1);
      int32_t idx[2 * 4 * 6];
      for (int i = 0; i < B * S * K; ++i) idx[i] = (int32_t)(rnd() % (T + 6)) - 3;
      for (int j = 0; j < K; ++j) idx[j] = -1;     /* an empty selection */
      idx[K] = idx[K + 1] = 2;                     /* a repeated entry */
      double *o = malloc(sizeof(double) * B * S * H * Dv);
      for (int ns = 0; ns <= 2; ns += 2)
        for (int gd = 0; gd <= 1; ++gd) {
          oracle_sparse_attn_pas(q, kc, vc, ns ? sk : NULL, ns ? sv : NULL, ns, idx,
                                 gd ? g : NULL, dt, B, S, T, P, H, Dqk, Dv, K, 0.2, gd, o);
          bad |= check_finite(o, (size_t)B * S * H * Dv, "sparse_attn");
        }
      oracle_sparse_attn_pas(q, kc, vc, NULL, NULL, 0, idx, g, dt, B, S, T, P, H, Dqk, Dv, K, 0.2,
                             Dv, o); /* elementwise gate */
      bad |= check_finite(o, (size_t)B * S * H * Dv, "sparse_attn elementwise");
      /* windows: narrower than, equal to and wider than the context, with an offset */
      int windows[3] = {1, 3, 50};
      for (int wi = 0; wi < 3; ++wi)
        for (int off = 0; off <= 2; off += 2) {
          int W = windows[wi];
          if (off > (P - W + 1 > 0 ? P - W + 1 : 0)) continue;
          int Tb = P + S - off;
          oracle_swa_attn_pas(q, kc, vc, sk, sv, 1, g, dt, 1, S, Tb, P, off, H, Dqk, Dv, W, 0.2,
                              1, o);
          bad |= check_finite(o, (size_t)S * H * Dv, "swa");
        }
      /* grouped KV heads: 6 query heads over the caches' 3 */
      void *q6 = fill(dt, (size_t)S * 6 * Dqk, 1), *g6 = fill(dt, (size_t)S * 6, 2);
      double *o6 = malloc(sizeof(double) * S * 6 * Dv);
      oracle_swa_attn_gqa(q6, kc, vc, g6, dt, 1, S, P + S, P, 0, 6, 3, Dqk, Dv, 4, 0.2, 1, o6);
      bad |= check_finite(o6, (size_t)S * 6 * Dv, "swa_gqa");
      free(q6), free(g6), free(o6);
      free(q), free(kc), free(vc), free(g), free(sk), free(sv), free(o);
    }
    /* indexer prologue with and without RoPE */
    {
      int B = 2, S = 3, P = 2, Q = 32, Hd = 40, HI = 2, D = 16;
      void *ql = fill(dt, (size_t)B * S * Q, 1), *hd = fill(dt, (size_t)B * S * Hd, 1);
      void *wq = fill(dt, (size_t)HI * D * Q, 0.2f), *wk = fill(dt, (size_t)D * Hd, 0.2f);
      void *nw = fill(dt, D, 1), *nb = fill(dt, D, 1), *wp = fill(dt, (size_t)HI * Hd, 0.2f);
      float cs[5 * 4], sn[5 * 4];
      for (int i = 0; i < 20; ++i) cs[i] = cosf((float)i), sn[i] = sinf((float)i);
      double *oq = malloc(sizeof(double) * B * S * HI * D), *ok = malloc(sizeof(double) * B * S * D),
             *ow = malloc(sizeof(double) * B * S * HI);
      for (int R = 0; R <= 8; R += 8)
        oracle_indexer_prologue(ql, hd, wq, wk, nw, nb, wp, R ? cs : NULL, R ? sn : NULL, dt, B, S,
                                P, Q, Hd, HI, D, R, 1e-5, oq, ok, ow);
      bad |= check_finite(oq, (size_t)B * S * HI * D, "prologue q");
      bad |= check_finite(ok, (size_t)B * S * D, "prologue k");
      free(ql), free(hd), free(wq), free(wk), free(nw), free(nb), free(wp), free(oq), free(ok),
          free(ow);
    }
  }
  /* FP8: codes of every representable magnitude, quantisation with an all-zero
   * row, and scores from the codes in every mode */
  {
    float v[1000];
    uint8_t c[1000];
    for (int i = 0; i < 1000; ++i) v[i] = unif() * 448.f * (float)ldexp(1.0, -(int)(rnd() % 16));
    v[0] = 0.f, v[1] = -0.f, v[2] = 448.f, v[3] = -448.f;
    oracle_e4m3_codes(v, 1000, c);
    int B = 1, S = 3, T = 7, HI = 2, DI = 32, P = 4;
    uint16_t *q = fill(1, (size_t)S * HI * DI, 3), *k = fill(1, (size_t)T * DI, 3);
    memset(k, 0, sizeof(uint16_t) * DI); /* an all-zero row */
    void *w = fill(1, (size_t)S * HI, 1);
    uint8_t *qc = malloc((size_t)S * HI * DI), *kc = malloc((size_t)T * DI);
    float *qs = malloc(sizeof(float) * S * HI), *ks = malloc(sizeof(float) * T);
    oracle_index_quant_fp8(q, S * HI, DI, qc, qs);
    oracle_index_quant_fp8(k, T, DI, kc, ks);
    double *o = malloc(sizeof(double) * S * T);
    for (int mode = 0; mode < 3; ++mode)
      oracle_index_scores_fp8(qc, qs, kc, ks, w, 1, B, S, T, P, HI, DI, 0.1, mode, o);
    free(q), free(k), free(w), free(qc), free(kc), free(qs), free(ks), free(o);
  }
  if (bad) {
    fprintf(stderr, "unexpected NaN in an oracle output\n");
    return 3;
  }
  printf("oracle sanitizer driver: ok\n");
  return 0;
}
