/*
 * dsa_oracle.c -- plain, slow, fp64 CPU reference for one DeepSeek-Sparse-
 * Attention (DSA) layer and its sliding-window (SWA) sibling.
 *
 * THIS IS TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it. The product path (the HIP library)
 * never calls it, and the two share no source, header, table or helper.
 *
 * Every function is the plain definition of its result, written out in the
 * order the pages give it:
 *   oracle_index_scores  -- lightning-indexer score with causal mask
 *                           [A.X-K2 page, "Sparse Gated Attention (SGA)"]
 *   oracle_topk          -- per-query top-k of a score row
 *                           [A.X-K2 page, SGA bullets and "index_topk"]
 *   oracle_sparse_attn   -- attention under the additive sparse mask AND the
 *                           causal mask, then the sigmoid output gate
 *                           [A.X-K2 page, "MLA + explicit sparse mask" steps
 *                           4-5 and "Attention output gate"; Spark-X2.5 page,
 *                           "forward pass" steps 1-3]
 *   oracle_swa_attn      -- sliding-window attention, window W keys
 *                           [Spark-X2.5 page, "why the gate" (sliding_window
 *                           512); openPangu-2.0 page §3.2]
 *   *_pas variants       -- the same two with parametric attention sinks:
 *                           n_sink learned K/V rows every query attends to
 *                           besides its selected or windowed keys
 *                           [openPangu-2.0 page §3.4 (PAS)]
 *   oracle_index_quant_fp8, oracle_index_scores_fp8
 *                        -- the indexer on FP8 operands: each q and k row is
 *                           rotated by a Hadamard matrix and stored as FP8
 *                           codes with one scale per row; scores are formed
 *                           from those codes [A.X-K2 page, implementation
 *                           notes: the reference indexer rotates with a
 *                           Hadamard transform and scores in FP8; the
 *                           rotation cancels since H q . H k = D q . k]
 *   oracle_indexer_prologue
 *                        -- the indexer's projections: q_idx from the query
 *                           LoRA bottleneck (wq_b), the key from the hidden
 *                           state (wk) through a LayerNorm, per-head weights
 *                           (weights_proj), half-split RoPE on q and k
 *                           [A.X-K2 page, SGA bullets and "two RoPE layouts"]
 *   oracle_mla_prologue  -- the main attention's projections: q_gate_proj on
 *                           [q_resid, q_compressed] split per head into the
 *                           query and the output gate, kv_a_proj_with_mqa to
 *                           the latent and the shared rope key, expand_kv
 *                           (kv_b_proj) of the latent into per-head k_nope and
 *                           v, interleaved RoPE on the rope slices
 *                           [A.X-K2 page, "MLA + explicit sparse mask" steps
 *                           1-3, "Attention output gate", "two RoPE layouts"]
 *   oracle_swa_attn_gqa  -- sliding-window attention whose K/V buffers hold
 *                           fewer heads than q (grouped KV heads)
 *                           [Spark-X2.5 page, "why the gate": 8 query heads,
 *                           2 KV heads, head_dim 256]
 * Decode is the same functions with S = 1 and past_len = T - 1.
 *
 * Arithmetic is IEEE double throughout; inputs are read in their storage type
 * (fp32, or bf16 bit patterns) and widened exactly. No blocking, fusion or
 * reordering beyond what the definitions state. Loops over independent
 * outputs are split across OpenMP threads; each output is computed by one
 * thread in a fixed order, so results do not depend on the thread count.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - ReLU placement in the indexer: per head, before the weighted sum
 *    (relu_mode 0). Mode 1 applies none (the formula as printed), mode 2
 *    applies it after the weighted sum.
 *  - Query s of a call sits at absolute position p = past_len + s and sees
 *    keys t <= p, itself included.
 *  - Top-k: order by (score descending, t ascending); -0.0 equals +0.0; slots
 *    whose score is -inf, or beyond the row, are emitted as -1.
 *  - Attention index lists are sets: negative entries, entries > p and
 *    entries >= T are ignored; a repeated entry selects its key once.
 *  - SWA window: the W keys p-W+1 .. p.
 *  - Gate: sigmoid(x) = 1 / (1 + exp(-x)), one scalar per (token, head)
 *    (gate_dim 1) or one per output element (gate_dim = v_dim).
 *  - Sinks (PAS): given per head as expanded K/V rows sink_k [n_sink,H,Dqk],
 *    sink_v [n_sink,H,Dv], shared by the whole batch; they carry no position,
 *    so no causal mask applies to them; the softmax runs over the sinks and
 *    the selected (or windowed) keys together.
 *  - Grouped KV heads: query head h reads KV head h / (H / H_kv), i.e.
 *    consecutive query heads share a KV head.
 *  - Indexer prologue: weights in the nn.Linear layout [out, in]; LayerNorm
 *    with the mean and the biased variance over idx_dim plus eps, then the
 *    affine weight and bias; RoPE on the last rope_dim dims of each index head
 *    and of the key: pair (j, j + rope_dim/2) of that slice rotates by the
 *    caller's (cos, sin) of position p and frequency j. The pages' bf16
 *    modules round each projection to bf16; the oracle keeps fp64 throughout.
 *  - MLA prologue: q_gate_proj reads the concatenation [q_resid, q_compressed]
 *    and its output for head h is the query (Dqk values, nope slice then rope
 *    slice) followed by the gate (Dv values); kv_a_proj_with_mqa's output is
 *    the latent (kv_lora_rank values) followed by the rope key (qk_rope
 *    values, one for all heads); expand_kv is kv_b_proj applied to the latent
 *    (no normalisation between: the page names none), whose output for head
 *    h is k_nope (qk_nope values) followed by v (Dv values). The interleaved
 *    RoPE rotates the pair (x_2j, x_2j+1) of a rope slice in place by the
 *    caller's (cos, sin) of position p and frequency j. The expanded key of
 *    head h is [k_nope_h | rotated rope key].
 *  - FP8 indexer (the page names the steps, not their details): the rotation
 *    is the Sylvester-ordered Walsh-Hadamard matrix with entries +-1 (no
 *    normalisation; scores divide by D instead), computed by the fast
 *    transform in fp32, stride 1 first. A row's scale is the power of two
 *    2^e with the smallest e such that max|y| * 2^-e <= 448, and each code is
 *    the OCP FP8 E4M3 value of y * 2^-e rounded to nearest, ties to even
 *    (largest finite 448, subnormal step 2^-9). An all-zero row has scale 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Storage types of the inputs. */
#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Indexer ReLU placement. */
#define ORACLE_RELU_PER_HEAD 0
#define ORACLE_RELU_NONE 1
#define ORACLE_RELU_POST_SUM 2

/* Read element i of an fp32 or bf16 array as an exact double. A bf16 value is
 * the upper 16 bits of the fp32 with the same value. */
static double rd(const void *base, int dtype, int64_t i) {
  if (dtype == ORACLE_F32) return (double)((const float *)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads of the parallel loops that follow (the CPU-baseline timing's
 * one-thread figure); results do not depend on it. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/*
 * Lightning-indexer scores [A.X-K2 page, SGA: the score formula and the
 * causal mask]:
 *   score[b,s,t] = sum_h w[b,s,h] * relu(scale * q[b,s,h,:] . k[b,t,:])
 * for t <= p = past_len + s, and -inf for t > p.
 *   q_idx [B,S,HI,DI], k_idx [B,T,DI], w [B,S,HI]  (dtype)
 *   out   [B,S,T] double
 */
void oracle_index_scores(const void *q_idx, const void *k_idx, const void *w,
                         int dtype, int B, int S, int T, int past_len, int HI,
                         int DI, double scale, int relu_mode, double *out) {
  int64_t n = (int64_t)B * S * T;
#pragma omp parallel for schedule(dynamic, 256)
  for (int64_t e = 0; e < n; ++e) {
    int64_t t = e % T;
    int64_t bs = e / T; /* b*S + s */
    int64_t s = bs % S;
    int64_t b = bs / S;
    int64_t p = (int64_t)past_len + s;
    if (t > p) {
      out[e] = -INFINITY;
      continue;
    }
    double total = 0.0;
    for (int h = 0; h < HI; ++h) {
      double dot = 0.0;
      for (int d = 0; d < DI; ++d)
        dot += rd(q_idx, dtype, (bs * HI + h) * DI + d) *
               rd(k_idx, dtype, (b * T + t) * DI + d);
      double u = scale * dot;
      double wh = rd(w, dtype, bs * HI + h);
      if (relu_mode == ORACLE_RELU_PER_HEAD)
        total += wh * (u > 0.0 ? u : 0.0);
      else
        total += wh * u;
    }
    if (relu_mode == ORACLE_RELU_POST_SUM && !(total > 0.0)) total = 0.0;
    out[e] = total;
  }
}

/*
 * FP8 E4M3 (OCP "e4m3fn": bias 7, 3 mantissa bits, no infinities, largest
 * finite 448) of a float with |v| <= 448, rounded to nearest, ties to even.
 * Written from the format's definition: subnormals are multiples of 2^-9
 * below 2^-6; a normal value 2^E (1 + m/8) has code (E + 7) << 3 | m.
 */
static uint8_t e4m3_rne(float v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs((double)v);
  if (a < 0x1p-6) { /* subnormal range (a result of 8 is the smallest normal) */
    double q = rint(a * 512.0);
    return (uint8_t)(sign | (uint8_t)q);
  }
  int E = ilogb(a);
  double m = rint((ldexp(a, -E) - 1.0) * 8.0);
  if (m >= 8.0) {
    m = 0.0;
    E += 1;
  }
  return (uint8_t)(sign | (uint8_t)(((E + 7) << 3) | (int)m));
}

/* FP8 E4M3 codes of n floats with |v| <= 448 (exposes e4m3_rne to the pins). */
void oracle_e4m3_codes(const float *v, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_rne(v[i]);
}

/* The value of an FP8 E4M3 code. */
static double e4m3_value(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return (c & 0x80) ? -v : v;
}

/*
 * Rotate and quantise rows of bf16 values to FP8 [A.X-K2 page, implementation
 * notes: Hadamard rotation, then FP8 quantisation, of the indexer's q and k].
 *   x [rows, dim] bf16 bits (dim a power of two, <= 4096)
 *   codes [rows, dim] FP8 E4M3, scales [rows]: row value = code * scale.
 */
void oracle_index_quant_fp8(const uint16_t *x, int64_t rows, int dim,
                            uint8_t *codes, float *scales) {
#pragma omp parallel
  {
    float *y = (float *)malloc(sizeof(float) * (size_t)dim);
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      for (int i = 0; i < dim; ++i) {
        uint32_t bits = (uint32_t)x[r * dim + i] << 16;
        memcpy(&y[i], &bits, sizeof(float));
      }
      /* fast Walsh-Hadamard transform in fp32: butterflies (a, b) ->
       * (a + b, a - b) on pairs (i, i + h), h = 1, 2, 4, ... */
      for (int h = 1; h < dim; h <<= 1)
        for (int i = 0; i < dim; i += 2 * h)
          for (int j = i; j < i + h; ++j) {
            float a = y[j], b = y[j + h];
            y[j] = a + b;
            y[j + h] = a - b;
          }
      float amax = 0.0f;
      for (int i = 0; i < dim; ++i)
        if (fabsf(y[i]) > amax) amax = fabsf(y[i]);
      if (amax == 0.0f) {
        scales[r] = 1.0f;
        for (int i = 0; i < dim; ++i) codes[r * dim + i] = 0;
        continue;
      }
      /* smallest e with amax * 2^-e <= 448 */
      int E = ilogbf(amax);
      int e = (ldexpf(amax, -(E - 8)) <= 448.0f) ? E - 8 : E - 7;
      scales[r] = ldexpf(1.0f, e);
      for (int i = 0; i < dim; ++i)
        codes[r * dim + i] = e4m3_rne(ldexpf(y[i], -e));
    }
    free(y);
  }
}

/*
 * Indexer scores from FP8 operands: the formula of oracle_index_scores on the
 * dequantised rotated rows, divided by dim (the rotation scales every dot
 * product by dim):
 *   score[b,s,t] = sum_h w[b,s,h] * relu(scale / DI * (qh . kt))
 *   qh = q_codes[b,s,h,:] * q_scales[b,s,h], kt = k_codes[b,t,:] * k_scales[b,t]
 * with the causal mask and relu_mode of oracle_index_scores.
 */
void oracle_index_scores_fp8(const uint8_t *q_codes, const float *q_scales,
                             const uint8_t *k_codes, const float *k_scales,
                             const void *w, int w_dtype, int B, int S, int T,
                             int past_len, int HI, int DI, double scale,
                             int relu_mode, double *out) {
  int64_t n = (int64_t)B * S * T;
#pragma omp parallel for schedule(dynamic, 256)
  for (int64_t e = 0; e < n; ++e) {
    int64_t t = e % T;
    int64_t bs = e / T;
    int64_t s = bs % S;
    int64_t b = bs / S;
    int64_t p = (int64_t)past_len + s;
    if (t > p) {
      out[e] = -INFINITY;
      continue;
    }
    double total = 0.0;
    for (int h = 0; h < HI; ++h) {
      const uint8_t *qc = q_codes + (bs * HI + h) * DI;
      const uint8_t *kc = k_codes + (b * T + t) * DI;
      double dot = 0.0;
      for (int d = 0; d < DI; ++d) dot += e4m3_value(qc[d]) * e4m3_value(kc[d]);
      double u = scale / DI * dot * (double)q_scales[bs * HI + h] *
                 (double)k_scales[b * T + t];
      double wh = rd(w, w_dtype, bs * HI + h);
      if (relu_mode == ORACLE_RELU_PER_HEAD)
        total += wh * (u > 0.0 ? u : 0.0);
      else
        total += wh * u;
    }
    if (relu_mode == ORACLE_RELU_POST_SUM && !(total > 0.0)) total = 0.0;
    out[e] = total;
  }
}

/*
 * The indexer's projections for S tokens at positions past_len + s [A.X-K2
 * page, SGA bullets: wq_b on the query LoRA bottleneck, wk + k_norm
 * (LayerNorm) on the key, weights_proj for the head weights; "two RoPE
 * layouts": the indexer's RoPE is half-split].
 *   q_lora [B,S,Q], hidden [B,S,Hd]; wq_b [HI*D, Q], wk [D, Hd],
 *   weights_proj [HI, Hd], k_norm_w / k_norm_b [D]   (dtype)
 *   rope_cos / rope_sin [T, R/2] fp32 (unused when R = 0)
 *   out_q [B,S,HI,D], out_k [B,S,D], out_w [B,S,HI]   double
 */
static void rope_half_split(double *x, int R, const float *cs, const float *sn) {
  int half = R / 2;
  for (int j = 0; j < half; ++j) {
    double a = x[j], b = x[j + half], c = cs[j], s = sn[j];
    x[j] = a * c - b * s;
    x[j + half] = b * c + a * s;
  }
}

void oracle_indexer_prologue(const void *q_lora, const void *hidden,
                             const void *wq_b, const void *wk,
                             const void *k_norm_w, const void *k_norm_b,
                             const void *weights_proj, const float *rope_cos,
                             const float *rope_sin, int dtype, int B, int S,
                             int past_len, int Q, int Hd, int HI, int D, int R,
                             double eps, double *out_q, double *out_k,
                             double *out_w) {
  int64_t n = (int64_t)B * S;
  int half = R / 2;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bs = 0; bs < n; ++bs) {
    int64_t p = past_len + bs % S;
    const float *cs = R > 0 ? rope_cos + p * half : NULL;
    const float *sn = R > 0 ? rope_sin + p * half : NULL;
    /* q_idx: wq_b applied to the query bottleneck, then RoPE per head */
    for (int o = 0; o < HI * D; ++o) {
      double acc = 0.0;
      for (int i = 0; i < Q; ++i)
        acc += rd(q_lora, dtype, bs * Q + i) * rd(wq_b, dtype, (int64_t)o * Q + i);
      out_q[bs * HI * D + o] = acc;
    }
    if (R > 0)
      for (int h = 0; h < HI; ++h)
        rope_half_split(out_q + (bs * HI + h) * D + (D - R), R, cs, sn);
    /* key: wk, LayerNorm, RoPE */
    double *k = out_k + bs * D;
    for (int o = 0; o < D; ++o) {
      double acc = 0.0;
      for (int i = 0; i < Hd; ++i)
        acc += rd(hidden, dtype, bs * Hd + i) * rd(wk, dtype, (int64_t)o * Hd + i);
      k[o] = acc;
    }
    double mean = 0.0, var = 0.0;
    for (int o = 0; o < D; ++o) mean += k[o];
    mean /= D;
    for (int o = 0; o < D; ++o) var += (k[o] - mean) * (k[o] - mean);
    var /= D;
    for (int o = 0; o < D; ++o)
      k[o] = (k[o] - mean) / sqrt(var + eps) * rd(k_norm_w, dtype, o) +
             rd(k_norm_b, dtype, o);
    if (R > 0) rope_half_split(k + (D - R), R, cs, sn);
    /* head weights */
    for (int o = 0; o < HI; ++o) {
      double acc = 0.0;
      for (int i = 0; i < Hd; ++i)
        acc += rd(hidden, dtype, bs * Hd + i) *
               rd(weights_proj, dtype, (int64_t)o * Hd + i);
      out_w[bs * HI + o] = acc;
    }
  }
}

/*
 * The main attention's projections for S tokens at positions past_len + s
 * [A.X-K2 page, "MLA + explicit sparse mask" steps 1-3: q_gate_proj produces
 * the query and the attention output gate together, kv_a_proj_with_mqa
 * compresses K/V to the kv_lora_rank latent plus the shared RoPE key, and
 * expand_kv expands the latent into full per-head keys and values (the cache
 * holds these expanded rows); "Attention output gate": the fused projection
 * reads [q_resid, q_compressed] and its output splits into a qk_head_dim
 * query and a v_head_dim gate; "two RoPE layouts": the main attention uses
 * the interleaved layout].
 *   q_resid [B,S,Qr], q_comp [B,S,Qc], hidden [B,S,Hd]        (dtype)
 *   wq_gate [H*(N+R+Dv), Qr+Qc], wkv_a [L+R, Hd], wkv_b [H*(N+Dv), L]
 *   rope_cos / rope_sin [T, R/2] fp32 (unused when R = 0)
 *   out_q [B,S,H,N+R], out_gate [B,S,H,Dv], out_k [B,S,H,N+R], out_v [B,S,H,Dv]
 *   (double; out_k / out_v are the cache rows of the S new tokens)
 */
static void rope_interleaved(double *x, int R, const float *cs, const float *sn) {
  for (int j = 0; j < R / 2; ++j) {
    double a = x[2 * j], b = x[2 * j + 1], c = cs[j], s = sn[j];
    x[2 * j] = a * c - b * s;
    x[2 * j + 1] = b * c + a * s;
  }
}

void oracle_mla_prologue(const void *q_resid, const void *q_comp, const void *hidden,
                         const void *wq_gate, const void *wkv_a, const void *wkv_b,
                         const float *rope_cos, const float *rope_sin, int dtype, int B,
                         int S, int past_len, int Qr, int Qc, int Hd, int L, int H, int N,
                         int R, int Dv, double *out_q, double *out_gate, double *out_k,
                         double *out_v) {
  int64_t n = (int64_t)B * S;
  int Dqk = N + R, Wq = Dqk + Dv, Wkv = N + Dv, Qin = Qr + Qc;
  int half = R / 2;
#pragma omp parallel
  {
    double *lat = (double *)malloc(sizeof(double) * (size_t)(L + R + 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t bs = 0; bs < n; ++bs) {
      int64_t p = past_len + bs % S;
      const float *cs = R > 0 ? rope_cos + p * half : NULL;
      const float *sn = R > 0 ? rope_sin + p * half : NULL;
      /* q_gate_proj on [q_resid, q_compressed]; head h: query then gate */
      for (int h = 0; h < H; ++h) {
        for (int c = 0; c < Wq; ++c) {
          int64_t o = (int64_t)h * Wq + c;
          double acc = 0.0;
          for (int i = 0; i < Qin; ++i) {
            double a = i < Qr ? rd(q_resid, dtype, bs * Qr + i)
                              : rd(q_comp, dtype, bs * Qc + (i - Qr));
            acc += a * rd(wq_gate, dtype, o * Qin + i);
          }
          if (c < Dqk)
            out_q[(bs * H + h) * Dqk + c] = acc;
          else
            out_gate[(bs * H + h) * Dv + (c - Dqk)] = acc;
        }
        if (R > 0) rope_interleaved(out_q + (bs * H + h) * Dqk + N, R, cs, sn);
      }
      /* kv_a_proj_with_mqa: latent, then the shared rope key */
      for (int c = 0; c < L + R; ++c) {
        double acc = 0.0;
        for (int i = 0; i < Hd; ++i)
          acc += rd(hidden, dtype, bs * Hd + i) * rd(wkv_a, dtype, (int64_t)c * Hd + i);
        lat[c] = acc;
      }
      if (R > 0) rope_interleaved(lat + L, R, cs, sn);
      /* expand_kv: kv_b_proj of the latent; head h: k_nope then v */
      for (int h = 0; h < H; ++h) {
        for (int c = 0; c < Wkv; ++c) {
          double acc = 0.0;
          for (int i = 0; i < L; ++i)
            acc += lat[i] * rd(wkv_b, dtype, ((int64_t)h * Wkv + c) * L + i);
          if (c < N)
            out_k[(bs * H + h) * Dqk + c] = acc;
          else
            out_v[(bs * H + h) * Dv + (c - N)] = acc;
        }
        for (int r = 0; r < R; ++r) out_k[(bs * H + h) * Dqk + N + r] = lat[L + r];
      }
    }
    free(lat);
  }
}

/* One candidate of a top-k row. */
typedef struct {
  float score;
  int32_t t;
} cand_t;

/* Order: higher score first, then lower position. -0.0 and +0.0 compare equal
 * under IEEE comparison, so they fall through to the position rule. */
static int cand_cmp(const void *pa, const void *pb) {
  const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  if (a->t < b->t) return -1;
  if (a->t > b->t) return 1;
  return 0;
}

/*
 * Per-row top-k [A.X-K2 page, SGA: keep the top index_topk positions, int32
 * [B,S,topk]]. Rows are fp32 (what the indexer stores); NaN is outside the
 * contract. The whole row is sorted by (score desc, t asc) and the first k
 * entries are emitted: t when its score is above -inf, else -1. Slots past
 * the end of the row are -1 as well.
 *   scores [R,T] float -> out [R,k] int32
 */
void oracle_topk(const float *scores, int64_t R, int64_t T, int k,
                 int32_t *out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < R; ++r) {
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(T > 0 ? T : 1));
    for (int64_t t = 0; t < T; ++t) {
      c[t].score = scores[r * T + t];
      c[t].t = (int32_t)t;
    }
    qsort(c, (size_t)T, sizeof(cand_t), cand_cmp);
    for (int j = 0; j < k; ++j) {
      int32_t v = -1;
      if (j < T && c[j].score > -INFINITY) v = c[j].t;
      out[r * k + j] = v;
    }
    free(c);
  }
}

/* sigmoid(x) = 1 / (1 + e^-x): exactly 0 at -inf, 1 at +inf, 1/2 at 0. */
static double sigm(double x) { return 1.0 / (1.0 + exp(-x)); }

/*
 * Softmax attention of one (b, s, h) query over the keys marked in sel[0..T)
 * and the n_sink sink rows (the gate is applied by the caller). Shared by the
 * DSA and SWA functions below (both are the same masked softmax, they differ
 * only in which keys are marked). The caches hold Hc heads per row and this
 * query reads cache head hc.
 *   qrow [Dqk] at q + qoff; key t row at kc + ((b*T + t)*Hc + hc)*Dqk,
 *   likewise vc with Dv; sink r at sk + (r*Hc + hc)*Dqk and
 *   sv + (r*Hc + hc)*Dv.
 *   logit has room for T + n_sink values. o [Dv] receives the result.
 */
static void masked_softmax_row(const void *q, int64_t qoff, const void *kc,
                               const void *vc, const void *sk, const void *sv,
                               int n_sink, int dtype, int64_t b, int64_t T,
                               int Hc, int hc, int Dqk, int Dv, double sm_scale,
                               const unsigned char *sel, double *logit,
                               double *o) {
  double mx = -INFINITY;
  int64_t nsel = 0;
  double *slog = logit + T; /* sink logits */
  for (int r = 0; r < n_sink; ++r) {
    double dot = 0.0;
    for (int d = 0; d < Dqk; ++d)
      dot += rd(q, dtype, qoff + d) *
             rd(sk, dtype, ((int64_t)r * Hc + hc) * (int64_t)Dqk + d);
    slog[r] = sm_scale * dot;
    if (slog[r] > mx) mx = slog[r];
    ++nsel;
  }
  for (int64_t t = 0; t < T; ++t) {
    if (!sel[t]) continue;
    double dot = 0.0;
    for (int d = 0; d < Dqk; ++d)
      dot += rd(q, dtype, qoff + d) *
             rd(kc, dtype, ((b * T + t) * Hc + hc) * (int64_t)Dqk + d);
    logit[t] = sm_scale * dot;
    if (logit[t] > mx) mx = logit[t];
    ++nsel;
  }
  for (int d = 0; d < Dv; ++d) o[d] = 0.0;
  if (nsel == 0) return; /* no visible selected key and no sink: output 0 */
  double den = 0.0;
  for (int r = 0; r < n_sink; ++r) {
    double e = exp(slog[r] - mx);
    den += e;
    for (int d = 0; d < Dv; ++d)
      o[d] += e * rd(sv, dtype, ((int64_t)r * Hc + hc) * (int64_t)Dv + d);
  }
  for (int64_t t = 0; t < T; ++t) {
    if (!sel[t]) continue;
    double e = exp(logit[t] - mx);
    den += e;
    for (int d = 0; d < Dv; ++d)
      o[d] += e * rd(vc, dtype, ((b * T + t) * Hc + hc) * (int64_t)Dv + d);
  }
  for (int d = 0; d < Dv; ++d) o[d] /= den;
}

/* Multiply the head output by its gate [A.X-K2 page, "Attention output gate";
 * Spark-X2.5 page, forward-pass steps 2-3]. gate_dim 0: no gate; 1: one logit
 * per (token, head), broadcast over v_dim; Dv: one logit per element. */
static void apply_gate(const void *gate, int dtype, int gate_dim, int64_t bs,
                       int H, int h, int Dv, double *o) {
  if (gate_dim == 0 || gate == NULL) return;
  if (gate_dim == 1) {
    double g = sigm(rd(gate, dtype, bs * H + h));
    for (int d = 0; d < Dv; ++d) o[d] *= g;
  } else {
    for (int d = 0; d < Dv; ++d)
      o[d] *= sigm(rd(gate, dtype, (bs * H + h) * (int64_t)Dv + d));
  }
}

/*
 * Sparse MLA attention [A.X-K2 page, "MLA + explicit sparse mask" step 4:
 * positions not chosen by the indexer get -inf, combined with the causal
 * mask; step 5 and "Attention output gate": output times sigmoid gate].
 *   q [B,S,H,Dqk] (nope slice then rope slice; the split does not change the
 *     dot product), k_cache [B,T,H,Dqk], v_cache [B,T,H,Dv] (expanded K/V),
 *   indices [B,S,topk] int32, gate [B,S,H] or [B,S,H,Dv] or NULL
 *   out [B,S,H,Dv] double
 */
void oracle_sparse_attn_pas(const void *q, const void *k_cache,
                            const void *v_cache, const void *sink_k,
                            const void *sink_v, int n_sink,
                            const int32_t *indices, const void *gate,
                            int dtype, int B, int S, int T, int past_len,
                            int H, int Dqk, int Dv, int topk, double sm_scale,
                            int gate_dim, double *out) {
  int64_t n = (int64_t)B * S * H;
#pragma omp parallel
  {
    unsigned char *sel = (unsigned char *)malloc((size_t)T);
    double *logit = (double *)malloc(sizeof(double) * ((size_t)T + n_sink));
#pragma omp for schedule(dynamic, 1)
    for (int64_t e = 0; e < n; ++e) {
      int h = (int)(e % H);
      int64_t bs = e / H;
      int64_t s = bs % S;
      int64_t b = bs / S;
      int64_t p = (int64_t)past_len + s;
      /* additive sparse mask AND causal mask */
      memset(sel, 0, (size_t)T);
      for (int j = 0; j < topk; ++j) {
        int64_t t = indices[bs * topk + j];
        if (t >= 0 && t <= p && t < T) sel[t] = 1;
      }
      double *o = out + e * Dv;
      masked_softmax_row(q, e * Dqk, k_cache, v_cache, sink_k, sink_v, n_sink,
                         dtype, b, T, H, h, Dqk, Dv, sm_scale, sel, logit, o);
      apply_gate(gate, dtype, gate_dim, bs, H, h, Dv, o);
    }
    free(logit);
    free(sel);
  }
}

void oracle_sparse_attn(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *indices, const void *gate, int dtype,
                        int B, int S, int T, int past_len, int H, int Dqk,
                        int Dv, int topk, double sm_scale, int gate_dim,
                        double *out) {
  oracle_sparse_attn_pas(q, k_cache, v_cache, NULL, NULL, 0, indices, gate,
                         dtype, B, S, T, past_len, H, Dqk, Dv, topk, sm_scale,
                         gate_dim, out);
}

/*
 * Sliding-window attention [Spark-X2.5 page: sliding_window 512;
 * openPangu-2.0 page §3.2: SWA layers see a fixed 512-token local window].
 * Query at p sees keys max(0, p-W+1) .. p. The K/V buffers hold T_buf rows;
 * buffer row j is absolute position kv_offset + j.
 *   q [B,S,H,Dqk], k_buf [B,T_buf,H,Dqk], v_buf [B,T_buf,H,Dv], gate as above
 *   out [B,S,H,Dv] double
 */
static void swa_attn(const void *q, const void *k_buf, const void *v_buf,
                     const void *sink_k, const void *sink_v, int n_sink,
                     const void *gate, int dtype, int B, int S, int T_buf,
                     int past_len, int kv_offset, int H, int H_kv, int Dqk,
                     int Dv, int window, double sm_scale, int gate_dim,
                     double *out) {
  int64_t n = (int64_t)B * S * H;
  int group = H / H_kv; /* query heads per KV head */
#pragma omp parallel
  {
    unsigned char *sel = (unsigned char *)malloc((size_t)T_buf);
    double *logit =
        (double *)malloc(sizeof(double) * ((size_t)T_buf + n_sink));
#pragma omp for schedule(dynamic, 1)
    for (int64_t e = 0; e < n; ++e) {
      int h = (int)(e % H);
      int64_t bs = e / H;
      int64_t s = bs % S;
      int64_t b = bs / S;
      int64_t p = (int64_t)past_len + s;
      int64_t lo = p - window + 1;
      if (lo < 0) lo = 0;
      for (int64_t j = 0; j < T_buf; ++j) {
        int64_t t = (int64_t)kv_offset + j;
        sel[j] = (t >= lo && t <= p) ? 1 : 0;
      }
      double *o = out + e * Dv;
      masked_softmax_row(q, e * Dqk, k_buf, v_buf, sink_k, sink_v, n_sink,
                         dtype, b, T_buf, H_kv, h / group, Dqk, Dv, sm_scale,
                         sel, logit, o);
      apply_gate(gate, dtype, gate_dim, bs, H, h, Dv, o);
    }
    free(logit);
    free(sel);
  }
}

void oracle_swa_attn_pas(const void *q, const void *k_buf, const void *v_buf,
                         const void *sink_k, const void *sink_v, int n_sink,
                         const void *gate, int dtype, int B, int S, int T_buf,
                         int past_len, int kv_offset, int H, int Dqk, int Dv,
                         int window, double sm_scale, int gate_dim,
                         double *out) {
  swa_attn(q, k_buf, v_buf, sink_k, sink_v, n_sink, gate, dtype, B, S, T_buf,
           past_len, kv_offset, H, H, Dqk, Dv, window, sm_scale, gate_dim, out);
}

void oracle_swa_attn(const void *q, const void *k_buf, const void *v_buf,
                     const void *gate, int dtype, int B, int S, int T_buf,
                     int past_len, int kv_offset, int H, int Dqk, int Dv,
                     int window, double sm_scale, int gate_dim, double *out) {
  swa_attn(q, k_buf, v_buf, NULL, NULL, 0, gate, dtype, B, S, T_buf, past_len,
           kv_offset, H, H, Dqk, Dv, window, sm_scale, gate_dim, out);
}

/*
 * Sliding-window attention with grouped KV heads [Spark-X2.5 page, "why the
 * gate": num_attention_heads 8, num_key_value_heads 2]. The buffers hold H_kv
 * heads (H_kv divides H): k_buf [B,T_buf,H_kv,Dqk], v_buf [B,T_buf,H_kv,Dv];
 * query head h reads KV head h / (H / H_kv). Everything else as
 * oracle_swa_attn.
 */
void oracle_swa_attn_gqa(const void *q, const void *k_buf, const void *v_buf,
                         const void *gate, int dtype, int B, int S, int T_buf,
                         int past_len, int kv_offset, int H, int H_kv, int Dqk,
                         int Dv, int window, double sm_scale, int gate_dim,
                         double *out) {
  swa_attn(q, k_buf, v_buf, NULL, NULL, 0, gate, dtype, B, S, T_buf, past_len,
           kv_offset, H, H_kv, Dqk, Dv, window, sm_scale, gate_dim, out);
}
