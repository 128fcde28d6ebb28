/*
 * gen_host.c -- host implementation of the seeded synthetic-input generator.
 *
 * This module holds none of the attention method's arithmetic: it only makes
 * reproducible inputs. gen_device.hip implements the same definition on the
 * GPU, and the two must agree bit for bit (a test checks this). Both sides
 * follow the definition below and nothing else.
 *
 * Definition
 *  - SplitMix64 (Steele, Lea & Flood, OOPSLA 2014; the finaliser as published
 *    by Vigna): the n-th output (n >= 1) of the generator seeded with `key` is
 *    mix(key + n * 0x9E3779B97F4A7C15), with
 *      mix(z): z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9;
 *              z = (z ^ (z >> 27)) * 0x94D049BB133111EB;
 *              return z ^ (z >> 31);
 *    all arithmetic modulo 2^64.
 *  - Stream key of a tensor: key = mix(seed * 2^20 + tensor_id).
 *  - Normal element i (i = 0, 1, ...): take outputs n = 3i+1, 3i+2, 3i+3,
 *    split each into four 16-bit lanes, and sum the twelve lanes (an integer
 *    in [0, 786420]). z = sum - 393210 is an Irwin-Hall variate with mean 0 and
 *    variance 65536^2 - 1. It is exact in fp32. The value is the fp32 product
 *    z * c, one correctly rounded multiply, where c = scale / sqrt(65536^2-1)
 *    is rounded to fp32 once by the caller. bf16 output is that fp32 rounded
 *    to nearest-even on bit 16.
 *  - Index rows: row r = b*S + s sees n = past_len + s + 1 positions. From
 *    h = output 1 of the stream keyed mix(key ^ (r * 0xD1B54A32D192ED03)):
 *    a = (h >> 32) mod n, bumped to 1 if 0, then incremented (wrapping n -> 1)
 *    until gcd(a, n) = 1; c = (h & 0xFFFFFFFF) mod n. Slot j < k holds
 *    (a*j + c) mod n when j < n, else -1. The k entries are distinct.
 *  - Score rows (synthetic fp32 inputs for the top-k): element (r, t) is the
 *    normal value of index r*T + t with scale 1, then by mode:
 *      0 as is; 1 rounded to a multiple of 1/8 (rint of z*8, divided by 8),
 *      which makes many exact ties; 2 negative values replaced by a zero whose
 *      sign is the lowest bit of the lane sum (a mix of +0.0 and -0.0);
 *    and -inf wherever t > past_len + s (the causal structure of real scores).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static uint64_t stream_key(uint64_t seed, int tensor_id) {
  return mix64((seed << 20) + (uint64_t)(uint32_t)tensor_id);
}

/* n-th output, n >= 1 */
static uint64_t sm_out(uint64_t key, uint64_t n) { return mix64(key + n * GOLDEN); }

static int32_t lane_sum(uint64_t key, uint64_t i) {
  int32_t s = 0;
  for (int j = 1; j <= 3; ++j) {
    uint64_t r = sm_out(key, 3 * i + (uint64_t)j);
    s += (int32_t)(r & 0xFFFF) + (int32_t)((r >> 16) & 0xFFFF) +
         (int32_t)((r >> 32) & 0xFFFF) + (int32_t)((r >> 48) & 0xFFFF);
  }
  return s;
}

static uint16_t to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* dtype 0: fp32, 1: bf16 bit patterns. Fills dst[0..n) with elements
 * start .. start+n-1 of the stream. */
void dsagen_normal_host(void *dst, int dtype, int64_t n, uint64_t seed,
                        int tensor_id, float cscale, int64_t start) {
  uint64_t key = stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < n; ++e) {
    int32_t z = lane_sum(key, (uint64_t)(start + e)) - 393210;
    volatile float zf = (float)z;
    float v = zf * cscale;
    if (dtype == 0)
      ((float *)dst)[e] = v;
    else
      ((uint16_t *)dst)[e] = to_bf16_rne(v);
  }
}

static uint64_t gcd64(uint64_t a, uint64_t b) {
  while (b) {
    uint64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

/* rows [row0, row0+nrows) of a [B*S, k] int32 index tensor */
void dsagen_indices_host(int32_t *dst, int64_t row0, int64_t nrows, int S,
                         int past_len, int k, uint64_t seed, int tensor_id) {
  uint64_t key = stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t rr = 0; rr < nrows; ++rr) {
    int64_t r = row0 + rr;
    int64_t s = r % S;
    uint64_t n = (uint64_t)past_len + (uint64_t)s + 1;
    uint64_t h = sm_out(mix64(key ^ ((uint64_t)r * 0xD1B54A32D192ED03ULL)), 1);
    uint64_t a = (h >> 32) % n;
    if (a == 0) a = 1;
    while (gcd64(a, n) != 1) {
      a += 1;
      if (a >= n) a = 1;
    }
    uint64_t c = (h & 0xFFFFFFFFULL) % n;
    for (int j = 0; j < k; ++j)
      dst[rr * k + j] = ((uint64_t)j < n) ? (int32_t)((a * (uint64_t)j + c) % n) : -1;
  }
}

/* rows [row0, row0+nrows) of a [B*S, T] fp32 score tensor */
void dsagen_scores_host(float *dst, int64_t row0, int64_t nrows, int S, int T,
                        int past_len, uint64_t seed, int tensor_id, int mode,
                        float cscale) {
  uint64_t key = stream_key(seed, tensor_id);
  int64_t n = nrows * (int64_t)T;
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < n; ++e) {
    int64_t rr = e / T, t = e % T;
    int64_t r = row0 + rr;
    int64_t s = r % S;
    uint64_t idx = (uint64_t)r * (uint64_t)T + (uint64_t)t;
    int32_t sum = lane_sum(key, idx);
    volatile float zf = (float)(sum - 393210);
    float v = zf * cscale;
    if (mode == 1) {
      volatile float x8 = v * 8.0f;
      v = rintf(x8) / 8.0f;
    } else if (mode == 2) {
      if (v < 0.0f) v = (sum & 1) ? -0.0f : 0.0f;
    }
    if (t > (int64_t)past_len + s) v = -INFINITY;
    dst[e] = v;
  }
}
