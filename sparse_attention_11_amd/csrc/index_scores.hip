// index_scores.hip -- lightning-indexer scores with causal mask (gfx950).
//
// score[b,s,t] = sum_h w[b,s,h] * relu(scale * q[b,s,h,:] . k[b,t,:]) for
// t <= p = past_len + s, -inf above (A.X-K2 page, "Sparse Gated Attention":
// per-head products with the shared index key, weighted head sum, ReLU,
// causal upper-triangle mask).
//
// The index key is shared by all index heads, so it is the stationary MFMA
// operand: a workgroup keeps a 128-key tile of k in registers and streams the
// per-head query tiles through the bf16 MFMA, one K = idx_dim product per
// head followed by the per-head ReLU and weighted accumulation in fp32.
// Scores are produced transposed (keys on the MFMA M axis) so that each lane
// owns one query column: the head weight is then a per-lane scalar.
//
// Kernels
//  idx_tile_kernel   prefill tiles of 128 queries x 128 keys, 4 waves, each
//                    wave 128 keys x 32 queries; only tiles on or below the
//                    causal diagonal are launched, paired (j, last-j) so every
//                    pair costs the same, pairs dealt to XCDs round-robin.
//  idx_fill_kernel   -inf for the key tiles above the diagonal.
//  idx_rows_kernel   few-query calls (decode): the index heads become the
//                    MFMA M axis; a wave streams 256 keys of k in blocks of 32.
//  idx_f32_kernel    fp32 inputs: plain fp32 loops (parity-size workloads).
#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kTileQ = 128;
constexpr int kTileK = 128;

// Key tiles a query tile needs (the causal triangle).
__host__ __device__ __forceinline__ int tiles_for_qtile(int qt, int S, int P, int nkt) {
  int last_q = min((qt + 1) * kTileQ, S) - 1;
  int c = (P + last_q) / kTileK + 1;
  return c < nkt ? c : nkt;
}

template <int DI, int MODE>
__global__ __launch_bounds__(256) void idx_tile_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ w,
                                                       float* __restrict__ scores, int S, int T,
                                                       int P, int HI, float scale, int nqt,
                                                       int nkt, int npairs, int maxlen) {
  constexpr int KS = DI / 16;
  const int b = blockIdx.y;
  // block -> (query tile, key tile)
  const int pid = blockIdx.x;
  const int xcd = pid & 7;
  const int n = pid >> 3;
  const int slot = n / maxlen;
  int u = n - slot * maxlen;
  const int j = slot * 8 + xcd;
  if (j >= npairs) return;
  const int qa = j, qb = nqt - 1 - j;
  const int ca = tiles_for_qtile(qa, S, P, nkt);
  int qt, kt;
  if (u < ca) {
    qt = qa;
    kt = u;
  } else {
    if (qb == qa) return;
    u -= ca;
    if (u >= tiles_for_qtile(qb, S, P, nkt)) return;
    qt = qb;
    kt = u;
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 31, lh = lane >> 5;
  const int q0 = qt * kTileQ, k0 = kt * kTileK;

  // stationary A operands: key rows (MFMA M), 8 dims per lane per k-step
  bf16x8_t a[4][KS];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = k0 + 32 * i + ln;
    const uint16_t* kp = k + ((int64_t)b * T + (t < T ? t : T - 1)) * DI + 8 * lh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t v = load16(kp + 16 * ks);
      if (t >= T) v = u32x4_t{0, 0, 0, 0};
      a[i][ks] = as_bf16x8(v);
    }
  }

  const int s = q0 + 32 * wave + ln;
  const int sc_ = s < S ? s : S - 1;
  const int64_t row = (int64_t)b * S + sc_;
  const uint16_t* qp = q + row * HI * DI + 8 * lh;
  const uint16_t* wp = w + row * HI;

  f32x16_t sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] = zero16();

  for (int h = 0; h < HI; ++h) {
    bf16x8_t bq[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bq[ks] = as_bf16x8(load16(qp + h * DI + 16 * ks));
    const float wh = bf16_to_f32(wp[h]) * scale;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x16_t acc = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma32x32x16(a[i][ks], bq[ks], acc);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = acc[e];
        if (MODE == 0) x = relu_f32(x);
        sc[i][e] = fmaf(wh, x, sc[i][e]);
      }
    }
  }
  if (s >= S) return;

  const int p = P + s;
  float* orow = scores + ((int64_t)b * S + s) * T;
  const bool vec = (T & 3) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int t0 = k0 + 32 * i + 8 * g + 4 * lh;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = sc[i][4 * g + r];
        if (MODE == 2) x = fmaxf(x, 0.0f);
        v[r] = (t0 + r <= p) ? x : -INFINITY;
      }
      if (vec && t0 + 3 < T) {
        *(float4*)(orow + t0) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t0 + r < T) orow[t0 + r] = v[r];
      }
    }
  }
}

// -inf for every key tile above the causal diagonal of its query tile.
__global__ __launch_bounds__(256) void idx_fill_kernel(float* __restrict__ scores, int S, int T,
                                                       int P, int nkt) {
  const int64_t row = blockIdx.x;  // b*S + s
  const int s = (int)(row % S);
  const int start = tiles_for_qtile(s / kTileQ, S, P, nkt) * kTileK;
  float* orow = scores + row * T;
  for (int t = start + threadIdx.x; t < T; t += blockDim.x) orow[t] = -INFINITY;
}

// Few queries per call: MFMA M = index heads (NHB blocks of 32), N = 32 keys.
// A wave streams kRowsKeys keys in blocks of 32; the query operand is loaded
// once per wave and the next block's keys are loaded during the current
// block's MFMAs.
constexpr int kRowsKeys = 256;  // keys per wave
template <int DI, int NHB, int MODE>
__global__ __launch_bounds__(256) void idx_rows_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ w,
                                                       float* __restrict__ scores, int S, int T,
                                                       int P, int HI, float scale) {
  constexpr int KS = DI / 16;
  constexpr int NB = kRowsKeys / 32;
  const int64_t row = blockIdx.y;
  const int b = (int)(row / S), s = (int)(row % S);
  const int p = P + s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 31, lh = lane >> 5;
  const int tbase = (blockIdx.x * 4 + wave) * kRowsKeys;
  float* orow = scores + row * T;
  if (tbase >= T) return;

  if (tbase > p) {  // the whole wave is above the diagonal
    for (int kb = 0; kb < NB; ++kb) {
      const int t = tbase + 32 * kb + ln;
      if (lh == 0 && t < T) orow[t] = -INFINITY;
    }
    return;
  }

  bf16x8_t a[NHB][KS];
  float wv[NHB][16];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int hh = 32 * hb + ln;
    const uint16_t* qp = q + (row * HI + (hh < HI ? hh : HI - 1)) * DI + 8 * lh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t v = load16(qp + 16 * ks);
      if (hh >= HI) v = u32x4_t{0, 0, 0, 0};
      a[hb][ks] = as_bf16x8(v);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = 32 * hb + 8 * (e >> 2) + 4 * lh + (e & 3);
      wv[hb][e] = m < HI ? bf16_to_f32(w[row * HI + m]) * scale : 0.0f;
    }
  }

  auto load_keys = [&](int kb, bf16x8_t* bk) {
    const int t = tbase + 32 * kb + ln;
    const bool tv = t < T && t <= p;
    const uint16_t* kp = k + ((int64_t)b * T + (tv ? t : 0)) * DI + 8 * lh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t v = load16(kp + 16 * ks);
      if (!tv) v = u32x4_t{0, 0, 0, 0};
      bk[ks] = as_bf16x8(v);
    }
  };
  bf16x8_t bk[KS], bn[KS];
  load_keys(0, bk);
  for (int kb = 0; kb < NB; ++kb) {
    const int t = tbase + 32 * kb + ln;
    const bool more = kb + 1 < NB && tbase + 32 * (kb + 1) <= p && tbase + 32 * (kb + 1) < T;
    if (more) load_keys(kb + 1, bn);
    float part = 0.0f;
    if (tbase + 32 * kb <= p) {
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        f32x16_t acc = zero16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma32x32x16(a[hb][ks], bk[ks], acc);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = acc[e];
          if (MODE == 0) x = fmaxf(x, 0.0f);
          part = fmaf(wv[hb][e], x, part);
        }
      }
      part += shfl_xor_f(part, 32);
      if (MODE == 2) part = fmaxf(part, 0.0f);
    }
    if (lh == 0 && t < T) orow[t] = (t <= p) ? part : -INFINITY;
    if (more) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bk[ks] = bn[ks];
    }
  }
}

// fp32 inputs: one thread per (row, key), plain loops in fp32.
__global__ __launch_bounds__(256) void idx_f32_kernel(const float* __restrict__ q,
                                                      const float* __restrict__ k,
                                                      const float* __restrict__ w,
                                                      float* __restrict__ scores, int S, int T,
                                                      int P, int HI, int DI, float scale,
                                                      int mode) {
  const int64_t row = blockIdx.y;
  const int b = (int)(row / S), s = (int)(row % S);
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  float* out = scores + row * T + t;
  if (t > P + s) {
    *out = -INFINITY;
    return;
  }
  const float* kp = k + ((int64_t)b * T + t) * DI;
  float total = 0.0f;
  for (int h = 0; h < HI; ++h) {
    const float* qp = q + (row * HI + h) * DI;
    float dot = 0.0f;
    for (int d = 0; d < DI; ++d) dot = fmaf(qp[d], kp[d], dot);
    float u = scale * dot;
    if (mode == 0) u = fmaxf(u, 0.0f);
    total = fmaf(w[row * HI + h], u, total);
  }
  if (mode == 2) total = fmaxf(total, 0.0f);
  *out = total;
}

template <int DI, int MODE>
hipError_t launch_tiles(const uint16_t* q, const uint16_t* k, const uint16_t* w, float* scores,
                        int B, int S, int T, int P, int HI, float scale, hipStream_t st) {
  const int nqt = (S + kTileQ - 1) / kTileQ;
  const int nkt = (T + kTileK - 1) / kTileK;
  const int npairs = (nqt + 1) / 2;
  int maxlen = 1;
  for (int j = 0; j < npairs; ++j) {
    int len = tiles_for_qtile(j, S, P, nkt);
    if (nqt - 1 - j != j) len += tiles_for_qtile(nqt - 1 - j, S, P, nkt);
    if (len > maxlen) maxlen = len;
  }
  const int64_t slots = (npairs + 7) / 8;
  const int64_t gx = 8 * slots * (int64_t)maxlen;
  if (gx > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((idx_tile_kernel<DI, MODE>), dim3((unsigned)gx, B), dim3(256), 0, st, q, k,
                     w, scores, S, T, P, HI, scale, nqt, nkt, npairs, maxlen);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // rows whose query tile does not reach the last key tile get -inf past it
  if (tiles_for_qtile(0, S, P, nkt) < nkt) {
    hipLaunchKernelGGL(idx_fill_kernel, dim3((unsigned)((int64_t)B * S)), dim3(256), 0, st, scores,
                       S, T, P, nkt);
    e = hipGetLastError();
  }
  return e;
}

template <int DI, int NHB, int MODE>
hipError_t launch_rows(const uint16_t* q, const uint16_t* k, const uint16_t* w, float* scores,
                       int B, int S, int T, int P, int HI, float scale, hipStream_t st) {
  hipLaunchKernelGGL((idx_rows_kernel<DI, NHB, MODE>), dim3((T + 4 * kRowsKeys - 1) / (4 * kRowsKeys), B * S),
                     dim3(256), 0, st, q, k, w, scores, S, T, P, HI, scale);
  return hipGetLastError();
}

template <int DI, int MODE>
hipError_t dispatch_rows(const uint16_t* q, const uint16_t* k, const uint16_t* w, float* scores,
                         int B, int S, int T, int P, int HI, float scale, hipStream_t st) {
  const int nhb = (HI + 31) / 32;
  switch (nhb) {
    case 1: return launch_rows<DI, 1, MODE>(q, k, w, scores, B, S, T, P, HI, scale, st);
    case 2: return launch_rows<DI, 2, MODE>(q, k, w, scores, B, S, T, P, HI, scale, st);
    case 3: return launch_rows<DI, 3, MODE>(q, k, w, scores, B, S, T, P, HI, scale, st);
    default: return launch_rows<DI, 4, MODE>(q, k, w, scores, B, S, T, P, HI, scale, st);
  }
}

template <int MODE>
hipError_t dispatch_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* w, float* scores,
                         int B, int S, int T, int P, int HI, int DI, float scale,
                         hipStream_t st) {
  // few queries per sequence and at most 128 index heads: head-major MFMA
  const bool rows = S < 32 && HI <= 128 && (int64_t)B * S <= 65535;
  if (rows) {
    switch (DI) {
      case 32: return dispatch_rows<32, MODE>(q, k, w, scores, B, S, T, P, HI, scale, st);
      case 64: return dispatch_rows<64, MODE>(q, k, w, scores, B, S, T, P, HI, scale, st);
      default: return dispatch_rows<128, MODE>(q, k, w, scores, B, S, T, P, HI, scale, st);
    }
  }
  switch (DI) {
    case 32: return launch_tiles<32, MODE>(q, k, w, scores, B, S, T, P, HI, scale, st);
    case 64: return launch_tiles<64, MODE>(q, k, w, scores, B, S, T, P, HI, scale, st);
    default: return launch_tiles<128, MODE>(q, k, w, scores, B, S, T, P, HI, scale, st);
  }
}

}  // namespace

hipError_t launch_index_scores(const void* q_idx, const void* k_idx, const void* w, float* scores,
                               int B, int S, int T, int past_len, int HI, int DI, float scale,
                               int relu_mode, int dtype, hipStream_t stream) {
  if (dtype == 0) {
    hipLaunchKernelGGL(idx_f32_kernel, dim3((T + 255) / 256, B * S), dim3(256), 0, stream,
                       (const float*)q_idx, (const float*)k_idx, (const float*)w, scores, S, T,
                       past_len, HI, DI, scale, relu_mode);
    return hipGetLastError();
  }
  const uint16_t* q = (const uint16_t*)q_idx;
  const uint16_t* k = (const uint16_t*)k_idx;
  const uint16_t* ww = (const uint16_t*)w;
  switch (relu_mode) {
    case 0: return dispatch_bf16<0>(q, k, ww, scores, B, S, T, past_len, HI, DI, scale, stream);
    case 1: return dispatch_bf16<1>(q, k, ww, scores, B, S, T, past_len, HI, DI, scale, stream);
    default: return dispatch_bf16<2>(q, k, ww, scores, B, S, T, past_len, HI, DI, scale, stream);
  }
}

}  // namespace dsa
