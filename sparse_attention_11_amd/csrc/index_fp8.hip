// index_fp8.hip -- the lightning indexer on FP8 operands (gfx950).
//
// The A.X-K2 page's implementation notes describe the reference indexer as a
// Hadamard rotation of q and k followed by FP8 quantisation and an FP8
// scoring kernel; the rotation cancels in the dot products (H q . H k =
// D q . k), so the scores approximate the bf16 ones.
//
// Kernels
//  quant_fp8_kernel   rows of D bf16 values -> Walsh-Hadamard transform (+-1
//                     entries, stride 1 first, fp32), one power-of-two scale
//                     per row (the smallest 2^e with max|y| 2^-e <= 448) and
//                     OCP E4M3 codes of y 2^-e, rounded to nearest even.
//                     D / 8 lanes per row, 8 values per lane: strides 1, 2, 4
//                     inside a lane, 8 .. D/2 across lanes.
//  idx8_tile_kernel   scores of 16 queries x 512 keys per workgroup on the
//                     same causal schedule as the bf16 kernel; each wave keeps
//                     128 keys' codes in registers as A operands of the gfx950
//                     v_mfma_f32_16x16x128_f8f6f4 (one instruction covers a
//                     whole 128-dim head); the queries' codes of 8 heads at a
//                     time are copied global -> LDS by the LDS-DMA path.
//                     score = k_scale[t] * sum_h (w_h q_scale_h scale / D)
//                     relu(codes_q . codes_k): positive row scales move
//                     outside the ReLU.
#include "common.h"
#include "idx_tiles.h"
#include "kernels.h"

namespace dsa {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8_t;  // 32 FP8 codes

// FP8 E4M3 code of a float with |v| <= 448, rounded to nearest, ties to even
// (subnormals are multiples of 2^-9 below 2^-6; a normal value 2^E (1 + m/8)
// has code (E + 7) << 3 | m). Every step is exact except the two rintf.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a < 0x1p-6f) return sign | (uint32_t)rintf(a * 512.0f);
  int E;
  frexpf(a, &E);  // a = f 2^E, f in [0.5, 1)
  E -= 1;         // a = mant 2^E, mant in [1, 2)
  float m = rintf((ldexpf(a, -E) - 1.0f) * 8.0f);
  if (m >= 8.0f) {
    m = 0.0f;
    E += 1;
  }
  return sign | (uint32_t)(((E + 7) << 3) | (int)m);
}

template <int D>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ x,
                                                        uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales,
                                                        int64_t rows) {
  constexpr int LPR = D / 8;  // lanes per row
  static_assert(LPR >= 1 && LPR <= 16, "a row lies inside one 16-lane DPP row");
  const int lane = threadIdx.x & 63;
  const int lr = lane % LPR;
  const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const bool valid = r < rows;
  const int64_t rr = valid ? r : rows - 1;  // every lane takes part in the exchanges
  const u32x4_t raw = load16(x + rr * D + 8 * lr);
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = __uint_as_float(raw[i] << 16);
    y[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
  }
  // strides 1, 2, 4 inside the lane
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((j & h) == 0) {
        const float a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
  // strides 8, 16, ... across lanes: the lane with the lower index holds a
  // (DPP lane exchanges: LPR <= 16 keeps a row inside one DPP row)
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) {
    const bool upper = (lr & m) != 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float o = __uint_as_float(lane_xor_u32(__float_as_uint(y[j]), m, lane));
      y[j] = upper ? o - y[j] : y[j] + o;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(y[j]));
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1)
    amax = fmaxf(amax, __uint_as_float(lane_xor_u32(__float_as_uint(amax), m, lane)));
  int e = 0;
  if (amax > 0.0f) {
    int E;
    frexpf(amax, &E);
    E -= 1;  // floor(log2 amax)
    e = (ldexpf(amax, -(E - 8)) <= 448.0f) ? E - 8 : E - 7;
  }
  uint32_t c[2] = {0u, 0u};
  if (amax > 0.0f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j >> 2] |= e4m3_rne(ldexpf(y[j], -e)) << (8 * (j & 3));
  }
  if (!valid) return;
  *(uint2*)(codes + r * D + 8 * lr) = make_uint2(c[0], c[1]);
  if (lr == 0) scales[r] = ldexpf(1.0f, e);
}

constexpr int kWaveK = 128;        // keys per wave (8 MFMA M blocks of 16)
constexpr int kStageBytes = 16384;  // 8 heads of 16 queries x 128 codes
constexpr int kDI = 128;
constexpr int kG = kStageBytes / (16 * kDI);  // heads per stage

__device__ __forceinline__ f32x4_t mfma_fp8(const i32x8_t& a, const i32x8_t& b, f32x4_t c) {
  // format 0 = FP8 E4M3 for both operands; zero scales select the unscaled form
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// One workgroup = 16 queries x 512 keys; wave w keeps keys 128w..128w+127 of
// the tile in registers: A operand kb holds keys 16 kb + lane % 16, codes
// 32 (lane / 16) .. +31 of each. The B operand of (head, query lq) uses the
// same code ranges, so the 128-term sums match. A stage's LDS image holds,
// per head, two 1 KB planes (codes 0-15 and 16-31 of each lane's 32), so
// each half of a B operand is one conflict-free 16-byte read per lane.
template <int MODE>
__global__ __launch_bounds__(256, 2) void idx8_tile_kernel(
    const uint8_t* __restrict__ qc, const float* __restrict__ qs, const uint8_t* __restrict__ kc,
    const float* __restrict__ ks, const uint16_t* __restrict__ w, float* __restrict__ scores,
    int S, int T, int P, int HI, float scale_d, int nqt, int nkt, int npairs, int maxlen) {
  __shared__ __attribute__((aligned(16))) uint8_t qsm[2][kStageBytes];
  const int b = blockIdx.y;
  IdxTile tile;
  if (!idx_tile_of(blockIdx.x, 16, S, P, nqt, nkt, npairs, maxlen, &tile)) return;
  const int qt = tile.qt, kt = tile.kt;
  DSA_CHECK(qt >= 0 && qt < nqt && kt >= 0 && kt < nkt, qt, kt);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lq = lane & 15, lg = lane >> 4;
  const int q0 = qt * 16;
  const int kw0 = kt * kIdxTileK + wave * kWaveK;
  const int64_t row = (int64_t)b * S + min(q0 + lq, S - 1);
  const bool active = kw0 <= P + min(q0 + 16, S) - 1;

  i32x8_t a[8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    const int t = kw0 + 16 * kb + lq;
    const uint8_t* kp = kc + ((int64_t)b * T + (t < T ? t : T - 1)) * kDI + 32 * lg;
    u32x4_t lo = u32x4_t{0, 0, 0, 0}, hi = u32x4_t{0, 0, 0, 0};
    if (active && t < T) {
      lo = load16(kp);
      hi = load16(kp + 16);
    }
    a[kb] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }

  // stage block n (16 per stage, 4 per wave) = (head n / 2, plane n % 2)
  const int nst = (HI + kG - 1) / kG;
  auto issue_stage = [&](int st, int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int blk = 4 * wave + r;
      // heads past HI copy the last head (finite operands for their zero weight)
      const int h = min(st * kG + blk / 2, HI - 1);
      const uint8_t* src = qc + (row * HI + h) * kDI + 32 * lg + 16 * (blk & 1);
      __builtin_amdgcn_global_load_lds(
          (const void*)src, (__attribute__((address_space(3))) void*)(&qsm[buf][blk * 1024]), 16,
          0, 0);
    }
  };
  // per-head weights of the next stage, w_h * q_scale_h * scale / D, as raw
  // loads (combined when their stage runs)
  uint16_t wn[kG];
  float sn[kG];
  auto load_weights = [&](int st) {
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      const int h = min(st * kG + g, HI - 1);
      wn[g] = w[row * HI + h];
      sn[g] = qs[row * HI + h];
    }
  };

  f32x4_t sc[8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) sc[kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  issue_stage(0, 0);
  load_weights(0);
  for (int st = 0; st < nst; ++st) {
    uint16_t wc[kG];
    float scur[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      wc[g] = wn[g];
      scur[g] = sn[g];
    }
    // stage st has landed (each wave drains its own copies before the
    // barrier) and every wave is done with the buffer stage st+1 overwrites
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    const int buf = st & 1;
    if (st + 1 < nst) {
      issue_stage(st + 1, buf ^ 1);
      load_weights(st + 1);
    }
    if (active) {
      auto read_op = [&](int g) {
        const u32x4_t lo = *(const u32x4_t*)(&qsm[buf][(2 * g) * 1024 + 16 * lane]);
        const u32x4_t hi = *(const u32x4_t*)(&qsm[buf][(2 * g + 1) * 1024 + 16 * lane]);
        return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      };
      i32x8_t bn = read_op(0);
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        const i32x8_t bq = bn;
        if (g + 1 < kG) bn = read_op(g + 1);  // next head's operand under this head's MFMAs
        f32x4_t acc[8];
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) acc[kb] = mfma_fp8(a[kb], bq, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f});
        const float wh = (st * kG + g < HI) ? bf16_to_f32(wc[g]) * scur[g] * scale_d : 0.0f;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x = acc[kb][e];
            if (MODE == 0) x = relu_bits(x);
            sc[kb][e] = fmaf(wh, x, sc[kb][e]);
          }
      }
    }
  }

  const bool vec = (T & 3) == 0;
  idx_fill_upper<16>(scores, tile, b, S, T, nkt, vec);
  // lane (lq, lg) holds keys kw0 + 16 kb + 4 lg + e of query q0 + lq
  const int s = q0 + lq;
  if (s >= S) return;
  const int p = P + s;
  float* orow = scores + ((int64_t)b * S + s) * T;
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    const int t0 = kw0 + 16 * kb + 4 * lg;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = t0 + e;
      float x = sc[kb][e] * ks[(int64_t)b * T + (t < T ? t : T - 1)];
      if (MODE == 2) x = relu_bits(x);
      v[e] = (t <= p) ? x : -INFINITY;
    }
    if (vec && t0 + 3 < T) {
      *(float4*)(orow + t0) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (t0 + e < T) orow[t0 + e] = v[e];
    }
  }
}

}  // namespace

#ifdef DSA_DEBUG
DSA_DEBUG_TAKE(index_fp8)
#endif

hipError_t launch_quant_fp8(const void* x, uint8_t* codes, float* scales, int64_t rows, int dim,
                            hipStream_t st) {
  const int rpw = 256 / (dim / 8);  // rows per workgroup
  const int64_t g = (rows + rpw - 1) / rpw;
  if (g > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const uint16_t* xx = (const uint16_t*)x;
  switch (dim) {
    case 32: hipLaunchKernelGGL((quant_fp8_kernel<32>), dim3((unsigned)g), dim3(256), 0, st, xx, codes, scales, rows); break;
    case 64: hipLaunchKernelGGL((quant_fp8_kernel<64>), dim3((unsigned)g), dim3(256), 0, st, xx, codes, scales, rows); break;
    case 128: hipLaunchKernelGGL((quant_fp8_kernel<128>), dim3((unsigned)g), dim3(256), 0, st, xx, codes, scales, rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_index_scores_fp8(const uint8_t* q_codes, const float* q_scales,
                                   const uint8_t* k_codes, const float* k_scales, const void* w,
                                   float* scores, int B, int S, int T, int P, int HI, int DI,
                                   float scale, int relu_mode, hipStream_t st) {
  if (DI != kDI) return hipErrorInvalidValue;
  const IdxGrid g = idx_grid(S, T, P, 16);
  if (g.gx > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const float sd = scale / (float)DI;  // the rotation multiplies every dot product by D
  const uint16_t* ww = (const uint16_t*)w;
#define DSA_IDX8(MODE)                                                                          \
  hipLaunchKernelGGL((idx8_tile_kernel<MODE>), dim3((unsigned)g.gx, B), dim3(256), 0, st, q_codes, \
                     q_scales, k_codes, k_scales, ww, scores, S, T, P, HI, sd, g.nqt, g.nkt,     \
                     g.npairs, g.maxlen)
  switch (relu_mode) {
    case 0: DSA_IDX8(0); break;
    case 1: DSA_IDX8(1); break;
    default: DSA_IDX8(2); break;
  }
#undef DSA_IDX8
  return hipGetLastError();
}

}  // namespace dsa
