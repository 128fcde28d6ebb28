// topk.hip -- per-row top-k of fp32 score rows (gfx950).
//
// Keeps, per row, the k positions with the largest scores (A.X-K2 page,
// "Sparse Gated Attention": the indexer returns the top index_topk
// positions), ordered by score descending and position ascending; -inf
// slots are reported as -1.
//
// Every element becomes a unique 64-bit key
//     key = orderable(score) << 32 | (0xFFFFFFFF - t)
// (orderable() is monotone in the float order and folds -0.0 onto +0.0), so
// "largest k keys" is exactly the required selection including the
// lower-position tie rule. A radix select over 8-bit digits, most significant
// first, finds the k-th largest key; it stops as soon as every key sharing the
// current prefix is needed. Keys >= that threshold are compacted into LDS and
// sorted with a bitonic network. Histograms are per wave (LDS atomics), the
// digit search is a wave-level suffix scan. One 1024-thread workgroup per
// row; rows up to 32768 elements stay in registers, longer rows are re-read
// from memory on every pass.
#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxK = 2048;

__device__ __forceinline__ uint64_t make_key(float sc, int t) {
  return ((uint64_t)orderable_key(sc) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t);
}

// EPT > 0: T <= kThreads * EPT, elements held in registers; EPT == 0: streamed.
template <int EPT>
__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores,
                                                        int32_t* __restrict__ out, int T, int k,
                                                        int k2) {
  __shared__ uint32_t hist[kWaves][256];
  __shared__ uint32_t total[256];
  __shared__ uint64_t sel[kMaxK];
  __shared__ uint64_t s_prefix;
  __shared__ int s_krem;
  __shared__ int s_done;
  __shared__ uint32_t s_cnt;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const float* srow = scores + row * (int64_t)T;

  uint32_t kreg[EPT > 0 ? EPT : 1];
  if (EPT > 0) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int t = tid + j * kThreads;
      kreg[j] = t < T ? orderable_key(srow[t]) : 0u;
    }
  }

  uint64_t prefix = 0, mask = 0;
  int krem = k;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int i = tid; i < kWaves * 256; i += kThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    if (EPT > 0) {
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int t = tid + j * kThreads;
        if (t < T) {
          const uint64_t key = ((uint64_t)kreg[j] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t);
          if ((key & mask) == prefix) atomicAdd(&hist[wave][(uint32_t)(key >> shift) & 255u], 1u);
        }
      }
    } else {
      for (int t = tid; t < T; t += kThreads) {
        const uint64_t key = make_key(srow[t], t);
        if ((key & mask) == prefix) atomicAdd(&hist[wave][(uint32_t)(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t c = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) c += hist[w][tid];
      total[tid] = c;
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 4l..4l+3; suffix sums over lanes (high digits first)
      const uint32_t b0 = total[4 * lane], b1 = total[4 * lane + 1], b2 = total[4 * lane + 2],
                     b3 = total[4 * lane + 3];
      const uint32_t local = b0 + b1 + b2 + b3;
      uint32_t x = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(x, off, 64);
        if (lane + off < 64) x += y;
      }
      const uint64_t ball = __ballot(x >= (uint32_t)krem);
      const int L = __popcll(ball) - 1;  // highest lane whose suffix reaches krem
      if (lane == L) {
        uint32_t cum = x - local;  // elements in digits above this lane's bins
        const uint32_t bins[4] = {b0, b1, b2, b3};
        int digit = 4 * lane;
        uint32_t above = cum;
        for (int q = 3; q >= 0; --q) {
          if (cum + bins[q] >= (uint32_t)krem) {
            digit = 4 * lane + q;
            above = cum;
            break;
          }
          cum += bins[q];
        }
        const int kr = krem - (int)above;
        s_prefix = prefix | ((uint64_t)digit << shift);
        s_krem = kr;
        s_done = (total[digit] == (uint32_t)kr) ? 1 : 0;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    mask |= (uint64_t)0xFF << shift;
    krem = s_krem;
    const int done = s_done;
    __syncthreads();
    if (done) break;
  }

  // compact keys >= threshold (exactly k of them)
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  const uint64_t thr = prefix;
  if (EPT > 0) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int t = tid + j * kThreads;
      if (t < T) {
        const uint64_t key = ((uint64_t)kreg[j] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t);
        if (key >= thr) {
          const uint32_t pos = atomicAdd(&s_cnt, 1u);
          if (pos < (uint32_t)kMaxK) sel[pos] = key;
        }
      }
    }
  } else {
    for (int t = tid; t < T; t += kThreads) {
      const uint64_t key = make_key(srow[t], t);
      if (key >= thr) {
        const uint32_t pos = atomicAdd(&s_cnt, 1u);
        if (pos < (uint32_t)kMaxK) sel[pos] = key;
      }
    }
  }
  for (int i = k + tid; i < k2; i += kThreads) sel[i] = 0;  // pad to a power of two
  __syncthreads();

  // bitonic sort, descending
  for (int size = 2; size <= k2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (k2 >> 1); i += kThreads) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const uint64_t a = sel[lo], c = sel[hi];
        const bool desc = (lo & size) == 0;
        if (desc ? (a < c) : (a > c)) {
          sel[lo] = c;
          sel[hi] = a;
        }
      }
      __syncthreads();
    }
  }

  int32_t* orow = out + row * (int64_t)k;
  for (int i = tid; i < k; i += kThreads) {
    const uint64_t key = sel[i];
    const uint32_t hi = (uint32_t)(key >> 32);
    orow[i] = (hi == DSA_NEG_INF_KEY) ? -1 : (int32_t)(0xFFFFFFFFu - (uint32_t)key);
  }
}

}  // namespace

size_t topk_workspace_bytes(int, int, int, int) { return 0; }

hipError_t launch_topk(const float* scores, int32_t* indices, int B, int S, int T, int topk,
                       void*, hipStream_t stream) {
  int k2 = 1;
  while (k2 < topk) k2 <<= 1;
  const int64_t rows = (int64_t)B * S;
  if (rows > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (T <= kThreads * 8)
    hipLaunchKernelGGL(topk_kernel<8>, dim3((unsigned)rows), dim3(kThreads), 0, stream, scores,
                       indices, T, topk, k2);
  else if (T <= kThreads * 32)
    hipLaunchKernelGGL(topk_kernel<32>, dim3((unsigned)rows), dim3(kThreads), 0, stream, scores,
                       indices, T, topk, k2);
  else
    hipLaunchKernelGGL(topk_kernel<0>, dim3((unsigned)rows), dim3(kThreads), 0, stream, scores,
                       indices, T, topk, k2);
  return hipGetLastError();
}

}  // namespace dsa
