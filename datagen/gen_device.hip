// gen_device.hip -- GPU implementation of the seeded synthetic-input generator.
//
// Same definition as gen_host.c (SplitMix64 stream, twelve-lane Irwin-Hall
// normal, affine index rows, synthetic score rows); the two must agree bit for
// bit. This module holds none of the attention method's arithmetic. It lets
// the benchmark and tests create multi-GiB caches directly in HBM instead of
// shipping them over PCIe.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t sm_out(uint64_t key, uint64_t n) {
  return mix64(key + n * GOLDEN);
}

__device__ __forceinline__ int32_t lane_sum(uint64_t key, uint64_t i) {
  int32_t s = 0;
#pragma unroll
  for (int j = 1; j <= 3; ++j) {
    uint64_t r = sm_out(key, 3 * i + (uint64_t)j);
    s += (int32_t)(r & 0xFFFF) + (int32_t)((r >> 16) & 0xFFFF) +
         (int32_t)((r >> 32) & 0xFFFF) + (int32_t)((r >> 48) & 0xFFFF);
  }
  return s;
}

__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static uint64_t host_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static uint64_t host_stream_key(uint64_t seed, int tensor_id) {
  return host_mix64((seed << 20) + (uint64_t)(uint32_t)tensor_id);
}

__global__ void normal_kernel(void* dst, int dtype, int64_t n, uint64_t key, float cscale,
                              int64_t start) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
    int32_t z = lane_sum(key, (uint64_t)(start + e)) - 393210;
    float v = __fmul_rn((float)z, cscale);
    if (dtype == 0)
      ((float*)dst)[e] = v;
    else
      ((uint16_t*)dst)[e] = to_bf16_rne(v);
  }
}

__device__ __forceinline__ uint64_t gcd64(uint64_t a, uint64_t b) {
  while (b) {
    uint64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

__global__ void indices_kernel(int32_t* dst, int64_t row0, int64_t nrows, int S, int past_len,
                               int k, uint64_t key) {
  int64_t rr = blockIdx.x;
  if (rr >= nrows) return;
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
  for (int j = threadIdx.x; j < k; j += blockDim.x)
    dst[rr * k + j] = ((uint64_t)j < n) ? (int32_t)((a * (uint64_t)j + c) % n) : -1;
}

__global__ void scores_kernel(float* dst, int64_t row0, int64_t nrows, int S, int T, int past_len,
                              uint64_t key, int mode, float cscale) {
  int64_t n = nrows * (int64_t)T;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
    int64_t rr = e / T, t = e % T;
    int64_t r = row0 + rr;
    int64_t s = r % S;
    uint64_t idx = (uint64_t)r * (uint64_t)T + (uint64_t)t;
    int32_t sum = lane_sum(key, idx);
    float v = __fmul_rn((float)(sum - 393210), cscale);
    if (mode == 1) {
      v = rintf(__fmul_rn(v, 8.0f)) / 8.0f;
    } else if (mode == 2) {
      if (v < 0.0f) v = (sum & 1) ? -0.0f : 0.0f;
    }
    if (t > (int64_t)past_len + s) v = -INFINITY;
    dst[e] = v;
  }
}

static int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

extern "C" {

int dsagen_normal_device(void* dst, int dtype, int64_t n, uint64_t seed, int tensor_id,
                         float cscale, int64_t start, hipStream_t stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(normal_kernel, dim3(grid_for(n)), dim3(256), 0, stream, dst, dtype, n,
                     host_stream_key(seed, tensor_id), cscale, start);
  return (int)hipGetLastError();
}

int dsagen_indices_device(int32_t* dst, int64_t row0, int64_t nrows, int S, int past_len, int k,
                          uint64_t seed, int tensor_id, hipStream_t stream) {
  if (nrows <= 0) return 0;
  if (nrows > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(indices_kernel, dim3((unsigned)nrows), dim3(256), 0, stream, dst, row0,
                     nrows, S, past_len, k, host_stream_key(seed, tensor_id));
  return (int)hipGetLastError();
}

int dsagen_scores_device(float* dst, int64_t row0, int64_t nrows, int S, int T, int past_len,
                         uint64_t seed, int tensor_id, int mode, float cscale,
                         hipStream_t stream) {
  if (nrows <= 0 || T <= 0) return 0;
  hipLaunchKernelGGL(scores_kernel, dim3(grid_for(nrows * (int64_t)T)), dim3(256), 0, stream,
                     dst, row0, nrows, S, T, past_len, host_stream_key(seed, tensor_id), mode,
                     cscale);
  return (int)hipGetLastError();
}

}  // extern "C"
