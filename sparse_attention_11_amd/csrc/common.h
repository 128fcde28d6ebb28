// common.h -- device-side helpers shared by the libdsa kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"  // (struct DebugRecord)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;  // MFMA bf16 operand (16 B / lane)
typedef __attribute__((ext_vector_type(16))) float f32x16_t;  // 32x32 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;    // 16x16 MFMA accumulator

#define DSA_LOG2E 1.4426950408889634f

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Two fp32 -> packed bf16x2 (lo in bits 0..15), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ u32x4_t load16(const void* p) { return *(const u32x4_t*)p; }

// Raw buffer resource over [base, base + bytes) (bytes clamped to 32 bits):
// a buffer load whose range lies past the end returns zeros instead of
// touching memory. The third dword is the gfx9-family untyped-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)n,
                                          0x00020000);
}
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D(16x16) += A(16x32) B(32x16): lane l holds A[l%16][8(l/16)+i] and
// B[8(l/16)+i][l%16] (i = 0..7); acc[j] = D[4(l/16)+j][l%16].
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// max(x, 0) as one signed-integer max on the bit pattern: every float with
// the sign bit set (negatives, -0) maps to +0, everything else is unchanged.
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// 2^x as the bare hardware instruction (no denormal-range fix-up): results
// below 2^-126 may flush to zero, which only ever drops negligible weights.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// x where bit `pos` of `bits` is set, else -inf: one bit-field extract that
// replicates the bit, then one bitwise select.
__device__ __forceinline__ float keep_or_neg_inf(float x, uint32_t bits, int pos) {
  const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)bits, pos, 1);
  return __uint_as_float((__float_as_uint(x) & sel) | (0xFF800000u & ~sel));
}

// sigmoid in fp32 as 1 / (1 + e^-x): exactly 0 at -inf, 1 at +inf, 1/2 at 0.
__device__ __forceinline__ float sigmoid_f32(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Order-preserving map of an fp32 score to u32 (larger float -> larger key),
// with -0.0 folded onto +0.0 so that the two tie.
__device__ __forceinline__ uint32_t orderable_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
#define DSA_NEG_INF_KEY 0x007FFFFFu  // orderable_key(-inf)

// acc + lo + hi of a packed bf16 pair, in fp32 (one v_dot2 with ones)
__device__ __forceinline__ float sum_bf16x2(uint32_t packed, float acc) {
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, packed), ones, acc, false);
}

// max of two floats as one v_max_f32 (no NaN-quieting of the inputs first).
// Like every inline-asm helper here it must only be given VALU results: the
// compiler does not insert the MFMA-to-VALU wait states before inline asm, so
// an MFMA result read here may be stale.
__device__ __forceinline__ float max_f32(float a, float b) {
  float r;
  asm("v_max_f32_e32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Transposing LDS read pair (gfx950 ds_read_b64_tr_b16): within each group of
// 16 lanes, lane 4j + q supplies a byte address a and lane i receives element
// i % 4 at a of lane 4j + i / 4 as its element j. Two reads `second` bytes
// apart fill an 8-element MFMA operand (first read -> elements 0..3).
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8_t lds_read_tr_pair(const uint16_t* lds, uint32_t byte_off,
                                                     uint32_t second) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const __attribute__((address_space(3))) char* base =
      (const __attribute__((address_space(3))) char*)lds;
  const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + byte_off));
  const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + byte_off + second));
  const i16x4_t lo = a, hi = b;
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}
// max of three floats as one v_max3_f32 (VALU results only, as max_f32)
__device__ __forceinline__ float max3_f32(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// max(x, x of lane l ^ 32): one cross-half lane swap, no LDS round trip
__device__ __forceinline__ float max_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_f32(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// x + (x of lane l ^ 32): one cross-half lane swap, no LDS round trip
__device__ __forceinline__ float sum_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Value of lane l ^ m (m = 1, 2, 4, 8, 16 or 32) without an LDS round trip:
// DPP quad permutes for 1 and 2, two mirrors for 4, a row rotate for 8, and
// the cross-row / cross-half permlane swaps for 16 and 32. m must fold to a
// constant at the call site.
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v, int m, int lane) {
  switch (m) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
    case 4: {  // i ^ 7 inside each half row, then i ^ 3 inside each quad
      const int r = __builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);  // row_half_mirror
      return (uint32_t)__builtin_amdgcn_mov_dpp(r, 0x1B, 0xF, 0xF, false);     // quad_perm 3,2,1,0
    }
    case 8: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);
    case 16: {
      const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return (lane & 16) ? r[0] : r[1];
    }
    default: {
      const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (lane & 32) ? r[0] : r[1];
    }
  }
}
// Inclusive prefix sum over the 64 lanes without LDS: DPP row shifts by 1,
// 2, 4, 8 inside each row of 16, then the row-15 and row-31 broadcasts
// carry row totals into the rows above.
__device__ __forceinline__ uint32_t wave_scan_incl_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}
// Sum over the 64 lanes, returned in every lane.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_incl_u32(x), 63);
}

__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t v, int m, int lane) {
  const uint32_t lo = lane_xor_u32((uint32_t)v, m, lane);
  const uint32_t hi = lane_xor_u32((uint32_t)(v >> 32), m, lane);
  return ((uint64_t)hi << 32) | lo;
}

// Lane-swap helpers (wave64).
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// ---------------------------------------------------------------- checks
// -DDSA_DEBUG builds: DSA_CHECK(cond, a, b) asserts an invariant a kernel
// relies on (an index inside its buffer, a count the algorithm fixes). A
// failure neither traps nor stops the kernel: it counts into this file's
// device record (struct DebugRecord, kernels.h) and keeps the first failure's
// line and the two values; the C ABI of a debug build synchronizes after each
// call and reports a non-zero count as DSA_ERR_CHECK. Release builds compile
// every check out. DSA_DEBUG_TAKE(name) defines the host function that reads
// and clears the record of the file it is placed in.
#ifdef DSA_DEBUG
static __device__ dsa::DebugRecord g_debug_record;
__device__ __noinline__ static void debug_fail(int line, long long a, long long b) {
  if (atomicAdd(&g_debug_record.count, 1u) == 0u) {
    g_debug_record.line = line;
    g_debug_record.a = a;
    g_debug_record.b = b;
  }
}
#define DSA_CHECK(cond, a, b)                                          \
  do {                                                                 \
    if (!(cond)) debug_fail(__LINE__, (long long)(a), (long long)(b)); \
  } while (0)
#define DSA_DEBUG_TAKE(name)                                                                    \
  int debug_take_##name(DebugRecord* out) {                                                     \
    if (hipMemcpyFromSymbol(out, HIP_SYMBOL(g_debug_record), sizeof(DebugRecord)) != hipSuccess) \
      return -1;                                                                                \
    if (out->count == 0u) return 0;                                                             \
    const DebugRecord zero = {0u, 0, 0, 0};                                                     \
    return hipMemcpyToSymbol(HIP_SYMBOL(g_debug_record), &zero, sizeof(DebugRecord)) ==         \
                   hipSuccess                                                                   \
               ? 1                                                                              \
               : -1;                                                                            \
  }
#else
#define DSA_CHECK(cond, a, b) ((void)0)
#endif
