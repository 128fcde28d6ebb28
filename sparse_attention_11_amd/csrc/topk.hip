// topk.hip -- per-row top-k of fp32 score rows (gfx950).
//
// Keeps, per row, the k positions with the largest scores (A.X-K2 page,
// "Sparse Gated Attention": the indexer returns the top index_topk
// positions), ordered by score descending and position ascending; -inf
// slots are reported as -1.
//
// Every finite score becomes a unique non-zero 64-bit key
//     key = orderable(score) << 32 | (0xFFFFFFFF - t)
// (orderable() is monotone in the float order and folds -0.0 onto +0.0), so
// "largest k keys" is exactly the required selection including the
// lower-position tie rule. -inf scores become key 0 and are never selected:
// if a row has only n < k finite scores, its last k - n slots are -1, which is
// what selecting -inf entries would print anyway. (Skipping them also keeps
// the causal half of every prefill row out of the histograms, where its
// identical keys would serialise the LDS atomics.)
//
// One workgroup (256, 512 or 1024 threads) per (row, segment):
//  1. count the valid keys; k' = min(k, count);
//  2. radix select of the k'-th largest key, most significant digit first,
//     11/11/10-bit digits per 32-bit half, one shared LDS histogram per
//     pass, a block suffix scan to pick the digit; it stops as soon as every
//     key sharing the current prefix is needed (normally after two or three
//     passes over the high half);
//  3. the k' keys >= threshold are compacted into LDS;
//  4. either a bitonic sort (descending; strides inside a thread run in
//     registers, inside a wave via lane swaps, only the widest through LDS)
//     and the index output, or, for the first stage of a long row, the
//     unsorted keys of the segment (padded with 0) for a second pass, or,
//     when the caller asks for no ordering, the compacted list itself.
// Rows longer than 16384 are split: segments of 16384 scores are reduced to
// k candidate keys each, groups of 16384 candidates are reduced again until
// at most 16384 remain, then one workgroup per row selects and sorts the
// final k. Every stage keeps its elements in registers.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kMaxK = 2048;
constexpr int kBins = 2048;
constexpr int kSegLen = 16384;  // segment length of the first stage (long rows)

__device__ __forceinline__ uint64_t score_key(float sc, int t) {
  if (sc == -INFINITY) return 0ull;
  return ((uint64_t)orderable_key(sc) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t);
}

// digit layout: pass 0..2 on the high word, 3..5 on the low word
__device__ __forceinline__ int digit_shift(int pass) {
  const int lo = (pass >= 3) ? 0 : 32;
  const int pp = pass % 3;
  return lo + (pp == 0 ? 21 : (pp == 1 ? 10 : 0));
}
__device__ __forceinline__ uint32_t digit_mask(int pass) { return (pass % 3 == 2) ? 0x3FFu : 0x7FFu; }

template <int NW>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* red) {
  v = wave_sum_u32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += red[w];
  return s;
}

// After a histogram pass: find the digit holding the krem-th largest key.
// Thread t owns bins BPT t .. BPT t + BPT - 1; a block suffix scan over
// threads (high digits first) locates the bin. Writes the digit, the count
// still needed inside it, and whether that bin is taken whole.
template <int NT>
__device__ __forceinline__ void pick_digit(const uint32_t* hist, uint32_t* red, int krem, int tid,
                                           int lane, int wave, int* s_krem, int* s_done,
                                           int* s_digit) {
  constexpr int BPT = kBins / NT, NW = NT / 64;
  uint32_t bins[BPT];
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    bins[q] = hist[BPT * tid + q];
    local += bins[q];
  }
  // inclusive suffix sum within the wave = wave total - exclusive prefix
  const uint32_t pre = wave_scan_incl_u32(local);
  const uint32_t x = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63) - pre + local;
  if (lane == 0) red[wave] = x;
  __syncthreads();
  uint32_t above_waves = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (w > wave) above_waves += red[w];
  const uint32_t suf = x + above_waves;   // keys in bins >= BPT*tid
  const uint32_t suf_next = suf - local;  // keys in bins >= BPT*tid + BPT
  if (suf >= (uint32_t)krem && suf_next < (uint32_t)krem) {
    uint32_t cum = suf_next;
    int q = BPT - 1;
    for (; q > 0; --q) {
      if (cum + bins[q] >= (uint32_t)krem) break;
      cum += bins[q];
    }
    const int kr = krem - (int)cum;
    *s_digit = BPT * tid + q;
    *s_krem = kr;
    *s_done = (bins[q] == (uint32_t)kr) ? 1 : 0;
  }
}

// Bitonic sort (descending) of the kk keys in sel[0..kk), padded with 0 to
// N = NT*E slots, then the positions of the first k to orow (-1 for padding).
// Strides inside a thread run in registers, inside a wave via lane swaps,
// only the widest through LDS (sel holds N keys). Keys are unique apart from
// the 0 padding, so one compare decides each exchange: a slot keeps its own
// key iff (own > partner) equals "this slot keeps the larger key"; both
// conditions are lane masks and meet in one mask XOR. Callers have published
// sel[0..kk) with a barrier.
template <int NT, int E>
__device__ __forceinline__ void sort_store(uint64_t* sel, int kk, int k, int32_t* orow) {
  const int tid = threadIdx.x, lane = tid & 63;
  constexpr int N = NT * E;
  uint64_t a[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid * E + e;
    a[e] = (i < kk) ? sel[i] : 0ull;
  }
#pragma unroll
  for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int pe = e ^ stride;
          if (pe > e) {
            const int i = tid * E + e;
            const bool desc = (i & size) == 0;  // larger key to the lower slot
            const uint64_t lo = a[e], hi = a[pe];
            const bool sw = (hi > lo) == desc;
            a[e] = sw ? hi : lo;
            a[pe] = sw ? lo : hi;
          }
        }
      } else {
        if (stride >= 64 * E) {
          __syncthreads();
#pragma unroll
          for (int e = 0; e < E; ++e) sel[tid * E + e] = a[e];
          __syncthreads();
        }
        // the slot's role depends on tid bits only (stride, size >= E)
        const int i0 = tid * E;
        const bool keep_max = ((i0 & stride) == 0) == ((i0 & size) == 0);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint64_t other =
              stride < 64 * E ? lane_xor_u64(a[e], stride / E, lane) : sel[(tid * E + e) ^ stride];
          a[e] = ((a[e] > other) == keep_max) ? a[e] : other;
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid * E + e;
    if (i < k) orow[i] = (a[e] == 0ull) ? -1 : (int32_t)(0xFFFFFFFFu - (uint32_t)a[e]);
  }
}

// Workgroup blockIdx.x handles elements [seg*seg_len, min(T, (seg+1)*seg_len))
// of row blockIdx.x / nseg (seg = blockIdx.x % nseg), where a row holds
// SRC 0: T fp32 scores; SRC 1: T 64-bit candidate keys (0 = empty).
// DST 0: sorted indices to out_idx[row, 0..k); DST 1: unsorted keys of this
//        segment to out_keys[(row*nseg + seg)*k ...], padded with 0.
// NT threads per workgroup (256, or 1024 when a stage has few workgroups).
// EPT > 0 keeps the elements in registers (range <= NT*EPT); EPT == 0 streams.
// E: sort elements per thread (the sort covers max(k, NT) = NT*E keys).
// Stages with at most 16 keys per thread are held to 64 registers so that
// 2048 threads (8 waves per SIMD) fit a CU; the 32-key stages need more.
template <int NT, int SRC, int DST, int EPT, int E>
__global__ __launch_bounds__(NT, (EPT <= 16 ? 2048 / NT : 1)) void topk_kernel(const void* __restrict__ src,
                                                        int32_t* __restrict__ out_idx,
                                                        uint64_t* __restrict__ out_keys, int T,
                                                        int k, int seg_len, int nseg, int order,
                                                        int S, int P) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t hist[kBins + 64];  // + one spare bin per lane
  // selected keys: k of them for a candidate stage, at most NT*E >= k for a
  // sorting stage (sized to that, so more workgroups fit a CU's LDS)
  constexpr int kSel = DST == 1 ? kMaxK : NT * E;
  __shared__ uint64_t sel[kSel];
  __shared__ uint32_t s_red[NW];
  __shared__ uint32_t s_col[(EPT > 0 ? EPT : 1) * NW];
  __shared__ int s_krem, s_done, s_digit;
  __shared__ uint32_t s_cnt;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x / nseg;
  const int seg = (int)(blockIdx.x % nseg);
  const int t0 = seg * seg_len;
  // valid length of a score row: T, or its causal bound when P >= 0
  const int L = (SRC == 0 && P >= 0) ? min(T, P + (int)(row % S) + 1) : T;
  const int n = max(0, min(L - t0, seg_len));
  const float* srow = (const float*)src + row * (int64_t)T;
  const uint64_t* krow = (const uint64_t*)src + row * (int64_t)T;
  auto load_key = [&](int j) -> uint64_t {
    if (SRC == 0) return score_key(srow[t0 + j], t0 + j);
    return krow[t0 + j];
  };
  // registers hold the high word only for score input (the low word is the
  // position, known from the slot), the whole key for candidate input
  using KT = typename std::conditional<SRC == 0, uint32_t, uint64_t>::type;
  KT kreg[EPT > 0 ? EPT : 1];
  auto reg_key = [&](int j) -> uint64_t {
    if (SRC == 1) return (uint64_t)kreg[j];
    const int t = t0 + tid + j * NT;
    return kreg[j] ? (((uint64_t)kreg[j] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t)) : 0ull;
  };
  uint32_t valid = 0;
  if (EPT > 0 && SRC == 0) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid + j * NT;
      const float sc = e < n ? srow[t0 + e] : -INFINITY;
      const uint32_t hi = (sc == -INFINITY) ? 0u : orderable_key(sc);
      kreg[j] = (KT)hi;
      valid += hi != 0u;
    }
  } else if (EPT > 0) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid + j * NT;
      const uint64_t key = e < n ? load_key(e) : 0ull;
      kreg[j] = (KT)key;
      valid += key != 0ull;
    }
  } else {
    for (int e = tid; e < n; e += NT) valid += load_key(e) != 0ull;
  }
  const int nvalid = (int)block_sum<NW>(valid, s_red);
  const int kk = min(k, nvalid);
  DSA_CHECK(kk <= kSel, kk, kSel);

  // Register path on score input: the selection is decided on the 32-bit
  // score key alone; ties at the threshold are resolved by position rank.
  if (EPT > 0 && SRC == 0) {
    uint32_t prefix = 0, mask = 0;
    int krem = kk;
    bool done = kk == 0;
    for (int pass = 0; pass < 3 && !done; ++pass) {
      const int shift = (pass == 0) ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t dmask = (pass == 2) ? 0x3FFu : 0x7FFu;
      for (int i = tid; i < kBins; i += NT) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        // non-matching keys count into a per-lane spare bin instead of branching
        const uint32_t hi = (uint32_t)kreg[j];
        const bool m = hi != 0u && (hi & mask) == prefix;
        atomicAdd(&hist[m ? ((hi >> shift) & dmask) : (uint32_t)(kBins + lane)], 1u);
      }
      __syncthreads();
      pick_digit<NT>(hist, s_red, krem, tid, lane, wave, &s_krem, &s_done, &s_digit);
      __syncthreads();
      prefix |= (uint32_t)s_digit << shift;
      mask |= dmask << shift;
      krem = s_krem;
      done = s_done != 0;
    }
    // done: every key >= prefix is taken. Otherwise the score key is fully
    // determined (prefix), all larger keys are taken, and among the keys equal
    // to it the krem lowest positions.
    if (tid == 0) s_cnt = 0;
    if (!done) {
      // positions t = t0 + 256 j + 64 wave + lane are ordered (j, wave, lane)
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const uint64_t b = __ballot((uint32_t)kreg[j] == prefix);
        if (lane == 0) s_col[j * NW + wave] = (uint32_t)__popcll(b);
      }
      __syncthreads();
      if (wave == 0) {  // exclusive prefix over the EPT*4 column counts
        constexpr int PER = EPT > 0 ? (EPT * NW + 63) / 64 : 1;
        uint32_t v[PER];
        uint32_t loc = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          const int i = lane * PER + q;
          v[q] = i < EPT * NW ? s_col[i] : 0u;
          loc += v[q];
        }
        const uint32_t x = wave_scan_incl_u32(loc);
        uint32_t run = x - loc;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          const int i = lane * PER + q;
          if (i < EPT * NW) s_col[i] = run;
          run += v[q];
        }
      }
    }
    __syncthreads();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // which of this thread's keys are taken (bit j), then an ordered compaction
    uint64_t takebits = 0;
    uint32_t ntake = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const uint32_t hi = (uint32_t)kreg[j];
      bool take;
      if (done) {
        take = hi != 0u && hi >= prefix;
      } else {
        const bool tie = hi == prefix;
        const uint64_t b = __ballot(tie);
        const uint32_t rank = s_col[j * NW + wave] + (uint32_t)__popcll(b & lt_mask);
        take = hi > prefix || (tie && rank < (uint32_t)krem);
      }
      takebits |= (uint64_t)take << j;
      ntake += take;
    }
    const uint32_t x = wave_scan_incl_u32(ntake);  // inclusive prefix over the wave
    if (lane == 63) s_red[wave] = x;
    __syncthreads();
    uint32_t base = x - ntake;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w < wave) base += s_red[w];
#ifdef DSA_DEBUG
    if (tid == 0) {  // the selection holds exactly kk keys
      uint32_t tot = 0;
      for (int w = 0; w < NW; ++w) tot += s_red[w];
      DSA_CHECK(tot == (uint32_t)kk, tot, kk);
    }
#endif
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      if ((takebits >> j) & 1ull) {
        const uint32_t t = (uint32_t)(t0 + tid + j * NT);
        if (base < (uint32_t)kSel) sel[base] = ((uint64_t)kreg[j] << 32) | (0xFFFFFFFFu - t);
        ++base;
      }
    }
    __syncthreads();
  } else {
    // 64-bit keys (candidate input, or streamed rows): radix select on both halves
    uint64_t prefix = 0, mask = 0;
    if (kk > 0) {
      int krem = kk;
      for (int pass = 0; pass < 6; ++pass) {
        const int shift = digit_shift(pass);
        const uint32_t dmask = digit_mask(pass);
        for (int i = tid; i < kBins; i += NT) hist[i] = 0;
        __syncthreads();
        if (EPT > 0) {
#pragma unroll
          for (int j = 0; j < EPT; ++j) {
            const uint64_t key = reg_key(j);
            if (key != 0ull && (key & mask) == prefix)
              atomicAdd(&hist[(uint32_t)(key >> shift) & dmask], 1u);
          }
        } else {
          for (int e = tid; e < n; e += NT) {
            const uint64_t key = load_key(e);
            if (key != 0ull && (key & mask) == prefix)
              atomicAdd(&hist[(uint32_t)(key >> shift) & dmask], 1u);
          }
        }
        __syncthreads();
        pick_digit<NT>(hist, s_red, krem, tid, lane, wave, &s_krem, &s_done, &s_digit);
        __syncthreads();
        prefix |= (uint64_t)s_digit << shift;
        mask |= (uint64_t)dmask << shift;
        krem = s_krem;
        if (s_done) break;
      }
    }
    // compact the kk keys >= threshold
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    if (kk > 0) {
      const uint64_t thr = prefix;
      if (EPT > 0) {  // ordered compaction: block prefix scan of per-thread counts
        uint64_t takebits = 0;
        uint32_t ntake = 0;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
          const uint64_t key = reg_key(j);
          const bool take = key != 0ull && key >= thr;
          takebits |= (uint64_t)take << j;
          ntake += take;
        }
        const uint32_t x = wave_scan_incl_u32(ntake);
        if (lane == 63) s_red[wave] = x;
        __syncthreads();
        uint32_t base = x - ntake;
#pragma unroll
        for (int w = 0; w < NW; ++w)
          if (w < wave) base += s_red[w];
#ifdef DSA_DEBUG
        if (tid == 0) {  // the keys >= the threshold are exactly kk
          uint32_t tot = 0;
          for (int w = 0; w < NW; ++w) tot += s_red[w];
          DSA_CHECK(tot == (uint32_t)kk, tot, kk);
        }
#endif
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
          if ((takebits >> j) & 1ull) {
            if (base < (uint32_t)kSel) sel[base] = reg_key(j);
            ++base;
          }
        }
      } else {
        for (int e = tid; e < n; e += NT) {
          const uint64_t key = load_key(e);
          if (key != 0ull && key >= thr) {
            const uint32_t pos = atomicAdd(&s_cnt, 1u);
            if (pos < (uint32_t)kSel) sel[pos] = key;
          }
        }
      }
    }
    __syncthreads();
  }

  if (EPT == 0 && SRC == 1 && tid == 0) DSA_CHECK(s_cnt == (uint32_t)kk || kk == 0, s_cnt, kk);
  if (DST == 1) {  // first stage of a long row: unsorted candidates
    uint64_t* o = out_keys + ((int64_t)row * nseg + seg) * k;
    for (int i = tid; i < k; i += NT) o[i] = (i < kk) ? sel[i] : 0ull;
    return;
  }
  // unsorted output: the compacted list as it stands (its order is fixed by
  // the thread layout, so it repeats from run to run)
  static_assert(EPT > 0, "a repeatable order needs the ordered (register) compaction");
  if (order != 0) {
    int32_t* orow = out_idx + row * (int64_t)k;
    for (int i = tid; i < k; i += NT)
      orow[i] = (i < kk) ? (int32_t)(0xFFFFFFFFu - (uint32_t)sel[i]) : -1;
    return;
  }

  sort_store<NT, E>(sel, kk, k, out_idx + row * (int64_t)k);
}

template <int NT, int SRC, int DST, int EPT>
hipError_t launch_e(const void* src, int32_t* idx, uint64_t* keys, int64_t blocks, int T, int k,
                    int seg_len, int nseg, hipStream_t st, int order, int S, int P) {
  const dim3 g((unsigned)blocks), b(NT);
  // sort width NT*E >= max(k, NT); k <= kMaxK = 8 * 256, so 1024 threads
  // need E <= 2 and 512 threads E <= 4
  constexpr int E4 = NT >= 1024 ? 2 : 4, E8 = NT >= 1024 ? 2 : (NT >= 512 ? 4 : 8);
  if (DST == 1 || k <= NT)
    hipLaunchKernelGGL((topk_kernel<NT, SRC, DST, EPT, 1>), g, b, 0, st, src, idx, keys, T, k, seg_len, nseg, order, S, P);
  else if (k <= 2 * NT)
    hipLaunchKernelGGL((topk_kernel<NT, SRC, DST, EPT, 2>), g, b, 0, st, src, idx, keys, T, k, seg_len, nseg, order, S, P);
  else if (k <= 4 * NT)
    hipLaunchKernelGGL((topk_kernel<NT, SRC, DST, EPT, E4>), g, b, 0, st, src, idx, keys, T, k, seg_len, nseg, order, S, P);
  else
    hipLaunchKernelGGL((topk_kernel<NT, SRC, DST, EPT, E8>), g, b, 0, st, src, idx, keys, T, k, seg_len, nseg, order, S, P);
  return hipGetLastError();
}

// A stage with few workgroups (few rows: decode, one long sequence) uses
// 1024-thread workgroups so that each row gets four times the lanes; a
// stage whose elements per workgroup are at most `range` keeps them in
// registers (range / NT each). Ranges of 16384 take 512 threads (32 keys
// each, 80 registers, 6 waves per SIMD) rather than 256 threads of 64 keys
// (150 registers, 3 waves per SIMD): measured on 16384-score segments of a
// 528384-key row, 4.23 -> 3.55 ms for 4096 rows, bit-identical.
template <int SRC, int DST, int RANGE>
hipError_t launch_stage(const void* src, int32_t* idx, uint64_t* keys, int64_t blocks, int T,
                        int k, int seg_len, int nseg, hipStream_t st, int order = 0, int S = 1,
                        int P = -1) {
  if (blocks < 256)
    return launch_e<1024, SRC, DST, RANGE / 1024>(src, idx, keys, blocks, T, k, seg_len, nseg, st, order, S, P);
  if (RANGE / 256 > 16)
    return launch_e<512, SRC, DST, RANGE / 512>(src, idx, keys, blocks, T, k, seg_len, nseg, st, order, S, P);
  return launch_e<256, SRC, DST, RANGE / 256>(src, idx, keys, blocks, T, k, seg_len, nseg, st, order, S, P);
}

constexpr int kCand = 16384;  // candidate keys one register-resident workgroup takes

// number of candidate-reduction passes and their group counts for a row of T scores
// (k <= 2048 < kCand, so every pass shrinks the candidate count)
int stage_groups(int T, int k, int* groups, int max_levels) {
  const int64_t nseg = ((int64_t)T + kSegLen - 1) / kSegLen;
  int64_t C = nseg * k;
  int lv = 0;
  groups[lv++] = (int)nseg;
  while (C > kCand && lv < max_levels) {
    const int64_t g = (C + kCand - 1) / kCand;
    groups[lv++] = (int)g;
    C = g * k;
  }
  return lv;
}

// ------------------------------------------------------------ few long rows
// Decode calls have a few rows of many scores. Instead of reducing every
// 16384-score segment to k candidates (k = 2048 is an eighth of a segment, so
// two or three passes over k-candidate sets), the threshold comes from one
// histogram of the whole row: the top 11 bits of every valid key (sign,
// exponent, two mantissa bits), summed over the row's chunks. The bin holding
// the k-th largest key bounds the selection from below, so the keys in that
// bin and above -- on indexer scores k plus a few hundred to a few thousand --
// are the only candidates.
//   row_hist_zero_kernel  clears the rows' histograms
//   row_hist_kernel       one workgroup per 2048-score chunk: LDS histogram,
//                         non-zero bins added to the row's
//   row_filter_kernel     per chunk: the threshold bin from the row's
//                         histogram, then the chunk's keys in that bin and
//                         above, in position order, into the chunk's own slots
//   row_select_kernel     one workgroup per row: the first digit of the radix
//                         select is that same bin (read off the row histogram),
//                         the rest runs on the candidates (held in registers
//                         when there are at most 16384, streamed otherwise),
//                         then an ordered compaction (position order) and
//                         either the bitonic sort (dsa_topk) or the compacted
//                         list itself (dsa_topk_unsorted).
constexpr int kRowChunk = 2048;      // scores per chunk: 256 threads x 8
constexpr int kRowMaxChunks = 1024;  // rows up to 2M scores take this path
constexpr int kRowRegKeys = 16;      // candidates per select thread kept in registers
// Copies of each row's histogram: chunk c adds into copy c % kRowHistCopies,
// and readers sum the copies. Spreads the device-scope atomics of a row's
// chunks (a single 528385-key row has 259) over more addresses.
#ifndef DSA_ROW_HIST_COPIES
#define DSA_ROW_HIST_COPIES 4
#endif
constexpr int kRowHistCopies = DSA_ROW_HIST_COPIES;

__global__ __launch_bounds__(256) void row_hist_zero_kernel(uint32_t* __restrict__ h, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) h[i] = 0u;
}

__global__ __launch_bounds__(256) void row_hist_kernel(const float* __restrict__ scores,
                                                       uint32_t* __restrict__ ghist, int T,
                                                       int nc, int S, int P) {
  constexpr int EPT = kRowChunk / 256;
  __shared__ uint32_t h[kBins];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x / nc;
  const int c = blockIdx.x % nc;
  const int L = P >= 0 ? min(T, P + (int)(row % S) + 1) : T;  // valid scores of the row
  const int t0 = c * kRowChunk, n = max(0, min(L - t0, kRowChunk));
  for (int i = tid; i < kBins; i += 256) h[i] = 0u;
  const float* sr = scores + row * (int64_t)T + t0;
  float f[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + 256 * j;
    f[j] = e < n ? sr[e] : -INFINITY;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < EPT; ++j)
    if (f[j] != -INFINITY) atomicAdd(&h[orderable_key(f[j]) >> 21], 1u);
  __syncthreads();
  uint32_t* gr = ghist + (row * kRowHistCopies + c % kRowHistCopies) * kBins;
  for (int i = tid; i < kBins; i += 256)
    if (h[i]) atomicAdd(&gr[i], h[i]);
}

// bin i of a row's histogram: the sum of its copies
__device__ __forceinline__ uint32_t row_bin(const uint32_t* __restrict__ ghist, int64_t row, int i) {
  uint32_t v = 0;
#pragma unroll
  for (int cp = 0; cp < kRowHistCopies; ++cp) v += ghist[(row * kRowHistCopies + cp) * kBins + i];
  return v;
}

__global__ __launch_bounds__(256) void row_filter_kernel(const float* __restrict__ scores,
                                                         const uint32_t* __restrict__ ghist,
                                                         uint64_t* __restrict__ cand,
                                                         uint32_t* __restrict__ cnt, int T,
                                                         int nc, int k, int S, int P) {
  constexpr int NT = 256, NW = 4, EPT = kRowChunk / 256;
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t s_red[NW];
  __shared__ uint32_t s_col[EPT * NW];
  __shared__ int s_krem, s_done, s_digit;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x / nc;
  const int c = blockIdx.x % nc;
  const int L = P >= 0 ? min(T, P + (int)(row % S) + 1) : T;  // valid scores of the row
  const int t0 = c * kRowChunk, n = max(0, min(L - t0, kRowChunk));
  // this chunk's scores first: their loads overlap the histogram work
  const float* sr = scores + row * (int64_t)T + t0;
  uint32_t hi[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + NT * j;
    const float f = e < n ? sr[e] : -INFINITY;
    hi[j] = f == -INFINITY ? 0u : orderable_key(f);
  }
  uint32_t tot = 0;
  for (int i = tid; i < kBins; i += NT) {
    const uint32_t v = row_bin(ghist, row, i);
    h[i] = v;
    tot += v;
  }
  tot = block_sum<NW>(tot, s_red);  // (its barriers also publish h)
  const int kk = (int)min((uint32_t)k, tot);
  uint32_t bmin = 0xFFFFFFFFu;  // no candidates when the row has no valid key
  if (kk > 0) {
    __syncthreads();  // every thread has read s_red before pick_digit reuses it
    pick_digit<NT>(h, s_red, kk, tid, lane, wave, &s_krem, &s_done, &s_digit);
    __syncthreads();
    bmin = (uint32_t)s_digit;
  }
  // keys in the threshold bin and above, in position order: positions t0 +
  // 256 j + 64 wave + lane are ordered (j, wave, lane)
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const bool take = hi[j] != 0u && (hi[j] >> 21) >= bmin;
    const uint64_t bal = __ballot(take);
    if (lane == 0) s_col[j * NW + wave] = (uint32_t)__popcll(bal);
  }
  __syncthreads();
  if (wave == 0) {  // exclusive prefix over the EPT x NW column counts
    constexpr int PER = (EPT * NW + 63) / 64;
    uint32_t v[PER];
    uint32_t loc = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int i = lane * PER + q;
      v[q] = i < EPT * NW ? s_col[i] : 0u;
      loc += v[q];
    }
    const uint32_t x = wave_scan_incl_u32(loc);
    uint32_t run = x - loc;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int i = lane * PER + q;
      if (i < EPT * NW) s_col[i] = run;
      run += v[q];
    }
    if (lane == 63) {
      DSA_CHECK(x <= (uint32_t)n, x, n);
      cnt[row * nc + c] = x;
    }
  }
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t* cr = cand + (row * nc + c) * (int64_t)kRowChunk;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const bool take = hi[j] != 0u && (hi[j] >> 21) >= bmin;
    const uint64_t bal = __ballot(take);
    if (take) {
      const uint32_t pos = s_col[j * NW + wave] + (uint32_t)__popcll(bal & lt_mask);
      const uint32_t t = (uint32_t)(t0 + tid + NT * j);
      cr[pos] = ((uint64_t)hi[j] << 32) | (uint64_t)(0xFFFFFFFFu - t);
    }
  }
}

__global__ __launch_bounds__(1024) void row_select_kernel(const uint64_t* __restrict__ cand,
                                                          const uint32_t* __restrict__ cnt,
                                                          const uint32_t* __restrict__ ghist,
                                                          int32_t* __restrict__ out, int nc, int k,
                                                          int order) {
  constexpr int NT = 1024, NW = 16, EPT = kRowRegKeys;
  static_assert(kRowMaxChunks <= NT, "one thread per chunk offset");
  static_assert(kMaxK == 2 * NT, "the sort covers kMaxK slots with two per thread");
  __shared__ uint32_t hist[kBins + 64];  // + one spare bin per lane
  __shared__ uint64_t sel[kMaxK];
  __shared__ uint32_t off[kRowMaxChunks + 1];
  __shared__ uint32_t s_red[NW];
  __shared__ uint32_t s_col[EPT * NW];
  __shared__ int s_krem, s_done, s_digit;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  // start of each chunk's candidates in the concatenation (chunk order =
  // position order), and the row histogram
  const uint32_t cv = tid < nc ? cnt[row * nc + tid] : 0u;
  const uint32_t xi = wave_scan_incl_u32(cv);
  if (lane == 63) s_red[wave] = xi;
  uint32_t tot = 0;
  for (int i = tid; i < kBins; i += NT) {
    const uint32_t v = row_bin(ghist, row, i);
    hist[i] = v;
    tot += v;
  }
  __syncthreads();
  uint32_t wbase = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (w < wave) wbase += s_red[w];
  if (tid < nc) off[tid] = wbase + xi - cv;
  if (tid == nc - 1) off[nc] = wbase + xi;
  tot = block_sum<NW>(tot, s_red);  // (its barriers also publish off and hist)
  const int C = (int)off[nc];
  const int kk = (int)min((uint32_t)k, tot);  // <= C: every key of the top k is a candidate
  if (tid == 0) DSA_CHECK(kk <= C, kk, C);
  auto slot = [&](int g) -> int64_t {  // the g-th candidate's slot: last chunk with off <= g
    int lo = 0, hi = nc;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= (uint32_t)g) lo = mid;
      else hi = mid;
    }
    return (row * nc + lo) * (int64_t)kRowChunk + (g - (int)off[lo]);
  };
  // first digit: the threshold bin, from the row histogram (the candidates
  // are exactly the keys in that bin and above)
  uint64_t prefix = 0, mask = 0;
  int krem = kk;
  bool done = kk == 0;
  if (kk > 0) {
    __syncthreads();  // every thread has read s_red before pick_digit reuses it
    pick_digit<NT>(hist, s_red, kk, tid, lane, wave, &s_krem, &s_done, &s_digit);
    __syncthreads();
    prefix = (uint64_t)s_digit << digit_shift(0);
    mask = (uint64_t)digit_mask(0) << digit_shift(0);
    krem = s_krem;
    done = s_done != 0;
  }
  if (C <= NT * EPT) {
    // candidates g = tid + NT j in registers; their order (j, wave, lane) is
    // the candidate order
    uint64_t kreg[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int g = tid + NT * j;
      kreg[j] = g < C ? cand[slot(g)] : 0ull;
    }
    for (int pass = 1; pass < 6 && !done; ++pass) {
      const int shift = digit_shift(pass);
      const uint32_t dmask = digit_mask(pass);
      for (int i = tid; i < kBins; i += NT) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        // non-matching keys count into a per-lane spare bin instead of branching
        const bool m = kreg[j] != 0ull && (kreg[j] & mask) == prefix;
        atomicAdd(&hist[m ? ((uint32_t)(kreg[j] >> shift) & dmask) : (uint32_t)(kBins + lane)], 1u);
      }
      __syncthreads();
      pick_digit<NT>(hist, s_red, krem, tid, lane, wave, &s_krem, &s_done, &s_digit);
      __syncthreads();
      prefix |= (uint64_t)s_digit << shift;
      mask |= (uint64_t)dmask << shift;
      krem = s_krem;
      done = s_done != 0;
    }
    // the kk keys >= prefix, in candidate order (ballot column counts, then
    // an exclusive prefix over them)
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const uint64_t bal = __ballot(kreg[j] != 0ull && kreg[j] >= prefix);
      if (lane == 0) s_col[j * NW + wave] = (uint32_t)__popcll(bal);
    }
    __syncthreads();
    if (wave == 0) {
      constexpr int PER = (EPT * NW + 63) / 64;
      uint32_t v[PER];
      uint32_t loc = 0;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        v[q] = s_col[lane * PER + q];
        loc += v[q];
      }
      const uint32_t x = wave_scan_incl_u32(loc);
      if (lane == 63) DSA_CHECK(x == (uint32_t)kk, x, kk);  // exactly kk keys >= prefix
      uint32_t run = x - loc;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        s_col[lane * PER + q] = run;
        run += v[q];
      }
    }
    __syncthreads();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const bool take = kreg[j] != 0ull && kreg[j] >= prefix;
      const uint64_t bal = __ballot(take);
      if (take) {
        const uint32_t pos = s_col[j * NW + wave] + (uint32_t)__popcll(bal & lt_mask);
        if (pos < (uint32_t)kMaxK) sel[pos] = kreg[j];
      }
    }
  } else {
    // many candidates (ties or a flat row): the same steps streaming from memory
    for (int pass = 1; pass < 6 && !done; ++pass) {
      const int shift = digit_shift(pass);
      const uint32_t dmask = digit_mask(pass);
      for (int i = tid; i < kBins; i += NT) hist[i] = 0;
      __syncthreads();
      for (int g = tid; g < C; g += NT) {
        const uint64_t key = cand[slot(g)];
        if ((key & mask) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & dmask], 1u);
      }
      __syncthreads();
      pick_digit<NT>(hist, s_red, krem, tid, lane, wave, &s_krem, &s_done, &s_digit);
      __syncthreads();
      prefix |= (uint64_t)s_digit << shift;
      mask |= (uint64_t)dmask << shift;
      krem = s_krem;
      done = s_done != 0;
    }
    uint32_t base = 0;
    for (int g0 = 0; g0 < C; g0 += NT) {
      const int g = g0 + tid;
      const uint64_t key = g < C ? cand[slot(g)] : 0ull;
      const bool take = key != 0ull && key >= prefix;
      const uint32_t x = wave_scan_incl_u32((uint32_t)take);
      if (lane == 63) s_red[wave] = x;
      __syncthreads();
      uint32_t before = 0, all = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if (w < wave) before += s_red[w];
        all += s_red[w];
      }
      const uint32_t pos = base + before + x - (uint32_t)take;
      if (take && pos < (uint32_t)kMaxK) sel[pos] = key;
      base += all;
      __syncthreads();
    }
    if (tid == 0) DSA_CHECK(base == (uint32_t)kk, base, kk);
  }
  __syncthreads();
  int32_t* orow = out + row * (int64_t)k;
  if (order != 0) {  // the compacted list: position order, -1 slots last
    for (int i = tid; i < k; i += NT)
      orow[i] = (i < kk) ? (int32_t)(0xFFFFFFFFu - (uint32_t)sel[i]) : -1;
    return;
  }
  sort_store<NT, kMaxK / NT>(sel, kk, k, orow);
}

// the histogram-threshold path: few rows (every stage of the segmented path
// would run fewer than 256 workgroups) of more than one segment
bool use_row_path(int64_t rows, int T) {
  if (T <= kSegLen) return false;
  const int64_t nseg = ((int64_t)T + kSegLen - 1) / kSegLen;
  const int64_t nc = ((int64_t)T + kRowChunk - 1) / kRowChunk;
  return rows * nseg < 256 && nc <= kRowMaxChunks;
}

size_t row_path_bytes(int64_t rows, int T) {
  const int64_t nc = ((int64_t)T + kRowChunk - 1) / kRowChunk;
  // candidates (one chunk's worth of slots per chunk), histograms, counts
  return (size_t)rows * nc * kRowChunk * sizeof(uint64_t) +
         (size_t)rows * kRowHistCopies * kBins * 4 + (size_t)rows * nc * 4;
}

hipError_t launch_row_path(const float* scores, int32_t* indices, int64_t rows, int T, int k,
                           void* workspace, hipStream_t st, int order, int S, int P) {
  const int nc = (int)(((int64_t)T + kRowChunk - 1) / kRowChunk);
  uint64_t* cand = (uint64_t*)workspace;
  uint32_t* ghist = (uint32_t*)(cand + rows * nc * (int64_t)kRowChunk);
  uint32_t* cnt = ghist + rows * kRowHistCopies * kBins;
  const int nh = (int)(rows * kRowHistCopies * kBins);
  hipLaunchKernelGGL(row_hist_zero_kernel, dim3((nh + 255) / 256), dim3(256), 0, st, ghist, nh);
  hipLaunchKernelGGL(row_hist_kernel, dim3((unsigned)(rows * nc)), dim3(256), 0, st, scores, ghist,
                     T, nc, S, P);
  hipLaunchKernelGGL(row_filter_kernel, dim3((unsigned)(rows * nc)), dim3(256), 0, st, scores,
                     ghist, cand, cnt, T, nc, k, S, P);
  hipLaunchKernelGGL(row_select_kernel, dim3((unsigned)rows), dim3(1024), 0, st, cand, cnt, ghist,
                     indices, nc, k, order);
  return hipGetLastError();
}

}  // namespace

#ifdef DSA_DEBUG
DSA_DEBUG_TAKE(topk)
#endif

size_t topk_workspace_bytes(int B, int S, int T, int topk) {
  if (T <= kSegLen) return 0;
  const int64_t rows = (int64_t)B * S;
  if (use_row_path(rows, T)) return row_path_bytes(rows, T);
  int groups[8];
  const int lv = stage_groups(T, topk, groups, 8);
  // two ping-pong candidate buffers: the first stage output and the largest later one
  const int64_t a = rows * groups[0] * (int64_t)topk;
  const int64_t b = lv > 1 ? rows * groups[1] * (int64_t)topk : 0;
  return (size_t)(a + b) * sizeof(uint64_t);
}

hipError_t launch_topk(const float* scores, int32_t* indices, int B, int S, int T, int topk,
                       void* workspace, hipStream_t st, int order, int causal_P) {
  const int64_t rows = (int64_t)B * S;
  if (T <= kSegLen) {  // one register-resident workgroup per row
    if (T <= 4096)
      return launch_stage<0, 0, 4096>(scores, indices, nullptr, rows, T, topk, T, 1, st, order, S,
                                      causal_P);
    return launch_stage<0, 0, kSegLen>(scores, indices, nullptr, rows, T, topk, T, 1, st, order, S,
                                       causal_P);
  }
  if (use_row_path(rows, T))
    return launch_row_path(scores, indices, rows, T, topk, workspace, st, order, S, causal_P);
  int groups[8];
  const int lv = stage_groups(T, topk, groups, 8);
  uint64_t* bufa = (uint64_t*)workspace;
  uint64_t* bufb = bufa + rows * groups[0] * (int64_t)topk;
  if (rows * groups[0] > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  // stage 1: k candidate keys per 16384-score segment
  hipError_t e = launch_stage<0, 1, kSegLen>(scores, nullptr, bufa, rows * groups[0], T, topk,
                                             kSegLen, groups[0], st, 0, S, causal_P);
  if (e != hipSuccess) return e;
  // candidate reductions: groups of kCand candidates -> k each
  int C = groups[0] * topk;
  uint64_t *in = bufa, *outb = bufb;
  for (int l = 1; l < lv; ++l) {
    e = launch_stage<1, 1, kCand>(in, nullptr, outb, rows * groups[l], C, topk, kCand, groups[l], st);
    if (e != hipSuccess) return e;
    C = groups[l] * topk;
    uint64_t* tmp = in;
    in = outb;
    outb = tmp;
  }
  // final selection and sort among at most kCand candidates per row (rows of
  // two segments have at most 4096: 16 per thread of a 256-thread workgroup)
  if (C <= 4096) return launch_stage<1, 0, 4096>(in, indices, nullptr, rows, C, topk, C, 1, st, order);
  return launch_stage<1, 0, kCand>(in, indices, nullptr, rows, C, topk, C, 1, st, order);
}

}  // namespace dsa
