// index_scores.hip -- lightning-indexer scores with causal mask (gfx950).
//
// score[b,s,t] = sum_h w[b,s,h] * relu(scale * q[b,s,h,:] . k[b,t,:]) for
// t <= p = past_len + s, -inf above (A.X-K2 page, "Sparse Gated Attention":
// per-head products with the shared index key, weighted head sum, ReLU,
// causal upper-triangle mask).
//
// The index key is shared by all index heads, so it is the stationary MFMA
// operand: each wave keeps 128 keys of k in registers and streams the
// per-head query operands through the bf16 MFMA, one K = idx_dim product per
// head followed by the per-head ReLU and weighted accumulation in fp32.
// Scores are produced transposed (keys on the MFMA M axis) so that each lane
// owns one query column: the head weight is then a per-lane scalar.
//
// Kernels
//  idx_tile_kernel   prefill tiles of 16 (or 32) queries x 512 keys, 4 waves,
//                    each wave 128 keys x the tile's queries with its keys
//                    held in registers and the queries' operands shared
//                    through LDS;
//                    only tiles on or below the causal diagonal are launched,
//                    paired (j, last-j) so every pair costs the same, pairs
//                    dealt to XCDs round-robin.
//  idx_rows_dma_kernel  few-query calls (decode) with up to 64 index heads:
//                    the index heads become the MFMA M axis; a wave streams 128
//                    or 512 keys of k in blocks of 32 through a two-slot LDS
//                    ring filled by LDS-DMA, each copy instruction reading 1 KB
//                    of whole key rows (32-byte pieces of 32 rows, as register
//                    loads in the operand layout take them, streamed at about
//                    4 TB/s; whole rows, swizzled in LDS for conflict-free
//                    operand reads, at about 5.8).
//  idx_rows_kernel   the same products with the keys loaded into registers
//                    one block ahead (more than 64 heads: their operands then
//                    need the register file at one wave per SIMD).
//  idx_f32_kernel    fp32 inputs: plain fp32 loops (parity-size workloads).
#include "common.h"
#include "idx_tiles.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kWaveK = 128;            // keys per wave (8 MFMA M blocks of 16)
constexpr int kTileK = 4 * kWaveK;     // keys per workgroup
static_assert(kTileK == kIdxTileK, "tile schedule");
constexpr int kStageBytes = 16384;     // query operands staged in LDS per step

// One workgroup = 16 QG queries x 512 keys; wave w keeps keys 128w..128w+127
// of the tile in registers as 16x16x32 MFMA A operands for the whole kernel,
// and multiplies them with QG groups of 16 queries in turn (QG = 2 halves the
// key loads per score where the per-score work is light).
// The queries' per-head operands are shared by the four waves: they are
// copied global -> LDS by the LDS-DMA path (no register staging), one stage
// of G heads at a time, double-buffered so that stage g+1 lands while stage
// g is multiplied. The LDS image of a stage is laid out exactly in operand
// lane order (1 KB per head, 32-dim step and 16-query group), so each B
// operand is one conflict-free 16-byte read per lane.
template <int DI, int QG, int MODE>
__global__ __launch_bounds__(256, 2) void idx_tile_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ w,
                                                          float* __restrict__ scores, int S,
                                                          int T, int P, int HI, float scale,
                                                          int nqt, int nkt, int npairs,
                                                          int maxlen, int two, int fill) {
  constexpr int kQG = QG;
  constexpr int kTileQ = 16 * QG;                      // queries per workgroup (MFMA N axis)
  constexpr int KS = DI / 32;                          // 32-dim steps per head
  constexpr int G = kStageBytes / (kTileQ * DI * 2);   // heads per stage
  static_assert(G * KS * kQG == 16, "a stage is 16 one-KB operand blocks, 4 per wave");
  __shared__ __attribute__((aligned(16))) uint8_t qs[2][kStageBytes];

  const int b = blockIdx.y;
  IdxTile2 tile;
  if (!idx_tile2_of(blockIdx.x, kTileQ, S, P, nqt, nkt, npairs, maxlen, two != 0, &tile)) return;
  const int kt = tile.kt;
  DSA_CHECK(tile.q1 >= 0 && tile.q1 < nqt && kt >= 0 && kt < nkt, tile.q1, kt);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int lq = lane & 15, lg = lane >> 4;
  const int kw0 = kt * kTileK + wave * kWaveK;  // first key of this wave
  // the query tile being multiplied: q1, then q2 with the same key registers
  int qt = tile.q1;
  int q0 = qt * kTileQ;
  int64_t row[kQG];  // this lane's query row of each group (clamped to S-1)
#pragma unroll
  for (int qg = 0; qg < kQG; ++qg) row[qg] = (int64_t)b * S + min(q0 + 16 * qg + lq, S - 1);
  // waves whose keys all lie above the tile's last query skip the products
  // (q1's causal range covers q2's, so q1 decides the key loads)
  bool active = kw0 <= P + min(q0 + kTileQ, S) - 1;

  bf16x8_t a[8][KS];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    const int t = kw0 + 16 * kb + lq;
    const uint16_t* kp = k + ((int64_t)b * T + (t < T ? t : T - 1)) * DI + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t v = u32x4_t{0, 0, 0, 0};
      if (active && t < T) v = load16(kp + 32 * ks);
      a[kb][ks] = as_bf16x8(v);
    }
  }

  // operand block n of a stage = (head n / (KS kQG), dims 32((n / kQG) % KS)
  // + 8 lg .. +8, query group n % kQG) of query lq; wave w copies 4w..4w+3
  const int nst = (HI + G - 1) / G;
  auto issue_stage = [&](int st, int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int blk = 4 * wave + r;
      const int qg = blk % kQG, ks = (blk / kQG) % KS;
      // heads past HI copy the last head (finite operands for the zero
      // weight they get), so every stage runs G heads without branches
      const int h = min(st * G + blk / (KS * kQG), HI - 1);
      const uint16_t* src = q + (row[qg] * HI + h) * DI + 32 * ks + 8 * lg;
      __builtin_amdgcn_global_load_lds(
          (const void*)src, (__attribute__((address_space(3))) void*)(&qs[buf][blk * 1024]), 16, 0,
          0);
    }
  };
  // head weights of the next stage as raw bf16 bits (heads past HI read the
  // last head's), converted and masked only when their stage runs so that
  // nothing waits on these loads before then
  uint16_t wn[kQG][G];
  auto load_weights = [&](int st) {
#pragma unroll
    for (int qg = 0; qg < kQG; ++qg)
#pragma unroll
      for (int g = 0; g < G; ++g) wn[qg][g] = w[row[qg] * HI + min(st * G + g, HI - 1)];
  };

  const bool vec = (T & 3) == 0;
  f32x4_t sc[kQG][8];
  for (int tl = 0; tl < (tile.q2 >= 0 ? 2 : 1); ++tl) {
  if (tl == 1) {  // the pair's earlier query tile with the same key registers
    qt = tile.q2;
    q0 = qt * kTileQ;
#pragma unroll
    for (int qg = 0; qg < kQG; ++qg) row[qg] = (int64_t)b * S + min(q0 + 16 * qg + lq, S - 1);
    active = kw0 <= P + min(q0 + kTileQ, S) - 1;
    __syncthreads();  // every wave is done with the previous tile's last stage buffer
  }
#pragma unroll
  for (int qg = 0; qg < kQG; ++qg)
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) sc[qg][kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  issue_stage(0, 0);
  load_weights(0);
  for (int st = 0; st < nst; ++st) {
    uint16_t wc[kQG][G];
#pragma unroll
    for (int qg = 0; qg < kQG; ++qg)
#pragma unroll
      for (int g = 0; g < G; ++g) wc[qg][g] = wn[qg][g];
    // stage st has landed (each wave drains its own copies, vmcnt(0), before
    // the barrier) and every wave is done with the buffer stage st+1 overwrites
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    const int buf = st & 1;
    if (st + 1 < nst) {
      issue_stage(st + 1, buf ^ 1);
      load_weights(st + 1);
    }
    if (active) {
      // B operands of one (head, query group) of the stage; the next pair's
      // are read from LDS while the current pair is multiplied
      auto read_ops = [&](int gq, bf16x8_t* dst) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          dst[ks] = as_bf16x8(*(const u32x4_t*)(
              &qs[buf][(((gq / kQG) * KS + ks) * kQG + gq % kQG) * 1024 + 16 * lane]));
      };
      bf16x8_t bqn[KS];
      read_ops(0, bqn);
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int qg = 0; qg < kQG; ++qg) {
          bf16x8_t bq[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) bq[ks] = bqn[ks];
          if (g * kQG + qg + 1 < G * kQG) read_ops(g * kQG + qg + 1, bqn);
          f32x4_t acc[8];
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) acc[kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
          // raised issue priority for the MFMA burst, so that the other wave
          // of the SIMD fills it with its ReLU/weight work (dsa-s32k about 1%)
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) acc[kb] = mfma16x16x32(a[kb][ks], bq[ks], acc[kb]);
          __builtin_amdgcn_s_setprio(0);
          const float wh = (st * G + g < HI) ? bf16_to_f32(wc[qg][g]) * scale : 0.0f;
#pragma unroll
          for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x = acc[kb][e];
              if (MODE == 0) x = relu_bits(x);
              sc[qg][kb][e] = fmaf(wh, x, sc[qg][kb][e]);
            }
        }
      }
    }
  }

  // lane (lq, lg) holds keys kw0 + 16 kb + 4 lg + e of query q0 + 16 qg + lq
#pragma unroll
  for (int qg = 0; qg < kQG; ++qg) {
    const int s = q0 + 16 * qg + lq;
    if (s >= S) continue;
    const int p = P + s;
    float* orow = scores + ((int64_t)b * S + s) * T;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const int t0 = kw0 + 16 * kb + 4 * lg;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = sc[qg][kb][e];
        if (MODE == 2) x = relu_bits(x);
        v[e] = (t0 + e <= p) ? x : -INFINITY;
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
  }  // query tiles
  if (fill) idx_fill_upper2<kTileQ>(scores, tile, b, S, T, nkt, vec);
}

// Few queries per call: MFMA M = index heads (NHB blocks of 32), N = 32 keys.
// A wave streams KPW keys in blocks of 32; the query operand is loaded
// once per wave and the next block's keys are loaded during the current
// block's MFMAs.
// KPW keys per wave: 512 where that still gives 2048 waves (fewer per-wave
// query loads), else 128 so that more waves stream the keys. Measured on
// one 528385-key row (32 heads): 512 keys 35.9 us, 256 32.0, 128 29.7; on
// 8 rows of 131072 (64 heads): 512 48.8 us, 256 54.2, 128 64.9.
constexpr int kRowsWaves = 2048;
template <int DI, int NHB, int MODE, int KPW>
__global__ __launch_bounds__(256) void idx_rows_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ w,
                                                       float* __restrict__ scores, int S, int T,
                                                       int P, int HI, float scale, int fill) {
  constexpr int KS = DI / 16;
  constexpr int NB = KPW / 32;
  const int64_t row = blockIdx.y;
  const int b = (int)(row / S), s = (int)(row % S);
  const int p = P + s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 31, lh = lane >> 5;
  const int tbase = (blockIdx.x * 4 + wave) * KPW;
  DSA_CHECK(p < T, p, T);  // the query's own key exists
  float* orow = scores + row * T;
  if (tbase >= T) return;

  if (tbase > p) {  // the whole wave is above the diagonal
    for (int kb = 0; kb < NB && fill; ++kb) {
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
          if (MODE == 0) x = relu_bits(x);
          part = fmaf(wv[hb][e], x, part);
        }
      }
      part = sum_other_half(part);
      if (MODE == 2) part = relu_bits(part);
    }
    if (lh == 0 && t < T) orow[t] = (t <= p) ? part : -INFINITY;
    if (more) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bk[ks] = bn[ks];
    }
  }
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// The KS B operands of one 32-key ring slot: operand ks of lane (ln, lh) is
// chunk 2 ks + lh of key ln, found at ln CH 16 + 16 ((2 ks + lh) ^ (ln % CH))
// (the slot layout of idx_rows_dma_kernel). The reads are issued and waited for
// in one asm statement: the slot was filled by LDS-DMA, whose completion the
// caller has already awaited with an exact vmcnt, and an LDS read the compiler
// can see would make it wait for every copy still in flight instead. Waiting
// inside the statement leaves no read in flight behind the compiler's back.
#define DSA_RB_READ(d, a) "ds_read_b128 %" #d ", %" #a "\n\t"
template <int KS, int CH>
__device__ __forceinline__ void read_block(const uint8_t* slot, int ln, int lh,
                                           bf16x8_t (&o)[KS]) {
  const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)slot +
                        (uint32_t)(ln * CH * 16);
  uint32_t a[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) a[ks] = base + 16u * (uint32_t)((2 * ks + lh) ^ (ln % CH));
  // outputs early-clobber: no result may land in an address not yet used
  u32x4_t r[KS];
  if constexpr (KS == 8) {
    asm volatile(DSA_RB_READ(0, 8) DSA_RB_READ(1, 9) DSA_RB_READ(2, 10) DSA_RB_READ(3, 11)
                     DSA_RB_READ(4, 12) DSA_RB_READ(5, 13) DSA_RB_READ(6, 14)
                         DSA_RB_READ(7, 15) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
                   "=&v"(r[6]), "=&v"(r[7])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
                   "v"(a[7])
                 : "memory");
  } else if constexpr (KS == 4) {
    asm volatile(DSA_RB_READ(0, 4) DSA_RB_READ(1, 5) DSA_RB_READ(2, 6) DSA_RB_READ(3, 7)
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                 : "memory");
  } else {
    static_assert(KS == 2, "idx_dim 32, 64 or 128");
    asm volatile(DSA_RB_READ(0, 2) DSA_RB_READ(1, 3) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1])
                 : "v"(a[0]), "v"(a[1])
                 : "memory");
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) o[ks] = as_bf16x8(r[ks]);
}
#undef DSA_RB_READ

// Few queries per call, the keys streamed through LDS: the products of
// idx_rows_kernel (same operands, same MFMA order, the same bits out), but a
// wave's keys arrive by LDS-DMA into a ring of two 32-key blocks, so that two
// blocks per wave are in flight while one is multiplied (the register form
// holds one), and its scores are kept in registers and stored at the end, so
// that the loop's only vector-memory operations are the block copies and
// vmcnt counts blocks exactly. The two slots are separate LDS arrays indexed
// statically (the loop is unrolled), which lets the compiler tell a slot
// being copied into from the one being read.
template <int DI, int NHB, int MODE, int KPW>
__global__ __launch_bounds__(256, 2) void idx_rows_dma_kernel(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ w,
                                                              float* __restrict__ scores, int S,
                                                              int T, int P, int HI, float scale,
                                                              int fill) {
  constexpr int KS = DI / 16;  // 1 KB copies per block (32 keys x 16 dims x 2 bytes)
  constexpr int CH = DI / 8;   // 16-byte chunks per key row
  constexpr int NB = KPW / 32;
  static_assert(NB >= 2, "two blocks in flight");
  __shared__ __attribute__((aligned(16))) uint8_t ring0[4][KS * 1024];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[4][KS * 1024];
  const int64_t row = blockIdx.y;
  const int b = (int)(row / S), s = (int)(row % S);
  const int p = P + s;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 31, lh = lane >> 5;
  const int tbase = (blockIdx.x * 4 + wave) * KPW;
  DSA_CHECK(p < T, p, T);  // the query's own key exists
  float* orow = scores + row * T;
  if (tbase >= T) return;

  if (tbase > p) {  // the whole wave is above the diagonal
    for (int kb = 0; kb < NB && fill; ++kb) {
      const int t = tbase + 32 * kb + ln;
      if (lh == 0 && t < T) orow[t] = -INFINITY;
    }
    return;
  }
  // blocks holding a key t <= p (every key of the others is masked)
  const int nv = min(NB, (p - tbase) / 32 + 1);
  DSA_CHECK(nv >= 1 && tbase + 32 * (nv - 1) <= p, nv, tbase);

  // A slot holds its 32 keys row-major (CH 16-byte chunks per key), chunk c
  // of key r in place c ^ (r % CH). Copy i brings rows 64/CH i .. : lane L
  // fills place L % CH of row 64/CH i + L / CH, i.e. chunk (L % CH) ^ (row %
  // CH), so every copy reads 1 KB of whole key rows (the lanes' 16-byte pieces
  // permuted within each row). Keys past the bound are clamped to p (masked at
  // the store).
  auto issue = [&](int kb) {
    uint8_t* dst = (kb & 1) ? &ring1[wave][0] : &ring0[wave][0];
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int r = i * (64 / CH) + lane / CH;
      const int t = min(tbase + 32 * kb + r, p);
      const int c = (lane % CH) ^ (r % CH);
      __builtin_amdgcn_global_load_lds(
          (const void*)(k + ((int64_t)b * T + t) * DI + 8 * c),
          (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16, 0, 0);
    }
  };

  // the first two blocks' copies go out before the query and weight loads
  const bool full = nv == NB;
  issue(0);
  if (full) issue(1);

  // query operands and head weights: every load issued unconditionally (heads
  // past HI read the last head's and are zeroed after), all in flight together
  // and converted only after the scheduling barrier, so one wait covers them
  u32x4_t qr[NHB][KS];
  uint16_t wr[NHB][16];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int hh = 32 * hb + ln;
    const uint16_t* qp = q + (row * HI + (hh < HI ? hh : HI - 1)) * DI + 8 * lh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qr[hb][ks] = load16(qp + 16 * ks);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = 32 * hb + 8 * (e >> 2) + 4 * lh + (e & 3);
      wr[hb][e] = w[row * HI + (m < HI ? m : HI - 1)];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  bf16x8_t a[NHB][KS];
  float wv[NHB][16];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const bool hv = 32 * hb + ln < HI;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a[hb][ks] = as_bf16x8(hv ? qr[hb][ks] : u32x4_t{0, 0, 0, 0});
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = 32 * hb + 8 * (e >> 2) + 4 * lh + (e & 3);
      const float x = bf16_to_f32(wr[hb][e]) * scale;
      wv[hb][e] = m < HI ? x : 0.0f;
    }
  }
  // the products of one block: the weighted head sum of its 32 keys
  auto block_scores = [&](const bf16x8_t (&bk)[KS]) {
    float part = 0.0f;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      f32x16_t acc = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma32x32x16(a[hb][ks], bk[ks], acc);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = acc[e];
        if (MODE == 0) x = relu_bits(x);
        part = fmaf(wv[hb][e], x, part);
      }
    }
    part = sum_other_half(part);
    if (MODE == 2) part = relu_bits(part);
    return part;
  };

  float res[NB];
  if (full) {
    // every block holds a visible key (all waves of a row but the one holding
    // its bound): a branch-free pipeline, so every wait count is exact
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      // block kb has landed once only the copies issued after it (those of
      // block kb + 1, when there is one) are outstanding
      if (kb + 1 < NB)
        wait_vmcnt<KS>();
      else
        wait_vmcnt<0>();
      bf16x8_t bk[KS];
      read_block<KS, CH>((kb & 1) ? &ring1[wave][0] : &ring0[wave][0], ln, lh, bk);
      if (kb + 2 < NB) issue(kb + 2);  // the slot's reads completed inside read_block
      res[kb] = block_scores(bk);
    }
  } else {
    // the wave holding the bound: one block at a time
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      res[kb] = 0.0f;
      if (kb < nv) {
        if (kb > 0) issue(kb);  // (block 0 was issued above)
        wait_vmcnt<0>();
        bf16x8_t bk[KS];
        read_block<KS, CH>((kb & 1) ? &ring1[wave][0] : &ring0[wave][0], ln, lh, bk);
        res[kb] = block_scores(bk);
      }
    }
  }
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) {
    const int t = tbase + 32 * kb + ln;
    if (lh == 0 && t < T) orow[t] = (t <= p) ? res[kb] : -INFINITY;
  }
}

// fp32 inputs: one thread per (row, key), plain loops in fp32.
__global__ __launch_bounds__(256) void idx_f32_kernel(const float* __restrict__ q,
                                                      const float* __restrict__ k,
                                                      const float* __restrict__ w,
                                                      float* __restrict__ scores, int S, int T,
                                                      int P, int HI, int DI, float scale,
                                                      int mode, int fill) {
  const int64_t row = blockIdx.y;
  const int b = (int)(row / S), s = (int)(row % S);
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  float* out = scores + row * T + t;
  if (t > P + s) {
    if (fill) *out = -INFINITY;
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

template <int DI, int QG, int MODE>
hipError_t launch_tiles(const uint16_t* q, const uint16_t* k, const uint16_t* w, float* scores,
                        int B, int S, int T, int P, int HI, float scale, int fill, hipStream_t st) {
  // Long contexts (many key tiles per query tile) share each key tile between
  // the pair's two query tiles. Measured with one 4096-query chunk after
  // 524288 keys (32 heads): 14.97 -> 13.97 ms; at S = T (32768 and 4096) it
  // gained nothing or lost 7%, so those keep one unit per workgroup.
  const bool two = (int64_t)T >= 8 * (int64_t)S;
  const IdxGrid g = idx_grid2(S, T, P, 16 * QG, two);
  if (g.gx > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((idx_tile_kernel<DI, QG, MODE>), dim3((unsigned)g.gx, B), dim3(256), 0, st, q,
                     k, w, scores, S, T, P, HI, scale, g.nqt, g.nkt, g.npairs, g.maxlen,
                     two ? 1 : 0, fill);
  return hipGetLastError();
}

template <int DI, int NHB, int MODE>
hipError_t launch_rows(const uint16_t* q, const uint16_t* k, const uint16_t* w, float* scores,
                       int B, int S, int T, int P, int HI, float scale, int fill, hipStream_t st) {
  const int64_t rows = (int64_t)B * S;
  auto waves = [&](int kpw) { return rows * ((T + kpw - 1) / kpw); };
  // up to 64 heads the keys stream through LDS (idx_rows_dma_kernel); more
  // heads keep their operands in registers at one wave per SIMD
#define DSA_ROWS_LAUNCH(KPW)                                                                     \
  if constexpr (NHB <= 2)                                                                        \
    hipLaunchKernelGGL((idx_rows_dma_kernel<DI, NHB, MODE, KPW>),                                \
                       dim3((T + 4 * KPW - 1) / (4 * KPW), (unsigned)rows), dim3(256), 0, st, q, \
                       k, w, scores, S, T, P, HI, scale, fill);                                  \
  else                                                                                           \
    hipLaunchKernelGGL((idx_rows_kernel<DI, NHB, MODE, KPW>), dim3((T + 4 * KPW - 1) / (4 * KPW), \
                       (unsigned)rows), dim3(256), 0, st, q, k, w, scores, S, T, P, HI, scale, fill)
  if (waves(512) >= kRowsWaves)
    DSA_ROWS_LAUNCH(512);
  else
    DSA_ROWS_LAUNCH(128);
#undef DSA_ROWS_LAUNCH
  return hipGetLastError();
}

template <int DI, int MODE>
hipError_t dispatch_rows(const uint16_t* q, const uint16_t* k, const uint16_t* w, float* scores,
                         int B, int S, int T, int P, int HI, float scale, int fill, hipStream_t st) {
  const int nhb = (HI + 31) / 32;
  switch (nhb) {
    case 1: return launch_rows<DI, 1, MODE>(q, k, w, scores, B, S, T, P, HI, scale, fill, st);
    case 2: return launch_rows<DI, 2, MODE>(q, k, w, scores, B, S, T, P, HI, scale, fill, st);
    case 3: return launch_rows<DI, 3, MODE>(q, k, w, scores, B, S, T, P, HI, scale, fill, st);
    default: return launch_rows<DI, 4, MODE>(q, k, w, scores, B, S, T, P, HI, scale, fill, st);
  }
}

template <int MODE>
hipError_t dispatch_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* w, float* scores,
                         int B, int S, int T, int P, int HI, int DI, float scale, int fill,
                         hipStream_t st) {
  // few queries per sequence and at most 128 index heads: head-major MFMA
  const bool rows = S < 32 && HI <= 128 && (int64_t)B * S <= 65535;
  if (rows) {
    switch (DI) {
      case 32: return dispatch_rows<32, MODE>(q, k, w, scores, B, S, T, P, HI, scale, fill, st);
      case 64: return dispatch_rows<64, MODE>(q, k, w, scores, B, S, T, P, HI, scale, fill, st);
      default: return dispatch_rows<128, MODE>(q, k, w, scores, B, S, T, P, HI, scale, fill, st);
    }
  }
  // Light per-score work (few index heads x small dim): two 16-query groups
  // per workgroup share each wave's key registers. Measured: 24 -> 22 us at
  // 4 heads x 64 (4096 x 4096); 3% slower at 64 heads x 128, where the
  // products dominate. (At dim 128 two groups' operands exceed the register
  // budget, so that dim always runs one group.)
  if (HI * DI <= 512 && DI <= 64) {
    switch (DI) {
      case 32: return launch_tiles<32, 2, MODE>(q, k, w, scores, B, S, T, P, HI, scale, fill, st);
      default: return launch_tiles<64, 2, MODE>(q, k, w, scores, B, S, T, P, HI, scale, fill, st);
    }
  }
  switch (DI) {
    case 32: return launch_tiles<32, 1, MODE>(q, k, w, scores, B, S, T, P, HI, scale, fill, st);
    case 64: return launch_tiles<64, 1, MODE>(q, k, w, scores, B, S, T, P, HI, scale, fill, st);
    default: return launch_tiles<128, 1, MODE>(q, k, w, scores, B, S, T, P, HI, scale, fill, st);
  }
}

}  // namespace

#ifdef DSA_DEBUG
DSA_DEBUG_TAKE(index_scores)
#endif

hipError_t launch_index_scores(const void* q_idx, const void* k_idx, const void* w, float* scores,
                               int B, int S, int T, int past_len, int HI, int DI, float scale,
                               int relu_mode, int dtype, hipStream_t stream, bool fill_masked) {
  const int fill = fill_masked ? 1 : 0;
  if (dtype == 0) {
    hipLaunchKernelGGL(idx_f32_kernel, dim3((T + 255) / 256, B * S), dim3(256), 0, stream,
                       (const float*)q_idx, (const float*)k_idx, (const float*)w, scores, S, T,
                       past_len, HI, DI, scale, relu_mode, fill);
    return hipGetLastError();
  }
  const uint16_t* q = (const uint16_t*)q_idx;
  const uint16_t* k = (const uint16_t*)k_idx;
  const uint16_t* ww = (const uint16_t*)w;
  switch (relu_mode) {
    case 0: return dispatch_bf16<0>(q, k, ww, scores, B, S, T, past_len, HI, DI, scale, fill, stream);
    case 1: return dispatch_bf16<1>(q, k, ww, scores, B, S, T, past_len, HI, DI, scale, fill, stream);
    default: return dispatch_bf16<2>(q, k, ww, scores, B, S, T, past_len, HI, DI, scale, fill, stream);
  }
}

}  // namespace dsa
