// attn_prefill.hip -- sparse (or sliding-window) MLA attention for many
// queries at once, bf16 MFMA on gfx950.
//
// DSA: each query attends only to its selected, causally visible keys; the
// selection acts as an additive 0/-inf mask on the attention logits (A.X-K2
// page, "MLA + explicit sparse mask", steps 4-5), followed by the sigmoid
// output gate (same page, "Attention output gate"; Spark-X2.5 page, forward
// pass steps 2-3). SWA: the mask is the window p-W+1 .. p instead (Spark-X2.5
// page: sliding_window 512; openPangu-2.0 page §3.2).
//
// Cost structure. The caches hold expanded per-head K/V and selections are
// per query, so gathering selected rows per query is a ~1 flop/byte stream.
// Dense flash tiles over the causal range, masked by a per-query selection
// bitmap, run at MFMA rate instead; every unselected logit is -inf and
// contributes exactly 0, so the result is the masked softmax itself.
//
// Layout of the work. One workgroup = one head, 128 queries (32 per wave).
// Logits are produced transposed, S^T = K Q^T (keys on the MFMA M axis), so a
// lane owns one query column: the softmax max/sum stay in registers except
// for one swap with the other half-wave. The 32x32 accumulator layout then
// holds keys {8g + 4*half + r}; the P.V product uses exactly that key order
// as its contraction index, so P never leaves registers: V stays row-major in
// LDS and its operand is read with gfx950's transposing LDS load, four keys
// per read, in that key order. Q^T stays in registers for the whole key loop.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kBQ = 128;  // queries per workgroup (32 per wave)
constexpr int kBN = 64;   // keys per step
constexpr float kLazyLog2 = 8.0f;  // largest exponent of an unnormalised weight p

// --------------------------------------------------------- selection bitmap
// bitmap[(b*S + s) * W32 + w] bit j  <=>  key 32w + j is selected and t <= p.
__global__ __launch_bounds__(256) void bitmap_lds_kernel(const int32_t* __restrict__ idx,
                                                         uint32_t* __restrict__ bm, int S, int T,
                                                         int P, int topk, int W32) {
  extern __shared__ uint32_t sbits[];
  const int64_t row = blockIdx.x;
  const int p = P + (int)(row % S);
  if (threadIdx.x == 0) DSA_CHECK(p < T && (int64_t)W32 * 32 >= T, p, T);  // the query's row exists
  for (int i = threadIdx.x; i < W32; i += blockDim.x) sbits[i] = 0;
  __syncthreads();
  const int32_t* ir = idx + row * topk;
  for (int j = threadIdx.x; j < topk; j += blockDim.x) {
    const int t = ir[j];
    if (t >= 0 && t <= p && t < T) atomicOr(&sbits[t >> 5], 1u << (t & 31));
  }
  __syncthreads();
  uint32_t* br = bm + row * W32;
  for (int i = threadIdx.x; i < W32; i += blockDim.x) br[i] = sbits[i];
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

__global__ __launch_bounds__(256) void bitmap_global_kernel(const int32_t* __restrict__ idx,
                                                            uint32_t* __restrict__ bm, int S,
                                                            int T, int P, int topk, int W32) {
  const int64_t row = blockIdx.x;
  const int p = P + (int)(row % S);
  const int32_t* ir = idx + row * topk;
  uint32_t* br = bm + row * W32;
  for (int j = threadIdx.x; j < topk; j += blockDim.x) {
    const int t = ir[j];
    if (t >= 0 && t <= p && t < T) atomicOr(&br[t >> 5], 1u << (t & 31));
  }
}

// Swizzle of the row-major V tile (rows of DV bf16 = VCH 16-byte chunks):
// chunk c of key row r is stored at chunk c ^ vt_xor(r). A transposing read
// covers four consecutive rows x 64 bytes per half-wave; the XOR moves those
// four row pieces into four different 16-bank groups (rows of 256 bytes all
// start at bank 0, rows of 128 bytes at bank 0 or 32).
template <int VCH>
__device__ __forceinline__ int vt_xor(int row) {
  return VCH >= 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// Buffer-row range [jlo, jhi] (64-aligned start) of the keys a 128-query tile
// can see: the causal range for the bitmap mask, the window range otherwise.
__host__ __device__ __forceinline__ void tile_range(int qt, int S, int P, int Tbuf, int kv_offset,
                                                    int window, int* jlo, int* jhi) {
  const int q0 = qt * kBQ;
  const int pmax = P + min(q0 + kBQ - 1, S - 1);
  int tlo = 0;
  if (window > 0) tlo = max(kv_offset, P + q0 - window + 1);
  *jlo = ((tlo - kv_offset) / kBN) * kBN;
  *jhi = min(pmax - kv_offset, Tbuf - 1);
}

__host__ __device__ __forceinline__ int tile_blocks(int qt, int S, int P, int Tbuf, int kv_offset,
                                                     int window) {
  int jlo, jhi;
  tile_range(qt, S, P, Tbuf, kv_offset, window, &jlo, &jhi);
  return jhi >= jlo ? (jhi - jlo) / kBN + 1 : 0;
}

// Work items run from the longest query tile down. When long tiles are split
// (at most M key blocks per item), start[o] is the first item of the o-th
// longest tile (tile nqt-1-o) and start[nqt] the item count; the table is
// built on the host and passed by value, so no kernel walks the tiles.
constexpr int kMaxSplitTiles = 128;  // calls with more query tiles never split
struct SplitTable {
  int start[kMaxSplitTiles + 1];
};

// Work item -> (query tile, split, number of splits).
__device__ __forceinline__ bool item_tile(int item, int nqt, int M, const SplitTable& tab, int* qt,
                                          int* split, int* nsplit) {
  if (M == 0x7FFFFFFF) {  // one item per tile
    if (item >= nqt) return false;
    *qt = nqt - 1 - item;
    *split = 0;
    *nsplit = 1;
    return true;
  }
  if (item >= tab.start[nqt]) return false;
  int lo = 0, hi = nqt;  // largest o with start[o] <= item
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tab.start[mid] <= item) lo = mid;
    else hi = mid;
  }
  *qt = nqt - 1 - lo;
  *split = item - tab.start[lo];
  *nsplit = tab.start[lo + 1] - tab.start[lo];
  return true;
}

// ------------------------------------------------------------ flash kernel
// MASK 0: selection bitmap (DSA); MASK 1: window [p-W+1, p] (SWA). SINK:
// whether attention-sink blocks come first (a separate instantiation, so the
// sink-free loop carries no sink checks).
//
// One workgroup = one head x 128 queries, wave w owning queries 32w..32w+31.
// Register budget is held to 256 per wave so two workgroups share a CU: one
// computes while the other waits on its barrier or loads. Inside a
// workgroup the next 64-key block is loaded into registers while the current
// block is computed (software pipelining) and written to LDS after a barrier.
template <int DQK, int DV, int MASK, bool SINK>
__global__ __launch_bounds__(256, (DV > 128 ? 1 : 2)) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ sk,
    const uint16_t* __restrict__ sv, int n_sink, const uint32_t* __restrict__ bm,
    const uint16_t* __restrict__ gate, uint16_t* __restrict__ out, float* __restrict__ part,
    int S, int Tbuf, int P, int kv_offset, int H, int HKV, int W32, int window, float scale_log2,
    int gate_dim, int nqt, int M, const SplitTable tab) {
  constexpr int KSQ = DQK / 16;
  constexpr int NDB = DV / 32;
  constexpr int KPAD = DQK + 8;           // bf16 elements per K row in LDS
  constexpr int KCH = DQK / 8;            // 16-byte chunks per K row
  constexpr int KLD = kBN * KCH / 256;    // K chunks per thread per block
  constexpr int VCH = DV / 8;             // 8-dv groups per V row
  constexpr int VUN = (kBN / 4) * VCH;    // (4 keys x 8 dv) units per block
  constexpr int VLD = (VUN + 255) / 256;  // units per thread
  static_assert((kBN * KCH) % 256 == 0, "K block must split evenly over 256 threads");
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBN * KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kBN * DV];
  // selection-mask calls start the logits' accumulators from the mask:
  // entry n holds, for 4 consecutive accumulator elements, 0 where bit j of
  // n is set (selected) and -inf where it is not; 0 + q.k is q.k exactly and
  // -inf + q.k is -inf, so the MFMA chain ends with the masked logits
  __shared__ __attribute__((aligned(16))) float mask_tab[16][4];
  if (MASK == 0 && threadIdx.x < 64)
    mask_tab[threadIdx.x >> 2][threadIdx.x & 3] = ((threadIdx.x >> 2) >> (threadIdx.x & 3)) & 1 ? 0.0f : -INFINITY;

  // XCD-aware order (selection-mask calls). Workgroups are dealt to the 8
  // XCDs round-robin by their linear id; this maps XCD x's share to one
  // contiguous range of the logical (item fastest, then head, then batch)
  // order, so the tiles running together on an XCD are mostly of one head and
  // stream the same K/V blocks (from key 0 up) through that XCD's L2 instead
  // of each XCD pulling every head's K/V from memory (dsa-s32k: 285 -> 152 GB
  // fetched per launch, 49.6 -> 46.2 ms). Window tiles read short, different
  // key ranges and keep the plain order.
  int item = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (MASK == 0) {
    const int64_t nx = gridDim.x, ny = gridDim.y;
    const int64_t N = nx * ny * gridDim.z;
    const int64_t L = blockIdx.x + nx * (blockIdx.y + ny * (int64_t)blockIdx.z);
    const int64_t x = L % 8, q8 = N / 8, r8 = N % 8;
    const int64_t lg = x * q8 + (x < r8 ? x : r8) + L / 8;
    item = (int)(lg % nx);
    h = (int)((lg / nx) % ny);
    b = (int)(lg / (nx * ny));
  }
  int qt, split, nsplit;
  if (!item_tile(item, nqt, M, tab, &qt, &split, &nsplit)) return;
  DSA_CHECK(qt >= 0 && qt < nqt && split >= 0 && split < nsplit, qt, split);
  DSA_CHECK(h < H && (nsplit == 1 || part != nullptr), h, nsplit);
  const int hk = h / (H / HKV);  // cache head: query heads come in groups of H / HKV
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, lh = lane >> 5;
  const int q0 = qt * kBQ;
  const int s = q0 + 32 * wave + ln;
  const bool svalid = s < S;
  const int sc = svalid ? s : S - 1;
  const int p = P + sc;  // absolute position of this lane's query
  const int64_t qrow = (int64_t)b * S + sc;

  bf16x8_t bq[KSQ];
  {
    const uint16_t* qp = q + (qrow * H + h) * DQK + 8 * lh;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) bq[ks] = as_bf16x8(load16(qp + 16 * ks));
  }

  // key range of this split of the tile, in buffer rows (row j = position kv_offset + j)
  int tjlo, tjhi;
  tile_range(qt, S, P, Tbuf, kv_offset, MASK == 1 ? window : 0, &tjlo, &tjhi);
  // (64-bit: M is INT_MAX when tiles are not split)
  const int jlo = (int)((int64_t)tjlo + (int64_t)split * M * kBN);
  const int jhi = (int)std::min<int64_t>(tjhi, (int64_t)jlo + (int64_t)M * kBN - 1);
  DSA_CHECK(jlo >= 0 && jhi < Tbuf, jlo, jhi);  // the item's key blocks lie in the buffer
  const int64_t kvrow0 = (int64_t)b * Tbuf;
  // Blocks of this item: first the attention-sink rows (split 0 only, every
  // query sees all of them, no position), then the cache rows jlo .. jhi.
  // Block bi < nsb holds sink rows 64 bi .. 64 bi + 63.
  const int nsb = (SINK && split == 0) ? (n_sink + kBN - 1) / kBN : 0;
  const int nblk = nsb + (jlo <= jhi ? (jhi - jlo) / kBN + 1 : 0);

  // ---- register prefetch of one key block. A K row of KCH 16-byte chunks is
  // covered by one or two power-of-two parts (24 = 16 + 8), so that a thread
  // keeps one byte offset per part and successive loads of a part add a
  // fixed row step (24 = 16 + 8, 12 = 8 + 4). Loads go through a buffer resource that ends at the
  // last row of this batch's buffer: rows past it read as zeros.
  constexpr int KP1 = (KCH == 24) ? 16 : (KCH == 12) ? 8 : KCH;  // chunks per row, part 1
  constexpr int KP2 = KCH - KP1;               // part 2 (0 or 8)
  constexpr int R1 = 256 / KP1, N1 = kBN / R1;  // rows per load, loads
  constexpr int R2 = KP2 ? 256 / KP2 : 1, N2 = KP2 ? kBN / R2 : 0;
  static_assert(N1 + N2 == KLD && (VLD == 1 || VUN == 256 * VLD), "load split");
  static_assert(256 % KP1 == 0 && (KP2 == 0 || 256 % KP2 == 0) && N1 * R1 == kBN &&
                    (KP2 == 0 || N2 * R2 == kBN),
                "every K row chunk is loaded exactly once");
  static_assert(VCH == 8 || VCH == 16 || VCH == 32, "the V swizzle keeps chunks inside a row");
  const int krow1 = tid / KP1, kc1 = tid % KP1;
  const int krow2 = KP2 ? tid / KP2 : 0, kc2 = KP2 ? KP1 + tid % KP2 : 0;
  const uint32_t rowb = (uint32_t)HKV * DQK * 2u;  // bytes between key rows
  const uint32_t kbo1 = krow1 * rowb + 16u * kc1, kbo2 = krow2 * rowb + 16u * kc2;
  // V unit n (4 key rows x 8 dv) of a block: thread tid takes n = tid + 256 u
  int vkg[VLD], vdg[VLD];
  const uint32_t vrowb = (uint32_t)HKV * DV * 2u;
  uint32_t vbo[VLD];
#pragma unroll
  for (int u = 0; u < VLD; ++u) {
    const int un = tid + 256 * u;
    vkg[u] = un / VCH;
    vdg[u] = un - vkg[u] * VCH;
    vbo[u] = 4 * vkg[u] * vrowb + 16u * vdg[u];
  }
  u32x4_t kpre[KLD];
  u32x4_t vpre[VLD][4];
  auto load_block = [&](int bi) {
    // rows of the buffer (cache or sinks) from the block's first row on
    const uint16_t *kp, *vp;
    int64_t rows;
    if (SINK && bi < nsb) {
      kp = sk + ((int64_t)bi * kBN * HKV + hk) * DQK;
      vp = sv + ((int64_t)bi * kBN * HKV + hk) * DV;
      rows = n_sink - bi * kBN;
    } else {
      const int jb = jlo + (bi - nsb) * kBN;
      kp = k + ((kvrow0 + jb) * HKV + hk) * DQK;
      vp = v + ((kvrow0 + jb) * HKV + hk) * DV;
      rows = (int64_t)Tbuf - jb;
    }
    const auto kr = make_rsrc(kp, rows * rowb - (int64_t)hk * DQK * 2);
    const auto vr = make_rsrc(vp, rows * vrowb - (int64_t)hk * DV * 2);
#pragma unroll
    for (int n = 0; n < N1; ++n) kpre[n] = buffer_load16(kr, kbo1 + n * R1 * rowb);
#pragma unroll
    for (int n = 0; n < N2; ++n) kpre[N1 + n] = buffer_load16(kr, kbo2 + n * R2 * rowb);
#pragma unroll
    for (int u = 0; u < VLD; ++u)
      if (tid + 256 * u < VUN) {
#pragma unroll
        for (int e = 0; e < 4; ++e) vpre[u][e] = buffer_load16(vr, vbo[u] + e * vrowb);
      }
  };
  // ---- registers -> LDS: K row-major (padded rows), V row-major (swizzled)
  auto store_block = [&]() {
#pragma unroll
    for (int n = 0; n < N1; ++n) *(u32x4_t*)(&Ks[(krow1 + n * R1) * KPAD + 8 * kc1]) = kpre[n];
#pragma unroll
    for (int n = 0; n < N2; ++n) *(u32x4_t*)(&Ks[(krow2 + n * R2) * KPAD + 8 * kc2]) = kpre[N1 + n];
#pragma unroll
    for (int u = 0; u < VLD; ++u)
      if (tid + 256 * u < VUN) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * vkg[u] + e;
          *(u32x4_t*)(&Vs[r * DV + 8 * (vdg[u] ^ vt_xor<VCH>(r))]) = vpre[u][e];
        }
      }
  };
  // Byte offset in Vs of this lane's transposing read for dv block d and the
  // first 16-key chunk: in each 16-lane group (g = lane / 16), lane 4j + q
  // addresses key row 4 * (lane / 32) + j, bytes 64 d + 32 (g & 1) + 8 q, and
  // lane i of the group receives dv 32 d + lane % 32 of those four rows; the
  // read 8 rows further gives the other four keys of the operand.
  uint32_t vrd[NDB];
  {
    const int g16 = lane >> 4, jr = (lane >> 2) & 3, qr = lane & 3;
    const int r = 4 * lh + jr;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const int chunk = 4 * d + 2 * (g16 & 1) + (qr >> 1);
      vrd[d] = (uint32_t)(r * DV * 2 + 16 * (chunk ^ vt_xor<VCH>(r)) + 8 * (qr & 1));
    }
  }

  float m = -INFINITY, l = 0.0f;
  const float lazy_thr = kLazyLog2 / scale_log2;  // raw-logit units
  f32x16_t o[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) o[d] = zero16();
  const uint32_t* bmrow = bm + qrow * (int64_t)W32;

  // selection-bitmap words of a block, loaded one block ahead like K and V;
  // a sink block's words mark its rows below n_sink
  uint32_t nbits[2] = {0u, 0u};
  auto load_bits = [&](int bi) {
    if (SINK && bi < nsb) {
      const int nv = min(kBN, n_sink - bi * kBN);  // >= 1
      nbits[0] = nv >= 32 ? 0xFFFFFFFFu : (1u << nv) - 1u;
      nbits[1] = nv >= 64 ? 0xFFFFFFFFu : (nv > 32 ? (1u << (nv - 32)) - 1u : 0u);
    } else if (MASK == 0) {
      const int w0 = (jlo + (bi - nsb) * kBN) >> 5;
      nbits[0] = (w0 < W32) ? bmrow[w0] : 0u;
      nbits[1] = (w0 + 1 < W32) ? bmrow[w0 + 1] : 0u;
    }
  };

  if (nblk > 0) {
    load_block(0);
    load_bits(0);
  }
  for (int bi = 0; bi < nblk; ++bi) {
    __syncthreads();  // every wave is done reading the previous block
    store_block();
    __syncthreads();
    const uint32_t bits[2] = {nbits[0], nbits[1]};
    const bool sinkb = SINK && bi < nsb;
    const int jb = jlo + (bi - nsb) * kBN;  // first cache row (cache blocks)

    // the next block's loads overlap this block's MFMA and softmax work
    if (bi + 1 < nblk) {
      load_block(bi + 1);
      load_bits(bi + 1);
    }

    // S^T for both 32-key halves, one masked online-softmax update over the
    // 64 keys, then O^T += V^T P^T for both halves
    // (the two halves' accumulation chains are interleaved, so consecutive
    // MFMAs never depend on each other)
    f32x16_t st[2] = {zero16(), zero16()};
    if (MASK == 0) {  // accumulators start at 0 (selected) or -inf: 4 elements per table read
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t wbits = bits[i] >> (4 * lh);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4_t m4 = *(const f32x4_t*)(&mask_tab[(wbits >> (8 * g)) & 0xFu][0]);
#pragma unroll
          for (int j = 0; j < 4; ++j) st[i][4 * g + j] = m4[j];
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bf16x8_t a = as_bf16x8(*(const u32x4_t*)(&Ks[(32 * i + ln) * KPAD + 16 * ks + 8 * lh]));
        st[i] = mfma32x32x16(a, bq[ks], st[i]);
      }
    if (DQK <= 192) {
      // K operand reads run about ten MFMAs ahead: the first twelve LDS reads
      // (mask table and K) are issued first, then one per MFMA (dsa-s32k K3
      // 44.6-44.9 -> 44.0-44.3 ms on one MI355X; 10 or 14 ahead were slower).
      // Dims 256 have no registers to spare for it.
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
      for (int r = 0; r < 2 * KSQ; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    // mask, then the running max on raw logits (scale > 0 keeps the order),
    // as a tree of three-input maxima (16 ops, 4 deep)
    float mx3[11];
#pragma unroll
    for (int i = 0; i < 2 && MASK != 0; ++i) {
      const uint32_t wbits = bits[i] >> (4 * lh);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x;
        if (sinkb) {
          x = keep_or_neg_inf(st[i][e], wbits, 8 * (e >> 2) + (e & 3));
        } else {
          const int jj = jb + 32 * i + 8 * (e >> 2) + 4 * lh + (e & 3);
          const int t = kv_offset + jj;
          x = ((jj < Tbuf) && (t <= p) && (t > p - window)) ? st[i][e] : -INFINITY;
        }
        st[i][e] = x;
      }
    }
    // (the first level reads the logits themselves, which are MFMA results
    // when the mask came in through the accumulators: that level uses the
    // compiler's max, whose operands get the MFMA-to-VALU wait states; the
    // inline-asm maxima only ever read VALU results)
#pragma unroll
    for (int r = 0; r < 10; ++r) {  // 30 of the 32 logits
      const int e0 = 3 * r;
      const float a = st[e0 >> 4][e0 & 15], b = st[(e0 + 1) >> 4][(e0 + 1) & 15],
                  c = st[(e0 + 2) >> 4][(e0 + 2) & 15];
      mx3[r] = MASK == 0 ? __builtin_fmaxf(__builtin_fmaxf(a, b), c) : max3_f32(a, b, c);
    }
    mx3[10] = MASK == 0 ? __builtin_fmaxf(st[1][14], st[1][15]) : max_f32(st[1][14], st[1][15]);
    float mx = max3_f32(max3_f32(mx3[0], mx3[1], mx3[2]), max3_f32(mx3[3], mx3[4], mx3[5]),
                        max3_f32(mx3[6], mx3[7], mx3[8]));
    mx = max3_f32(mx, mx3[9], mx3[10]);
    mx = max_other_half(mx);
    // The reference max m only moves when the block max exceeds it by more
    // than kLazyLog2 in log2 units, so p = 2^(c(x - m)) stays below
    // 2^kLazyLog2 and O, l are rescaled rarely. Any m gives the same O / l.
    const bool bump = mx > m + lazy_thr;
    const bool resc = bump && (m != -INFINITY);  // m = -inf: O and l are still 0
    const float mnew = bump ? mx : m;
    const float nms = (mnew == -INFINITY) ? 0.0f : -mnew * scale_log2;
    const float alpha = resc ? exp2_hw((m - mnew) * scale_log2) : 1.0f;
    m = mnew;
    // weights rounded to bf16 once; the row sum is taken over the same
    // rounded weights that P.V multiplies (one bf16 dot2 per pair)
    uint32_t pk[2][2][4];  // [32-key half][16-key chunk][packed pair]
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = exp2_hw(fmaf(st[i][e], scale_log2, nms));
        const float p1 = exp2_hw(fmaf(st[i][e + 1], scale_log2, nms));
        const uint32_t pp = pack_bf16x2(p0, p1);
        psum = sum_bf16x2(pp, psum);
        pk[i][e >> 3][(e & 7) >> 1] = pp;
      }
    l = l * alpha + psum;
    if (__any(resc)) {
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8_t pb = as_bf16x8(u32x4_t{pk[i][c][0], pk[i][c][1], pk[i][c][2], pk[i][c][3]});
        const uint32_t crow = (uint32_t)(16 * (2 * i + c) * DV * 2);  // first row of the chunk
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
          const bf16x8_t va = lds_read_tr_pair(Vs, vrd[d] + crow, 8 * DV * 2);
          o[d] = mfma32x32x16(va, pb, o[d]);
        }
      }
  }

  // ---- normalise, gate, store
  const float ltot = l + shfl_xor_f(l, 32);
  if (nsplit > 1) {  // partial state (unnormalised O, max, sum) for the merge kernel
    float* pp = part + ((((int64_t)b * H + h) * gridDim.x + item) * kBQ + 32 * wave + ln) *
                           (DV + 4);
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(float4*)(pp + 32 * d + 8 * g + 4 * lh) =
            make_float4(o[d][4 * g], o[d][4 * g + 1], o[d][4 * g + 2], o[d][4 * g + 3]);
    if (lh == 0) {
      pp[DV] = m;
      pp[DV + 1] = ltot;
    }
    return;
  }
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  if (!svalid) return;
  float g1 = 1.0f;
  if (gate_dim == 1) g1 = sigmoid_f32(bf16_to_f32(gate[qrow * H + h]));
  uint16_t* orow = out + (qrow * H + h) * DV;
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dv0 = 32 * d + 8 * g + 4 * lh;
      float r4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float gg = g1;
        if (gate_dim > 1) gg = sigmoid_f32(bf16_to_f32(gate[(qrow * H + h) * DV + dv0 + r]));
        r4[r] = o[d][4 * g + r] * inv * gg;
      }
      uint2 pkd;
      pkd.x = pack_bf16x2(r4[0], r4[1]);
      pkd.y = pack_bf16x2(r4[2], r4[3]);
      *(uint2*)(orow + dv0) = pkd;
    }
  }
}

// ------------------------------------------------- ping-pong flash kernel
// Selection-mask calls without sinks or split tiles. One workgroup of 8
// waves = one head x 256 queries: waves 0-3 (group A) own queries 0..127 of
// the tile, waves 4-7 (group B) queries 128..255, so each SIMD runs one wave
// of each group. The groups run half a block apart and alternate at every
// workgroup barrier: while one group is in its MFMA phase (S(j) = K(j) Q^T
// with the mask in the accumulators, then O += V(j-1)^T P(j-1)^T), the other
// is in its VALU phase (the online softmax of its latest S, and staging the
// next K block (A) or V block (B) from registers into LDS). The MFMA work of
// one wave then runs under the VALU work of the other instead of after it.
// K(j) and V(j-1) are read in the same phase, so both are double-buffered.
// Per query the arithmetic is that of prefill_kernel, block by block; group A
// also walks the tile's last (at most two) blocks, which its queries cannot
// see: their bits are clear, so they add nothing.
constexpr int kBQ2 = 256;  // queries per ping-pong workgroup
// The ping-pong kernel runs when its grid has at least this many workgroups
// (one per CU at a time): on smaller grids the prefill_kernel's twice as many
// 128-query workgroups fill the GPU better.
constexpr int64_t kPingPongMinGrid = 1024;

template <int DQK, int DV>
__global__ __launch_bounds__(512, 1) void prefill_pp_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint32_t* __restrict__ bm,
    const uint16_t* __restrict__ gate, uint16_t* __restrict__ out, int S, int Tbuf, int P, int H,
    int HKV, int W32, float scale_log2, int gate_dim, int nqt) {
  constexpr int KSQ = DQK / 16;
  constexpr int NDB = DV / 32;
  constexpr int KPAD = DQK + 8;
  constexpr int KCH = DQK / 8;
  constexpr int KLD = kBN * KCH / 256;   // K chunks per group-A thread per block
  constexpr int VCH = DV / 8;
  constexpr int VUN = (kBN / 4) * VCH;   // (4 keys x 8 dv) units per block
  static_assert((kBN * KCH) % 256 == 0 && VUN <= 256, "one group of 256 threads stages a block");
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBN * KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kBN * DV];
  __shared__ __attribute__((aligned(16))) float mask_tab[16][4];  // as in prefill_kernel
  if (threadIdx.x < 64)
    mask_tab[threadIdx.x >> 2][threadIdx.x & 3] = ((threadIdx.x >> 2) >> (threadIdx.x & 3)) & 1 ? 0.0f : -INFINITY;

  // XCD-aware order, as in prefill_kernel
  int item, h, b;
  {
    const int64_t nx = gridDim.x, ny = gridDim.y;
    const int64_t N = nx * ny * gridDim.z;
    const int64_t L = blockIdx.x + nx * (blockIdx.y + ny * (int64_t)blockIdx.z);
    const int64_t x = L % 8, q8 = N / 8, r8 = N % 8;
    const int64_t lg = x * q8 + (x < r8 ? x : r8) + L / 8;
    item = (int)(lg % nx);
    h = (int)((lg / nx) % ny);
    b = (int)(lg / (nx * ny));
  }
  const int qt = nqt - 1 - item;  // longest tiles first
  DSA_CHECK(qt >= 0 && qt < nqt && h < H, qt, h);
  const int hk = h / (H / HKV);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: group A, 1: group B
  const int tg = tid & 255;   // thread index inside the group
  const int ln = lane & 31, lh = lane >> 5;
  const int q0 = qt * kBQ2;
  const int s = q0 + 32 * wave + ln;
  const bool svalid = s < S;
  const int sc = svalid ? s : S - 1;
  const int64_t qrow = (int64_t)b * S + sc;

  bf16x8_t bq[KSQ];
  {
    const uint16_t* qp = q + (qrow * H + h) * DQK + 8 * lh;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) bq[ks] = as_bf16x8(load16(qp + 16 * ks));
  }
  // causal key range of the whole tile: rows 0 .. jhi
  const int jhi = min(P + min(q0 + kBQ2 - 1, S - 1), Tbuf - 1);
  const int nblk = jhi / kBN + 1;
  DSA_CHECK(jhi >= 0 && jhi < Tbuf, jhi, Tbuf);
  const int64_t kvrow0 = (int64_t)b * Tbuf;

  // ---- K staging by group A (the chunk split of prefill_kernel, over 256 threads)
  constexpr int KP1 = (KCH == 24) ? 16 : (KCH == 12) ? 8 : KCH;
  constexpr int KP2 = KCH - KP1;
  constexpr int R1 = 256 / KP1, N1 = kBN / R1;
  constexpr int R2 = KP2 ? 256 / KP2 : 1, N2 = KP2 ? kBN / R2 : 0;
  static_assert(N1 + N2 == KLD, "load split");
  const int krow1 = tg / KP1, kc1 = tg % KP1;
  const int krow2 = KP2 ? tg / KP2 : 0, kc2 = KP2 ? KP1 + tg % KP2 : 0;
  const uint32_t rowb = (uint32_t)HKV * DQK * 2u;
  const uint32_t kbo1 = krow1 * rowb + 16u * kc1, kbo2 = krow2 * rowb + 16u * kc2;
  // ---- V staging by group B: unit tg = 4 key rows x 8 dv
  const int vkg = tg / VCH, vdg = tg - (tg / VCH) * VCH;
  const bool vact = tg < VUN;
  const uint32_t vrowb = (uint32_t)HKV * DV * 2u;
  const uint32_t vbo = 4 * vkg * vrowb + 16u * vdg;
  // a wave stages only K (group A) or only V (group B): one register set
  constexpr int NPRE = KLD > 4 ? KLD : 4;
  u32x4_t pre[NPRE];
  auto load_k = [&](int bi) {
    const int jb = bi * kBN;
    const auto kr = make_rsrc(k + ((kvrow0 + jb) * HKV + hk) * DQK,
                              (int64_t)(Tbuf - jb) * rowb - (int64_t)hk * DQK * 2);
#pragma unroll
    for (int n = 0; n < N1; ++n) pre[n] = buffer_load16(kr, kbo1 + n * R1 * rowb);
#pragma unroll
    for (int n = 0; n < N2; ++n) pre[N1 + n] = buffer_load16(kr, kbo2 + n * R2 * rowb);
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int n = 0; n < N1; ++n) *(u32x4_t*)(&Ks[buf][(krow1 + n * R1) * KPAD + 8 * kc1]) = pre[n];
#pragma unroll
    for (int n = 0; n < N2; ++n)
      *(u32x4_t*)(&Ks[buf][(krow2 + n * R2) * KPAD + 8 * kc2]) = pre[N1 + n];
  };
  auto load_v = [&](int bi) {
    const int jb = bi * kBN;
    const auto vr = make_rsrc(v + ((kvrow0 + jb) * HKV + hk) * DV,
                              (int64_t)(Tbuf - jb) * vrowb - (int64_t)hk * DV * 2);
    if (vact) {
#pragma unroll
      for (int e = 0; e < 4; ++e) pre[e] = buffer_load16(vr, vbo + e * vrowb);
    }
  };
  auto store_v = [&](int buf) {
    if (vact) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * vkg + e;
        *(u32x4_t*)(&Vs[buf][r * DV + 8 * (vdg ^ vt_xor<VCH>(r))]) = pre[e];
      }
    }
  };
  // transposing-read offsets of the V operand, as in prefill_kernel
  uint32_t vrd[NDB];
  {
    const int g16 = lane >> 4, jr = (lane >> 2) & 3, qr = lane & 3;
    const int r = 4 * lh + jr;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const int chunk = 4 * d + 2 * (g16 & 1) + (qr >> 1);
      vrd[d] = (uint32_t)(r * DV * 2 + 16 * (chunk ^ vt_xor<VCH>(r)) + 8 * (qr & 1));
    }
  }

  float m = -INFINITY, l = 0.0f;
  const float lazy_thr = kLazyLog2 / scale_log2;
  f32x16_t o[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) o[d] = zero16();
  f32x16_t st[2] = {zero16(), zero16()};
  uint32_t pk[2][2][4] = {};
  // bitmap words of the next block, loaded unconditionally (clamped to the
  // row) so that no control flow merges them; words past the row are
  // cleared where they are used. They go through a buffer resource like the
  // K and V loads: loads of one kind return in order, so the wait for these
  // words skips the K or V prefetch issued after them.
  // (the resource starts at the wave's first row, which is wave-uniform; each
  // lane's row is an offset: a per-lane resource would serialise the loads)
  const int rowbase = __builtin_amdgcn_readfirstlane(min(q0 + 32 * wave, S - 1));
  const auto bmr = make_rsrc(bm + ((int64_t)b * S + rowbase) * W32, (int64_t)32 * W32 * 4);
  const uint32_t boff = (uint32_t)(sc - rowbase) * (uint32_t)W32 * 4u;
  DSA_CHECK(sc >= rowbase && sc - rowbase < 32, sc, rowbase);  // the lane's row is in the resource
  uint32_t nbits[2];
  auto load_bits = [&](int bi) {
    const int w0 = min(2 * bi, W32 - 1), w1 = min(2 * bi + 1, W32 - 1);
    nbits[0] = __builtin_amdgcn_raw_buffer_load_b32(bmr, boff + 4 * w0, 0, 0);
    nbits[1] = __builtin_amdgcn_raw_buffer_load_b32(bmr, boff + 4 * w1, 0, 0);
  };
  // MFMA phase of block j: S(j) (j < nblk) and O += V(j-1)^T P(j-1)^T (j > 0)
  auto pv_part = [&](int j) {
    const uint16_t* Vb = Vs[(j - 1) & 1];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8_t pb = as_bf16x8(u32x4_t{pk[i][c][0], pk[i][c][1], pk[i][c][2], pk[i][c][3]});
        const uint32_t crow = (uint32_t)(16 * (2 * i + c) * DV * 2);
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
          const bf16x8_t va = lds_read_tr_pair(Vb, vrd[d] + crow, 8 * DV * 2);
          o[d] = mfma32x32x16(va, pb, o[d]);
        }
      }
  };
  // the logits' accumulators start from the mask of block bi (0 where the
  // key is selected, -inf where not; the table of prefill_kernel)
  auto mask_init = [&](int bi) {
    const uint32_t bits[2] = {2 * bi < W32 ? nbits[0] : 0u, 2 * bi + 1 < W32 ? nbits[1] : 0u};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t wbits = bits[i] >> (4 * lh);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4_t m4 = *(const f32x4_t*)(&mask_tab[(wbits >> (8 * g)) & 0xFu][0]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) st[i][4 * g + jj] = m4[jj];
      }
    }
  };
  auto s_part = [&](int j) {
    mask_init(j);
    const uint16_t* Kb = Ks[j & 1];
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bf16x8_t a = as_bf16x8(*(const u32x4_t*)(&Kb[(32 * i + ln) * KPAD + 16 * ks + 8 * lh]));
        st[i] = mfma32x32x16(a, bq[ks], st[i]);
      }
    load_bits(min(j + 1, nblk - 1));
  };
  // The wave in its MFMA phase runs at raised issue priority, so that when
  // both waves of a SIMD are ready the arbiter issues its MFMAs and operand
  // reads before the other wave's softmax (dsa-s32k 42.4 -> 39.6 ms; level 3
  // measures the same, raising the softmax phase instead gains nothing).
  // Each MFMA's PV operands (two transposing reads) are read about four MFMAs
  // ahead: eight reads first, then two per MFMA (without the hint the compiler
  // reads one operand ahead and every MFMA waits on LDS); the K reads follow
  // prefill_kernel's hint (mask table and four K reads ahead).
  auto pv_hint = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };
  auto s_hint = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
    for (int r = 0; r < 2 * KSQ; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  auto mfma_first = [&]() {  // block 0: S only
    __builtin_amdgcn_s_setprio(1);
    s_part(0);
    s_hint();
    __builtin_amdgcn_s_setprio(0);
  };
  // 0 < j < nblk: S(j), then PV(j-1). With S first, the softmax of the next
  // VALU phase finds its logits finished, and the MFMAs still draining at the
  // barrier are PV ones, which nothing needs before the next MFMA phase
  // (dsa-s32k 36.2 -> 35.4 ms against PV first)
  auto mfma_full = [&](int j) {
    __builtin_amdgcn_s_setprio(1);
    s_part(j);
    s_hint();
    pv_part(j);
    pv_hint();
    __builtin_amdgcn_s_setprio(0);
  };
  auto mfma_last = [&]() {  // after the last block: PV(nblk-1) only
    __builtin_amdgcn_s_setprio(1);
    pv_part(nblk);
    pv_hint();
    __builtin_amdgcn_s_setprio(0);
  };
  // VALU phase: masked online softmax of the latest S into P (prefill_kernel's arithmetic)
  auto softmax = [&]() {
    float mx3[11];
#pragma unroll
    for (int r = 0; r < 10; ++r) {
      const int e0 = 3 * r;
      const float a = st[e0 >> 4][e0 & 15], bb = st[(e0 + 1) >> 4][(e0 + 1) & 15],
                  c = st[(e0 + 2) >> 4][(e0 + 2) & 15];
      mx3[r] = __builtin_fmaxf(__builtin_fmaxf(a, bb), c);
    }
    mx3[10] = __builtin_fmaxf(st[1][14], st[1][15]);
    float mx = max3_f32(max3_f32(mx3[0], mx3[1], mx3[2]), max3_f32(mx3[3], mx3[4], mx3[5]),
                        max3_f32(mx3[6], mx3[7], mx3[8]));
    mx = max3_f32(mx, mx3[9], mx3[10]);
    mx = max_other_half(mx);
    const bool bump = mx > m + lazy_thr;
    const bool resc = bump && (m != -INFINITY);
    const float mnew = bump ? mx : m;
    const float nms = (mnew == -INFINITY) ? 0.0f : -mnew * scale_log2;
    const float alpha = resc ? exp2_hw((m - mnew) * scale_log2) : 1.0f;
    m = mnew;
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = exp2_hw(fmaf(st[i][e], scale_log2, nms));
        const float p1 = exp2_hw(fmaf(st[i][e + 1], scale_log2, nms));
        const uint32_t pp = pack_bf16x2(p0, p1);
        psum = sum_bf16x2(pp, psum);
        pk[i][e >> 3][(e & 7) >> 1] = pp;
      }
    l = l * alpha + psum;
    if (__any(resc)) {
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
    }
  };

  // Phase 2j: A computes block j on MFMA; B runs the softmax of block j-1 and
  // stages V(j) (its buffer last held V(j-2), read up to phase 2j-1).
  // Phase 2j+1: A runs the softmax of block j and stages K(j+1) (its buffer
  // last held K(j-1), read up to phase 2j-1); B computes block j on MFMA.
  // Each group runs its own loop (so that only its own state is live across
  // iterations), with the first and last block peeled so that the loop body
  // is straight-line code, and every prefetch is issued unconditionally
  // (block index clamped to the last block; a stage past it lands in a buffer
  // nobody reads again): no control flow merges in-flight registers, which
  // would make the compiler wait for the loads. Both groups execute
  // 2 nblk + 2 barriers.
  load_bits(0);
  if (grp == 0) {
    load_k(0);
    store_k(0);
    load_k(min(1, nblk - 1));
    __syncthreads();
    mfma_first();
    __syncthreads();
    softmax();
    store_k(1);
    load_k(min(2, nblk - 1));
    __syncthreads();
    for (int j = 1; j < nblk; ++j) {
      mfma_full(j);
      __syncthreads();
      softmax();
      store_k((j + 1) & 1);
      load_k(min(j + 2, nblk - 1));
      __syncthreads();
    }
    mfma_last();
    __syncthreads();
  } else {
    load_v(0);
    __syncthreads();
    store_v(0);
    load_v(min(1, nblk - 1));
    __syncthreads();
    mfma_first();
    __syncthreads();
    for (int j = 1; j < nblk; ++j) {
      softmax();
      store_v(j & 1);
      load_v(min(j + 1, nblk - 1));
      __syncthreads();
      mfma_full(j);
      __syncthreads();
    }
    softmax();
    __syncthreads();
    mfma_last();
  }

  // ---- normalise, gate, store
  const float ltot = sum_other_half(l);
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  if (!svalid) return;
  float g1 = 1.0f;
  if (gate_dim == 1) g1 = sigmoid_f32(bf16_to_f32(gate[qrow * H + h]));
  uint16_t* orow = out + (qrow * H + h) * DV;
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dv0 = 32 * d + 8 * g + 4 * lh;
      float r4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float gg = g1;
        if (gate_dim > 1) gg = sigmoid_f32(bf16_to_f32(gate[(qrow * H + h) * DV + dv0 + r]));
        r4[r] = o[d][4 * g + r] * inv * gg;
      }
      uint2 pkd;
      pkd.x = pack_bf16x2(r4[0], r4[1]);
      pkd.y = pack_bf16x2(r4[2], r4[3]);
      *(uint2*)(orow + dv0) = pkd;
    }
  }
}

// Combines the splits of each split tile: out = sum_s 2^(c(m_s - M)) O_s /
// sum_s 2^(c(m_s - M)) l_s, then the gate. A workgroup covers 8 query rows
// of one (tile, head, b), 32 threads per row and 4 output dims per thread,
// and issues every split's loads before combining them (up to kMergeUnroll
// splits in flight; longer lists run in chunks).
// query rows per merge workgroup: DV / 4 threads per row
template <int DV>
constexpr int merge_rows() { return 256 / (DV / 4) < 8 ? 256 / (DV / 4) : 8; }
constexpr int kMergeUnroll = 8;
template <int DV>
__global__ __launch_bounds__(256) void merge_splits_kernel(const float* __restrict__ part,
                                                           const uint16_t* __restrict__ gate,
                                                           uint16_t* __restrict__ out, int S,
                                                           int H, int items, int nqt,
                                                           float scale_log2, int gate_dim,
                                                           const SplitTable tab) {
  constexpr int TPR = DV / 4;  // threads per query row
  constexpr int kMergeRows = merge_rows<DV>();
  static_assert(TPR * kMergeRows <= 256 && kBQ % kMergeRows == 0, "row group must fit the workgroup");
  const int qt = blockIdx.x / (kBQ / kMergeRows);
  const int rg = blockIdx.x % (kBQ / kMergeRows);
  const int h = blockIdx.y, b = blockIdx.z;
  // first item of this tile and its number of splits
  const int base = tab.start[nqt - 1 - qt];
  const int c = tab.start[nqt - qt] - base;
  DSA_CHECK(c >= 1 && base + c <= items, base, c);
  if (c <= 1 || (int)threadIdx.x >= TPR * kMergeRows) return;
  const int qi = rg * kMergeRows + threadIdx.x / TPR, dv0 = 4 * (threadIdx.x % TPR);
  const int s = qt * kBQ + qi;
  if (s >= S) return;
  const int64_t split_stride = (int64_t)kBQ * (DV + 4);
  const float* pt = part + (((int64_t)b * H + h) * items + base) * split_stride + qi * (DV + 4);
  const int64_t qrow = (int64_t)b * S + s;
  const uint16_t g1raw = gate_dim == 1 ? gate[qrow * H + h] : (uint16_t)0;  // issued early
  // loads are unconditional (split indices past the last one re-read it and
  // get weight 0) so that every load of a chunk is in flight at once
  float mx = -INFINITY;
  for (int s0 = 0; s0 < c; s0 += kMergeUnroll) {
    float ms[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) ms[u] = pt[min(s0 + u, c - 1) * split_stride + DV];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) mx = fmaxf(mx, ms[u]);
  }
  float L = 0.0f, acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < c; s0 += kMergeUnroll) {
    float2 ml[kMergeUnroll];
    float4 o4[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const float* q = pt + min(s0 + u, c - 1) * split_stride;
      ml[u] = *(const float2*)(q + DV);
      o4[u] = *(const float4*)(q + dv0);
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const float w = (s0 + u >= c || ml[u].x == -INFINITY) ? 0.0f : exp2f((ml[u].x - mx) * scale_log2);
      L += w * ml[u].y;
      acc[0] += w * o4[u].x;
      acc[1] += w * o4[u].y;
      acc[2] += w * o4[u].z;
      acc[3] += w * o4[u].w;
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  float g1 = 1.0f;
  if (gate_dim == 1) g1 = sigmoid_f32(bf16_to_f32(g1raw));
  float r4[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float gg = g1;
    if (gate_dim > 1) gg = sigmoid_f32(bf16_to_f32(gate[(qrow * H + h) * DV + dv0 + r]));
    r4[r] = acc[r] * inv * gg;
  }
  uint2 pkd;
  pkd.x = pack_bf16x2(r4[0], r4[1]);
  pkd.y = pack_bf16x2(r4[2], r4[3]);
  *(uint2*)(out + (qrow * H + h) * DV + dv0) = pkd;
}

struct SplitPlan {
  int nqt, M, items;
  SplitTable tab;
};

// Splits long query tiles when the plain grid is too small to fill the GPU:
// at most M key blocks per work item, about 1024 items in total. The bound
// uses past_len = T - S (the longest tiles a call with this T can have).
// Only selection-mask (DSA) calls split: there kv_offset = 0 and T >= P + S,
// so T - S bounds past_len and the bound plan covers every actual call.
// Window (SWA) tiles are short by construction and never split, nor are
// calls with more than kMaxSplitTiles query tiles (their grid is large).
SplitPlan make_split_plan(int B, int S, int T, int P, int H, int kv_offset, int window) {
  SplitPlan pl;
  pl.nqt = (int)(((int64_t)S + kBQ - 1) / kBQ);
  pl.M = 0x7FFFFFFF;  // no split
  if (window <= 0 && kv_offset == 0 && (int64_t)B * H * pl.nqt < 1024 &&
      pl.nqt <= kMaxSplitTiles) {
    int64_t total_bound = 0;
    for (int t = 0; t < pl.nqt; ++t) total_bound += tile_blocks(t, S, T - S, T, 0, 0);
    total_bound *= (int64_t)B * H;
    const int64_t m = (total_bound + 1023) / 1024;
    pl.M = (int)std::max<int64_t>(16, m);
  }
  pl.items = 0;
  for (int o = 0; o < pl.nqt; ++o) {
    if (o <= kMaxSplitTiles) pl.tab.start[o] = pl.items;
    const int nb = tile_blocks(pl.nqt - 1 - o, S, P, T, kv_offset, window);
    pl.items += nb > pl.M ? (nb + pl.M - 1) / pl.M : 1;
  }
  if (pl.nqt <= kMaxSplitTiles) pl.tab.start[pl.nqt] = pl.items;
  return pl;
}

template <int DQK, int DV>
hipError_t launch_dims(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const uint16_t* sk, const uint16_t* sv, int n_sink,
                       const uint32_t* bm, const uint16_t* gate, uint16_t* out, int B, int S,
                       int Tbuf, int P, int kv_offset, int H, int Hkv, int W32, int window,
                       float scale_log2, int gate_dim, float* part, hipStream_t st) {
  const SplitPlan pl = make_split_plan(B, S, Tbuf, P, H, kv_offset, window);
  if (pl.items != pl.nqt && part == nullptr) return hipErrorInvalidValue;  // no partial buffer
  if constexpr (DQK <= 192 && DV <= 128) {
    const int nqt2 = (int)(((int64_t)S + kBQ2 - 1) / kBQ2);
    if (window <= 0 && n_sink == 0 && pl.items == pl.nqt && (int64_t)B * H * nqt2 >= kPingPongMinGrid) {
      hipLaunchKernelGGL((prefill_pp_kernel<DQK, DV>), dim3(nqt2, H, B), dim3(512), 0, st, q, k,
                         v, bm, gate, out, S, Tbuf, P, H, Hkv, W32, scale_log2, gate_dim, nqt2);
      return hipGetLastError();
    }
  }
  const dim3 grid(pl.items, H, B);
#define DSA_FLASH_LAUNCH(MK, SK)                                                                 \
  hipLaunchKernelGGL((prefill_kernel<DQK, DV, MK, SK>), grid, dim3(256), 0, st, q, k, v, sk, sv,   \
                     n_sink, bm, gate, out, part, S, Tbuf, P, kv_offset, H, Hkv, W32, window,     \
                     scale_log2, gate_dim, pl.nqt, pl.M, pl.tab)
  if (window > 0) {
    if (n_sink > 0)
      DSA_FLASH_LAUNCH(1, true);
    else
      DSA_FLASH_LAUNCH(1, false);
  } else {
    if (n_sink > 0)
      DSA_FLASH_LAUNCH(0, true);
    else
      DSA_FLASH_LAUNCH(0, false);
  }
#undef DSA_FLASH_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.items == pl.nqt) return e;
  hipLaunchKernelGGL((merge_splits_kernel<DV>), dim3(pl.nqt * (kBQ / merge_rows<DV>()), H, B), dim3(256),
                     0, st, part, gate, out, S, H, pl.items, pl.nqt, scale_log2, gate_dim, pl.tab);
  return hipGetLastError();
}

constexpr int kBitmapLdsMaxWords = 12288;  // 48 KiB of LDS

}  // namespace

#ifdef DSA_DEBUG
DSA_DEBUG_TAKE(attn_prefill)
#endif

bool prefill_mfma_supported(int dtype, int S, int Dqk, int Dv) {
  if (dtype != 1 || S < 16) return false;
  // (96: A.X-K2-Light's qk_head_dim, nope 64 + rope 32)
  return (Dqk == 64 && Dv == 64) || (Dqk == 128 && Dv == 128) || (Dqk == 192 && Dv == 128) ||
         (Dqk == 256 && Dv == 128) || (Dqk == 128 && Dv == 64) || (Dqk == 256 && Dv == 256) ||
         (Dqk == 96 && Dv == 64) || (Dqk == 96 && Dv == 128);
}

void prefill_work_plan(int B, int S, int T, int P, int H, int kv_offset, int window, int* n_tiles,
                       int* n_items, int* max_blocks, int* item_start, int cap) {
  const SplitPlan pl = make_split_plan(B, S, T, P, H, kv_offset, window);
  *n_tiles = pl.nqt;
  *n_items = pl.items;
  *max_blocks = pl.M;
  if (item_start && cap >= pl.nqt + 1) {
    if (pl.nqt <= kMaxSplitTiles) {
      for (int o = 0; o <= pl.nqt; ++o) item_start[o] = pl.tab.start[o];
    } else {  // never split: one item per tile, longest first
      for (int o = 0; o <= pl.nqt; ++o) item_start[o] = o;
    }
  }
}

size_t bitmap_bytes(int B, int S, int T) {
  return (size_t)B * (size_t)S * (size_t)(((int64_t)T + 31) / 32) * sizeof(uint32_t);
}

size_t prefill_mfma_workspace_bytes(int B, int S, int T, int H, int Dv) {
  // bitmap, 256-byte aligned, then partial states if long tiles get split
  const size_t bmb = (bitmap_bytes(B, S, T) + 255) / 256 * 256;
  const SplitPlan pl = make_split_plan(B, S, T, T - S, H, 0, 0);
  if (pl.items == pl.nqt) return bmb;
  return bmb + (size_t)B * H * pl.items * kBQ * (Dv + 4) * sizeof(float);
}

hipError_t launch_prefill_mfma(const void* q, const void* k, const void* v, const void* sink_k,
                               const void* sink_v, int n_sink, const int32_t* indices,
                               const void* gate, void* out, int B, int S, int T, int past_len,
                               int kv_offset, int H, int Hkv, int Dqk, int Dv, int topk, int window,
                               float sm_scale, int gate_dim, void* workspace, hipStream_t st) {
  const int W32 = (int)(((int64_t)T + 31) / 32);
  uint32_t* bm = (uint32_t*)workspace;
  // partial states follow the (256-byte aligned) bitmap; only DSA calls have them
  float* part = nullptr;
  if (window <= 0 && prefill_mfma_workspace_bytes(B, S, T, H, Dv) >
                         (bitmap_bytes(B, S, T) + 255) / 256 * 256)
    part = (float*)((char*)workspace + (bitmap_bytes(B, S, T) + 255) / 256 * 256);
  const int64_t rows = (int64_t)B * S;
  if (window <= 0) {
    if (W32 <= kBitmapLdsMaxWords) {
      hipLaunchKernelGGL(bitmap_lds_kernel, dim3((unsigned)rows), dim3(256),
                         W32 * sizeof(uint32_t), st, indices, bm, S, T, past_len, topk, W32);
    } else {
      const int64_t n = rows * W32;
      const int64_t g = std::min<int64_t>((n + 255) / 256, 65536);
      hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)g), dim3(256), 0, st, bm, n);
      hipLaunchKernelGGL(bitmap_global_kernel, dim3((unsigned)rows), dim3(256), 0, st, indices,
                         bm, S, T, past_len, topk, W32);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const float sl2 = sm_scale * DSA_LOG2E;
  const uint16_t *qq = (const uint16_t*)q, *kk = (const uint16_t*)k, *vv = (const uint16_t*)v,
                 *gg = (const uint16_t*)gate;
  uint16_t* oo = (uint16_t*)out;
#define DSA_PREFILL_CASE(A, C)                                                                    \
  if (Dqk == A && Dv == C)                                                                        \
    return launch_dims<A, C>(qq, kk, vv, (const uint16_t*)sink_k, (const uint16_t*)sink_v, n_sink, \
                             bm, gg, oo, B, S, T, past_len, kv_offset, H, Hkv, W32, window,    \
                             sl2, gate_dim, part, st);
  DSA_PREFILL_CASE(64, 64)
  DSA_PREFILL_CASE(96, 64)
  DSA_PREFILL_CASE(96, 128)
  DSA_PREFILL_CASE(128, 64)
  DSA_PREFILL_CASE(128, 128)
  DSA_PREFILL_CASE(192, 128)
  DSA_PREFILL_CASE(256, 128)
  DSA_PREFILL_CASE(256, 256)
#undef DSA_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
