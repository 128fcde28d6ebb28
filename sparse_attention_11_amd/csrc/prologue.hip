// prologue.hip -- the indexer's projections in front of the lightning indexer
// (gfx950).
//
// A.X-K2 page, SGA ("Sparse Gated Attention") bullets: the indexer has its own
// light projections, wq_b on the query LoRA bottleneck and wk followed by a
// LayerNorm (k_norm) on the key, and per-head weights from weights_proj; its
// key cache is appended to by update_indexer. "Two RoPE layouts": the
// indexer uses the non-interleaved (half-split) rotary layout.
//
// Kernels
//  gemm_bf16_kernel   C[M,N] = A[M,K] W[N,K]^T (nn.Linear weights), bf16 in,
//                     fp32 accumulate, bf16 out. Tiles of 128 x 128 (K steps
//                     of 64) or, for wide outputs, 256 x 128 (K steps of 32),
//                     4 waves of 64 x 64 or 128 x 64, v_mfma_f32_32x32x16_bf16
//                     with both operands read K-contiguous from LDS
//                     (double-buffered, the next step loaded into registers
//                     under the current MFMAs); the MFMA forms C^T so that a
//                     lane stores four consecutive columns at once.
//                     The A operand may be two row-major matrices side by
//                     side (a concatenation along K read in place), and the
//                     epilogue may scatter columns into the main attention's
//                     tensors (the MLA side below).
//  rope_q_kernel      half-split RoPE on the last rope_dim dims of every
//                     index head, in place.
//  ln_rope_k_kernel   LayerNorm over idx_dim (fp32 statistics), then the
//                     same RoPE, written into the key cache rows
//                     past_len .. past_len + S - 1.
//
// The main attention's projections (A.X-K2 page, "MLA + explicit sparse
// mask" steps 1-3 and "Attention output gate"; interleaved RoPE, "two RoPE
// layouts") run as three GEMMs whose epilogues write the attention's inputs
// directly:
//   kv_a_proj_with_mqa  hidden -> [latent | rope key]: the latent to the
//                       workspace, the rope key rotated and written into the
//                       rope slice of every head's cache row
//   expand_kv           latent -> per head [k_nope | v]: into the nope slice of
//                       the key cache rows and the value cache rows
//   q_gate_proj         [q_resid | q_compressed] -> per head [query | gate]:
//                       the query (rope slice rotated) and the gate
// A lane holds four consecutive output columns, so every interleaved rotary
// pair (2j, 2j + 1) is in one lane and no group of four straddles a head or
// a slice (every width is a multiple of 16).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kGBN = 128;  // output columns per workgroup
// rows per workgroup (BM) and K step (BK): 128 x 64 for skinny outputs, 256
// x 32 for wide ones (half the L2 -> CU operand bytes per flop of the square
// tile, same LDS footprint). LDS rows are padded by 8 bf16 (16 bytes), which
// keeps the 16-byte operand reads of 32 consecutive rows conflict-free.
template <int BM>
constexpr int gemm_bk() { return BM == 256 ? 32 : 64; }
constexpr int kGroupedTiles = 8;  // column tiles up to which a row tile stays on one XCD

// Two weight / output pairs share one pass over A (the key and head-weight
// projections both read the hidden state): column tiles 0 .. nt1-1 belong to
// (W1, C1), the rest to (W2, C2). With few column tiles (skinny outputs, A
// the big operand) tile ids are dealt so that the column tiles of one row
// tile run back to back on the same XCD (the A tile is then an L2 hit for
// all but the first); with many, column tiles vary fastest over all XCDs, so
// each XCD's L2 holds only its share of W for the row tiles in flight.
struct GemmOut {
  const uint16_t* W;
  uint16_t* C;
  int N, ldc;
};
// Optional RoPE epilogue (q_idx): heads of D dims, rotary slice = the last R
// dims of each head (R 32 or 64), row m at position P + m % S.
struct GemmRope {
  const float* cosb;
  const float* sinb;
  int D, R, S, P;
};

// The A operand: rows of A1 (K1 wide) followed, along K, by rows of A2 (K -
// K1 wide; unused when K1 = K). K1 is a multiple of 32, so a 16-byte chunk
// lies in one of the two.
struct GemmA {
  const uint16_t* A1;
  const uint16_t* A2;
  int K1;
};
// Epilogues of the main attention's projections (EPI 1..3 below): token row
// m = b * S + s sits at position P + s of caches with T rows.
struct GemmMla {
  uint16_t* q;     // [M, H, N + R]       (EPI 1)
  uint16_t* gate;  // [M, H, Dv]          (EPI 1)
  uint16_t* kc;    // [B, T, H, N + R]    (EPI 2: rope slices, EPI 3: nope slices)
  uint16_t* vc;    // [B, T, H, Dv]       (EPI 3)
  uint16_t* lat;   // [M, L]              (EPI 2)
  const float* cosb;
  const float* sinb;  // [T, R / 2]
  int H, N, R, Dv, L, S, T, P;
};

__device__ __forceinline__ void store4_bf16(uint16_t* p, float a, float b, float c, float d) {
  uint2 pk;
  pk.x = pack_bf16x2(a, b);
  pk.y = pack_bf16x2(c, d);
  *(uint2*)p = pk;
}

// Interleaved RoPE of the two pairs (x0, x1), (x2, x3) at rotary indices j0,
// j0 + 1 of position p.
__device__ __forceinline__ void rope_interleaved4(float* x, const GemmMla& e, int p, int j0) {
  const int half = e.R / 2;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float c = e.cosb[(int64_t)p * half + j0 + u], s = e.sinb[(int64_t)p * half + j0 + u];
    const float a = x[2 * u], b = x[2 * u + 1];
    x[2 * u] = a * c - b * s;
    x[2 * u + 1] = b * c + a * s;
  }
}

// Columns n .. n + 3 of token row m, scattered by the MLA epilogues.
template <int EPI>
__device__ __forceinline__ void mla_store4(const GemmMla& e, int m, int n, float* x) {
  const int b = m / e.S, s = m - b * e.S, p = e.P + s;
  const int Dqk = e.N + e.R;
  DSA_CHECK(p < e.T || EPI == 1, p, e.T);  // cache rows past_len + s exist
  if (EPI == 1) {  // q_gate_proj: head h = [query (Dqk) | gate (Dv)]
    const int W = Dqk + e.Dv, h = n / W, c = n - h * W;
    if (c < Dqk) {
      if (c >= e.N) rope_interleaved4(x, e, p, (c - e.N) >> 1);
      store4_bf16(e.q + ((int64_t)m * e.H + h) * Dqk + c, x[0], x[1], x[2], x[3]);
    } else {
      store4_bf16(e.gate + ((int64_t)m * e.H + h) * e.Dv + (c - Dqk), x[0], x[1], x[2], x[3]);
    }
  } else if (EPI == 2) {  // kv_a_proj_with_mqa: [latent (L) | rope key (R)]
    if (n < e.L) {
      store4_bf16(e.lat + (int64_t)m * e.L + n, x[0], x[1], x[2], x[3]);
    } else {
      const int r = n - e.L;
      rope_interleaved4(x, e, p, r >> 1);
      uint16_t* row = e.kc + ((int64_t)b * e.T + p) * e.H * Dqk + e.N + r;
      for (int h = 0; h < e.H; ++h) store4_bf16(row + (int64_t)h * Dqk, x[0], x[1], x[2], x[3]);
    }
  } else {  // expand_kv: head h = [k_nope (N) | v (Dv)]
    const int W = e.N + e.Dv, h = n / W, c = n - h * W;
    const int64_t cr = ((int64_t)b * e.T + p) * e.H + h;
    if (c < e.N)
      store4_bf16(e.kc + cr * Dqk + c, x[0], x[1], x[2], x[3]);
    else
      store4_bf16(e.vc + cr * e.Dv + (c - e.N), x[0], x[1], x[2], x[3]);
  }
}

// RHALF: half the rotary width (16 or 32) for the RoPE epilogue, 0 for none;
// a compile-time constant so that every rotary pair's registers are fixed.
// EPI 0: C = A W^T into (o1, o2); EPI 1..3: the MLA epilogues above (o1.N is
// the output width).
// KSTRAD (EPI 1 only): the concatenation point K1 is not a multiple of the K
// step, so one step straddles the two A matrices.
template <int RHALF, int BM, int EPI, bool KSTRAD = false>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmA ga, GemmOut o1, GemmOut o2,
                                                           int M, int K, int ntiles_n, int nt1,
                                                           GemmRope rp, GemmMla mla) {
  constexpr int kGBM = BM, kGBK = gemm_bk<BM>();
  constexpr int kWM = BM / 2;                  // rows per wave (2 x 2 waves)
  constexpr int kWI = kWM / 32;                // 32-row MFMA blocks per wave
  constexpr int kCPR = kGBK / 8;               // 16-byte chunks per tile row
  constexpr int kGLdA = kGBM * kCPR / 256;     // A chunks per thread
  constexpr int kGLdW = kGBN * kCPR / 256;     // W chunks per thread
  // tile rows of kGBK bf16 without padding; the 16-byte chunk c of row r is
  // stored at chunk c ^ ((r / (16 / kCPR)) % kCPR), so that both the stores
  // (kCPR lanes per row, 16 / kCPR rows per 16 lanes) and the MFMA operand
  // reads (16 rows, one chunk) of a 16-lane phase hit 64 distinct banks
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kGBM * kGBK];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][kGBN * kGBK];
  auto swz = [](int r, int c) { return c ^ ((r / (16 / kCPR)) % kCPR); };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int pid = blockIdx.x;
  int mt, nt;
  if (ntiles_n <= kGroupedTiles) {  // the row tile's column tiles together on one XCD
    const int xcd = pid & 7, q = pid >> 3;
    mt = (q / ntiles_n) * 8 + xcd;
    nt = q % ntiles_n;
  } else {
    mt = pid / ntiles_n;
    nt = pid % ntiles_n;
  }
  const int m0 = mt * kGBM;
  if (m0 >= M) return;
  const bool second = nt >= nt1;
  const uint16_t* __restrict__ W = second ? o2.W : o1.W;
  uint16_t* __restrict__ C = second ? o2.C : o1.C;
  const int N = second ? o2.N : o1.N, ldc = second ? o2.ldc : o1.ldc;
  const int n0 = (second ? nt - nt1 : nt) * kGBN;

  // global -> register staging, two K steps ahead: the data of step s is
  // loaded at the start of step s - 2 into register set s & 1 and written to
  // LDS at the end of step s - 1, so each load has two steps of MFMAs to land.
  // The loads are branch-free buffer loads over per-tile resources (rows past
  // M or N read as zeros; a chunk past K is sent past the resource's end), so
  // the compiler counts them exactly and the LDS write of step s - 1's data
  // waits only for those loads, not for the ones step s has just issued (with
  // a conditional load per chunk it waited for everything, a full memory
  // latency per K step).
  // (only q_gate_proj reads two A matrices; the other instantiations see one)
  const int lda1 = EPI == 1 ? ga.K1 : K, lda2 = K - ga.K1;
  const auto rA1 = make_rsrc(ga.A1 + (int64_t)m0 * lda1, (int64_t)(M - m0) * lda1 * 2);
  const auto rA2 = make_rsrc(EPI == 1 ? ga.A2 + (int64_t)m0 * lda2 : ga.A1,
                             EPI == 1 ? (int64_t)(M - m0) * lda2 * 2 : 0);
  const auto rW = make_rsrc(W + (int64_t)n0 * K, (int64_t)(N - n0) * K * 2);
  constexpr uint32_t kPast = 0xFFFFFFF0u;  // an offset past every resource
  u32x4_t ra[2][kGLdA], rw[2][kGLdW];
  auto load_tile = [&](auto set_c, int k0) {
    constexpr int SET = decltype(set_c)::value;
#pragma unroll
    for (int i = 0; i < kGLdA; ++i) {
      const int c = tid + 256 * i, r = c / kCPR, kc = 8 * (c % kCPR);
      const int k = k0 + kc;
      if constexpr (EPI == 1 && KSTRAD) {
        // a step straddles K1 (K1 % 32 == 0, so a chunk does not), and a
        // resource is uniform: each chunk reads both matrices, the side it is
        // not in sent past the end
        const bool in1 = k < ga.K1, in2 = !in1 && k < K;
        ra[SET][i] = buffer_load16(rA1, in1 ? (uint32_t)(r * lda1 + k) * 2u : kPast) |
                     buffer_load16(rA2, in2 ? (uint32_t)(r * lda2 + (k - ga.K1)) * 2u : kPast);
      } else if constexpr (EPI == 1) {  // the whole step lies in A1 or in A2
        const bool a2 = k0 >= ga.K1;
        const uint32_t off = a2 ? (uint32_t)(r * lda2 + (k - ga.K1)) * 2u
                                : (uint32_t)(r * lda1 + k) * 2u;
        ra[SET][i] = buffer_load16(a2 ? rA2 : rA1, k < K ? off : kPast);
      } else {
        ra[SET][i] = buffer_load16(rA1, k < K ? (uint32_t)(r * lda1 + k) * 2u : kPast);
      }
    }
#pragma unroll
    for (int i = 0; i < kGLdW; ++i) {
      const int c = tid + 256 * i, r = c / kCPR, kc = 8 * (c % kCPR);
      const int k = k0 + kc;
      rw[SET][i] = buffer_load16(rW, k < K ? (uint32_t)(r * K + k) * 2u : kPast);
    }
  };
  auto store_tile = [&](auto set_c, int buf) {
    constexpr int SET = decltype(set_c)::value;
#pragma unroll
    for (int i = 0; i < kGLdA; ++i) {
      const int c = tid + 256 * i, r = c / kCPR, kc = 8 * (c % kCPR);
      *(u32x4_t*)(&As[buf][r * kGBK + 8 * swz(r, kc / 8)]) = ra[SET][i];
    }
#pragma unroll
    for (int i = 0; i < kGLdW; ++i) {
      const int c = tid + 256 * i, r = c / kCPR, kc = 8 * (c % kCPR);
      *(u32x4_t*)(&Ws[buf][r * kGBK + 8 * swz(r, kc / 8)]) = rw[SET][i];
    }
  };

  f32x16_t acc[kWI][2];
#pragma unroll
  for (int i = 0; i < kWI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero16();

  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < kGBK / 16; ++s) {
      bf16x8_t a[kWI], b[2];
#pragma unroll
      for (int i = 0; i < kWI; ++i) {
        const int r = wm * kWM + 32 * i + (lane & 31);
        a[i] = as_bf16x8(*(const u32x4_t*)(&As[buf][r * kGBK + 8 * swz(r, 2 * s + (lane >> 5))]));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + 32 * j + (lane & 31);
        b[j] = as_bf16x8(*(const u32x4_t*)(&Ws[buf][r * kGBK + 8 * swz(r, 2 * s + (lane >> 5))]));
      }
#pragma unroll
      for (int i = 0; i < kWI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(b[j], a[i], acc[i][j]);
    }
  };
  const int nk = (K + kGBK - 1) / kGBK;
  const std::integral_constant<int, 0> S0;
  const std::integral_constant<int, 1> S1;
  // one K step: loads of step kt + 2 into set kt & 1 (written to LDS at the
  // end of step kt - 1, so free), MFMAs on buffer kt & 1, then step kt + 1's
  // data (loaded two steps ago) into the other buffer (last read before the
  // previous barrier)
  auto step = [&](int kt, auto cur, auto nxt) {
    // (past the last step every chunk lies past K and reads nothing: no branch,
    // so the wait counts stay exact)
    load_tile(cur, (kt + 2) * kGBK);
    compute(decltype(cur)::value);
    if (kt + 1 < nk) {
      store_tile(nxt, decltype(nxt)::value);
      __syncthreads();
    }
  };

  load_tile(S0, 0);
  if (nk > 1) load_tile(S1, kGBK);
  store_tile(S0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, S0, S1);
    if (kt + 1 < nk) step(kt + 1, S1, S0);
  }
  // the MFMA computes C^T: lane l holds C[m][n] for m = 32 i + l % 32 and
  // n = 32 j + 8 g + 4 (l / 32) + r (e = 4 g + r) of the wave's tile, so each
  // group of four is one 8-byte store of consecutive columns
  if (RHALF > 0) {
    // A wave's 64 columns lie inside one head (D = 64 or 128, 64-aligned), so
    // a rotary pair (d, d + R/2) sits in one lane: R/2 = 32 is the next 32-
    // column block j, R/2 = 16 the group g + 2 of the same block.
    constexpr int half = RHALF;
    const int hd0 = (n0 + wn * 64) % rp.D;  // head dim of the wave's first column
#pragma unroll
    for (int i = 0; i < kWI; ++i) {
      const int m = m0 + wm * kWM + 32 * i + (lane & 31);
      const int p = rp.P + (m < M ? m : M - 1) % rp.S;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int d = hd0 + 32 * j + 8 * g + 4 * (lane >> 5) + r;
            const int jj = d - (rp.D - rp.R);  // index in the rotary slice
            if (jj < 0 || jj >= half) continue;
            // partner at d + half: (j + 1, g) for half 32, (j, g + 2) for 16
            constexpr int dj = half == 32 ? 1 : 0, dg = half == 32 ? 0 : 2;
            const int j2 = j + dj, g2 = g + dg;
            if (j2 > 1 || g2 > 3) continue;  // folds at compile time (unrolled loops)
            const float cs = rp.cosb[(int64_t)p * half + jj], sn = rp.sinb[(int64_t)p * half + jj];
            const float x1 = acc[i][j][4 * g + r], x2 = acc[i][j2][4 * g2 + r];
            acc[i][j][4 * g + r] = x1 * cs - x2 * sn;
            acc[i][j2][4 * g2 + r] = x2 * cs + x1 * sn;
          }
    }
  }
  if (EPI > 0) {
#pragma unroll
    for (int i = 0; i < kWI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = m0 + wm * kWM + 32 * i + (lane & 31);
        if (m >= M) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * 64 + 32 * j + 8 * g + 4 * (lane >> 5);
          if (n >= N) continue;  // (widths are multiples of 4)
          float x[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                        acc[i][j][4 * g + 3]};
          mla_store4<EPI>(mla, m, n, x);
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < kWI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = m0 + wm * kWM + 32 * i + (lane & 31);
      if (m >= M) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 64 + 32 * j + 8 * g + 4 * (lane >> 5);
        uint16_t* cp = C + (int64_t)m * ldc + n;
        if (n + 3 < N && ((ldc | n) & 3) == 0) {
          uint2 pk;
          pk.x = pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
          pk.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          *(uint2*)cp = pk;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) cp[r] = f32_to_bf16(acc[i][j][4 * g + r]);
        }
      }
    }
}

// Half-split RoPE of one (x1, x2) pair: (x1 cos - x2 sin, x2 cos + x1 sin).
__device__ __forceinline__ void rope_pair(float& x1, float& x2, float c, float s) {
  const float a = x1, b = x2;
  x1 = a * c - b * s;
  x2 = b * c + a * s;
}

// q [M, HI, D] in place: one thread per (row, head, pair j < R / 2); the pair
// is (D - R + j, D - R + j + R / 2). Row m is token s = m % S at p = P + s.
__global__ __launch_bounds__(256) void rope_q_kernel(uint16_t* __restrict__ q,
                                                     const float* __restrict__ cosb,
                                                     const float* __restrict__ sinb, int64_t M,
                                                     int S, int P, int HI, int D, int R) {
  const int half = R / 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * HI * half) return;
  const int j = (int)(i % half);
  const int64_t mh = i / half;
  const int64_t m = mh / HI;
  const int p = P + (int)(m % S);
  uint16_t* row = q + mh * D + (D - R);
  float x1 = bf16_to_f32(row[j]), x2 = bf16_to_f32(row[j + half]);
  rope_pair(x1, x2, cosb[(int64_t)p * half + j], sinb[(int64_t)p * half + j]);
  row[j] = f32_to_bf16(x1);
  row[j + half] = f32_to_bf16(x2);
}

// One wave per key row (D = 64 .. 256 values, D / 64 per lane): LayerNorm
// with fp32 mean and biased variance, affine gamma / beta, then the RoPE of
// the last R dims, stored to cache row b * T + P + s.
__global__ __launch_bounds__(256) void ln_rope_k_kernel(const uint16_t* __restrict__ kraw,
                                                        const uint16_t* __restrict__ gamma,
                                                        const uint16_t* __restrict__ beta,
                                                        const float* __restrict__ cosb,
                                                        const float* __restrict__ sinb,
                                                        uint16_t* __restrict__ kcache, int64_t M,
                                                        int S, int T, int P, int D, int R,
                                                        float eps) {
  __shared__ float rowbuf[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m = (int64_t)blockIdx.x * 4 + wave;
  if (m >= M) return;  // whole waves only: no workgroup barrier below
  const int per = D / 64;
  float x[4];
  float sum = 0.0f;
  for (int c = 0; c < per; ++c) {
    x[c] = bf16_to_f32(kraw[m * D + lane + 64 * c]);
    sum += x[c];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  const float mean = sum / (float)D;
  float var = 0.0f;
  for (int c = 0; c < per; ++c) {
    const float d = x[c] - mean;
    var += d * d;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) var += __shfl_xor(var, off, 64);
  const float inv = 1.0f / sqrtf(var / (float)D + eps);
  for (int c = 0; c < per; ++c) {
    const int d = lane + 64 * c;
    rowbuf[wave][d] = (x[c] - mean) * inv * bf16_to_f32(gamma[d]) + bf16_to_f32(beta[d]);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int b = (int)(m / S), s = (int)(m % S), p = P + s;
  const int half = R / 2, r0 = D - R;
  DSA_CHECK(p < T, p, T);  // the key's cache row exists
  uint16_t* out = kcache + ((int64_t)b * T + p) * D;
  for (int c = 0; c < per; ++c) {
    const int d = lane + 64 * c;
    float v = rowbuf[wave][d];
    if (d >= r0) {  // the rotary slice: pair (r0 + j, r0 + j + half)
      const int j = (d - r0) % half;
      const float cs = cosb[(int64_t)p * half + j], sn = sinb[(int64_t)p * half + j];
      const float x1 = rowbuf[wave][r0 + j], x2 = rowbuf[wave][r0 + j + half];
      v = (d - r0 < half) ? x1 * cs - x2 * sn : x2 * cs + x1 * sn;
    }
    out[d] = f32_to_bf16(v);
  }
}

}  // namespace

#ifdef DSA_DEBUG
DSA_DEBUG_TAKE(prologue)
#endif

namespace {
hipError_t gemm_launch(GemmA ga, GemmOut o1, GemmOut o2, int M, int K, const GemmRope* rp,
                       hipStream_t st, int epi = 0, const GemmMla* mla = nullptr) {
  if (K % 32 != 0 || ga.K1 % 32 != 0 || ga.K1 > K) return hipErrorInvalidValue;
  const int nt1 = (o1.N + kGBN - 1) / kGBN, nt2 = o2.N > 0 ? (o2.N + kGBN - 1) / kGBN : 0;
  const int ntn = nt1 + nt2;
  // wide outputs: 256-row tiles (still >= 2 workgroups per CU at M = 32768)
  const int bm = (ntn > kGroupedTiles && (int64_t)((M + 255) / 256) * ntn >= 2048) ? 256 : 128;
  const int64_t mtiles = (M + bm - 1) / bm;
  const int64_t g = (ntn <= kGroupedTiles ? (mtiles + 7) / 8 * 8 : mtiles) * ntn;
  if (g > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const GemmMla ml = mla ? *mla : GemmMla{};
#define DSA_GEMM_LAUNCH(RH, BMV, EP, RP)                                                         \
  hipLaunchKernelGGL((gemm_bf16_kernel<RH, BMV, EP>), dim3((unsigned)g), dim3(256), 0, st, ga,  \
                     o1, o2, M, K, ntn, nt1, RP, ml)
#define DSA_GEMM_BM(BMV)                                           \
  if (epi == 1 && ga.K1 % gemm_bk<BMV>() != 0) {                   \
    hipLaunchKernelGGL((gemm_bf16_kernel<0, BMV, 1, true>), dim3((unsigned)g), dim3(256), 0, st, \
                       ga, o1, o2, M, K, ntn, nt1, GemmRope{}, ml);                          \
  } else if (epi == 1) {                                           \
    DSA_GEMM_LAUNCH(0, BMV, 1, GemmRope{});                        \
  } else if (epi == 2) {                                           \
    DSA_GEMM_LAUNCH(0, BMV, 2, GemmRope{});                        \
  } else if (epi == 3) {                                           \
    DSA_GEMM_LAUNCH(0, BMV, 3, GemmRope{});                        \
  } else if (rp && rp->R == 64) {                                  \
    DSA_GEMM_LAUNCH(32, BMV, 0, *rp);                              \
  } else if (rp && rp->R == 32) {                                  \
    DSA_GEMM_LAUNCH(16, BMV, 0, *rp);                              \
  } else {                                                         \
    DSA_GEMM_LAUNCH(0, BMV, 0, GemmRope{});                        \
  }
  if (bm == 256) {
    DSA_GEMM_BM(256)
  } else {
    DSA_GEMM_BM(128)
  }
#undef DSA_GEMM_BM
#undef DSA_GEMM_LAUNCH
  return hipGetLastError();
}

GemmA one_a(const void* A, int K) { return GemmA{(const uint16_t*)A, nullptr, K}; }
}  // namespace

hipError_t launch_gemm_bf16(const void* A, const void* W, void* C, int M, int N, int K, int ldc,
                            hipStream_t st) {
  return gemm_launch(one_a(A, K), GemmOut{(const uint16_t*)W, (uint16_t*)C, N, ldc},
                     GemmOut{nullptr, nullptr, 0, 0}, M, K, nullptr, st);
}

hipError_t launch_indexer_prologue(const void* q_lora, const void* hidden, const void* wq_b,
                                   const void* wk, const void* k_norm_weight,
                                   const void* k_norm_bias, const void* weights_proj,
                                   const float* rope_cos, const float* rope_sin, void* q_idx,
                                   void* k_idx_cache, void* w, int B, int S, int T, int past_len,
                                   int q_lora_rank, int hidden_dim, int HI, int DI, int R,
                                   float eps, void* workspace, hipStream_t st) {
  const int M = B * S;
  // q_idx = q_lora wq_b^T, with the RoPE in the epilogue where a rotary pair
  // sits in one lane (idx_dim 64 or 128, rope_dim 32 or 64)
  const bool fused = (DI == 64 || DI == 128) && (R == 32 || R == 64);
  const GemmRope rp{rope_cos, rope_sin, DI, R, S, past_len};
  hipError_t e = gemm_launch(one_a(q_lora, q_lora_rank),
                             GemmOut{(const uint16_t*)wq_b, (uint16_t*)q_idx, HI * DI,
                                             HI * DI},
                             GemmOut{nullptr, nullptr, 0, 0}, M, q_lora_rank, fused ? &rp : nullptr,
                             st);
  if (e != hipSuccess) return e;
  // the key and head-weight projections in one pass over the hidden state
  e = gemm_launch(one_a(hidden, hidden_dim), GemmOut{(const uint16_t*)wk, (uint16_t*)workspace, DI, DI},
                  GemmOut{(const uint16_t*)weights_proj, (uint16_t*)w, HI, HI}, M, hidden_dim,
                  nullptr, st);
  if (e != hipSuccess) return e;
  if (R > 0 && !fused) {
    const int64_t n = (int64_t)M * HI * (R / 2);
    hipLaunchKernelGGL(rope_q_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       (uint16_t*)q_idx, rope_cos, rope_sin, (int64_t)M, S, past_len, HI, DI, R);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(ln_rope_k_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, st,
                     (const uint16_t*)workspace, (const uint16_t*)k_norm_weight,
                     (const uint16_t*)k_norm_bias, rope_cos, rope_sin, (uint16_t*)k_idx_cache,
                     (int64_t)M, S, T, past_len, DI, R, eps);
  return hipGetLastError();
}

hipError_t launch_mla_prologue(const void* q_resid, const void* q_comp, const void* hidden,
                               const void* wq_gate, const void* wkv_a, const void* wkv_b,
                               const float* rope_cos, const float* rope_sin, void* q, void* gate,
                               void* k_cache, void* v_cache, int B, int S, int T, int past_len,
                               int Qr, int Qc, int Hd, int L, int H, int N, int R, int Dv,
                               void* workspace, hipStream_t st) {
  const int M = B * S;
  GemmMla e{(uint16_t*)q,          (uint16_t*)gate, (uint16_t*)k_cache, (uint16_t*)v_cache,
            (uint16_t*)workspace, rope_cos,        rope_sin,           H,
            N,                    R,               Dv,                 L,
            S,                    T,               past_len};
  const GemmOut none{nullptr, nullptr, 0, 0};
  // kv_a_proj_with_mqa: the latent (workspace) and the rotated rope key
  hipError_t err = gemm_launch(one_a(hidden, Hd), GemmOut{(const uint16_t*)wkv_a, nullptr, L + R, 0},
                               none, M, Hd, nullptr, st, 2, &e);
  if (err != hipSuccess) return err;
  // expand_kv: per-head k_nope and v from the latent
  err = gemm_launch(one_a(workspace, L), GemmOut{(const uint16_t*)wkv_b, nullptr, H * (N + Dv), 0},
                    none, M, L, nullptr, st, 3, &e);
  if (err != hipSuccess) return err;
  // q_gate_proj on [q_resid, q_compressed]: query (rope slice rotated) and gate
  return gemm_launch(GemmA{(const uint16_t*)q_resid, (const uint16_t*)q_comp, Qr},
                     GemmOut{(const uint16_t*)wq_gate, nullptr, H * (N + R + Dv), 0}, none, M,
                     Qr + Qc, nullptr, st, 1, &e);
}

}  // namespace dsa
