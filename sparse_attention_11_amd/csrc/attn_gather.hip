// attn_gather.hip -- split-K row-gather attention + merge (gfx950).
//
// For few queries (decode: one token per sequence) the work is a stream of
// whole selected cache rows: with token-major caches one selected position is
// one contiguous [H, D] row (A.X-K2 page: the cache holds expanded K/V; the
// indexer's positions are shared by all heads). Split form: the selection is
// split into chunks; a workgroup takes one chunk for 32 heads, keeps an
// online softmax per head and writes a partial state (m, l, o[Dv]); the merge
// kernel combines the chunks, applies the sigmoid gate (A.X-K2 page,
// "Attention output gate"; Spark-X2.5 page, forward pass) and stores the
// output. Whole-row form (bf16 grids of at least 256 (row, head) pairs):
// one workgroup per (row, head) whose 32 lane groups take slices of the list
// and are combined in LDS, with no partial states and no second launch.
//
// Lane layout: 8 lanes per head, 8 heads per wave, 4 waves = 32 heads. A
// head's K row (Dqk elements) is read as 16-byte chunks, lane j of the head
// taking chunks j, j+8, ...; each load instruction therefore covers 128
// contiguous bytes per head and 1 KiB per wave. The per-head dot product is
// reduced over the 8 lanes with three xor-swaps. Four tokens are in flight
// per step.
//
// The same kernels serve the fp32 path and sliding-window attention (the
// window is an implicit list p, p-1, ..., p-W+1). Attention sinks
// (openPangu-2.0 page §3.4, PAS) are n_sink extra entries in front of the
// list: entry r < n_sink is sink row r, visible to every query.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kG = 4;          // tokens in flight per step (G = 8 when a split holds 8 entries)
constexpr int kMaxSplit = 256;  // splits of one row's selection (merge weights live in LDS)

template <int DT>
struct Elem;
template <>
struct Elem<0> {  // fp32
  static constexpr int kPer16 = 4;
  __device__ static void unpack(const u32x4_t& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
};
template <>
struct Elem<1> {  // bf16
  static constexpr int kPer16 = 8;
  __device__ static void unpack(const u32x4_t& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  }
};

// Online softmax over the entries [e0, e1) of one query row for one head:
// the 8 lanes of the head (lane `sub` holds chunks sub, sub + 8, ...) load G
// tokens' K and V chunks at once, reduce the logits over the 8 lanes and
// update (m, l, o): o unnormalised, m in log2 units (qf is pre-scaled).
// WIN 0: indices list; WIN 1: window p, p-1, ..., p-window+1.
// KC / VC: 16-byte chunks per lane of a head's K / V row (chunk c of a row
// belongs to lane c % 8 of the head's 8 lanes). G: tokens whose loads are in
// flight together.
template <int DT, int WIN, int KC, int VC, int G>
__device__ __forceinline__ void gather_span(
    const float (&qf)[KC][Elem<DT>::kPer16], const char* __restrict__ kb,
    const char* __restrict__ vb, const char* __restrict__ skb, const char* __restrict__ svb,
    int n_sink, const int32_t* __restrict__ irow, int e0, int e1, int p, int64_t kvrow0,
    int Tbuf, int kv_offset, int window, int hk, int HKV, int DQK, int DV, int sub, int lane,
    float& m, float& l, float (&o)[VC][Elem<DT>::kPer16]) {
  using E = Elem<DT>;
  constexpr int EP = E::kPer16;
  constexpr int esz = DT ? 2 : 4;
  const int nck = DQK / EP, ncv = DV / EP;
  auto pos_of = [&](int ent) -> int {  // (sink entries: unused)
    const int le = ent - n_sink;
    if (WIN) return p - le;
    return (ent < e1 && le >= 0) ? irow[le] : -1;
  };
  int tn[G];  // positions of the next group (index loads run one group ahead)
#pragma unroll
  for (int g = 0; g < G; ++g) tn[g] = pos_of(e0 + g);

  for (int base = e0; base < e1; base += G) {
    int jrow[G];
    bool ok[G];
    bool snk[G];  // uniform over the head's 8 lanes: they share their entries
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int ent = base + g;
      const int t = tn[g];
      const int j = t - kv_offset;
      snk[g] = ent < n_sink;
      ok[g] = (ent < e1) && t >= 0 && t <= p && j >= 0 && j < Tbuf;
      if (WIN) ok[g] = ok[g] && ent - n_sink < window;
      if (snk[g]) ok[g] = ent < e1;
      jrow[g] = snk[g] ? ent : (ok[g] ? j : 0);
      DSA_CHECK(!ok[g] || (jrow[g] >= 0 && jrow[g] < (snk[g] ? n_sink : Tbuf)), jrow[g], ent);
    }
    // all K and V chunks of the group in flight at once
    u32x4_t kr[G][KC], vr[G][VC];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const char* krow =
          snk[g] ? skb + (((int64_t)jrow[g] * HKV + hk) * (int64_t)DQK) * esz
                 : kb + (((kvrow0 + jrow[g]) * HKV + hk) * (int64_t)DQK) * esz;
      const char* vrow =
          snk[g] ? svb + (((int64_t)jrow[g] * HKV + hk) * (int64_t)DV) * esz
                 : vb + (((kvrow0 + jrow[g]) * HKV + hk) * (int64_t)DV) * esz;
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const int c = sub + 8 * i;
        kr[g][i] = (c < nck) ? load16(krow + (int64_t)c * EP * esz) : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < VC; ++i) {
        const int c = sub + 8 * i;
        vr[g][i] = (c < ncv) ? load16(vrow + (int64_t)c * EP * esz) : u32x4_t{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) tn[g] = pos_of(base + G + g);

    // logits
    float x[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        float kf[EP];
        E::unpack(kr[g][i], kf);
#pragma unroll
        for (int e = 0; e < EP; ++e) dot = fmaf(qf[i][e], kf[e], dot);
      }
      // sum over the 8 lanes of this head (DPP lane exchanges, no LDS)
      dot += __uint_as_float(lane_xor_u32(__float_as_uint(dot), 1, lane));
      dot += __uint_as_float(lane_xor_u32(__float_as_uint(dot), 2, lane));
      dot += __uint_as_float(lane_xor_u32(__float_as_uint(dot), 4, lane));
      x[g] = ok[g] ? dot : -INFINITY;
    }
    float mx = m;
#pragma unroll
    for (int g = 0; g < G; ++g) mx = fmaxf(mx, x[g]);
    const float muse = (mx == -INFINITY) ? 0.0f : mx;
    const float alpha = exp2_hw(m - muse);
    m = mx;
    float pg[G];
    float ps = 0.0f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      pg[g] = exp2_hw(x[g] - muse);  // 0 for a skipped slot (x = -inf)
      ps += pg[g];
    }
    l = l * alpha + ps;
#pragma unroll
    for (int i = 0; i < VC; ++i)
#pragma unroll
      for (int e = 0; e < EP; ++e) o[i][e] *= alpha;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (!ok[g]) continue;  // never multiply a skipped row (it may hold anything)
#pragma unroll
      for (int i = 0; i < VC; ++i) {
        float vf[EP];
        E::unpack(vr[g][i], vf);
#pragma unroll
        for (int e = 0; e < EP; ++e) o[i][e] = fmaf(pg[g], vf[e], o[i][e]);
      }
    }
  }
}

// The query's chunks of one head, pre-scaled by scale * log2(e).
template <int DT, int KC>
__device__ __forceinline__ void load_q(const void* __restrict__ qv, int64_t row, int H, int hh,
                                       int DQK, int sub, float scale_log2,
                                       float (&qf)[KC][Elem<DT>::kPer16]) {
  using E = Elem<DT>;
  constexpr int EP = E::kPer16;
  constexpr int esz = DT ? 2 : 4;
  const int nck = DQK / EP;
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const int c = sub + 8 * i;
#pragma unroll
    for (int e = 0; e < EP; ++e) qf[i][e] = 0.0f;
    if (c < nck) {
      const u32x4_t x = load16((const char*)qv + ((row * H + hh) * (int64_t)DQK + c * EP) * esz);
      E::unpack(x, qf[i]);
#pragma unroll
      for (int e = 0; e < EP; ++e) qf[i][e] *= scale_log2;
    }
  }
}

// Split-K form: a workgroup takes entries split*per_split .. of one row for
// 32 heads (8 per wave) and writes their partial states for merge_kernel.
template <int DT, int WIN, int KC, int VC, int G>
__global__ __launch_bounds__(256) void gather_kernel(
    const void* __restrict__ qv, const void* __restrict__ kv, const void* __restrict__ vv,
    const void* __restrict__ skv, const void* __restrict__ svv, int n_sink,
    const int32_t* __restrict__ idx, float* __restrict__ part, int S, int Tbuf, int P,
    int kv_offset, int H, int HKV, int DQK, int DV, int nent, int per_split, int nsplit,
    int window, float scale_log2) {
  constexpr int EP = Elem<DT>::kPer16;
  const int split = (int)(blockIdx.x % (unsigned)nsplit);
  const int64_t row = blockIdx.x / (unsigned)nsplit;
  const int b = (int)(row / S), s = (int)(row % S);
  const int p = P + s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & 7;
  const int h = 32 * blockIdx.y + 8 * wave + (lane >> 3);
  const bool hvalid = h < H;
  const int hh = hvalid ? h : H - 1;
  const int hk = hh / (H / HKV);  // cache head: query heads come in groups of H / HKV
  const int ncv = DV / EP;

  float qf[KC][EP];
  load_q<DT, KC>(qv, row, H, hh, DQK, sub, scale_log2, qf);
  float m = -INFINITY, l = 0.0f;
  float o[VC][EP];
#pragma unroll
  for (int i = 0; i < VC; ++i)
#pragma unroll
    for (int e = 0; e < EP; ++e) o[i][e] = 0.0f;
  // entries 0 .. n_sink-1 are the sinks, n_sink .. nent-1 the list
  const int e0 = split * per_split;
  const int e1 = min(nent, e0 + per_split);
  const int32_t* irow = idx + row * (int64_t)(nent - n_sink);
  gather_span<DT, WIN, KC, VC, G>(qf, (const char*)kv, (const char*)vv, (const char*)skv,
                                  (const char*)svv, n_sink, irow, e0, e1, p, (int64_t)b * Tbuf,
                                  Tbuf, kv_offset, window, hk, HKV, DQK, DV, sub, lane, m, l, o);

  if (!hvalid) return;
  // partial state: [row][split][h][DV + 4] = o[0..DV), m, l (16-byte rows)
  float* pr = part + ((row * nsplit + split) * H + h) * (int64_t)(DV + 4);
#pragma unroll
  for (int i = 0; i < VC; ++i) {
    const int c = sub + 8 * i;
    if (c < ncv) {
#pragma unroll
      for (int e = 0; e < EP; ++e) pr[c * EP + e] = o[i][e];
    }
  }
  if (sub == 0) {
    pr[DV] = m;
    pr[DV + 1] = l;
  }
}

// Whole-row form (no partial states, no merge launch): one workgroup per
// (row, head); its 32 groups of 8 lanes take contiguous slices of the row's
// entries, and their (m, l, o) are combined in LDS as merge_kernel combines
// splits, then gated and stored.
constexpr int kWgGroups = 32;
template <int DT, int WIN, int KC, int VC, int G>
__global__ __launch_bounds__(256) void gather_wg_kernel(
    const void* __restrict__ qv, const void* __restrict__ kv, const void* __restrict__ vv,
    const void* __restrict__ skv, const void* __restrict__ svv, int n_sink,
    const int32_t* __restrict__ idx, const void* __restrict__ gate, void* __restrict__ out,
    int S, int Tbuf, int P, int kv_offset, int H, int HKV, int DQK, int DV, int nent,
    int window, float scale_log2, int gate_dim) {
  constexpr int EP = Elem<DT>::kPer16;
  constexpr int kDVMax = 8 * VC * EP;  // largest DV this instantiation serves
  __shared__ float gm[kWgGroups], gl[kWgGroups];
  __shared__ float go[kWgGroups][kDVMax];
  __shared__ float wsh[kWgGroups];
  const int64_t rh = blockIdx.x;  // row * H + h
  const int64_t row = rh / H;
  const int h = (int)(rh % H);
  const int b = (int)(row / S), s = (int)(row % S);
  const int p = P + s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int grp = tid >> 3, sub = lane & 7;
  const int hk = h / (H / HKV);
  const int ncv = DV / EP;

  float qf[KC][EP];
  load_q<DT, KC>(qv, row, H, h, DQK, sub, scale_log2, qf);
  float m = -INFINITY, l = 0.0f;
  float o[VC][EP];
#pragma unroll
  for (int i = 0; i < VC; ++i)
#pragma unroll
    for (int e = 0; e < EP; ++e) o[i][e] = 0.0f;
  const int per = (nent + kWgGroups - 1) / kWgGroups;
  const int e0 = min(nent, grp * per), e1 = min(nent, e0 + per);
  const int32_t* irow = idx + row * (int64_t)(nent - n_sink);
  gather_span<DT, WIN, KC, VC, G>(qf, (const char*)kv, (const char*)vv, (const char*)skv,
                                  (const char*)svv, n_sink, irow, e0, e1, p, (int64_t)b * Tbuf,
                                  Tbuf, kv_offset, window, hk, HKV, DQK, DV, sub, lane, m, l, o);
#pragma unroll
  for (int i = 0; i < VC; ++i) {
    const int c = sub + 8 * i;
    if (c < ncv) {
#pragma unroll
      for (int e = 0; e < EP; ++e) go[grp][c * EP + e] = o[i][e];
    }
  }
  if (sub == 0) {
    gm[grp] = m;
    gl[grp] = l;
  }
  __syncthreads();
  // weights 2^(m_g - M) over the groups (M = the largest m), as merge_kernel
  float M = -INFINITY;
#pragma unroll
  for (int g = 0; g < kWgGroups; ++g) M = fmaxf(M, gm[g]);
  const float Muse = (M == -INFINITY) ? 0.0f : M;
  if (tid < kWgGroups) wsh[tid] = gm[tid] != -INFINITY ? exp2f(gm[tid] - Muse) : 0.0f;
  __syncthreads();
  if (tid >= DV) return;
  float L = 0.0f, acc = 0.0f;
#pragma unroll
  for (int g = 0; g < kWgGroups; ++g) {
    L = fmaf(wsh[g], gl[g], L);
    acc = fmaf(go[g][tid], wsh[g], acc);
  }
  float gg = 1.0f;
  if (gate_dim == 1)
    gg = sigmoid_f32(DT ? bf16_to_f32(((const uint16_t*)gate)[rh]) : ((const float*)gate)[rh]);
  else if (gate_dim > 1)
    gg = sigmoid_f32(DT ? bf16_to_f32(((const uint16_t*)gate)[rh * DV + tid])
                        : ((const float*)gate)[rh * DV + tid]);
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const float r = acc * inv * gg;
  if (DT)
    ((uint16_t*)out)[rh * DV + tid] = f32_to_bf16(r);
  else
    ((float*)out)[rh * DV + tid] = r;
}

// One workgroup per (row, head). Thread i < nsplit reads split i's (m, l) and
// forms its weight w_i = 2^(m_i - M) (M = the largest m); the output columns
// are then summed over the splits by 256 / (DV / 4) groups of threads, each
// taking every G-th split with eight splits' loads in flight, and the groups
// are added through LDS. Every split is read once and the whole workgroup
// waits on only a few memory round trips.
template <int DT>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part,
                                                    const void* __restrict__ gate,
                                                    void* __restrict__ out, int H, int DV,
                                                    int nsplit, int gate_dim) {
  __shared__ float wsh[kMaxSplit];
  __shared__ float red[2][4];
  __shared__ float4 accsh[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t rh = blockIdx.x;  // row * H + h
  const int64_t row = rh / H;
  const int h = (int)(rh % H);
  const int64_t sstride = (int64_t)H * (DV + 4);
  const float* pbase = part + (row * nsplit * H + h) * (int64_t)(DV + 4);
  if (threadIdx.x == 0) DSA_CHECK(nsplit >= 1 && nsplit <= kMaxSplit, nsplit, kMaxSplit);
  // columns: group j of G sums splits j, j + G, ...; thread (j, cg) owns
  // output columns 4 cg .. 4 cg + 3. Its first kPre splits' columns are
  // loaded before anything else, together with the (m, l) pairs, so the
  // workgroup waits on one round of loads; longer lists loop after.
  const int ncg = DV / 4, G = 256 / ncg;
  const int cg = tid % ncg, j = tid / ncg;
  const float* pc = pbase + 4 * cg;
  // the gate values this thread applies, loaded up front with the rest
  float graw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (gate_dim == 1) {
    graw[0] = DT ? bf16_to_f32(((const uint16_t*)gate)[rh]) : ((const float*)gate)[rh];
  } else if (gate_dim > 1 && tid < ncg) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t gi = rh * DV + 4 * tid + c;
      graw[c] = DT ? bf16_to_f32(((const uint16_t*)gate)[gi]) : ((const float*)gate)[gi];
    }
  }
  constexpr int kPre = 32;
  float4 x[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int sp = j + G * u;
    x[u] = (j < G && sp < nsplit) ? *(const float4*)(pc + sp * sstride)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float mt = -INFINITY, lt = 0.0f;
  if (tid < nsplit) {
    mt = pbase[tid * sstride + DV];
    lt = pbase[tid * sstride + DV + 1];
  }
  float M = mt;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if (lane == 0) red[0][wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  const float Muse = (M == -INFINITY) ? 0.0f : M;
  const float wt = (tid < nsplit && mt != -INFINITY) ? exp2f(mt - Muse) : 0.0f;
  if (tid < nsplit) wsh[tid] = wt;
  float L = wt * lt;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off, 64);
  if (lane == 0) red[1][wave] = L;
  __syncthreads();
  L = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (j < G) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int sp = j + G * u;
      const float ww = sp < nsplit ? wsh[sp] : 0.0f;
      acc.x = fmaf(x[u].x, ww, acc.x);
      acc.y = fmaf(x[u].y, ww, acc.y);
      acc.z = fmaf(x[u].z, ww, acc.z);
      acc.w = fmaf(x[u].w, ww, acc.w);
    }
    for (int sp = j + G * kPre; sp < nsplit; sp += G) {
      const float4 y = *(const float4*)(pc + sp * sstride);
      const float ww = wsh[sp];
      acc.x = fmaf(y.x, ww, acc.x);
      acc.y = fmaf(y.y, ww, acc.y);
      acc.z = fmaf(y.z, ww, acc.z);
      acc.w = fmaf(y.w, ww, acc.w);
    }
  }
  accsh[tid] = acc;
  __syncthreads();
  if (tid >= ncg) return;
  float4 t = accsh[tid];
  for (int jj = 1; jj < G; ++jj) {
    const float4 y = accsh[jj * ncg + tid];
    t.x += y.x;
    t.y += y.y;
    t.z += y.z;
    t.w += y.w;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const float tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int d = 4 * tid + c;
    float gg = 1.0f;
    if (gate_dim == 1) gg = sigmoid_f32(graw[0]);
    if (gate_dim > 1) gg = sigmoid_f32(graw[c]);
    const float r = tv[c] * inv * gg;
    if (DT)
      ((uint16_t*)out)[rh * DV + d] = f32_to_bf16(r);
    else
      ((float*)out)[rh * DV + d] = r;
  }
}

struct Plan {
  int nsplit, per_split;
  int nsplit_bound;  // splits the workspace is sized for (>= nsplit, monotone in nent)
};

Plan make_plan(int64_t rows, int H, int64_t nent_in) {
  // (callers clamp the entry count to the visible positions; the clamp here
  // only keeps the arithmetic in range)
  const int nent = (int)std::min<int64_t>(nent_in, 0x3FFFFFFF);
  const int64_t hgroups = ((int64_t)H + 31) / 32;
  const int64_t base = rows * hgroups;
  // about 512 workgroups: enough to keep HBM busy, while fewer splits mean
  // less partial-state traffic through the merge
  int nsplit = (int)std::max<int64_t>(1, (512 + base - 1) / base);
  // at least one group of kG entries per split (measured on a 512-key window
  // decode: 16 entries per split 15.7 us, 8 12.1, 4 11.4)
  const int max_split = std::max(1, (nent + kG - 1) / kG);
  nsplit = std::min(std::min(nsplit, max_split), kMaxSplit);
  const int bound = nsplit;  // never decreases as nent grows
  int per = (nent + nsplit - 1) / nsplit;
  per = (per + kG - 1) / kG * kG;
  nsplit = (nent + per - 1) / per;
  return {nsplit, per, bound};
}

}  // namespace

#ifdef DSA_DEBUG
DSA_DEBUG_TAKE(attn_gather)
#endif

size_t gather_workspace_bytes(int64_t rows, int H, int Dv, int64_t nentries) {
  // sized for the bound, so a call with fewer entries (a window clamped to the
  // visible positions) never needs more than a query with more entries
  const Plan pl = make_plan(rows, H, nentries);
  return (size_t)rows * pl.nsplit_bound * H * (size_t)(Dv + 4) * sizeof(float);
}

hipError_t launch_gather(const void* q, const void* k, const void* v, const void* sink_k,
                         const void* sink_v, int n_sink, const int32_t* indices,
                         const void* gate, void* out, int B, int S, int T, int past_len,
                         int kv_offset, int H, int Hkv, int Dqk, int Dv, int topk,
                         int window, float sm_scale, int gate_dim, int dtype, void* workspace,
                         hipStream_t st) {
  const int64_t rows = (int64_t)B * S;
  const int nent = n_sink + (window > 0 ? window : topk);
  const float sl2w = sm_scale * DSA_LOG2E;
  // bf16 calls whose (row, head) grid fills the GPU take the whole-row kernel
  // (no partial states, no merge launch): decode-b8 245 -> 239 us back to
  // back. Few rows stay split across the GPU: one 2048-entry row of 32 heads
  // takes 17.5 us split and 36 us whole-row (one CU's bandwidth per head);
  // a 512-key window of 32 heads gains 1 us back to back but nothing inside
  // the decode step, and dims 256 lose (14 -> 18 us at spark-swa).
  if (dtype == 1 && Dv <= 256 && Dqk <= 256 && rows * H >= 256) {
    if (rows * H > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
#define DSA_WG_LAUNCH(WIN, KC, VC)                                                                 \
  hipLaunchKernelGGL((gather_wg_kernel<1, WIN, KC, VC, 2 * kG>), dim3((unsigned)(rows * H)), \
                     dim3(256), 0, st, q, k, v, sink_k, sink_v, n_sink, indices, gate, out, S, T,   \
                     past_len, kv_offset, H, Hkv, Dqk, Dv, nent, window, sl2w, gate_dim)
#define DSA_WG_VC(WIN, KC)                       \
  switch ((Dv + 63) / 64) {                      \
    case 1: DSA_WG_LAUNCH(WIN, KC, 1); break;    \
    case 2: DSA_WG_LAUNCH(WIN, KC, 2); break;    \
    case 3: DSA_WG_LAUNCH(WIN, KC, 3); break;    \
    default: DSA_WG_LAUNCH(WIN, KC, 4); break;   \
  }
#define DSA_WG_KC(WIN)                           \
  switch ((Dqk + 63) / 64) {                     \
    case 1: DSA_WG_VC(WIN, 1); break;            \
    case 2: DSA_WG_VC(WIN, 2); break;            \
    case 3: DSA_WG_VC(WIN, 3); break;            \
    default: DSA_WG_VC(WIN, 4); break;           \
  }
    if (window > 0) {
      DSA_WG_KC(1)
    } else {
      DSA_WG_KC(0)
    }
#undef DSA_WG_KC
#undef DSA_WG_VC
#undef DSA_WG_LAUNCH
    return hipGetLastError();
  }
  const Plan pl = make_plan(rows, H, nent);
  float* part = (float*)workspace;
  const dim3 grid((unsigned)(rows * pl.nsplit), (H + 31) / 32);
  if (rows * pl.nsplit > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const float sl2 = sm_scale * DSA_LOG2E;
  // splits of 8 entries (few rows: one long selection spread over the GPU)
  // load all 8 tokens at once; bf16 only (fp32 rows are twice the registers)
  const bool g8 = dtype == 1 && pl.per_split == 2 * kG;
#define DSA_GATHER_G(DT, WIN, KC, VC, GG)                                                          \
  hipLaunchKernelGGL((gather_kernel<DT, WIN, KC, VC, GG>), grid, dim3(256), 0, st, q, k, v, sink_k, \
                     sink_v, n_sink, indices, part, S, T, past_len, kv_offset, H, Hkv, Dqk, Dv,    \
                     nent, pl.per_split, pl.nsplit, window, sl2)
#define DSA_GATHER(DT, WIN, KC, VC)              \
  if (DT == 1 && g8)                             \
    DSA_GATHER_G(DT, WIN, KC, VC, (DT == 1 ? 2 * kG : kG)); \
  else                                           \
    DSA_GATHER_G(DT, WIN, KC, VC, kG)
#define DSA_GATHER_VC(DT, WIN, KC)            \
  switch (vc) {                               \
    case 1: DSA_GATHER(DT, WIN, KC, 1); break; \
    case 2: DSA_GATHER(DT, WIN, KC, 2); break; \
    case 3: DSA_GATHER(DT, WIN, KC, 3); break; \
    default: DSA_GATHER(DT, WIN, KC, 4); break; \
  }
#define DSA_GATHER_KC(DT, WIN)                  \
  switch (kc) {                                 \
    case 1: DSA_GATHER_VC(DT, WIN, 1); break;   \
    case 2: DSA_GATHER_VC(DT, WIN, 2); break;   \
    case 3: DSA_GATHER_VC(DT, WIN, 3); break;   \
    default: DSA_GATHER_VC(DT, WIN, 4); break;  \
  }
  // chunks per lane: bf16 rows carry 8 values per 16 bytes, fp32 rows 4
  const int per = dtype == 1 ? 64 : 32;
  const int kc = (Dqk + per - 1) / per, vc = (Dv + per - 1) / per;
  if (dtype == 1) {
    if (window > 0) {
      DSA_GATHER_KC(1, 1)
    } else {
      DSA_GATHER_KC(1, 0)
    }
  } else if (kc > 4 || vc > 4) {  // fp32 head dims above 128
    if (window > 0) {
      DSA_GATHER(0, 1, 8, 8);
    } else {
      DSA_GATHER(0, 0, 8, 8);
    }
  } else {
    if (window > 0) {
      DSA_GATHER_KC(0, 1)
    } else {
      DSA_GATHER_KC(0, 0)
    }
  }
#undef DSA_GATHER_KC
#undef DSA_GATHER_VC
#undef DSA_GATHER
#undef DSA_GATHER_G
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nrh = rows * H;
  if (nrh > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (dtype == 1)
    hipLaunchKernelGGL(merge_kernel<1>, dim3((unsigned)nrh), dim3(256), 0, st, part, gate, out, H,
                       Dv, pl.nsplit, gate_dim);
  else
    hipLaunchKernelGGL(merge_kernel<0>, dim3((unsigned)nrh), dim3(256), 0, st, part, gate, out, H,
                       Dv, pl.nsplit, gate_dim);
  return hipGetLastError();
}

}  // namespace dsa
