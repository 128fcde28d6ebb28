// idx_tiles.h -- the causal tile schedule shared by the prefill indexer
// kernels (bf16 in index_scores.hip, FP8 in index_fp8.hip).
//
// A workgroup computes one (query tile, key tile) unit of TQ queries x 512
// keys. Only units on or below the causal diagonal are launched: query tiles
// are paired (j, nqt-1-j) so that every pair costs about the same, and pairs
// are dealt to the 8 XCDs round-robin (block id mod 8). The same workgroups
// write -inf over the pair's units above the diagonal, so no separate pass
// re-touches HBM.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kIdxTileK = 512;  // keys per workgroup

// Key tiles a query tile of tq queries needs (the causal triangle).
__host__ __device__ __forceinline__ int idx_tiles_for_qtile(int qt, int tq, int S, int P,
                                                            int nkt) {
  const int last_q = min((qt + 1) * tq, S) - 1;
  const int c = (P + last_q) / kIdxTileK + 1;
  return c < nkt ? c : nkt;
}

struct IdxTile {
  int qt, kt;  // the unit this workgroup multiplies
  int v;       // its index among the pair's ca + cb workgroups
  int qa, qb;  // the pair's query tiles
  int ca, cb;  // their numbers of key tiles on or below the diagonal
};

// Unit of workgroup pid; false when pid has none (grid padding).
__device__ __forceinline__ bool idx_tile_of(int pid, int tq, int S, int P, int nqt, int nkt,
                                            int npairs, int maxlen, IdxTile* o) {
  const int xcd = pid & 7;
  const int n = pid >> 3;
  const int slot = n / maxlen;
  int u = n - slot * maxlen;
  const int j = slot * 8 + xcd;
  if (j >= npairs) return false;
  o->qa = j;
  o->qb = nqt - 1 - j;
  o->ca = idx_tiles_for_qtile(o->qa, tq, S, P, nkt);
  o->cb = o->qb == o->qa ? 0 : idx_tiles_for_qtile(o->qb, tq, S, P, nkt);
  o->v = u;
  if (u < o->ca) {
    o->qt = o->qa;
    o->kt = u;
    return true;
  }
  if (o->qb == o->qa) return false;
  u -= o->ca;
  if (u >= o->cb) return false;
  o->qt = o->qb;
  o->kt = u;
  return true;
}

// -inf over the pair's units above the diagonal: the (nkt - ca) + (nkt - cb)
// units are dealt round-robin to its ca + cb workgroups (256 threads each).
template <int TQ>
__device__ __forceinline__ void idx_fill_upper(float* scores, const IdxTile& t, int b, int S,
                                               int T, int nkt, bool vec) {
  const int na = nkt - t.ca, nunits = na + (t.qb == t.qa ? 0 : nkt - t.cb);
  for (int un = t.v; un < nunits; un += t.ca + t.cb) {
    const int fq = un < na ? t.qa : t.qb;
    const int fk = un < na ? t.ca + un : t.cb + (un - na);
    const int tid = threadIdx.x;
#pragma unroll
    for (int rr = 0; rr < TQ; rr += 16) {
      const int fs = fq * TQ + rr + tid / 16;
      if (fs >= S) continue;
      float* frow = scores + ((int64_t)b * S + fs) * T;
#pragma unroll
      for (int i = 0; i < kIdxTileK / 64; ++i) {
        const int t0 = fk * kIdxTileK + 4 * (tid % 16 + 16 * i);
        if (vec && t0 + 3 < T) {
          *(float4*)(frow + t0) = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (t0 + e < T) frow[t0 + e] = -INFINITY;
        }
      }
    }
  }
}

// Key-stationary form for long contexts: the pair's workgroups each take one
// key tile u and multiply it with qb (the later query tile, u < cb) and, when
// u < ca, with qa as well, so the key tile is loaded once for both (with
// two = false the plain schedule above, one unit per workgroup). The fill
// deals the pair's units above the diagonal over its nwg workgroups.
struct IdxTile2 {
  int kt, v, nwg;  // key tile; index among the pair's nwg workgroups
  int q1, q2;      // query tiles to multiply (q2 < 0: just q1)
  int qa, qb, ca, cb;
};

__device__ __forceinline__ bool idx_tile2_of(int pid, int tq, int S, int P, int nqt, int nkt,
                                             int npairs, int maxlen, bool two, IdxTile2* o) {
  const int xcd = pid & 7;
  const int n = pid >> 3;
  const int slot = n / maxlen;
  const int u = n - slot * maxlen;
  const int j = slot * 8 + xcd;
  if (j >= npairs) return false;
  o->qa = j;
  o->qb = nqt - 1 - j;
  o->ca = idx_tiles_for_qtile(o->qa, tq, S, P, nkt);
  o->cb = o->qb == o->qa ? 0 : idx_tiles_for_qtile(o->qb, tq, S, P, nkt);
  o->v = u;
  o->q2 = -1;
  if (!two || o->cb == 0) {  // one unit per workgroup
    o->nwg = o->ca + o->cb;
    if (u >= o->nwg) return false;
    o->q1 = u < o->ca ? o->qa : o->qb;
    o->kt = u < o->ca ? u : u - o->ca;
    return true;
  }
  o->nwg = o->cb;  // ca <= cb: qb's causal range covers qa's
  if (u >= o->nwg) return false;
  o->kt = u;
  o->q1 = o->qb;
  if (u < o->ca) o->q2 = o->qa;
  return true;
}

template <int TQ>
__device__ __forceinline__ void idx_fill_upper2(float* scores, const IdxTile2& t, int b, int S,
                                                int T, int nkt, bool vec) {
  const int na = nkt - t.ca, nunits = na + (t.qb == t.qa ? 0 : nkt - t.cb);
  for (int un = t.v; un < nunits; un += t.nwg) {
    const int fq = un < na ? t.qa : t.qb;
    const int fk = un < na ? t.ca + un : t.cb + (un - na);
    const int tid = threadIdx.x;
#pragma unroll
    for (int rr = 0; rr < TQ; rr += 16) {
      const int fs = fq * TQ + rr + tid / 16;
      if (fs >= S) continue;
      float* frow = scores + ((int64_t)b * S + fs) * T;
#pragma unroll
      for (int i = 0; i < kIdxTileK / 64; ++i) {
        const int t0 = fk * kIdxTileK + 4 * (tid % 16 + 16 * i);
        if (vec && t0 + 3 < T) {
          *(float4*)(frow + t0) = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (t0 + e < T) frow[t0 + e] = -INFINITY;
        }
      }
    }
  }
}

// Grid of the schedule for one batch row (x) -- host side.
struct IdxGrid {
  int nqt, nkt, npairs, maxlen;
  int64_t gx;
};

inline IdxGrid idx_grid(int S, int T, int P, int tq) {
  IdxGrid g;
  g.nqt = (int)(((int64_t)S + tq - 1) / tq);
  g.nkt = (int)(((int64_t)T + kIdxTileK - 1) / kIdxTileK);
  g.npairs = (g.nqt + 1) / 2;
  g.maxlen = 1;
  for (int j = 0; j < g.npairs; ++j) {
    int len = idx_tiles_for_qtile(j, tq, S, P, g.nkt);
    if (g.nqt - 1 - j != j) len += idx_tiles_for_qtile(g.nqt - 1 - j, tq, S, P, g.nkt);
    if (len > g.maxlen) g.maxlen = len;
  }
  g.gx = 8 * (int64_t)((g.npairs + 7) / 8) * g.maxlen;
  return g;
}

// Grid of the key-stationary form (two = true): pairs have cb workgroups.
inline IdxGrid idx_grid2(int S, int T, int P, int tq, bool two) {
  IdxGrid g = idx_grid(S, T, P, tq);
  if (!two) return g;
  g.maxlen = 1;
  for (int j = 0; j < g.npairs; ++j) {
    const int qb = g.nqt - 1 - j;
    const int len = idx_tiles_for_qtile(qb, tq, S, P, g.nkt);  // cb (the middle tile: ca)
    if (len > g.maxlen) g.maxlen = len;
  }
  g.gx = 8 * (int64_t)((g.npairs + 7) / 8) * g.maxlen;
  return g;
}

}  // namespace dsa
