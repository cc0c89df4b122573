// Top-k / top-p warping of the sampling rows the walk visits, selected
// exactly by the workgroups that share a sequence's walk.
//
// What is computed ("LLM speculative decoding: EAGLE", jingming.pro, sec. 1:
// the distribution speculative sampling preserves is the one after the
// temperature, top-k and top-p processing; the draft's q gets the same
// processing because it must be what the drafted tokens were drawn from):
// tokens are ranked by probability, ties to the lower id; top-k keeps the
// first k; top-p then keeps the shortest rank prefix whose mass reaches
// top_p times the mass top-k kept; the kept probabilities are renormalised.
//
// Ranking by probability is ranking by logit (exp is monotone), so a kept set
// is "every token at or above a threshold" in the order (logit desc, id asc),
// and the threshold is found by radix selection over the row, with no sort:
//   level 0      256 bins of 1/8 octave of mass below the row max
//                (digit 255 = the max's bin, digit 0 = everything at least
//                2^-31.875 below it); the digit is a monotone function of the
//                logit, so its bins are contiguous in the ranking
//   levels 1-4   the bytes of an order-preserving 32-bit key of the logit,
//                among the tokens of the chosen level-0 bin
// Every level histograms the candidates (count and mass) per workgroup in
// LDS, publishes the histogram, meets at the sequence barrier and merges all
// of them in a fixed order; every workgroup then takes the same decision:
// the bin where the running count (top-k) or mass (top-p), summed from the
// top, reaches what is still needed. A selection ends as soon as the chosen
// bin is taken whole (top-k) or holds a single token (top-p); tokens with
// one logit value are ordered by id in a last pass only when the cut falls
// inside such a tie group.
//
// Masses are fixed point: a token's mass relative to the row max, exp2((z -
// m) log2(e) / T) <= 1, formed in fp64, times 2^S with S = min(52, 63 -
// ceil(log2 V)) (so V of them cannot overflow 64 bits), truncated to an
// integer. Integer sums do not depend on the order of addition, so the
// histograms can use LDS atomics and the result is still bitwise
// reproducible; a running mass is off by less than V * 2^-S of the max
// token's mass, which places the top-p cut as fp64 arithmetic would unless
// the cut lies within that distance of moving. The kept mass normalises the
// warped row.
#pragma once

#include "walk_common.h"

namespace sv {

typedef unsigned long long u64;

constexpr int kWarpBins = 256;

// A threshold in the ranking: a token is kept when (digit0, key, -id) is at
// least (b, key, -idx) lexicographically.
struct WarpThr {
  int b;
  uint32_t key;
  int idx;
};

__device__ __forceinline__ WarpThr warp_none() { return WarpThr{-1, 0u, 0x7fffffff}; }

// Order-preserving key of a finite logit (-0 ranks as +0).
__device__ __forceinline__ uint32_t warp_key(float z) {
  uint32_t u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Level-0 digit: 255 - floor(8 log2(e) (m - z) / T), clamped to [0, 255];
// l2t8 = 8 log2(e) / T. fl(m - z) and the product are monotone in z, so the
// digit never decreases as z grows.
__device__ __forceinline__ int warp_digit0(float z, float m, float l2t8) {
  const float t = (m - z) * l2t8;   // >= 0 when m is the row max; NaN goes to digit 0
  return 255 - ((t < 255.0f) ? ((t > 0.0f) ? (int)t : 0) : 255);
}

// l2td = log2(e) / T in fp64; scale = 2^S.
__device__ __forceinline__ u64 warp_qmass(float z, float m, double l2td, double scale) {
  return (u64)(exp2(((double)z - (double)m) * l2td) * scale);
}

__device__ __forceinline__ bool warp_in(const WarpThr& t, int d0, uint32_t key, int idx) {
  return d0 > t.b || (d0 == t.b && (key > t.key || (key == t.key && idx <= t.idx)));
}

// The kept set of one warped row: inside the top-k threshold a and the top-p
// threshold b (warp_none() for a step not applied).
struct WarpRow {
  WarpThr a, b;
  float m;     // row max
};

__device__ __forceinline__ bool warp_kept(const WarpRow& w, float z, int idx, float l2t8) {
  const int d0 = warp_digit0(z, w.m, l2t8);
  const uint32_t k = warp_key(z);
  return warp_in(w.a, d0, k, idx) && warp_in(w.b, d0, k, idx);
}

// Selection state of one row; uniform across the workgroup (lives in LDS).
struct WarpSel {
  float m;         // row max
  int active;      // still selecting
  int mode;        // 0: count (top-k), 1: mass (top-p)
  int level;       // level of the next histogram
  int b0;          // chosen level-0 digit
  uint32_t kp;     // chosen key bytes so far (level - 1 of them)
  u64 need;        // count or mass still to take from the current candidates
  u64 above;       // mass of the tokens ranked above the current candidates
  int tie_r;       // > 0: the cut is the tie_r-th id of the final tie group
  WarpThr rst;     // restriction: the earlier (top-k) threshold
  WarpThr res;     // the selected threshold
  u64 kept;        // kept mass (fixed point)
};

// Is token (z, idx) a candidate of the current level, and its digit.
__device__ __forceinline__ bool warp_candidate(const WarpSel& S, float z, int idx, float l2t8,
                                               int* digit) {
  const int d0 = warp_digit0(z, S.m, l2t8);
  const uint32_t key = warp_key(z);
  if (!warp_in(S.rst, d0, key, idx)) return false;
  if (S.level == 0) {
    *digit = d0;
    return true;
  }
  if (d0 != S.b0) return false;
  if (S.level > 1 && (key >> (40 - 8 * S.level)) != S.kp) return false;
  *digit = (int)((key >> (32 - 8 * S.level)) & 255u);
  return true;
}

// Histogram of the current level over tiles [t0, t1) of the active rows into
// LDS hc / hm ([2][256], zeroed by the caller). Level-0 digit 0 (the far
// tail, where most of a sharp row sits) is summed per lane and added once
// per wave.
template <bool VEC>
__device__ void warp_hist(const float* zt, const float* zd, int V, int t0, int t1, float l2t,
                          double l2td, double scale, const WarpSel* sel, unsigned* hc, u64* hm) {
  const int wave = threadIdx.x >> 6;
  const float l2t8 = l2t * 8.0f;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const WarpSel S = sel[r];
    if (!S.active) continue;
    const float* z = r ? zd : zt;
    unsigned tc = 0;
    u64 tm = 0;
    for (int t = t0 + wave; t < t1; t += 4) {
      float x[4];
      int idx[4];
      load_tile4<VEC>(z, t * kStatTile, V, x, idx);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int dig = 0;
        if (idx[e] >= V || !warp_candidate(S, x[e], idx[e], l2t8, &dig)) continue;
        const u64 q = warp_qmass(x[e], S.m, l2td, scale);
        if (S.level == 0 && dig == 0) {
          tc += 1u;
          tm += q;
        } else {
          atomicAdd(&hc[r * kWarpBins + dig], 1u);
          atomicAdd(&hm[r * kWarpBins + dig], q);
        }
      }
    }
    if (S.level == 0) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        tc += __shfl_xor(tc, o, 64);
        tm += __shfl_xor(tm, o, 64);
      }
      if (lane_id() == 0 && tc != 0u) {
        atomicAdd(&hc[r * kWarpBins], tc);
        atomicAdd(&hm[r * kWarpBins], tm);
      }
    }
  }
}

// Merge the G published histograms (thread t owns bin t) and take the
// level's decision for every active row. Returns false when a decision was
// impossible (a count or mass beyond what the candidates hold; not expected).
__device__ bool warp_choose(WarpSel* sel, const unsigned* pc, const u64* pm, int G, float top_p,
                            u64* s_tot /*[2][2][4]*/, int* s_found /*[2]*/) {
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  bool ok = true;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const WarpSel S = sel[r];
    if (!S.active) continue;
    u64 cnt = 0, ms = 0;
    for (int w = 0; w < G; ++w) {
      cnt += xload_u(pc + ((size_t)w * 2 + r) * kWarpBins + t);
      ms += xload_u(pm + ((size_t)w * 2 + r) * kWarpBins + t);
    }
    // suffix sums over the bins (bins >= t), by wave then across waves
    u64 sc = cnt, sm = ms;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const u64 yc = __shfl_down(sc, o, 64);
      const u64 ym = __shfl_down(sm, o, 64);
      if (lane + o < 64) {
        sc += yc;
        sm += ym;
      }
    }
    __syncthreads();
    if (lane == 0) {
      s_tot[(r * 2 + 0) * 4 + wave] = sc;
      s_tot[(r * 2 + 1) * 4 + wave] = sm;
    }
    if (t == 0) s_found[r] = 0;
    __syncthreads();
    u64 total_m = 0;
    for (int w = 0; w < 4; ++w) {
      total_m += s_tot[(r * 2 + 1) * 4 + w];
      if (w > wave) {
        sc += s_tot[(r * 2 + 0) * 4 + w];
        sm += s_tot[(r * 2 + 1) * 4 + w];
      }
    }
    u64 need = S.need;
    if (S.mode == 1 && S.level == 0) {
      // the top-p goal: the first rank whose running mass reaches top_p times
      // the mass of the candidates (the whole row, or what top-k kept)
      need = (u64)ceil((double)top_p * (double)total_m);
      if (need == 0) need = 1;
    }
    const u64 incl = S.mode ? sm : sc;
    const u64 own = S.mode ? ms : cnt;
    const u64 excl = incl - own;
    if (excl < need && need <= incl) {
      WarpSel n = S;
      const int L = S.level;
      const u64 c = cnt, bm = ms;
      n.above = S.above + (sm - ms);
      n.need = need - excl;
      if (L == 0) {
        n.b0 = t;
        n.kp = 0u;
      } else {
        n.kp = (S.kp << 8) | (uint32_t)t;
      }
      const uint32_t low = (L == 0) ? 0u : (n.kp << (32 - 8 * L));
      const bool whole = S.mode ? (c == 1) : (n.need == c);
      if (whole) {
        n.res = WarpThr{n.b0, low, 0x7fffffff};
        n.kept = n.above + bm;
        n.active = 0;
      } else if (L == 4) {
        // one logit value: equal masses; the cut is the r-th of them by id
        const u64 mm = bm / c;
        u64 rr = S.mode ? (n.need + mm - 1) / mm : n.need;
        if (rr > c) rr = c;
        n.kept = n.above + rr * mm;
        n.res = WarpThr{n.b0, n.kp, 0x7fffffff};
        n.tie_r = (rr < c) ? (int)rr : 0;
        n.active = 0;
      } else {
        n.level = L + 1;
      }
      sel[r] = n;
      s_found[r] = 1;
    }
    __syncthreads();
    if (!s_found[r]) {
      ok = false;
      if (t == 0) {
        sel[r].active = 0;
        sel[r].res = warp_none();
        sel[r].kept = 1ull;
      }
    }
    __syncthreads();
  }
  return ok;
}

// Number of tokens of the final tie group of row S in tiles [t0, t1).
__device__ int warp_tie_count(const float* z, int V, int t0, int t1, const WarpSel& S, float l2t8,
                              int* sh) {
  int n = 0;
  const int v1 = min(V, t1 * kStatTile);
  for (int v = t0 * kStatTile + (int)threadIdx.x; v < v1; v += kThreads) {
    const float x = z[v];
    const int d0 = warp_digit0(x, S.m, l2t8);
    const uint32_t key = warp_key(x);
    if (d0 == S.res.b && key == S.res.key && warp_in(S.rst, d0, key, v)) ++n;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o, 64);
  __syncthreads();
  if (lane_id() == 0) sh[threadIdx.x >> 6] = n;
  __syncthreads();
  return sh[0] + sh[1] + sh[2] + sh[3];
}

// Id of the r-th token (1-based, ascending id) of the final tie group of row S
// in tiles [t0, t1); -1 if there are fewer.
__device__ int warp_tie_find(const float* z, int V, int t0, int t1, const WarpSel& S, float l2t8,
                             int r, int* sh) {
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int v1 = min(V, t1 * kStatTile);
  int before = 0;
  for (int base = t0 * kStatTile; base < v1; base += kThreads) {
    const int v = base + (int)threadIdx.x;
    bool c = false;
    if (v < v1) {
      const float x = z[v];
      const int d0 = warp_digit0(x, S.m, l2t8);
      const uint32_t key = warp_key(x);
      c = d0 == S.res.b && key == S.res.key && warp_in(S.rst, d0, key, v);
    }
    const unsigned long long m = __ballot(c);
    __syncthreads();
    if (lane == 0) sh[wave] = __popcll(m);
    __syncthreads();
    int off = before;
    for (int w = 0; w < wave; ++w) off += sh[w];
    const int rank = off + __popcll(m & ((1ull << lane) - 1ull)) + 1;
    const int tile_total = sh[0] + sh[1] + sh[2] + sh[3];
    __syncthreads();
    if (c && rank == r) sh[4] = v;
    if (before < r && r <= before + tile_total) {
      __syncthreads();
      return sh[4];
    }
    before += tile_total;
  }
  return -1;
}

}  // namespace sv
