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

constexpr int kLevelSub = 5;      // the sub-bin histogram of a dense level-0 bin
constexpr int kWarpCapW = 256;    // gathered candidates per workgroup and row
constexpr int kWarpCapT = 1024;   // gathered candidates per row in total (sorted in LDS)

// Sub-bin digit of t = (m - z) * l2t8 inside its level-0 bin (t < 255):
// 255 - floor(256 * frac(t)). 256 * t is exact in fp32, so the sub-bins nest
// in the level-0 bins and stay monotone in z.
__device__ __forceinline__ int warp_d1(float t) {
  const float tc = (t > 0.0f) ? t : 0.0f;
  return 255 - ((int)(tc * 256.0f) - 256 * (int)tc);
}

// Selection state of one row; uniform across the workgroup (lives in LDS).
struct WarpSel {
  float m;         // row max
  int active;      // still selecting
  int gather;      // the next pass gathers the candidates (else it histograms `level`)
  int mode;        // 0: count (top-k), 1: mass (top-p)
  int level;       // next histogram: 0 mass digit, kLevelSub sub-bins, 1..4 key bytes
  int b0;          // chosen level-0 digit
  int sub;         // candidates restricted to sub-bin b1 of bin b0
  int b1;
  int nomass;      // top-k alone: the level-0 histogram counts only, and the gather pass
                   // sums the exact mass ranked above the candidates (and of a whole bin)
  int whole;       // nomass: bin b0 is kept whole; the gather pass only sums its mass
  uint32_t kp;     // chosen key bytes so far (level - 1 of them)
  u64 need;        // count or mass still to take from the current candidates
  u64 above;       // mass of the tokens ranked above the current candidates
  u64 need0;       // need and above right after the level-0 decision (the top-p step
  u64 above0;      // derives its level-0 histogram from the top-k step's)
  int tie_r;       // > 0: the cut is the tie_r-th id of the final tie group
  WarpThr rst;     // restriction: the earlier (top-k) threshold
  WarpThr res;     // the selected threshold
  u64 kept;        // kept mass (fixed point)
};

// Wave-uniform copies (the selection state lives in LDS; reading it through
// readfirstlane tells the compiler it is uniform, so the mode tests below are
// scalar branches outside the token loops).
__device__ __forceinline__ int rfl_i(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float rfl_f(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
__device__ __forceinline__ WarpThr warp_thr_uniform(const WarpThr& t) {
  return WarpThr{rfl_i(t.b), (uint32_t)rfl_i((int)t.key), rfl_i(t.idx)};
}
__device__ __forceinline__ WarpRow warp_row_uniform(const WarpRow& w) {
  return WarpRow{warp_thr_uniform(w.a), warp_thr_uniform(w.b), rfl_f(w.m)};
}

// What one pass does for one row.
enum { kPassCount0 = 0, kPassHist0 = 1, kPassHistSub = 2, kPassHistKey = 3, kPassGather = 4 };

// One row's pass over tiles [t0, t1), specialised by KIND: a histogram into
// hc / hm ([256] of this row; level-0 digit 0, the far tail, summed per lane
// and added once per wave), or the candidates appended to this workgroup's
// list gl ([kWarpCapW][key, mass], counted in *gcnt; entries past the
// capacity are only counted) with, for a nomass row, the exact masses ranked
// above the candidates and of the candidates summed into gred[0], gred[1].
template <bool VEC, int KIND>
__device__ __forceinline__ void warp_row_pass(const float* z, int V, int t0, int t1, float m,
                                              float l2t8, double l2td, double scale,
                                              WarpThr rst, int b0, int b1, int sub, int level,
                                              uint32_t kp, int nomass, int whole, unsigned* hc,
                                              u64* hm, unsigned* gcnt, u64* gred, u64* gl) {
  const int wave = threadIdx.x >> 6;
  unsigned tc = 0;
  u64 tm = 0, abv = 0, binm = 0;
  constexpr int kU = 4;   // tiles in flight per wave
  for (int t = t0 + wave; t < t1; t += 4 * kU) {
    float x[kU][4];
    int idx[kU][4];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int tt = t + 4 * u;
      if (tt < t1) {
        load_tile4<VEC>(z, tt * kStatTile, V, x[u], idx[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) { x[u][e] = 0.0f; idx[u][e] = V; }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int id = idx[u][e];
        const float zv = x[u][e];
        const float tv = (m - zv) * l2t8;
        const int d0 = 255 - ((tv < 255.0f) ? ((tv > 0.0f) ? (int)tv : 0) : 255);
        const uint32_t key = warp_key(zv);
        const bool ok = id < V && warp_in(rst, d0, key, id);
        if (KIND == kPassCount0) {
          if (ok && d0 == 0) tc += 1u;
          else if (ok) atomicAdd(&hc[d0], 1u);
        } else if (KIND == kPassHist0) {
          if (ok) {
            const u64 q = warp_qmass(zv, m, l2td, scale);
            if (d0 == 0) {
              tc += 1u;
              tm += q;
            } else {
              atomicAdd(&hc[d0], 1u);
              atomicAdd(&hm[d0], q);
            }
          }
        } else if (KIND == kPassHistSub) {
          if (ok && d0 == b0) {
            const int dig = warp_d1(tv);
            atomicAdd(&hc[dig], 1u);
            atomicAdd(&hm[dig], warp_qmass(zv, m, l2td, scale));
          }
        } else if (KIND == kPassHistKey) {
          const bool c = ok && d0 == b0 && (!sub || warp_d1(tv) == b1) &&
                         (level == 1 || (key >> (40 - 8 * level)) == kp);
          if (c) {
            const int dig = (int)((key >> (32 - 8 * level)) & 255u);
            atomicAdd(&hc[dig], 1u);
            atomicAdd(&hm[dig], warp_qmass(zv, m, l2td, scale));
          }
        } else {
          const int d1 = sub ? warp_d1(tv) : 0;
          const bool cand = ok && d0 == b0 && (!sub || d1 == b1);
          const bool above = ok && nomass && (d0 > b0 || (sub && d0 == b0 && d1 > b1));
          if (cand) {
            const u64 q = warp_qmass(zv, m, l2td, scale);
            if (nomass) binm += q;
            if (!whole) {
              const unsigned pos = atomicAdd(gcnt, 1u);
              if (pos < (unsigned)kWarpCapW) {
                u64* slot = gl + (size_t)pos * 2;
                xstore_u(slot, ((u64)key << 32) | (u64)(0xFFFFFFFFu - (uint32_t)id));
                xstore_u(slot + 1, q);
              }
            }
          } else if (above) {
            abv += warp_qmass(zv, m, l2td, scale);
          }
        }
      }
  }
  if (KIND == kPassCount0 || KIND == kPassHist0) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      tc += __shfl_xor(tc, o, 64);
      if (KIND == kPassHist0) tm += __shfl_xor(tm, o, 64);
    }
    if (lane_id() == 0 && tc != 0u) {
      atomicAdd(&hc[0], tc);
      if (KIND == kPassHist0) atomicAdd(&hm[0], tm);
    }
  } else if (KIND == kPassGather) {
    if (nomass) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        abv += __shfl_xor(abv, o, 64);
        binm += __shfl_xor(binm, o, 64);
      }
      if (lane_id() == 0) {
        atomicAdd(&gred[0], abv);
        atomicAdd(&gred[1], binm);
      }
    }
  }
}

// One pass over tiles [t0, t1) for every active row (see warp_row_pass);
// hc / hm are [2][256] and zeroed by the caller, gcnt [2], gred [2][2],
// glist this workgroup's [2 rows][kWarpCapW][2].
template <bool VEC>
__device__ __forceinline__ void warp_pass(const float* zt, const float* zd, int V, int t0, int t1,
                                          float l2t, double l2td, double scale,
                                          const WarpSel* sel, unsigned* hc, u64* hm,
                                          unsigned* gcnt, u64* gred, u64* glist) {
  const float l2t8 = l2t * 8.0f;
#pragma unroll 1
  for (int r = 0; r < 2; ++r) {
    const WarpSel& S = sel[r];
    if (!rfl_i(S.active)) continue;
    const float m = rfl_f(S.m);
    const WarpThr rst = warp_thr_uniform(S.rst);
    const int gather = rfl_i(S.gather), level = rfl_i(S.level), nomass = rfl_i(S.nomass);
    const int b0 = rfl_i(S.b0), b1 = rfl_i(S.b1), sub = rfl_i(S.sub), whole = rfl_i(S.whole);
    const uint32_t kp = (uint32_t)rfl_i((int)S.kp);
    const float* z = r ? zd : zt;
    unsigned* hcr = hc + r * kWarpBins;
    u64* hmr = hm + r * kWarpBins;
    u64* gl = glist + (size_t)r * kWarpCapW * 2;
#define SV_WARP_ROW(K)                                                                      \
  warp_row_pass<VEC, K>(z, V, t0, t1, m, l2t8, l2td, scale, rst, b0, b1, sub, level, kp,   \
                        nomass, whole, hcr, hmr, gcnt + r, gred + 2 * r, gl)
    if (gather) SV_WARP_ROW(kPassGather);
    else if (level == 0 && nomass) SV_WARP_ROW(kPassCount0);
    else if (level == 0) SV_WARP_ROW(kPassHist0);
    else if (level == kLevelSub) SV_WARP_ROW(kPassHistSub);
    else SV_WARP_ROW(kPassHistKey);
#undef SV_WARP_ROW
  }
}

// The level's decision for row r from its histogram: thread t holds bin t's
// count and mass (cnt, ms), merged over the workgroups or derived. Every
// workgroup decides identically. keep_c / keep_m (or null) receive the
// level-0 histogram for a later top-p step. Returns false when no bin could
// be chosen (a count or mass beyond what the candidates hold; not expected).
__device__ __forceinline__ bool warp_decide(WarpSel* sel, int r, u64 cnt, u64 ms, float top_p,
                            u64* s_tot /*[8]*/, int* s_found, unsigned* keep_c, u64* keep_m) {
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const WarpSel S = sel[r];
  if (keep_c != nullptr && S.level == 0) {
    keep_c[t] = (unsigned)cnt;
    keep_m[t] = ms;
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
    s_tot[wave] = sc;
    s_tot[4 + wave] = sm;
  }
  if (t == 0) *s_found = 0;
  __syncthreads();
  u64 total_m = 0;
  for (int w = 0; w < 4; ++w) {
    total_m += s_tot[4 + w];
    if (w > wave) {
      sc += s_tot[w];
      sm += s_tot[4 + w];
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
      n.need0 = n.need;
      n.above0 = n.above;
      if (S.mode ? (c == 1) : (n.need == c)) {      // the bin is taken whole
        if (S.nomass) {
          n.whole = 1;                              // its exact mass comes from a pass
          n.gather = 1;
        } else {
          n.res = WarpThr{t, 0u, 0x7fffffff};
          n.kept = n.above + bm;
          n.active = 0;
        }
      } else if (c <= (u64)kWarpCapT || S.nomass) {
        // (a nomass row gathers even a dense bin: the pass also sums the
        // exact mass ranked above it, and an overflowing list then falls
        // back to the key-byte histograms)
        n.gather = 1;
      } else {
        n.level = (t == 0) ? 1 : kLevelSub;         // the far tail has no sub-bins
      }
    } else if (L == kLevelSub) {
      n.b1 = t;
      n.sub = 1;
      if (c <= (u64)kWarpCapT) n.gather = 1;
      else n.level = 1;
    } else {
      n.kp = (S.kp << 8) | (uint32_t)t;
      if (S.mode ? (c == 1) : (n.need == c)) {
        n.res = WarpThr{n.b0, n.kp << (32 - 8 * L), 0x7fffffff};
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
    }
    sel[r] = n;
    *s_found = 1;
  }
  __syncthreads();
  const bool ok = *s_found != 0;
  if (!ok && t == 0) {
    sel[r].active = 0;
    sel[r].res = warp_none();
    sel[r].kept = 1ull;
  }
  __syncthreads();
  return ok;
}

// Merge the G published histograms of row r (all loads in flight, clamped
// index, fixed-order sum) and decide.
__device__ __forceinline__ bool warp_choose_row(WarpSel* sel, int r, const unsigned* pc, const u64* pm, int G,
                                float top_p, u64* s_tot, int* s_found, unsigned* keep_c,
                                u64* keep_m) {
  const int t = threadIdx.x;
  unsigned cw[kWalkGroupsMax];
  u64 mw[kWalkGroupsMax];
#pragma unroll
  for (int w = 0; w < kWalkGroupsMax; ++w) {
    const size_t at = ((size_t)min(w, G - 1) * 2 + r) * kWarpBins + t;
    cw[w] = xload_u(pc + at);
    mw[w] = xload_u(pm + at);
  }
  u64 cnt = 0, ms = 0;
#pragma unroll
  for (int w = 0; w < kWalkGroupsMax; ++w) {
    if (w < G) {
      cnt += cw[w];
      ms += mw[w];
    }
  }
  return warp_decide(sel, r, cnt, ms, top_p, s_tot, s_found, keep_c, keep_m);
}

// Finish a gathering row r: read the G workgroups' published counts (and,
// nomass, the exact masses above the candidates and of the candidates:
// counts is [G][2 rows][count, above, bin]) and lists, sort the candidates
// by (key desc, id asc) in LDS (sk, sm hold kWarpCapT entries) and cut at
// what is still needed: the need-th candidate (top-k) or the first whose
// running mass reaches it (top-p). A whole nomass bin only takes its mass.
// When a list overflowed, the row falls back to the key-byte histograms.
// Returns false when the cut could not be placed (not expected).
__device__ __forceinline__ bool warp_gather_finish(WarpSel* sel, int r, const u64* counts, const u64* lists,
                                   int G, u64* sk, u64* sm, u64* s_tot /*[8]*/,
                                   int* s_cnt /*[kWalkGroupsMax]*/, int* s_found) {
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  WarpSel S = sel[r];
  __syncthreads();
  if (t < G) {                           // sm / sk serve as scratch for the parts here
    const u64* c = counts + ((size_t)t * 2 + r) * 3;
    s_cnt[t] = (int)xload_u(c);
    sm[t] = xload_u(c + 1);
    sk[t] = xload_u(c + 2);
  }
  __syncthreads();
  int total = 0;
  bool over = false;
  u64 above = 0, binm = 0;
  for (int w = 0; w < G; ++w) {
    total += s_cnt[w];
    over = over || s_cnt[w] > kWarpCapW;
    above += sm[w];
    binm += sk[w];
  }
  __syncthreads();
  if (S.nomass) S.above = above;         // exact: every token ranked above the candidates
  if (S.whole) {
    if (t == 0) {
      WarpSel n = S;
      n.res = WarpThr{S.b0, 0u, 0x7fffffff};
      n.kept = S.above + binm;
      n.active = 0;
      n.gather = 0;
      sel[r] = n;
    }
    __syncthreads();
    return true;
  }
  if (over || total > kWarpCapT || total < 1) {
    if (t == 0) {
      sel[r].above = S.above;
      sel[r].gather = 0;
      sel[r].level = 1;
    }
    __syncthreads();
    return total >= 1;
  }
  int n = 2;
  while (n < total) n <<= 1;
  for (int i = t; i < n; i += kThreads) {
    u64 k = 0ull, q = 0ull;
    if (i < total) {
      int w = 0, off = 0;
      while (off + s_cnt[w] <= i) {    // the list holding entry i (prefix over workgroups)
        off += s_cnt[w];
        ++w;
      }
      const u64* e = lists + (((size_t)w * 2 + r) * kWarpCapW + (i - off)) * 2;
      k = xload_u(e);
      q = xload_u(e + 1);
    }
    sk[i] = k;
    sm[i] = q;
  }
  __syncthreads();
  // bitonic sort, descending by key (padding entries have key 0 and sink)
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < n; i += kThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;
          const u64 a = sk[i], b = sk[j];
          if (desc ? (a < b) : (a > b)) {
            sk[i] = b;
            sk[j] = a;
            const u64 qa = sm[i];
            sm[i] = sm[j];
            sm[j] = qa;
          }
        }
      }
      __syncthreads();
    }
  }
  // running masses: every thread owns a contiguous chunk of n / 256 entries
  const int per = (n + kThreads - 1) / kThreads;
  const int i0 = min(n, t * per), i1 = min(n, i0 + per);
  u64 own = 0;
  for (int i = i0; i < i1; ++i) own += sm[i];
  u64 incl = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const u64 y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (t == 0) *s_found = 0;
  if (lane == 63) s_tot[wave] = incl;
  __syncthreads();
  u64 run = incl - own;
  for (int w = 0; w < wave; ++w) run += s_tot[w];
  // run = mass of the entries before this chunk
  for (int i = i0; i < i1 && i < total; ++i) {
    const u64 after = run + sm[i];
    const bool cut = S.mode ? (run < S.need && S.need <= after) : (i + 1 == (int)S.need);
    if (cut) {
      WarpSel ns = S;
      ns.res = WarpThr{S.b0, (uint32_t)(sk[i] >> 32), (int)(0xFFFFFFFFu - (uint32_t)sk[i])};
      ns.kept = S.above + after;
      ns.active = 0;
      ns.gather = 0;
      sel[r] = ns;
      *s_found = 1;
    }
    run = after;
  }
  __syncthreads();
  const bool ok = *s_found != 0;
  if (!ok && t == 0) {
    sel[r].active = 0;
    sel[r].gather = 0;
    sel[r].res = warp_none();
    sel[r].kept = 1ull;
  }
  __syncthreads();
  return ok;
}

// Number of tokens of the final tie group of row S in tiles [t0, t1).
__device__ __forceinline__ int warp_tie_count(const float* z, int V, int t0, int t1, const WarpSel& S, float l2t8,
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
__device__ __forceinline__ int warp_tie_find(const float* z, int V, int t0, int t1, const WarpSel& S, float l2t8,
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
