// Tree preparation: validates each sequence's packed tree and inputs and
// derives what the attention and sampling kernels need from the parent array.
//
// The packed tree and its mask follow "LLM speculative decoding: EAGLE"
// (jingming.pro) sec. 4.2 "Attention Mask" and the EAGLE-2 excerpts
// (modelers.csdn.net) sec. 2.3.2: the drafted nodes are flattened into one
// sequence and node j may see the prefix, its ancestors and itself. Here the
// ancestor-or-self set of node j is a 64-bit mask (bit a = node a), and the
// children of every slot are listed in ascending node index, the order in
// which multi-round speculative sampling tests them.
#include <algorithm>

#include "sv_internal.h"

namespace sv {

// Attention scheduling: one more block of the preparation launch per
// candidate split length c (in key tiles). Its items are the (sequence,
// split) pairs of every sequence whose prefix length is valid: a range of T
// key tiles makes ceil(T / c) splits, all of c tiles but the last. They are
// listed longest first (a counting sort on the tile count; the order inside
// one count is that of the atomics and does not matter, since each item
// writes its own results). The hardware hands out blocks in grid order to
// whichever CU frees first, so this is longest-processing-time-first list
// scheduling: the short last splits fill the end of the grid instead of
// leaving CUs idle behind long ones.
//
// The block also estimates the makespan of that schedule. The HG attention
// blocks of an item over P CUs act like one item on each of M = P / HG
// machines. A block costs its tiles plus a fixed 8.5 tiles (the query
// loads, the pipeline fill and the partial stores, measured at about 8.5
// key tiles' streaming time), counted in half tiles. The full splits, all
// equal, spread evenly; the last splits (at most one per sequence) then go
// one by one, longest first, to the least loaded machine, as the hardware's
// greedy dispatch places them (one machine per lane, so M <= 64). With more
// machines, or more than kExactLasts last splits, the estimate assigns every
// item in snake order (0..M-1, M-1..0, ...) instead, a close and cheaper
// stand-in. The attention kernels take the candidate with the lowest
// estimate.
struct SchedArgs {
  int32_t* sched;      // kSchedCands schedules, `stride` int32 apart
  int stride;          // int32 per schedule: 4 of header, then B * max_splits items
  int max_splits;      // item = b * max_splits + split
  int machines;        // M
  // M when some sequence samples (T > 0) and attention runs beside sampling
  // on a share of the CUs (0: never). A greedy walk is short, so attention
  // beside it keeps every CU and ends first.
  int side_machines;
  const float* temperature;
  int cand[kSchedCands];
};

constexpr int kExactLasts = 128;
constexpr uint32_t kLoadSat = (1u << 26) - 1;   // machine loads saturate here (half tiles)

// Key tiles of sequence b's attention range; 0 when its prefix length is not
// in [1, max_prefix] (such a sequence is flagged and gets no attention block).
__device__ __forceinline__ int seq_key_tiles(const int32_t* __restrict__ kv_offset, int b, int N,
                                             int max_prefix) {
  const long long total = (long long)kv_offset[b + 1] - kv_offset[b];
  const long long L = total - N;
  if (L < 1 || L > max_prefix) return 0;
  return (int)((total + kKeyTile - 1) / kKeyTile);
}

__device__ __forceinline__ unsigned long long block_cost(int tiles) {
  return 17ull + 2ull * (unsigned)tiles;
}

__device__ void attn_candidate(int B, int N, int max_prefix, const int32_t* __restrict__ kv_offset,
                               const SchedArgs& sa, int j) {
  const int lane = threadIdx.x;             // one wave
  const int c = sa.cand[j];
  int M = sa.machines;
  if (sa.side_machines > 0) {
    bool sampled = false;
    for (int b = lane; b < B; b += 64) sampled |= sa.temperature[b] > 0.0f;
    if (__ballot(sampled) != 0ull) M = sa.side_machines;
  }
  int32_t* out = sa.sched + (size_t)j * sa.stride;
  __shared__ int cnt[kMaxChunkTiles + 1];     // last splits per length
  __shared__ int start[kMaxChunkTiles + 1];   // their next position
  __shared__ unsigned long long load[kSchedMachines];
  __shared__ int nfull, fullpos;
  for (int t = lane; t <= c; t += 64) cnt[t] = 0;
  if (lane == 0) {
    nfull = 0;
    fullpos = 0;
  }
  __syncthreads();
  for (int b = lane; b < B; b += 64) {
    const int T = seq_key_tiles(kv_offset, b, N, max_prefix);
    if (T == 0) continue;
    const int ns = (T + c - 1) / c;
    const int last = T - (ns - 1) * c;
    atomicAdd(&nfull, last == c ? ns : ns - 1);
    if (last < c) atomicAdd(&cnt[last], 1);
  }
  __syncthreads();
  // positions: the full splits first, then last splits by length c-1 .. 1;
  // lane l scans lengths c-1-u for u in [l*k, (l+1)*k)
  const int k = (c - 1 + 63) / 64;
  int local = 0;
  for (int u = lane * k; u < min((lane + 1) * k, c - 1); ++u) local += cnt[c - 1 - u];
  int incl = local;
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  const int nlast = __shfl(incl, 63, 64);
  const int count = nfull + nlast;
  int base = nfull + incl - local;
  for (int u = lane * k; u < min((lane + 1) * k, c - 1); ++u) {
    start[c - 1 - u] = base;
    base += cnt[c - 1 - u];
  }
  const bool exact = nlast <= kExactLasts && M <= 64;
  // machine loads: with the exact estimate, the full splits spread evenly
  // (nfull = q M + r: r machines take q + 1 of them)
  const int q = nfull / M, r = nfull - q * M;
  for (int m = lane; m < M; m += 64)
    load[m] = exact ? (unsigned long long)(q + (m < r ? 1 : 0)) * block_cost(c) : 0ull;
  __syncthreads();
  auto place = [&](int pos, int item, int tiles) {
    out[4 + pos] = item;
    if (!exact) {
      const int rr = pos / M;
      const int m = (rr & 1) ? M - 1 - (pos - rr * M) : pos - rr * M;
      atomicAdd(&load[m], block_cost(tiles));
    }
  };
  for (int b = lane; b < B; b += 64) {
    const int T = seq_key_tiles(kv_offset, b, N, max_prefix);
    if (T == 0) continue;
    const int ns = (T + c - 1) / c;
    const int last = T - (ns - 1) * c;
    const int nf = last == c ? ns : ns - 1;
    if (nf > 0) {
      const int at = atomicAdd(&fullpos, nf);
      for (int sp = 0; sp < nf; ++sp) place(at + sp, b * sa.max_splits + sp, c);
    }
    if (last < c) place(atomicAdd(&start[last], 1), b * sa.max_splits + ns - 1, last);
  }
  __syncthreads();
  if (exact && nlast > 0) {
    // last splits longest first, each onto the least loaded machine (lowest
    // index among equals); machine m's load in lane m; lengths in groups of
    // 64, lane i on length hi - i
    uint32_t my = lane < M ? (uint32_t)min(load[lane], (unsigned long long)kLoadSat) : kLoadSat;
    for (int hi = c - 1; hi >= 1; hi -= 64) {
      const int len = hi - lane;
      const int n = len >= 1 ? cnt[len] : 0;
      uint64_t mask = __ballot(n > 0);
      while (mask) {
        const int i = __builtin_ctzll(mask);
        mask &= mask - 1;
        const uint32_t add = (uint32_t)block_cost(hi - i);
        const int ni = __shfl(n, i, 64);
        for (int e = 0; e < ni; ++e) {
          const uint32_t key = lane < M ? (my << 6) | (uint32_t)lane : 0xffffffffu;
          if ((int)(wave_min_u32(key) & 63) == lane) my = min(my + add, kLoadSat);
        }
      }
    }
    if (lane < M) load[lane] = my;
    __syncthreads();
  }
  unsigned long long mk = 0;
  for (int m = lane; m < M; m += 64) mk = load[m] > mk ? load[m] : mk;
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long v = __shfl_xor(mk, o, 64);
    mk = v > mk ? v : mk;
  }
  if (lane == 0) {
    out[0] = count;
    out[1] = c * kKeyTile;
    out[2] = (int32_t)(uint32_t)(mk & 0xffffffffull);
    out[3] = (int32_t)(uint32_t)(mk >> 32);
  }
}

// One wave per sequence. Writes, for sequence b:
//   anc[b*R + s]        ancestor-or-self mask of slot s (slot 0: 0)
//   nkids[b*R + s]      number of children of slot s
//   kids[(b*R+s)*maxc + i]  i-th child (ascending node index)
//   flags[b]            SV_SEQ_ERR_* bits
//   bar[b]              0 (the sampling walk's barrier counter)
//   xtag[b][2][64][2]   0 (the walk's exchange words), when given
// With a KV layout (kv_offset), blocks B .. B + kSchedCands - 1 write the
// attention schedules.
// With `distinct` (siblings drawn without replacement), two children of one
// slot with the same token are an input error for sequences with T > 0.
__global__ __launch_bounds__(64) void k_tree_prep(
    int N, int V, int maxc, int max_prefix, int distinct, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ token, const float* __restrict__ temperature,
    const int32_t* __restrict__ kv_offset, uint64_t* __restrict__ anc,
    int32_t* __restrict__ nkids, int32_t* __restrict__ kids, int32_t* __restrict__ flags,
    int32_t* __restrict__ bar, unsigned long long* __restrict__ xtag, int B, SchedArgs sa) {
  const int b = blockIdx.x;
  if (b >= B) {
    attn_candidate(B, N, max_prefix, kv_offset, sa, b - B);
    return;
  }
  const int lane = threadIdx.x;
  const int R = N + 1;
  __shared__ int par[kMaxNodes];
  __shared__ int tok[kMaxNodes];
  __shared__ int s_err;
  if (lane == 0) s_err = 0;
  int err = 0;
  if (lane < N) {
    const int p = parent[(size_t)b * N + lane];
    par[lane] = p;
    if (p < -1 || p >= lane) err |= SV_SEQ_ERR_TREE;
    if (token != nullptr) {
      const int t = token[(size_t)b * N + lane];
      tok[lane] = t;
      if (t < 0 || t >= V) err |= SV_SEQ_ERR_TOKEN;
    }
  }
  if (lane == 0) {
    if (temperature != nullptr) {
      const float T = temperature[b];
      if (!(T >= 0.0f) || T == INFINITY) err |= SV_SEQ_ERR_TEMPERATURE;
    }
    if (kv_offset != nullptr) {
      const long long L = (long long)kv_offset[b + 1] - kv_offset[b] - N;
      if (L < 1 || L > max_prefix) err |= SV_SEQ_ERR_PREFIX;
    }
  }
  __syncthreads();
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  const bool tree_ok = (s_err & SV_SEQ_ERR_TREE) == 0;
  if (distinct && token != nullptr && temperature != nullptr && temperature[b] > 0.0f &&
      lane < N && tree_ok) {
    bool dup = false;
    for (int i = 0; i < lane; ++i) dup |= (par[i] == par[lane] && tok[i] == tok[lane]);
    if (dup) atomicOr(&s_err, SV_SEQ_ERR_TOKEN);
  }

  // children lists, one slot per lane (R may exceed 64 by one)
  for (int s = lane; s < R; s += 64) {
    int cnt = 0;
    if (tree_ok) {
      for (int j = s; j < N; ++j) {          // a child of slot s has index >= s
        if (par[j] + 1 == s) {
          if (cnt < maxc) kids[((size_t)b * R + s) * maxc + cnt] = j;
          ++cnt;
        }
      }
    }
    if (cnt > maxc) atomicOr(&s_err, SV_SEQ_ERR_TREE);
    nkids[(size_t)b * R + s] = cnt < maxc ? cnt : maxc;
  }

  // ancestor-or-self masks; parent[j] < j bounds the walk by j steps
  if (lane < N) {
    uint64_t m = 0;
    if (tree_ok) {
      int x = lane;
      while (x >= 0) {
        m |= (uint64_t)1 << x;
        x = par[x];
      }
    }
    anc[(size_t)b * R + lane + 1] = m;
  }
  if (lane == 0) anc[(size_t)b * R] = 0;
  __syncthreads();
  if (lane == 0) {
    flags[b] = s_err;
    bar[b] = 0;
  }
  if (xtag != nullptr) {
    // phase 0 in both exchange buffers: no residual exchange has happened
    constexpr int kWords = 2 * kWalkGroupsPlainMax * kWalkXWords;
    for (int i = lane; i < kWords; i += 64) xtag[(size_t)b * kWords + i] = 0ull;
  }
}

hipError_t launch_tree_prep(const Plan& P, const Args& a, bool check_prefix, hipStream_t s,
                            bool clear_walk, int cu_share) {
  SchedArgs sa{};
  int extra = 0;
  if (check_prefix) {      // with a KV layout: one more block per candidate split length
    extra = P.n_cand;
    sa.sched = ws_attn_sched(P, a.ws);
    sa.stride = (int)P.sched_stride;
    sa.max_splits = P.max_splits;
    const int hg = P.Hkv * P.attn_rg;
    sa.machines = std::max(1, std::min(kSchedMachines, device_cus() / hg));
    if (cu_share > 1 && a.temperature != nullptr) {
      sa.side_machines = std::max(1, std::min(kSchedMachines, device_cus() / cu_share / hg));
      sa.temperature = a.temperature;
    }
    for (int j = 0; j < kSchedCands; ++j) sa.cand[j] = P.cand_tiles[j];
  }
  hipLaunchKernelGGL(k_tree_prep, dim3(P.B + extra), dim3(64), 0, s, P.N, P.V, P.max_children,
                     P.max_prefix, P.sampling == SV_SAMPLE_DISTINCT ? 1 : 0, a.parent, a.token,
                     a.temperature, check_prefix ? a.kv_offset : nullptr, ws_anc(P, a.ws),
                     ws_nkids(P, a.ws), ws_kids(P, a.ws), ws_flags(P, a.ws), ws_bar(P, a.ws),
                     clear_walk ? ws_xtag(P, a.ws) : nullptr, P.B, sa);
  return hipGetLastError();
}

}  // namespace sv
