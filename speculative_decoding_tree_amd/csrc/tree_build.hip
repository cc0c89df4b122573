// EAGLE-2 context-aware dynamic draft tree: expansion by global acceptance
// value, reranking, flattening.
//
// What is computed ("LLM speculative decoding: EAGLE", jingming.pro, sec.
// 4.2.1; "EAGLE / EAGLE-2" excerpts, modelers.csdn.net, sec. 2.3.1-2.3.2):
// a drafted node's value is the product of the draft model's probabilities
// along its path from the root (the root's value is 1). Each expansion step
// takes the draft model's next-token logits at the nodes of the current
// frontier, gives every such node the C most probable tokens as children
// (ties: lower token id), and makes the K children of highest value (ties:
// earlier creation) the next frontier. After the last step every node is
// ranked by value (higher first), depth (shallower first) and creation
// order; the first m form the draft tree, flattened in that order. A child's
// value never exceeds its parent's (its probability is at most 1, and the
// fp32 product rounds monotonically), so every kept node's parent is kept
// and precedes it: the parent array satisfies parent[j] < j, the packed
// order the verification step reads.
//
// State lives in caller-owned device arrays (the pool): for sequence b,
// node id j < pool_count[b] has pool_token/parent/value/depth[b*P + j],
// created in order; frontier[b*K .. b*K + frontier_count[b]) holds the pool
// ids to expand next (-1 = the root).
//
// Kernels:
//   k_tree_init    one thread per sequence: frontier = {root}, empty pool.
//   k_expand_seg   one block per (16384-token segment of a frontier row,
//                  sequence): the segment's (max, sum of exp) and its C best
//                  tokens, from registers, into the workspace.
//   k_expand_merge one block per sequence: merges each row's segments into
//                  its C children, commits them and picks the next frontier
//                  by rank counting.
//   k_tree_finalize one block per sequence: sorts every pool node by rank
//                  key in LDS (bitonic), keeps the first m and writes the
//                  flattened tree.
#include "sv_internal.h"

namespace sv {

constexpr int kMaxChildren = 16;          // C <= 16 per expanded node
constexpr int kMaxExpand = 16;            // K <= 16 nodes per frontier
constexpr int kMaxPool = 1024;            // pool capacity per sequence
constexpr int kFinalThreads = 1024;

struct TreePool {
  int32_t* token;
  int32_t* parent;
  float* value;
  int32_t* depth;
  int32_t* count;
};

__global__ void k_tree_init(int B, int K, int32_t* frontier, int32_t* frontier_count,
                            int32_t* pool_count, int32_t* status) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  frontier[(size_t)b * K] = -1;
  frontier_count[b] = 1;
  pool_count[b] = 0;
  status[b] = 0;
}

// (z, v) ranks ahead of (z2, v2): larger logit, then lower token id
__device__ __forceinline__ bool ahead(float z, int v, float z2, int v2) {
  return z > z2 || (z == z2 && v < v2);
}

// Wave-wide "ahead-most" of one (value, token) pair per lane, in every lane.
// Inside each 16-lane row: DPP exchanges xor 1, xor 2 (quad permutes), then
// the half-row and row mirrors; across rows: permlane16 and permlane32 swaps,
// each followed by a choice between the two values it leaves in the lane
// (the choice is symmetric, so which of them came from the partner does not
// matter). All VALU work, no LDS round trips.
template <int CTRL>
__device__ __forceinline__ void dpp_ahead(float& v, int& i) {
  const float v2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
  const int i2 = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xF, 0xF, false);
  if (ahead(v2, i2, v, i)) {
    v = v2;
    i = i2;
  }
}

__device__ __forceinline__ void wave_ahead_max(float& v, int& i) {
  dpp_ahead<0xB1>(v, i);    // quad_perm [1, 0, 3, 2]
  dpp_ahead<0x4E>(v, i);    // quad_perm [2, 3, 0, 1]
  dpp_ahead<0x141>(v, i);   // half-row mirror
  dpp_ahead<0x140>(v, i);   // row mirror
  {
    const auto rv = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const auto ri = __builtin_amdgcn_permlane16_swap((unsigned)i, (unsigned)i, false, false);
    const float a = __uint_as_float(rv[0]), b2 = __uint_as_float(rv[1]);
    const int ia = (int)ri[0], ib = (int)ri[1];
    if (ahead(b2, ib, a, ia)) { v = b2; i = ib; } else { v = a; i = ia; }
  }
  {
    const auto rv = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const auto ri = __builtin_amdgcn_permlane32_swap((unsigned)i, (unsigned)i, false, false);
    const float a = __uint_as_float(rv[0]), b2 = __uint_as_float(rv[1]);
    const int ia = (int)ri[0], ib = (int)ri[1];
    if (ahead(b2, ib, a, ia)) { v = b2; i = ib; } else { v = a; i = ia; }
  }
}

// Expansion, first kernel: one block of kSegThreads per (segment of a
// frontier row, sequence). A segment of up to kSegLen tokens is loaded into
// registers at once (kSegPerLane values per lane, every load in flight
// together). Pass one over the registers gives the segment's (max, sum of
// exp) and each lane's best token. Every wave's C-th best lane-best is a
// lower bound for the row's C-th best token (the wave holds C distinct tokens
// ranking at or ahead of it), so pass two appends to the wave's LDS buffer
// only the tokens that rank at or ahead of the best such bound: a few dozen
// per segment. A buffer that would overflow is compacted to its C best,
// which raises the bound further. The waves' C best then merge into the
// segment's C best, written to the workspace with the segment's statistics.
constexpr int kSegThreads = 512;
constexpr int kSegWaves = kSegThreads / 64;
constexpr int kSegPerLane = 32;
constexpr int kSegLen = kSegThreads * kSegPerLane;   // 16384 tokens
static_assert((long long)kTreeMaxVocab <= 64LL * kSegLen, "a merge lane per segment");
constexpr int kCandBuf = 256;                        // per wave
constexpr int kMergeThreads = 64 * kMaxExpand;       // one wave per frontier row

struct SegOut {
  float* v;    // [B][K][S][kMaxChildren] the segment's best logits, in order
  int* t;      // [B][K][S][kMaxChildren] their tokens
  float* m;    // [B][K][S] segment max
  float* s;    // [B][K][S] sum of exp(z - max) over the segment
};

// A buffered candidate: one 8-byte LDS entry, read with one ds_read_b64.
struct Cand {
  float v;
  int t;
};

// How many of buf[0 .. n8) rank ahead of (v, t); n8 is a multiple of 8 and
// entries past the real ones hold empty markers (never ahead of anything).
// Eight independent reads in flight per step.
__device__ __forceinline__ int rank_in(const Cand* buf, int n8, float v, int t) {
  int r = 0;
  for (int o = 0; o < n8; o += 8) {
    Cand c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = buf[o + k];
#pragma unroll
    for (int k = 0; k < 8; ++k) r += ahead(c[k].v, c[k].t, v, t) ? 1 : 0;
  }
  return r;
}

// Keep the C best of the wave's n buffered candidates in slots 0 .. C-1, in
// order (empty markers past n); returns how many were kept and the
// threshold: the C-th best, or the old threshold when fewer than C are
// buffered. Every lane ranks its entries (lane, lane + 64, ...) against the
// whole buffer; entries are distinct, so the ranks are a permutation.
// Wave-wide; LDS accesses of one wave run in order. Out of line: it runs at
// the end and when a buffer could overflow.
struct Compacted {
  int kept;
  float tv;
  int ti;
};

__device__ __attribute__((noinline)) Compacted compact_candidates(Cand* buf, int n, int C,
                                                                  float tv, int ti) {
  const int lane = threadIdx.x & 63;
  constexpr int kPer = kCandBuf / 64;
  const int n8 = (n + 7) & ~7;
  for (int e = n + lane; e < n8; e += 64) buf[e] = Cand{-INFINITY, 0x7fffffff};
  __builtin_amdgcn_wave_barrier();
  Cand mine[kPer];
  int rank[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = lane + 64 * k;
    mine[k] = (e < n) ? buf[e] : Cand{-INFINITY, 0x7fffffff};
    rank[k] = (e < n) ? rank_in(buf, n8, mine[k].v, mine[k].t) : kCandBuf;
  }
  // every lane has read the buffer before its first slots are rewritten
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    if (rank[k] < C) buf[rank[k]] = mine[k];
  for (int r = n + lane; r < C; r += 64) buf[r] = Cand{-INFINITY, 0x7fffffff};
  __builtin_amdgcn_wave_barrier();
  Compacted out{min(n, C), tv, ti};
  if (out.kept == C) {
    out.tv = buf[C - 1].v;
    out.ti = buf[C - 1].t;
  }
  return out;
}

template <bool VEC>
__global__ __launch_bounds__(kSegThreads) void k_expand_seg(
    const float* __restrict__ logits, int V, int K, int C, int S, const int32_t* frontier_count,
    int32_t* status, SegOut out) {
  __shared__ Cand s_cand[kSegWaves][kCandBuf];
  __shared__ Cand s_best[kSegWaves * kMaxChildren];
  __shared__ int s_n[kSegWaves];
  __shared__ float s_wm[kSegWaves], s_ws[kSegWaves];
  __shared__ float s_tv[kSegWaves];
  __shared__ int s_ti[kSegWaves];
  __shared__ int s_bad;
  __shared__ int s_skip;
  const int i = blockIdx.x / S;
  const int sg = blockIdx.x % S;
  const int b = blockIdx.y;
  // Other blocks of this launch may set error bits in status[b] while this
  // block starts: one thread reads it and the whole block takes its verdict,
  // so no wave passes a barrier that an exited wave skipped.
  if (threadIdx.x == 0)
    s_skip = (i >= frontier_count[b] || (__atomic_load_n(&status[b], __ATOMIC_RELAXED) &
                                         kSeqErrMask)) ? 1 : 0;
  __syncthreads();
  if (s_skip) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* z = logits + ((size_t)b * K + i) * V;
  const int t_begin = sg * kSegLen;
  const int len = min(V - t_begin, kSegLen);     // tokens of this segment

  // the segment in registers: value k of this lane is token t_begin + off(k),
  // rising in k; values past the segment read as -inf (their addresses are
  // clamped, so every load is valid and in flight at once)
  float x[kSegPerLane];
  auto off = [&](int k) {
    return VEC ? 4 * (tid + kSegThreads * (k >> 2)) + (k & 3) : tid + kSegThreads * k;
  };
  if (VEC) {
#pragma unroll
    for (int u = 0; u < kSegPerLane / 4; ++u) {
      const int o = 4 * (tid + kSegThreads * u);
      const float4 f = *(const float4*)(z + t_begin + min(o, len - 4));
      const bool ok = o < len;      // len is a multiple of 4 here
      x[4 * u] = ok ? f.x : -INFINITY;
      x[4 * u + 1] = ok ? f.y : -INFINITY;
      x[4 * u + 2] = ok ? f.z : -INFINITY;
      x[4 * u + 3] = ok ? f.w : -INFINITY;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kSegPerLane; ++k) {
      const int o = tid + kSegThreads * k;
      const float f = z[t_begin + min(o, len - 1)];
      x[k] = (o < len) ? f : -INFINITY;
    }
  }
  // the lane's first token inside the segment, and how many it holds
  const int n_valid = VEC ? min(kSegPerLane, max(0, 4 * ((len / 4 - tid + kSegThreads - 1) / kSegThreads)))
                          : min(kSegPerLane, max(0, (len - tid + kSegThreads - 1) / kSegThreads));

  // pass one: statistics and the lane's best token (the first maximum, i.e.
  // the lowest id; a lane holding only -inf values takes its first token)
  float mx = -INFINITY;
  bool bad = false;
#pragma unroll
  for (int k = 0; k < kSegPerLane; ++k) {
    bad |= isnan(x[k]) || x[k] == INFINITY;
    mx = fmaxf(mx, x[k]);
  }
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (n_valid > 0) {
    bi = t_begin + off(0);
#pragma unroll
    for (int k = 0; k < kSegPerLane; ++k)
      if (x[k] > bv) {
        bv = x[k];
        bi = t_begin + off(k);
      }
  }
  float sm = 0.0f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int k = 0; k < kSegPerLane; ++k) sm += __builtin_amdgcn_exp2f((x[k] - mx) * kLog2e);
  }
  float wm = mx;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o, 64));
  float ws = (mx == -INFINITY) ? 0.0f : sm * __builtin_amdgcn_exp2f((mx - wm) * kLog2e);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ws += __shfl_xor(ws, o, 64);

  // the wave's bound: the C-th best of its lanes' best tokens (C rounds of a
  // wave argmax, each winner dropping out)
  Cand* buf = s_cand[wave];
  float tv = -INFINITY;
  int ti = 0x7fffffff;
  {
    float hv = bv;
    int hi = bi;
    for (int r = 0; r < C; ++r) {
      float wv = hv;
      int wi = hi;
      wave_ahead_max(wv, wi);
      if (hi == wi && hv == wv) {
        hv = -INFINITY;
        hi = 0x7fffffff;
      }
      tv = wv;
      ti = wi;
    }
  }
  const bool wbad = __ballot(bad) != 0;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (lane == 0) {
    s_wm[wave] = wm;
    s_ws[wave] = ws;
    s_tv[wave] = tv;
    s_ti[wave] = ti;
    s_n[wave] = 0;
    if (wbad) s_bad = 1;
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0) atomicOr(&status[b], SV_SEQ_ERR_NONFINITE);
    return;
  }
  // the strongest bound of any wave (the empty marker if no wave has C tokens)
  for (int w = 0; w < kSegWaves; ++w)
    if (ahead(s_tv[w], s_ti[w], tv, ti)) {
      tv = s_tv[w];
      ti = s_ti[w];
    }
  auto admit = [&](float v, int t) { return ahead(v, t, tv, ti) || (v == tv && t == ti); };

  // pass two: only lanes whose best token is admitted can hold admitted
  // tokens; they append them from their registers through an LDS counter.
  // If more than the buffer holds are admitted (only with massive ties) the
  // wave starts over on a slow path that reads the values again and
  // compacts the buffer whenever it fills, which raises the bound.
  if (admit(bv, bi)) {
#pragma unroll
    for (int k = 0; k < kSegPerLane; ++k) {
      const int t = t_begin + off(k);
      if (k < n_valid && admit(x[k], t)) {
        const int pos = atomicAdd(&s_n[wave], 1);
        if (pos < kCandBuf) buf[pos] = Cand{x[k], t};
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  int n = __builtin_amdgcn_readfirstlane(s_n[wave]);
  if (n > kCandBuf) {
    n = 0;
    for (int k = 0; k < kSegPerLane; ++k) {
      const int t = t_begin + off(k);
      const float v = (k < n_valid) ? z[t] : -INFINITY;
      const bool pass = k < n_valid && admit(v, t);
      unsigned long long mask = __ballot(pass);
      if (mask == 0ull) continue;
      if (n + __popcll(mask) > kCandBuf) {
        const Compacted r = compact_candidates(buf, n, C, tv, ti);
        n = r.kept;
        tv = r.tv;
        ti = r.ti;
        mask = __ballot(k < n_valid && admit(v, t));
      }
      if ((mask >> lane) & 1ull) {
        const int pos = n + __builtin_amdgcn_mbcnt_hi(
                                (unsigned)(mask >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0));
        buf[pos] = Cand{v, t};
      }
      n += __popcll(mask);
    }
  }
  compact_candidates(buf, n, C, tv, ti);   // slots 0 .. C-1: the wave's C best
  for (int r = lane; r < C; r += 64) s_best[wave * C + r] = buf[r];
  __syncthreads();
  if (wave != 0) return;

  // the segment's C best among the waves' lists: lane l holds entries l and
  // l + 64 of the kSegWaves * C, ranked against all of them. Real tokens are
  // distinct and rank ahead of every empty marker, so they take ranks
  // 0 .. real - 1; slots real .. C - 1 get markers.
  const size_t row = ((size_t)b * K + i) * S + sg;
  const int total = kSegWaves * C;   // <= 128, a multiple of 8
  int real = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = lane + 64 * h;
    const Cand c = (e < total) ? s_best[e] : Cand{-INFINITY, 0x7fffffff};
    const bool is_real = c.t != 0x7fffffff;
    real += __popcll(__ballot(is_real));
    if (is_real) {
      const int rank = rank_in(s_best, total, c.v, c.t);
      if (rank < C) {
        out.v[row * kMaxChildren + rank] = c.v;
        out.t[row * kMaxChildren + rank] = c.t;
      }
    }
  }
  for (int r = real + lane; r < C; r += 64) {
    out.v[row * kMaxChildren + r] = -INFINITY;
    out.t[row * kMaxChildren + r] = 0x7fffffff;
  }
  if (lane == 0) {
    float m = -INFINITY;
    for (int w = 0; w < kSegWaves; ++w) m = fmaxf(m, s_wm[w]);
    float sum = 0.0f;
    for (int w = 0; w < kSegWaves; ++w)
      sum += (s_wm[w] == -INFINITY) ? 0.0f : s_ws[w] * __builtin_amdgcn_exp2f((s_wm[w] - m) * kLog2e);
    out.m[row] = m;
    out.s[row] = sum;
  }
}

// Expansion, second kernel: one block per sequence, wave w merging frontier
// row w's segments (statistics, then C rounds over the S list heads) into its
// C children; then the next frontier by rank counting over the children.
// The segments' statistics (one lane each) and lists (LDS) are loaded with
// every load in flight before the rounds start, so the rounds wait on LDS,
// not on a memory round trip each; rows with more than 64 segments or
// kMergeCand list entries read their lists from memory instead.
constexpr int kMergeCand = 256;   // list entries (S * C) staged per frontier row
__global__ __launch_bounds__(kMergeThreads) void k_expand_merge(int K, int C, int P, int S,
                                                                int32_t* frontier,
                                                                int32_t* frontier_count,
                                                                TreePool pool, int32_t* status,
                                                                SegOut seg) {
  __shared__ float s_val[kMaxExpand * kMaxChildren];
  __shared__ float s_cv[kMaxExpand][kMergeCand];
  __shared__ int s_ct[kMaxExpand][kMergeCand];
  __shared__ int s_err;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_in = frontier_count[b];
  const int base = pool.count[b];
  const int st = status[b];
  // this wave's frontier entry, read beside the counts (an entry past n_in
  // is never used), and then its node's value and depth, so the dependent
  // loads take two round trips before the merge instead of four
  const int f_raw = (wave < K) ? frontier[(size_t)b * K + wave] : -1;
  const bool overflow = base + n_in * C > P;
  const int f = (wave < n_in) ? f_raw : -1;
  float pv = 1.0f;
  int pd = 0;
  if (f >= 0 && !(st & kSeqErrMask) && !overflow) {
    pv = pool.value[(size_t)b * P + f];
    pd = pool.depth[(size_t)b * P + f];
  }
  if (tid == 0) s_err = 0;
  __syncthreads();   // every read of the frontier and counts is done
  if ((st & kSeqErrMask) || overflow) {
    if (tid == 0) {
      if (!(st & kSeqErrMask)) status[b] = st | SV_SEQ_ERR_POOL;
      frontier_count[b] = 0;
    }
    return;
  }
  const bool staged = S <= 64 && S * C <= kMergeCand;
  float sgm = -INFINITY, sgs = 0.0f;     // lane sg: segment sg's (max, sum)
  if (wave < n_in && staged) {
    const size_t row0 = ((size_t)b * K + wave) * S;
    if (lane < S) {
      sgm = seg.m[row0 + lane];
      sgs = seg.s[row0 + lane];
    }
    for (int idx = lane; idx < S * C; idx += 64) {
      const size_t at = (row0 + idx / C) * kMaxChildren + idx % C;
      s_cv[wave][idx] = seg.v[at];
      s_ct[wave][idx] = seg.t[at];
    }
  }
  __syncthreads();   // the staged lists are visible to every lane of their wave
  if (wave < n_in) {
    const size_t row0 = ((size_t)b * K + wave) * S;
    // row statistics in segment order, as a plain loop over the segments
    float rm = -INFINITY;
    float rs = 0.0f;
    if (staged) {
      for (int sg = 0; sg < S; ++sg) rm = fmaxf(rm, __shfl(sgm, sg, 64));
      for (int sg = 0; sg < S; ++sg) {
        const float m = __shfl(sgm, sg, 64);
        const float sv = __shfl(sgs, sg, 64);
        rs += (m == -INFINITY) ? 0.0f : sv * __builtin_amdgcn_exp2f((m - rm) * kLog2e);
      }
    } else {
      for (int sg = 0; sg < S; ++sg) rm = fmaxf(rm, seg.m[row0 + sg]);
      for (int sg = 0; sg < S; ++sg) {
        const float m = seg.m[row0 + sg];
        rs += (m == -INFINITY) ? 0.0f : seg.s[row0 + sg] * __builtin_amdgcn_exp2f((m - rm) * kLog2e);
      }
    }
    if (rm == -INFINITY) {
      if (lane == 0) s_err = 1;
    } else {
      int ptr = 0;
      for (int r = 0; r < C; ++r) {
        float hv = -INFINITY;
        int hi = 0x7fffffff;
        if (lane < S && ptr < C) {
          if (staged) {
            hv = s_cv[wave][lane * C + ptr];
            hi = s_ct[wave][lane * C + ptr];
          } else {
            hv = seg.v[(row0 + lane) * kMaxChildren + ptr];
            hi = seg.t[(row0 + lane) * kMaxChildren + ptr];
          }
        }
        float wv = hv;
        int wi = hi;
        wave_ahead_max(wv, wi);
        if (lane < S && hi == wi && hv == wv) ++ptr;
        if (lane == 0) {
          const float val = pv * (__builtin_amdgcn_exp2f((wv - rm) * kLog2e) / rs);
          const size_t slot = (size_t)b * P + base + wave * C + r;
          pool.token[slot] = wi;
          pool.parent[slot] = f;
          pool.value[slot] = val;
          pool.depth[slot] = pd + 1;
          s_val[wave * C + r] = val;
        }
      }
    }
  }
  __syncthreads();
  if (s_err) {
    if (tid == 0) {
      status[b] = st | SV_SEQ_ERR_NONFINITE;
      frontier_count[b] = 0;
    }
    return;
  }
  const int n_new = n_in * C;   // <= 256
  if (tid < n_new) {
    const float v = s_val[tid];
    int rank = 0;
    for (int u = 0; u < n_new; ++u) {
      const float vu = s_val[u];
      rank += (vu > v || (vu == v && u < tid)) ? 1 : 0;
    }
    if (rank < K) frontier[(size_t)b * K + rank] = base + tid;
  }
  if (tid == 0) {
    frontier_count[b] = min(K, n_new);
    pool.count[b] = base + n_new;
  }
}

// Rank order as one 64-bit key, ascending: value descending (values are
// products of probabilities, >= 0, so their bit patterns order like the
// values; inverted for descending), then depth, then pool id.
__device__ __forceinline__ unsigned long long rank_key(float v, int d, int id) {
  const unsigned int vb = ~__float_as_uint(v);
  return ((unsigned long long)vb << 32) | ((unsigned long long)(unsigned)d << 16) |
         (unsigned long long)(unsigned)id;
}

__global__ __launch_bounds__(kFinalThreads / 2) void k_tree_finalize(int P, int m, TreePool pool,
                                                                     int32_t* parent,
                                                                     int32_t* node_token,
                                                                     int32_t* node_pool_id,
                                                                     int32_t* n_kept) {
  // bitonic sort of kMaxPool keys (padding keys sort last), one
  // compare-exchange per thread per stage
  __shared__ unsigned long long s_key[kMaxPool];
  __shared__ int s_rank[kMaxPool];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int cnt = min(pool.count[b], P);
  for (int j = tid; j < kMaxPool; j += kFinalThreads / 2)
    s_key[j] = (j < cnt) ? rank_key(pool.value[(size_t)b * P + j], pool.depth[(size_t)b * P + j], j)
                         : ~0ull;
  __syncthreads();
  for (int k = 2; k <= kMaxPool; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      // pair (lo, lo + j) for this thread's index among kMaxPool / 2 pairs
      const int lo = 2 * tid - (tid & (j - 1));
      const int hi = lo + j;
      const bool up = (lo & k) == 0;
      const unsigned long long a = s_key[lo], c = s_key[hi];
      if ((a > c) == up) {
        s_key[lo] = c;
        s_key[hi] = a;
      }
      __syncthreads();
    }
  }
  for (int p = tid; p < cnt; p += kFinalThreads / 2) s_rank[(int)(s_key[p] & 0xFFFF)] = p;
  __syncthreads();
  const int kept = min(m, cnt);
  for (int r = tid; r < m; r += kFinalThreads / 2) {
    if (r < kept) {
      const int j = (int)(s_key[r] & 0xFFFF);
      const int pj = pool.parent[(size_t)b * P + j];
      parent[(size_t)b * m + r] = (pj < 0) ? -1 : s_rank[pj];
      node_token[(size_t)b * m + r] = pool.token[(size_t)b * P + j];
      node_pool_id[(size_t)b * m + r] = j;
    } else {
      parent[(size_t)b * m + r] = -1;
      node_token[(size_t)b * m + r] = -1;
      node_pool_id[(size_t)b * m + r] = -1;
    }
  }
  if (tid == 0) n_kept[b] = kept;
}

hipError_t launch_tree_init(int B, int K, int32_t* frontier, int32_t* frontier_count,
                            int32_t* pool_count, int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_tree_init, dim3((B + 255) / 256), dim3(256), 0, s, B, K, frontier,
                     frontier_count, pool_count, status);
  return hipGetLastError();
}

int tree_segments(int V) { return (V + kSegLen - 1) / kSegLen; }

size_t tree_workspace_bytes(int B, int K, int V) {
  const size_t rows = (size_t)B * K * tree_segments(V);
  return rows * kMaxChildren * (sizeof(float) + sizeof(int)) + rows * 2 * sizeof(float);
}

hipError_t launch_tree_expand(int B, int V, int K, int C, int P, const float* logits,
                              int32_t* frontier, int32_t* frontier_count, int32_t* token,
                              int32_t* parent, float* value, int32_t* depth, int32_t* count,
                              int32_t* status, void* ws, hipStream_t s) {
  TreePool pool{token, parent, value, depth, count};
  const int S = tree_segments(V);
  const size_t rows = (size_t)B * K * S;
  SegOut seg;
  seg.v = (float*)ws;
  seg.t = (int*)(seg.v + rows * kMaxChildren);
  seg.m = (float*)(seg.t + rows * kMaxChildren);
  seg.s = seg.m + rows;
  const bool vec = (V % 4 == 0) && (((uintptr_t)logits & 15u) == 0);
  if (vec)
    hipLaunchKernelGGL(k_expand_seg<true>, dim3(K * S, B), dim3(kSegThreads), 0, s, logits, V, K,
                       C, S, frontier_count, status, seg);
  else
    hipLaunchKernelGGL(k_expand_seg<false>, dim3(K * S, B), dim3(kSegThreads), 0, s, logits, V,
                       K, C, S, frontier_count, status, seg);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(k_expand_merge, dim3(B), dim3(kMergeThreads), 0, s, K, C, P, S, frontier,
                     frontier_count, pool, status, seg);
  return hipGetLastError();
}

hipError_t launch_tree_finalize(int B, int P, int m, const int32_t* token, const int32_t* parent,
                                const float* value, const int32_t* depth, const int32_t* count,
                                int32_t* out_parent, int32_t* out_token, int32_t* out_pool_id,
                                int32_t* n_kept, hipStream_t s) {
  TreePool pool{(int32_t*)token, (int32_t*)parent, (float*)value, (int32_t*)depth,
                (int32_t*)count};
  hipLaunchKernelGGL(k_tree_finalize, dim3(B), dim3(kFinalThreads / 2), 0, s, P, m, pool,
                     out_parent, out_token, out_pool_id, n_kept);
  return hipGetLastError();
}

}  // namespace sv
