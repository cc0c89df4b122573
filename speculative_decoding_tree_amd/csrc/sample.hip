// Multi-round speculative sampling down the packed draft tree, fused over the
// vocabulary, with no host round trip.
//
// What is computed:
//  - "LLM speculative decoding: EAGLE" (jingming.pro) sec. 2.3: a drafted
//    token x is accepted when r <= p(x)/q(x); on rejection one token is drawn
//    from norm(max(0, p - q)); if every drafted token is accepted a bonus
//    token is drawn from the next target distribution.
//  - EAGLE excerpts (modelers.csdn.net) sec. 1.3.2 and 1.7: at a node with k
//    candidate children the test is applied to each child in turn; after a
//    rejection the adjusted distribution becomes the target for the next
//    child; only when all k are rejected is the adjusted distribution sampled.
//    Greedy mode compares each child with the target argmax.
//  - Temperature: p = softmax(z_target / T), q = softmax(z_draft / T).
//
// One-scalar form of the adjusted targets. After i rejections at slot s the
// adjusted target is p_i = (p - c_i q)_+ / N_i, with c_0 = 0, N_0 = 1,
// c_{i+1} = c_i + N_i and N_{i+1} = sum_v (p - c_{i+1} q)_+ : subtracting q
// from a distribution of the form (p - c q)_+/N and renormalising gives
// (p - (c + N) q)_+ / N' because the positive part of p - c q only shrinks
// where p - c q is already positive. So every adjusted distribution of a slot
// is fixed by one scalar c, and its mass is one vocabulary pass. The
// acceptance test of the i-th child, u * q(x) <= p_{i-1}(x), becomes
// u * N_{i-1} * q(x) <= (p(x) - c_{i-1} q(x))_+ .
//
// Siblings drawn without replacement (SV_SAMPLE_DISTINCT): the i-th sibling
// came from q_i = q / S_i on the tokens not drawn before it, S_i = 1 - their
// draft mass. The same one-scalar form holds with c_{i+1} = c_i + N_i / S_i
// (a rejected token x has p(x) < c_{i+1} q(x), so it keeps zero weight), and
// the test becomes u * N_i * q(x) <= S_i * (p(x) - c_i q(x))_+ .
//
// Work is done only where the walk needs it. The first child of every slot
// is tested against the plain target (c_0 = 0, N_0 = 1), so a vocabulary pass
// is needed only when a child is rejected, and draft statistics only at the
// slots the walk visits: a few passes per sequence instead of one per
// (slot, child). The walk is sequential, so each sampling sequence gets a
// group of workgroups that split every vocabulary pass and meet at a
// sequence-wide barrier (a counter in the workspace). The grid is sized to
// be resident at once on an idle GPU, and a sequence's workgroups are
// consecutive in dispatch order, so a sequence that waits at a barrier waits
// only for its own workgroups (dispatched after earlier sequences', never
// behind later ones) or for other kernels' blocks to retire. Grids above
// half of the GPU are launched cooperatively.
//   k_row_stats    per (row, 256-token tile) target statistics: max and sum of
//                  exp((z - max)/T), or the argmax for T = 0 (only when the
//                  LM-head GEMM did not produce them in its epilogue).
//   k_slot_combine one wave per row merges the tile statistics of the target
//                  row into its (max, sum) or (argmax value, index).
//   k_walk         G workgroups per sequence: the walk with its draft
//                  statistics and residual passes, then the final draw by a
//                  scan over 256-token tile masses and a block prefix sum
//                  inside one tile (workgroup 0).
// Reductions use fixed orders (no float atomics), so results are bitwise
// reproducible for a given G.
#include "warp_select.h"

namespace sv {

struct SampleParams {
  const float* logits;     // [B*R, V]
  const float* draft;      // [B*R, V]
  const int32_t* token;    // [B*N]
  const float* uniforms;   // [B*R]
  const float* temperature;
  const int32_t* nkids;    // [B*R]
  const int32_t* kids;     // [B*R, maxc]
  const int32_t* flags;    // [B]
  RowStat* tstat;          // [B*R, CT] tile statistics, target rows
  RowStat* slot_t;         // [B*R] merged target statistics
  const int32_t* parent;   // [B*N]
  RowStat* dpart;          // [B*R, dparts] draft statistics of internal sampling slots, per part
  RowStat* slot_q;         // [B*R] their merged draft statistics
  int dparts;              // parts per draft row (1..kDraftPartsMax)
  int draft_done;          // draft statistics computed up front (else by the walk, lazily)
  unsigned long long* xtag;  // [B, 2, 64, kXWords] (phase, value) words of the exchanges
  float* tmass;            // [B, 2, CT] tile masses of the last two residual passes
  int32_t* bar;            // [B] barrier counters, zero at launch
  int B, N, R, V, C, CT, maxc;
  int target_done;         // target tile statistics already written (GEMM epilogue)
  int distinct;            // siblings drawn without replacement (SV_SAMPLE_DISTINCT)
  int top_k;               // > 0 and < V: keep the top_k most probable tokens of p and q
  float top_p;             // in (0, 1): then the shortest prefix reaching this mass
  double mass_scale;       // 2^S: fixed-point unit of the selection masses
  double mass_unit;        // 2^-S
  unsigned* whc;           // [B][2][G][2][256] selection histograms (warping only)
  unsigned long long* whm; // [B][2][G][2][256]
  int* wtie;               // [B][2][G][2]
  int* wtidx;              // [B][2][2]
  unsigned long long* wgl; // [B][2][G][2][kWarpCapW][2] gathered candidates (key, mass)
  unsigned long long* wgcnt; // [B][2][G][2][3] their counts, masses above, masses
  int32_t* accept_len;
  int32_t* accept_path;
  int32_t* out_tokens;
  int32_t* seq_status;
  sv_debug dbg;
};

constexpr int kTilesPerChunk = kVocabChunk / kStatTile;   // 16, 4 per wave
static_assert(kWalkGroupsMax <= kWalkGroupsPlainMax && kWalkGroupsPlainMax <= 64,
              "one lane per workgroup partial");

// ---------------------------------------------------------------------------
// reductions in fixed orders
// ---------------------------------------------------------------------------

__device__ int block_min_int(int v, int* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return min(min(sh[0], sh[1]), min(sh[2], sh[3]));
}

__device__ int block_max_int(int v, int* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return max(max(sh[0], sh[1]), max(sh[2], sh[3]));
}

// (value, index) max with the lowest index among equal values
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(v, o, 64);
    const int i2 = __shfl_xor(i, o, 64);
    argmax_merge(v, i, v2, i2);
  }
}

// Merge n tile statistics of a sampling row into (max, sum exp((z-max)/T)).
// Tiles a lane loads before using any (one memory round trip for rows of up
// to 64 * kMergeBatch tiles); each lane still visits its tiles c = lane,
// lane + 64, ... in order, so the sums are those of a plain strided loop.
constexpr int kMergeBatch = 8;

__device__ __forceinline__ RowStat wave_merge_stats(const RowStat* st, int n, float l2t) {
  const int lane = lane_id();
  float m = -INFINITY;
  float s = 0.0f;
  if (n <= 64 * kMergeBatch) {
    RowStat r[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int c = lane + 64 * i;
      r[i] = c < n ? st[c] : RowStat{-INFINITY, 0.0f};
    }
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) m = fmaxf(m, r[i].m);
    m = wave_max(m);
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i)
      if (lane + 64 * i < n)
        s += (r[i].m == -INFINITY) ? r[i].s : r[i].s * fast_exp2((r[i].m - m) * l2t);
  } else {
    for (int c = lane; c < n; c += 64) m = fmaxf(m, st[c].m);
    m = wave_max(m);
    for (int c = lane; c < n; c += 64) {
      const RowStat r = st[c];
      s += (r.m == -INFINITY) ? r.s : r.s * fast_exp2((r.m - m) * l2t);
    }
  }
  RowStat out;
  out.m = m;
  out.s = wave_sum(s);     // a NaN tile marker propagates
  return out;
}

// Merge n tile argmax statistics: (value, lowest index); value NaN if any tile was.
__device__ __forceinline__ RowStat wave_merge_argmax(const RowStat* st, int n) {
  const int lane = lane_id();
  float v = -INFINITY;
  int idx = 0x7fffffff;
  bool bad = false;
  for (int c0 = 0; c0 < n; c0 += 64 * kMergeBatch) {
    RowStat r[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int c = c0 + lane + 64 * i;
      r[i] = c < n ? st[c] : RowStat{-INFINITY, __int_as_float(0x7fffffff)};
    }
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (c0 + lane + 64 * i >= n) continue;
      if (isnan(r[i].m)) bad = true;
      else argmax_merge(v, idx, r[i].m, __float_as_int(r[i].s));
    }
  }
  wave_argmax(v, idx);
  const bool any_bad = __ballot(bad) != 0;
  RowStat out;
  out.m = any_bad ? NAN : v;
  out.s = __int_as_float(idx);
  return out;
}

// ---------------------------------------------------------------------------
// target row statistics per (row, 256-token tile); a block covers 16 tiles
// ---------------------------------------------------------------------------

template <bool VEC>
__device__ __forceinline__ void row_stats_chunk(const SampleParams& p, int chunk, int row) {
  const int b = row / p.R;
  if (p.flags[b] & kSeqErrMask) return;
  const float T = p.temperature[b];
  const bool greedy = (T == 0.0f);
  const float* z = p.logits + (size_t)row * p.V;
  RowStat* out = p.tstat + (size_t)row * p.CT;
  const int wave = threadIdx.x >> 6;
  const float l2t = greedy ? 0.0f : kLog2e / T;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int tile = chunk * kTilesPerChunk + 4 * wave + q;
    if (tile >= p.CT) break;
    float x[4];
    int idx[4];
    load_tile4<VEC>(z, tile * kStatTile, p.V, x, idx);
    bool bad = false;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (idx[e] < p.V && !isfinite(x[e])) bad = true;
    const bool any_bad = __ballot(bad) != 0;
    RowStat r;
    if (greedy) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (idx[e] < p.V && x[e] > bv) {
          bv = x[e];
          bi = idx[e];
        }
      wave_argmax(bv, bi);
      r.m = any_bad ? NAN : bv;
      r.s = __int_as_float(bi);
    } else {
      const float mx = wave_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) s += fast_exp2((x[e] - mx) * l2t);
      s = wave_sum(s);
      r.m = mx;
      r.s = any_bad ? NAN : s;
    }
    if (lane_id() == 0) out[tile] = r;
  }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_row_stats(SampleParams p) {
  row_stats_chunk<VEC>(p, blockIdx.x, blockIdx.y);
}

// ---------------------------------------------------------------------------
// per-slot merge of the target statistics: one wave per row
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void k_slot_combine(SampleParams p) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.B * p.R) return;
  const int b = row / p.R;
  const int lane = lane_id();
  if (p.flags[b] & kSeqErrMask) return;
  const float T = p.temperature[b];
  float s0 = 0.f, s1 = 0.f;
  int am = -1;
  if (T == 0.0f) {
    const RowStat r = wave_merge_argmax(p.tstat + (size_t)row * p.CT, p.CT);
    if (lane == 0) p.slot_t[row] = r;
    s0 = r.m;
    am = __float_as_int(r.s);
  } else {
    const RowStat r = wave_merge_stats(p.tstat + (size_t)row * p.CT, p.CT, kLog2e / T);
    if (lane == 0) p.slot_t[row] = r;
    s0 = r.m;
    s1 = r.s;
    if (p.draft_done && p.nkids[row] > 0) {
      const RowStat q = wave_merge_stats(p.dpart + (size_t)row * p.dparts, p.dparts, kLog2e / T);
      if (lane == 0) {
        p.slot_q[row] = q;
        if (p.dbg.slot_stats != nullptr) {
          p.dbg.slot_stats[(size_t)row * 4 + 2] = q.m;
          p.dbg.slot_stats[(size_t)row * 4 + 3] = q.s;
        }
      }
    }
  }
  if (lane == 0) {
    if (p.dbg.slot_stats != nullptr) {
      p.dbg.slot_stats[(size_t)row * 4 + 0] = s0;
      p.dbg.slot_stats[(size_t)row * 4 + 1] = s1;
    }
    if (p.dbg.slot_argmax != nullptr) p.dbg.slot_argmax[row] = am;
  }
}

// ---------------------------------------------------------------------------
// the walk
// ---------------------------------------------------------------------------

// (max, sum exp2((z - max) * l2t)) of a row over tiles [t0, t1), with the sum
// NaN when a value is not finite. One pass over memory: a wave loads up to 8
// of its tiles at once and folds them into per-lane (max, sum) pairs, which
// merge across lanes and waves at the end. Result valid in thread 0.
template <bool VEC>
__device__ __forceinline__ RowStat block_row_stats(const float* z, int V, int t0, int t1, float l2t,
                                   RowStat* sh) {
  const int wave = threadIdx.x >> 6;
  constexpr int kU = 8;   // tiles in flight per wave
  float m = -INFINITY, s = 0.0f;
  bool bad = false;
  for (int t = t0 + wave; t < t1; t += 4 * kU) {
    float x[kU][4];
    int idx[kU][4];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int tt = t + 4 * u;
      if (tt < t1) load_tile4<VEC>(z, tt * kStatTile, V, x[u], idx[u]);
      else {
#pragma unroll
        for (int e = 0; e < 4; ++e) { x[u][e] = -INFINITY; idx[u][e] = V; }
      }
    }
    float cm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (idx[u][e] < V && !isfinite(x[u][e])) bad = true;
        cm = fmaxf(cm, x[u][e]);
      }
    if (cm != -INFINITY) {
      float cs = 0.0f;
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) cs += fast_exp2((x[u][e] - cm) * l2t);
      const float nm = fmaxf(m, cm);
      s = (m == -INFINITY ? 0.0f : s * fast_exp2((m - nm) * l2t)) + cs * fast_exp2((cm - nm) * l2t);
      m = nm;
    }
  }
  const float wm = wave_max(m);
  float ws = wave_sum((m == -INFINITY) ? 0.0f : s * fast_exp2((m - wm) * l2t));
  if (__ballot(bad) != 0) ws = NAN;
  __syncthreads();
  if (lane_id() == 0) sh[wave] = RowStat{wm, ws};
  __syncthreads();
  RowStat r{-INFINITY, 0.0f};
  if (threadIdx.x == 0) {
    float mm = -INFINITY;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, sh[w].m);
    float ss = 0.0f;
    for (int w = 0; w < 4; ++w)
      ss += (sh[w].m == -INFINITY) ? sh[w].s : sh[w].s * fast_exp2((sh[w].m - mm) * l2t);
    r = RowStat{mm, ss};
  }
  return r;
}

// Tile masses of (p - ci q)_+ over tiles [t0, t1) into out[tile]; returns
// their sum (valid in thread 0). WARP: p and q are zero outside their kept
// sets (wt, wd); USEQ = false drops q (the warped target's own tile masses).
template <bool VEC, bool WARP, bool USEQ>
__device__ __forceinline__ float block_residual(const float* zt, const float* zd, int V, int t0, int t1,
                                float mp, float ip, float mq, float iq, float ci, float l2t,
                                const WarpRow& wt, const WarpRow& wd, float* out, float* sh) {
  const int wave = threadIdx.x >> 6;
  constexpr int kU = WARP ? 4 : 8;   // tiles in flight per wave (target and draft each)
  const float l2t8 = l2t * 8.0f;
  float wsum = 0.0f;
  for (int t = t0 + wave; t < t1; t += 4 * kU) {
    float xt[kU][4], xd[kU][4];
    int idx[kU][4];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int tt = t + 4 * u;
      if (tt < t1) {
        load_tile4<VEC>(zt, tt * kStatTile, V, xt[u], idx[u]);
        if (USEQ) load_tile4<VEC>(zd, tt * kStatTile, V, xd[u], idx[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) { xt[u][e] = xd[u][e] = -INFINITY; idx[u][e] = V; }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (idx[u][e] < V) {
          float pv = fast_exp2((xt[u][e] - mp) * l2t) * ip;
          if (WARP && !warp_kept(wt, xt[u][e], idx[u][e], l2t8)) pv = 0.0f;
          float qv = 0.0f;
          if (USEQ) {
            qv = fast_exp2((xd[u][e] - mq) * l2t) * iq;
            if (WARP && !warp_kept(wd, xd[u][e], idx[u][e], l2t8)) qv = 0.0f;
          }
          acc += fmaxf(0.0f, pv - ci * qv);
        }
      }
      acc = wave_sum(acc);
      const int tt = t + 4 * u;
      if (tt < t1) {
        wsum += acc;
        if (lane_id() == 0) xstore(out + tt, acc);
      }
    }
  }
  __syncthreads();
  if (lane_id() == 0) sh[wave] = wsum;
  __syncthreads();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

// mass of tile t of the terminal distribution (a residual pass, or the target)
// Draft statistics of every slot with children of a sampling sequence, up
// front: part `blockIdx.x` of the row's tiles reduced to (max, sum of
// exp((z - max)/T)) with the walk's own one-pass block reduction; the slot
// combine merges the parts. Other rows exit at once.
template <bool VEC>
__device__ __forceinline__ void draft_stats_part(const SampleParams& p, int part, int row) {
  __shared__ RowStat sh[4];
  const int b = row / p.R;
  if (p.flags[b] & kSeqErrMask) return;
  const float T = p.temperature[b];
  if (T == 0.0f || p.nkids[row] == 0) return;
  int t0, t1;
  wg_tiles(p.CT, p.dparts, part, &t0, &t1);
  const RowStat r =
      block_row_stats<VEC>(p.draft + (size_t)row * p.V, p.V, t0, t1, kLog2e / T, sh);
  if (threadIdx.x == 0) p.dpart[(size_t)row * p.dparts + part] = r;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_draft_stats(SampleParams p) {
  draft_stats_part<VEC>(p, blockIdx.x, blockIdx.y);
}

// Both passes in one launch when both run (the target statistics did not come
// from the GEMM epilogue and the draft statistics are computed up front):
// blocks x < C take the target row's chunk x, the others draft part x - C.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_row_draft_stats(SampleParams p) {
  if ((int)blockIdx.x < p.C) row_stats_chunk<VEC>(p, blockIdx.x, blockIdx.y);
  else draft_stats_part<VEC>(p, blockIdx.x - p.C, blockIdx.y);
}

__device__ __forceinline__ float tile_mass(const SampleParams& p, int row, const float* tm,
                                           int t, float mp, float ip, float l2t) {
  if (tm == nullptr) {
    const RowStat r = p.tstat[(size_t)row * p.CT + t];
    return (r.m == -INFINITY) ? 0.0f : r.s * fast_exp2((r.m - mp) * l2t) * ip;
  }
  return xload(tm + t);
}

__device__ __forceinline__ float wave_incl_scan(float v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

// Writes the outputs of sequence b (workgroup 0).
__device__ __forceinline__ void write_outputs(const SampleParams& p, int b, int status, int plen,
                              const int* path, int token) {
  const int N = p.N, R = p.R;
  const bool err = (status & kSeqErrMask) != 0;
  for (int j = threadIdx.x; j < N; j += kThreads)
    p.accept_path[(size_t)b * N + j] = (!err && j < plen) ? path[j] : -1;
  for (int j = threadIdx.x; j < R; j += kThreads) {
    int t = -1;
    if (!err) {
      if (j < plen) t = p.token[(size_t)b * N + path[j]];
      else if (j == plen) t = token;
    }
    p.out_tokens[(size_t)b * R + j] = t;
  }
  if (threadIdx.x == 0) {
    p.accept_len[b] = err ? -1 : plen;
    p.seq_status[b] = status;
  }
}

// Barrier of the sequence's G workgroups: a tagged exchange without payload
// on the walk's phase counter (the same counter and buffers as its residual
// and draft-statistics exchanges, so the buffers keep alternating by phase
// parity across all of them). Every wave's earlier stores are complete
// before this workgroup's word is stored, so after the barrier every
// workgroup sees them. False when the bounded wait gave up.
__device__ __forceinline__ bool walk_barrier(const SampleParams& p, int b, unsigned* xphase, int G,
                                             float (*xv)[kXWords], int* s_flag) {
  ++*xphase;
  unsigned long long* xbuf =
      p.xtag + ((size_t)b * 2 + (*xphase & 1)) * kWalkGroupsPlainMax * kXWords;
  const float none[1] = {0.0f};
  return tagged_exchange<1>(xbuf, *xphase, none, G, xv, s_flag);
}

// Top-k / top-p thresholds of a visited slot: the target row and, when
// with_draft, the draft row, selected together (the two rows share every
// barrier). Every workgroup of the sequence takes part and ends with the
// same thresholds and kept masses. Returns false when a barrier wait gave
// up; sets *bad when a selection was impossible (not expected).
struct WarpLds {
  WarpSel sel[2];
  unsigned hc[2 * kWarpBins];
  u64 hm[2 * kWarpBins];
  u64 sk[kWarpCapT];
  u64 sm[kWarpCapT];
  unsigned h0c[2 * kWarpBins];   // the top-k step's level-0 histograms, for top-p
  u64 h0m[2 * kWarpBins];
  u64 tot[8];
  u64 gred[4];
  unsigned gcnt[2];
  int cntw[kWalkGroupsMax];
  int found[2];
  int sh[8];
};

template <bool VEC>
__device__ __forceinline__ bool warp_slot(const SampleParams& p, int b, int wg, int G, int t0, int t1,
                          const float* zt, const float* zd, float mt, float md, bool with_draft,
                          float l2t, double l2td, int* target, unsigned* xphase,
                          float (*xv)[kXWords], int* s_flag, WarpLds& L,
                          WarpRow* wrow, float* kept, bool* bad) {
  const int tid = threadIdx.x;
  const bool use_k = p.top_k > 0 && p.top_k < p.V;
  const bool use_p = p.top_p > 0.0f && p.top_p < 1.0f;
  const float l2t8 = l2t * 8.0f;
  const size_t hist = (size_t)2 * G * 2 * kWarpBins;    // one sequence, both phases
  unsigned* whc = p.whc + (size_t)b * hist;
  u64* whm = p.whm + (size_t)b * hist;
  int* wtie = p.wtie + (size_t)b * 2 * G * 2;
  int* wtidx = p.wtidx + (size_t)b * 2 * 2;
  u64* wgcnt = p.wgcnt + (size_t)b * 2 * G * 2 * 3;
  const size_t glen = (size_t)2 * kWarpCapW * 2;        // one workgroup's lists, both rows
  u64* wgl = p.wgl + (size_t)b * 2 * G * glen;
  WarpThr ra[2] = {warp_none(), warp_none()};
  WarpThr rb[2] = {warp_none(), warp_none()};
  u64 kq[2] = {0ull, 0ull};
  for (int step = 0; step < 2; ++step) {
    if (step == 0 ? !use_k : !use_p) continue;
    // top-p after top-k starts from the top-k step's level-0 histogram cut to
    // its kept set: bins above its cut bin whole, the cut bin's kept part
    const bool derived = (step == 1 && use_k);
    u64 dc[2] = {0ull, 0ull}, dm[2] = {0ull, 0ull};
    if (derived) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const WarpSel A = L.sel[r];
        if (tid > A.b0) {
          dc[r] = L.h0c[r * kWarpBins + tid];
          dm[r] = L.h0m[r * kWarpBins + tid];
        } else if (tid == A.b0) {
          dc[r] = A.need0;
          dm[r] = A.kept - A.above0;
        }
      }
    }
    __syncthreads();
    if (tid < 2) {
      WarpSel S;
      S.m = tid ? md : mt;
      S.active = (tid == 0 || with_draft) ? 1 : 0;
      S.mode = step;
      S.level = 0;
      S.gather = 0;
      S.b0 = 0;
      S.sub = 0;
      S.b1 = 0;
      S.nomass = (step == 0 && !use_p) ? 1 : 0;
      S.whole = 0;
      S.kp = 0u;
      S.need = (step == 0) ? (u64)p.top_k : 0ull;   // top-p: set from the level-0 total
      S.above = 0ull;
      S.need0 = 0ull;
      S.above0 = 0ull;
      S.tie_r = 0;
      S.rst = (step == 1) ? (tid ? ra[1] : ra[0]) : warp_none();
      S.res = warp_none();
      S.kept = 0ull;
      L.sel[tid] = S;
    }
    __syncthreads();
    if (derived) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (!L.sel[r].active) continue;
        if (!warp_decide(L.sel, r, dc[r], dm[r], p.top_p, L.tot, &L.found[0], nullptr, nullptr))
          *bad = true;
      }
    }
    // Each round is one pass over the rows and one barrier: rows that
    // histogram publish their bins, rows that gather publish their candidates.
    while (L.sel[0].active || L.sel[1].active) {
      for (int i = tid; i < 2 * kWarpBins; i += kThreads) {
        L.hc[i] = 0u;
        L.hm[i] = 0ull;
      }
      if (tid < 2) L.gcnt[tid] = 0u;
      if (tid < 4) L.gred[tid] = 0ull;
      __syncthreads();
      const int ph = (*target / G) & 1;
      unsigned* pc = whc + (size_t)ph * G * 2 * kWarpBins;
      u64* pm = whm + (size_t)ph * G * 2 * kWarpBins;
      u64* gc = wgcnt + (size_t)ph * G * 2 * 3;
      u64* gl = wgl + (size_t)ph * G * glen;
      warp_pass<VEC>(zt, zd, p.V, t0, t1, l2t, l2td, p.mass_scale, L.sel, L.hc, L.hm, L.gcnt,
                     L.gred, gl + (size_t)wg * glen);
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (!L.sel[r].active) continue;
        if (L.sel[r].gather) {
          if (tid < 3) {
            const u64 v = (tid == 0) ? (u64)L.gcnt[r] : L.gred[r * 2 + tid - 1];
            xstore_u(gc + ((size_t)wg * 2 + r) * 3 + tid, v);
          }
        } else {
          const size_t at = ((size_t)wg * 2 + r) * kWarpBins + tid;
          xstore_u(pc + at, L.hc[r * kWarpBins + tid]);
          xstore_u(pm + at, L.hm[r * kWarpBins + tid]);
        }
      }
      *target += G;
      if (!walk_barrier(p, b, xphase, G, xv, s_flag)) return false;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (!L.sel[r].active) continue;
        const bool okr = L.sel[r].gather
                             ? warp_gather_finish(L.sel, r, gc, gl, G, L.sk, L.sm, L.tot, L.cntw,
                                                  &L.found[0])
                             : warp_choose_row(L.sel, r, pc, pm, G, p.top_p, L.tot, &L.found[0],
                                               (step == 0 && use_p) ? L.h0c + r * kWarpBins
                                                                    : nullptr,
                                               L.h0m + r * kWarpBins);
        if (!okr) *bad = true;
      }
    }
    // the cut inside a group of equal logits: the r-th id of the group, found
    // by the workgroup whose tiles hold it
    const bool tie0 = L.sel[0].tie_r > 0, tie1 = L.sel[1].tie_r > 0;
    if (tie0 || tie1) {
      int cnt[2] = {0, 0};
      if (tie0) cnt[0] = warp_tie_count(zt, p.V, t0, t1, L.sel[0], l2t8, L.sh);
      if (tie1) cnt[1] = warp_tie_count(zd, p.V, t0, t1, L.sel[1], l2t8, L.sh);
      int* pt = wtie + (size_t)((*target / G) & 1) * G * 2;
      if (tid == 0) {
        xstore_u(pt + wg * 2 + 0, cnt[0]);
        xstore_u(pt + wg * 2 + 1, cnt[1]);
      }
      *target += G;
      if (!walk_barrier(p, b, xphase, G, xv, s_flag)) return false;
      int* ti = wtidx + (size_t)((*target / G) & 1) * 2;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int rr = L.sel[r].tie_r;
        if (rr <= 0) continue;
        int cws[kWalkGroupsMax];
#pragma unroll
        for (int w = 0; w < kWalkGroupsMax; ++w) cws[w] = xload_u(pt + min(w, G - 1) * 2 + r);
        int before = 0, mine = 0;
#pragma unroll
        for (int w = 0; w < kWalkGroupsMax; ++w) {
          if (w < wg) before += cws[w];
          if (w == wg) mine = cws[w];
        }
        if (before < rr && rr <= before + mine) {
          const int id = warp_tie_find(r ? zd : zt, p.V, t0, t1, L.sel[r], l2t8, rr - before, L.sh);
          if (tid == 0) xstore_u(ti + r, id);
        }
      }
      *target += G;
      if (!walk_barrier(p, b, xphase, G, xv, s_flag)) return false;
      if (tid < 2 && L.sel[tid].tie_r > 0) L.sel[tid].res.idx = xload_u(ti + tid);
      __syncthreads();
      if ((tie0 && L.sel[0].res.idx < 0) || (tie1 && L.sel[1].res.idx < 0)) *bad = true;
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (step == 0) ra[r] = L.sel[r].res;
      else rb[r] = L.sel[r].res;
      kq[r] = L.sel[r].kept;
    }
  }
  wrow[0] = WarpRow{ra[0], rb[0], mt};
  wrow[1] = WarpRow{ra[1], rb[1], md};
  kept[0] = (float)((double)kq[0] * p.mass_unit);
  kept[1] = (float)((double)kq[1] * p.mass_unit);
  return true;
}

// Four workgroups per CU without warping (128 VGPRs, a few spills): the
// walk's grid then stays within half of the GPU at 32 sequences (see
// launch_sampling); two with warping, whose selection state needs ~250.
template <bool VEC, bool WARP>
__global__ __launch_bounds__(kThreads, WARP ? 2 : 4) void k_walk(SampleParams p) {
  __shared__ int s_path[kMaxNodes];
  __shared__ int s_int[8];
  __shared__ RowStat s_rs[4];
  __shared__ float s_f[4];
  __shared__ float wtot[4];
  __shared__ int shi[4];
  __shared__ int s_flag;
  __shared__ float s_xv[64][kXWords];
  __shared__ int s_tile, s_token, s_clamp;
  __shared__ float s_run, s_target;
  __shared__ WarpLds s_warp;
  const int wg = blockIdx.x;
  const int G = gridDim.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int N = p.N, R = p.R, CT = p.CT;
  const int flags = p.flags[b];
  if (flags & kSeqErrMask) {
    if (wg == 0) write_outputs(p, b, flags, 0, s_path, -1);
    return;
  }
  const float T = p.temperature[b];
  const bool greedy = (T == 0.0f);

  if (greedy) {
    // argmax comparisons only: workgroup 0, wave 0, lanes test the children
    if (wg != 0) return;
    if (tid == 0) {
      s_int[0] = 0;       // path length
      s_int[1] = flags;   // status
      s_int[2] = -1;      // final token
    }
    __syncthreads();
    if (wave == 0) {
      // Everything the walk can read, loaded at once: lane j holds node j's
      // parent slot and token, lane s slot s's argmax statistics (slot 64,
      // the deepest leaf of a 64-node chain, is read when reached). The walk
      // itself is then ballots over registers.
      int my_ps = -1, my_tok = -1;
      if (lane < N) {
        my_ps = p.parent[(size_t)b * N + lane] + 1;
        my_tok = p.token[(size_t)b * N + lane];
      }
      const RowStat my_st = (lane < R) ? p.slot_t[(size_t)b * R + lane] : RowStat{0.0f, 0.0f};
      int s = 0, plen = 0, status = 0, tok = -1;
      while (true) {
        const RowStat st = (s < 64) ? RowStat{__shfl(my_st.m, s, 64), __shfl(my_st.s, s, 64)}
                                    : p.slot_t[(size_t)b * R + s];
        if (isnan(st.m)) {
          status |= SV_SEQ_ERR_NONFINITE;
          break;
        }
        const int a = __float_as_int(st.s);
        // the first child (ascending node index) whose token is the argmax
        const unsigned long long m = __ballot(lane < N && my_ps == s && my_tok == a);
        if (m == 0ull) {
          tok = a;
          break;
        }
        const int nxt = __ffsll((long long)m) - 1;
        if (lane == 0) s_path[plen] = nxt;
        ++plen;
        s = nxt + 1;
      }
      if (lane == 0) {
        s_int[0] = plen;
        s_int[1] |= status;
        s_int[2] = tok;
      }
    }
    __syncthreads();
    write_outputs(p, b, s_int[1], s_int[0], s_path, s_int[2]);
    return;
  }

  // ---- sampling: the walk, shared by the G workgroups of the sequence ----
  const float l2t = kLog2e / T;
  int status = flags;
  if (wg == 0) {
    bool warn = false;
    for (int j = tid; j < R; j += kThreads) clamp_uniform(p.uniforms[(size_t)b * R + j], &warn);
    if (tid == 0) s_int[3] = 0;
    __syncthreads();
    if (warn) atomicOr(&s_int[3], SV_SEQ_WARN_UNIFORM);
    __syncthreads();
    status |= s_int[3];
  }
  int t0, t1;
  wg_tiles(CT, G, wg, &t0, &t1);
  int target = 0;          // G times the selection barriers passed (buffer parity)
  unsigned xphase = 0;     // phase of the last exchange or barrier among the workgroups
  int s = 0, plen = 0;
  float mp = 0.0f, ip = 1.0f;
  float mq = 0.0f, iq = 1.0f, c = 0.0f, n = 1.0f, S = 1.0f;
  int eff = 0, effbuf = 1;
  bool ok = true;
  const float l2t8 = l2t * 8.0f;
  WarpRow wt, wd;
  wt.a = wt.b = wd.a = wd.b = warp_none();
  wt.m = wd.m = 0.0f;
  // With the draft statistics computed up front (and no warping, whose kept
  // sets are found at each visited slot), every value a test can read is
  // loaded at once before the walk: lane j holds node j's parent slot, its
  // target and draft probabilities p(x), q(x) at its token under that slot's
  // statistics, and its uniform; lane s holds slot s's target and draft
  // statistics (slot 64, the deepest leaf of a 64-node chain, is read when
  // reached). The walk then moves through the tree by ballots over these
  // registers; only rejections cost a vocabulary pass.
  const bool pre = !WARP && p.draft_done;
  int my_ps = -1;
  float my_px = 0.0f, my_qx = 0.0f, my_u = 0.0f;
  RowStat my_st{0.0f, 0.0f}, my_sq{0.0f, 0.0f};
  if (pre) {
    if (lane < R) {
      my_st = p.slot_t[(size_t)b * R + lane];
      my_sq = p.slot_q[(size_t)b * R + lane];
    }
    if (lane < N) {
      my_ps = p.parent[(size_t)b * N + lane] + 1;
      const int x = p.token[(size_t)b * N + lane];
      const size_t prow = (size_t)b * R + my_ps;
      const float zx = p.logits[prow * p.V + x];
      const float dx = p.draft[prow * p.V + x];
      const RowStat pt = p.slot_t[prow];
      const RowStat pq = p.slot_q[prow];
      my_px = fast_exp2((zx - pt.m) * l2t) * (1.0f / pt.s);
      my_qx = fast_exp2((dx - pq.m) * l2t) * (1.0f / pq.s);
      bool w = false;
      my_u = clamp_uniform(p.uniforms[(size_t)b * R + lane], &w);
    }
  }
  for (int depth = 0; depth <= N; ++depth) {
    const int row = b * R + s;
    const unsigned long long kidmask = pre ? __ballot(lane < N && my_ps == s) : 0ull;
    const int nk = pre ? __popcll(kidmask) : p.nkids[row];
    const RowStat st = (pre && s < 64)
                           ? RowStat{__shfl(my_st.m, s, 64), __shfl(my_st.s, s, 64)}
                           : p.slot_t[row];
    c = 0.0f;
    n = 1.0f;
    S = 1.0f;
    eff = 0;
    effbuf = 1;
    if (!isfinite(st.s) || !(st.s > 0.0f)) {
      status |= SV_SEQ_ERR_NONFINITE;
      break;
    }
    mp = st.m;
    ip = 1.0f / st.s;
    if (!WARP && nk == 0) break;   // a leaf: the bonus token comes from the plain target
    const float* zt = p.logits + (size_t)row * p.V;
    const float* zd = p.draft + (size_t)row * p.V;
    if (nk > 0 && p.draft_done) {
      // draft statistics computed up front (k_draft_stats + k_slot_combine)
      const RowStat q = (pre && s < 64) ? RowStat{__shfl(my_sq.m, s, 64), __shfl(my_sq.s, s, 64)}
                                        : p.slot_q[row];
      if (!isfinite(q.s) || !(q.s > 0.0f)) {
        status |= SV_SEQ_ERR_NONFINITE;
        break;
      }
      mq = q.m;
      iq = 1.0f / q.s;
    } else if (nk > 0) {
    // draft statistics of this slot
    const RowStat qs = block_row_stats<VEC>(p.draft + (size_t)row * p.V, p.V, t0, t1, l2t, s_rs);
    // the workgroups' partials by tagged exchange (see tagged_exchange)
    ++xphase;
    unsigned long long* xbuf =
        p.xtag + ((size_t)b * 2 + (xphase & 1)) * kWalkGroupsPlainMax * kXWords;
    const float mine[2] = {qs.m, qs.s};
    if (!tagged_exchange<2>(xbuf, xphase, mine, G, s_xv, &s_flag)) {
      ok = false;
      break;
    }
    {
      // lane w holds workgroup w's partial, then a fixed butterfly (the same
      // in every workgroup)
      RowStat r{-INFINITY, 0.0f};
      if (lane < G) {
        r.m = s_xv[lane][0];
        r.s = s_xv[lane][1];
      }
      const float mm = wave_max(r.m);
      const float ss = wave_sum((r.m == -INFINITY) ? r.s : r.s * fast_exp2((r.m - mm) * l2t));
      if (!isfinite(ss) || !(ss > 0.0f)) {
        status |= SV_SEQ_ERR_NONFINITE;
        break;
      }
      mq = mm;
      iq = 1.0f / ss;
      if (wg == 0 && tid == 0 && p.dbg.slot_stats != nullptr) {
        p.dbg.slot_stats[(size_t)row * 4 + 2] = mm;
        p.dbg.slot_stats[(size_t)row * 4 + 3] = ss;
      }
    }
    }
    if (WARP) {
      // the warped rows: p and q restricted to their kept sets, renormalised
      WarpRow wr[2];
      float kept[2];
      bool bad = false;
      if (!warp_slot<VEC>(p, b, wg, G, t0, t1, zt, zd, mp, mq, nk > 0, l2t,
                          1.4426950408889634 / (double)T, &target, &xphase, s_xv, &s_flag,
                          s_warp, wr, kept,
                          &bad)) {
        ok = false;
        break;
      }
      if (bad || !(kept[0] > 0.0f) || (nk > 0 && !(kept[1] > 0.0f))) {
        status |= SV_SEQ_ERR_INTERNAL;
        break;
      }
      wt = warp_row_uniform(wr[0]);
      wd = warp_row_uniform(wr[1]);
      ip = 1.0f / kept[0];
      if (nk > 0) iq = 1.0f / kept[1];
      if (wg == 0 && tid == 0 && p.dbg.slot_stats != nullptr) {
        p.dbg.slot_stats[(size_t)row * 4 + 1] = kept[0];
        if (nk > 0) p.dbg.slot_stats[(size_t)row * 4 + 3] = kept[1];
      }
      if (nk == 0) break;
    }
    bool accepted = false;
    float prev = 1.0f;
    // the children's nodes, target and draft logits and uniforms, one lane per
    // child (up to 64), loaded together
    int cnode = 0, ckt = 1, ckd = 1;
    float czt = 0.0f, czd = 0.0f, cu = 0.0f;
    unsigned long long rest = kidmask;   // children not yet tested (prefetched walk)
    if (!pre && lane < nk) {
      cnode = p.kids[(size_t)row * p.maxc + lane];
      const int x = p.token[(size_t)b * N + cnode];
      czt = zt[x];
      czd = zd[x];
      if (WARP) {
        ckt = warp_kept(wt, czt, x, l2t8) ? 1 : 0;
        ckd = warp_kept(wd, czd, x, l2t8) ? 1 : 0;
      }
      bool w = false;
      cu = clamp_uniform(p.uniforms[(size_t)b * R + cnode], &w);
    }
    for (int i = 1; i <= nk; ++i) {
      // the i-th child, tested against the target adjusted by its i-1
      // rejected elder siblings
      int node;
      float px, qx, u;
      if (pre) {
        node = __ffsll((long long)rest) - 1;
        rest &= rest - 1;
        px = __shfl(my_px, node, 64);
        qx = __shfl(my_qx, node, 64);
        u = __shfl(my_u, node, 64);
      } else {
        node = __shfl(cnode, i - 1, 64);
        px = fast_exp2((__shfl(czt, i - 1, 64) - mp) * l2t) * ip;
        qx = fast_exp2((__shfl(czd, i - 1, 64) - mq) * l2t) * iq;
        if (WARP) {
          if (!__shfl(ckt, i - 1, 64)) px = 0.0f;
          if (!__shfl(ckd, i - 1, 64)) qx = 0.0f;
        }
        u = __shfl(cu, i - 1, 64);
      }
      const float num = fmaxf(0.0f, px - c * qx);
      if (wg == 0 && tid == 0 && p.dbg.node_ratio != nullptr)
        p.dbg.node_ratio[(size_t)b * N + node] = (qx > 0.0f) ? S * num / (n * qx) : INFINITY;
      if (u * n * qx <= S * num) {
        if (tid == 0) s_path[plen] = node;
        ++plen;
        s = node + 1;
        accepted = true;
        break;
      }
      // residual pass i: the mass of (p - (c + n / S) q)_+
      const float ci = c + n / S;
      const int wbuf = effbuf ^ 1;
      float* out = p.tmass + ((size_t)b * 2 + wbuf) * CT;
      const float part = block_residual<VEC, WARP, true>(zt, zd, p.V, t0, t1, mp, ip, mq, iq, ci,
                                                         l2t, wt, wd, out, s_f);
      ++xphase;
      unsigned long long* xbuf =
          p.xtag + ((size_t)b * 2 + (xphase & 1)) * kWalkGroupsPlainMax * kXWords;
      const float mine[1] = {part};
      if (!tagged_exchange<1>(xbuf, xphase, mine, G, s_xv, &s_flag)) {
        ok = false;
        break;
      }
      const float mi = wave_sum(lane < G ? s_xv[lane][0] : 0.0f);
      if (wg == 0 && tid == 0 && p.dbg.residual_mass != nullptr)
        p.dbg.residual_mass[(size_t)row * p.maxc + (i - 1)] = mi / prev;
      if (mi > 0.0f && isfinite(mi)) {
        c = ci;
        n = mi;
        eff = i;
        effbuf = wbuf;
        prev = mi;
      } else {
        status |= SV_SEQ_WARN_RESIDUAL;
      }
      if (p.distinct && i < nk) {
        // the next sibling was drawn from q with this token removed:
        // q_i = q / S on the tokens not yet drawn, S = 1 - their mass so far
        const float rest = S - qx;
        if (rest > 0.0f) S = rest;
        else status |= SV_SEQ_WARN_RESIDUAL;
      }
    }
    if (!ok || !accepted) break;   // all children rejected: s is the terminal slot
  }
  if (WARP && ok && !(status & kSeqErrMask) && eff == 0) {
    // the terminal draw is from the warped target itself: its tile masses
    const int wbuf = effbuf ^ 1;
    float* out = p.tmass + ((size_t)b * 2 + wbuf) * CT;
    block_residual<VEC, true, false>(p.logits + (size_t)(b * R + s) * p.V, nullptr, p.V, t0, t1,
                                     mp, ip, 0.0f, 0.0f, 0.0f, l2t, wt, wd, out, s_f);
    target += G;
    if (walk_barrier(p, b, &xphase, G, s_xv, &s_flag)) effbuf = wbuf;
    else ok = false;
  }
  if (!ok) status |= SV_SEQ_ERR_INTERNAL;
  if (wg != 0) return;

  // ---- final draw (workgroup 0) ----
  __syncthreads();
  if (tid == 0) {
    s_token = -1;
    s_clamp = 0;
  }
  __syncthreads();
  if (!(status & kSeqErrMask)) {
    const int row = b * R + s;
    const float* tm = (eff > 0 || WARP) ? p.tmass + ((size_t)b * 2 + effbuf) * CT : nullptr;
    if (wave == 0) {
      bool w = false;
      const float u = clamp_uniform(p.uniforms[(size_t)b * R + N], &w);
      // Tile masses of the terminal distribution, 8 consecutive tiles per
      // lane (512 per round, all loads of a round in flight together).
      constexpr int kPL = 8;
      float total = 0.0f;
      for (int c0 = 0; c0 < CT; c0 += 64 * kPL) {
        float ls = 0.0f;
#pragma unroll
        for (int k = 0; k < kPL; ++k) {
          const int t = c0 + kPL * lane + k;
          ls += (t < CT) ? tile_mass(p, row, tm, t, mp, ip, l2t) : 0.0f;
        }
        total += __shfl(wave_incl_scan(ls), 63, 64);
      }
      const float tgt = u * total;
      // first tile in ascending order with positive mass whose inclusive
      // cumulative mass exceeds the target
      float run = 0.0f, before = 0.0f;
      int j = -1, last_pos = -1;
      for (int c0 = 0; c0 < CT && j < 0; c0 += 64 * kPL) {
        float tmv[kPL];
        float ls = 0.0f;
#pragma unroll
        for (int k = 0; k < kPL; ++k) {
          const int t = c0 + kPL * lane + k;
          tmv[k] = (t < CT) ? tile_mass(p, row, tm, t, mp, ip, l2t) : 0.0f;
          ls += tmv[k];
        }
        const float incl = wave_incl_scan(ls);
        float cum = run + (incl - ls);
        int hitk = -1, lastk = -1;
        float bef = 0.0f;
#pragma unroll
        for (int k = 0; k < kPL; ++k) {
          if (tmv[k] > 0.0f) {
            lastk = k;
            if (hitk < 0 && cum + tmv[k] > tgt) {
              hitk = k;
              bef = cum;
            }
          }
          cum += tmv[k];
        }
        const unsigned long long hit = __ballot(hitk >= 0);
        const unsigned long long pos = __ballot(lastk >= 0);
        if (pos) {
          const int lp = 63 - __clzll((long long)pos);
          last_pos = c0 + kPL * lp + __shfl(lastk, lp, 64);
        }
        if (hit) {
          const int f = __ffsll((long long)hit) - 1;
          j = c0 + kPL * f + __shfl(hitk, f, 64);
          before = __shfl(bef, f, 64);
        }
        run += __shfl(incl, 63, 64);
      }
      int clamp = 0;
      if (j < 0) {
        // rounding defeated every tile comparison: draw from the last positive tile
        j = last_pos >= 0 ? last_pos : 0;
        clamp = 1;
        before = 0.0f;
        for (int base = 0; base < j; base += 64) {
          const int t = base + lane;
          before += wave_sum((t < j) ? tile_mass(p, row, tm, t, mp, ip, l2t) : 0.0f);
        }
      }
      if (lane == 0) {
        s_clamp = clamp;
        s_tile = j;
        s_run = before;
        s_target = tgt;
      }
    }
    __syncthreads();
    // block prefix sum over the chosen tile, one token per thread
    const int v = s_tile * kStatTile + tid;
    float wv = 0.0f;
    if (v < p.V) {
      const float zv = p.logits[(size_t)row * p.V + v];
      float pv = fast_exp2((zv - mp) * l2t) * ip;
      if (WARP && !warp_kept(wt, zv, v, l2t8)) pv = 0.0f;
      if (eff == 0) {
        wv = pv;
      } else {
        const float dv = p.draft[(size_t)row * p.V + v];
        float qv = fast_exp2((dv - mq) * l2t) * iq;
        if (WARP && !warp_kept(wd, dv, v, l2t8)) qv = 0.0f;
        wv = fmaxf(0.0f, pv - c * qv);
      }
    }
    const float incl = wave_incl_scan(wv);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    float acc = s_run;
    for (int k = 0; k < wave; ++k) acc += wtot[k];
    acc += incl;
    const int first = (wv > 0.0f && acc > s_target) ? v : 0x7fffffff;
    const int lastpos = (wv > 0.0f) ? v : -1;
    const int first_all = block_min_int(first, shi);
    const int last_all = block_max_int(lastpos, shi);
    if (tid == 0) {
      if (first_all != 0x7fffffff) {
        s_token = first_all;
      } else {
        s_token = last_all >= 0 ? last_all : s_tile * kStatTile;
        s_clamp = 1;
      }
    }
  }
  __syncthreads();
  write_outputs(p, b, status | (s_clamp ? SV_SEQ_WARN_CDF_CLAMP : 0), plen, s_path, s_token);
}

// Workgroups of this walk kernel instance the GPU holds at once (occupancy x
// CUs); 0 when the runtime cannot tell.
static long long walk_capacity(int variant, const void* fn) {
  static int per_cu_cache[4] = {-1, -1, -1, -1};
  int per_cu = __atomic_load_n(&per_cu_cache[variant], __ATOMIC_RELAXED);
  if (per_cu < 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess)
      per_cu = 0;
    __atomic_store_n(&per_cu_cache[variant], per_cu, __ATOMIC_RELAXED);
  }
  return (long long)per_cu * device_cus();
}

// Workgroups per sampling sequence: the more, the faster each vocabulary pass,
// but the more arrivals at every barrier, and the walk is mostly barrier
// latency. Up to 64 (16 with top-k / top-p) while the walk's grid stays
// within 512 workgroups and each workgroup keeps at least 8 statistics tiles
// (at least 16 per sequence), then limited so that the whole grid is resident
// at once on an idle GPU (the barriers rely on it). Measured: 16 the best of 1-32
// at 32 sequences of V = 128256; at one sequence 32-64 slightly better than
// 16 at V = 128256, 16 slightly better at V = 32000, and fewer than 16 slower
// everywhere. variant indexes the kernel instance (float4 loads, warping).
static int walk_groups(int B, int CT, int variant, long long cap) {
  int g = (variant & 2) ? kWalkGroupsMax : kWalkGroupsPlainMax;
  while (g > 16 && ((long long)g * B > 512 || 8 * g > CT)) g >>= 1;
  while (g > 1 && (long long)g * B > cap) g >>= 1;
  return g;
}

hipError_t launch_sampling(const Plan& P, const Args& a, const float* logits, bool target_done,
                           hipStream_t s) {
  SampleParams p;
  p.logits = logits;
  p.draft = a.draft;
  p.token = a.token;
  p.uniforms = a.uniforms;
  p.temperature = a.temperature;
  p.nkids = ws_nkids(P, a.ws);
  p.kids = ws_kids(P, a.ws);
  p.flags = ws_flags(P, a.ws);
  p.tstat = ws_tstat(P, a.ws);
  p.slot_t = (RowStat*)(a.ws + P.off_slot_t);
  p.parent = a.parent;
  p.dpart = (RowStat*)(a.ws + P.off_dpart);
  p.slot_q = (RowStat*)(a.ws + P.off_slot_q);
  // The draft statistics of every internal sampling slot in one parallel
  // pass, instead of a barrier phase of the walk at each slot it visits, and
  // then a walk whose tests read prefetched registers. That pays when the
  // draft rows are few (the batch-1 shapes); for a large batch the pass over
  // every internal row costs more than the phases of the few slots the walks
  // visit (measured at 32 x 61 slots, V = 128256: sampling stage 0.148 ms up
  // front against 0.131 ms lazily).
  p.draft_done = ((size_t)P.B * P.R * P.V * sizeof(float) <= kDraftUpFrontBytes) ? 1 : 0;
  p.dparts = 1;
  p.xtag = ws_xtag(P, a.ws);
  p.tmass = (float*)(a.ws + P.off_tmass);
  p.bar = ws_bar(P, a.ws);
  p.B = P.B;
  p.N = P.N;
  p.R = P.R;
  p.V = P.V;
  p.C = P.C;
  p.CT = P.CT;
  p.maxc = P.max_children;
  p.target_done = target_done ? 1 : 0;
  p.distinct = (P.sampling == SV_SAMPLE_DISTINCT) ? 1 : 0;
  p.top_k = P.top_k;
  p.top_p = P.top_p;
  {
    int lg = 0;   // ceil(log2 V)
    while ((1ll << lg) < P.V) ++lg;
    const int shift = (63 - lg < 52) ? 63 - lg : 52;
    p.mass_scale = ldexp(1.0, shift);
    p.mass_unit = ldexp(1.0, -shift);
  }
  p.whc = (unsigned*)(a.ws + P.off_whc);
  p.whm = (unsigned long long*)(a.ws + P.off_whm);
  p.wtie = (int*)(a.ws + P.off_wtie);
  p.wtidx = (int*)(a.ws + P.off_wtidx);
  p.wgl = (unsigned long long*)(a.ws + P.off_wgl);
  p.wgcnt = (unsigned long long*)(a.ws + P.off_wgcnt);
  p.accept_len = a.accept_len;
  p.accept_path = a.accept_path;
  p.out_tokens = a.out_tokens;
  p.seq_status = a.seq_status;
  p.dbg = a.dbg;
  const int rows = P.B * P.R;
  // float4 loads need 16-byte aligned rows
  const bool vec = (P.V % 4 == 0) && (((uintptr_t)logits | (uintptr_t)a.draft) & 15) == 0;
  hipError_t e;
  if (p.draft_done) {
    // parts per draft row: about 1024 blocks over all rows (most rows of a
    // batch are leaves or greedy and exit), at least one tile each; a budget
    // of 4096 blocks (8-tile parts at 61 rows) was 1-1.5% slower per step
    int parts = (1024 + rows - 1) / rows;
    parts = parts < 1 ? 1 : (parts > kDraftPartsMax ? kDraftPartsMax : parts);
    parts = parts > P.CT ? P.CT : parts;
    p.dparts = parts;
  }
  if (!target_done && p.draft_done) {
    const dim3 grid(P.C + p.dparts, rows);
    if (vec)
      hipLaunchKernelGGL(k_row_draft_stats<true>, grid, dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL(k_row_draft_stats<false>, grid, dim3(kThreads), 0, s, p);
  } else if (!target_done) {
    if (vec)
      hipLaunchKernelGGL(k_row_stats<true>, dim3(P.C, rows), dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL(k_row_stats<false>, dim3(P.C, rows), dim3(kThreads), 0, s, p);
  } else if (p.draft_done) {
    if (vec)
      hipLaunchKernelGGL(k_draft_stats<true>, dim3(p.dparts, rows), dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL(k_draft_stats<false>, dim3(p.dparts, rows), dim3(kThreads), 0, s, p);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_slot_combine, dim3((rows + 3) / 4), dim3(kThreads), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool warp = P.warp != 0;
  const void* fns[4] = {(const void*)k_walk<false, false>, (const void*)k_walk<true, false>,
                        (const void*)k_walk<false, true>, (const void*)k_walk<true, true>};
  const int variant = (vec ? 1 : 0) + (warp ? 2 : 0);
  const void* fn = fns[variant];
  const long long cap = walk_capacity(variant, fn);
  const int G = walk_groups(P.B, P.CT, variant, cap);
  // blockIdx.x = workgroup of the sequence, blockIdx.y = sequence: dispatch
  // order is x-fastest, so each sequence's group is contiguous in it, and the
  // grid fits the idle GPU (G > 1). Alone, such a grid cannot stall its own
  // barriers whatever other kernels run beside it; several overlapping walks
  // could, once together they need more residency than the GPU has. A grid
  // within half of the GPU (the few-sequence shapes, and 32 sequences x 16)
  // takes a plain launch: the cooperative one cost ~16 us per step in the
  // runtime, and two such walks always fit together. A larger grid keeps the
  // cooperative launch and its residency guarantee. G = 1 (one workgroup per
  // sequence, any number of sequences) has no barrier between workgroups and
  // is always a plain launch.
  const dim3 grid(G, P.B);
  if (G == 1 || (long long)G * P.B * kPlainWalkShare <= cap) {
    switch (variant) {
      case 0: hipLaunchKernelGGL((k_walk<false, false>), grid, dim3(kThreads), 0, s, p); break;
      case 1: hipLaunchKernelGGL((k_walk<true, false>), grid, dim3(kThreads), 0, s, p); break;
      case 2: hipLaunchKernelGGL((k_walk<false, true>), grid, dim3(kThreads), 0, s, p); break;
      default: hipLaunchKernelGGL((k_walk<true, true>), grid, dim3(kThreads), 0, s, p); break;
    }
    return hipGetLastError();
  }
  void* args[] = {&p};
  return hipLaunchCooperativeKernel(fn, grid, dim3(kThreads), args, 0, s);
}

}  // namespace sv
