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
// Data-parallel formulation used here. After i rejections at slot s the
// adjusted target is p_i = (p - c_i q)_+ / N_i, with c_0 = 0, N_0 = 1,
// c_{i+1} = c_i + N_i and N_{i+1} = sum_v (p - c_{i+1} q)_+ : subtracting q
// from a distribution of the form (p - c q)_+/N and renormalising gives
// (p - (c + N) q)_+ / N' because the positive part of p - c q only shrinks
// where p - c q is already positive. So every adjusted distribution of a
// slot is fixed by one scalar c, and its mass is one vocabulary pass. The
// acceptance test of the i-th child, u * q(x) <= p_{i-1}(x), becomes
// u * N_{i-1} * q(x) <= (p(x) - c_{i-1} q(x))_+ . None of this depends on the
// walk's outcome, so it is computed for all slots in parallel:
//   k_row_stats   per (row, 256-token tile): max and sum of exp((z - max)/T)
//                 of draft rows of slots with children, and of target rows
//                 unless the LM-head GEMM already produced them in its
//                 epilogue; argmax partials for greedy rows.
//   k_slot_combine one wave per row merges the tile statistics into the
//                 row's (max, sum) or (argmax value, index).
//   k_chain_pass  pass i for every slot with >= i children: the decision of
//                 its i-th child and the tile masses of (p - c_i q)_+ (the
//                 masses the final inverse-CDF draw scans).
//   k_walk        one block per sequence: walks the precomputed decisions
//                 root-down, then draws the final token by a scan over tile
//                 masses and a block prefix sum inside one 256-token tile.
// Reductions use fixed orders (no float atomics), so results are bitwise
// reproducible.
#include "sv_internal.h"

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
  RowStat* dstat;          // [B*R, CT] tile statistics, draft rows
  RowStat* slot_t;         // [B*R] merged target statistics
  RowStat* slot_d;         // [B*R] merged draft statistics
  float* chain;            // [B*R, maxc, CT] tile masses of (p - c_i q)_+
  float* cpart;            // [B*R, maxc, C] the same masses summed per block (16 tiles)
  int32_t* node_acc;       // [B*N]
  int B, N, R, V, C, CT, maxc;
  int target_done;         // target tile statistics already written (GEMM epilogue)
  int32_t* accept_len;
  int32_t* accept_path;
  int32_t* out_tokens;
  int32_t* seq_status;
  sv_debug dbg;
};

constexpr int kThreads = 256;
constexpr int kTilesPerChunk = kVocabChunk / kStatTile;   // 16, 4 per wave

// ---------------------------------------------------------------------------
// reductions in fixed orders (no float atomics): lane-strided partials, then
// butterflies; block results combine the 4 waves in order
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

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Sum of n values; every lane of the wave gets the same result.
__device__ __forceinline__ float wave_sum_chunks(const float* v, int n) {
  float s = 0.0f;
  for (int c = lane_id(); c < n; c += 64) s += v[c];
  return wave_sum(s);
}

// Merge n tile statistics of a sampling row into (max, sum exp((z-max)/T)).
__device__ __forceinline__ RowStat wave_merge_stats(const RowStat* st, int n, float l2t) {
  float m = -INFINITY;
  for (int c = lane_id(); c < n; c += 64) m = fmaxf(m, st[c].m);
  m = wave_max(m);
  float s = 0.0f;
  for (int c = lane_id(); c < n; c += 64) {
    const RowStat r = st[c];
    s += (r.m == -INFINITY) ? r.s : r.s * fast_exp2((r.m - m) * l2t);
  }
  RowStat out;
  out.m = m;
  out.s = wave_sum(s);     // a NaN tile marker propagates
  return out;
}

// Merge n tile argmax statistics: (value, lowest index); value NaN if any tile was.
__device__ __forceinline__ RowStat wave_merge_argmax(const RowStat* st, int n) {
  float v = -INFINITY;
  int idx = 0x7fffffff;
  bool bad = false;
  for (int c = lane_id(); c < n; c += 64) {
    const RowStat r = st[c];
    if (isnan(r.m)) bad = true;
    else argmax_merge(v, idx, r.m, __float_as_int(r.s));
  }
  wave_argmax(v, idx);
  const bool any_bad = __ballot(bad) != 0;
  RowStat out;
  out.m = any_bad ? NAN : v;
  out.s = __int_as_float(idx);
  return out;
}

// (c, N) of the adjusted target after k rejections at a slot, from the block
// sums of passes 1..k (p_k = (p - c q)_+ / N). A pass whose mass is not
// positive and finite keeps the previous distribution (*fallback). *eff = the
// last pass whose distribution is in effect (0 = the plain target).
__device__ __forceinline__ void wave_chain_state(const float* cpart_row, int C, int k,
                                                 float* c_out, float* n_out, int* eff,
                                                 bool* fallback) {
  float c = 0.0f, n = 1.0f;
  int e = 0;
  for (int kk = 1; kk <= k; ++kk) {
    const float m = wave_sum_chunks(cpart_row + (size_t)(kk - 1) * C, C);
    if (m > 0.0f && isfinite(m)) {
      c = c + n;
      n = m;
      e = kk;
    } else {
      *fallback = true;
    }
  }
  *c_out = c;
  *n_out = n;
  *eff = e;
}

// Four values of one 256-token tile for this lane (tokens in ascending order
// within the lane); out-of-range tokens read as -inf.
template <bool VEC>
__device__ __forceinline__ void load_tile4(const float* z, int v0, int V, float (&x)[4],
                                           int (&idx)[4]) {
  const int lane = lane_id();
  if (VEC) {
    const int v = v0 + 4 * lane;
    if (v + 3 < V) {
      const float4 f = *(const float4*)(z + v);
      x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (v + e < V) ? z[v + e] : -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) idx[e] = v + e;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = v0 + lane + 64 * e;
      idx[e] = v;
      x[e] = (v < V) ? z[v] : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// row statistics per (row, 256-token tile); a block covers 16 tiles, 4 per wave
// ---------------------------------------------------------------------------

template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_row_stats(SampleParams p) {
  const int chunk = blockIdx.x;
  const int row = blockIdx.y;
  // z = 0 target rows, z = 1 draft rows; a single z plane covers draft rows
  // only when the target statistics came from the GEMM epilogue
  const bool draft = p.target_done || blockIdx.z == 1;
  const int b = row / p.R;
  if (p.flags[b] & kSeqErrMask) return;
  const float T = p.temperature[b];
  const bool greedy = (T == 0.0f);
  if (draft && (greedy || p.nkids[row] == 0)) return;
  const float* z = (draft ? p.draft : p.logits) + (size_t)row * p.V;
  RowStat* out = (draft ? p.dstat : p.tstat) + (size_t)row * p.CT;
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

// ---------------------------------------------------------------------------
// per-slot merge: one wave per row
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void k_slot_combine(SampleParams p) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.B * p.R) return;
  const int b = row / p.R;
  const int lane = lane_id();
  if (p.flags[b] & kSeqErrMask) return;
  const float T = p.temperature[b];
  float dbgv[4] = {0.f, 0.f, 0.f, 0.f};
  int am = -1;
  if (T == 0.0f) {
    const RowStat r = wave_merge_argmax(p.tstat + (size_t)row * p.CT, p.CT);
    if (lane == 0) p.slot_t[row] = r;
    dbgv[0] = r.m;
    am = __float_as_int(r.s);
  } else {
    const float l2t = kLog2e / T;
    const RowStat r = wave_merge_stats(p.tstat + (size_t)row * p.CT, p.CT, l2t);
    if (lane == 0) p.slot_t[row] = r;
    dbgv[0] = r.m;
    dbgv[1] = r.s;
    if (p.nkids[row] > 0) {
      const RowStat d = wave_merge_stats(p.dstat + (size_t)row * p.CT, p.CT, l2t);
      if (lane == 0) p.slot_d[row] = d;
      dbgv[2] = d.m;
      dbgv[3] = d.s;
    }
  }
  if (lane == 0) {
    if (p.dbg.slot_stats != nullptr)
      for (int k = 0; k < 4; ++k) p.dbg.slot_stats[(size_t)row * 4 + k] = dbgv[k];
    if (p.dbg.slot_argmax != nullptr) p.dbg.slot_argmax[row] = am;
  }
}

// ---------------------------------------------------------------------------
// residual passes; a block covers 16 tiles of one slot row, 4 per wave
// ---------------------------------------------------------------------------

template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_chain_pass(SampleParams p, int pass) {
  const int chunk = blockIdx.x;
  const int row = blockIdx.y;
  const int b = row / p.R;
  if (p.flags[b] & kSeqErrMask) return;
  const float T = p.temperature[b];
  if (T == 0.0f || p.nkids[row] < pass) return;
  const float l2t = kLog2e / T;
  const RowStat st = p.slot_t[row];
  const RowStat sd = p.slot_d[row];
  const float mp = st.m, ip = 1.0f / st.s, mq = sd.m, iq = 1.0f / sd.s;
  // every wave computes the same chain state (same loads, same order)
  float c, n;
  int eff;
  bool fb = false;
  wave_chain_state(p.cpart + (size_t)row * p.maxc * p.C, p.C, pass - 1, &c, &n, &eff, &fb);
  const float ci = c + n;
  const float* zt = p.logits + (size_t)row * p.V;
  const float* zd = p.draft + (size_t)row * p.V;
  float* out = p.chain + ((size_t)row * p.maxc + (pass - 1)) * p.CT;
  const int wave = threadIdx.x >> 6;
  __shared__ float s_wsum[4];
  float wtot = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int tile = chunk * kTilesPerChunk + 4 * wave + q;
    if (tile >= p.CT) break;
    float xt[4], xd[4];
    int idx[4];
    load_tile4<VEC>(zt, tile * kStatTile, p.V, xt, idx);
    load_tile4<VEC>(zd, tile * kStatTile, p.V, xd, idx);
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (idx[e] < p.V) {
        const float pv = fast_exp2((xt[e] - mp) * l2t) * ip;
        const float qv = fast_exp2((xd[e] - mq) * l2t) * iq;
        acc += fmaxf(0.0f, pv - ci * qv);
      }
    }
    acc = wave_sum(acc);
    wtot += acc;
    if (lane_id() == 0) out[tile] = acc;
  }
  if (lane_id() == 0) s_wsum[wave] = wtot;
  __syncthreads();
  if (threadIdx.x == 0)
    p.cpart[((size_t)row * p.maxc + (pass - 1)) * p.C + chunk] =
        (s_wsum[0] + s_wsum[1]) + (s_wsum[2] + s_wsum[3]);
  if (chunk == 0 && threadIdx.x == 0) {
    // the pass-th child, tested against the target adjusted by its pass-1
    // rejected elder siblings
    const int node = p.kids[(size_t)row * p.maxc + (pass - 1)];
    const int x = p.token[(size_t)b * p.N + node];
    const float px = fast_exp2((zt[x] - mp) * l2t) * ip;
    const float qx = fast_exp2((zd[x] - mq) * l2t) * iq;
    const float num = fmaxf(0.0f, px - c * qx);
    bool warn = false;
    const float u = clamp_uniform(p.uniforms[(size_t)b * p.R + node], &warn);
    p.node_acc[(size_t)b * p.N + node] = (u * n * qx <= num) ? 1 : 0;
    if (p.dbg.node_ratio != nullptr)
      p.dbg.node_ratio[(size_t)b * p.N + node] = (qx > 0.0f) ? num / (n * qx) : INFINITY;
  }
}

// ---------------------------------------------------------------------------
// the walk and the final draw: one block per sequence
// ---------------------------------------------------------------------------

// mass of tile t of the terminal distribution (pass `eff`, or the target)
__device__ __forceinline__ float tile_mass(const SampleParams& p, int row, int eff, int t,
                                           float mp, float ip, float l2t) {
  if (eff == 0) {
    const RowStat r = p.tstat[(size_t)row * p.CT + t];
    return (r.m == -INFINITY) ? 0.0f : r.s * fast_exp2((r.m - mp) * l2t) * ip;
  }
  return p.chain[((size_t)row * p.maxc + (eff - 1)) * p.CT + t];
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

__global__ __launch_bounds__(kThreads) void k_walk(SampleParams p) {
  __shared__ int s_path[kMaxNodes];
  __shared__ int s_plen, s_term, s_k, s_token, s_status, s_tile, s_clamp;
  __shared__ float s_target, s_run, s_c, s_mp, s_ip, s_mq, s_iq;
  __shared__ int shi[4];
  __shared__ float wtot[4];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int N = p.N, R = p.R, CT = p.CT;
  const int flags = p.flags[b];
  if (flags & kSeqErrMask) {
    for (int j = tid; j < N; j += kThreads) p.accept_path[(size_t)b * N + j] = -1;
    for (int j = tid; j < R; j += kThreads) p.out_tokens[(size_t)b * R + j] = -1;
    if (tid == 0) {
      p.accept_len[b] = -1;
      p.seq_status[b] = flags;
    }
    return;
  }
  const float T = p.temperature[b];
  const bool greedy = (T == 0.0f);
  const float l2t = greedy ? 0.0f : kLog2e / T;
  if (tid == 0) {
    s_status = flags;
    s_plen = 0;
    s_token = -1;
    s_clamp = 0;
    s_k = 0;
    s_term = 0;
  }
  __syncthreads();
  if (!greedy) {
    bool warn = false;
    for (int j = tid; j < R; j += kThreads) clamp_uniform(p.uniforms[(size_t)b * R + j], &warn);
    if (warn) atomicOr(&s_status, SV_SEQ_WARN_UNIFORM);
    if (p.dbg.residual_mass != nullptr) {
      for (int s = wave; s < R; s += 4) {
        const int row = b * R + s;
        float prev = 1.0f;
        for (int i = 0; i < p.nkids[row]; ++i) {
          const float m = wave_sum_chunks(p.cpart + ((size_t)row * p.maxc + i) * p.C, p.C);
          if (lane == 0) p.dbg.residual_mass[(size_t)row * p.maxc + i] = m / prev;
          if (m > 0.0f && isfinite(m)) prev = m;
        }
      }
    }
  }
  __syncthreads();

  // the walk: wave 0, lanes test the children of a slot in parallel
  if (wave == 0) {
    int s = 0, plen = 0, status = 0;
    while (true) {
      const int row = b * R + s;
      const int nk = p.nkids[row];
      int node = -1;
      bool pick = false;
      if (lane < nk) node = p.kids[(size_t)row * p.maxc + lane];
      if (greedy) {
        const RowStat st = p.slot_t[row];
        if (isnan(st.m)) {
          status |= SV_SEQ_ERR_NONFINITE;
          break;
        }
        const int a = __float_as_int(st.s);
        if (lane < nk) pick = (p.token[(size_t)b * N + node] == a);
        const unsigned long long m = __ballot(pick);
        if (m == 0ull) {
          if (lane == 0) s_token = a;
          break;
        }
        const int first = __ffsll((long long)m) - 1;
        const int nxt = __shfl(node, first, 64);
        if (lane == 0) s_path[plen] = nxt;
        ++plen;
        s = nxt + 1;
      } else {
        if (nk > 0) {
          const RowStat st = p.slot_t[row];
          const RowStat sd = p.slot_d[row];
          if (!isfinite(st.s) || !isfinite(sd.s)) {
            status |= SV_SEQ_ERR_NONFINITE;
            break;
          }
        }
        if (lane < nk) pick = p.node_acc[(size_t)b * N + node] != 0;
        const unsigned long long m = __ballot(pick);
        if (m == 0ull) {
          if (lane == 0) s_k = nk;
          break;
        }
        const int first = __ffsll((long long)m) - 1;
        const int nxt = __shfl(node, first, 64);
        if (lane == 0) s_path[plen] = nxt;
        ++plen;
        s = nxt + 1;
      }
    }
    if (lane == 0) {
      s_plen = plen;
      s_term = s;
      s_status |= status;
    }
  }
  __syncthreads();

  if (!greedy && !(s_status & kSeqErrMask)) {
    // terminal distribution: the target at s_term after s_k rejections
    const int row = b * R + s_term;
    if (wave == 0) {
      const RowStat st = p.slot_t[row];
      const float mp = st.m, ip = 1.0f / st.s;
      bool bad = !isfinite(st.s) || !(st.s > 0.0f);
      float mq = 0.0f, iq = 1.0f, c = 0.0f, n = 1.0f;
      int eff = 0;
      bool fb = false;
      if (s_k > 0) {
        const RowStat sd = p.slot_d[row];
        mq = sd.m;
        iq = 1.0f / sd.s;
        bad = bad || !isfinite(sd.s) || !(sd.s > 0.0f);
        wave_chain_state(p.cpart + (size_t)row * p.maxc * p.C, p.C, s_k, &c, &n, &eff, &fb);
      }
      bool w = false;
      const float u = clamp_uniform(p.uniforms[(size_t)b * R + N], &w);
      // inclusive scan of tile masses in ascending order, 64 tiles at a time
      float total = 0.0f;
      for (int base = 0; base < CT; base += 64) {
        const int t = base + lane;
        const float cs = (t < CT) ? tile_mass(p, row, eff, t, mp, ip, l2t) : 0.0f;
        total += __shfl(wave_incl_scan(cs), 63, 64);
      }
      const float target = u * total;
      float run = 0.0f, before = 0.0f;
      int j = -1, last_pos = -1;
      for (int base = 0; base < CT && j < 0; base += 64) {
        const int t = base + lane;
        const float cs = (t < CT) ? tile_mass(p, row, eff, t, mp, ip, l2t) : 0.0f;
        const float incl = wave_incl_scan(cs);
        const unsigned long long hit = __ballot(t < CT && cs > 0.0f && run + incl > target);
        const unsigned long long pos = __ballot(t < CT && cs > 0.0f);
        if (pos) last_pos = base + 63 - __clzll((long long)pos);
        if (hit) {
          const int f = __ffsll((long long)hit) - 1;
          j = base + f;
          before = run + __shfl(incl - cs, f, 64);
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
          before += wave_sum((t < j) ? tile_mass(p, row, eff, t, mp, ip, l2t) : 0.0f);
        }
      }
      if (lane == 0) {
        if (bad) s_status |= SV_SEQ_ERR_NONFINITE;
        if (fb) s_status |= SV_SEQ_WARN_RESIDUAL;
        s_clamp = clamp;
        s_mp = mp;
        s_ip = ip;
        s_mq = mq;
        s_iq = iq;
        s_c = c;
        s_k = eff;
        s_tile = j;
        s_run = before;
        s_target = target;
      }
    }
    __syncthreads();
    if (!(s_status & kSeqErrMask)) {
      // block prefix sum over the chosen tile, one token per thread
      const int v = s_tile * kStatTile + tid;
      float wv = 0.0f;
      if (v < p.V) {
        const float pv = fast_exp2((p.logits[(size_t)row * p.V + v] - s_mp) * l2t) * s_ip;
        if (s_k == 0) {
          wv = pv;
        } else {
          const float qv = fast_exp2((p.draft[(size_t)row * p.V + v] - s_mq) * l2t) * s_iq;
          wv = fmaxf(0.0f, pv - s_c * qv);
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
  }
  __syncthreads();

  const int plen = s_plen;
  const bool err = (s_status & kSeqErrMask) != 0;
  for (int j = tid; j < N; j += kThreads)
    p.accept_path[(size_t)b * N + j] = (!err && j < plen) ? s_path[j] : -1;
  for (int j = tid; j < R; j += kThreads) {
    int t = -1;
    if (!err) {
      if (j < plen) t = p.token[(size_t)b * N + s_path[j]];
      else if (j == plen) t = s_token;
    }
    p.out_tokens[(size_t)b * R + j] = t;
  }
  if (tid == 0) {
    p.accept_len[b] = err ? -1 : plen;
    p.seq_status[b] = s_status | (s_clamp ? SV_SEQ_WARN_CDF_CLAMP : 0);
  }
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
  p.dstat = (RowStat*)(a.ws + P.off_dstat);
  p.slot_t = (RowStat*)(a.ws + P.off_slot_t);
  p.slot_d = (RowStat*)(a.ws + P.off_slot_d);
  p.chain = (float*)(a.ws + P.off_chain);
  p.cpart = (float*)(a.ws + P.off_cpart);
  p.node_acc = (int32_t*)(a.ws + P.off_node_acc);
  p.B = P.B;
  p.N = P.N;
  p.R = P.R;
  p.V = P.V;
  p.C = P.C;
  p.CT = P.CT;
  p.maxc = P.max_children;
  p.target_done = target_done ? 1 : 0;
  p.accept_len = a.accept_len;
  p.accept_path = a.accept_path;
  p.out_tokens = a.out_tokens;
  p.seq_status = a.seq_status;
  p.dbg = a.dbg;
  const int rows = P.B * P.R;
  // float4 loads need 16-byte aligned rows
  const bool vec = (P.V % 4 == 0) && (((uintptr_t)logits | (uintptr_t)a.draft) & 15) == 0;
  const dim3 gstats(P.C, rows, target_done ? 1 : 2);
  if (vec)
    hipLaunchKernelGGL(k_row_stats<true>, gstats, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(k_row_stats<false>, gstats, dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_slot_combine, dim3((rows + 3) / 4), dim3(kThreads), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (P.N > 0) {
    for (int pass = 1; pass <= P.max_children; ++pass) {
      if (vec)
        hipLaunchKernelGGL(k_chain_pass<true>, dim3(P.C, rows), dim3(kThreads), 0, s, p, pass);
      else
        hipLaunchKernelGGL(k_chain_pass<false>, dim3(P.C, rows), dim3(kThreads), 0, s, p, pass);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(k_walk, dim3(P.B), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace sv
