// Tree-masked attention over a prefix KV cache and a packed draft tree.
//
// What is computed ("LLM speculative decoding: EAGLE", jingming.pro, sec. 4.2
// "Attention Mask"; EAGLE-2 excerpts, modelers.csdn.net, sec. 2.3.2): slot 0
// (the root) attends to the L prefix rows of its sequence; node j attends to
// those and to the tree rows of its ancestors and itself. Scores are
// q.k / sqrt(D), softmax over the visible keys, output = weighted sum of V.
// All R = N + 1 slots and the G = Hq / Hkv query heads of one KV head share
// that head's K/V, so one block streams a K/V split once for R*G query rows.
//
// Layout: kv [rows, 2, Hkv, D] (K then V per token row), node_hidden
// [B*R, Hq*D] holds the queries, out [B*R, Hq, D] fp32.
//
// Decomposition: grid (split, kv_head * row_groups, batch). A split is a
// contiguous key range of `chunk_keys` keys; single-split (sequence, head)
// pairs write normalised rows directly, multi-split ones write the
// unnormalised accumulator with its (max, sum) for the merge kernel.
#include "sv_internal.h"

namespace sv {

struct AttnParams {
  const void* kv;
  const int32_t* kv_offset;
  const void* q;
  const uint64_t* anc;
  const int32_t* flags;
  float* out;
  float* part_acc;   // [B][Hkv*RG][max_splits][rb][D]
  float2* part_ml;   // [B][Hkv*RG][max_splits][rb]
  int N, R, Hq, Hkv, G, rows_g, rb, RG, chunk_keys, max_splits;
  float scale_log2;  // log2(e) / sqrt(D)
};

__device__ __forceinline__ bool key_visible(int t, int L, int key_end, uint64_t anc) {
  if (t >= key_end) return false;
  if (t < L) return true;
  return (anc >> (t - L)) & 1ull;
}

// ---------------------------------------------------------------------------
// bf16, D = 128: MFMA 16x16x32 for S^T = K Q^T and O^T = V^T P^T
// ---------------------------------------------------------------------------
//
// Block = 8 waves (2 per SIMD, so one wave's softmax overlaps another's
// MFMAs); wave w owns QT query tiles of 16 rows, the block 128*QT rows.
// Per 64-key tile:
//   K tile [64][128] bf16 in LDS, rows padded to 272 B (conflict-free 16 B
//   fragment reads); V tile stored transposed Vt[128][64] bf16, rows padded
//   to 144 B, so a lane reads its 4 consecutive keys of one d as 8 bytes.
//   Waves 0-3 stage K and waves 4-7 stage V through registers; the next
//   tile's global loads are in flight during the current tile's math.
//   S^T (keys x queries) puts each query's scores in one lane column: the
//   row max needs only a reduction across the 4 lane groups, and the scores
//   already sit in the B-operand layout of the P^T product (the key order
//   inside the MFMA's k dimension is any order A and B agree on).
// Softmax: scores stay unscaled until exp2(fma(s, log2e/sqrt(D), -m)), with
// m a reference max in scaled units. The accumulator is rescaled only when
// a row's tile max exceeds its reference by more than 8 (a factor 256), so
// exponentials stay below 2^8 and the common case skips the rescale; the
// result (acc / sum) is exact for any reference.

constexpr int kD = 128;
constexpr int kKS = kD * 2 + 16;          // K row stride in LDS (bytes)
constexpr int kVS = kKeyTile * 2 + 16;    // Vt row stride in LDS (bytes)
constexpr float kRescaleSlack = 8.0f;     // log2 units

template <int QT>
__global__ __launch_bounds__(512, 1) void k_attn_mfma(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char lds_k[kKeyTile * kKS];
  __shared__ __attribute__((aligned(16))) char lds_v[kD * kVS];

  const int b = blockIdx.z;
  const int grp = blockIdx.y;
  const int g = grp / p.RG;
  const int rg = grp % p.RG;
  const int split = blockIdx.x;
  if (p.flags[b] & kSeqErrMask) return;
  const int base = p.kv_offset[b];
  const int total = p.kv_offset[b + 1] - base;
  const int L = total - p.N;
  const int nsplit = (total + p.chunk_keys - 1) / p.chunk_keys;
  if (split >= nsplit) return;
  const int key_begin = split * p.chunk_keys;
  const int key_end = min(total, key_begin + p.chunk_keys);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 15;      // row/column inside a 16x16 tile
  const int lg = lane >> 4;      // lane group 0..3

  const bf16_t* kv = (const bf16_t*)p.kv;
  const bf16_t* qp = (const bf16_t*)p.q;
  const size_t row_elems = (size_t)2 * p.Hkv * kD;
  const size_t hidden = (size_t)p.Hq * kD;
  const float sc = p.scale_log2;

  // query fragments and per-column ancestor masks
  bf16x8 qf[QT][4];
  uint64_t anc_q[QT];
  int qrow[QT];
  int nt_valid = 0;
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int tile_first = rg * p.rb + (wave * QT + t) * 16;
    const int qq = tile_first + lr;
    if (tile_first < p.rows_g) nt_valid = t + 1;
    qrow[t] = qq;
    anc_q[t] = 0;
    if (qq < p.rows_g) {
      const int slot = qq / p.G;
      const int h = g * p.G + qq % p.G;
      const bf16x8* src = (const bf16x8*)(qp + ((size_t)b * p.R + slot) * hidden + (size_t)h * kD);
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) qf[t][ds] = src[ds * 4 + lg];
      anc_q[t] = p.anc[(size_t)b * p.R + slot];
    } else {
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) qf[t][ds] = bf16x8{};
    }
  }

  f32x4 o[QT][8];
  float m_ref[QT], l_part[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    m_ref[t] = -INFINITY;
    l_part[t] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // global -> register staging: threads 0-255 move K, 256-511 move V
  const bool stage_k = tid < 256;
  const int st = tid & 255;
  const int v_kg = st & 15;      // V: keys 4*v_kg .. 4*v_kg+3
  const int v_dg = st >> 4;      // V: d = 8*v_dg .. 8*v_dg+7
  uint4 reg[4];
  auto load_tile = [&](int tile0) {
    if (stage_k) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = st + 256 * j;
        const int key = tile0 + (c >> 4);
        reg[j] = make_uint4(0, 0, 0, 0);
        if (key < key_end)
          reg[j] = *(const uint4*)(kv + (size_t)(base + key) * row_elems + (size_t)g * kD +
                                   (c & 15) * 8);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = tile0 + 4 * v_kg + j;
        reg[j] = make_uint4(0, 0, 0, 0);
        if (key < key_end)
          reg[j] = *(const uint4*)(kv + (size_t)(base + key) * row_elems +
                                   (size_t)(p.Hkv + g) * kD + v_dg * 8);
      }
    }
  };
  auto store_tile = [&]() {
    if (stage_k) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = st + 256 * j;
        *(uint4*)(lds_k + (c >> 4) * kKS + (c & 15) * 16) = reg[j];
      }
    } else {
      const uint32_t* w0 = (const uint32_t*)&reg[0];
      const uint32_t* w1 = (const uint32_t*)&reg[1];
      const uint32_t* w2 = (const uint32_t*)&reg[2];
      const uint32_t* w3 = (const uint32_t*)&reg[3];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wi = e >> 1;
        uint32_t lo, hi;
        if (e & 1) {
          lo = (w0[wi] >> 16) | (w1[wi] & 0xFFFF0000u);
          hi = (w2[wi] >> 16) | (w3[wi] & 0xFFFF0000u);
        } else {
          lo = (w0[wi] & 0xFFFFu) | (w1[wi] << 16);
          hi = (w2[wi] & 0xFFFFu) | (w3[wi] << 16);
        }
        *(uint2*)(lds_v + (v_dg * 8 + e) * kVS + v_kg * 8) = make_uint2(lo, hi);
      }
    }
  };

  const int ntiles = (key_end - key_begin + kKeyTile - 1) / kKeyTile;
  load_tile(key_begin);
  for (int it = 0; it < ntiles; ++it) {
    const int tile0 = key_begin + it * kKeyTile;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (it + 1 < ntiles) load_tile(tile0 + kKeyTile);
    if (nt_valid == 0) continue;

    // S^T = K Q^T for 4 key tiles x QT query tiles (unscaled scores)
    f32x4 s[QT][4];
#pragma unroll
    for (int t = 0; t < QT; ++t)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        const bf16x8 a = *(const bf16x8*)(lds_k + (16 * kt + lr) * kKS + (32 * ds + 8 * lg) * 2);
#pragma unroll
        for (int t = 0; t < QT; ++t)
          if (t < nt_valid) s[t][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[t][ds], s[t][kt], 0, 0, 0);
      }
    }

    const bool need_mask = (tile0 + kKeyTile > L) || (tile0 + kKeyTile > key_end);
    bf16x8 pb[QT][2];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      if (t >= nt_valid) continue;
      if (need_mask) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!key_visible(tile0 + 16 * kt + 4 * lg + i, L, key_end, anc_q[t]))
              s[t][kt][i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        mx = fmaxf(mx, fmaxf(fmaxf(s[t][kt][0], s[t][kt][1]), fmaxf(s[t][kt][2], s[t][kt][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mx_s = mx * sc;                     // scaled; -inf when all masked
      if (__ballot(mx_s > m_ref[t] + kRescaleSlack)) {
        const float m_new = fmaxf(m_ref[t], mx_s);
        const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_ref[t] - m_new);
        m_ref[t] = m_new;
        l_part[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          o[t][dt][0] *= alpha;
          o[t][dt][1] *= alpha;
          o[t][dt][2] *= alpha;
          o[t][dt][3] *= alpha;
        }
      }
      const float off = (m_ref[t] == -INFINITY) ? 0.0f : -m_ref[t];
      float psum = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(fmaf(s[t][kt][i], sc, off));
          s[t][kt][i] = e;
          psum += e;
        }
      l_part[t] += psum;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = (bf16_t)s[t][2 * ks][i];
          v[4 + i] = (bf16_t)s[t][2 * ks + 1][i];
        }
        pb[t][ks] = v;
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const char* row = lds_v + (16 * dt + lr) * kVS;
        const uint2 a0 = *(const uint2*)(row + (32 * ks + 4 * lg) * 2);
        const uint2 a1 = *(const uint2*)(row + (32 * ks + 16 + 4 * lg) * 2);
        uint4 av = make_uint4(a0.x, a0.y, a1.x, a1.y);
        const bf16x8 a = *(const bf16x8*)&av;
#pragma unroll
        for (int t = 0; t < QT; ++t)
          if (t < nt_valid) o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[t][ks], o[t][dt], 0, 0, 0);
      }
    }
  }

  // epilogue
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    if (t >= nt_valid) continue;
    float l = l_part[t];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int qq = qrow[t];
    if (qq >= p.rows_g) continue;
    const int slot = qq / p.G;
    const int h = g * p.G + qq % p.G;
    if (nsplit == 1) {
      const float inv = 1.0f / l;
      float* dst = p.out + (((size_t)b * p.R + slot) * p.Hq + h) * kD;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *(float4*)(dst + 16 * dt + 4 * lg) =
            make_float4(o[t][dt][0] * inv, o[t][dt][1] * inv, o[t][dt][2] * inv, o[t][dt][3] * inv);
    } else {
      const size_t pidx = (((size_t)b * gridDim.y + grp) * p.max_splits + split) * p.rb +
                          (qq - rg * p.rb);
      float* dst = p.part_acc + pidx * kD;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *(float4*)(dst + 16 * dt + 4 * lg) = make_float4(o[t][dt][0], o[t][dt][1], o[t][dt][2], o[t][dt][3]);
      if (lg == 0) p.part_ml[pidx] = make_float2(m_ref[t], l);
    }
  }
}

// ---------------------------------------------------------------------------
// VALU kernel: fp32 storage, or bf16 with D = 64. 32 query rows per block,
// 8 per wave; lane k scores key k of the tile, lanes then own d columns.
// ---------------------------------------------------------------------------

template <typename TIn>
__device__ __forceinline__ float ld_val(const TIn* p) { return (float)*p; }

template <typename TIn, int D>
__global__ __launch_bounds__(256) void k_attn_valu(AttnParams p) {
  constexpr int RBV = 32;
  constexpr int RPW = 8;
  constexpr int DPL = D / 64;     // d columns per lane
  __shared__ float Ks[kKeyTile][D + 1];
  __shared__ float Vs[kKeyTile][D];
  __shared__ float Qs[RBV][D];
  __shared__ float Acc[RBV][D];
  __shared__ float Ms[RBV], Ls[RBV];
  __shared__ uint64_t Anc[RBV];
  __shared__ float Ps[4][kKeyTile];

  const int b = blockIdx.z;
  const int grp = blockIdx.y;
  const int g = grp / p.RG;
  const int rg = grp % p.RG;
  const int split = blockIdx.x;
  if (p.flags[b] & kSeqErrMask) return;
  const int base = p.kv_offset[b];
  const int total = p.kv_offset[b + 1] - base;
  const int L = total - p.N;
  const int nsplit = (total + p.chunk_keys - 1) / p.chunk_keys;
  if (split >= nsplit) return;
  const int key_begin = split * p.chunk_keys;
  const int key_end = min(total, key_begin + p.chunk_keys);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const TIn* kv = (const TIn*)p.kv;
  const TIn* qp = (const TIn*)p.q;
  const size_t row_elems = (size_t)2 * p.Hkv * D;
  const size_t hidden = (size_t)p.Hq * D;

  for (int i = tid; i < RBV * D; i += 256) {
    const int r = i / D, dd = i % D;
    const int qq = rg * RBV + r;
    float v = 0.0f;
    if (qq < p.rows_g) {
      const int slot = qq / p.G, h = g * p.G + qq % p.G;
      v = ld_val(qp + ((size_t)b * p.R + slot) * hidden + (size_t)h * D + dd);
    }
    Qs[r][dd] = v;
    Acc[r][dd] = 0.0f;
  }
  if (tid < RBV) {
    const int qq = rg * RBV + tid;
    Ms[tid] = -INFINITY;
    Ls[tid] = 0.0f;
    Anc[tid] = (qq < p.rows_g) ? p.anc[(size_t)b * p.R + qq / p.G] : 0;
  }

  for (int tile0 = key_begin; tile0 < key_end; tile0 += kKeyTile) {
    __syncthreads();
    for (int i = tid; i < kKeyTile * D; i += 256) {
      const int k = i / D, dd = i % D;
      const int key = tile0 + k;
      float kvk = 0.0f, kvv = 0.0f;
      if (key < key_end) {
        const TIn* row = kv + (size_t)(base + key) * row_elems;
        kvk = ld_val(row + (size_t)g * D + dd);
        kvv = ld_val(row + (size_t)(p.Hkv + g) * D + dd);
      }
      Ks[k][dd] = kvk;
      Vs[k][dd] = kvv;
    }
    __syncthreads();
    for (int r = 0; r < RPW; ++r) {
      const int qr = wave * RPW + r;
      float sc = 0.0f;
#pragma unroll 8
      for (int dd = 0; dd < D; ++dd) sc += Qs[qr][dd] * Ks[lane][dd];
      sc *= p.scale_log2;
      if (!key_visible(tile0 + lane, L, key_end, Anc[qr])) sc = -INFINITY;
      const float m_old = Ms[qr];
      const float m_new = fmaxf(m_old, wave_max(sc));
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = fast_exp2(m_old - m_use);
      const float e = fast_exp2(sc - m_use);
      const float esum = wave_sum(e);
      Ps[wave][lane] = e;
      __syncthreads();
      if (lane == 0) {
        Ms[qr] = m_new;
        Ls[qr] = Ls[qr] * alpha + esum;
      }
#pragma unroll
      for (int j = 0; j < DPL; ++j) {
        float a = Acc[qr][lane + 64 * j] * alpha;
        for (int k = 0; k < kKeyTile; ++k) a += Ps[wave][k] * Vs[k][lane + 64 * j];
        Acc[qr][lane + 64 * j] = a;
      }
      __syncthreads();
    }
  }

  for (int r = 0; r < RPW; ++r) {
    const int ql = wave * RPW + r;
    const int qq = rg * RBV + ql;
    if (qq >= p.rows_g) continue;
    const int slot = qq / p.G, h = g * p.G + qq % p.G;
    if (nsplit == 1) {
      float* dst = p.out + (((size_t)b * p.R + slot) * p.Hq + h) * D;
#pragma unroll
      for (int j = 0; j < DPL; ++j) dst[lane + 64 * j] = Acc[ql][lane + 64 * j] / Ls[ql];
    } else {
      const size_t pidx = (((size_t)b * gridDim.y + grp) * p.max_splits + split) * p.rb + ql;
#pragma unroll
      for (int j = 0; j < DPL; ++j) p.part_acc[pidx * D + lane + 64 * j] = Acc[ql][lane + 64 * j];
      if (lane == 0) p.part_ml[pidx] = make_float2(Ms[ql], Ls[ql]);
    }
  }
}

// ---------------------------------------------------------------------------
// merge of split partials (log-sum-exp in base 2), and zero rows for
// sequences with an error. A thread owns 4 consecutive d of one row; grid
// (rows / rows-per-block, Hkv*RG, B), 256 threads.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_attn_merge(AttnParams p, int D) {
  const int tpr = D / 4;               // threads per row
  const int rpb = 256 / tpr;           // rows per block
  const int b = blockIdx.z, grp = blockIdx.y;
  const int g = grp / p.RG, rg = grp % p.RG;
  const int qloc = blockIdx.x * rpb + threadIdx.x / tpr;
  const int d = (threadIdx.x % tpr) * 4;
  if (qloc >= p.rb) return;
  const int qq = rg * p.rb + qloc;
  if (qq >= p.rows_g) return;
  const int slot = qq / p.G, h = g * p.G + qq % p.G;
  float4* dst = (float4*)(p.out + (((size_t)b * p.R + slot) * p.Hq + h) * D + d);
  if (p.flags[b] & kSeqErrMask) {
    *dst = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const int total = p.kv_offset[b + 1] - p.kv_offset[b];
  const int nsplit = (total + p.chunk_keys - 1) / p.chunk_keys;
  if (nsplit <= 1) return;        // written directly by the attention kernel
  const size_t pbase = (((size_t)b * gridDim.y + grp) * p.max_splits) * p.rb + qloc;
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, p.part_ml[pbase + (size_t)s * p.rb].x);
  float l = 0.0f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < nsplit; ++s) {
    const size_t pi = pbase + (size_t)s * p.rb;
    const float2 ml = p.part_ml[pi];
    if (ml.x == -INFINITY) continue;
    const float w = fast_exp2(ml.x - m);
    const float4 v = *(const float4*)(p.part_acc + pi * D + d);
    l += ml.y * w;
    a.x += v.x * w;
    a.y += v.y * w;
    a.z += v.z * w;
    a.w += v.w * w;
  }
  const float inv = 1.0f / l;
  *dst = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
}

hipError_t launch_attention(const Plan& P, const Args& a, hipStream_t s) {
  AttnParams p;
  p.kv = a.kv;
  p.kv_offset = a.kv_offset;
  p.q = a.hidden;
  p.anc = ws_anc(P, a.ws);
  p.flags = ws_flags(P, a.ws);
  p.out = a.attn_out;
  p.part_acc = (float*)(a.ws + P.off_part_acc);
  p.part_ml = (float2*)(a.ws + P.off_part_ml);
  p.N = P.N;
  p.R = P.R;
  p.Hq = P.Hq;
  p.Hkv = P.Hkv;
  p.G = P.G;
  p.rows_g = P.rows_g;
  p.rb = P.attn_rb;
  p.RG = P.attn_rg;
  p.chunk_keys = P.chunk_keys;
  p.max_splits = P.max_splits;
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)P.D);
  const dim3 grid(P.max_splits, P.Hkv * P.attn_rg, P.B);
  if (P.attn_mfma) {
    if (P.attn_qt == 2)
      hipLaunchKernelGGL(k_attn_mfma<2>, grid, dim3(512), 0, s, p);
    else
      hipLaunchKernelGGL(k_attn_mfma<1>, grid, dim3(512), 0, s, p);
  } else if (P.dtype == SV_F32) {
    if (P.D == 128)
      hipLaunchKernelGGL((k_attn_valu<float, 128>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((k_attn_valu<float, 64>), grid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((k_attn_valu<bf16_t, 64>), grid, dim3(256), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rpb = 256 / (P.D / 4);
  hipLaunchKernelGGL(k_attn_merge, dim3((P.attn_rb + rpb - 1) / rpb, P.Hkv * P.attn_rg, P.B),
                     dim3(256), 0, s, p, P.D);
  return hipGetLastError();
}

}  // namespace sv
