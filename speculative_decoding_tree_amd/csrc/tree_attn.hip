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
// Decomposition: a split is a contiguous key range of one sequence, of a
// length the tree preparation chose for this call from the actual prefix
// lengths; single-split (sequence, head) pairs write normalised rows
// directly, multi-split ones write the unnormalised accumulator with its
// (max, sum) for the merge kernel. The grid is one-dimensional: block i takes
// work item i / HG of the chosen schedule (the (sequence, split) pairs,
// longest first) and head group i % HG, so the blocks that run together read
// adjacent head slices of the same token rows, and the short last splits of
// the sequences fill the end of the grid instead of leaving CUs idle behind
// long ones.
#include "sv_internal.h"

namespace sv {

struct AttnParams {
  const void* kv;
  const int32_t* kv_offset;
  const void* q;
  const uint64_t* anc;
  const int32_t* flags;
  float* out;        // [B*R][Hq][D] fp32, or null
  uint16_t* out16;   // the same as bf16 (round to nearest even), or null
  float* part_acc;   // [B][Hkv*RG][max_splits][rb][D]
  float2* part_ml;   // [B][Hkv*RG][max_splits][rb]
  // n_cand schedules, sched_stride int32 apart: {item count, split keys,
  // estimated makespan lo, hi}, then item i at [4 + i] = b * max_splits + split
  const int32_t* sched;
  int32_t* nsplit;   // [B] splits of each sequence, for the merge
  int sched_stride, n_cand;
  int B, N, R, Hq, Hkv, G, rows_g, rb, RG, HG, max_splits;
  float scale_log2;  // log2(e) / sqrt(D)
};

// Item w of the schedule the tree preparation estimated fastest (lowest
// makespan, saturated at 2^26 - 1 half tiles; ties to the shorter split), with
// that schedule's item count and split length, the same in every lane of the
// wave. Lane j reads the header and item w of schedule j together, so the
// choice costs one memory round trip. Every lane of the wave must be active.
struct AttnPick {
  int count, chunk, item;
};
__device__ __forceinline__ AttnPick attn_pick(const AttnParams& p, int w) {
  const int lane = threadIdx.x & 63;
  uint32_t key = 0xffffffffu;
  int count = 0, chunk = 0, item = 0;
  if (lane < p.n_cand) {
    const int32_t* sj = p.sched + (size_t)lane * p.sched_stride;
    const int4 h = *(const int4*)sj;
    item = sj[4 + w];   // w < B * max_splits: inside the schedule
    count = h.x;
    chunk = h.y;
    const uint32_t cost = (h.w != 0 || (uint32_t)h.z > 0x3ffffffu) ? 0x3ffffffu : (uint32_t)h.z;
    key = (cost << 6) | (uint32_t)lane;
  }
  const int j = __builtin_amdgcn_readfirstlane((int)(wave_min_u32(key) & 63));
  AttnPick r;
  // (the schedules never hold more than B * max_splits items or splits
  // shorter than one key tile; the clamps keep every later index in bounds)
  r.count = min(__builtin_amdgcn_readfirstlane(__shfl(count, j, 64)), p.B * p.max_splits);
  r.chunk = max(__builtin_amdgcn_readfirstlane(__shfl(chunk, j, 64)), kKeyTile);
  r.item = __builtin_amdgcn_readfirstlane(__shfl(item, j, 64));
  return r;
}

// The (sequence, head group, split) of this block and the split length;
// false when the block has no work item.
__device__ __forceinline__ bool attn_item(const AttnParams& p, int* b, int* grp, int* split,
                                          int* chunk) {
  const int w = (int)(blockIdx.x / (unsigned)p.HG);
  *grp = (int)blockIdx.x - w * p.HG;
  const AttnPick pk = attn_pick(p, w);
  if (w >= pk.count) return false;
  *b = pk.item / p.max_splits;
  *split = pk.item - *b * p.max_splits;
  *chunk = pk.chunk;
  return (unsigned)*b < (unsigned)p.B;
}

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
//
// K/V streaming: key tiles of 64 rows go global -> LDS with
// global_load_lds_dwordx4 (no register staging) into a ring of 4 stages of
// 32 KB (K tile, then V tile, both row-major with 256-byte rows), so three
// tiles are in flight while one is consumed; one barrier per tile. One
// wave-instruction moves 4 rows (lane l lands at row l/16, 16-byte position
// l%16); the lane picks which 16-byte chunk of its row it fetches, so rows
// are XOR-swizzled on 16-byte chunks: K by (row & 15), which spreads a
// fragment read of 16 rows over all 16 positions; V by 2*(row & 7), which
// spreads the 4 rows x 32 bytes of a transposed read over 8 positions.
//
// S^T (keys x queries) puts each query's scores in one lane column: the row
// max needs only a reduction across the 4 lane groups, and the scores already
// sit in the B-operand layout of the P^T product (the key order inside the
// MFMA's k dimension is any order A and B agree on). The V^T operand comes
// from row-major V with ds_read_b64_tr_b16: per 16-lane group, source lane s
// addresses V[k0 + s/4][d0 + 4(s%4)] and lane j receives V[k0 + i][d0 + j],
// i = 0..3, i.e. 4 consecutive keys of one d column.
//
// Softmax: scores stay unscaled until exp2(fma(s, log2e/sqrt(D), -m)), with
// m a reference max in scaled units. The accumulator is rescaled only when
// a row's tile max exceeds its reference by more than 8 (a factor 256), so
// exponentials stay below 2^8 and the common case skips the rescale; the
// result (acc / sum) is exact for any reference.

typedef __attribute__((address_space(3))) void attn_lds_void_t;
typedef __attribute__((address_space(1))) void attn_glb_void_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// Stores 4 consecutive output values of row element e0 to whichever of the
// fp32 and bf16 outputs are given.
__device__ __forceinline__ void store_out4(const AttnParams& p, size_t e0, float4 v) {
  if (p.out != nullptr) *(float4*)(p.out + e0) = v;
  if (p.out16 != nullptr) {
    const uint32_t lo = (uint32_t)to_bf16_bits(v.x) | ((uint32_t)to_bf16_bits(v.y) << 16);
    const uint32_t hi = (uint32_t)to_bf16_bits(v.z) | ((uint32_t)to_bf16_bits(v.w) << 16);
    *(uint2*)(p.out16 + e0) = make_uint2(lo, hi);
  }
}

constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;                  // one K or V row of a head
constexpr int kOpBytes = kKeyTile * kRowBytes;     // 16 KB: K (or V) of a key tile
constexpr int kStageBytes = 2 * kOpBytes;
constexpr int kStages = 4;
constexpr float kRescaleSlack = 8.0f;     // log2 units

__device__ __forceinline__ int swz_k(int row) { return row & 15; }
__device__ __forceinline__ int swz_v(int row) { return (row & 7) << 1; }

// max over the 4 lane groups (lanes l, l^16, l^32, l^48): each permlane swap
// leaves the two values of a lane pair in the two results
__device__ __forceinline__ float xlg_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ds_read_b64_tr_b16 as inline asm. Through the builtin, the compiler's
// wait-count pass makes every such read wait for all in-flight global->LDS
// loads (it cannot tell that they target other stages of the ring), which
// would drain the K/V prefetch once per tile. The asm reads are invisible to
// that pass, so their results are fenced explicitly by lds_wait_all().
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
template <int OFF>
__device__ __forceinline__ u32x2_t ds_read_tr16(uint32_t lds_addr) {
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "i"(OFF));
  return r;
}

// vmcnt(n) with expcnt / lgkmcnt left at their maximum (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

template <int QT>
__global__ __launch_bounds__(512, 1) void k_attn_mfma(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[kStages * kStageBytes];

  int b, grp, split, chunk;
  if (!attn_item(p, &b, &grp, &split, &chunk)) return;
  const int g = grp / p.RG;
  const int rg = grp % p.RG;
  if (p.flags[b] & kSeqErrMask) return;
  const int base = p.kv_offset[b];
  const int total = p.kv_offset[b + 1] - base;
  const int L = total - p.N;
  const int nsplit = (total + chunk - 1) / chunk;
  if (split >= nsplit) return;
  if (split == 0 && grp == 0 && threadIdx.x == 0) p.nsplit[b] = nsplit;
  const int key_begin = split * chunk;
  const int key_end = min(total, key_begin + chunk);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform in SGPRs
  const int lane = tid & 63;
  const int lr = lane & 15;      // row/column inside a 16x16 tile
  const int lg = lane >> 4;      // lane group 0..3

  const bf16_t* kv = (const bf16_t*)p.kv;
  const bf16_t* qp = (const bf16_t*)p.q;
  const size_t row_elems = (size_t)2 * p.Hkv * kD;
  const size_t hidden = (size_t)p.Hq * kD;
  const float sc = p.scale_log2;

  // K/V streaming: this lane's rows and source chunks in its wave's 2 + 2
  // instructions per tile (rows 8*wave + 4*j + lane/16)
  const bf16_t* kbase = kv + (size_t)base * row_elems + (size_t)g * kD;
  const bf16_t* vbase = kv + (size_t)base * row_elems + (size_t)(p.Hkv + g) * kD;
  const int ntiles = (key_end - key_begin + kKeyTile - 1) / kKeyTile;
  // this lane's source rows in the tile (8 wave + 4 j + lane / 16) and their
  // swizzled chunks, as pointers to the next tile to copy: tiles are issued
  // in order, so a full tile advances them by 64 rows; the split's last
  // tile clamps rows past its end to a valid row
  const bf16_t* ksrc[2];
  const bf16_t* vsrc[2];
  int trow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 8 * wave + 4 * j + (lane >> 4);
    trow[j] = row;
    ksrc[j] = kbase + (size_t)(key_begin + row) * row_elems + ((lr ^ swz_k(row)) << 3);
    vsrc[j] = vbase + (size_t)(key_begin + row) * row_elems + ((lr ^ swz_v(row)) << 3);
  }
  const size_t tile_elems = (size_t)kKeyTile * row_elems;
  auto issue = [&](int t) {
    char* sb = lds + (t % kStages) * kStageBytes;
    const int tile0 = key_begin + t * kKeyTile;
    const bool full = tile0 + kKeyTile <= key_end;     // wave-uniform
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r0 = 8 * wave + 4 * j;
      const bf16_t* ks = ksrc[j];
      const bf16_t* vs = vsrc[j];
      if (!full) {
        const ptrdiff_t back =
            (ptrdiff_t)(tile0 + trow[j] - min(tile0 + trow[j], key_end - 1)) * (ptrdiff_t)row_elems;
        ks -= back;
        vs -= back;
      }
      __builtin_amdgcn_global_load_lds((attn_glb_void_t*)ks,
                                       (attn_lds_void_t*)(sb + r0 * kRowBytes), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((attn_glb_void_t*)vs,
                                       (attn_lds_void_t*)(sb + kOpBytes + r0 * kRowBytes), 16, 0,
                                       0);
      ksrc[j] += tile_elems;
      vsrc[j] += tile_elems;
    }
  };
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t)
    if (t < ntiles) issue(t);

  // query fragments and per-column ancestor masks; a wave computes all QT
  // tiles once it has a valid one (rows past rows_g hold zero queries and are
  // never stored), and skips the math when it has none
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

  // o: the accumulators of O^T; lsum: the row sums of P, taken by the same
  // MFMA with an all-ones A operand (every output row is the column sum of
  // P^T, i.e. the query's sum over the tile's keys of the bf16 P values the
  // products use), so the softmax adds no per-score sums
  f32x4 o[QT][8], lsum[QT];
  float m_ref[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    m_ref[t] = -INFINITY;
    lsum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (bf16_t)1.0f;

  // per-lane LDS offsets of the fragment reads (stage-relative)
  int koff[4];     // K rows 16*kt + lr; the chunk swizzle of those rows is lr
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) koff[kt] = (16 * kt + lr) * kRowBytes;
  // V^T reads: rows 32*ks + 4*lg + lr/4 (and +16, same swizzle), columns
  // 16*dt + 4*(lr%4): chunk 2*dt + (lr%4)/2, byte (lr%2)*8 inside it
  int voff[2][8];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int row = 32 * ks + 4 * lg + (lr >> 2);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      voff[ks][dt] = kOpBytes + row * kRowBytes +
                     (((2 * dt + ((lr & 3) >> 1)) ^ swz_v(row)) << 4) + (lr & 1) * 8;
  }
  // LDS byte address of the ring (the asm reads take raw LDS addresses)
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;

  for (int it = 0; it < ntiles; ++it) {
    if (it + 2 < ntiles) wait_vm<8>();
    else if (it + 1 < ntiles) wait_vm<4>();
    else wait_vm<0>();
    __syncthreads();   // tile `it` landed for every wave; stage (it - 1) % 4 is free
    if (it + kStages - 1 < ntiles) issue(it + kStages - 1);
    if (nt_valid == 0) continue;
    const int tile0 = key_begin + it * kKeyTile;
    const char* stg = lds + (it % kStages) * kStageBytes;

    // S^T = K Q^T for 4 key subtiles x QT query tiles (unscaled scores); the
    // 4 K fragments of a d-step are read together, one d-step ahead
    f32x4 s[QT][4];
#pragma unroll
    for (int t = 0; t < QT; ++t)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 ka[2][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      ka[0][kt] = *(const bf16x8*)(stg + koff[kt] + ((lg ^ lr) << 4));
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      if (ds + 1 < 4) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          ka[(ds + 1) & 1][kt] =
              *(const bf16x8*)(stg + koff[kt] + (((4 * (ds + 1) + lg) ^ lr) << 4));
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int t = 0; t < QT; ++t)
          s[t][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ds & 1][kt], qf[t][ds], s[t][kt], 0, 0, 0);
    }

    // V^T fragments of the first 32 keys, read while the softmax runs
    u32x2_t vlo[8], vhi[8];
    const uint32_t stg_addr = lds_base + (uint32_t)(it % kStages) * kStageBytes;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      vlo[dt] = ds_read_tr16<0>(stg_addr + voff[0][dt]);
      vhi[dt] = ds_read_tr16<16 * kRowBytes>(stg_addr + voff[0][dt]);
    }

    // visibility: keys past the split end, and tree keys outside the query's
    // ancestor set (only tiles that reach the tree rows or the split end)
    if ((tile0 + kKeyTile > L) || (tile0 + kKeyTile > key_end)) {
      const int P = min(max(min(L, key_end) - tile0, 0), 64);   // visible prefix keys [0, P)
      const int E = min(max(key_end - tile0, 0), 64);           // keys inside the split [0, E)
      const uint64_t pm = P >= 64 ? ~0ull : ((1ull << P) - 1ull);
      const uint64_t em = E >= 64 ? ~0ull : ((1ull << E) - 1ull);
      const int dsh = L - tile0;                                // key k <-> ancestor bit k - dsh
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        uint64_t tm = 0;
        if (dsh >= 0 && dsh < 64) tm = anc_q[t] << dsh;
        else if (dsh < 0 && dsh > -64) tm = anc_q[t] >> (-dsh);
        const uint64_t ml = ((pm | tm) & em) >> (4 * lg);     // bit 16*kt + i: key 16*kt + 4*lg + i
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const uint32_t nib = (uint32_t)(ml >> (16 * kt));
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!((nib >> i) & 1u)) s[t][kt][i] = -INFINITY;
        }
      }
    }

    bf16x8 pb[QT][2];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        mx = fmaxf(mx, fmaxf(fmaxf(s[t][kt][0], s[t][kt][1]), fmaxf(s[t][kt][2], s[t][kt][3])));
      mx = xlg_max(mx);
      const float mx_s = mx * sc;                     // scaled; -inf when all masked
      if (__ballot(mx_s > m_ref[t] + kRescaleSlack)) {
        const float m_new = fmaxf(m_ref[t], mx_s);
        const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_ref[t] - m_new);
        m_ref[t] = m_new;
        lsum[t][0] *= alpha;
        lsum[t][1] *= alpha;
        lsum[t][2] *= alpha;
        lsum[t][3] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          o[t][dt][0] *= alpha;
          o[t][dt][1] *= alpha;
          o[t][dt][2] *= alpha;
          o[t][dt][3] *= alpha;
        }
      }
      const float off = (m_ref[t] == -INFINITY) ? 0.0f : -m_ref[t];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[t][kt][i] = fast_exp2(fmaf(s[t][kt][i], sc, off));
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

    // O^T += V^T P^T; A slots 0-3 = keys 32ks + 4lg + 0..3, slots 4-7 = the
    // same + 16, matching the key order of pb
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // the 16 reads of this half are complete (the asm names them, so the
      // MFMAs below cannot move above the wait)
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(vlo[0]), "+v"(vlo[1]), "+v"(vlo[2]), "+v"(vlo[3]), "+v"(vlo[4]),
                     "+v"(vlo[5]), "+v"(vlo[6]), "+v"(vlo[7]), "+v"(vhi[0]), "+v"(vhi[1]),
                     "+v"(vhi[2]), "+v"(vhi[3]), "+v"(vhi[4]), "+v"(vhi[5]), "+v"(vhi[6]),
                     "+v"(vhi[7]));
      bf16x8 va[8];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const u32x2_t both[2] = {vlo[dt], vhi[dt]};
        va[dt] = *(const bf16x8*)both;
      }
      if (ks == 0) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          vlo[dt] = ds_read_tr16<0>(stg_addr + voff[1][dt]);
          vhi[dt] = ds_read_tr16<16 * kRowBytes>(stg_addr + voff[1][dt]);
        }
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int t = 0; t < QT; ++t)
          o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], pb[t][ks], o[t][dt], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < QT; ++t)
        lsum[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[t][ks], lsum[t], 0, 0, 0);
    }
  }

  // epilogue
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const float l = lsum[t][0];     // every row of the sum tile holds the query's sum
    const int qq = qrow[t];
    if (qq >= p.rows_g) continue;
    const int slot = qq / p.G;
    const int h = g * p.G + qq % p.G;
    if (nsplit == 1) {
      const float inv = 1.0f / l;
      const size_t e0 = (((size_t)b * p.R + slot) * p.Hq + h) * kD;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        store_out4(p, e0 + 16 * dt + 4 * lg,
                   make_float4(o[t][dt][0] * inv, o[t][dt][1] * inv, o[t][dt][2] * inv,
                               o[t][dt][3] * inv));
    } else {
      const size_t pidx = (((size_t)b * p.HG + grp) * p.max_splits + split) * p.rb +
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
// VALU kernel: fp32 storage, or bf16 with D = 64. Up to 32 query rows per
// block; wave w takes rows w, w + 4, ... of those that hold a query, so a
// block with few rows (5 at batch 1 with 4 x 64 heads) spends one or two row
// passes per key tile, not eight. In a row pass lane k scores key k of the
// tile, then lanes own d columns. Only the K/V tile is shared between waves;
// a row's probabilities, statistics and accumulator belong to its wave, so
// the row passes need no block barrier. Dot products and the P V sums run
// four partial sums each, to break the dependent FMA chains.
// ---------------------------------------------------------------------------

template <typename TIn>
__device__ __forceinline__ float ld_val(const TIn* p) { return (float)*p; }

template <typename TIn, int D>
__global__ __launch_bounds__(256) void k_attn_valu(AttnParams p) {
  constexpr int RBV = 32;
  constexpr int DPL = D / 64;     // d columns per lane
  static_assert(D % 4 == 0 && kKeyTile % 4 == 0, "partial sums");
  __shared__ float Ks[kKeyTile][D + 1];
  __shared__ float Vs[kKeyTile][D];
  __shared__ float Qs[RBV][D];
  __shared__ float Acc[RBV][D];
  __shared__ float Ms[RBV], Ls[RBV];
  __shared__ uint64_t Anc[RBV];
  __shared__ float Ps[4][kKeyTile];

  int b, grp, split, chunk;
  if (!attn_item(p, &b, &grp, &split, &chunk)) return;
  const int g = grp / p.RG;
  const int rg = grp % p.RG;
  if (p.flags[b] & kSeqErrMask) return;
  const int base = p.kv_offset[b];
  const int total = p.kv_offset[b + 1] - base;
  const int L = total - p.N;
  const int nsplit = (total + chunk - 1) / chunk;
  if (split >= nsplit) return;
  if (split == 0 && grp == 0 && threadIdx.x == 0) p.nsplit[b] = nsplit;
  const int key_begin = split * chunk;
  const int key_end = min(total, key_begin + chunk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nrows = min(RBV, p.rows_g - rg * RBV);   // rows of this block with a query (>= 1)
  const TIn* kv = (const TIn*)p.kv;
  const TIn* qp = (const TIn*)p.q;
  const size_t row_elems = (size_t)2 * p.Hkv * D;
  const size_t hidden = (size_t)p.Hq * D;

  // every load of a staging loop is issued before the first LDS store, so the
  // loop waits for one memory latency, not one per element
  constexpr int kQPer = RBV * D / 256, kKVPer = kKeyTile * D / 256;
  static_assert(RBV * D % 256 == 0 && kKeyTile * D % 256 == 0, "staging loops");
  {
    float v[kQPer];
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
      const int i = tid + 256 * u, r = i / D, dd = i % D;
      const int qq = rg * RBV + r;
      v[u] = 0.0f;
      if (qq < p.rows_g) {
        const int slot = qq / p.G, h = g * p.G + qq % p.G;
        v[u] = ld_val(qp + ((size_t)b * p.R + slot) * hidden + (size_t)h * D + dd);
      }
    }
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
      const int i = tid + 256 * u;
      Qs[i / D][i % D] = v[u];
      Acc[i / D][i % D] = 0.0f;
    }
  }
  if (tid < RBV) {
    const int qq = rg * RBV + tid;
    Ms[tid] = -INFINITY;
    Ls[tid] = 0.0f;
    Anc[tid] = (qq < p.rows_g) ? p.anc[(size_t)b * p.R + qq / p.G] : 0;
  }

  for (int tile0 = key_begin; tile0 < key_end; tile0 += kKeyTile) {
    float kvk[kKVPer], kvv[kKVPer];
#pragma unroll
    for (int u = 0; u < kKVPer; ++u) {
      const int i = tid + 256 * u, k = i / D, dd = i % D;
      const int key = tile0 + k;
      kvk[u] = 0.0f;
      kvv[u] = 0.0f;
      if (key < key_end) {
        const TIn* row = kv + (size_t)(base + key) * row_elems;
        kvk[u] = ld_val(row + (size_t)g * D + dd);
        kvv[u] = ld_val(row + (size_t)(p.Hkv + g) * D + dd);
      }
    }
    __syncthreads();               // the previous tile's row passes are done with Ks / Vs
#pragma unroll
    for (int u = 0; u < kKVPer; ++u) {
      const int i = tid + 256 * u;
      Ks[i / D][i % D] = kvk[u];
      Vs[i / D][i % D] = kvv[u];
    }
    __syncthreads();
    // wave-uniform loop; every access below is to this wave's own row or
    // Ps[wave], which LDS orders within the wave
    for (int qr = wave; qr < nrows; qr += 4) {
      float d4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
      for (int dd = 0; dd < D; dd += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) d4[u] += Qs[qr][dd + u] * Ks[lane][dd + u];
      }
      float sc = ((d4[0] + d4[1]) + (d4[2] + d4[3])) * p.scale_log2;
      if (!key_visible(tile0 + lane, L, key_end, Anc[qr])) sc = -INFINITY;
      const float m_old = Ms[qr];
      const float m_new = fmaxf(m_old, wave_max(sc));
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = fast_exp2(m_old - m_use);
      const float e = fast_exp2(sc - m_use);
      const float esum = wave_sum(e);
      Ps[wave][lane] = e;
      if (lane == 0) {
        Ms[qr] = m_new;
        Ls[qr] = Ls[qr] * alpha + esum;
      }
#pragma unroll
      for (int j = 0; j < DPL; ++j) {
        float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
        for (int k = 0; k < kKeyTile; k += 4) {
#pragma unroll
          for (int u = 0; u < 4; ++u) a4[u] += Ps[wave][k + u] * Vs[k + u][lane + 64 * j];
        }
        Acc[qr][lane + 64 * j] = Acc[qr][lane + 64 * j] * alpha + ((a4[0] + a4[1]) + (a4[2] + a4[3]));
      }
    }
  }

  for (int ql = wave; ql < nrows; ql += 4) {
    const int qq = rg * RBV + ql;
    const int slot = qq / p.G, h = g * p.G + qq % p.G;
    if (nsplit == 1) {
      const size_t e0 = (((size_t)b * p.R + slot) * p.Hq + h) * D;
#pragma unroll
      for (int j = 0; j < DPL; ++j) {
        const float v = Acc[ql][lane + 64 * j] / Ls[ql];
        if (p.out != nullptr) p.out[e0 + lane + 64 * j] = v;
        if (p.out16 != nullptr) p.out16[e0 + lane + 64 * j] = to_bf16_bits(v);
      }
    } else {
      const size_t pidx = (((size_t)b * p.HG + grp) * p.max_splits + split) * p.rb + ql;
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
  const size_t e0 = (((size_t)b * p.R + slot) * p.Hq + h) * D + d;
  if (p.flags[b] & kSeqErrMask) {
    store_out4(p, e0, make_float4(0.f, 0.f, 0.f, 0.f));
    return;
  }
  // (every sequence without an error has a first split, which recorded the
  // split count; at most max_splits)
  const int nsplit = min(p.nsplit[b], p.max_splits);
  if (nsplit <= 1) return;        // written directly by the attention kernel
  const size_t pbase = (((size_t)b * p.HG + grp) * p.max_splits) * p.rb + qloc;
  // Splits go in batches of kMB whose loads are all issued before they are
  // used (one memory round trip per batch, not per split); the arithmetic
  // and its order are those of a plain loop over the splits.
  constexpr int kMB = 8;
  float m = -INFINITY;
  for (int s0 = 0; s0 < nsplit; s0 += kMB) {
    float mx[kMB];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
      mx[i] = (s0 + i < nsplit) ? p.part_ml[pbase + (size_t)(s0 + i) * p.rb].x : -INFINITY;
#pragma unroll
    for (int i = 0; i < kMB; ++i) m = fmaxf(m, mx[i]);
  }
  float l = 0.0f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nsplit; s0 += kMB) {
    float2 ml[kMB];
    float4 v[kMB];
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
      ml[i] = make_float2(-INFINITY, 0.0f);
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s0 + i < nsplit) {
        const size_t pi = pbase + (size_t)(s0 + i) * p.rb;
        ml[i] = p.part_ml[pi];
        v[i] = *(const float4*)(p.part_acc + pi * D + d);
      }
    }
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
      if (ml[i].x == -INFINITY) continue;     // an empty split, or past the last one
      const float w = fast_exp2(ml[i].x - m);
      l += ml[i].y * w;
      a.x += v[i].x * w;
      a.y += v[i].y * w;
      a.z += v[i].z * w;
      a.w += v[i].w * w;
    }
  }
  const float inv = 1.0f / l;
  store_out4(p, e0, make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv));
}

hipError_t launch_attention(const Plan& P, const Args& a, hipStream_t s) {
  AttnParams p;
  p.kv = a.kv;
  p.kv_offset = a.kv_offset;
  p.q = a.hidden;
  p.anc = ws_anc(P, a.ws);
  p.flags = ws_flags(P, a.ws);
  p.out = a.attn_out;
  p.out16 = a.attn_out16;
  p.part_acc = (float*)(a.ws + P.off_part_acc);
  p.part_ml = (float2*)(a.ws + P.off_part_ml);
  p.B = P.B;
  p.N = P.N;
  p.R = P.R;
  p.Hq = P.Hq;
  p.Hkv = P.Hkv;
  p.G = P.G;
  p.rows_g = P.rows_g;
  p.rb = P.attn_rb;
  p.RG = P.attn_rg;
  p.HG = P.Hkv * P.attn_rg;
  p.sched = ws_attn_sched(P, a.ws);
  p.nsplit = ws_attn_nsplit(P, a.ws);
  p.sched_stride = (int)P.sched_stride;
  p.n_cand = P.n_cand;
  p.max_splits = P.max_splits;
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)P.D);
  const dim3 grid((unsigned)((size_t)P.B * P.max_splits * p.HG));
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
