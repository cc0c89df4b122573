// LM head: logits[r, v] = sum_k x[r, k] * w[v, k] for every tree slot
// ("LLM speculative decoding: EAGLE", jingming.pro, sec. 3.1: the frozen target
// LM head maps each node's last-layer feature to a vocabulary distribution).
//
// x [M, K] and w [N, K] are both K-contiguous, which is the operand layout
// the MFMA wants for A (rows of x) and B (columns = rows of w): every lane
// loads 8 consecutive k of one row. Output fp32 [M, N].
//
// bf16: MFMA 16x16x32 with fp32 accumulation, LDS-staged tiles with the
// next K-slab's global loads in flight during the current slab's math. The
// grid runs the M blocks of one N band back to back, so a band of w is
// fetched from HBM once and reused (through L2/MALL) by all M blocks.
// fp32 (small shapes only): one wave per (8 rows, column), lanes split K.
//
// In the verification call the large-M kernel also reduces each row of its
// 256 x 256 output tile to the sampling statistics of that row and 256-token
// tile (max and sum of exp((z - max)/T), or the argmax for T = 0), while the
// accumulators are still in registers; sampling then never re-reads the
// target logits to normalise them.
#include <type_traits>

#include "sv_internal.h"

namespace sv {

template <int MT, int NT, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm_bf16(const bf16_t* __restrict__ X,
                                                            const bf16_t* __restrict__ W,
                                                            float* __restrict__ C, int M, int N,
                                                            int K) {
  constexpr int BM = 16 * MT * WM;
  constexpr int BN = 16 * NT * WN;
  constexpr int BK = 64;
  constexpr int NTH = 64 * WM * WN;
  constexpr int SA = BK * 2 + 16;                 // LDS row stride (bytes), conflict-free reads
  constexpr int CA = (BM * 8 + NTH - 1) / NTH;    // 16-byte chunks per thread, A tile
  constexpr int CB = (BN * 8 + NTH - 1) / NTH;    // 16-byte chunks per thread, B tile
  __shared__ __attribute__((aligned(16))) char As[BM * SA];
  __shared__ __attribute__((aligned(16))) char Bs[BN * SA];

  const int m0 = blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int wm = wave / WN, wn = wave % WN;

  uint4 ra[CA], rb[CB];
  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < CA; ++j) {
      const int c = tid + NTH * j;
      const int row = c >> 3, part = c & 7;
      ra[j] = make_uint4(0, 0, 0, 0);
      if (c < BM * 8 && m0 + row < M)
        ra[j] = *(const uint4*)(X + (size_t)(m0 + row) * K + k0 + part * 8);
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int c = tid + NTH * j;
      const int row = c >> 3, part = c & 7;
      rb[j] = make_uint4(0, 0, 0, 0);
      if (c < BN * 8 && n0 + row < N)
        rb[j] = *(const uint4*)(W + (size_t)(n0 + row) * K + k0 + part * 8);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int j = 0; j < CA; ++j) {
      const int c = tid + NTH * j;
      if (c < BM * 8) *(uint4*)(As + (c >> 3) * SA + (c & 7) * 16) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int c = tid + NTH * j;
      if (c < BN * 8) *(uint4*)(Bs + (c >> 3) * SA + (c & 7) * 16) = rb[j];
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + BK < K) load(k0 + BK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[MT], bfr[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        af[i] = *(const bf16x8*)(As + (wm * MT * 16 + 16 * i + lr) * SA + (32 * ks + 8 * lg) * 2);
#pragma unroll
      for (int j = 0; j < NT; ++j)
        bfr[j] = *(const bf16x8*)(Bs + (wn * NT * 16 + 16 * j + lr) * SA + (32 * ks + 8 * lg) * 2);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // lane holds C[4*lg + e][lr] of every 16x16 tile
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int n = n0 + wn * NT * 16 + 16 * j + lr;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * MT * 16 + 16 * i + 4 * lg + e;
        if (m < M) C[(size_t)m * N + n] = acc[i][j][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large M (batched rows): 256 x 256 block tile, K slab 64, 8 waves of
// 128 x 64 each (128 fp32 accumulators per lane), two waves per SIMD so one
// wave's LDS reads and barrier waits overlap the other's MFMAs.
//
// Operand slabs go global -> LDS with global_load_lds_dwordx4 (no register
// staging): one wave-instruction moves 64 lanes x 16 B = 8 rows of 128 B, lane
// l landing at row 8*q + l/8, 16-byte position l%8 of the instruction's LDS
// span. The lane chooses which global chunk it fetches, so the LDS rows are
// XOR-swizzled: logical 16-byte chunk c of row r sits at position
// c ^ ((r >> 1) & 7). The 16 lanes of a fragment read (rows r0..r0+15, one
// chunk) then touch 16 distinct 16-byte bank groups.
// LDS holds a ring of two X slabs and a ring of three W slabs (160 KB): W,
// streamed from HBM, is issued two slabs ahead, X (re-read through L2) one.
//
// Tile order: blocks are dealt to the 8 XCDs round-robin, so block i runs on
// XCD i % 8. Block i takes logical tile (i % 8) * tiles_per_xcd + i / 8, which
// gives each XCD a contiguous range of N bands with all M blocks of a band
// next to each other: a band of W is fetched once and shared through that
// XCD's L2 by the M blocks, and X (small) is re-read from L2/MALL.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr int kBig = 256;       // block tile edge (M and N)
constexpr int kBigK = 64;       // K slab
constexpr int kSlabBytes = kBig * kBigK * 2;   // one operand's 256 rows of a 64-deep slab
constexpr int kXSlabs = 2;                     // X ring (one slab ahead)
constexpr int kWSlabs = 3;                     // W ring (two slabs ahead)

__device__ __forceinline__ int big_swz(int row) { return (row >> 1) & 7; }

// Wait until this wave's global->LDS loads have landed (vmcnt(0); expcnt and
// lgkmcnt left at their maximum). The compiler does not count those loads as
// LDS writes, so the barrier that publishes a slab needs this explicit wait.
__device__ __forceinline__ void wait_lds_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// The same with up to N of this wave's newest loads still in flight (loads
// complete in issue order). vmcnt is six bits: the low four sit in bits 3:0
// of the immediate, the high two in bits 15:14.
template <int N>
__device__ __forceinline__ void wait_lds_dma_but() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// DPP lane exchanges inside a 16-lane row: xor 1, xor 2 (quad permutes),
// then the half-row and row mirrors; after the four steps every lane of the
// row holds the reduction over its 16 lanes.
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- lane 7 - i within 8
constexpr int kDppMirror = 0x140;       // lane i <- lane 15 - i within 16

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f<kDppMirror>(v));
}

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v + dpp_f<kDppMirror>(v);
}

__device__ __forceinline__ int row16_min(int v) {
  v = min(v, dpp_i<kDppXor1>(v));
  v = min(v, dpp_i<kDppXor2>(v));
  v = min(v, dpp_i<kDppHalfMirror>(v));
  return min(v, dpp_i<kDppMirror>(v));
}

template <bool STATS, bool SEG = false>
__global__ __launch_bounds__(512, 1) void k_gemm_bf16_big(const bf16_t* __restrict__ X,
                                                          const bf16_t* __restrict__ W,
                                                          float* __restrict__ C, int M, int N,
                                                          int K, int MB, int T,
                                                          int tiles_per_xcd, HeadStats hs,
                                                          GemmSegs sg) {
  // One LDS object (a second __shared__ variable would make the compiler wait
  // for every in-flight global->LDS load before each fragment read): a ring
  // of two X slabs and a ring of three W slabs, 160 KB. W streams from HBM
  // and is issued two slabs ahead; X (small, re-read through L2) one slab
  // ahead. After the K loop the same memory holds the epilogue's tables.
  __shared__ __attribute__((aligned(1024))) char lds[(kXSlabs + kWSlabs) * kSlabBytes];
  auto xslab = [&](int buf) { return lds + buf * kSlabBytes; };
  auto wslab = [&](int buf) { return lds + (kXSlabs + buf) * kSlabBytes; };
  const int bi = blockIdx.x;
  const int t = (bi & 7) * tiles_per_xcd + (bi >> 3);
  if (t >= T) return;
  // SEG: the tile's segment (weights, output, width) by its 256-column band,
  // and its K split (each split writes its own partial output)
  int m0, n0, Nn = N, kbeg = 0, Kc = K;
  const bf16_t* Wsrc = W;
  float* Cdst = C;
  if constexpr (SEG) {
    const int per_split = MB * sg.band0[sg.count];
    const int ks = t / per_split, tt = t - ks * per_split;
    const int band = tt / MB;
    int sgi = 0;
    if (sg.count > 1 && band >= sg.band0[1]) sgi = 1;
    if (sg.count > 2 && band >= sg.band0[2]) sgi = 2;
    Wsrc = sg.w[sgi];
    Cdst = sg.c[sgi] + (size_t)ks * sg.split_stride[sgi];
    Nn = sg.n[sgi];
    m0 = (tt % MB) * kBig;
    n0 = (band - sg.band0[sgi]) * kBig;
    kbeg = ks * sg.kc;
    Kc = sg.kc;
  } else {
    m0 = (t % MB) * kBig;
    n0 = (t / MB) * kBig;
  }
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;      // wave tile: rows 128*wm.., cols 64*wn..
  const int lr = lane & 15, lg = lane >> 4;
  // STATS: log2(e)/T of row m0 + tid's sequence (0 greedy, -1 no statistics),
  // one register across the K loop; the epilogue puts it in LDS
  float row_l2t = -1.0f;
  if constexpr (STATS) {
    const int m = m0 + tid;
    if (tid < kBig && m < M) {
      const int b = m / hs.R;
      if (!(hs.flags[b] & kSeqErrMask)) {
        const float Tb = hs.temperature[b];
        row_l2t = (Tb == 0.0f) ? 0.0f : kLog2e / Tb;
      }
    }
  }

  // this lane's source offsets for the 4 A and 4 B wave-instructions of a slab
  int offA[4], offB[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (j * 8 + wave) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ big_swz(row);
    const int ra = min(m0 + row, M - 1) - m0;     // rows past the edge re-read a valid row;
    const int rb = min(n0 + row, Nn - 1) - n0;    // their results are never stored
    offA[j] = ra * K + c * 8;
    offB[j] = rb * K + c * 8;
  }
  const bf16_t* Xb = X + (size_t)m0 * K + kbeg;
  const bf16_t* Wb = Wsrc + (size_t)n0 * K + kbeg;
  auto issue_x = [&](int buf, int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r0 = (j * 8 + wave) * 8;
      __builtin_amdgcn_global_load_lds((glb_void_t*)(Xb + offA[j] + k0),
                                       (lds_void_t*)(xslab(buf) + r0 * 128), 16, 0, 0);
    }
  };
  auto issue_w = [&](int buf, int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r0 = (j * 8 + wave) * 8;
      __builtin_amdgcn_global_load_lds((glb_void_t*)(Wb + offB[j] + k0),
                                       (lds_void_t*)(wslab(buf) + r0 * 128), 16, 0, 0);
    }
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The K loop, specialised on MV, the number of this wave's 16-row tiles
  // that hold rows below M (8 unless the block overhangs the last row).
  // Tiles past M skip their fragment reads and MFMAs (their accumulators
  // stay zero and are never stored); every variant issues the same slab
  // loads and meets the same barriers. A wave with no valid row only moves
  // slabs.
  auto kloop = [&](auto mv_tag) {
  constexpr int MV = decltype(mv_tag)::value;
  auto read_frags = [&](int kt, int ks, bf16x8 (&a)[8], bf16x8 (&b)[4]) {
    const char* As = xslab(kt & 1);
    const char* Bs = wslab(kt % kWSlabs);
    const int c = 4 * ks + lg;
#pragma unroll
    for (int i = 0; i < MV; ++i) {
      const int r = wm * 128 + 16 * i + lr;
      a[i] = *(const bf16x8*)(As + r * 128 + ((c ^ big_swz(r)) << 4));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 64 + 16 * j + lr;
      b[j] = *(const bf16x8*)(Bs + r * 128 + ((c ^ big_swz(r)) << 4));
    }
  };
  auto mma = [&](const bf16x8 (&a)[8], const bf16x8 (&b)[4]) {
#pragma unroll
    for (int i = 0; i < MV; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  // Software pipeline over k-steps: the next k-step's fragments are read from
  // LDS while the current k-step's MFMAs run. Slab kt's X lives in X buffer
  // kt & 1, its W in W buffer kt % 3. The one barrier per slab, between its
  // two k-steps, publishes slab kt+1 and frees both of slab kt's buffers:
  // X for slab kt+2, W for slab kt+3. Each iteration issues X before W, so
  // at the barrier vmcnt(4) waits for slab kt+1's X (issued one iteration
  // earlier) and W (two earlier) while the newest W slab stays in flight.
  const int nk = Kc / kBigK;   // >= 1
  bf16x8 ca[8], cb[4], na[8], nb[4];
  // Instruction interleaving inside each half step (scheduling groups: 0x008
  // MFMA, 0x100 LDS read, 0x010 global->LDS load): the fragment reads and the
  // slab loads are spread between the MFMAs from the start of the half step,
  // so the reads land well before the next half step needs them and the MFMA
  // pipe never waits behind a burst of address arithmetic.
  auto step = [&](int kt, auto issue_x_next, auto issue_w_next, auto read_next) {
    if constexpr (MV > 0) {
      read_frags(kt, 1, na, nb);
      mma(ca, cb);
    }
    if constexpr (MV == 8) {
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // slab kt+1 complete; slab kt+2's W (issued last iteration, after its X)
    // may stay in flight when it exists
    if (kt + 2 < nk) wait_lds_dma_but<4>();
    else wait_lds_dma();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    constexpr bool kIssueX = decltype(issue_x_next)::value;
    constexpr bool kIssueW = decltype(issue_w_next)::value;
    constexpr bool kRead = decltype(read_next)::value;
    constexpr int kIssued = (kIssueX ? 4 : 0) + (kIssueW ? 4 : 0);
    if constexpr (kIssueX) issue_x(kt & 1, (kt + 2) * kBigK);
    if constexpr (kIssueW) issue_w(kt % kWSlabs, (kt + 3) * kBigK);
    if constexpr (kRead && MV > 0) read_frags(kt + 1, 0, ca, cb);
    if constexpr (MV > 0) mma(na, nb);
    if constexpr (MV == 8 && kIssued > 0) {
#pragma unroll
      for (int i = 0; i < kIssued; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      }
    }
    if constexpr (MV == 8 && kRead) {
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      }
    }
    if constexpr (MV == 8)
      __builtin_amdgcn_sched_group_barrier(0x008, 32 - kIssued - (kRead ? 12 : 0), 1);
    __builtin_amdgcn_sched_barrier(0);
  };
  using yes = std::true_type;
  using no = std::false_type;
  // prologue: slab 0, slab 1, then slab 2's W; wait for slab 0
  issue_x(0, 0);
  issue_w(0, 0);
  if (nk > 1) {
    issue_x(1, kBigK);
    issue_w(1, kBigK);
  }
  if (nk > 2) issue_w(2, 2 * kBigK);
  if (nk > 2) wait_lds_dma_but<12>();
  else if (nk > 1) wait_lds_dma_but<8>();
  else wait_lds_dma();
  __syncthreads();
  if constexpr (MV > 0) read_frags(0, 0, ca, cb);
  int kt = 0;
  for (; kt + 3 < nk; ++kt) step(kt, yes{}, yes{}, yes{});
  if (kt + 2 < nk) step(kt++, yes{}, no{}, yes{});
  if (kt + 1 < nk) step(kt++, no{}, no{}, yes{});
  step(kt, no{}, no{}, no{});
  };
  {
    const int rows_left = M - m0 - wm * 128;    // wave-uniform
    if (rows_left > 64) kloop(std::integral_constant<int, 8>{});
    else if (rows_left > 32) kloop(std::integral_constant<int, 4>{});
    else if (rows_left > 16) kloop(std::integral_constant<int, 2>{});
    else if (rows_left > 0) kloop(std::integral_constant<int, 1>{});
    else kloop(std::integral_constant<int, 0>{});
  }

  if constexpr (!STATS) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + 16 * j + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + wm * 128 + 16 * i + 4 * lg + e;
          if (m < M && n < Nn) Cdst[(size_t)m * Nn + n] = acc[i][j][e];
        }
      }
    }
  } else {
    // Row statistics of this 256-column tile. A row's 64 columns in this
    // wave sit in 4 registers of the 16 lanes of one DPP row (lane group lg),
    // so each row reduces in-lane over j, then across its 16 lanes; the four
    // column waves (wn) then merge through LDS in column order. Every row
    // takes the same branch-free steps (max, lowest argmax column, sum of
    // exponentials) so the 32 rows of a lane interleave; a row keeps what its
    // temperature needs. Logits of greedy rows are only stored on request:
    // the argmax statistics are all that sampling reads of them.
    RowStat* part = (RowStat*)lds;             // [4 wn][256 rows]
    float* s_l2t = (float*)(lds + 4 * kBig * sizeof(RowStat));
    __syncthreads();                           // every wave is done with the slabs
    if (tid < kBig) s_l2t[tid] = row_l2t;
    __syncthreads();
    int col[4];
    bool colok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      col[j] = n0 + wn * 64 + 16 * j + lr;
      colok[j] = col[j] < N;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (m0 + wm * 128 + 16 * i >= M) break;   // this and later row tiles lie past M
      const int rb = wm * 128 + 16 * i + 4 * lg;
      const float4 l4 = *(const float4*)&s_l2t[rb];
      const float l2ts[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float l2t = l2ts[e];        // uniform over the 16 lanes of the row
        // the wave's four rows here (one per lane group) are rows 4 apart of
        // one 16-row tile, nearly always of one sequence: the sum of
        // exponentials runs only if one of them samples, the argmax only if
        // one is greedy (a greedy row's NaN marker is then the check alone,
        // as the exponentials it skips are finite)
        const bool any_sampled = __ballot(l2t > 0.0f) != 0;
        const bool any_greedy = __ballot(l2t == 0.0f) != 0;
        const int m = m0 + rb + e;
        if (m < M && (l2t > 0.0f || hs.store_all)) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (colok[j]) C[(size_t)m * N + col[j]] = acc[i][j][e];
        }
        // Columns past N hold a copy of column N - 1 (clamped W rows), so the
        // finiteness check may read them unmasked.
        float x[4];
        float chk = 0.0f;                 // NaN iff a logit of the tile is not finite
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[j] = colok[j] ? acc[i][j][e] : -INFINITY;
          chk = fmaf(acc[i][j][e], 0.0f, chk);
        }
        const float mx = row16_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        float sm = chk;
        if (any_sampled) {
          const float mref = (mx == -INFINITY) ? 0.0f : mx;
          const float sl = (l2t > 0.0f) ? l2t : 1.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) sm += __builtin_amdgcn_exp2f((x[j] - mref) * sl);
        }
        sm = row16_sum(sm);
        int ix = 0x7fffffff;
        if (any_greedy) {
#pragma unroll
          for (int j = 3; j >= 0; --j) ix = (colok[j] && x[j] == mx) ? col[j] : ix;
          ix = row16_min(ix);
        }
        RowStat r;
        r.m = (l2t > 0.0f || !isnan(sm)) ? mx : NAN;
        r.s = (l2t > 0.0f) ? sm : __int_as_float(ix);
        if (lr == 0 && l2t >= 0.0f) part[wn * kBig + rb + e] = r;
      }
    }
    __syncthreads();
    if (tid < kBig) {
      const float l2t = s_l2t[tid];
      const int m = m0 + tid;
      if (l2t >= 0.0f) {
        RowStat r;
        if (l2t > 0.0f) {
          float mx = -INFINITY;
#pragma unroll
          for (int w = 0; w < 4; ++w) mx = fmaxf(mx, part[w * kBig + tid].m);
          float sm = 0.0f;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const RowStat q = part[w * kBig + tid];
            sm += (q.m == -INFINITY) ? q.s : q.s * __builtin_amdgcn_exp2f((q.m - mx) * l2t);
          }
          r.m = mx;
          r.s = sm;
        } else {
          float v = -INFINITY;
          int ix = 0x7fffffff;
          bool bad = false;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const RowStat q = part[w * kBig + tid];
            const int qi = __float_as_int(q.s);
            if (isnan(q.m)) bad = true;
            else if (q.m > v || (q.m == v && qi < ix)) {
              v = q.m;
              ix = qi;
            }
          }
          r.m = bad ? NAN : v;
          r.s = __int_as_float(ix);
        }
        hs.tstat[(size_t)m * ((N + kBig - 1) / kBig) + n0 / kBig] = r;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Few rows (M <= 32, the batch-1 shapes): the weight stream is the whole cost
// (each of the V x K weights meets at most 32 rows), so the kernels are built
// to keep HBM busy, not the matrix cores. Every wave owns NU consecutive rows
// of W and streams them over the whole K straight into registers, D 64-deep
// chunks ahead: the register file (512 KB per CU) holds far more loads in
// flight than a slab ring in LDS could. A = W, B = X, so a lane's four results
// of a 16 x 16 tile are four consecutive vocabulary entries of one row: one
// 16-byte store.
//
// X (at most 32 x K, L2-resident) is as many bytes per wave as its W rows when
// NU = BM; read straight from L2 it doubles what every CU pulls through its
// vector memory path, which costs ~15% at 27 x 8192. k_gemm_stream_lds stages
// X in LDS one K segment at a time, shared by the block's four waves;
// k_gemm_stream reads it from L2 and serves K that is not a multiple of the
// segment.
// ---------------------------------------------------------------------------

template <int NU, int BM, int D>
__global__ __launch_bounds__(256) void k_gemm_stream(const bf16_t* __restrict__ X,
                                                     const bf16_t* __restrict__ W,
                                                     float* __restrict__ C, int M, int N, int K) {
  constexpr int NT = NU / 16;       // 16-row W tiles of the wave
  constexpr int MT = BM / 16;       // 16-row X tiles
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = (blockIdx.x * 4 + wave) * NU;
  if (n0 >= N) return;              // no barriers: a wave may leave alone
  const int nchunks = K / 64;

  // A 64-deep chunk feeds two MFMA k-steps. Lane (lr, lg) loads the 32
  // contiguous bytes k = 64 c + 16 lg .. + 15 of its row: the first 8 values
  // are its slots of the first k-step, the next 8 of the second. X and W use
  // the same assignment, so every product still pairs equal k; and the four
  // lane groups of a row read its whole 128-byte line at once.
  const bf16_t* wp[NT];
  const bf16_t* xp[MT];
#pragma unroll
  for (int t = 0; t < NT; ++t) wp[t] = W + (size_t)min(n0 + 16 * t + lr, N - 1) * K + 16 * lg;
#pragma unroll
  for (int j = 0; j < MT; ++j) xp[j] = X + (size_t)min(16 * j + lr, M - 1) * K + 16 * lg;

  bf16x8 wf[D][2][NT], xf[D][2][MT];
  auto load = [&](int c, bf16x8 (&w)[2][NT], bf16x8 (&x)[2][MT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      w[0][t] = *(const bf16x8*)(wp[t] + 64 * c);
      w[1][t] = *(const bf16x8*)(wp[t] + 64 * c + 8);
    }
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      x[0][j] = *(const bf16x8*)(xp[j] + 64 * c);
      x[1][j] = *(const bf16x8*)(xp[j] + 64 * c + 8);
    }
  };
  f32x4 acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const bf16x8 (&w)[2][NT], const bf16x8 (&x)[2][MT]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < MT; ++j)
          acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[h][t], x[h][j], acc[t][j], 0, 0, 0);
  };
  // D chunks in flight (nchunks >= D; the launcher checks): chunk c lives in
  // slot c % D. A steady-state loop in which every chunk, once its MFMAs are
  // issued, reloads its slot with the chunk D ahead; then the last D to 2D - 1
  // chunks with uniform guards.
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, wf[d], xf[d]);
  int c0 = 0;
  for (; c0 + 2 * D <= nchunks; c0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      mma(wf[d], xf[d]);
      load(c0 + D + d, wf[d], xf[d]);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) {
    mma(wf[d], xf[d]);
    if (c0 + D + d < nchunks) load(c0 + D + d, wf[d], xf[d]);
  }
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (c0 + D + d < nchunks) mma(wf[d], xf[d]);

  // lane holds C[m = 16 j + lr][n = n0 + 16 t + 4 lg + e], e = 0..3
  const bool vec_store = (N & 3) == 0;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = n0 + 16 * t + 4 * lg;
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int m = 16 * j + lr;
      if (m >= M) continue;
      float* dst = C + (size_t)m * N + n;
      if (vec_store && n + 3 < N) {
        *(float4*)dst = make_float4(acc[t][j][0], acc[t][j][1], acc[t][j][2], acc[t][j][3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < N) dst[e] = acc[t][j][e];
      }
    }
  }
}

// X in LDS. The block's WAVES waves own WAVES * NU consecutive weight rows;
// the K range is cut into segments of KS, and segment g of X (BM rows x KS,
// rows past M repeat row M - 1) lives in LDS buffer g % 2, each row padded by
// 16 bytes so that the 16 rows a fragment read touches fall in distinct banks.
// Segment g + 1 is loaded into registers at the start of segment g and written
// to its buffer at the end, behind the weight loads of the whole segment, so
// waiting for it holds nothing up; one barrier per segment publishes it and
// releases the buffer the next write overwrites. (A global -> LDS fetch would
// skip the registers, but the compiler then makes every LDS read after it
// wait for it, and with it for every weight load in flight.) The weight
// chunks keep streaming across segment boundaries. In chunk c, lane
// (lr, lg) = (lane % 16, lane / 16) loads weight k = 64 c + 8 lg .. + 7 of
// its row (first MFMA k-step) and 64 c + 32 + 8 lg .. + 7 (second), and reads
// X with the same assignment.
template <int NU, int BM, int D, int KS, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemm_stream_lds(const bf16_t* __restrict__ X,
                                                               const bf16_t* __restrict__ W,
                                                               float* __restrict__ C, int M,
                                                               int N, int K) {
  constexpr int NT = NU / 16, MT = BM / 16;
  constexpr int CPS = KS / 64;                // 64-deep chunks per segment
  constexpr int RS = KS * 2 + 16;             // padded LDS row stride, bytes
  constexpr int PPR = KS * 2 / 1024;          // 1 KB pieces per X row segment
  constexpr int PW = BM * PPR / WAVES;        // pieces per wave
  static_assert(PPR >= 1 && CPS % D == 0 && CPS >= 2 && BM * PPR % WAVES == 0,
                "segment shape");
  __shared__ __attribute__((aligned(16))) char xs[2][BM * RS];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = (blockIdx.x * WAVES + wave) * NU;   // may be >= N: the wave still
                                                     // stages X and meets the barriers
  const int nseg = K / KS;

  bf16x8 xst[PW];                             // X pieces on their way to LDS
  auto load_x = [&](int g) {
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int piece = wave + WAVES * i, r = piece / PPR, q = piece % PPR;
      xst[i] = *(const bf16x8*)(X + (size_t)min(r, M - 1) * K + (size_t)g * KS + q * 512 +
                                lane * 8);
    }
  };
  auto store_x = [&](int g) {
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int piece = wave + WAVES * i, r = piece / PPR, q = piece % PPR;
      *(bf16x8*)(xs[g & 1] + r * RS + q * 1024 + lane * 16) = xst[i];
    }
  };
  const bf16_t* wp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) wp[t] = W + (size_t)min(n0 + 16 * t + lr, N - 1) * K + 8 * lg;
  bf16x8 wf[D][2][NT];
  auto load_w = [&](int c, bf16x8 (&w)[2][NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      w[0][t] = *(const bf16x8*)(wp[t] + 64 * c);
      w[1][t] = *(const bf16x8*)(wp[t] + 64 * c + 32);
    }
  };
  bf16x8 xf[2][2][MT];                        // X fragments, one chunk ahead
  auto read_x = [&](int buf, int cc, bf16x8 (&x)[2][MT]) {
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        x[h][j] = *(const bf16x8*)(xs[buf] + (16 * j + lr) * RS + (64 * cc + 32 * h + 8 * lg) * 2);
  };
  f32x4 acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const bf16x8 (&w)[2][NT], const bf16x8 (&x)[2][MT]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < MT; ++j)
          acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[h][t], x[h][j], acc[t][j], 0, 0, 0);
  };

  // One segment. Before the last, every chunk has a chunk D ahead (D <= CPS)
  // and X of the next segment is staged; in the last, only chunks
  // cc + D < CPS load. Both conditions are compile-time: loads under a
  // run-time guard would make the compiler's waits at the loop head assume
  // the newest load may be any of them.
  auto segment = [&](int g, auto last) {
    constexpr bool kLast = decltype(last)::value;
    const int buf = g & 1;
    read_x(buf, 0, xf[0]);
#pragma unroll
    for (int cc = 0; cc < CPS; ++cc) {
      if (cc + 1 < CPS) read_x(buf, cc + 1, xf[(cc + 1) & 1]);
      mma(wf[cc % D], xf[cc & 1]);
      if (!kLast || cc + D < CPS) load_w(g * CPS + cc + D, wf[cc % D]);
      if (!kLast && cc == 0) load_x(g + 1);
      if (!kLast && cc == CPS - 1) store_x(g + 1);
      // keep each chunk's loads in issue order behind its MFMAs: clustering
      // them (the scheduler's choice in one long block) makes the MFMAs of a
      // later chunk wait for every load in flight
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  load_x(0);
  store_x(0);
#pragma unroll
  for (int d = 0; d < D; ++d) load_w(d, wf[d]);     // K / 64 >= CPS >= D
  __syncthreads();
  for (int g = 0; g + 1 < nseg; ++g) {
    segment(g, std::false_type{});
    __syncthreads();
  }
  segment(nseg - 1, std::true_type{});
  if (n0 >= N) return;

  // lane holds C[m = 16 j + lr][n = n0 + 16 t + 4 lg + e], e = 0..3
  const bool vec_store = (N & 3) == 0;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = n0 + 16 * t + 4 * lg;
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int m = 16 * j + lr;
      if (m >= M) continue;
      float* dst = C + (size_t)m * N + n;
      if (vec_store && n + 3 < N) {
        *(float4*)dst = make_float4(acc[t][j][0], acc[t][j][1], acc[t][j][2], acc[t][j][3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < N) dst[e] = acc[t][j][e];
      }
    }
  }
}

int device_cus() {
  static int cus[64] = {};     // 0 = not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = __atomic_load_n(&cus[dev], __ATOMIC_RELAXED);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    __atomic_store_n(&cus[dev], n, __ATOMIC_RELAXED);
  }
  return n;
}

template <int NU, int BM, int D>
static hipError_t gemm_stream(const void* x, const void* w, float* out, int M, int N, int K,
                              hipStream_t s) {
  const int units = (N + NU - 1) / NU;
  hipLaunchKernelGGL((k_gemm_stream<NU, BM, D>), dim3((units + 3) / 4), dim3(256), 0, s,
                     (const bf16_t*)x, (const bf16_t*)w, out, M, N, K);
  return hipGetLastError();
}

// X staged in LDS when K is a multiple of the segment: 16 weight rows per
// wave, four waves per block, 8 chunks in flight; the segment keeps the two X
// buffers at ~66 KB so that two blocks share a CU.
template <int BM>
static hipError_t gemm_stream_lds(const void* x, const void* w, float* out, int M, int N, int K,
                                  hipStream_t s) {
  constexpr int KS = BM == 16 ? 1024 : 512;
  constexpr int kWaves = 4, kNU = 16;
  const long long units = ((long long)N + kNU - 1) / kNU;
  hipLaunchKernelGGL((k_gemm_stream_lds<kNU, BM, 8, KS, kWaves>),
                     dim3((unsigned)((units + kWaves - 1) / kWaves)), dim3(64 * kWaves), 0, s,
                     (const bf16_t*)x, (const bf16_t*)w, out, M, N, K);
  return hipGetLastError();
}

// Few rows. K a multiple of the X segment: the LDS-staged kernel. Otherwise X
// comes from L2 and every wave owns one unit of NU weight rows (NU = 16 NT),
// with NT the smallest power of two that spreads the vocabulary over about 4
// waves per CU (one per SIMD; the register file then holds the loads in
// flight), and D chunks of loads so that at least D - 1 chunks, ~32 KB of W,
// are on the way at any time; larger units re-read X less often. K must be a
// multiple of 64 and at least 64 * 16.
template <int BM>
static hipError_t gemm_few_rows_bm(const void* x, const void* w, float* out, int M, int N, int K,
                                   hipStream_t s) {
  if (K % (BM == 16 ? 1024 : 512) == 0) return gemm_stream_lds<BM>(x, w, out, M, N, K, s);
  const long long tiles = ((long long)N + 15) / 16;
  const long long waves = 4LL * device_cus();
  if (tiles > 4 * waves) return gemm_stream<128, BM, 3>(x, w, out, M, N, K, s);
  if (tiles > 2 * waves) return gemm_stream<64, BM, 5>(x, w, out, M, N, K, s);
  if (tiles > waves) return gemm_stream<32, BM, 9>(x, w, out, M, N, K, s);
  return gemm_stream<16, BM, 16>(x, w, out, M, N, K, s);
}

static hipError_t gemm_few_rows(const void* x, const void* w, float* out, int M, int N, int K,
                                hipStream_t s) {
  if (M <= 16) return gemm_few_rows_bm<16>(x, w, out, M, N, K, s);
  return gemm_few_rows_bm<32>(x, w, out, M, N, K, s);
}

__global__ __launch_bounds__(64) void k_gemm_f32(const float* __restrict__ X,
                                                 const float* __restrict__ W,
                                                 float* __restrict__ C, int M, int N, int K) {
  const int n = blockIdx.x;
  const int m0 = blockIdx.y * 8;
  const int lane = threadIdx.x;
  float acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.0f;
  for (int k = lane; k < K; k += 64) {
    const float w = W[(size_t)n * K + k];
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (m0 + r < M) acc[r] += X[(size_t)(m0 + r) * K + k] * w;
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == 0 && m0 + r < M) C[(size_t)(m0 + r) * N + n] = v;
  }
}

template <int MT, int NT, int WM, int WN>
static hipError_t gemm(const void* x, const void* w, float* out, int M, int N, int K,
                       hipStream_t s) {
  constexpr int BM = 16 * MT * WM, BN = 16 * NT * WN;
  const dim3 grid((M + BM - 1) / BM, (N + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm_bf16<MT, NT, WM, WN>), grid, dim3(64 * WM * WN), 0, s,
                     (const bf16_t*)x, (const bf16_t*)w, out, M, N, K);
  return hipGetLastError();
}

hipError_t launch_lm_head(int dtype, int M, int K, int N, const void* x, const void* w,
                          float* out, const HeadStats* st, bool* stats_done, hipStream_t s) {
  *stats_done = false;
  if (dtype == SV_F32) {
    hipLaunchKernelGGL(k_gemm_f32, dim3(N, (M + 7) / 8), dim3(64), 0, s, (const float*)x,
                       (const float*)w, out, M, N, K);
    return hipGetLastError();
  }
  // up to 32 rows: every wave streams its own rows of W into registers. With
  // 33-64 rows each wave would also re-read 64 rows of X per weight chunk, and
  // the LDS-staged tiles below share X between the waves of a block instead
  // (0.207 against 0.30 ms at 61 x 4096 x 128256 on one box).
  if (M <= 32 && K % 64 == 0 && K >= 1024) return gemm_few_rows(x, w, out, M, N, K, s);
  if (M <= 16) return gemm<1, 4, 1, 4>(x, w, out, M, N, K, s);
  if (M <= 32) return gemm<2, 4, 1, 4>(x, w, out, M, N, K, s);
  if (M <= 64) return gemm<4, 4, 1, 4>(x, w, out, M, N, K, s);
  if (M < 512) return gemm<4, 8, 2, 2>(x, w, out, M, N, K, s);
  const int MB = (M + kBig - 1) / kBig, NB = (N + kBig - 1) / kBig;
  const int T = MB * NB;
  const int per_xcd = (T + 7) / 8;
  GemmSegs nosg{};
  if (st != nullptr) {
    hipLaunchKernelGGL((k_gemm_bf16_big<true, false>), dim3(per_xcd * 8), dim3(512), 0, s,
                       (const bf16_t*)x, (const bf16_t*)w, out, M, N, K, MB, T, per_xcd, *st,
                       nosg);
    *stats_done = true;
  } else {
    HeadStats none = {nullptr, nullptr, 1, nullptr, 1};
    hipLaunchKernelGGL((k_gemm_bf16_big<false, false>), dim3(per_xcd * 8), dim3(512), 0, s,
                       (const bf16_t*)x, (const bf16_t*)w, out, M, N, K, MB, T, per_xcd, none,
                       nosg);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_segments(int M, int K, const void* x, const GemmSegs& sg0, int ksplit,
                                hipStream_t s) {
  if (M < 512 || ksplit < 1 || K % (kBigK * ksplit) != 0) {
    // small or odd shapes: one plain launch per segment (no K split)
    if (ksplit != 1) return hipErrorInvalidValue;
    bool sd = false;
    for (int i = 0; i < sg0.count; ++i)
      if (launch_lm_head(SV_BF16, M, K, sg0.n[i], x, sg0.w[i], sg0.c[i], nullptr, &sd, s) !=
          hipSuccess)
        return hipErrorLaunchFailure;
    return hipSuccess;
  }
  GemmSegs sg = sg0;
  sg.band0[0] = 0;
  for (int i = 0; i < sg.count; ++i) sg.band0[i + 1] = sg.band0[i] + (sg.n[i] + kBig - 1) / kBig;
  sg.kc = K / ksplit;
  const int MB = (M + kBig - 1) / kBig;
  const int T = MB * sg.band0[sg.count] * ksplit;
  const int per_xcd = (T + 7) / 8;
  HeadStats none = {nullptr, nullptr, 1, nullptr, 1};
  hipLaunchKernelGGL((k_gemm_bf16_big<false, true>), dim3(per_xcd * 8), dim3(512), 0, s,
                     (const bf16_t*)x, (const bf16_t*)sg.w[0], sg.c[0], M, sg.n[0], K, MB, T,
                     per_xcd, none, sg);
  return hipGetLastError();
}

}  // namespace sv
