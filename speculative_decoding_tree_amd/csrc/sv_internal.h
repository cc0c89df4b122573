// Internal declarations of the HIP library behind include/specverify.h.
// gfx950 (CDNA4) only: wave64, MFMA bf16 16x16x32, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

constexpr int kMaxNodes = 64;       // ancestor sets are 64-bit masks
constexpr int kVocabChunk = 4096;   // vocabulary tokens per sampling block
constexpr int kStatTile = 256;      // vocabulary tokens per statistics tile (= LM-head GEMM tile)
constexpr int kKeyTile = 64;        // attention key tile
constexpr int kSchedCands = 32;     // attention split lengths tried per call (one prep block each)
constexpr int kSeqErrMask = 0xFF;   // seq_status bits that are errors
constexpr int kSeqErrPath = SV_SEQ_ERR_PATH;   // sv_compact_cache: invalid path or region
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// Per-(row, 256-token tile) statistics of a logits row. For sampling rows:
// the tile max m and s = sum exp((z - m)/T), s = NaN if the tile holds a
// non-finite logit. For greedy rows: the tile max logit in m (NaN if the
// tile holds a non-finite logit) and its lowest index (bit pattern) in s.
struct RowStat {
  float m;
  float s;
};

// Host-side launch plan and workspace carving, a pure function of the shape.
struct Plan {
  int B, N, R, Hq, Hkv, D, G, d, V, dtype, max_prefix, max_children, sampling;
  int top_k;        // as given (0 = off)
  float top_p;      // as given (0 or 1 = off)
  int warp;         // top-k or top-p changes a sampling row: 0 < top_k < V or 0 < top_p < 1
  int C;            // vocabulary chunks of kVocabChunk (sampling blocks)
  int CT;           // statistics tiles of kStatTile
  // attention
  int rows_g;       // R * G query rows per KV head
  bool attn_mfma;   // bf16 with D == 128: MFMA kernel, else VALU kernel
  int attn_qt;      // MFMA: 16-row query tiles per wave (1 or 4)
  int attn_rb;      // query rows per block
  int attn_rg;      // row groups per KV head
  int chunk_keys;   // shortest split the device may choose (keys); sizes the partials
  int max_splits;   // splits of the longest sequence at that length
  int n_cand;       // candidate split lengths (the device picks one per call)
  int cand_tiles[kSchedCands];  // ascending, in key tiles
  size_t sched_stride;         // int32 per candidate schedule (header + items)
  // workspace offsets (bytes)
  size_t off_anc, off_nkids, off_kids, off_flags;
  size_t off_part_acc, off_part_ml, off_sched, off_nsplit;
  size_t off_logits, off_tstat, off_slot_t, off_xtag, off_tmass, off_bar;
  size_t off_dpart, off_slot_q;   // draft statistics computed up front (per part, per slot)
  size_t off_whc, off_whm, off_wtie, off_wtidx;   // top-k / top-p selection (warp only)
  size_t off_wgl, off_wgcnt;                      // its gathered candidates
  size_t bytes_attn_end;   // end of what attention needs
  size_t total;
};

// Builds the plan; returns SV_OK or a synchronous error code. Host only.
// sampling_only carves only what sv_sample uses (no attention partials, no
// logits).
int make_plan(const sv_problem* p, Plan* plan, bool sampling_only = false);

// Raw device pointers of a call (any may be null when unused by a stage).
struct Args {
  const void* kv;
  const int32_t* kv_offset;
  const void* hidden;
  const int32_t* parent;
  const int32_t* token;
  const void* lm_head;
  const float* draft;
  const float* uniforms;
  const float* temperature;
  const float* logits_in;   // sv_sample: caller's logits
  float* attn_out;          // may be null when attn_out16 is given
  uint16_t* attn_out16;     // optional bf16 copy of the attention output
  int32_t* accept_len;
  int32_t* accept_path;
  int32_t* out_tokens;
  int32_t* seq_status;
  sv_debug dbg;
  char* ws;
};

// Stage launchers (asynchronous on `stream`; return hipSuccess or the launch error).
// clear_walk: also zero the walk's residual-exchange words (callers whose
// workspace holds the sampling buffers). cu_share: when some sequence
// samples (T > 0), the attention schedules are sized for 1 / cu_share of the
// device's CUs (attention that runs beside the sampling walk, which then
// keeps the rest)
hipError_t launch_tree_prep(const Plan& P, const Args& a, bool check_prefix, hipStream_t s,
                            bool clear_walk = true, int cu_share = 1);
hipError_t launch_attention(const Plan& P, const Args& a, hipStream_t s);
// Row statistics the LM-head GEMM can produce in its epilogue (per row and
// 256-column tile; see RowStat), for rows of the sequence of row / R.
struct HeadStats {
  const float* temperature;   // [B]
  const int32_t* flags;       // [B] sequences with an error are skipped
  int R;                      // rows per sequence
  RowStat* tstat;             // [M, ceil(V / kStatTile)]
  int store_all;              // store every logit (else only rows with T > 0)
};

// Returns hipSuccess or the launch error; *stats_done tells whether `st`
// (may be null) was filled by the GEMM epilogue. When it was, logits of rows
// with T == 0 or of sequences with an error are stored only if st->store_all.
hipError_t launch_lm_head(int dtype, int M, int d, int V, const void* x, const void* w,
                          float* out, const HeadStats* st, bool* stats_done, hipStream_t s);
hipError_t launch_sampling(const Plan& P, const Args& a, const float* logits, bool target_done,
                           hipStream_t s);
// sv_sample's pointer checks and its launch sequence on a workspace `ws` of
// at least P.total bytes (host; synchronous status codes).
int check_sample_args(const Plan& P, const int32_t* parent, const int32_t* node_token,
                      const float* logits, const float* draft_logits, const float* uniforms,
                      const float* temperature, int32_t* accept_len, int32_t* accept_path,
                      int32_t* out_tokens, int32_t* seq_status);
int sample_call(const Plan& P, const int32_t* parent, const int32_t* node_token,
                const float* logits, const float* draft_logits, const float* uniforms,
                const float* temperature, int32_t* accept_len, int32_t* accept_path,
                int32_t* out_tokens, int32_t* seq_status, const sv_debug* dbg, char* ws,
                hipStream_t s);
// Up to three column segments of one bf16 GEMM over the same rows x [M, K],
// segment i: c[i] [M, n[i]] = x w[i]^T with w[i] [n[i], K]; with a K split of
// ksplit, split j writes the partial sum over its K range to
// c[i] + j * split_stride[i]. The Q/K/V projection of the layer share runs as
// one launch; its O projection splits K. Small M runs one plain launch per
// segment (ksplit must then be 1). band0 and kc are filled by the launcher.
struct GemmSegs {
  const bf16_t* w[3];
  float* c[3];
  int n[3];
  int band0[4];
  int count;
  int kc;
  size_t split_stride[3];
};
hipError_t launch_gemm_segments(int M, int K, const void* x, const GemmSegs& sg, int ksplit,
                                hipStream_t s);
hipError_t launch_compact_cache(void* cache, long long layer_stride, int n_layers, int row_bytes,
                                int B, int N, const int32_t* kv_offset,
                                const int32_t* prefix_len, const int32_t* accept_len,
                                const int32_t* accept_path, int32_t* new_prefix_len,
                                int32_t* status, bool vec16, hipStream_t s);
hipError_t launch_tree_init(int B, int K, int32_t* frontier, int32_t* frontier_count,
                            int32_t* pool_count, int32_t* status, hipStream_t s);
size_t tree_workspace_bytes(int B, int K, int V);
constexpr int kTreeMaxVocab = 1 << 20;   // 64 segments of 16384 tokens (one merge lane each)
hipError_t launch_tree_expand(int B, int V, int K, int C, int P, const float* logits,
                              int32_t* frontier, int32_t* frontier_count, int32_t* token,
                              int32_t* parent, float* value, int32_t* depth, int32_t* count,
                              int32_t* status, void* ws, hipStream_t s);
hipError_t launch_tree_finalize(int B, int P, int m, const int32_t* token, const int32_t* parent,
                                const float* value, const int32_t* depth, const int32_t* count,
                                int32_t* out_parent, int32_t* out_token, int32_t* out_pool_id,
                                int32_t* n_kept, hipStream_t s);
size_t layer_workspace_bytes(const Plan& P);
hipError_t launch_layer_share(const Plan& P, const Args& a, const void* wq, const void* wk,
                              const void* wv, const void* wo, double theta, void* kv,
                              void* out_hidden, float* attn_out, hipStream_t s);

// Workspace views.
inline uint64_t* ws_anc(const Plan& P, char* ws) { return (uint64_t*)(ws + P.off_anc); }
inline int32_t* ws_nkids(const Plan& P, char* ws) { return (int32_t*)(ws + P.off_nkids); }
inline int32_t* ws_kids(const Plan& P, char* ws) { return (int32_t*)(ws + P.off_kids); }
inline int32_t* ws_flags(const Plan& P, char* ws) { return (int32_t*)(ws + P.off_flags); }
inline RowStat* ws_tstat(const Plan& P, char* ws) { return (RowStat*)(ws + P.off_tstat); }
inline int32_t* ws_bar(const Plan& P, char* ws) { return (int32_t*)(ws + P.off_bar); }
inline unsigned long long* ws_xtag(const Plan& P, char* ws) {
  return (unsigned long long*)(ws + P.off_xtag);
}
// Attention schedules, one per candidate split length, sched_stride int32
// apart: header {item count, split keys, estimated makespan (int64, low word
// first)}, then item i at [4 + i] = b * max_splits + split, longest first.
inline int32_t* ws_attn_sched(const Plan& P, char* ws) { return (int32_t*)(ws + P.off_sched); }
inline int32_t* ws_attn_nsplit(const Plan& P, char* ws) { return (int32_t*)(ws + P.off_nsplit); }
constexpr int kMaxChunkTiles = 1024;  // longest attention split, in key tiles
constexpr int kSchedMachines = 1024;  // bound on the machines of the makespan estimate
// Compute units of the current device (cached per device).
int device_cus();
// workgroups per sampling sequence in the walk (upper bound; sizes the workspace)
constexpr int kWalkGroupsMax = 16;        // with top-k / top-p (its tables are unrolled over it)
constexpr int kWalkGroupsPlainMax = 64;   // without (one lane per workgroup partial)
constexpr int kWalkXWords = 2;            // tagged words per workgroup slot of a walk exchange
constexpr int kPlainWalkShare = 2;        // plain walk launch when the grid is <= 1/2 of the GPU
constexpr int kSideAttnShare = 4;         // attention beside sampling: schedules for 1/4 of the CUs
// parts of a draft row whose statistics are reduced up front (upper bound)
constexpr int kDraftPartsMax = 64;
// draft statistics are computed up front when all draft rows together take at
// most this many bytes (else lazily, at the slots the walk visits)
constexpr size_t kDraftUpFrontBytes = size_t(256) << 20;

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// fp32 -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Minimum over the 64 lanes of a wave, in every lane, without LDS: DPP
// within rows of 16 lanes (quad swaps, then the half-row and row mirrors),
// then the permlane swaps across rows. Every lane of the wave must be active.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half mirror
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = min(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return min(r[0], r[1]);
}

// Clamp a uniform into [0, 1 - 2^-24]; NaN -> 0. Sets *warn when it changed.
__device__ __forceinline__ float clamp_uniform(float u, bool* warn) {
  const float hi = 0.99999994f;  // 1 - 2^-24
  if (!(u >= 0.0f)) { *warn = true; return 0.0f; }
  if (u > hi) { *warn = true; return hi; }
  return u;
}

}  // namespace sv
