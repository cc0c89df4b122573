// The C ABI of include/specverify.h: argument checks (pure host code, run
// before any HIP call), the launch plan and workspace carving, and the
// stream-ordered launch sequence of the verification step.
#include <limits.h>
#include <math.h>
#include <string.h>

#include <cmath>

#include "sv_internal.h"

namespace sv {

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static int check_problem(const sv_problem* p) {
  if (p == nullptr) return SV_ERR_NULL;
  if (p->dtype != SV_BF16 && p->dtype != SV_F32) return SV_ERR_DTYPE;
  if (p->batch < 1 || p->n_nodes < 0 || p->n_nodes > kMaxNodes) return SV_ERR_SHAPE;
  if (p->n_q_heads < 1 || p->n_kv_heads < 1 || p->n_q_heads % p->n_kv_heads != 0)
    return SV_ERR_SHAPE;
  if (p->head_dim != 64 && p->head_dim != 128) return SV_ERR_SHAPE;
  if ((long long)p->n_q_heads * p->head_dim != p->hidden) return SV_ERR_SHAPE;
  if (p->vocab < 1 || p->vocab > (1 << 30)) return SV_ERR_SHAPE;
  if (p->max_prefix < 1 || p->max_prefix > (1 << 28)) return SV_ERR_SHAPE;
  if (p->max_children < 1 || p->max_children > kMaxNodes) return SV_ERR_SHAPE;
  if (p->sampling != SV_SAMPLE_IID && p->sampling != SV_SAMPLE_DISTINCT) return SV_ERR_SHAPE;
  if (p->top_k < 0 || !(p->top_p >= 0.0f && p->top_p <= 1.0f)) return SV_ERR_SHAPE;
  // grid limits: rows of the sampling grids and the batch dimension
  if ((long long)p->batch * (p->n_nodes + 1) > 65535) return SV_ERR_SHAPE;
  return SV_OK;
}

int make_plan(const sv_problem* pr, Plan* P, bool sampling_only) {
  const int rc = check_problem(pr);
  if (rc != SV_OK) return rc;
  Plan& q = *P;
  q.B = pr->batch;
  q.N = pr->n_nodes;
  q.R = q.N + 1;
  q.Hq = pr->n_q_heads;
  q.Hkv = pr->n_kv_heads;
  q.D = pr->head_dim;
  q.G = q.Hq / q.Hkv;
  q.d = pr->hidden;
  q.V = pr->vocab;
  q.dtype = pr->dtype;
  q.max_prefix = pr->max_prefix;
  q.max_children = pr->max_children;
  q.sampling = pr->sampling;
  q.top_k = pr->top_k;
  q.top_p = pr->top_p;
  q.warp = ((q.top_k > 0 && q.top_k < pr->vocab) || (q.top_p > 0.0f && q.top_p < 1.0f)) ? 1 : 0;
  q.C = (q.V + kVocabChunk - 1) / kVocabChunk;
  q.CT = (q.V + kStatTile - 1) / kStatTile;

  q.rows_g = q.R * q.G;
  q.attn_mfma = (q.dtype == SV_BF16 && q.D == 128);
  if (q.attn_mfma) {
    q.attn_qt = q.rows_g <= 128 ? 1 : 2;
    q.attn_rb = 128 * q.attn_qt;
  } else {
    q.attn_qt = 0;
    q.attn_rb = 32;
  }
  q.attn_rg = (q.rows_g + q.attn_rb - 1) / q.attn_rb;
  const long long max_keys = (long long)q.max_prefix + q.N;
  const long long tiles_max = (max_keys + kKeyTile - 1) / kKeyTile;
  const long long total_tiles = (long long)q.B * q.Hkv * q.attn_rg * tiles_max;
  // Split lengths: the device chooses per call, from the actual prefix
  // lengths, among kSchedCands lengths spaced geometrically from the shortest
  // (about 6 splits per CU for the longest prefix bound, at least 2 tiles; it
  // sizes the split partials) to the longest sequence's whole key range.
  long long lo = (total_tiles + 1535) / 1536;
  if (lo < 2) lo = 2;
  const long long hi = tiles_max < kMaxChunkTiles ? tiles_max : kMaxChunkTiles;
  if (lo > hi) lo = hi;
  q.chunk_keys = (int)(lo * kKeyTile);
  q.max_splits = (int)((max_keys + q.chunk_keys - 1) / q.chunk_keys);
  q.n_cand = kSchedCands;
  for (int j = 0; j < kSchedCands; ++j) {
    const double f = (double)j / (kSchedCands - 1);
    long long c = (long long)llround((double)lo * pow((double)hi / (double)lo, f));
    if (c < lo) c = lo;
    if (c > hi) c = hi;
    q.cand_tiles[j] = (int)c;
  }
  if (q.max_splits > 65535 || (long long)q.Hkv * q.attn_rg > 65535) return SV_ERR_SHAPE;
  // the attention grid is one-dimensional: (sequence, split) items x head groups
  if ((long long)q.B * q.max_splits * q.Hkv * q.attn_rg > 0x7fffffffLL) return SV_ERR_SHAPE;

  const size_t BR = (size_t)q.B * q.R;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  q.off_anc = take(sizeof(uint64_t) * BR);
  q.off_nkids = take(sizeof(int32_t) * BR);
  q.off_kids = take(sizeof(int32_t) * BR * q.max_children);
  q.off_flags = take(sizeof(int32_t) * q.B);
  // a sampling-only plan (sv_sample on the static scratch) leaves out the
  // attention partials and the logits, which that call never touches
  const size_t nparts =
      sampling_only ? 0 : (size_t)q.B * q.Hkv * q.attn_rg * q.max_splits * q.attn_rb;
  q.off_part_acc = take(sizeof(float) * nparts * q.D);
  q.off_part_ml = take(sizeof(float) * 2 * nparts);
  q.sched_stride = sampling_only ? 0 : align_up(4 + (size_t)q.B * q.max_splits, 4);
  q.off_sched = take(sizeof(int32_t) * q.n_cand * q.sched_stride);
  q.off_nsplit = take(sampling_only ? 0 : sizeof(int32_t) * q.B);
  q.bytes_attn_end = off;
  q.off_logits = take(sampling_only ? 0 : sizeof(float) * BR * q.V);
  q.off_tstat = take(sizeof(RowStat) * BR * q.CT);
  q.off_slot_t = take(sizeof(RowStat) * BR);
  q.off_dpart = take(sizeof(RowStat) * BR * kDraftPartsMax);
  q.off_slot_q = take(sizeof(RowStat) * BR);
  // walk partials, double-buffered by barrier phase
  q.off_xtag = take(sizeof(uint64_t) * q.B * 2 * kWalkGroupsPlainMax * kWalkXWords);
  q.off_tmass = take(sizeof(float) * q.B * 2 * q.CT);
  // top-k / top-p selection: per sequence, phase, workgroup and row (target,
  // draft) histograms of 256 bins, tie-group counts and cut ids
  const size_t wsel = q.warp ? (size_t)q.B * 2 * kWalkGroupsMax * 2 : 0;
  q.off_whc = take(sizeof(uint32_t) * wsel * 256);
  q.off_whm = take(sizeof(uint64_t) * wsel * 256);
  q.off_wtie = take(sizeof(int32_t) * wsel);
  q.off_wtidx = take(sizeof(int32_t) * (q.warp ? (size_t)q.B * 4 : 0));
  // gathered candidates: per sequence, phase, workgroup and row, 256 entries of (key, mass)
  q.off_wgl = take(sizeof(uint64_t) * wsel * 256 * 2);
  q.off_wgcnt = take(sizeof(uint64_t) * wsel * 3);
  q.off_bar = take(sizeof(int32_t) * q.B);
  q.total = off;
  return SV_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static int check_workspace(const Plan& P, void* ws, size_t bytes) {
  if (ws == nullptr) return SV_ERR_WORKSPACE;
  if (bytes < P.total) return SV_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255u) != 0) return SV_ERR_ALIGN;
  return SV_OK;
}

int check_sample_args(const Plan& P, const int32_t* parent, const int32_t* node_token,
                      const float* logits, const float* draft_logits, const float* uniforms,
                      const float* temperature, int32_t* accept_len, int32_t* accept_path,
                      int32_t* out_tokens, int32_t* seq_status) {
  if (!logits || !draft_logits || !uniforms || !temperature || !accept_len || !out_tokens ||
      !seq_status)
    return SV_ERR_NULL;
  if (P.N > 0 && (!parent || !node_token || !accept_path)) return SV_ERR_NULL;
  return SV_OK;
}

int sample_call(const Plan& P, const int32_t* parent, const int32_t* node_token,
                const float* logits, const float* draft_logits, const float* uniforms,
                const float* temperature, int32_t* accept_len, int32_t* accept_path,
                int32_t* out_tokens, int32_t* seq_status, const sv_debug* dbg, char* ws,
                hipStream_t s) {
  Args a;
  memset(&a, 0, sizeof(a));
  a.parent = parent;
  a.token = node_token;
  a.draft = draft_logits;
  a.uniforms = uniforms;
  a.temperature = temperature;
  a.accept_len = accept_len;
  a.accept_path = accept_path;
  a.out_tokens = out_tokens;
  a.seq_status = seq_status;
  if (dbg) a.dbg = *dbg;
  a.ws = ws;
  (void)hipGetLastError();
  if (launch_tree_prep(P, a, false, s) != hipSuccess) return SV_ERR_HIP;
  if (launch_sampling(P, a, logits, false, s) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

}  // namespace sv

using namespace sv;

extern "C" {

int sv_version(void) { return 200; }

const char* sv_status_string(int s) {
  switch (s) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE: return "unsupported or inconsistent problem shape";
    case SV_ERR_DTYPE: return "dtype must be SV_BF16 or SV_F32";
    case SV_ERR_WORKSPACE: return "workspace missing or smaller than sv_workspace_size()";
    case SV_ERR_HIP: return "HIP launch or device query failed";
    case SV_ERR_ALIGN: return "pointer misaligned (16 bytes; workspace 256 bytes)";
    case SV_ERR_SCRATCH:
      return "problem needs more than the static scratch of sv_sample_noalloc "
             "(SV_NOALLOC_SCRATCH_BYTES); use sv_sample with a workspace";
    default: return "unknown status";
  }
}

const char* sv_seq_status_string(int bit) {
  switch (bit) {
    case 0: return "ok";
    case SV_SEQ_ERR_TREE: return "sequence: invalid parent array or too many children";
    case SV_SEQ_ERR_TOKEN: return "sequence: drafted token outside [0, vocab)";
    case SV_SEQ_ERR_TEMPERATURE: return "sequence: temperature negative or not finite";
    case SV_SEQ_ERR_PREFIX: return "sequence: prefix length outside [1, max_prefix]";
    case SV_SEQ_ERR_NONFINITE: return "sequence: non-finite logits on the walked slots";
    case SV_SEQ_ERR_INTERNAL: return "sequence: a wait between the workgroups of the walk gave up";
    case SV_SEQ_ERR_PATH: return "sequence: accept path or cache region not valid for compaction";
    case SV_SEQ_ERR_POOL: return "sequence: draft-tree pool capacity exceeded";
    case SV_SEQ_WARN_UNIFORM: return "sequence: a uniform outside [0, 1) was clamped";
    case SV_SEQ_WARN_RESIDUAL: return "sequence: a residual mass was not positive; kept the previous distribution";
    case SV_SEQ_WARN_CDF_CLAMP: return "sequence: inverse-CDF draw clamped to the last positive token";
    default: return "unknown status";
  }
}

int sv_workspace_size(const sv_problem* prob, size_t* bytes) {
  if (bytes == nullptr) return SV_ERR_NULL;
  Plan P;
  const int rc = make_plan(prob, &P);
  if (rc != SV_OK) return rc;
  *bytes = P.total;
  return SV_OK;
}

// A second stream for the attention stage. Attention and sampling both read
// only the tree preparation's outputs and write disjoint memory, and the walk
// is latency-bound (at most a few hundred resident workgroups, mostly waiting
// at sequence barriers), so attention can run beside sampling after the LM
// head: the caller's stream forks to this stream and joins it again before
// the call's last work in stream order. One stream and one pair of events
// per host thread and device, created on first use and never destroyed (a
// HIP call from a thread-exit or process-exit handler could run after the
// runtime is gone); a later call re-records the events, which leaves earlier
// waits on them as they were. Null when the runtime cannot create them: then
// every stage runs on the caller's stream.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxSideDevices = 64;

static SideStream* side_stream() {
  static thread_local SideStream side[kMaxSideDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return nullptr;
  SideStream& x = side[dev];
  if (x.s != nullptr) return &x;
  const unsigned ev_flags = hipEventDisableTiming | hipEventDisableSystemFence;
  hipStream_t st = nullptr;
  hipEvent_t f = nullptr, j = nullptr;
  if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
  if (hipEventCreateWithFlags(&f, ev_flags) != hipSuccess ||
      hipEventCreateWithFlags(&j, ev_flags) != hipSuccess) {
    if (f != nullptr) (void)hipEventDestroy(f);
    (void)hipStreamDestroy(st);
    return nullptr;
  }
  x.s = st;
  x.fork = f;
  x.join = j;
  return &x;
}

int sv_verify_tree(const sv_problem* prob, const void* kv, const int32_t* kv_offset,
                   const void* node_hidden, const int32_t* parent, const int32_t* node_token,
                   const void* lm_head, const float* draft_logits, const float* uniforms,
                   const float* temperature, float* attn_out, int32_t* accept_len,
                   int32_t* accept_path, int32_t* out_tokens, int32_t* seq_status,
                   const sv_debug* dbg, void* workspace, size_t workspace_bytes,
                   sv_stream_t stream) {
  Plan P;
  int rc = make_plan(prob, &P);
  if (rc != SV_OK) return rc;
  if (!kv || !kv_offset || !node_hidden || !lm_head || !draft_logits || !uniforms ||
      !temperature || !attn_out || !accept_len || !out_tokens || !seq_status)
    return SV_ERR_NULL;
  if (P.N > 0 && (!parent || !node_token || !accept_path)) return SV_ERR_NULL;
  if (!aligned16(kv) || !aligned16(node_hidden) || !aligned16(lm_head) ||
      !aligned16(draft_logits) || !aligned16(attn_out))
    return SV_ERR_ALIGN;
  if (dbg && dbg->logits && !aligned16(dbg->logits)) return SV_ERR_ALIGN;
  rc = check_workspace(P, workspace, workspace_bytes);
  if (rc != SV_OK) return rc;

  Args a;
  memset(&a, 0, sizeof(a));
  a.kv = kv;
  a.kv_offset = kv_offset;
  a.hidden = node_hidden;
  a.parent = parent;
  a.token = node_token;
  a.lm_head = lm_head;
  a.draft = draft_logits;
  a.uniforms = uniforms;
  a.temperature = temperature;
  a.attn_out = attn_out;
  a.accept_len = accept_len;
  a.accept_path = accept_path;
  a.out_tokens = out_tokens;
  a.seq_status = seq_status;
  if (dbg) a.dbg = *dbg;
  a.ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  float* logits = (dbg && dbg->logits) ? dbg->logits : (float*)(a.ws + P.off_logits);
  sv_event_t* ev = dbg ? dbg->stage_events : nullptr;
  auto mark_on = [&](int i, hipStream_t st) {
    return ev == nullptr || ev[i] == nullptr || hipEventRecord((hipEvent_t)ev[i], st) == hipSuccess;
  };
  auto mark = [&](int i) { return mark_on(i, s); };
  // Below 512 rows (the few-sequence shapes) attention is small and the
  // sampling stage is mostly launch and barrier latency: attention goes to
  // the side stream after the LM head and runs beside sampling (5-7% off the
  // step at batch 1). When some sequence samples, its schedule is then sized
  // for a quarter of the CUs: sampling's kernels keep the rest instead of
  // sharing SIMDs with attention blocks, and attention still ends within the
  // walk. A greedy walk is too short for that and keeps the full schedule.
  // With many rows both stages are large, contend for HBM and CUs, and the
  // overlap measured no gain; attention then runs first on the caller's
  // stream.
  SideStream* side = P.B * P.R < 512 ? side_stream() : nullptr;
  if (!mark(2 * SV_STAGE_PREP) ||
      launch_tree_prep(P, a, true, s, true, side != nullptr ? kSideAttnShare : 1) != hipSuccess ||
      !mark(2 * SV_STAGE_PREP + 1))
    return SV_ERR_HIP;
  auto attention_on = [&](hipStream_t st) {
    return mark_on(2 * SV_STAGE_ATTENTION, st) && launch_attention(P, a, st) == hipSuccess &&
           mark_on(2 * SV_STAGE_ATTENTION + 1, st);
  };
  if (side == nullptr && !attention_on(s)) return SV_ERR_HIP;
  HeadStats hs;
  hs.temperature = temperature;
  hs.flags = ws_flags(P, a.ws);
  hs.R = P.R;
  hs.tstat = ws_tstat(P, a.ws);
  hs.store_all = (dbg && dbg->logits) ? 1 : 0;
  bool stats_done = false;
  if (!mark(2 * SV_STAGE_LM_HEAD) ||
      launch_lm_head(P.dtype, P.B * P.R, P.d, P.V, node_hidden, lm_head, logits, &hs,
                     &stats_done, s) != hipSuccess ||
      !mark(2 * SV_STAGE_LM_HEAD + 1))
    return SV_ERR_HIP;
  if (side != nullptr) {
    if (hipEventRecord(side->fork, s) != hipSuccess ||
        hipStreamWaitEvent(side->s, side->fork, 0) != hipSuccess || !attention_on(side->s) ||
        hipEventRecord(side->join, side->s) != hipSuccess)
      return SV_ERR_HIP;
  }
  const bool sampled =
      mark(2 * SV_STAGE_SAMPLING) && launch_sampling(P, a, logits, stats_done, s) == hipSuccess &&
      mark(2 * SV_STAGE_SAMPLING + 1);
  // join even when sampling failed to launch, so the caller's stream never
  // runs ahead of work still queued on the side stream
  if (side != nullptr && hipStreamWaitEvent(s, side->join, 0) != hipSuccess) return SV_ERR_HIP;
  return sampled ? SV_OK : SV_ERR_HIP;
}

int sv_tree_attention(const sv_problem* prob, const void* kv, const int32_t* kv_offset,
                      const void* node_hidden, const int32_t* parent, float* attn_out,
                      int32_t* seq_status, void* workspace, size_t workspace_bytes,
                      sv_stream_t stream) {
  Plan P;
  int rc = make_plan(prob, &P);
  if (rc != SV_OK) return rc;
  if (!kv || !kv_offset || !node_hidden || !attn_out || !seq_status) return SV_ERR_NULL;
  if (P.N > 0 && !parent) return SV_ERR_NULL;
  if (!aligned16(kv) || !aligned16(node_hidden) || !aligned16(attn_out)) return SV_ERR_ALIGN;
  rc = check_workspace(P, workspace, workspace_bytes);
  if (rc != SV_OK) return rc;
  Args a;
  memset(&a, 0, sizeof(a));
  a.kv = kv;
  a.kv_offset = kv_offset;
  a.hidden = node_hidden;
  a.parent = parent;
  a.attn_out = attn_out;
  a.seq_status = seq_status;
  a.ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (launch_tree_prep(P, a, true, s) != hipSuccess) return SV_ERR_HIP;
  if (launch_attention(P, a, s) != hipSuccess) return SV_ERR_HIP;
  if (hipMemcpyAsync(seq_status, ws_flags(P, a.ws), sizeof(int32_t) * P.B,
                     hipMemcpyDeviceToDevice, s) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

int sv_lm_head(const sv_problem* prob, int32_t rows, const void* hidden, const void* lm_head,
               float* logits, sv_stream_t stream) {
  if (prob == nullptr) return SV_ERR_NULL;
  if (prob->dtype != SV_BF16 && prob->dtype != SV_F32) return SV_ERR_DTYPE;
  if (rows < 1 || rows > 65535 * 256 || prob->hidden < 1 || prob->vocab < 1) return SV_ERR_SHAPE;
  if (prob->dtype == SV_BF16 && prob->hidden % 64 != 0) return SV_ERR_SHAPE;
  if (prob->dtype == SV_F32 && (long long)(rows + 7) / 8 > 65535) return SV_ERR_SHAPE;
  if (!hidden || !lm_head || !logits) return SV_ERR_NULL;
  if (!aligned16(hidden) || !aligned16(lm_head)) return SV_ERR_ALIGN;
  (void)hipGetLastError();
  bool stats_done = false;
  if (launch_lm_head(prob->dtype, rows, prob->hidden, prob->vocab, hidden, lm_head, logits,
                     nullptr, &stats_done, (hipStream_t)stream) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

int sv_sample(const sv_problem* prob, const int32_t* parent, const int32_t* node_token,
              const float* logits, const float* draft_logits, const float* uniforms,
              const float* temperature, int32_t* accept_len, int32_t* accept_path,
              int32_t* out_tokens, int32_t* seq_status, const sv_debug* dbg, void* workspace,
              size_t workspace_bytes, sv_stream_t stream) {
  Plan P;
  int rc = make_plan(prob, &P);
  if (rc != SV_OK) return rc;
  rc = check_sample_args(P, parent, node_token, logits, draft_logits, uniforms, temperature,
                         accept_len, accept_path, out_tokens, seq_status);
  if (rc != SV_OK) return rc;
  rc = check_workspace(P, workspace, workspace_bytes);
  if (rc != SV_OK) return rc;
  return sample_call(P, parent, node_token, logits, draft_logits, uniforms, temperature,
                     accept_len, accept_path, out_tokens, seq_status, dbg, (char*)workspace,
                     (hipStream_t)stream);
}

int sv_compact_cache(void* cache, int64_t layer_stride, int32_t n_layers, int32_t row_bytes,
                     int32_t batch, int32_t n_nodes, const int32_t* kv_offset,
                     const int32_t* prefix_len, const int32_t* accept_len,
                     const int32_t* accept_path, int32_t* new_prefix_len, int32_t* status,
                     sv_stream_t stream) {
  if (batch < 0 || batch > 65535 || n_nodes < 0 || n_nodes > 64 || n_layers < 1 ||
      n_layers > 65535 || row_bytes < 4 || row_bytes % 4 != 0 || layer_stride < 0)
    return SV_ERR_SHAPE;
  if (batch == 0) return SV_OK;
  if (!cache || !kv_offset || !prefix_len || !accept_len || !new_prefix_len) return SV_ERR_NULL;
  if (n_nodes > 0 && !accept_path) return SV_ERR_NULL;
  if (((uintptr_t)cache & 3u) != 0 || layer_stride % 4 != 0) return SV_ERR_ALIGN;
  const bool vec16 = aligned16(cache) && layer_stride % 16 == 0 && row_bytes % 16 == 0;
  (void)hipGetLastError();
  if (launch_compact_cache(cache, layer_stride, n_layers, row_bytes, batch, n_nodes, kv_offset,
                           prefix_len, accept_len, accept_path, new_prefix_len, status, vec16,
                           (hipStream_t)stream) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

int sv_tree_init(int32_t batch, int32_t n_expand, int32_t* frontier, int32_t* frontier_count,
                 int32_t* pool_count, int32_t* seq_status, sv_stream_t stream) {
  if (batch < 1 || batch > 65535 || n_expand < 1 || n_expand > 16) return SV_ERR_SHAPE;
  if (!frontier || !frontier_count || !pool_count || !seq_status) return SV_ERR_NULL;
  (void)hipGetLastError();
  if (launch_tree_init(batch, n_expand, frontier, frontier_count, pool_count, seq_status,
                       (hipStream_t)stream) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

int sv_tree_workspace_size(int32_t batch, int32_t n_expand, int32_t vocab, size_t* bytes) {
  if (!bytes) return SV_ERR_NULL;
  if (batch < 1 || batch > 65535 || n_expand < 1 || n_expand > 16 || vocab < 1 ||
      vocab > kTreeMaxVocab)
    return SV_ERR_SHAPE;
  *bytes = tree_workspace_bytes(batch, n_expand, vocab);
  return SV_OK;
}

int sv_tree_expand(int32_t batch, int32_t vocab, int32_t n_expand, int32_t n_children,
                   int32_t pool_capacity, const float* draft_logits, int32_t* frontier,
                   int32_t* frontier_count, int32_t* pool_token, int32_t* pool_parent,
                   float* pool_value, int32_t* pool_depth, int32_t* pool_count,
                   int32_t* seq_status, void* workspace, size_t workspace_bytes,
                   sv_stream_t stream) {
  if (batch < 1 || batch > 65535 || n_expand < 1 || n_expand > 16 || n_children < 1 ||
      n_children > 16 || n_expand * n_children > 256 || vocab < n_children ||
      vocab > kTreeMaxVocab || pool_capacity < 1 || pool_capacity > 1024)
    return SV_ERR_SHAPE;
  if (!draft_logits || !frontier || !frontier_count || !pool_token || !pool_parent ||
      !pool_value || !pool_depth || !pool_count || !seq_status)
    return SV_ERR_NULL;
  if (((uintptr_t)draft_logits & 3u) != 0) return SV_ERR_ALIGN;
  if (!workspace || workspace_bytes < tree_workspace_bytes(batch, n_expand, vocab))
    return SV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SV_ERR_ALIGN;
  (void)hipGetLastError();
  if (launch_tree_expand(batch, vocab, n_expand, n_children, pool_capacity, draft_logits,
                         frontier, frontier_count, pool_token, pool_parent, pool_value,
                         pool_depth, pool_count, seq_status, workspace,
                         (hipStream_t)stream) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

int sv_tree_finalize(int32_t batch, int32_t pool_capacity, int32_t m, const int32_t* pool_token,
                     const int32_t* pool_parent, const float* pool_value,
                     const int32_t* pool_depth, const int32_t* pool_count, int32_t* parent,
                     int32_t* node_token, int32_t* node_pool_id, int32_t* n_kept,
                     sv_stream_t stream) {
  if (batch < 1 || batch > 65535 || pool_capacity < 1 || pool_capacity > 1024 || m < 1 ||
      m > 64)
    return SV_ERR_SHAPE;
  if (!pool_token || !pool_parent || !pool_value || !pool_depth || !pool_count || !parent ||
      !node_token || !node_pool_id || !n_kept)
    return SV_ERR_NULL;
  (void)hipGetLastError();
  if (launch_tree_finalize(batch, pool_capacity, m, pool_token, pool_parent, pool_value,
                           pool_depth, pool_count, parent, node_token, node_pool_id, n_kept,
                           (hipStream_t)stream) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

int sv_layer_workspace_size(const sv_problem* prob, size_t* bytes) {
  if (!bytes) return SV_ERR_NULL;
  Plan P;
  const int rc = make_plan(prob, &P);
  if (rc != SV_OK) return rc;
  *bytes = layer_workspace_bytes(P);
  return SV_OK;
}

int sv_layer_share(const sv_problem* prob, const void* hidden, const void* wq, const void* wk,
                   const void* wv, const void* wo, float rope_theta, void* kv,
                   const int32_t* kv_offset, const int32_t* parent, void* out_hidden,
                   float* attn_out, int32_t* seq_status, void* workspace,
                   size_t workspace_bytes, sv_stream_t stream) {
  Plan P;
  int rc = make_plan(prob, &P);
  if (rc != SV_OK) return rc;
  if (P.dtype != SV_BF16) return SV_ERR_DTYPE;
  if (P.D != 128 || !(rope_theta > 0.0f) || !std::isfinite(rope_theta)) return SV_ERR_SHAPE;
  if (!hidden || !wq || !wk || !wv || !wo || !kv || !kv_offset || !out_hidden || !seq_status)
    return SV_ERR_NULL;
  if (P.N > 0 && !parent) return SV_ERR_NULL;
  if (!aligned16(hidden) || !aligned16(wq) || !aligned16(wk) || !aligned16(wv) ||
      !aligned16(wo) || !aligned16(kv) || !aligned16(out_hidden) ||
      (attn_out && !aligned16(attn_out)))
    return SV_ERR_ALIGN;
  if (!workspace || workspace_bytes < layer_workspace_bytes(P)) return SV_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return SV_ERR_ALIGN;
  Args a;
  memset(&a, 0, sizeof(a));
  a.kv = kv;
  a.kv_offset = kv_offset;
  a.hidden = hidden;
  a.parent = parent;
  a.seq_status = seq_status;
  a.ws = (char*)workspace;
  (void)hipGetLastError();
  if (launch_layer_share(P, a, wq, wk, wv, wo, (double)rope_theta, kv, out_hidden, attn_out,
                         (hipStream_t)stream) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

}  // extern "C"
