/*
 * specverify.h - C ABI of the MI355X (gfx950) verification stage of tree
 * speculative sampling: tree-masked attention over a prefix KV cache and a
 * packed draft tree, LM-head logits for every tree slot, and multi-round
 * speculative sampling (or greedy argmax comparison) down the tree.
 *
 * What each call computes is stated on the source pages:
 *  - "LLM speculative decoding: EAGLE" (jingming.pro), sec. 2.2-2.3:
 *    speculative sampling (accept a drafted token with probability
 *    min(1, p/q); on rejection resample from norm(max(0, p - q)); if every
 *    drafted token passes, draw a bonus token from the next target
 *    distribution); sec. 4.2: the tree is packed into one sequence and the
 *    attention mask lets each node see the prefix and its own ancestors.
 *  - "EAGLE / EAGLE-2" excerpts (modelers.csdn.net), sec. 1.3.2 and 1.7:
 *    one target forward with tree attention scores every tree node; at each
 *    node speculative sampling is applied recursively over its candidate
 *    children (SpecInfer-style multi-round sampling); greedy decoding compares
 *    with the target argmax.
 *
 * Conventions shared by every call
 *  - Slots: a sequence with N draft nodes has R = N + 1 slots. Slot 0 is the
 *    root (the last committed token); slot j + 1 is node j. Row-major arrays
 *    "[B*R, ...]" hold sequence b's slot s at row b*R + s.
 *  - Tree: parent[b*N + j] in [-1, j); -1 = child of the root. Children of a
 *    slot are tested in ascending node index.
 *  - KV cache: kv is [sum_b (L_b + N), 2, Hkv, D] (K then V per token row).
 *    Sequence b owns rows kv_offset[b] .. kv_offset[b+1]-1 = L_b + N rows:
 *    the first L_b rows are its prefix (the last of them is the root token),
 *    the next N rows are the K/V of its N tree nodes in packed order.
 *    Slot 0 attends to the L_b prefix rows; node j also attends to the tree
 *    rows of its ancestors and itself. Query head h reads KV head
 *    h / (Hq / Hkv); scores are q.k / sqrt(D).
 *  - Queries and LM-head input: node_hidden [B*R, Hq*D]; slot row r holds the
 *    query of head h at columns h*D .. h*D + D - 1, and the same row is the
 *    feature the LM head maps to logits.
 *  - Temperature T >= 0 per sequence: p = softmax(target_logits / T),
 *    q = softmax(draft_logits / T); T = 0 selects greedy verification.
 *  - Uniforms [B*R] in [0, 1): u[b*R + j] tests node j (accept when
 *    u*q(x) <= p(x)); u[b*R + N] drives the single final draw (the smallest
 *    token whose cumulative weight exceeds u times the total weight).
 *  - Pointers are device pointers unless a comment says host. All calls are
 *    asynchronous on `stream`; the library allocates no memory, keeps no
 *    state between calls beyond a one-time device query, and is thread-safe
 *    when concurrent calls use distinct workspaces and outputs.
 *  - Return value: SV_OK, or a synchronous error (argument check or launch
 *    failure). Problems found in the data on the device are reported per
 *    sequence in seq_status (bit flags below); a sequence with an error bit
 *    set gets accept_len = -1 and all-(-1) paths and tokens.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A hipStream_t; NULL means the null stream. */
typedef struct ihipStream_t* sv_stream_t;

/* A hipEvent_t. */
typedef struct ihipEvent_t* sv_event_t;

/* Stages of sv_verify_tree (indexes of sv_debug.stage_events). Below 512 rows (B*R)
 * they are launched as prep, LM head, then attention (on the library's second stream)
 * beside sampling; from 512 rows as prep, attention, LM head, sampling. */
enum { SV_STAGE_PREP = 0, SV_STAGE_ATTENTION = 1, SV_STAGE_LM_HEAD = 2, SV_STAGE_SAMPLING = 3,
       SV_NUM_STAGES = 4 };

/* Storage type of kv, node_hidden and lm_head. Logits are always fp32. */
enum { SV_BF16 = 0, SV_F32 = 1 };

/* How the drafted siblings of a slot were sampled (sv_problem.sampling; T > 0
 * only). SV_SAMPLE_IID: independent draws from the slot's draft distribution
 * q (duplicates allowed). SV_SAMPLE_DISTINCT: draws without replacement, so
 * the i-th sibling came from q with the earlier siblings' tokens removed and
 * renormalised; the acceptance test and the residual step use that
 * distribution, and duplicate sibling tokens are an input error. */
enum { SV_SAMPLE_IID = 0, SV_SAMPLE_DISTINCT = 1 };

/* Synchronous status codes (return values). */
enum {
  SV_OK = 0,
  SV_ERR_NULL = 1,      /* a required pointer is NULL */
  SV_ERR_SHAPE = 2,     /* batch < 1, N outside [0, 64], Hq % Hkv != 0, hidden != Hq*D,
                           D not 64 or 128, vocab < 1, max_prefix < 1,
                           max_children outside [1, 64], sampling not an SV_SAMPLE_*
                           value, or a size overflow */
  SV_ERR_DTYPE = 3,     /* dtype is neither SV_BF16 nor SV_F32 */
  SV_ERR_WORKSPACE = 4, /* workspace NULL or smaller than sv_workspace_size() */
  SV_ERR_HIP = 5,       /* a HIP launch or device query failed */
  SV_ERR_ALIGN = 6,     /* a pointer misses the 16-byte alignment the kernels load with */
  SV_ERR_SCRATCH = 7    /* sv_sample_noalloc: the problem needs more scratch than
                           SV_NOALLOC_SCRATCH_BYTES */
};

/* Per-sequence device status bits (seq_status[b]). Bits 0-7 are errors. */
enum {
  SV_SEQ_ERR_TREE = 1 << 0,        /* parent[j] outside [-1, j), or a slot has more
                                      than max_children children */
  SV_SEQ_ERR_TOKEN = 1 << 1,       /* node_token outside [0, vocab), or (SV_SAMPLE_DISTINCT,
                                      T > 0) two siblings with the same token */
  SV_SEQ_ERR_TEMPERATURE = 1 << 2, /* T < 0 or not finite */
  SV_SEQ_ERR_PREFIX = 1 << 3,      /* L_b = kv_offset[b+1] - kv_offset[b] - N outside
                                      [1, max_prefix] */
  SV_SEQ_ERR_NONFINITE = 1 << 4,   /* NaN/Inf logits on a slot the walk used (sv_tree_expand:
                                      a draft row with NaN, +inf or no finite logit) */
  SV_SEQ_ERR_INTERNAL = 1 << 5,    /* a bounded wait between the workgroups sharing a
                                      sequence's walk gave up (not expected) */
  SV_SEQ_ERR_PATH = 1 << 6,        /* sv_compact_cache: accept_len outside [-1, N], an
                                      accept path not strictly increasing inside [0, N),
                                      or L_b + N rows past the sequence's region */
  SV_SEQ_ERR_POOL = 1 << 7,        /* sv_tree_expand: the step would overflow the
                                      sequence's pool capacity (nothing was added) */
  SV_SEQ_WARN_UNIFORM = 1 << 8,    /* a uniform outside [0, 1) was clamped to
                                      [0, 1 - 2^-24] (NaN -> 0) */
  SV_SEQ_WARN_RESIDUAL = 1 << 9,   /* a residual mass came out <= 0 (impossible in exact
                                      arithmetic); the previous distribution was kept */
  SV_SEQ_WARN_CDF_CLAMP = 1 << 10  /* rounding defeated the inverse-CDF comparison; the
                                      last token with positive weight was drawn */
};

/* Problem shape. All sequences share N; prefix lengths may differ. */
typedef struct {
  int32_t batch;        /* B >= 1 */
  int32_t n_nodes;      /* N in [0, 64] draft nodes per sequence */
  int32_t n_q_heads;    /* Hq */
  int32_t n_kv_heads;   /* Hkv, divides Hq */
  int32_t head_dim;     /* D: 64 or 128 */
  int32_t hidden;       /* d, must equal Hq * D */
  int32_t vocab;        /* V >= 1 */
  int32_t dtype;        /* SV_BF16 or SV_F32 */
  int32_t max_prefix;   /* upper bound on every L_b (sizes the attention grid) */
  int32_t max_children; /* upper bound on the children of any slot (1..64); sizes the
                           number of residual passes */
  int32_t sampling;     /* SV_SAMPLE_IID or SV_SAMPLE_DISTINCT */
  int32_t top_k;        /* >= 0; 0 < top_k < vocab keeps only the top_k most probable
                           tokens of every sampling row of p and q (see below) */
  float top_p;          /* in [0, 1]; 0 < top_p < 1 then keeps the shortest prefix of
                           the remaining tokens, most probable first, whose mass
                           reaches top_p times their mass; 0 and 1 mean no cut */
} sv_problem;

/* Top-k / top-p warping ("LLM speculative decoding: EAGLE" (jingming.pro),
 * sec. 1: the distribution that speculative sampling preserves is the one
 * after temperature, top-k and top-p processing). With top_k or top_p active,
 * both p = softmax(z/T) and q = softmax(z_draft/T) of every slot the walk
 * uses are restricted to their kept sets and renormalised before the tests,
 * the residuals and the final draw; tokens rank by probability, ties to the
 * lower id; top-k is applied first, top-p to what it kept. The drafted tokens
 * must come from the warped q. Greedy rows (T = 0) are unaffected. The cost
 * is a radix selection over each visited row (a few vocabulary passes). */

/* Optional device outputs of intermediate stages; any member may be NULL. */
typedef struct {
  float* logits;      /* [B*R, V] target logits. When set, sv_verify_tree writes the
                         logits here instead of into the workspace. */
  float* slot_stats;  /* [B*R, 4]: max and sum of exp((z - max)/T) of the target row,
                         then of the draft row; greedy rows hold the argmax logit in
                         [0]. Rebuild p(v) = exp((z_v - m)/T) / S. Draft entries are
                         written for every slot with children of a sampling
                         (T > 0) sequence when all B*R draft rows together take at
                         most 256 MB (their statistics are then computed up
                         front), else only for the slots with children that the
                         walk visited; others are left untouched. With top-k / top-p, the sums of the rows the walk
                         visited are their kept masses (p(v) = 0 outside the kept
                         set). */
  int32_t* slot_argmax; /* [B*R] target argmax (lowest index on ties) of greedy rows,
                           -1 elsewhere */
  float* node_ratio;  /* [B*N] the test value p_{s,i-1}(x)/q_s(x) of node j, where
                         node j is the i-th child of slot s and p_{s,i-1} is the target
                         after its i-1 earlier siblings were rejected (written for the
                         nodes the walk tested, T > 0; +inf when q_s(x) = 0) */
  float* residual_mass; /* [B*R, max_children]: entry i-1 is the mass Z_i of
                           max(0, p_{s,i-1} - q_s) for the rejections the walk made
                           (T > 0); other entries are left untouched */
  sv_event_t* stage_events; /* host array of 2*SV_NUM_STAGES caller-created events, or
                               NULL: event 2i is recorded before stage i's first
                               kernel, event 2i+1 after its last (sv_verify_tree
                               only), on the stream the stage runs on (attention's
                               on the library's second stream below 512 rows), for
                               per-stage device times; a NULL entry is not recorded
                               (time only the stages of interest: every recorded
                               event adds a little to the step) */
} sv_debug;

/* Library version: major*10000 + minor*100 + patch (200 = 0.2.0: sv_problem carries
 * sampling, top_k and top_p). A binding built for another version's struct layouts
 * must not call the library. */
int sv_version(void);

/* Text for a synchronous status code (a return value). */
const char* sv_status_string(int status);

/* Text for one seq_status bit (0 gives "ok"). */
const char* sv_seq_status_string(int bit);

/* Workspace bytes sv_verify_tree / sv_tree_attention / sv_sample need for
 * `prob` (host pointers). Pure host arithmetic; touches no device. */
int sv_workspace_size(const sv_problem* prob, size_t* bytes);

/*
 * The whole verification step for B sequences (see the conventions above):
 * the verification stage of "EAGLE / EAGLE-2" excerpts (modelers.csdn.net),
 * sec. 1.3.2 (one target forward with tree attention over the packed draft
 * tree, then speculative sampling down the tree, sec. 1.7).
 * Inputs:  kv, kv_offset [B+1] int32, node_hidden, parent [B*N], node_token
 *          [B*N], lm_head [V, d], draft_logits [B*R, V] fp32 (row of slot s =
 *          the draft distribution that proposed s's children; rows of leaf
 *          slots are not read), uniforms [B*R] fp32, temperature [B] fp32.
 * Outputs: attn_out [B*R, Hq, D] fp32 (tree attention of every slot),
 *          accept_len [B] (accepted nodes n, -1 on error), accept_path [B*N]
 *          (the accepted node indices root-down, -1 padded), out_tokens
 *          [B*R] (the n accepted drafted tokens, then the corrected or bonus
 *          token, -1 padded), seq_status [B].
 * dbg may be NULL. workspace: device memory of at least sv_workspace_size()
 * bytes, 256-byte aligned, owned by the caller; its contents on entry do not
 * matter. 16-byte alignment is required of kv, node_hidden, lm_head,
 * draft_logits and attn_out.
 * Streams: the step is ordered on `stream` like any launch. Below 512 rows
 * (B*R), the attention stage runs on a second stream that the library owns (one
 * per host thread and device, created on first use): `stream` forks to it after
 * the LM head, sampling runs on `stream` meanwhile, and `stream` waits for it
 * before the step's last work, so later work on `stream` sees every output.
 * Without that stream (creation failed) every stage runs on `stream`.
 */
int sv_verify_tree(const sv_problem* prob,
                   const void* kv, const int32_t* kv_offset,
                   const void* node_hidden,
                   const int32_t* parent, const int32_t* node_token,
                   const void* lm_head,
                   const float* draft_logits, const float* uniforms,
                   const float* temperature,
                   float* attn_out,
                   int32_t* accept_len, int32_t* accept_path, int32_t* out_tokens,
                   int32_t* seq_status,
                   const sv_debug* dbg,
                   void* workspace, size_t workspace_bytes, sv_stream_t stream);

/* Tree attention alone ("LLM speculative decoding: EAGLE" (jingming.pro),
 * sec. 4.2: the draft tree is packed behind the prefix and the mask lets each
 * node see the prefix and its own ancestors, itself included; "EAGLE /
 * EAGLE-2" excerpts (modelers.csdn.net), sec. 1.6.1 and 2.3.2).
 * attn_out [B*R, Hq, D] fp32, row b*R + s = slot s of sequence b: slot 0
 * attends to the L_b prefix rows, node j to those and to the tree rows of its
 * ancestors and itself. Inputs as for sv_verify_tree; workspace as
 * sv_workspace_size() states. seq_status [B] receives the tree and prefix
 * checks; sequences with an error get zero rows. Errors: SV_ERR_NULL,
 * SV_ERR_SHAPE, SV_ERR_DTYPE, SV_ERR_ALIGN, SV_ERR_WORKSPACE, SV_ERR_HIP. */
int sv_tree_attention(const sv_problem* prob,
                      const void* kv, const int32_t* kv_offset,
                      const void* node_hidden, const int32_t* parent,
                      float* attn_out, int32_t* seq_status,
                      void* workspace, size_t workspace_bytes, sv_stream_t stream);

/* LM head alone ("LLM speculative decoding: EAGLE" (jingming.pro), sec. 3.1:
 * the target's frozen LM head maps each position's last-layer feature to
 * vocabulary logits; "EAGLE / EAGLE-2" excerpts, sec. 1.3.2: one target
 * forward scores every tree node). logits [M, V] fp32 = hidden [M, d] x
 * lm_head[V, d]^T, row-major, for any M >= 1 (prob->batch, n_nodes,
 * max_prefix and max_children are not read; M = rows; d = prob->hidden,
 * a multiple of 64 for bf16). hidden and lm_head are bf16 or fp32 as
 * prob->dtype says, 16-byte aligned. Needs no workspace. Errors:
 * SV_ERR_NULL, SV_ERR_DTYPE, SV_ERR_SHAPE, SV_ERR_ALIGN, SV_ERR_HIP. */
int sv_lm_head(const sv_problem* prob, int32_t rows,
               const void* hidden, const void* lm_head, float* logits,
               sv_stream_t stream);

/* Sampling alone ("LLM speculative decoding: EAGLE" (jingming.pro), sec. 2.3:
 * accept a drafted token x with probability min(1, p(x)/q(x)); on rejection
 * continue from norm(max(0, p - q)); when every draft passes, draw the bonus
 * token from the next target distribution; "EAGLE / EAGLE-2" excerpts
 * (modelers.csdn.net), sec. 1.7: at a tree node the sampler is invoked again
 * on the next candidate after a rejection, and the adjusted distribution is
 * sampled only when all candidates are rejected; greedy decoding compares
 * with the target argmax). From given target logits [B*R, V] fp32 (the
 * caller's LM head), with the other inputs and all outputs as for
 * sv_verify_tree except attn_out. kv_offset is not needed (prefix checks are
 * skipped). Errors: as sv_verify_tree. */
int sv_sample(const sv_problem* prob,
              const int32_t* parent, const int32_t* node_token,
              const float* logits, const float* draft_logits,
              const float* uniforms, const float* temperature,
              int32_t* accept_len, int32_t* accept_path, int32_t* out_tokens,
              int32_t* seq_status, const sv_debug* dbg,
              void* workspace, size_t workspace_bytes, sv_stream_t stream);

/*
 * sv_sample without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Arguments, outputs and errors are those of sv_sample,
 * minus the workspace: its scratch (ancestor masks, child lists, per-tile
 * target statistics, the walk's exchange buffers and barrier counters, the
 * top-k / top-p selection buffers) lives in a static device array of
 * SV_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends. Problems needing more return SV_ERR_SCRATCH before
 * any HIP call (batch 32 x 61 slots at V = 128256 needs 8.6 MB, 22.7 MB
 * with top-k / top-p). The first call on a device looks the array's
 * address up (hipGetSymbolAddress, SV_ERR_HIP if that fails); no call
 * allocates. Every call on one GPU uses that GPU's one array, and every
 * kernel re-initialises what it reads of it, so a call's results never
 * depend on an earlier call's; calls that overlap in time on one GPU (two
 * streams, two host threads) race on the array and must be serialised by
 * the caller.
 */
#define SV_NOALLOC_SCRATCH_BYTES (64u << 20)
int sv_sample_noalloc(const sv_problem* prob,
                      const int32_t* parent, const int32_t* node_token,
                      const float* logits, const float* draft_logits,
                      const float* uniforms, const float* temperature,
                      int32_t* accept_len, int32_t* accept_path, int32_t* out_tokens,
                      int32_t* seq_status, const sv_debug* dbg, sv_stream_t stream);

/*
 * KV-cache compaction after acceptance, in place. "EAGLE / EAGLE-2" excerpts
 * (modelers.csdn.net), sec. 1.3.2: the accepted tokens are kept for the next
 * drafting round; "EAGLE (ICML 2024) close reading" (edgeai1.github.io),
 * sec. 5: after a rejection both the target's and the draft decoder's caches
 * are cut back. For every sequence b with n = accept_len[b] >= 0 and every
 * layer l:
 *   row kv_offset[b] + L_b + i  <-  row kv_offset[b] + L_b + accept_path[b*N + i],  i < n
 * with L_b = prefix_len[b], and new_prefix_len[b] = L_b + n. The packed tree
 * puts parents first, so the kept rows come out in decode order. Rows from
 * L_b + n on keep stale contents (free for the next tree); the corrected or
 * bonus token has no row yet.
 * cache: layer l's row r starts at (char*)cache + l*layer_stride + r*row_bytes.
 *   A row is any per-token record of row_bytes bytes (a multiple of 4): the
 *   target's K/V [2, Hkv, D] as sv_verify_tree reads it, the draft decoder's
 *   K/V, or per-token features. Layers must not overlap. 16-byte moves are
 *   used when cache, layer_stride and row_bytes are multiples of 16.
 * kv_offset [B+1], prefix_len [B], accept_len [B], accept_path [B*N]: device
 *   int32, accept_len / accept_path as sv_verify_tree writes them. Sequence b's
 *   tree rows must lie inside its region: kv_offset[b] + L_b + N <= kv_offset[b+1].
 * new_prefix_len [B]: device out. status [B]: device out (0 or
 *   SV_SEQ_ERR_PATH), may be NULL.
 * accept_len = -1 (a sequence sv_verify_tree flagged) leaves the sequence
 * alone with new_prefix_len = L_b and status 0; an invalid length, path or
 * region leaves it alone with status SV_SEQ_ERR_PATH. All caller-owned; no
 * workspace. Errors: SV_ERR_NULL (a required pointer NULL while batch > 0),
 * SV_ERR_SHAPE (batch outside [0, 65535], N outside [0, 64], n_layers outside
 * [1, 65535], row_bytes < 4 or not a multiple of 4, layer_stride < 0),
 * SV_ERR_ALIGN (cache or layer_stride not a multiple of 4), SV_ERR_HIP.
 */
int sv_compact_cache(void* cache, int64_t layer_stride, int32_t n_layers, int32_t row_bytes,
                     int32_t batch, int32_t n_nodes,
                     const int32_t* kv_offset, const int32_t* prefix_len,
                     const int32_t* accept_len, const int32_t* accept_path,
                     int32_t* new_prefix_len, int32_t* status, sv_stream_t stream);

/*
 * EAGLE-2 context-aware dynamic draft tree ("LLM speculative decoding: EAGLE"
 * (jingming.pro), sec. 4.2.1; "EAGLE / EAGLE-2" excerpts (modelers.csdn.net),
 * sec. 2.3.1-2.3.2). A drafted node's value is the product of the draft
 * model's probabilities (softmax of its logits, T = 1) along its path from the
 * root; the root's value is 1. Each expansion step gives every frontier node
 * its C most probable tokens as children (ties: lower token id) and makes the
 * K children of highest value the next frontier (ties: earlier creation,
 * i.e. by frontier position, then child rank). Finalizing ranks every node by
 * value (higher first), then depth (shallower first), then creation order,
 * and keeps the first m, flattened in that order: parent[j] < j, the packed
 * order sv_verify_tree takes. The draft model's forward between steps is the
 * caller's.
 *
 * The pool (caller-owned device arrays, capacity P per sequence): node
 * j < pool_count[b] of sequence b is pool_token / pool_parent (pool id, -1 =
 * the root) / pool_value (fp32) / pool_depth (root = 0) [b*P + j], in creation
 * order. frontier [B*K] holds the pool ids to expand next (-1 = the root),
 * frontier_count [B] how many. seq_status [B] collects error bits; a sequence
 * with an error stops expanding.
 *
 * sv_tree_init: frontier = {root}, empty pool, seq_status = 0.
 * sv_tree_workspace_size: bytes of scratch sv_tree_expand needs for
 *   (batch, n_expand, vocab); pure host arithmetic.
 * sv_tree_expand: draft_logits [B, K, V] fp32; row i of sequence b is the
 *   draft model's next-token logits at frontier[b*K + i], for i <
 *   frontier_count[b] (other rows are not read). Appends frontier_count[b]*C
 *   children to the pool and rewrites frontier / frontier_count. workspace:
 *   caller-owned device memory of sv_tree_workspace_size() bytes, 16-byte
 *   aligned, contents irrelevant on entry.
 *   Per-sequence errors: SV_SEQ_ERR_NONFINITE (a row with NaN, +inf or no
 *   finite logit), SV_SEQ_ERR_POOL (the pool would overflow).
 * sv_tree_finalize: parent [B*m] (indices into the flattened tree, -1 =
 *   root), node_token [B*m], node_pool_id [B*m], n_kept [B] = min(m, pool
 *   size); entries past n_kept are -1.
 * Limits: batch in [1, 65535], K and C in [1, 16] with K*C <= 256,
 * C <= V <= 1048576 (sv_tree_expand), P in [1, 1024], m in [1, 64]. Errors: SV_ERR_SHAPE, SV_ERR_NULL,
 * SV_ERR_ALIGN (draft_logits not 4-byte aligned, workspace not 16-byte
 * aligned), SV_ERR_WORKSPACE (workspace smaller than needed), SV_ERR_HIP.
 */
int sv_tree_init(int32_t batch, int32_t n_expand, int32_t* frontier, int32_t* frontier_count,
                 int32_t* pool_count, int32_t* seq_status, sv_stream_t stream);
int sv_tree_workspace_size(int32_t batch, int32_t n_expand, int32_t vocab, size_t* bytes);
int sv_tree_expand(int32_t batch, int32_t vocab, int32_t n_expand, int32_t n_children,
                   int32_t pool_capacity, const float* draft_logits,
                   int32_t* frontier, int32_t* frontier_count,
                   int32_t* pool_token, int32_t* pool_parent, float* pool_value,
                   int32_t* pool_depth, int32_t* pool_count, int32_t* seq_status,
                   void* workspace, size_t workspace_bytes, sv_stream_t stream);
int sv_tree_finalize(int32_t batch, int32_t pool_capacity, int32_t m,
                     const int32_t* pool_token, const int32_t* pool_parent,
                     const float* pool_value, const int32_t* pool_depth,
                     const int32_t* pool_count,
                     int32_t* parent, int32_t* node_token, int32_t* node_pool_id,
                     int32_t* n_kept, sv_stream_t stream);

/*
 * The full verify-layer share ("LLM speculative decoding: EAGLE"
 * (jingming.pro), sec. 3.1 and 4.2; "EAGLE (ICML 2024) close reading"
 * (edgeai1.github.io), sec. 5: tree position ids). For every slot of every
 * sequence: q = h Wq^T; for every node, k = h Wk^T and v = h Wv^T; q and k
 * rotated by position (root L_b - 1, node j at L_b - 1 + depth(j)); the nodes'
 * rotated K and V written to their cache rows (kv rows kv_offset[b] + L_b + j,
 * the layout of sv_verify_tree); tree attention of q over the prefix and the
 * ancestors (the root's K/V is cache row L_b - 1, not recomputed); out_hidden
 * = bf16(h + attn Wo^T), the input of the LM head. Rotary pairs are
 * (i, i + D/2), angle pos * rope_theta^(-2i/D). No norms or MLP.
 * hidden, out_hidden [B*R, d]; wq [Hq*D, d]; wk, wv [Hkv*D, d]; wo [d, Hq*D]:
 * bf16, row-major, 16-byte aligned. kv: in/out (node rows written). attn_out
 * [B*R, Hq, D] fp32 optional (NULL to skip). seq_status [B] as
 * sv_tree_attention reports it. Requires dtype SV_BF16 and head_dim 128;
 * rope_theta > 0 and finite. workspace: sv_layer_workspace_size() bytes,
 * 256-byte aligned. Errors: as sv_tree_attention, and SV_ERR_SHAPE for a bad
 * rope_theta.
 */
int sv_layer_workspace_size(const sv_problem* prob, size_t* bytes);
int sv_layer_share(const sv_problem* prob, const void* hidden, const void* wq, const void* wk,
                   const void* wv, const void* wo, float rope_theta,
                   void* kv, const int32_t* kv_offset, const int32_t* parent,
                   void* out_hidden, float* attn_out, int32_t* seq_status,
                   void* workspace, size_t workspace_bytes, sv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
