"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Stage-isolated checks (attention alone, LM head alone, sampling fed the
oracle's logits) keep one stage's error out of the next stage's check; the
end-to-end checks run sv_verify_tree on every registered workload, the batched
one at full size with the oracle evaluated on sampled sequences.
"""
import numpy as np
import pytest
import torch

from oracle import verify as ov
from speculative_decoding_tree_amd import lib, synth
from speculative_decoding_tree_amd.runner import DeviceBatch

from parity_util import (MARGIN_STAGE, TOL_ATTN, TOL_LOGIT, TOL_PROB, attn_rel_err, compare_rounds,
                         compare_rounds_e2e, logit_delta, path_excluded, widened)

pytestmark = pytest.mark.gpu

MINI = synth.Workload(
    name="mini_ragged", batch=3, n_nodes=12, n_q_heads=8, n_kv_heads=2, head_dim=128,
    vocab=5000, dtype=synth.BF16, prefix=("list", (1, 77, 300)), tree=("seeded", 4), w_std=0.05,
    draft=("perturbed", 0.5), temperature=("list", (0.0, 0.7, 1.3)))

MINI_F32 = MINI.with_(name="mini_f32", dtype=synth.F32, head_dim=64, n_q_heads=4, n_kv_heads=4)
# 152064 tokens = 594 statistics tiles per row: the slot combine's merge of
# more than 512 tiles (its strided path rather than one batch per lane)
MINI_WIDE = MINI.with_(name="mini_v152k", vocab=152064)

SMALL = ["chain_v1k", "eagle1_7b_t0", "eagle1_7b_t1", "share_70b"]
# 150 short ragged sequences: more last splits than the attention schedule's
# exact makespan estimate takes (its snake-order fallback); 2 KV heads give it
# 128 machines as well
MANY = MINI.with_(name="many_short", batch=150, n_nodes=4, vocab=1000, prefix=("uniform", 1, 300),
                  tree=("chain",), temperature=("split", 0.0, 1.0))


def _run(inp, dbg=True):
    db = DeviceBatch.create(inp)
    d = db.debug_buffers() if dbg else None
    db.verify(dbg=d)
    torch.cuda.synchronize()
    res = db.results()
    if d:
        res.update({k: v.cpu().numpy() for k, v in d.items()})
    return db, res


def _oracle_logits(inp, rows=None):
    w = widened(inp)
    h = w["node_hidden"] if rows is None else w["node_hidden"][rows]
    return ov.lm_head(h, w["lm_head"])


# ---------------------------------------------------------------------------
# LM head alone
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("name", ["chain_v1k", "eagle1_7b_t1", "share_70b", "gqa_8b"])
def test_lm_head_matches_oracle(name):
    inp = synth.generate(name, seed=0)
    _, res = _run(inp)
    ref = _oracle_logits(inp)
    err = np.abs(res["logits"].astype(np.float64) - ref).max()
    print(f"{name}: max |logit err| = {err:.3e}", flush=True)
    assert err <= TOL_LOGIT


@pytest.mark.parametrize("rows", [1, 5, 16, 17, 33, 64, 65, 130, 300, 512, 600, 1000,
                                  # batched-row GEMM: the last 256-row block's lower and
                                  # upper waves on each side of the 16/32/64-row steps of
                                  # its valid-tile loop variants
                                  528, 529, 544, 545, 576, 577, 656, 657, 672, 673, 704,
                                  705, 767])
def test_lm_head_entry_point_ragged_rows(rows):
    rng = np.random.default_rng(rows)
    d, V = 256, 4099                    # ragged vocabulary tile tail
    h = synth.to_bf16_bits(rng.standard_normal((rows, d)).astype(np.float32))
    w = synth.to_bf16_bits((rng.standard_normal((V, d)) * 0.05).astype(np.float32))
    prob = lib.make_problem(1, 0, 2, 2, 128, V, lib.SV_BF16, 1, 1)
    out = torch.full((rows, V), float("nan"), device="cuda")
    lib.sv_lm_head(prob, rows, torch.from_numpy(h.view(np.int16)).cuda(),
                   torch.from_numpy(w.view(np.int16)).cuda(), out)
    torch.cuda.synchronize()
    ref = ov.lm_head(synth.widen(h, "bf16"), synth.widen(w, "bf16"))
    assert np.abs(out.cpu().numpy() - ref).max() <= TOL_LOGIT


# ---------------------------------------------------------------------------
# attention alone
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("wl", [MINI, MINI_F32, MANY] + SMALL + ["gqa_8b"],
                         ids=lambda w: w if isinstance(w, str) else w.name)
def test_attention_matches_oracle(wl):
    inp = synth.generate(wl, seed=1)
    _, res = _run(inp, dbg=False)
    w = widened(inp)
    W = inp.workload
    ref = ov.tree_attention(w["node_hidden"], w["kv"], inp.kv_offset, inp.prefix_len,
                            inp.parent, W.n_nodes, W.n_q_heads, W.n_kv_heads, W.head_dim)
    err = attn_rel_err(res["attn_out"], ref)
    print(f"{W.name}: attention max rel err = {err:.3e}", flush=True)
    assert err <= TOL_ATTN


def test_attention_entry_point_equals_full_step():
    inp = synth.generate(MINI, seed=2)
    db, res = _run(inp, dbg=False)
    out = torch.empty_like(db.t["attn_out"])
    st = torch.empty_like(db.t["seq_status"])
    lib.sv_tree_attention(db.prob, db.t["kv"], db.t["kv_offset"], db.t["node_hidden"],
                          db.t["parent"], out, st, db.workspace)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), res["attn_out"])
    assert (st.cpu().numpy() == 0).all()


# ---------------------------------------------------------------------------
# sampling fed the oracle's logits (rounded to fp32)
# ---------------------------------------------------------------------------


def _sample_with_logits(inp, logits32):
    db = DeviceBatch.create(inp)
    W = inp.workload
    B, N, R = W.batch, W.n_nodes, W.rows
    t = db.t
    lg = torch.from_numpy(logits32).cuda()
    d = db.debug_buffers()
    d.pop("logits")
    lib.sv_sample(db.prob, t["parent"], t["node_token"], lg, t["draft_logits"], t["uniforms"],
                  t["temperature"], t["accept_len"], t["accept_path"], t["out_tokens"],
                  t["seq_status"], dbg=d, workspace=db.workspace)
    torch.cuda.synchronize()
    res = db.results()
    res.update({k: v.cpu().numpy() for k, v in d.items()})
    return res


def _check_probabilities(inp, logits64, res, rounds):
    """Probabilities rebuilt from the GPU's slot statistics vs the oracle's:
    the target at every slot, the draft at every slot with children that the
    walk visited (the walk computes draft statistics nowhere else)."""
    W = inp.workload
    R, N = W.rows, W.n_nodes
    worst = 0.0
    for b in range(W.batch):
        T = float(inp.temperature[b])
        if T == 0.0:
            continue
        r = rounds[b]
        visited = {0} | {j + 1 for j in r.path}
        for s in range(R):
            row = b * R + s
            m, S = res["slot_stats"][row, 0], res["slot_stats"][row, 1]
            p_gpu = np.exp((logits64[row] - m) / T) / S
            worst = max(worst, np.abs(p_gpu - ov.softmax_t(logits64[row], T)).max())
            kids = [j for j in range(N) if inp.parent[b * N + j] == s - 1]
            mq, Sq = res["slot_stats"][row, 2], res["slot_stats"][row, 3]
            if kids and s in visited and not path_excluded(r, T):
                assert np.isfinite(mq) and np.isfinite(Sq), (b, s)
            if kids and np.isfinite(mq):
                zd = inp.draft_logits[row].astype(np.float64)
                q_gpu = np.exp((zd - mq) / T) / Sq
                worst = max(worst, np.abs(q_gpu - ov.softmax_t(zd, T)).max())
    return worst


@pytest.mark.parametrize("wl", [MINI, MINI_WIDE, MANY] + SMALL + ["gqa_8b"],
                         ids=lambda w: w if isinstance(w, str) else w.name)
def test_sampling_stage_matches_oracle(wl):
    inp = synth.generate(wl, seed=3)
    W = inp.workload
    logits32 = _oracle_logits(inp).astype(np.float32)
    res = _sample_with_logits(inp, logits32)
    logits64 = logits32.astype(np.float64)
    rounds, _, _, _ = ov.sample_batch(logits64, inp.draft_logits.astype(np.float64), inp.parent,
                                      inp.node_token, inp.uniforms, inp.temperature, W.n_nodes)
    npath, nfin, excl, bad = compare_rounds(rounds, inp.temperature, res["accept_len"],
                                            res["accept_path"], res["out_tokens"], W.n_nodes,
                                            margin=MARGIN_STAGE)
    print(f"{W.name}: paths {npath}, final tokens {nfin}, excluded {excl}", flush=True)
    assert not bad, bad[:3]
    assert (res["seq_status"] & lib.SEQ_ERR_MASK == 0).all()
    assert _check_probabilities(inp, logits64, res, rounds) <= TOL_PROB
    # per-node test values against the oracle's on the walked tests of rounds
    # whose path is compared (the GPU tests exactly those nodes there)
    for b, r in enumerate(rounds):
        if path_excluded(r, float(inp.temperature[b])):
            continue
        for t in r.tests:
            g = res["node_ratio"][b * W.n_nodes + t.node]
            assert abs(g - t.ratio) <= 1e-4 * max(1.0, abs(t.ratio)), (b, t, g)


def _warp_top_p(W):
    # the C ABI carries top_p as fp32; the oracle takes the same value
    return float(np.float32(W.top_p)) if 0.0 < W.top_p < 1.0 else 1.0


def _kept_sets_agree(r, z_gpu, z_ref, T, top_k, top_p):
    """Whether warping keeps the same tokens on the GPU's and the oracle's
    target logits at every slot the round visited (the draft rows are the same
    input on both sides)."""
    for s in r.visited:
        a = ov.warp(ov.softmax_t(z_gpu[s], T), top_k, top_p) > 0.0
        b = ov.warp(ov.softmax_t(z_ref[s], T), top_k, top_p) > 0.0
        if not np.array_equal(a, b):
            return False
    return True


def _compare_e2e(inp, ref, res, min_final_frac=0.5):
    """End-to-end rounds against the oracle, two ways.

    (a) Against the full fp64 oracle: the exclusion windows come from the
        measured logit error of each sequence (parity_util.e2e_exclusions).
    (b) The oracle's sampling run on the GPU's own fp32 logits, compared at the
        stage margin: this isolates the sampling of the timed path from the
        LM head's rounding, and compares most final draws.
    Both must be free of mismatches; (b) must compare every path it does not
    exclude by the stated |u - p/q| rule and, for batches of 8 or more, at
    least `min_final_frac` of the final draws."""
    W = inp.workload
    B, N, R = W.batch, W.n_nodes, W.rows
    wr = W.children == "distinct"
    tp = _warp_top_p(W)
    warped = W.top_k > 0 or tp < 1.0
    gl = res["logits"]
    deltas = [logit_delta(gl[b * R:(b + 1) * R], ref.logits[b * R:(b + 1) * R])
              for b in range(B)]
    assert max(deltas) <= TOL_LOGIT
    keep = list(range(B))
    if warped:
        keep = [b for b in range(B) if float(inp.temperature[b]) == 0.0 or _kept_sets_agree(
            ref.rounds[b], gl[b * R:(b + 1) * R], ref.logits[b * R:(b + 1) * R],
            float(inp.temperature[b]), W.top_k, tp)]
    sel_rows = np.concatenate([np.arange(b * R, (b + 1) * R) for b in keep]) if keep else []
    sel_nodes = np.concatenate([np.arange(b * N, (b + 1) * N) for b in keep]) if keep else []
    npath, nfin, excl, bad = compare_rounds_e2e(
        [ref.rounds[b] for b in keep], inp.temperature[keep], res["accept_len"][keep],
        res["accept_path"][sel_nodes], res["out_tokens"][sel_rows], N,
        [deltas[b] for b in keep], ref.logits[sel_rows], inp.draft_logits[sel_rows],
        inp.node_token[sel_nodes], wr, W.top_k, tp)
    assert not bad, bad[:3]
    excl += B - len(keep)
    # (b) the oracle's sampling on the GPU's logits
    rounds_g, _, _, _ = ov.sample_batch(gl.astype(np.float64), inp.draft_logits.astype(np.float64),
                                        inp.parent, inp.node_token, inp.uniforms,
                                        inp.temperature, N, wr, W.top_k, tp)
    np2, nf2, ex2, bad2 = compare_rounds(rounds_g, inp.temperature, res["accept_len"],
                                         res["accept_path"], res["out_tokens"], N,
                                         margin=MARGIN_STAGE)
    assert not bad2, bad2[:3]
    if B >= 8:
        assert nf2 >= min_final_frac * B, (nf2, B)
    print(f"{W.name}: max logit delta {max(deltas):.2e}; vs fp64 oracle: paths {npath}, "
          f"final tokens {nfin}, excluded {excl}; vs oracle sampling on GPU logits: paths "
          f"{np2}, final tokens {nf2}, excluded {ex2}; accept_len {res['accept_len'].tolist()}",
          flush=True)
    return [npath, nfin, excl]


# ---------------------------------------------------------------------------
# many rounds on one context: fresh candidates and uniforms per copy
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("name,copies", [("chain_v1k", 64), ("eagle1_7b_t1", 48),
                                         ("share_70b", 48), ("gqa_8b", 24)])
def test_sampling_many_rounds(name, copies):
    base = synth.generate(name, seed=11)
    inp = synth.replicate_rounds(base, copies, seed=12)
    W = inp.workload
    logits32 = np.tile(_oracle_logits(base)[:W.rows].astype(np.float32), (copies, 1))
    res = _sample_with_logits(inp, logits32)
    rounds, _, _, _ = ov.sample_batch(logits32.astype(np.float64),
                                      inp.draft_logits.astype(np.float64), inp.parent,
                                      inp.node_token, inp.uniforms, inp.temperature, W.n_nodes)
    npath, nfin, excl, bad = compare_rounds(rounds, inp.temperature, res["accept_len"],
                                            res["accept_path"], res["out_tokens"], W.n_nodes,
                                            margin=MARGIN_STAGE)
    lens = np.bincount(res["accept_len"], minlength=1).tolist()
    print(f"{W.name}: paths {npath}, final tokens {nfin}, excluded {excl}; "
          f"accept-length histogram {lens}", flush=True)
    assert not bad, bad[:3]
    assert npath >= 0.9 * copies and nfin >= 0.5 * copies


@pytest.mark.parametrize("name,copies", [("eagle1_7b_t1", 16), ("gqa_8b", 8)])
def test_verify_tree_many_rounds(name, copies):
    base = synth.generate(name, seed=13)
    inp = synth.replicate_rounds(base, copies, seed=14)
    W = inp.workload
    _, res = _run(inp)
    w = widened(inp)
    # one oracle forward serves every copy: the context is the same
    ref_logits = ov.lm_head(w["node_hidden"][:W.rows], w["lm_head"])
    assert np.abs(res["logits"] - np.tile(ref_logits, (copies, 1))).max() <= TOL_LOGIT
    rounds, _, _, _ = ov.sample_batch(np.tile(ref_logits, (copies, 1)),
                                      inp.draft_logits.astype(np.float64), inp.parent,
                                      inp.node_token, inp.uniforms, inp.temperature, W.n_nodes)
    R = W.rows
    deltas = [logit_delta(res["logits"][b * R:(b + 1) * R], ref_logits) for b in range(copies)]
    npath, nfin, excl, bad = compare_rounds_e2e(rounds, inp.temperature, res["accept_len"],
                                                res["accept_path"], res["out_tokens"], W.n_nodes,
                                                deltas, [ref_logits] * copies, inp.draft_logits,
                                                inp.node_token)
    print(f"{W.name}: paths {npath}, final tokens {nfin}, excluded {excl} "
          f"(max logit delta {max(deltas):.1e})", flush=True)
    assert not bad, bad[:3]
    assert npath >= 0.9 * copies


# ---------------------------------------------------------------------------
# the whole step
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("wl", [MINI, MINI_F32, MANY] + SMALL,
                         ids=lambda w: w if isinstance(w, str) else w.name)
def test_verify_tree_end_to_end(wl):
    inp = synth.generate(wl, seed=4)
    W = inp.workload
    _, res = _run(inp)
    w = widened(inp)
    ref = ov.verify_batch(w["node_hidden"], w["kv"], inp.kv_offset, inp.prefix_len, inp.parent,
                          inp.node_token, w["lm_head"], inp.draft_logits, inp.uniforms,
                          inp.temperature, W.n_nodes, W.n_q_heads, W.n_kv_heads, W.head_dim)
    assert attn_rel_err(res["attn_out"], ref.attn_out) <= TOL_ATTN
    assert np.abs(res["logits"] - ref.logits).max() <= TOL_LOGIT
    _compare_e2e(inp, ref, res)
    assert (res["seq_status"] & lib.SEQ_ERR_MASK == 0).all()


def test_gqa_8b_end_to_end():
    inp = synth.generate("gqa_8b", seed=0)
    W = inp.workload
    _, res = _run(inp)
    w = widened(inp)
    ref = ov.verify_batch(w["node_hidden"], w["kv"], inp.kv_offset, inp.prefix_len, inp.parent,
                          inp.node_token, w["lm_head"], inp.draft_logits, inp.uniforms,
                          inp.temperature, W.n_nodes, W.n_q_heads, W.n_kv_heads, W.head_dim)
    assert attn_rel_err(res["attn_out"], ref.attn_out) <= TOL_ATTN
    assert np.abs(res["logits"] - ref.logits).max() <= TOL_LOGIT
    _compare_e2e(inp, ref, res)


class _LazyOracleLogits:
    """Oracle logits of one sequence's rows, computed (fp64) on first use:
    the walk reads only the slots it visits."""

    def __init__(self, hidden_rows, weight):
        self.h = hidden_rows
        self.w = weight
        self.rows = {}

    def __getitem__(self, s):
        if s not in self.rows:
            self.rows[s] = ov.lm_head(self.h[s:s + 1], self.w)[0]
        return self.rows[s]

    def __len__(self):
        return len(self.h)


def test_batch32_bench_configuration_full_size():
    """The batched workload at full size (32 sequences, 1952 rows, V = 128256)
    in the launch configuration the benchmark times.

    Run 1 is the benchmark's call: stage events only, so the LM-head GEMM's
    epilogue reduces every row to its sampling statistics and stores logits
    only for the rows of sampled (T > 0) sequences. Run 2 reads the
    statistics back (slot statistics, argmax, test values, residual masses)
    with the same store pattern (still no debug logits). Run 3 also asks for
    every row's logits. All three are bitwise equal in every output. Then,
    for all 32 sequences:
      - the oracle's walk on the GPU's own fp32 logits, compared at the stage
        margin (every path, and most final draws);
      - p rebuilt from the epilogue's slot statistics within 1e-5 of the
        oracle's softmax of the same logits, on every row of every sampled
        sequence; the greedy rows' argmax is the lowest-index argmax of the
        row's logits;
      - every round against the fp64 oracle (its logits computed for the
        slots its walk visits), windows from the measured logit error;
      - the GPU logits of those rows within 1e-2 of the oracle's, and tree
        attention of the root and of the last node of every sequence within
        1e-2 relative.
    """
    inp = synth.generate("batch32_8b", seed=0)
    W = inp.workload
    B, N, R, V = W.batch, W.n_nodes, W.rows, W.vocab
    db = DeviceBatch.create(inp)
    outs = []
    ev = lib.StageEvents(stages=("lm_head",))
    db.verify(dbg={"stage_events": ev})            # run 1: the benchmark's timed call
    torch.cuda.synchronize()
    outs.append(db.results())
    stage_ms = ev.elapsed()
    ev.destroy()
    assert list(stage_ms) == ["lm_head"] and stage_ms["lm_head"] > 0.0, stage_ms
    d2 = db.debug_buffers()
    d2.pop("logits")
    db.verify(dbg=d2)                              # run 2: statistics back, same stores
    torch.cuda.synchronize()
    outs.append(db.results())
    d3 = db.debug_buffers()
    db.verify(dbg=d3)                              # run 3: every row's logits as well
    torch.cuda.synchronize()
    outs.append(db.results())
    for k in outs[0]:
        np.testing.assert_array_equal(outs[0][k], outs[1][k], err_msg=k)
        np.testing.assert_array_equal(outs[0][k], outs[2][k], err_msg=k)
    st2 = {k: v.cpu().numpy() for k, v in d2.items()}
    st3 = {k: v.cpu().numpy() for k, v in d3.items()}
    for k in st2:
        np.testing.assert_array_equal(st2[k], st3[k], err_msg=k)
    res = outs[0]
    assert (res["seq_status"] & lib.SEQ_ERR_MASK == 0).all(), res["seq_status"]
    gl = st3["logits"]
    T = inp.temperature
    sampled = [b for b in range(B) if T[b] > 0.0]
    assert 0 < len(sampled) < B

    # sampling of the timed path on its own logits, every sequence
    rounds_g, _, _, _ = ov.sample_batch(gl, inp.draft_logits, inp.parent, inp.node_token,
                                        inp.uniforms, T, N)
    np_g, nf_g, ex_g, bad = compare_rounds(rounds_g, T, res["accept_len"], res["accept_path"],
                                           res["out_tokens"], N, margin=MARGIN_STAGE)
    assert not bad, bad[:3]
    assert nf_g >= B // 2, (nf_g, B)

    # the epilogue's statistics: p within 1e-5 on every row of every sampled
    # sequence; the greedy rows' argmax bit-exact
    worst = 0.0
    for b in sampled:
        for r in range(b * R, (b + 1) * R):
            z = gl[r].astype(np.float64)
            m, S = st2["slot_stats"][r, 0], st2["slot_stats"][r, 1]
            p_gpu = np.exp((z - m) / T[b]) / S
            worst = max(worst, float(np.abs(p_gpu - ov.softmax_t(z, T[b])).max()))
    assert worst <= TOL_PROB, worst
    for b in range(B):
        if T[b] == 0.0:
            for r in range(b * R, (b + 1) * R):
                assert st2["slot_argmax"][r] == int(np.argmax(gl[r])), r

    # every round against the fp64 oracle, logits of the visited slots only
    w = widened(inp)
    rounds, deltas, zts = [], [], []
    for b in range(B):
        rows = slice(b * R, (b + 1) * R)
        zt = _LazyOracleLogits(w["node_hidden"][rows], w["lm_head"])
        zts.append(zt)
        r = ov.verify_round(zt, inp.draft_logits[rows], inp.parent[b * N:(b + 1) * N],
                            inp.node_token[b * N:(b + 1) * N], inp.uniforms[rows], float(T[b]))
        rounds.append(r)
        deltas.append(max(logit_delta(gl[b * R + s], zt[s]) for s in zt.rows))
    assert max(deltas) <= TOL_LOGIT, max(deltas)
    np_o, nf_o, ex_o, bad = compare_rounds_e2e(rounds, T, res["accept_len"], res["accept_path"],
                                               res["out_tokens"], N, deltas, zts,
                                               inp.draft_logits, inp.node_token)
    assert not bad, bad[:3]
    assert np_o >= B - 4, (np_o, ex_o)

    # tree attention of the root and of the last node of every sequence
    L = inp.prefix_len
    worst_attn = 0.0
    for b in range(B):
        base = int(inp.kv_offset[b])
        kv_b = w["kv"][base: base + int(L[b]) + N]
        for s in (0, R - 1):
            q = w["node_hidden"][b * R + s].reshape(W.n_q_heads, W.head_dim)
            o = ov.tree_attention_slot(q, kv_b[:, 0], kv_b[:, 1], int(L[b]),
                                       inp.parent[b * N:(b + 1) * N], s, W.n_kv_heads)
            worst_attn = max(worst_attn, attn_rel_err(res["attn_out"][b * R + s][None], o[None]))
    assert worst_attn <= TOL_ATTN, worst_attn
    print(f"batch32 bench configuration: stage ms {stage_ms}; on GPU logits paths {np_g} "
          f"finals {nf_g} excluded {ex_g}; vs fp64 oracle paths {np_o} finals {nf_o} excluded "
          f"{ex_o} (max logit delta {max(deltas):.2e}); max p err {worst:.2e}; attention "
          f"{worst_attn:.2e}; accept_len {res['accept_len'].tolist()}", flush=True)

    # properties that hold for every sequence
    for b in range(B):
        n = int(res["accept_len"][b])
        path = res["accept_path"][b * N:(b + 1) * N]
        prev = -1
        for c in path[:n]:
            assert inp.parent[b * N + c] == prev
            prev = c
        assert (path[n:] == -1).all()
        toks = res["out_tokens"][b * R:(b + 1) * R]
        assert 0 <= toks[n] < V and (toks[n + 1:] == -1).all()
        if T[b] == 0.0:
            # greedy: the emitted tokens are the argmax of the visited slots
            slots = [0] + [int(c) + 1 for c in path[:n]]
            for i, s in enumerate(slots):
                assert toks[i] == int(st2["slot_argmax"][b * R + s])


# Below 512 rows the tile GEMMs k_gemm_bf16<MT, NT, WM, WN> write every
# row's logits and the statistics kernel reduces them: 39 rows (<4,4,1,4>),
# 244 rows (<4,8,2,2>) and 26 rows at hidden size 512 (<2,4,1,4>; the
# streaming kernels need at least 1024), each with a ragged last vocabulary
# tile and greedy and sampled sequences.
TILE39 = MINI.with_(name="tile_39rows")
TILE244 = MINI.with_(name="tile_244rows", batch=4, n_nodes=60, vocab=20000, tree=("seeded", 6),
                     prefix=("list", (64, 300, 17, 129)),
                     temperature=("list", (0.0, 1.0, 0.6, 1.4)))
TILE26 = MINI.with_(name="tile_26rows_k512", batch=2, n_q_heads=4, n_kv_heads=2,
                    prefix=("list", (50, 200)), temperature=("list", (1.0, 0.0)))


@pytest.mark.parametrize("wl", [TILE39, TILE244, TILE26], ids=lambda w: w.name)
def test_tile_gemm_statistics_configuration(wl):
    """Row statistics below 512 rows in the step's own launch configuration.
    Run 1 records stage events only (what the benchmark times), run 2 reads
    the statistics back, run 3 also every row's logits: all outputs bitwise
    equal. p rebuilt from the slot statistics is within 1e-5 of the softmax of
    the GPU's logits on every row of every sampled sequence; a greedy row's
    argmax is the lowest-index argmax of its logits; the rounds match the
    oracle's on the GPU's logits and on its own fp64 logits."""
    inp = synth.generate(wl, seed=6)
    W = inp.workload
    B, N, R = W.batch, W.n_nodes, W.rows
    db = DeviceBatch.create(inp)
    outs = []
    ev = lib.StageEvents(stages=("lm_head",))
    db.verify(dbg={"stage_events": ev})
    torch.cuda.synchronize()
    outs.append(db.results())
    ev.destroy()
    d2 = db.debug_buffers()
    d2.pop("logits")
    db.verify(dbg=d2)
    torch.cuda.synchronize()
    outs.append(db.results())
    d3 = db.debug_buffers()
    db.verify(dbg=d3)
    torch.cuda.synchronize()
    outs.append(db.results())
    for k in outs[0]:
        np.testing.assert_array_equal(outs[0][k], outs[1][k], err_msg=k)
        np.testing.assert_array_equal(outs[0][k], outs[2][k], err_msg=k)
    st2 = {k: v.cpu().numpy() for k, v in d2.items()}
    st3 = {k: v.cpu().numpy() for k, v in d3.items()}
    for k in st2:
        np.testing.assert_array_equal(st2[k], st3[k], err_msg=k)
    res = dict(outs[0])
    assert (res["seq_status"] & lib.SEQ_ERR_MASK == 0).all(), res["seq_status"]
    gl = st3["logits"]
    T = inp.temperature
    assert (T > 0.0).any() and (T == 0.0).any()
    worst = 0.0
    for b in range(B):
        for r in range(b * R, (b + 1) * R):
            if T[b] > 0.0:
                z = gl[r].astype(np.float64)
                m, S = st2["slot_stats"][r, 0], st2["slot_stats"][r, 1]
                p_gpu = np.exp((z - m) / T[b]) / S
                worst = max(worst, float(np.abs(p_gpu - ov.softmax_t(z, T[b])).max()))
            else:
                assert st2["slot_argmax"][r] == int(np.argmax(gl[r])), r
    assert worst <= TOL_PROB, worst
    w = widened(inp)
    ref = ov.verify_batch(w["node_hidden"], w["kv"], inp.kv_offset, inp.prefix_len, inp.parent,
                          inp.node_token, w["lm_head"], inp.draft_logits, inp.uniforms,
                          inp.temperature, N, W.n_q_heads, W.n_kv_heads, W.head_dim)
    assert attn_rel_err(res["attn_out"], ref.attn_out) <= TOL_ATTN
    res["logits"] = gl
    _compare_e2e(inp, ref, res)


def test_deterministic_reruns():
    inp = synth.generate(MINI, seed=5)
    db = DeviceBatch.create(inp)
    outs = []
    for _ in range(2):
        d = db.debug_buffers()
        db.verify(dbg=d)
        torch.cuda.synchronize()
        r = db.results()
        r["logits"] = d["logits"].cpu().numpy()
        outs.append(r)
    for k in outs[0]:
        np.testing.assert_array_equal(outs[0][k], outs[1][k])


@pytest.mark.parametrize("rows,V", [(1, 32000), (5, 128256), (11, 32000), (16, 32000),
                                    (17, 32001), (27, 32000), (32, 70000), (33, 32000),
                                    (61, 128256), (64, 65536), (64, 1000)])
def test_lm_head_few_rows_streaming(rows, V):
    """Up to 32 rows take the weight-streaming GEMM with X staged in LDS per K
    segment (16-byte stores when V % 4 == 0, element stores otherwise); 33-64
    rows the LDS-tiled GEMM: every row against the oracle at K = 4096."""
    rng = np.random.default_rng(rows * 7 + V)
    d = 4096
    h = synth.to_bf16_bits(rng.standard_normal((rows, d)).astype(np.float32))
    w = synth.to_bf16_bits((rng.standard_normal((V, d)) * 0.02).astype(np.float32))
    prob = lib.make_problem(1, 0, 32, 8, 128, V, lib.SV_BF16, 1, 1)
    out = torch.full((rows, V), float("nan"), device="cuda")
    lib.sv_lm_head(prob, rows, torch.from_numpy(h.view(np.int16)).cuda(),
                   torch.from_numpy(w.view(np.int16)).cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    ref = ov.lm_head(synth.widen(h, "bf16"), synth.widen(w, "bf16"))
    err = np.abs(got - ref).max()
    print(f"rows {rows} V {V}: max |logit err| = {err:.3e}", flush=True)
    assert err <= TOL_LOGIT


@pytest.mark.parametrize("rows,d", [(11, 1024), (16, 2048), (11, 1536), (27, 1536), (27, 1088),
                                    (32, 2560), (3, 8192), (17, 1024)])
def test_lm_head_few_rows_k_segments(rows, d):
    """The few-row GEMM over K: one X segment (K = 1024 at <= 16 rows), several,
    K that is a multiple of 512 but not of 1024 (the 16-row tile falls back to
    reading X from L2, the 32-row tile keeps 512-deep segments), and K that is
    neither (both fall back), with a ragged vocabulary; every row against the
    oracle."""
    rng = np.random.default_rng(rows * 31 + d)
    V = 5003
    h = synth.to_bf16_bits(rng.standard_normal((rows, d)).astype(np.float32))
    w = synth.to_bf16_bits((rng.standard_normal((V, d)) * 0.02).astype(np.float32))
    prob = lib.make_problem(1, 0, d // 64, d // 64, 64, V, lib.SV_BF16, 1, 1)
    out = torch.full((rows, V), float("nan"), device="cuda")
    lib.sv_lm_head(prob, rows, torch.from_numpy(h.view(np.int16)).cuda(),
                   torch.from_numpy(w.view(np.int16)).cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    ref = ov.lm_head(synth.widen(h, "bf16"), synth.widen(w, "bf16"))
    err = np.abs(got - ref).max()
    print(f"rows {rows} d {d}: max |logit err| = {err:.3e}", flush=True)
    assert err <= TOL_LOGIT


@pytest.mark.parametrize("rows,d", [(700, 4096), (1952, 4096), (520, 8192)])
def test_lm_head_long_k_many_rows(rows, d):
    """Many K slabs through the batched-row GEMM path (its slab pipeline runs
    64-128 slabs here), against the oracle on every row."""
    rng = np.random.default_rng(rows + d)
    V = 1500
    h = synth.to_bf16_bits(rng.standard_normal((rows, d)).astype(np.float32))
    w = synth.to_bf16_bits((rng.standard_normal((V, d)) * 0.02).astype(np.float32))
    prob = lib.make_problem(1, 0, d // 128, d // 128, 128, V, lib.SV_BF16, 1, 1)
    out = torch.full((rows, V), float("nan"), device="cuda")
    lib.sv_lm_head(prob, rows, torch.from_numpy(h.view(np.int16)).cuda(),
                   torch.from_numpy(w.view(np.int16)).cuda(), out)
    torch.cuda.synchronize()
    ref = ov.lm_head(synth.widen(h, "bf16"), synth.widen(w, "bf16"))
    err = np.abs(out.cpu().numpy() - ref).max()
    print(f"rows {rows} d {d}: max |logit err| = {err:.3e}", flush=True)
    assert err <= TOL_LOGIT
