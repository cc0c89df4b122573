"""GPU edge cases and the statistical test of the sampling kernel."""
import numpy as np
import pytest
import torch
from scipy import stats

from oracle import verify as ov
from speculative_decoding_tree_amd import lib, synth
from speculative_decoding_tree_amd.runner import DeviceBatch

from parity_util import compare_rounds, compare_rounds_e2e, logit_delta, widened

pytestmark = pytest.mark.gpu

BASE = synth.Workload(
    name="edge", batch=2, n_nodes=6, n_q_heads=4, n_kv_heads=2, head_dim=128, vocab=700,
    dtype=synth.BF16, prefix=("list", (5, 130)), tree=("seeded", 3), w_std=0.1,
    draft=("perturbed", 0.7), temperature=("list", (0.0, 1.0)))


def _verify(inp, mutate=None, max_prefix=None):
    db = DeviceBatch.create(inp, max_prefix=max_prefix)
    if mutate:
        mutate(db.t)
    d = db.debug_buffers()
    db.verify(dbg={"logits": d["logits"]})
    torch.cuda.synchronize()
    res = db.results()
    res["logits"] = d["logits"].cpu().numpy()
    return res


def _oracle(inp):
    W = inp.workload
    w = widened(inp)
    return ov.verify_batch(w["node_hidden"], w["kv"], inp.kv_offset, inp.prefix_len, inp.parent,
                           inp.node_token, w["lm_head"], inp.draft_logits, inp.uniforms,
                           inp.temperature, W.n_nodes, W.n_q_heads, W.n_kv_heads, W.head_dim)


def _assert_parity(inp, res):
    """Rounds against the fp64 oracle, with exclusion windows from the measured
    logit error of each sequence."""
    ref = _oracle(inp)
    W = inp.workload
    R = W.rows
    deltas = [logit_delta(res["logits"][b * R:(b + 1) * R], ref.logits[b * R:(b + 1) * R])
              for b in range(W.batch)]
    _, _, _, bad = compare_rounds_e2e(ref.rounds, inp.temperature, res["accept_len"],
                                      res["accept_path"], res["out_tokens"], W.n_nodes, deltas,
                                      ref.logits, inp.draft_logits, inp.node_token)
    assert not bad, bad
    return ref


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_no_nodes(T):
    wl = BASE.with_(n_nodes=0, tree=("chain",), temperature=("all", T))
    inp = synth.generate(wl, seed=1)
    res = _verify(inp)
    _assert_parity(inp, res)
    assert (res["accept_len"] == 0).all()


@pytest.mark.parametrize("tree", [("chain",), ("star",)])
def test_sixty_four_nodes(tree):
    wl = BASE.with_(n_nodes=64, tree=tree, temperature=("list", (0.0, 0.9)),
                    draft=("perturbed", 0.05))
    inp = synth.generate(wl, seed=2)
    res = _verify(inp)
    _assert_parity(inp, res)
    assert (res["seq_status"] & lib.SEQ_ERR_MASK == 0).all()


@pytest.mark.parametrize("V", [1, 3, 4096, 4097, 9000])
def test_vocab_sizes(V):
    wl = BASE.with_(vocab=V, n_nodes=min(6, V) if V > 1 else 2,
                    tree=("seeded", 2) if V > 1 else ("chain",))
    inp = synth.generate(wl, seed=3)
    res = _verify(inp)
    _assert_parity(inp, res)


def test_bad_tree_token_temperature_prefix_are_per_sequence():
    wl = BASE.with_(batch=5, prefix=("list", (5, 9, 30, 64, 100)),
                    temperature=("list", (1.0, 1.0, 1.0, 1.0, 0.0)))
    inp = synth.generate(wl, seed=4)
    N = wl.n_nodes

    def mutate(t):
        par = t["parent"].clone()
        par[1 * N + 3] = 5                        # seq 1: parent[3] >= 3
        t["parent"].copy_(par)
        tok = t["node_token"].clone()
        tok[2 * N + 1] = wl.vocab                 # seq 2: token out of range
        t["node_token"].copy_(tok)
        temp = t["temperature"].clone()
        temp[3] = -1.0                            # seq 3: negative temperature
        t["temperature"].copy_(temp)

    res = _verify(inp, mutate, max_prefix=99)     # seq 4: L = 100 > max_prefix
    st = res["seq_status"]
    assert st[0] == 0
    assert st[1] & lib.SEQ_ERR_TREE
    assert st[2] & lib.SEQ_ERR_TOKEN
    assert st[3] & lib.SEQ_ERR_TEMPERATURE
    assert st[4] & lib.SEQ_ERR_PREFIX
    assert (res["accept_len"][1:] == -1).all()
    R = wl.rows
    assert (res["out_tokens"][R:] == -1).all()
    assert (res["attn_out"][R:] == 0).all()
    # the healthy sequence is unaffected
    good = synth.generate(wl.with_(batch=1, prefix=("list", (5,)), temperature=("all", 1.0)),
                          seed=4)
    assert res["accept_len"][0] >= 0
    del good


def test_uniform_out_of_range_is_clamped_and_flagged():
    inp = synth.generate(BASE, seed=5)
    R = BASE.rows

    def mutate(t):
        u = t["uniforms"].clone()
        u[R + BASE.n_nodes] = 1.5                 # seq 1 (T = 1): final uniform
        t["uniforms"].copy_(u)

    res = _verify(inp, mutate)
    assert res["seq_status"][1] & lib.SEQ_WARN_UNIFORM
    assert res["accept_len"][1] >= 0


def test_nonfinite_logits_flagged():
    inp = synth.generate(BASE.with_(temperature=("all", 1.0)), seed=6)
    inp.draft_logits[0, 3] = np.nan               # seq 0 root draft row (root has children)
    res = _verify(inp)
    assert res["seq_status"][0] & lib.SEQ_ERR_NONFINITE
    assert res["accept_len"][0] == -1
    assert res["seq_status"][1] & lib.SEQ_ERR_MASK == 0


def test_sampling_distribution_chi_square_and_bitwise_agreement():
    """Many independent rounds in one launch: V = 32, four candidates at the
    root, depth 2, fixed target/draft rows; the first emitted token must
    follow the root target distribution, and every non-excluded round must
    match the oracle exactly."""
    rng = np.random.default_rng(77)
    V, T = 32, 1.0
    parent1 = np.array([-1, -1, -1, -1, 0, 0, 1, 2], dtype=np.int32)
    N = len(parent1)
    R = N + 1
    B = 7000
    zt = rng.normal(0, 1.0, (R, V)).astype(np.float32)
    zd = (zt + rng.normal(0, 1.0, (R, V))).astype(np.float32)
    q = [np.exp(zd[s].astype(np.float64) / T) for s in range(R)]
    q = [x / x.sum() for x in q]
    tokens = np.empty((B, N), dtype=np.int32)
    for j in range(N):
        tokens[:, j] = rng.choice(V, size=B, p=q[parent1[j] + 1])
    uniforms = rng.random((B, R), dtype=np.float32)
    logits = np.tile(zt, (B, 1))
    draft = np.tile(zd, (B, 1))
    parent = np.tile(parent1, B)
    prob = lib.make_problem(B, N, 2, 2, 128, V, lib.SV_BF16, 1, 4)
    ws = torch.empty(lib.sv_workspace_size(prob), dtype=torch.uint8, device="cuda")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    acc_len = torch.empty(B, dtype=torch.int32, device="cuda")
    acc_path = torch.empty(B * N, dtype=torch.int32, device="cuda")
    out_tok = torch.empty(B * R, dtype=torch.int32, device="cuda")
    status = torch.empty(B, dtype=torch.int32, device="cuda")
    lib.sv_sample(prob, dev(parent), dev(tokens.reshape(-1)), dev(logits), dev(draft),
                  dev(uniforms.reshape(-1)), dev(np.full(B, T, np.float32)), acc_len, acc_path,
                  out_tok, status, workspace=ws)
    torch.cuda.synchronize()
    out_tok = out_tok.cpu().numpy()
    first = out_tok.reshape(B, R)[:, 0]
    counts = np.bincount(first, minlength=V).astype(np.float64)
    p = np.exp(zt[0].astype(np.float64) / T)
    p /= p.sum()
    exp = p * B
    order = np.argsort(exp)
    obs_p, exp_p, ao, ae = [], [], 0.0, 0.0
    for i in order:
        ao += counts[i]
        ae += exp[i]
        if ae >= 5:
            obs_p.append(ao)
            exp_p.append(ae)
            ao = ae = 0.0
    if ae > 0:
        obs_p[-1] += ao
        exp_p[-1] += ae
    pval = stats.chisquare(obs_p, exp_p).pvalue
    print(f"chi-square p-value {pval:.4f}", flush=True)
    assert pval >= 1e-3
    rounds, _, _, _ = ov.sample_batch(logits.astype(np.float64), draft.astype(np.float64), parent,
                                      tokens.reshape(-1), uniforms.reshape(-1),
                                      np.full(B, T), N)
    npath, nfin, excl, bad = compare_rounds(rounds, np.full(B, T), acc_len.cpu().numpy(),
                                            acc_path.cpu().numpy(), out_tok, N)
    print(f"paths {npath} final tokens {nfin} excluded {excl}", flush=True)
    assert not bad, bad[:3]
    assert npath > 0.99 * B and nfin > 0.95 * B
