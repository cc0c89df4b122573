"""The end-to-end exclusion windows of the GPU parity tests, checked on the
CPU: a walk run on logits perturbed by at most delta must agree with the
oracle's walk on every round the windows do not exclude, and the windows must
leave most rounds compared. The "GPU" here is the oracle itself on perturbed
logits, so a window that is too narrow shows up as a mismatch."""
import numpy as np
import pytest

from oracle import verify as ov

from parity_util import compare_rounds_e2e


def _tree(rng, n, max_kids=4):
    parent = []
    kids = {-1: 0}
    for j in range(n):
        while True:
            p = int(rng.integers(-1, j))
            if kids.get(p, 0) < max_kids:
                break
        kids[p] = kids.get(p, 0) + 1
        kids[j] = 0
        parent.append(p)
    return np.array(parent, dtype=np.int32)


def _draw_children(rng, zd, parent, T, distinct):
    """Drafted tokens: each slot's children drawn from q = softmax(zd/T),
    i.i.d. or without replacement."""
    N = len(parent)
    tok = np.zeros(N, dtype=np.int32)
    for s in range(N + 1):
        kids = [j for j in range(N) if parent[j] == s - 1]
        if not kids:
            continue
        q = ov.softmax_t(zd[s], T)
        if distinct:
            picks = rng.choice(len(q), size=len(kids), replace=False, p=q)
        else:
            picks = rng.choice(len(q), size=len(kids), replace=True, p=q)
        tok[kids] = picks
    return tok


@pytest.mark.parametrize("delta", [2e-5, 3e-4])
@pytest.mark.parametrize("draft,distinct,T", [("perturbed", False, 1.0), ("independent", False, 1.0),
                                              ("perturbed", True, 0.7), ("independent", False, 0.0)])
def test_windows_hold_under_bounded_logit_error(draft, distinct, T, delta):
    """No mismatch at any delta; at a delta a few times the GPU's measured
    one (about 1e-5 at K = 4096), most paths and finals stay compared."""
    rng = np.random.default_rng(17)
    B, N, V = 48, 12, 1500
    R = N + 1
    zt = rng.normal(0, 1.5, (B * R, V))
    zd = zt + rng.normal(0, 0.5, zt.shape) if draft == "perturbed" else rng.normal(0, 2, zt.shape)
    parent = np.concatenate([_tree(rng, N) for _ in range(B)])
    tokens = np.concatenate([_draw_children(rng, zd[b * R:(b + 1) * R], parent[b * N:(b + 1) * N],
                                            T if T > 0 else 1.0, distinct) for b in range(B)])
    u = rng.random(B * R)
    temp = np.full(B, T)
    ref, _, _, _ = ov.sample_batch(zt, zd, parent, tokens, u, temp, N, distinct)
    z_gpu = zt + rng.uniform(-delta, delta, zt.shape)
    _, g_len, g_path, g_tok = ov.sample_batch(z_gpu, zd, parent, tokens, u, temp, N, distinct)
    deltas = [float(np.abs(z_gpu[b * R:(b + 1) * R] - zt[b * R:(b + 1) * R]).max())
              for b in range(B)]
    npath, nfin, excl, bad = compare_rounds_e2e(ref, temp, g_len, g_path, g_tok, N, deltas, zt,
                                                zd, tokens, distinct)
    assert not bad, bad[:3]
    if delta <= 2e-5:
        assert npath >= 0.8 * B, (npath, excl)
        if T > 0:
            assert nfin >= 0.3 * B, nfin


def test_windows_catch_a_larger_error():
    """Logits moved by far more than the delta the windows are given: some
    compared round disagrees (so the comparison is not vacuous)."""
    rng = np.random.default_rng(18)
    B, N, V = 64, 8, 400
    R = N + 1
    zt = rng.normal(0, 1.5, (B * R, V))
    zd = zt + rng.normal(0, 0.5, zt.shape)
    parent = np.concatenate([_tree(rng, N) for _ in range(B)])
    tokens = np.concatenate([_draw_children(rng, zd[b * R:(b + 1) * R], parent[b * N:(b + 1) * N],
                                            1.0, False) for b in range(B)])
    u = rng.random(B * R)
    temp = np.ones(B)
    ref, _, _, _ = ov.sample_batch(zt, zd, parent, tokens, u, temp, N)
    z_gpu = zt + rng.normal(0, 0.3, zt.shape)
    _, g_len, g_path, g_tok = ov.sample_batch(z_gpu, zd, parent, tokens, u, temp, N)
    _, _, _, bad = compare_rounds_e2e(ref, temp, g_len, g_path, g_tok, N, [1e-6] * B, zt, zd,
                                      tokens)
    assert bad
