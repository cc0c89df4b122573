"""The seeded input generator: shapes, tree properties, storage formats."""
import numpy as np
import pytest
import torch
from scipy import stats

from speculative_decoding_tree_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.0, -2.5, 1.00390625, 1.01171875]   # exact and tie cases
    ours = synth.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("depth,n", [(6, 60), (5, 26), (3, 10), (1, 4)])
def test_seeded_tree_properties(depth, n):
    for seed in range(20):
        rng = np.random.default_rng(seed)
        par = synth.seeded_tree(rng, n, depth)
        assert len(par) == n
        assert all(-1 <= p < j for j, p in enumerate(par))
        dep = []
        for j, p in enumerate(par):
            dep.append(1 if p < 0 else dep[p] + 1)
        assert max(dep) == depth
        assert dep == sorted(dep)              # breadth-first numbering
        assert synth.children_count(par).max() <= synth.SEEDED_BRANCHING


def test_workload_shapes_small():
    inp = synth.generate("chain_v1k", seed=0)
    wl = inp.workload
    assert inp.kv.shape == (128 + 4, 2, 4, 64) and inp.kv.dtype == np.float32
    assert inp.node_hidden.shape == (5, 256)
    assert inp.lm_head.shape == (1024, 256)
    assert inp.draft_logits.shape == (5, 1024)
    assert list(inp.parent) == [-1, 0, 1, 2]
    assert inp.uniforms.shape == (5,) and (inp.uniforms < 1).all() and (inp.uniforms >= 0).all()
    assert inp.kv_offset.tolist() == [0, 132]
    assert wl.rows == 5 and inp.max_children == 1
    # same seed, same inputs
    again = synth.generate("chain_v1k", seed=0)
    np.testing.assert_array_equal(inp.kv, again.kv)
    np.testing.assert_array_equal(inp.node_token, again.node_token)


def test_greedy_tokens_are_top_k_of_draft():
    wl = synth.workload("eagle1_7b_t0", vocab=512, n_q_heads=2, n_kv_heads=2, head_dim=64,
                        prefix=("fixed", 16))
    inp = synth.generate(wl, seed=3)
    zd = inp.draft_logits
    order = np.argsort(-zd[0], kind="stable")
    root_kids = [j for j, p in enumerate(inp.parent) if p == -1]
    assert [int(inp.node_token[j]) for j in root_kids] == order[:len(root_kids)].tolist()


def test_sampled_tokens_follow_draft_distribution():
    # Gumbel-max draws from softmax(z / T): chi-square on a tiny vocabulary
    wl = synth.workload("chain_v1k", vocab=8, n_nodes=1, head_dim=64, n_q_heads=1,
                        n_kv_heads=1, prefix=("fixed", 2), temperature=("all", 0.7),
                        draft=("normal", 1.0))
    rng = np.random.default_rng(1)
    z = rng.normal(0, 1, (2, 8)).astype(np.float32)
    counts = np.zeros(8)
    for _ in range(20000):
        counts[synth._draw_tokens(rng, z, np.array([-1]), 0.7)[0]] += 1
    p = np.exp(z[0].astype(np.float64) / 0.7)
    p /= p.sum()
    assert stats.chisquare(counts, p * counts.sum()).pvalue > 1e-3
    del wl


def test_ragged_prefixes_and_offsets():
    wl = synth.workload("batch32_8b", batch=4, vocab=256, n_q_heads=4, n_kv_heads=2,
                        head_dim=64, prefix=("uniform", 3, 40), n_nodes=7,
                        tree=("seeded", 3))
    inp = synth.generate(wl, seed=5)
    assert (inp.prefix_len >= 3).all() and (inp.prefix_len <= 40).all()
    np.testing.assert_array_equal(np.diff(inp.kv_offset), inp.prefix_len + 7)
    assert inp.kv.shape[0] == inp.kv_offset[-1]
    assert inp.kv.dtype == np.uint16
    assert inp.temperature.tolist() == [0.0, 0.0, 1.0, 1.0]


def test_replicate_rounds_shares_context_and_redraws_draws():
    wl = synth.workload("eagle1_7b_t1", vocab=300, n_q_heads=2, n_kv_heads=2, head_dim=64,
                        prefix=("fixed", 12))
    base = synth.generate(wl, seed=1)
    rep = synth.replicate_rounds(base, 5, seed=2)
    R, N = wl.rows, wl.n_nodes
    assert rep.workload.batch == 5
    for c in range(5):
        np.testing.assert_array_equal(rep.kv[c * (12 + N):(c + 1) * (12 + N)], base.kv)
        np.testing.assert_array_equal(rep.node_hidden[c * R:(c + 1) * R], base.node_hidden)
        np.testing.assert_array_equal(rep.parent[c * N:(c + 1) * N], base.parent)
    assert len({tuple(rep.uniforms[c * R:(c + 1) * R]) for c in range(5)}) == 5
    np.testing.assert_array_equal(np.diff(rep.kv_offset), rep.prefix_len + N)
