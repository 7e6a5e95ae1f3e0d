"""Pins of the tree-verification oracle (reading R15).

* A chain-shaped tree gives exactly the chain rules (a separate, vectorised code path).
* Sampled trees are lossless: over many random trees with several candidates per node,
  the first emitted token follows p at the root and the second, after an accepted draft
  x1, follows the target distribution after x1 (chi-square, alpha = 0.01 with a
  Bonferroni split).  A planted mistake (no residual update after a rejected
  candidate) must fail the same test.
* Greedy trees emit the longest root path whose tokens are the target argmaxes.
"""
import numpy as np
import pytest
from scipy import stats

import oracle
import oracle.tree as otree


def _dirichlet(rng, shape, V, a=1.0):
    x = rng.gamma(a, size=shape + (V,))
    return x / x.sum(-1, keepdims=True)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_chain_tree_is_the_chain_rule(seed):
    rng = np.random.default_rng(seed)
    B, K, V = 40, 5, 7
    p = _dirichlet(rng, (B, K + 1), V)
    q = _dirichlet(rng, (B, K), V)
    draft = np.array([[rng.choice(V, p=q[b, j]) for j in range(K)] for b in range(B)])
    coins = rng.random((B, K + 1))
    parent = np.tile(np.arange(K), (B, 1))  # node j+1's parent is node j
    t = oracle.accept_tree_sample(p, q, draft, parent, coins)
    c = oracle.accept_sample(p, q, draft, coins)
    np.testing.assert_array_equal(t["accepted"], c["accepted"])
    np.testing.assert_array_equal(t["emitted"], c["emitted"])
    z = rng.standard_normal((B, K + 1, V))
    draft_g = np.where(rng.random((B, K)) < 0.7, z[:, :K].argmax(-1), rng.integers(0, V, (B, K)))
    tg = oracle.accept_tree_greedy(z, draft_g, parent)
    cg = oracle.accept_greedy(z, draft_g)
    np.testing.assert_array_equal(tg["accepted"], cg["accepted"])
    np.testing.assert_array_equal(tg["emitted"], cg["emitted"])


# tree: root with 3 candidates, each with 2 candidates of its own (N = 10 nodes)
_PARENT = np.array([0, 0, 0, 1, 1, 2, 2, 3, 3])
_DEPTH1 = [1, 2, 3]


def _law_trials(n, seed):
    rng = np.random.default_rng(seed)
    V, N = 5, 10
    p_root = np.array([0.5, 0.2, 0.15, 0.1, 0.05])
    q_root = np.array([0.1, 0.15, 0.2, 0.25, 0.3])
    p_child = _dirichlet(np.random.default_rng(99), (V,), V)      # target after token x1
    q_child = _dirichlet(np.random.default_rng(98), (V,), V)      # drafter after token x1
    p = np.empty((n, N, V))
    q = np.empty((n, N - 1, V))
    tokens = np.empty((n, N - 1), np.int64)
    cum_root = np.cumsum(q_root)
    t1 = np.minimum(np.searchsorted(cum_root, rng.random((n, 3)), side="right"), V - 1)
    p[:, 0], q[:, 0] = p_root, q_root
    tokens[:, 0:3] = t1
    for i, node in enumerate(_DEPTH1):
        x1 = t1[:, i]
        p[:, node], q[:, node] = p_child[x1], q_child[x1]
        cq = np.cumsum(q_child[x1], axis=-1)
        for k, leaf in enumerate((4 + 2 * i, 5 + 2 * i)):
            x2 = np.minimum((cq < rng.random((n, 1))).sum(-1), V - 1)
            tokens[:, leaf - 1] = x2
            p[:, leaf] = _dirichlet(rng, (n,), V)  # target at depth 2 (bonus only)
            if leaf < N - 1:
                q[:, leaf] = q_root
    parent = np.tile(_PARENT, (n, 1))
    coins = rng.random((n, N))
    return oracle.accept_tree_sample(p, q, tokens, parent, coins), p_root, p_child


def _chi2_ok(counts, probs, alpha):
    n = counts.sum()
    return stats.chisquare(counts, n * probs).pvalue > alpha


def _lossless(n=60000, seed=5):
    out, p_root, p_child = _law_trials(n, seed)
    em, acc = out["emitted"], out["accepted"]
    V = len(p_root)
    tests = [(np.bincount(em[:, 0], minlength=V), p_root)]
    for x1 in range(V):
        sel = (acc >= 1) & (em[:, 0] == x1)
        if sel.sum() > 2000:
            tests.append((np.bincount(em[sel, 1], minlength=V), p_child[x1]))
    alpha = 0.01 / len(tests)
    return all(_chi2_ok(c, pr, alpha) for c, pr in tests), out


def test_sampled_tree_is_lossless():
    ok, out = _lossless()
    assert ok
    assert 0.2 < (out["accepted"] >= 1).mean() < 0.95 and (out["accepted"] == 2).mean() > 0.05


def test_tree_without_residual_update_is_caught(monkeypatch):
    monkeypatch.setattr(otree, "next_residual", lambda r, q_u, p_u: (p_u.copy(), False))
    ok, _ = _lossless(n=30000)
    assert not ok


def test_greedy_tree_follows_the_argmax_path():
    rng = np.random.default_rng(3)
    B, N, V = 50, 12, 6
    z = rng.standard_normal((B, N, V))
    amax = z.argmax(-1)
    parent = np.array([[rng.integers(j) for j in range(1, N)] for _ in range(B)])
    # half the candidates carry the argmax of their parent
    tokens = np.where(rng.random((B, N - 1)) < 0.5, amax[np.arange(B)[:, None], parent], rng.integers(0, V, (B, N - 1)))
    out = oracle.accept_tree_greedy(z, tokens, parent)
    for b in range(B):
        ch = oracle.tree_children(parent[b], N)
        node, seq = 0, []
        while True:  # brute force: the lowest-index matching child at every level
            m = [c for c in ch[node] if tokens[b, c - 1] == amax[b, node]]
            if not m:
                seq.append(amax[b, node])
                break
            seq.append(tokens[b, m[0] - 1])
            node = m[0]
        A = len(seq) - 1
        assert out["accepted"][b] == A
        np.testing.assert_array_equal(out["emitted"][b, : A + 1], seq)
        assert all(out["emitted"][b, i] == amax[b, out["path"][b, i]] for i in range(A + 1))
