"""Pins of the commit oracle (reading R14) against sequential decoding of a toy target.

Whatever the acceptance decided, the cache and the recurrent state after a commit must
be those of feeding the committed tokens one at a time.  Steps without a draft are mixed
with steps with one, the case the hybrid-model engine got wrong ([WB] n-gram pitfalls).
Mistakes planted in the oracle's output (one input too many or too few, a chain commit
applied to a tree) must fail the same check.
"""
import numpy as np
import pytest

import oracle
from tests.commit_session import Session, ToyTarget


def _run(tree, steps=14, seed=3, mutate=None, Kmax=5):
    s = Session(ToyTarget(seed=seed), Kmax=Kmax, seed=seed + 1)
    rng = np.random.default_rng(seed + 2)
    for it in range(steps):
        # every other step has no draft for some requests (k = 0)
        k = rng.integers(0, Kmax + 1, size=s.B)
        if it % 2 == 1:
            k[rng.random(s.B) < 0.6] = 0
        tokens, parent, depth, snap = s.verify_pass(k, tree=tree)
        A, path = s.accept(k, parent, tree=tree)
        kv, L, st = oracle.commit(s.kv, s.seq_len, s.block_table, A, k, s.state, snap, path if tree else None)
        if mutate is not None:
            kv, L, st = mutate(kv, L, st, s, A, k, snap, path)
        s.apply(kv, L, st, tokens, A, path)
        s.check()
    return s


@pytest.mark.parametrize("tree", [False, True], ids=["chain", "tree"])
def test_commit_matches_sequential_decoding(tree):
    s = _run(tree)
    assert min(len(c) for c in s.committed) > 10


def test_no_draft_steps_alternating():
    """Steps alternate between no draft and a full draft block, all accepted or none."""
    s = Session(ToyTarget(seed=9), Kmax=4, seed=10)
    for it in range(10):
        k = np.full(s.B, 0 if it % 2 == 0 else 4)
        tokens, parent, depth, snap = s.verify_pass(k)
        A = np.array([0, 4, 2])[: s.B] if it % 2 else np.zeros(s.B, np.int64)
        path = np.tile(np.arange(5), (s.B, 1))
        kv, L, st = oracle.commit(s.kv, s.seq_len, s.block_table, A, k, s.state, snap)
        s.apply(kv, L, st, tokens, A, path)
        s.check()


def test_flagged_request_is_left_unchanged():
    s = Session(ToyTarget(seed=5), seed=6)
    k = np.array([3, 3, 3])
    tokens, parent, depth, snap = s.verify_pass(k)
    A = np.array([2, -1, 0])
    kv, L, st = oracle.commit(s.kv, s.seq_len, s.block_table, A, k, s.state, snap)
    assert L[1] == s.seq_len[1] and np.array_equal(st[1], s.state[1])
    assert L[0] == s.seq_len[0] + 3 and L[2] == s.seq_len[2] + 1


def _off_by_one_len(kv, L, st, s, A, k, snap, path):
    return kv, L - (A >= 0), st


def _state_one_late(kv, L, st, s, A, k, snap, path):
    st = st.copy()
    for b in range(s.B):
        if 0 <= A[b] < k[b]:
            st[b] = snap[b, A[b] + 1]
    return kv, L, st


def _chain_commit_on_tree(kv, L, st, s, A, k, snap, path):
    return oracle.commit(s.kv, s.seq_len, s.block_table, A, k, s.state, snap, None)


@pytest.mark.parametrize("mutate,tree", [(_off_by_one_len, False), (_state_one_late, False),
                                         (_chain_commit_on_tree, True)],
                         ids=["length-one-short", "state-one-input-late", "tree-without-compaction"])
def test_planted_commit_mistakes_are_caught(mutate, tree):
    with pytest.raises(AssertionError):
        _run(tree, mutate=mutate)
