"""GPU parity of spec_verify_tree against the tree oracle (reading R15).

Draft tokens of a tree come from the oracle's drafter: for a sampled tree every child
of node u is an independent inverse-CDF draw from q_u (its own draft coin); for a
greedy tree the children of u carry the top-k tokens of u's draft logits, in order.
Logits are compared with the logit tolerance; accepted depths, paths and emitted tokens
must match, except where the first differing decision is a near tie of a stated class
(|u - ratio| < 1e-4 for a candidate test, a top-1/top-2 gap below 1e-3 for an argmax,
the final coin within 1e-4 of a boundary of the oracle's CDF).  The tree path output
is then committed with spec_commit and checked against the commit oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from draft_block_verification_spec_amd import binding as bd
from draft_block_verification_spec_amd import workload as wl
from tests import parity as pt

pytestmark = pytest.mark.gpu


def _f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _draft_tokens(z_d, parent, coins, T):
    """[B, K] tokens: child c of node u ~ q_u (coin coins[c-1]), or u's top-k at T == 0."""
    B, K = parent.shape
    tok = np.zeros((B, K), np.int64)
    for b in range(B):
        rank = {}
        for j in range(K):
            u = int(parent[b, j])
            if T == 0.0:
                r = rank.get(u, 0)
                rank[u] = r + 1
                tok[b, j] = np.argsort(-z_d[b, u], kind="stable")[r]
            else:
                tok[b, j], _, _ = oracle.inverse_cdf(oracle.softmax_t(z_d[b, u], T), coins[b, j])
    return tok


def _case(wk, rep, kind, T):
    data = wl.generate(wk, rep)
    W = oracle.Weights.from_bits(data)
    B, K = wk.B, wk.K
    parent = wl.tree_parents(B, K, kind, seed=rep)
    h64 = oracle.from_bf16_bits(data["h"])
    hd64 = oracle.from_bf16_bits(data["h_draft"])
    z_t = oracle.lm_logits(W.w_lm, oracle.target_hidden(h64, W))
    z_d = oracle.lm_logits(W.w_lm, hd64)
    tokens = _draft_tokens(z_d, parent, data["draft_coins"].astype(np.float64), T)
    coins = data["coins"].astype(np.float64)
    if T == 0.0:
        ref = oracle.accept_tree_greedy(z_t, tokens, parent)
    else:
        ref = oracle.accept_tree_sample(oracle.softmax_t(z_t, T), oracle.softmax_t(z_d, T), tokens, parent, coins)
    ref["z_t"], ref["z_d"] = z_t, z_d
    return data, W, parent, tokens, coins, ref


def _first_diff(ref, b, parent, A_g, path_g, em_g, coins, T):
    """None when the first differing decision of request b is an allowed near tie."""
    A_o, path_o, em_o = int(ref["accepted"][b]), ref["path"][b], ref["emitted"][b]
    if A_g == A_o and np.array_equal(path_g[: A_g + 1], path_o[: A_o + 1]) and np.array_equal(
            em_g[: A_g + 1], em_o[: A_o + 1]):
        return None
    i = 1
    while i <= min(A_g, A_o) and path_g[i] == path_o[i]:
        i += 1
    same_path = A_g == A_o and i > A_o
    node = int(path_o[A_o]) if same_path else int(path_o[i - 1])
    if T == 0.0:
        z = ref["z_t"][b, node]
        top = np.sort(z)[-2:]
        return None if top[1] - top[0] < pt.GAP_BAND else f"request {b}: argmax path differs at node {node}"
    if not same_path:
        dec = [d for d in ref["decisions"][b] if d[0] >= 1 and parent[b, d[0] - 1] == node]
        if any(abs(c - min(1.0, r)) < pt.RATIO_BAND for _, r, c, _ in dec):
            return None
        return f"request {b}: candidate decision at node {node} differs (gpu depth {A_g}, oracle {A_o})"
    lo, hi = ref["cdf"][b]
    u = coins[b, -1]
    if min(abs(u - lo), abs(u - hi)) < pt.CDF_BAND:
        return None
    return f"request {b}: final token differs: gpu {em_g[A_g]} oracle {em_o[A_o]}"


def _run(wk, rep, kind, T):
    data, W, parent, tokens, coins, ref = _case(wk, rep, kind, T)
    w = pt.dev_weights(data)
    print(f"spec_verify_tree {wk.name} B={wk.B} K={wk.K} {kind} T={T}", flush=True)
    out = bd.spec_verify_tree(w, pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"]), _i32(tokens), _i32(parent),
                              _f32(coins), T, diag=True, logits=True)
    torch.cuda.synchronize()
    assert int(out.dev_status.item()) == 0
    B, K = wk.B, wk.K
    lg = out.logits.cpu().numpy()
    assert np.abs(lg[: B * (K + 1)] - ref["z_t"].reshape(B * (K + 1), -1)).max() <= pt.LOGIT_TOL
    if T > 0.0:
        assert np.abs(lg[B * (K + 1):] - ref["z_d"].reshape(B * K, -1)).max() <= pt.LOGIT_TOL
    acc, em, path = (x.cpu().numpy() for x in (out.accepted_len, out.emitted, out.path))
    bad = [m for b in range(B) if (m := _first_diff(ref, b, parent, int(acc[b]), path[b], em[b], coins, T))]
    assert not bad, bad
    for b in range(B):
        assert np.all(path[b, acc[b] + 1:] == -1) and np.all(em[b, acc[b] + 1:] == -1)
        assert all(parent[b, path[b, i] - 1] == path[b, i - 1] for i in range(1, acc[b] + 1))
    tau = float(out.tau.item())
    assert abs(tau - float(np.mean(acc + 1))) < 1e-6
    return out, data, parent, tokens, ref


TREE63 = wl.Workload("tree63", 93, B=2, K=63, d=64, d_ff=0, V=1000, T=1.0, sigma=0.4)


@pytest.mark.parametrize("T", [0.0, 1.0], ids=["greedy", "sample"])
@pytest.mark.parametrize("kind", ["random", "topk"])
# B = 12 (K = 7): 96 greedy / 180 sampled LM-head rows (128 x 128 and 192 x 192 tiles);
# B = 20: 160 / 300 rows (one and two row tiles of 160 x 256, four statistics slots per
# column tile); the largest tree the entry point takes (K = 63: 64 nodes).
@pytest.mark.parametrize("wk", [wl.SMALL, wl.SMALL_WIDE, wl.SMALL_BATCH.with_batch(12), wl.SMALL_BATCH.with_batch(20),
                                TREE63], ids=lambda w: f"{w.name}-b{w.B}")
def test_tree_reduced(wk, kind, T):
    _run(wk, 0, kind, T if T == 0.0 else wk.T)


@pytest.mark.parametrize("T", [0.0, 1.0], ids=["greedy", "sample"])
def test_tree_chain_matches_chain_entry_points(T):
    wk = wl.SMALL_BATCH.with_batch(12)
    out, data, parent, tokens, ref = _run(wk, 1, "chain", T)
    w = pt.dev_weights(data)
    if T == 0.0:
        c = bd.spec_verify_greedy(w, pt.dev_bf16(data["h"]), _i32(tokens))
    else:
        c = bd.spec_verify_sample(w, pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"]), _i32(tokens),
                                  _f32(data["coins"]), T)
    torch.cuda.synchronize()
    A = out.accepted_len.cpu().numpy()
    same = A == c.accepted_len.cpu().numpy()
    same &= np.all(out.emitted.cpu().numpy() == c.emitted.cpu().numpy(), axis=1)
    assert same.mean() >= 1.0 - 1.0 / wk.B, "chain trees differ from the chain entry points beyond one near tie"


@pytest.mark.parametrize("T", [0.0, 1.0], ids=["greedy", "sample"])
@pytest.mark.parametrize("rep", [0, 1])
def test_tree_block16_full(rep, T):
    """The 16-token block (d = 4096, d_ff = 12288, V = 151936) as a top-k tree of depth 3."""
    _run(wl.BLOCK16, rep, "topk", T)


def test_tree_bad_parent_and_token_flagged():
    wk = wl.SMALL.with_batch(3)
    data, W, parent, tokens, coins, ref = _case(wk, 2, "random", wk.T)
    parent = parent.copy()
    tokens = tokens.copy()
    parent[1, 2] = 3  # node 3's parent must be in 0..2
    tokens[2, 0] = wk.V
    out = bd.spec_verify_tree(pt.dev_weights(data), pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"]),
                              _i32(tokens), _i32(parent), _f32(coins), wk.T)
    torch.cuda.synchronize()
    acc = out.accepted_len.cpu().numpy()
    assert acc[1] == -1 and acc[2] == -1 and acc[0] >= 0
    assert int(out.dev_status.item()) in (bd.SV_DEV_BAD_TREE, bd.SV_DEV_BAD_TOKEN)
    assert np.all(out.path.cpu().numpy()[1:] == -1)


def test_tree_path_commits():
    """Tree verification then spec_commit with its path: the cache keeps the accepted path."""
    wk = wl.SMALL_BATCH.with_batch(12)
    out, data, parent, tokens, ref = _run(wk, 2, "topk", wk.T)
    B, K = wk.B, wk.K
    rng = np.random.default_rng(5)
    bs, eb, layers = 4, 32, 2
    max_blocks = 12
    seq = rng.integers(0, 20, size=B).astype(np.int32)
    nblk = B * max_blocks
    table = rng.permutation(nblk).reshape(B, max_blocks).astype(np.int32)
    kv = rng.integers(0, 256, size=(layers, 2, nblk, bs, eb), dtype=np.uint8)
    rs = rng.integers(0, 256, size=(B, 64), dtype=np.uint8)
    sn = rng.integers(0, 256, size=(B, K + 1, 64), dtype=np.uint8)
    acc, path = out.accepted_len.cpu().numpy(), out.path.cpu().numpy()
    kv_e, L_e, st_e = oracle.commit(kv, seq, table, acc, np.full(B, K), rs, sn, np.where(path < 0, 0, path))
    kv_d, seq_d, rs_d = torch.from_numpy(kv).cuda(), _i32(seq), torch.from_numpy(rs).cuda()
    bd.spec_commit(out.accepted_len, seq_d, Kmax=K, kv=kv_d, block_table=_i32(table), rec_state=rs_d,
                   rec_snap=torch.from_numpy(sn).cuda(), path=out.path)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(seq_d.cpu().numpy(), L_e)
    assert np.array_equal(kv_d.cpu().numpy(), kv_e) and np.array_equal(rs_d.cpu().numpy(), st_e)


def test_tree_meeting_timeout_is_reported():
    """With the blocks' wait bound set to zero polls every meeting of a sampled tree fails:
    the requests are flagged with SV_DEV_TIMEOUT and their outputs are -1 (no hang)."""
    wk = wl.SMALL.with_batch(3)
    data, W, parent, tokens, coins, ref = _case(wk, 3, "topk", wk.T)
    args = (pt.dev_weights(data), pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"]), _i32(tokens), _i32(parent),
            _f32(coins), wk.T)
    out = bd.spec_verify_tree(*args, wait_polls=0)
    torch.cuda.synchronize()
    acc = out.accepted_len.cpu().numpy()
    # a request whose walk needs no residual pass before its draw still meets once (the draw's pass)
    assert np.all(acc == -1)
    assert int(out.dev_status.item()) == bd.SV_DEV_TIMEOUT
    assert np.all(out.emitted.cpu().numpy() == -1)
    out = bd.spec_verify_tree(*args)
    torch.cuda.synchronize()
    assert int(out.dev_status.item()) == 0 and np.all(out.accepted_len.cpu().numpy() >= 0)


@pytest.mark.parametrize("T", [0.0, 1.0], ids=["greedy", "sample"])
def test_tree_without_drafts(T):
    """K = 0: the tree is its root; greedy emits the argmax, sampling draws from p."""
    wk = wl.SMALL.with_batch(4)
    data = wl.generate(wk, 5)
    W = oracle.Weights.from_bits(data)
    h = data["h"][:, :1]
    coins = data["coins"][:, -1:].astype(np.float64)
    z_t = oracle.lm_logits(W.w_lm, oracle.target_hidden(oracle.from_bf16_bits(h), W))
    empty = np.zeros((wk.B, 0), np.int64)
    if T == 0.0:
        ref = oracle.accept_tree_greedy(z_t, empty, empty)
    else:
        ref = oracle.accept_tree_sample(oracle.softmax_t(z_t, T), np.zeros((wk.B, 0, wk.V)), empty, empty, coins)
    out = bd.spec_verify_tree(pt.dev_weights(data), pt.dev_bf16(h), pt.dev_bf16(data["h_draft"][:, :0]),
                              torch.zeros(wk.B, 0, dtype=torch.int32, device="cuda"),
                              torch.zeros(wk.B, 0, dtype=torch.int32, device="cuda"), _f32(coins), T)
    torch.cuda.synchronize()
    assert int(out.dev_status.item()) == 0
    np.testing.assert_array_equal(out.accepted_len.cpu().numpy(), 0)
    em = out.emitted.cpu().numpy()[:, 0]
    for b in range(wk.B):
        if em[b] != ref["emitted"][b, 0]:
            if T == 0.0:
                top = np.sort(z_t[b, 0])[-2:]
                assert top[1] - top[0] < pt.GAP_BAND
            else:
                lo, hi = ref["cdf"][b]
                assert min(abs(coins[b, 0] - lo), abs(coins[b, 0] - hi)) < pt.CDF_BAND
