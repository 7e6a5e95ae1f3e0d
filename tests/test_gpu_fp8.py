"""GPU parity with FP8 weights (reading R13: E4M3 codes, one fp32 scale per output row).

The oracle decodes the same codes exactly and multiplies by the row scales
(``oracle.Weights.from_fp8``); the library streams the codes, converts them to bf16
MFMA operands and scales each output row after the reduction.  Shapes: the full
16-token block (whole 4096-value chunks of K) and reduced shapes whose K is not a
multiple of 4096 (the general streaming path), all within the rows the
weight-streaming kernel takes.
"""
import numpy as np
import pytest
import torch

import oracle
from draft_block_verification_spec_amd import binding as bd
from draft_block_verification_spec_amd import workload as wl
from tests import parity as pt
from tests.test_gpu_parity import ODD, _run_greedy, _run_sample

pytestmark = pytest.mark.gpu

# reduced shapes with at most 16 target rows (MLP) and 32 LM-head rows; the last has
# d = 192 and d_ff = 576 (6 and 18 k-steps of 32 on the general path) and an odd V
SMALL8 = [wl.SMALL.with_batch(2), wl.SMALL_WIDE.with_batch(3), wl.TINY.with_batch(3), ODD.with_batch(2)]


@pytest.mark.parametrize("wk", SMALL8, ids=lambda w: f"{w.name}-B{w.B}")
def test_fp8_sample_reduced(wk):
    _run_sample(wk, fp8=True)


@pytest.mark.parametrize("wk", SMALL8, ids=lambda w: f"{w.name}-B{w.B}")
def test_fp8_greedy_reduced(wk):
    _run_greedy(wk, fp8=True)


@pytest.mark.parametrize("rep", [0, 1])
def test_fp8_block16_sample(rep):
    _run_sample(wl.BLOCK16, rep, fp8=True)


def test_fp8_block16_greedy():
    _run_greedy(wl.BLOCK16, fp8=True)


def test_fp8_propose_matches_oracle_drafter():
    """The drafter step with FP8 weights: argmax drafts and conf = 1 at T = 0; inverse-CDF
    drafts and top-1 probabilities at the workload's temperature."""
    wk = wl.BLOCK16
    data = wl.to_fp8(wl.generate(wk))
    W = oracle.Weights.from_fp8(data)
    w = pt.dev_fp8_weights(data)
    hd = pt.dev_bf16(data["h_draft"])
    coins = torch.from_numpy(data["draft_coins"].astype(np.float32)).cuda()
    for T in (wk.T, 0.0):
        ref = pt.oracle_drafts(W, data, T)
        x, conf = bd.spec_draft_propose(w, hd, coins, T)
        torch.cuda.synchronize()
        x = x.cpu().numpy()
        conf = conf.cpu().numpy()
        z = ref["logits"]
        if T == 0.0:
            sure = oracle.row_stats(z)["gap"] >= pt.GAP_BAND
            np.testing.assert_array_equal(x[sure], ref["draft"][sure])
            np.testing.assert_array_equal(conf, np.ones_like(conf))
        else:
            C = np.cumsum(oracle.softmax_t(z, T), axis=-1)
            u = data["draft_coins"].astype(np.float64)
            for idx in zip(*np.nonzero(x != ref["draft"])):
                assert np.min(np.abs(C[idx] - u[idx])) < pt.CDF_BAND, f"draft token differs at {idx}"
            np.testing.assert_allclose(conf, ref["conf"], atol=pt.PROB_TOL)


def test_fp8_rejects_batches_past_the_streaming_kernel():
    """FP8 weights on a batch whose products would not stream (64 target rows): invalid."""
    wk = wl.SMALL.with_batch(8)
    data = wl.to_fp8(wl.generate(wk))
    w = pt.dev_fp8_weights(data)
    draft = torch.zeros(wk.B, wk.K, dtype=torch.int32, device="cuda")
    with pytest.raises(bd.SpecVerifyError):
        bd.spec_verify_greedy(w, pt.dev_bf16(data["h"]), draft)


@pytest.mark.parametrize("T", [0.0, 1.0], ids=["greedy", "sample"])
def test_fp8_tree_block16(T):
    """Tree verification with FP8 weights: the 16-token block as a top-k tree.  Greedy: the
    children of a node are its best draft tokens in rank order.  Sampled: every child is drawn
    from its parent's q with its own coin (the rule is lossless for such children)."""
    wk = wl.BLOCK16
    data = wl.to_fp8(wl.generate(wk, 1))
    W = oracle.Weights.from_fp8(data)
    w = pt.dev_fp8_weights(data)
    parent = wl.tree_parents(wk.B, wk.K, "topk")
    hd64 = oracle.from_bf16_bits(data["h_draft"])
    z_t = oracle.lm_logits(W.w_lm, oracle.target_hidden(oracle.from_bf16_bits(data["h"]), W))
    z_d = oracle.lm_logits(W.w_lm, hd64)
    coins = data["coins"].astype(np.float64)
    tok = np.zeros((wk.B, wk.K), np.int64)
    if T == 0.0:
        for j in range(wk.K):  # child j+1 of node u: u's (rank)-th best draft token
            u = int(parent[0, j])
            r = int(np.sum(parent[0, :j] == u))
            tok[0, j] = np.argsort(-z_d[0, u], kind="stable")[r]
    else:
        q_par = oracle.softmax_t(z_d[0, parent[0]], T)  # [K, V]: q of each child's parent
        tok[0] = oracle.inverse_cdf(q_par, data["draft_coins"][0].astype(np.float64))[0]
    if T == 0.0:
        ref = oracle.accept_tree_greedy(z_t, tok, parent)
    else:
        ref = oracle.accept_tree_sample(oracle.softmax_t(z_t, T), oracle.softmax_t(z_d, T), tok, parent, coins)
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    out = bd.spec_verify_tree(w, pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"]), i32(tok), i32(parent),
                              torch.from_numpy(coins.astype(np.float32)).cuda(), T, logits=True)
    torch.cuda.synchronize()
    assert int(out.dev_status.item()) == 0
    lg = out.logits.cpu().numpy()
    assert np.abs(lg[: wk.K + 1] - z_t[0]).max() <= pt.LOGIT_TOL
    A = int(out.accepted_len.item())
    path, em = out.path.cpu().numpy()[0], out.emitted.cpu().numpy()[0]
    if A == ref["accepted"][0] and np.array_equal(em[: A + 1], ref["emitted"][0, : A + 1]):
        return
    # a difference must come from a near tie of a stated class
    if T == 0.0:
        node = int(ref["path"][0, min(A, int(ref["accepted"][0]))])
        top = np.sort(z_t[0, node])[-2:]
        assert top[1] - top[0] < pt.GAP_BAND
    else:
        near = [abs(c - min(1.0, r)) < pt.RATIO_BAND for _, r, c, _ in ref["decisions"][0]]
        lo, hi = ref["cdf"][0]
        assert any(near) or min(abs(coins[0, -1] - lo), abs(coins[0, -1] - hi)) < pt.CDF_BAND
