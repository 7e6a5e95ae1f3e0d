"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The oracle recomputes every output it can afford: all rows of the B=1 block, every draft
row and every request of the scheduled batches (their schedule is the oracle's own, from
its own confidences), and a sample of the requests of the other batched shapes (requests
are independent, so a request's rows can be checked one by one).
"""
import numpy as np
import pytest
import torch

import oracle
from draft_block_verification_spec_amd import binding as bd
from draft_block_verification_spec_amd import workload as wl
from tests import parity as pt
from tests.test_gpu_parity import _final_rows, _schedule_agrees

pytestmark = pytest.mark.gpu


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


_cache = {}


def _setup(wk, rep=0):
    key = (wk.name, wk.B, rep)
    if key not in _cache:
        _cache.clear()
        data = wl.generate(wk, rep)
        W = oracle.Weights.from_bits(data)
        _cache[key] = (data, W, pt.dev_weights(data))
    return _cache[key]


def _check_rows(lg_gpu, ref_rows):
    err = np.abs(lg_gpu.astype(np.float64) - ref_rows).max()
    assert err <= pt.LOGIT_TOL, f"logit error {err}"
    return err


@pytest.mark.parametrize("rep", [0, 1])
def test_block16_sample_full(rep):
    wk = wl.BLOCK16
    data, W, w = _setup(wk, rep)
    h64, hd64 = oracle.from_bf16_bits(data["h"]), oracle.from_bf16_bits(data["h_draft"])
    draft = oracle.propose(W, hd64, wk.T, data["draft_coins"])["draft"]
    coins = data["coins"].astype(np.float64)
    ref = oracle.verify_sample(W, h64, hd64, draft, coins, wk.T)
    out = bd.spec_verify_sample(w, pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"]), _i32(draft),
                                _f32(data["coins"]), wk.T, diag=True, logits=True)
    torch.cuda.synchronize()
    assert int(out.dev_status.item()) == 0
    V = wk.V
    _check_rows(out.logits.cpu().numpy(),
                np.concatenate([ref["logits_t"].reshape(-1, V), ref["logits_d"].reshape(-1, V)]))
    dg = out.diag.cpu().numpy().astype(np.float64)
    K = wk.K
    assert np.abs(dg[:K, 5] - ref["p_x"][0]).max() <= pt.PROB_TOL
    assert np.abs(dg[K + 1:, 5] - ref["q_x"][0]).max() <= pt.PROB_TOL
    acc, em = out.accepted_len.cpu().numpy(), out.emitted.cpu().numpy()
    pt.count_bands(ref, coins, "sample")
    lg = out.logits.cpu().numpy()
    rows = _final_rows(lg, wk.B, K, wk.T)
    pt.assert_decisions(ref, acc, em, lambda b: pt.first_diff_sample(ref, int(acc[b]), em[b], b, coins, K, rows(b, K)),
                        "block16 sample")


@pytest.mark.parametrize("rep", [0, 1])
def test_block16_greedy_full(rep):
    wk = wl.BLOCK16
    data, W, w = _setup(wk, rep)
    h64, hd64 = oracle.from_bf16_bits(data["h"]), oracle.from_bf16_bits(data["h_draft"])
    draft = oracle.propose(W, hd64, 0.0, None)["draft"]
    ref = oracle.verify_greedy(W, h64, draft)
    out = bd.spec_verify_greedy(w, pt.dev_bf16(data["h"]), _i32(draft), diag=True, logits=True)
    torch.cuda.synchronize()
    _check_rows(out.logits.cpu().numpy(), ref["logits_t"].reshape(-1, wk.V))
    acc, em = out.accepted_len.cpu().numpy(), out.emitted.cpu().numpy()
    gap = ref["gap_t"]

    def classify(b):
        j = min(int(acc[b]), int(ref["accepted"][b]))
        if gap[b, j] < pt.GAP_BAND:
            pt.note("argmax_gap")
            return None
        return f"row {j} gap {gap[b, j]}"

    pt.count_bands(ref, None, "greedy")
    pt.assert_decisions(ref, acc, em, classify, "block16 greedy")


@pytest.mark.parametrize("B", [8, 32, 128])
def test_sweep_greedy_sampled_requests(B):
    wk = wl.SWEEP.with_batch(B)
    data, W, w = _setup(wk)
    hd_dev = pt.dev_bf16(data["h_draft"])
    # drafts: the library's own drafter at T = 0 (argmax of the draft logits); checked below
    x_gpu, _ = bd.spec_draft_propose(w, hd_dev, None, 0.0)
    out = bd.spec_verify_greedy(w, pt.dev_bf16(data["h"]), x_gpu.contiguous(), diag=True, logits=True)
    torch.cuda.synchronize()
    draft = x_gpu.cpu().numpy().astype(np.int64)
    lg = out.logits.cpu().numpy()
    acc, em = out.accepted_len.cpu().numpy(), out.emitted.cpu().numpy()
    K = wk.K
    rng = np.random.default_rng(B)
    sample = np.unique(np.concatenate([[0, B - 1], rng.choice(B, size=min(B, 6), replace=False)]))
    for b in sample:
        rows = slice(b, b + 1)
        ref = oracle.verify_greedy(W, oracle.from_bf16_bits(data["h"][rows]), draft[rows])
        _check_rows(lg[b * (K + 1):(b + 1) * (K + 1)], ref["logits_t"][0])
        # the drafts themselves: argmax of the oracle's draft logits (up to near ties)
        zd = oracle.lm_logits(W.w_lm, oracle.from_bf16_bits(data["h_draft"][b]))
        st = oracle.row_stats(zd)
        sure = st["gap"] >= pt.GAP_BAND
        np.testing.assert_array_equal(draft[b][sure], st["argmax"][sure])
        gap = ref["gap_t"]

        def classify(_b):
            j = min(int(acc[b]), int(ref["accepted"][0]))
            if gap[0, j] < pt.GAP_BAND:
                pt.note("argmax_gap")
                return None
            return f"request {b} row {j}"

        pt.count_bands(ref, None, "greedy")
        pt.assert_decisions(ref, acc[b:b + 1], em[b:b + 1], classify, f"sweep B={B}")


def _sched_check(wk):
    """The whole scheduled batch against the oracle: every draft row's confidence and logits,
    the oracle's own schedule (from its own confidences), and for every request the schedule
    agrees on, its verified rows' logits and its decisions."""
    data, W, w = _setup(wk)
    B, K, V = wk.B, wk.K, wk.V
    hd_dev = pt.dev_bf16(data["h_draft"])
    x_gpu, conf_gpu = bd.spec_draft_propose(w, hd_dev, _f32(data["draft_coins"]), wk.T)
    out = bd.spec_verify_scheduled(w, pt.dev_bf16(data["h"]), hd_dev, x_gpu.contiguous(), _f32(data["coins"]), wk.T,
                                   wk.threshold, wk.budget, diag=True, logits=True)
    torch.cuda.synchronize()
    assert int(out.dev_status.item()) == 0
    draft = x_gpu.cpu().numpy().astype(np.int64)
    vl = out.verify_len.cpu().numpy()
    dg = out.diag.cpu().numpy().astype(np.float64)
    conf = dg[B * (K + 1):, 6].reshape(B, K)
    np.testing.assert_allclose(conf, conf_gpu.cpu().numpy(), atol=pt.PROB_TOL)
    coins = data["coins"].astype(np.float64)
    ref = oracle.verify_scheduled(W, oracle.from_bf16_bits(data["h"]), oracle.from_bf16_bits(data["h_draft"]), draft,
                                  coins, wk.T, wk.threshold, wk.budget)
    np.testing.assert_allclose(conf, ref["conf"], atol=pt.PROB_TOL)
    lg = out.logits.cpu().numpy()
    _check_rows(lg[B * (K + 1):], ref["logits_d"].reshape(-1, V))
    same = _schedule_agrees(vl, ref, wk)
    assert (vl + 1).sum() <= wk.budget
    assert np.all((vl >= 0) & (vl <= K))
    acc, em = out.accepted_len.cpu().numpy(), out.emitted.cpu().numpy()
    lt = lg[: B * (K + 1)].reshape(B, K + 1, V)
    for b in np.nonzero(same)[0]:
        kb = int(vl[b])
        _check_rows(lt[b, : kb + 1], ref["logits_t"][b, : kb + 1])
        assert np.all(em[b, kb + 1:] == -1)
    sel = np.nonzero(same)[0]
    sub = {k: (v[sel] if isinstance(v, np.ndarray) and v.shape[:1] == (B,) else v) for k, v in ref.items()}
    pt.count_bands(sub, coins[sel], "sample")
    rows = _final_rows(lg, B, K, wk.T)
    pt.assert_decisions(sub, acc[sel], em[sel],
                        lambda i: pt.first_diff_sample(sub, int(acc[sel[i]]), em[sel[i]], i, coins[sel], int(vl[sel[i]]),
                                                       rows(sel[i], int(vl[sel[i]]))),
                        f"{wk.name} (all {len(sel)} requests the schedule agrees on)")
    return vl


def test_sched_literal():
    vl = _sched_check(wl.SCHED)
    assert vl.min() >= 0


def test_sched_stress_budget_binds():
    vl = _sched_check(wl.SCHED_STRESS)
    assert (vl + 1).sum() == wl.SCHED_STRESS.budget


def test_wide_sample_sampled_requests():
    wk = wl.WIDE
    data, W, w = _setup(wk)
    B, K, V = wk.B, wk.K, wk.V
    hd_dev = pt.dev_bf16(data["h_draft"])
    x_gpu, _ = bd.spec_draft_propose(w, hd_dev, _f32(data["draft_coins"]), wk.T)
    out = bd.spec_verify_sample(w, pt.dev_bf16(data["h"]), hd_dev, x_gpu.contiguous(), _f32(data["coins"]), wk.T,
                                diag=True, logits=True)
    torch.cuda.synchronize()
    assert int(out.dev_status.item()) == 0
    draft = x_gpu.cpu().numpy().astype(np.int64)
    lg = out.logits.cpu().numpy()
    acc, em = out.accepted_len.cpu().numpy(), out.emitted.cpu().numpy()
    coins = data["coins"].astype(np.float64)
    for b in (0, 13, B - 1):
        sl = slice(b, b + 1)
        ref = oracle.verify_sample(W, oracle.from_bf16_bits(data["h"][sl]), oracle.from_bf16_bits(data["h_draft"][sl]),
                                   draft[sl], coins[sl], wk.T)
        _check_rows(lg[b * (K + 1):(b + 1) * (K + 1)], ref["logits_t"][0])
        _check_rows(lg[B * (K + 1) + b * K: B * (K + 1) + (b + 1) * K], ref["logits_d"][0])
        A = int(acc[b])
        pt.count_bands(ref, coins[sl], "sample")
        rows = _final_rows(lg, B, K, wk.T)(b, K)
        pt.assert_decisions(ref, acc[sl], em[sl], lambda _b: pt.first_diff_sample(ref, A, em[b], 0, coins[sl], K, rows),
                            f"wide request {b}")


def test_wide_greedy_sampled_requests():
    """The wide model greedy: 160 rows, so gate/up and the LM head run on 160 x 256 tiles
    (waves side by side); logits of sampled requests and every decision checked."""
    wk = wl.WIDE
    data, W, w = _setup(wk)
    B, K = wk.B, wk.K
    x_gpu, _ = bd.spec_draft_propose(w, pt.dev_bf16(data["h_draft"]), None, 0.0)
    out = bd.spec_verify_greedy(w, pt.dev_bf16(data["h"]), x_gpu.contiguous(), diag=True, logits=True)
    torch.cuda.synchronize()
    assert int(out.dev_status.item()) == 0
    draft = x_gpu.cpu().numpy().astype(np.int64)
    lg = out.logits.cpu().numpy()
    acc, em = out.accepted_len.cpu().numpy(), out.emitted.cpu().numpy()
    for b in (0, 17, B - 1):
        sl = slice(b, b + 1)
        ref = oracle.verify_greedy(W, oracle.from_bf16_bits(data["h"][sl]), draft[sl])
        _check_rows(lg[b * (K + 1):(b + 1) * (K + 1)], ref["logits_t"][0])
        gap = ref["gap_t"]

        def classify(_b, b=b, ref=ref, gap=gap):
            j = min(int(acc[b]), int(ref["accepted"][0]))
            if gap[0, j] < pt.GAP_BAND:
                pt.note("argmax_gap")
                return None
            return f"wide greedy request {b} row {j}"

        pt.count_bands(ref, None, "greedy")
        pt.assert_decisions(ref, acc[sl], em[sl], classify, f"wide greedy request {b}")
