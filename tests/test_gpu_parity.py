"""GPU parity of the HIP verification path against the fp64 oracle (C ABI via ctypes).

Reduced shapes span several GEMM tiles and ragged tails (V = 5003, 12347, 4099, 3001;
M not a multiple of 16) and are compared element by element; the full-size shapes
are in test_gpu_fullsize.py.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from draft_block_verification_spec_amd import binding as bd
from draft_block_verification_spec_amd import workload as wl
from tests import parity as pt

pytestmark = pytest.mark.gpu


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _weights(wk, rep, fp8):
    """Inputs, oracle weights and device weights (bf16, or FP8 codes + row scales)."""
    data = wl.generate(wk, rep)
    if fp8:
        data = wl.to_fp8(data)
        return data, oracle.Weights.from_fp8(data), pt.dev_fp8_weights(data)
    return data, oracle.Weights.from_bits(data), pt.dev_weights(data)


def _final_rows(lg, B, K, T):
    """rows(b, K_b)(A): the GPU's logit rows of request b's final draw at accepted length A,
    out of the logits in call order (target rows [B*(K+1)], then draft rows [B*K])."""
    def rows(b, K_b):
        return lambda A: (lg[b * (K + 1) + A], lg[B * (K + 1) + b * K + A] if A < K_b else None, T)
    return rows


def _run_sample(wk, rep=0, check_hidden=True, fp8=False, edit=None):
    data, W, w = _weights(wk, rep, fp8)
    if edit is not None:  # inputs changed on the host before either side sees them
        data = edit(data, wk)
    T = wk.T
    draft = pt.oracle_drafts(W, data, T)["draft"]
    h64 = oracle.from_bf16_bits(data["h"])
    hd64 = oracle.from_bf16_bits(data["h_draft"])
    coins = data["coins"].astype(np.float64)
    ref = oracle.verify_sample(W, h64, hd64, draft, coins, T)
    out = bd.spec_verify_sample(w, pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"]), _i32(draft),
                                _f32(data["coins"]), T, diag=True, logits=True, hidden=wk.d_ff > 0)
    torch.cuda.synchronize()
    B, K, V = wk.B, wk.K, wk.V
    assert int(out.dev_status.item()) == bd.SV_DEV_OK
    # logits of target and draft rows
    lg = out.logits.cpu().numpy().astype(np.float64)
    ref_lg = np.concatenate([ref["logits_t"].reshape(-1, V), ref["logits_d"].reshape(-1, V)])
    err = np.abs(lg - ref_lg).max()
    assert err <= pt.LOGIT_TOL, f"logit error {err}"
    if check_hidden and wk.d_ff > 0:
        pt.check_hidden(out.hidden, ref["y"], W, h64)
    # p(x) on target rows j < K, q(x) and the confidence on draft rows
    dg = out.diag.cpu().numpy().astype(np.float64)
    dt = dg[: B * (K + 1)].reshape(B, K + 1, -1)
    dd = dg[B * (K + 1):].reshape(B, K, -1)
    rt = (np.arange(B)[:, None] * (K + 1) + np.arange(K)[None, :]).ravel()
    rd = B * (K + 1) + np.arange(B * K)
    pt.check_probs(dt[:, :K, 5], lg[rt], ref_lg[rt], draft, ref["p_x"], T, "p(x)")
    pt.check_probs(dd[:, :, 5], lg[rd], ref_lg[rd], draft, ref["q_x"], T, "q(x)")
    pt.check_probs(dd[:, :, 6], lg[rd], ref_lg[rd], None, ref["conf"], T, "confidence")
    pt.check_lse(dt[:, :, 0], lg[: B * (K + 1)], ref_lg[: B * (K + 1)], ref["lse_t"], T, "target lse")
    pt.check_lse(dd[:, :, 0], lg[rd], ref_lg[rd], ref["lse_d"], T, "draft lse")
    # decisions
    acc = out.accepted_len.cpu().numpy()
    em = out.emitted.cpu().numpy()
    pt.count_bands(ref, coins, "sample")
    rows = _final_rows(lg, B, K, T)
    mism = pt.assert_decisions(ref, acc, em,
                               lambda b: pt.first_diff_sample(ref, int(acc[b]), em[b], b, coins, K, rows(b, K)),
                               f"sample {wk.name}")
    tau = float(out.tau.item())
    assert tau == pytest.approx(np.mean(acc + 1), rel=1e-6)
    c = out.counters.cpu().numpy()
    assert c[0] == acc.sum() and c[1] == B * K and c[2] == (acc + 1).sum()
    return ref, out, mism


@pytest.mark.parametrize("name", ["small", "small_wide", "small_batch"])
def test_sample_parity(name):
    _run_sample(wl.PRESETS[name])


def test_sample_parity_tiny_steps():
    """Tiny configuration (d=64, V=512, no MLP): 2000 verify steps in one call; the
    fp32 values are rounded to bf16 for both sides."""
    _run_sample(wl.TINY.with_batch(2000))


def _run_greedy(wk, rep=0, fp8=False, edit=None):
    data, W, w = _weights(wk, rep, fp8)
    if edit is not None:
        data = edit(data, wk)
    draft = pt.oracle_drafts(W, data, 0.0)["draft"]
    ref = oracle.verify_greedy(W, oracle.from_bf16_bits(data["h"]), draft)
    out = bd.spec_verify_greedy(w, pt.dev_bf16(data["h"]), _i32(draft), diag=True, logits=True,
                                hidden=wk.d_ff > 0)
    torch.cuda.synchronize()
    B, K, V = wk.B, wk.K, wk.V
    assert int(out.dev_status.item()) == bd.SV_DEV_OK
    if wk.d_ff > 0:
        pt.check_hidden(out.hidden, ref["y"], W, oracle.from_bf16_bits(data["h"]))
    lg = out.logits.cpu().numpy().astype(np.float64)
    err = np.abs(lg - ref["logits_t"].reshape(-1, V)).max()
    assert err <= pt.LOGIT_TOL, f"logit error {err}"
    dg = out.diag.cpu().numpy().reshape(B, K + 1, -1)
    gap = ref["gap_t"]
    am = dg[:, :, 1].astype(np.int64)
    sure = gap >= pt.GAP_BAND
    np.testing.assert_array_equal(am[sure], ref["argmax"][sure])
    acc = out.accepted_len.cpu().numpy()
    em = out.emitted.cpu().numpy()

    def classify(b):
        A_o, A_g = int(ref["accepted"][b]), int(acc[b])
        j = min(A_o, A_g)
        if gap[b, j] < pt.GAP_BAND:
            pt.note("argmax_gap")
            return None
        return f"greedy decision differs at row {j} (gap {gap[b, j]:.2e})"

    pt.count_bands(ref, None, "greedy")
    pt.assert_decisions(ref, acc, em, classify, f"greedy {wk.name}")
    # every emitted token is the target argmax of its row (the greedy invariant, on GPU output)
    for b in range(B):
        for j in range(int(acc[b]) + 1):
            assert em[b, j] == am[b, j] or gap[b, j] < pt.GAP_BAND
    return ref, out


# Two reduced shapes aimed at tiling paths of the larger-batch GEMMs:
#  * 20 requests x 8 rows = 160 target rows: gate/up and down run on 192-row tiles (one row
#    tile per column tile), the 300-row sampled LM head on two row tiles of 160 x 256
#    (waves side by side, four statistics slots per column tile);
#  * 128 requests x 8 rows = 1024 rows, V = 24000: 94 column tiles of 256 x 4 row tiles =
#    376 tiles = one round of 256 + 120, so columns [0, 16384) run as 256 x 256 tiles and
#    the ragged rest (7616 columns, 240 tiles of 256 x 128) as a second launch whose
#    argmax indices and statistic slots are offset; with d_ff = 12288 gate/up splits the
#    same way (outputs [0, 8192) on 256 x 256 tiles, the rest on 256 x 128).
MLP160 = wl.Workload("mlp160", 14, B=20, K=7, d=256, d_ff=1536, V=5003, T=1.0, sigma=(0.3, 1.2))
LM_SPLIT = wl.Workload("lm_split", 15, B=128, K=7, d=256, d_ff=12288, V=24000, T=1.0, sigma=(0.3, 1.2))


# Blocks longer than the 64 acceptance decisions one wave takes at a time (the batched
# acceptance kernels), and a 32-row batch on the small-batch tail.  With no MLP and no
# drafter noise every draft row equals its target row, so p = q: every draft is accepted
# (exactly: the ratio is exp(0)) and the final token is the bonus draw from row K.  With
# the draft rows from position 66 on taken from another draw, the drafts there no longer
# follow the target and the first rejection falls in the second block of 64 (the oracle
# puts it at 66 for both requests, in both modes; no greedy row is within the near-tie band).
LONG70 = wl.Workload("long70", 90, B=2, K=70, d=64, d_ff=0, V=1000, T=1.0, sigma=0.0)
LONG64 = wl.Workload("long64", 91, B=1, K=64, d=64, d_ff=0, V=1000, T=1.0, sigma=0.0)
SAME15 = wl.Workload("same_rows15", 92, B=2, K=15, d=64, d_ff=0, V=1000, T=1.0, sigma=0.0)


def _draft_rows_from_another_draw(j0):
    def edit(data, wk):
        hd = data["h_draft"].copy()
        hd[:, j0:] = wl.generate(wk, 1, weights=False)["h_draft"][:, j0:]
        return {**data, "h_draft": hd}
    return edit


@pytest.mark.parametrize("wk", [LONG70, LONG64, SAME15], ids=lambda w: w.name)
def test_equal_rows_accept_every_draft(wk):
    _, out, _ = _run_sample(wk)
    assert (out.accepted_len.cpu().numpy() == wk.K).all()
    _, out = _run_greedy(wk)
    assert (out.accepted_len.cpu().numpy() == wk.K).all()


def test_long_block_rejects_in_second_block():
    edit = _draft_rows_from_another_draw(66)
    ref, out, _ = _run_sample(LONG70, edit=edit)
    assert (out.accepted_len.cpu().numpy() == 66).all() and (ref["accepted"] == 66).all()
    ref, out = _run_greedy(LONG70, edit=edit)
    assert (out.accepted_len.cpu().numpy() == 66).all() and (ref["accepted"] == 66).all()


def test_sample_parity_160_rows():
    _run_sample(MLP160)


def test_greedy_parity_160_rows():
    _run_greedy(MLP160)


def test_greedy_parity_lm_head_in_two_launches():
    _run_greedy(LM_SPLIT)


# The LM head at 257-320 rows runs on two row tiles of 160: sampled at 288 rows (the wide
# model's shape: 32 requests, 4 drafts) and 258 rows (86 requests, one draft: the second
# row tile 98 rows live); greedy at 320 rows (both row tiles full) and 288 rows.
LM160 = [wl.Workload("lm160_288", 23, B=32, K=4, d=512, d_ff=1536, V=12347, T=0.7, sigma=0.6),
         wl.Workload("lm160_320", 24, B=40, K=7, d=256, d_ff=512, V=5003, T=1.0, sigma=(0.3, 1.2)),
         wl.Workload("lm160_258", 25, B=86, K=1, d=256, d_ff=512, V=4099, T=1.0, sigma=0.4)]


# 160 rows with d_ff = 16896: gate/up on 160 x 256 tiles (one round of 132 tiles against
# two rounds of 264 192 x 128 ones), the LM head on one 160-row tile.
MLP160_FF = wl.Workload("mlp160_ff", 26, B=20, K=7, d=256, d_ff=16896, V=5003, T=1.0, sigma=(0.3, 1.2))


def test_greedy_parity_160_rows_wide_ff():
    _run_greedy(MLP160_FF)


# 160 rows with d = 8192, d_ff = 2048: the down projection on 160 x 256 tiles with 8
# K-splits (32 column tiles x 8 = 256 workgroups) and the fixed-order reduce; the MLP
# output is compared element by element.
MLP160_D8K = wl.Workload("mlp160_d8k", 27, B=20, K=7, d=8192, d_ff=2048, V=5003, T=1.0, sigma=(0.3, 1.2))


def test_greedy_parity_160_rows_down_split_k():
    _run_greedy(MLP160_D8K)


def test_sample_parity_160_rows_wide_ff():
    _run_sample(MLP160_FF)


@pytest.mark.parametrize("wk", [LM160[0], LM160[2]], ids=lambda w: w.name)
def test_sample_parity_lm_head_160_row_tiles(wk):
    _run_sample(wk)


@pytest.mark.parametrize("B", [40, 36], ids=["320-rows", "288-rows"])
def test_greedy_parity_lm_head_160_row_tiles(B):
    _run_greedy(LM160[1].with_batch(B))


# The LM head at 161-192 rows runs on 192 x 192 tiles (three 32-column blocks per wave):
# greedy at 168 and 192 rows, sampled at 180 rows (20 requests, 4 drafts).
@pytest.mark.parametrize("B", [21, 24], ids=["168-rows", "192-rows"])
def test_greedy_parity_lm_head_192_tiles(B):
    _run_greedy(LM160[1].with_batch(B))


def test_sample_parity_lm_head_192_tiles():
    _run_sample(LM160[0].with_batch(20))


# The LM head at 193-256 rows runs on one 256 x 256 row tile: greedy at 256 rows with
# V = 70000 (274 column tiles: one round of 256 on 256 x 256 tiles, the ragged 4464
# columns as a second launch of 256 x 128 tiles), at 200 rows with V = 48000 (one partial
# round, no split); sampled at 240 rows (16 requests: 128 target + 112 draft rows).
LM256 = wl.Workload("lm256", 28, B=32, K=7, d=256, d_ff=512, V=70000, T=1.0, sigma=(0.3, 1.2))


@pytest.mark.parametrize("B,V", [(32, 70000), (25, 48000)], ids=["256-rows-split", "200-rows"])
def test_greedy_parity_lm_head_256_tiles(B, V):
    _run_greedy(replace(LM256, V=V).with_batch(B))


def test_sample_parity_lm_head_256_tiles():
    _run_sample(LM256.with_batch(16))


# Sizes that are not multiples of 128: d = 192 and d_ff = 576 put the 64-row LM head and
# down projection on 64-wide slices (64 x 128, two stages), the 16-row weight-streaming
# kernels on their general-K path (6 and 18 k-steps of 32, the rest of a 4096-wide chunk
# masked), and V = 3001 (odd) on the scalar paths of the sampling tails.
ODD = wl.Workload("odd_dims", 33, B=8, K=7, d=192, d_ff=576, V=3001, T=1.0, sigma=(0.3, 1.2))


@pytest.mark.parametrize("B", [8, 2], ids=["64-rows", "16-rows"])
def test_greedy_parity_odd_dims(B):
    _run_greedy(ODD.with_batch(B))


@pytest.mark.parametrize("B", [8, 2], ids=["120-rows", "30-rows"])
def test_sample_parity_odd_dims(B):
    _run_sample(ODD.with_batch(B))


@pytest.mark.parametrize("name", ["small", "small_wide", "small_batch", "tiny"])
def test_greedy_parity(name):
    wk = wl.PRESETS[name]
    if name == "tiny":
        wk = wk.with_batch(2000)
    _run_greedy(wk)


def test_greedy_drafts_from_target_accept_everything():
    """When the drafts are the target's own argmax the whole block is accepted and the
    bonus token is the argmax of the last row."""
    wk = wl.SMALL
    data = wl.generate(wk)
    W = oracle.Weights.from_bits(data)
    y = oracle.target_hidden(oracle.from_bf16_bits(data["h"]), W)
    z = oracle.lm_logits(W.w_lm, y)
    st = oracle.row_stats(z)
    draft = st["argmax"][:, :-1]
    w = pt.dev_weights(data)
    out = bd.spec_verify_greedy(w, pt.dev_bf16(data["h"]), _i32(draft))
    torch.cuda.synchronize()
    acc = out.accepted_len.cpu().numpy()
    ok = st["gap"].min(axis=1) >= pt.GAP_BAND
    assert np.all(acc[ok] == wk.K)
    assert float(out.tau.item()) == pytest.approx(np.mean(acc + 1))


# Shapes of the small-batch tail (B * (K+1) <= 32) beyond the ones above: V a multiple
# of 4 (16-byte logit loads) at reduced size, no drafts at all (K = 0: the one token is
# drawn from p), and the scheduled mode with two requests (budget binding).
TAIL_VEC = wl.Workload("tail_vec", 16, B=2, K=7, d=256, d_ff=512, V=8192, T=1.0, sigma=0.4)
NO_DRAFTS = wl.Workload("no_drafts", 17, B=4, K=0, d=256, d_ff=512, V=5003, T=1.0, sigma=0.4)
SCHED_TAIL = wl.Workload("sched_tail", 18, B=2, K=15, d=256, d_ff=512, V=8192, T=1.0, sigma=(0.3, 1.2),
                         gain=(4.0, 32.0), threshold=0.3, budget=12)


def test_sample_parity_small_tail_vec():
    _run_sample(TAIL_VEC)


def test_sample_without_drafts():
    wk = NO_DRAFTS
    data = wl.generate(wk)
    W = oracle.Weights.from_bits(data)
    coins = data["coins"].astype(np.float64)
    draft = np.zeros((wk.B, 0), dtype=np.int64)
    ref = oracle.verify_sample(W, oracle.from_bf16_bits(data["h"]), oracle.from_bf16_bits(data["h_draft"]), draft,
                               coins, wk.T)
    w = pt.dev_weights(data)
    out = bd.spec_verify_sample(w, pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"]), _i32(draft),
                                _f32(data["coins"]), wk.T, logits=True)
    torch.cuda.synchronize()
    assert int(out.dev_status.item()) == bd.SV_DEV_OK
    lg = out.logits.cpu().numpy().astype(np.float64)
    assert np.abs(lg - ref["logits_t"].reshape(-1, wk.V)).max() <= pt.LOGIT_TOL
    acc, em = out.accepted_len.cpu().numpy(), out.emitted.cpu().numpy()
    assert np.all(acc == 0)
    rows = _final_rows(lg, wk.B, 0, wk.T)
    pt.assert_decisions(ref, acc, em, lambda b: pt.first_diff_sample(ref, 0, em[b], b, coins, 0, rows(b, 0)),
                        "no drafts")
    assert float(out.tau.item()) == pytest.approx(1.0)


def test_scheduled_parity_small():
    _run_scheduled(wl.SMALL_SCHED)


def test_scheduled_parity_small_tail():
    _run_scheduled(SCHED_TAIL)


# A binding budget above 128 rows: the verify GEMMs span two row tiles of 128.
SCHED_200 = wl.Workload("sched_200", 19, B=24, K=15, d=256, d_ff=512, V=3001, T=1.0, sigma=(0.3, 1.2),
                        gain=(4.0, 32.0), threshold=0.3, budget=200)


def test_scheduled_parity_two_row_tiles():
    _run_scheduled(SCHED_200)


# A budget that does not bind: the verify GEMMs are planned for 512 rows (two row tiles
# of 256) while 142 rows are verified, so only the first row tile is live, the down
# projection takes its split-K path, and of each pair of launches (plans for at most 128
# rows and for the budget) the budget-sized one works.
SCHED_LOOSE = wl.Workload("sched_loose", 22, B=64, K=15, d=256, d_ff=512, V=3001, T=1.0, sigma=(0.3, 1.2),
                          gain=(1.0, 2.5), threshold=0.3, budget=512)


def test_scheduled_parity_budget_not_binding():
    vl = _run_scheduled(SCHED_LOOSE, expect_bound=False)
    assert 128 < (vl + 1).sum() <= 192, (vl + 1).sum()


# The same batch with a higher threshold: 105 rows verified, so the launches planned for
# at most 128 rows (128 x 256 LM-head tiles) do the work and the budget-sized ones return.
SCHED_FEW = replace(SCHED_LOOSE, name="sched_few", threshold=0.5)


def test_scheduled_parity_few_rows_small_plans():
    vl = _run_scheduled(SCHED_FEW, expect_bound=False)
    assert 64 < (vl + 1).sum() <= 128, (vl + 1).sum()


# A 160-row budget: the budget-sized LM head uses 160 x 256 tiles (four statistics slots
# per column tile) and the small plan 128 x 256 ones (two).  Binding (160 rows: the
# budget-sized launches work) and not binding (105 rows: the small ones work).
SCHED_160 = replace(SCHED_200, name="sched_160", budget=160)
SCHED_160_FEW = replace(SCHED_LOOSE, name="sched_160_few", threshold=0.5, budget=160)


def test_scheduled_parity_budget_160_binding():
    vl = _run_scheduled(SCHED_160)
    assert (vl + 1).sum() == 160


def test_scheduled_parity_budget_160_few_rows():
    vl = _run_scheduled(SCHED_160_FEW, expect_bound=False)
    assert 64 < (vl + 1).sum() <= 128, (vl + 1).sum()


# A binding 300-row budget: the budget-sized verify LM head runs on two row tiles of 160
# (four statistics slots per column tile), the small plan beside it on 128-row tiles.
SCHED_300 = replace(SCHED_200, name="sched_300", budget=300)


def test_scheduled_parity_budget_300_binding():
    vl = _run_scheduled(SCHED_300)
    assert (vl + 1).sum() == 300


# A binding 192-row budget: the budget-sized verify LM head on one row tile of 192 x 192.
SCHED_192 = replace(SCHED_200, name="sched_192", budget=192)


def test_scheduled_parity_budget_192_binding():
    vl = _run_scheduled(SCHED_192)
    assert (vl + 1).sum() == 192


# The largest batch the scheduled call takes: 8192 requests of one draft each, so the
# schedule's keys, key histogram and lengths need 68 KiB of LDS (over the 64 KiB a launch
# gets by default); the budget binds (3808 of the 8192 drafts kept).
SCHED_MAX = wl.Workload("sched_max", 96, B=8192, K=1, d=64, d_ff=0, V=257, T=1.0, sigma=(0.3, 1.2),
                        gain=(1.0, 8.0), threshold=0.3, budget=12000)


def test_scheduled_parity_largest_batch():
    _run_scheduled(SCHED_MAX)


def _run_scheduled(wk, expect_bound=True):
    data = wl.generate(wk)
    W = oracle.Weights.from_bits(data)
    T = wk.T
    draft = pt.oracle_drafts(W, data, T)["draft"]
    coins = data["coins"].astype(np.float64)
    ref = oracle.verify_scheduled(W, oracle.from_bf16_bits(data["h"]), oracle.from_bf16_bits(data["h_draft"]), draft,
                                  coins, T, wk.threshold, wk.budget)
    assert bool(ref["budget_bound"]) == expect_bound, "budget binding not as the shape intends"
    w = pt.dev_weights(data)
    out = bd.spec_verify_scheduled(w, pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"]), _i32(draft),
                                   _f32(data["coins"]), T, wk.threshold, wk.budget, diag=True, logits=True)
    torch.cuda.synchronize()
    B, K, V = wk.B, wk.K, wk.V
    assert int(out.dev_status.item()) == bd.SV_DEV_OK
    dg = out.diag.cpu().numpy().astype(np.float64)
    dd = dg[B * (K + 1):].reshape(B, K, -1)
    lg = out.logits.cpu().numpy().astype(np.float64)
    ref_ld = ref["logits_d"].reshape(-1, V)
    np.testing.assert_allclose(lg[B * (K + 1):], ref_ld, atol=pt.LOGIT_TOL, rtol=0)
    pt.check_probs(dd[:, :, 6], lg[B * (K + 1):], ref_ld, None, ref["conf"], T, "confidence")
    vl = out.verify_len.cpu().numpy()
    same = _schedule_agrees(vl, ref, wk)
    assert (vl + 1).sum() <= wk.budget
    # every request the schedule agrees on: its verified target rows' logits (scattered back
    # to their unpacked rows) and its decisions
    lt = lg[: B * (K + 1)].reshape(B, K + 1, V)
    for b in np.nonzero(same)[0]:
        kb = int(vl[b])
        err = np.abs(lt[b, : kb + 1] - ref["logits_t"][b, : kb + 1]).max()
        assert err <= pt.LOGIT_TOL
    acc = out.accepted_len.cpu().numpy()
    em = out.emitted.cpu().numpy()
    sel = np.nonzero(same)[0]
    sub = {k: (v[sel] if isinstance(v, np.ndarray) and v.shape[:1] == (B,) else v) for k, v in ref.items()}
    pt.count_bands(sub, coins[sel], "sample")
    rows = _final_rows(lg, B, K, T)
    pt.assert_decisions(sub, acc[sel], em[sel],
                        lambda i: pt.first_diff_sample(sub, int(acc[sel[i]]), em[sel[i]], i, coins[sel], int(vl[sel[i]]),
                                                       rows(sel[i], int(vl[sel[i]]))),
                        "scheduled")
    c = out.counters.cpu().numpy()
    assert c[1] == vl.sum() and c[2] == (acc + 1).sum()
    return vl


def _schedule_agrees(vl, ref, wk):
    """Requests whose verify length equals the oracle's.  Where they differ, the survival
    products must lie within SURV_BAND of the threshold or of a 1/1024 key boundary (reading
    R11): a request whose own survival is near the threshold, or any request when the budget
    cut falls on a near-tie key (it can move positions between requests)."""
    same = vl == ref["verify_len"]
    if same.all():
        return same
    s = ref["survival"]
    near_thr = np.abs(s - wk.threshold) < pt.SURV_BAND
    near_key = np.abs(1024 * s - np.round(1024 * s)) < 1024 * pt.SURV_BAND
    for b in np.nonzero(~same)[0]:
        assert near_thr[b].any() or (ref["budget_bound"] and near_key.any()), \
            f"request {b}: verify length {vl[b]} vs {ref['verify_len'][b]} without a near tie"
        pt.note("survival")
    TALLY_SCHED.append(int((~same).sum()))
    return same


TALLY_SCHED: list = []


# The drafter step over 20 draft rows (streaming kernel) and over 140, 168 and 280 rows
# (LM head on 160 x 256, 192 x 192 and two row tiles of 160 x 256).
@pytest.mark.parametrize("wk", [wl.SMALL_WIDE, wl.SMALL_BATCH.with_batch(20), wl.SMALL_BATCH.with_batch(24),
                                wl.SMALL_BATCH.with_batch(40)], ids=lambda w: f"{w.name}-b{w.B}")
def test_propose_parity(wk):
    data = wl.generate(wk)
    W = oracle.Weights.from_bits(data)
    w = pt.dev_weights(data)
    hd = pt.dev_bf16(data["h_draft"])
    for T in (wk.T, 0.0):
        ref = pt.oracle_drafts(W, data, T)
        x, conf = bd.spec_draft_propose(w, hd, _f32(data["draft_coins"]), T)
        torch.cuda.synchronize()
        x = x.cpu().numpy()
        z = ref["logits"]
        if T == 0.0:
            gap = oracle.row_stats(z)["gap"]
            sure = gap >= pt.GAP_BAND
            np.testing.assert_array_equal(x[sure], ref["draft"][sure])
        else:
            q = oracle.softmax_t(z, T)
            C = np.cumsum(q, axis=-1)
            u = data["draft_coins"].astype(np.float64)
            diff = x != ref["draft"]
            for idx in zip(*np.nonzero(diff)):
                cdf = C[idx]
                assert np.min(np.abs(cdf - u[idx])) < pt.CDF_BAND, f"draft token differs at {idx}"
            np.testing.assert_allclose(conf.cpu().numpy(), ref["conf"], atol=pt.PROB_TOL)


def test_bad_draft_token_sets_status():
    wk = wl.SMALL
    data = wl.generate(wk)
    W = oracle.Weights.from_bits(data)
    draft = pt.oracle_drafts(W, data, wk.T)["draft"].copy()
    draft[1, 2] = wk.V  # out of range
    w = pt.dev_weights(data)
    out = bd.spec_verify_sample(w, pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"]), _i32(draft),
                                _f32(data["coins"]), wk.T)
    torch.cuda.synchronize()
    assert int(out.dev_status.item()) == bd.SV_DEV_BAD_TOKEN
    acc = out.accepted_len.cpu().numpy()
    em = out.emitted.cpu().numpy()
    assert acc[1] == -1 and np.all(em[1] == -1)
    assert acc[0] >= 0 and acc[2] >= 0
    # greedy as well, and a clean call afterwards resets the status
    gd = pt.oracle_drafts(W, data, 0.0)["draft"].copy()
    gd[2, 0] = -5
    out2 = bd.spec_verify_greedy(w, pt.dev_bf16(data["h"]), _i32(gd))
    torch.cuda.synchronize()
    assert int(out2.dev_status.item()) == bd.SV_DEV_BAD_TOKEN
    assert out2.accepted_len.cpu().numpy()[2] == -1
    gd[2, 0] = 0
    bd.spec_verify_greedy(w, pt.dev_bf16(data["h"]), _i32(gd), out=out2)
    torch.cuda.synchronize()
    assert int(out2.dev_status.item()) == bd.SV_DEV_OK


def test_deterministic_and_optional_outputs():
    """Two identical calls give bit-identical results (no float atomics); optional
    outputs may be omitted without changing the decisions."""
    wk = wl.SMALL_BATCH
    data = wl.generate(wk)
    W = oracle.Weights.from_bits(data)
    draft = _i32(pt.oracle_drafts(W, data, wk.T)["draft"])
    w = pt.dev_weights(data)
    h, hd, u = pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"]), _f32(data["coins"])
    o1 = bd.spec_verify_sample(w, h, hd, draft, u, wk.T, diag=True, logits=True, hidden=True)
    o2 = bd.spec_verify_sample(w, h, hd, draft, u, wk.T, diag=True, logits=True, hidden=True)
    o3 = bd.spec_verify_sample(w, h, hd, draft, u, wk.T)
    torch.cuda.synchronize()
    assert torch.equal(o1.logits, o2.logits)
    assert torch.equal(o1.hidden.view(torch.int16), o2.hidden.view(torch.int16))
    assert torch.equal(o1.emitted, o2.emitted) and torch.equal(o1.emitted, o3.emitted)
    assert torch.equal(o1.accepted_len, o3.accepted_len)
    assert torch.equal(o1.diag.nan_to_num(), o2.diag.nan_to_num())


def test_scheduled_workspace_reuse_across_plans():
    """One workspace and one set of outputs for calls that alternate between the two
    plans of the verify pass (105 rows verified: the plans for at most 128 rows work;
    142 rows: the budget-sized ones): every call is bit-identical to the same call on a
    fresh workspace, so nothing a previous call left behind (statistics slots, the slot
    count the LM head reports, partials) leaks into the next."""
    data = wl.generate(SCHED_LOOSE)
    W = oracle.Weights.from_bits(data)
    w = pt.dev_weights(data)
    T = SCHED_LOOSE.T
    draft = _i32(pt.oracle_drafts(W, data, T)["draft"])
    h, hd, u = pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"]), _f32(data["coins"])
    B, K = SCHED_LOOSE.B, SCHED_LOOSE.K
    ws = bd.workspace(bd.SV_MODE_SCHEDULED, B, K, w, h.device)
    out = bd.make_outputs(B, K, h.device, mode=bd.SV_MODE_SCHEDULED, V=SCHED_LOOSE.V, d=SCHED_LOOSE.d, diag=True,
                          logits=True)
    for thr in (0.5, 0.3, 0.5, 0.3):
        fresh = bd.spec_verify_scheduled(w, h, hd, draft, u, T, thr, SCHED_LOOSE.budget, diag=True, logits=True)
        bd.spec_verify_scheduled(w, h, hd, draft, u, T, thr, SCHED_LOOSE.budget, out=out, ws=ws)
        torch.cuda.synchronize()
        assert int(out.dev_status.item()) == bd.SV_DEV_OK
        vl = out.verify_len.cpu().numpy()
        rows = int((vl + 1).sum())
        assert (64 < rows <= 128) if thr == 0.5 else (rows > 128), rows
        assert torch.equal(out.verify_len, fresh.verify_len)
        assert torch.equal(out.accepted_len, fresh.accepted_len)
        assert torch.equal(out.emitted, fresh.emitted)
        assert torch.equal(out.counters, fresh.counters)
        # every draft row is written by each call; target rows up to each request's
        # verified length (the rest of the reused outputs keep an earlier call's values)
        nt = B * (K + 1)
        assert torch.equal(out.diag[nt:].nan_to_num(), fresh.diag[nt:].nan_to_num())
        assert torch.equal(out.logits[nt:], fresh.logits[nt:])
        dt_o, dt_f = out.diag[:nt].view(B, K + 1, -1), fresh.diag[:nt].view(B, K + 1, -1)
        lt_o, lt_f = out.logits[:nt].view(B, K + 1, -1), fresh.logits[:nt].view(B, K + 1, -1)
        for b in range(B):
            k = int(vl[b]) + 1
            assert torch.equal(dt_o[b, :k].nan_to_num(), dt_f[b, :k].nan_to_num())
            assert torch.equal(lt_o[b, :k], lt_f[b, :k])
