"""Exact argmax ties (reading R6: the lowest index wins) across the places where the
library merges partial row statistics: different workgroups of the weight-streaming LM
head, different column tiles of the tiled LM head, and the two launches of a tiled LM
head whose last columns run as a second launch (statistic slots after the first launch's,
argmax indices offset by the first launch's columns).

Row t1 of W_lm is made a copy of row t0 = the target argmax of a row, half a vocabulary
away (before or after t0), so the two logits of every row are equal bit for bit on both
sides: the same products summed in the same order.  The oracle's argmax (numpy: the first
maximum) is the lowest index; the GPU must return exactly that, and greedy verification
with the oracle's argmax tokens as drafts must accept the whole block.
"""
import numpy as np
import pytest
import torch

import oracle
from draft_block_verification_spec_amd import binding as bd
from draft_block_verification_spec_amd import workload as wl
from tests import parity as pt
from tests.test_gpu_parity import LM_SPLIT, MLP160

pytestmark = pytest.mark.gpu


def _with_duplicates(data, W, wk):
    """Copy W_lm row t0 (a target row's argmax) into row t1 = t0 +- V/2 for as many target rows
    as possible without two copies touching the same row; returns the modified bf16 bits."""
    h64 = oracle.from_bf16_bits(data["h"]).reshape(-1, wk.d)
    z = oracle.lm_logits(W.w_lm, oracle.target_hidden(h64, W))
    am = z.argmax(-1)
    bits = data["w_lm"].copy()
    used, pairs = set(), []
    half = wk.V // 2
    for t0 in am:
        t0 = int(t0)
        t1 = t0 + half if t0 < half else t0 - half
        if t0 in used or t1 in used:
            continue
        bits[t1] = bits[t0]
        used.update((t0, t1))
        pairs.append((t0, t1))
    return bits, pairs


@pytest.mark.parametrize("wk", [wl.SMALL, MLP160, LM_SPLIT], ids=["stream", "tiled", "two-launch"])
def test_exact_ties_go_to_the_lowest_index(wk):
    data = dict(wl.generate(wk))
    W0 = oracle.Weights.from_bits(data)
    data["w_lm"], pairs = _with_duplicates(data, W0, wk)
    assert len(pairs) >= 3
    W = oracle.Weights.from_bits(data)
    h64 = oracle.from_bf16_bits(data["h"])
    z = oracle.lm_logits(W.w_lm, oracle.target_hidden(h64, W))  # [B, K+1, V]
    st = oracle.row_stats(z)
    top = z.max(-1, keepdims=True)
    n_max = (z == top).sum(-1)
    tied = n_max >= 2
    assert tied.sum() >= 3, "the construction should tie several rows exactly"
    # both directions occur: the lower copy sits before and after the original argmax
    t0s = {p[0] for p in pairs}
    low = st["argmax"][tied]
    assert any(int(a) in t0s for a in low) and any(int(a) not in t0s for a in low)
    draft = st["argmax"][:, :-1]
    w = pt.dev_weights(data)
    out = bd.spec_verify_greedy(w, pt.dev_bf16(data["h"]), torch.from_numpy(draft.astype(np.int32)).cuda(),
                                diag=True, logits=True)
    torch.cuda.synchronize()
    assert int(out.dev_status.item()) == bd.SV_DEV_OK
    B, K = wk.B, wk.K
    dg = out.diag.cpu().numpy().reshape(B, K + 1, -1)
    am_gpu = dg[:, :, 1].astype(np.int64)
    lg = out.logits.cpu().numpy().reshape(B, K + 1, -1)
    # the GPU's logits tie exactly where the oracle's do
    for b, j in zip(*np.nonzero(tied)):
        t = np.nonzero(z[b, j] == top[b, j])[0]
        assert np.all(lg[b, j, t] == lg[b, j, t[0]]), (b, j, t)
    np.testing.assert_array_equal(am_gpu[tied], st["argmax"][tied])
    sure = ~tied & (st["gap"] >= pt.GAP_BAND)
    np.testing.assert_array_equal(am_gpu[sure], st["argmax"][sure])
    # greedy with the argmax drafts: every request accepts all K, bonus = argmax of row K
    acc, em = out.accepted_len.cpu().numpy(), out.emitted.cpu().numpy()
    ok = (st["gap"] >= pt.GAP_BAND) | tied
    full = ok.all(axis=1)
    assert np.all(acc[full] == K)
    np.testing.assert_array_equal(em[full], st["argmax"][full])
