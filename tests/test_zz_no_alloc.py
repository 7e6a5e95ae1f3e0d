"""The allocation-free sampled verification (spec_verify_sample_noalloc) against the
entry point it mirrors (spec_verify_sample with a caller workspace), through the C ABI.

Both run the same kernels, so every output must be bit-identical; two calls in a row,
the second with a smaller batch, check that the shared static scratch is reused
correctly (its previous contents do not leak into the next call).  The oracle comparison
of spec_verify_sample itself lives in the parity tests."""
import numpy as np
import pytest
import torch

import oracle
from draft_block_verification_spec_amd import binding as bd
from draft_block_verification_spec_amd import workload as wl
from tests import parity as pt

pytestmark = pytest.mark.gpu


def _case(wk, rep, oracle_drafts=True):
    data = wl.generate(wk, rep)
    if oracle_drafts:
        draft = pt.oracle_drafts(oracle.Weights.from_bits(data), data, wk.T)["draft"]
    else:
        draft = np.random.default_rng(rep).integers(0, wk.V, size=(wk.B, wk.K))
    dev = lambda x, t: torch.from_numpy(np.ascontiguousarray(x, dtype=t)).cuda()
    return (pt.dev_weights(data), pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"]), dev(draft, np.int32),
            dev(data["coins"], np.float32), wk.T)


def _same(a, b):
    for n in ("accepted_len", "emitted", "tau", "counters", "dev_status"):
        assert torch.equal(getattr(a, n), getattr(b, n)), n
    assert torch.equal(a.logits, b.logits)
    assert torch.equal(a.diag.nan_to_num(), b.diag.nan_to_num())
    assert torch.equal(a.hidden.view(torch.int16), b.hidden.view(torch.int16))


def test_noalloc_matches_caller_workspace_twice():
    # first the larger batch, then a smaller one on the same scratch
    for wk, rep in ((wl.SMALL_WIDE, 3), (wl.SMALL.with_batch(2), 4)):
        args = _case(wk, rep)
        ref = bd.spec_verify_sample(*args, diag=True, logits=True, hidden=True)
        got = bd.spec_verify_sample_noalloc(*args, diag=True, logits=True, hidden=True)
        torch.cuda.synchronize()
        assert int(got.dev_status.item()) == bd.SV_DEV_OK
        _same(ref, got)


def test_noalloc_full_block():
    """The 16-token block (B = 1, K = 15) fits the static scratch; the call after a larger
    one of another shape gives the caller-workspace result again."""
    wk = wl.BLOCK16
    args = _case(wk, 0)
    ref = bd.spec_verify_sample(*args, logits=True)
    got = bd.spec_verify_sample_noalloc(*args, logits=True)
    torch.cuda.synchronize()
    assert torch.equal(ref.emitted, got.emitted) and torch.equal(ref.accepted_len, got.accepted_len)
    assert torch.equal(ref.logits, got.logits) and torch.equal(ref.tau, got.tau)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    wk = wl.SMALL.with_batch(4096)
    args = _case(wk, 0, oracle_drafts=False)
    assert bd.sv_workspace_bytes(bd.SV_MODE_SAMPLE, wk.B, wk.K, args[0]) > bd.SV_STATIC_SCRATCH_BYTES
    with pytest.raises(bd.SpecVerifyError, match="static scratch"):
        bd.spec_verify_sample_noalloc(*args)
