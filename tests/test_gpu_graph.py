"""Calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

A call enqueues kernels only: no allocation, memset, copy or host synchronisation, and
every counter a kernel relies on is zeroed by an earlier kernel of the same call.  So a
caller may capture a call once and replay it.  Each test warms the call up eagerly,
captures it on fixed buffers, then replays it several times with unrelated eager work and
synchronisations in between.  Every replay must equal the eager call bit for bit, also
after new inputs are copied into the captured input buffers.  The greedy, sampled and
allocation-free entry points are covered, on the streaming kernels (the 16-token block)
and on the tiled ones (40 requests of 8 rows), the block with FP8 weights, and the scheduled one (24 requests, the
verify GEMMs gated on the device-side row count).  Before each replay the logits and
diagnostics are refilled with NaN, as the eager reference's fresh buffers are, so every
replay must also write every row the eager call writes.  The drafter step (sampled and
argmax, streaming and tiled) and the commit (chain and tree, in place: its state is
restored before each replay) are captured the same way.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from draft_block_verification_spec_amd import binding as bd
from draft_block_verification_spec_amd import workload as wl
from tests import parity as pt

pytestmark = pytest.mark.gpu

FIELDS = ("accepted_len", "emitted", "tau", "counters", "dev_status")


def _inputs(wk, data, dev, seed):
    draft = np.random.default_rng(seed).integers(0, wk.V, size=(wk.B, wk.K))
    return (pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"]),
            torch.from_numpy(draft.astype(np.int32)).to(dev),
            torch.from_numpy(np.ascontiguousarray(data["coins"], dtype=np.float32)).to(dev))


def _same(a, b, what):
    for n in FIELDS:
        assert torch.equal(getattr(a, n), getattr(b, n)), f"{what}: {n}"
    if a.verify_len is not None:
        assert torch.equal(a.verify_len, b.verify_len), f"{what}: verify_len"
    if a.logits is not None:
        assert torch.equal(a.logits.nan_to_num(), b.logits.nan_to_num()), f"{what}: logits"
    if a.diag is not None:
        assert torch.equal(a.diag.nan_to_num(), b.diag.nan_to_num()), f"{what}: diag"


def _eager_work(dev, out=None, refill=()):
    """Unrelated eager work, then the output buffers refilled as fresh ones are."""
    x = torch.randn(512, 512, device=dev)
    (x @ x).sum().item()
    fills = [(t, float("nan")) for t in ((out.logits, out.diag) if out is not None else ()) if t is not None]
    for t, v in fills + list(refill):
        t.fill_(v)
    torch.cuda.synchronize()


def _check_graph(wk, mode, noalloc=False, fp8=False):
    dev = torch.device("cuda", 0)
    data = wl.generate(wk)
    if fp8:
        data = wl.to_fp8(data)
    w = pt.dev_fp8_weights(data) if fp8 else pt.dev_weights(data)
    h, hd, draft, u = _inputs(wk, data, dev, 1)
    B, K = wk.B, wk.K
    m = {"greedy": bd.SV_MODE_GREEDY, "sample": bd.SV_MODE_SAMPLE, "scheduled": bd.SV_MODE_SCHEDULED}[mode]
    logits = wk.V * (B * (K + 1) + (B * K if m != bd.SV_MODE_GREEDY else 0)) <= (1 << 26)
    out = bd.make_outputs(B, K, dev, mode=m, V=wk.V, d=wk.d, diag=True, logits=logits)
    ws = None if noalloc else bd.workspace(m, B, K, w, dev)

    def call(o, wsp):
        if mode == "greedy":
            return bd.spec_verify_greedy(w, h, draft, out=o, ws=wsp)
        if mode == "scheduled":
            return bd.spec_verify_scheduled(w, h, hd, draft, u, wk.T, wk.threshold, wk.budget, out=o, ws=wsp)
        if noalloc:
            return bd.spec_verify_sample_noalloc(w, h, hd, draft, u, wk.T, out=o)
        return bd.spec_verify_sample(w, h, hd, draft, u, wk.T, out=o, ws=wsp)

    def eager_reference():
        o = bd.make_outputs(B, K, dev, mode=m, V=wk.V, d=wk.d, diag=True, logits=logits)
        call(o, None if noalloc else bd.workspace(m, B, K, w, dev))
        torch.cuda.synchronize()
        return o

    # warm-up on the capture buffers (first-use attributes and device lookups happen here)
    call(out, ws)
    torch.cuda.synchronize()
    ref = eager_reference()
    assert int(ref.dev_status.item()) == bd.SV_DEV_OK
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, ws)
    for rep in range(3):
        _eager_work(dev, out)
        g.replay()
        torch.cuda.synchronize()
        _same(out, ref, f"{wk.name} {mode} replay {rep}")
    # new inputs in the captured buffers
    d2 = wl.generate(wk, 1, weights=False)
    h2, hd2, draft2, u2 = _inputs(wk, d2, dev, 2)
    h.copy_(h2)
    hd.copy_(hd2)
    draft.copy_(draft2)
    u.copy_(u2)
    torch.cuda.synchronize()
    ref2 = eager_reference()
    # the new inputs change the row statistics, so a replay that reused the old ones would fail
    assert not torch.equal(ref2.diag.nan_to_num(), ref.diag.nan_to_num())
    for rep in range(2):
        _eager_work(dev, out)
        g.replay()
        torch.cuda.synchronize()
        _same(out, ref2, f"{wk.name} {mode} new inputs, replay {rep}")


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_graph_replay_block16(mode):
    _check_graph(wl.BLOCK16, mode)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_graph_replay_tiled(mode):
    _check_graph(wl.SMALL_BATCH, mode)


def test_graph_replay_noalloc():
    _check_graph(wl.BLOCK16, "sample", noalloc=True)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_graph_replay_fp8(mode):
    """FP8 E4M3 weights with row scales on the streaming kernels."""
    _check_graph(wl.BLOCK16, mode, fp8=True)


def test_graph_replay_scheduled():
    _check_graph(wl.SMALL_SCHED, "scheduled")


@pytest.mark.parametrize("wk", [wl.BLOCK16, wl.SMALL_BATCH], ids=lambda w: w.name)
def test_graph_replay_propose(wk):
    """The drafter step over every draft row: 15 rows on the streaming kernels, 280 rows on
    the tiled ones; sampled (the rows' coins) and argmax."""
    dev = torch.device("cuda", 0)
    data = wl.generate(wk)
    w = pt.dev_weights(data)
    rows = pt.dev_bf16(data["h_draft"]).reshape(-1, wk.d).contiguous()
    n = rows.shape[0]
    coins = torch.from_numpy(np.ascontiguousarray(data["draft_coins"], dtype=np.float32).reshape(-1)).to(dev)
    d2 = wl.generate(wk, 1, weights=False)
    rows2 = pt.dev_bf16(d2["h_draft"]).reshape(-1, wk.d).contiguous()
    coins2 = torch.from_numpy(np.ascontiguousarray(d2["draft_coins"], dtype=np.float32).reshape(-1)).to(dev)
    rows0, coins0 = rows.clone(), coins.clone()
    for T in (wk.T, 0.0):
        c = coins if T > 0 else None
        rows.copy_(rows0)
        coins.copy_(coins0)
        ws = bd.workspace(bd.SV_MODE_PROPOSE, n, 0, w, dev)
        x = torch.empty(n, dtype=torch.int32, device=dev)
        conf = torch.empty(n, dtype=torch.float32, device=dev)

        def call():
            bd.spec_draft_propose(w, rows, c, T, draft_out=x, conf_out=conf, ws=ws)

        def eager_reference():
            rx, rc = bd.spec_draft_propose(w, rows, c, T)
            torch.cuda.synchronize()
            return rx.clone(), rc.clone()

        call()
        torch.cuda.synchronize()
        ref = eager_reference()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
        for k in range(3):
            _eager_work(dev, refill=((x, -7), (conf, float("nan"))))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(x, ref[0]) and torch.equal(conf, ref[1]), f"{wk.name} T={T} replay {k}"
        rows.copy_(rows2)
        coins.copy_(coins2)
        torch.cuda.synchronize()
        ref2 = eager_reference()
        # new rows change the drafts (the confidences are 1 at T = 0)
        assert not (torch.equal(ref2[0], ref[0]) and torch.equal(ref2[1], ref[1]))
        for k in range(2):
            _eager_work(dev, refill=((x, -7), (conf, float("nan"))))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(x, ref2[0]) and torch.equal(conf, ref2[1]), f"{wk.name} T={T} new rows, replay {k}"


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("tree", [False, True], ids=["chain", "tree"])
def test_graph_replay_commit(tree):
    """The commit of the small paged-cache case (chain and tree).  It works in place, so the
    cache, lengths, recurrent states and status are restored eagerly before each replay."""
    cw = replace(wl.COMMIT_SMALL, name="commit_small_tree", index=22, tree=True) if tree else wl.COMMIT_SMALL
    c = wl.commit_case(cw, 0)
    kv0, seq0, rs0 = _cuda(c["kv"]), _cuda(c["seq_len"]), _cuda(c["rec_state"])
    kv, seq, rs = kv0.clone(), seq0.clone(), rs0.clone()
    sn, acc, vl, bt = _cuda(c["rec_snap"]), _cuda(c["accepted_len"]), _cuda(c["verify_len"]), _cuda(c["block_table"])
    path = _cuda(c["path"]) if tree else None
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def call():
        bd.spec_commit(acc, seq, Kmax=cw.Kmax, kv=kv, block_table=bt, rec_state=rs, rec_snap=sn, verify_len=vl,
                       path=path, dev_status=status)

    def restore():
        kv.copy_(kv0)
        seq.copy_(seq0)
        rs.copy_(rs0)
        status.zero_()
        torch.cuda.synchronize()

    restore()
    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (kv, seq, rs, status)]
    # a chain's accepted entries are already in place; a tree's are moved along the path
    assert not torch.equal(ref[1], seq0) and not torch.equal(ref[2], rs0), "the case commits nothing"
    assert torch.equal(ref[0], kv0) != tree, "cache bytes moved as the case expects"
    restore()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for k in range(3):
        _eager_work(torch.device("cuda", 0))
        restore()
        g.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((kv, seq, rs, status), ref, ("kv", "seq_len", "rec_state", "dev_status")):
            assert torch.equal(got, want), f"{cw.name} replay {k}: {name}"
