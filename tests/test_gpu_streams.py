"""Concurrent calls on two streams, each with its own workspace and outputs.

Calls share no state beyond cached device properties, so a greedy and a sampled call
(or a scheduled call and a drafter step) running at the same time on two streams (default
priority) must give what each gives alone.  Both are issued several times in alternation, so the kernels of the two calls
overlap on the device; every result is compared bit for bit with the same call made on
its own.
"""
import numpy as np
import pytest
import torch

from draft_block_verification_spec_amd import binding as bd
from draft_block_verification_spec_amd import workload as wl
from tests import parity as pt

pytestmark = pytest.mark.gpu


def _same(a, b, what):
    for n in ("accepted_len", "emitted", "tau", "counters", "dev_status"):
        assert torch.equal(getattr(a, n), getattr(b, n)), f"{what}: {n}"
    assert torch.equal(a.diag.nan_to_num(), b.diag.nan_to_num()), f"{what}: diag"


@pytest.mark.parametrize("wk", [wl.SMALL_BATCH, wl.BLOCK16], ids=lambda w: w.name)
def test_two_streams_match_one_at_a_time(wk):
    dev = torch.device("cuda", 0)
    data = wl.generate(wk)
    w = pt.dev_weights(data)
    h, hd = pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"])
    draft = torch.from_numpy(np.random.default_rng(3).integers(0, wk.V, size=(wk.B, wk.K)).astype(np.int32)).to(dev)
    u = torch.from_numpy(np.ascontiguousarray(data["coins"], dtype=np.float32)).to(dev)
    B, K = wk.B, wk.K

    # every workspace and output is allocated before any launch and kept alive until the
    # final synchronisation (a freed buffer could be reused while the other stream runs)
    def buffers(mode):
        return (bd.make_outputs(B, K, dev, mode=mode, V=wk.V, d=wk.d, diag=True), bd.workspace(mode, B, K, w, dev))

    def greedy(buf, stream=None):
        return bd.spec_verify_greedy(w, h, draft, out=buf[0], ws=buf[1], stream=stream)

    def sample(buf, stream=None):
        return bd.spec_verify_sample(w, h, hd, draft, u, wk.T, out=buf[0], ws=buf[1], stream=stream)

    bg, bs = buffers(bd.SV_MODE_GREEDY), buffers(bd.SV_MODE_SAMPLE)
    ref_g, ref_s = greedy(bg), sample(bs)
    torch.cuda.synchronize()
    assert int(ref_g.dev_status.item()) == 0 and int(ref_s.dev_status.item()) == 0
    bufs = [(kind, buffers(bd.SV_MODE_GREEDY if kind == "greedy" else bd.SV_MODE_SAMPLE))
            for _ in range(4) for kind in ("greedy", "sample")]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = [(kind, greedy(buf, s1) if kind == "greedy" else sample(buf, s2)) for kind, buf in bufs]
    torch.cuda.synchronize()
    for i, (kind, o) in enumerate(outs):
        _same(o, ref_g if kind == "greedy" else ref_s, f"{wk.name} {kind} call {i}")


def test_binding_allocations_survive_other_streams():
    """Without caller buffers the binding allocates the workspace and outputs on torch's
    current stream and records them on the call's stream: while the calls run on two other
    streams, fresh allocations of the same sizes on the current stream (filled at once)
    must not land on their memory."""
    wk = wl.SMALL_BATCH
    dev = torch.device("cuda", 0)
    data = wl.generate(wk)
    w = pt.dev_weights(data)
    h, hd = pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"])
    draft = torch.from_numpy(np.random.default_rng(4).integers(0, wk.V, size=(wk.B, wk.K)).astype(np.int32)).to(dev)
    u = torch.from_numpy(np.ascontiguousarray(data["coins"], dtype=np.float32)).to(dev)
    ref_g = bd.spec_verify_greedy(w, h, draft, diag=True)
    ref_s = bd.spec_verify_sample(w, h, hd, draft, u, wk.T, diag=True)
    torch.cuda.synchronize()
    n_g = bd.sv_workspace_bytes(bd.SV_MODE_GREEDY, wk.B, wk.K, w)
    n_s = bd.sv_workspace_bytes(bd.SV_MODE_SAMPLE, wk.B, wk.K, w)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs, junk = [], []
    for _ in range(4):
        outs.append(("greedy", bd.spec_verify_greedy(w, h, draft, diag=True, stream=s1)))
        outs.append(("sample", bd.spec_verify_sample(w, h, hd, draft, u, wk.T, diag=True, stream=s2)))
        for n in (n_g, n_s):  # the sizes the dropped workspaces had
            junk.append(torch.full((n,), 255, dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    for i, (kind, o) in enumerate(outs):
        _same(o, ref_g if kind == "greedy" else ref_s, f"{kind} call {i}")


def test_scheduled_and_drafter_on_two_streams():
    """The scheduled call (device-side schedule, gated GEMM launches) on one stream and the
    drafter step over every draft row on another, alternating four times each."""
    wk = wl.SMALL_SCHED
    dev = torch.device("cuda", 0)
    data = wl.generate(wk)
    w = pt.dev_weights(data)
    h, hd = pt.dev_bf16(data["h"]), pt.dev_bf16(data["h_draft"])
    draft = torch.from_numpy(np.random.default_rng(5).integers(0, wk.V, size=(wk.B, wk.K)).astype(np.int32)).to(dev)
    u = torch.from_numpy(np.ascontiguousarray(data["coins"], dtype=np.float32)).to(dev)
    rows = hd.reshape(-1, wk.d).contiguous()
    n = rows.shape[0]
    coins = torch.from_numpy(np.ascontiguousarray(data["draft_coins"], dtype=np.float32).reshape(-1)).to(dev)
    m = bd.SV_MODE_SCHEDULED

    def sched_buf():
        return (bd.make_outputs(wk.B, wk.K, dev, mode=m, V=wk.V, d=wk.d, diag=True), bd.workspace(m, wk.B, wk.K, w, dev))

    def prop_buf():
        return (torch.empty(n, dtype=torch.int32, device=dev), torch.empty(n, dtype=torch.float32, device=dev),
                bd.workspace(bd.SV_MODE_PROPOSE, n, 0, w, dev))

    def sched(buf, stream=None):
        bd.spec_verify_scheduled(w, h, hd, draft, u, wk.T, wk.threshold, wk.budget, out=buf[0], ws=buf[1],
                                 stream=stream)

    def prop(buf, stream=None):
        bd.spec_draft_propose(w, rows, coins, wk.T, draft_out=buf[0], conf_out=buf[1], ws=buf[2], stream=stream)

    ref_s, ref_p = sched_buf(), prop_buf()
    sched(ref_s)
    prop(ref_p)
    torch.cuda.synchronize()
    assert int(ref_s[0].dev_status.item()) == 0
    bufs = [(sched_buf(), prop_buf()) for _ in range(4)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for bs, bp in bufs:
        sched(bs, s1)
        prop(bp, s2)
    torch.cuda.synchronize()
    for i, (bs, bp) in enumerate(bufs):
        _same(bs[0], ref_s[0], f"scheduled call {i}")
        assert torch.equal(bs[0].verify_len, ref_s[0].verify_len), f"scheduled call {i}: verify_len"
        assert torch.equal(bp[0], ref_p[0]) and torch.equal(bp[1], ref_p[1]), f"drafter call {i}"
