"""GPU parity of spec_commit against the commit oracle (reading R14): byte-exact cache,
cache lengths and recurrent states; requests whose commit does not fit are left alone
and flagged.  The toy-session test drives the GPU commit through a session mixing steps
with and without drafts and checks sequential decoding after every step."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from draft_block_verification_spec_amd import binding as bd
from draft_block_verification_spec_amd import workload as wl
from tests.commit_session import Session, ToyTarget

pytestmark = pytest.mark.gpu

SMALL_TREE = replace(wl.COMMIT_SMALL, name="commit_small_tree", index=22, tree=True)
# the longest verify block the commit takes (Kmax = 63: one lane per depth in one wave)
LONG63 = wl.CommitWorkload("commit_long63", 94, B=6, Kmax=63, n_layers=2, entry_bytes=48, block_size=4,
                           rec_bytes=48, ctx=(0, 40), invalid=1)
LONG63_TREE = replace(LONG63, name="commit_long63_tree", index=95, tree=True)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _expected(cw, c, use_kv=True, use_rec=True):
    acc = c["accepted_len"].copy()
    acc[c["invalid"]] = -1
    kv = c["kv"] if use_kv else np.zeros((0, 2, c["n_blocks"], cw.block_size, cw.entry_bytes), np.uint8)
    rs = c["rec_state"] if use_rec else np.zeros((cw.B, 0), np.uint8)
    sn = c["rec_snap"] if use_rec else np.zeros((cw.B, cw.Kmax + 1, 0), np.uint8)
    return oracle.commit(kv, c["seq_len"], c["block_table"], acc, c["verify_len"], rs, sn,
                         c["path"] if cw.tree else None)


def _run(cw, c, use_kv=True, use_rec=True, pass_verify_len=True):
    kv = _dev(c["kv"]) if use_kv else None
    rs = _dev(c["rec_state"]) if use_rec else None
    sn = _dev(c["rec_snap"]) if use_rec else None
    seq = _dev(c["seq_len"])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    print(f"spec_commit {cw.name} B={cw.B} Kmax={cw.Kmax} tree={cw.tree} kv={use_kv} rec={use_rec}", flush=True)
    bd.spec_commit(_dev(c["accepted_len"]), seq, Kmax=cw.Kmax, kv=kv,
                   block_table=_dev(c["block_table"]) if use_kv else None, rec_state=rs, rec_snap=sn,
                   verify_len=_dev(c["verify_len"]) if pass_verify_len else None,
                   path=_dev(c["path"]) if cw.tree else None, dev_status=status)
    torch.cuda.synchronize()
    return (kv.cpu().numpy() if use_kv else None, seq.cpu().numpy(), rs.cpu().numpy() if use_rec else None,
            int(status.item()))


@pytest.mark.parametrize("cw", [wl.COMMIT_SMALL, SMALL_TREE, LONG63, LONG63_TREE],
                         ids=["chain", "tree", "chain63", "tree63"])
@pytest.mark.parametrize("rep", [0, 1])
def test_commit_matches_oracle(cw, rep):
    c = wl.commit_case(cw, rep)
    kv_e, L_e, st_e = _expected(cw, c)
    kv, L, st, status = _run(cw, c)
    np.testing.assert_array_equal(L, L_e)
    assert np.array_equal(st, st_e), "recurrent states differ"
    assert np.array_equal(kv, kv_e), "cache bytes differ"
    assert status == (bd.SV_DEV_BAD_COMMIT if len(c["invalid"]) else bd.SV_DEV_OK)


@pytest.mark.parametrize("use_kv,use_rec", [(True, False), (False, True)], ids=["kv-only", "state-only"])
def test_commit_partial_caches(use_kv, use_rec):
    c = wl.commit_case(SMALL_TREE, 3)
    kv_e, L_e, st_e = _expected(SMALL_TREE, c, use_kv, use_rec)
    kv, L, st, _ = _run(SMALL_TREE, c, use_kv, use_rec)
    np.testing.assert_array_equal(L, L_e)
    if use_kv:
        assert np.array_equal(kv, kv_e)
    if use_rec:
        assert np.array_equal(st, st_e)


def test_commit_without_verify_len_uses_kmax():
    cw = wl.COMMIT_SMALL
    c = wl.commit_case(cw, 4)
    full = np.full(cw.B, cw.Kmax, np.int32)
    # with k_b = Kmax the case's invalid requests (A_b = k_b + 1) may fit: apply the rule to all
    acc = c["accepted_len"]
    kv_e, L_e, st_e = oracle.commit(c["kv"], c["seq_len"], c["block_table"], np.where(acc <= cw.Kmax, acc, -1), full,
                                    c["rec_state"], c["rec_snap"])
    kv, L, st, status = _run(cw, c, pass_verify_len=False)
    np.testing.assert_array_equal(L, L_e)
    assert np.array_equal(st, st_e) and np.array_equal(kv, kv_e)
    assert status == (bd.SV_DEV_BAD_COMMIT if (acc > cw.Kmax).any() else bd.SV_DEV_OK)


def test_commit_full_size_tree():
    """The benchmark's commit: B = 64, Kmax = 15, 8 layers of 2 KiB entries, 1 MiB of state."""
    cw = wl.COMMIT
    c = wl.commit_case(cw)
    kv_e, L_e, st_e = _expected(cw, c)
    kv, L, st, status = _run(cw, c)
    np.testing.assert_array_equal(L, L_e)
    assert np.array_equal(st, st_e), "recurrent states differ"
    assert np.array_equal(kv, kv_e), "cache bytes differ"
    assert status == bd.SV_DEV_OK


def _gpu_commit(s, A, k, snap, path, tree):
    kv = _dev(s.kv)
    seq = _dev(s.seq_len.astype(np.int32))
    st = _dev(s.state)
    bd.spec_commit(_dev(A.astype(np.int32)), seq, Kmax=s.Kmax, kv=kv, block_table=_dev(s.block_table),
                   rec_state=st, rec_snap=_dev(snap), verify_len=_dev(k.astype(np.int32)),
                   path=_dev(path.astype(np.int32)) if tree else None)
    torch.cuda.synchronize()
    return kv.cpu().numpy(), seq.cpu().numpy().astype(np.int64), st.cpu().numpy()


@pytest.mark.parametrize("tree", [False, True], ids=["chain", "tree"])
def test_commit_session_matches_sequential_decoding(tree):
    s = Session(ToyTarget(seed=11), Kmax=5, seed=12)
    rng = np.random.default_rng(13)
    for it in range(10):
        k = rng.integers(0, s.Kmax + 1, size=s.B)
        if it % 2 == 1:
            k[:] = 0
        tokens, parent, depth, snap = s.verify_pass(k, tree=tree)
        A, path = s.accept(k, parent, tree=tree)
        kv, L, st = _gpu_commit(s, A, k, snap, path, tree)
        s.apply(kv, L, st, tokens, A, path)
        s.check()
