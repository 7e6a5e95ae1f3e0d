"""Edge shapes of the vocabulary against the oracle: the largest vocabulary the library
accepts (2^19 tokens: 256 sampling chunks of 2048) and one-, two- and three-token
vocabularies.  Each runs through both sampled tails (B*(K+1) <= 32 rows: acceptance and
draw in the small-batch tail; more rows: the batched acceptance and draw) and greedy
verification.  A one-token vocabulary has p = q = 1 everywhere: every draft is accepted
and the bonus token is token 0; with two or three tokens rejections and residual draws
occur.  Decisions are compared as in the other parity tests."""
import numpy as np
import pytest

from draft_block_verification_spec_amd import workload as wl
from tests.test_gpu_parity import _run_greedy, _run_sample

pytestmark = pytest.mark.gpu

V_MAX = 1 << 19


def _wk(V, B, seed):
    return wl.Workload(f"v{V}_b{B}", seed, B=B, K=3, d=64, d_ff=0, V=V, T=1.0, sigma=0.4)


@pytest.mark.parametrize("B", [2, 12], ids=["small-tail", "batched-tail"])
def test_sample_parity_max_vocabulary(B):
    _run_sample(_wk(V_MAX, B, 40 + B))


def test_greedy_parity_max_vocabulary():
    _run_greedy(_wk(V_MAX, 12, 43))


@pytest.mark.parametrize("V", [1, 2, 3])
@pytest.mark.parametrize("B", [4, 16], ids=["small-tail", "batched-tail"])
def test_sample_parity_tiny_vocabularies(V, B):
    ref, out, _ = _run_sample(_wk(V, B, 50 + 4 * V + B))
    if V == 1:
        assert np.all(out.accepted_len.cpu().numpy() == 3)
        assert np.all(out.emitted.cpu().numpy() == 0)


@pytest.mark.parametrize("V", [1, 2, 3])
def test_greedy_parity_tiny_vocabularies(V):
    wk = _wk(V, 16, 70 + V)
    ref, out = _run_greedy(wk)
    if V == 1:
        assert np.all(out.accepted_len.cpu().numpy() == wk.K)
