"""Seeded synthetic inputs for the draft-block verification step.

This module only *draws* data: weights, hidden states, draft noise and uniform
coins, rounded to bf16 bit patterns.  It holds none of the verification
arithmetic (no matmul, no softmax, no acceptance rule), so the oracle and the
GPU library can both consume what it returns without sharing any of the
method's code.

Recipe (every array is reproducible from ``seed = 20261202 + 100*index + repeat``):

* One child ``SeedSequence`` per stream, in this order: LM head, gate, up,
  down, target hidden, draft noise, draft-sampling coins, verify coins,
  per-request parameters.  Large streams are cut into chunks of 2**22
  elements, each chunk with its own grandchild seed, so generation can run on
  several threads and still be deterministic.
* Normals are drawn in fp32, scaled in fp32 and rounded to bf16
  (round-to-nearest-even on the fp32 bit pattern).
* ``W_lm ~ N(0, lm_scale**2 / d)``; ``W_gate, W_up ~ N(0, 1/d)``;
  ``W_down ~ N(0, 1/d_ff)`` (fan-in scaling; the pages give no MLP scale).
* ``h ~ N(0, 1)`` of shape ``[B, K+1, d]``; the draft hidden is
  ``gain_b * (h[:, :K] + sigma_b * eps)`` (MTP/EAGLE-style perturbation of the
  same rows), with ``sigma_b`` fixed or uniform per request and ``gain_b`` 1 or
  log-uniform per request.
* Coins are fp32 multiples of 2**-24 in [0, 1): ``draft_coins [B, K]`` drive
  the drafter's own sampling, ``coins [B, K+1]`` drive verification
  (``coins[:, j]`` for draft position j+1, ``coins[:, K]`` for the final sample).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
import os

import numpy as np

BASE_SEED = 20261202
CHUNK = 1 << 22
_STREAMS = ("w_lm", "w_gate", "w_up", "w_down", "h", "noise", "draft_coins", "coins", "params")


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic verification batch."""

    name: str
    index: int            # seed slot
    B: int                # concurrent requests
    K: int                # draft tokens per request (K_max in scheduled mode)
    d: int                # hidden size
    d_ff: int             # SwiGLU width; 0 = no MLP (y = h)
    V: int                # vocabulary
    T: float = 1.0        # temperature used by sampled / scheduled verification
    sigma: float | tuple = 0.5      # draft noise std, or (lo, hi) uniform per request
    gain: tuple | None = None       # (lo, hi) log-uniform per-request gain on the draft hidden
    lm_scale: float = 2.5
    threshold: float = 0.3          # survival threshold (scheduled mode)
    budget: int = 0                 # verified-position budget (scheduled mode)

    @property
    def M_t(self) -> int:
        return self.B * (self.K + 1)

    def with_batch(self, B: int) -> "Workload":
        return replace(self, B=B)

    def weight_bytes(self) -> int:
        return 2 * (self.V * self.d + 3 * self.d * self.d_ff)


# Presets.  Shapes follow the pages' workloads: a 16-token parallel-drafter block
# (K=15), K=7 parallel drafters under load, a DSpark-style scheduled batch, and a
# short MTP-like draft on a wide model.
TINY = Workload("tiny", 0, B=1, K=4, d=64, d_ff=0, V=512, T=1.0, sigma=0.5)
BLOCK16 = Workload("block16", 1, B=1, K=15, d=4096, d_ff=12288, V=151936, T=1.0, sigma=0.7)
SWEEP = Workload("sweep", 2, B=128, K=7, d=4096, d_ff=12288, V=151936, T=1.0, sigma=(0.3, 1.2))
SCHED = Workload("sched", 3, B=64, K=15, d=4096, d_ff=12288, V=151936, T=1.0, sigma=(0.3, 1.2),
                 threshold=0.3, budget=512)
SCHED_STRESS = replace(SCHED, name="sched_stress", gain=(4.0, 32.0))
WIDE = Workload("wide", 4, B=32, K=4, d=8192, d_ff=28672, V=128256, T=0.7, sigma=0.6)

# Reduced shapes that the oracle finishes in seconds while still spanning several
# GPU tiles and a ragged tail in every dimension the kernels tile.
SMALL = Workload("small", 10, B=3, K=5, d=256, d_ff=512, V=5003, T=1.0, sigma=0.4)
SMALL_WIDE = Workload("small_wide", 11, B=5, K=4, d=512, d_ff=1536, V=12347, T=0.7, sigma=0.6)
SMALL_BATCH = Workload("small_batch", 12, B=40, K=7, d=256, d_ff=768, V=4099, T=1.0, sigma=(0.3, 1.2))
SMALL_SCHED = Workload("small_sched", 13, B=24, K=15, d=256, d_ff=512, V=3001, T=1.0, sigma=(0.3, 1.2),
                       gain=(4.0, 32.0), threshold=0.3, budget=96)

PRESETS = {w.name: w for w in (TINY, BLOCK16, SWEEP, SCHED, SCHED_STRESS, WIDE,
                               SMALL, SMALL_WIDE, SMALL_BATCH, SMALL_SCHED)}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round-to-nearest-even on the integer representation."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(ss: np.random.SeedSequence, shape, scale: float) -> np.ndarray:
    """N(0, scale**2) drawn in fp32 and rounded to bf16 bits, chunked over threads."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nchunks = max(1, -(-n // CHUNK))
    kids = ss.spawn(nchunks)
    s32 = np.float32(scale)

    def work(i):
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        x = g.standard_normal(hi - lo, dtype=np.float32)
        x *= s32
        out[lo:hi] = f32_to_bf16_bits(x)

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def _normal_f32(ss: np.random.SeedSequence, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, -(-n // CHUNK))
    kids = ss.spawn(nchunks)
    for i in range(nchunks):
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        np.random.Generator(np.random.PCG64(kids[i])).standard_normal(hi - lo, dtype=np.float32,
                                                                       out=out[lo:hi])
    return out.reshape(shape)


def _coins(ss: np.random.SeedSequence, shape) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(ss))
    return (g.integers(0, 1 << 24, size=shape, dtype=np.int64).astype(np.float32)
            * np.float32(2.0 ** -24))


def seed_for(w: Workload, repeat: int = 0) -> int:
    return BASE_SEED + 100 * w.index + repeat


def generate(w: Workload, repeat: int = 0, *, weights: bool = True, keep_f32: bool = False) -> dict:
    """Draw one batch.

    Returns a dict of numpy arrays: bf16 bit patterns (uint16) for ``w_lm``,
    ``w_gate``, ``w_up``, ``w_down`` (absent when ``d_ff == 0``), ``h``
    ``[B, K+1, d]`` and ``h_draft`` ``[B, K, d]``; fp32 ``draft_coins [B, K]``,
    ``coins [B, K+1]``, ``sigma [B]``, ``gain [B]``.  With ``keep_f32`` the
    unrounded fp32 ``h_f32``, ``h_draft_f32`` and ``w_lm_f32`` are kept too (the
    tiny configuration's statistics are taken on fp32 values).
    """
    root = np.random.SeedSequence(seed_for(w, repeat))
    ss = dict(zip(_STREAMS, root.spawn(len(_STREAMS))))
    out: dict = {}
    B, K, d = w.B, w.K, w.d
    if weights:
        if keep_f32:
            wl = _normal_f32(ss["w_lm"], (w.V, d)) * np.float32(w.lm_scale / np.sqrt(d))
            out["w_lm_f32"] = wl
            out["w_lm"] = f32_to_bf16_bits(wl)
        else:
            out["w_lm"] = _normal_bf16(ss["w_lm"], (w.V, d), w.lm_scale / np.sqrt(d))
        if w.d_ff:
            out["w_gate"] = _normal_bf16(ss["w_gate"], (w.d_ff, d), 1.0 / np.sqrt(d))
            out["w_up"] = _normal_bf16(ss["w_up"], (w.d_ff, d), 1.0 / np.sqrt(d))
            out["w_down"] = _normal_bf16(ss["w_down"], (d, w.d_ff), 1.0 / np.sqrt(w.d_ff))
    g = np.random.Generator(np.random.PCG64(ss["params"]))
    if isinstance(w.sigma, tuple):
        sigma = g.uniform(w.sigma[0], w.sigma[1], size=B).astype(np.float32)
    else:
        sigma = np.full(B, w.sigma, dtype=np.float32)
    if w.gain is not None:
        lo, hi = np.log(w.gain[0]), np.log(w.gain[1])
        gain = np.exp(g.uniform(lo, hi, size=B)).astype(np.float32)
    else:
        gain = np.ones(B, dtype=np.float32)
    h32 = _normal_f32(ss["h"], (B, K + 1, d))
    eps = _normal_f32(ss["noise"], (B, K, d))
    hd32 = gain[:, None, None] * (h32[:, :K, :] + sigma[:, None, None] * eps)
    out["h"] = f32_to_bf16_bits(h32)
    out["h_draft"] = f32_to_bf16_bits(hd32)
    if keep_f32:
        out["h_f32"] = h32
        out["h_draft_f32"] = hd32.astype(np.float32)
    out["draft_coins"] = _coins(ss["draft_coins"], (B, K))
    out["coins"] = _coins(ss["coins"], (B, K + 1))
    out["sigma"] = sigma
    out["gain"] = gain
    return out


def to_fp8(data: dict) -> dict:
    """FP8 copy of a batch's weights: for every matrix (``lm``, ``gate``, ``up``,
    ``down``) one fp32 scale per output row, ``s = max|w_row| / 448``, and the E4M3
    codes of ``w / s`` (``q_*``, uint8, rounded to nearest even by torch's float8
    conversion).  The bf16 weights are dropped; activations and coins are kept."""
    import torch

    out = {k: v for k, v in data.items() if not k.startswith("w_")}
    for name in ("lm", "gate", "up", "down"):
        bits = data.get("w_" + name)
        if bits is None:
            continue
        w = torch.from_numpy(np.ascontiguousarray(bits).astype(np.int32) << 16).view(torch.float32)
        amax = w.abs().amax(dim=1).clamp_min(torch.finfo(torch.float32).tiny)
        scale = (amax / 448.0).to(torch.float32)
        q = (w / scale[:, None]).to(torch.float8_e4m3fn)
        out["q_" + name] = q.view(torch.uint8).numpy()
        out["s_" + name] = scale.numpy()
    return out


@dataclass(frozen=True)
class CommitWorkload:
    """Cached target state around one commit: a paged KV cache and recurrent states.

    ``ctx``: cache length range before the verify block; ``tree``: verify blocks are
    random trees (node j's parent uniform in 0..j-1) instead of chains."""
    name: str
    index: int
    B: int
    Kmax: int
    n_layers: int
    entry_bytes: int
    block_size: int
    rec_bytes: int
    ctx: tuple = (0, 64)
    tree: bool = False
    invalid: int = 0  # requests given an accepted length or path that does not fit (for error tests)


# The confidence-scheduled batch (B = 64, 16-token blocks) on a hybrid target: 8 attention
# layers with 8 KV heads x 128 bf16 values per token (2 KiB entries) and 1 MiB of
# linear-attention state per request; tree-shaped verify blocks.
COMMIT = CommitWorkload("commit", 20, B=64, Kmax=15, n_layers=8, entry_bytes=2048, block_size=16,
                        rec_bytes=1 << 20, ctx=(256, 768), tree=True)
COMMIT_SMALL = CommitWorkload("commit_small", 21, B=12, Kmax=7, n_layers=3, entry_bytes=48, block_size=4,
                              rec_bytes=(1 << 15) + 48, ctx=(0, 40), tree=False, invalid=2)


def commit_case(cw: CommitWorkload, repeat: int = 0, *, big: bool = True) -> dict:
    """Seeded inputs of one commit.  Small int32 arrays always; with ``big`` also the byte
    arrays (kv [n_layers, 2, n_blocks, block_size, entry_bytes], rec_state [B, rec_bytes],
    rec_snap [B, Kmax+1, rec_bytes]) as uint8.  Verify lengths k_b are uniform in 0..Kmax
    (k_b = 0 for a quarter of the requests); a chain accepts a uniform prefix length, a tree
    accepts the root path of a uniform node; ``invalid`` requests get A_b = k_b + 1 (chain)
    or a path that is not increasing (tree); one request in eight is flagged (A_b = -1)."""
    rng = np.random.default_rng(BASE_SEED + 100 * cw.index + repeat)
    B, K1 = cw.B, cw.Kmax + 1
    seq_len = rng.integers(cw.ctx[0], cw.ctx[1] + 1, size=B).astype(np.int32)
    k = rng.integers(0, K1, size=B).astype(np.int32)
    k[rng.random(B) < 0.25] = 0
    max_blocks = (int(seq_len.max()) + K1 + cw.block_size - 1) // cw.block_size + 1
    n_blocks = B * max_blocks + 3
    block_table = rng.permutation(n_blocks)[: B * max_blocks].reshape(B, max_blocks).astype(np.int32)
    acc = np.zeros(B, np.int32)
    path = np.zeros((B, K1), np.int32)
    for b in range(B):
        if cw.tree:
            parent = [-1] + [int(rng.integers(j)) for j in range(1, k[b] + 1)]
            node = int(rng.integers(k[b] + 1))
            chain = [node]
            while chain[-1] != 0:
                chain.append(parent[chain[-1]])
            chain.reverse()
        else:
            chain = list(range(int(rng.integers(k[b] + 1)) + 1))
        acc[b] = len(chain) - 1
        path[b, : len(chain)] = chain
    acc[rng.random(B) < 0.125] = -1
    bad = rng.choice(B, size=cw.invalid, replace=False) if cw.invalid else np.zeros(0, np.int64)
    for b in bad:
        if cw.tree and acc[b] >= 1:
            path[b, 1] = path[b, 0]
        else:
            acc[b] = k[b] + 1
    out = {"seq_len": seq_len, "verify_len": k, "accepted_len": acc, "path": path, "block_table": block_table,
           "n_blocks": n_blocks, "invalid": np.asarray(bad, np.int64)}
    if big:
        out["kv"] = rng.integers(0, 256, size=(cw.n_layers, 2, n_blocks, cw.block_size, cw.entry_bytes), dtype=np.uint8)
        out["rec_state"] = rng.integers(0, 256, size=(B, cw.rec_bytes), dtype=np.uint8)
        out["rec_snap"] = rng.integers(0, 256, size=(B, K1, cw.rec_bytes), dtype=np.uint8)
    return out


def tree_parents(B: int, K: int, kind: str = "topk", seed: int = 0) -> np.ndarray:
    """Parents [B, K] of verify trees of K+1 nodes (node j+1's parent in 0..j).

    ``chain``: node j+1 follows node j.  ``random``: parent uniform in 0..j.  ``topk``: the
    shape of an EAGLE-style tree built with top-k candidates per draft step (SGLang's
    num-steps / eagle-topk / num-draft-tokens), breadth first: the root has 4 children,
    every depth-1 node 2, every deeper node 1, in node order until K nodes exist."""
    if kind == "chain":
        return np.tile(np.arange(K, dtype=np.int32), (B, 1))
    if kind == "random":
        rng = np.random.default_rng(BASE_SEED + 7 + seed)
        return np.array([[rng.integers(j + 1) for j in range(K)] for _ in range(B)], np.int32).reshape(B, K)
    assert kind == "topk"
    par, level = [], [0]
    while len(par) < K:
        nxt = []
        for u in level:
            fan = 4 if u == 0 else (2 if par[u - 1] == 0 else 1)
            for _ in range(fan):
                if len(par) < K:
                    par.append(u)
                    nxt.append(len(par))
        level = nxt
    return np.tile(np.array(par, np.int32), (B, 1))
