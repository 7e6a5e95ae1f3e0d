"""Tree (multi-candidate) verification.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: [MISHA] "EAGLE" (EAGLE-2 builds the candidate tree dynamically) and "Medusa"
(several continuations assembled into a candidate tree and checked by the target in
one pass with tree attention); [VLLM26] SGLang EAGLE-3 settings (draft steps = depth,
top-k candidates per step, a token budget for verification).  The pages state no
acceptance rule for a tree.  Reading R15:

* a verify tree has N = K + 1 nodes per request; node 0 is the last emitted token, node
  j >= 1 carries draft token tokens[j-1] and has parent parent[j-1] < j (parents come
  first); the target row of node j gives p_j (its distribution for the next token), the
  draft row of node j gives q_j, the distribution node j's children were drawn from;
* greedy: from the root, move to the first child (lowest index) whose token is the
  target argmax at the current node; stop when no child matches and emit that argmax;
* sampled: Statement 1 ([WB] "A bit of theory") applied to the children of the current
  node one after another, in index order: child c with token x passes when
  coins[c-1] < min(1, r(x) / q_u(x)), where r starts as p_u and after each rejected
  child becomes the normalised max(0, r - q_u) (p_u again if that is all zero, as in
  the chain's fallback); the first child that passes becomes the current node; when
  every child fails, or the node has none, the emitted token is drawn from r by inverse
  CDF with coins[N-1].  With a chain (parent of node j+1 is node j) both rules are the
  chain rules exactly.
"""
from __future__ import annotations

import numpy as np

from .verify import (Weights, inverse_cdf, lm_logits, softmax_t, target_hidden)


def children(parent_row, N: int) -> list[list[int]]:
    """Children of every node of one request's tree, in increasing index order."""
    ch = [[] for _ in range(N)]
    for j in range(1, N):
        ch[int(parent_row[j - 1])].append(j)
    return ch


def next_residual(r, q_u, p_u):
    """The distribution after a rejected child: normalised max(0, r - q_u), or p_u when
    that is all zero.  Returns (r', fell_back)."""
    w = np.maximum(0.0, r - q_u)
    s = w.sum()
    if s > 0.0:
        return w / s, False
    return p_u.copy(), True


def accept_tree_greedy(z_t, tokens, parent) -> dict:
    """z_t: [B, N, V] target logits per node; tokens, parent: [B, N-1] (node j+1)."""
    z_t = np.asarray(z_t, dtype=np.float64)
    B, N, _ = z_t.shape
    amax = z_t.argmax(axis=-1)
    acc = np.zeros(B, np.int64)
    path = np.full((B, N), -1, np.int64)
    emitted = np.full((B, N), -1, np.int64)
    for b in range(B):
        ch = children(parent[b], N)
        node, depth = 0, 0
        path[b, 0] = 0
        while True:
            nxt = [c for c in ch[node] if int(tokens[b, c - 1]) == amax[b, node]]
            if not nxt:
                emitted[b, depth] = amax[b, node]
                break
            node = nxt[0]
            depth += 1
            path[b, depth] = node
            emitted[b, depth - 1] = int(tokens[b, node - 1])
        acc[b] = depth
    return {"accepted": acc, "path": path, "emitted": emitted, "argmax": amax}


def accept_tree_sample(p, q, tokens, parent, coins) -> dict:
    """p: [B, N, V] target distributions per node; q: [B, N-1, V] draft distributions at
    nodes 0..N-2; tokens, parent: [B, N-1]; coins: [B, N] (coins[j-1] tests node j,
    coins[N-1] draws the emitted token).  Also returns every decision taken (node tested,
    ratio, coin) and the CDF bounds of the final draw, to classify near ties."""
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    coins = np.asarray(coins, dtype=np.float64)
    B, N, _ = p.shape
    acc = np.zeros(B, np.int64)
    path = np.full((B, N), -1, np.int64)
    emitted = np.full((B, N), -1, np.int64)
    decisions = [[] for _ in range(B)]
    cdf = np.zeros((B, 2))
    fallback = np.zeros(B, bool)
    for b in range(B):
        ch = children(parent[b], N)
        node, depth = 0, 0
        path[b, 0] = 0
        while True:
            r = p[b, node].copy()
            moved = False
            for c in ch[node]:
                x = int(tokens[b, c - 1])
                qx = q[b, node, x]
                ratio = r[x] / qx if qx > 0 else np.inf
                ok = coins[b, c - 1] < min(1.0, ratio)
                decisions[b].append((c, ratio, coins[b, c - 1], ok))
                if ok:
                    node = c
                    depth += 1
                    path[b, depth] = c
                    emitted[b, depth - 1] = x
                    moved = True
                    break
                r, fb = next_residual(r, q[b, node], p[b, node])
                fallback[b] |= fb
            if not moved:
                v, lo, hi = inverse_cdf(r, coins[b, N - 1])
                emitted[b, depth] = int(v)
                cdf[b] = (lo, hi)
                break
        acc[b] = depth
    return {"accepted": acc, "path": path, "emitted": emitted, "decisions": decisions, "cdf": cdf,
            "fallback": fallback}


def verify_tree_greedy(w: Weights, h, tokens, parent) -> dict:
    """h: [B, N, d] target hidden rows per node (fp64 values of bf16 inputs)."""
    z_t = lm_logits(w.w_lm, target_hidden(h, w))
    out = accept_tree_greedy(z_t, tokens, parent)
    out["logits_t"] = z_t
    return out


def verify_tree_sample(w: Weights, h, h_draft, tokens, parent, coins, T: float) -> dict:
    """h: [B, N, d]; h_draft: [B, N-1, d] draft rows of nodes 0..N-2."""
    z_t = lm_logits(w.w_lm, target_hidden(h, w))
    z_d = lm_logits(w.w_lm, h_draft)
    out = accept_tree_sample(softmax_t(z_t, T), softmax_t(z_d, T), tokens, parent, coins)
    out["logits_t"] = z_t
    out["logits_d"] = z_d
    return out
