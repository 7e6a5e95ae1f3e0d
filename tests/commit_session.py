"""A toy hybrid target for testing the commit step (test infrastructure).

Every attention layer caches one entry per token whose bytes depend on the token and
its position (so a misplaced or stale entry is visible), and one recurrent layer keeps
the state S <- lam * S + k(t) v(t)^T in float64 (so a state taken one input too early or
too late is visible).  A verify pass writes the entries and state snapshots of its
inputs the way a target forward does; ``sequential`` feeds committed tokens one at a
time, which is what speculative decoding must reproduce ([MISHA] "The KV cache and
speculative decoding work together"; [WB] n-gram pitfalls on the hybrid model).
"""
from __future__ import annotations

import numpy as np

LAM = 0.9


class ToyTarget:
    def __init__(self, n_layers=2, entry_bytes=16, vocab=40, max_pos=160, dk=2, seed=0):
        rng = np.random.default_rng(seed)
        self.entry = rng.integers(0, 256, size=(n_layers, 2, vocab, max_pos, entry_bytes), dtype=np.uint8)
        self.kvec = rng.standard_normal((vocab, dk))
        self.vvec = rng.standard_normal((vocab, dk))
        self.n_layers, self.entry_bytes, self.vocab, self.dk = n_layers, entry_bytes, vocab, dk

    @property
    def rec_bytes(self) -> int:
        return self.dk * self.dk * 8

    def step_state(self, S, t):
        return LAM * S + np.outer(self.kvec[t], self.vvec[t])

    def sequential(self, tokens):
        """Cache entries [n_layers, 2, len, entry_bytes] and final state of feeding tokens."""
        ent = np.stack([self.entry[:, :, t, p] for p, t in enumerate(tokens)], axis=2) if tokens else \
            np.zeros((self.n_layers, 2, 0, self.entry_bytes), np.uint8)
        S = np.zeros((self.dk, self.dk))
        for t in tokens:
            S = self.step_state(S, t)
        return ent, S


class Session:
    """B requests over a paged cache: verify passes write, a commit function keeps."""

    def __init__(self, target: ToyTarget, B=3, block_size=4, n_blocks=200, max_blocks=40, Kmax=5, seed=1):
        self.t = target
        self.B, self.bs, self.Kmax = B, block_size, Kmax
        self.rng = np.random.default_rng(seed)
        self.kv = self.rng.integers(0, 256, size=(target.n_layers, 2, n_blocks, block_size, target.entry_bytes),
                                    dtype=np.uint8)
        perm = self.rng.permutation(n_blocks)[: B * max_blocks]
        self.block_table = perm.reshape(B, max_blocks).astype(np.int32)
        self.seq_len = np.zeros(B, np.int64)
        self.state = np.zeros((B, target.rec_bytes), np.uint8)
        self.committed = [[] for _ in range(B)]  # tokens with a cache entry, in order
        self.next_input = [int(self.rng.integers(target.vocab)) for _ in range(B)]

    def _slot(self, b, pos):
        return self.block_table[b, pos // self.bs], pos % self.bs

    def _state_of(self, b):
        return self.state[b].view(np.float64).reshape(self.t.dk, self.t.dk)

    def verify_pass(self, k, tree=False):
        """Write the entries and snapshots of one verify block per request.

        Chain: inputs [next_input, d_1 .. d_k].  Tree: node 0 = next_input, node j has a
        parent in 0..j-1 and sits at cache slot L + j with position L + depth(j).
        Returns (tokens [B, Kmax+1], parent [B, Kmax+1], depth [B, Kmax+1], snap)."""
        B, K1 = self.B, self.Kmax + 1
        tokens = np.zeros((B, K1), np.int64)
        parent = np.full((B, K1), -1, np.int64)
        depth = np.zeros((B, K1), np.int64)
        snap = np.zeros((B, K1, self.t.rec_bytes), np.uint8)
        for b in range(B):
            L = int(self.seq_len[b])
            tokens[b, 0] = self.next_input[b]
            for j in range(1, k[b] + 1):
                tokens[b, j] = self.rng.integers(self.t.vocab)
                parent[b, j] = self.rng.integers(j) if tree else j - 1
                depth[b, j] = depth[b, parent[b, j]] + 1
            S0 = self._state_of(b)
            states = []
            for j in range(k[b] + 1):
                prev = S0 if j == 0 else states[parent[b, j]]
                states.append(self.t.step_state(prev, tokens[b, j]))
                snap[b, j] = states[-1].reshape(-1).view(np.uint8)
                blk, off = self._slot(b, L + j)
                self.kv[:, :, blk, off] = self.t.entry[:, :, tokens[b, j], L + depth[b, j]]
        return tokens, parent, depth, snap

    def accept(self, k, parent, tree=False):
        """Random acceptance: a chain prefix length, or a random tree node's root path."""
        A = np.zeros(self.B, np.int64)
        path = np.zeros((self.B, self.Kmax + 1), np.int64)
        for b in range(self.B):
            if tree:
                node = int(self.rng.integers(k[b] + 1))
                chain = [node]
                while chain[-1] != 0:
                    chain.append(int(parent[b, chain[-1]]))
                chain.reverse()
            else:
                chain = list(range(int(self.rng.integers(k[b] + 1)) + 1))
            A[b] = len(chain) - 1
            path[b, : len(chain)] = chain
        return A, path

    def apply(self, new_kv, new_seq_len, new_state, tokens, A, path):
        """Take a commit's results and record the tokens it committed."""
        self.kv, self.seq_len, self.state = new_kv, np.asarray(new_seq_len, np.int64), new_state
        for b in range(self.B):
            if A[b] < 0:
                continue
            self.committed[b] += [int(tokens[b, j]) for j in path[b, : A[b] + 1]]
            self.next_input[b] = int(self.rng.integers(self.t.vocab))

    def check(self):
        """The cache and state equal feeding the committed tokens one at a time."""
        for b in range(self.B):
            ent, S = self.t.sequential(self.committed[b])
            n = len(self.committed[b])
            assert int(self.seq_len[b]) == n, f"request {b}: cache length {self.seq_len[b]} != {n} committed"
            for p in range(n):
                blk, off = self._slot(b, p)
                if not np.array_equal(self.kv[:, :, blk, off], ent[:, :, p]):
                    raise AssertionError(f"request {b}: cache entry at position {p} is not token {p}'s")
            if not np.array_equal(self._state_of(b), S):
                raise AssertionError(f"request {b}: recurrent state differs from sequential decoding")
