"""Commit after verification: cached target state kept for the accepted prefix only.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* [MISHA] "The KV cache and speculative decoding work together": the target checks the whole
  speculative block and keeps its cached state only for the part that was accepted; the
  work done for the rejected tail is thrown away.
* [WB] "Why hybrid attention matters for speculation" and the n-gram pitfalls: on a
  hybrid model (linear-attention layers beside full attention) the engine corrupted
  answers when it mishandled the linear-attention recurrent state across steps with and
  without a draft.

Reading R14 (the pages give the idea, not the bookkeeping):
* the verify pass of request b feeds k_b + 1 inputs - the last emitted token (input 0)
  and the k_b drafts - and the target's forward wrote their keys/values at cache
  positions L_b + j (L_b = seq_len[b], the tokens already cached), and the state of every
  recurrent layer after input j into snapshot j;
* after acceptance of A_b drafts, inputs 0 .. A_b are the committed ones: their cache
  entries stay, the cache length becomes L_b + A_b + 1, the entries beyond are dropped,
  and each recurrent state becomes snapshot A_b.  A step without a draft (k_b = 0) commits
  its one input the same way (snapshot 0);
* tree verification: node j of the verified tree was written at L_b + j, and the accepted
  path p_0 = 0, p_1, ..., p_A (node of depth i at p_i) is moved to positions L_b + i; the
  recurrent state becomes the snapshot of node p_A;
* a request whose accepted length is negative (a verify call flagged its inputs) is left
  unchanged.

Cache layout (bytes): kv[layer, half, block, slot] holds one token's keys (half 0) or
values (half 1) for one layer; position p of request b lives in block
block_table[b, p // block_size] at slot p % block_size.
"""
from __future__ import annotations

import numpy as np


def commit(kv, seq_len, block_table, accepted_len, verify_len, rec_state, rec_snap, path=None):
    """Apply the commit of reading R14 and return (kv, seq_len, rec_state) as new arrays.

    kv: uint8 [n_layers, 2, n_blocks, block_size, entry_bytes] (may have n_layers = 0);
    seq_len: [B]; block_table: [B, max_blocks]; accepted_len: [B]; verify_len: [B];
    rec_state: uint8 [B, rec_bytes]; rec_snap: uint8 [B, Kmax + 1, rec_bytes];
    path: [B, Kmax + 1] node index of the accepted path at each depth, or None (chain).
    """
    kv = np.array(kv, copy=True)
    rec_state = np.array(rec_state, copy=True)
    seq_len = np.array(seq_len, dtype=np.int64, copy=True)
    bs = kv.shape[3]
    B = len(seq_len)
    for b in range(B):
        A = int(accepted_len[b])
        if A < 0:
            continue
        assert A <= int(verify_len[b])
        L = int(seq_len[b])
        nodes = list(range(A + 1)) if path is None else [int(x) for x in path[b][: A + 1]]
        for i, j in enumerate(nodes):
            if j == i:
                continue
            src, dst = L + j, L + i
            sb, so = block_table[b][src // bs], src % bs
            db, do = block_table[b][dst // bs], dst % bs
            kv[:, :, db, do, :] = kv[:, :, sb, so, :]
        seq_len[b] = L + A + 1
        rec_state[b] = rec_snap[b, nodes[-1]]
    return kv, seq_len, rec_state
