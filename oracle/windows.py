"""Per-slot window states committed after the accepted rows, written out plainly.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the HIP library shares no code with it.

What it computes (FreeToken PR #844 "MTP drafts for the Qwen3.5 family and
Flash-Next", Design: besides the GDN state, a slot carries other states, a
second conv history and an n-gram context of token ids; the verify reads
their live values and stages, per verify row, what that row appends; the
commit then restores each of them as it stands after the accepted rows,
sharing one upload of the slot and count indices with the GDN commit).

Reading (parity unpinned for the layout, which the page does not give): a
window state holds, per slot, the last L entries of its stream, oldest first,
each entry a fixed number of bytes. Verify row t of request b stages the
entry that row appends, rows[b][t]. Committing n accepted rows replaces the
slot's window with the last L entries of [window (L entries) | rows[b][0..n-1]],
that is entries n .. n+L-1 of the concatenation. n = 0 leaves the slot as it
is; a padding request (slot id -1) is skipped; a slot id outside [-1, P) or an
accept length outside [0, R] skips the request and sets bit 0 or bit 1 of the
returned error word, as the GDN commit does.

The GDN conv history is one such window (entries of C channels, L = W - 1):
the tests check that this function and the C oracle's conv commit agree.
"""
from __future__ import annotations

import numpy as np

ERR_SLOT = 1
ERR_ACCEPT = 2


def commit_window(state, rows, slot_ids, accept_len):
    """state [P][L][...] (updated in place), rows [B][R][...] of the same
    entry shape and dtype, slot_ids [B], accept_len [B]. Returns the error
    word (bit 0: slot id out of range, bit 1: accept length out of range)."""
    state = np.asarray(state)
    rows = np.asarray(rows)
    P, L = state.shape[0], state.shape[1]
    B, R = rows.shape[0], rows.shape[1]
    err = 0
    for b in range(B):
        s, n = int(slot_ids[b]), int(accept_len[b])
        if s == -1:
            continue
        if s < -1 or s >= P:
            err |= ERR_SLOT
            continue
        if n < 0 or n > R:
            err |= ERR_ACCEPT
            continue
        if n == 0:
            continue
        window = np.concatenate([state[s], rows[b, :n]], axis=0)   # L + n entries, oldest first
        state[s] = window[n:n + L]
    return err
