"""Greedy acceptance of speculative draft tokens, written out plainly.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the HIP library shares no code with it.

Verify row 0 of a request holds its pending token and row t (t >= 1) the
draft token d_t; g_t is the target model's greedy token after row t
(FreeToken PR #844, Design: the target scores [pending, d1..dk] and n tokens
are accepted). Speculative decoding must reproduce greedy decoding token for
token (FreeToken issue #828, Design), so d_{t+1} is kept only if it equals
g_t, the token greedy decoding would emit after row t, and every earlier
draft was kept. The accept length n counts the pending row and the kept
drafts (at most k + 1: FreeToken PR #844, End-to-end); the target's greedy
token after the last kept row, g_{n-1}, is the next pending token. A padding
request (slot id -1) accepts nothing.
"""
import numpy as np


def greedy_accept(draft, target, slot_ids=None):
    """draft [B][R-1], target [B][R] int -> (accept_len [B], next_token [B]) int32."""
    target = np.asarray(target)
    B, R = target.shape
    draft = np.asarray(draft).reshape(B, R - 1)
    accept = np.zeros(B, np.int32)
    nxt = np.full(B, -1, np.int32)
    for b in range(B):
        if slot_ids is not None and int(slot_ids[b]) == -1:
            continue
        n = 1
        for t in range(1, R):
            if int(draft[b][t - 1]) != int(target[b][t - 1]):
                break
            n += 1
        accept[b] = n
        nxt[b] = int(target[b][n - 1])
    return accept, nxt
