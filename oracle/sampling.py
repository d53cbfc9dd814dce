"""Speculative (rejection) sampling of draft tokens, written out plainly.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the HIP library shares no code with it.

What it computes (FreeToken issue #828 "Speculative decoding: MTP and
DFlash", Plan: the target side verifies drafts with rejection sampling and
per-row presence and frequency penalties; lmdeploy PR #5006, What's included,
Verification path: speculative sampling op kernels). The pages print no
formula; this is the standard speculative sampling rule, which keeps the
emitted tokens distributed exactly as the target's own sampling would:

  Verify row 0 of request b holds its pending token, row t (1 <= t < R) the
  draft token d_t. Row t's target distribution p_t is the softmax of its
  logits after the penalties, divided by the temperature T:

      l'_t[v] = l_t[v] - frequency * c_t[v] - presence * [c_t[v] > 0]
      p_t     = softmax(l'_t / T)

  where c_t[v] counts v among the request's earlier output (prior_counts)
  and the tokens of rows 0..t (the pending token and d_1..d_t): row t sees
  the tokens decoding would have emitted before it ("per-row" penalties).

  For t = 0 .. R-2, draft d_{t+1} (drawn by the drafter from q_t) is accepted
  when u_t * q_t(d_{t+1}) <= p_t(d_{t+1}) with u_t uniform in [0, 1), i.e. with
  probability min(1, p_t / q_t). The first rejection at row t ends the run:
  accept_len = t + 1 rows are committed and the next pending token is drawn
  from the residual max(0, p_t - q_t) (normalised). If every draft is
  accepted, accept_len = R and the next token is drawn from p_{R-1}.
  Without draft probabilities the drafter is taken to be greedy: q_t is one
  on d_{t+1} and zero elsewhere.

Random numbers. Both draws are Gumbel-max draws, argmax_v (log w_v + G_v)
with G_v = -log(-log U_v), which samples v with probability w_v / sum(w):
no cumulative sum decides the index, so the oracle and the device agree on
it whenever the two best keys are not within rounding of each other. U comes
from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
Easy as 1, 2, 3", SC'11), keyed by the call's 64-bit seed:
  - G of row t, vocab entry v: counter (v >> 2, t, b, 0), word v & 3;
  - u_t: counter (0, t, b, 1), word 0;
  - U = (2 * (word >> 9) + 1) / 2^24: the top 23 bits as an odd fraction,
    in (0, 1) and exact in fp32 as well as fp64.

Reading where the pages are silent (parity unpinned: no page value fixes
them): the penalties act on the logits before the temperature, the pending
token (when given) counts towards every row's penalties, a zero draft
probability accepts the draft, and padding requests (slot id -1) get
accept_len 0 and next token -1.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds, elementwise over broadcast uint64 arrays
    holding 32-bit values: ctr = (c0, c1, c2, c3), key = (k0, k1). Returns
    the four output words."""
    c0, c1, c2, c3 = (np.asarray(x, np.uint64) & MASK for x in ctr)
    k0, k1 = (np.asarray(x, np.uint64) & MASK for x in key)
    for r in range(10):
        if r:
            k0 = (k0 + W0) & MASK
            k1 = (k1 + W1) & MASK
        p0 = np.uint64(M0) * c0          # 64-bit products of 32-bit values
        p1 = np.uint64(M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0) & MASK, lo1, (hi0 ^ c3 ^ k1) & MASK, lo0
    return c0, c1, c2, c3


def _key(seed):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & MASK, seed >> 32


def _unit(word):
    """A 32-bit word as a uniform in (0, 1): (2 * (word >> 9) + 1) / 2^24."""
    w = np.asarray(word, np.uint64) >> np.uint64(9)
    return (2.0 * w.astype(np.float64) + 1.0) / 16777216.0


def gumbel_row(seed, b, t, vocab):
    """G_v = -log(-log U_v) for v in 0..vocab-1 of row t of request b."""
    v = np.arange(vocab, dtype=np.uint64)
    words = philox4x32_10((v >> np.uint64(2), t, b, 0), _key(seed))
    w = np.choose((v & np.uint64(3)).astype(np.int64), words)
    return -np.log(-np.log(_unit(w)))


def accept_uniform(seed, b, t):
    """u_t of request b, in (0, 1)."""
    return float(_unit(philox4x32_10((0, t, b, 1), _key(seed))[0]))


def penalized_logits(logits_row, counts, presence, frequency):
    """l' = l - frequency * c - presence * [c > 0], fp64."""
    c = np.asarray(counts, np.float64)
    return np.asarray(logits_row, np.float64) - frequency * c - presence * (c > 0)


def row_counts(prior, pending, draft, t, vocab):
    """c_t: prior output counts plus the tokens of rows 0..t (the pending
    token is left out when it is None)."""
    c = np.zeros(vocab, np.int64) if prior is None else np.asarray(prior, np.int64).copy()
    toks = ([] if pending is None else [int(pending)]) + [int(x) for x in draft[:t]]
    for tok in toks:
        c[tok] += 1
    return c


def softmax(x):
    z = np.exp(x - np.max(x))
    return z / np.sum(z)


def speculative_sample(logits, draft, seed, temperature, draft_probs=None, pending=None, prior_counts=None,
                       presence=None, frequency=None, slot_ids=None, details=False):
    """logits [B][R][V] (any float), draft [B][R-1] int, draft_probs [B][R-1][V]
    or None (greedy drafter), pending [B] (needed with penalties), prior_counts
    [B][V] or None, temperature / presence / frequency [B] (None: no penalty),
    slot_ids [B] or None. Returns (accept_len [B], next_token [B]) int32, and
    with details=True also a list of per-request dicts with the decisions'
    margins (how far each comparison was from a tie)."""
    logits = np.asarray(logits, np.float64)
    B, R, V = logits.shape
    draft = np.asarray(draft).reshape(B, R - 1)
    accept = np.zeros(B, np.int32)
    nxt = np.full(B, -1, np.int32)
    info = []
    for b in range(B):
        if slot_ids is not None and int(slot_ids[b]) == -1:
            info.append(None)
            continue
        T = float(temperature[b])
        pres = 0.0 if presence is None else float(presence[b])
        freq = 0.0 if frequency is None else float(frequency[b])
        pend = None if pending is None else int(pending[b])
        prior = None if prior_counts is None else prior_counts[b]
        use_pen = pres != 0.0 or freq != 0.0
        p_rows = []
        for t in range(R):
            row = logits[b, t]
            if use_pen:
                row = penalized_logits(row, row_counts(prior, pend, draft[b], t, V), pres, freq)
            p_rows.append(softmax(row / T))
        margins = []
        n = R
        for t in range(R - 1):
            d = int(draft[b, t])
            q = np.zeros(V)
            if draft_probs is None:
                q[d] = 1.0
            else:
                q = np.asarray(draft_probs[b, t], np.float64)
            u = accept_uniform(seed, b, t)
            lhs, rhs = u * q[d], p_rows[t][d]
            margins.append(abs(lhs - rhs) / max(lhs, rhs, 1e-300))
            if not lhs <= rhs:
                n = t + 1
                resid = np.maximum(p_rows[t] - q, 0.0)
                keys = np.full(V, -np.inf)
                pos = resid > 0
                keys[pos] = np.log(resid[pos]) + gumbel_row(seed, b, t, V)[pos]
                break
        if n == R:
            keys = np.log(p_rows[R - 1]) + gumbel_row(seed, b, R - 1, V)
        order = np.argsort(-keys, kind="stable")
        accept[b] = n
        nxt[b] = int(order[0])
        if details:
            gap = keys[order[0]] - keys[order[1]] if V > 1 else np.inf
            info.append({"accept_margins": margins, "argmax_gap": float(gap), "row": n - 1 if n < R else R - 1,
                         "key": float(keys[order[0]])})
    if details:
        return accept, nxt, info
    return accept, nxt
