"""Verification attention over a paged KV cache, written out plainly.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the HIP library shares no code with it.

The full-attention layers of a hybrid model score the same k+1 verify rows
as its GatedDeltaNet layers, against the request's KV cache kept in pages
(lmdeploy PR #5006, What's included, Verification path: verification
attention over paged KV). Readings where the page is silent:

  - the verify rows' own keys and values are already in the cache, at
    positions seq_len - rows .. seq_len - 1; row t sees positions
    0 .. seq_len - rows + t (causal within the rows, as decoding would);
  - query head h reads KV head h / (Hq / Hkv);
  - scores are scale * q.k, softmax over the visible positions, o = p.V;
  - position p of request b lives in page block_table[b][p // page_size],
    slot p % page_size; cache layout [pages][page_size][Hkv][D];
  - seq_len 0 marks a padding request (output left zero).

Everything is computed in fp64 over the stored (bf16-rounded) inputs.
"""
import numpy as np


def verify_attention(q, k_cache, v_cache, block_table, seq_lens, page_size, scale):
    """q [B][R][Hq][D], caches [pages][page_size][Hkv][D] -> o [B][R][Hq][D] fp64."""
    q = np.asarray(q, np.float64)
    B, R, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    o = np.zeros((B, R, Hq, D))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        pos = np.arange(L)
        pages = np.asarray(block_table[b])[pos // page_size]
        K = np.asarray(k_cache[pages, pos % page_size], np.float64)   # [L][Hkv][D]
        V = np.asarray(v_cache[pages, pos % page_size], np.float64)
        for t in range(R):
            last = L - R + t          # the last position row t sees
            for h in range(Hq):
                g = h // G
                s = scale * (K[:last + 1, g] @ q[b, t, h])
                s = s - s.max()
                p = np.exp(s)
                p = p / p.sum()
                o[b, t, h] = p @ V[:last + 1, g]
    return o
