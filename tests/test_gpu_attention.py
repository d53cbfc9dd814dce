"""Verification attention on the device against the oracle, element by
element: ragged lengths across pages and splits, every verify row count,
query-head groups, both head dims, padding, and the error flags."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle import attention  # noqa: E402
from linear_attention_verify_amd import binding as bd  # noqa: E402
from linear_attention_verify_amd import workloads as wl  # noqa: E402

DEV = "cuda"
ATOL, RTOL = 3e-3, 1e-2


def _bits_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def _run(w, d, table=None, seq=None):
    s = w.shape
    desc = bd.attn_desc(s)
    table = d["block_table"] if table is None else table
    seq = d["seq_lens"] if seq is None else seq
    q = _bits_to_dev(d["q"])
    kc = _bits_to_dev(d["k_cache"])
    vc = _bits_to_dev(d["v_cache"])
    bt = torch.from_numpy(np.ascontiguousarray(table, np.int32)).to(DEV)
    sl = torch.from_numpy(np.ascontiguousarray(seq, np.int32)).to(DEV)
    nbytes = bd.gdn_spec_attn_scratch_bytes(desc, w.batch, w.rows, table.shape[1])
    scratch = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    bd.gdn_spec_attn_verify(desc, q, kc, vc, bt, sl, scratch, out, err)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), int(err.item())


def _oracle(w, d, seq=None):
    f = lambda a: wl.bf16_bits_to_f32(a)
    seq = d["seq_lens"] if seq is None else seq
    return attention.verify_attention(f(d["q"]), f(d["k_cache"]), f(d["v_cache"]), d["block_table"],
                                      seq, w.shape.page_size, w.shape.scale)


CASES = [
    # d, Hq, Hkv, page, rows, batch, min_len, max_len
    (128, 4, 2, 32, 3, 3, 3, 200),
    (128, 8, 1, 64, 1, 2, 1, 700),
    (256, 16, 2, 64, 9, 3, 9, 1500),
    (256, 16, 2, 32, 4, 4, 33, 300),
    (128, 2, 2, 32, 9, 2, 9, 2100),
    (256, 32, 2, 64, 4, 2, 64, 900),    # 64 queries per KV head: one full group of query tiles
    (128, 16, 1, 32, 8, 2, 100, 500),   # 128 queries, the most one KV head takes: two groups
    (128, 8, 2, 128, 5, 3, 5, 900),     # pages of four key tiles
    (256, 16, 2, 256, 9, 2, 9, 1600),   # pages of eight key tiles
    (128, 4, 1, 96, 3, 3, 3, 700),      # a page size that is not a power of two (three key tiles)
    (128, 4, 4, 32, 1, 3, 1, 300),      # one query per KV head: one query tile, one computing wave
    (256, 16, 8, 64, 3, 2, 3, 900),     # eight KV heads
]


@pytest.mark.parametrize("case", CASES, ids=["d%d-hq%d-hkv%d-p%d-r%d" % c[:5] for c in CASES])
def test_matches_oracle(case):
    d_, hq, hkv, page, rows, batch, lo, hi = case
    w = wl.AttnWorkload("t", wl.AttnShape(hq, hkv, d_, page), batch=batch, rows=rows, min_len=lo,
                        max_len=hi, seed=sum(case), padding=(1,) if batch > 2 else ())
    d = wl.draw_attention(w)
    print("attention", case, "seq", d["seq_lens"].tolist(), flush=True)
    got, err = _run(w, d)
    assert err == 0
    want = _oracle(w, d)
    np.testing.assert_allclose(got, want, atol=ATOL, rtol=RTOL)
    if batch > 2:
        assert not np.any(got[1])


def test_lengths_at_every_edge():
    """seq_len = rows (no committed context), page and split boundaries on both sides."""
    w = wl.AttnWorkload("edges", wl.AttnShape(8, 2, 128, 32), batch=9, rows=4, min_len=4, max_len=1100, seed=5)
    d = wl.draw_attention(w)
    seq = np.array([4, 31, 32, 33, 255, 256, 257, 1023, 1100], np.int32)
    # the draw gave each request pages for its own length: rebuild the table for these lengths
    need = -(-seq // 32)
    pages = d["k_cache"].shape[0]
    assert need.sum() <= pages
    table = np.full((9, w.max_blocks), -1, np.int32)
    perm = np.random.default_rng(0).permutation(pages)
    off = 0
    for b in range(9):
        table[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    d = dict(d, seq_lens=seq, block_table=table)
    got, err = _run(w, d)
    assert err == 0
    np.testing.assert_allclose(got, _oracle(w, d), atol=ATOL, rtol=RTOL)


def test_pieces_that_some_rows_cannot_see():
    """A piece of the split whose positions all lie past what some verify
    row sees (a pair's short last tile, cut off by itself) must add nothing
    to that row. Lengths 40 and 161 with 9 rows and 13 blocks of 32 give
    seven workgroups of three tiles, and three such pieces."""
    w = wl.AttnWorkload("unseen", wl.AttnShape(8, 2, 128, 32), batch=2, rows=9, min_len=9, max_len=416, seed=13)
    d = wl.draw_attention(w)
    seq = np.array([40, 161], np.int32)
    need = -(-seq // 32)
    table = np.full((2, w.max_blocks), -1, np.int32)
    perm = np.random.default_rng(1).permutation(d["k_cache"].shape[0])
    table[0, :need[0]] = perm[:need[0]]
    table[1, :need[1]] = perm[need[0]:need[0] + need[1]]
    d = dict(d, seq_lens=seq, block_table=table)
    got, err = _run(w, d)
    assert err == 0
    assert not np.isnan(got).any()
    np.testing.assert_allclose(got, _oracle(w, d), atol=ATOL, rtol=RTOL)


def test_bad_pages_and_lengths_are_flagged():
    w = wl.AttnWorkload("bad", wl.AttnShape(4, 2, 128, 32), batch=4, rows=3, min_len=40, max_len=90, seed=6)
    d = wl.draw_attention(w)
    table = d["block_table"].copy()
    table[1, 0] = d["k_cache"].shape[0] + 5     # page outside the cache
    seq = d["seq_lens"].copy()
    seq[2] = 2                                   # below rows
    got, err = _run(w, d, table=table, seq=seq)
    assert err == 1 | 4
    assert not np.any(got[1]) and not np.any(got[2])
    ok = [0, 3]
    want = _oracle(w, dict(d, seq_lens=seq), seq=np.where(np.isin(np.arange(4), ok), seq, 0))
    np.testing.assert_allclose(got[ok], want[ok], atol=ATOL, rtol=RTOL)


def test_bad_page_inside_a_request_is_flagged():
    """A page id outside the pool in the middle of a request (its third
    block): that request is zero on both KV heads and flagged, the others
    are exact."""
    w = wl.AttnWorkload("bad-mid", wl.AttnShape(8, 2, 128, 64), batch=3, rows=4, min_len=300, max_len=600, seed=9)
    d = wl.draw_attention(w)
    table = d["block_table"].copy()
    table[1, 2] = -3
    print("bad page inside request 1, seq", d["seq_lens"].tolist(), flush=True)
    got, err = _run(w, d, table=table)
    assert err == 1
    assert not np.any(got[1])
    ok = [0, 2]
    want = _oracle(w, d, seq=np.where(np.isin(np.arange(3), ok), d["seq_lens"], 0))
    np.testing.assert_allclose(got[ok], want[ok], atol=ATOL, rtol=RTOL)


def test_full_size_batch():
    """The 64-request, 9-row workload at its real lengths, in the launch
    configuration the bench times: every output against the oracle."""
    w = wl.ATTN_WORKLOADS["attn-b64"]
    d = wl.draw_attention(w)
    got, err = _run(w, d)
    assert err == 0
    np.testing.assert_allclose(got, _oracle(w, d), atol=ATOL, rtol=RTOL)
    # every request: o is a convex combination of the value rows it sees, so
    # each column lies between their least and greatest entry (up to bf16)
    assert np.isfinite(got).all()
    s_, G = w.shape, w.shape.num_q_heads // w.shape.num_kv_heads
    for b, L in enumerate(d["seq_lens"]):
        pos = np.arange(L)
        V = wl.bf16_bits_to_f32(d["v_cache"][d["block_table"][b][pos // s_.page_size], pos % s_.page_size])
        lo, hi = V.min(axis=0), V.max(axis=0)                   # [Hkv][D], over all positions
        o = got[b].reshape(w.rows, s_.num_kv_heads, G, s_.head_dim)
        assert (o >= lo[None, :, None, :] - 0.02).all() and (o <= hi[None, :, None, :] + 0.02).all(), b


def test_single_request_full_oracle():
    """The single-request workload (one request, 3 verify rows, 2048 positions)
    checked in full: few workgroups, each a run of tiles of one pair."""
    w = wl.ATTN_WORKLOADS["attn-single"]
    d = wl.draw_attention(w)
    got, err = _run(w, d)
    assert err == 0
    np.testing.assert_allclose(got, _oracle(w, d), atol=ATOL, rtol=RTOL)


def test_long_sequence_merges_many_records():
    """One request of 8192 positions: each (request, KV head) pair is cut over
    many workgroups, so the combine merges dozens of partial records."""
    w = wl.AttnWorkload("long", wl.AttnShape(16, 2, 256, 64), batch=1, rows=9, min_len=8192, max_len=8192, seed=21)
    d = wl.draw_attention(w)
    got, err = _run(w, d)
    assert err == 0
    np.testing.assert_allclose(got, _oracle(w, d), atol=ATOL, rtol=RTOL)


def test_slots_past_the_sequence_may_hold_nan():
    """Cache slots past a request's length (in its last page) hold NaN: they
    are masked out and must not reach the output through P V."""
    w = wl.AttnWorkload("nan-tail", wl.AttnShape(8, 2, 128, 64), batch=3, rows=4, min_len=70, max_len=250, seed=8)
    d = wl.draw_attention(w)
    kc, vc = d["k_cache"].copy(), d["v_cache"].copy()
    nan_bits = np.uint16(0x7FC1)
    for b in range(w.batch):
        L = int(d["seq_lens"][b])
        last_page = d["block_table"][b, (L - 1) // 64]
        kc[last_page, L % 64 or 64:] = nan_bits
        vc[last_page, L % 64 or 64:] = nan_bits
    d2 = dict(d, k_cache=kc, v_cache=vc)
    got, err = _run(w, d2)
    assert err == 0
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, _oracle(w, d), atol=ATOL, rtol=RTOL)
