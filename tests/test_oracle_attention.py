"""Pins of the verification-attention oracle: closed forms, invariances the
definition fixes, a hand-worked case and a library routine (scaled dot-product
attention with an explicit mask, in fp64 on the CPU)."""
import numpy as np
import pytest

from oracle import attention


def _case(rng, B=3, R=4, Hq=4, Hkv=2, D=8, page=4, lens=(9, 4, 13)):
    lens = np.asarray(lens)
    nblk = int(np.ceil(lens.max() / page))
    P = B * nblk + 3
    perm = rng.permutation(P)[:B * nblk].reshape(B, nblk)
    q = rng.standard_normal((B, R, Hq, D))
    kc = rng.standard_normal((P, page, Hkv, D))
    vc = rng.standard_normal((P, page, Hkv, D))
    return q, kc, vc, perm, lens, page


def test_hand_case():
    # one request, one head, D = 2, two positions, one verify row:
    # q = [1, 0], k0 = [0, 0], k1 = [ln 3, 0], scale 1 -> scores 0, ln 3 ->
    # weights 1/4, 3/4; v0 = [4, 0], v1 = [0, 8] -> o = [1, 6]
    q = np.array([[[[1.0, 0.0]]]])
    kc = np.array([[[[0.0, 0.0]], [[np.log(3.0), 0.0]]]])
    vc = np.array([[[[4.0, 0.0]], [[0.0, 8.0]]]])
    o = attention.verify_attention(q, kc, vc, np.array([[0]]), np.array([2]), 2, 1.0)
    np.testing.assert_allclose(o[0, 0, 0], [1.0, 6.0], atol=1e-12)


def test_equal_keys_average_the_visible_values():
    rng = np.random.default_rng(1)
    q, kc, vc, bt, lens, page = _case(rng)
    kc[:] = rng.standard_normal(kc.shape[-1])          # every key the same vector
    o = attention.verify_attention(q, kc, vc, bt, lens, page, 0.7)
    R = q.shape[1]
    for b in range(len(lens)):
        pos = np.arange(lens[b])
        V = vc[bt[b][pos // page], pos % page]
        for t in range(R):
            want = V[:lens[b] - R + t + 1].mean(axis=0)   # [Hkv][D]
            for h in range(q.shape[2]):
                np.testing.assert_allclose(o[b, t, h], want[h // 2], atol=1e-12)


def test_single_visible_position_returns_its_value():
    rng = np.random.default_rng(2)
    q, kc, vc, bt, _, page = _case(rng, R=1, lens=(1, 1, 1))
    o = attention.verify_attention(q, kc, vc, bt, np.array([1, 1, 1]), page, 1.0)
    for b in range(3):
        for h in range(4):
            np.testing.assert_allclose(o[b, 0, h], vc[bt[b][0], 0, h // 2], atol=1e-12)


def test_later_positions_do_not_reach_earlier_rows():
    rng = np.random.default_rng(3)
    q, kc, vc, bt, lens, page = _case(rng)
    o = attention.verify_attention(q, kc, vc, bt, lens, page, 0.5)
    # change the key and value of each request's last position: only row R-1 may move
    kc2, vc2 = kc.copy(), vc.copy()
    for b, L in enumerate(lens):
        p = L - 1
        kc2[bt[b][p // page], p % page] += 3.0
        vc2[bt[b][p // page], p % page] -= 2.0
    o2 = attention.verify_attention(q, kc2, vc2, bt, lens, page, 0.5)
    assert np.array_equal(o[:, :-1], o2[:, :-1])
    assert not np.allclose(o[:, -1], o2[:, -1])


def test_page_placement_does_not_matter():
    rng = np.random.default_rng(4)
    q, kc, vc, bt, lens, page = _case(rng)
    perm = rng.permutation(kc.shape[0])                # move every page elsewhere
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    o = attention.verify_attention(q, kc, vc, bt, lens, page, 0.9)
    o2 = attention.verify_attention(q, kc2, vc2, perm[bt], lens, page, 0.9)
    assert np.array_equal(o, o2)


def test_matches_library_attention_with_a_mask():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    q, kc, vc, bt, lens, page = _case(rng, Hq=6, Hkv=3)
    scale = 0.35
    o = attention.verify_attention(q, kc, vc, bt, lens, page, scale)
    B, R, Hq, D = q.shape
    G = Hq // kc.shape[2]
    for b in range(B):
        L = lens[b]
        pos = np.arange(L)
        K = torch.from_numpy(kc[bt[b][pos // page], pos % page])    # [L][Hkv][D]
        V = torch.from_numpy(vc[bt[b][pos // page], pos % page])
        Qb = torch.from_numpy(q[b]).transpose(0, 1)                # [Hq][R][D]
        Kb = K.repeat_interleave(G, dim=1).transpose(0, 1)         # [Hq][L][D]
        Vb = V.repeat_interleave(G, dim=1).transpose(0, 1)
        mask = torch.from_numpy(pos[None, :] <= (L - R + np.arange(R))[:, None])   # [R][L]
        ref = torch.nn.functional.scaled_dot_product_attention(Qb, Kb, Vb, attn_mask=mask, scale=scale)
        np.testing.assert_allclose(o[b], ref.transpose(0, 1).numpy(), atol=1e-12)


def test_padding_request_stays_zero():
    rng = np.random.default_rng(6)
    q, kc, vc, bt, _, page = _case(rng)
    o = attention.verify_attention(q, kc, vc, bt, np.array([9, 0, 13]), page, 1.0)
    assert not o[1].any()


MUTANTS = [
    ("sees_one_position_too_many", "            last = L - R + t          # the last position row t sees",
     "            last = min(L - R + t + 1, L - 1)"),
    ("sees_one_position_too_few", "            last = L - R + t          # the last position row t sees",
     "            last = max(L - R + t - 1, 0)"),
    ("head_map_modulo", "                g = h // G", "                g = h % Hkv"),
    ("scale_dropped", "                s = scale * (K[:last + 1, g] @ q[b, t, h])", "                s = K[:last + 1, g] @ q[b, t, h]"),
    ("page_slot_swapped", "        pages = np.asarray(block_table[b])[pos // page_size]",
     "        pages = np.asarray(block_table[b])[pos % len(block_table[b])]"),
]


@pytest.mark.parametrize("name,before,after", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, before, after):
    """Each planted mistake makes one of the pins above fail."""
    src = open(attention.__file__).read()
    assert src.count(before) == 1, name
    ns = {}
    exec(compile(src.replace(before, after), "mutant_" + name, "exec"), ns)
    mutant = type("M", (), {"verify_attention": staticmethod(ns["verify_attention"])})
    pins = [test_hand_case, test_equal_keys_average_the_visible_values,
            test_single_visible_position_returns_its_value, test_later_positions_do_not_reach_earlier_rows,
            test_page_placement_does_not_matter, test_matches_library_attention_with_a_mask]
    caught = False
    saved = attention.verify_attention
    try:
        attention.verify_attention = mutant.verify_attention
        for pin in pins:
            try:
                pin()
            except (AssertionError, IndexError, ValueError):
                caught = True
                break
    finally:
        attention.verify_attention = saved
    assert caught, name
