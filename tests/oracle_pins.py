"""Pins for the CPU oracle: checks against what the definition and hand work fix.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises ``AssertionError`` when the
oracle disagrees. They run on the real oracle (``test_oracle_pins.py``) and on
copies of it with one planted mistake each (``test_oracle_mutants.py``), every
one of which must trip at least one pin.

Nothing here calls the oracle to make an expected value. The expected values
come from hand work (``tests/golden``), closed forms of the recurrence, and an
independent formulation (the product of per-row transition matrices, with the
conv done by ``numpy.convolve``).
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass, replace

import numpy as np

from linear_attention_verify_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@dataclass(frozen=True)
class Shape:
    num_k_heads: int = 1
    num_v_heads: int = 1
    d_k: int = 2
    d_v: int = 2
    conv_width: int = 4
    dtype: str = "f32"
    act: str = "none"
    scale: float = 1.0
    l2_eps: float = 0.0

    @property
    def conv_channels(self):
        return 2 * self.num_k_heads * self.d_k + self.num_v_heads * self.d_v


def identity_taps(C, W):
    cw = np.zeros((C, W), np.float32)
    cw[:, W - 1] = 1.0
    return cw


def pack_x(shape, q_rows, k_rows, v_rows):
    """x [1][R][C] from per-row q (HK*d_k), k (HK*d_k), v (HV*d_v) values."""
    R = len(q_rows)
    x = np.zeros((1, R, shape.conv_channels), np.float32)
    nq = shape.num_k_heads * shape.d_k
    for t in range(R):
        x[0, t, :nq] = np.ravel(q_rows[t])
        x[0, t, nq:2 * nq] = np.ravel(k_rows[t])
        x[0, t, 2 * nq:] = np.ravel(v_rows[t])
    return x


def gates(vals, HV):
    return np.repeat(np.asarray(vals, np.float32).reshape(1, -1, 1), HV, axis=2)


def pool_from_math(S_list):
    """Pool array [1][HV][d_k][d_v] from math-orientation d_v x d_k states."""
    return np.ascontiguousarray(np.stack([np.asarray(S, np.float32).T for S in S_list])[None])


# ---------------------------------------------------------------------------
# independent formulation: conv by numpy.convolve, transition-matrix products
# ---------------------------------------------------------------------------

def reference_by_transitions(shape, S0_math, hist, cw, x, alpha, beta):
    """One request. S0_math [HV][d_v][d_k], hist [W-1][C], cw [C][W], x [R][C],
    alpha/beta [R][HV] (all float64). Returns (o [R][HV][d_v], S_t [R][HV][d_v][d_k]).

    Conv: y[t, c] = (window_c * taps_c)[t] computed as a 'valid' numpy
    convolution with the reversed taps. State: S_t = S_{t-1} A_t + beta_t v_t k_t^T
    with A_t = alpha_t (I - beta_t k_t k_t^T), unrolled as
    S_t = S_0 A_1...A_t + sum_s beta_s v_s k_s^T A_{s+1}...A_t.
    """
    HK, HV, dk, dv, W = shape.num_k_heads, shape.num_v_heads, shape.d_k, shape.d_v, shape.conv_width
    R, C = x.shape
    y = np.empty((R, C))
    for c in range(C):
        window = np.concatenate([hist[:, c], x[:, c]])
        y[:, c] = np.convolve(window, cw[c, ::-1], mode="valid")
    if shape.act == "silu":
        y = y * (0.5 * (1.0 + np.tanh(0.5 * y)))   # logistic via tanh
    nq = HK * dk
    q = y[:, :nq].reshape(R, HK, dk)
    k = y[:, nq:2 * nq].reshape(R, HK, dk)
    v = y[:, 2 * nq:].reshape(R, HV, dv)
    qn = q / np.sqrt(np.sum(q * q, axis=2, keepdims=True) + shape.l2_eps)
    kn = k / np.sqrt(np.sum(k * k, axis=2, keepdims=True) + shape.l2_eps)
    group = HV // HK
    o = np.zeros((R, HV, dv))
    states = np.zeros((R, HV, dv, dk))
    I = np.eye(dk)
    for h in range(HV):
        kh = h // group
        A = [alpha[t, h] * (I - beta[t, h] * np.outer(kn[t, kh], kn[t, kh])) for t in range(R)]
        for t in range(R):
            prod = np.linalg.multi_dot([S0_math[h]] + A[:t + 1]) if t >= 0 else None
            S = prod.copy()
            for s in range(t + 1):
                tail = np.eye(dk)
                for m in range(s + 1, t + 1):
                    tail = tail @ A[m]
                S += beta[s, h] * np.outer(v[s, h], kn[s, kh]) @ tail
            states[t, h] = S
            o[t, h] = shape.scale * (S @ qn[t, kh])
    return o, states


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_conv_ring_hand(orc):
    """tests/golden/conv_ring.json: conv outputs and the history after n rows."""
    g = golden("conv_ring.json")
    # one key head and one value head of width 1: channels q, k, v each see the
    # same history and inputs; with beta = 1 and d = 1, S_t = v_t so o_t = y_v[t].
    for act, expect in (("none", g["conv_out"]), ("silu", g["silu_out"])):
        shape = Shape(d_k=1, d_v=1, act=act, l2_eps=0.0)
        C, W = shape.conv_channels, shape.conv_width
        hist = np.tile(np.asarray(g["history"], np.float32)[:, None], (1, C))[None]
        cw = np.tile(np.asarray(g["taps"], np.float32), (C, 1))
        x = np.tile(np.asarray(g["inputs"], np.float32)[:, None], (1, C))[None]
        R = x.shape[1]
        alpha, beta = gates([0.7] * R, 1), gates([1.0] * R, 1)
        ssm = np.full((1, 1, 1, 1), 0.25, np.float32)
        out, snap, err = orc.verify(shape, ssm, hist, cw, x, alpha, beta,
                                    np.array([0], np.int32), R, want_snapshots=True)
        assert err == 0
        # the taps 0.1..0.4 are stored as fp32 (each off by < 3e-8 relative)
        np.testing.assert_allclose(out[0, :, 0, 0], expect, rtol=0, atol=1e-6)
        np.testing.assert_allclose(snap[0, :, 0, 0, 0], expect, rtol=0, atol=1e-6)
        for n, want in g["history_after_commit"].items():
            s2, h2 = ssm.copy(), hist.copy()
            err = orc.commit(shape, s2, h2, cw, x, alpha, beta, np.array([0], np.int32),
                             np.array([int(n)], np.int32), R)
            assert err == 0
            for c in range(C):
                assert h2[0, :, c].tolist() == want, (n, c, h2[0, :, c])


def pin_recurrence_d2_hand(orc):
    """tests/golden/hand_d2.json: two rows at d = 2, exact to fp64 rounding."""
    g = golden("hand_d2.json")
    shape = Shape()
    C, W = shape.conv_channels, shape.conv_width
    rows = g["rows"]
    R = len(rows)
    x = pack_x(shape, [r["q"] for r in rows], [r["k"] for r in rows], [r["v"] for r in rows])
    alpha = gates([r["alpha"] for r in rows], 1)
    beta = gates([r["beta"] for r in rows], 1)
    ssm = pool_from_math([g["S0"]])
    assert ssm.ravel().tolist() == g["S0_pool_order"]
    hist = np.zeros((1, W - 1, C), np.float32)
    cw = identity_taps(C, W)
    out, snap, err = orc.verify(shape, ssm, hist, cw, x, alpha, beta, np.array([0], np.int32),
                                R, want_snapshots=True)
    assert err == 0
    for t, r in enumerate(rows):
        np.testing.assert_allclose(out[0, t, 0], r["o"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(snap[0, t, 0].T, r["S"], rtol=0, atol=1e-12)
    s2 = ssm.copy()
    assert orc.commit(shape, s2, hist.copy(), cw, x, alpha, beta, np.array([0], np.int32),
                      np.array([R], np.int32), R) == 0
    np.testing.assert_allclose(s2[0, 0].T, rows[-1]["S"], rtol=0, atol=1e-7)


def _random_case(shape, R, seed, alpha=None, beta=None, hist=None):
    rng = np.random.default_rng(seed)
    C, W, HV = shape.conv_channels, shape.conv_width, shape.num_v_heads
    S0 = rng.standard_normal((HV, shape.d_v, shape.d_k)).astype(np.float32)
    hist = rng.standard_normal((1, W - 1, C)).astype(np.float32) if hist is None else hist
    cw = (rng.standard_normal((C, W)) / np.sqrt(W)).astype(np.float32)
    x = rng.standard_normal((1, R, C)).astype(np.float32)
    a = rng.uniform(0.9, 1.0, (1, R, HV)).astype(np.float32) if alpha is None else alpha
    b = rng.uniform(0.0, 1.0, (1, R, HV)).astype(np.float32) if beta is None else beta
    return S0, hist, cw, x, a, b


def pin_identity_gate(orc):
    """alpha = 1, beta = 0: S unchanged bitwise, o_t = S_0 q_hat_t."""
    shape = Shape(num_k_heads=2, num_v_heads=4, d_k=8, d_v=8, act="none", l2_eps=1e-6)
    R = 3
    HV = shape.num_v_heads
    S0, _, _, x, _, _ = _random_case(shape, R, 11)
    C, W = shape.conv_channels, shape.conv_width
    hist = np.zeros((1, W - 1, C), np.float32)
    cw = identity_taps(C, W)
    alpha, beta = gates([1.0] * R, HV), gates([0.0] * R, HV)
    ssm = pool_from_math(list(S0))
    out, snap, err = orc.verify(shape, ssm, hist, cw, x, alpha, beta, np.array([0], np.int32),
                                R, want_snapshots=True)
    assert err == 0
    for t in range(R):
        assert np.array_equal(snap[0, t].astype(np.float32), ssm[0])
    nq = shape.num_k_heads * shape.d_k
    q = x[0, :, :nq].astype(np.float64).reshape(R, shape.num_k_heads, shape.d_k)
    qn = q / np.linalg.norm(q, axis=2, keepdims=True)
    for h in range(HV):
        want = np.einsum("ij,tj->ti", S0[h].astype(np.float64), qn[:, h // 2])
        np.testing.assert_allclose(out[0, :, h], want, rtol=1e-6, atol=1e-6)
    s2 = ssm.copy()
    assert orc.commit(shape, s2, hist.copy(), cw, x, alpha, beta, np.array([0], np.int32),
                      np.array([R], np.int32), R) == 0
    assert np.array_equal(s2.view(np.uint32), ssm.view(np.uint32))


def pin_write_back(orc):
    """alpha arbitrary, beta = 1, unit k: the updated state maps k_t to v_t."""
    shape = Shape(num_k_heads=1, num_v_heads=2, d_k=8, d_v=8, act="none", l2_eps=0.0)
    R = 4
    HV = shape.num_v_heads
    S0, _, _, x, alpha, _ = _random_case(shape, R, 12)
    C, W = shape.conv_channels, shape.conv_width
    nq = shape.d_k
    x[0, :, nq:2 * nq] /= np.linalg.norm(x[0, :, nq:2 * nq], axis=1, keepdims=True)
    beta = gates([1.0] * R, HV)
    ssm = pool_from_math(list(S0))
    _, snap, err = orc.verify(shape, ssm, np.zeros((1, W - 1, C), np.float32), identity_taps(C, W),
                              x, alpha, beta, np.array([0], np.int32), R, want_snapshots=True)
    assert err == 0
    for t in range(R):
        k = x[0, t, nq:2 * nq].astype(np.float64)
        k = k / np.linalg.norm(k)
        for h in range(HV):
            v = x[0, t, 2 * nq + h * shape.d_v:2 * nq + (h + 1) * shape.d_v]
            np.testing.assert_allclose(snap[0, t, h].T @ k, v, rtol=0, atol=1e-6)


def pin_beta_zero_decay(orc):
    """beta = 0: S_t = (alpha_1 ... alpha_t) S_0, per value head."""
    shape = Shape(num_k_heads=2, num_v_heads=4, d_k=4, d_v=4, act="silu", l2_eps=1e-6)
    R = 5
    HV = shape.num_v_heads
    S0, hist, cw, x, alpha, _ = _random_case(shape, R, 13)
    beta = gates([0.0] * R, HV)
    ssm = pool_from_math(list(S0))
    _, snap, err = orc.verify(shape, ssm, hist, cw, x, alpha, beta, np.array([0], np.int32),
                              R, want_snapshots=True)
    assert err == 0
    decay = np.cumprod(alpha[0].astype(np.float64), axis=0)      # [R][HV]
    for t in range(R):
        for h in range(HV):
            np.testing.assert_allclose(snap[0, t, h].T, decay[t, h] * S0[h], rtol=1e-13, atol=0)


def pin_orthonormal_keys(orc):
    """k_t = e_t, beta = 1: column j of S_n is (prod of later alphas) v_j for
    written columns and (prod of all alphas) times column j of S_0 otherwise."""
    shape = Shape(num_k_heads=1, num_v_heads=2, d_k=6, d_v=5, act="none", l2_eps=0.0)
    R = 4
    HV, dk = shape.num_v_heads, shape.d_k
    S0, _, _, x, alpha, _ = _random_case(shape, R, 14)
    C, W = shape.conv_channels, shape.conv_width
    x[0, :, dk:2 * dk] = 0.0
    for t in range(R):
        x[0, t, dk + t] = 2.0                   # normalises to e_t
    beta = gates([1.0] * R, HV)
    ssm = pool_from_math(list(S0))
    _, snap, err = orc.verify(shape, ssm, np.zeros((1, W - 1, C), np.float32), identity_taps(C, W),
                              x, alpha, beta, np.array([0], np.int32), R, want_snapshots=True)
    assert err == 0
    a = alpha[0].astype(np.float64)
    for n in range(1, R + 1):
        for h in range(HV):
            Sn = snap[0, n - 1, h].T                 # d_v x d_k
            for j in range(dk):
                if j < n:
                    v = x[0, j, 2 * dk + h * shape.d_v:2 * dk + (h + 1) * shape.d_v]
                    want = np.prod(a[j + 1:n, h]) * v.astype(np.float64)
                else:
                    want = np.prod(a[:n, h]) * S0[h][:, j].astype(np.float64)
                np.testing.assert_allclose(Sn[:, j], want, rtol=1e-13, atol=1e-14)


def pin_transition_products(orc):
    """Random case with GQA (HK = 2, HV = 4), SiLU, eps, scale != 1 and a
    non-trivial conv: outputs and states match the transition-matrix form."""
    shape = Shape(num_k_heads=2, num_v_heads=4, d_k=6, d_v=5, act="silu", l2_eps=1e-6, scale=0.7)
    R = 4
    S0, hist, cw, x, alpha, beta = _random_case(shape, R, 15)
    ssm = pool_from_math(list(S0))
    out, snap, err = orc.verify(shape, ssm, hist, cw, x, alpha, beta, np.array([0], np.int32),
                                R, want_snapshots=True)
    assert err == 0
    o_ref, s_ref = reference_by_transitions(
        shape, S0.astype(np.float64), hist[0].astype(np.float64), cw.astype(np.float64),
        x[0].astype(np.float64), alpha[0].astype(np.float64), beta[0].astype(np.float64))
    np.testing.assert_allclose(out[0], o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(np.swapaxes(snap[0], 2, 3), s_ref, rtol=1e-11, atol=1e-12)


def pin_decode_equivalence(orc):
    """verify(R) then commit(n) leaves what n single decode steps leave (conv
    history bitwise; S to fp32 rounding), and verify leaves the pool untouched."""
    shape = Shape(num_k_heads=2, num_v_heads=4, d_k=4, d_v=4, act="silu", l2_eps=1e-6)
    R = 4
    S0, hist, cw, x, alpha, beta = _random_case(shape, R, 16)
    ssm0 = pool_from_math(list(S0))
    ssm, conv = ssm0.copy(), hist.copy()
    out, _, err = orc.verify(shape, ssm, conv, cw, x, alpha, beta, np.array([0], np.int32), R)
    assert err == 0
    assert np.array_equal(ssm.view(np.uint32), ssm0.view(np.uint32))
    assert np.array_equal(conv, hist)
    for n in range(R + 1):
        s_c, h_c = ssm0.copy(), hist.copy()
        assert orc.commit(shape, s_c, h_c, cw, x, alpha, beta, np.array([0], np.int32),
                          np.array([n], np.int32), R) == 0
        s_d, h_d = ssm0.copy(), hist.copy()
        for t in range(n):
            o_t, err = orc.decode_step(shape, s_d, h_d, cw, x[:, t], alpha[:, t], beta[:, t],
                                       np.array([0], np.int32))
            assert err == 0
            np.testing.assert_allclose(o_t[0], out[0, t], rtol=1e-5, atol=1e-6)
        assert np.array_equal(h_c, h_d), n
        np.testing.assert_allclose(s_c, s_d, rtol=1e-5, atol=1e-6)


def pin_bf16_storage(orc):
    """The same (bf16-exact) values stored as bf16 or as fp32 give identical results."""
    w = wl.small_workload(wl.LayerShape(2, 4, 8, 8, dtype="bf16"), batch=2, rows=3, num_slots=5,
                          seed=17)
    slot_ids, accept = wl.draw_requests(w)
    d = wl.draw_layer(w)
    ssm, conv = wl.build_pools(w, d, slot_ids)
    sh16 = w.shape
    sh32 = replace(w.shape, dtype="f32")
    f = wl.bf16_bits_to_f32
    o16, _, e16 = orc.verify(sh16, ssm, conv, d["conv_w"], d["x"], d["alpha"], d["beta"], slot_ids, 3)
    o32, _, e32 = orc.verify(sh32, ssm, f(conv), f(d["conv_w"]), f(d["x"]), f(d["alpha"]),
                             f(d["beta"]), slot_ids, 3)
    assert e16 == 0 and e32 == 0
    assert np.all(np.isfinite(o16))
    assert np.array_equal(o16, o32)
    s16, c16 = ssm.copy(), conv.copy()
    s32, c32 = ssm.copy(), f(conv)
    assert orc.commit(sh16, s16, c16, d["conv_w"], d["x"], d["alpha"], d["beta"], slot_ids, accept, 3) == 0
    assert orc.commit(sh32, s32, c32, f(d["conv_w"]), f(d["x"]), f(d["alpha"]), f(d["beta"]),
                      slot_ids, accept, 3) == 0
    assert np.array_equal(s16.view(np.uint32), s32.view(np.uint32))
    assert np.array_equal(f(c16).view(np.uint32), c32.view(np.uint32))


def pin_slot_table(orc):
    """Requests read and write their own slots: a batch equals one-request runs,
    padding gives zeros and commits nothing, untouched slots keep their bits,
    bad slots and accept lengths are flagged and skipped."""
    w = wl.small_workload(wl.LayerShape(2, 4, 8, 8, dtype="f32"), batch=4, rows=3, num_slots=9,
                          seed=18)
    slot_ids, accept = wl.draw_requests(w)
    d = wl.draw_layer(w)
    slot_ids[2] = -1
    ssm, conv = wl.build_pools(w, d, slot_ids)
    sh = w.shape
    out, _, err = orc.verify(sh, ssm, conv, d["conv_w"], d["x"], d["alpha"], d["beta"], slot_ids, 3)
    assert err == 0
    assert not np.any(out[2])
    for b in (0, 1, 3):
        o1, _, e1 = orc.verify(sh, ssm, conv, d["conv_w"], d["x"][b:b + 1], d["alpha"][b:b + 1],
                               d["beta"][b:b + 1], slot_ids[b:b + 1], 3)
        assert e1 == 0 and np.all(np.isfinite(o1))
        assert np.array_equal(o1[0], out[b])
    s2, c2 = ssm.copy(), conv.copy()
    assert orc.commit(sh, s2, c2, d["conv_w"], d["x"], d["alpha"], d["beta"], slot_ids, accept, 3) == 0
    active = set(int(s) for s in slot_ids if s >= 0)
    for s in range(w.num_slots):
        same = np.array_equal(s2[s].view(np.uint32), ssm[s].view(np.uint32))
        assert same == (s not in active), s
    # out-of-range slot and accept length: flagged, pool untouched
    bad = slot_ids.copy()
    bad[0] = w.num_slots
    _, _, err = orc.verify(sh, ssm, conv, d["conv_w"], d["x"], d["alpha"], d["beta"], bad, 3)
    assert err & 1
    s3, c3 = ssm.copy(), conv.copy()
    bad_acc = accept.copy()
    bad_acc[:] = 4
    err = orc.commit(sh, s3, c3, d["conv_w"], d["x"], d["alpha"], d["beta"], slot_ids, bad_acc, 3)
    assert err & 2
    assert np.array_equal(s3.view(np.uint32), ssm.view(np.uint32))


def pin_commit_row_selection(orc):
    """commit(n) equals the verify snapshot after row n-1, not its neighbours."""
    w = wl.small_workload(wl.LayerShape(2, 4, 16, 16, dtype="f32"), batch=1, rows=5, num_slots=2,
                          seed=19)
    slot_ids, _ = wl.draw_requests(w)
    d = wl.draw_layer(w)
    ssm, conv = wl.build_pools(w, d, slot_ids)
    sh = w.shape
    _, snap, err = orc.verify(sh, ssm, conv, d["conv_w"], d["x"], d["alpha"], d["beta"], slot_ids,
                              5, want_snapshots=True)
    assert err == 0
    s = int(slot_ids[0])
    for n in range(1, 6):
        s2, c2 = ssm.copy(), conv.copy()
        assert orc.commit(sh, s2, c2, d["conv_w"], d["x"], d["alpha"], d["beta"], slot_ids,
                          np.array([n], np.int32), 5) == 0
        dist = [np.max(np.abs(s2[s] - snap[0, t])) for t in range(5)]
        assert int(np.argmin(dist)) == n - 1 and dist[n - 1] < 1e-6, (n, dist)


PINS = [
    pin_conv_ring_hand,
    pin_recurrence_d2_hand,
    pin_identity_gate,
    pin_write_back,
    pin_beta_zero_decay,
    pin_orthonormal_keys,
    pin_transition_products,
    pin_decode_equivalence,
    pin_bf16_storage,
    pin_slot_table,
    pin_commit_row_selection,
]
