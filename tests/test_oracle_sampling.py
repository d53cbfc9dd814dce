"""Pins of the speculative-sampling oracle (oracle/sampling.py), on the CPU.

None of them re-types the oracle's formulas:
  - Philox4x32-10 against its published known-answer vectors;
  - Gumbel-max draws against the softmax they sample (chi-square);
  - the defining property of speculative sampling: whatever the drafter's
    distribution q, the first token a verify emits is distributed as the
    target's p_0 (chi-square, with and without draft probabilities);
  - q = p accepts every draft;
  - hand-worked per-row penalties;
  - near-zero temperature reduces to the greedy acceptance oracle;
  - planted mistakes in a copy of the module each fail one of the above.
"""
import importlib.util
import json
import os
import tempfile

import numpy as np
import pytest

from oracle import acceptance
from oracle import sampling as smp

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _chi2_ok(counts, probs, n):
    """Pearson chi-square of observed counts against n * probs, with a fixed
    critical value for p = 1e-4 at the degrees of freedom used here."""
    exp = n * np.asarray(probs)
    stat = float(np.sum((np.asarray(counts) - exp) ** 2 / exp))
    crit = {3: 21.1, 4: 23.5, 5: 25.7}[len(probs) - 1]
    return stat < crit, stat


def pin_philox_kat(mod=smp):
    kat = json.load(open(os.path.join(GOLDEN, "philox_kat.json")))
    for vec in kat["vectors"]:
        ctr = [int(x, 16) for x in vec["ctr"]]
        key = [int(x, 16) for x in vec["key"]]
        out = [int(x) for x in mod.philox4x32_10(ctr, key)]
        assert out == [int(x, 16) for x in vec["out"]], vec


def pin_gumbel_frequencies(mod=smp):
    """R = 1 (no drafts): the emitted token is a Gumbel-max draw from p_0."""
    V, B = 5, 12000
    row = np.array([0.3, -1.0, 1.2, 0.0, 0.7])
    T = 0.8
    logits = np.broadcast_to(row, (B, 1, V))
    _, nxt = mod.speculative_sample(logits, np.zeros((B, 0), np.int32), seed=1234, temperature=np.full(B, T))
    p = np.exp(row / T) / np.sum(np.exp(row / T))
    ok, stat = _chi2_ok(np.bincount(nxt, minlength=V), p, B)
    assert ok, stat


def _emitted_first(mod, logits, q, greedy, B, seed):
    """First emitted token after row 0 of B requests sharing row 0's logits
    (R = 2): the accepted draft, or the replacement."""
    rng = np.random.default_rng(seed)
    V = logits.shape[-1]
    if greedy:
        draft = np.full((B, 1), int(np.argmax(q)), np.int32)
        dp = None
    else:
        draft = rng.choice(V, size=(B, 1), p=q).astype(np.int32)   # the drafter's own draw
        dp = np.broadcast_to(q, (B, 1, V))
    lg = np.broadcast_to(logits, (B, 2, V))
    n, nxt = mod.speculative_sample(lg, draft, seed=seed, temperature=np.ones(B), draft_probs=dp)
    return np.where(n == 2, draft[:, 0], nxt)


def pin_first_token_is_target_distributed(mod=smp):
    V, B = 5, 12000
    l0 = np.array([0.5, 1.5, -0.3, 0.9, 0.1])
    logits = np.stack([l0, np.zeros(V)])
    p0 = np.exp(l0) / np.sum(np.exp(l0))
    q = np.array([0.05, 0.1, 0.45, 0.3, 0.1])      # far from p0
    for greedy in (False, True):
        tok = _emitted_first(mod, logits, q, greedy, B, seed=77 + greedy)
        ok, stat = _chi2_ok(np.bincount(tok, minlength=V), p0, B)
        assert ok, (greedy, stat)


def pin_equal_distributions_accept_everything(mod=smp):
    rng = np.random.default_rng(5)
    B, R, V = 50, 4, 7
    logits = rng.standard_normal((B, R, V))
    p = np.exp(logits) / np.exp(logits).sum(-1, keepdims=True)
    draft = np.array([[rng.choice(V, p=p[b, t]) for t in range(R - 1)] for b in range(B)], np.int32)
    n, _ = mod.speculative_sample(logits, draft, seed=9, temperature=np.ones(B), draft_probs=p[:, :R - 1])
    assert (n == R).all()


def pin_penalties_by_hand(mod=smp):
    g = json.load(open(os.path.join(GOLDEN, "penalties_hand.json")))
    for t, want in enumerate(g["rows"]):
        c = mod.row_counts(np.array(g["prior_counts"]), g["pending"], g["draft"], t, g["vocab"])
        got = mod.penalized_logits(np.array(g["logits"]), c, g["presence"], g["frequency"])
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def pin_cold_temperature_is_greedy(mod=smp):
    rng = np.random.default_rng(11)
    B, R, V = 200, 5, 9
    logits = rng.permuted(np.tile(np.arange(V, dtype=np.float64), (B, R, 1)), axis=2)   # distinct, 1 apart
    target = logits.argmax(-1).astype(np.int32)
    draft = np.where(rng.random((B, R - 1)) < 0.7, target[:, :-1], rng.integers(0, V, (B, R - 1))).astype(np.int32)
    n, nxt = mod.speculative_sample(logits, draft, seed=3, temperature=np.full(B, 0.01))
    n_g, nxt_g = acceptance.greedy_accept(draft, target)
    assert np.array_equal(n, n_g) and np.array_equal(nxt, nxt_g)


# cheapest first: a planted mistake stops at the first pin it fails
PINS = [pin_philox_kat, pin_penalties_by_hand, pin_equal_distributions_accept_everything,
        pin_cold_temperature_is_greedy, pin_gumbel_frequencies, pin_first_token_is_target_distributed]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_sampling_oracle_pin(pin):
    pin()


def test_padding_requests():
    logits = np.zeros((3, 2, 4))
    n, nxt = smp.speculative_sample(logits, np.zeros((3, 1), np.int32), seed=1, temperature=np.ones(3),
                                    slot_ids=np.array([0, -1, 2]))
    assert n[1] == 0 and nxt[1] == -1 and n[0] >= 1 and n[2] >= 1


MUTANTS = {
    "residual without the clamp": ("resid = np.maximum(p_rows[t] - q, 0.0)", "resid = np.abs(p_rows[t] - q)"),
    "residual is p": ("resid = np.maximum(p_rows[t] - q, 0.0)", "resid = p_rows[t].copy()"),
    "acceptance with p and q swapped": ("lhs, rhs = u * q[d], p_rows[t][d]", "lhs, rhs = u * p_rows[t][d], q[d]"),
    "penalty counts stop a row early": ("toks = ([] if pending is None else [int(pending)]) + [int(x) for x in draft[:t]]",
                                        "toks = ([] if pending is None else [int(pending)]) + [int(x) for x in draft[:max(t - 1, 0)]]"),
    "presence weighted by the count": ("return np.asarray(logits_row, np.float64) - frequency * c - presence * (c > 0)",
                                       "return np.asarray(logits_row, np.float64) - frequency * c - presence * c"),
    "temperature applied twice": ("p_rows.append(softmax(row / T))", "p_rows.append(softmax(row / T / T))"),
    "one Gumbel word per counter": ("w = np.choose((v & np.uint64(3)).astype(np.int64), words)", "w = words[0]"),
    "a Philox round with the key words swapped": ("c0, c1, c2, c3 = (hi1 ^ c1 ^ k0) & MASK, lo1, (hi0 ^ c3 ^ k1) & MASK, lo0",
                                                  "c0, c1, c2, c3 = (hi1 ^ c1 ^ k1) & MASK, lo1, (hi0 ^ c3 ^ k0) & MASK, lo0"),
    "bonus drawn from the first row": ("keys = np.log(p_rows[R - 1]) + gumbel_row(seed, b, R - 1, V)",
                                       "keys = np.log(p_rows[0]) + gumbel_row(seed, b, R - 1, V)"),
}


def _load_variant(text):
    d = tempfile.mkdtemp(prefix="sampling_mutant_")
    path = os.path.join(d, "sampling_variant.py")
    with open(path, "w") as f:
        f.write(text)
    spec = importlib.util.spec_from_file_location("sampling_variant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name):
    old, new = MUTANTS[name]
    src = open(smp.__file__).read()
    assert src.count(old) == 1, name
    mod = _load_variant(src.replace(old, new))
    for pin in PINS:
        try:
            pin(mod)
        except AssertionError:
            return
    raise AssertionError("no pin caught: " + name)
