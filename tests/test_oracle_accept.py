"""Pins of the greedy-acceptance oracle: hand-derived cases
(tests/golden/accept_greedy.json), an independent vectorised formulation on
random tables, and planted mistakes that the pins must catch."""
import json
import os

import numpy as np
import pytest

from oracle import acceptance

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "accept_greedy.json")))


def _run(fn, case):
    R = len(case["target"])
    draft = np.asarray(case["draft"], np.int64).reshape(1, R - 1)
    target = np.asarray([case["target"]], np.int64)
    n, nxt = fn(draft, target, np.asarray([case["slot"]]))
    return int(n[0]), int(nxt[0])


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=[c["why"] for c in GOLDEN["cases"]])
def test_hand_cases(case):
    assert _run(acceptance.greedy_accept, case) == (case["accept_len"], case["next_token"])


def _vectorised(draft, target):
    """accept_len = 1 + index of the first mismatch among the drafts (or all of
    them): a cumulative product of the match mask, a different route to the
    same count."""
    match = (draft == target[:, :-1]).astype(np.int64)
    kept = np.cumprod(match, axis=1).sum(axis=1)
    n = 1 + kept
    return n, target[np.arange(len(n)), n - 1]


@pytest.mark.parametrize("seed", range(4))
def test_matches_vectorised_form(seed):
    rng = np.random.default_rng(seed)
    B, R = 200, 1 + seed * 2 + 2
    target = rng.integers(0, 4, size=(B, R))       # few symbols: long kept runs happen
    draft = np.where(rng.random((B, R - 1)) < 0.7, target[:, :-1], rng.integers(0, 4, size=(B, R - 1)))
    n, nxt = acceptance.greedy_accept(draft, target)
    n2, nxt2 = _vectorised(draft, target)
    assert np.array_equal(n, n2) and np.array_equal(nxt, nxt2)
    assert n.min() >= 1 and n.max() <= R


MUTANTS = [
    ("count_starts_at_zero", "        n = 1\n        for t", "        n = 0\n        for t"),
    ("compares_own_row", "int(draft[b][t - 1]) != int(target[b][t - 1])", "int(draft[b][t - 1]) != int(target[b][t])"),
    ("next_is_one_late", "nxt[b] = int(target[b][n - 1])", "nxt[b] = int(target[b][min(n, R - 1)])"),
    ("keeps_going_after_mismatch", "                break\n", "                continue\n"),
    ("padding_not_skipped", "int(slot_ids[b]) == -1", "int(slot_ids[b]) == -2"),
]


@pytest.mark.parametrize("name,before,after", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, before, after):
    src = open(acceptance.__file__).read()
    assert src.count(before) == 1, name
    ns = {}
    exec(compile(src.replace(before, after), "mutant_" + name, "exec"), ns)
    fn = ns["greedy_accept"]
    caught = any(_run(fn, c) != (c["accept_len"], c["next_token"]) for c in GOLDEN["cases"])
    assert caught, name
