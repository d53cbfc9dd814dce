"""Pins of the window-state commit oracle (oracle/windows.py), on the CPU.

None of them re-types the oracle's one line of arithmetic:
  - hand-worked windows (tests/golden/window_hand.json), a window shorter and
    one longer than the verify rows;
  - the GDN conv history is such a window: committing the raw verify rows
    into it must give bit for bit what the C oracle's conv commit gives;
  - multi-dimensional entries move whole;
  - padding, n = 0, bad slots and bad accept lengths;
  - planted mistakes in a copy of the module each fail one of the above.
"""
import importlib.util
import json
import os
import tempfile

import numpy as np
import pytest

import oracle
from oracle import windows as win
from linear_attention_verify_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pin_hand(mod=win):
    g = json.load(open(os.path.join(GOLDEN, "window_hand.json")))
    for case in (g, g["long_window"]):
        for n, want in case["after"].items():
            state = np.array([case["window"]], np.int32)
            rows = np.array([case["rows"]], np.int32)
            err = mod.commit_window(state, rows, np.array([0]), np.array([int(n)]))
            assert err == 0 and state[0].tolist() == want, (n, state[0].tolist(), want)


def pin_conv_history_is_a_window(mod=win):
    tiny = wl.Workload(name="t", shape=wl.WORKLOADS["tiny-fp32"].shape, batch=5, rows=4, num_slots=9, seed=3)
    for work in (tiny,):
        sid, acc = wl.draw_requests(work)
        acc = np.array([0, 1, 2, 4, 3][:work.batch], np.int32)
        sid = sid.copy()
        sid[2] = -1
        d = wl.draw_layer(work)
        ssm, conv = wl.build_pools(work, d, sid)
        conv_ref = conv.copy()
        err = oracle.Oracle().commit(work.shape, ssm.copy(), conv_ref, d["conv_w"], d["x"], d["alpha"], d["beta"],
                                     sid, acc, work.rows)
        assert err == 0
        conv_win = conv.copy()
        err = mod.commit_window(conv_win, d["x"], sid, acc)
        assert err == 0
        assert np.array_equal(conv_win.view(np.uint8), conv_ref.view(np.uint8))


def pin_entries_move_whole(mod=win):
    rng = np.random.default_rng(4)
    state = rng.standard_normal((3, 2, 2, 3)).astype(np.float32)   # P = 3 slots, L = 2 entries of 2 x 3
    rows = rng.standard_normal((2, 3, 2, 3)).astype(np.float32)    # B = 2, R = 3
    before = state.copy()
    err = mod.commit_window(state, rows, np.array([2, 0]), np.array([3, 1]))
    assert err == 0
    assert np.array_equal(state[2], rows[0, 1:3])
    assert np.array_equal(state[0], np.stack([before[0, 1], rows[1, 0]]))
    assert np.array_equal(state[1], before[1])


def pin_skips_and_errors(mod=win):
    state = np.arange(12, dtype=np.int32).reshape(4, 3)
    rows = np.full((4, 2, ), 99, np.int32).reshape(4, 2)
    before = state.copy()
    err = mod.commit_window(state, rows, np.array([-1, 7, 1, 2]), np.array([2, 1, 3, 0]))
    assert err == win.ERR_SLOT | win.ERR_ACCEPT
    assert np.array_equal(state, before)   # padding, bad slot, bad length, n = 0: nothing moves


PINS = [pin_hand, pin_entries_move_whole, pin_skips_and_errors, pin_conv_history_is_a_window]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_window_oracle_pin(pin):
    pin()


MUTANTS = {
    "one entry early": ("state[s] = window[n:n + L]", "state[s] = window[n - 1:n - 1 + L]"),
    "rows not taken": ("window = np.concatenate([state[s], rows[b, :n]], axis=0)",
                       "window = np.concatenate([state[s], rows[b, :max(n - 1, 0)]], axis=0)"),
    "newest rows first": ("window = np.concatenate([state[s], rows[b, :n]], axis=0)",
                          "window = np.concatenate([state[s], rows[b, :n][::-1]], axis=0)"),
    "n = 0 taken as one row": ("        if n == 0:\n            continue\n", "        if n == 0:\n            n = 1\n"),
    "bad slot committed": ("            err |= ERR_SLOT\n            continue\n", "            err |= ERR_SLOT\n"),
}


def _load_variant(text):
    d = tempfile.mkdtemp(prefix="windows_mutant_")
    path = os.path.join(d, "windows_variant.py")
    with open(path, "w") as f:
        f.write(text)
    spec = importlib.util.spec_from_file_location("windows_variant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name):
    old, new = MUTANTS[name]
    src = open(win.__file__).read()
    assert src.count(old) == 1, name
    mod = _load_variant(src.replace(old, new))
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, IndexError, ValueError):
            return
    raise AssertionError("no pin caught: " + name)
