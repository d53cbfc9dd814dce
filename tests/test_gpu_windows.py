"""Window states committed with the GDN layers (gdn_spec_commit_all) against
the window oracle (oracle/windows.py), bit for bit: the other per-slot states
a commit restores after the accepted rows (FreeToken PR #844, Design: a
second conv history and an n-gram context of token ids, staged per verify
row, committed with the GDN state on one upload of the slot and count
indices)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import gpu_harness as gh  # noqa: E402
import oracle  # noqa: E402
import parity as par  # noqa: E402
from oracle import windows as win  # noqa: E402
from linear_attention_verify_amd import binding as bd  # noqa: E402
from linear_attention_verify_amd import workloads as wl  # noqa: E402

DEV = "cuda"


def _windows(rng, B, R, P, specs):
    """specs: (length, entry shape, numpy dtype) per window -> host (state, rows) pairs."""
    out = []
    for length, entry, dt in specs:
        if dt == "bf16":
            state = wl.f32_to_bf16_bits(rng.standard_normal((P, length) + entry).astype(np.float32)).view(np.int16)
            rows = wl.f32_to_bf16_bits(rng.standard_normal((B, R) + entry).astype(np.float32)).view(np.int16)
        elif np.issubdtype(dt, np.integer):
            state = rng.integers(0, 1 << 20, (P, length) + entry).astype(dt)
            rows = rng.integers(0, 1 << 20, (B, R) + entry).astype(dt)
        else:
            state = rng.standard_normal((P, length) + entry).astype(np.float32)
            rows = rng.standard_normal((B, R) + entry).astype(np.float32)
        out.append((state, rows))
    return out


def _to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


SPECS = [
    (3, (96,), "bf16"),       # a conv history: W - 1 = 3 entries of 96 bf16 channels
    (2, (), np.int32),        # an n-gram context: the last 2 token ids
    (5, (8, 3), np.float32),  # entries of 2-D blocks, a window longer than the rows
    (2, (4096,), "bf16"),     # 8 KiB entries: several chunks per window
]


def test_windows_alone_match_the_oracle():
    rng = np.random.default_rng(31)
    B, R, P = 7, 4, 11
    sid = rng.choice(P, B, replace=False).astype(np.int32)
    sid[3] = -1
    acc = np.array([0, 1, 2, 3, 4, 4, 1], np.int32)
    host = _windows(rng, B, R, P, SPECS)
    dev = [(_to_dev(s), _to_dev(r)) for s, r in host]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    print("windows alone B=%d R=%d" % (B, R), flush=True)
    bd.gdn_spec_commit_all(None, [], dev, _to_dev(sid), _to_dev(acc), R, "replay", err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for (s, r), (ds, _) in zip(host, dev):
        ref = s.copy()
        assert win.commit_window(ref, r, sid, acc) == 0
        assert np.array_equal(ds.cpu().numpy(), ref)   # every slot, touched or not, bit for bit


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
def test_windows_with_gdn_layers_in_one_launch(mode):
    shape = wl.LayerShape(num_k_heads=2, num_v_heads=4, d_k=128, d_v=128, dtype="bf16")
    w = wl.small_workload(shape, batch=6, rows=5, num_slots=9, seed=702)
    sid, acc = wl.draw_requests(w)
    sid[1] = -1
    acc[4] = 0
    cases = [gh.make_case(w, layer=layer, mode=mode, slot_ids=sid, accept=acc) for layer in range(2)]
    for c in cases:
        gh.verify(c)
    torch.cuda.synchronize()
    before = [(c.ssm.clone(), c.conv.clone()) for c in cases]
    for c in cases:
        gh.commit(c)
    torch.cuda.synchronize()
    want = [(c.ssm.clone(), c.conv.clone()) for c in cases]
    for c, (s0, c0) in zip(cases, before):
        c.ssm.copy_(s0)
        c.conv.copy_(c0)

    rng = np.random.default_rng(32)
    host = _windows(rng, w.batch, w.rows, w.num_slots, SPECS[:3])
    dev = [(_to_dev(s), _to_dev(r)) for s, r in host]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    print("windows + 2 layers %s" % mode, flush=True)
    bd.gdn_spec_commit_all(cases[0].desc, [(c.ssm, c.conv, c.scratch) for c in cases], dev, cases[0].slot_ids,
                           cases[0].accept, w.rows, mode, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for c, (ws, wc) in zip(cases, want):   # the GDN layers as gdn_spec_commit gives them
        assert torch.equal(c.ssm.view(torch.int32), ws.view(torch.int32))
        assert torch.equal(c.conv.view(torch.int16), wc.view(torch.int16))
    par.assert_matches(cases[0], par.oracle_step(oracle.Oracle(), cases[0]))
    for (s, r), (ds, _) in zip(host, dev):
        ref = s.copy()
        assert win.commit_window(ref, r, sid, acc) == 0
        assert np.array_equal(ds.cpu().numpy(), ref)


def test_window_errors_leave_the_request_untouched():
    rng = np.random.default_rng(33)
    B, R, P = 4, 3, 5
    sid = np.array([0, 7, 2, 3], np.int32)        # 7 is outside this window's 5 slots: bit 0
    acc = np.array([2, 1, 4, 1], np.int32)        # 4 > R: bit 1
    host = _windows(rng, B, R, P, [(3, (), np.int32)])
    s, r = host[0]
    ds, dr = _to_dev(s), _to_dev(r)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    bd.gdn_spec_commit_all(None, [], [(ds, dr)], _to_dev(sid), _to_dev(acc), R, "replay", err)
    torch.cuda.synchronize()
    assert int(err.item()) == 3
    ref = s.copy()
    assert win.commit_window(ref, r, sid, acc) == 3
    assert np.array_equal(ds.cpu().numpy(), ref)
    assert np.array_equal(ref[2], s[2])           # the request with a bad length kept its window
