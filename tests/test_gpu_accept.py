"""Device-side greedy acceptance against the oracle, bit for bit, and fed
straight into the commit (the accept lengths never leave the device)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import gpu_harness as gh  # noqa: E402
import oracle  # noqa: E402
from oracle import acceptance  # noqa: E402
from linear_attention_verify_amd import binding as bd  # noqa: E402
from linear_attention_verify_amd import workloads as wl  # noqa: E402

DEV = "cuda"


def _device_accept(draft, target, slot_ids, rows):
    B = target.shape[0]
    d = torch.from_numpy(np.ascontiguousarray(draft, np.int32)).to(DEV) if rows > 1 else None
    t = torch.from_numpy(np.ascontiguousarray(target, np.int32)).to(DEV)
    s = None if slot_ids is None else torch.from_numpy(np.asarray(slot_ids, np.int32)).to(DEV)
    n = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    nxt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    bd.gdn_spec_accept_greedy(d, t, s, rows, n, nxt)
    torch.cuda.synchronize()
    return n.cpu().numpy(), nxt.cpu().numpy()


@pytest.mark.parametrize("rows", [1, 2, 4, 9])
@pytest.mark.parametrize("batch", [1, 64, 300])
def test_accept_matches_oracle(rows, batch):
    rng = np.random.default_rng(rows * 1000 + batch)
    target = rng.integers(0, 3, size=(batch, rows)).astype(np.int32)
    draft = np.where(rng.random((batch, rows - 1)) < 0.75, target[:, :-1],
                     rng.integers(0, 3, size=(batch, rows - 1))).astype(np.int32)
    slots = np.arange(batch, dtype=np.int32)
    slots[rng.random(batch) < 0.1] = -1
    print("accept rows=%d batch=%d" % (rows, batch), flush=True)
    n, nxt = _device_accept(draft, target, slots, rows)
    n_ref, nxt_ref = acceptance.greedy_accept(draft, target, slots)
    assert np.array_equal(n, n_ref) and np.array_equal(nxt, nxt_ref)
    n2, _ = _device_accept(draft, target, None, rows)
    assert np.array_equal(n2, acceptance.greedy_accept(draft, target)[0])


def test_drawn_tokens_realise_the_workload_accept_lengths():
    w = wl.WORKLOADS["saturated-b64"]
    _, accept = wl.draw_requests(w)
    draft, target = wl.draw_tokens(w, accept)
    n, _ = _device_accept(draft, target, None, w.rows)
    assert np.array_equal(n, accept)


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
def test_device_acceptance_feeds_the_commit(mode):
    """verify -> device acceptance -> commit, with padding: the committed
    state and history equal the oracle's for the oracle's accept lengths."""
    w = wl.WORKLOADS["low-concurrency"]
    sid, acc = wl.draw_requests(w)
    sid[3] = -1
    c = gh.make_case(w, mode=mode, slot_ids=sid)
    draft, target = wl.draw_tokens(w, acc)
    n_ref, _ = acceptance.greedy_accept(draft, target, sid)
    gh.verify(c)
    bd.gdn_spec_accept_greedy(torch.from_numpy(draft).to(DEV), torch.from_numpy(target).to(DEV), c.slot_ids,
                              w.rows, c.accept)   # the commit reads these lengths
    gh.commit(c)
    torch.cuda.synchronize()
    assert int(c.err.item()) == 0
    assert np.array_equal(c.accept.cpu().numpy(), n_ref)

    orc = oracle.Oracle()
    reqs = np.arange(w.batch)
    hs, hc, hsid = gh.host_pools_for(c, reqs)
    d = c.draw
    e = orc.commit(w.shape, hs, hc, d["conv_w"], d["x"], d["alpha"], d["beta"], hsid, n_ref, w.rows,
                   nthreads=16)
    assert e == 0
    act = hsid >= 0
    slots = torch.from_numpy(sid[act].astype(np.int64)).to(DEV)
    satol, srtol = gh.state_tolerances(w.shape)
    np.testing.assert_allclose(c.ssm[slots].cpu().numpy(), hs[hsid[act]], atol=satol, rtol=srtol)
    conv_gpu = gh.to_storage_numpy(c.conv[slots], w.shape.dtype)
    assert np.array_equal(conv_gpu.view(np.uint8), hc[hsid[act]].view(np.uint8))
