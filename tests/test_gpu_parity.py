"""GPU parity: the HIP verify/commit against the CPU oracle, through the C ABI.

Element by element on the same seeded inputs: o of every verify row, the
committed state of every request's slot, and the conv history (bitwise: it is
a copy of raw inputs). Untouched slots must keep their NaN sentinels bit for
bit; the error flag must stay clear.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from linear_attention_verify_amd import workloads as wl  # noqa: E402
import gpu_harness as gh  # noqa: E402


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def _log(msg):
    print(msg, flush=True)


def check_layer(orc, c, requests=None, nthreads=16):
    """Runs verify + commit on the device and compares with the oracle on
    `requests` (all by default)."""
    w, s = c.w, c.w.shape
    reqs = np.arange(w.batch) if requests is None else np.asarray(requests)
    ssm_before = c.ssm.clone()
    conv_before = c.conv.clone()
    gh.verify(c)
    torch.cuda.synchronize()
    assert torch.equal(c.ssm.view(torch.int32), ssm_before.view(torch.int32)), "verify wrote the state"
    assert torch.equal(c.conv.view(torch.int16 if s.dtype == "bf16" else torch.int32),
                       conv_before.view(torch.int16 if s.dtype == "bf16" else torch.int32))
    gh.commit(c)
    torch.cuda.synchronize()
    assert int(c.err.item()) == 0

    hs, hc, hsid = gh.host_pools_for(c, reqs)
    d = c.draw
    sub = lambda a: np.ascontiguousarray(a[reqs])
    o_ref, _, err = orc.verify(s, hs, hc, d["conv_w"], sub(d["x"]), sub(d["alpha"]), sub(d["beta"]),
                               hsid, w.rows, nthreads=nthreads)
    assert err == 0
    err = orc.commit(s, hs, hc, d["conv_w"], sub(d["x"]), sub(d["alpha"]), sub(d["beta"]), hsid,
                     np.ascontiguousarray(c.accept_np[reqs]), w.rows, nthreads=nthreads)
    assert err == 0

    atol, rtol = gh.tolerances(s)
    o_gpu = gh.tensor_f64(c.out, s.dtype)[reqs]
    np.testing.assert_allclose(o_gpu, o_ref, atol=atol, rtol=rtol)

    compare_states(c, reqs, hs, hc, hsid)


def compare_states(c, reqs, hs, hc, hsid):
    """Committed state (tolerance) and conv history (bitwise) of the active requests."""
    s = c.w.shape
    act = hsid >= 0
    sl = c.slot_ids_np[reqs][act].astype(np.int64)
    assert ((sl >= 0) & (sl < c.w.num_slots)).all(), "slot index outside the pool"
    slots = torch.from_numpy(sl).to(c.ssm.device)
    s_gpu = c.ssm[slots].cpu().numpy()
    satol, srtol = gh.state_tolerances(s)
    np.testing.assert_allclose(s_gpu, hs[hsid[act]], atol=satol, rtol=srtol)
    conv_gpu = gh.to_storage_numpy(c.conv[slots], s.dtype)
    assert np.array_equal(conv_gpu.view(np.uint8), hc[hsid[act]].view(np.uint8)), "conv history differs"


def check_untouched(c):
    """Every slot no request owns keeps its sentinel bits."""
    w, s = c.w, c.w.shape
    mask = torch.ones(w.num_slots, dtype=torch.bool, device=c.ssm.device)
    sid = c.slot_ids_np
    active = sid[(sid >= 0) & (sid < w.num_slots)].astype(np.int64)
    mask[torch.from_numpy(active).to(c.ssm.device)] = False
    rest = c.ssm[mask].view(torch.int32)
    assert bool((rest == int(np.int32(wl.F32_SENTINEL.view(np.int32)))).all())
    if s.dtype == "bf16":
        crest = c.conv[mask].view(torch.int16)
        assert bool((crest == int(np.int16(wl.BF16_SENTINEL.view(np.int16)))).all())


SMALL = ["tiny-fp32", "single-stream", "low-concurrency"]


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
@pytest.mark.parametrize("name", SMALL)
def test_workload_parity(orc, name, mode):
    w = wl.WORKLOADS[name]
    _log("parity %s %s B=%d R=%d" % (name, mode, w.batch, w.rows))
    c = gh.make_case(w, mode=mode)
    check_layer(orc, c)
    check_untouched(c)


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
def test_saturated_b64_parity(orc, mode):
    """Batch 64, 9 rows, geometric accept lengths: every request against the oracle."""
    w = wl.WORKLOADS["saturated-b64"]
    _log("parity saturated-b64 %s" % mode)
    c = gh.make_case(w, mode=mode)
    check_layer(orc, c)
    check_untouched(c)


def test_stack36_parity(orc):
    """36 layers, 128 requests: all layers verified, then all committed (the
    order of a real step); sampled layers and requests against the oracle."""
    w = wl.WORKLOADS["stack36"]
    slot_ids, accept = wl.draw_requests(w)
    layers = [0, 17, 35]
    sample = np.random.default_rng(99).choice(w.batch, size=12, replace=False)
    cases = []
    for layer in range(w.layers):
        if layer in layers:
            c = gh.make_case(w, layer=layer, slot_ids=slot_ids, accept=accept)
        else:
            # filled on the device: part of the 36-layer launch sequence, not compared
            c = gh.make_device_case(w, layer, slot_ids, accept)
        cases.append(c)
    _log("stack36: %d layers resident" % len(cases))
    before = {l: cases[l].ssm.clone() for l in layers}
    for c in cases:
        gh.verify(c)
    torch.cuda.synchronize()
    for l in layers:
        assert torch.equal(before[l].view(torch.int32), cases[l].ssm.view(torch.int32))
    for c in cases:
        gh.commit(c)
    torch.cuda.synchronize()
    for c in cases:
        assert int(c.err.item()) == 0
        assert bool(torch.isfinite(c.out.float()).all())
    for l in layers:
        c = cases[l]
        assert int(c.err.item()) == 0
        _compare_after(orc, c, sample)
        check_untouched(c)


def _compare_after(orc, c, reqs):
    """The oracle, started from the drawn committed state, against the device results."""
    w, s, d = c.w, c.w.shape, c.draw
    hs, hc, hsid = gh.host_pools_for(c, reqs)
    sub = lambda a: np.ascontiguousarray(a[reqs])
    o_ref, _, err = orc.verify(s, hs, hc, d["conv_w"], sub(d["x"]), sub(d["alpha"]), sub(d["beta"]),
                               hsid, w.rows, nthreads=16)
    assert err == 0
    assert orc.commit(s, hs, hc, d["conv_w"], sub(d["x"]), sub(d["alpha"]), sub(d["beta"]), hsid,
                      np.ascontiguousarray(c.accept_np[reqs]), w.rows, nthreads=16) == 0
    atol, rtol = gh.tolerances(s)
    np.testing.assert_allclose(gh.tensor_f64(c.out, s.dtype)[reqs], o_ref, atol=atol, rtol=rtol)
    compare_states(c, reqs, hs, hc, hsid)


@pytest.mark.parametrize("rows", list(range(1, 10)))
@pytest.mark.parametrize("d,dtype", [(32, "f32"), (64, "bf16"), (128, "bf16")])
def test_rows_and_head_dims(orc, rows, d, dtype):
    """Every row count 1..9 at every supported head dim, ragged accept lengths
    (0..rows), padding and GQA (2 value heads per key head)."""
    shape = wl.LayerShape(num_k_heads=2, num_v_heads=4, d_k=d, d_v=d, dtype=dtype)
    w = wl.small_workload(shape, batch=5, rows=rows, num_slots=11, seed=100 + rows)
    slot_ids, _ = wl.draw_requests(w)
    slot_ids[3] = -1
    accept = np.array([rows, 0, 1, min(2, rows), max(rows - 1, 0)], np.int32)
    c = gh.make_case(w, slot_ids=slot_ids, accept=accept)
    _log("rows=%d d=%d %s" % (rows, d, dtype))
    check_layer(orc, c)
    check_untouched(c)
    assert not bool(c.out[3].float().abs().sum())


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
@pytest.mark.parametrize("rows", [3, 9])
@pytest.mark.parametrize("hk,hv", [(3, 3), (2, 8), (3, 6)])
def test_head_groups_at_d128(orc, hk, hv, rows, mode):
    """Value heads per key head G = 1 (one head per workgroup), 4 (two pairs of
    value heads per key head, only the first storing its q/k inputs) and 2
    with an odd key-head count."""
    shape = wl.LayerShape(num_k_heads=hk, num_v_heads=hv, d_k=128, d_v=128, dtype="bf16")
    w = wl.small_workload(shape, batch=3, rows=rows, num_slots=7, seed=300 + rows + hv)
    c = gh.make_case(w, mode=mode)
    _log("G hk=%d hv=%d rows=%d %s" % (hk, hv, rows, mode))
    check_layer(orc, c)
    check_untouched(c)


@pytest.mark.parametrize("name", ["tiny-fp32", "low-concurrency"])
def test_replay_and_snapshot_agree_bitwise(name):
    w = wl.WORKLOADS[name]
    cr = gh.make_case(w, mode="replay")
    cs = gh.make_case(w, mode="snapshot")
    for c in (cr, cs):
        gh.verify(c)
        gh.commit(c)
    torch.cuda.synchronize()
    assert torch.equal(cr.out.view(torch.int16 if w.shape.dtype == "bf16" else torch.int32),
                       cs.out.view(torch.int16 if w.shape.dtype == "bf16" else torch.int32))
    assert torch.equal(cr.ssm.view(torch.int32), cs.ssm.view(torch.int32))


def test_deterministic_reruns():
    w = wl.WORKLOADS["low-concurrency"]
    a = gh.make_case(w)
    b = gh.make_case(w)
    for c in (a, b):
        gh.verify(c)
        gh.commit(c)
    torch.cuda.synchronize()
    assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))
    assert torch.equal(a.ssm.view(torch.int32), b.ssm.view(torch.int32))
    assert torch.equal(a.conv.view(torch.int16), b.conv.view(torch.int16))


def test_steps_in_sequence_match_decode_steps(orc):
    """verify(R) + commit(n) on the GPU leaves what n single-row verify+commit
    calls leave: conv history bitwise, state to tolerance."""
    shape = wl.LayerShape(num_k_heads=2, num_v_heads=4, d_k=64, d_v=64, dtype="f32")
    w = wl.small_workload(shape, batch=3, rows=5, num_slots=6, seed=7)
    slot_ids, _ = wl.draw_requests(w)
    accept = np.array([5, 3, 1], np.int32)
    big = gh.make_case(w, slot_ids=slot_ids, accept=accept)
    gh.verify(big)
    gh.commit(big)
    # one row at a time on a copy of the same pools, taps and inputs
    w1 = wl.small_workload(shape, batch=3, rows=1, num_slots=6, seed=7)
    fresh = gh.make_case(w, slot_ids=slot_ids, accept=accept)
    step = gh.make_case(w1, slot_ids=slot_ids, accept=np.ones(3, np.int32))
    step.ssm.copy_(fresh.ssm)
    step.conv.copy_(fresh.conv)
    step.conv_w.copy_(fresh.conv_w)
    for t in range(5):
        step.x.copy_(fresh.x[:, t:t + 1])
        step.alpha.copy_(fresh.alpha[:, t:t + 1])
        step.beta.copy_(fresh.beta[:, t:t + 1])
        step.accept.copy_(torch.from_numpy((accept > t).astype(np.int32)))
        gh.verify(step)
        gh.commit(step)
    torch.cuda.synchronize()
    assert int(big.err.item()) == 0 and int(step.err.item()) == 0
    assert torch.equal(big.conv.view(torch.int32), step.conv.view(torch.int32))
    np.testing.assert_allclose(big.ssm.cpu().numpy(), step.ssm.cpu().numpy(), atol=1e-5, rtol=1e-4)


def test_bad_slots_and_accept_lengths_are_flagged():
    shape = wl.LayerShape(num_k_heads=2, num_v_heads=4, d_k=32, d_v=32, dtype="f32")
    w = wl.small_workload(shape, batch=4, rows=3, num_slots=6, seed=5)
    slot_ids, _ = wl.draw_requests(w)
    bad = slot_ids.copy()
    bad[1] = 6            # out of range
    accept = np.array([2, 2, 4, 0], np.int32)   # request 2: > rows
    c = gh.make_case(w, slot_ids=bad, accept=accept)
    base = gh.make_case(w, slot_ids=bad, accept=accept)
    gh.verify(c)
    torch.cuda.synchronize()
    assert int(c.err.item()) & 1
    assert not bool(c.out[1].abs().sum())
    c.err.zero_()
    gh.commit(c)
    torch.cuda.synchronize()
    assert int(c.err.item()) == 3
    # request 0 committed; 1 (bad slot), 2 (bad accept), 3 (accept 0) untouched
    for b in (2, 3):
        s = int(bad[b])
        assert torch.equal(c.ssm[s].view(torch.int32), base.ssm[s].view(torch.int32))
        assert torch.equal(c.conv[s].view(torch.int32), base.conv[s].view(torch.int32))
    s0 = int(bad[0])
    assert not torch.equal(c.ssm[s0].view(torch.int32), base.ssm[s0].view(torch.int32))


def test_empty_batch_is_a_no_op():
    from linear_attention_verify_amd import binding as bd
    w = wl.WORKLOADS["tiny-fp32"]
    c = gh.make_case(w)
    empty = torch.empty(0, dtype=torch.int32, device="cuda")
    bd.gdn_spec_verify(c.desc, c.ssm, c.conv, c.conv_w, c.x, c.alpha, c.beta, empty, w.rows,
                       "replay", c.scratch, c.out, c.err)
    bd.gdn_spec_commit(c.desc, c.ssm, c.conv, empty, empty, w.rows, "replay", c.scratch, c.err)
    torch.cuda.synchronize()
    assert int(c.err.item()) == 0
