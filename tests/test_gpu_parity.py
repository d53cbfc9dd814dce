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
import parity as par  # noqa: E402


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def _log(msg):
    print(msg, flush=True)


check_layer = par.check_layer
check_untouched = par.check_untouched


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


@pytest.mark.parametrize("commit", ["fused", "per-layer"])
def test_stack36_parity(orc, commit):
    """36 layers, 128 requests: all layers verified, then all committed (the
    order of a real step), in one launch for every layer (gdn_spec_commit_layers)
    or one launch per layer; every request of three layers against the oracle."""
    from linear_attention_verify_amd import binding as bd
    w = wl.WORKLOADS["stack36"]
    slot_ids, accept = wl.draw_requests(w)
    layers = [0, 17, 35]
    cases = []
    for layer in range(w.layers):
        if layer in layers:
            c = gh.make_case(w, layer=layer, slot_ids=slot_ids, accept=accept)
        else:
            # filled on the device: part of the 36-layer launch sequence, not compared
            c = gh.make_device_case(w, layer, slot_ids, accept)
        cases.append(c)
    _log("stack36 %s: %d layers resident" % (commit, len(cases)))
    before = {l: cases[l].ssm.clone() for l in layers}
    for c in cases:
        gh.verify(c)
    torch.cuda.synchronize()
    for l in layers:
        assert torch.equal(before[l].view(torch.int32), cases[l].ssm.view(torch.int32))
    del before
    if commit == "fused":
        err = torch.zeros(1, dtype=torch.int32, device=cases[0].ssm.device)
        bd.gdn_spec_commit_layers(cases[0].desc, [(c.ssm, c.conv, c.scratch) for c in cases],
                                  cases[0].slot_ids, cases[0].accept, w.rows, "replay", err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
    else:
        for c in cases:
            gh.commit(c)
        torch.cuda.synchronize()
    for c in cases:
        assert int(c.err.item()) == 0
        assert bool(torch.isfinite(c.out.float()).all())
    for l in layers:
        c = cases[l]
        _log("stack36 %s: layer %d against the oracle" % (commit, l))
        par.assert_matches(c, par.oracle_step(orc, c))
        check_untouched(c)
    del cases
    torch.cuda.empty_cache()


PAIRS = [(32, "f32"), (32, "bf16"), (64, "f32"), (64, "bf16"), (128, "f32"), (128, "bf16")]


def _rows_case(rows, d, dtype, mode):
    shape = wl.LayerShape(num_k_heads=2, num_v_heads=4, d_k=d, d_v=d, dtype=dtype)
    w = wl.small_workload(shape, batch=5, rows=rows, num_slots=11, seed=100 + rows)
    slot_ids, _ = wl.draw_requests(w)
    slot_ids[3] = -1
    accept = np.array([rows, 0, 1, min(2, rows), max(rows - 1, 0)], np.int32)
    return gh.make_case(w, slot_ids=slot_ids, accept=accept, mode=mode)


@pytest.mark.parametrize("rows", list(range(1, 10)))
@pytest.mark.parametrize("d,dtype", PAIRS)
def test_rows_and_head_dims(orc, rows, d, dtype):
    """Every row count 1..9 at every supported (head dim, storage type),
    ragged accept lengths (0..rows), padding and GQA (2 value heads per key
    head; at d = 128 the matrix-core kernel, staged for bf16 and per channel
    for fp32)."""
    c = _rows_case(rows, d, dtype, "replay")
    _log("rows=%d d=%d %s replay" % (rows, d, dtype))
    check_layer(orc, c)
    check_untouched(c)
    assert not bool(c.out[3].float().abs().sum())


@pytest.mark.parametrize("rows", [1, 3, 9])
@pytest.mark.parametrize("d,dtype", PAIRS)
def test_rows_and_head_dims_snapshot(orc, rows, d, dtype):
    c = _rows_case(rows, d, dtype, "snapshot")
    _log("rows=%d d=%d %s snapshot" % (rows, d, dtype))
    check_layer(orc, c)
    check_untouched(c)
    assert not bool(c.out[3].float().abs().sum())


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
@pytest.mark.parametrize("rows", [3, 9])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hk,hv", [(3, 3), (2, 8), (3, 6)])
def test_head_groups_at_d128(orc, hk, hv, dtype, rows, mode):
    """Value heads per key head G = 1 (one head per workgroup), 4 (two pairs of
    value heads per key head, only the first storing its q/k inputs) and 2
    with an odd key-head count."""
    shape = wl.LayerShape(num_k_heads=hk, num_v_heads=hv, d_k=128, d_v=128, dtype=dtype)
    w = wl.small_workload(shape, batch=3, rows=rows, num_slots=7, seed=300 + rows + hv)
    c = gh.make_case(w, mode=mode)
    _log("G hk=%d hv=%d %s rows=%d %s" % (hk, hv, dtype, rows, mode))
    check_layer(orc, c)
    check_untouched(c)


@pytest.mark.parametrize("rows", [1, 2, 3, 5, 8, 9])
def test_large_batch_kernel_at_every_row_count(orc, rows):
    """512 (request, value-head pair) units at d = 128, bf16: the one-round
    kernel (smaller batches take the split kernel), ragged accept lengths and
    two padding requests; every request against the oracle."""
    w = wl.small_workload(wl.QWEN3_NEXT_LAYER, batch=32, rows=rows, num_slots=80, seed=900 + rows)
    slot_ids, _ = wl.draw_requests(w)
    slot_ids[[5, 17]] = -1
    accept = np.random.default_rng(rows).integers(0, rows + 1, size=32).astype(np.int32)
    c = gh.make_case(w, slot_ids=slot_ids, accept=accept)
    _log("one-round kernel rows=%d" % rows)
    check_layer(orc, c)
    check_untouched(c)
    assert not bool(c.out[[5, 17]].float().abs().sum())


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
@pytest.mark.parametrize("d,dtype", PAIRS)
def test_identity_gate_leaves_the_state_bitwise(orc, d, dtype, mode):
    """alpha = 1, beta = 0 on every row: each correction e_t is zero, so the
    committed state equals the drawn one bit for bit, and o_t = scale S_0 q_t
    (against the oracle)."""
    shape = wl.LayerShape(num_k_heads=2, num_v_heads=4, d_k=d, d_v=d, dtype=dtype)
    w = wl.small_workload(shape, batch=4, rows=6, num_slots=9, seed=500 + d)
    draw = wl.draw_layer(w)
    draw["alpha"] = wl.to_storage(np.ones_like(wl.storage_to_f32(draw["alpha"], dtype)), dtype)
    draw["beta"] = wl.to_storage(np.zeros_like(wl.storage_to_f32(draw["beta"], dtype)), dtype)
    slot_ids, _ = wl.draw_requests(w)
    accept = np.array([6, 3, 1, 5], np.int32)
    c = gh.make_case(w, slot_ids=slot_ids, accept=accept, draw=draw, mode=mode)
    _log("identity gate d=%d %s %s" % (d, dtype, mode))
    ssm0 = c.ssm.clone()
    check_layer(orc, c)
    assert torch.equal(c.ssm.view(torch.int32), ssm0.view(torch.int32)), "state changed under alpha=1, beta=0"


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (128, "f32"), (64, "f32"), (32, "bf16")])
def test_zero_and_eps_dominated_keys_and_queries(orc, d, dtype, mode):
    """Conv taps set to zero or scaled by 1e-4 on chosen q/k channels: key head
    0's q is zero (its heads' o must come out zero), key head 1's k is zero
    (e_t = b_t v_t, S_n = (prod a) S_0), and key head 2's q and k are so small
    that sum x^2 is below l2_eps, so the normalisation is decided by eps."""
    shape = wl.LayerShape(num_k_heads=3, num_v_heads=6, d_k=d, d_v=d, dtype=dtype)
    w = wl.small_workload(shape, batch=3, rows=5, num_slots=8, seed=600 + d)
    draw = wl.draw_layer(w)
    cw = wl.storage_to_f32(draw["conv_w"], dtype).copy()
    HK = shape.num_k_heads
    q0 = slice(0, d)
    k1 = slice(HK * d + d, HK * d + 2 * d)
    q2, k2 = slice(2 * d, 3 * d), slice(HK * d + 2 * d, HK * d + 3 * d)
    cw[q0] = 0.0
    cw[k1] = 0.0
    cw[q2] *= 1e-4
    cw[k2] *= 1e-4
    draw["conv_w"] = wl.to_storage(cw, dtype)
    c = gh.make_case(w, draw=draw, mode=mode)
    _log("zero/eps keys d=%d %s %s" % (d, dtype, mode))
    check_layer(orc, c)
    o = c.out.float()
    assert not bool(o[:, :, 0:2].abs().sum()), "a zero query gave a non-zero output"
    assert bool(o[:, :, 4:6].abs().sum()), "eps-dominated heads came out zero"


@pytest.mark.parametrize("name", ["tiny-fp32", "single-stream", "low-concurrency", "saturated-b64"])
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
    calls leave: conv history bitwise, state to tolerance; both are also
    compared with the oracle, and each single-row call's o with the oracle's
    o of that row (for requests that have accepted every earlier row)."""
    shape = wl.LayerShape(num_k_heads=2, num_v_heads=4, d_k=64, d_v=64, dtype="f32")
    w = wl.small_workload(shape, batch=3, rows=5, num_slots=6, seed=7)
    slot_ids, _ = wl.draw_requests(w)
    accept = np.array([5, 3, 1], np.int32)
    big = gh.make_case(w, slot_ids=slot_ids, accept=accept)
    ref = par.oracle_step(orc, big)
    gh.verify(big)
    gh.commit(big)
    # one row at a time on a copy of the same pools, taps and inputs
    w1 = wl.small_workload(shape, batch=3, rows=1, num_slots=6, seed=7)
    fresh = gh.make_case(w, slot_ids=slot_ids, accept=accept)
    step = gh.make_case(w1, slot_ids=slot_ids, accept=np.ones(3, np.int32))
    step.ssm.copy_(fresh.ssm)
    step.conv.copy_(fresh.conv)
    step.conv_w.copy_(fresh.conv_w)
    atol, rtol = gh.tolerances(shape)
    for t in range(5):
        step.x.copy_(fresh.x[:, t:t + 1])
        step.alpha.copy_(fresh.alpha[:, t:t + 1])
        step.beta.copy_(fresh.beta[:, t:t + 1])
        step.accept.copy_(torch.from_numpy((accept > t).astype(np.int32)))
        gh.verify(step)
        gh.commit(step)
        torch.cuda.synchronize()
        live = np.flatnonzero(accept > t)
        np.testing.assert_allclose(step.out.cpu().numpy()[live, 0], ref.out[live, t], atol=atol, rtol=rtol)
    torch.cuda.synchronize()
    assert int(big.err.item()) == 0 and int(step.err.item()) == 0
    assert torch.equal(big.conv.view(torch.int32), step.conv.view(torch.int32))
    np.testing.assert_allclose(big.ssm.cpu().numpy(), step.ssm.cpu().numpy(), atol=1e-5, rtol=1e-4)
    par.assert_matches(big, ref)
    par.assert_states_match(big, ref, ssm=step.ssm, conv=step.conv)


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
