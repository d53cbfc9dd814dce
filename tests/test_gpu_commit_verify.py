"""Commit-verify (gdn_spec_commit_verify): one launch that commits the
previous step's accepted rows into the state on its way into this step's
verify (FreeToken issue #828, Design: the verify only reads the state, the
commit replays the accepted rows; lmdeploy PR #5006, Verification path: a
gated-delta-rule verify-and-commit kernel mode).

Checked bit for bit against gdn_spec_commit followed by gdn_spec_verify
(pool, history, outputs and the new stash), with batches rearranged between
the steps (a request leaving, one joining, padding, a permuted order), and
against the oracle's commit then verify."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import gpu_harness as gh  # noqa: E402
import oracle  # noqa: E402
from linear_attention_verify_amd import binding as bd  # noqa: E402
from linear_attention_verify_amd import workloads as wl  # noqa: E402

DEV = "cuda"
QWEN = wl.LayerShape(num_k_heads=16, num_v_heads=32, d_k=128, d_v=128, dtype="bf16")
# four value heads per key head: two workgroups (pairs) share a key head's q/k channels
GQA4 = wl.LayerShape(num_k_heads=8, num_v_heads=32, d_k=128, d_v=128, dtype="bf16")


def _zero_scratch(desc, B, R, mode="replay"):
    return torch.zeros(max(bd.gdn_spec_scratch_bytes(desc, B, R, mode), 16), dtype=torch.uint8, device=DEV)


def _plan(sid1, P, seed):
    """The next step's batch: every step-1 request but one (all of them in a
    batch of one or two), shuffled, plus a request on a free slot and a
    padding row. Returns (slot ids, source rows, the step-1 rows left behind)."""
    rng = np.random.default_rng(seed)
    B1 = len(sid1)
    keep = np.sort(rng.choice(B1, B1 - 1 if B1 > 2 else B1, replace=False))
    dropped = np.setdiff1d(np.arange(B1), keep)
    new_slot = int(rng.choice(np.setdiff1d(np.arange(P), sid1)))
    order = [int(r) for r in keep] + [-1, -2]
    rng.shuffle(order)
    sid2, src = [], []
    for r in order:
        if r >= 0:
            sid2.append(int(sid1[r]))
            src.append(r)
        elif r == -1:
            sid2.append(new_slot)
            src.append(-1)
        else:
            sid2.append(-1)
            src.append(int(rng.integers(0, B1)))   # a padding row's source is ignored
    return np.array(sid2, np.int32), np.array(src, np.int32), dropped, new_slot


def _two_steps(R, B1, seed, accept_edges=True, shape=QWEN, mode="replay"):
    w = wl.small_workload(shape, batch=B1, rows=R, num_slots=3 * B1 + 2, seed=seed)
    sid1, acc1 = wl.draw_requests(w)
    if accept_edges:
        acc1[0] = R                                # every row accepted
        if B1 > 1:
            acc1[1] = 0                            # nothing accepted
    c = gh.make_case(w, slot_ids=sid1, accept=acc1, mode=mode)
    sid2, src, dropped, new_slot = _plan(sid1, w.num_slots, seed + 1)
    w2 = wl.small_workload(shape, batch=len(sid2), rows=R, num_slots=w.num_slots, seed=seed + 2)
    d2 = wl.draw_layer(w2, 0)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    c.ssm[new_slot] = torch.randn(c.ssm[new_slot].shape, generator=gen, device=DEV)
    c.conv[new_slot] = torch.randn(c.conv[new_slot].shape, generator=gen, device=DEV).to(torch.bfloat16)
    return c, w2, d2, sid2, src, dropped


def _step2(c, w2, d2, sid2):
    s = c.w.shape
    ins = {k: gh.storage_tensor(d2[k], s.dtype) for k in ("x", "alpha", "beta")}
    out = torch.full((w2.batch, w2.rows, s.num_v_heads, s.d_v), float("nan"), dtype=torch.bfloat16, device=DEV)
    return ins, out, torch.from_numpy(sid2).to(DEV)


def _run_both(c, w2, d2, sid2, src, dropped):
    """Returns (reference, fused) tuples of (ssm, conv, out, new scratch, err)."""
    R = c.w.rows
    gh.verify(c)                                    # step 1, the previous step's stash in c.scratch
    torch.cuda.synchronize()
    ssm0, conv0 = c.ssm.clone(), c.conv.clone()
    ins, out, sid2_t = _step2(c, w2, d2, sid2)

    # commit, then verify
    gh.commit(c)
    sb = _zero_scratch(c.desc, w2.batch, R, c.mode)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    bd.gdn_spec_verify(c.desc, c.ssm, c.conv, c.conv_w, ins["x"], ins["alpha"], ins["beta"], sid2_t, R, c.mode,
                       sb, out, err)
    torch.cuda.synchronize()
    ref = (c.ssm.clone(), c.conv.clone(), out.clone(), sb.clone(), int(err.item()) | int(c.err.item()))

    # the rows left behind committed on their own, the rest with the verify
    c.ssm.copy_(ssm0)
    c.conv.copy_(conv0)
    c.err.zero_()
    lone = np.full_like(c.slot_ids_np, -1)
    lone[dropped] = c.slot_ids_np[dropped]
    bd.gdn_spec_commit(c.desc, c.ssm, c.conv, torch.from_numpy(lone).to(DEV), c.accept, R, c.mode, c.scratch,
                       c.err)
    sb2 = _zero_scratch(c.desc, w2.batch, R, c.mode)
    out.fill_(float("nan"))
    err2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    print("commit-verify %s B=%d->%d R=%d" % (c.mode, c.w.batch, w2.batch, R), flush=True)
    bd.gdn_spec_commit_verify(c.desc, c.ssm, c.conv, c.conv_w, ins["x"], ins["alpha"], ins["beta"], sid2_t, R, sb2,
                              torch.from_numpy(src).to(DEV), c.scratch, c.slot_ids, c.accept, out, err2,
                              host_slot_ids=sid2, host_src_row=src, mode=c.mode)
    torch.cuda.synchronize()
    fused = (c.ssm.clone(), c.conv.clone(), out.clone(), sb2.clone(), int(err2.item()) | int(c.err.item()))
    return ref, fused


def _bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
@pytest.mark.parametrize("R,B1,shape", [
    (4, 16, QWEN), (9, 16, QWEN),              # one unit per compute unit or more (one-round / snapshot kernel)
    (3, 1, QWEN), (9, 1, QWEN), (4, 6, QWEN),  # the split kernel (fewer)
    (4, 16, GQA4), (3, 2, GQA4),               # a key head shared by two pairs, both kernels
])
def test_commit_verify_equals_commit_then_verify(R, B1, shape, mode):
    c, w2, d2, sid2, src, dropped = _two_steps(R, B1=B1, seed=900 + 10 * R + B1, shape=shape, mode=mode)
    ref, fused = _run_both(c, w2, d2, sid2, src, dropped)
    assert ref[4] == 0 and fused[4] == 0
    for name, a, b in zip(("state", "history", "outputs", "stash"), ref[:4], fused[:4]):
        assert _bits_equal(a, b), name


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
def test_commit_verify_at_the_saturated_batch(mode):
    """64 requests x 9 rows, every request continued in place (the serving
    loop's usual case and the benchmark's launch), bit for bit."""
    w = wl.WORKLOADS["saturated-b64"]
    c = gh.make_case(w, mode=mode)
    d2 = wl.draw_layer(w, 1)
    ident = np.arange(w.batch, dtype=np.int32)
    ref, fused = _run_both(c, w, d2, c.slot_ids_np, ident, np.zeros(0, np.int64))
    assert ref[4] == 0 and fused[4] == 0
    for name, a, b in zip(("state", "history", "outputs", "stash"), ref[:4], fused[:4]):
        assert _bits_equal(a, b), name


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
@pytest.mark.parametrize("B1", [16, 3])
def test_commit_verify_matches_the_oracle(B1, mode):
    """The oracle's commit of step 1 then its verify of step 2, on the whole
    pool: outputs to the bf16 tolerance, states to the fp32 one, conv
    histories bit for bit (both kernels, both modes)."""
    R = 4
    c, w2, d2, sid2, src, dropped = _two_steps(R, B1=B1, seed=950 + B1, mode=mode)
    s = c.w.shape
    host_ssm = c.ssm.cpu().numpy().copy()
    host_conv = gh.to_storage_numpy(c.conv, s.dtype).copy()
    _, fused = _run_both(c, w2, d2, sid2, src, dropped)
    assert fused[4] == 0
    orc = oracle.Oracle()
    d1 = c.draw
    assert orc.commit(s, host_ssm, host_conv, d1["conv_w"], d1["x"], d1["alpha"], d1["beta"], c.slot_ids_np,
                      c.accept_np, R, nthreads=16) == 0
    o_ref, _, err = orc.verify(s, host_ssm, host_conv, d1["conv_w"], d2["x"], d2["alpha"], d2["beta"], sid2, R,
                               nthreads=16)
    assert err == 0
    atol, rtol = gh.tolerances(s)
    np.testing.assert_allclose(gh.tensor_f64(fused[2], s.dtype), o_ref, atol=atol, rtol=rtol)
    touched = np.unique(np.concatenate([c.slot_ids_np, sid2[sid2 >= 0]]))
    satol, srtol = gh.state_tolerances(s)
    np.testing.assert_allclose(fused[0].cpu().numpy()[touched], host_ssm[touched], atol=satol, rtol=srtol)
    conv_gpu = gh.to_storage_numpy(fused[1], s.dtype)
    assert np.array_equal(conv_gpu[touched], host_conv[touched])


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
@pytest.mark.parametrize("B1", [16, 8])
def test_commit_verify_errors_skip_the_request(B1, mode):
    """A source row outside the previous batch or naming another slot (bit 2),
    an accept length outside [0, rows] (bit 1) and a slot outside the pool
    (bit 0): each such request gets zero outputs and its slot keeps its state;
    the others are committed and verified as usual (both kernels)."""
    R = 4
    c, w2, d2, sid2, src, dropped = _two_steps(R, B1=B1, seed=970 + B1, accept_edges=False, mode=mode)
    gh.verify(c)
    torch.cuda.synchronize()
    live = np.flatnonzero((sid2 >= 0) & (src >= 0))
    b_far, b_other, b_acc, b_slot = live[:4]
    src = src.copy()
    sid2 = sid2.copy()
    src[b_far] = c.w.batch + 3                                   # outside the previous batch
    src[b_other] = src[live[4]]                                  # names another request's row
    acc = c.accept_np.copy()
    acc[src[b_acc]] = R + 1                                      # accept length out of range
    c.accept.copy_(torch.from_numpy(acc))
    bad_slot_owner = sid2[b_slot]
    sid2[b_slot] = c.w.num_slots + 5                             # slot outside the pool
    ins, out, sid2_t = _step2(c, w2, d2, sid2)
    before_ssm, before_conv = c.ssm.clone(), c.conv.clone()
    sb = _zero_scratch(c.desc, w2.batch, R, mode)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    bd.gdn_spec_commit_verify(c.desc, c.ssm, c.conv, c.conv_w, ins["x"], ins["alpha"], ins["beta"], sid2_t, R, sb,
                              torch.from_numpy(src).to(DEV), c.scratch, c.slot_ids, c.accept, out, err, mode=mode)
    torch.cuda.synchronize()
    assert int(err.item()) == 7
    for b in (b_far, b_other, b_acc, b_slot):
        assert bool((out[b].float() == 0).all()), b
    for b in (b_far, b_other, b_acc):
        s_ = int(sid2[b])
        assert _bits_equal(c.ssm[s_], before_ssm[s_]) and _bits_equal(c.conv[s_], before_conv[s_]), b
    s_ = int(bad_slot_owner)                                     # its request never reached the pool
    assert _bits_equal(c.ssm[s_], before_ssm[s_])
    ok = np.setdiff1d(live, [b_far, b_other, b_acc, b_slot])
    changed = [int(sid2[b]) for b in ok if c.accept_np[src[b]] > 0]
    assert changed and all(not _bits_equal(c.ssm[s_], before_ssm[s_]) for s_ in changed)


def test_commit_verify_replays_from_a_graph():
    """Two consecutive commit-verify steps (the scratch buffers trading
    places) captured in one HIP graph replay to the bits of the eager
    launches, three times, with eager work between the replays (FreeToken PR
    #844, Tests: a captured verify replays bitwise; the call only enqueues
    kernels on the caller's stream)."""
    w = wl.small_workload(QWEN, batch=16, rows=4, num_slots=40, seed=990)
    c = gh.make_case(w)
    s = c.w.shape
    d2, d3 = wl.draw_layer(w, 1), wl.draw_layer(w, 2)
    ins2 = [gh.storage_tensor(d2[k], s.dtype) for k in ("x", "alpha", "beta")]
    ins3 = [gh.storage_tensor(d3[k], s.dtype) for k in ("x", "alpha", "beta")]
    gh.verify(c)                                       # step 1: scratch A holds its stash
    torch.cuda.synchronize()
    sa_, sb_ = c.scratch.clone(), _zero_scratch(c.desc, w.batch, w.rows)
    ident = torch.arange(w.batch, dtype=torch.int32, device=DEV)
    out = torch.empty_like(c.out)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    steps = [bd.PreparedCommitVerify(c.desc, c.ssm, c.conv, c.conv_w, *ins2, c.slot_ids, w.rows, sb_, ident, sa_,
                                     c.slot_ids, c.accept, out, err),
             bd.PreparedCommitVerify(c.desc, c.ssm, c.conv, c.conv_w, *ins3, c.slot_ids, w.rows, sa_, ident, sb_,
                                     c.slot_ids, c.accept, out, err)]
    ssm0, conv0, a0 = c.ssm.clone(), c.conv.clone(), sa_.clone()

    def restore():
        c.ssm.copy_(ssm0)
        c.conv.copy_(conv0)
        sa_.copy_(a0)
        sb_.zero_()
        out.fill_(float("nan"))
        err.zero_()

    restore()
    for st in steps:
        st()
    torch.cuda.synchronize()
    want = (c.ssm.clone(), c.conv.clone(), out.clone(), sa_.clone())
    assert int(err.item()) == 0

    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for st in steps:
            st.args = st.args[:-1] + (torch.cuda.current_stream().cuda_stream,)
            st()
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device=DEV)
    for rep in range(3):
        restore()
        junk.mul_(1.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (c.ssm, c.conv, out, sa_)
        for name, a, b in zip(("state", "history", "outputs", "stash"), want, got):
            assert _bits_equal(a, b), (rep, name)
        assert int(err.item()) == 0


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
@pytest.mark.parametrize("B", [16, 3])
def test_commit_verify_chains_over_steps(B, mode):
    """Four steps: a plain verify, then three commit-verify launches, each
    committing the step before it (so a fused launch commits from a fused
    launch's scratch, including the history it kept), then a plain commit of
    the last. The pool and every step's outputs equal those of verify then
    commit at every step, bit for bit, and the oracle's sequence of commits
    and verifies within tolerance."""
    R = 4
    w = wl.small_workload(QWEN, batch=B, rows=R, num_slots=2 * B + 1, seed=1200 + B)
    c = gh.make_case(w, mode=mode)
    s = c.w.shape
    rng = np.random.default_rng(1300 + B)
    draws = [c.draw] + [wl.draw_layer(w, k) for k in (1, 2, 3)]
    accepts = [rng.integers(0, R + 1, B).astype(np.int32) for _ in range(4)]
    host_ssm = c.ssm.cpu().numpy().copy()
    host_conv = gh.to_storage_numpy(c.conv, s.dtype).copy()
    ssm0, conv0 = c.ssm.clone(), c.conv.clone()
    ident = torch.arange(B, dtype=torch.int32, device=DEV)

    def inputs(d):
        return [gh.storage_tensor(d[k], s.dtype) for k in ("x", "alpha", "beta")]

    # serial: verify, commit at every step
    outs_serial = []
    sc = _zero_scratch(c.desc, B, R, mode)
    for d, acc in zip(draws, accepts):
        out = torch.empty_like(c.out)
        bd.gdn_spec_verify(c.desc, c.ssm, c.conv, c.conv_w, *inputs(d), c.slot_ids, R, mode, sc, out, c.err)
        bd.gdn_spec_commit(c.desc, c.ssm, c.conv, c.slot_ids, torch.from_numpy(acc).to(DEV), R, mode, sc, c.err)
        outs_serial.append(out)
    torch.cuda.synchronize()
    assert int(c.err.item()) == 0
    want_ssm, want_conv = c.ssm.clone(), c.conv.clone()

    # fused: a plain verify, three commit-verify launches, a plain commit
    c.ssm.copy_(ssm0)
    c.conv.copy_(conv0)
    bufs = [_zero_scratch(c.desc, B, R, mode), _zero_scratch(c.desc, B, R, mode)]
    accs = [torch.from_numpy(a).to(DEV) for a in accepts]
    outs = []
    out = torch.empty_like(c.out)
    bd.gdn_spec_verify(c.desc, c.ssm, c.conv, c.conv_w, *inputs(draws[0]), c.slot_ids, R, mode, bufs[0], out, c.err)
    outs.append(out)
    for k in (1, 2, 3):
        out = torch.empty_like(c.out)
        print("chain %s B=%d step %d" % (mode, B, k), flush=True)
        bd.gdn_spec_commit_verify(c.desc, c.ssm, c.conv, c.conv_w, *inputs(draws[k]), c.slot_ids, R, bufs[k % 2],
                                  ident, bufs[(k - 1) % 2], c.slot_ids, accs[k - 1], out, c.err, mode=mode)
        outs.append(out)
    bd.gdn_spec_commit(c.desc, c.ssm, c.conv, c.slot_ids, accs[3], R, mode, bufs[1], c.err)
    torch.cuda.synchronize()
    assert int(c.err.item()) == 0
    for k in range(4):
        assert _bits_equal(outs[k], outs_serial[k]), k
    assert _bits_equal(c.ssm, want_ssm) and _bits_equal(c.conv, want_conv)

    # the oracle's steps
    orc = oracle.Oracle()
    atol, rtol = gh.tolerances(s)
    for k, (d, acc) in enumerate(zip(draws, accepts)):
        o_ref, _, e = orc.verify(s, host_ssm, host_conv, draws[0]["conv_w"], d["x"],
                                 d["alpha"], d["beta"], c.slot_ids_np, R, nthreads=16)
        assert e == 0
        np.testing.assert_allclose(gh.tensor_f64(outs[k], s.dtype), o_ref, atol=atol, rtol=rtol)
        assert orc.commit(s, host_ssm, host_conv, draws[0]["conv_w"], d["x"], d["alpha"], d["beta"], c.slot_ids_np,
                          acc, R, nthreads=16) == 0
    sl = c.slot_ids_np
    satol, srtol = gh.state_tolerances(s)
    np.testing.assert_allclose(c.ssm.cpu().numpy()[sl], host_ssm[sl], atol=satol, rtol=srtol)
    assert np.array_equal(gh.to_storage_numpy(c.conv, s.dtype)[sl], host_conv[sl])
