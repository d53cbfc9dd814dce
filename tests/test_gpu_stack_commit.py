"""One launch commits every layer of a stack: bit for bit the per-layer
commits and within tolerance of the oracle, in both modes, with padding and
per-layer pools of different sizes (FreeToken PR #844, Design: one upload of
the slot and count indices serves every state the commit restores)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import gpu_harness as gh  # noqa: E402
import oracle  # noqa: E402
import parity as par  # noqa: E402
from linear_attention_verify_amd import binding as bd  # noqa: E402
from linear_attention_verify_amd import workloads as wl  # noqa: E402


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (32, "f32")])
def test_stack_commit_matches_per_layer_commits(d, dtype, mode):
    orc = oracle.Oracle()
    shape = wl.LayerShape(num_k_heads=2, num_v_heads=4, d_k=d, d_v=d, dtype=dtype)
    L = 3
    base = wl.small_workload(shape, batch=6, rows=5, num_slots=9, seed=700)
    sid, acc = wl.draw_requests(base)
    sid[2] = -1
    acc[4] = 0
    print("stack commit d=%d %s %s" % (d, dtype, mode), flush=True)
    cases = []
    for layer in range(L):
        # layers keep their own pool sizes; the slot table fits the smallest
        w = wl.small_workload(shape, batch=6, rows=5, num_slots=9 + 3 * layer, seed=700)
        c = gh.make_case(w, layer=layer, mode=mode, slot_ids=sid, accept=acc)
        gh.verify(c)
        cases.append(c)
    torch.cuda.synchronize()
    before = [(c.ssm.clone(), c.conv.clone()) for c in cases]

    for c in cases:                       # per-layer commits
        gh.commit(c)
    torch.cuda.synchronize()
    want = [(c.ssm.clone(), c.conv.clone()) for c in cases]
    assert all(int(c.err.item()) == 0 for c in cases)

    for c, (s0, c0) in zip(cases, before):
        c.ssm.copy_(s0)
        c.conv.copy_(c0)
    err = torch.zeros(1, dtype=torch.int32, device=cases[0].ssm.device)
    bd.gdn_spec_commit_layers(cases[0].desc, [(c.ssm, c.conv, c.scratch) for c in cases], cases[0].slot_ids,
                              cases[0].accept, base.rows, mode, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for layer, (c, (ws, wc)) in enumerate(zip(cases, want)):
        assert torch.equal(_bits(c.ssm), _bits(ws)), layer
        assert torch.equal(_bits(c.conv), _bits(wc)), layer
        par.assert_matches(c, par.oracle_step(orc, c))
        par.check_untouched(c)


def test_stack_commit_flags_bad_lengths_once_per_call():
    shape = wl.LayerShape(num_k_heads=2, num_v_heads=4, d_k=64, d_v=64, dtype="bf16")
    w = wl.small_workload(shape, batch=3, rows=3, num_slots=5, seed=701)
    sid, acc = wl.draw_requests(w)
    acc[1] = 4                            # above rows: bit 1, that request untouched
    cases = [gh.make_case(w, layer=layer, slot_ids=sid, accept=acc) for layer in range(2)]
    for c in cases:
        gh.verify(c)
    torch.cuda.synchronize()
    before = [c.ssm[int(sid[1])].clone() for c in cases]
    err = torch.zeros(1, dtype=torch.int32, device=cases[0].ssm.device)
    bd.gdn_spec_commit_layers(cases[0].desc, [(c.ssm, c.conv, c.scratch) for c in cases], cases[0].slot_ids,
                              cases[0].accept, w.rows, "replay", err)
    torch.cuda.synchronize()
    assert int(err.item()) == 2
    for c, b0 in zip(cases, before):
        assert torch.equal(_bits(c.ssm[int(sid[1])]), _bits(b0))
