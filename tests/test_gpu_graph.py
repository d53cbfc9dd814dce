"""Verify + commit captured in a HIP graph.

Both calls only enqueue kernels on the caller's stream: no allocation, no
synchronisation, no device-memory read on the host (LightLLM PR #1330,
Summary: the verify dispatch is capture-safe, no device-to-host syncs). A
captured verify + commit therefore replays to the bits of the eager launches
(FreeToken PR #844, Tests: a captured verify replay equals the eager verify
bitwise). A graph captured for a fixed batch serves fewer live requests when
the rest of the slot table is padding (-1), as a serving engine pads batches
to its captured sizes (LightLLM PR #1330, Summary: padding of the captured
decode batch).

Every replay is checked against the eager result, with eager work and
synchronisation between the replays, and against the CPU oracle.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import gpu_harness as gh  # noqa: E402
import oracle  # noqa: E402
import parity as par  # noqa: E402
from linear_attention_verify_amd import workloads as wl  # noqa: E402


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


def _restore(c, ssm0, conv0):
    c.ssm.copy_(ssm0)
    c.conv.copy_(conv0)
    c.out.fill_(float("nan"))
    c.err.zero_()


def _eager(c, ssm0, conv0):
    _restore(c, ssm0, conv0)
    gh.verify(c)
    gh.commit(c)
    torch.cuda.synchronize()
    return c.out.clone(), c.ssm.clone(), c.conv.clone()


def _capture(c):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gh.verify(c)   # the binding launches on torch's current stream: the capture stream
        gh.commit(c)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
@pytest.mark.parametrize("name", ["tiny-fp32", "low-concurrency"])
def test_graph_replays_match_eager_bitwise(orc, name, mode):
    w = wl.WORKLOADS[name]
    print("graph %s %s" % (name, mode), flush=True)
    c = gh.make_case(w, mode=mode)
    ref = par.oracle_step(orc, c)
    ssm0, conv0 = c.ssm.clone(), c.conv.clone()
    out_e, ssm_e, conv_e = _eager(c, ssm0, conv0)
    assert int(c.err.item()) == 0

    _restore(c, ssm0, conv0)
    g = _capture(c)
    scratch_junk = torch.randn(1 << 20, device=c.ssm.device)
    for rep in range(3):
        _restore(c, ssm0, conv0)
        scratch_junk.mul_(1.5)          # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(c.err.item()) == 0, rep
        assert torch.equal(_bits(c.out), _bits(out_e)), rep
        assert torch.equal(_bits(c.ssm), _bits(ssm_e)), rep
        assert torch.equal(_bits(c.conv), _bits(conv_e)), rep
        par.assert_matches(c, ref)
        par.check_untouched(c)


def test_padded_graph_batch_matches_live_requests(orc):
    """Capture at batch 8; run 5 live requests with the last 3 slots -1. The
    live requests' outputs and committed states equal an eager batch of the 5
    alone and the oracle's; padding rows come out zero and no other slot
    changes."""
    shape = wl.LayerShape(num_k_heads=2, num_v_heads=4, d_k=128, d_v=128, dtype="bf16")
    w8 = wl.small_workload(shape, batch=8, rows=4, num_slots=12, seed=401)
    sid8, acc8 = wl.draw_requests(w8)
    sid8[5:] = -1
    acc8[5:] = 0
    c8 = gh.make_case(w8, slot_ids=sid8, accept=acc8)
    ssm0, conv0 = c8.ssm.clone(), c8.conv.clone()

    w5 = wl.small_workload(shape, batch=5, rows=4, num_slots=12, seed=401)
    d5 = {k: (v if k == "conv_w" else np.ascontiguousarray(v[:5])) for k, v in c8.draw.items()}
    c5 = gh.make_case(w5, slot_ids=sid8[:5], accept=acc8[:5], draw=d5)
    out5, ssm5, conv5 = _eager(c5, c5.ssm.clone(), c5.conv.clone())

    ref = par.oracle_step(orc, c8, requests=np.arange(5))
    _restore(c8, ssm0, conv0)
    g = _capture(c8)
    for rep in range(2):
        _restore(c8, ssm0, conv0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(c8.err.item()) == 0
        assert torch.equal(_bits(c8.out[:5]), _bits(out5)), rep
        assert not bool(c8.out[5:].float().abs().sum()), rep
        assert torch.equal(_bits(c8.ssm), _bits(ssm5)), rep
        assert torch.equal(_bits(c8.conv), _bits(conv5)), rep
        par.assert_matches(c8, ref)
        par.check_untouched(c8)
