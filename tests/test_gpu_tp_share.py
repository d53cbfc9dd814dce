"""One rank's share of the layer under tensor parallelism over value heads
(TP4: 4 key / 8 value heads, 2,048 conv channels, as the pages' TP4 runs
shard the model; FreeToken PR #844, End-to-end): the path runs unchanged on
the shard, so the share is checked as any layer is, every request against
the oracle, and the commit-verify bit for bit against commit then verify."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import gpu_harness as gh  # noqa: E402
import oracle  # noqa: E402
import parity as par  # noqa: E402
from linear_attention_verify_amd import binding as bd  # noqa: E402
from linear_attention_verify_amd import workloads as wl  # noqa: E402

DEV = "cuda"


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
@pytest.mark.parametrize("name", wl.TP_SHARES)
def test_tp_share_parity(orc, name, mode):
    w = wl.WORKLOADS[name]
    print("tp share parity %s %s B=%d" % (name, mode, w.batch), flush=True)
    c = gh.make_case(w, mode=mode)
    par.check_layer(orc, c)
    par.check_untouched(c)


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
@pytest.mark.parametrize("name", wl.TP_SHARES)
def test_tp_share_commit_verify(name, mode):
    w = wl.WORKLOADS[name]
    c = gh.make_case(w, mode=mode)
    s = w.shape
    gh.verify(c)
    torch.cuda.synchronize()
    ssm0, conv0 = c.ssm.clone(), c.conv.clone()
    d2 = wl.draw_layer(w, 1)
    ins = [gh.storage_tensor(d2[k], s.dtype) for k in ("x", "alpha", "beta")]
    ident = torch.arange(w.batch, dtype=torch.int32, device=DEV)
    nbytes = bd.gdn_spec_scratch_bytes(c.desc, w.batch, w.rows, mode)
    print("tp share commit-verify %s %s" % (name, mode), flush=True)
    # commit then verify
    gh.commit(c)
    sa = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    out_a = torch.empty_like(c.out)
    bd.gdn_spec_verify(c.desc, c.ssm, c.conv, c.conv_w, *ins, c.slot_ids, w.rows, mode, sa, out_a, c.err)
    torch.cuda.synchronize()
    ref = (c.ssm.clone(), c.conv.clone(), out_a, sa)
    # one launch
    c.ssm.copy_(ssm0)
    c.conv.copy_(conv0)
    sb = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    out_b = torch.empty_like(c.out)
    bd.gdn_spec_commit_verify(c.desc, c.ssm, c.conv, c.conv_w, *ins, c.slot_ids, w.rows, sb, ident, c.scratch,
                              c.slot_ids, c.accept, out_b, c.err, mode=mode)
    torch.cuda.synchronize()
    assert int(c.err.item()) == 0
    for label, a, b in zip(("state", "history", "outputs", "stash"), ref, (c.ssm, c.conv, out_b, sb)):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), label
