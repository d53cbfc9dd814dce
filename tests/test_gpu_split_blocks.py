"""The small-batch verify splits each (request, value-head pair) over 16, 8
or 4 workgroups (blocks of 16, 32 or 64 state rows) by batch size. Every
result element takes the same operations in the same order whatever the
block, so a request's outputs and the state its commit leaves are the same
bits at batch 1, 2 and 3 (one block size each at 32 value heads), in both
commit modes, and match the oracle."""
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


def _bits(t):
    return t.contiguous().view(torch.uint8)


@pytest.mark.parametrize("mode", ["replay", "snapshot"])
@pytest.mark.parametrize("R", [3, 9])
def test_request_bits_do_not_depend_on_the_block_size(mode, R):
    w = wl.small_workload(QWEN, batch=3, rows=R, num_slots=7, seed=1400 + R)
    sid = np.array([5, 1, 3], np.int32)
    acc = np.array([2, R, 1], np.int32)
    c = gh.make_case(w, slot_ids=sid, accept=acc, mode=mode)
    ssm0, conv0 = c.ssm.clone(), c.conv.clone()
    results = {}
    for B in (1, 2, 3):   # 16, 32, 48 units: 16-, 32- and 64-row blocks
        c.ssm.copy_(ssm0)
        c.conv.copy_(conv0)
        c.err.zero_()
        out = torch.full((B, R, QWEN.num_v_heads, QWEN.d_v), float("nan"), dtype=torch.bfloat16, device=DEV)
        scratch = torch.zeros(bd.gdn_spec_scratch_bytes(c.desc, B, R, mode), dtype=torch.uint8, device=DEV)
        print("split blocks %s R=%d B=%d" % (mode, R, B), flush=True)
        bd.gdn_spec_verify(c.desc, c.ssm, c.conv, c.conv_w, c.x[:B], c.alpha[:B], c.beta[:B], c.slot_ids[:B], R,
                           mode, scratch, out, c.err)
        bd.gdn_spec_commit(c.desc, c.ssm, c.conv, c.slot_ids[:B], c.accept[:B], R, mode, scratch, c.err)
        torch.cuda.synchronize()
        assert int(c.err.item()) == 0
        results[B] = (out[0].clone(), c.ssm[sid[0]].clone(), c.conv[sid[0]].clone())
    for B in (2, 3):
        for a, b in zip(results[1], results[B]):
            assert torch.equal(_bits(a), _bits(b)), B

    # and request 0 against the oracle (verify outputs, committed state and history)
    s = w.shape
    host_ssm = ssm0.cpu().numpy().copy()
    host_conv = gh.to_storage_numpy(conv0, s.dtype).copy()
    d = c.draw
    orc = oracle.Oracle()
    o_ref, _, e = orc.verify(s, host_ssm, host_conv, d["conv_w"], d["x"][:1], d["alpha"][:1], d["beta"][:1],
                             sid[:1], R, nthreads=16)
    assert e == 0
    atol, rtol = gh.tolerances(s)
    np.testing.assert_allclose(gh.tensor_f64(results[1][0][None], s.dtype), o_ref, atol=atol, rtol=rtol)
    assert orc.commit(s, host_ssm, host_conv, d["conv_w"], d["x"][:1], d["alpha"][:1], d["beta"][:1], sid[:1],
                      acc[:1], R, nthreads=16) == 0
    satol, srtol = gh.state_tolerances(s)
    np.testing.assert_allclose(results[1][1].cpu().numpy(), host_ssm[sid[0]], atol=satol, rtol=srtol)
    assert np.array_equal(gh.to_storage_numpy(results[1][2][None], s.dtype)[0], host_conv[sid[0]])
