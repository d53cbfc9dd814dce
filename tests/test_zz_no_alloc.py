"""The allocation-free verification attention (gdn_spec_attn_verify_static)
against the call that takes a scratch buffer, through the C ABI: two calls in
a row on the library's device array, the second on a smaller batch, each
equal to gdn_spec_attn_verify on the same inputs (the same kernels, so bit for
bit, which is within the attention tolerance), error flags included."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from linear_attention_verify_amd import binding as bd  # noqa: E402
from linear_attention_verify_amd import workloads as wl  # noqa: E402

DEV = "cuda"


def _bits(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def _inputs(w):
    d = wl.draw_attention(w)
    return (bd.attn_desc(w.shape), _bits(d["q"]), _bits(d["k_cache"]), _bits(d["v_cache"]),
            torch.from_numpy(d["block_table"]).to(DEV), torch.from_numpy(d["seq_lens"]).to(DEV))


def _both(w):
    desc, q, kc, vc, bt, sl = _inputs(w)
    nbytes = bd.gdn_spec_attn_scratch_bytes(desc, w.batch, w.rows, bt.shape[1])
    assert nbytes <= bd.ATTN_STATIC_SCRATCH_BYTES
    scratch = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    out_ref = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    err_ref = torch.zeros(1, dtype=torch.int32, device=DEV)
    bd.gdn_spec_attn_verify(desc, q, kc, vc, bt, sl, scratch, out_ref, err_ref)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    bd.gdn_spec_attn_verify_static(desc, q, kc, vc, bt, sl, out, err)
    torch.cuda.synchronize()
    return out, err, out_ref, err_ref


def test_static_scratch_matches_the_scratch_call_twice():
    big = wl.ATTN_WORKLOADS["attn-b64"]
    small = wl.AttnWorkload("no-alloc-small", wl.AttnShape(8, 2, 128, 32), batch=5, rows=4, min_len=40,
                            max_len=700, seed=77, padding=(3,))
    for w in (big, small):
        print("static scratch: %s B=%d R=%d" % (w.name, w.batch, w.rows), flush=True)
        out, err, out_ref, err_ref = _both(w)
        assert int(err.item()) == int(err_ref.item()) == 0
        assert bool(torch.isfinite(out.float()).all())
        assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16))
        np.testing.assert_allclose(out.float().cpu().numpy(), out_ref.float().cpu().numpy(), atol=3e-3, rtol=1e-2)
