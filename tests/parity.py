"""Comparisons of device results with the CPU oracle, shared by the GPU tests.

Element by element on the same seeded inputs: o of every verify row (to the
tolerance of the storage type), the committed state of every request's slot
(fp32 tolerance) and the conv history (bitwise: it is a copy of raw inputs).
Untouched slots must keep their NaN sentinels bit for bit.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import gpu_harness as gh
from linear_attention_verify_amd import workloads as wl


@dataclass
class OracleResult:
    reqs: np.ndarray
    out: np.ndarray       # [len(reqs)][R][HV][d_v] fp64
    ssm: np.ndarray       # host pool after the commit, request i in slot i
    conv: np.ndarray
    sid: np.ndarray       # oracle slot of each sampled request (-1: padding)


def oracle_step(orc, c: gh.LayerCase, requests=None, accept=None, nthreads=16) -> OracleResult:
    """The oracle's verify + commit of `requests` (all by default), started
    from the committed state the case was drawn with."""
    w, s, d = c.w, c.w.shape, c.draw
    reqs = np.arange(w.batch) if requests is None else np.asarray(requests)
    acc = c.accept_np if accept is None else np.asarray(accept, np.int32)
    hs, hc, hsid = gh.host_pools_for(c, reqs)
    sub = lambda a: np.ascontiguousarray(a[reqs])
    o_ref, _, err = orc.verify(s, hs, hc, d["conv_w"], sub(d["x"]), sub(d["alpha"]), sub(d["beta"]),
                               hsid, w.rows, nthreads=nthreads)
    assert err == 0
    err = orc.commit(s, hs, hc, d["conv_w"], sub(d["x"]), sub(d["alpha"]), sub(d["beta"]), hsid,
                     np.ascontiguousarray(acc[reqs]), w.rows, nthreads=nthreads)
    assert err == 0
    return OracleResult(reqs, o_ref, hs, hc, hsid)


def assert_out_matches(c: gh.LayerCase, ref: OracleResult, out=None):
    s = c.w.shape
    atol, rtol = gh.tolerances(s)
    o_gpu = gh.tensor_f64(c.out if out is None else out, s.dtype)[ref.reqs]
    np.testing.assert_allclose(o_gpu, ref.out, atol=atol, rtol=rtol)


def assert_states_match(c: gh.LayerCase, ref: OracleResult, ssm=None, conv=None):
    """Committed state (tolerance) and conv history (bitwise) of the active requests."""
    s = c.w.shape
    ssm = c.ssm if ssm is None else ssm
    conv = c.conv if conv is None else conv
    act = ref.sid >= 0
    sl = c.slot_ids_np[ref.reqs][act].astype(np.int64)
    assert ((sl >= 0) & (sl < c.w.num_slots)).all(), "slot index outside the pool"
    slots = torch.from_numpy(sl).to(ssm.device)
    s_gpu = ssm[slots].cpu().numpy()
    satol, srtol = gh.state_tolerances(s)
    np.testing.assert_allclose(s_gpu, ref.ssm[ref.sid[act]], atol=satol, rtol=srtol)
    conv_gpu = gh.to_storage_numpy(conv[slots], s.dtype)
    assert np.array_equal(conv_gpu.view(np.uint8), ref.conv[ref.sid[act]].view(np.uint8)), "conv history differs"


def assert_matches(c: gh.LayerCase, ref: OracleResult):
    assert_out_matches(c, ref)
    assert_states_match(c, ref)


def check_untouched(c: gh.LayerCase, ssm=None, conv=None):
    """Every slot no request owns keeps its sentinel bits."""
    w, s = c.w, c.w.shape
    ssm = c.ssm if ssm is None else ssm
    conv = c.conv if conv is None else conv
    mask = torch.ones(w.num_slots, dtype=torch.bool, device=ssm.device)
    sid = c.slot_ids_np
    active = sid[(sid >= 0) & (sid < w.num_slots)].astype(np.int64)
    mask[torch.from_numpy(active).to(ssm.device)] = False
    rest = ssm[mask].view(torch.int32)
    assert bool((rest == int(np.int32(wl.F32_SENTINEL.view(np.int32)))).all())
    if s.dtype == "bf16":
        crest = conv[mask].view(torch.int16)
        assert bool((crest == int(np.int16(wl.BF16_SENTINEL.view(np.int16)))).all())
    else:
        crest = conv[mask].view(torch.int32)
        assert bool((crest == int(np.int32(wl.F32_SENTINEL.view(np.int32)))).all())


def check_layer(orc, c: gh.LayerCase, requests=None, nthreads=16) -> OracleResult:
    """Verify + commit on the device, the pool checked unchanged by the
    verify, then everything compared with the oracle on `requests`."""
    s = c.w.shape
    ssm_before = c.ssm.clone()
    conv_before = c.conv.clone()
    gh.verify(c)
    torch.cuda.synchronize()
    assert torch.equal(c.ssm.view(torch.int32), ssm_before.view(torch.int32)), "verify wrote the state"
    cv = torch.int16 if s.dtype == "bf16" else torch.int32
    assert torch.equal(c.conv.view(cv), conv_before.view(cv)), "verify wrote the conv history"
    gh.commit(c)
    torch.cuda.synchronize()
    assert int(c.err.item()) == 0
    ref = oracle_step(orc, c, requests, nthreads=nthreads)
    assert_matches(c, ref)
    return ref
