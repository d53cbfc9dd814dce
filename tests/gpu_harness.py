"""Device-side set-up shared by the GPU tests, smoke() and the benchmark.

Draws a workload with the shared seeded generator, places it in device memory
(pools full of NaN sentinels with the drawn states at the requests' slots) and
calls the C ABI through the binding. Holds no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from linear_attention_verify_amd import binding as bd
from linear_attention_verify_amd import workloads as wl

DEV = "cuda"


def storage_tensor(a: np.ndarray, dtype: str, device=DEV) -> torch.Tensor:
    """numpy storage array (fp32, or bf16 bits as uint16) -> device tensor."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_storage_numpy(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if dtype == "f32":
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def tensor_f64(t: torch.Tensor, dtype: str) -> np.ndarray:
    return wl.storage_to_f32(to_storage_numpy(t, dtype), dtype).astype(np.float64)


@dataclass
class LayerCase:
    w: wl.Workload
    layer: int
    draw: dict
    slot_ids_np: np.ndarray
    accept_np: np.ndarray
    ssm: torch.Tensor
    conv: torch.Tensor
    conv_w: torch.Tensor
    x: torch.Tensor
    alpha: torch.Tensor
    beta: torch.Tensor
    slot_ids: torch.Tensor
    accept: torch.Tensor
    out: torch.Tensor
    err: torch.Tensor
    scratch: torch.Tensor
    desc: bd.GdnLayerDesc
    mode: str


def device_pools(w: wl.Workload, draw: dict, slot_ids: np.ndarray, device=DEV):
    """Pools on the device: sentinels, then the drawn states at the active slots."""
    s = w.shape
    ssm = torch.full((w.num_slots, s.num_v_heads, s.d_k, s.d_v), 0, dtype=torch.int32, device=device)
    ssm.fill_(int(np.int32(wl.F32_SENTINEL.view(np.int32))))
    ssm = ssm.view(torch.float32)
    conv_shape = (w.num_slots, s.conv_width - 1, s.conv_channels)
    if s.dtype == "f32":
        conv = torch.empty(conv_shape, dtype=torch.int32, device=device)
        conv.fill_(int(np.int32(wl.F32_SENTINEL.view(np.int32))))
        conv = conv.view(torch.float32)
    else:
        conv = torch.empty(conv_shape, dtype=torch.int16, device=device)
        conv.fill_(int(np.int16(wl.BF16_SENTINEL.view(np.int16))))
        conv = conv.view(torch.bfloat16)
    # only slots inside the pool get a state; an out-of-range id (the tests of
    # the error flag use one) must never reach a device-side index
    valid = (slot_ids >= 0) & (slot_ids < w.num_slots)
    if valid.any():
        idx = torch.from_numpy(slot_ids[valid].astype(np.int64)).to(device)
        ssm[idx] = torch.from_numpy(np.ascontiguousarray(draw["ssm_active"][valid])).to(device)
        conv[idx] = storage_tensor(draw["conv_active"][valid], s.dtype, device)
    return ssm, conv


def make_case(w: wl.Workload, layer: int = 0, mode: str = "replay", slot_ids=None, accept=None,
              draw=None, device=DEV) -> LayerCase:
    s = w.shape
    sid, acc = wl.draw_requests(w)
    sid = sid if slot_ids is None else np.asarray(slot_ids, np.int32)
    acc = acc if accept is None else np.asarray(accept, np.int32)
    d = wl.draw_layer(w, layer) if draw is None else draw
    ssm, conv = device_pools(w, d, sid, device)
    desc = bd.layer_desc(s)
    nbytes = bd.gdn_spec_scratch_bytes(desc, w.batch, w.rows, mode)
    odt = torch.float32 if s.dtype == "f32" else torch.bfloat16
    return LayerCase(
        w=w, layer=layer, draw=d, slot_ids_np=sid, accept_np=acc, ssm=ssm, conv=conv,
        conv_w=storage_tensor(d["conv_w"], s.dtype, device),
        x=storage_tensor(d["x"], s.dtype, device),
        alpha=storage_tensor(d["alpha"], s.dtype, device),
        beta=storage_tensor(d["beta"], s.dtype, device),
        slot_ids=torch.from_numpy(sid).to(device),
        accept=torch.from_numpy(acc).to(device),
        out=torch.full((w.batch, w.rows, s.num_v_heads, s.d_v), float("nan"), dtype=odt,
                       device=device),
        err=torch.zeros(1, dtype=torch.int32, device=device),
        scratch=torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device),
        desc=desc, mode=mode)


def verify(c: LayerCase, stream=None):
    bd.gdn_spec_verify(c.desc, c.ssm, c.conv, c.conv_w, c.x, c.alpha, c.beta, c.slot_ids,
                       c.w.rows, c.mode, c.scratch, c.out, c.err, stream)


def commit(c: LayerCase, stream=None):
    bd.gdn_spec_commit(c.desc, c.ssm, c.conv, c.slot_ids, c.accept, c.w.rows, c.mode, c.scratch,
                       c.err, stream)


def host_pools_for(c: LayerCase, requests):
    """Host pools holding only the given requests' committed states (slots 0..k-1),
    for running the oracle on a sample; returns (ssm, conv, slot_ids)."""
    w, d = c.w, c.draw
    reqs = np.asarray(requests)
    sub = wl.Workload(name=w.name, shape=w.shape, batch=len(reqs), rows=w.rows,
                      num_slots=max(len(reqs), 1))
    # padding requests stay padding for the oracle
    sid = np.where(c.slot_ids_np[reqs] >= 0, np.arange(len(reqs)), -1).astype(np.int32)
    sub_draw = {"ssm_active": d["ssm_active"][reqs], "conv_active": d["conv_active"][reqs]}
    ssm, conv = wl.build_pools(sub, sub_draw, sid)
    return ssm, conv, sid


def tolerances(shape):
    """atol, rtol: fp32 inputs 1e-5 / 1e-4; bf16 inputs 2e-3 / 1e-2."""
    return (1e-5, 1e-4) if shape.dtype == "f32" else (2e-3, 1e-2)


def state_tolerances(shape):
    """The state stays fp32 in both dtypes; only the GPU's fp32 arithmetic
    separates it from the oracle, so it is held to the fp32 bar."""
    return 1e-5, 1e-4


def make_device_case(w: wl.Workload, layer: int, slot_ids, accept, mode: str = "replay",
                     device=DEV) -> LayerCase:
    """A layer drawn on the device with a seeded torch generator (same
    distributions as the host draw). For layers that fill out a launch
    configuration but are not compared with the oracle; ``draw`` is None."""
    s = w.shape
    gen = torch.Generator(device=device)
    gen.manual_seed(1_000_003 * (w.seed + 1) + layer)
    B, R, C, W, HV = w.batch, w.rows, s.conv_channels, s.conv_width, s.num_v_heads
    sdt = torch.float32 if s.dtype == "f32" else torch.bfloat16
    f32 = dict(dtype=torch.float32, device=device, generator=gen)
    sid = np.asarray(slot_ids, np.int32)
    acc = np.asarray(accept, np.int32)
    ssm, conv = device_pools(w, {"ssm_active": np.zeros((0,), np.float32),
                                 "conv_active": np.zeros((0,), np.float32)}, sid[:0], device)
    sel = (sid >= 0) & (sid < w.num_slots)
    idx = torch.from_numpy(sid[sel].astype(np.int64)).to(device)
    n = int(idx.numel())
    ssm[idx] = torch.randn((n, HV, s.d_k, s.d_v), **f32)
    conv[idx] = torch.randn((n, W - 1, C), **f32).to(sdt)
    desc = bd.layer_desc(s)
    nbytes = bd.gdn_spec_scratch_bytes(desc, B, R, mode)
    return LayerCase(
        w=w, layer=layer, draw=None, slot_ids_np=sid, accept_np=acc, ssm=ssm, conv=conv,
        conv_w=(torch.randn((C, W), **f32) / float(np.sqrt(W))).to(sdt),
        x=torch.randn((B, R, C), **f32).to(sdt),
        alpha=(0.9 + 0.1 * torch.rand((B, R, HV), **f32)).to(sdt),
        beta=torch.rand((B, R, HV), **f32).to(sdt),
        slot_ids=torch.from_numpy(sid).to(device),
        accept=torch.from_numpy(acc).to(device),
        out=torch.full((B, R, HV, s.d_v), float("nan"), dtype=sdt, device=device),
        err=torch.zeros(1, dtype=torch.int32, device=device),
        scratch=torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device),
        desc=desc, mode=mode)
