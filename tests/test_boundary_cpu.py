"""The C ABI on the host: the library loads, exports every declared symbol and
refuses bad arguments before anything reaches the GPU (FreeToken PR #844,
Summary: rejection at config time). No call here launches a kernel: every
argument set is one the library must reject, or has batch 0."""
import ctypes
import os
import re

import pytest

from linear_attention_verify_amd import binding as bd
from linear_attention_verify_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn_spec.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIBRARY):
        from linear_attention_verify_amd import build
        build.build()
    return bd.load_library()


def declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.dirname(HEADER))):
        if h.endswith(".h"):
            text = open(os.path.join(os.path.dirname(HEADER), h)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdn_\w+)\s*\(", text, re.M))
    return sorted(names)


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(bd.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError):
        bd.load_library(str(tmp_path / "absent.so"))


def _align(v):
    return (v + 255) // 256 * 256


@pytest.mark.parametrize("name", wl.WORKLOAD_ORDER)
@pytest.mark.parametrize("mode", ["replay", "snapshot"])
def test_scratch_bytes(lib, name, mode):
    w = wl.WORKLOADS[name]
    s = w.shape
    B, R, HK, HV, D, C = w.batch, w.rows, s.num_k_heads, s.num_v_heads, s.d_k, s.conv_channels
    # raw row inputs, e_t per value head, k_t per key head, a_t per value head, the history read
    want = (_align(B * R * C * s.elem_bytes) + _align(B * R * HV * D * 4) + _align(B * HK * R * D * 4)
            + _align(B * HV * R * 4) + _align(B * (s.conv_width - 1) * C * s.elem_bytes))
    if mode == "snapshot":
        want += _align(B * R * HV * D * D * 4)
    assert bd.gdn_spec_scratch_bytes(bd.layer_desc(s), B, R, mode) == want


def _status_verify(lib, desc, pool, batch=2, rows=3, mode=0, scratch=4096, nbytes=1 << 30,
                   ptr=4096, slot=4096, conv_w=None, x=None):
    return lib.gdn_spec_verify(ctypes.byref(desc) if desc is not None else None,
                               ctypes.byref(pool) if pool is not None else None,
                               ptr if conv_w is None else conv_w, ptr if x is None else x, ptr, ptr, slot,
                               batch, rows, mode, scratch, nbytes, ptr, None, None)


def _status_commit(lib, desc, pool, batch=2, rows=3, mode=0, scratch=4096, nbytes=1 << 30,
                   ptr=4096):
    return lib.gdn_spec_commit(ctypes.byref(desc) if desc is not None else None,
                               ctypes.byref(pool) if pool is not None else None,
                               ptr, ptr, batch, rows, mode, scratch, nbytes, None, None)


def good_desc(**kw):
    s = wl.LayerShape(num_k_heads=2, num_v_heads=4, d_k=32, d_v=32, dtype="f32")
    d = bd.layer_desc(s)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def good_pool():
    return bd.GdnPool(4096, 4096, 8)


@pytest.mark.parametrize("field,value,status", [
    ("num_k_heads", 0, bd.GDN_ERR_INVALID_ARG),
    ("num_v_heads", 3, bd.GDN_ERR_INVALID_ARG),      # not a multiple of HK = 2
    ("d_k", 96, bd.GDN_ERR_UNSUPPORTED),
    ("d_v", 64, bd.GDN_ERR_UNSUPPORTED),              # d_k != d_v
    ("conv_width", 3, bd.GDN_ERR_UNSUPPORTED),
    ("dtype", 7, bd.GDN_ERR_INVALID_ARG),
    ("act", 5, bd.GDN_ERR_INVALID_ARG),
])
def test_bad_descriptor_is_refused(lib, field, value, status):
    d = good_desc(**{field: value})
    assert _status_verify(lib, d, good_pool()) == status
    assert _status_commit(lib, d, good_pool()) == status
    out = ctypes.c_size_t(0)
    assert lib.gdn_spec_scratch_bytes(ctypes.byref(d), 2, 3, 0, ctypes.byref(out)) == status


def test_bad_arguments_are_refused(lib):
    d, p = good_desc(), good_pool()
    inv = bd.GDN_ERR_INVALID_ARG
    assert _status_verify(lib, None, p) == inv
    assert _status_verify(lib, d, None) == inv
    assert _status_verify(lib, d, bd.GdnPool(None, 4096, 8)) == inv
    assert _status_verify(lib, d, bd.GdnPool(4096, 4096, 0)) == inv
    assert _status_verify(lib, d, bd.GdnPool(4100, 4096, 8)) == inv      # ssm not 16-byte aligned
    assert _status_verify(lib, d, bd.GdnPool(4096, 4100, 8)) == inv      # conv not 16-byte aligned
    assert _status_commit(lib, d, bd.GdnPool(4096, 4104, 8)) == inv
    assert _status_verify(lib, d, p, rows=0) == inv
    assert _status_verify(lib, d, p, rows=10) == inv
    assert _status_verify(lib, d, p, batch=-1) == inv
    assert _status_verify(lib, d, p, mode=2) == inv
    assert _status_verify(lib, d, p, scratch=None) == inv
    assert _status_verify(lib, d, p, scratch=4104) == inv                # misaligned scratch
    assert _status_verify(lib, d, p, slot=None) == inv
    assert _status_verify(lib, d, p, ptr=None) == inv
    assert _status_verify(lib, d, p, x=4104) == inv                      # x not 16-byte aligned
    assert _status_verify(lib, d, p, conv_w=4100) == inv                 # conv_w not 16-byte aligned
    assert _status_commit(lib, d, p, ptr=None) == inv
    assert _status_commit(lib, d, p, rows=10) == inv


def _status_commit_layers(lib, desc, pools, scratch, layers, batch=2, rows=3, nbytes=1 << 30):
    import ctypes as ct
    P = (bd.GdnPool * max(len(pools), 1))(*pools) if pools is not None else None
    S = (ct.c_void_p * max(len(scratch), 1))(*scratch) if scratch is not None else None
    return lib.gdn_spec_commit_layers(ct.byref(desc), P, S, layers, 4096, 4096, batch, rows, 0, nbytes,
                                      None, None)


def test_commit_layers_arguments_are_refused(lib):
    d, p = good_desc(), good_pool()
    inv = bd.GDN_ERR_INVALID_ARG
    assert _status_commit_layers(lib, d, [p], [4096], 0) == inv            # no layers
    assert _status_commit_layers(lib, d, [p] * 65, [4096] * 65, 65) == inv  # above 64
    assert _status_commit_layers(lib, d, None, [4096], 1) == inv
    assert _status_commit_layers(lib, d, [p], None, 1) == inv
    assert _status_commit_layers(lib, d, [p, bd.GdnPool(4096, 4100, 8)], [4096, 4096], 2) == inv
    assert _status_commit_layers(lib, d, [p, p], [4096, 4104], 2) == inv    # misaligned scratch
    assert _status_commit_layers(lib, d, [p, p], [4096, None], 2) == inv
    need = bd.gdn_spec_scratch_bytes(d, 2, 3, "replay")
    assert _status_commit_layers(lib, d, [p, p], [4096, 4096], 2, nbytes=need - 1) == bd.GDN_ERR_SCRATCH_TOO_SMALL
    assert _status_commit_layers(lib, d, [p, p], [4096, 4096], 2, batch=0) == bd.GDN_OK


def test_commit_all_arguments_are_refused(lib):
    """gdn_spec_commit_all (GDN layers and window states in one launch) refuses
    counts out of range, missing or misaligned window pointers and entries
    that are not a positive multiple of 4 bytes, before any launch."""
    INV, UNS = bd.GDN_ERR_INVALID_ARG, bd.GDN_ERR_UNSUPPORTED
    fake = 0x100000   # never dereferenced: every call below is refused first

    def call(windows, nw, layers=0, batch=2, rows=3):
        arr = (bd.GdnSlotWindow * max(len(windows), 1))(*windows)
        return lib.gdn_spec_commit_all(None, None, None, layers, arr if windows else None, nw, fake, fake, batch,
                                       rows, 0, 0, None, None)

    good = bd.GdnSlotWindow(fake, fake, 4, 3, 16)
    assert call([], 0) == INV                                          # nothing to commit
    assert call([good] * 17, 17) == INV                                # more than 16 windows
    assert call([good], 1, layers=-1) == INV
    assert call([good], 1, layers=65) == INV
    assert call([good], 1, layers=1) == INV                            # layers without pools
    assert call([good], 1, rows=0) == INV
    assert call([good], 1, rows=10) == INV
    assert call([good], 1, batch=-1) == INV
    for bad in (bd.GdnSlotWindow(None, fake, 4, 3, 16), bd.GdnSlotWindow(fake, None, 4, 3, 16),
                bd.GdnSlotWindow(fake + 2, fake, 4, 3, 16), bd.GdnSlotWindow(fake, fake + 1, 4, 3, 16),
                bd.GdnSlotWindow(fake, fake, 0, 3, 16), bd.GdnSlotWindow(fake, fake, 4, 0, 16),
                bd.GdnSlotWindow(fake, fake, 4, 3, 6), bd.GdnSlotWindow(fake, fake, 4, 3, 0)):
        assert call([good, bad], 2) == INV
    assert call([bd.GdnSlotWindow(fake, fake, 4, 1 << 20, 1 << 12)], 1) == UNS   # words past an int32 index
    assert call([good], 1, batch=0) == bd.GDN_OK                       # empty batch: nothing launched


def test_accept_greedy_arguments_are_refused(lib):
    inv = bd.GDN_ERR_INVALID_ARG
    f = lib.gdn_spec_accept_greedy
    assert f(4096, 4096, None, 2, 0, 4096, None, None) == inv      # rows 0
    assert f(4096, 4096, None, 2, 10, 4096, None, None) == inv     # rows > 9
    assert f(4096, 4096, None, -1, 3, 4096, None, None) == inv     # negative batch
    assert f(None, 4096, None, 2, 3, 4096, None, None) == inv      # drafts needed when rows > 1
    assert f(4096, None, None, 2, 3, 4096, None, None) == inv
    assert f(4096, 4096, None, 2, 3, None, None, None) == inv
    assert f(None, None, None, 0, 3, None, None, None) == bd.GDN_OK  # empty batch launches nothing


def test_small_scratch_is_refused(lib):
    d, p = good_desc(), good_pool()
    need = bd.gdn_spec_scratch_bytes(d, 2, 3, "replay")
    assert _status_verify(lib, d, p, nbytes=need - 1) == bd.GDN_ERR_SCRATCH_TOO_SMALL
    assert _status_commit(lib, d, p, nbytes=need - 1) == bd.GDN_ERR_SCRATCH_TOO_SMALL
    snap = bd.gdn_spec_scratch_bytes(d, 2, 3, "snapshot")
    assert _status_verify(lib, d, p, mode=1, nbytes=snap - 1) == bd.GDN_ERR_SCRATCH_TOO_SMALL


def test_empty_batch_returns_before_launching(lib):
    d, p = good_desc(), good_pool()
    assert _status_verify(lib, d, p, batch=0, scratch=None, nbytes=0, ptr=None, slot=None) == bd.GDN_OK
    assert _status_commit(lib, d, p, batch=0, scratch=None, nbytes=0, ptr=None) == bd.GDN_OK


def test_strerror(lib):
    for st in range(5):
        assert bd.gdn_strerror(st)
    assert bd.gdn_strerror(99) == "unknown status"


def test_product_code_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "linear_attention_verify_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, re.M), f
                assert "gdn_oracle" not in text, f


def _attn_desc(**kw):
    d = bd.GdnAttnDesc(8, 2, 128, 32, 0.088)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("field,value,status", [
    ("num_q_heads", 0, bd.GDN_ERR_INVALID_ARG),
    ("num_q_heads", 7, bd.GDN_ERR_INVALID_ARG),       # not a multiple of the KV heads
    ("head_dim", 64, bd.GDN_ERR_UNSUPPORTED),
    ("page_size", 16, bd.GDN_ERR_UNSUPPORTED),        # not a multiple of 32
    ("num_kv_heads", 0, bd.GDN_ERR_INVALID_ARG),
    ("scale", 0.0, bd.GDN_ERR_INVALID_ARG),
    ("scale", -0.5, bd.GDN_ERR_INVALID_ARG),
    ("scale", float("inf"), bd.GDN_ERR_INVALID_ARG),
    ("scale", float("nan"), bd.GDN_ERR_INVALID_ARG),
])
def test_attention_descriptor_is_refused(lib, field, value, status):
    import ctypes as ct
    out = ct.c_size_t(0)
    assert lib.gdn_spec_attn_scratch_bytes(ct.byref(_attn_desc(**{field: value})), 2, 3, 4, ct.byref(out)) == status


def test_attention_arguments_are_refused(lib):
    import ctypes as ct
    d = _attn_desc()
    inv = bd.GDN_ERR_INVALID_ARG
    out = ct.c_size_t(0)
    assert lib.gdn_spec_attn_scratch_bytes(ct.byref(d), 2, 10, 4, ct.byref(out)) == inv       # rows > 9
    assert lib.gdn_spec_attn_scratch_bytes(ct.byref(_attn_desc(num_q_heads=64, num_kv_heads=1)), 2, 3, 4,
                                           ct.byref(out)) == bd.GDN_ERR_UNSUPPORTED           # 192 queries
    assert lib.gdn_spec_attn_scratch_bytes(ct.byref(_attn_desc(num_q_heads=2048, num_kv_heads=2048)), 2, 3, 4,
                                           ct.byref(out)) == bd.GDN_ERR_UNSUPPORTED           # past 1024 KV heads
    need = bd.gdn_spec_attn_scratch_bytes(d, 2, 3, 4)
    f = lambda **kw: lib.gdn_spec_attn_verify(
        ct.byref(d), kw.get("q", 4096), 4096, 4096, kw.get("pages", 8), 4096, kw.get("mb", 4), 4096,
        kw.get("batch", 2), 3, kw.get("scratch", 4096), kw.get("nbytes", need), kw.get("out", 4096), None, None)
    assert f(q=None) == inv
    assert f(q=4104) == inv                 # misaligned
    assert f(out=4104) == inv
    assert f(out=None) == inv
    assert f(pages=0) == inv
    assert f(mb=0) == inv
    assert f(scratch=None) == inv
    assert f(nbytes=need - 1) == bd.GDN_ERR_SCRATCH_TOO_SMALL
    assert f(batch=0, q=None, scratch=None) == bd.GDN_OK


def test_static_attention_refuses_before_launching(lib):
    """The allocation-free attention call checks its arguments, and that the
    batch fits its device array, before any HIP call: a batch whose records
    need more than the array returns GDN_ERR_SCRATCH_TOO_SMALL."""
    import ctypes as ct
    assert bd.ATTN_STATIC_SCRATCH_BYTES == 64 << 20
    d = _attn_desc(num_q_heads=1024, num_kv_heads=1024, head_dim=256)
    need = bd.gdn_spec_attn_scratch_bytes(d, 4, 3, 4)
    assert need > bd.ATTN_STATIC_SCRATCH_BYTES
    f = lambda desc, **kw: lib.gdn_spec_attn_verify_static(
        ct.byref(desc), kw.get("q", 4096), 4096, 4096, 8, 4096, 4, 4096, kw.get("batch", 4), kw.get("rows", 3),
        kw.get("out", 4096), None, None)
    assert f(d) == bd.GDN_ERR_SCRATCH_TOO_SMALL
    assert bd.gdn_spec_attn_scratch_bytes(d, 3, 3, 4) <= bd.ATTN_STATIC_SCRATCH_BYTES   # 3 requests fit
    small = _attn_desc()
    assert f(small, q=None) == bd.GDN_ERR_INVALID_ARG
    assert f(small, out=4104) == bd.GDN_ERR_INVALID_ARG
    assert f(small, rows=10) == bd.GDN_ERR_INVALID_ARG
    assert f(small, batch=0, q=None, out=None) == bd.GDN_OK


def test_sample_arguments_are_refused(lib):
    import ctypes as ct
    inv = bd.GDN_ERR_INVALID_ARG
    out = ct.c_size_t(0)
    assert lib.gdn_spec_sample_scratch_bytes(4, 10, 1000, ct.byref(out)) == inv     # rows > 9
    assert lib.gdn_spec_sample_scratch_bytes(4, 3, 0, ct.byref(out)) == inv         # empty vocabulary
    assert lib.gdn_spec_sample_scratch_bytes(-1, 3, 10, ct.byref(out)) == inv
    need = bd.gdn_spec_sample_scratch_bytes(4, 3, 1000)
    assert need > 0
    good = bd.GdnSampleInputs(4096, None, 4096, None, None, 4096, None, None, None)

    def f(inputs=good, dtype=bd.GDN_BF16, batch=4, rows=3, scratch=4096, nbytes=need, acc=4096, nxt=4096):
        return lib.gdn_spec_accept_sample(ct.byref(inputs) if inputs is not None else None, dtype, batch, rows, 1000,
                                          ct.c_uint64(1), scratch, nbytes, acc, nxt, None, None)
    assert f(inputs=None) == inv
    assert f(inputs=bd.GdnSampleInputs(None, None, 4096, None, None, 4096, None, None, None)) == inv   # no logits
    assert f(inputs=bd.GdnSampleInputs(4096, None, None, None, None, 4096, None, None, None)) == inv   # no drafts
    assert f(inputs=bd.GdnSampleInputs(4096, None, 4096, None, None, None, None, None, None)) == inv   # no temperature
    assert f(dtype=7) == inv
    assert f(acc=None) == inv
    assert f(scratch=4104) == inv                                        # misaligned
    assert f(nbytes=need - 1) == bd.GDN_ERR_SCRATCH_TOO_SMALL
    assert f(batch=0, inputs=None, scratch=None, acc=None, nxt=None) == bd.GDN_OK


def _status_commit_verify(lib, desc, pool, batch=2, rows=3, scratch=0x100000, prev=0x200000, prev_batch=2,
                          nbytes=1 << 16, pnbytes=1 << 16, src=4096, prev_slots=4096, prev_acc=4096, ptr=4096,
                          mode=0):
    return lib.gdn_spec_commit_verify(ctypes.byref(desc), ctypes.byref(pool), ptr, ptr, ptr, ptr, ptr, batch, rows,
                                      mode, scratch, nbytes, src, prev, pnbytes, prev_slots, prev_acc, prev_batch, ptr,
                                      None, None)


def test_commit_verify_arguments_are_refused(lib):
    """gdn_spec_commit_verify runs on the d = 128 bf16 kernels (an even number
    of value heads per key head), and refuses a missing
    source table or previous step, a negative previous batch and a scratch
    that overlaps the previous step's, before any launch."""
    INV, UNS = bd.GDN_ERR_INVALID_ARG, bd.GDN_ERR_UNSUPPORTED
    q = bd.layer_desc(wl.LayerShape(num_k_heads=2, num_v_heads=4, d_k=128, d_v=128, dtype="bf16"))
    p = good_pool()
    assert _status_commit_verify(lib, good_desc(), p) == UNS                        # fp32 storage
    d64 = bd.layer_desc(wl.LayerShape(num_k_heads=2, num_v_heads=4, d_k=64, d_v=64, dtype="bf16"))
    assert _status_commit_verify(lib, d64, p) == UNS                                # d = 64
    g1 = bd.layer_desc(wl.LayerShape(num_k_heads=2, num_v_heads=2, d_k=128, d_v=128, dtype="bf16"))
    assert _status_commit_verify(lib, g1, p) == UNS                                 # one value head per key head
    assert _status_commit_verify(lib, q, p, prev_batch=-1) == INV
    assert _status_commit_verify(lib, q, p, src=None) == INV
    assert _status_commit_verify(lib, q, p, prev=None) == INV
    assert _status_commit_verify(lib, q, p, prev=0x100008) == INV                    # misaligned previous scratch
    assert _status_commit_verify(lib, q, p, prev_slots=None) == INV
    assert _status_commit_verify(lib, q, p, prev_acc=None) == INV
    assert _status_commit_verify(lib, q, p, prev=0x100000 + 256) == INV              # overlaps this step's scratch
    assert _status_commit_verify(lib, q, p, nbytes=256) == bd.GDN_ERR_SCRATCH_TOO_SMALL
    assert _status_commit_verify(lib, q, p, pnbytes=256) == bd.GDN_ERR_SCRATCH_TOO_SMALL
    assert _status_commit_verify(lib, q, p, batch=0, prev=None, prev_slots=None, prev_acc=None, pnbytes=0,
                                 prev_batch=0) == bd.GDN_OK                       # no previous step needs no buffers
    assert _status_commit_verify(lib, q, p, rows=10) == INV
    assert _status_commit_verify(lib, q, p, mode=2) == INV
    assert _status_commit_verify(lib, q, p, mode=1) == bd.GDN_ERR_SCRATCH_TOO_SMALL   # snapshot scratch is larger
    assert _status_commit_verify(lib, q, p, batch=0) == bd.GDN_OK                    # nothing launched
