"""ctypes binding of libgdn_spec.so (the C ABI in include/gdn_spec.h).

Argument marshalling only: torch tensors (device memory) become raw pointers,
the current torch stream becomes the hipStream_t; every step of the path runs
in the HIP kernels. There is no fallback: if the library is not built, loading
it raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libgdn_spec.so")

GDN_OK = 0
GDN_ERR_INVALID_ARG = 1
GDN_ERR_UNSUPPORTED = 2
GDN_ERR_SCRATCH_TOO_SMALL = 3
GDN_ERR_HIP = 4

GDN_F32 = 0
GDN_BF16 = 1
GDN_COMMIT_REPLAY = 0
GDN_COMMIT_SNAPSHOT = 1
GDN_ACT_SILU = 0
GDN_ACT_NONE = 1

MODES = {"replay": GDN_COMMIT_REPLAY, "snapshot": GDN_COMMIT_SNAPSHOT}

EXPORTS = ("gdn_spec_scratch_bytes", "gdn_spec_verify", "gdn_spec_commit", "gdn_spec_commit_verify",
           "gdn_spec_commit_layers",
           "gdn_spec_commit_all", "gdn_spec_accept_greedy", "gdn_strerror", "gdn_spec_attn_scratch_bytes", "gdn_spec_attn_verify",
           "gdn_spec_attn_verify_static", "gdn_spec_sample_scratch_bytes", "gdn_spec_accept_sample")

# bytes of the device array behind gdn_spec_attn_verify_static (GDN_SPEC_ATTN_STATIC_SCRATCH_BYTES)
ATTN_STATIC_SCRATCH_BYTES = 64 << 20


class GdnLayerDesc(ctypes.Structure):
    _fields_ = [
        ("num_k_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("d_k", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("conv_width", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("act", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("l2_eps", ctypes.c_float),
    ]


class GdnPool(ctypes.Structure):
    _fields_ = [
        ("ssm", ctypes.c_void_p),
        ("conv", ctypes.c_void_p),
        ("num_slots", ctypes.c_int32),
    ]


class GdnSlotWindow(ctypes.Structure):
    _fields_ = [
        ("state", ctypes.c_void_p),
        ("rows", ctypes.c_void_p),
        ("num_slots", ctypes.c_int32),
        ("length", ctypes.c_int32),
        ("entry_bytes", ctypes.c_int32),
    ]


class GdnAttnDesc(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class GdnSampleInputs(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "logits", "draft_probs", "draft", "pending", "prior_counts", "temperature", "presence", "frequency",
        "slot_ids")]


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s (status %d)" % (where, gdn_strerror(status), status))
        self.status = status


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIBRARY
    if not os.path.exists(p):
        raise RuntimeError(
            "%s is not built; run `python -m linear_attention_verify_amd.build`" % p)
    lib = ctypes.CDLL(p)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    pdesc, ppool = ctypes.POINTER(GdnLayerDesc), ctypes.POINTER(GdnPool)
    lib.gdn_spec_scratch_bytes.restype = ctypes.c_int
    lib.gdn_spec_scratch_bytes.argtypes = [pdesc, i32, i32, ctypes.c_int, ctypes.POINTER(sz)]
    lib.gdn_spec_verify.restype = ctypes.c_int
    lib.gdn_spec_verify.argtypes = [pdesc, ppool, vp, vp, vp, vp, vp, i32, i32, ctypes.c_int,
                                    vp, sz, vp, vp, vp]
    lib.gdn_spec_commit.restype = ctypes.c_int
    lib.gdn_spec_commit.argtypes = [pdesc, ppool, vp, vp, i32, i32, ctypes.c_int, vp, sz, vp, vp]
    lib.gdn_spec_commit_verify.restype = ctypes.c_int
    lib.gdn_spec_commit_verify.argtypes = [pdesc, ppool, vp, vp, vp, vp, vp, i32, i32, ctypes.c_int, vp, sz, vp, vp,
                                           sz, vp, vp, i32, vp, vp, vp]
    lib.gdn_spec_commit_layers.restype = ctypes.c_int
    lib.gdn_spec_commit_layers.argtypes = [pdesc, ppool, ctypes.POINTER(vp), i32, vp, vp, i32, i32,
                                           ctypes.c_int, sz, vp, vp]
    lib.gdn_spec_commit_all.restype = ctypes.c_int
    lib.gdn_spec_commit_all.argtypes = [pdesc, ppool, ctypes.POINTER(vp), i32, ctypes.POINTER(GdnSlotWindow), i32,
                                        vp, vp, i32, i32, ctypes.c_int, sz, vp, vp]
    lib.gdn_spec_accept_greedy.restype = ctypes.c_int
    lib.gdn_spec_accept_greedy.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp]
    pattn = ctypes.POINTER(GdnAttnDesc)
    lib.gdn_spec_attn_scratch_bytes.restype = ctypes.c_int
    lib.gdn_spec_attn_scratch_bytes.argtypes = [pattn, i32, i32, i32, ctypes.POINTER(sz)]
    lib.gdn_spec_attn_verify.restype = ctypes.c_int
    lib.gdn_spec_attn_verify.argtypes = [pattn, vp, vp, vp, i32, vp, i32, vp, i32, i32, vp, sz, vp, vp, vp]
    lib.gdn_spec_attn_verify_static.restype = ctypes.c_int
    lib.gdn_spec_attn_verify_static.argtypes = [pattn, vp, vp, vp, i32, vp, i32, vp, i32, i32, vp, vp, vp]
    lib.gdn_spec_sample_scratch_bytes.restype = ctypes.c_int
    lib.gdn_spec_sample_scratch_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
    lib.gdn_spec_accept_sample.restype = ctypes.c_int
    lib.gdn_spec_accept_sample.argtypes = [ctypes.POINTER(GdnSampleInputs), i32, i32, i32, i32, ctypes.c_uint64,
                                           vp, sz, vp, vp, vp, vp]
    lib.gdn_strerror.restype = ctypes.c_char_p
    lib.gdn_strerror.argtypes = [ctypes.c_int]
    if path is None:
        _lib = lib
    return lib


def layer_desc(shape) -> GdnLayerDesc:
    """Descriptor from any object with the LayerShape fields."""
    return GdnLayerDesc(
        shape.num_k_heads, shape.num_v_heads, shape.d_k, shape.d_v, shape.conv_width,
        GDN_F32 if shape.dtype == "f32" else GDN_BF16,
        GDN_ACT_SILU if shape.act == "silu" else GDN_ACT_NONE,
        float(shape.scale), float(shape.l2_eps))


def _mode(mode) -> int:
    return MODES[mode] if isinstance(mode, str) else int(mode)


def _ptr(t):
    """Device pointer of a torch tensor (None -> NULL). Callers check the
    tensor with _check first."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _torch():
    import torch
    return torch


def _storage_dtype(desc):
    torch = _torch()
    return torch.float32 if int(desc.dtype) == GDN_F32 else torch.bfloat16


def _check(t, name, dtype, shape=None, device=None, optional=False, min_numel=None):
    """Refuses, before any pointer reaches the library, a tensor the C ABI
    would misread: not a torch tensor on a GPU, on another device than the
    call's other buffers, of another dtype, not contiguous, or of another
    shape (an exact tuple; None entries match any extent) or too small.
    The library cannot see buffer sizes, so these checks are what stands
    between a wrong tensor and an out-of-bounds access on the device."""
    torch = _torch()
    if t is None:
        if optional:
            return
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor, got %s" % (name, type(t).__name__))
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None:
        got = tuple(t.shape)
        if len(got) != len(shape) or any(w is not None and g != w for g, w in zip(got, shape)):
            raise ValueError("%s has shape %s, expected %s" % (name, got, tuple("*" if w is None else w for w in shape)))
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError("%s holds %d elements, at least %d needed" % (name, t.numel(), min_numel))
    if not t.is_cuda:
        raise ValueError("%s must be in GPU memory (got device %s)" % (name, t.device))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, the call's other buffers on %s" % (name, t.device, device))


def _layer_dims(desc):
    HK, HV, dk, dv, W = (int(desc.num_k_heads), int(desc.num_v_heads), int(desc.d_k), int(desc.d_v),
                         int(desc.conv_width))
    return HK, HV, dk, dv, W, 2 * HK * dk + HV * dv


def _check_pool(desc, ssm, conv):
    """The pool tensors of one layer; returns (device, num_slots)."""
    torch = _torch()
    HK, HV, dk, dv, W, C = _layer_dims(desc)
    _check(ssm, "ssm", torch.float32, (None, HV, dk, dv))
    P = int(ssm.shape[0])
    _check(conv, "conv", _storage_dtype(desc), (P, W - 1, C), device=ssm.device)
    return ssm.device, P


def _check_slot_table(slot_ids, device, batch=None):
    torch = _torch()
    _check(slot_ids, "slot_ids", torch.int32, (None,) if batch is None else (batch,), device=device)
    return int(slot_ids.shape[0])


def check_slot_ids_host(slot_ids, num_slots):
    """Opt-in check of a host copy of a slot table: every id is -1 (padding)
    or in [0, num_slots), and no two requests share a slot. Two requests on
    one slot would have two sets of workgroups committing into the same
    state, with no defined result. The library cannot see this without a
    device-to-host read, so the check runs on a table the caller still holds
    on the host (a list, a numpy array or a CPU tensor). Raises ValueError."""
    import numpy as np
    if hasattr(slot_ids, "detach"):
        if slot_ids.is_cuda:
            raise ValueError("check_slot_ids_host takes the host copy of the slot table")
        slot_ids = slot_ids.detach().numpy()
    a = np.asarray(slot_ids)
    if a.ndim != 1 or not np.issubdtype(a.dtype, np.integer):
        raise ValueError("slot table must be a 1-D integer array")
    bad = (a < -1) | (a >= num_slots)
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise ValueError("slot id %d of request %d is outside [-1, %d)" % (int(a[i]), i, num_slots))
    live = a[a >= 0]
    uniq, counts = np.unique(live, return_counts=True)
    if (counts > 1).any():
        s = int(uniq[np.flatnonzero(counts > 1)[0]])
        reqs = np.flatnonzero(a == s).tolist()
        raise ValueError("slot %d is shared by requests %s" % (s, reqs))


def check_src_rows_host(src_row, prev_batch, slot_ids=None):
    """Opt-in check of a host copy of a commit-verify's source-row table:
    every entry is -1 or a row of the previous batch [0, prev_batch), and no
    previous row is named twice (its accepted rows would be committed twice).
    With the host slot table, padding requests (slot -1), whose source is
    ignored, are left out. Raises ValueError."""
    import numpy as np

    def host(t, what):
        if hasattr(t, "detach"):
            if t.is_cuda:
                raise ValueError("check_src_rows_host takes the host copy of the %s" % what)
            t = t.detach().numpy()
        return np.asarray(t)
    a = host(src_row, "source-row table")
    if a.ndim != 1 or not np.issubdtype(a.dtype, np.integer):
        raise ValueError("source-row table must be a 1-D integer array")
    if slot_ids is not None:
        sl = host(slot_ids, "slot table")
        if sl.shape != a.shape:
            raise ValueError("slot table and source-row table differ in length")
        a = np.where(sl == -1, -1, a)
    bad = (a < -1) | (a >= prev_batch)
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise ValueError("source row %d of request %d is outside [-1, %d)" % (int(a[i]), i, prev_batch))
    live = a[a >= 0]
    uniq, counts = np.unique(live, return_counts=True)
    if (counts > 1).any():
        r = int(uniq[np.flatnonzero(counts > 1)[0]])
        raise ValueError("previous row %d is named by requests %s" % (r, np.flatnonzero(a == r).tolist()))


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def gdn_strerror(status: int) -> str:
    return load_library().gdn_strerror(int(status)).decode()


def gdn_spec_scratch_bytes(desc: GdnLayerDesc, batch: int, rows: int, mode="replay") -> int:
    out = ctypes.c_size_t(0)
    st = load_library().gdn_spec_scratch_bytes(ctypes.byref(desc), batch, rows, _mode(mode),
                                               ctypes.byref(out))
    if st != GDN_OK:
        raise GdnError(st, "gdn_spec_scratch_bytes")
    return out.value


def make_pool(ssm, conv) -> GdnPool:
    return GdnPool(_ptr(ssm), _ptr(conv), int(ssm.shape[0]))


def _nbytes(t):
    return t.numel() * t.element_size()


def _check_verify_args(desc, ssm, conv, conv_w, x, alpha, beta, slot_ids, rows, scratch, out, err_flag):
    """Every tensor of a verify call against the header's layouts; returns the batch."""
    torch = _torch()
    dev, _ = _check_pool(desc, ssm, conv)
    HK, HV, dk, dv, W, C = _layer_dims(desc)
    B = _check_slot_table(slot_ids, dev)
    st = _storage_dtype(desc)
    if B > 0:
        _check(conv_w, "conv_w", st, (C, W), device=dev)
        _check(x, "x", st, (B, rows, C), device=dev)
        _check(alpha, "alpha", st, (B, rows, HV), device=dev)
        _check(beta, "beta", st, (B, rows, HV), device=dev)
        _check(out, "out", st, (B, rows, HV, dv), device=dev)
        _check(scratch, "scratch", torch.uint8, device=dev)
    _check(err_flag, "err_flag", torch.int32, device=dev, optional=True, min_numel=1)
    return B


def _check_commit_args(desc, ssm, conv, slot_ids, accept_len, scratch, err_flag):
    torch = _torch()
    dev, _ = _check_pool(desc, ssm, conv)
    B = _check_slot_table(slot_ids, dev)
    if B > 0:
        _check(accept_len, "accept_len", torch.int32, (B,), device=dev)
        _check(scratch, "scratch", torch.uint8, device=dev)
    _check(err_flag, "err_flag", torch.int32, device=dev, optional=True, min_numel=1)
    return B


def gdn_spec_verify(desc, ssm, conv, conv_w, x, alpha, beta, slot_ids, rows, mode, scratch, out,
                    err_flag=None, stream=None, host_slot_ids=None):
    """Verify `rows` rows of every request; tensors are device tensors in the
    header's layouts (checked here). With `host_slot_ids` (the caller's host
    copy of slot_ids), the slot table is also checked for range and for
    requests sharing a slot."""
    B = _check_verify_args(desc, ssm, conv, conv_w, x, alpha, beta, slot_ids, rows, scratch, out, err_flag)
    if host_slot_ids is not None:
        check_slot_ids_host(host_slot_ids, int(ssm.shape[0]))
    pool = make_pool(ssm, conv)
    st = load_library().gdn_spec_verify(
        ctypes.byref(desc), ctypes.byref(pool), _ptr(conv_w), _ptr(x), _ptr(alpha), _ptr(beta),
        _ptr(slot_ids), B, rows, _mode(mode), _ptr(scratch), _nbytes(scratch) if B else 0, _ptr(out),
        _ptr(err_flag), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_spec_verify")


def gdn_spec_commit(desc, ssm, conv, slot_ids, accept_len, rows, mode, scratch, err_flag=None,
                    stream=None, host_slot_ids=None):
    """Commit accept_len[b] rows of each request verified on this scratch
    (tensors checked as for gdn_spec_verify)."""
    B = _check_commit_args(desc, ssm, conv, slot_ids, accept_len, scratch, err_flag)
    if host_slot_ids is not None:
        check_slot_ids_host(host_slot_ids, int(ssm.shape[0]))
    pool = make_pool(ssm, conv)
    st = load_library().gdn_spec_commit(
        ctypes.byref(desc), ctypes.byref(pool), _ptr(slot_ids), _ptr(accept_len), B, rows,
        _mode(mode), _ptr(scratch), _nbytes(scratch) if B else 0, _ptr(err_flag), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_spec_commit")


def _check_commit_verify_args(desc, ssm, conv, conv_w, x, alpha, beta, slot_ids, rows, scratch, src_row,
                              prev_scratch, prev_slot_ids, prev_accept_len, out, err_flag):
    """A commit-verify call: this step's verify tensors, the source-row table
    and the previous step's slot table, accept lengths and scratch. Returns
    (batch, previous batch)."""
    torch = _torch()
    B = _check_verify_args(desc, ssm, conv, conv_w, x, alpha, beta, slot_ids, rows, scratch, out, err_flag)
    dev = ssm.device
    Bp = 0 if prev_slot_ids is None else _check_slot_table(prev_slot_ids, dev)
    if B > 0:
        _check(src_row, "src_row", torch.int32, (B,), device=dev)
    if Bp > 0:
        _check(prev_accept_len, "prev_accept_len", torch.int32, (Bp,), device=dev)
        _check(prev_scratch, "prev_scratch", torch.uint8, device=dev)
    return B, Bp


class PreparedCommitVerify:
    """gdn_spec_commit_verify on fixed device tensors: commits the previous
    step's accepted rows (prev_slot_ids, prev_accept_len, prev_scratch) into
    the slots src_row maps them to, then verifies this step's rows, in one
    launch. Checked and turned into ctypes arguments once."""

    def __init__(self, desc, ssm, conv, conv_w, x, alpha, beta, slot_ids, rows, scratch, src_row, prev_scratch,
                 prev_slot_ids, prev_accept_len, out, err_flag=None, stream=None, host_slot_ids=None,
                 host_src_row=None, mode="replay"):
        B, Bp = _check_commit_verify_args(desc, ssm, conv, conv_w, x, alpha, beta, slot_ids, rows, scratch, src_row,
                                          prev_scratch, prev_slot_ids, prev_accept_len, out, err_flag)
        if host_slot_ids is not None:
            check_slot_ids_host(host_slot_ids, int(ssm.shape[0]))
        if host_src_row is not None:
            check_src_rows_host(host_src_row, Bp, host_slot_ids)
        self.lib = load_library()
        self._keep = (ssm, conv, conv_w, x, alpha, beta, slot_ids, scratch, src_row, prev_scratch, prev_slot_ids,
                      prev_accept_len, out, err_flag)
        self.desc = desc
        self.pool = make_pool(ssm, conv)
        self.args = (ctypes.byref(self.desc), ctypes.byref(self.pool), _ptr(conv_w), _ptr(x), _ptr(alpha),
                     _ptr(beta), _ptr(slot_ids), B, rows, _mode(mode), _ptr(scratch), _nbytes(scratch) if B else 0,
                     _ptr(src_row),
                     _ptr(prev_scratch) if Bp else None, _nbytes(prev_scratch) if Bp else 0,
                     _ptr(prev_slot_ids) if Bp else None, _ptr(prev_accept_len) if Bp else None, Bp, _ptr(out),
                     _ptr(err_flag), _stream(stream))

    def __call__(self):
        st = self.lib.gdn_spec_commit_verify(*self.args)
        if st != GDN_OK:
            raise GdnError(st, "gdn_spec_commit_verify")


def gdn_spec_commit_verify(desc, ssm, conv, conv_w, x, alpha, beta, slot_ids, rows, scratch, src_row, prev_scratch,
                           prev_slot_ids, prev_accept_len, out, err_flag=None, stream=None, host_slot_ids=None,
                           host_src_row=None, mode="replay"):
    """Commit the previous step's accepted rows and verify this step's rows in
    one launch (replay or snapshot mode); src_row[b] names the previous batch
    row pending on slot_ids[b], or -1. With host copies of the slot and
    source-row tables (host_slot_ids, host_src_row), those are checked too."""
    PreparedCommitVerify(desc, ssm, conv, conv_w, x, alpha, beta, slot_ids, rows, scratch, src_row, prev_scratch,
                         prev_slot_ids, prev_accept_len, out, err_flag, stream, host_slot_ids, host_src_row, mode)()


class PreparedCommitLayers:
    """gdn_spec_commit_layers over fixed per-layer (ssm, conv, scratch) device
    tensors, checked and turned into ctypes arguments once."""

    def __init__(self, desc, layers, slot_ids, accept_len, rows, mode, err_flag=None, stream=None,
                 host_slot_ids=None):
        if not layers:
            raise ValueError("no layers")
        for ssm, conv, sc in layers:
            B = _check_commit_args(desc, ssm, conv, slot_ids, accept_len, sc, err_flag)
            if host_slot_ids is not None:
                check_slot_ids_host(host_slot_ids, int(ssm.shape[0]))
        self.lib = load_library()
        self._keep = (layers, slot_ids, accept_len, err_flag)
        self.desc = desc
        L = len(layers)
        self.pools = (GdnPool * L)(*[make_pool(ssm, conv) for ssm, conv, _ in layers])
        self.scratch = (ctypes.c_void_p * L)(*[_ptr(sc) for _, _, sc in layers])
        nbytes = min(_nbytes(sc) for _, _, sc in layers)
        self.args = (ctypes.byref(self.desc), self.pools, self.scratch, L, _ptr(slot_ids), _ptr(accept_len),
                     B, rows, _mode(mode), nbytes, _ptr(err_flag), _stream(stream))

    def __call__(self):
        st = self.lib.gdn_spec_commit_layers(*self.args)
        if st != GDN_OK:
            raise GdnError(st, "gdn_spec_commit_layers")


def gdn_spec_commit_layers(desc, layers, slot_ids, accept_len, rows, mode, err_flag=None, stream=None,
                           host_slot_ids=None):
    """Commit every layer in one launch; layers = [(ssm, conv, scratch), ...] device tensors."""
    PreparedCommitLayers(desc, layers, slot_ids, accept_len, rows, mode, err_flag, stream, host_slot_ids)()


def _check_window(state, rows_t, B, R, device):
    """A window state [P][L][...] and its staged rows [B][R][...]: same dtype
    and entry shape, entries a multiple of 4 bytes; returns the descriptor."""
    torch = _torch()
    if not isinstance(state, torch.Tensor) or state.dim() < 2:
        raise ValueError("window state must be a tensor [slots][length][...]")
    _check(state, "window state", state.dtype, tuple(state.shape), device=device)
    _check(rows_t, "window rows", state.dtype, (B, R) + tuple(state.shape[2:]), device=device)
    entry = state.element_size()
    for e in state.shape[2:]:
        entry *= int(e)
    if entry % 4 or entry == 0:
        raise ValueError("window entries are %d bytes, a positive multiple of 4 is needed" % entry)
    return GdnSlotWindow(_ptr(state), _ptr(rows_t), int(state.shape[0]), int(state.shape[1]), entry)


class PreparedCommitAll:
    """gdn_spec_commit_all: GDN layers [(ssm, conv, scratch), ...] and window
    states [(state, rows), ...] committed in one launch, checked and turned
    into ctypes arguments once."""

    def __init__(self, desc, layers, windows, slot_ids, accept_len, rows, mode, err_flag=None, stream=None,
                 host_slot_ids=None):
        torch = _torch()
        if not layers and not windows:
            raise ValueError("nothing to commit")
        B = dev = None
        for ssm, conv, sc in layers:
            B = _check_commit_args(desc, ssm, conv, slot_ids, accept_len, sc, err_flag)
            dev = ssm.device
            if host_slot_ids is not None:
                check_slot_ids_host(host_slot_ids, int(ssm.shape[0]))
        if B is None:
            B = _check_slot_table(slot_ids, None)
            dev = slot_ids.device
            _check(accept_len, "accept_len", torch.int32, (B,), device=dev)
            _check(err_flag, "err_flag", torch.int32, (None,), device=dev, optional=True)
        wins = [_check_window(st, rw, B, rows, dev) for st, rw in windows]
        if host_slot_ids is not None:
            for st, _ in windows:
                check_slot_ids_host(host_slot_ids, int(st.shape[0]))
        self.lib = load_library()
        self._keep = (layers, windows, slot_ids, accept_len, err_flag)
        self.desc = desc
        L = len(layers)
        self.pools = (GdnPool * max(L, 1))(*[make_pool(ssm, conv) for ssm, conv, _ in layers])
        self.scratch = (ctypes.c_void_p * max(L, 1))(*[_ptr(sc) for _, _, sc in layers])
        self.windows = (GdnSlotWindow * max(len(wins), 1))(*wins)
        nbytes = min(_nbytes(sc) for _, _, sc in layers) if layers else 0
        self.args = (ctypes.byref(self.desc) if desc is not None else None, self.pools if L else None,
                     self.scratch if L else None, L, self.windows if wins else None, len(wins), _ptr(slot_ids),
                     _ptr(accept_len), B, rows, _mode(mode), nbytes, _ptr(err_flag), _stream(stream))

    def __call__(self):
        st = self.lib.gdn_spec_commit_all(*self.args)
        if st != GDN_OK:
            raise GdnError(st, "gdn_spec_commit_all")


def gdn_spec_commit_all(desc, layers, windows, slot_ids, accept_len, rows, mode, err_flag=None, stream=None,
                        host_slot_ids=None):
    """Commit GDN layers [(ssm, conv, scratch), ...] and window states
    [(state [P][L][...], rows [B][R][...]), ...] in one launch."""
    PreparedCommitAll(desc, layers, windows, slot_ids, accept_len, rows, mode, err_flag, stream, host_slot_ids)()


def _check_accept_args(draft, target, slot_ids, rows, accept_len, next_token):
    torch = _torch()
    _check(target, "target", torch.int32, (None, rows))
    dev = target.device
    B = int(target.shape[0])
    _check(draft, "draft", torch.int32, (B, rows - 1), device=dev, optional=rows == 1)
    _check(slot_ids, "slot_ids", torch.int32, (B,), device=dev, optional=True)
    _check(accept_len, "accept_len", torch.int32, (B,), device=dev)
    _check(next_token, "next_token", torch.int32, (B,), device=dev, optional=True)
    return B


def gdn_spec_accept_greedy(draft, target, slot_ids, rows, accept_len, next_token=None, stream=None):
    """accept_len (and next_token) from the draft and target greedy tokens, on the device."""
    B = _check_accept_args(draft, target, slot_ids, rows, accept_len, next_token)
    st = load_library().gdn_spec_accept_greedy(_ptr(draft), _ptr(target), _ptr(slot_ids), B, rows,
                                               _ptr(accept_len), _ptr(next_token), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_spec_accept_greedy")


class Prepared:
    """Verify and commit on fixed device tensors, checked and turned into
    ctypes arguments once, so that issuing a launch costs one foreign call."""

    def __init__(self, desc, ssm, conv, conv_w, x, alpha, beta, slot_ids, accept_len, rows, mode,
                 scratch, out, err_flag=None, stream=None):
        B = _check_verify_args(desc, ssm, conv, conv_w, x, alpha, beta, slot_ids, rows, scratch, out, err_flag)
        _check_commit_args(desc, ssm, conv, slot_ids, accept_len, scratch, err_flag)
        self.lib = load_library()
        self._keep = (ssm, conv, conv_w, x, alpha, beta, slot_ids, accept_len, scratch, out, err_flag)
        self.desc = desc
        self.pool = make_pool(ssm, conv)
        st = _stream(stream)
        m = _mode(mode)
        self.vargs = (ctypes.byref(self.desc), ctypes.byref(self.pool), _ptr(conv_w), _ptr(x),
                      _ptr(alpha), _ptr(beta), _ptr(slot_ids), B, rows, m, _ptr(scratch),
                      _nbytes(scratch), _ptr(out), _ptr(err_flag), st)
        self.cargs = (ctypes.byref(self.desc), ctypes.byref(self.pool), _ptr(slot_ids),
                      _ptr(accept_len), B, rows, m, _ptr(scratch), _nbytes(scratch),
                      _ptr(err_flag), st)

    def verify(self):
        st = self.lib.gdn_spec_verify(*self.vargs)
        if st != GDN_OK:
            raise GdnError(st, "gdn_spec_verify")

    def commit(self):
        st = self.lib.gdn_spec_commit(*self.cargs)
        if st != GDN_OK:
            raise GdnError(st, "gdn_spec_commit")


class PreparedAccept:
    """gdn_spec_accept_greedy on fixed device tensors, checked and turned into
    ctypes arguments once."""

    def __init__(self, draft, target, slot_ids, rows, accept_len, next_token=None, stream=None):
        B = _check_accept_args(draft, target, slot_ids, rows, accept_len, next_token)
        self.lib = load_library()
        self._keep = (draft, target, slot_ids, accept_len, next_token)
        self.args = (_ptr(draft), _ptr(target), _ptr(slot_ids), B, rows,
                     _ptr(accept_len), _ptr(next_token), _stream(stream))

    def __call__(self):
        st = self.lib.gdn_spec_accept_greedy(*self.args)
        if st != GDN_OK:
            raise GdnError(st, "gdn_spec_accept_greedy")


def attn_desc(shape) -> GdnAttnDesc:
    """Descriptor from any object with the AttnShape fields."""
    return GdnAttnDesc(shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.page_size,
                       float(shape.scale))


def gdn_spec_attn_scratch_bytes(desc: GdnAttnDesc, batch: int, rows: int, max_blocks: int) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().gdn_spec_attn_scratch_bytes(ctypes.byref(desc), batch, rows, max_blocks,
                                                    ctypes.byref(out))
    if st != GDN_OK:
        raise GdnError(st, "gdn_spec_attn_scratch_bytes")
    return out.value


def _check_attn_args(desc, q, k_cache, v_cache, block_table, seq_lens, scratch, out, err_flag, static=False):
    torch = _torch()
    Hq, Hkv, D, page = int(desc.num_q_heads), int(desc.num_kv_heads), int(desc.head_dim), int(desc.page_size)
    _check(q, "q", torch.bfloat16, (None, None, Hq, D))
    dev = q.device
    B, R = int(q.shape[0]), int(q.shape[1])
    _check(k_cache, "k_cache", torch.bfloat16, (None, page, Hkv, D), device=dev)
    _check(v_cache, "v_cache", torch.bfloat16, tuple(k_cache.shape), device=dev)
    _check(block_table, "block_table", torch.int32, (B, None), device=dev)
    _check(seq_lens, "seq_lens", torch.int32, (B,), device=dev)
    _check(out, "out", torch.bfloat16, (B, R, Hq, D), device=dev)
    if not static:
        _check(scratch, "scratch", torch.uint8, device=dev)
    _check(err_flag, "err_flag", torch.int32, device=dev, optional=True, min_numel=1)
    return B, R


class PreparedAttn:
    """gdn_spec_attn_verify on fixed device tensors, checked and turned into
    ctypes arguments once. q [B][R][Hq][D], caches [pages][page_size][Hkv][D]
    (bf16), block_table [B][max_blocks] and seq_lens [B] (int32), out like q."""

    def __init__(self, desc, q, k_cache, v_cache, block_table, seq_lens, scratch, out, err_flag=None,
                 stream=None):
        B, R = _check_attn_args(desc, q, k_cache, v_cache, block_table, seq_lens, scratch, out, err_flag)
        self.lib = load_library()
        self._keep = (q, k_cache, v_cache, block_table, seq_lens, scratch, out, err_flag)
        self.desc = desc
        self.args = (ctypes.byref(self.desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), int(k_cache.shape[0]),
                     _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens), B, R, _ptr(scratch),
                     _nbytes(scratch), _ptr(out), _ptr(err_flag), _stream(stream))

    def __call__(self):
        st = self.lib.gdn_spec_attn_verify(*self.args)
        if st != GDN_OK:
            raise GdnError(st, "gdn_spec_attn_verify")


def gdn_spec_attn_verify(desc, q, k_cache, v_cache, block_table, seq_lens, scratch, out, err_flag=None,
                         stream=None):
    PreparedAttn(desc, q, k_cache, v_cache, block_table, seq_lens, scratch, out, err_flag, stream)()


def gdn_spec_attn_verify_static(desc, q, k_cache, v_cache, block_table, seq_lens, out, err_flag=None,
                                stream=None):
    """gdn_spec_attn_verify on the library's own device array instead of a
    scratch argument: no allocation anywhere (tensors checked as there)."""
    B, R = _check_attn_args(desc, q, k_cache, v_cache, block_table, seq_lens, None, out, err_flag, static=True)
    st = load_library().gdn_spec_attn_verify_static(
        ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), int(k_cache.shape[0]), _ptr(block_table),
        int(block_table.shape[1]), _ptr(seq_lens), B, R, _ptr(out), _ptr(err_flag), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_spec_attn_verify_static")


def gdn_spec_sample_scratch_bytes(batch: int, rows: int, vocab: int) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().gdn_spec_sample_scratch_bytes(batch, rows, vocab, ctypes.byref(out))
    if st != GDN_OK:
        raise GdnError(st, "gdn_spec_sample_scratch_bytes")
    return out.value


class PreparedSample:
    """gdn_spec_accept_sample on fixed device tensors, checked and turned into
    ctypes arguments once; the seed is given per call. logits [B][R][V] fp32
    or bf16, draft [B][R-1] int32, the optional inputs as in the header."""

    def __init__(self, logits, draft, temperature, accept_len, next_token, scratch, draft_probs=None,
                 pending=None, prior_counts=None, presence=None, frequency=None, slot_ids=None, err_flag=None,
                 stream=None):
        torch = _torch()
        if logits is None or logits.dim() != 3:
            raise ValueError("logits must be [batch][rows][vocab]")
        if logits.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("logits must be float32 or bfloat16, got %s" % logits.dtype)
        B, R, V = (int(x) for x in logits.shape)
        _check(logits, "logits", logits.dtype, (B, R, V))
        dev = logits.device
        _check(draft, "draft", torch.int32, (B, R - 1), device=dev, optional=R == 1)
        _check(draft_probs, "draft_probs", torch.float32, (B, R - 1, V), device=dev, optional=True)
        _check(pending, "pending", torch.int32, (B,), device=dev, optional=True)
        _check(prior_counts, "prior_counts", torch.int32, (B, V), device=dev, optional=True)
        _check(temperature, "temperature", torch.float32, (B,), device=dev)
        _check(presence, "presence", torch.float32, (B,), device=dev, optional=True)
        _check(frequency, "frequency", torch.float32, (B,), device=dev, optional=True)
        _check(slot_ids, "slot_ids", torch.int32, (B,), device=dev, optional=True)
        _check(accept_len, "accept_len", torch.int32, (B,), device=dev)
        _check(next_token, "next_token", torch.int32, (B,), device=dev)
        _check(scratch, "scratch", torch.uint8, device=dev, min_numel=gdn_spec_sample_scratch_bytes(B, R, V))
        _check(err_flag, "err_flag", torch.int32, device=dev, optional=True, min_numel=1)
        self.lib = load_library()
        self._keep = (logits, draft, temperature, accept_len, next_token, scratch, draft_probs, pending,
                      prior_counts, presence, frequency, slot_ids, err_flag)
        self.inputs = GdnSampleInputs(_ptr(logits), _ptr(draft_probs), _ptr(draft), _ptr(pending),
                                      _ptr(prior_counts), _ptr(temperature), _ptr(presence), _ptr(frequency),
                                      _ptr(slot_ids))
        self.head = (ctypes.byref(self.inputs), GDN_F32 if logits.dtype == torch.float32 else GDN_BF16, B, R, V)
        self.tail = (_ptr(scratch), _nbytes(scratch), _ptr(accept_len), _ptr(next_token), _ptr(err_flag),
                     _stream(stream))

    def __call__(self, seed: int):
        st = self.lib.gdn_spec_accept_sample(*self.head, ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
                                             *self.tail)
        if st != GDN_OK:
            raise GdnError(st, "gdn_spec_accept_sample")


def gdn_spec_accept_sample(logits, draft, temperature, seed, accept_len, next_token, scratch, **optional):
    """Speculative sampling on the device (see PreparedSample for the inputs)."""
    PreparedSample(logits, draft, temperature, accept_len, next_token, scratch, **optional)(seed)
