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

EXPORTS = ("gdn_spec_scratch_bytes", "gdn_spec_verify", "gdn_spec_commit", "gdn_spec_commit_layers",
           "gdn_spec_accept_greedy", "gdn_strerror", "gdn_spec_attn_scratch_bytes", "gdn_spec_attn_verify")


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


class GdnAttnDesc(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


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
    lib.gdn_spec_commit_layers.restype = ctypes.c_int
    lib.gdn_spec_commit_layers.argtypes = [pdesc, ppool, ctypes.POINTER(vp), i32, vp, vp, i32, i32,
                                           ctypes.c_int, sz, vp, vp]
    lib.gdn_spec_accept_greedy.restype = ctypes.c_int
    lib.gdn_spec_accept_greedy.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp]
    pattn = ctypes.POINTER(GdnAttnDesc)
    lib.gdn_spec_attn_scratch_bytes.restype = ctypes.c_int
    lib.gdn_spec_attn_scratch_bytes.argtypes = [pattn, i32, i32, i32, ctypes.POINTER(sz)]
    lib.gdn_spec_attn_verify.restype = ctypes.c_int
    lib.gdn_spec_attn_verify.argtypes = [pattn, vp, vp, vp, i32, vp, i32, vp, i32, i32, vp, sz, vp, vp, vp]
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
    """Device pointer of a torch tensor (None -> NULL; ints pass through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


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
    return GdnPool(_ptr(ssm), _ptr(conv), int(ssm.shape[0]) if hasattr(ssm, "shape") else 0)


def _nbytes(t):
    return t.numel() * t.element_size()


def gdn_spec_verify(desc, ssm, conv, conv_w, x, alpha, beta, slot_ids, rows, mode, scratch, out,
                    err_flag=None, stream=None, batch=None):
    """Verify `rows` rows of every request; tensors are device tensors in the header's layouts."""
    pool = make_pool(ssm, conv)
    B = int(slot_ids.shape[0]) if batch is None else batch
    st = load_library().gdn_spec_verify(
        ctypes.byref(desc), ctypes.byref(pool), _ptr(conv_w), _ptr(x), _ptr(alpha), _ptr(beta),
        _ptr(slot_ids), B, rows, _mode(mode), _ptr(scratch), _nbytes(scratch), _ptr(out),
        _ptr(err_flag), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_spec_verify")


def gdn_spec_commit(desc, ssm, conv, slot_ids, accept_len, rows, mode, scratch, err_flag=None,
                    stream=None, batch=None):
    """Commit accept_len[b] rows of each request verified on this scratch."""
    pool = make_pool(ssm, conv)
    B = int(slot_ids.shape[0]) if batch is None else batch
    st = load_library().gdn_spec_commit(
        ctypes.byref(desc), ctypes.byref(pool), _ptr(slot_ids), _ptr(accept_len), B, rows,
        _mode(mode), _ptr(scratch), _nbytes(scratch), _ptr(err_flag), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_spec_commit")


class PreparedCommitLayers:
    """gdn_spec_commit_layers over fixed per-layer (ssm, conv, scratch) device
    tensors, ctypes arguments built once."""

    def __init__(self, desc, layers, slot_ids, accept_len, rows, mode, err_flag=None, stream=None):
        self.lib = load_library()
        self._keep = (layers, slot_ids, accept_len, err_flag)
        self.desc = desc
        L = len(layers)
        self.pools = (GdnPool * L)(*[make_pool(ssm, conv) for ssm, conv, _ in layers])
        self.scratch = (ctypes.c_void_p * L)(*[_ptr(sc) for _, _, sc in layers])
        nbytes = min(_nbytes(sc) for _, _, sc in layers)
        self.args = (ctypes.byref(self.desc), self.pools, self.scratch, L, _ptr(slot_ids), _ptr(accept_len),
                     int(slot_ids.shape[0]), rows, _mode(mode), nbytes, _ptr(err_flag), _stream(stream))

    def __call__(self):
        st = self.lib.gdn_spec_commit_layers(*self.args)
        if st != GDN_OK:
            raise GdnError(st, "gdn_spec_commit_layers")


def gdn_spec_commit_layers(desc, layers, slot_ids, accept_len, rows, mode, err_flag=None, stream=None):
    """Commit every layer in one launch; layers = [(ssm, conv, scratch), ...] device tensors."""
    PreparedCommitLayers(desc, layers, slot_ids, accept_len, rows, mode, err_flag, stream)()


def gdn_spec_accept_greedy(draft, target, slot_ids, rows, accept_len, next_token=None, stream=None,
                           batch=None):
    """accept_len (and next_token) from the draft and target greedy tokens, on the device."""
    B = int(target.shape[0]) if batch is None else batch
    st = load_library().gdn_spec_accept_greedy(_ptr(draft), _ptr(target), _ptr(slot_ids), B, rows,
                                               _ptr(accept_len), _ptr(next_token), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_spec_accept_greedy")


class Prepared:
    """Verify and commit on fixed device tensors with the ctypes arguments built
    once, so that issuing a launch costs one foreign call."""

    def __init__(self, desc, ssm, conv, conv_w, x, alpha, beta, slot_ids, accept_len, rows, mode,
                 scratch, out, err_flag=None, stream=None):
        self.lib = load_library()
        self._keep = (ssm, conv, conv_w, x, alpha, beta, slot_ids, accept_len, scratch, out, err_flag)
        self.desc = desc
        self.pool = make_pool(ssm, conv)
        B = int(slot_ids.shape[0])
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
    """gdn_spec_accept_greedy on fixed device tensors, ctypes arguments built once."""

    def __init__(self, draft, target, slot_ids, rows, accept_len, next_token=None, stream=None):
        self.lib = load_library()
        self._keep = (draft, target, slot_ids, accept_len, next_token)
        self.args = (_ptr(draft), _ptr(target), _ptr(slot_ids), int(target.shape[0]), rows,
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


class PreparedAttn:
    """gdn_spec_attn_verify on fixed device tensors, ctypes arguments built once.
    q [B][R][Hq][D], caches [pages][page_size][Hkv][D] (bf16), block_table
    [B][max_blocks] and seq_lens [B] (int32), out like q."""

    def __init__(self, desc, q, k_cache, v_cache, block_table, seq_lens, scratch, out, err_flag=None,
                 stream=None):
        self.lib = load_library()
        self._keep = (q, k_cache, v_cache, block_table, seq_lens, scratch, out, err_flag)
        self.desc = desc
        B, R = int(q.shape[0]), int(q.shape[1])
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
