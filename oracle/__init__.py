"""CPU oracle for the GatedDeltaNet speculative verify/commit step.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. It wraps the plain C
reference in ``gdn_oracle.c`` (fp64, row by row); it imports nothing from the
HIP library's package and shares no code with it.

Arguments are numpy arrays in the storage layouts the C file documents; bf16
tensors are ``uint16`` bit patterns. ``shape`` is any object with the fields
num_k_heads, num_v_heads, d_k, d_v, conv_width, dtype ("f32"/"bf16"), act
("silu"/"none"), scale and l2_eps.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "gdn_oracle.c")
LIBRARY = os.path.join(HERE, "libgdn_oracle.so")

ERR_SLOT = 1
ERR_ACCEPT = 2
ERR_ARGS = 1 << 30


class _Desc(ctypes.Structure):
    _fields_ = [
        ("num_k_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("d_k", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("conv_width", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("act", ctypes.c_int32),
        ("pad_", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("l2_eps", ctypes.c_double),
    ]


def compile_library(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the C oracle with gcc (OpenMP over requests)."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


def build() -> str:
    return compile_library()


def compile_variant(source_text: str, workdir: str | None = None) -> str:
    """Compile a modified copy of the oracle (used by the mutation tests)."""
    workdir = workdir or tempfile.mkdtemp(prefix="gdn_oracle_")
    src = os.path.join(workdir, "variant.c")
    with open(src, "w") as f:
        f.write(source_text)
    return compile_library(src, os.path.join(workdir, "libvariant.so"))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    def __init__(self, lib_path: str | None = None):
        path = lib_path or LIBRARY
        if lib_path is None and not os.path.exists(path):
            compile_library()
        self.lib = ctypes.CDLL(path)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        self.lib.oracle_verify.restype = ctypes.c_int
        self.lib.oracle_verify.argtypes = [ctypes.POINTER(_Desc), vp, vp, i32, vp, vp, vp, vp,
                                           vp, i32, i32, vp, vp, i32]
        self.lib.oracle_commit.restype = ctypes.c_int
        self.lib.oracle_commit.argtypes = [ctypes.POINTER(_Desc), vp, vp, i32, vp, vp, vp, vp,
                                           vp, vp, i32, i32, i32]
        self.lib.oracle_decode_step.restype = ctypes.c_int
        self.lib.oracle_decode_step.argtypes = [ctypes.POINTER(_Desc), vp, vp, i32, vp, vp, vp,
                                                vp, vp, i32, vp, i32]

    @staticmethod
    def _desc(shape) -> _Desc:
        return _Desc(shape.num_k_heads, shape.num_v_heads, shape.d_k, shape.d_v,
                     shape.conv_width, 0 if shape.dtype == "f32" else 1,
                     0 if shape.act == "silu" else 1, 0, float(shape.scale), float(shape.l2_eps))

    @staticmethod
    def _c(a, dtype):
        a = np.ascontiguousarray(a)
        if a.dtype != dtype:
            raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
        return a

    def _store(self, shape):
        return np.float32 if shape.dtype == "f32" else np.uint16

    def verify(self, shape, ssm, conv, conv_w, x, alpha, beta, slot_ids, rows,
               want_snapshots=False, nthreads=1):
        """Returns (out [B][R][HV][d_v] fp64, snapshots [B][R][HV][d_k][d_v] fp64 or None, err)."""
        st = self._store(shape)
        ssm = self._c(ssm, np.float32)
        conv, conv_w, x = self._c(conv, st), self._c(conv_w, st), self._c(x, st)
        alpha, beta = self._c(alpha, st), self._c(beta, st)
        slot_ids = self._c(slot_ids, np.int32)
        B = slot_ids.shape[0]
        out = np.zeros((B, rows, shape.num_v_heads, shape.d_v), np.float64)
        snap = (np.zeros((B, rows, shape.num_v_heads, shape.d_k, shape.d_v), np.float64)
                if want_snapshots else None)
        d = self._desc(shape)
        err = self.lib.oracle_verify(ctypes.byref(d), _ptr(ssm), _ptr(conv), ssm.shape[0],
                                     _ptr(conv_w), _ptr(x), _ptr(alpha), _ptr(beta),
                                     _ptr(slot_ids), B, rows, _ptr(out), _ptr(snap), nthreads)
        return out, snap, err

    def commit(self, shape, ssm, conv, conv_w, x, alpha, beta, slot_ids, accept_len, rows,
               nthreads=1):
        """Commits in place into ``ssm`` and ``conv`` (which must be contiguous); returns err."""
        st = self._store(shape)
        for a, t in ((ssm, np.float32), (conv, st)):
            if a.dtype != t or not a.flags.c_contiguous:
                raise TypeError("pool arrays must be contiguous %s" % np.dtype(t))
        conv_w, x = self._c(conv_w, st), self._c(x, st)
        alpha, beta = self._c(alpha, st), self._c(beta, st)
        slot_ids = self._c(slot_ids, np.int32)
        accept_len = self._c(accept_len, np.int32)
        d = self._desc(shape)
        return self.lib.oracle_commit(ctypes.byref(d), _ptr(ssm), _ptr(conv), ssm.shape[0],
                                      _ptr(conv_w), _ptr(x), _ptr(alpha), _ptr(beta),
                                      _ptr(slot_ids), _ptr(accept_len), slot_ids.shape[0],
                                      rows, nthreads)

    def decode_step(self, shape, ssm, conv, conv_w, x_t, alpha_t, beta_t, slot_ids, nthreads=1):
        """One decode step in place; x_t [B][C], gates [B][HV]. Returns (out [B][HV][d_v], err)."""
        st = self._store(shape)
        for a, t in ((ssm, np.float32), (conv, st)):
            if a.dtype != t or not a.flags.c_contiguous:
                raise TypeError("pool arrays must be contiguous %s" % np.dtype(t))
        conv_w, x_t = self._c(conv_w, st), self._c(x_t, st)
        alpha_t, beta_t = self._c(alpha_t, st), self._c(beta_t, st)
        slot_ids = self._c(slot_ids, np.int32)
        B = slot_ids.shape[0]
        out = np.zeros((B, shape.num_v_heads, shape.d_v), np.float64)
        d = self._desc(shape)
        err = self.lib.oracle_decode_step(ctypes.byref(d), _ptr(ssm), _ptr(conv), ssm.shape[0],
                                          _ptr(conv_w), _ptr(x_t), _ptr(alpha_t), _ptr(beta_t),
                                          _ptr(slot_ids), B, _ptr(out), nthreads)
        return out, err


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
