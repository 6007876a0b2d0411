"""CPU oracle for the sparse Flash-MLA Softmax-L1Norm.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product
library (``sparse_mla_attention_02_amd``) never imports it and shares no code
with it; the only thing both sides share is the input generator in
``workloads``, which holds none of the operation's arithmetic.

Two formulations live here:

* ``smla_oracle.c`` (wrapped by :func:`lse` and :func:`l1norm`): the
  three-stage formula of the "SparseFlashMlaSoftmaxL1Norm" article (section
  三阶段计算公式) evaluated entry by entry in double precision, OpenMP over
  query rows.
* :mod:`oracle.brute`: a dense NumPy formulation for tiny inputs (full score
  matrix, boolean selection and visibility masks). It is the brute-force pin
  of the C code.

Parity status of each function, with what pins it, is listed in
``tests/test_oracle_pins.py``; every function here is pinned.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "smla_oracle.c")
_LIBPATH = os.path.join(_HERE, "liboracle.so")
_LIB = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIBPATH) or \
            os.path.getmtime(_LIBPATH) < os.path.getmtime(_SRC):
        tmp = _LIBPATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIBPATH)
    return _LIBPATH


class COracle:
    """ctypes handle on one build of ``smla_oracle.c``."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        common = [_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                  _i64, _i64, ctypes.c_double, _p, _i64]
        lib.oracle_lse.argtypes = [_p] + common + [_p, _p]
        lib.oracle_lse.restype = ctypes.c_int
        lib.oracle_l1norm.argtypes = [_p, _p, _p] + common[1:] + [_i64, _i64, _p]
        lib.oracle_l1norm.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def lse(self, p, rows: Optional[Sequence[int]] = None):
        """Forward log-sum-exp over each row's used entries, rounded to fp32.

        Returns ``(lse_rows (nrows, G) float32, nused (nrows,) int32)``.
        """
        a = _Args(p, rows)
        out = np.empty((len(a.rows), p.groups), dtype=np.float32)
        nused = np.empty((len(a.rows),), dtype=np.int32)
        rc = self.lib.oracle_lse(_ptr(a.q), *a.common(), _ptr(out), _ptr(nused))
        if rc != 0:
            raise ValueError("oracle_lse: undecodable row id")
        return out, nused

    def fill_lse(self, p):
        """Set ``p.softmax_lse`` to the oracle's lse for every row; returns nused."""
        l, nused = self.lse(p)
        p.softmax_lse = l.reshape(p.lse_shape())
        return nused

    def l1norm(self, p, rows: Optional[Sequence[int]] = None, softmax_lse=None):
        """The operation's output rows (nrows, W) float32 for the listed rows.

        ``softmax_lse`` defaults to ``p.softmax_lse`` (shape (B,N2,S1,G) or
        (N2,T1,G)).
        """
        a = _Args(p, rows)
        full = p.softmax_lse if softmax_lse is None else softmax_lse
        if full is None:
            raise ValueError("no softmax_lse given")
        full = np.asarray(full, dtype=np.float32).reshape(p.rows, p.groups)
        l = np.ascontiguousarray(full[a.rows])
        out = np.empty((len(a.rows), p.out_width), dtype=np.float32)
        rc = self.lib.oracle_l1norm(_ptr(a.q), _ptr(a.k), _ptr(l), *a.common()[1:],
                                    int(bool(getattr(p, "kwide", False))), p.out_width,
                                    _ptr(out))
        if rc != 0:
            raise ValueError("oracle_l1norm: undecodable row id or a column past the width")
        return out

    def num_threads(self) -> int:
        """Threads an OpenMP region of this build runs with."""
        return int(self.lib.oracle_num_threads())


def default() -> COracle:
    """The oracle built from the committed source."""
    global _LIB
    if _LIB is None:
        _LIB = COracle(build(force=False))
    return _LIB


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


class _Args:
    """Marshalled, contiguous views of a Problem for the C oracle."""

    def __init__(self, p, rows: Optional[Sequence[int]]):
        R, G, D = p.rows, p.groups, p.head_dim
        if p.heads_k != 1:
            raise ValueError("the oracle covers N2 == 1 only")
        self.rows = np.arange(R, dtype=np.int64) if rows is None else \
            np.ascontiguousarray(rows, dtype=np.int64)
        qf = p.q.reshape(R, G, D)
        if rows is not None:
            import torch
            qf = qf[torch.from_numpy(self.rows)]
        self.q = np.ascontiguousarray(qf.float().numpy())
        self.k = np.ascontiguousarray(p.k.reshape(-1, D).float().numpy())
        # None: the dense case (every key of the row's sequence)
        self.idx = None if p.sparse_indices is None else _c32(p.sparse_indices.reshape(R, p.topk))
        self.tlen = _c32(None if p.topk_length is None else p.topk_length.reshape(R))
        self.cu_q = _c32(p.cu_seqlens_q)
        self.cu_k = _c32(p.cu_seqlens_k)
        self.res = _c32(p.cmp_residual_k)
        self.su_q = _c32(getattr(p, "seqused_q", None))
        self.su_k = _c32(getattr(p, "seqused_k", None))
        self.layout = 0 if p.layout == "BSND" else 1
        self.dims = (self.layout, p.batch, p.seqlen_q, p.seqlen_k, G, D, p.topk,
                     p.mask_mode, p.cmp_ratio)
        self.scale = float(p.softmax_scale)

    def common(self):
        return [_ptr(self.k), _ptr(self.idx), _ptr(self.tlen), _ptr(self.cu_q),
                _ptr(self.cu_k), _ptr(self.res), _ptr(self.su_q), _ptr(self.su_k),
                *self.dims, self.scale,
                _ptr(self.rows), len(self.rows)]


def lse(p, rows: Optional[Sequence[int]] = None):
    """See :meth:`COracle.lse`."""
    return default().lse(p, rows)


def fill_lse(p):
    """See :meth:`COracle.fill_lse`."""
    return default().fill_lse(p)


def l1norm(p, rows: Optional[Sequence[int]] = None, softmax_lse=None):
    """See :meth:`COracle.l1norm`."""
    return default().l1norm(p, rows, softmax_lse)


def num_threads() -> int:
    """See :meth:`COracle.num_threads`."""
    return default().num_threads()
