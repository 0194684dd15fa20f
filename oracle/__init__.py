"""CPU oracle for submanifold 3x3x3 sparse convolution (SubMConv3d).

TEST INFRASTRUCTURE ONLY.  Only `tests/`, `__graft_entry__.smoke()` and the
benchmark's CPU-baseline leg may import this package.  The product library
never imports, links or runs anything here, and this package imports nothing
from the product library.

Two independent implementations of the same definition:

* `reference` (O1): a Python dict of coordinates and float64 numpy matmuls.
* `dense` (O2): C code with a dense int32 index volume and double-precision
  loops, built with gcc by `build_oracle()` into `oracle/_lib/`.

Parity status: every function is pinned by CPU tests against brute force,
dense torch conv3d, closed forms, invariants and hand-worked examples
(tests/test_oracle_*.py, tests/golden/).  Three conventions are fixed here
where the pages are silent and are "parity unpinned" against the upstream
implementations, which no available artefact can settle:
  - the kernel orientation (correlation by default, `flip` for the mirror);
  - the channel layout inside a space-to-depth row (slot-major: slot s holds
    channels [s C, (s+1) C));
  - the order of the coarse rows of space-to-depth and downsample (ascending
    (b, z, y, x)).
Within each convention the functions are pinned as above.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import reference
from .reference import OracleError

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dense_oracle.c")
_LIBDIR = os.path.join(_HERE, "_lib")
_LIB = os.path.join(_LIBDIR, "libdense_oracle.so")
_lib = None


def build_oracle(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O3 -fopenmp, baseline x86-64 ISA)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    os.makedirs(_LIBDIR, exist_ok=True)
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                           "-o", tmp, _SRC])
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build_oracle()
        lib = ctypes.CDLL(_LIB)
        i32p = ctypes.POINTER(ctypes.c_int32)
        f64p = ctypes.POINTER(ctypes.c_double)
        lib.oracle_neighbors.argtypes = [i32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, i32p]
        lib.oracle_forward.argtypes = [f64p, f64p, f64p, i32p, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                       ctypes.c_int64, f64p]
        lib.oracle_subdivide.argtypes = [i32p, ctypes.c_int64, i32p]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int32]
        lib.oracle_set_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


_ERRORS = {-1: "invalid argument", -2: "coordinate out of range", -3: "duplicate coordinate",
           -6: "out of memory"}


def _check(rc):
    if rc != 0:
        raise OracleError(_ERRORS.get(rc, "error %d" % rc))


class dense:
    """O2: the C dense-volume oracle."""

    @staticmethod
    def neighbor_table(coords: np.ndarray, res: int, batch: int = None) -> np.ndarray:
        c = np.ascontiguousarray(coords, dtype=np.int32)
        if batch is None:
            batch = int(c[:, 0].max()) + 1 if len(c) else 1
        nbr = np.empty((len(c), 27), np.int32)
        _check(_load().oracle_neighbors(_ptr(c, ctypes.c_int32), len(c), res, batch,
                                        _ptr(nbr, ctypes.c_int32)))
        return nbr

    @staticmethod
    def forward(feats, weight, bias, nbr, flip=False, rows=None) -> np.ndarray:
        f = np.ascontiguousarray(feats, dtype=np.float64)
        w = np.ascontiguousarray(weight, dtype=np.float64)
        nb = np.ascontiguousarray(nbr, dtype=np.int32)
        n, cin = f.shape
        cout = w.shape[0]
        r0, r1 = (0, n) if rows is None else rows
        out = np.zeros((n, cout), np.float64)
        bp = None
        if bias is not None:
            b = np.ascontiguousarray(bias, dtype=np.float64)
            bp = _ptr(b, ctypes.c_double)
        _check(_load().oracle_forward(_ptr(f, ctypes.c_double), _ptr(w, ctypes.c_double), bp,
                                      _ptr(nb, ctypes.c_int32), n, cin, cout, int(bool(flip)),
                                      r0, r1, _ptr(out, ctypes.c_double)))
        return out

    @staticmethod
    def subdivide(coords: np.ndarray) -> np.ndarray:
        c = np.ascontiguousarray(coords, dtype=np.int32)
        out = np.empty((8 * len(c), 4), np.int32)
        _check(_load().oracle_subdivide(_ptr(c, ctypes.c_int32), len(c), _ptr(out, ctypes.c_int32)))
        return out

    @staticmethod
    def num_threads() -> int:
        return int(_load().oracle_num_threads())

    @staticmethod
    def set_threads(threads: int) -> None:
        """Threads of the parallel loops from now on (1 for the single-thread timing)."""
        _check(_load().oracle_set_threads(int(threads)))


__all__ = ["reference", "dense", "build_oracle", "OracleError"]
