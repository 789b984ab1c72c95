"""Dequantisation and the plain contraction (oracle).

Test infrastructure only: see the package docstring for who may use it.

[W01] paragraph on group-wise affine integer quantisation: a weight is
``w = (q - z) * s`` with ``s`` and ``z`` shared by the 128 consecutive
entries of one group along the reduction dimension, and the layer computes
``y = W x`` from those weights.  [W01] paragraph on the Hadamard transform:
the activations are rotated at run time with the same rotation that was
folded into the weights, so the layer computes ``y = W' (R x)``.
[W02] "Recipe": the tied embedding / output head is quantised without the
rotation, so its activations are used as they are.

The result is defined plainly: ``y[m][n] = sum_k What[n][k] * x'[m][k]`` with
``What`` the dequantised weight in fp64 and ``x'`` the explicitly rotated
activations in fp64.  The sum is a triple loop in C (``contract.c``).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .hadamard import rht

GROUP = 128
_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_contract.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ``contract.c`` with gcc into ``oracle/_contract.so``."""
    src = os.path.join(_HERE, "contract.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC",
                               "-shared", src, "-o", tmp])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.oracle_contract.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int]
        lib.oracle_contract.restype = None
        _lib = lib
    return _lib


def default_threads() -> int:
    return len(os.sched_getaffinity(0))


def contract(w_hat: np.ndarray, x: np.ndarray, threads: int | None = None) -> np.ndarray:
    """``y[m][n] = sum_k w_hat[n][k] * x[m][k]`` by the C triple loop, fp64."""
    w_hat = np.ascontiguousarray(w_hat, dtype=np.float64)
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float64)
    n, k = w_hat.shape
    m, k2 = x.shape
    if k != k2:
        raise ValueError("reduction sizes differ")
    y = np.empty((m, n), dtype=np.float64)
    _load().oracle_contract(w_hat.ctypes.data, x.ctypes.data, y.ctypes.data,
                            m, n, k, int(threads or default_threads()))
    return y


def dequant(q: np.ndarray, s: np.ndarray, z: np.ndarray, group: int = GROUP) -> np.ndarray:
    """``What[n][k] = (q[n][k] - z[n][k // group]) * s[n][k // group]`` in fp64."""
    q = np.asarray(q)
    n, k = q.shape
    gidx = np.arange(k) // group
    s64 = np.asarray(s, dtype=np.float16).astype(np.float64)[:, gidx]
    z64 = np.asarray(z, dtype=np.float16).astype(np.float64)[:, gidx]
    return (q.astype(np.float64) - z64) * s64


def linear(q, s, z, x, sign_bits=None, threads: int | None = None) -> np.ndarray:
    """The layer's output in fp64: rotate ``x`` (if signs are given), dequantise, contract."""
    x64 = np.atleast_2d(np.asarray(x)).astype(np.float64)
    xr = rht(x64, sign_bits) if sign_bits is not None else x64
    return contract(dequant(q, s, z), xr, threads)
