"""CPU reference ("oracle") for distance-bound triangle smoothing.

TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the CPU-baseline
leg of the benchmark are the only callers.  The GPU library and its Python
binding never import this package, and this package imports nothing of
theirs; the two share only the seeded input generator.

`oracle.c` holds the arithmetic (one Floyd-Warshall round per intermediate
atom, upper bounds before lower bounds, front/back buffers, fp32, with
round-to-nearest or with sums rounded up and differences rounded down), following
GPU Gems 2, Ch. 43 "GPU Computing for Protein Structure Prediction" (study
notes), §2-§4 and §6.  `check.py` holds the plain definitions of the input
checks the library's validator reports.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
SO = os.path.join(HERE, "libdbs_oracle.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc (plain -O2, OpenMP, no fast-math; the
    rounding mode is honoured, -frounding-math)."""
    tmp = SO + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", "-frounding-math", SRC, "-lm", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, SO)
    return SO


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(SO):
            build()
        lib = ctypes.CDLL(SO)
        f32p = ctypes.POINTER(ctypes.c_float)
        i64 = ctypes.c_int64
        lib.dbs_oracle_rounds.argtypes = [f32p, f32p, i64, i64, i64, i64, ctypes.c_int]
        lib.dbs_oracle_rounds.restype = ctypes.c_int
        lib.dbs_oracle_rounds_directed.argtypes = [f32p, f32p, i64, i64, i64, i64,
                                                   ctypes.c_int]
        lib.dbs_oracle_rounds_directed.restype = ctypes.c_int
        lib.dbs_oracle_smooth.argtypes = [f32p, f32p, i64, i64, ctypes.c_int]
        lib.dbs_oracle_smooth.restype = ctypes.c_int
        lib.dbs_oracle_max_threads.restype = ctypes.c_int
        lib.dbs_oracle_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def _prep(U, L):
    U = np.array(U, dtype=np.float32, copy=True, order="C")
    L = np.array(L, dtype=np.float32, copy=True, order="C")
    if U.shape != L.shape or U.ndim not in (2, 3) or U.shape[-1] != U.shape[-2]:
        raise ValueError(f"bad shapes {U.shape} {L.shape}")
    n = U.shape[-1]
    batch = 1 if U.ndim == 2 else U.shape[0]
    return U, L, n, batch


def rounds(U, L, k_begin: int, k_end: int, threads: int = 0):
    """Rounds k_begin..k_end-1 of a pass; returns new (U, L) float32 arrays."""
    U, L, n, batch = _prep(U, L)
    f32p = ctypes.POINTER(ctypes.c_float)
    rc = load().dbs_oracle_rounds(U.ctypes.data_as(f32p), L.ctypes.data_as(f32p),
                                  n, batch, k_begin, k_end, threads)
    if rc != 0:
        raise ValueError(f"dbs_oracle_rounds failed ({rc})")
    return U, L


def smooth(U, L, threads: int = 0):
    """One full pass (every intermediate atom); returns new (U, L)."""
    U, L, n, batch = _prep(U, L)
    return rounds(U, L, 0, n, threads)


def rounds_directed(U, L, k_begin: int, k_end: int, threads: int = 0):
    """rounds() with upper-bound sums rounded toward +inf and lower-bound
    differences toward -inf; returns new (U, L) float32 arrays."""
    U, L, n, batch = _prep(U, L)
    f32p = ctypes.POINTER(ctypes.c_float)
    rc = load().dbs_oracle_rounds_directed(U.ctypes.data_as(f32p), L.ctypes.data_as(f32p),
                                           n, batch, k_begin, k_end, threads)
    if rc != 0:
        raise ValueError(f"dbs_oracle_rounds_directed failed ({rc})")
    return U, L


def smooth_directed(U, L, threads: int = 0):
    """A full pass with directed rounding; returns new (U, L)."""
    U, L, n, batch = _prep(U, L)
    return rounds_directed(U, L, 0, n, threads)


def max_threads() -> int:
    return int(load().dbs_oracle_max_threads())
