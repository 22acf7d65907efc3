"""Python face of the fp64 CPU oracle (oracle/ns_oracle.c).

TEST INFRASTRUCTURE: only tests/, the package smoke check and bench.py's
cpu_baseline leg import this module. It imports nothing from the GPU package.

The oracle is Muon's quintic Newton-Schulz iteration written out in plain
loops (see the header of ns_oracle.c for the definition and its sources).
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libns_oracle.so")

# Muon's quintic coefficients. The GPU library receives them as fp32, so the
# oracle iterates the same polynomial: the fp32 values widened to fp64.
QUINTIC = tuple(float(np.float32(v)) for v in (3.4445, -4.7750, 2.0315))
EPS = 1e-7

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python oracle/build.py`")
        _lib = ctypes.CDLL(LIB_PATH)
        d = ctypes.POINTER(ctypes.c_double)
        _lib.ns_oracle_f64_sched.argtypes = [
            d, d, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, d,
            ctypes.c_int32, ctypes.c_double]
        _lib.ns_oracle_f64_sched.restype = ctypes.c_int
        _lib.ns_oracle_frobenius.argtypes = [d, ctypes.c_int64, ctypes.c_int64]
        _lib.ns_oracle_frobenius.restype = ctypes.c_double
    return _lib


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def frobenius(g) -> float:
    g = np.ascontiguousarray(g, dtype=np.float64)
    if g.ndim != 2:
        raise ValueError("expected a 2-D matrix")
    return float(lib().ns_oracle_frobenius(_dptr(g), g.shape[0], g.shape[1]))


def newton_schulz(g, steps: int = 5, coeffs=QUINTIC, eps: float = EPS) -> np.ndarray:
    """Newton-Schulz orthogonalization of one matrix in fp64.

    g       2-D array of any real dtype; converted exactly to float64.
    steps   iteration count.
    coeffs  (a, b, c) used at every step, or a (steps, 3) array giving one
            triple per step.
    eps     added to ||G||_F before the division.
    Returns a new float64 array of g's shape.
    """
    g = np.ascontiguousarray(np.asarray(g, dtype=np.float64))
    if g.ndim != 2:
        raise ValueError("expected a 2-D matrix")
    cf = np.ascontiguousarray(np.asarray(coeffs, dtype=np.float64))
    per_step = 1 if cf.ndim == 2 else 0
    if per_step and cf.shape != (steps, 3):
        raise ValueError("per-step coefficients must have shape (steps, 3)")
    if not per_step and cf.shape != (3,):
        raise ValueError("coeffs must hold (a, b, c)")
    out = np.zeros_like(g)
    if g.size == 0:
        return out
    rc = lib().ns_oracle_f64_sched(_dptr(g), _dptr(out), g.shape[0], g.shape[1],
                                   int(steps), _dptr(cf), per_step, float(eps))
    if rc != 0:
        raise RuntimeError(f"ns_oracle_f64_sched failed with status {rc}")
    return out
