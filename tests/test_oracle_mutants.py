"""How strong the oracle's pins are: a plausible mistake planted in a copy of
the oracle must fail at least one pin that the oracle itself passes.

Each mutant is oracle/ns_oracle.c with one textual change (a dropped term, a
wrong sign, a wrong index, a transposed or missing operand, eps in the wrong
place, a step too few, the wrong coefficient row), written to a temporary
directory and compiled with gcc. The committed oracle is never modified. The
pins applied are those of tests/test_oracle_pins.py in small form: the SVD
closed form U p^(k)(S / (||G||_F + eps)) V^T for wide, tall, square and 1xN
shapes and several step counts, eps at a norm where it is a 10% effect, and a
per-step coefficient schedule.

Mutations that cannot change the result are left out on purpose: the
orientation (Newton-Schulz commutes with transposition in exact arithmetic)
and reading A or B transposed in a product (both are symmetric)."""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "oracle", "ns_oracle.c")
QUINTIC = tuple(float(np.float32(v)) for v in (3.4445, -4.7750, 2.0315))

SCALE = "    const double scale = ns_oracle_frobenius(in, rows, cols) + eps;"
POLY = "            bm[e] = cb * a[e] + cc * aa[e];"
UPDATE = "            xn[e] = ca * x[e] + bx[e];"
MUTANTS = [
    ("sign of b", POLY, "            bm[e] = -cb * a[e] + cc * aa[e];"),
    ("c A^2 term dropped", POLY, "            bm[e] = cb * a[e];"),
    ("a X term dropped", UPDATE, "            xn[e] = bx[e];"),
    ("a X replaced by X", UPDATE, "            xn[e] = x[e] + bx[e];"),
    ("wrong row in X X^T", "        const double* xj = x + j * n;", "        const double* xj = x + i * n;"),
    ("A^2 replaced by A", "        matmul(a, a, m, m, m, aa);", "        memcpy(aa, a, sizeof(double) * m * m);"),
    ("eps added to the squared norm", SCALE,
     "    const double scale = sqrt(ns_oracle_frobenius(in, rows, cols) * ns_oracle_frobenius(in, rows, cols)"
     " + eps);"),
    ("eps dropped", SCALE, "    const double scale = ns_oracle_frobenius(in, rows, cols);"),
    ("norm without its square root", "    return sqrt(s);", "    return s;"),
    ("one step too few", "    for (int32_t t = 0; t < steps; ++t) {", "    for (int32_t t = 1; t < steps; ++t) {"),
    ("per-step coefficients from the wrong row", "coeffs + 3 * t", "coeffs + t"),
    ("tall input not transposed", "        transpose(in, rows, cols, x);",
     "        memcpy(x, in, sizeof(double) * m * n);"),
    ("tall result not transposed back", "        transpose(x, m, n, out);",
     "        memcpy(out, x, sizeof(double) * m * n);"),
]


def _compile(text, workdir, name):
    src = os.path.join(workdir, name + ".c")
    lib = os.path.join(workdir, name + ".so")
    with open(src, "w") as f:
        f.write(text)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off", src,
                    "-o", lib, "-lm"], check=True, capture_output=True)
    h = ctypes.CDLL(lib)
    d = ctypes.POINTER(ctypes.c_double)
    h.ns_oracle_f64_sched.argtypes = [d, d, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, d, ctypes.c_int32,
                                      ctypes.c_double]
    h.ns_oracle_f64_sched.restype = ctypes.c_int
    return h


def _run(h, g, steps, coeffs, eps=1e-7):
    g = np.ascontiguousarray(g, dtype=np.float64)
    cf = np.ascontiguousarray(np.asarray(coeffs, dtype=np.float64))
    out = np.zeros_like(g)
    d = ctypes.POINTER(ctypes.c_double)
    rc = h.ns_oracle_f64_sched(g.ctypes.data_as(d), out.ctypes.data_as(d), g.shape[0], g.shape[1], steps,
                               cf.ctypes.data_as(d), 1 if cf.ndim == 2 else 0, eps)
    assert rc == 0
    return out


def _closed_form(g, sched, eps=1e-7):
    u, s, vt = np.linalg.svd(g, full_matrices=False)
    x = s / (np.sqrt(np.sum(g * g)) + eps)
    for a, b, c in sched:
        x = a * x + b * x ** 3 + c * x ** 5
    return (u * x) @ vt


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _failed_pins(h):
    """Names of the pins the library at `h` fails."""
    failed = []
    rng = np.random.default_rng(2024)
    for shape in [(5, 9), (9, 5), (6, 6), (1, 7), (7, 1)]:
        g = rng.standard_normal(shape)
        for steps in (1, 3, 5):
            if _rel(_run(h, g, steps, QUINTIC), _closed_form(g, [QUINTIC] * steps)) > 1e-12:
                failed.append(f"closed form {shape} x {steps}")
    g = 1e-6 * rng.standard_normal((6, 9)) / 7.0   # eps = 1e-7 is a 10% effect here
    if _rel(_run(h, g, 5, QUINTIC), _closed_form(g, [QUINTIC] * 5)) > 1e-12:
        failed.append("eps at a tiny norm")
    sched = np.array([[3.4445, -4.7750, 2.0315], [2.0, -1.5, 0.5], [1.5, -0.5, 0.0]])
    g = rng.standard_normal((8, 11))
    if _rel(_run(h, g, 3, sched), _closed_form(g, sched)) > 1e-12:
        failed.append("per-step schedule")
    return failed


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    return str(tmp_path_factory.mktemp("oracle_mutants"))


@pytest.fixture(scope="module")
def source():
    with open(SOURCE) as f:
        return f.read()


def test_unmodified_copy_passes_every_pin(workdir, source):
    assert _failed_pins(_compile(source, workdir, "control")) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(workdir, source, name, old, new):
    assert source.count(old) == 1, f"mutation site not found once: {old!r}"
    h = _compile(source.replace(old, new), workdir, "m%d" % MUTANTS.index((name, old, new)))
    failed = _failed_pins(h)
    assert failed, f"the planted mistake '{name}' passes every pin"
