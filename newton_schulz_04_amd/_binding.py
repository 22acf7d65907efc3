"""ctypes binding of libns.so (include/ns.h): argument marshalling only.

Every step of the orthogonalization runs in the library's HIP kernels. The
library is loaded on first use; if it has not been built the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libns.so")

NS_BF16, NS_FP32 = 0, 1
# device scratch of ns_orthogonalize_batched_noalloc (NS_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 256 << 20
STATUS = {0: "NS_OK", 1: "NS_EINVAL", 2: "NS_EDTYPE", 3: "NS_ENOMEM", 4: "NS_EHIP"}
QUINTIC = (3.4445, -4.7750, 2.0315)
PROFILE_KINDS = ("norm_partial", "norm_final", "prep", "syrk", "poly", "update",
                 "small", "scale_out")

_lib: Optional[ctypes.CDLL] = None


class NSError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import "
                           "__graft_entry__ as g; g.build()'` or "
                           "`python newton_schulz_04_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    L.ns_orthogonalize_batched.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(i64), i32, i32,
                                           ctypes.POINTER(ctypes.c_float), i32, vp]
    L.ns_orthogonalize_batched.restype = ctypes.c_int
    L.ns_orthogonalize_batched_sched.argtypes = L.ns_orthogonalize_batched.argtypes
    L.ns_orthogonalize_batched_sched.restype = ctypes.c_int
    L.ns_orthogonalize_batched_noalloc.argtypes = L.ns_orthogonalize_batched.argtypes
    L.ns_orthogonalize_batched_noalloc.restype = ctypes.c_int
    L.ns_orthogonalize_chunked.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(i64), ctypes.POINTER(i32),
                                           ctypes.POINTER(i64), i32, i32, ctypes.POINTER(ctypes.c_float),
                                           i32, vp]
    L.ns_orthogonalize_chunked.restype = ctypes.c_int
    L.ns_plan_ranks.argtypes = [ctypes.POINTER(i64), ctypes.POINTER(i64), i32, i32, i64, i64, i32, i32,
                                ctypes.POINTER(i32), ctypes.POINTER(i64), ctypes.POINTER(i32),
                                ctypes.POINTER(i64), ctypes.POINTER(i32), ctypes.POINTER(i64)]
    L.ns_plan_ranks.restype = ctypes.c_int
    L.ns_workspace_bytes.argtypes = [ctypes.POINTER(i64), i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.ns_workspace_bytes.restype = ctypes.c_int
    L.ns_release_workspace.argtypes = [vp]
    L.ns_release_workspace.restype = ctypes.c_int
    L.ns_last_error.argtypes = []
    L.ns_last_error.restype = ctypes.c_char_p
    L.ns_version.argtypes = []
    L.ns_version.restype = ctypes.c_char_p
    L.ns_compute_cost.argtypes = [i64, i64]
    L.ns_compute_cost.restype = i64
    L.ns_plan_classify.argtypes = [ctypes.POINTER(i64), i32, i32, ctypes.POINTER(i32)]
    L.ns_plan_classify.restype = ctypes.c_int
    L.ns_plan_tiles.argtypes = [ctypes.POINTER(i64), i32, i32, i32, ctypes.POINTER(i32), i64,
                                ctypes.POINTER(i64), ctypes.POINTER(i32)]
    L.ns_plan_tiles.restype = ctypes.c_int
    L.ns_profile_enable.argtypes = [i32]
    L.ns_profile_enable.restype = ctypes.c_int
    L.ns_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64), i32]
    L.ns_profile_read.restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int):
    if rc != 0:
        raise NSError(rc, lib().ns_last_error().decode())


def _shapes_array(shapes: Sequence[Sequence[int]]):
    flat = [int(v) for s in shapes for v in s]
    return (ctypes.c_int64 * max(1, len(flat)))(*flat)


def last_error() -> str:
    return lib().ns_last_error().decode()


def version() -> str:
    return lib().ns_version().decode()


def compute_cost(rows: int, cols: int) -> int:
    return int(lib().ns_compute_cost(rows, cols))


def _is_schedule(coeffs) -> bool:
    """True for a sequence of (a, b, c) triples, False for one triple."""
    if coeffs is None:
        return False
    first = list(coeffs)[0] if len(coeffs) else None
    return first is not None and hasattr(first, "__len__")


def orthogonalize_raw(ptrs, shapes, steps: int, coeffs, dtype: int, stream: int = 0,
                      count: Optional[int] = None, noalloc: bool = False) -> int:
    """Direct call of ns_orthogonalize_batched (one (a, b, c) triple), of
    ns_orthogonalize_batched_sched (a sequence of triples, one per step) or,
    with noalloc, of ns_orthogonalize_batched_noalloc; returns the status
    code. `ptrs` are integers (device addresses; 0 = NULL), `shapes` (rows,
    cols) pairs; None for either passes NULL. For contract tests."""
    n = len(shapes) if count is None else count
    p = None if ptrs is None else (ctypes.c_void_p * max(1, len(ptrs)))(*[v or None for v in ptrs])
    s = None if shapes is None else _shapes_array(shapes)
    st = ctypes.c_void_p(stream or None)
    if _is_schedule(coeffs):
        flat = [float(v) for t in coeffs for v in t]
        c = (ctypes.c_float * max(1, len(flat)))(*flat)
        return int(lib().ns_orthogonalize_batched_sched(p, s, n, steps, c, dtype, st))
    c = None if coeffs is None else (ctypes.c_float * 3)(*coeffs)
    if noalloc:
        return int(lib().ns_orthogonalize_batched_noalloc(p, s, n, steps, c, dtype, st))
    return int(lib().ns_orthogonalize_batched(p, s, n, steps, c, dtype, st))


def orthogonalize(tensors, steps: int = 5, coeffs=QUINTIC, stream=None, noalloc: bool = False):
    """Orthogonalize a list of 2-D CUDA tensors (all bf16 or all fp32) in place
    on `stream` (default: the current stream). `coeffs` is one (a, b, c)
    triple for every step, or a sequence of `steps` triples (a schedule).
    noalloc: use ns_orthogonalize_batched_noalloc (one triple only; the batch
    must fit NS_NOALLOC_SCRATCH_BYTES). Returns the list."""
    import torch
    tensors = list(tensors)
    if not tensors:
        return tensors
    dt = tensors[0].dtype
    if dt == torch.bfloat16:
        code = NS_BF16
    elif dt == torch.float32:
        code = NS_FP32
    else:
        raise TypeError(f"unsupported dtype {dt}; use bfloat16 or float32")
    dev = tensors[0].device
    for t in tensors:
        if t.dim() != 2:
            raise ValueError("every matrix must be 2-D")
        if t.dtype != dt:
            raise TypeError("all matrices of a call must share one dtype")
        if t.device != dev or dev.type != "cuda":
            raise ValueError("all matrices must be on the same CUDA device")
        if t.numel() and not t.is_contiguous():
            raise ValueError("matrices must be contiguous (row-major)")
    ptrs = [t.data_ptr() if t.numel() else 0 for t in tensors]
    shapes = [tuple(t.shape) for t in tensors]
    with torch.cuda.device(dev):
        s = torch.cuda.current_stream() if stream is None else stream
        if _is_schedule(coeffs) and len(coeffs) != steps:
            raise ValueError("a coefficient schedule needs one (a, b, c) triple per step")
        if noalloc and _is_schedule(coeffs):
            raise ValueError("the no-allocation entry point takes one (a, b, c) triple")
        rc = orthogonalize_raw(ptrs, shapes, steps, coeffs, code, s.cuda_stream, noalloc=noalloc)
    _check(rc)
    return tensors


def orthogonalize_chunked_raw(chunk_ptrs, chunk_rows, nchunks, cols, steps: int, coeffs,
                              dtype: int, stream: int = 0) -> int:
    """Direct call of ns_orthogonalize_chunked; returns the status code.
    None for an array passes NULL. For contract tests."""
    def arr(ctype, vals):
        return None if vals is None else (ctype * max(1, len(vals)))(*vals)
    p = None if chunk_ptrs is None else (ctypes.c_void_p * max(1, len(chunk_ptrs)))(
        *[v or None for v in chunk_ptrs])
    c = None if coeffs is None else (ctypes.c_float * 3)(*coeffs)
    count = 0 if nchunks is None else len(nchunks)
    return int(lib().ns_orthogonalize_chunked(p, arr(ctypes.c_int64, chunk_rows), arr(ctypes.c_int32, nchunks),
                                              arr(ctypes.c_int64, cols), count, steps, c, dtype,
                                              ctypes.c_void_p(stream or None)))


def orthogonalize_chunked(matrices, steps: int = 5, coeffs=QUINTIC, stream=None):
    """Orthogonalize matrices given as lists of row blocks (2-D CUDA tensors
    with the matrix's column count, stacked top to bottom; blocks may have 0
    rows) in place: each matrix is treated as the concatenation of its
    blocks and the result lands back in them. Returns `matrices`."""
    import torch
    matrices = [list(m) for m in matrices]
    blocks = [b for m in matrices for b in m]
    if not blocks:
        return matrices
    dt = blocks[0].dtype
    if dt == torch.bfloat16:
        code = NS_BF16
    elif dt == torch.float32:
        code = NS_FP32
    else:
        raise TypeError(f"unsupported dtype {dt}; use bfloat16 or float32")
    dev = blocks[0].device
    cols = []
    for m in matrices:
        if not m:
            cols.append(0)
            continue
        c = m[0].shape[1] if m[0].dim() == 2 else -1
        for b in m:
            if b.dim() != 2 or b.shape[1] != c:
                raise ValueError("the blocks of a matrix must be 2-D with one column count")
            if b.dtype != dt or b.device != dev or dev.type != "cuda":
                raise ValueError("all blocks must share one dtype and CUDA device")
            if b.numel() and not b.is_contiguous():
                raise ValueError("blocks must be contiguous (row-major)")
        cols.append(c)
    ptrs = [b.data_ptr() if b.numel() else 0 for b in blocks]
    rows = [b.shape[0] for b in blocks]
    with torch.cuda.device(dev):
        s = torch.cuda.current_stream() if stream is None else stream
        rc = orthogonalize_chunked_raw(ptrs, rows, [len(m) for m in matrices], cols, steps, coeffs, code,
                                       s.cuda_stream)
    _check(rc)
    return matrices


def plan_ranks(numel, cost, world: int, bucket_size: int, align: int = 1, by_cost: bool = True,
               absorb: bool = True):
    """ns_plan_ranks: place parameters (numel, Newton-Schulz cost; backprop
    order) onto `world` ranks in buckets. Returns a dict with per-parameter
    `rank`, `offset`, `bucket`, per-bucket `bucket_elems` and per-rank
    `rank_cost`."""
    n = len(numel)
    if len(cost) != n:
        raise ValueError("numel and cost must have one entry per parameter")
    k = max(1, n)
    rank = (ctypes.c_int32 * k)()
    off = (ctypes.c_int64 * k)()
    bkt = (ctypes.c_int32 * k)()
    be = (ctypes.c_int64 * k)()
    nb = ctypes.c_int32(0)
    rc_ = (ctypes.c_int64 * max(1, world))()
    _check(lib().ns_plan_ranks((ctypes.c_int64 * k)(*numel), (ctypes.c_int64 * k)(*cost), n, world,
                               bucket_size, align, int(by_cost), int(absorb), rank, off, bkt, be,
                               ctypes.byref(nb), rc_))
    return {"rank": list(rank)[:n], "offset": list(off)[:n], "bucket": list(bkt)[:n],
            "bucket_elems": list(be)[:nb.value], "rank_cost": list(rc_)[:world]}


def workspace_bytes(shapes, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().ns_workspace_bytes(_shapes_array(shapes), len(shapes), dtype, ctypes.byref(out)))
    return int(out.value)


def release_workspace(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    _check(lib().ns_release_workspace(ctypes.c_void_p(s.cuda_stream or None)))


def plan_classify(shapes, dtype: int):
    kinds = (ctypes.c_int32 * max(1, len(shapes)))()
    _check(lib().ns_plan_classify(_shapes_array(shapes), len(shapes), dtype, kinds))
    return [int(kinds[i]) for i in range(len(shapes))]


def plan_tiles(shapes, dtype: int, stage: int):
    """Tile list of a GEMM stage in launch order: [(matrix, bi, bj, kdepth)]
    and the tile edge."""
    n = ctypes.c_int64(0)
    ts = ctypes.c_int32(0)
    _check(lib().ns_plan_tiles(_shapes_array(shapes), len(shapes), dtype, stage, None, 0,
                               ctypes.byref(n), ctypes.byref(ts)))
    buf = (ctypes.c_int32 * max(4, 4 * n.value))()
    _check(lib().ns_plan_tiles(_shapes_array(shapes), len(shapes), dtype, stage, buf, n.value,
                               ctypes.byref(n), ctypes.byref(ts)))
    return [tuple(buf[4 * i: 4 * i + 4]) for i in range(n.value)], ts.value


def profile_enable(on: bool):
    _check(lib().ns_profile_enable(1 if on else 0))


def profile_read():
    """{kind: (total_ms, launches)} since the last profile_enable(True)."""
    k = len(PROFILE_KINDS)
    ms = (ctypes.c_double * k)()
    cnt = (ctypes.c_int64 * k)()
    _check(lib().ns_profile_read(ms, cnt, k))
    return {name: (float(ms[i]), int(cnt[i])) for i, name in enumerate(PROFILE_KINDS)}
