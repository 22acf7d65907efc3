"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
the same seeded inputs, at sizes the oracle finishes in seconds. Tolerance per
matrix, relative Frobenius error: 2e-2 for bf16, 1e-4 for fp32; zero rows,
zero columns and padding must come back as exact +0.0."""
import numpy as np
import pytest
import torch

import newton_schulz_04_amd as ns
from newton_schulz_04_amd import workloads
from nsutil import TOL, coeffs32, gpu_run, oracle_run, rel_err, zero_bits
from oracle import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ns.lib()


def test_tiny_fp32_workload():
    cases = workloads.tiny_fp32()
    out = gpu_run([c.mat for c in cases])
    for c, y in zip(cases, out):
        ref = oracle_run(c.mat)
        e = rel_err(y, ref)
        assert e <= TOL[torch.float32], e
    assert zero_bits(out[3][56:])
    assert out[3][:56].abs().min() > 0


def test_attn_gate_workload_padded():
    cases = workloads.attn_gate()
    out = gpu_run([c.mat for c in cases])
    raw_out = gpu_run([c.tags["raw"] for c in cases])
    for c, y, yr in zip(cases, out, raw_out):
        real = c.real_rows
        ref = oracle_run(c.tags["raw"])
        assert rel_err(y[real], ref) <= TOL[torch.bfloat16]
        assert zero_bits(y[~real])
        # zero-row padding leaves the real rows bitwise unchanged
        assert torch.equal(y[real].view(torch.int16), yr.view(torch.int16))


LARGE_SHAPES = [(300, 520), (520, 300), (256, 256), (33, 100), (100, 33), (257, 513),
                (513, 257), (64, 2000), (700, 1000), (1000, 700), (96, 96),
                # few rows, many columns: clustered singular values, where the
                # diagonals of A and B dominate and their rounding matters most
                (33, 1000), (1000, 33), (64, 2304)]


@pytest.mark.parametrize("shape", LARGE_SHAPES)
def test_large_bf16_vs_oracle(shape):
    g = workloads.gaussian(shape, seed=11, index=shape[0] * 7 + shape[1])
    (y,) = gpu_run([g])
    e = rel_err(y, oracle_run(g))
    assert e <= TOL[torch.bfloat16], e


CUBIC = (1.5, -0.5, 0.0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(300, 520), (24, 300)])
def test_constant_schedule_is_bitwise_the_plain_call(dtype, shape):
    g = workloads.gaussian(shape, seed=21, index=shape[0], dtype=dtype)
    (a,) = gpu_run([g], steps=5)
    (b,) = gpu_run([g], steps=5, coeffs=[ns.QUINTIC] * 5)
    iv = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(a.view(iv), b.view(iv))


@pytest.mark.parametrize("dtype,shape", [(torch.bfloat16, (300, 520)), (torch.bfloat16, (520, 300)),
                                         (torch.float32, (257, 300)), (torch.float32, (24, 300)),
                                         (torch.bfloat16, (24, 2304))])
def test_schedule_vs_oracle(dtype, shape):
    # three quintic steps, then cubic steps toward the polar factor
    sched = [ns.QUINTIC] * 3 + [CUBIC] * 4
    g = workloads.gaussian(shape, seed=22, index=shape[1], dtype=dtype)
    (y,) = gpu_run([g], steps=len(sched), coeffs=sched)
    ref = oracle.newton_schulz(g.float().numpy(), steps=len(sched),
                               coeffs=np.array([coeffs32(c) for c in sched]))
    e = rel_err(y, ref)
    assert e <= TOL[dtype], e


def test_fp32_schedule_reaches_polar_factor():
    # quintic steps move the spectrum into [0.68, 1.2], cubic steps then
    # converge to U V^T (a fixed point of the cubic map)
    g = workloads.gaussian((96, 160), seed=23, dtype=torch.float32)
    sched = [ns.QUINTIC] * 5 + [CUBIC] * 20
    (y,) = gpu_run([g], steps=len(sched), coeffs=sched)
    u, _, vt = np.linalg.svd(g.double().numpy(), full_matrices=False)
    assert rel_err(y, u @ vt) <= 1e-4


@pytest.mark.parametrize("rank,shape", [(16, (256, 1024)), (40, (600, 300)), (1, (96, 700))])
def test_low_rank_bf16_vs_oracle(rank, shape):
    # Exactly low-rank input: directions outside the row space grow by about
    # a per step from whatever rounding puts there, so X must be carried
    # between steps more precisely than one bf16 rounding.
    gen = torch.Generator().manual_seed(rank * 1000 + shape[0])
    left = torch.randn((shape[0], rank), generator=gen, dtype=torch.float64)
    right = torch.randn((rank, shape[1]), generator=gen, dtype=torch.float64)
    g = (left @ right).to(torch.bfloat16)
    (y,) = gpu_run([g])
    e = rel_err(y, oracle_run(g))
    assert e <= TOL[torch.bfloat16], e


@pytest.mark.parametrize("shape", [(300, 520), (520, 300), (64, 100), (257, 300), (40, 40),
                                   (64, 32), (17, 900)])
def test_fp32_vs_oracle(shape):
    g = workloads.gaussian(shape, seed=12, index=shape[0], dtype=torch.float32)
    (y,) = gpu_run([g])
    e = rel_err(y, oracle_run(g))
    assert e <= TOL[torch.float32], e


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(300, 520), (520, 300), (24, 300), (300, 24)])
def test_zero_rows_and_columns_exact(dtype, shape):
    g = workloads.gaussian(shape, seed=13, dtype=dtype)
    g[[0, 7, shape[0] - 1]] = 0
    g[:, [3, shape[1] - 1]] = 0
    (y,) = gpu_run([g])
    assert zero_bits(y[[0, 7, shape[0] - 1]])
    assert zero_bits(y[:, [3, shape[1] - 1]])
    assert rel_err(y, oracle_run(g)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_all_zero_matrices(dtype):
    mats = [torch.zeros(s, dtype=dtype) for s in [(300, 520), (24, 100), (1, 1)]]
    for y in gpu_run(mats):
        assert zero_bits(y)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("steps", [0, 1, 2, 3])
def test_step_counts(dtype, steps):
    mats = [workloads.gaussian(s, seed=14, index=i, dtype=dtype)
            for i, s in enumerate([(300, 520), (20, 70), (70, 20)])]
    out = gpu_run(mats, steps=steps)
    for g, y in zip(mats, out):
        assert rel_err(y, oracle_run(g, steps=steps)) <= TOL[dtype]


def test_cubic_fp32_reaches_polar_factor():
    g = workloads.gaussian((200, 300), seed=15, dtype=torch.float32)
    cubic = (1.5, -0.5, 0.0)
    (y,) = gpu_run([g], steps=30, coeffs=cubic)
    assert rel_err(y, oracle_run(g, steps=30, coeffs=cubic)) <= 1e-4
    u, _, vt = np.linalg.svd(g.double().numpy(), full_matrices=False)
    assert rel_err(y, u @ vt) <= 1e-4


def test_one_by_n_and_scalars():
    for shape in [(1, 1), (1, 257), (257, 1), (2, 3)]:
        for dtype in (torch.bfloat16, torch.float32):
            g = workloads.gaussian(shape, seed=16, dtype=dtype)
            (y,) = gpu_run([g])
            assert rel_err(y, oracle_run(g)) <= TOL[dtype]


def _mixed_batch(dtype):
    shapes = [(300, 520), (24, 2304), (0, 17), (520, 300), (64, 32), (33, 40), (9, 0), (256, 1000)]
    return [workloads.gaussian(s, seed=17, index=i, dtype=dtype) if 0 not in s
            else torch.zeros(s, dtype=dtype) for i, s in enumerate(shapes)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_batch_results_independent_of_batch(dtype):
    mats = _mixed_batch(dtype)
    together = gpu_run(mats)
    alone = [gpu_run([m])[0] for m in mats]
    perm = [3, 7, 0, 5, 1, 6, 2, 4]
    shuffled = gpu_run([mats[i] for i in perm])
    iv = torch.int16 if dtype == torch.bfloat16 else torch.int32
    for i, (a, b) in enumerate(zip(together, alone)):
        assert a.shape == mats[i].shape
        assert torch.equal(a.view(iv), b.view(iv)), i
    for k, i in enumerate(perm):
        assert torch.equal(shuffled[k].view(iv), together[i].view(iv)), i
    for g, y in zip(mats, together):
        if g.numel():
            assert rel_err(y, oracle_run(g)) <= TOL[dtype]


def test_repeated_calls_and_plan_cache():
    mats = [workloads.gaussian((300, 520), seed=18).cuda(), workloads.gaussian((24, 100), seed=19).cuda()]
    pristine = [m.clone() for m in mats]
    ns.orthogonalize(mats)
    first = [m.clone() for m in mats]
    for m, p in zip(mats, pristine):
        m.copy_(p)
    ns.orthogonalize(mats)                    # same pointers: cached plan
    for a, b in zip(mats, first):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    other = [workloads.gaussian((700, 300), seed=20).cuda()]
    ns.orthogonalize(other)                   # different plan in between
    for m, p in zip(mats, pristine):
        m.copy_(p)
    ns.orthogonalize(mats)
    for a, b in zip(mats, first):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_side_stream_matches_default_stream():
    g = workloads.gaussian((520, 300), seed=21).cuda()
    a, b = g.clone(), g.clone()
    ns.orthogonalize([a])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ns.orthogonalize([b], stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ns.release_workspace(s)


def test_contract_errors_leave_buffers_untouched():
    g = workloads.gaussian((300, 520), seed=22).cuda()
    before = g.clone()
    p = g.data_ptr()
    assert ns.orthogonalize_raw([p, p], [(300, 520), (-1, 3)], 5, ns.QUINTIC, ns.NS_BF16) == 1
    assert ns.orthogonalize_raw([p], [(300, 520)], 5, ns.QUINTIC, 5) == 2
    assert ns.orthogonalize_raw([p], [(300, 520)], -2, ns.QUINTIC, ns.NS_BF16) == 1
    assert ns.orthogonalize_raw([p], [(300, 520)], 5, None, ns.NS_BF16) == 1
    assert ns.orthogonalize_raw([p, 0], [(300, 520), (0, 4)], 0, None, ns.NS_BF16) == 0
    torch.cuda.synchronize()
    # the last call was valid (steps = 0): G / (||G|| + eps)
    ref = before.float() / (before.float().norm() + 1e-7)
    assert rel_err(g.cpu(), ref.cpu().double().numpy()) <= 1e-2
    canary = torch.full((64,), 7.0, device="cuda")
    assert ns.orthogonalize_raw([canary.data_ptr()], [(0, 64)], 5, ns.QUINTIC, ns.NS_FP32) == 0
    assert ns.orthogonalize_raw([], [], 5, ns.QUINTIC, ns.NS_FP32) == 0
    torch.cuda.synchronize()
    assert bool((canary == 7.0).all())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(32, 2304), (33, 2304), (2304, 32), (2304, 33)])
def test_small_large_boundary(dtype, shape):
    # m = 32 is the last small-path size, m = 33 the first tiled one
    g = workloads.gaussian(shape, seed=41, index=shape[0], dtype=dtype)
    (y,) = gpu_run([g])
    assert rel_err(y, oracle_run(g)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(24, 1024), (24, 1025), (1025, 24), (32, 796), (32, 797), (5, 2389),
                                   (5, 4000)])
def test_small_path_slices(dtype, shape):
    # The small-matrix kernel gives each 512-column slice of X its own
    # workgroup (its Gram piece in 256-column chunks) and sums the pieces in
    # slice order: two whole slices (24 x 1024), a last slice of one column
    # (24 x 1025 and its transpose), ragged last slices and chunks (32 x 796,
    # 32 x 797, 5 x 2389), eight slices (5 x 4000). Alone and in one batch,
    # against the oracle; a matrix's bits do not depend on the batch.
    g = workloads.gaussian(shape, seed=43, index=shape[0] * 7 + shape[1], dtype=dtype)
    (y,) = gpu_run([g])
    assert rel_err(y, oracle_run(g)) <= TOL[dtype]
    other = workloads.gaussian((16, 300), seed=43, index=1, dtype=dtype)
    y2, _ = gpu_run([g, other])
    assert torch.equal(y.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       y2.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))


@pytest.mark.parametrize("shape", [(520, 300), (300, 520)])
def test_unaligned_base_pointer(shape):
    # a matrix starting 2 bytes past a 16-byte boundary takes the element-wise
    # load paths and must give the bits of an aligned copy
    g = workloads.gaussian(shape, seed=42, index=shape[0])
    buf = torch.zeros(g.numel() + 16, dtype=g.dtype, device="cuda")
    view = buf[1:1 + g.numel()].view(shape)
    view.copy_(g.cuda())
    ref = g.cuda().contiguous()
    ns.orthogonalize([view, ref])
    torch.cuda.synchronize()
    assert torch.equal(view.view(torch.int16), ref.view(torch.int16))
    assert buf[0].item() == 0 and not bool(buf[1 + g.numel():].view(torch.int16).any())


@pytest.mark.parametrize("shape", [(24, 300), (300, 520)])
def test_nan_propagates(shape):
    # NaN and Inf are not checked: a NaN input element makes the norm, hence
    # every output element, NaN; the call itself completes normally
    g = workloads.gaussian(shape, seed=43)
    g[3, 5] = float("nan")
    (y,) = gpu_run([g])
    assert bool(torch.isnan(y.float()).all())


def test_many_small_matrices_one_call():
    shapes = [(r, c) for r in (1, 7, 18, 24, 32) for c in (32, 100, 2304)] * 20
    gs = [workloads.gaussian(s, seed=44, index=i) for i, s in enumerate(shapes)]
    ys = gpu_run(gs)
    for i in range(0, len(gs), 37):
        assert rel_err(ys[i], oracle_run(gs[i])) <= TOL[torch.bfloat16]
    # results do not depend on the batch
    for i in (0, 150, 299):
        (alone,) = gpu_run([gs[i]])
        assert torch.equal(alone.view(torch.int16), ys[i].view(torch.int16))
