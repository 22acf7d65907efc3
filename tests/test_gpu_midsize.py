"""GPU parity at sizes that reach every kernel path the full-size workloads
take, against the live fp64 oracle, element by element.

Paths that only batches of more than 256 tiles or 2048-multiple shapes reach:
  * the half tiles of a symmetric stage's split last round
    (k_gemm<0, 0|1, 0, 1>): a stage of n > 256 tiles whose last round holds
    r = n mod 256 <= 128 tiles runs those as 2r half tiles after the whole
    ones, in the same launch;
  * tile lists of more than one round (n > 256) in every stage;
  * padded row pitches: an operand row of 4096 bytes times an odd number
    gets 128 bytes of padding (bf16 m = 2048, 6144, 10240; fp32 rows of
    1024, 3072 elements);
  * the last update step writing a wide (rows <= cols, restaged by rows) and
    a tall (rows > cols) caller matrix.
The zero-padding cases of the workloads (dion PR #74, Fix: shards padded with
zero rows) and the 8192x6144 remainder matrices (xtuner PR #2069) run these
same paths at full size; here the oracle runs on the whole result."""
import numpy as np
import pytest
import torch

import newton_schulz_04_amd as ns
from newton_schulz_04_amd import workloads
from nsutil import TOL, gpu_run, oracle_run, rel_err, zero_bits

pytestmark = pytest.mark.gpu

TILE_ROUND = 256   # compute units of the device the tile lists are cut for


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ns.lib()


def _tail(shapes, dtype, stage):
    """Matrix indices owning the half tiles of a symmetric stage, and r."""
    tiles, edge = ns.plan_tiles(shapes, dtype, stage)
    n = len(tiles)
    r = n % TILE_ROUND
    assert edge == 256
    if n <= TILE_ROUND or r == 0 or r > TILE_ROUND // 2:
        return set(), 0
    tail = tiles[n - r:]
    assert all(t[1] != t[2] for t in tail), "a diagonal tile in the split round"
    return {t[0] for t in tail}, r


def test_midsize_bf16_batch_reaches_full_size_paths():
    # 8 matrices with m = 2048 (A, B, X_lo rows of 4096 bytes: padded pitch),
    # n = 2304: 36 upper tiles each, 288 per symmetric launch (one full round
    # and a split tail of 32), 72 update tiles each (576, three rounds);
    # alternately wide and tall
    shapes = [(2048, 2304) if i % 2 == 0 else (2304, 2048) for i in range(8)]
    for stage in (0, 1):
        owners, r = _tail(shapes, ns.NS_BF16, stage)
        assert r == 32 and owners, (stage, r)
    owners = sorted(_tail(shapes, ns.NS_BF16, 0)[0] | _tail(shapes, ns.NS_BF16, 1)[0])
    assert len(ns.plan_tiles(shapes, ns.NS_BF16, 2)[0]) == 576
    gs = [workloads.gaussian(s, seed=61, index=i) for i, s in enumerate(shapes)]
    ys = gpu_run(gs)
    for y in ys:
        assert bool(torch.isfinite(y.float()).all())
    # the oracle on the matrices that own half tiles, plus one of the other
    # orientation
    check = owners[:2]
    if not any(shapes[i][0] > shapes[i][1] for i in check):
        check.append(next(i for i in range(8) if shapes[i][0] > shapes[i][1]))
    if not any(shapes[i][0] < shapes[i][1] for i in check):
        check.append(next(i for i in range(8) if shapes[i][0] < shapes[i][1]))
    for i in check:
        ref = oracle_run(gs[i])
        e = rel_err(ys[i], ref)
        print(f"matrix {i} {shapes[i]}: rel err {e:.3e} (half-tile owner: {i in owners})", flush=True)
        assert e <= TOL[torch.bfloat16], (i, e)
        # every 256 x 256 output block on its own
        y = ys[i].float().numpy().astype(np.float64)
        for r0 in range(0, y.shape[0], 256):
            for c0 in range(0, y.shape[1], 256):
                blk = ref[r0:r0 + 256, c0:c0 + 256]
                eb = np.linalg.norm(y[r0:r0 + 256, c0:c0 + 256] - blk) / np.linalg.norm(blk)
                assert eb <= TOL[torch.bfloat16], (i, r0, c0, eb)
    # alone (36 whole tiles, no split) the owners give the same bits
    for i in owners:
        (alone,) = gpu_run([gs[i]])
        assert torch.equal(alone.view(torch.int16), ys[i].view(torch.int16)), i


def test_midsize_fp32_batch_padded_pitch_and_rounds():
    # fp32: A, B and X^T rows of 1024 floats (4096 bytes: padded pitch);
    # 24 update tiles per matrix, 288 per launch (two rounds)
    shapes = [(1024, 1536) if i % 3 else (1536, 1024) for i in range(12)]
    assert len(ns.plan_tiles(shapes, ns.NS_FP32, 2)[0]) == 288
    gs = [workloads.gaussian(s, seed=62, index=i, dtype=torch.float32) for i, s in enumerate(shapes)]
    ys = gpu_run(gs)
    upd, _ = ns.plan_tiles(shapes, ns.NS_FP32, 2)
    # the matrices of the first and of the last tile of the update launch,
    # and one of each orientation
    check = sorted({upd[0][0], upd[-1][0], 0, 1})
    for i in check:
        e = rel_err(ys[i], oracle_run(gs[i]))
        print(f"fp32 matrix {i} {shapes[i]}: rel err {e:.3e}", flush=True)
        assert e <= TOL[torch.float32], (i, e)


@pytest.mark.parametrize("shape", [(300, 1024), (1024, 300), (1024, 1024)])
def test_fp32_padded_pitch(shape):
    # rows of X (fp32 path: 1024 floats) at the padded pitch
    g = workloads.gaussian(shape, seed=63, index=shape[0], dtype=torch.float32)
    (y,) = gpu_run([g])
    e = rel_err(y, oracle_run(g))
    assert e <= TOL[torch.float32], e


def test_tiny_fp32_padding_is_bitwise():
    # the tiny batch's matrix 3 has rows 56..63 zero: its real rows equal,
    # bit for bit, the result for the 56 x 32 matrix without them
    cases = workloads.tiny_fp32()
    out = gpu_run([c.mat for c in cases])
    (cut,) = gpu_run([cases[3].mat[:56].contiguous()])
    assert zero_bits(out[3][56:])
    assert torch.equal(out[3][:56].view(torch.int32), cut.view(torch.int32))
    assert rel_err(cut, oracle_run(cases[3].mat[:56])) <= TOL[torch.float32]


# Huge entries: the norm's squares would overflow fp32 (entries above about
# 1.8e19); every finite input still normalizes like the fp64 oracle.
NORM_CASES = [
    ("bf16 tiled, one 1e20 entry", torch.bfloat16, (300, 520), "one", 1e20),
    ("bf16 small, one 1e20 entry", torch.bfloat16, (24, 300), "one", 1e20),
    ("bf16 tiled, one row of 1e30", torch.bfloat16, (520, 300), "row", 1e30),
    ("bf16 tiled, all entries x 1e35", torch.bfloat16, (257, 300), "all", 1e35),
    ("fp32 tiled, all entries x 1e30", torch.float32, (257, 300), "all", 1e30),
    ("fp32 tiled, entries near FLT_MAX", torch.float32, (300, 520), "all", 5e37),
    ("fp32 small, all entries x 1e30", torch.float32, (20, 400), "all", 1e30),
]


@pytest.mark.parametrize("name,dtype,shape,how,big", NORM_CASES, ids=[c[0] for c in NORM_CASES])
def test_huge_entries_normalize_like_the_oracle(name, dtype, shape, how, big):
    g = workloads.gaussian(shape, seed=64, index=shape[0], dtype=torch.float32)
    if how == "one":
        g[5, 7] = big
    elif how == "row":
        g[3] = g[3] * big
    else:
        g = g * big
    g = g.to(dtype)
    assert bool(torch.isfinite(g.float()).all())
    (y,) = gpu_run([g])
    ref = oracle_run(g)
    assert np.isfinite(ref).all()
    e = rel_err(y, ref)
    assert e <= TOL[dtype], (name, e)


def test_norm_scaling_keeps_ordinary_inputs_bitwise():
    # entries below 2^40 are summed unscaled: a matrix and the same matrix
    # with one entry raised to 2^39 and back give the bits of a plain run
    g = workloads.gaussian((300, 520), seed=65)
    (a,) = gpu_run([g])
    (b,) = gpu_run([g.clone()])
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    h = g.clone()
    h[0, 0] = 2.0 ** 39
    (y,) = gpu_run([h])
    assert rel_err(y, oracle_run(h)) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("shape", [(20, 300), (300, 20), (40, 300)])
def test_more_steps_than_a_schedule_holds(shape):
    # the plain call takes any step count (a schedule holds at most 64):
    # 70 cubic steps converge to the polar factor on both size classes
    g = workloads.gaussian(shape, seed=66, index=shape[0], dtype=torch.float32)
    cubic = (1.5, -0.5, 0.0)
    (y,) = gpu_run([g], steps=70, coeffs=cubic)
    assert rel_err(y, oracle_run(g, steps=70, coeffs=cubic)) <= TOL[torch.float32]
    u, _, vt = np.linalg.svd(g.double().numpy(), full_matrices=False)
    assert rel_err(y, u @ vt) <= TOL[torch.float32]


@pytest.mark.parametrize("dtype,shape", [(torch.bfloat16, (8, 200000)), (torch.float32, (150000, 20))])
def test_small_path_wide_slices(dtype, shape):
    # n > 131072: a small matrix's columns go into slices of 1024 (at most
    # 256 slices), each workgroup looping over several 512- and 256-column
    # chunks; against the oracle, and bitwise the same inside a batch
    g = workloads.gaussian(shape, seed=67, index=shape[0], dtype=dtype)
    (y,) = gpu_run([g])
    assert rel_err(y, oracle_run(g)) <= TOL[dtype]
    other = workloads.gaussian((16, 300), seed=67, index=1, dtype=dtype)
    y2, _ = gpu_run([g, other])
    iv = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(y.view(iv), y2.view(iv))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_small_threshold_and_check_mode_from_environment(monkeypatch, dtype):
    # the same 24 x 300 matrix on the small path (default) and, with
    # NS_SMALL_M=8, on the tiled path: both against the oracle; NS_CHECK=1
    # (wait and check after every launch) gives the same bits
    g = workloads.gaussian((24, 300), seed=68, dtype=dtype)
    ref = oracle_run(g)
    monkeypatch.delenv("NS_SMALL_M", raising=False)
    monkeypatch.delenv("NS_CHECK", raising=False)
    (small,) = gpu_run([g])
    monkeypatch.setenv("NS_SMALL_M", "8")
    (tiled,) = gpu_run([g])
    monkeypatch.setenv("NS_CHECK", "1")
    (checked,) = gpu_run([g])
    assert rel_err(small, ref) <= TOL[dtype] and rel_err(tiled, ref) <= TOL[dtype]
    iv = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(tiled.view(iv), checked.view(iv))


@pytest.mark.parametrize("steps", [5, 8])
def test_fp32_exactly_low_rank_error_is_that_of_plain_fp32(steps):
    # An exactly rank-4 input: fp32 rounding noise in its null space grows by
    # about a = 3.4445 per step (a^5 ~ 485, a^8 ~ 2e4), so an fp32
    # evaluation need not stay within 1e-4 of the fp64 oracle here. The tiled fp32
    # path must stay within a small factor of a plain fp32 evaluation of the
    # same iteration (numpy, fp32 products).
    gen = workloads.generator(90, steps)
    g = (torch.randn(856, 4, generator=gen) @ torch.randn(4, 535, generator=gen)).float()
    (y,) = gpu_run([g], steps=steps)
    ref = oracle_run(g, steps=steps)
    a, b, c = (np.float32(v) for v in ns.QUINTIC)
    x = g.numpy().T.copy()                       # 535 x 856: rows <= cols
    x = x / (np.float32(np.linalg.norm(x.astype(np.float64))) + np.float32(1e-7))
    for _ in range(steps):
        A = x @ x.T
        x = a * x + (b * A + c * (A @ A)) @ x
    plain = rel_err(torch.from_numpy(x.T.copy()), ref)
    e = rel_err(y, ref)
    print(f"steps {steps}: library fp32 {e:.2e}, plain fp32 {plain:.2e}", flush=True)
    assert e <= 5 * plain and e <= 1e-2, (e, plain)
