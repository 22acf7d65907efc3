"""Matrices passed as row blocks (ns_orthogonalize_chunked) against the same
matrices passed whole: the row-block call must give the bits of the whole
matrix's result, block by block, for ragged and padded splits, empty blocks,
blocks not aligned to 16 bytes, both dtypes, both size classes and steps = 0.
The whole-matrix results are themselves checked against the oracle elsewhere;
here one case per class is also compared with the oracle directly."""
import numpy as np
import pytest
import torch

import newton_schulz_04_amd as ns
from newton_schulz_04_amd import workloads
from nsutil import TOL, oracle_run, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ns.lib()


def _blocks(g, rows, offset=0):
    """Copies of g's row blocks in one device buffer, block k starting
    `offset` elements after the previous block's end (offset 1 makes every
    block 2 bytes off a 16-byte boundary for bf16)."""
    cols = g.shape[1]
    total = sum(rows) * cols + offset * (len(rows) + 1)
    buf = torch.zeros(total + 8, dtype=g.dtype, device="cuda")
    out, at, r0 = [], offset, 0
    for r in rows:
        b = buf[at:at + r * cols].view(r, cols)
        b.copy_(g[r0:r0 + r].cuda())
        out.append(b)
        at += r * cols + offset
        r0 += r
    return buf, out


def _check(g, rows, steps=5, offset=0):
    whole = g.cuda().contiguous()
    ns.orthogonalize([whole], steps=steps)
    _, blocks = _blocks(g, rows, offset)
    ns.orthogonalize_chunked([blocks], steps=steps)
    torch.cuda.synchronize()
    got = torch.cat([b for b in blocks], dim=0)
    iv = torch.int16 if g.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(got.view(iv), whole.view(iv))
    return got.cpu()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape,rows", [
    ((2100, 700), [700, 0, 650, 750]),           # tall: transposed path, ragged, an empty shard
    ((300, 1000), [100, 100, 100]),              # wide: equal blocks
    ((520, 300), [1, 255, 0, 264]),              # a one-row block
    ((24, 300), [10, 0, 14]),                    # small path
])
def test_blocks_match_whole_matrix(dtype, shape, rows):
    g = workloads.gaussian(shape, seed=31, index=shape[0], dtype=dtype)
    y = _check(g, rows)
    if rows == [700, 0, 650, 750] or rows == [10, 0, 14]:
        assert rel_err(y, oracle_run(g)) <= TOL[dtype]


@pytest.mark.parametrize("shape,rows", [((2100, 700), [700, 650, 750]), ((300, 1000), [150, 150]),
                                        ((24, 300), [12, 12])])
def test_blocks_off_16_byte_boundaries(shape, rows):
    g = workloads.gaussian(shape, seed=32, index=shape[1])
    _check(g, rows, offset=1)


def test_blocks_steps_zero():
    g = workloads.gaussian((520, 300), seed=33)
    _check(g, [200, 0, 320], steps=0)


def test_attention_gate_shards():
    # an 18 x 2304 gate split over 8 ranks as (3,3,3,3,3,3,0,0): ragged, and
    # padded to 3 rows per shard (the last two shards all zero)
    g = workloads.attn_gate_raw(0)
    y = _check(g, [3, 3, 3, 3, 3, 3, 0, 0])
    assert rel_err(y, oracle_run(g)) <= TOL[torch.bfloat16]
    padded = torch.cat([g, torch.zeros(6, 2304, dtype=g.dtype)], dim=0)
    yp = _check(padded, [3] * 8)
    assert not bool(yp[18:].view(torch.int16).any())
    assert torch.equal(yp[:18].view(torch.int16), y.view(torch.int16))


def test_batch_of_chunked_matrices():
    # several matrices with different block layouts in one call
    gs = [workloads.gaussian(s, seed=35, index=i) for i, s in enumerate([(300, 520), (2100, 700), (24, 300)])]
    layouts = [[100, 200], [1000, 0, 1100], [24]]
    wholes = [g.cuda().contiguous() for g in gs]
    ns.orthogonalize(wholes)
    bufs, blocks = zip(*[_blocks(g, r) for g, r in zip(gs, layouts)])
    ns.orthogonalize_chunked(list(blocks))
    torch.cuda.synchronize()
    for w, bl in zip(wholes, blocks):
        assert torch.equal(torch.cat(list(bl)).view(torch.int16), w.view(torch.int16))
