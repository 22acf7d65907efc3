"""ns_orthogonalize_batched_noalloc (for callers that cannot allocate)
against ns_orthogonalize_batched through the C ABI: the same bits, on two
calls in a row, the second with a smaller batch, for both dtypes; a batch
that does not fit the static scratch array is rejected before anything is
enqueued; the call captured into a HIP graph replays with the eager bits."""
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


def _both(mats):
    """Results of the allocating and of the no-allocation entry point."""
    a = [m.cuda() for m in mats]
    b = [m.cuda() for m in mats]
    ns.orthogonalize(a)
    torch.cuda.synchronize()
    ns.orthogonalize(b, noalloc=True)
    torch.cuda.synchronize()
    return a, b


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_the_allocating_call(dtype):
    # first call: attention-gate-sized small matrices, tiled matrices of both
    # orientations and one with 2048 rows (36 symmetric tiles); second call: a
    # smaller batch, so the scratch array still holds the first call's data
    first = [workloads.gaussian((24, 2304), seed=81, index=i, dtype=dtype, scale=0.02) for i in range(8)]
    first += [workloads.gaussian(s, seed=82, index=i, dtype=dtype)
              for i, s in enumerate([(300, 520), (520, 300), (2048, 1536), (0, 9)])]
    second = [workloads.gaussian(s, seed=83, index=i, dtype=dtype) for i, s in enumerate([(40, 70), (17, 300)])]
    for batch in (first, second):
        a, b = _both(batch)
        for x, y in zip(a, b):
            assert torch.equal(_bits(x), _bits(y))
        k = max(range(len(batch)), key=lambda i: batch[i].numel())
        assert rel_err(b[k].cpu(), oracle_run(batch[k])) <= TOL[dtype]


def test_noalloc_rejects_a_batch_larger_than_the_scratch():
    g = workloads.gaussian((8192, 6144), seed=84).cuda()
    before = g.clone()
    need = ns.workspace_bytes([(8192, 6144)], ns.NS_BF16)
    assert need + 256 > ns.NOALLOC_SCRATCH_BYTES
    rc = ns.orthogonalize_raw([g.data_ptr()], [(8192, 6144)], 5, ns.QUINTIC, ns.NS_BF16,
                              torch.cuda.current_stream().cuda_stream, noalloc=True)
    assert rc == 1 and "no-allocation" in ns.last_error()
    torch.cuda.synchronize()
    assert torch.equal(_bits(g), _bits(before))
    # and a batch that fits still runs after the rejection
    a, b = _both([workloads.gaussian((300, 520), seed=85)])
    assert torch.equal(_bits(a[0]), _bits(b[0]))


def test_noalloc_under_hip_graph_capture():
    # What the entry point is for: captured into a HIP graph (its launches
    # are kernels only: no allocation, no memset, no copy), then replayed on
    # fresh inputs, with eager work that uses the same scratch array and
    # synchronizations between the replays; every replay gives the eager
    # call's bits
    shapes = [(24, 2304), (300, 520), (520, 300)]
    pristine = [workloads.gaussian(s, seed=86, index=i).cuda() for i, s in enumerate(shapes)]
    eager = [p.clone() for p in pristine]
    ns.orthogonalize(eager, noalloc=True)   # (also looks the scratch address up, before any capture)
    torch.cuda.synchronize()
    bufs = [p.clone() for p in pristine]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ns.orthogonalize(bufs, noalloc=True)
    torch.cuda.synchronize()
    for rep in range(3):
        for b, p in zip(bufs, pristine):
            b.copy_(p)
        other = [workloads.gaussian((40, 300), seed=87, index=rep).cuda()]
        ns.orthogonalize(other, noalloc=True)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for b, e in zip(bufs, eager):
            assert torch.equal(_bits(b), _bits(e)), rep
