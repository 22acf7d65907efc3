"""The library never waits for the device (microsoft/dion PR #74, "Fix
megabatch_orthogonalize_async hang on empty FSDP2 shards": the Concrete repro
is a host-side hang, and the review thread is about a hidden sync point).

With the stream kept busy by a large batch, many calls that each need a new
plan and a metadata upload (distinct pointer sets, so none hits the plan
cache) must each return at once, while the stream still has pending work."""
import time

import pytest
import torch

import newton_schulz_04_amd as ns
from newton_schulz_04_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ns.lib()


def test_calls_return_while_the_stream_is_busy():
    stream = torch.cuda.Stream()
    busy = [workloads.gaussian((8192, 6144), seed=71, index=i).cuda() for i in range(4)]
    calls = 24   # uploads in flight at once, beyond any small fixed staging pool
    smalls = [[workloads.gaussian((300, 520), seed=72, index=i).cuda(),
               workloads.gaussian((20, 700), seed=72, index=100 + i).cuda()] for i in range(calls)]
    with torch.cuda.stream(stream):
        # reference bits for every small batch, computed before the timed part
        ref = []
        for pair in smalls:
            c = [t.clone() for t in pair]
            ns.orthogonalize(c, stream=stream)
            ref.append(c)
        torch.cuda.synchronize()
        ns.release_workspace(stream)
        # refill the workspace at its large size, then queue about 100 ms
        # of work (5 calls over four 8192 x 6144 matrices)
        ns.orthogonalize(busy, stream=stream)
        torch.cuda.synchronize()
        for _ in range(5):
            ns.orthogonalize(busy, stream=stream)
        assert not stream.query(), "the busy batch finished before the test calls"
        host = []
        for pair in smalls:
            t0 = time.perf_counter()
            ns.orthogonalize(pair, stream=stream)
            host.append(time.perf_counter() - t0)
        pending = not stream.query()
    stream.synchronize()
    print(f"host ms per call: max {1e3 * max(host):.2f}, mean {1e3 * sum(host) / len(host):.2f}", flush=True)
    assert pending, "the stream drained during the calls: some call waited for the device"
    assert max(host) < 0.025, f"a call took {max(host) * 1e3:.1f} ms of host time"
    for got, want in zip(smalls, ref):
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ns.release_workspace(stream)
