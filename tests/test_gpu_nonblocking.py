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


def test_host_threads_on_their_own_streams():
    # Entry points may be called from several host threads: four threads,
    # each with its own stream (so its own workspace and plan cache), run
    # mixed batches concurrently; every result equals the one-thread result
    import threading
    batches = []
    for t in range(4):
        shapes = [(300, 520), (24, 700), (520, 300 + 8 * t), (40, 2304)]
        batches.append([workloads.gaussian(s, seed=73, index=10 * t + i) for i, s in enumerate(shapes)])
    expect = []
    for b in batches:
        dev = [g.cuda() for g in b]
        ns.orthogonalize(dev)
        torch.cuda.synchronize()
        expect.append([d.cpu() for d in dev])
    results = [None] * 4
    errors = []

    def work(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                out = []
                for _ in range(3):
                    dev = [g.to("cuda", non_blocking=False) for g in batches[t]]
                    ns.orthogonalize(dev, stream=s)
                    out = dev
                s.synchronize()
                results[t] = [d.cpu() for d in out]
            ns.release_workspace(s)
        except Exception as e:  # reported below, in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    for got, want in zip(results, expect):
        assert got is not None
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
