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
from nsutil import TOL, oracle_run, rel_err

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


def test_release_workspace_while_work_is_in_flight():
    # ns_release_workspace frees the device workspace with stream-ordered
    # frees: released right after a call is enqueued (the stream still busy),
    # the call completes with its own bits, and the next call on the stream
    # allocates a fresh workspace in stream order
    stream = torch.cuda.Stream()
    first = [workloads.gaussian((2048, 2304), seed=74, index=i) for i in range(4)]
    second = [workloads.gaussian((1024, 1536), seed=75, index=i) for i in range(3)] + \
             [workloads.gaussian((24, 700), seed=75, index=9)]
    want = []
    for batch in (first, second):
        dev = [g.cuda() for g in batch]
        ns.orthogonalize(dev)
        torch.cuda.synchronize()
        want.append([d.cpu() for d in dev])
    with torch.cuda.stream(stream):
        a = [g.cuda() for g in first]
        b = [g.cuda() for g in second]
        torch.cuda.synchronize()
        ns.orthogonalize(a, stream=stream)
        in_flight = not stream.query()
        ns.release_workspace(stream)
        ns.orthogonalize(b, stream=stream)
        ns.release_workspace(stream)
    stream.synchronize()
    assert in_flight, "the first call finished before the release: nothing was in flight"
    for got, exp in zip((a, b), want):
        for x, y in zip(got, exp):
            assert torch.equal(x.cpu().view(torch.int16), y.view(torch.int16))


def test_more_batches_than_the_plan_cache_holds():
    # 72 distinct batches in a row (the cache keeps 64 plans per stream), then
    # some of them again: evicted plans are rebuilt and give the same bits
    batches = [[workloads.gaussian((40 + i % 5, 300), seed=76, index=2 * i),
                workloads.gaussian((20, 260 + i), seed=76, index=2 * i + 1)] for i in range(72)]
    devs = [[g.cuda() for g in b] for b in batches]
    for d in devs:
        ns.orthogonalize(d)
    torch.cuda.synchronize()
    first = [[x.cpu() for x in d] for d in devs]
    again = (0, 1, 71)
    for i in again:
        for x, g in zip(devs[i], batches[i]):
            x.copy_(g)
        ns.orthogonalize(devs[i])
    torch.cuda.synchronize()
    for i in again:
        for x, y in zip(devs[i], first[i]):
            assert torch.equal(x.cpu().view(torch.int16), y.view(torch.int16)), i
    for i in (0, 35):
        for x, g in zip(first[i], batches[i]):
            assert rel_err(x, oracle_run(g)) <= TOL[torch.bfloat16]
