"""Calls on distinct streams may run concurrently: several host threads, each
with its own compute and copy streams and buffers, drive whole training
steps (double-buffered forward walk and backward walk) through the library
at the same time.  Each thread's outputs must equal the serial run's bit for
bit.  ctypes releases the interpreter lock for the duration of a foreign
call, so the library calls really overlap."""

import threading

import pytest
import torch

from test_graph_gpu import Step

pytestmark = pytest.mark.gpu


def test_concurrent_calls_on_distinct_streams():
    B, H, P, C, d = 1, 2, 4, 160, 128
    print(f"threads B={B} H={H} P={P} C={C} d={d}", flush=True)
    steps = [Step(B, H, P, C, d, rank, causal=rank % 2 == 0) for rank in range(P)]
    want = []
    for s in steps:
        s.run()
        torch.cuda.synchronize()
        want.append(s.outputs())
    for s in steps:
        for t in [s.o, s.lse, s.dq, *s.dk, *s.dv]:
            t.fill_(float("nan"))
    torch.cuda.synchronize()

    errors = []
    start = threading.Barrier(len(steps))

    def work(s):
        try:
            stream = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(stream):
                for _ in range(3):
                    s.run()
            stream.synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(s,)) for s in steps]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for n, (s, w) in enumerate(zip(steps, want)):
        for m, (a, b) in enumerate(zip(s.outputs(), w)):
            assert torch.equal(a, b), f"thread {n}: output {m} differs from the serial run"
