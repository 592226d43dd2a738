"""Concurrent calls from two host threads on one stream (C ABI).

The large-token path keeps one scratch latent per (device, stream); calls
that grow it move to a larger buffer and keep the old one.  Two threads issuing calls of growing
token counts on the same stream must each get exactly the result of the same
call made alone: the scratch of one call must not be freed or overwritten
between its two kernels by the other thread's call.
"""
from __future__ import annotations

import threading

import numpy as np
import pytest

from gpu_util import DevInputs, dev, host, say
from latent_moe_output_amd import binding, synth

pytestmark = pytest.mark.gpu

TS = (200, 900, 2000)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    binding.load()
    prev = binding.lt_set_skinny_max_tokens(-1)
    yield
    binding.lt_set_skinny_max_tokens(-1 if prev == 64 else prev)


def test_two_threads_one_stream_growing_scratch():
    import torch

    wls = {T: synth.Workload("threads", T=T, L=1024, H=1024, P=1, c0=0, n=1024, ld_out=1024,
                             part_std=0.6) for T in TS}
    inputs = {T: DevInputs(synth.generate(wls[T], seed=T)) for T in TS}
    s = torch.cuda.Stream()
    sh = s.cuda_stream

    def call(T, out):
        di, wl = inputs[T], wls[T]
        return binding.lt_latent_tail(di.partials, 1, T, wl.L, di.norm_w, wl.eps, di.W, wl.H,
                                      0, wl.n, out, wl.ld_out, sh)

    # each call alone (fresh out copies), one after the other; uploads run
    # on PyTorch's stream, so synchronise before the calls on `s`
    ref = {}
    for T in TS:
        out = inputs[T].d["out"].copy()
        o = dev(out)
        torch.cuda.synchronize()
        say("threads: reference T=%d" % T)
        binding.check(call(T, o))
        s.synchronize()
        ref[T] = host(o)

    # the same calls from two threads at once, starting from no scratch so
    # that the buffer grows while both threads are issuing
    s.synchronize()
    assert binding.lt_release_scratch() == binding.LT_OK
    n_calls = 6
    outs = [[dev(inputs[TS[(i + k) % 3]].d["out"].copy()) for i in range(n_calls)]
            for k in range(2)]
    torch.cuda.synchronize()
    status = [[None] * n_calls for _ in range(2)]
    start = threading.Barrier(2)

    def worker(k):
        start.wait()
        for i in range(n_calls):
            status[k][i] = call(TS[(i + k) % 3], outs[k][i])

    say("threads: two threads x %d calls on one stream" % n_calls)
    th = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    s.synchronize()
    for k in range(2):
        for i in range(n_calls):
            T = TS[(i + k) % 3]
            assert status[k][i] == binding.LT_OK, binding.lt_status_string(status[k][i])
            np.testing.assert_array_equal(host(outs[k][i]), ref[T],
                                          err_msg="thread %d call %d T=%d" % (k, i, T))


def test_per_thread_stream_keeps_scratch_per_thread():
    """hipStreamPerThread names a different stream in every host thread: two
    threads calling on it at once, with growing token counts, each get
    exactly the result of the same call made alone (each thread has its own
    scratch latent)."""
    import torch

    per_thread = 2                        # hipStreamPerThread
    wls = {T: synth.Workload("pts", T=T, L=1024, H=1024, P=2, c0=0, n=1024, ld_out=1024,
                             part_std=0.6) for T in TS}
    inputs = {T: DevInputs(synth.generate(wls[T], seed=100 + T)) for T in TS}
    ref = {}
    for T in TS:
        say("per-thread stream: reference T=%d" % T)
        binding.check(inputs[T].call(wls[T]))
        torch.cuda.synchronize()
        ref[T] = host(inputs[T].out)
    assert binding.lt_release_scratch() == binding.LT_OK
    n_calls = 6
    outs = [[dev(inputs[TS[(i + k) % 3]].d["out"].copy()) for i in range(n_calls)]
            for k in range(2)]
    torch.cuda.synchronize()
    status = [[None] * n_calls for _ in range(2)]
    start = threading.Barrier(2)

    def worker(k):
        start.wait()
        for i in range(n_calls):
            T = TS[(i + k) % 3]
            di, wl = inputs[T], wls[T]
            status[k][i] = binding.lt_latent_tail(di.partials, 2, T, wl.L, di.norm_w, wl.eps,
                                                  di.W, wl.H, 0, wl.n, outs[k][i], wl.ld_out,
                                                  per_thread)

    say("per-thread stream: two threads x %d calls" % n_calls)
    th = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    for k in range(2):
        for i in range(n_calls):
            T = TS[(i + k) % 3]
            assert status[k][i] == binding.LT_OK, binding.lt_status_string(status[k][i])
            np.testing.assert_array_equal(host(outs[k][i]), ref[T],
                                          err_msg="thread %d call %d T=%d" % (k, i, T))

