"""lt_latent_tail_noalloc, through the C ABI, against lt_latent_tail.

The entry point for callers that cannot allocate must give the same bits as
the allocating one on the same inputs, call after call (its fixed scratch
keeps the last call's contents, so a smaller call follows a larger one), must
refuse a latent beyond its fixed scratch before launching anything, and
needs no lt_reserve to be captured into a HIP graph.
"""
from __future__ import annotations

import numpy as np
import pytest

from gpu_util import DevInputs, host, say
from latent_moe_output_amd import binding, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    binding.load()
    binding.lt_set_skinny_max_tokens(-1)
    yield
    binding.lt_set_skinny_max_tokens(-1)


def _sync():
    import torch

    torch.cuda.synchronize()


def _call(fn, di, wl, stream=None):
    P, T, L = di.d["partials"].shape
    return fn(di.partials, P, T, L, di.norm_w, wl.eps, di.W, wl.H, wl.c0, wl.n, di.out,
              wl.ld_out, stream)


def _both(wl, seed, what):
    """(allocating result, noalloc result) of one call on the same inputs."""
    d = synth.generate(wl, seed=seed)
    a, b = DevInputs(d), DevInputs(d)
    say("noalloc: %s allocating T=%d P=%d path=%d" % (what, wl.T, wl.P,
                                                      binding.lt_path_for(wl.T, wl.n)))
    binding.check(_call(binding.lt_latent_tail, a, wl))
    _sync()
    say("noalloc: %s noalloc T=%d" % (what, wl.T))
    binding.check(_call(binding.lt_latent_tail_noalloc, b, wl))
    _sync()
    return host(a.out), host(b.out)


@pytest.mark.parametrize("P,norm", [(3, True), (1, True), (2, False)])
def test_noalloc_matches_allocating_entry_point_twice(P, norm):
    """Two calls in a row through the fixed scratch, the second smaller (fewer
    tokens, a narrower latent, another window): both equal lt_latent_tail."""
    first = synth.Workload("na1", T=2000, L=1024, H=3000, P=P, c0=40, n=2900, ld_out=3008,
                           norm=norm, part_std=0.6)
    second = synth.Workload("na2", T=300, L=520, H=2000, P=P, c0=3, n=1500, ld_out=2004,
                            norm=norm, part_std=0.6)
    for k, wl in enumerate((first, second)):
        ref, got = _both(wl, seed=50 + k + 10 * P, what="call %d" % k)
        np.testing.assert_array_equal(got, ref, err_msg="call %d P=%d norm=%s" % (k, P, norm))


def test_noalloc_weight_streaming_and_unscratched_paths():
    """Decode sizes and one partial without the norm use no scratch at all;
    beyond the scratch limit such calls still run."""
    for wl in (synth.WORKLOADS["decode"].with_T(16),
               synth.Workload("na_big", T=9000, L=1024, H=1024, P=1, c0=0, n=1024,
                              ld_out=1024, norm=False, part_std=0.6)):
        ref, got = _both(wl, seed=60, what=wl.name)
        np.testing.assert_array_equal(got, ref, err_msg=wl.name)


def test_noalloc_refuses_latent_beyond_its_scratch():
    """T * L over LT_NOALLOC_MAX_LATENT on the scratch path: refused before
    any launch, out untouched."""
    T, L = 8193, 1024
    assert T * L > binding.LT_NOALLOC_MAX_LATENT
    wl = synth.Workload("na_over", T=T, L=L, H=256, P=2, c0=0, n=256, ld_out=256,
                        part_std=0.6)
    d = synth.generate(wl, seed=61)
    di = DevInputs(d)
    say("noalloc: over the limit")
    assert _call(binding.lt_latent_tail_noalloc, di, wl) == binding.LT_ERR_SCRATCH_LIMIT
    _sync()
    np.testing.assert_array_equal(host(di.out), d["out"])


def test_noalloc_captured_without_reserve():
    """Captured into a HIP graph on a fresh stream with no lt_reserve, then
    replayed with eager work (and eager noalloc calls of another size)
    between replays: every replay equals the eager result."""
    import torch

    wl = synth.Workload("na_graph", T=777, L=1024, H=2048, P=2, c0=512, n=1024, ld_out=2048,
                        part_std=0.7)
    other = synth.Workload("na_other", T=1500, L=1024, H=1024, P=3, c0=0, n=1024,
                           ld_out=1024, part_std=0.6)
    d = synth.generate(wl, seed=62)
    di = DevInputs(d)
    say("noalloc graph: eager")
    binding.check(_call(binding.lt_latent_tail_noalloc, di, wl))
    _sync()
    expected = host(di.out)
    do = DevInputs(synth.generate(other, seed=63))
    binding.check(_call(binding.lt_latent_tail, do, other))
    _sync()
    expected_other = host(do.out)

    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    di.reset_out()
    _sync()
    say("noalloc graph: capture")
    with torch.cuda.graph(g, stream=s):
        status = _call(binding.lt_latent_tail_noalloc, di, wl, stream=torch.cuda.current_stream())
    assert status == binding.LT_OK
    for rep in range(3):
        do.reset_out()
        _sync()
        say("noalloc graph: eager other %d" % rep)
        binding.check(_call(binding.lt_latent_tail_noalloc, do, other))
        _sync()
        np.testing.assert_array_equal(host(do.out), expected_other)
        di.reset_out()
        _sync()
        junk = torch.randn(1 << 20, device="cuda").sum()
        say("noalloc graph: replay %d" % rep)
        g.replay()
        _sync()
        np.testing.assert_array_equal(host(di.out), expected, err_msg="replay %d" % rep)
        del junk
    del g
