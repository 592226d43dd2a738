"""GPU parity of the residual form, lt_latent_tail_residual, through the C ABI.

`out` must match the oracle as for lt_latent_tail; `resid` must match the
oracle's residual within the same tolerance, equal bf16(prefix + out) of the
GPU's own `out` bit for bit (the add is exact before its one rounding), and
be untouched outside the window.  Both paths (weight streaming and
norm + GEMM), the vector and the element-wise epilogues, separate and
in-place residual buffers, and the full-size prefill shape on every element.
"""
from __future__ import annotations

import numpy as np
import pytest

from gpu_util import DevInputs, assert_window_close, dev, eps32, host, say
from latent_moe_output_amd import binding, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    binding.load()
    prev = binding.lt_set_skinny_max_tokens(-1)
    yield
    binding.lt_set_skinny_max_tokens(-1 if prev == 64 else prev)


def _bf16_add(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """PyTorch's bf16 add of two bit-pattern arrays (CPU)."""
    import torch

    ta = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    tb = torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)
    return (ta + tb).view(torch.int16).numpy().view(np.uint16)


def _res_inputs(wl, ld_pre, ld_res, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    prefix = synth.to_bf16_bits(rng.standard_normal((wl.T, ld_pre)) * 3.0)
    resid0 = synth.to_bf16_bits(rng.standard_normal((wl.T, ld_res)) * 7.0 + 100.0)
    return prefix, resid0


def _call(di, wl, prefix_d, ld_pre, resid_d, ld_res, stream=None):
    P, T, L = di.d["partials"].shape
    H = di.d["W"].shape[0]
    ld = di.d["out"].shape[1]
    return binding.lt_latent_tail_residual(di.partials, P, T, L, di.norm_w, wl.eps, di.W, H,
                                           wl.c0, wl.n, di.out, ld, prefix_d, ld_pre, resid_d,
                                           ld_res, stream)


def _check(what, wl, got_out, got_res, ref_out, ref_res, prefix, resid0, rows=None):
    c0, n = wl.c0, wl.n
    assert_window_close(got_out, ref_out, c0, n, what + " out")
    sel = slice(None) if rows is None else rows
    assert_window_close(got_res[sel], ref_res, c0, n, what + " resid")
    # the residual is exactly bf16(prefix + out') of the GPU's own out'
    want = _bf16_add(prefix[:, c0:c0 + n], got_out[:, c0:c0 + n])
    np.testing.assert_array_equal(got_res[:, c0:c0 + n], want, err_msg=what + " resid add")
    outside = np.ones(got_res.shape, dtype=bool)
    outside[:, c0:c0 + n] = False
    np.testing.assert_array_equal(got_res[outside], resid0[outside], err_msg=what + " outside")


CASES = [
    # T, L, H, P, c0, n, ld_out, ld_pre, ld_res, forced threshold (-1 = default)
    (16, 1024, 7168, 1, 0, 7168, 7168, 7168, 7168, -1),   # decode, vector epilogue
    (5, 1024, 700, 2, 3, 517, 705, 709, 701, -1),         # skinny, element-wise epilogue
    (40, 264, 900, 3, 8, 880, 904, 912, 896, -1),         # skinny, two token tiles
    (130, 1024, 1536, 2, 64, 1024, 1544, 1552, 1560, -1),  # GEMM, LDS epilogue
    (129, 1024, 520, 1, 3, 517, 523, 525, 527, -1),        # GEMM, element-wise epilogue
    (64, 1024, 1536, 2, 64, 1024, 1544, 1552, 1560, 0),    # forced GEMM at a skinny size
    (100, 1024, 1536, 2, 64, 1024, 1544, 1552, 1560, 1000),  # forced skinny, two launches
    (2000, 1032, 7110, 1, 8, 7100, 7112, 7120, 7128, -1),  # 256 x 256 slot ring, K tail, ragged
    (2560, 1024, 7100, 1, 8, 7090, 7112, 7120, 7128, -1),  # ring, last round in halves, ragged
]


@pytest.mark.parametrize("T,L,H,P,c0,n,ld,ldp,ldr,thr", CASES)
def test_residual_matches_oracle(T, L, H, P, c0, n, ld, ldp, ldr, thr):
    from oracle import oracle

    binding.lt_set_skinny_max_tokens(thr)
    try:
        wl = synth.Workload("resid", T=T, L=L, H=H, P=P, c0=c0, n=n, ld_out=ld, part_std=0.6)
        d = synth.generate(wl, seed=T + c0)
        prefix, resid0 = _res_inputs(wl, ldp, ldr, seed=T)
        di = DevInputs(d)
        pd, rd = dev(prefix), dev(resid0)
        say("case resid T=%d L=%d H=%d c0=%d n=%d ld=%d/%d/%d thr=%d path=%d" % (
            T, L, H, c0, n, ld, ldp, ldr, thr, binding.lt_path_for(T, n)))
        binding.check(_call(di, wl, pd, ldp, rd, ldr))
        import torch

        torch.cuda.synchronize()
        ref_out, ref_res = oracle.latent_tail_residual(d["partials"], d["norm_w"], eps32(wl),
                                                       d["W"], c0, n, d["out"], prefix,
                                                       resid=resid0)
        _check("T=%d" % T, wl, host(di.out), host(rd), ref_out, ref_res, prefix, resid0)
    finally:
        binding.lt_set_skinny_max_tokens(-1)


@pytest.mark.parametrize("T", [8, 300])
def test_residual_in_place(T):
    """resid == prefix: the window is updated in place, the rest kept."""
    from oracle import oracle

    wl = synth.Workload("resid_ip", T=T, L=1024, H=2048, P=2, c0=128, n=1536, ld_out=2048,
                        part_std=0.6)
    d = synth.generate(wl, seed=3 * T)
    prefix, _ = _res_inputs(wl, 2056, 8, seed=T + 1)
    di = DevInputs(d)
    pd = dev(prefix)
    say("case resid in place T=%d path=%d" % (T, binding.lt_path_for(T, wl.n)))
    binding.check(_call(di, wl, pd, 2056, pd, 2056))
    import torch

    torch.cuda.synchronize()
    ref_out, ref_res = oracle.latent_tail_residual(d["partials"], d["norm_w"], eps32(wl), d["W"],
                                                   wl.c0, wl.n, d["out"], prefix, in_place=True)
    _check("in place T=%d" % T, wl, host(di.out), host(pd), ref_out, ref_res, prefix, prefix)


def test_residual_prefill_full():
    """Full-size prefill shape (T = 8192, n = 7168) on the 256 x 256 slot
    ring, compared with the oracle on every element of both buffers."""
    from oracle import oracle

    wl = synth.WORKLOADS["prefill"]
    d = synth.generate(wl, seed=0)
    prefix, resid0 = _res_inputs(wl, wl.ld_out, wl.ld_out, seed=9)
    di = DevInputs(d)
    pd, rd = dev(prefix), dev(resid0)
    say("case resid prefill (full size)")
    binding.check(_call(di, wl, pd, wl.ld_out, rd, wl.ld_out))
    import torch

    torch.cuda.synchronize()
    ref_out, ref_res = oracle.latent_tail_residual(d["partials"], d["norm_w"], eps32(wl), d["W"],
                                                   wl.c0, wl.n, d["out"], prefix, resid=resid0)
    _check("prefill", wl, host(di.out), host(rd), ref_out, ref_res, prefix, resid0)


def test_plain_and_residual_forms_give_the_same_out():
    """The residual form changes nothing about `out` (bit for bit)."""
    wl = synth.Workload("same", T=777, L=1024, H=7168, P=1, c0=0, n=7168, ld_out=7168)
    d = synth.generate(wl, seed=12)
    a, b = DevInputs(d), DevInputs(d)
    prefix, resid0 = _res_inputs(wl, 7168, 7168, seed=2)
    say("case plain vs residual T=777")
    binding.check(a.call(wl))
    binding.check(_call(b, wl, dev(prefix), 7168, dev(resid0), 7168))
    import torch

    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(a.out), host(b.out))


@pytest.mark.parametrize("T", [8, 700])
def test_residual_graph_capture_and_replay(T):
    """The residual form captured into a HIP graph (after lt_reserve) and
    replayed with eager work between replays: every replay matches eager."""
    import torch

    wl = synth.Workload("res_graph", T=T, L=1024, H=2048, P=2, c0=256, n=1536, ld_out=2048,
                        part_std=0.6)
    d = synth.generate(wl, seed=5)
    prefix, resid0 = _res_inputs(wl, 2048, 2048, seed=6)
    di = DevInputs(d)
    pd, rd = dev(prefix), dev(resid0)
    say("graph residual eager T=%d" % T)
    binding.check(_call(di, wl, pd, 2048, rd, 2048))
    torch.cuda.synchronize()
    want_out, want_res = host(di.out), host(rd)

    s = torch.cuda.Stream()
    assert binding.lt_reserve(T, wl.L, s) == binding.LT_OK
    g = torch.cuda.CUDAGraph()
    rd0 = dev(resid0)
    di.reset_out()
    rd.copy_(rd0)
    torch.cuda.synchronize()
    say("graph residual capture T=%d" % T)
    with torch.cuda.graph(g, stream=s):
        status = _call(di, wl, pd, 2048, rd, 2048, stream=torch.cuda.current_stream())
    assert status == binding.LT_OK
    for rep in range(3):
        di.reset_out()
        rd.copy_(rd0)
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()
        say("graph residual replay %d T=%d" % (rep, T))
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(di.out), want_out)
        np.testing.assert_array_equal(host(rd), want_res)
        del junk
    del g
