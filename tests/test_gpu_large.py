"""Largest sizes through the C ABI: byte offsets past 2**32.

The large-token path on a 4.3 GB `out` (T = 300,000, two partials of 1.2 GB
together, ragged last token tile) and the weight-streaming path with a row
stride that puts its later rows past 4 GiB.  Inputs are drawn on the device
(synth.generate_device); the oracle sees host copies of sampled rows: rows
on both sides of the 4 GiB mark, tile edges and the last rows.
"""
from __future__ import annotations

import numpy as np
import pytest

from gpu_util import assert_window_close, host, say
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
    torch.cuda.empty_cache()


def _run_sampled(wl, rows, cols, seed, what):
    import torch

    from oracle import oracle

    d = synth.generate_device(wl, seed=seed)
    idx = torch.tensor(rows, device=d["out"].device)
    before = host(d["out"][:, :cols].index_select(0, idx))
    say("case %s T=%d P=%d ld=%d path=%d" % (what, wl.T, wl.P, wl.ld_out,
                                              binding.lt_path_for(wl.T, wl.n)))
    binding.check(binding.lt_latent_tail(d["partials"], wl.P, wl.T, wl.L, d["norm_w"], wl.eps,
                                         d["W"], wl.H, wl.c0, wl.n, d["out"], wl.ld_out, None))
    torch.cuda.synchronize()
    after = host(d["out"][:, :cols].index_select(0, idx))
    ref = oracle.latent_tail(host(d["partials"].index_select(1, idx)),
                             host(d["norm_w"]) if d["norm_w"] is not None else None,
                             float(np.float32(wl.eps)), host(d["W"]), wl.c0, wl.n, before)
    del d
    torch.cuda.empty_cache()
    assert_window_close(after, ref, wl.c0, wl.n, what)


def test_large_token_path_out_past_4gib():
    T, ld = 300_000, 7176
    wl = synth.Workload("huge", T=T, L=1024, H=7168, P=2, c0=0, n=7168, ld_out=ld, part_std=0.6)
    assert binding.lt_path_for(T, wl.n) == 2
    cross = (1 << 32) // (2 * ld)            # first row that starts past 4 GiB
    rng = np.random.Generator(np.random.PCG64(5))
    rows = sorted({0, 1, 255, 256, cross - 1, cross, cross + 1, T - 225, T - 224, T - 1,
                   *rng.integers(0, T, 6).tolist()})
    _run_sampled(wl, rows, ld, seed=21, what="huge prefill")


def test_weight_streaming_row_stride_past_4gib():
    T, ld = 40, 60_000_000                   # rows 36.. start past 4 GiB
    wl = synth.Workload("wide", T=T, L=1024, H=7168, P=1, c0=8, n=7100, ld_out=ld, part_std=0.6)
    assert binding.lt_path_for(T, wl.n) == 1
    _run_sampled(wl, list(range(T)), 7168 + 64, seed=22, what="wide decode")


def test_pingpong_gemm_row_stride_past_4gib():
    """The 256 x 128 ping-pong kernel (T = 1000 over 7168 columns) with a row
    stride of about 4.2 M elements: its 32-bit in-tile offsets stay below
    1.1 GB while token tiles from row 512 on start past 4 GiB."""
    T, ld = 1000, 4_194_312
    wl = synth.Workload("pp_wide", T=T, L=1024, H=7168, P=1, c0=0, n=7168, ld_out=ld,
                        part_std=0.6)
    assert binding.lt_path_for(T, wl.n) == 2
    cross = -(-(1 << 32) // (2 * ld))        # first row that starts past 4 GiB
    rng = np.random.Generator(np.random.PCG64(9))
    rows = sorted({0, 1, 63, 64, 127, 128, cross - 1, cross, cross + 1, 895, 896, T - 1,
                   *rng.integers(0, T, 6).tolist()})
    _run_sampled(wl, rows, 7168 + 8, seed=24, what="ping-pong wide")
