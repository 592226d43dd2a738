"""Shared helpers for the GPU parity tests (device buffers, comparisons).

All device buffers are torch int16 tensors holding bf16 bit patterns; the
library sees raw device pointers.  Nothing here computes the tail.
"""
from __future__ import annotations

import sys

import numpy as np

from latent_moe_output_amd import binding, synth

RTOL = 1.6e-2
ATOL = 3e-2


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, device="cuda"):
    import torch

    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).to(device)


def host(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


class DevInputs:
    """Device copies of one input set; `out` is fresh from `reset_out()`."""

    def __init__(self, d: dict, device="cuda"):
        import torch

        self.d = d
        self.partials = dev(d["partials"], device)
        self.norm_w = dev(d["norm_w"], device) if d["norm_w"] is not None else None
        self.W = dev(d["W"], device)
        self.out0 = dev(d["out"], device)
        self.out = torch.empty_like(self.out0)
        self.reset_out()

    def reset_out(self):
        self.out.copy_(self.out0)

    def call(self, wl, eps=None, c0=None, n=None, T=None, stream=None) -> int:
        P, Tp, L = self.d["partials"].shape
        H = self.d["W"].shape[0]
        ld = self.d["out"].shape[1]
        return binding.lt_latent_tail(
            self.partials, P, Tp if T is None else T, L, self.norm_w,
            wl.eps if eps is None else eps, self.W, H, wl.c0 if c0 is None else c0,
            wl.n if n is None else n, self.out, ld, stream)


def eps32(wl) -> float:
    return float(np.float32(wl.eps))


def assert_window_close(got: np.ndarray, ref: np.ndarray, c0: int, n: int, what: str = ""):
    """|got - ref| <= ATOL + RTOL*|ref| inside [c0, c0+n); bit-exact elsewhere."""
    g = synth.bf16_bits_to_f64(got[:, c0:c0 + n])
    r = synth.bf16_bits_to_f64(ref[:, c0:c0 + n])
    bad = ~(np.abs(g - r) <= ATOL + RTOL * np.abs(r))
    if bad.any():
        t, j = np.argwhere(bad)[0]
        raise AssertionError(
            "%s: %d of %d window elements out of tolerance; first at row %d col %d: "
            "gpu %r oracle %r" % (what, int(bad.sum()), bad.size, t, c0 + j, g[t, j], r[t, j]))
    outside = np.ones(got.shape, dtype=bool)
    outside[:, c0:c0 + n] = False
    if not np.array_equal(got[outside], ref[outside]):
        idx = np.argwhere(outside & (got != ref))[0]
        raise AssertionError("%s: element outside the window changed at %s" % (what, tuple(idx)))
