"""Seeded synthetic inputs for the latent-MoE output tail.

This module is shared by the tests, the benchmark and the smoke check.  It
holds the workload recipes (shapes and value distributions) and a seeded
sampler, and nothing of the tail's own arithmetic: it never sums, normalises,
projects or rounds anything the way the method does.  Random draws are made
in float64 with numpy's PCG64 and stored as bf16 bit patterns (``uint16``)
through PyTorch's float32 -> bfloat16 cast; that conversion only decides
which sample values exist and plays no part in the computation under test.

Draw order per input set (fixed, so a seed names one input set):
partials [P][T][L] -> norm weight [L] -> W [H][L] -> out [T][ld_out] ->
outlier mask and outlier signs.  The norm weight is drawn even when the norm
is disabled, so that both variants of a workload share W and out.

Workloads follow the pages' setting -- the Kimi-K3 latent-MoE tail at its
production shape on one tensor-parallel rank or replicated -- with synthetic
values standing in for the serving benchmarks the pages measure with:

* ``tiny``     T=5, L=64, H=128, one partial, full columns.
* ``decode``   T in {1, 8, 16}, L=1024, H=7168, one partial, full columns.
* ``shard``    T=256, 8 partials ~N(0, 0.35), window c0=3*896, n=896.
* ``prefill``  T=8192, one partial, full columns.
* ``ragged``   T=8191, 4 partials ~N(0, 0.5), window c0=7*896, n=896,
               +-1e4 outliers at 0.1% density over the whole out buffer;
               ``ragged_nonorm`` is the same inputs with the norm disabled.

Common values: partial ~N(0,1) unless stated, norm weight 1 + 0.1 N(0,1),
W ~N(0, 0.02), shared output ~N(0, 1), eps = 1e-6.  N(mu, s) names the
standard deviation s.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    L: int
    H: int
    P: int
    c0: int
    n: int
    ld_out: int
    part_std: float = 1.0
    norm: bool = True
    eps: float = 1e-6
    w_std: float = 0.02
    out_std: float = 1.0
    outlier_density: float = 0.0
    outlier_value: float = 1e4

    def with_T(self, T: int) -> "Workload":
        return replace(self, T=int(T))


WORKLOADS = {
    "tiny": Workload("tiny", T=5, L=64, H=128, P=1, c0=0, n=128, ld_out=128),
    "decode": Workload("decode", T=16, L=1024, H=7168, P=1, c0=0, n=7168, ld_out=7168),
    "shard": Workload("shard", T=256, L=1024, H=7168, P=8, c0=3 * 896, n=896,
                      ld_out=7168, part_std=0.35),
    "prefill": Workload("prefill", T=8192, L=1024, H=7168, P=1, c0=0, n=7168, ld_out=7168),
    "ragged": Workload("ragged", T=8191, L=1024, H=7168, P=4, c0=7 * 896, n=896,
                       ld_out=7168, part_std=0.5, outlier_density=1e-3),
    "ragged_nonorm": Workload("ragged_nonorm", T=8191, L=1024, H=7168, P=4, c0=7 * 896,
                              n=896, ld_out=7168, part_std=0.5, outlier_density=1e-3,
                              norm=False),
}

DECODE_TOKENS = (1, 8, 16)


def to_bf16_bits(x) -> np.ndarray:
    """float array -> uint16 bf16 bit patterns via PyTorch's bfloat16 cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f64(h) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact widening)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def generate(wl: Workload, seed: int = 0) -> dict:
    """One input set for workload ``wl``; every array is bf16 bits (uint16).

    Returns dict(partials [P][T][L], norm_w [L] or None, W [H][L],
    out [T][ld_out]).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    partials = to_bf16_bits(rng.standard_normal((wl.P, wl.T, wl.L)) * wl.part_std)
    norm_w = to_bf16_bits(1.0 + 0.1 * rng.standard_normal(wl.L))
    W = to_bf16_bits(rng.standard_normal((wl.H, wl.L)) * wl.w_std)
    out_f = rng.standard_normal((wl.T, wl.ld_out)) * wl.out_std
    if wl.outlier_density > 0:
        mask = rng.random((wl.T, wl.ld_out)) < wl.outlier_density
        sign = np.where(rng.random((wl.T, wl.ld_out)) < 0.5, -1.0, 1.0)
        out_f = np.where(mask, sign * wl.outlier_value, out_f)
    out = to_bf16_bits(out_f)
    return dict(partials=partials, norm_w=norm_w if wl.norm else None, W=W, out=out)


def generate_device(wl: Workload, seed: int = 0, device="cuda") -> dict:
    """The same distributions as generate(), drawn on the device by torch's
    seeded generator, for shapes too large to draw on the host.  Every entry
    is an int16 tensor of bf16 bit patterns (fp32 draws rounded to bf16, so
    not bit-identical to generate()); outliers are not drawn."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def draw(shape, std, mean=0.0):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        return (x * std + mean).to(torch.bfloat16).view(torch.int16)

    partials = draw((wl.P, wl.T, wl.L), wl.part_std)
    norm_w = draw((wl.L,), 0.1, 1.0)
    W = draw((wl.H, wl.L), wl.w_std)
    out = draw((wl.T, wl.ld_out), wl.out_std)
    return dict(partials=partials, norm_w=norm_w if wl.norm else None, W=W, out=out)
