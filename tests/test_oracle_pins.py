"""Pins for the CPU fp64 oracle: checks against things other than itself.

The pages print no numeric worked example, so the oracle is pinned by
(a) a hand-derived exact example (tests/golden/hand_example.txt),
(b) closed forms of RMSNorm (constant rows, two-level rows, eps inside the
    root) from the definition used by [PR51253 Key source snippets,
    `_check_matches_replicated`],
(c) invariants the pages fix: only the window changes
    ([PR51253 Key source snippets, `_check_writes_only_its_own_shard`]),
    concatenated column shards equal the full projection
    ([PR50383 Key source snippets, `_shard_up_proj_tail`]), splitting a
    partial sum leaves it unchanged,
(d) library routines: PyTorch's float32 -> bfloat16 cast for rounding,
    numpy's fp64 matmul for the textbook GEMM special case,
(e) exact-arithmetic brute force (Python fractions / decimal) on tiny inputs.

[PR51253] = prhub report of vLLM PR #51253 (ROCm shard of the latent-MoE
up-projection); [PR50383] = prhub report of vLLM PR #50383 (column-parallel
up-projection tier).
"""
from __future__ import annotations

import decimal
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

from exact_bf16 import bf16_fraction, bits_of, nearest_check
from latent_moe_output_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
EPS32 = float(np.float32(1e-6))


def _f64(h):
    return synth.bf16_bits_to_f64(h)


# --------------------------------------------------------------------------
# bf16 rounding
# --------------------------------------------------------------------------

def test_rounding_matches_torch_cast_on_float32_values(oracle_mod):
    """For float32-representable inputs one RNE step is exactly PyTorch's
    float32 -> bfloat16 cast (a library routine)."""
    import torch

    rng = np.random.Generator(np.random.PCG64(1))
    u = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2**16, size=4000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    special = np.array([0x00000000, 0x80000000, 0x00000001, 0x00008000, 0x00018000,
                        0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0xFF7FFFFF, 0x3F808000,
                        0x3F818000, 0x007F8000, 0x00800000], dtype=np.uint32)
    u = np.concatenate([u, ties, special])
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle_mod.f64_to_bf16(float(x)) for x in f], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "first mismatch: %r -> 0x%04x, torch 0x%04x" % (
        f[bad[0]], got[bad[0]], ref[bad[0]])


def test_rounding_is_nearest_even_on_doubles(oracle_mod):
    """Doubles that are not float32 values (where a float32 detour would round
    twice): the result must be the nearest bf16, ties to even."""
    rng = np.random.Generator(np.random.PCG64(2))
    xs = list(rng.standard_normal(3000) * np.exp2(rng.integers(-30, 30, 3000)))
    # exact ties and near-ties below float32 resolution
    for base in (1.0, 1.5, -3.25, 2.0**-100, 1.0 + 2.0**-7):
        half = 2.0 ** (np.floor(np.log2(abs(base))) - 8)
        xs += [base + half, base - half, base + half + 2.0**-40 * abs(base),
               base + half - 2.0**-40 * abs(base), base + 3 * half]
    xs += [2.0**-133 * 0.5, 2.0**-133 * 1.5, 2.0**-133 * 0.5000001, 2.0**-130 * 1.3]
    for x in xs:
        h = oracle_mod.f64_to_bf16(x)
        err = nearest_check(h, Fraction(x))
        assert err is None, err


def test_rounding_specials(oracle_mod):
    assert oracle_mod.f64_to_bf16(float("inf")) == 0x7F80
    assert oracle_mod.f64_to_bf16(float("-inf")) == 0xFF80
    assert oracle_mod.f64_to_bf16(-0.0) == 0x8000
    assert oracle_mod.f64_to_bf16(3.5e38) == 0x7F80        # beyond max finite
    assert oracle_mod.f64_to_bf16(3.389e38) == 0x7F7F
    assert oracle_mod.f64_to_bf16(3.38e38) == 0x7F7E
    nan = oracle_mod.f64_to_bf16(float("nan"))
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0
    assert oracle_mod.bf16_to_f64(0x3F80) == 1.0
    assert oracle_mod.bf16_to_f64(0xC0A0) == -5.0


# --------------------------------------------------------------------------
# hand-worked golden example
# --------------------------------------------------------------------------

def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *rest = line.split()
            vals[key] = [float(v) for v in rest]
    return vals


def test_hand_worked_example(oracle_mod):
    g = _read_golden("hand_example.txt")
    T, L, H, P = (int(g[k][0]) for k in ("T", "L", "H", "P"))
    ld, c0, n = (int(g[k][0]) for k in ("ld_out", "c0", "n"))
    eps = g["eps"][0]
    partials = bits_of(g["partials"]).reshape(P, T, L)
    norm_w = bits_of(g["norm_w"])
    W = bits_of(g["W"]).reshape(H, L)
    out = bits_of(g["out"]).reshape(T, ld)

    y = oracle_mod.latent(partials, norm_w, eps)
    np.testing.assert_array_equal(y, bits_of(g["latent"]).reshape(T, L))
    got = oracle_mod.latent_tail(partials, norm_w, eps, W, c0, n, out)
    np.testing.assert_array_equal(got, bits_of(g["expected_out"]).reshape(T, ld))

    y0 = oracle_mod.latent(partials, None, eps)
    np.testing.assert_array_equal(y0, bits_of(g["latent_nonorm"]).reshape(T, L))
    got0 = oracle_mod.latent_tail(partials, None, eps, W, c0, n, out)
    np.testing.assert_array_equal(got0, bits_of(g["expected_out_nonorm"]).reshape(T, ld))


def test_hand_worked_residual(oracle_mod):
    """The residual update of the hand example, including a tie that rounds
    to the even neighbour, with and without the norm, separate and in place."""
    g = _read_golden("hand_example.txt")
    T, L, H, P = (int(g[k][0]) for k in ("T", "L", "H", "P"))
    ld, c0, n = (int(g[k][0]) for k in ("ld_out", "c0", "n"))
    eps = g["eps"][0]
    partials = bits_of(g["partials"]).reshape(P, T, L)
    norm_w = bits_of(g["norm_w"])
    W = bits_of(g["W"]).reshape(H, L)
    out = bits_of(g["out"]).reshape(T, ld)
    prefix = bits_of(g["prefix"]).reshape(T, ld)
    for nw, ko, kr in ((norm_w, "expected_out", "expected_resid"),
                       (None, "expected_out_nonorm", "expected_resid_nonorm")):
        for in_place in (False, True):
            o, r = oracle_mod.latent_tail_residual(partials, nw, eps, W, c0, n, out, prefix,
                                                   in_place=in_place)
            np.testing.assert_array_equal(o, bits_of(g[ko]).reshape(T, ld))
            np.testing.assert_array_equal(r, bits_of(g[kr]).reshape(T, ld))


# --------------------------------------------------------------------------
# RMSNorm closed forms
# --------------------------------------------------------------------------

def _norm_w(L, seed):
    return synth.to_bf16_bits(1.0 + 0.3 * np.random.Generator(np.random.PCG64(seed)).standard_normal(L))


@pytest.mark.parametrize("L", [8, 64, 1024])
def test_constant_row_gives_norm_weight(oracle_mod, L):
    """A constant row c != 0 normalises to sign(c) * w (c^2 >> eps); a zero row to 0."""
    w = _norm_w(L, 3)
    rows = [1.5, -0.75, 0.0, 96.0, -2.0**-2]
    partials = np.stack([bits_of(np.full(L, c)) for c in rows])[None]
    y = oracle_mod.latent(partials, w, EPS32)
    for t, c in enumerate(rows):
        if c > 0:
            np.testing.assert_array_equal(y[t], w)
        elif c < 0:
            np.testing.assert_array_equal(y[t], w ^ 0x8000)
        else:
            np.testing.assert_array_equal(_f64(y[t]), 0.0)


def test_constant_row_through_identity_projection(oracle_mod):
    """Observed through the projection with W = I and out = 0: out == latent."""
    L = 64
    w = _norm_w(L, 4)
    partials = np.stack([bits_of(np.full(L, c)) for c in (2.0, -0.5, 0.0)])[None]
    W = bits_of(np.eye(L))
    out = np.zeros((3, L), dtype=np.uint16)
    got = oracle_mod.latent_tail(partials, w, EPS32, W, 0, L, out)
    np.testing.assert_array_equal(got[0], w)
    np.testing.assert_array_equal(got[1], w ^ 0x8000)
    np.testing.assert_array_equal(_f64(got[2]), 0.0)


@pytest.mark.parametrize("c,eps", [(1.0, 3.0), (2.0, 12.0), (0.5, 0.75)])
def test_eps_is_added_inside_the_root(oracle_mod, c, eps):
    """Constant row c with eps = 3 c^2: r = 1 / (2|c|), so latent = w / 2 exactly."""
    L = 32
    w = _norm_w(L, 5)
    partials = bits_of(np.full((1, 1, L), c))
    y = oracle_mod.latent(partials, w, eps)
    np.testing.assert_array_equal(_f64(y[0]), _f64(w) / 2)


@pytest.mark.parametrize("m", [-3, 0, 2])
def test_two_level_row(oracle_mod, m):
    """Row alternating 1 and 7: mean square 25, r = 1/5; with w = 5 * 2^m the
    latent is exactly [2^m, 7 * 2^m, ...]."""
    L = 16
    row = np.tile([1.0, 7.0], L // 2)
    partials = bits_of(row)[None, None]
    w = bits_of(np.full(L, 5.0 * 2.0**m))
    y = oracle_mod.latent(partials, w, EPS32)
    np.testing.assert_array_equal(_f64(y[0]), row * 2.0**m)


def test_norm_disabled_passes_the_sum(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(6))
    x = synth.to_bf16_bits(rng.standard_normal((1, 3, 40)))
    np.testing.assert_array_equal(oracle_mod.latent(x, None, EPS32), x[0])


# --------------------------------------------------------------------------
# partial sum and its bf16 storage round trip
# --------------------------------------------------------------------------

def test_partial_split_invariance(oracle_mod):
    """[X, Y, -Y] and [X/2, X/2] sum exactly to X: same result as [X] alone."""
    wl = synth.WORKLOADS["tiny"]
    d = synth.generate(wl, seed=7)
    X = d["partials"]
    Y = synth.generate(wl, seed=8)["partials"]
    half = synth.to_bf16_bits(_f64(X) / 2)           # halving a bf16 is exact here
    assert np.all(_f64(half) * 2 == _f64(X))
    ref = oracle_mod.latent_tail(X, d["norm_w"], EPS32, d["W"], wl.c0, wl.n, d["out"])
    for stack in (np.concatenate([X, Y, Y ^ 0x8000]), np.concatenate([half, half])):
        got = oracle_mod.latent_tail(stack, d["norm_w"], EPS32, d["W"], wl.c0, wl.n, d["out"])
        np.testing.assert_array_equal(got, ref)


def test_partial_sum_is_rounded_to_bf16_before_use(oracle_mod):
    """The reduced latent is stored as bf16: 1 + 3*2^-9 becomes 1 + 2^-7, so
    (s0 - 1) projected with weight [1, -1] gives 2^-7, not 3*2^-9."""
    partials = bits_of([[[1.0, 1.0]], [[3 * 2.0**-9, 0.0]]])   # P=2, T=1, L=2
    W = bits_of([[1.0, -1.0]])
    out = np.zeros((1, 1), dtype=np.uint16)
    got = oracle_mod.latent_tail(partials, None, EPS32, W, 0, 1, out)
    assert _f64(got)[0, 0] == 2.0**-7
    rng = np.random.Generator(np.random.PCG64(9))
    parts = synth.to_bf16_bits(rng.standard_normal((3, 4, 24)))
    y = oracle_mod.latent(parts, None, EPS32)
    exact = [[sum(bf16_fraction(parts[p, t, k]) for p in range(3)) for k in range(24)]
             for t in range(4)]
    for t in range(4):
        for k in range(24):
            err = nearest_check(int(y[t, k]), exact[t][k])
            assert err is None, err


# --------------------------------------------------------------------------
# projection, window and beta-add
# --------------------------------------------------------------------------

def test_textbook_gemm_special_case(oracle_mod):
    """Norm off, one partial: out_window = bf16(C + A @ B^T), checked against
    numpy's fp64 matmul within the half-ulp bound of the final rounding."""
    rng = np.random.Generator(np.random.PCG64(10))
    T, L, H, c0, n, ld = 6, 1024, 300, 37, 211, 301
    A = synth.to_bf16_bits(rng.standard_normal((1, T, L)))
    B = synth.to_bf16_bits(rng.standard_normal((H, L)) * 0.02)
    C = synth.to_bf16_bits(rng.standard_normal((T, ld)))
    got = oracle_mod.latent_tail(A, None, EPS32, B, c0, n, C)
    ref = _f64(C)[:, c0:c0 + n] + _f64(A[0]) @ _f64(B)[c0:c0 + n].T
    g = _f64(got)[:, c0:c0 + n]
    # |got - ref| <= half a bf16 step at |ref| (plus fp64 summation slack)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0**-126))) - 7)
    assert np.all(np.abs(g - ref) <= 0.5 * step * (1 + 1e-9) + 1e-12)
    np.testing.assert_array_equal(np.delete(got, np.s_[c0:c0 + n], axis=1),
                                  np.delete(C, np.s_[c0:c0 + n], axis=1))


def test_dyadic_exact_projection(oracle_mod):
    """Small-integer latent and dyadic W: the projection sum is exact in
    integers, so the result must be the nearest bf16 of the exact value."""
    rng = np.random.Generator(np.random.PCG64(11))
    T, L, H = 3, 1024, 48
    A = rng.integers(-2, 3, (1, T, L)).astype(np.float64)
    Bq = rng.integers(-2, 3, (H, L))
    C = rng.integers(-64, 65, (T, H)).astype(np.float64) / 8
    got = oracle_mod.latent_tail(bits_of(A), None, EPS32, bits_of(Bq / 16.0), 0, H, bits_of(C))
    exact = A[0].astype(np.int64) @ Bq.T.astype(np.int64)        # in units of 1/16
    for t in range(T):
        for j in range(H):
            x = Fraction(int(exact[t, j]), 16) + Fraction(C[t, j])
            err = nearest_check(int(got[t, j]), x)
            assert err is None, (t, j, err)


def test_shards_concatenate_to_full_projection(oracle_mod):
    """Column shards c0 = k*H/8, n = H/8 written one after another reproduce
    the full-window call bit for bit."""
    wl = synth.Workload("s", T=7, L=128, H=256, P=2, c0=0, n=256, ld_out=260)
    d = synth.generate(wl, seed=12)
    full = oracle_mod.latent_tail(d["partials"], d["norm_w"], EPS32, d["W"], 0, wl.H, d["out"])
    acc = d["out"].copy()
    for k in range(8):
        acc = oracle_mod.latent_tail(d["partials"], d["norm_w"], EPS32, d["W"],
                                     k * wl.H // 8, wl.H // 8, acc)
    np.testing.assert_array_equal(acc, full)


def test_only_the_window_changes(oracle_mod):
    """Sentinels (NaN payloads, -0.0, +-9984, denormals) outside the window and
    in the row padding survive bit for bit; odd offsets included."""
    T, L, H, ld = 4, 64, 40, 45
    wl = synth.Workload("w", T=T, L=L, H=H, P=1, c0=0, n=H, ld_out=ld)
    d = synth.generate(wl, seed=13)
    sentinels = np.array([0x7FA1, 0xFFC3, 0x8000, 0x461C, 0xC61C, 0x0001], dtype=np.uint16)
    out = np.resize(sentinels, (T, ld)).astype(np.uint16)
    for c0, n in ((1, 5), (0, 1), (39, 1), (7, 33)):
        got = oracle_mod.latent_tail(d["partials"], d["norm_w"], EPS32, d["W"], c0, n, out)
        mask = np.zeros((T, ld), dtype=bool)
        mask[:, c0:c0 + n] = True
        np.testing.assert_array_equal(got[~mask], out[~mask])
        assert np.any(got[mask] != out[mask])


def test_empty_calls_are_noops(oracle_mod):
    wl = synth.WORKLOADS["tiny"]
    d = synth.generate(wl, seed=14)
    np.testing.assert_array_equal(
        oracle_mod.latent_tail(d["partials"], d["norm_w"], EPS32, d["W"], 3, 0, d["out"]),
        d["out"])
    empty = np.zeros((1, 0, wl.L), dtype=np.uint16)
    assert oracle_mod.latent_tail(empty, d["norm_w"], EPS32, d["W"], 0, 4,
                                  np.zeros((0, wl.ld_out), np.uint16)).shape == (0, wl.ld_out)


def test_bad_arguments_are_rejected(oracle_mod):
    wl = synth.WORKLOADS["tiny"]
    d = synth.generate(wl, seed=15)
    with pytest.raises(ValueError):
        oracle_mod.latent_tail(d["partials"], d["norm_w"], EPS32, d["W"], 100, 29, d["out"])
    with pytest.raises(ValueError):
        oracle_mod.latent_tail(d["partials"], d["norm_w"], EPS32, d["W"], 0, 4,
                               np.zeros((wl.T, wl.H - 1), np.uint16))


# --------------------------------------------------------------------------
# brute force in exact / high-precision arithmetic
# --------------------------------------------------------------------------

def _brute_force_check(oracle_mod, wl, seed, eps):
    d = synth.generate(wl, seed=seed)
    P, T, L = d["partials"].shape
    y = oracle_mod.latent(d["partials"], d["norm_w"], eps)
    ctx = decimal.Context(prec=60)
    for t in range(T):
        s = []
        for k in range(L):
            ex = sum(bf16_fraction(d["partials"][p, t, k]) for p in range(P))
            # storage round trip of the sum: must be the nearest bf16, ties even
            cand = [h for h in _candidates(ex)]
            s.append(_nearest_from(cand, ex))
        if d["norm_w"] is None:
            for k in range(L):
                assert int(y[t, k]) == s[k] or bf16_fraction(y[t, k]) == bf16_fraction(s[k])
            continue
        ms = sum(bf16_fraction(h) ** 2 for h in s) / L + Fraction(eps)
        dm = ctx.divide(decimal.Decimal(ms.numerator), decimal.Decimal(ms.denominator))
        r = Fraction(ctx.divide(decimal.Decimal(1), ctx.sqrt(dm)))
        for k in range(L):
            v = bf16_fraction(s[k]) * r * bf16_fraction(d["norm_w"][k])
            err = nearest_check(int(y[t, k]), v)
            assert err is None, (t, k, err)
    got = oracle_mod.latent_tail(d["partials"], d["norm_w"], eps, d["W"], wl.c0, wl.n, d["out"])
    Wf = [[bf16_fraction(h) for h in row] for row in d["W"][wl.c0:wl.c0 + wl.n]]
    yf = [[bf16_fraction(h) for h in row] for row in y]
    for t in range(T):
        for j in range(wl.n):
            x = bf16_fraction(d["out"][t, wl.c0 + j]) + sum(a * b for a, b in zip(yf[t], Wf[j]))
            err = nearest_check(int(got[t, wl.c0 + j]), x)
            assert err is None, (t, j, err)


def _candidates(x: Fraction):
    f = float(x)
    h = int(np.array([f], dtype=np.float32).view(np.uint32)[0] >> 16)
    return [(h + d) & 0xFFFF for d in (-1, 0, 1, 2)]


def _nearest_from(cands, x):
    for h in cands:
        if (h & 0x7F80) != 0x7F80 and nearest_check(h, x) is None:
            return h
    raise AssertionError("no nearest bf16 among candidates for %r" % float(x))


def test_brute_force_tiny_workload(oracle_mod):
    """The tiny workload (T=5, L=64, H=128, one partial) in exact rational /
    60-digit decimal arithmetic: latent and output are the nearest bf16 of the
    exact values at each of the three rounding points."""
    _brute_force_check(oracle_mod, synth.WORKLOADS["tiny"], 0, EPS32)


def test_brute_force_three_partials_window(oracle_mod):
    wl = synth.Workload("bf3", T=3, L=32, H=24, P=3, c0=5, n=11, ld_out=27, part_std=0.6)
    _brute_force_check(oracle_mod, wl, 16, EPS32)


def test_brute_force_norm_disabled(oracle_mod):
    wl = synth.Workload("bf0", T=2, L=48, H=16, P=2, c0=3, n=9, ld_out=16, norm=False)
    _brute_force_check(oracle_mod, wl, 17, EPS32)


# --------------------------------------------------------------------------
# residual update after the tail
# --------------------------------------------------------------------------

def test_residual_matches_torch_bf16_add(oracle_mod):
    """R4 is PyTorch's bf16 add of the prefix and the tail's output (the sum
    of two bf16 values rounds correctly through float32), checked against
    torch on a ragged window, with prefix outliers and ties."""
    import torch

    wl = synth.Workload("res", T=7, L=72, H=40, P=2, c0=3, n=29, ld_out=45, part_std=0.6,
                        outlier_density=0.05)
    d = synth.generate(wl, seed=21)
    rng = np.random.Generator(np.random.PCG64(5))
    prefix = synth.to_bf16_bits(rng.standard_normal((wl.T, wl.ld_out + 2)) * 4.0)
    resid0 = synth.to_bf16_bits(rng.standard_normal((wl.T, wl.ld_out + 2)))
    out_new = oracle_mod.latent_tail(d["partials"], d["norm_w"], EPS32, d["W"], wl.c0, wl.n,
                                     d["out"])
    o, r = oracle_mod.latent_tail_residual(d["partials"], d["norm_w"], EPS32, d["W"], wl.c0,
                                           wl.n, d["out"], prefix, resid=resid0)
    np.testing.assert_array_equal(o, out_new)
    win = slice(wl.c0, wl.c0 + wl.n)
    tp = torch.from_numpy(prefix[:, win].astype(np.int16)).view(torch.bfloat16)
    to = torch.from_numpy(out_new[:, win].astype(np.int16)).view(torch.bfloat16)
    want = (tp + to).view(torch.int16).numpy().astype(np.uint16)
    np.testing.assert_array_equal(r[:, win], want)
    keep = np.ones(r.shape, dtype=bool)
    keep[:, win] = False
    np.testing.assert_array_equal(r[keep], resid0[keep])


def test_residual_of_zero_prefix_is_the_output(oracle_mod):
    """prefix = +0: the residual window equals the tail's output value for
    value (bf16(0 + x) = x; a -0 output becomes +0)."""
    wl = synth.Workload("res0", T=5, L=64, H=33, P=1, c0=0, n=33, ld_out=33)
    d = synth.generate(wl, seed=4)
    prefix = np.zeros((wl.T, wl.ld_out), dtype=np.uint16)
    o, r = oracle_mod.latent_tail_residual(d["partials"], d["norm_w"], EPS32, d["W"], 0, wl.n,
                                           d["out"], prefix)
    np.testing.assert_array_equal(synth.bf16_bits_to_f64(r), synth.bf16_bits_to_f64(o))


def test_residual_rejects_short_strides(oracle_mod):
    wl = synth.Workload("resb", T=2, L=8, H=6, P=1, c0=2, n=4, ld_out=6)
    d = synth.generate(wl, seed=1)
    with pytest.raises(ValueError):
        oracle_mod.latent_tail_residual(d["partials"], d["norm_w"], EPS32, d["W"], 2, 4,
                                        d["out"], np.zeros((2, 5), dtype=np.uint16))
