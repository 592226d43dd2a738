"""Pins for the oracle of the AttnRes zero-block path (state update + norm).

[PR50593] = prhub report of vLLM PR #50593, "[Kimi-K3][AMD] Fuse AttnRes
state updates and norms".  Its Implementation section, item 1, defines the
fused update: prefix + delta in high precision, one round trip to bf16
storage precision, that value used as the residual source (prefix updated in
place) and written to the block-write slot, output RMSNorm with its variance
out of bf16; with zero valid blocks the aggregated value is the prefix.

The oracle is pinned by
(a) a hand-derived exact example (tests/golden/attn_res_hand_example.txt)
    over every combination of the three switches (delta, block write, norm),
(b) closed forms of RMSNorm: constant rows give +-w, eps = 3c^2 gives
    r = 1/(2|c|), a two-level row fixes the mean over H,
(c) library routines: PyTorch's bf16 add for the update, PyTorch's float64
    F.rms_norm for the norm,
(d) invariants: untouched slots and buffers, -0 as the delta's identity,
(e) exact-arithmetic brute force (fractions / 60-digit decimal) on small rows.
"""
from __future__ import annotations

import decimal
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest

from exact_bf16 import bf16_fraction, bits_of, nearest_check
from latent_moe_output_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
EPS32 = float(np.float32(1e-6))


def _golden():
    vals = {}
    for line in open(os.path.join(GOLDEN, "attn_res_hand_example.txt")):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *rest = line.split()
        vals[key] = rest
    T, H, S = int(vals["T"][0]), int(vals["H"][0]), int(vals["slots"][0])

    def arr(key, shape):
        return bits_of([float(x) for x in vals[key]]).reshape(shape)

    return dict(T=T, H=H, S=S, idx=int(vals["block_idx"][0]), eps=float(vals["eps"][0]),
                prefix=arr("prefix", (T, H)), delta=arr("delta", (T, H)),
                norm_w=arr("norm_w", (H,)), updated=arr("updated_prefix", (T, H)),
                out=arr("expected_out", (T, H)))


def _sentinel_block(T, S, H):
    return np.resize(np.array([0x7FA1, 0x8000, 0x461C, 0xC61C, 0x0001, 0x3F80], np.uint16),
                     (T, S, H)).astype(np.uint16)


@pytest.mark.parametrize("has_delta,write_block,norm",
                         list(itertools.product([True, False], repeat=3)))
def test_hand_worked_example(oracle_mod, has_delta, write_block, norm):
    g = _golden()
    T, H, S = g["T"], g["H"], g["S"]
    # without the delta the prefix is already the updated value
    prefix = g["prefix"] if has_delta else g["updated"]
    block = _sentinel_block(T, S, H) if write_block else None
    pre, blk, out = oracle_mod.attn_res_zero_block(
        prefix, g["delta"] if has_delta else None, block, g["idx"] if write_block else -1,
        g["norm_w"] if norm else None, g["eps"])
    np.testing.assert_array_equal(pre, g["updated"])          # bit patterns, -0 included
    np.testing.assert_array_equal(out, g["out"] if norm else g["updated"])
    if write_block:
        want = _sentinel_block(T, S, H)
        want[:, g["idx"], :] = g["updated"]
        np.testing.assert_array_equal(blk, want)


@pytest.mark.parametrize("H", [128, 1024, 7168])
def test_constant_rows_normalise_to_weight(oracle_mod, H):
    """A constant row c (c^2 >> eps) normalises to sign(c) * w exactly; a zero
    row to 0."""
    rng = np.random.Generator(np.random.PCG64(20))
    w = synth.to_bf16_bits(1 + 0.2 * rng.standard_normal(H))
    cs = [1.5, -0.75, 0.0, 40.0, -3.0]
    prefix = bits_of(np.repeat(np.array(cs)[:, None], H, axis=1))
    _, _, out = oracle_mod.attn_res_zero_block(prefix, None, None, -1, w, EPS32)
    for t, c in enumerate(cs):
        if c > 0:
            np.testing.assert_array_equal(out[t], w)
        elif c < 0:
            np.testing.assert_array_equal(out[t], w ^ 0x8000)
        else:
            assert np.all(synth.bf16_bits_to_f64(out[t]) == 0.0)


@pytest.mark.parametrize("c,eps", [(1.0, 3.0), (2.0, 12.0), (0.5, 0.75)])
def test_eps_is_added_inside_the_root(oracle_mod, c, eps):
    """mean(c^2) + 3c^2 = 4c^2, so r = 1/(2|c|) and out = w/2 exactly; eps
    added outside the root or left out would change it."""
    H = 64
    w = bits_of(np.array([1.0, -1.5, 0.25, 3.0] * (H // 4)))
    prefix = bits_of(np.full((1, H), c))
    _, _, out = oracle_mod.attn_res_zero_block(prefix, None, None, -1, w, eps)
    want = synth.to_bf16_bits(synth.bf16_bits_to_f64(w) / 2)
    np.testing.assert_array_equal(out[0], want)


@pytest.mark.parametrize("m", [1, 3, 7])
def test_two_level_row(oracle_mod, m):
    """Row of H/2 ones and H/2 sevens: mean(x^2) = 25, r = 1/5 with eps = 0
    (the mean divides by H, not H - 1; it squares, not takes abs)."""
    H = 16 * m
    x = np.array([1.0, 7.0] * (H // 2))
    w = bits_of(np.full(H, 5.0))
    _, _, out = oracle_mod.attn_res_zero_block(bits_of(x[None]), None, None, -1, w, 0.0)
    np.testing.assert_array_equal(out[0], bits_of(x))


def _bf16_add(a, b):
    import torch

    ta = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    tb = torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)
    return (ta + tb).view(torch.int16).numpy().view(np.uint16)


def test_update_matches_torch_bf16_add(oracle_mod):
    """The updated prefix is PyTorch's bf16 add (the unfused
    `prefix_sum + hidden_states` of [PR50593 Key source snippets,
    `forward_attn_residual`]), exact ties included; without the norm the
    output is that same value and the block slot holds it."""
    rng = np.random.Generator(np.random.PCG64(21))
    T, H, S = 9, 1024, 4
    prefix = synth.to_bf16_bits(rng.standard_normal((T, H)) * 4)
    delta = synth.to_bf16_bits(rng.standard_normal((T, H)) * np.exp2(rng.integers(-12, 3, (T, H))))
    # exact ties: delta = half a bf16 spacing of the prefix
    pf = synth.bf16_bits_to_f64(prefix[:2])
    half = np.exp2(np.floor(np.log2(np.abs(pf))) - 8) * np.sign(pf)
    delta[:2] = synth.to_bf16_bits(half)
    block = _sentinel_block(T, S, H)
    pre, blk, out = oracle_mod.attn_res_zero_block(prefix, delta, block, 2, None, 0.0)
    want = _bf16_add(prefix, delta)
    np.testing.assert_array_equal(pre, want)
    np.testing.assert_array_equal(out, want)
    np.testing.assert_array_equal(blk[:, 2, :], want)
    keep = np.ones(S, bool)
    keep[2] = False
    np.testing.assert_array_equal(blk[:, keep, :], _sentinel_block(T, S, H)[:, keep, :])


@pytest.mark.parametrize("H", [128, 1024, 7168])
def test_norm_is_nearest_bf16_of_torch_rms_norm(oracle_mod, H):
    """The output is the nearest bf16 (ties even) of PyTorch's float64
    F.rms_norm of the updated prefix over H with the norm weight and eps."""
    import torch

    rng = np.random.Generator(np.random.PCG64(22 + H))
    T = 5
    prefix = synth.to_bf16_bits(rng.standard_normal((T, H)))
    delta = synth.to_bf16_bits(rng.standard_normal((T, H)) * 0.3)
    w = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(H))
    pre, _, out = oracle_mod.attn_res_zero_block(prefix, delta, None, -1, w, EPS32)
    x = torch.from_numpy(synth.bf16_bits_to_f64(pre))
    y = torch.nn.functional.rms_norm(x, (H,), torch.from_numpy(synth.bf16_bits_to_f64(w)),
                                     EPS32).numpy()
    for t in range(T):
        for h in range(0, H, max(1, H // 97)):
            err = nearest_check(int(out[t, h]), Fraction(float(y[t, h])))
            assert err is None, (t, h, err)


def test_negative_zero_delta_is_the_identity(oracle_mod):
    """delta = -0 everywhere (the exact additive identity, -0 + -0 = -0)
    gives the result of no delta, bit for bit, prefix included."""
    rng = np.random.Generator(np.random.PCG64(23))
    T, H = 4, 256
    prefix = synth.to_bf16_bits(rng.standard_normal((T, H)))
    prefix[0, :8] = 0x8000
    w = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(H))
    a = oracle_mod.attn_res_zero_block(prefix, None, None, -1, w, EPS32)
    b = oracle_mod.attn_res_zero_block(prefix, np.full((T, H), 0x8000, np.uint16), None, -1,
                                       w, EPS32)
    np.testing.assert_array_equal(a[0], prefix)
    np.testing.assert_array_equal(b[0], prefix)
    np.testing.assert_array_equal(a[2], b[2])


def test_without_delta_the_prefix_is_untouched(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(24))
    prefix = synth.to_bf16_bits(rng.standard_normal((3, 128)))
    pre, blk, _ = oracle_mod.attn_res_zero_block(prefix, None, None, -1, None, 0.0)
    np.testing.assert_array_equal(pre, prefix)
    assert blk is None


def test_bad_arguments_are_rejected(oracle_mod):
    prefix = np.zeros((2, 16), np.uint16)
    with pytest.raises(ValueError):
        oracle_mod.attn_res_zero_block(prefix, None, np.zeros((2, 2, 16), np.uint16), 2, None, 0.0)
    with pytest.raises(ValueError):
        oracle_mod.attn_res_zero_block(prefix, np.zeros((2, 8), np.uint16), None, -1, None, 0.0)
    pre, _, out = oracle_mod.attn_res_zero_block(np.zeros((0, 16), np.uint16), None, None, -1,
                                                 None, 0.0)
    assert pre.shape == (0, 16) and out.shape == (0, 16)


@pytest.mark.parametrize("H,seed", [(24, 30), (40, 31)])
def test_brute_force(oracle_mod, H, seed):
    """Small rows in exact arithmetic: the updated prefix is the nearest bf16
    of the exact sum, the output the nearest bf16 of p' * r * w with r from
    60-digit decimal arithmetic."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T = 3
    prefix = synth.to_bf16_bits(rng.standard_normal((T, H)) * 2)
    delta = synth.to_bf16_bits(rng.standard_normal((T, H)) * np.exp2(rng.integers(-10, 2, (T, H))))
    w = synth.to_bf16_bits(1 + 0.2 * rng.standard_normal(H))
    eps = EPS32
    pre, blk, out = oracle_mod.attn_res_zero_block(prefix, delta, np.zeros((T, 2, H), np.uint16),
                                                   0, w, eps)
    ctx = decimal.Context(prec=60)
    for t in range(T):
        for h in range(H):
            ex = bf16_fraction(prefix[t, h]) + bf16_fraction(delta[t, h])
            assert nearest_check(int(pre[t, h]), ex) is None, (t, h)
            assert blk[t, 0, h] == pre[t, h]
        ms = sum(bf16_fraction(x) ** 2 for x in pre[t]) / H + Fraction(eps)
        dm = ctx.divide(decimal.Decimal(ms.numerator), decimal.Decimal(ms.denominator))
        r = Fraction(ctx.divide(decimal.Decimal(1), ctx.sqrt(dm)))
        for h in range(H):
            v = bf16_fraction(pre[t, h]) * r * bf16_fraction(w[h])
            err = nearest_check(int(out[t, h]), v)
            assert err is None, (t, h, err)
