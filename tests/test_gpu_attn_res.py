"""GPU parity of lt_attn_res_zero_block (the AttnRes zero-block path) against
the oracle, through the C ABI.

[PR50593] = prhub report of vLLM PR #50593, "[Kimi-K3][AMD] Fuse AttnRes
state updates and norms".  Its Implementation section, item 3, describes the
contract test this follows: token counts 1, 7, 17, 3 and 320, hidden sizes
128, 1024 and 7168, combinations of the delta / block-write / output-norm
switches; return value, in-place prefix update, untouched block storage and
output checked.  Here every switch combination runs on every (tokens, hidden)
pair with zero valid blocks.

Bar: the updated prefix, the block slot and the output without the norm are
exact (one rounding of an exact sum), so they must equal the oracle bit for
bit; the normalised output must be within |d| <= 3e-2 + 1.6e-2*|ref| of the
oracle and at most one bf16 step from it; every element the call must not
write is bit-identical.  Item 4's HIP graph capture and replay at varying
shapes is tested too.
"""
from __future__ import annotations

import itertools
import os

import numpy as np
import pytest

from exact_bf16 import bits_of
from gpu_util import ATOL, RTOL, dev, host, say
from latent_moe_output_amd import binding, synth

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
EPS32 = float(np.float32(1e-6))
SLOTS = 9                                   # room for the pages' 0-8 blocks


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    binding.load()


def _sync():
    import torch

    torch.cuda.synchronize()


def _inputs(T, H, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    prefix = synth.to_bf16_bits(rng.standard_normal((T, H)) * 2.0)
    delta = synth.to_bf16_bits(rng.standard_normal((T, H)) * np.exp2(rng.integers(-9, 2, (T, H))))
    block = np.resize(np.array([0x7FA1, 0x8000, 0x461C, 0xC61C, 0x0001, 0x3F80], np.uint16),
                      (T, SLOTS, H)).astype(np.uint16)
    w = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(H))
    out0 = np.full((T, H), 0x7FC1, np.uint16)
    return prefix, delta, block, w, out0


def _run(prefix, delta, block, idx, w, eps, out0, stream=None):
    """GPU results (prefix', block', out) for one call."""
    T, H = prefix.shape
    pd, dd = dev(prefix), (dev(delta) if delta is not None else None)
    bd = dev(block) if block is not None else None
    wd = dev(w) if w is not None else None
    od = dev(out0)
    _sync()
    st = binding.lt_attn_res_zero_block(pd, dd, T, H, bd, SLOTS if block is not None else 0,
                                        idx, wd, eps, od, stream)
    binding.check(st)
    _sync()
    return host(pd), (host(bd).reshape(block.shape) if bd is not None else None), host(od)


def _compare(got, ref, norm, what):
    g_pre, g_blk, g_out = got
    r_pre, r_blk, r_out = ref
    np.testing.assert_array_equal(g_pre, r_pre, err_msg=what + " prefix")
    if r_blk is not None:
        np.testing.assert_array_equal(g_blk, r_blk, err_msg=what + " block")
    if not norm:
        np.testing.assert_array_equal(g_out, r_out, err_msg=what + " out")
        return
    g = synth.bf16_bits_to_f64(g_out)
    r = synth.bf16_bits_to_f64(r_out)
    bad = ~(np.abs(g - r) <= ATOL + RTOL * np.abs(r))
    assert not bad.any(), "%s: %d outputs out of tolerance" % (what, int(bad.sum()))
    steps = int(np.abs(_order_key(g_out) - _order_key(r_out)).max())
    assert steps <= 1, "%s: %d bf16 steps from the oracle" % (what, steps)


def _order_key(h):
    """bf16 bit patterns -> integers in value order (adjacent values differ by 1)."""
    h = h.astype(np.int64)
    return np.where(h & 0x8000, -(h & 0x7FFF), h)


COMBOS = list(itertools.product([True, False], repeat=3))   # delta, block write, norm


@pytest.mark.parametrize("has_delta,write_block,norm", COMBOS)
@pytest.mark.parametrize("T", [1, 7, 17, 3, 320])
@pytest.mark.parametrize("H", [128, 1024, 7168])
def test_contract_matrix(H, T, has_delta, write_block, norm):
    from oracle import oracle

    prefix, delta, block, w, out0 = _inputs(T, H, seed=T * 31 + H)
    idx = (T + H) % SLOTS if write_block else -1
    args = (prefix, delta if has_delta else None, block if write_block else None, idx,
            w if norm else None, EPS32)
    say("attn_res T=%d H=%d delta=%s block=%d norm=%s" % (T, H, has_delta, idx, norm))
    got = _run(*args, out0)
    ref = oracle.attn_res_zero_block(*args)
    _compare(got, ref, norm, "T=%d H=%d d=%s b=%s n=%s" % (T, H, has_delta, write_block, norm))


def _random_cases(count=48, seed=77):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(count):
        T = int(np.exp(rng.uniform(0, np.log(3000))))
        H = 8 * int(rng.integers(1, 1025))
        sw = rng.random(3) < 0.6
        cases.append((i, T, H, bool(sw[0]), bool(sw[1]), bool(sw[2])))
    return cases


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: "r%02d_T%d_H%d_%d%d%d" % (
    c[0], c[1], c[2], c[3], c[4], c[5]))
def test_random_shapes(case):
    """48 seeded random (tokens, hidden, switches) draws over the whole
    supported range (H a multiple of 8 up to 8192), against the oracle."""
    from oracle import oracle

    i, T, H, has_delta, write_block, norm = case
    prefix, delta, block, w, out0 = _inputs(T, H, seed=900 + i)
    idx = (i * 5) % SLOTS if write_block else -1
    args = (prefix, delta if has_delta else None, block if write_block else None, idx,
            w if norm else None, EPS32)
    say("attn_res random %d: T=%d H=%d delta=%s block=%d norm=%s" % (i, T, H, has_delta, idx, norm))
    _compare(_run(*args, out0), oracle.attn_res_zero_block(*args), norm, "random %d" % i)


def test_hand_worked_example_bit_exact():
    """The hand-derived values of tests/golden/attn_res_hand_example.txt (two
    exact ties of the storage round trip, a -0 output) through the GPU.  The
    kernel's rows are multiples of 8 wide, so each 4-wide row is repeated
    twice: the mean over the 8 columns equals the mean over the 4, and every
    value stays the hand-derived one."""
    vals = {}
    for line in open(os.path.join(GOLDEN, "attn_res_hand_example.txt")):
        line = line.split("#", 1)[0].strip()
        if line:
            k, *rest = line.split()
            vals[k] = rest
    T, H = int(vals["T"][0]), int(vals["H"][0])

    def rep(k, shape):
        a = bits_of([float(x) for x in vals[k]]).reshape(shape)
        return np.concatenate([a, a], axis=-1)

    prefix, delta = rep("prefix", (T, H)), rep("delta", (T, H))
    updated, want_out = rep("updated_prefix", (T, H)), rep("expected_out", (T, H))
    w = rep("norm_w", (H,))
    idx, eps = int(vals["block_idx"][0]), float(vals["eps"][0])
    blk = np.zeros((T, SLOTS, 2 * H), np.uint16)
    say("attn_res hand example")
    got_pre, got_blk, got_out = _run(prefix, delta, blk, idx, w, eps,
                                     np.zeros((T, 2 * H), np.uint16))
    np.testing.assert_array_equal(got_pre, updated)
    np.testing.assert_array_equal(got_blk[:, idx, :], updated)
    np.testing.assert_array_equal(got_out, want_out)        # bit patterns, -0 included
    # without the norm the output is the updated prefix
    _, _, got_out2 = _run(prefix, delta, None, -1, None, 0.0, np.zeros((T, 2 * H), np.uint16))
    np.testing.assert_array_equal(got_out2, updated)


@pytest.mark.parametrize("H", [128, 1024, 7168])
def test_constant_rows_normalise_to_weight(H):
    rng = np.random.Generator(np.random.PCG64(70))
    w = synth.to_bf16_bits(1 + 0.2 * rng.standard_normal(H))
    cs = [1.5, -0.75, 0.0, 40.0, -3.0]
    prefix = bits_of(np.repeat(np.array(cs)[:, None], H, axis=1))
    say("attn_res constant rows H=%d" % H)
    _, _, out = _run(prefix, None, None, -1, w, EPS32, np.zeros((len(cs), H), np.uint16))
    for t, c in enumerate(cs):
        if c > 0:
            np.testing.assert_array_equal(out[t], w)
        elif c < 0:
            np.testing.assert_array_equal(out[t], w ^ 0x8000)
        else:
            assert np.all(synth.bf16_bits_to_f64(out[t]) == 0.0)


@pytest.mark.parametrize("T,H", [(5, 8), (9, 520), (11, 1544), (3, 2048), (6, 3000), (2, 4096),
                                 (33, 4104), (4, 8192), (2048, 7168), (8192, 1024)])
def test_ragged_and_large_shapes(T, H):
    """Rows that end inside a lane's chunk range (H not a multiple of 512),
    the widest row, and prefill-sized token counts; all switches on.  The
    widths cover every workgroup shape of the kernel: 1, 2, 4 and 8 waves
    per row with one 16-byte chunk per lane, and 8 waves with two."""
    from oracle import oracle

    prefix, delta, block, w, out0 = _inputs(T, H, seed=T + H)
    args = (prefix, delta, block, SLOTS - 1, w, EPS32)
    say("attn_res shape T=%d H=%d" % (T, H))
    _compare(_run(*args, out0), oracle.attn_res_zero_block(*args), True, "T=%d H=%d" % (T, H))


def test_deterministic():
    prefix, delta, block, w, out0 = _inputs(320, 7168, seed=71)
    say("attn_res determinism")
    a = _run(prefix, delta, block, 3, w, EPS32, out0)
    b = _run(prefix, delta, block, 3, w, EPS32, out0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_graph_replay_at_varying_shapes():
    """[PR50593 Implementation, item 4]: calls captured into HIP graphs at
    several shapes and replayed interleaved, with eager work between replays;
    every replay equals the eager result."""
    import torch

    shapes = [(1, 7168), (17, 1024), (320, 7168), (3, 128)]
    bufs, expected = {}, {}
    for T, H in shapes:
        prefix, delta, block, w, out0 = _inputs(T, H, seed=72 + T)
        d = dict(p0=dev(prefix), p=dev(prefix), d=dev(delta), b0=dev(block), b=dev(block),
                 w=dev(w), o=dev(out0))
        bufs[(T, H)] = d
        _sync()
        say("attn_res graph eager T=%d H=%d" % (T, H))
        binding.check(binding.lt_attn_res_zero_block(d["p"], d["d"], T, H, d["b"], SLOTS, 2,
                                                     d["w"], EPS32, d["o"], None))
        _sync()
        expected[(T, H)] = (host(d["p"]), host(d["b"]), host(d["o"]))
    s = torch.cuda.Stream()
    graphs = {}
    for (T, H), d in bufs.items():
        d["p"].copy_(d["p0"])
        d["b"].copy_(d["b0"])
        _sync()
        g = torch.cuda.CUDAGraph()
        say("attn_res graph capture T=%d H=%d" % (T, H))
        with torch.cuda.graph(g, stream=s):
            st = binding.lt_attn_res_zero_block(d["p"], d["d"], T, H, d["b"], SLOTS, 2, d["w"],
                                                EPS32, d["o"], torch.cuda.current_stream())
        assert st == binding.LT_OK
        graphs[(T, H)] = g
    for rep, key in enumerate([shapes[2], shapes[0], shapes[3], shapes[1], shapes[2], shapes[0]]):
        d = bufs[key]
        d["p"].copy_(d["p0"])
        d["b"].copy_(d["b0"])
        d["o"].fill_(0)
        _sync()
        junk = torch.randn(1 << 18, device="cuda").sum()
        say("attn_res graph replay %d T=%d H=%d" % (rep, *key))
        graphs[key].replay()
        _sync()
        for got, want in zip((host(d["p"]), host(d["b"]), host(d["o"])), expected[key]):
            np.testing.assert_array_equal(got, want, err_msg="replay %d %s" % (rep, key))
        del junk
    del graphs


def test_invalid_arguments_touch_nothing():
    T, H = 4, 1024
    prefix, delta, block, w, out0 = _inputs(T, H, seed=73)
    pd, dd, bd, wd, od = dev(prefix), dev(delta), dev(block), dev(w), dev(out0)
    _sync()
    say("attn_res invalid arguments")
    call = binding.lt_attn_res_zero_block
    assert call(pd, dd, T, H, bd, SLOTS, SLOTS, wd, EPS32, od) == binding.LT_ERR_INVALID_ARG
    assert call(pd, dd, T, H, bd, SLOTS, 0, wd, -1.0, od) == binding.LT_ERR_INVALID_ARG
    assert call(pd, dd, T, H, None, SLOTS, 0, wd, EPS32, od) == binding.LT_ERR_INVALID_ARG
    assert call(pd, dd, T, H - 4, bd, SLOTS, 0, wd, EPS32, od) == binding.LT_ERR_UNSUPPORTED
    assert call(pd, dd, T, H, bd, SLOTS, 0, wd, EPS32, pd) == binding.LT_ERR_INVALID_ARG
    assert call(pd, dd, T, H, bd, SLOTS, 0, wd, EPS32,
                od.data_ptr() + 2) == binding.LT_ERR_UNSUPPORTED
    assert call(pd, dd, 0, H, bd, SLOTS, 0, wd, EPS32, od) == binding.LT_OK
    _sync()
    np.testing.assert_array_equal(host(pd), prefix)
    np.testing.assert_array_equal(host(bd).reshape(block.shape), block)
    np.testing.assert_array_equal(host(od), out0)
