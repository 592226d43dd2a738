"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bar: |gpu - oracle| <= 3e-2 + 1.6e-2 * |oracle| on every window element,
and bit-identical everywhere else; bit-exact where the arithmetic is exact
(dyadic inputs, identity projections, split partials, shards).

Workloads are the seeded recipes of latent_moe_output_amd.synth.  Every
workload, the full prefill and ragged sizes included (launched exactly as
the benchmark launches them), is compared with the oracle element by element
over the whole buffer; the oracle runs on all host cores.
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


@pytest.fixture()
def forced():
    """Force the dispatcher threshold for one test, restoring the default."""
    def _set(t):
        binding.lt_set_skinny_max_tokens(t)
    yield _set
    binding.lt_set_skinny_max_tokens(-1)


def _sync():
    import torch

    torch.cuda.synchronize()


def _run_full(wl, seed=0, **kw):
    """GPU result and oracle result for the whole buffer."""
    from oracle import oracle

    d = synth.generate(wl, seed=seed)
    di = DevInputs(d)
    say("case %s T=%d L=%d H=%d P=%d c0=%d n=%d ld=%d norm=%s seed=%d path=%d" % (
        wl.name, wl.T, wl.L, wl.H, wl.P, wl.c0, wl.n, wl.ld_out, wl.norm, seed,
        binding.lt_path_for(wl.T, wl.n)))
    binding.check(di.call(wl, **kw))
    _sync()
    got = host(di.out)
    ref = oracle.latent_tail(d["partials"], d["norm_w"], eps32(wl), d["W"], wl.c0, wl.n, d["out"])
    return d, got, ref


# --------------------------------------------------------------------------
# the configured workloads
# --------------------------------------------------------------------------

def test_tiny_workload():
    wl = synth.WORKLOADS["tiny"]
    _, got, ref = _run_full(wl)
    assert_window_close(got, ref, wl.c0, wl.n, "tiny")


@pytest.mark.parametrize("T", synth.DECODE_TOKENS)
def test_decode_workload(T):
    wl = synth.WORKLOADS["decode"].with_T(T)
    _, got, ref = _run_full(wl)
    assert_window_close(got, ref, wl.c0, wl.n, "decode T=%d" % T)


@pytest.mark.parametrize("T,seed", [(1, 10), (5, 11), (8, 12), (16, 13), (5, 14)])
def test_pages_token_sweep(T, seed):
    """The token counts the pages' own equivalence test sweeps ([PR51253 Key
    source snippets, `_check_matches_replicated`]: 1, 5, 8, 16, 5), on the
    decode shape with a fresh seed per entry."""
    wl = synth.WORKLOADS["decode"].with_T(T)
    _, got, ref = _run_full(wl, seed=seed)
    assert_window_close(got, ref, wl.c0, wl.n, "pages sweep T=%d seed=%d" % (T, seed))


def test_shard_workload():
    wl = synth.WORKLOADS["shard"]
    _, got, ref = _run_full(wl)
    assert_window_close(got, ref, wl.c0, wl.n, "shard")


@pytest.mark.parametrize("name", ["prefill", "ragged", "ragged_nonorm"])
def test_large_workload_full(name):
    """Full-size call, launched exactly as the benchmark launches it (one
    call on the default dispatch), compared with the oracle on every element
    of the whole buffer: the window within tolerance, everything else bit for
    bit ([PR51253 Key source snippets, `_check_matches_replicated`] compares
    the whole output)."""
    wl = synth.WORKLOADS[name]
    _, got, ref = _run_full(wl)
    assert_window_close(got, ref, wl.c0, wl.n, name)


@pytest.mark.parametrize("T,n,c0,ld,P,L", [
    (2000, 7100, 37, 7168, 2, 1024),   # 256 x 256 tiles, 2 stages (224 tiles), ragged both ways
    (1000, 7100, 5, 7120, 1, 1024),    # 128 x 128 tiles, 2 stages
    (500, 7100, 11, 7128, 3, 1024),    # 128 x 128 tiles, 4 stages
    (300, 3000, 8, 3016, 1, 1024),     # 64 x 64 tiles, 4 waves, 4 stages
    (130, 7168, 0, 7176, 1, 1024),     # 64 x 128 tiles, 4 waves, 4 stages
    (130, 7168, 24, 7200, 2, 1032),    # 64 x 128 with a K tail
    (129, 7100, 3, 7112, 1, 1096),     # 64 x 64 with a K tail, ragged T and n
    (2000, 7100, 64, 7168, 1, 1032),   # 256 x 256, LDS epilogue, K tail (L % 128 != 0)
    (1000, 7100, 33, 7136, 2, 1096),   # 128 x 128 / 2 stages with a K tail (unaligned window)
    (500, 7100, 3, 7112, 1, 1160),     # 128 x 128 / 4 stages with a K tail
    (1500, 4000, 1, 4008, 1, 2048),    # widest latent, 128 x 128 / 2 stages (384 tiles)
    (900, 7100, 6, 7112, 2, 1024),     # 128 x 128 / 2 stages, 2 tiles per CU (392 tiles)
    (320, 7100, 5, 7112, 1, 1032),     # 128 x 128 / 4 stages where 64 x 128 needs 2 rounds
    # 256 x 256 on the five-slot ring: every phase of the last K stage
    # (K stages mod 5 = 0..4), the shortest ring (3 stages) and the two-stage
    # kernel below it (2 stages)
    (2000, 7100, 0, 7104, 1, 1240),    # 20 K stages
    (2000, 7100, 8, 7112, 2, 1096),    # 18
    (2000, 7100, 16, 7120, 1, 1160),   # 19
    (2048, 7168, 0, 7176, 1, 1024),    # 16, interior tiles only
    (2000, 7100, 0, 7104, 1, 192),     # 3
    (2000, 7100, 0, 7104, 1, 128),     # 2: two-stage kernel
    # ring launches whose last round is split into 128 x 256 halves (280 tiles:
    # 256 whole, 24 as 48 halves): interior, a ragged last column tile whose
    # second half has 60 columns, and one whose second half is empty (ragged
    # T, K tail)
    (2560, 7168, 0, 7176, 1, 1024),
    (2560, 7100, 0, 7104, 1, 1024),
    (2500, 7012, 8, 7024, 2, 1096),
    # one ring round below 224 tiles, where 128 x 128 tiles would need two
    # rounds of two per CU: 140 tiles (interior), 168 (ragged T and n, K tail)
    (1280, 7168, 0, 7176, 1, 1024),
    (1300, 7100, 16, 7120, 2, 1096),
    # 256 x 128 ping-pong tiles (about one round of 140 .. 240 of them, aligned
    # window): every nk mod 3 with and without a K tail, ragged T (down to 10
    # rows in the last token tile, so its second out quarter is empty) and
    # ragged n (a chunk that crosses the window's end), the widest latent
    # and the fewest K stages it takes (4)
    (1024, 7168, 0, 7176, 1, 1024),    # 224 tiles, interior, nk = 16
    (1000, 7100, 32, 7136, 2, 1096),   # nk = 18, K tail, ragged T and n
    (700, 6000, 8, 6016, 1, 1000),     # nk = 16, K tail, 144 tiles
    (900, 5000, 24, 5032, 3, 1088),    # nk = 17
    (650, 7100, 16, 7120, 1, 1032),    # nk = 17, K tail, 10 rows in the last token tile
    (1500, 4000, 0, 4008, 1, 2048),    # nk = 32
    (600, 7100, 0, 7104, 1, 264),      # nk = 5, K tail
    (640, 7168, 0, 7176, 1, 256),      # nk = 4
    (800, 7100, 0, 7104, 1, 1152),     # nk = 18
    # aligned windows with fewer than 140 tiles of 256 x 128 (128 x 128 tiles,
    # four or two stages): every nk mod 3 with and without a K tail, ragged T
    # (4 rows in the last token tile) and n
    (300, 7100, 8, 7112, 1, 1000),     # nk = 16, K tail
    (500, 7100, 0, 7104, 1, 1160),     # nk = 19, K tail
    (400, 7168, 0, 7176, 2, 1088),     # nk = 17
    (260, 6000, 16, 6024, 1, 1032),    # nk = 17, K tail, 4 rows in the last token tile
    (450, 7100, 24, 7128, 1, 1152),    # nk = 18
    (350, 7000, 0, 7008, 1, 1096),     # nk = 18, K tail
    (320, 7168, 0, 7176, 1, 1024),     # nk = 16, interior
])
def test_gemm_tile_shapes(T, n, c0, ld, P, L):
    """Each GEMM tile shape the dispatcher picks, on ragged T and n with an
    offset window, compared with the oracle on every element (the 2048 x 7168
    case runs the exact 256 x 256 ring instance the benchmark times at
    T = 8192)."""
    wl = synth.Workload("tiles", T=T, L=L, H=c0 + n + 3, P=P, c0=c0, n=n, ld_out=ld,
                        part_std=0.6)
    assert binding.lt_path_for(T, n) == 2
    _, got, ref = _run_full(wl, seed=T + n)
    assert_window_close(got, ref, c0, n, "tiles T=%d n=%d" % (T, n))


# --------------------------------------------------------------------------
# dispatch boundary and forced paths
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [63, 64, 65, 100])
@pytest.mark.parametrize("thr", [0, 1000, -1])
def test_dispatch_boundary_both_paths(T, thr, forced):
    forced(thr)
    wl = synth.Workload("boundary", T=T, L=1024, H=1536, P=2, c0=320, n=800, ld_out=1544,
                        part_std=0.7)
    _, got, ref = _run_full(wl, seed=T)
    assert_window_close(got, ref, wl.c0, wl.n, "T=%d thr=%d" % (T, thr))


@pytest.mark.parametrize("P", [1, 3])
def test_paths_give_identical_latents(P, forced):
    """With W = I (H = L) and out = 0 the output is the latent itself; the
    weight-streaming and GEMM paths must produce the same bits, and those
    bits must be the oracle's latent within tolerance (one partial: both
    kernels stage the tile through LDS; three: both sum in registers)."""
    from oracle import oracle

    L, T = 1024, 48
    rng = np.random.Generator(np.random.PCG64(3))
    parts = synth.to_bf16_bits(rng.standard_normal((P, T, L)) * 0.6)
    nw = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(L))
    eye = synth.to_bf16_bits(np.eye(L))
    outs = []
    for thr in (1000, 0):
        forced(thr)
        d = dict(partials=parts, norm_w=nw, W=eye, out=np.zeros((T, L), np.uint16))
        di = DevInputs(d)
        wl = synth.Workload("eye", T=T, L=L, H=L, P=P, c0=0, n=L, ld_out=L)
        say("identity latent P=%d thr=%d" % (P, thr))
        binding.check(di.call(wl))
        _sync()
        outs.append(host(di.out))
    assert np.array_equal(outs[0], outs[1])
    y = oracle.latent(parts, nw, eps32(synth.WORKLOADS["tiny"]))
    assert_window_close(outs[0], y, 0, L, "identity latent")


# --------------------------------------------------------------------------
# exact cases: bit-exact against the oracle
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [5, 40, 200])
@pytest.mark.parametrize("P", [1, 2])
def test_dyadic_inputs_are_bit_exact(T, P):
    """Norm off, small-integer latent, W in {-2..2}/16: every partial sum and
    projection is exact in fp32, so only the final rounding remains and the
    GPU must equal the oracle bit for bit (one partial: the latent staged
    through LDS goes straight to the projection)."""
    from oracle import oracle

    rng = np.random.Generator(np.random.PCG64(4))
    L, H = 1024, 640
    A = rng.integers(-2, 3, (P, T, L)).astype(np.float64)
    Wm = rng.integers(-2, 3, (H, L)) / 16.0
    C = rng.integers(-512, 513, (T, H)) / 8.0
    d = dict(partials=synth.to_bf16_bits(A), norm_w=None, W=synth.to_bf16_bits(Wm),
             out=synth.to_bf16_bits(C))
    wl = synth.Workload("dyadic", T=T, L=L, H=H, P=P, c0=64, n=520, ld_out=H, norm=False)
    di = DevInputs(d)
    say("dyadic T=%d P=%d" % (T, P))
    binding.check(di.call(wl))
    _sync()
    ref = oracle.latent_tail(d["partials"], None, 0.0, d["W"], wl.c0, wl.n, d["out"])
    np.testing.assert_array_equal(host(di.out), ref)


@pytest.mark.parametrize("T", [16, 300])
def test_constant_rows_normalise_to_weight(T):
    """Constant rows normalise to +-w (c^2 >> eps) and zero rows to 0; seen
    bit-exactly through W = I."""
    L = 512
    rng = np.random.Generator(np.random.PCG64(5))
    nw = synth.to_bf16_bits(1 + 0.2 * rng.standard_normal(L))
    cs = np.resize(np.array([1.5, -0.75, 0.0, 40.0, -3.0]), T)
    parts = synth.to_bf16_bits(np.repeat(cs[:, None], L, axis=1))[None]
    d = dict(partials=parts, norm_w=nw, W=synth.to_bf16_bits(np.eye(L)),
             out=np.zeros((T, L), np.uint16))
    di = DevInputs(d)
    wl = synth.Workload("const", T=T, L=L, H=L, P=1, c0=0, n=L, ld_out=L)
    say("constant rows T=%d" % T)
    binding.check(di.call(wl))
    _sync()
    got = host(di.out)
    for t, c in enumerate(cs):
        if c > 0:
            np.testing.assert_array_equal(got[t], nw)
        elif c < 0:
            np.testing.assert_array_equal(got[t], nw ^ 0x8000)
        else:
            assert np.all(synth.bf16_bits_to_f64(got[t]) == 0.0)


@pytest.mark.parametrize("T", [8, 257])
def test_shards_concatenate_bit_exact(T):
    """Eight column shards c0 = k*H/8 written in turn equal the full call bit
    for bit (the accumulation order of an element does not depend on the
    window)."""
    wl = synth.Workload("shards", T=T, L=1024, H=1792, P=2, c0=0, n=1792, ld_out=1800,
                        part_std=0.7)
    d = synth.generate(wl, seed=6)
    full = DevInputs(d)
    say("shards T=%d full" % T)
    binding.check(full.call(wl))
    part = DevInputs(d)
    for k in range(8):
        binding.check(part.call(wl, c0=k * 224, n=224))
    _sync()
    np.testing.assert_array_equal(host(part.out), host(full.out))


def test_pingpong_tiles_bit_exact():
    """The ping-pong 256 x 128 kernel (the full 7168-column window at T = 1000)
    equals, bit for bit, eight 896-column shards that run the 32 x 64 and
    128 x 128 kernels, and two unaligned half windows that run 128 x 128."""
    wl = synth.Workload("pingpong", T=1000, L=1024, H=7176, P=1, c0=0, n=7168,
                        ld_out=7176, part_std=0.7)
    d = synth.generate(wl, seed=23)
    full = DevInputs(d)
    say("ping-pong tiles: full window")
    binding.check(full.call(wl))
    part = DevInputs(d)
    for k in range(8):
        say("ping-pong tiles: shard %d" % k)
        binding.check(part.call(wl, c0=k * 896, n=896))
    _sync()
    np.testing.assert_array_equal(host(part.out), host(full.out))
    odd = DevInputs(d)
    binding.check(odd.call(wl, c0=0, n=3581))
    binding.check(odd.call(wl, c0=3581, n=3587))
    _sync()
    np.testing.assert_array_equal(host(odd.out), host(full.out))


def test_split_last_round_bit_exact():
    """A ring launch whose last round runs as half-width tiles (T = 2560 over
    7168 columns: 280 tiles of 256 x 256, the last 24 as 48 halves) equals,
    bit for bit, eight 896-column shards that run the 128 x 128 kernel: the
    halves keep every output's K order."""
    wl = synth.Workload("split_round", T=2560, L=1024, H=7168, P=1, c0=0, n=7168,
                        ld_out=7168, part_std=0.7)
    d = synth.generate(wl, seed=17)
    full = DevInputs(d)
    say("split last round: full window")
    binding.check(full.call(wl))
    part = DevInputs(d)
    for k in range(8):
        say("split last round: shard %d" % k)
        binding.check(part.call(wl, c0=k * 896, n=896))
    _sync()
    np.testing.assert_array_equal(host(part.out), host(full.out))


@pytest.mark.parametrize("T,H,norm,L", [(7, 512, True, 1024), (20, 7168, True, 1024),
                                        (48, 512, True, 1024), (48, 512, False, 1024),
                                        (64, 7168, True, 1024), (130, 512, True, 1024),
                                        (130, 512, False, 1024), (300, 512, True, 264),
                                        (1000, 1024, False, 1024), (1023, 512, True, 1024),
                                        (1023, 512, False, 1024), (1024, 512, True, 1024),
                                        (2048, 7168, False, 1024), (2048, 7168, True, 1024)])
def test_split_partials_bit_exact(T, H, norm, L):
    """[X, Y, -Y] and [X/2, X/2] give the same bits as [X].  With the norm off
    the large-token path multiplies one partial in place and sums several
    first, so this also ties the two routes together; the norm kernel splits
    a 16-token tile over 1..16 workgroups depending on T (T = 130 to 2048
    here), staging one partial straight into LDS and summing several in
    registers; on the weight-streaming path (T <= 64) one partial is staged
    through LDS (two tiles at a time past 32 tokens) while several are summed
    in registers.  The one-partial result is checked against the oracle on
    three rows."""
    from oracle import oracle

    wl = synth.Workload("split", T=T, L=L, H=H, P=1, c0=0, n=H, ld_out=H, norm=norm)
    d = synth.generate(wl, seed=7)
    X = d["partials"]
    Y = synth.generate(wl, seed=8)["partials"]
    half = synth.to_bf16_bits(synth.bf16_bits_to_f64(X) / 2)
    results = []
    for parts in (X, np.concatenate([X, Y, Y ^ 0x8000]), np.concatenate([half, half])):
        dd = dict(d, partials=parts)
        di = DevInputs(dd)
        say("split partials T=%d H=%d L=%d norm=%s P=%d" % (T, H, L, norm, parts.shape[0]))
        binding.check(di.call(wl))
        _sync()
        results.append(host(di.out))
    np.testing.assert_array_equal(results[1], results[0])
    np.testing.assert_array_equal(results[2], results[0])
    rows = sorted({0, T // 2, T - 1})
    ref = oracle.latent_tail(X[:, rows, :], d["norm_w"], eps32(wl), d["W"], 0, H, d["out"][rows])
    assert_window_close(results[0][rows], ref, 0, H, "split T=%d norm=%s" % (T, norm))


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,L,H,P,c0,n,ld", [
    (3, 8, 40, 1, 1, 5, 45),          # smallest latent, odd window
    (9, 72, 100, 2, 37, 63, 101),     # ragged latent (not a multiple of 64/128)
    (70, 72, 100, 3, 0, 100, 100),    # same, GEMM path
    (5, 2048, 300, 1, 13, 257, 333),  # widest latent, skinny
    (90, 2048, 300, 2, 13, 257, 333), # widest latent, GEMM
    (1, 1024, 7168, 1, 7167, 1, 7168),  # last column only
    (33, 1024, 520, 1, 3, 517, 523),  # odd c0 and stride: scalar epilogue
    (129, 1024, 520, 1, 3, 517, 523), # same on the GEMM path
    (300, 1024, 1000, 5, 8, 991, 1016),
])
def test_edge_shapes(T, L, H, P, c0, n, ld):
    wl = synth.Workload("edge", T=T, L=L, H=H, P=P, c0=c0, n=n, ld_out=ld, part_std=0.6)
    _, got, ref = _run_full(wl, seed=T + L)
    assert_window_close(got, ref, c0, n, "edge T=%d L=%d" % (T, L))


@pytest.mark.parametrize("T", [1, 17, 33, 64])
@pytest.mark.parametrize("n,L", [(7168, 1024), (7100, 1024), (5000, 264), (4097, 1024),
                                 (9000, 520), (12, 1024)])
@pytest.mark.parametrize("P", [1, 2])
def test_skinny_row_blocks(T, n, L, P, forced):
    """Weight-streaming path over window widths whose row blocks (4..32 rows,
    one or two MFMA tiles, a short last block) cover every epilogue case, with
    the latent staged through LDS (one partial) and summed in registers (two)."""
    forced(64)
    wl = synth.Workload("rowblk", T=T, L=L, H=n + 11, P=P, c0=5, n=n, ld_out=n + 13,
                        part_std=0.6)
    assert binding.lt_path_for(T, n) == 1
    _, got, ref = _run_full(wl, seed=T * 7 + n)
    assert_window_close(got, ref, 5, n, "rowblk T=%d n=%d L=%d" % (T, n, L))


@pytest.mark.parametrize("T", [32, 33, 64])
@pytest.mark.parametrize("L", [1536, 2048])
@pytest.mark.parametrize("P", [1, 2])
def test_skinny_widest_latent_full_launches(T, L, P, forced):
    """Latents over 1024 wide run at most 32 tokens per weight-streaming
    launch (two 16-token tiles; staged through LDS, 128 KB, with one partial):
    a full launch, a launch plus one token, and two full launches."""
    forced(64)
    wl = synth.Workload("wide", T=T, L=L, H=1100, P=P, c0=9, n=1031, ld_out=1104,
                        part_std=0.6)
    assert binding.lt_path_for(T, wl.n) == 1
    _, got, ref = _run_full(wl, seed=T + L + P)
    assert_window_close(got, ref, wl.c0, wl.n, "wide T=%d L=%d P=%d" % (T, L, P))


def test_sentinels_outside_window_survive():
    """NaN payloads, -0.0 and +-9984 outside the window and in the padding."""
    from oracle import oracle

    T, L, H, ld = 70, 256, 96, 103
    wl = synth.Workload("sent", T=T, L=L, H=H, P=1, c0=17, n=41, ld_out=ld)
    d = synth.generate(wl, seed=9)
    sentinels = np.array([0x7FA1, 0xFFC3, 0x8000, 0x461C, 0xC61C, 0x0001], dtype=np.uint16)
    out = np.resize(sentinels, (T, ld)).astype(np.uint16)
    out[:, 17:58] = d["out"][:, 17:58]
    d["out"] = out
    for thr in (1000, 0):
        binding.lt_set_skinny_max_tokens(thr)
        di = DevInputs(d)
        say("sentinels thr=%d" % thr)
        binding.check(di.call(wl))
        _sync()
        ref = oracle.latent_tail(d["partials"], d["norm_w"], eps32(wl), d["W"], 17, 41, out)
        assert_window_close(host(di.out), ref, 17, 41, "sentinels thr=%d" % thr)
    binding.lt_set_skinny_max_tokens(-1)


def test_empty_calls_launch_nothing():
    wl = synth.WORKLOADS["tiny"]
    d = synth.generate(wl, seed=10)
    di = DevInputs(d)
    say("empty calls")
    assert di.call(wl, T=0) == binding.LT_OK
    assert di.call(wl, n=0) == binding.LT_OK
    _sync()
    np.testing.assert_array_equal(host(di.out), d["out"])


def test_invalid_arguments_leave_out_untouched():
    wl = synth.WORKLOADS["tiny"]
    d = synth.generate(wl, seed=11)
    di = DevInputs(d)
    P, T, L = d["partials"].shape
    say("invalid arguments")
    cases = [
        dict(c0=100, n=29),                     # window beyond H
        dict(eps=float("nan")),
        dict(eps=-1.0),
    ]
    for kw in cases:
        assert di.call(wl, **kw) == binding.LT_ERR_INVALID_ARG, kw
    # misaligned W
    assert binding.lt_latent_tail(di.partials, P, T, L, di.norm_w, 1e-6, di.W.data_ptr() + 2,
                                  wl.H - 1, 0, 4, di.out, wl.ld_out) == binding.LT_ERR_UNSUPPORTED
    # out overlapping W
    assert binding.lt_latent_tail(di.partials, P, T, L, di.norm_w, 1e-6, di.W, wl.H, 0, 4,
                                  di.W, wl.ld_out) == binding.LT_ERR_INVALID_ARG
    # L not a multiple of 8
    assert binding.lt_latent_tail(di.partials, P, T, L - 4, di.norm_w, 1e-6, di.W, wl.H, 0, 4,
                                  di.out, wl.ld_out) == binding.LT_ERR_UNSUPPORTED
    _sync()
    np.testing.assert_array_equal(host(di.out), d["out"])


# --------------------------------------------------------------------------
# determinism, streams, graph capture
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [16, 1000])
def test_bitwise_deterministic(T):
    wl = synth.WORKLOADS["decode"].with_T(T)
    d = synth.generate(wl, seed=12)
    di = DevInputs(d)
    outs = []
    for _ in range(3):
        di.reset_out()
        say("determinism T=%d" % T)
        binding.check(di.call(wl))
        _sync()
        outs.append(host(di.out))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_non_default_stream():
    import torch

    wl = synth.WORKLOADS["shard"]
    d = synth.generate(wl, seed=13)
    di = DevInputs(d)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("side stream")
    binding.check(di.call(wl, stream=s))
    s.synchronize()
    got_side = host(di.out)
    di.reset_out()
    binding.check(di.call(wl))
    _sync()
    np.testing.assert_array_equal(got_side, host(di.out))


@pytest.mark.parametrize("T", [8, 777])
def test_graph_capture_and_replay(T):
    """Capture one call into a HIP graph (after lt_reserve) and replay it
    several times, with eager work and synchronisation between replays; every
    replay must match the eager result."""
    import torch

    wl = synth.Workload("graph", T=T, L=1024, H=2048, P=2, c0=512, n=1024, ld_out=2048,
                        part_std=0.7)
    d = synth.generate(wl, seed=14)
    di = DevInputs(d)
    say("graph eager T=%d" % T)
    binding.check(di.call(wl))
    _sync()
    expected = host(di.out)

    s = torch.cuda.Stream()
    assert binding.lt_reserve(T, wl.L, s) == binding.LT_OK
    g = torch.cuda.CUDAGraph()
    di.reset_out()
    torch.cuda.synchronize()
    say("graph capture T=%d" % T)
    with torch.cuda.graph(g, stream=s):
        status = di.call(wl, stream=torch.cuda.current_stream())
    assert status == binding.LT_OK
    for rep in range(4):
        di.reset_out()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()     # eager work between replays
        say("graph replay %d T=%d" % (rep, T))
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(di.out), expected)
        del junk
    del g


@pytest.mark.parametrize("T", [2560, 1000])
def test_split_ring_graph_replay(T):
    """The ring launch whose last round runs as half tiles (T = 2560 over
    7168 columns) and the ping-pong 256 x 128 kernel (T = 1000), each
    captured into a HIP graph after lt_reserve and replayed three times with
    eager work in between: every replay equals the eager call bit for bit."""
    import torch

    wl = synth.Workload("split_graph", T=T, L=1024, H=7168, P=1, c0=0, n=7168,
                        ld_out=7168, part_std=0.7)
    di = DevInputs(synth.generate(wl, seed=23))
    say("graph T=%d: eager" % T)
    binding.check(di.call(wl))
    _sync()
    want = host(di.out)
    s = torch.cuda.Stream()
    assert binding.lt_reserve(wl.T, wl.L, s) == binding.LT_OK
    di.reset_out()
    _sync()
    g = torch.cuda.CUDAGraph()
    say("graph T=%d: capture" % T)
    with torch.cuda.graph(g, stream=s):
        status = di.call(wl, stream=torch.cuda.current_stream())
    assert status == binding.LT_OK
    for rep in range(3):
        di.reset_out()
        _sync()
        junk = torch.randn(1 << 20, device="cuda").sum()
        say("graph T=%d: replay %d" % (T, rep))
        g.replay()
        _sync()
        np.testing.assert_array_equal(host(di.out), want)
        del junk
    del g


def test_graphs_of_several_shapes_survive_scratch_growth():
    """Graph replay at varying shapes ([PR50593 Implementation, item 4]):
    graphs captured at T = 8 (weight streaming), 100 and 777 (sum+RMSNorm
    and GEMM through the stream's scratch) after lt_reserve(777); a call that
    would have to grow the scratch under capture is refused; an eager
    T = 2000 call on the same stream then grows the scratch; the graphs are
    replayed interleaved with each other and with further eager calls, and
    every replay must match its eager result bit for bit (the buffer a graph
    captured is kept when a larger one takes over)."""
    import torch

    from oracle import oracle

    def wl_of(T):
        return synth.Workload("gshape", T=T, L=1024, H=2048, P=2, c0=512, n=1024, ld_out=2048,
                              part_std=0.7)

    shapes = (8, 100, 777)
    inputs = {T: DevInputs(synth.generate(wl_of(T), seed=40 + T)) for T in shapes + (2000,)}
    expected = {}
    for T in shapes + (2000,):
        say("graph shapes: eager T=%d" % T)
        binding.check(inputs[T].call(wl_of(T)))
        _sync()
        expected[T] = host(inputs[T].out)
    d2 = inputs[2000].d
    ref2000 = oracle.latent_tail(d2["partials"], d2["norm_w"], eps32(wl_of(2000)), d2["W"], 512,
                                 1024, d2["out"])
    assert_window_close(expected[2000], ref2000, 512, 1024, "graph shapes eager T=2000")

    s = torch.cuda.Stream()
    assert binding.lt_release_scratch() == binding.LT_OK
    assert binding.lt_reserve(777, 1024, s) == binding.LT_OK
    graphs = {}
    for T in shapes:
        inputs[T].reset_out()
        _sync()
        g = torch.cuda.CUDAGraph()
        say("graph shapes: capture T=%d" % T)
        with torch.cuda.graph(g, stream=s):
            status = inputs[T].call(wl_of(T), stream=torch.cuda.current_stream())
        assert status == binding.LT_OK
        graphs[T] = g
    # growth is refused while the stream is being captured (nothing launched)
    big = inputs[2000]
    big.reset_out()
    _sync()
    g_bad = torch.cuda.CUDAGraph()
    marker = torch.zeros(4, device="cuda")
    say("graph shapes: capture that would grow the scratch")
    with torch.cuda.graph(g_bad, stream=s):
        marker.add_(1.0)
        status = big.call(wl_of(2000), stream=torch.cuda.current_stream())
    assert status == binding.LT_ERR_NO_MEMORY
    del g_bad
    _sync()
    np.testing.assert_array_equal(host(big.out), d2["out"])

    order = (777, 8, 100, 777, 100, 8)
    for rep, T in enumerate(order):
        # an eager call on the capture stream between replays; the first one
        # grows the scratch past what the graphs captured
        big.reset_out()
        _sync()
        say("graph shapes: eager T=2000 before replay %d" % rep)
        binding.check(big.call(wl_of(2000), stream=s))
        s.synchronize()
        np.testing.assert_array_equal(host(big.out), expected[2000])
        inputs[T].reset_out()
        _sync()
        say("graph shapes: replay %d of T=%d" % (rep, T))
        graphs[T].replay()
        _sync()
        np.testing.assert_array_equal(host(inputs[T].out), expected[T],
                                      err_msg="replay %d T=%d" % (rep, T))
    del graphs

