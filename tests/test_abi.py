"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The shared library must load, export every function declared in
include/*.h, and reject bad arguments before touching the GPU.
"""
from __future__ import annotations

import glob
import os
import re

import pytest

from latent_moe_output_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"LT_API\s+[\w\s\*]*?\b(lt_\w+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for must in ("lt_latent_tail", "lt_status_string", "lt_reserve", "lt_set_skinny_max_tokens"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_only_the_c_abi_is_exported():
    import subprocess

    res = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH],
                         capture_output=True, text=True, check=True)
    text_syms = [ln.split()[-1] for ln in res.stdout.splitlines() if " T " in ln]
    assert sorted(text_syms) == _declared_functions()


def test_version_and_status_strings(lib):
    assert "gfx950" in binding.lt_version()
    for code in range(6):
        assert binding.lt_status_string(code).startswith("LT_")
    assert binding.lt_status_string(99) == "unknown lt status"


def test_dispatcher_threshold(lib):
    prev = binding.lt_set_skinny_max_tokens(-1)
    try:
        assert binding.lt_get_skinny_max_tokens() == 64
        assert binding.lt_path_for(0, 7168) == 0
        assert binding.lt_path_for(5, 0) == 0
        assert binding.lt_path_for(64, 7168) == 1
        assert binding.lt_path_for(65, 7168) == 2
        assert binding.lt_set_skinny_max_tokens(0) == 64
        assert binding.lt_path_for(1, 7168) == 2
        binding.lt_set_skinny_max_tokens(1 << 20)
        assert binding.lt_path_for(8192, 7168) == 1
    finally:
        binding.lt_set_skinny_max_tokens(-1 if prev == 64 else prev)


FAKE = 1 << 32   # a 16-byte-aligned address that is never dereferenced


@pytest.mark.parametrize("kw,code", [
    (dict(n_partials=0), binding.LT_ERR_INVALID_ARG),
    (dict(T=-1), binding.LT_ERR_INVALID_ARG),
    (dict(L=0), binding.LT_ERR_INVALID_ARG),
    (dict(H=0), binding.LT_ERR_INVALID_ARG),
    (dict(c0=-1), binding.LT_ERR_INVALID_ARG),
    (dict(n=-1), binding.LT_ERR_INVALID_ARG),
    (dict(c0=7000, n=200), binding.LT_ERR_INVALID_ARG),
    (dict(ld_out=7167), binding.LT_ERR_INVALID_ARG),
    (dict(eps=float("inf")), binding.LT_ERR_INVALID_ARG),
    (dict(eps=float("nan")), binding.LT_ERR_INVALID_ARG),
    (dict(eps=-1e-6), binding.LT_ERR_INVALID_ARG),
    (dict(partials=None), binding.LT_ERR_INVALID_ARG),
    (dict(W=None), binding.LT_ERR_INVALID_ARG),
    (dict(out=None), binding.LT_ERR_INVALID_ARG),
    (dict(L=1020), binding.LT_ERR_UNSUPPORTED),
    (dict(L=4096), binding.LT_ERR_UNSUPPORTED),
    (dict(partials=FAKE + 8), binding.LT_ERR_UNSUPPORTED),
    (dict(W=FAKE + 2), binding.LT_ERR_UNSUPPORTED),
    (dict(norm_w=FAKE + 4), binding.LT_ERR_UNSUPPORTED),
    (dict(out=FAKE + 1), binding.LT_ERR_UNSUPPORTED),
    (dict(out=FAKE), binding.LT_ERR_INVALID_ARG),            # out == partials
    (dict(out=FAKE + (1 << 20)), binding.LT_ERR_INVALID_ARG),  # out inside W
])
def test_invalid_arguments_are_rejected_before_launch(lib, kw, code):
    args = dict(partials=FAKE, n_partials=1, T=16, L=1024, norm_w=FAKE + (1 << 30), eps=1e-6,
                W=FAKE + (1 << 20), H=7168, c0=0, n=7168, out=FAKE + (1 << 31), ld_out=7168)
    args.update(kw)
    assert binding.lt_latent_tail(**args) == code


def test_empty_calls_return_ok_without_launch(lib):
    args = dict(partials=FAKE, n_partials=1, T=16, L=1024, norm_w=None, eps=1e-6,
                W=FAKE + (1 << 20), H=7168, c0=0, n=7168, out=FAKE + (1 << 31), ld_out=7168)
    assert binding.lt_latent_tail(**dict(args, T=0)) == binding.LT_OK
    assert binding.lt_latent_tail(**dict(args, n=0)) == binding.LT_OK
    assert binding.lt_latent_tail(**dict(args, T=0, partials=None, W=None, out=None)) == binding.LT_OK


def test_reserve_rejects_bad_sizes(lib):
    assert binding.lt_reserve(-1, 1024) == binding.LT_ERR_INVALID_ARG
    assert binding.lt_reserve(4, 0) == binding.LT_ERR_INVALID_ARG
    assert binding.lt_reserve(0, 1024) == binding.LT_OK


# residual form: its extra arguments are validated before anything launches
_RES_BASE = dict(partials=FAKE, n_partials=1, T=16, L=1024, norm_w=FAKE + (1 << 30), eps=1e-6,
                 W=FAKE + (1 << 20), H=7168, c0=8, n=7000, out=FAKE + (1 << 31), ld_out=7168,
                 prefix=FAKE + (1 << 33), ld_prefix=7168, resid=FAKE + (1 << 34),
                 ld_resid=7168)


@pytest.mark.parametrize("kw,code", [
    (dict(prefix=None), binding.LT_ERR_INVALID_ARG),
    (dict(resid=None), binding.LT_ERR_INVALID_ARG),
    (dict(ld_prefix=7007), binding.LT_ERR_INVALID_ARG),          # below c0 + n
    (dict(ld_resid=7007), binding.LT_ERR_INVALID_ARG),
    (dict(prefix=FAKE + (1 << 33) + 1), binding.LT_ERR_UNSUPPORTED),
    (dict(resid=FAKE + (1 << 34) + 1), binding.LT_ERR_UNSUPPORTED),
    (dict(resid=FAKE + (1 << 31) + 64), binding.LT_ERR_INVALID_ARG),   # resid inside out
    (dict(prefix=FAKE + (1 << 31)), binding.LT_ERR_INVALID_ARG),       # prefix is out
    (dict(resid=FAKE + (1 << 20)), binding.LT_ERR_INVALID_ARG),        # resid inside W
    (dict(resid=FAKE), binding.LT_ERR_INVALID_ARG),                    # resid is partials
    (dict(resid=FAKE + (1 << 33) + 2), binding.LT_ERR_INVALID_ARG),    # shifted onto prefix
    (dict(resid=FAKE + (1 << 33), ld_resid=7176), binding.LT_ERR_INVALID_ARG),  # same base, other stride
    (dict(eps=-1.0), binding.LT_ERR_INVALID_ARG),                      # the tail's own checks
    (dict(L=1000 + 4), binding.LT_ERR_UNSUPPORTED),
])
def test_residual_invalid_arguments_are_rejected(lib, kw, code):
    assert binding.lt_latent_tail_residual(**dict(_RES_BASE, **kw)) == code


def test_residual_empty_calls_launch_nothing(lib):
    assert binding.lt_latent_tail_residual(**dict(_RES_BASE, T=0)) == binding.LT_OK
    assert binding.lt_latent_tail_residual(**dict(_RES_BASE, n=0)) == binding.LT_OK


def test_noalloc_entry_point_validates_like_the_tail(lib):
    """lt_latent_tail_noalloc shares the tail's argument checks (all before
    any launch); empty calls return LT_OK."""
    args = dict(partials=FAKE, n_partials=1, T=16, L=1024, norm_w=FAKE + (1 << 30), eps=1e-6,
                W=FAKE + (1 << 20), H=7168, c0=0, n=7168, out=FAKE + (1 << 31), ld_out=7168)
    for kw, code in ((dict(n_partials=0), binding.LT_ERR_INVALID_ARG),
                     (dict(eps=-1.0), binding.LT_ERR_INVALID_ARG),
                     (dict(L=1020), binding.LT_ERR_UNSUPPORTED),
                     (dict(out=FAKE), binding.LT_ERR_INVALID_ARG),
                     (dict(T=0), binding.LT_OK), (dict(n=0), binding.LT_OK)):
        assert binding.lt_latent_tail_noalloc(**dict(args, **kw)) == code, kw


_AR = dict(prefix=FAKE, delta=FAKE + (1 << 24), T=4, H=1024, block_residual=FAKE + (1 << 25),
           num_slots=3, block_idx=1, norm_w=FAKE + (1 << 26), eps=1e-6, out=FAKE + (1 << 27))


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), binding.LT_ERR_INVALID_ARG),
    (dict(H=0), binding.LT_ERR_INVALID_ARG),
    (dict(block_idx=3), binding.LT_ERR_INVALID_ARG),
    (dict(block_idx=-2), binding.LT_ERR_INVALID_ARG),
    (dict(num_slots=-1, block_idx=-1), binding.LT_ERR_INVALID_ARG),
    (dict(eps=float("nan")), binding.LT_ERR_INVALID_ARG),
    (dict(eps=-1.0), binding.LT_ERR_INVALID_ARG),
    (dict(prefix=None), binding.LT_ERR_INVALID_ARG),
    (dict(out=None), binding.LT_ERR_INVALID_ARG),
    (dict(block_residual=None), binding.LT_ERR_INVALID_ARG),
    (dict(H=1020), binding.LT_ERR_UNSUPPORTED),
    (dict(H=8200), binding.LT_ERR_UNSUPPORTED),
    (dict(prefix=FAKE + 8), binding.LT_ERR_UNSUPPORTED),
    (dict(delta=FAKE + (1 << 24) + 2), binding.LT_ERR_UNSUPPORTED),
    (dict(norm_w=FAKE + (1 << 26) + 4), binding.LT_ERR_UNSUPPORTED),
    (dict(out=FAKE + (1 << 27) + 8), binding.LT_ERR_UNSUPPORTED),
    (dict(block_residual=FAKE + (1 << 25) + 8), binding.LT_ERR_UNSUPPORTED),
    (dict(out=FAKE), binding.LT_ERR_INVALID_ARG),                     # out is prefix
    (dict(out=FAKE + (1 << 25) + 2048), binding.LT_ERR_INVALID_ARG),  # out inside the block
    (dict(block_residual=FAKE + (1 << 24)), binding.LT_ERR_INVALID_ARG),  # block is delta
    (dict(delta=FAKE + 4096), binding.LT_ERR_INVALID_ARG),            # delta inside prefix
    (dict(norm_w=FAKE + 1024), binding.LT_ERR_INVALID_ARG),           # weight inside prefix
    (dict(T=0), binding.LT_OK),
    (dict(T=0, prefix=None, out=None), binding.LT_OK),
])
def test_attn_res_arguments_are_checked_before_launch(lib, kw, code):
    assert binding.lt_attn_res_zero_block(**dict(_AR, **kw)) == code


def test_attn_res_optional_buffers_may_be_null(lib):
    """No delta, no block write, no norm: only prefix and out are needed (T
    = 0, so nothing launches)."""
    assert binding.lt_attn_res_zero_block(FAKE, None, 0, 1024, None, 0, -1, None, 0.0,
                                          FAKE + (1 << 27)) == binding.LT_OK
