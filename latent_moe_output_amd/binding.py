"""ctypes binding of liblatenttail.so (the C ABI in include/latent_tail.h).

Argument marshalling only: every function forwards to the C entry point of
the same name.  Pointer arguments accept an integer device address, a torch
tensor (its ``data_ptr()``) or ``None``; ``stream`` accepts an integer
hipStream_t, a ``torch.cuda.Stream`` or ``None`` (the default stream).

The library is loaded on first use from this package directory.  There is no
fallback: if it has not been built, the call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblatenttail.so")

LT_OK = 0
LT_ERR_INVALID_ARG = 1
LT_ERR_UNSUPPORTED = 2
LT_ERR_NO_MEMORY = 3
LT_ERR_HIP = 4
LT_ERR_SCRATCH_LIMIT = 5
LT_NOALLOC_MAX_LATENT = 8 * 1024 * 1024
LT_ATTN_RES_MAX_H = 8192
LT_MAX_L = 2048

_lib = None


class LtError(RuntimeError):
    def __init__(self, status: int):
        self.status = int(status)
        super().__init__(lt_status_string(status))


def load():
    """Load liblatenttail.so (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "liblatenttail.so is not built (%s); run `python -m latent_moe_output_amd.build`"
            % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.lt_latent_tail.argtypes = [vp, ctypes.c_int, i64, i64, vp, ctypes.c_float, vp, i64,
                                   i64, i64, vp, i64, vp]
    lib.lt_latent_tail.restype = ctypes.c_int
    lib.lt_latent_tail_noalloc.argtypes = [vp, ctypes.c_int, i64, i64, vp, ctypes.c_float, vp,
                                           i64, i64, i64, vp, i64, vp]
    lib.lt_latent_tail_noalloc.restype = ctypes.c_int
    lib.lt_latent_tail_residual.argtypes = [vp, ctypes.c_int, i64, i64, vp, ctypes.c_float, vp,
                                            i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.lt_latent_tail_residual.restype = ctypes.c_int
    lib.lt_attn_res_zero_block.argtypes = [vp, vp, i64, i64, vp, i64, i64, vp, ctypes.c_float,
                                           vp, vp]
    lib.lt_attn_res_zero_block.restype = ctypes.c_int
    lib.lt_status_string.argtypes = [ctypes.c_int]
    lib.lt_status_string.restype = ctypes.c_char_p
    lib.lt_reserve.argtypes = [i64, i64, vp]
    lib.lt_reserve.restype = ctypes.c_int
    lib.lt_release_scratch.argtypes = []
    lib.lt_release_scratch.restype = ctypes.c_int
    lib.lt_set_skinny_max_tokens.argtypes = [i64]
    lib.lt_set_skinny_max_tokens.restype = i64
    lib.lt_get_skinny_max_tokens.argtypes = []
    lib.lt_get_skinny_max_tokens.restype = i64
    lib.lt_path_for.argtypes = [i64, i64]
    lib.lt_path_for.restype = ctypes.c_int
    lib.lt_set_kernel_events.argtypes = [vp, vp]
    lib.lt_set_kernel_events.restype = ctypes.c_int
    lib.lt_version.argtypes = []
    lib.lt_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    dp = getattr(x, "data_ptr", None)
    if dp is not None:
        return int(dp())
    raise TypeError("expected a device address, a tensor or None, got %r" % type(x))


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    cs = getattr(s, "cuda_stream", None)
    if cs is not None:
        return int(cs)
    raise TypeError("expected a hipStream_t address, a torch.cuda.Stream or None")


def lt_latent_tail(partials, n_partials, T, L, norm_w, eps, W, H, c0, n, out, ld_out,
                   stream=None) -> int:
    """Forward to the C entry point; returns its status code."""
    return int(load().lt_latent_tail(_ptr(partials), int(n_partials), int(T), int(L),
                                      _ptr(norm_w), float(eps), _ptr(W), int(H), int(c0),
                                      int(n), _ptr(out), int(ld_out), _stream(stream)))


def lt_latent_tail_noalloc(partials, n_partials, T, L, norm_w, eps, W, H, c0, n, out, ld_out,
                           stream=None) -> int:
    """Forward to the C entry point; returns its status code."""
    return int(load().lt_latent_tail_noalloc(_ptr(partials), int(n_partials), int(T), int(L),
                                              _ptr(norm_w), float(eps), _ptr(W), int(H), int(c0),
                                              int(n), _ptr(out), int(ld_out), _stream(stream)))


def lt_latent_tail_residual(partials, n_partials, T, L, norm_w, eps, W, H, c0, n, out, ld_out,
                            prefix, ld_prefix, resid, ld_resid, stream=None) -> int:
    """Forward to the C entry point; returns its status code."""
    return int(load().lt_latent_tail_residual(
        _ptr(partials), int(n_partials), int(T), int(L), _ptr(norm_w), float(eps), _ptr(W),
        int(H), int(c0), int(n), _ptr(out), int(ld_out), _ptr(prefix), int(ld_prefix),
        _ptr(resid), int(ld_resid), _stream(stream)))


def lt_attn_res_zero_block(prefix, delta, T, H, block_residual, num_slots, block_idx, norm_w,
                           eps, out, stream=None) -> int:
    """Forward to the C entry point; returns its status code."""
    return int(load().lt_attn_res_zero_block(_ptr(prefix), _ptr(delta), int(T), int(H),
                                              _ptr(block_residual), int(num_slots),
                                              int(block_idx), _ptr(norm_w), float(eps),
                                              _ptr(out), _stream(stream)))


def lt_status_string(status: int) -> str:
    return load().lt_status_string(int(status)).decode()


def lt_reserve(max_T, L, stream=None) -> int:
    return int(load().lt_reserve(int(max_T), int(L), _stream(stream)))


def lt_release_scratch() -> int:
    return int(load().lt_release_scratch())


def lt_set_skinny_max_tokens(t: int) -> int:
    return int(load().lt_set_skinny_max_tokens(int(t)))


def lt_get_skinny_max_tokens() -> int:
    return int(load().lt_get_skinny_max_tokens())


def lt_path_for(T, n) -> int:
    return int(load().lt_path_for(int(T), int(n)))


def lt_set_kernel_events(before, after) -> int:
    """before/after: raw hipEvent_t handles (ints) or None."""
    return int(load().lt_set_kernel_events(before, after))


def lt_version() -> str:
    return load().lt_version().decode()


def check(status: int) -> None:
    """Raise LtError unless status is LT_OK."""
    if status != LT_OK:
        raise LtError(status)
