"""CPU fp64 oracle for the latent-MoE output tail (Python side).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The HIP library and
its binding never import it, and it imports nothing from them.

The arithmetic lives in ``lto.c`` (plain C, fp64, OpenMP over rows); this file
only builds that shared object with gcc and marshals numpy arrays into it.
bf16 values travel as ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lto.c")
_LIB = os.path.join(_HERE, "liblto.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile lto.c into liblto.so with gcc (-O2, no FMA contraction)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    i64 = ctypes.c_int64
    lib.lto_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.lto_bf16_to_f64.restype = ctypes.c_double
    lib.lto_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.lto_f64_to_bf16.restype = ctypes.c_uint16
    lib.lto_max_threads.argtypes = []
    lib.lto_max_threads.restype = ctypes.c_int
    lib.lto_latent.argtypes = [u16p, ctypes.c_int, i64, i64, u16p, ctypes.c_double, u16p]
    lib.lto_latent.restype = ctypes.c_int
    lib.lto_latent_tail.argtypes = [u16p, ctypes.c_int, i64, i64, u16p, ctypes.c_double,
                                    u16p, i64, i64, i64, u16p, i64, ctypes.c_int]
    lib.lto_latent_tail.restype = ctypes.c_int
    lib.lto_latent_tail_residual.argtypes = [u16p, ctypes.c_int, i64, i64, u16p, ctypes.c_double,
                                             u16p, i64, i64, i64, u16p, i64, u16p, i64, u16p,
                                             i64, ctypes.c_int]
    lib.lto_latent_tail_residual.restype = ctypes.c_int
    lib.lto_attn_res_zero_block.argtypes = [u16p, u16p, i64, i64, u16p, i64, i64, u16p,
                                            ctypes.c_double, u16p]
    lib.lto_attn_res_zero_block.restype = ctypes.c_int
    _lib = lib
    return lib


def _u16(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 arrays must be uint16 bit patterns, got %s" % a.dtype)
    return a


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_uint16)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def max_threads() -> int:
    return int(_load().lto_max_threads())


def f64_to_bf16(x: float) -> int:
    """bf16 bits of x, round to nearest, ties to even (the oracle's rounding)."""
    return int(_load().lto_f64_to_bf16(float(x)))


def bf16_to_f64(h: int) -> float:
    return float(_load().lto_bf16_to_f64(int(h)))


def latent(partials, norm_w, eps):
    """y[T][L] bf16 bits: partial sum, bf16 round trip, optional RMSNorm.

    partials: uint16 [P][T][L]; norm_w: uint16 [L] or None.
    """
    p = _u16(partials)
    P, T, L = p.shape
    w = _u16(norm_w)
    if w is not None and w.shape != (L,):
        raise ValueError("norm_w must have shape (L,)")
    y = np.zeros((T, L), dtype=np.uint16)
    rc = _load().lto_latent(_ptr(p), P, T, L, _ptr(w), float(eps), _ptr(y))
    if rc != 0:
        raise ValueError("lto_latent rejected its arguments")
    return y


def latent_tail(partials, norm_w, eps, W, c0, n, out, nthreads=0):
    """Return a copy of ``out`` ([T][ld_out] uint16) with the window updated.

    partials [P][T][L], W [H][L], out [T][ld_out]; all uint16 bf16 bits.
    """
    p = _u16(partials)
    P, T, L = p.shape
    Wm = _u16(W)
    H = Wm.shape[0]
    if Wm.shape != (H, L):
        raise ValueError("W must be [H][L]")
    w = _u16(norm_w)
    o = np.array(_u16(out), copy=True)
    if o.ndim != 2 or o.shape[0] != T:
        raise ValueError("out must be [T][ld_out]")
    ld = o.shape[1]
    rc = _load().lto_latent_tail(_ptr(p), P, T, L, _ptr(w), float(eps), _ptr(Wm), H,
                                 int(c0), int(n), _ptr(o), ld, int(nthreads))
    if rc != 0:
        raise ValueError("lto_latent_tail rejected its arguments")
    return o


def latent_tail_residual(partials, norm_w, eps, W, c0, n, out, prefix, resid=None,
                         in_place=False, nthreads=0):
    """Return (out', resid') copies: the tail's updated ``out`` and the
    residual buffer with bf16(prefix + out') written on the window.

    prefix [T][ld_prefix]; resid [T][ld_resid] (its columns outside the window
    are kept) or None for a copy of prefix; in_place=True passes the prefix
    buffer itself as resid (resid must then be None).
    """
    p = _u16(partials)
    P, T, L = p.shape
    Wm = _u16(W)
    H = Wm.shape[0]
    w = _u16(norm_w)
    o = np.array(_u16(out), copy=True)
    pre = np.array(_u16(prefix), copy=True)
    if in_place:
        if resid is not None:
            raise ValueError("in_place takes no separate resid")
        r = pre
    else:
        r = np.array(_u16(resid if resid is not None else prefix), copy=True)
    if o.ndim != 2 or o.shape[0] != T or pre.shape[0] != T or r.shape[0] != T:
        raise ValueError("out, prefix and resid must have T rows")
    rc = _load().lto_latent_tail_residual(_ptr(p), P, T, L, _ptr(w), float(eps), _ptr(Wm), H,
                                          int(c0), int(n), _ptr(o), o.shape[1], _ptr(pre),
                                          pre.shape[1], _ptr(r), r.shape[1], int(nthreads))
    if rc != 0:
        raise ValueError("lto_latent_tail_residual rejected its arguments")
    return o, r


def attn_res_zero_block(prefix, delta, block, block_idx, norm_w, eps):
    """AttnRes state update + output norm with no valid blocks.

    prefix [T][H], delta [T][H] or None, block [T][S][H] or None (with
    block_idx < 0), norm_w [H] or None; uint16 bf16 bits.  Returns copies
    (prefix', block', out) after the update; block' is None when block is.
    """
    pre = np.array(_u16(prefix), copy=True)
    if pre.ndim != 2:
        raise ValueError("prefix must be [T][H]")
    T, H = pre.shape
    dl = _u16(delta)
    if dl is not None and dl.shape != (T, H):
        raise ValueError("delta must be [T][H]")
    blk = None if block is None else np.array(_u16(block), copy=True)
    S = 0 if blk is None else blk.shape[1]
    if blk is not None and (blk.ndim != 3 or blk.shape[0] != T or blk.shape[2] != H):
        raise ValueError("block must be [T][S][H]")
    w = _u16(norm_w)
    if w is not None and w.shape != (H,):
        raise ValueError("norm_w must have shape (H,)")
    out = np.zeros((T, H), dtype=np.uint16)
    rc = _load().lto_attn_res_zero_block(_ptr(pre), _ptr(dl), T, H, _ptr(blk), S,
                                         int(block_idx), _ptr(w), float(eps), _ptr(out))
    if rc != 0:
        raise ValueError("lto_attn_res_zero_block rejected its arguments")
    return pre, blk, out

