"""CPU oracle for the W8A8 CausalConv3d path (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of the
benchmark may import this package.  The product path (the HIP library and its
Python binding) never imports, loads or calls it, and the two share no code.

The arithmetic lives in ``qvae_oracle.c`` (plain C, compiled with gcc
``-O2 -ffp-contract=off``: one IEEE binary32 operation per step of the W8A8
path, exact int64 sums; the native-precision conv and the RMSNorm + SiLU
prologue in binary64, rounded once).  This module is argument marshalling between numpy arrays and that
library.  See the header of ``qvae_oracle.c`` for what each step computes and
the passages of the ComfyUI-Qwen-VAE-Triton v0.2.0 page that define it.

Parity unpinned: none.  Every function is pinned by tests under ``tests/``
(brute force, float64 library convolution, closed forms, invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qvae_oracle.c")
_LIB = os.path.join(_HERE, "libqvae_oracle.so")

OK = 0
EOVERFLOW = 1
EARG = 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (CPU only; no HIP toolchain involved)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = f32
        L.oracle_f32_to_bf16.argtypes = [f32]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_scale_from_absmax.argtypes = [f32, f32]
        L.oracle_scale_from_absmax.restype = f32
        L.oracle_quantize_weights.argtypes = [P, i32, i32, i32, i32, i32, f32, P, P]
        L.oracle_quantize_weights.restype = i32
        L.oracle_act_absmax.argtypes = [P, i64]
        L.oracle_act_absmax.restype = f32
        L.oracle_act_quantize.argtypes = [P, i64, f32, P]
        L.oracle_act_quantize.restype = None
        L.oracle_conv_acc_positions.argtypes = [P, P, P] + [i32] * 9 + [P, i64, P]
        L.oracle_conv_acc_positions.restype = i32
        L.oracle_conv_acc.argtypes = [P, P, P] + [i32] * 9 + [P]
        L.oracle_conv_acc.restype = i32
        L.oracle_epilogue.argtypes = [P, i64, i32, f32, P, P, P]
        L.oracle_epilogue.restype = None
        L.oracle_epilogue_f32.argtypes = [P, i64, i32, f32, P, P, P]
        L.oracle_epilogue_f32.restype = None
        L.oracle_layer.argtypes = ([P, P, P, P, P] + [i32] * 9 +
                                   [f32, P, i64, P, P, P, P])
        L.oracle_layer.restype = i32
        L.oracle_conv_bf16_positions.argtypes = [P, P, P, P] + [i32] * 9 + [P, i64, P, P]
        L.oracle_conv_bf16_positions.restype = i32
        L.oracle_bf16_from_f64.argtypes = [ctypes.c_double]
        L.oracle_bf16_from_f64.restype = ctypes.c_uint16
        L.oracle_rmsnorm_silu.argtypes = [P, i64, i32, P, f32, P]
        L.oracle_rmsnorm_silu.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


# ---------------------------------------------------------------- scalars
def bf16_to_f32(h: int) -> float:
    return lib().oracle_bf16_to_f32(int(h))


def f32_to_bf16(f: float) -> int:
    return lib().oracle_f32_to_bf16(float(np.float32(f)))


def scale_from_absmax(absmax: float, clip_ratio: float = 1.0) -> np.float32:
    return np.float32(lib().oracle_scale_from_absmax(float(absmax), float(clip_ratio)))


# ---------------------------------------------------------------- weights
def quantize_weights(w: np.ndarray, clip_ratio: float = 1.0):
    """w float32 [Cout][Cin][kt][kh][kw] -> (wq int8 [Cout][kt][kh][kw][Cin], s_w float32 [Cout])."""
    w = _c(w, np.float32)
    Cout, Cin, kt, kh, kw = w.shape
    wq = np.empty((Cout, kt, kh, kw, Cin), np.int8)
    s_w = np.empty((Cout,), np.float32)
    rc = lib().oracle_quantize_weights(_ptr(w), Cout, Cin, kt, kh, kw,
                                       float(clip_ratio), _ptr(wq), _ptr(s_w))
    if rc != OK:
        raise ValueError(f"oracle_quantize_weights failed: {rc}")
    return wq, s_w


# ---------------------------------------------------------------- activations
def act_absmax(x_bf16_bits: np.ndarray) -> np.float32:
    x = _c(x_bf16_bits, np.uint16)
    return np.float32(lib().oracle_act_absmax(_ptr(x), x.size))


def act_quantize(x_bf16_bits: np.ndarray, s: float) -> np.ndarray:
    x = _c(x_bf16_bits, np.uint16)
    q = np.empty(x.shape, np.int8)
    lib().oracle_act_quantize(_ptr(x), x.size, float(np.float32(s)), _ptr(q))
    return q


def act_absmax_quant(x_bf16_bits: np.ndarray, clip_ratio: float = 1.0):
    """-> (absmax float32, s_x float32, xq int8 of x's shape)."""
    a = act_absmax(x_bf16_bits)
    s = scale_from_absmax(a, clip_ratio)
    return a, s, act_quantize(x_bf16_bits, s)


# ---------------------------------------------------------------- convolution
def conv_acc(xq: np.ndarray, wq: np.ndarray, cache: np.ndarray | None = None,
             positions: np.ndarray | None = None) -> np.ndarray:
    """INT32 accumulators.

    xq int8 [N][T][H][W][Cin]; wq int8 [Cout][kt][kh][kw][Cin];
    cache int8 [N][kt-1][H][W][Cin] or None.  With ``positions`` (flattened
    ((n*T+t)*H+h)*W+w indices) returns [len(positions)][Cout], else
    [N][T][H][W][Cout].
    """
    xq = _c(xq, np.int8)
    wq = _c(wq, np.int8)
    N, T, H, W, Cin = xq.shape
    Cout, kt, kh, kw, Cin2 = wq.shape
    if Cin2 != Cin:
        raise ValueError("Cin mismatch")
    if cache is not None:
        cache = _c(cache, np.int8)
        if cache.shape != (N, kt - 1, H, W, Cin):
            raise ValueError(f"cache shape {cache.shape}")
    if positions is None:
        acc = np.empty((N, T, H, W, Cout), np.int32)
        rc = lib().oracle_conv_acc(_ptr(xq), _ptr(cache), _ptr(wq), N, T, H, W,
                                   Cin, Cout, kt, kh, kw, _ptr(acc))
    else:
        pos = _c(np.asarray(positions, np.int64), np.int64)
        acc = np.empty((pos.size, Cout), np.int32)
        rc = lib().oracle_conv_acc_positions(_ptr(xq), _ptr(cache), _ptr(wq), N, T,
                                             H, W, Cin, Cout, kt, kh, kw, _ptr(pos),
                                             pos.size, _ptr(acc))
    if rc != OK:
        raise ValueError(f"oracle conv failed: {rc}")
    return acc


def epilogue(acc: np.ndarray, s_x: float, s_w: np.ndarray, bias: np.ndarray | None):
    """INT32 acc [..., Cout] -> bf16 bits (uint16) of the same shape."""
    acc = _c(acc, np.int32)
    s_w = _c(s_w, np.float32)
    Cout = acc.shape[-1]
    b = None if bias is None else _c(bias, np.float32)
    y = np.empty(acc.shape, np.uint16)
    lib().oracle_epilogue(_ptr(acc), acc.size // Cout, Cout, float(np.float32(s_x)),
                          _ptr(s_w), _ptr(b), _ptr(y))
    return y


def epilogue_f32(acc: np.ndarray, s_x: float, s_w: np.ndarray, bias: np.ndarray | None):
    acc = _c(acc, np.int32)
    s_w = _c(s_w, np.float32)
    Cout = acc.shape[-1]
    b = None if bias is None else _c(bias, np.float32)
    y = np.empty(acc.shape, np.float32)
    lib().oracle_epilogue_f32(_ptr(acc), acc.size // Cout, Cout, float(np.float32(s_x)),
                              _ptr(s_w), _ptr(b), _ptr(y))
    return y


def layer(x_bf16_bits, wq, s_w, bias, cache=None, positions=None, clip_ratio=1.0):
    """Whole layer (absmax -> quantize -> conv -> epilogue) on the CPU.

    Returns (y bf16 bits [npos][Cout] or [N][T][H][W][Cout], s_x)."""
    x = _c(x_bf16_bits, np.uint16)
    wq = _c(wq, np.int8)
    s_w = _c(s_w, np.float32)
    N, T, H, W, Cin = x.shape
    Cout, kt, kh, kw, _ = wq.shape
    b = None if bias is None else _c(bias, np.float32)
    if cache is not None:
        cache = _c(cache, np.int8)
    if positions is None:
        npos = N * T * H * W
        pos = None
        yshape = (N, T, H, W, Cout)
    else:
        pos = _c(np.asarray(positions, np.int64), np.int64)
        npos = pos.size
        yshape = (npos, Cout)
    xq = np.empty(x.shape, np.int8)
    acc = np.empty((npos, Cout), np.int32)
    y = np.empty(yshape, np.uint16)
    sx = ctypes.c_float(0.0)
    rc = lib().oracle_layer(_ptr(x), _ptr(cache), _ptr(wq), _ptr(s_w), _ptr(b), N, T,
                            H, W, Cin, Cout, kt, kh, kw, float(clip_ratio), _ptr(pos),
                            npos, _ptr(xq), _ptr(acc), _ptr(y),
                            ctypes.cast(ctypes.pointer(sx), ctypes.c_void_p))
    if rc != OK:
        raise ValueError(f"oracle layer failed: {rc}")
    return y, np.float32(sx.value)


# ---------------------------------------------------------------- native-precision conv
def conv_bf16(x_bf16_bits, w_bf16_bits, bias=None, cache=None, positions=None):
    """bf16 conv of the layers a preset leaves unquantized.

    x uint16 bf16 bits [N][T][H][W][Cin]; w uint16 bf16 bits
    [Cout][Cin][kt][kh][kw]; bias float32 [Cout] or None; cache uint16
    [N][kt-1][H][W][Cin] or None.  Returns (z, mag), float64 of shape
    [npos][Cout] (or [N][T][H][W][Cout] without ``positions``): z the exact
    value (before any rounding to bf16), mag the sum of |x w| plus |bias|."""
    x = _c(x_bf16_bits, np.uint16)
    w = _c(w_bf16_bits, np.uint16)
    N, T, H, W, Cin = x.shape
    Cout, Cin2, kt, kh, kw = w.shape
    if Cin2 != Cin:
        raise ValueError("Cin mismatch")
    b = None if bias is None else _c(bias, np.float32)
    if cache is not None:
        cache = _c(cache, np.uint16)
        if cache.shape != (N, kt - 1, H, W, Cin):
            raise ValueError(f"cache shape {cache.shape}")
    if positions is None:
        npos, pos, shape = N * T * H * W, None, (N, T, H, W, Cout)
    else:
        pos = _c(np.asarray(positions, np.int64), np.int64)
        npos, shape = pos.size, (pos.size, Cout)
    z = np.empty(shape, np.float64)
    mag = np.empty(shape, np.float64)
    rc = lib().oracle_conv_bf16_positions(_ptr(x), _ptr(cache), _ptr(w), _ptr(b), N, T, H, W, Cin, Cout,
                                          kt, kh, kw, _ptr(pos), npos, _ptr(z), _ptr(mag))
    if rc != OK:
        raise ValueError(f"oracle bf16 conv failed: {rc}")
    return z, mag


# ---------------------------------------------------------------- RMSNorm + SiLU
def bf16_from_f64(d: float) -> int:
    """bf16 bits of a binary64 value, rounded once (nearest, ties to even)."""
    return int(lib().oracle_bf16_from_f64(float(d)))


def rmsnorm_silu(x_bf16_bits: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x uint16 bf16 bits [..., C] (channels last) -> h uint16 bf16 bits, same shape.

    h = bf16_rne(SiLU(x * gamma / sqrt(mean(x^2) + eps))), evaluated in binary64
    and rounded once (the definition, not the GPU pass's binary32 sequence)."""
    x = _c(x_bf16_bits, np.uint16)
    g = _c(gamma, np.float32)
    C = x.shape[-1]
    if g.shape != (C,):
        raise ValueError("gamma must be [C]")
    h = np.empty(x.shape, np.uint16)
    rc = lib().oracle_rmsnorm_silu(_ptr(x), x.size // C, C, _ptr(g), float(np.float32(eps)), _ptr(h))
    if rc != OK:
        raise ValueError(f"oracle rmsnorm_silu failed: {rc}")
    return h
