"""Thin Python binding of libqvae (ctypes): argument marshalling only.

Every step of the path runs in the HIP kernels behind the C ABI declared in
``include/qvae.h``; this module only turns torch tensors into device pointers
and the current torch stream into a ``hipStream_t``.  Torch provides device
memory and streams.  There is no fallback here: a missing library or a
non-zero status raises ``QvaeError`` (the caller decides what to do, e.g. run
its native-precision layer instead).

Names follow the C entry points:
  quantize_weights        -> qvae_quantize_weights
  act_absmax              -> qvae_act_absmax
  act_quantize            -> qvae_act_quantize
  act_absmax_quant        -> qvae_act_absmax_quant
  act_absmax_quant_noalloc -> qvae_act_absmax_quant_noalloc
  causalconv3d_w8a8       -> qvae_causalconv3d_w8a8
  causalconv3d_w8a8_acc32 -> qvae_causalconv3d_w8a8_acc32
  causalconv3d_w8a8_absmax -> qvae_causalconv3d_w8a8_absmax
  select_layer            -> qvae_select_layer
  pack_weights_bf16       -> qvae_pack_weights_bf16
  causalconv3d_bf16       -> qvae_causalconv3d_bf16
  rmsnorm_silu            -> qvae_rmsnorm_silu
  rmsnorm_silu_absmax     -> qvae_rmsnorm_silu_absmax
  causalconv3d_w8a8_qin   -> qvae_causalconv3d_w8a8_qin
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqvae.so")

OK, EINVAL, EUNSUPPORTED, ELAUNCH, EFORCED = 0, -1, -2, -3, -4
PRESET_NATIVE, PRESET_CONSERVATIVE, PRESET_BALANCED, PRESET_AGGRESSIVE = 0, 1, 2, 3
PRESETS = {"native": PRESET_NATIVE, "conservative": PRESET_CONSERVATIVE, "balanced": PRESET_BALANCED,
           "aggressive": PRESET_AGGRESSIVE}
ABSMAX_WORDS = 513   # QVAE_ABSMAX_WORDS: word 0 = bf16 bits of max|x|, then partial maxima


class QvaeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        text = strerror(status) if _lib is not None else ""
        super().__init__(f"{where}: {text} (status {status})" if text else f"{where} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqvae.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise QvaeError(ELAUNCH, f"HIP library not built: {LIB_PATH} is missing "
                                     "(run python -m w8a8_int8_quantized_act_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.qvae_version.argtypes = []
        L.qvae_version.restype = i32
        L.qvae_strerror.argtypes = [i32]
        L.qvae_strerror.restype = ctypes.c_char_p
        L.qvae_quantize_weights.argtypes = [P, i32, i32, i32, i32, i32, f32, P, P, P]
        L.qvae_quantize_weights.restype = i32
        L.qvae_act_absmax.argtypes = [P, i64, P, P]
        L.qvae_act_absmax.restype = i32
        L.qvae_act_quantize.argtypes = [P, i64, f32, P, P, P, P]
        L.qvae_act_quantize.restype = i32
        L.qvae_act_absmax_quant.argtypes = [P, i64, f32, P, P, P, P]
        L.qvae_act_absmax_quant.restype = i32
        L.qvae_act_absmax_quant_noalloc.argtypes = [P, i64, f32, P, P, P]
        L.qvae_act_absmax_quant_noalloc.restype = i32
        L.qvae_causalconv3d_w8a8.argtypes = [P, P, P, P, P, P] + [i32] * 9 + [P, P]
        L.qvae_causalconv3d_w8a8.restype = i32
        L.qvae_causalconv3d_w8a8_absmax.argtypes = [P, P, P, P, P, P] + [i32] * 9 + [P, P, P]
        L.qvae_causalconv3d_w8a8_absmax.restype = i32
        L.qvae_causalconv3d_w8a8_acc32.argtypes = [P, P, P] + [i32] * 9 + [P, P]
        L.qvae_causalconv3d_w8a8_acc32.restype = i32
        L.qvae_select_layer.argtypes = [i32, ctypes.c_char_p] + [i32] * 6
        L.qvae_select_layer.restype = i32
        L.qvae_pack_weights_bf16.argtypes = [P] + [i32] * 5 + [P, P]
        L.qvae_pack_weights_bf16.restype = i32
        L.qvae_causalconv3d_bf16.argtypes = [P, P, P, P] + [i32] * 9 + [P, P]
        L.qvae_causalconv3d_bf16.restype = i32
        L.qvae_rmsnorm_silu.argtypes = [P, i64, i32, P, f32, P, P]
        L.qvae_rmsnorm_silu.restype = i32
        L.qvae_rmsnorm_silu_absmax.argtypes = [P, i64, i32, P, f32, P, P, P]
        L.qvae_rmsnorm_silu_absmax.restype = i32
        L.qvae_causalconv3d_w8a8_qin.argtypes = [P, P, P, f32, P, P, P] + [i32] * 9 + [P, P, P]
        L.qvae_causalconv3d_w8a8_qin.restype = i32
        L.qvae_init.argtypes = []
        L.qvae_init.restype = i32
        _lib = L
    return _lib


def init():
    """qvae_init: load the library's GPU code for the current device now (optional)."""
    _check(lib().qvae_init(), "qvae_init")


def strerror(status: int) -> str:
    return lib().qvae_strerror(int(status)).decode()


def _check(status: int, where: str):
    if status != OK:
        raise QvaeError(status, where)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _absmax_buf(t: torch.Tensor, name: str = "absmax_bits"):
    """An activation-maximum buffer: int32 on the device, at least ABSMAX_WORDS words."""
    _dev(t, name, torch.int32)
    if t.numel() < ABSMAX_WORDS:
        raise ValueError(f"{name} must hold {ABSMAX_WORDS} int32 words, got {t.numel()}")
    return t


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _vec(t: torch.Tensor | None, name: str, n: int, dtype=torch.float32):
    """A per-channel device vector with at least n elements (None passes)."""
    if t is None:
        return None
    _dev(t, name, dtype)
    if t.numel() < n:
        raise ValueError(f"{name} must hold at least {n} elements, got {t.numel()}")
    return t


def _out(t: torch.Tensor | None, name: str, shape, dtype, device):
    """The caller's output tensor (checked: device, dtype, exact shape,
    contiguous), or a new one."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _dev(t, name, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


# ------------------------------------------------------------------ weights
def packed_weight_shape(Cout, Cin, kt, kh, kw):
    """Shape of the packed INT8 weights: [Cout/32][kt][Cin/32][kh][kw][64][16]."""
    return (Cout // 32, kt, Cin // 32, kh, kw, 64, 16)


def quantize_weights(w: torch.Tensor, clip_ratio: float = 1.0, stream=None):
    """w float32 [Cout][Cin][kt][kh][kw] -> (wq int8 packed [Cout/32][kt][Cin/32][kh][kw][64][16],
    w_scale float32 [Cout]); see qvae.h for the packing."""
    _dev(w, "w", torch.float32)
    Cout, Cin, kt, kh, kw = w.shape
    if Cout % 32 or Cin % 32:
        raise QvaeError(EUNSUPPORTED, "quantize_weights: Cout and Cin must be multiples of 32")
    wq = torch.empty(packed_weight_shape(Cout, Cin, kt, kh, kw), dtype=torch.int8, device=w.device)
    ws = torch.empty((Cout,), dtype=torch.float32, device=w.device)
    _check(lib().qvae_quantize_weights(_p(w), Cout, Cin, kt, kh, kw, float(clip_ratio),
                                       _p(wq), _p(ws), _stream(stream)), "qvae_quantize_weights")
    return wq, ws


def packed_weight_shape_bf16(Cout, Cin, kt, kh, kw):
    """Shape of the packed bf16 weights: [Cout/32][kt][Cin/16][kh][kw][64][8]."""
    return (Cout // 32, kt, Cin // 16, kh, kw, 64, 8)


def pack_weights_bf16(w: torch.Tensor, stream=None):
    """w bf16 [Cout][Cin][kt][kh][kw] -> packed bf16 [Cout/32][kt][Cin/16][kh][kw][64][8]
    (a permutation; see qvae.h)."""
    _dev(w, "w", torch.bfloat16)
    Cout, Cin, kt, kh, kw = w.shape
    if Cout % 32 or Cin % 16:
        raise QvaeError(EUNSUPPORTED, "pack_weights_bf16: Cout must be a multiple of 32, Cin of 16")
    wp = torch.empty(packed_weight_shape_bf16(Cout, Cin, kt, kh, kw), dtype=torch.bfloat16, device=w.device)
    _check(lib().qvae_pack_weights_bf16(_p(w), Cout, Cin, kt, kh, kw, _p(wp), _stream(stream)),
           "qvae_pack_weights_bf16")
    return wp


def select_layer(preset, name: str, Cin: int, Cout: int, k=(3, 3, 3), top_channels: int = 384) -> bool:
    """True if the preset runs this decoder Conv3d in W8A8 (host-side plan)."""
    p = PRESETS[preset] if isinstance(preset, str) else int(preset)
    r = lib().qvae_select_layer(p, name.encode(), int(Cin), int(Cout), int(k[0]), int(k[1]), int(k[2]),
                                int(top_channels))
    if r < 0:
        raise QvaeError(r, "qvae_select_layer")
    return r == 1


# ------------------------------------------------------------------ activations
def _bits_view(x: torch.Tensor):
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError(f"x must hold bf16 values, got {x.dtype}")
    return x


def act_absmax(x: torch.Tensor, absmax_bits: torch.Tensor | None = None, stream=None):
    """First activation pass: partial maxima into the int32 [ABSMAX_WORDS] buffer
    (word 0 is filled in by act_quantize)."""
    _dev(_bits_view(x), "x")
    if absmax_bits is None:
        absmax_bits = torch.empty((ABSMAX_WORDS,), dtype=torch.int32, device=x.device)
    _absmax_buf(absmax_bits)
    _check(lib().qvae_act_absmax(_p(x), x.numel(), _p(absmax_bits), _stream(stream)), "qvae_act_absmax")
    return absmax_bits


def act_quantize(x: torch.Tensor, absmax_bits: torch.Tensor, clip_ratio: float = 1.0,
                 x_scale: torch.Tensor | None = None, xq: torch.Tensor | None = None, stream=None):
    """-> (x_scale float32 [1], xq int8 of x's shape)."""
    _dev(_bits_view(x), "x")
    if x_scale is None:
        x_scale = torch.empty((1,), dtype=torch.float32, device=x.device)
    _vec(x_scale, "x_scale", 1)
    xq = _out(xq, "xq", x.shape, torch.int8, x.device)
    _absmax_buf(absmax_bits)
    _check(lib().qvae_act_quantize(_p(x), x.numel(), float(clip_ratio), _p(absmax_bits), _p(x_scale),
                                   _p(xq), _stream(stream)), "qvae_act_quantize")
    return x_scale, xq


def act_absmax_quant(x: torch.Tensor, clip_ratio: float = 1.0, absmax_bits=None, x_scale=None, xq=None,
                     stream=None):
    """-> (absmax_bits int32 [ABSMAX_WORDS] (word 0 = bf16 bits of max|x|), x_scale float32 [1],
    xq int8 of x's shape)."""
    _dev(_bits_view(x), "x")
    dev = x.device
    if absmax_bits is None:
        absmax_bits = torch.empty((ABSMAX_WORDS,), dtype=torch.int32, device=dev)
    if x_scale is None:
        x_scale = torch.empty((1,), dtype=torch.float32, device=dev)
    _vec(x_scale, "x_scale", 1)
    xq = _out(xq, "xq", x.shape, torch.int8, dev)
    _absmax_buf(absmax_bits)
    _check(lib().qvae_act_absmax_quant(_p(x), x.numel(), float(clip_ratio), _p(absmax_bits), _p(x_scale),
                                       _p(xq), _stream(stream)), "qvae_act_absmax_quant")
    return absmax_bits, x_scale, xq


def act_absmax_quant_noalloc(x: torch.Tensor, clip_ratio: float = 1.0, x_scale=None, xq=None, stream=None):
    """qvae_act_absmax_quant_noalloc: both passes with the activation-maximum
    words in the library's static scratch (no workspace; with x_scale and xq
    given, nothing is allocated) -> (x_scale float32 [1], xq int8 of x's shape)."""
    _dev(_bits_view(x), "x")
    if x_scale is None:
        x_scale = torch.empty((1,), dtype=torch.float32, device=x.device)
    _vec(x_scale, "x_scale", 1)
    xq = _out(xq, "xq", x.shape, torch.int8, x.device)
    _check(lib().qvae_act_absmax_quant_noalloc(_p(x), x.numel(), float(clip_ratio), _p(x_scale), _p(xq),
                                               _stream(stream)), "qvae_act_absmax_quant_noalloc")
    return x_scale, xq


# ------------------------------------------------------------------ norm + SiLU prologue
def rmsnorm_silu(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6, out: torch.Tensor | None = None,
                 absmax_bits: torch.Tensor | None = None, with_absmax: bool = False, stream=None):
    """h = SiLU(RMSNorm(x)) over the last (channel) axis of a channels-last bf16 tensor.

    Returns h, or (h, absmax_bits) with ``with_absmax`` (the partial maxima of
    |h| for act_quantize(h, absmax_bits))."""
    _dev(x, "x", torch.bfloat16)
    _dev(gamma, "gamma", torch.float32)
    C = x.shape[-1]
    if gamma.shape != (C,):
        raise ValueError("gamma must be [C]")
    if out is None:
        out = torch.empty_like(x)
    else:
        _dev(out, "out", torch.bfloat16)
        if out.shape != x.shape:
            raise ValueError("out shape")
    npix = x.numel() // C
    if with_absmax:
        if absmax_bits is None:
            absmax_bits = torch.empty((ABSMAX_WORDS,), dtype=torch.int32, device=x.device)
        _absmax_buf(absmax_bits)
        _check(lib().qvae_rmsnorm_silu_absmax(_p(x), npix, C, _p(gamma), float(eps), _p(out), _p(absmax_bits),
                                              _stream(stream)), "qvae_rmsnorm_silu_absmax")
        return out, absmax_bits
    _check(lib().qvae_rmsnorm_silu(_p(x), npix, C, _p(gamma), float(eps), _p(out), _stream(stream)),
           "qvae_rmsnorm_silu")
    return out


# ------------------------------------------------------------------ convolution
def _conv_dims(xq, wq, cache):
    _dev(xq, "xq", torch.int8)
    _dev(wq, "wq", torch.int8)
    N, T, H, W, Cin = xq.shape
    if wq.dim() != 7 or tuple(wq.shape[5:]) != (64, 16):
        raise ValueError("wq must be the packed [Cout/32][kt][Cin/32][kh][kw][64][16] tensor")
    Cout, kt, Cin2, kh, kw = wq.shape[0] * 32, wq.shape[1], wq.shape[2] * 32, wq.shape[3], wq.shape[4]
    if Cin2 != Cin:
        raise ValueError(f"Cin mismatch: xq has {Cin}, wq has {Cin2}")
    if cache is not None:
        _dev(cache, "cache", torch.int8)
        if tuple(cache.shape) != (N, kt - 1, H, W, Cin):
            raise ValueError(f"cache must be [N][kt-1][H][W][Cin] = {(N, kt - 1, H, W, Cin)}, "
                             f"got {tuple(cache.shape)}")
    return N, T, H, W, Cin, Cout, kt, kh, kw


def causalconv3d_w8a8(xq: torch.Tensor, x_scale: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                      bias: torch.Tensor | None = None, cache: torch.Tensor | None = None,
                      out: torch.Tensor | None = None, stream=None):
    """xq int8 [N][T][H][W][Cin] -> y bf16 [N][T][H][W][Cout]."""
    N, T, H, W, Cin, Cout, kt, kh, kw = _conv_dims(xq, wq, cache)
    _vec(x_scale, "x_scale", 1)
    _vec(w_scale, "w_scale", Cout)
    _vec(bias, "bias", Cout)
    out = _out(out, "out", (N, T, H, W, Cout), torch.bfloat16, xq.device)
    _check(lib().qvae_causalconv3d_w8a8(_p(xq), _p(x_scale), _p(cache), _p(wq), _p(w_scale), _p(bias),
                                        N, T, H, W, Cin, Cout, kt, kh, kw, _p(out), _stream(stream)),
           "qvae_causalconv3d_w8a8")
    return out


def causalconv3d_w8a8_absmax(xq: torch.Tensor, x_scale: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                             bias: torch.Tensor | None = None, cache: torch.Tensor | None = None,
                             out: torch.Tensor | None = None, y_absmax: torch.Tensor | None = None, stream=None):
    """causalconv3d_w8a8 that also leaves the partial maxima of |y| in an
    activation-maximum buffer -> (y, y_absmax); act_quantize(y, y_absmax)
    then quantizes y without its absmax pass."""
    N, T, H, W, Cin, Cout, kt, kh, kw = _conv_dims(xq, wq, cache)
    _vec(x_scale, "x_scale", 1)
    _vec(w_scale, "w_scale", Cout)
    _vec(bias, "bias", Cout)
    out = _out(out, "out", (N, T, H, W, Cout), torch.bfloat16, xq.device)
    if y_absmax is None:
        y_absmax = torch.empty((ABSMAX_WORDS,), dtype=torch.int32, device=xq.device)
    _absmax_buf(y_absmax, "y_absmax")
    _check(lib().qvae_causalconv3d_w8a8_absmax(_p(xq), _p(x_scale), _p(cache), _p(wq), _p(w_scale), _p(bias),
                                               N, T, H, W, Cin, Cout, kt, kh, kw, _p(out), _p(y_absmax),
                                               _stream(stream)), "qvae_causalconv3d_w8a8_absmax")
    return out, y_absmax


def causalconv3d_w8a8_acc32(xq: torch.Tensor, wq: torch.Tensor, cache: torch.Tensor | None = None,
                            out: torch.Tensor | None = None, stream=None):
    """Raw INT32 accumulators [N][T][H][W][Cout] (verification export)."""
    N, T, H, W, Cin, Cout, kt, kh, kw = _conv_dims(xq, wq, cache)
    out = _out(out, "out", (N, T, H, W, Cout), torch.int32, xq.device)
    _check(lib().qvae_causalconv3d_w8a8_acc32(_p(xq), _p(cache), _p(wq), N, T, H, W, Cin, Cout, kt, kh, kw,
                                              _p(out), _stream(stream)), "qvae_causalconv3d_w8a8_acc32")
    return out


def causalconv3d_w8a8_qin(x: torch.Tensor, absmax_bits: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                          bias: torch.Tensor | None = None, cache: torch.Tensor | None = None,
                          clip_ratio: float = 1.0, out: torch.Tensor | None = None,
                          x_scale: torch.Tensor | None = None, stream=None):
    """The W8A8 conv on bf16 x [N][T][H][W][Cin]: quantizes x (and the bf16 cache)
    itself with the scale from absmax_bits (partial maxima of x) -> (y, x_scale)."""
    _dev(x, "x", torch.bfloat16)
    _dev(wq, "wq", torch.int8)
    N, T, H, W, Cin = x.shape
    if wq.dim() != 7 or tuple(wq.shape[5:]) != (64, 16):
        raise ValueError("wq must be the packed [Cout/32][kt][Cin/32][kh][kw][64][16] tensor")
    Cout, kt, Cin2, kh, kw = wq.shape[0] * 32, wq.shape[1], wq.shape[2] * 32, wq.shape[3], wq.shape[4]
    if Cin2 != Cin:
        raise ValueError(f"Cin mismatch: x has {Cin}, wq has {Cin2}")
    if cache is not None:
        _dev(cache, "cache", torch.bfloat16)
        if tuple(cache.shape) != (N, kt - 1, H, W, Cin):
            raise ValueError(f"cache must be [N][kt-1][H][W][Cin] = {(N, kt - 1, H, W, Cin)}")
    _vec(w_scale, "w_scale", Cout)
    _vec(bias, "bias", Cout)
    out = _out(out, "out", (N, T, H, W, Cout), torch.bfloat16, x.device)
    if x_scale is None:
        x_scale = torch.empty((1,), dtype=torch.float32, device=x.device)
    _vec(x_scale, "x_scale", 1)
    _absmax_buf(absmax_bits)
    _check(lib().qvae_causalconv3d_w8a8_qin(_p(x), _p(cache), _p(absmax_bits), float(clip_ratio), _p(wq),
                                            _p(w_scale), _p(bias), N, T, H, W, Cin, Cout, kt, kh, kw,
                                            _p(x_scale), _p(out), _stream(stream)), "qvae_causalconv3d_w8a8_qin")
    return out, x_scale


def causalconv3d_bf16(x: torch.Tensor, wp: torch.Tensor, bias: torch.Tensor | None = None,
                      cache: torch.Tensor | None = None, out: torch.Tensor | None = None, stream=None):
    """Native-precision conv: x bf16 [N][T][H][W][Cin], wp from pack_weights_bf16,
    cache bf16 [N][kt-1][H][W][Cin] or None -> y bf16 [N][T][H][W][Cout]."""
    _dev(x, "x", torch.bfloat16)
    _dev(wp, "wp", torch.bfloat16)
    N, T, H, W, Cin = x.shape
    if wp.dim() != 7 or tuple(wp.shape[5:]) != (64, 8):
        raise ValueError("wp must be the packed [Cout/32][kt][Cin/16][kh][kw][64][8] tensor")
    Cout, kt, Cin2, kh, kw = wp.shape[0] * 32, wp.shape[1], wp.shape[2] * 16, wp.shape[3], wp.shape[4]
    if Cin2 != Cin:
        raise ValueError(f"Cin mismatch: x has {Cin}, wp has {Cin2}")
    if cache is not None:
        _dev(cache, "cache", torch.bfloat16)
        if tuple(cache.shape) != (N, kt - 1, H, W, Cin):
            raise ValueError(f"cache must be [N][kt-1][H][W][Cin] = {(N, kt - 1, H, W, Cin)}")
    _vec(bias, "bias", Cout)
    out = _out(out, "out", (N, T, H, W, Cout), torch.bfloat16, x.device)
    _check(lib().qvae_causalconv3d_bf16(_p(x), _p(cache), _p(wp), _p(bias), N, T, H, W, Cin, Cout, kt, kh, kw,
                                        _p(out), _stream(stream)), "qvae_causalconv3d_bf16")
    return out


def layer_forward(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor, bias: torch.Tensor | None = None,
                  cache: torch.Tensor | None = None, clip_ratio: float = 1.0, stream=None):
    """One W8A8 CausalConv3d layer: absmax -> quantize -> implicit-GEMM conv.

    x bf16 [N][T][H][W][Cin] -> (y bf16 [N][T][H][W][Cout], x_scale, xq)."""
    _, x_scale, xq = act_absmax_quant(x, clip_ratio, stream=stream)
    y = causalconv3d_w8a8(xq, x_scale, wq, w_scale, bias, cache, stream=stream)
    return y, x_scale, xq
