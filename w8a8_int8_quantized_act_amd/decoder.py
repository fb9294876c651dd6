"""The decoder Conv3d layers a preset chooses from, and a per-layer runner.

Page "ComfyUI-Qwen-VAE-Triton v0.2.0", section "Three presets explained": the
patch covers 28 Conv3d layers of the Qwen VAE decoder; Conservative runs 15
of them in W8A8 (the highest channel level), Balanced 22 (the two highest
levels, the bottom 96-channel level native), Aggressive 26 (all but
decoder.upsamples.14.residual.2 and .6, which a fixed rule keeps native); any
error falls back to native precision (fixed-parameter paragraph).

The page names counts and two layers, not the architecture.  The layer table
below is a reading of the Wan / Qwen-Image VAE decoder that those names and
counts fit: base width 96 with multipliers (1, 2, 4, 4), so the levels run
at 384, 384, 192 and 96 channels; a middle stage of two residual blocks
(middle.0 and middle.2, an attention block between them) at the latent size;
then four up-sampling levels of three residual blocks each, with a spatial
2x up-sampling block after each of the first three (whose convolution halves
the channels).  Each residual block holds two 3x3x3 CausalConv3d layers,
residual.2 (Cin -> Cout) and residual.6 (Cout -> Cout): 2 x 2 + 4 x 3 x 2 = 28.
The selection rules themselves are in the library (qvae_select_layer).

The runner is control flow only: every layer runs in the library's kernels,
W8A8 (absmax, then quantize + INT8 conv or the conv that quantizes its own
input) or native bf16, and a W8A8 layer whose calls return an error status
runs the native conv instead.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import ops

TOP_CHANNELS = 384
# Frames on which the decoder benchmark's "quantize in the conv" variant uses
# the input-quantizing conv (the HBM-bound 96-channel top level).  The runner
# itself quantizes with the quantize pass unless asked otherwise: at 96 @
# 1024x1024 the input-quantizing conv takes 151-160 us against 142-150 us for
# the quantize pass and the conv together (the pass leaves the codes in the
# last-level cache for the conv), and the two-step path is faster still on
# the smaller levels.
QIN_MIN_PIXELS = 512 * 1024


@dataclass(frozen=True)
class DecoderConv:
    name: str
    Cin: int
    Cout: int
    H: int          # spatial size of the layer's input and output
    W: int
    k: tuple = (3, 3, 3)


def residual_convs(out_h: int = 1024, out_w: int = 1024, base: int = 96, mult=(1, 2, 4, 4),
                   blocks_per_level: int = 3):
    """The 28 residual-block convolutions of the decoder for an out_h x out_w
    image (latent size out / 8), in execution order."""
    ups = len(mult) - 1
    if out_h % (1 << ups) or out_w % (1 << ups):
        raise ValueError(f"output size must be a multiple of {1 << ups}")
    h, w = out_h >> ups, out_w >> ups
    dims = [base * m for m in (mult[-1],) + tuple(reversed(mult))]
    layers = []
    for blk in (0, 2):
        layers.append(DecoderConv(f"decoder.middle.{blk}.residual.2", dims[0], dims[0], h, w))
        layers.append(DecoderConv(f"decoder.middle.{blk}.residual.6", dims[0], dims[0], h, w))
    idx = 0
    for i, (cin, cout) in enumerate(zip(dims[:-1], dims[1:])):
        if i > 0:
            cin //= 2          # the previous level's up-sampling conv halves the channels
        for _ in range(blocks_per_level):
            layers.append(DecoderConv(f"decoder.upsamples.{idx}.residual.2", cin, cout, h, w))
            layers.append(DecoderConv(f"decoder.upsamples.{idx}.residual.6", cout, cout, h, w))
            cin = cout
            idx += 1
        if i != len(mult) - 1:
            idx += 1           # the up-sampling block
            h, w = 2 * h, 2 * w
    return layers


def plan(preset, layers, top_channels: int = TOP_CHANNELS):
    """{layer name: True if W8A8} for a preset ("native", "conservative",
    "balanced", "aggressive" or its number)."""
    return {L.name: ops.select_layer(preset, L.name, L.Cin, L.Cout, L.k, top_channels) for L in layers}


_code_loaded = False


class PlannedConv:
    """One decoder Conv3d run as the preset says, with per-layer fallback.

    w: bf16 [Cout][Cin][kt][kh][kw] on the device (the VAE's own weights);
    bias: float32 [Cout] or None.  The native packed weights are always kept:
    they serve the native layers and the fallback of the W8A8 ones."""

    def __init__(self, name: str, w: torch.Tensor, bias: torch.Tensor | None, preset,
                 top_channels: int = TOP_CHANNELS, clip_ratio: float = 1.0,
                 quantize_in_conv: bool | None = None):
        self.name = name
        # W8A8 layers: quantize x inside the conv (absmax pass + the input-quantizing
        # conv) or with the quantize pass (absmax + quantize + conv).  None picks the
        # latter: with the quantize pass leaving large tensors' codes in the
        # last-level cache for the conv, it measured at least as fast on every
        # decoder level; the results are identical.
        self.quantize_in_conv = quantize_in_conv
        global _code_loaded
        if not _code_loaded:
            # the library's GPU code is loaded at set-up, not in the first decoder step
            try:
                ops.init()
            except ops.QvaeError:
                pass   # the calls below report the failure (or fall back)
            _code_loaded = True
        Cout, Cin, kt, kh, kw = w.shape
        self.bias = bias
        self.clip_ratio = clip_ratio
        self.wp = ops.pack_weights_bf16(w)
        self.w8a8 = ops.select_layer(preset, name, Cin, Cout, (kt, kh, kw), top_channels)
        self.fallbacks = 0
        self.wq = self.ws = None
        if self.w8a8:
            try:
                # bf16 -> float32 is an exact widening; the quantizer reads float32
                self.wq, self.ws = ops.quantize_weights(w.float(), clip_ratio)
            except ops.QvaeError:
                self.w8a8 = False
                self.fallbacks += 1

    def uses_quantize_in_conv(self, x: torch.Tensor) -> bool:
        return bool(self.quantize_in_conv)

    def __call__(self, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        if self.w8a8:
            try:
                if self.uses_quantize_in_conv(x):
                    am = ops.act_absmax(x)
                    y, _ = ops.causalconv3d_w8a8_qin(x, am, self.wq, self.ws, self.bias,
                                                     clip_ratio=self.clip_ratio, out=out)
                    return y
                _, xs, xq = ops.act_absmax_quant(x, self.clip_ratio)
                return ops.causalconv3d_w8a8(xq, xs, self.wq, self.ws, self.bias, out=out)
            except ops.QvaeError:
                self.fallbacks += 1
        return ops.causalconv3d_bf16(x, self.wp, self.bias, out=out)
