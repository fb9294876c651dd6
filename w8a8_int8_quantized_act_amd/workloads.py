"""Seeded synthetic inputs for the W8A8 CausalConv3d layers.

This module draws inputs and nothing else: it holds none of the method's
arithmetic (no scale, no rounding to int8, no convolution).  Both the HIP path
and the CPU oracle consume the bytes it produces.

Shapes stand in for the CausalConv3d layers of a Qwen-Image / Wan-style VAE
decoder (the layer family named on the ComfyUI-Qwen-VAE-Triton v0.2.0 page,
intro paragraph); the page's own workload needs trained model files that are
not available, so every tensor here is random.

Recipe (per conv, one ``torch.Generator`` per workload, draws in this order):
  x  ~ N(0,1) float32 drawn as [N][Cin][T][H][W]; then the workload's
       transform (SiLU-like ``z*sigmoid(z)``, or 5 % i.i.d. outliers scaled
       x20 with the mask drawn right after x); then cast to bf16 (round to
       nearest even) and laid out channels-last [N][T][H][W][Cin];
  w  ~ N(0, 0.02) float32 [Cout][Cin][kt][kh][kw];
  b  ~ N(0, 0.01) float32 [Cout].
Level sweeps draw their levels in order from one generator.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass
class ConvSpec:
    name: str
    N: int
    Cin: int
    Cout: int
    T: int
    H: int
    W: int
    k: tuple = (3, 3, 3)
    x_kind: str = "normal"          # "normal" | "silu" | "outlier"
    zero_cache: bool = False        # pass an explicit all-zero (kt-1)-frame cache
    chunks: int = 1                 # >1: chunked causal decode over T
    proj_cout: int = 0              # >0: add a 1x1x1 projection Cin -> proj_cout

    @property
    def kt(self):
        return self.k[0]

    @property
    def numel(self):
        return self.N * self.T * self.H * self.W * self.Cin

    @property
    def positions(self):
        return self.N * self.T * self.H * self.W


@dataclass
class Workload:
    key: str
    seed: int
    convs: list = field(default_factory=list)
    description: str = ""


def _wl():
    w = {}
    w["single_96_t4_32"] = Workload(
        "single_96_t4_32", 0,
        [ConvSpec("c96_t4_32x32", 1, 96, 96, 4, 32, 32)],
        "single CausalConv3d 3x3x3, Cin=Cout=96, [1,96,4,32,32], causal front pad 2")
    w["latent_384_128_cache"] = Workload(
        "latent_384_128_cache", 1,
        [ConvSpec("c384_t1_128x128_cache", 1, 384, 384, 1, 128, 128,
                  x_kind="outlier", zero_cache=True)],
        "latent-level CausalConv3d 3x3x3, Cin=Cout=384, [1,384,1,128,128], 5% x20 "
        "outliers, explicit 2-frame zero cache")
    w["sweep_1024"] = Workload(
        "sweep_1024", 2,
        [ConvSpec("c384_128x128", 1, 384, 384, 1, 128, 128, x_kind="silu"),
         ConvSpec("c384_256x256", 1, 384, 384, 1, 256, 256, x_kind="silu"),
         ConvSpec("c192_512x512", 1, 192, 192, 1, 512, 512, x_kind="silu"),
         ConvSpec("c96_1024x1024", 1, 96, 96, 1, 1024, 1024, x_kind="silu")],
        "decoder levels for a 1024x1024 output, T=1, SiLU-like activations")
    w["sweep_840x1256"] = Workload(
        "sweep_840x1256", 3,
        [ConvSpec("c384_105x157", 1, 384, 384, 1, 105, 157),
         ConvSpec("c384_210x314", 1, 384, 384, 1, 210, 314),
         ConvSpec("c192_420x628", 1, 192, 192, 1, 420, 628),
         ConvSpec("c96_840x1256", 1, 96, 96, 1, 840, 1256)],
        "decoder levels for an 840x1256 output (odd, non-tile-multiple sizes), T=1")
    w["video_384_t8_chunked"] = Workload(
        "video_384_t8_chunked", 4,
        [ConvSpec("c384_t8_90x160_chunked", 1, 384, 384, 8, 90, 160, chunks=4,
                  proj_cout=192)],
        "chunked causal decode: [1,384,8,90,160] as 4 chunks of 2 frames with a "
        "2-frame cache, plus a 1x1x1 384->192 projection on the same input")
    return w


WORKLOADS = _wl()
WORKLOAD_ORDER = ["single_96_t4_32", "latent_384_128_cache", "sweep_1024",
                  "sweep_840x1256", "video_384_t8_chunked"]


@dataclass
class ConvInputs:
    spec: ConvSpec
    x: np.ndarray          # uint16 bf16 bits, [N][T][H][W][Cin]
    w: np.ndarray          # float32 [Cout][Cin][kt][kh][kw]
    b: np.ndarray          # float32 [Cout]
    w_proj: np.ndarray | None = None   # float32 [Cp][Cin][1][1][1]
    b_proj: np.ndarray | None = None


def _bf16_bits_ndhwc(x: torch.Tensor) -> np.ndarray:
    xb = x.to(torch.bfloat16).permute(0, 2, 3, 4, 1).contiguous()
    return xb.view(torch.int16).numpy().view(np.uint16)


def draw_conv(spec: ConvSpec, gen: torch.Generator) -> ConvInputs:
    shape = (spec.N, spec.Cin, spec.T, spec.H, spec.W)
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if spec.x_kind == "silu":
        x = x * torch.sigmoid(x)
    elif spec.x_kind == "outlier":
        mask = torch.rand(shape, generator=gen, dtype=torch.float32) < 0.05
        x = torch.where(mask, x * 20.0, x)
    elif spec.x_kind != "normal":
        raise ValueError(spec.x_kind)
    kt, kh, kw = spec.k
    w = torch.randn((spec.Cout, spec.Cin, kt, kh, kw), generator=gen,
                    dtype=torch.float32) * 0.02
    b = torch.randn((spec.Cout,), generator=gen, dtype=torch.float32) * 0.01
    out = ConvInputs(spec, _bf16_bits_ndhwc(x), w.numpy(), b.numpy())
    del x
    if spec.proj_cout:
        wp = torch.randn((spec.proj_cout, spec.Cin, 1, 1, 1), generator=gen,
                         dtype=torch.float32) * 0.02
        bp = torch.randn((spec.proj_cout,), generator=gen, dtype=torch.float32) * 0.01
        out.w_proj, out.b_proj = wp.numpy(), bp.numpy()
    return out


def draw_workload(key: str, only: int | None = None):
    """All convs of a workload, drawn in order from its seed.  ``only`` keeps
    one level (earlier levels are still drawn so the stream stays the same)."""
    wl = WORKLOADS[key]
    gen = torch.Generator().manual_seed(wl.seed)
    out = []
    for i, spec in enumerate(wl.convs):
        ci = draw_conv(spec, gen)
        if only is None or only == i:
            out.append(ci)
        else:
            del ci
        if only is not None and i >= only:
            break
    return out


def draw_custom(seed: int, N, Cin, Cout, T, H, W, k=(3, 3, 3), x_kind="normal",
                x_scale: float = 1.0) -> ConvInputs:
    """A small conv of any shape with the same recipe (for parity sweeps)."""
    gen = torch.Generator().manual_seed(seed)
    spec = ConvSpec(f"custom_s{seed}", N, Cin, Cout, T, H, W, k=tuple(k), x_kind=x_kind)
    ci = draw_conv(spec, gen)
    if x_scale != 1.0:
        xf = torch.from_numpy(ci.x.view(np.int16)).view(torch.bfloat16).float() * x_scale
        ci.x = xf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return ci


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact; a change of representation)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)
