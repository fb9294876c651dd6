"""GPU parity of the native-precision path (the layers a preset leaves
unquantized) and of the per-layer preset runner, through the C ABI.

Bar for the bf16 conv (FP32 accumulation in the matrix cores' order, so not
bit-exact against any fixed order): against the oracle's exact value z and
magnitude sum m = sum |x w| + |bias| of every checked output,
  |y - z| <= e + 2^-8 (|z| + e),   e = (K/16 + 16) 2^-23 m,
where K = Cin kt kh kw: at most one FP32 rounding per 16-product matrix step
plus the products' sum inside a step (at most 16 terms), doubled for safety,
then the bf16 rounding (half an ulp, at most 2^-8 relative).  On top of the
bound, at least 97 % of the outputs must equal bf16_rne(z) exactly.
Where results must be identical by construction (zero cache vs front
padding, chunked vs unchunked, the runner vs the entry point it calls),
the test asks for bit equality.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.layout import pack_weights_bf16 as pack_ref
from tests.test_gpu_parity import DEV, bf16_bits, sample_positions, to_dev_bits, ulp_dist
from w8a8_int8_quantized_act_amd import decoder
from w8a8_int8_quantized_act_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w8a8_int8_quantized_act_amd import ops as o
    o.lib()
    return o


def _bits(t):
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _draw(seed, N, T, H, W, Cin, Cout, k, with_cache, x_kind="silu"):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(N, T, H, W, Cin, generator=g)
    if x_kind == "silu":
        x = x * torch.sigmoid(x)
    w = torch.randn(Cout, Cin, *k, generator=g) * 0.05
    b = (torch.randn(Cout, generator=g) * 0.05).numpy()
    cache = _bits(torch.randn(N, k[0] - 1, H, W, Cin, generator=g)) if with_cache and k[0] > 1 else None
    return _bits(x), _bits(w), b, cache


def _check(y_bits, z, mag, K):
    y = wl.bf16_bits_to_f32(y_bits).astype(np.float64)
    e = (K / 16 + 16) * 2.0 ** -23 * mag
    bound = e + 2.0 ** -8 * (np.abs(z) + e) + 1e-38
    over = np.abs(y - z) > bound
    assert not over.any(), f"{over.sum()} outputs outside the bound, worst ratio {np.max(np.abs(y - z) / bound):.3g}"
    zr = torch.from_numpy(np.ascontiguousarray(z)).to(torch.float32).to(torch.bfloat16)
    same = np.mean(zr.view(torch.int16).numpy().view(np.uint16) == y_bits)
    assert same >= 0.97, f"only {same:.4f} of the outputs equal bf16_rne(z)"


def _run(ops, x, w, b, cache):
    wp = ops.pack_weights_bf16(to_dev_bits(w))
    y = ops.causalconv3d_bf16(to_dev_bits(x), wp, torch.from_numpy(b).to(DEV),
                              None if cache is None else to_dev_bits(cache))
    torch.cuda.synchronize()
    return wp, y


SMALL = [
    # N, T, H, W, Cin, Cout, k, cache
    (1, 3, 19, 37, 96, 96, (3, 3, 3), False),
    (2, 2, 11, 13, 48, 64, (3, 3, 3), True),
    (1, 1, 9, 40, 16, 32, (3, 3, 3), False),
    (1, 2, 20, 31, 384, 192, (1, 1, 1), False),
    (1, 3, 8, 24, 64, 96, (3, 1, 1), True),
    (1, 1, 25, 18, 192, 192, (1, 3, 3), False),
    (1, 1, 17, 33, 384, 384, (3, 3, 3), True),
    (1, 1, 1, 1, 16, 32, (3, 3, 3), False),
    (1, 2, 12, 20, 192, 384, (3, 3, 3), False),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}x{c[1]}x{c[2]}x{c[3]}_c{c[4]}-{c[5]}_k{''.join(map(str, c[6]))}"
                                             f"{'_cache' if c[7] else ''}" for c in SMALL])
def test_bf16_conv_small_full(ops, case):
    N, T, H, W, Cin, Cout, k, with_cache = case
    x, w, b, cache = _draw(500 + sum(case[:6]), N, T, H, W, Cin, Cout, k, with_cache)
    wp, y = _run(ops, x, w, b, cache)
    assert np.array_equal(wp.view(torch.int16).cpu().numpy().view(np.uint16), pack_ref(w))
    z, mag = oracle.conv_bf16(x, w, b, cache)
    _check(bf16_bits(y), z, mag, Cin * k[0] * k[1] * k[2])


@pytest.mark.parametrize("shape,with_cache", [((1, 96, 1, 1024, 1024), False), ((1, 384, 1, 128, 128), True),
                                              ((1, 192, 2, 420, 628), False), ((1, 384, 3, 105, 157), True)],
                         ids=["c96_1024", "c384_128_cache", "c192_420x628_t2", "c384_105x157_t3_cache"])
def test_bf16_conv_decoder_sizes_sampled(ops, shape, with_cache):
    N, C, T, H, W = shape
    x, w, b, cache = _draw(600 + C + T, N, T, H, W, C, C, (3, 3, 3), with_cache)
    _, y = _run(ops, x, w, b, cache)
    pos = sample_positions(N, T, H, W, 600, 13)
    z, mag = oracle.conv_bf16(x, w, b, cache, positions=pos)
    got = bf16_bits(y.reshape(-1, C)[torch.from_numpy(pos).to(DEV)])
    _check(got, z, mag, C * 27)


def test_bf16_conv_zero_cache_and_chunks_bit_exact(ops):
    N, T, H, W, C = 1, 4, 40, 72, 384
    x, w, b, _ = _draw(700, N, T, H, W, C, C, (3, 3, 3), False)
    xd = to_dev_bits(x)
    wp = ops.pack_weights_bf16(to_dev_bits(w))
    bd = torch.from_numpy(b).to(DEV)
    full = ops.causalconv3d_bf16(xd, wp, bd)
    zc = ops.causalconv3d_bf16(xd, wp, bd, torch.zeros((N, 2, H, W, C), dtype=torch.bfloat16, device=DEV))
    chunked = torch.empty_like(full)
    ops.causalconv3d_bf16(xd[:, :2].contiguous(), wp, bd, out=chunked[:, :2])
    ops.causalconv3d_bf16(xd[:, 2:].contiguous(), wp, bd, xd[:, :2].contiguous(), out=chunked[:, 2:])
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), zc.view(torch.int16))
    # frames 2, 3 with the cache see the same taps, but in the unchunked call frames 0, 1
    # come from the input, not a cache: same values, same order -> the same FP32 sums
    assert torch.equal(full.view(torch.int16), chunked.view(torch.int16))


# ------------------------------------------------------------------ the preset runner
@pytest.fixture(scope="module")
def stack(ops):
    """The 28 decoder convs at a 128 x 128 output (16 x 16 latent), with
    seeded bf16 weights, float32 biases and one bf16 input per layer."""
    layers = decoder.residual_convs(128, 128)
    g = torch.Generator().manual_seed(800)
    data = []
    for L in layers:
        w = (torch.randn(L.Cout, L.Cin, 3, 3, 3, generator=g) * 0.03).to(torch.bfloat16)
        b = torch.randn(L.Cout, generator=g) * 0.02
        x = torch.randn(1, 1, L.H, L.W, L.Cin, generator=g)
        x = (x * torch.sigmoid(x)).to(torch.bfloat16)
        data.append((L, w.to(DEV), b.to(DEV), x.to(DEV)))
    return data


@pytest.mark.parametrize("preset,count", [("native", 0), ("conservative", 15), ("balanced", 22),
                                          ("aggressive", 26)])
def test_runner_follows_the_plan(ops, stack, preset, count):
    n_w8a8 = 0
    for L, w, b, x in stack:
        conv = decoder.PlannedConv(L.name, w, b, preset)
        y = conv(x)
        if conv.w8a8:
            n_w8a8 += 1
            wq, ws = ops.quantize_weights(w.float())
            _, xs, xq = ops.act_absmax_quant(x)
            ref = ops.causalconv3d_w8a8(xq, xs, wq, ws, b)
        else:
            ref = ops.causalconv3d_bf16(x, ops.pack_weights_bf16(w), b)
        torch.cuda.synchronize()
        assert conv.fallbacks == 0
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), L.name
    assert n_w8a8 == count


def test_runner_quantize_in_conv_equals_two_step(ops, stack):
    # the input-quantizing conv gives the runner's W8A8 layers bit-identical results
    for L, w, b, x in stack[:12]:
        two = decoder.PlannedConv(L.name, w, b, "balanced", quantize_in_conv=False)
        one = decoder.PlannedConv(L.name, w, b, "balanced", quantize_in_conv=True)
        assert two.w8a8 == one.w8a8
        y2, y1 = two(x), one(x)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), L.name


def test_runner_w8a8_layer_against_the_oracle(ops, stack):
    L, w, b, x = stack[10]                     # decoder.upsamples.4.residual.2, 192 -> 384 @ 32x32
    conv = decoder.PlannedConv(L.name, w, b, "balanced")
    assert conv.w8a8 and L.Cin == 192 and L.Cout == 384
    y = conv(x)
    torch.cuda.synchronize()
    wq, ws = oracle.quantize_weights(w.float().cpu().numpy())
    ref, _ = oracle.layer(bf16_bits(x), wq, ws, b.cpu().numpy())
    assert ulp_dist(bf16_bits(y), ref).max() == 0


def test_runner_falls_back_per_layer(ops, stack, monkeypatch):
    L, w, b, x = stack[0]
    native = ops.causalconv3d_bf16(x, ops.pack_weights_bf16(w), b)
    loaded = decoder.PlannedConv(L.name, w, b, "aggressive")     # quantized while W8A8 works
    assert loaded.w8a8
    monkeypatch.setenv("QVAE_FORCE_FAIL", "w8a8")
    y1 = loaded(x)                                              # the W8A8 calls fail -> native
    fresh = decoder.PlannedConv(L.name, w, b, "aggressive")     # weight quantization fails at load
    y2 = fresh(x)
    torch.cuda.synchronize()
    assert loaded.fallbacks == 1 and fresh.fallbacks == 1 and not fresh.w8a8
    assert torch.equal(y1.view(torch.int16), native.view(torch.int16))
    assert torch.equal(y2.view(torch.int16), native.view(torch.int16))
    monkeypatch.delenv("QVAE_FORCE_FAIL")
    y3 = loaded(x)
    torch.cuda.synchronize()
    assert loaded.fallbacks == 1 and not torch.equal(y3.view(torch.int16), native.view(torch.int16))
