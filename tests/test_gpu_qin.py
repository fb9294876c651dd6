"""GPU parity of the conv that quantizes its own bf16 input (and cache):
bit for bit against the oracle (quantize the tensor the cache and x belong to,
then the INT32 conv and the epilogue) on small shapes, and against the
library's own two-step path (quantize pass + conv) at decoder sizes."""
import numpy as np
import pytest
import torch

import oracle
from tests.test_gpu_parity import DEV, bf16_bits, f32_bits, sample_positions, to_dev_bits, ulp_dist

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w8a8_int8_quantized_act_amd import ops as o
    o.lib()
    return o


def _draw(seed, N, T, H, W, Cin, Cout, k, with_cache, kind="silu", scale=1.0):
    g = torch.Generator().manual_seed(seed)
    frames = T + (k[0] - 1 if with_cache else 0)
    full = torch.randn(N, frames, H, W, Cin, generator=g) * scale
    if kind == "silu":
        full = full * torch.sigmoid(full)
    w = (torch.randn(Cout, Cin, *k, generator=g) * 0.03).numpy()
    b = (torch.randn(Cout, generator=g) * 0.01).numpy()
    fb = full.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return fb, w, b


def _run(ops, fb, w, b, T, kt, with_cache, clip=1.0):
    full_d = to_dev_bits(fb)
    x = full_d[:, kt - 1:].contiguous() if with_cache else full_d
    cache = full_d[:, :kt - 1].contiguous() if with_cache else None
    am = ops.act_absmax(full_d)                      # the maxima of the tensor x and its cache belong to
    wq, ws = ops.quantize_weights(torch.from_numpy(w).to(DEV), clip)
    bd = torch.from_numpy(b).to(DEV)
    y, xs = ops.causalconv3d_w8a8_qin(x, am, wq, ws, bd, cache, clip_ratio=clip)
    # the two-step path on the same inputs
    xs2, xq_full = ops.act_quantize(full_d, am, clip)
    xq = xq_full[:, kt - 1:].contiguous() if with_cache else xq_full
    cq = xq_full[:, :kt - 1].contiguous() if with_cache else None
    y2 = ops.causalconv3d_w8a8(xq, xs2, wq, ws, bd, cq)
    torch.cuda.synchronize()
    return y, xs, y2, xs2, am, xq_full


SMALL = [
    # N, T, H, W, Cin, Cout, k, cache
    (1, 3, 19, 37, 64, 96, (3, 3, 3), True),
    (2, 2, 11, 13, 96, 64, (3, 3, 3), False),
    (1, 1, 17, 33, 384, 384, (3, 3, 3), True),
    (1, 2, 20, 31, 384, 192, (1, 1, 1), False),
    (1, 3, 8, 24, 64, 96, (3, 1, 1), True),
    (1, 1, 25, 18, 192, 192, (1, 3, 3), False),
    (1, 1, 1, 1, 32, 32, (3, 3, 3), False),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}x{c[1]}x{c[2]}x{c[3]}_c{c[4]}-{c[5]}_k{''.join(map(str, c[6]))}"
                                             f"{'_cache' if c[7] else ''}" for c in SMALL])
def test_qin_small_against_oracle(ops, case):
    N, T, H, W, Cin, Cout, k, with_cache = case
    fb, w, b = _draw(1000 + sum(case[:6]), N, T, H, W, Cin, Cout, k, with_cache)
    y, xs, y2, xs2, am, _ = _run(ops, fb, w, b, T, k[0], with_cache)
    wq, ws = oracle.quantize_weights(w)
    a, s, q_full = oracle.act_absmax_quant(fb)
    kt = k[0]
    xq = q_full[:, kt - 1:] if with_cache else q_full
    cq = q_full[:, :kt - 1] if with_cache else None
    ref = oracle.epilogue(oracle.conv_acc(np.ascontiguousarray(xq), wq,
                                          None if cq is None else np.ascontiguousarray(cq)), s, ws, b)
    assert f32_bits(xs.item()) == f32_bits(s)
    assert int(am[0].item()) == f32_bits(a) >> 16
    assert ulp_dist(bf16_bits(y), ref).max() == 0
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("shape,with_cache", [((1, 96, 1, 1024, 1024), False), ((1, 192, 1, 512, 512), False),
                                              ((1, 384, 1, 256, 256), False), ((1, 384, 1, 128, 128), True),
                                              ((1, 384, 2, 105, 157), False), ((2, 96, 2, 90, 160), True)],
                         ids=["c96_1024", "c192_512", "c384_256", "c384_128_cache", "c384_105x157_t2",
                              "c96_n2_90x160_t2_cache"])
def test_qin_decoder_sizes_equal_two_step(ops, shape, with_cache):
    N, C, T, H, W = shape
    fb, w, b = _draw(1100 + C + T, N, T, H, W, C, C, (3, 3, 3), with_cache)
    y, xs, y2, xs2, am, xq_full = _run(ops, fb, w, b, T, 3, with_cache)
    assert f32_bits(xs.item()) == f32_bits(xs2.item())
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    # and the oracle on sampled positions
    pos = sample_positions(N, T, H, W, 200, 21)
    wq, ws = oracle.quantize_weights(w)
    a, s, q_full = oracle.act_absmax_quant(fb)
    assert np.array_equal(xq_full.cpu().numpy(), q_full)
    xq = np.ascontiguousarray(q_full[:, 2:] if with_cache else q_full)
    cq = np.ascontiguousarray(q_full[:, :2]) if with_cache else None
    ref = oracle.epilogue(oracle.conv_acc(xq, wq, cq, positions=pos), s, ws, b)
    assert ulp_dist(bf16_bits(y.reshape(-1, C)[torch.from_numpy(pos).to(DEV)]), ref).max() == 0


def test_qin_clip_and_zero_input(ops):
    N, T, H, W, C = 1, 2, 23, 29, 96
    fb, w, b = _draw(1200, N, T, H, W, C, C, (3, 3, 3), True, kind="normal", scale=3.0)
    y, xs, y2, xs2, _, xq_full = _run(ops, fb, w, b, T, 3, True, clip=0.5)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert f32_bits(xs.item()) == f32_bits(xs2.item())
    assert int((xq_full.abs() == 127).sum().item()) > 100          # the clamp fired
    # an all-zero tensor: scale 0, every code 0, y = bias
    z = np.zeros_like(fb)
    y0, xs0, y02, _, _, _ = _run(ops, z, w, b, T, 3, True)
    assert xs0.item() == 0.0
    assert torch.equal(y0.view(torch.int16), y02.view(torch.int16))
    bb = torch.from_numpy(b).to(torch.bfloat16).view(torch.int16).to(DEV)
    assert torch.equal(y0.view(torch.int16).reshape(-1, C), bb.expand(N * T * H * W, C))


def test_binding_rejects_a_short_maximum_buffer(ops):
    x = torch.zeros(1, 1, 4, 4, 32, dtype=torch.bfloat16, device=DEV)
    for bad in (torch.zeros(100, dtype=torch.int32, device=DEV), torch.zeros(513, dtype=torch.float32, device=DEV)):
        with pytest.raises(ValueError):
            ops.act_quantize(x, bad)
