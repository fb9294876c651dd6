"""GPU parity of the norm + SiLU pass (with and without the fused activation
maximum) against the oracle, through the C ABI.

The oracle computes h = bf16_rne(SiLU(x * gamma / sqrt(mean(x^2) + eps))) in
binary64, rounded once; the pass computes the same quantity in binary32 with
its own exp.  Bar: every GPU value within one bf16 ulp of the oracle's (ordinal
distance of the bit patterns), and at least 99.9 % of them equal.  What is
built on h is integer and exact, so it is compared bit for bit against the
oracle run on the GPU's own h: the fused maximum, the scale, the codes and the
conv's output.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.test_gpu_parity import DEV, bf16_bits, f32_bits, sample_positions, to_dev_bits, ulp_dist

pytestmark = pytest.mark.gpu

MIN_EQUAL = 0.999   # share of h values equal to the oracle's (the rest one ulp away)


def _check_h(got, ref):
    d = ulp_dist(got, ref)
    assert d.max() <= 1, f"{np.count_nonzero(d > 1)} values more than one ulp off, first at {np.argwhere(d > 1)[:3].tolist()}"
    ne = np.count_nonzero(d)
    assert ne <= max(2, (1 - MIN_EQUAL) * d.size), f"{ne} of {d.size} values differ by one ulp"


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w8a8_int8_quantized_act_amd import ops as o
    o.lib()
    return o


def _draw(seed, npix, C, kind="silu", scale=1.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(npix, C, generator=g) * scale
    if kind == "silu":
        x = x * torch.sigmoid(x)
    if npix > 5:
        x[5] = 0.0                                         # an all-zero pixel
    gamma = (1.0 + 0.2 * torch.randn(C, generator=g)).float()
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), gamma.numpy()


CASES = [(1, 8, 1e-6), (7, 96, 1e-6), (1000, 96, 1e-6), (333, 192, 0.1), (129, 384, 1e-6), (16384, 384, 1e-6),
         (4097, 480, 1e-6), (3001, 16, 1e-3), (65536 + 17, 192, 1e-6)]


@pytest.mark.parametrize("npix,C,eps", CASES, ids=[f"{c[0]}x{c[1]}_eps{c[2]:g}" for c in CASES])
def test_rmsnorm_silu_within_one_ulp(ops, npix, C, eps):
    xb, gamma = _draw(900 + C + npix % 97, npix, C)
    x = to_dev_bits(xb).view(npix, C)
    gd = torch.from_numpy(gamma).to(DEV)
    h = ops.rmsnorm_silu(x, gd, eps)
    stale = torch.full((ops.ABSMAX_WORDS,), 0x7F7F, dtype=torch.int32, device=DEV)
    h2, am = ops.rmsnorm_silu(x, gd, eps, absmax_bits=stale, with_absmax=True)
    xs, xq = ops.act_quantize(h2, am)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_silu(xb.reshape(npix, C), gamma, eps)
    got = bf16_bits(h)
    _check_h(got, ref)
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16))
    # the fused maximum, the scale and the codes: exact, from the GPU's h
    a, s, q = oracle.act_absmax_quant(got)
    assert int(am[0].item()) == f32_bits(a) >> 16
    assert f32_bits(xs.item()) == f32_bits(s)
    assert np.array_equal(xq.cpu().numpy(), q)


def test_rmsnorm_silu_full_level_and_large_values(ops):
    # the 96-channel level at 1024 x 1024 (100 M values), and inputs scaled by 1000
    for npix, C, scale, seed in [(1024 * 1024, 96, 1.0, 950), (50000, 96, 1000.0, 951)]:
        xb, gamma = _draw(seed, npix, C, kind="normal", scale=scale)
        x = to_dev_bits(xb).view(npix, C)
        h, am = ops.rmsnorm_silu(x, torch.from_numpy(gamma).to(DEV), 1e-6, with_absmax=True)
        xs, xq = ops.act_quantize(h, am)
        torch.cuda.synchronize()
        ref = oracle.rmsnorm_silu(xb.reshape(npix, C), gamma, 1e-6)
        got = bf16_bits(h)
        _check_h(got, ref)
        a, s, q = oracle.act_absmax_quant(got)
        assert int(am[0].item()) == f32_bits(a) >> 16
        assert f32_bits(xs.item()) == f32_bits(s)
        assert np.array_equal(xq.cpu().numpy(), q)


def test_rmsnorm_silu_wide_gamma_and_near_ties(ops):
    """Normalised values far outside the SiLU's central range (|n| up to a few
    hundred: exp(-n) overflows below n ~ -88.7, and |n| > 64 takes the pass's
    correctly rounded division), and enough values (4 M) that quotients next
    to a bf16 rounding boundary (about 3 in 65536) occur hundreds of times."""
    for npix, C, gscale, seed in [(20000, 96, 40.0, 952), (1 << 15, 128, 1.0, 953)]:
        xb, gamma = _draw(seed, npix, C, kind="normal")
        gamma = (gamma * gscale * np.where(np.arange(C) % 3 == 0, -1.0, 1.0)).astype(np.float32)
        x = to_dev_bits(xb).view(npix, C)
        h = ops.rmsnorm_silu(x, torch.from_numpy(gamma).to(DEV), 1e-6)
        torch.cuda.synchronize()
        ref = oracle.rmsnorm_silu(xb.reshape(npix, C), gamma, 1e-6)
        _check_h(bf16_bits(h), ref)


def test_residual_branch_norm_silu_quantize_conv(ops):
    """x -> RMSNorm + SiLU (with the fused maximum) -> quantize (no absmax pass)
    -> W8A8 conv: h against the oracle's within one ulp, then the oracle's
    quantizer and conv on the GPU's h against the GPU's scale and output."""
    N, T, H, W, C = 1, 2, 37, 45, 192
    xb, gamma = _draw(960, N * T * H * W, C, kind="normal")
    g = torch.Generator().manual_seed(961)
    w = (torch.randn(C, C, 3, 3, 3, generator=g) * 0.03).numpy()
    b = (torch.randn(C, generator=g) * 0.01).numpy()
    x = to_dev_bits(xb).view(N, T, H, W, C)
    h, am = ops.rmsnorm_silu(x, torch.from_numpy(gamma).to(DEV), 1e-6, with_absmax=True)
    xs, xq = ops.act_quantize(h, am)
    wq_d, ws_d = ops.quantize_weights(torch.from_numpy(w).to(DEV))
    y = ops.causalconv3d_w8a8(xq, xs, wq_d, ws_d, torch.from_numpy(b).to(DEV))
    torch.cuda.synchronize()
    hg = bf16_bits(h)
    _check_h(hg.reshape(-1, C), oracle.rmsnorm_silu(xb.reshape(N * T * H * W, C), gamma, 1e-6))
    wq, ws = oracle.quantize_weights(w)
    pos = sample_positions(N, T, H, W, 400, 17)
    yref, s = oracle.layer(hg, wq, ws, b, positions=pos)
    assert f32_bits(xs.item()) == f32_bits(s)
    assert ulp_dist(bf16_bits(y.reshape(-1, C)[torch.from_numpy(pos).to(DEV)]), yref).max() == 0


def test_rmsnorm_silu_rejects(ops):
    x = torch.zeros(4, 96, dtype=torch.bfloat16, device=DEV)
    gd = torch.ones(96, device=DEV)
    for eps in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(ops.QvaeError) as e:
            ops.rmsnorm_silu(x, gd, eps)
        assert e.value.status == ops.EINVAL
    with pytest.raises(ops.QvaeError) as e:
        ops.rmsnorm_silu(torch.zeros(4, 100, dtype=torch.bfloat16, device=DEV), torch.ones(100, device=DEV))
    assert e.value.status == ops.EUNSUPPORTED
    with pytest.raises(ops.QvaeError) as e:
        ops.rmsnorm_silu(torch.zeros(4, 512, dtype=torch.bfloat16, device=DEV), torch.ones(512, device=DEV))
    assert e.value.status == ops.EUNSUPPORTED


def test_residual_branches_in_hip_graph(ops):
    """Both residual branches captured once and replayed several times, with eager
    work in between; every replay equals the eager result bit for bit."""
    N, T, H, W, C = 1, 2, 23, 31, 96
    xb, gamma = _draw(970, N * T * H * W, C, kind="normal")
    g = torch.Generator().manual_seed(971)
    w = (torch.randn(C, C, 3, 3, 3, generator=g) * 0.03).to(torch.bfloat16)
    b = (torch.randn(C, generator=g) * 0.01).to(DEV)
    x = to_dev_bits(xb).view(N, T, H, W, C)
    gd = torch.from_numpy(gamma).to(DEV)
    wq, ws = ops.quantize_weights(w.float().to(DEV))
    wp = ops.pack_weights_bf16(w.to(DEV))
    h = torch.empty_like(x)
    am = torch.empty((ops.ABSMAX_WORDS,), dtype=torch.int32, device=DEV)
    xs = torch.empty((1,), dtype=torch.float32, device=DEV)
    xq = torch.empty(x.shape, dtype=torch.int8, device=DEV)
    y8 = torch.empty_like(x)
    yn = torch.empty_like(x)
    # eager references
    he, ame = ops.rmsnorm_silu(x, gd, 1e-6, with_absmax=True)
    xse, xqe = ops.act_quantize(he, ame)
    y8e = ops.causalconv3d_w8a8(xqe, xse, wq, ws, b)
    yne = ops.causalconv3d_bf16(ops.rmsnorm_silu(x, gd, 1e-6), wp, b)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops.rmsnorm_silu(x, gd, 1e-6, out=h, absmax_bits=am, with_absmax=True)
        ops.act_quantize(h, am, x_scale=xs, xq=xq)
        ops.causalconv3d_w8a8(xq, xs, wq, ws, b, out=y8)
        ops.rmsnorm_silu(x, gd, 1e-6, out=h)
        ops.causalconv3d_bf16(h, wp, b, out=yn)
    for rep in range(4):
        y8.zero_()
        yn.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y8.view(torch.int16), y8e.view(torch.int16)), f"W8A8 branch, replay {rep}"
        assert torch.equal(yn.view(torch.int16), yne.view(torch.int16)), f"native branch, replay {rep}"
        other = ops.rmsnorm_silu(x, gd, 0.5)                    # eager work between replays
        torch.cuda.synchronize()
        del other


def _silu64(n):
    return n / (1.0 + np.exp(-n))


def _near_tie_gammas(C, r, seed):
    """Per-channel gammas for a pixel of all-ones x (so n_c = r * gamma_c up to
    binary32 rounding) whose SiLU value sits within a few binary32 ulps of a
    bf16 rounding boundary (the midpoint between two bf16 values), solved for
    with the binary64 SiLU."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < C:
        # positive values up to 12; negative ones above SiLU's minimum (~ -0.278)
        mag = float(rng.uniform(0.05, 12.0)) if rng.random() < 0.7 else -float(rng.uniform(0.01, 0.27))
        t_bits = (int(np.float32(mag).view(np.uint32)) & 0xFFFF0000) | 0x8000   # a bf16 midpoint
        T = float(np.uint32(t_bits).view(np.float32))
        n = T if T > 0 else -1.0
        for _ in range(60):   # Newton on n / (1 + exp(-n)) = T (binary64)
            s = 1.0 / (1.0 + np.exp(-n))
            f, df = n * s - T, s + n * s * (1.0 - s)
            if df == 0.0:
                break
            n -= f / df
        g = np.float32(n / float(r))
        v = _silu64(float(np.float32(r * g)))
        if abs(v - T) <= 4 * 2.0 ** -24 * abs(T):
            out.append(g)
    return np.array(out, dtype=np.float32)


def test_rmsnorm_silu_values_at_bf16_boundaries(ops):
    """Every value of pixel 0 (x = 1 in all channels) has its SiLU within a few
    binary32 ulps of a bf16 rounding boundary, where the pass's reciprocal-based
    quotient may be one binary32 ulp off and must take the correctly rounded
    division; the other pixels are ordinary data.  Each value stays within one
    ulp of the oracle's."""
    C, eps = 96, 1e-6
    r = 1.0 / np.sqrt(1.0 + eps)
    gamma = _near_tie_gammas(C, r, 77)
    ones = np.float32(1.0).view(np.uint32) >> 16
    xb, _ = _draw(954, 300, C)
    xb = xb.reshape(300, C).copy()
    xb[0, :] = ones
    x = to_dev_bits(xb).view(300, C)
    h = ops.rmsnorm_silu(x, torch.from_numpy(gamma).to(DEV), eps)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_silu(xb, gamma, eps)
    got = bf16_bits(h)
    assert ulp_dist(got[0], ref[0]).max() <= 1
    _check_h(got[1:], ref[1:])
