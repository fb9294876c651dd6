"""Pins for the CPU oracle, against things other than itself.

Each test ties one oracle function to a value the mathematics fixes: a
closed form, an invariant, brute force on tiny inputs, a float64 library
convolution on integer-valued tensors (exact, since every partial sum is an
integer below 2^53), or a derived error bound against the unquantized float
convolution.  The scheme being pinned is the one on the ComfyUI-Qwen-VAE-Triton
v0.2.0 page, section "Three presets explained": symmetric per-output-channel
INT8 weights, dynamic symmetric INT8 activations, INT32 accumulation, FP32
rescale, output in the activation precision, clip ratio 1.0 (the page's
fixed value; ratios below 1, where the clamp to +-127 fires, are pinned too).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from tests.bruteforce import conv_acc_bruteforce
from w8a8_int8_quantized_act_amd import workloads as wl


def bits(x_f32):
    """float32 values that are exactly representable in bf16 -> bf16 bits."""
    a = np.asarray(x_f32, np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def f32(b):
    return wl.bf16_bits_to_f32(np.asarray(b, np.uint16))


# --------------------------------------------------------------- bf16 rounding
@pytest.mark.parametrize("val,expect", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),              # exactly half an ulp above 1: tie -> even (1.0)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),          # half an ulp above 1+2^-7: tie -> even (1+2^-6)
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # just above the tie -> up
    (1.0 + 2.0 ** -8 - 2.0 ** -20, 0x3F80),  # just below the tie -> down
    (-(1.0 + 2.0 ** -8), 0xBF80),
    (-(1.0 + 3 * 2.0 ** -8), 0xBF82),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (3.0, 0x4040),
    (2.0 ** -126, 0x0080),                  # smallest normal
    (2.0 ** -130, 0x0008),                  # subnormal, exact
    (255.5, 0x4380),                        # 255.5 = 0x437F8000: tie, 0x437F odd -> 0x4380 (256)
])
def test_bf16_rne_closed_form(oracle, val, expect):
    assert oracle.f32_to_bf16(np.float32(val)) == expect


def test_bf16_roundtrip_exact(oracle):
    for h in [0x0001, 0x3F80, 0x7F7F, 0x8001, 0xC2F7, 0x1234]:
        assert oracle.f32_to_bf16(oracle.bf16_to_f32(h)) == h


def test_bf16_rne_matches_torch_cast(oracle):
    # torch's float32 -> bfloat16 cast is an independent round-to-nearest-even
    g = torch.Generator().manual_seed(7)
    v = (torch.randn(4000, generator=g) * torch.exp(torch.randn(4000, generator=g) * 4)).float()
    ref = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(float(t)) for t in v.numpy()], np.uint16)
    assert np.array_equal(ref, got)


# --------------------------------------------------------------- activation quantization
def test_rne_special_case_scale_one(oracle):
    # absmax 127 -> s = fl(127/127) = 1, so q is x rounded half to even.
    x = np.array([127.0, 0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 3.5, -3.5, 126.5, -126.5,
                  0.25, -0.75, 0.0, -127.0], np.float32)
    a, s, q = oracle.act_absmax_quant(bits(x))
    assert a == np.float32(127.0) and s == np.float32(1.0)
    assert q.tolist() == [127, 0, 0, 2, -2, 2, -2, 4, -4, 126, -126, 0, -1, 0, -127]


def test_act_absmax_is_max_magnitude(oracle):
    x = np.array([0.5, -3.0, 2.0, -0.125], np.float32)
    assert oracle.act_absmax(bits(x)) == np.float32(3.0)
    assert oracle.act_absmax(bits(np.zeros(5, np.float32))) == 0.0


def test_act_scale_closed_form(oracle):
    # s = fl(a / 127) in binary32
    for a in [1.0, 3.0, 20.5, 0.0078125, 65280.0]:
        assert oracle.scale_from_absmax(a) == np.float32(np.float32(a) / np.float32(127.0))
    # clip ratio multiplies the max before the division
    assert oracle.scale_from_absmax(2.0, 0.5) == np.float32(1.0) / np.float32(127.0)


def test_act_quantize_invariants(oracle):
    g = torch.Generator().manual_seed(11)
    x = (torch.randn(50000, generator=g) * 3).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    a, s, q = oracle.act_absmax_quant(xb)
    xf = f32(xb).astype(np.float64)
    # the extreme element maps to +-127, and nothing is clamped at clip 1.0
    assert np.abs(q.astype(int)).max() == 127
    assert q[np.argmax(np.abs(xf))] == (127 if xf[np.argmax(np.abs(xf))] > 0 else -127)
    # dequantization error at most half a step (plus the division's rounding)
    err = np.abs(xf - q.astype(np.float64) * float(s))
    assert np.all(err <= float(s) * (0.5 + 2.0 ** -17))
    # odd symmetry of round-half-to-even
    qn = oracle.act_quantize(xb ^ np.uint16(0x8000), s)
    assert np.array_equal(qn.astype(int), -q.astype(int))
    # monotone in x
    order = np.argsort(xf, kind="stable")
    assert np.all(np.diff(q[order].astype(int)) >= 0)


def test_act_quantize_matches_numpy_rint(oracle):
    # numpy's float32 division and rint (half to even) are an independent library path
    g = torch.Generator().manual_seed(12)
    x = (torch.randn(200000, generator=g) * 5).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    a, s, q = oracle.act_absmax_quant(xb)
    ref = np.clip(np.rint(f32(xb) / np.float32(s)), -127, 127).astype(np.int8)
    assert np.array_equal(q, ref)


def test_act_quantize_all_zero(oracle):
    a, s, q = oracle.act_absmax_quant(np.zeros(64, np.uint16))
    assert a == 0 and s == 0 and not q.any()


@pytest.mark.parametrize("clip,min_clamped", [(0.5, 500), (0.9, 5)])
def test_act_quantize_clip_below_one(oracle, clip, min_clamped):
    # a clip ratio below 1 shrinks the scale; the clamp maps the clipped tail to +-127
    g = torch.Generator().manual_seed(14)
    x = (torch.randn(50000, generator=g) * 3).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    a, s, q = oracle.act_absmax_quant(xb, clip)
    assert a == oracle.act_absmax(xb)
    assert s == np.float32(np.float32(clip) * np.float32(a)) / np.float32(127)
    assert s < oracle.scale_from_absmax(a)
    xf = f32(xb).astype(np.float64)
    qi = q.astype(int)
    # numpy's float32 division and rint (half to even), then the clamp
    ref = np.clip(np.rint(f32(xb) / np.float32(s)), -127, 127).astype(np.int8)
    assert np.array_equal(q, ref)
    # beyond 128 steps the code is +-127 with the sign of x, and the clamp really fires
    far = np.abs(xf) >= 128.0 * float(s)
    assert far.sum() >= min_clamped
    assert np.all(qi[far] == np.where(xf[far] > 0, 127, -127))
    # inside the clip range the usual half-step error bound holds
    inside = np.abs(xf) <= 127.0 * float(s)
    err = np.abs(xf[inside] - qi[inside] * float(s))
    assert np.all(err <= float(s) * (0.5 + 2.0 ** -17))
    # odd symmetry and monotonicity survive the clamp
    qn = oracle.act_quantize(xb ^ np.uint16(0x8000), s)
    assert np.array_equal(qn.astype(int), -qi)
    order = np.argsort(xf, kind="stable")
    assert np.all(np.diff(qi[order]) >= 0)


# --------------------------------------------------------------- weight quantization
def test_weight_quant_per_channel_closed_form(oracle):
    w = np.zeros((3, 2, 3, 3, 3), np.float32)
    w[0, 1, 2, 1, 0] = 1.27        # max of channel 0
    w[0, 0, 0, 0, 0] = -0.635      # half of it
    w[1, 0, 1, 1, 1] = -2.54       # channel 1: negative max
    # channel 2 stays all-zero
    wq, s_w = oracle.quantize_weights(w)
    assert s_w[0] == np.float32(np.float32(1.27) / np.float32(127))
    assert s_w[1] == np.float32(np.float32(2.54) / np.float32(127))
    assert s_w[2] == 0
    # layout: [Cout][Cin][kt][kh][kw] -> [Cout][kt][kh][kw][Cin]
    assert wq[0, 2, 1, 0, 1] == 127
    assert wq[0, 0, 0, 0, 0] == -64           # -63.5 (about) rounds away from the tie
    assert wq[1, 1, 1, 1, 0] == -127
    assert not wq[2].any()
    assert np.count_nonzero(wq) == 3


def test_weight_quant_matches_numpy(oracle):
    g = torch.Generator().manual_seed(13)
    w = (torch.randn(32, 16, 3, 3, 3, generator=g) * 0.02).numpy()
    wq, s_w = oracle.quantize_weights(w)
    a = np.abs(w).reshape(32, -1).max(axis=1).astype(np.float32)
    s_ref = (a / np.float32(127)).astype(np.float32)
    assert np.array_equal(s_w, s_ref)
    q_ref = np.clip(np.rint(w / s_ref[:, None, None, None, None]), -127, 127).astype(np.int8)
    assert np.array_equal(wq, q_ref.transpose(0, 2, 3, 4, 1))
    # each channel's extreme weight maps to +-127
    assert np.all(np.abs(wq.reshape(32, -1).astype(int)).max(axis=1) == 127)


def test_weight_quant_clip_half_closed_form(oracle):
    # max 2.0 and clip 0.5: s = fl(1.0 / 127); weights at or beyond 1.0 clamp to +-127
    w = np.zeros((2, 32, 1, 1, 1), np.float32)
    w[0, :6, 0, 0, 0] = [2.0, -1.0, 1.5, 0.25, -0.125, 10.0 / 127.0]
    w[1, 3, 0, 0, 0] = -4.0
    w[1, 4, 0, 0, 0] = 1.0
    wq, s_w = oracle.quantize_weights(w, 0.5)
    assert s_w[0] == np.float32(1.0) / np.float32(127)
    assert s_w[1] == np.float32(2.0) / np.float32(127)
    assert wq[0, 0, 0, 0, :6].tolist() == [127, -127, 127, 32, -16, 10]
    # 1.0 / fl(2/127) rounds to exactly 63.5 in binary32: a tie, which goes to the even code
    assert wq[1, 0, 0, 0, 3] == -127 and wq[1, 0, 0, 0, 4] == 64
    assert np.count_nonzero(wq) == 8


@pytest.mark.parametrize("clip", [0.5, 0.9])
def test_weight_quant_clip_matches_numpy(oracle, clip):
    g = torch.Generator().manual_seed(15)
    w = (torch.randn(32, 16, 3, 3, 3, generator=g) * 0.02).numpy()
    wq, s_w = oracle.quantize_weights(w, clip)
    a = np.abs(w).reshape(32, -1).max(axis=1).astype(np.float32)
    s_ref = ((np.float32(clip) * a).astype(np.float32) / np.float32(127)).astype(np.float32)
    assert np.array_equal(s_w, s_ref)
    q_ref = np.clip(np.rint(w / s_ref[:, None, None, None, None]), -127, 127).astype(np.int8)
    assert np.array_equal(wq, q_ref.transpose(0, 2, 3, 4, 1))
    # every channel has clamped weights at these ratios (randn's tail beyond clip * max)
    clamped = (np.abs(wq.reshape(32, -1).astype(int)) == 127).sum(axis=1)
    assert np.all(clamped >= 1)


# --------------------------------------------------------------- the INT32 contraction
def _rand_int8(g, shape, lo=-127, hi=127):
    return torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int64).numpy().astype(np.int8)


def _torch_f64_conv(xq, wq, cache=None):
    """float64 torch conv3d over integer-valued tensors (exact)."""
    N, T, H, W, Cin = xq.shape
    Cout, kt, kh, kw, _ = wq.shape
    x = torch.from_numpy(xq.astype(np.float64)).permute(0, 4, 1, 2, 3)   # N C T H W
    if cache is not None:
        c = torch.from_numpy(cache.astype(np.float64)).permute(0, 4, 1, 2, 3)
        x = torch.cat([c, x], dim=2)
    else:
        x = F.pad(x, (0, 0, 0, 0, kt - 1, 0))
    x = F.pad(x, ((kw - 1) // 2, (kw - 1) // 2, (kh - 1) // 2, (kh - 1) // 2, 0, 0))
    w = torch.from_numpy(wq.astype(np.float64)).permute(0, 4, 1, 2, 3)   # Co Ci kt kh kw
    y = F.conv3d(x, w)
    return y.permute(0, 2, 3, 4, 1).numpy()


@pytest.mark.parametrize("with_cache", [False, True])
@pytest.mark.parametrize("k", [(3, 3, 3), (1, 1, 1), (3, 1, 1), (1, 3, 3)])
def test_conv_bruteforce_tiny(oracle, with_cache, k):
    if with_cache and k[0] == 1:
        pytest.skip("no cache frames when kt = 1")
    g = torch.Generator().manual_seed(21)
    N, T, H, W, Cin, Cout = 2, 3, 4, 5, 3, 4
    xq = _rand_int8(g, (N, T, H, W, Cin))
    wq = _rand_int8(g, (Cout,) + k + (Cin,))
    cache = _rand_int8(g, (N, k[0] - 1, H, W, Cin)) if with_cache else None
    got = oracle.conv_acc(xq, wq, cache)
    ref = conv_acc_bruteforce(xq.astype(int).tolist(), wq.astype(int).tolist(),
                              None if cache is None else cache.astype(int).tolist())
    assert np.array_equal(got, np.array(ref, np.int64))


@pytest.mark.parametrize("with_cache", [False, True])
def test_conv_matches_f64_library_conv(oracle, with_cache):
    g = torch.Generator().manual_seed(22)
    N, T, H, W, Cin, Cout = 1, 4, 9, 11, 32, 32
    xq = _rand_int8(g, (N, T, H, W, Cin))
    wq = _rand_int8(g, (Cout, 3, 3, 3, Cin))
    cache = _rand_int8(g, (N, 2, H, W, Cin)) if with_cache else None
    got = oracle.conv_acc(xq, wq, cache)
    ref = _torch_f64_conv(xq, wq, cache)
    assert np.array_equal(got.astype(np.float64), ref)


def test_conv_extreme_values_no_overflow(oracle):
    # all -127 inputs and +127 weights: |acc| = 127^2 * Cin * taps exactly
    N, T, H, W, Cin, Cout = 1, 3, 4, 4, 384, 32
    xq = np.full((N, T, H, W, Cin), -127, np.int8)
    wq = np.full((Cout, 3, 3, 3, Cin), 127, np.int8)
    acc = oracle.conv_acc(xq, wq)
    # interior position at t = 2: all 27 taps hit data
    assert acc[0, 2, 1, 1, 0] == -127 * 127 * Cin * 27
    # corner at t = 0: 1 temporal tap, 2x2 spatial taps
    assert acc[0, 0, 0, 0, 5] == -127 * 127 * Cin * 4


def test_conv_t1_reduces_to_conv2d(oracle):
    # T = 1 without cache: only the last temporal tap touches data.
    g = torch.Generator().manual_seed(23)
    Cin, Cout, H, W = 32, 64, 7, 13
    xq = _rand_int8(g, (1, 1, H, W, Cin))
    wq = _rand_int8(g, (Cout, 3, 3, 3, Cin))
    acc = oracle.conv_acc(xq, wq)
    x2 = torch.from_numpy(xq[0, 0].astype(np.float64)).permute(2, 0, 1)[None]
    w2 = torch.from_numpy(wq[:, 2].astype(np.float64)).permute(0, 3, 1, 2)
    ref = F.conv2d(x2, w2, padding=1)[0].permute(1, 2, 0).numpy()
    assert np.array_equal(acc[0, 0].astype(np.float64), ref)


def test_zero_cache_equals_front_padding(oracle):
    g = torch.Generator().manual_seed(24)
    xq = _rand_int8(g, (1, 3, 6, 7, 32))
    wq = _rand_int8(g, (32, 3, 3, 3, 32))
    a = oracle.conv_acc(xq, wq)
    b = oracle.conv_acc(xq, wq, np.zeros((1, 2, 6, 7, 32), np.int8))
    assert np.array_equal(a, b)


def test_chunked_equals_unchunked(oracle):
    g = torch.Generator().manual_seed(25)
    T = 8
    xq = _rand_int8(g, (1, T, 5, 6, 32))
    wq = _rand_int8(g, (32, 3, 3, 3, 32))
    full = oracle.conv_acc(xq, wq)
    parts = []
    for c in range(4):
        cache = None if c == 0 else xq[:, 2 * c - 2:2 * c]
        parts.append(oracle.conv_acc(np.ascontiguousarray(xq[:, 2 * c:2 * c + 2]), wq, cache))
    assert np.array_equal(full, np.concatenate(parts, axis=1))


def test_causality(oracle):
    g = torch.Generator().manual_seed(26)
    xq = _rand_int8(g, (1, 6, 5, 5, 32))
    wq = _rand_int8(g, (32, 3, 3, 3, 32))
    base = oracle.conv_acc(xq, wq)
    t0 = 2
    xq2 = xq.copy()
    xq2[:, t0 + 1:] = _rand_int8(g, xq2[:, t0 + 1:].shape)
    pert = oracle.conv_acc(xq2, wq)
    assert np.array_equal(base[:, :t0 + 1], pert[:, :t0 + 1])
    assert not np.array_equal(base[:, t0 + 1:], pert[:, t0 + 1:])


def test_conv_odd_symmetry(oracle):
    g = torch.Generator().manual_seed(27)
    xq = _rand_int8(g, (1, 2, 4, 6, 32))
    wq = _rand_int8(g, (32, 3, 3, 3, 32))
    assert np.array_equal(oracle.conv_acc(-xq, wq), -oracle.conv_acc(xq, wq))


@pytest.mark.parametrize("with_cache", [False, True])
@pytest.mark.parametrize("k", [(3, 3, 3), (1, 1, 1)])
def test_conv_positions_equal_full_tensor(oracle, with_cache, k):
    """The position-list form (what the full-size GPU parity tests sample the
    oracle through) gives the rows of the float64 library conv at exactly the
    listed flattened ((n*T + t)*H + h)*W + w positions, in the order given,
    repeats included; a position outside the tensor is rejected."""
    if with_cache and k[0] == 1:
        pytest.skip("no cache frames when kt = 1")
    g = torch.Generator().manual_seed(29)
    N, T, H, W, Cin, Cout = 2, 3, 5, 7, 32, 64
    xq = _rand_int8(g, (N, T, H, W, Cin))
    wq = _rand_int8(g, (Cout,) + k + (Cin,))
    cache = _rand_int8(g, (N, k[0] - 1, H, W, Cin)) if with_cache else None
    total = N * T * H * W
    rng = np.random.default_rng(3)
    pos = np.concatenate([rng.permutation(total), [0, total - 1, 17, 17, W, H * W, T * H * W]]).astype(np.int64)
    ref = _torch_f64_conv(xq, wq, cache).reshape(-1, Cout)
    got = oracle.conv_acc(xq, wq, cache, positions=pos)
    assert got.shape == (pos.size, Cout)
    assert np.array_equal(got.astype(np.float64), ref[pos])
    assert np.array_equal(got, oracle.conv_acc(xq, wq, cache).reshape(-1, Cout)[pos])
    for bad in ([total], [-1]):
        with pytest.raises(ValueError):
            oracle.conv_acc(xq, wq, cache, positions=np.array(bad, np.int64))


@pytest.mark.parametrize("with_cache", [False, True])
def test_layer_positions_equal_full_tensor(oracle, with_cache):
    """The whole layer at a position list equals the full layer's rows at those
    positions, and both equal the step-by-step path (absmax, scale, quantize,
    float64 library conv, epilogue) at those rows."""
    g = torch.Generator().manual_seed(30)
    N, T, H, W, Cin, Cout = 1, 3, 6, 9, 32, 32
    x = _bf16_bits_of(torch.randn(N, T, H, W, Cin, generator=g) * 3.0)
    w = (torch.randn(Cout, Cin, 3, 3, 3, generator=g) * 0.05).numpy()
    b = (torch.randn(Cout, generator=g) * 0.1).numpy()
    wq, ws = oracle.quantize_weights(w)
    cache = _rand_int8(g, (N, 2, H, W, Cin)) if with_cache else None
    total = N * T * H * W
    pos = np.concatenate([np.random.default_rng(4).permutation(total)[:60], [0, total - 1, 5, 5]]).astype(np.int64)
    y_full, s_full = oracle.layer(x, wq, ws, b, cache=cache)
    y_pos, s_pos = oracle.layer(x, wq, ws, b, cache=cache, positions=pos)
    assert s_full == s_pos
    assert y_pos.shape == (pos.size, Cout)
    assert np.array_equal(y_pos, y_full.reshape(-1, Cout)[pos])
    a = np.abs(f32(x)).max()
    s = np.float32(np.float32(a) / np.float32(127.0))
    assert s_pos == s
    xq = oracle.act_quantize(x, s)
    acc = _torch_f64_conv(xq, wq, cache).reshape(-1, Cout)[pos].astype(np.int32)
    assert np.array_equal(y_pos, oracle.epilogue(acc, s, ws, b))


# --------------------------------------------------------------- epilogue
def test_epilogue_closed_form(oracle):
    acc = np.array([[3, -5, 0, 1000, 7]], np.int32)
    s_w = np.array([0.25, 0.5, 2.0, 2.0 ** -10, 1.0], np.float32)
    b = np.array([0.0, 1.0, -0.5, 0.0, 2.0 ** -9], np.float32)
    y = oracle.epilogue(acc, np.float32(0.5), s_w, b)
    # 3*0.125 = 0.375 ; -5*0.25+1 = -0.25 ; 0*1-0.5 = -0.5 ;
    # 1000*2^-11 = 0.48828125 = 0x3EFA0000 -> bf16 0x3EFA exact ;
    # 7*0.5 + 2^-9 = 3.501953125: bf16 step at 3.5 is 2^-6, remainder 2^-9 < half -> 3.5
    assert y[0].tolist() == [0x3EC0, 0xBE80, 0xBF00, 0x3EFA, 0x4060]
    assert oracle.epilogue(acc, np.float32(0.5), s_w, None)[0, 1] == 0xBFA0   # -5*0.25 = -1.25


def test_epilogue_single_fma_rounding(oracle):
    # acc*m + b done as one fused operation: with m = 1+2^-23 and acc = 2^23+1,
    # the exact product 2^23 + 2 + 2^-23 plus b = -2^23 gives 2 + 2^-23 -> 2.0
    # after one rounding; a separate multiply would round the product to
    # 2^23+2 first (same result here), so also check a case where they differ:
    # acc = 3, m = 1/3 rounded, b = -1: fma keeps the tiny residual.
    m = np.float32(1.0) / np.float32(3.0)
    y32 = oracle.epilogue_f32(np.array([[3]], np.int32), np.float32(1.0),
                              np.array([m], np.float32), np.array([-1.0], np.float32))
    exact = 3 * np.float64(m) - 1.0
    assert y32[0, 0] == np.float32(exact) and y32[0, 0] != 0.0


def test_zero_activation_gives_bias(oracle):
    x = np.zeros((1, 2, 3, 4, 32), np.uint16)
    g = torch.Generator().manual_seed(28)
    w = (torch.randn(32, 32, 3, 3, 3, generator=g) * 0.02).numpy()
    b = (torch.randn(32, generator=g) * 0.01).numpy()
    wq, s_w = oracle.quantize_weights(w)
    y, s_x = oracle.layer(x, wq, s_w, b)
    assert s_x == 0
    bb = np.array([oracle.f32_to_bf16(v) for v in b], np.uint16)
    assert np.array_equal(y, np.broadcast_to(bb, y.shape))


# --------------------------------------------------------------- end-to-end pins
def _delta_weights(C, i, j, l, value=1.0):
    w = np.zeros((C, C, 3, 3, 3), np.float32)
    for c in range(C):
        w[c, c, i, j, l] = value
    return w


def _ulp_dist(a_bits, b_bits):
    """ordinal distance between bf16 bit patterns (monotone in value)."""
    def ordv(h):
        h = h.astype(np.int64)
        return np.where(h & 0x8000, -(h & 0x7FFF), h)
    return np.abs(ordv(a_bits) - ordv(b_bits))


def test_delta_kernel_identity(oracle):
    C = 32
    ci = wl.draw_custom(31, 1, C, C, 3, 6, 7)
    b = ci.b
    wq, s_w = oracle.quantize_weights(_delta_weights(C, 2, 1, 1))
    assert np.all(s_w == np.float32(1.0) / np.float32(127.0))
    assert np.count_nonzero(wq) == C and np.all(wq[:, 2, 1, 1, :].diagonal() == 127)
    y, s_x = oracle.layer(ci.x, wq, s_w, b)
    a, s, xq = oracle.act_absmax_quant(ci.x)
    # y = dequant(x) + b within one bf16 ulp
    expect = np.array([oracle.f32_to_bf16(v) for v in
                       (xq.astype(np.float64) * float(s) + b.astype(np.float64)).ravel()],
                      np.uint16).reshape(y.shape)
    assert np.all(_ulp_dist(y, expect) <= 1)


@pytest.mark.parametrize("j,l,dh,dw", [(0, 0, -1, -1), (0, 2, -1, 1), (2, 1, 1, 0), (1, 0, 0, -1)])
def test_delta_kernel_spatial_shift(oracle, j, l, dh, dw):
    # tap (j, l) reads input (h + j - 1, w + l - 1): a shifted delta moves the image
    C = 32
    g = torch.Generator().manual_seed(32)
    xq = _rand_int8(g, (1, 2, 5, 6, C))
    wq = np.zeros((C, 3, 3, 3, C), np.int8)
    for c in range(C):
        wq[c, 2, j, l, c] = 1
    acc = oracle.conv_acc(xq, wq)
    H, W = 5, 6
    for h in range(H):
        for w in range(W):
            hs, ws = h + dh, w + dw
            exp = xq[0, :, hs, ws] if (0 <= hs < H and 0 <= ws < W) else 0
            assert np.array_equal(acc[0, :, h, w], np.broadcast_to(exp, (2, C)))


@pytest.mark.parametrize("with_cache", [False, True])
def test_delta_kernel_temporal(oracle, with_cache):
    # temporal tap 0 reads frame t-2: zero (or the oldest cache frame) for t < 2
    C = 32
    g = torch.Generator().manual_seed(33)
    xq = _rand_int8(g, (1, 4, 3, 4, C))
    cache = _rand_int8(g, (1, 2, 3, 4, C)) if with_cache else None
    wq = np.zeros((C, 3, 3, 3, C), np.int8)
    for c in range(C):
        wq[c, 0, 1, 1, c] = 1
    acc = oracle.conv_acc(xq, wq, cache)
    for t in range(4):
        if t >= 2:
            exp = xq[0, t - 2]
        elif with_cache:
            exp = cache[0, t]
        else:
            exp = np.zeros_like(xq[0, 0])
        assert np.array_equal(acc[0, t], exp.astype(np.int32))


@pytest.mark.parametrize("x_kind,x_scale", [("normal", 1.0), ("silu", 1.0), ("normal", 20.0)])
def test_quantized_conv_within_derived_bound(oracle, x_kind, x_scale):
    """bf16 W8A8 output vs the float64 convolution of the unquantized bf16 x and
    float32 w, within the bound derived from the quantization steps:
      x = s_x (q_x + dx), w = s_w (q_w + dw), |dx|,|dw| <= e = 1/2 + 2^-17
      => |sum x w - s_x s_w sum q_x q_w| <= s_x s_w sum_k (e(|q_x|+|q_w|) + e^2)
    plus the FP32 epilogue (2^-22 relative) and the bf16 rounding (2^-8 relative)."""
    N, T, H, W, C = 1, 3, 8, 9, 64
    ci = wl.draw_custom(41, N, C, C, T, H, W, x_kind=x_kind, x_scale=x_scale)
    wq, s_w = oracle.quantize_weights(ci.w)
    a, s_x, xq = oracle.act_absmax_quant(ci.x)
    acc = oracle.conv_acc(xq, wq)
    y = f32(oracle.epilogue(acc, s_x, s_w, ci.b)).astype(np.float64)

    xf = torch.from_numpy(f32(ci.x).astype(np.float64)).permute(0, 4, 1, 2, 3)
    pad = lambda t: F.pad(F.pad(t, (0, 0, 0, 0, 2, 0)), (1, 1, 1, 1, 0, 0))
    y_ref = F.conv3d(pad(xf), torch.from_numpy(ci.w.astype(np.float64)),
                     torch.from_numpy(ci.b.astype(np.float64)))
    y_ref = y_ref.permute(0, 2, 3, 4, 1).numpy()

    e = 0.5 + 2.0 ** -17
    qx_abs = torch.from_numpy(np.abs(xq.astype(np.float64))).permute(0, 4, 1, 2, 3)
    ones = torch.ones_like(qx_abs)
    wq_abs = torch.from_numpy(np.abs(wq.astype(np.float64))).permute(0, 4, 1, 2, 3)
    sum_qx = F.conv3d(pad(qx_abs), torch.ones_like(wq_abs)).permute(0, 2, 3, 4, 1).numpy()
    sum_qw = F.conv3d(pad(ones), wq_abs).permute(0, 2, 3, 4, 1).numpy()
    nvalid = F.conv3d(pad(ones), torch.ones_like(wq_abs)).permute(0, 2, 3, 4, 1).numpy()
    sxsw = float(s_x) * s_w.astype(np.float64)
    bound = (sxsw * (e * (sum_qx + sum_qw) + e * e * nvalid)
             + 2.0 ** -8 * np.abs(y)
             + 2.0 ** -22 * (np.abs(acc) * sxsw + np.abs(ci.b.astype(np.float64)))
             + 1e-12)
    ratio = np.abs(y - y_ref) / bound
    assert ratio.max() <= 1.0
    # and the typical error is far inside the worst case (random rounding errors)
    assert np.sqrt(np.mean((y - y_ref) ** 2)) < 0.2 * np.sqrt(np.mean(bound ** 2))


def test_layer_clip_below_one_bruteforce(oracle):
    """The whole layer at clip 0.5 against numpy quantization + the pure-Python
    convolution + the (separately pinned) epilogue."""
    g = torch.Generator().manual_seed(16)
    N, T, H, W, Cin, Cout = 1, 2, 3, 4, 32, 32
    xb = (torch.randn(N, T, H, W, Cin, generator=g) * 2).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    w = (torch.randn(Cout, Cin, 3, 3, 3, generator=g) * 0.05).numpy()
    b = (torch.randn(Cout, generator=g) * 0.1).numpy()
    wq, s_w = oracle.quantize_weights(w, 0.5)
    y, s_x = oracle.layer(xb, wq, s_w, b, clip_ratio=0.5)
    xf = f32(xb)
    a = np.abs(xf).max()
    s_ref = np.float32(np.float32(0.5) * a) / np.float32(127)
    assert s_x == s_ref
    xq = np.clip(np.rint(xf / s_ref), -127, 127).astype(np.int8)
    assert np.count_nonzero(np.abs(xq.astype(int)) == 127) > 10
    acc = np.array(conv_acc_bruteforce(xq.astype(int).tolist(), wq.astype(int).tolist()), np.int32)
    assert np.array_equal(y, oracle.epilogue(acc, s_x, s_w, b))


# --------------------------------------------------------------- native-precision conv (bf16)
def _bf16_bits_of(t):
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("with_cache", [False, True])
def test_bf16_conv_integer_values_bruteforce(oracle, with_cache):
    # small integers are exact in bf16, so the exact conv is the integer conv
    g = torch.Generator().manual_seed(31)
    N, T, H, W, Cin, Cout = 1, 3, 4, 5, 3, 4
    xi = torch.randint(-9, 10, (N, T, H, W, Cin), generator=g)
    wi = torch.randint(-9, 10, (Cout, Cin, 3, 3, 3), generator=g)
    ci = torch.randint(-9, 10, (N, 2, H, W, Cin), generator=g) if with_cache else None
    z, mag = oracle.conv_bf16(_bf16_bits_of(xi.float()), _bf16_bits_of(wi.float()), None,
                              None if ci is None else _bf16_bits_of(ci.float()))
    w_cl = wi.permute(0, 2, 3, 4, 1).tolist()          # [Cout][kt][kh][kw][Cin] for the brute force
    ref = conv_acc_bruteforce(xi.tolist(), w_cl, None if ci is None else ci.tolist())
    assert np.array_equal(z, np.array(ref, np.float64))
    ref_abs = conv_acc_bruteforce(xi.abs().tolist(), wi.abs().permute(0, 2, 3, 4, 1).tolist(),
                                  None if ci is None else ci.abs().tolist())
    assert np.array_equal(mag, np.array(ref_abs, np.float64))


@pytest.mark.parametrize("k,with_cache", [((3, 3, 3), False), ((3, 3, 3), True), ((1, 1, 1), False),
                                          ((3, 1, 1), True), ((1, 3, 3), False)])
def test_bf16_conv_matches_f64_library_conv(oracle, k, with_cache):
    g = torch.Generator().manual_seed(32)
    N, T, H, W, Cin, Cout = 2, 3, 7, 9, 16, 32
    kt, kh, kw = k
    x = _bf16_bits_of(torch.randn(N, T, H, W, Cin, generator=g) * 2)
    w = _bf16_bits_of(torch.randn(Cout, Cin, kt, kh, kw, generator=g) * 0.1)
    b = (torch.randn(Cout, generator=g) * 0.1).numpy()
    cache = _bf16_bits_of(torch.randn(N, kt - 1, H, W, Cin, generator=g)) if with_cache else None
    z, mag = oracle.conv_bf16(x, w, b, cache)
    xt = torch.from_numpy(f32(x).astype(np.float64)).permute(0, 4, 1, 2, 3)
    if cache is not None:
        xt = torch.cat([torch.from_numpy(f32(cache).astype(np.float64)).permute(0, 4, 1, 2, 3), xt], dim=2)
    else:
        xt = F.pad(xt, (0, 0, 0, 0, kt - 1, 0))
    xt = F.pad(xt, ((kw - 1) // 2, (kw - 1) // 2, (kh - 1) // 2, (kh - 1) // 2, 0, 0))
    wt = torch.from_numpy(f32(w).astype(np.float64))
    ref = F.conv3d(xt, wt, torch.from_numpy(b.astype(np.float64))).permute(0, 2, 3, 4, 1).numpy()
    assert np.all(np.abs(z - ref) <= 1e-12 * mag + 1e-300)
    ref_mag = F.conv3d(xt.abs(), wt.abs(), torch.from_numpy(np.abs(b).astype(np.float64)))
    assert np.allclose(mag, ref_mag.permute(0, 2, 3, 4, 1).numpy(), rtol=1e-12, atol=0)


def test_bf16_conv_zero_cache_and_causality(oracle):
    g = torch.Generator().manual_seed(33)
    N, T, H, W, Cin, Cout = 1, 4, 5, 6, 16, 32
    x = _bf16_bits_of(torch.randn(N, T, H, W, Cin, generator=g))
    w = _bf16_bits_of(torch.randn(Cout, Cin, 3, 3, 3, generator=g) * 0.1)
    z0, _ = oracle.conv_bf16(x, w)
    zc, _ = oracle.conv_bf16(x, w, cache=np.zeros((N, 2, H, W, Cin), np.uint16))
    assert np.array_equal(z0, zc)
    x2 = x.copy()
    x2[:, 2:] = _bf16_bits_of(torch.randn(N, T - 2, H, W, Cin, generator=g))    # change frames 2, 3
    z2, _ = oracle.conv_bf16(x2, w)
    assert np.array_equal(z0[:, :2], z2[:, :2])                                 # frames 0, 1 unchanged
    assert not np.array_equal(z0[:, 2:], z2[:, 2:])
    # positions give the same values as the full tensor
    pos = np.array([0, 7, 29, N * T * H * W - 1])
    zp, _ = oracle.conv_bf16(x, w, positions=pos)
    assert np.array_equal(zp, z0.reshape(-1, Cout)[pos])


# --------------------------------------------------------------- RMSNorm + SiLU prologue
def _bf16_round_f64(v):
    """bf16 bits of float64 values rounded once, to nearest with ties to even,
    by rounding the float64 bit pattern at its 8th significant bit (normal
    bf16 range only; the test data stays inside it or is exactly zero)."""
    v = np.asarray(v, np.float64)
    u = v.view(np.uint64)
    mag = u & np.uint64(0x7FFFFFFFFFFFFFFF)
    kept = mag >> np.uint64(45)
    dropped = mag & np.uint64((1 << 45) - 1)
    half = np.uint64(1 << 44)
    up = (dropped > half) | ((dropped == half) & ((kept & np.uint64(1)) == 1))
    kept = kept + up.astype(np.uint64)
    r = ((kept << np.uint64(45)) | (u & np.uint64(1 << 63))).view(np.float64)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("val,expect", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                   # tie -> even
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),      # above the tie by less than a binary32 ulp: rounded
                                                 # once it goes up (via binary32 it would tie to even)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),               # tie -> even
    (-(1.0 + 2.0 ** -8 + 2.0 ** -40), 0xBF81),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (255.5, 0x4380),                             # tie, 0x437F odd -> 256
    (2.0 ** -126, 0x0080),                       # smallest normal
    (2.0 ** -134, 0x0000),                       # half the subnormal step: tie -> 0
    (3 * 2.0 ** -134, 0x0002),                   # 1.5 steps: tie -> 2 steps
    (2.0 ** -130, 0x0008),                       # subnormal, exact
    (3.0e38, 0x7F62),                            # large finite
])
def test_bf16_from_f64_closed_form(oracle, val, expect):
    assert oracle.bf16_from_f64(val) == expect


def test_bf16_from_f64_against_exact_rationals(oracle):
    # Python's round() on an exact Fraction is round-half-to-even: an independent
    # route to the correctly rounded bf16 value (8 significant bits)
    import math
    from fractions import Fraction
    rng = np.random.default_rng(5)
    vals = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000),
                           # binary64 values next to bf16 ties
                           (1 + (2 * rng.integers(0, 128, 500) + 1) * 2.0 ** -8) *
                           2.0 ** rng.integers(-60, 60, 500) * (1 + rng.integers(-3, 4, 500) * 2.0 ** -50)])
    for v in vals:
        v = float(v)
        _, e = math.frexp(v)
        q = Fraction(2) ** (e - 8)
        r = round(Fraction(v) / q) * q
        ref = int(np.float32(float(r)).view(np.uint32)) >> 16
        assert oracle.bf16_from_f64(v) == ref, v
    assert np.array_equal(np.array([oracle.bf16_from_f64(float(v)) for v in vals[:500]], np.uint16),
                          _bf16_round_f64(vals[:500]))


@pytest.mark.parametrize("C,eps,kind", [(96, 1e-6, "normal"), (384, 1e-6, "silu"), (192, 0.1, "normal"),
                                        (8, 1e-6, "large"), (16, 1e-3, "wide_gamma")])
def test_rmsnorm_silu_against_torch_float64(oracle, C, eps, kind):
    """h against torch's own RMSNorm and SiLU in float64 (F.rms_norm, F.silu),
    rounded to bf16 once: equal bit for bit."""
    g = torch.Generator().manual_seed(40 + C)
    x = torch.randn(500, C, generator=g)
    if kind == "silu":
        x = x * torch.sigmoid(x)
    elif kind == "large":
        x = x * 1000.0
    x[3] = 0.0                                              # an all-zero pixel: h = 0
    xb = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    gamma = (1.0 + 0.2 * torch.randn(C, generator=g)).numpy().astype(np.float32)
    if kind == "wide_gamma":                                # |n| up to a few hundred, both signs
        gamma = (gamma * 40.0 * np.where(np.arange(C) % 3 == 0, -1.0, 1.0)).astype(np.float32)
    h = oracle.rmsnorm_silu(xb, gamma, eps)
    x64 = torch.from_numpy(f32(xb).astype(np.float64))
    n = F.rms_norm(x64, (C,), weight=torch.from_numpy(gamma.astype(np.float64)), eps=float(np.float32(eps)))
    ref = F.silu(n).numpy()
    refb = _bf16_round_f64(ref)
    refb[ref == 0.0] = (np.signbit(ref[ref == 0.0]).astype(np.uint16) << 15)
    tiny = np.abs(ref) < 2.0 ** -120                        # outside the helper's normal range
    assert np.array_equal(h[~tiny], refb[~tiny])
    assert np.all(np.abs(f32(h[tiny])) < 2.0 ** -119)
    assert not (h[3] & 0x7FFF).any()                       # +-0 (the sign of x * gamma)
    # gamma is per channel: swapping two channels' gammas changes only those channels
    g2 = gamma.copy()
    g2[[0, 1]] = g2[[1, 0]]
    h2 = oracle.rmsnorm_silu(xb, g2, eps)
    assert np.array_equal(h2[:, 2:], h[:, 2:])


def test_rmsnorm_silu_closed_form(oracle):
    # a pixel of equal powers of two: mean(x^2) = a^2 exactly, so with eps = 2^-60
    # n = sign(a) * gamma * (1 - ~2^-61) and h = bf16(n / (1 + exp(-n)))
    import math
    from fractions import Fraction
    C = 64
    for a, gam in [(0.25, 2.0), (-4.0, 0.5), (1.0, 1.0), (2.0, 100.0), (-1.0, 100.0), (0.5, 0.0)]:
        xb = bits(np.full((1, C), a, np.float32))
        h = oracle.rmsnorm_silu(xb, np.full(C, gam, np.float32), 2.0 ** -60)
        n = math.copysign(gam, a)
        ref = n / (1 + math.exp(-n))
        if ref == 0.0:
            expect = 0x8000 if math.copysign(1.0, ref) < 0 else 0
        else:
            _, e = math.frexp(ref)
            q = Fraction(2) ** (e - 8)
            expect = int(np.float32(float(round(Fraction(ref) / q) * q)).view(np.uint32)) >> 16
        assert np.all(h == expect), (a, gam, h[0, 0], expect)
    # SiLU(n) = n for large n, and -0 for very negative n (exp(-n) overflows)
    h = oracle.rmsnorm_silu(bits(np.full((1, 4), 1.0, np.float32)), np.full(4, 200.0, np.float32), 2.0 ** -60)
    assert np.all(h == 0x4348)                               # 200
    h = oracle.rmsnorm_silu(bits(np.full((1, 4), -1.0, np.float32)), np.full(4, 1000.0, np.float32), 2.0 ** -60)
    assert np.all(h == 0x8000)


def test_layer_causality_end_to_end(oracle):
    """Whole layer (dynamic scale included): changing frames after t0 while keeping
    every |x| below the tensor maximum (held in frame 0) leaves the outputs of
    frames <= t0 unchanged, bit for bit."""
    g = torch.Generator().manual_seed(28)
    N, T, H, W, C = 1, 5, 6, 7, 32
    x = torch.randn(N, T, H, W, C, generator=g)
    x[0, 0, 0, 0, 0] = 8.0                                  # the maximum, in a past frame
    x2 = x.clone()
    t0 = 1
    x2[:, t0 + 1:] = (torch.rand(N, T - t0 - 1, H, W, C, generator=g) * 2 - 1) * 7.5
    xb = _bf16_bits_of(x)
    xb2 = _bf16_bits_of(x2)
    w = (torch.randn(C, C, 3, 3, 3, generator=g) * 0.05).numpy()
    b = (torch.randn(C, generator=g) * 0.1).numpy()
    wq, ws = oracle.quantize_weights(w)
    y, s = oracle.layer(xb, wq, ws, b)
    y2, s2 = oracle.layer(xb2, wq, ws, b)
    assert s == s2
    assert np.array_equal(y[:, :t0 + 1], y2[:, :t0 + 1])
    assert not np.array_equal(y[:, t0 + 1:], y2[:, t0 + 1:])
