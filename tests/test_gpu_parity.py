"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: INT8 codes, scales (as bit patterns) and INT32 accumulators bit-exact;
bf16 outputs within 1 bf16 ulp of the oracle's bf16 (ordinal distance of the
bit patterns), which is the stated tolerance for the FP32-rescaled output.
Small shapes are compared element by element over the whole output; the full
workload sizes are compared on sampled output positions (corners, edges,
tile seams, ragged tails, random) plus properties that hold at any size
(chunked == unchunked, zero cache == front padding).
"""
import numpy as np
import pytest
import torch

import oracle
from tests.layout import pack_weight_codes
from w8a8_int8_quantized_act_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w8a8_int8_quantized_act_amd import ops as o
    o.lib()          # raises when the HIP library is missing
    return o


DEV = "cuda:0"


def to_dev_bits(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def ulp_dist(a, b):
    def ordv(h):
        h = h.astype(np.int64)
        return np.where(h & 0x8000, -(h & 0x7FFF), h)
    return np.abs(ordv(a) - ordv(b))


def f32_bits(v) -> int:
    return int(np.float32(v).view(np.uint32))


# ------------------------------------------------------------------ activation quantization
def _check_act(ops, x_bits, clip=1.0):
    xd = to_dev_bits(x_bits)
    absmax_bits, x_scale, xq = ops.act_absmax_quant(xd, clip)
    torch.cuda.synchronize()
    a, s, q = oracle.act_absmax_quant(x_bits, clip)
    assert int(absmax_bits[0].item()) == f32_bits(a) >> 16
    assert f32_bits(x_scale.item()) == f32_bits(s)
    got = xq.cpu().numpy()
    bad = np.count_nonzero(got != q)
    assert bad == 0, f"{bad} of {q.size} codes differ"
    return q


def _bits_of(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("n", [1, 7, 8, 15, 16, 17, 4097, 65536 * 3 + 5])
def test_act_quant_sizes(ops, n):
    g = torch.Generator().manual_seed(100 + n % 97)
    _check_act(ops, _bits_of(torch.randn(n, generator=g) * 3))


@pytest.mark.parametrize("n", [(16 << 20) - 3, (16 << 20) + 11])
def test_act_quant_both_store_policies(ops, n):
    # the quantize pass stores the codes of tensors from 16 Mi elements on with
    # the default cache policy and smaller ones non-temporally: both sides of
    # that size, bit-exact against the oracle
    g = torch.Generator().manual_seed(200 + n % 89)
    _check_act(ops, _bits_of(torch.randn(n, generator=g) * 3))


def test_act_quant_outliers_large(ops):
    g = torch.Generator().manual_seed(101)
    x = torch.randn(3_000_011, generator=g)
    m = torch.rand(x.shape, generator=g) < 0.05
    _check_act(ops, _bits_of(torch.where(m, x * 20, x)))


def test_act_quant_ties_scale_one(ops):
    # absmax 127 -> scale exactly 1: x.5 values are ties and go to the even code
    vals = [127.0] + [k + 0.5 for k in range(-127, 127)] + [-127.0, 0.0, -0.0, 0.25, -0.75]
    _check_act(ops, _bits_of(torch.tensor(vals * 37, dtype=torch.float32)))


def test_act_quant_near_ties(ops):
    # many values whose quotient lands within a few ulps of a half-integer
    g = torch.Generator().manual_seed(102)
    base = torch.randint(-126, 126, (200_000,), generator=g).float() + 0.5
    a = torch.tensor([93.0])      # scale 93/127: quotients are near, not at, the ties
    x = torch.cat([a, base * (93.0 / 127.0)])
    _check_act(ops, _bits_of(x))


def test_act_quant_split_entry_points(ops):
    # the two passes called one by one (same buffers) give the combined call's result
    g = torch.Generator().manual_seed(104)
    xb = _bits_of(torch.randn(1_000_003, generator=g) * 2)
    xd = to_dev_bits(xb)
    absmax = ops.act_absmax(xd)
    xs, xq = ops.act_quantize(xd, absmax)
    torch.cuda.synchronize()
    a, s, q = oracle.act_absmax_quant(xb)
    assert int(absmax[0].item()) == f32_bits(a) >> 16
    assert f32_bits(xs.item()) == f32_bits(s)
    assert np.array_equal(xq.cpu().numpy(), q)


def test_act_quant_zero_and_tiny(ops):
    _check_act(ops, np.zeros(1000, np.uint16))
    _check_act(ops, np.array([0x8000] * 33, np.uint16))           # -0.0 only
    g = torch.Generator().manual_seed(103)
    tiny = torch.randn(5000, generator=g) * 1e-39                 # bf16 subnormals: 1/s is not finite
    _check_act(ops, _bits_of(tiny))
    big = torch.randn(5000, generator=g) * 1e37
    _check_act(ops, _bits_of(big))


@pytest.mark.parametrize("clip", [0.5, 0.9, 0.25, 1e-3])
@pytest.mark.parametrize("n", [17, 4097, 1_000_003])
def test_act_quant_clip_below_one(ops, clip, n):
    # below clip 1 the scale shrinks and the clamp maps the tail to +-127
    g = torch.Generator().manual_seed(105 + n % 89)
    x = torch.randn(n, generator=g) * 3
    m = torch.rand(x.shape, generator=g) < 0.05
    q = _check_act(ops, _bits_of(torch.where(m, x * 20, x)), clip)
    if n > 1000:
        assert np.count_nonzero(np.abs(q.astype(np.int16)) == 127) > 1


# ------------------------------------------------------------------ weight quantization
@pytest.mark.parametrize("shape", [(384, 384, 3, 3, 3), (192, 384, 1, 1, 1), (96, 96, 3, 3, 3), (32, 64, 3, 1, 1)])
def test_weight_quant_bitexact(ops, shape):
    g = torch.Generator().manual_seed(200 + shape[0])
    w = torch.randn(shape, generator=g) * 0.02
    w[1] = 0.0                                   # an all-zero channel
    w[2].view(-1)[5] = 0.5                       # a channel with one large weight
    wq, ws = ops.quantize_weights(w.to(DEV))
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_weights(w.numpy())
    assert np.array_equal(ws.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(wq.cpu().numpy(), pack_weight_codes(rq))


@pytest.mark.parametrize("clip", [0.5, 0.9])
@pytest.mark.parametrize("shape", [(384, 384, 3, 3, 3), (96, 96, 3, 3, 3), (192, 384, 1, 1, 1)])
def test_weight_quant_clip_below_one(ops, shape, clip):
    g = torch.Generator().manual_seed(210 + shape[0])
    w = torch.randn(shape, generator=g) * 0.02
    w[1] = 0.0
    wq, ws = ops.quantize_weights(w.to(DEV), clip)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_weights(w.numpy(), clip)
    assert np.array_equal(ws.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(wq.cpu().numpy(), pack_weight_codes(rq))
    assert np.count_nonzero(np.abs(rq.astype(np.int16)) == 127) > shape[0]


# ------------------------------------------------------------------ the convolution, small shapes
SMALL = [
    # N, T, H, W, Cin, Cout, k, cache
    (1, 4, 32, 32, 96, 96, (3, 3, 3), False),
    (2, 3, 19, 37, 64, 192, (3, 3, 3), False),
    (1, 2, 17, 33, 64, 384, (3, 3, 3), True),
    (1, 1, 9, 40, 32, 96, (3, 3, 3), True),
    (2, 2, 11, 13, 96, 64, (3, 3, 3), False),
    (1, 3, 5, 7, 32, 32, (3, 3, 3), True),
    (1, 1, 1, 1, 32, 32, (3, 3, 3), False),
    (1, 2, 20, 31, 384, 192, (1, 1, 1), False),
    (1, 3, 8, 24, 64, 96, (3, 1, 1), True),
    (1, 1, 25, 18, 192, 192, (1, 3, 3), False),
]


def _small_inputs(case, seed):
    N, T, H, W, Cin, Cout, k, with_cache = case
    ci = wl.draw_custom(seed, N, Cin, Cout, T, H, W, k=k)
    wq, ws = oracle.quantize_weights(ci.w)
    a, s, xq = oracle.act_absmax_quant(ci.x)
    cache = None
    if with_cache and k[0] > 1:
        g = torch.Generator().manual_seed(seed + 1)
        cache = torch.randint(-127, 128, (N, k[0] - 1, H, W, Cin), generator=g,
                              dtype=torch.int64).numpy().astype(np.int8)
    return ci, wq, ws, s, xq, cache


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}x{c[1]}x{c[2]}x{c[3]}_c{c[4]}-{c[5]}_k{''.join(map(str, c[6]))}"
                                             f"{'_cache' if c[7] else ''}" for c in SMALL])
def test_conv_small_full(ops, case):
    ci, wq, ws, s, xq, cache = _small_inputs(case, 300 + sum(case[:6]))
    ref_acc = oracle.conv_acc(xq, wq, cache)
    ref_y = oracle.epilogue(ref_acc, s, ws, ci.b)

    xq_d = torch.from_numpy(xq).to(DEV)
    wq_d = torch.from_numpy(pack_weight_codes(wq)).to(DEV)
    cache_d = None if cache is None else torch.from_numpy(cache).to(DEV)
    acc = ops.causalconv3d_w8a8_acc32(xq_d, wq_d, cache_d)
    y = ops.causalconv3d_w8a8(xq_d, torch.tensor([s], device=DEV), wq_d, torch.from_numpy(ws).to(DEV),
                              torch.from_numpy(ci.b).to(DEV), cache_d)
    torch.cuda.synchronize()
    got_acc = acc.cpu().numpy()
    bad = np.argwhere(got_acc != ref_acc)
    assert bad.shape[0] == 0, f"{bad.shape[0]} accumulators differ, first at {bad[:4].tolist()}"
    d = ulp_dist(bf16_bits(y), ref_y)
    assert d.max() <= 1
    assert np.count_nonzero(d) == 0, f"{np.count_nonzero(d)} bf16 outputs differ by 1 ulp"


def test_conv_no_bias(ops):
    ci, wq, ws, s, xq, cache = _small_inputs((1, 2, 9, 21, 64, 96, (3, 3, 3), False), 350)
    ref_y = oracle.epilogue(oracle.conv_acc(xq, wq), s, ws, None)
    y = ops.causalconv3d_w8a8(torch.from_numpy(xq).to(DEV), torch.tensor([s], device=DEV),
                              torch.from_numpy(pack_weight_codes(wq)).to(DEV), torch.from_numpy(ws).to(DEV), None)
    torch.cuda.synchronize()
    assert ulp_dist(bf16_bits(y), ref_y).max() == 0


def test_layer_end_to_end_small(ops):
    # bf16 x -> (GPU absmax, quantize, weight quant, conv) vs the oracle's layer
    ci = wl.draw_custom(360, 1, 96, 96, 3, 23, 29, x_kind="silu")
    wq_d, ws_d = ops.quantize_weights(torch.from_numpy(ci.w).to(DEV))
    y, xs, xq = ops.layer_forward(to_dev_bits(ci.x), wq_d, ws_d, torch.from_numpy(ci.b).to(DEV))
    torch.cuda.synchronize()
    wq, ws = oracle.quantize_weights(ci.w)
    ref_y, ref_s = oracle.layer(ci.x, wq, ws, ci.b)
    assert f32_bits(xs.item()) == f32_bits(ref_s)
    assert ulp_dist(bf16_bits(y), ref_y).max() == 0


# ------------------------------------------------------------------ full workload sizes
def sample_positions(N, T, H, W, n_random, seed):
    """Flattened (n, t, h, w) positions: corners, image edges, tile seams of
    8/16/32-pixel tiles, the ragged last row/column, and random ones."""
    rng = np.random.default_rng(seed)
    hs = sorted(set([0, 1, H - 2, H - 1] + [v for m in (8, 16) for k in range(m, H, m * 5) for v in (k - 1, k)]))
    ws = sorted(set([0, 1, W - 2, W - 1] + [v for m in (16, 32) for k in range(m, W, m * 5) for v in (k - 1, k)]))
    hs = [h for h in hs if 0 <= h < H]
    ws = [w for w in ws if 0 <= w < W]
    pos = []
    for n in range(N):
        for t in sorted(set([0, T - 1, min(1, T - 1), min(2, T - 1)])):
            for h in hs:
                for w in (ws[:3] + ws[-3:]):
                    pos.append(((n * T + t) * H + h) * W + w)
            for w in ws:
                for h in (hs[:2] + hs[-2:]):
                    pos.append(((n * T + t) * H + h) * W + w)
    pos += list(rng.integers(0, N * T * H * W, n_random))
    return np.unique(np.array(pos, np.int64))


def _run_full_conv(ops, ci, cache_zero=False):
    spec = ci.spec
    kt = spec.k[0]
    x_d = to_dev_bits(ci.x)
    wq_d, ws_d = ops.quantize_weights(torch.from_numpy(ci.w).to(DEV))
    b_d = torch.from_numpy(ci.b).to(DEV)
    absmax, xs, xq_d = ops.act_absmax_quant(x_d)
    cache_d = None
    if cache_zero:
        cache_d = torch.zeros((spec.N, kt - 1, spec.H, spec.W, spec.Cin), dtype=torch.int8, device=DEV)
    y = ops.causalconv3d_w8a8(xq_d, xs, wq_d, ws_d, b_d, cache_d)
    acc = ops.causalconv3d_w8a8_acc32(xq_d, wq_d, cache_d)
    torch.cuda.synchronize()
    return dict(x_d=x_d, wq_d=wq_d, ws_d=ws_d, b_d=b_d, absmax=absmax, xs=xs, xq_d=xq_d, y=y, acc=acc,
                cache_d=cache_d)


def _compare_full(ops, ci, r, n_random=1500, seed=0, cache_zero=False):
    spec = ci.spec
    wq, ws = oracle.quantize_weights(ci.w)
    assert np.array_equal(r["wq_d"].cpu().numpy(), pack_weight_codes(wq))
    assert np.array_equal(r["ws_d"].cpu().numpy().view(np.uint32), ws.view(np.uint32))
    a, s, xq = oracle.act_absmax_quant(ci.x)
    assert int(r["absmax"][0].item()) == f32_bits(a) >> 16
    assert f32_bits(r["xs"].item()) == f32_bits(s)
    got_xq = r["xq_d"].cpu().numpy()
    assert np.array_equal(got_xq, xq), f"{np.count_nonzero(got_xq != xq)} codes differ"
    # nothing is clamped at clip ratio 1.0: the largest code is exactly 127 in magnitude
    assert np.abs(xq.astype(np.int16)).max() == 127
    pos = sample_positions(spec.N, spec.T, spec.H, spec.W, n_random, seed)
    cache = np.zeros((spec.N, spec.k[0] - 1, spec.H, spec.W, spec.Cin), np.int8) if cache_zero else None
    ref_acc = oracle.conv_acc(xq, wq, cache, positions=pos)
    ref_y = oracle.epilogue(ref_acc, s, ws, ci.b)
    got_acc = r["acc"].reshape(-1, spec.Cout)[torch.from_numpy(pos).to(DEV)].cpu().numpy()
    got_y = bf16_bits(r["y"].reshape(-1, spec.Cout)[torch.from_numpy(pos).to(DEV)])
    assert np.array_equal(got_acc, ref_acc), f"{np.count_nonzero(got_acc != ref_acc)} accumulators differ"
    d = ulp_dist(got_y, ref_y)
    assert d.max() <= 1 and np.count_nonzero(d) == 0
    # the bf16 output and the INT32 export agree everywhere (same contraction, same epilogue)
    return pos


@pytest.mark.parametrize("shape,cache_kind", [
    ((2, 384, 3, 60, 120), None),      # 384 ragged 8x16 tiles: workgroups run several, frames with 1..3 taps
    ((2, 384, 3, 60, 120), "random"),  # the same with a nonzero prev-frame cache (all taps valid)
    ((1, 192, 2, 250, 136), None),     # 288 ragged 16x16 tiles of 192 channels
    ((1, 384, 1, 105, 157), "random"), # 6x16 tiles (180 of them in one round), ragged bottom row
])
def test_conv_several_tiles_per_workgroup(ops, shape, cache_kind):
    """Shapes with more pixel tiles than CUs, so a workgroup runs tiles in a
    row and prefetches the next tile's first halo and weights; checked against
    the oracle on sampled positions (tile seams, ragged edges, every frame)."""
    N, C, T, H, W = shape
    ci = wl.draw_custom(70 + C + (1 if cache_kind else 0), N, C, C, T, H, W)
    spec = ci.spec
    wq, ws = oracle.quantize_weights(ci.w)
    a, s, xq = oracle.act_absmax_quant(ci.x)
    cache = None
    if cache_kind == "random":
        g = np.random.default_rng(5)
        cache = g.integers(-127, 128, (N, 2, H, W, C)).astype(np.int8)
    wq_d, ws_d = ops.quantize_weights(torch.from_numpy(ci.w).to(DEV))
    _, xs_d, xq_d = ops.act_absmax_quant(to_dev_bits(ci.x))
    b_d = torch.from_numpy(ci.b).to(DEV)
    cache_d = None if cache is None else torch.from_numpy(cache).to(DEV)
    y = ops.causalconv3d_w8a8(xq_d, xs_d, wq_d, ws_d, b_d, cache_d)
    acc = ops.causalconv3d_w8a8_acc32(xq_d, wq_d, cache_d)
    torch.cuda.synchronize()
    assert np.array_equal(xq_d.cpu().numpy(), xq)
    pos = sample_positions(N, T, H, W, 300, 7)
    ref_acc = oracle.conv_acc(xq, wq, cache, positions=pos)
    ref_y = oracle.epilogue(ref_acc, s, ws, ci.b)
    pos_d = torch.from_numpy(pos).to(DEV)
    got_acc = acc.reshape(-1, C)[pos_d].cpu().numpy()
    got_y = bf16_bits(y.reshape(-1, C)[pos_d])
    assert np.array_equal(got_acc, ref_acc), f"{np.count_nonzero(got_acc != ref_acc)} accumulators differ"
    assert ulp_dist(got_y, ref_y).max() == 0


@pytest.mark.parametrize("shape,k,cache_kind", [
    ((2, 64, 3, 11, 20), (3, 3, 3), "random"),   # ragged 8x16 / 16x16 tiles, cache
    ((1, 96, 2, 33, 47), (3, 3, 3), None),       # 96-channel tiles (two workgroups per CU)
    ((1, 384, 1, 40, 56), (3, 3, 3), "zero"),    # split K (few pixel tiles)
    ((2, 384, 3, 60, 120), (3, 3, 3), None),     # several tiles per workgroup
    ((1, 192, 2, 19, 23), (1, 1, 1), None),      # 1x1x1
    ((1, 64, 1, 400, 264), (3, 3, 3), None),     # narrow tiles, three workgroups per CU: the grid is capped at 512
    ((1, 192, 2, 250, 136), (3, 3, 3), "random"),  # 192-channel 16x16 tiles (16x16 matrix tiles), ragged edges
    ((1, 384, 1, 105, 157), (3, 3, 3), None),      # 6x16 pixel tiles
])
def test_conv_output_absmax_feeds_the_next_quantize(ops, shape, k, cache_kind):
    """The conv that also reports the partial maxima of its output: y is the
    plain conv's bit for bit, word 0 after the next quantize pass is max |y|
    over the output (out-of-image lanes excluded), and that pass quantizes y
    exactly as the two-pass quantizer does."""
    N, C, T, H, W = shape
    ci = wl.draw_custom(90 + C + T, N, C, C, T, H, W, k=k)
    kt = k[0]
    wq_d, ws_d = ops.quantize_weights(torch.from_numpy(ci.w).to(DEV))
    _, xs_d, xq_d = ops.act_absmax_quant(to_dev_bits(ci.x))
    b_d = torch.from_numpy(ci.b).to(DEV)
    cache_d = None
    if cache_kind == "zero":
        cache_d = torch.zeros((N, kt - 1, H, W, C), dtype=torch.int8, device=DEV)
    elif cache_kind == "random":
        g = torch.Generator().manual_seed(3)
        cache_d = torch.randint(-127, 128, (N, kt - 1, H, W, C), generator=g, dtype=torch.int8).to(DEV)
    y_plain = ops.causalconv3d_w8a8(xq_d, xs_d, wq_d, ws_d, b_d, cache_d)
    stale = torch.full((ops.ABSMAX_WORDS,), 0x7F7F, dtype=torch.int32, device=DEV)   # stale maxima everywhere
    y, y_absmax = ops.causalconv3d_w8a8_absmax(xq_d, xs_d, wq_d, ws_d, b_d, cache_d, y_absmax=stale)
    ys, yq = ops.act_quantize(y, y_absmax)
    a2, ys2, yq2 = ops.act_absmax_quant(y)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_plain.view(torch.int16))
    yb = bf16_bits(y)
    true_max = int((yb & 0x7FFF).max())
    assert int(y_absmax[0].item()) == true_max
    assert int(a2[0].item()) == true_max
    assert f32_bits(ys.item()) == f32_bits(ys2.item())
    assert torch.equal(yq, yq2)
    # and against the oracle's quantizer of y
    a_o, s_o, q_o = oracle.act_absmax_quant(yb)
    assert f32_bits(a_o) >> 16 == true_max and f32_bits(ys.item()) == f32_bits(s_o)
    assert np.array_equal(yq.cpu().numpy(), q_o)


@pytest.mark.parametrize("shape,cache_kind", [
    ((1, 384, 2, 105, 157), None),          # latent level, odd sizes
    ((1, 384, 2, 210, 314), "random"),      # second level, with a prev-frame cache
    ((1, 192, 3, 420, 628), None),          # third level, three frames
    ((1, 96, 2, 840, 1256), "random"),      # full-resolution level, with a cache
], ids=["c384_105x157_t2", "c384_210x314_t2_cache", "c192_420x628_t3", "c96_840x1256_t2_cache"])
def test_levels_multi_frame_clip_below_one(ops, shape, cache_kind):
    """Every decoder level with several frames, activations quantized at clip 0.5
    and weights at clip 0.9 (both clamps active), through the layer entry and the
    conv that reports its output maximum, whose partial maxima then feed the next
    layer's quantizer at clip 0.5; checked against the oracle on sampled positions."""
    N, C, T, H, W = shape
    clip_x, clip_w = 0.5, 0.9
    ci = wl.draw_custom(400 + C + T, N, C, C, T, H, W, x_kind="silu")
    cache = None
    if cache_kind == "random":
        cache = np.random.default_rng(9).integers(-127, 128, (N, 2, H, W, C)).astype(np.int8)
    cache_d = None if cache is None else torch.from_numpy(cache).to(DEV)
    wq_d, ws_d = ops.quantize_weights(torch.from_numpy(ci.w).to(DEV), clip_w)
    b_d = torch.from_numpy(ci.b).to(DEV)
    x_d = to_dev_bits(ci.x)
    y, xs_d, xq_d = ops.layer_forward(x_d, wq_d, ws_d, b_d, cache_d, clip_ratio=clip_x)
    y2, y_absmax = ops.causalconv3d_w8a8_absmax(xq_d, xs_d, wq_d, ws_d, b_d, cache_d)
    ys_d, yq_d = ops.act_quantize(y2, y_absmax, clip_x)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    wq, ws = oracle.quantize_weights(ci.w, clip_w)
    assert np.array_equal(ws_d.cpu().numpy().view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(wq_d.cpu().numpy(), pack_weight_codes(wq))
    a, s, xq = oracle.act_absmax_quant(ci.x, clip_x)
    assert f32_bits(xs_d.item()) == f32_bits(s)
    got_xq = xq_d.cpu().numpy()
    assert np.array_equal(got_xq, xq), f"{np.count_nonzero(got_xq != xq)} codes differ"
    assert np.count_nonzero(np.abs(xq.astype(np.int16)) == 127) > 100        # the clamp fired
    pos = sample_positions(N, T, H, W, 800, 11)
    pos_d = torch.from_numpy(pos).to(DEV)
    ref_y = oracle.epilogue(oracle.conv_acc(xq, wq, cache, positions=pos), s, ws, ci.b)
    assert ulp_dist(bf16_bits(y.reshape(-1, C)[pos_d]), ref_y).max() == 0
    # the next layer's quantizer on this output, from the fused partial maxima
    yb = bf16_bits(y)
    a2, s2, q2 = oracle.act_absmax_quant(yb, clip_x)
    assert f32_bits(ys_d.item()) == f32_bits(s2)
    assert np.array_equal(yq_d.cpu().numpy(), q2)


def test_workload_single_96_t4_32_full(ops):
    ci = wl.draw_workload("single_96_t4_32")[0]
    r = _run_full_conv(ops, ci)
    wq, ws = oracle.quantize_weights(ci.w)
    y_ref, s = oracle.layer(ci.x, wq, ws, ci.b)
    assert f32_bits(r["xs"].item()) == f32_bits(s)
    assert ulp_dist(bf16_bits(r["y"]), y_ref).max() == 0
    a, s, xq = oracle.act_absmax_quant(ci.x)
    assert np.array_equal(r["acc"].cpu().numpy(), oracle.conv_acc(xq, wq))


def test_workload_latent_384_128_cache(ops):
    ci = wl.draw_workload("latent_384_128_cache")[0]
    r = _run_full_conv(ops, ci, cache_zero=True)
    _compare_full(ops, ci, r, seed=1, cache_zero=True)
    # a zero cache equals causal front padding, bit for bit, at full size
    y2 = ops.causalconv3d_w8a8(r["xq_d"], r["xs"], r["wq_d"], r["ws_d"], r["b_d"], None)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), r["y"].view(torch.int16))


@pytest.mark.parametrize("level", [0, 1, 2, 3])
def test_workload_sweep_1024(ops, level):
    ci = wl.draw_workload("sweep_1024", only=level)[0]
    r = _run_full_conv(ops, ci)
    _compare_full(ops, ci, r, seed=20 + level)


@pytest.mark.parametrize("level", [0, 1, 2, 3])
def test_workload_sweep_840x1256(ops, level):
    ci = wl.draw_workload("sweep_840x1256", only=level)[0]
    r = _run_full_conv(ops, ci)
    _compare_full(ops, ci, r, seed=30 + level)


def test_workload_video_chunked(ops):
    ci = wl.draw_workload("video_384_t8_chunked")[0]
    spec = ci.spec
    x_d = to_dev_bits(ci.x)
    wq_d, ws_d = ops.quantize_weights(torch.from_numpy(ci.w).to(DEV))
    b_d = torch.from_numpy(ci.b).to(DEV)
    wp_d, wps_d = ops.quantize_weights(torch.from_numpy(ci.w_proj).to(DEV))
    bp_d = torch.from_numpy(ci.b_proj).to(DEV)
    _, xs, xq_d = ops.act_absmax_quant(x_d)        # one scale over all 8 frames
    full = ops.causalconv3d_w8a8(xq_d, xs, wq_d, ws_d, b_d)
    chunked = torch.empty_like(full)
    fpc = spec.T // spec.chunks
    for c in range(spec.chunks):
        cache = None if c == 0 else xq_d[:, fpc * c - 2:fpc * c]
        ops.causalconv3d_w8a8(xq_d[:, fpc * c:fpc * (c + 1)], xs, wq_d, ws_d, b_d, cache,
                              out=chunked[:, fpc * c:fpc * (c + 1)])
    proj = ops.causalconv3d_w8a8(xq_d, xs, wp_d, wps_d, bp_d)
    acc = ops.causalconv3d_w8a8_acc32(xq_d, wq_d)
    torch.cuda.synchronize()
    # chunked decode equals the single pass, bit for bit
    assert torch.equal(full.view(torch.int16), chunked.view(torch.int16))
    # both against the oracle on sampled positions
    wq, ws = oracle.quantize_weights(ci.w)
    wp, wps = oracle.quantize_weights(ci.w_proj)
    a, s, xq = oracle.act_absmax_quant(ci.x)
    assert np.array_equal(xq_d.cpu().numpy(), xq)
    pos = sample_positions(spec.N, spec.T, spec.H, spec.W, 1500, 4)
    pos_d = torch.from_numpy(pos).to(DEV)
    ref_acc = oracle.conv_acc(xq, wq, None, positions=pos)
    assert np.array_equal(acc.reshape(-1, spec.Cout)[pos_d].cpu().numpy(), ref_acc)
    ref_y = oracle.epilogue(ref_acc, s, ws, ci.b)
    assert ulp_dist(bf16_bits(chunked.reshape(-1, spec.Cout)[pos_d]), ref_y).max() == 0
    ref_p = oracle.epilogue(oracle.conv_acc(xq, wp, None, positions=pos), s, wps, ci.b_proj)
    assert ulp_dist(bf16_bits(proj.reshape(-1, spec.proj_cout)[pos_d]), ref_p).max() == 0


def test_layer_step_in_hip_graph(ops):
    # absmax -> quantize -> conv captured once and replayed several times, with
    # the program's own eager work in between; every replay equals the eager result
    ci = wl.draw_custom(370, 1, 192, 192, 2, 21, 35, x_kind="silu")
    x = to_dev_bits(ci.x)
    wq, ws = ops.quantize_weights(torch.from_numpy(ci.w).to(DEV))
    b = torch.from_numpy(ci.b).to(DEV)
    absmax = torch.empty((ops.ABSMAX_WORDS,), dtype=torch.int32, device=DEV)
    xs = torch.empty((1,), dtype=torch.float32, device=DEV)
    xq = torch.empty(x.shape, dtype=torch.int8, device=DEV)
    y = torch.empty((1, 2, 21, 35, 192), dtype=torch.bfloat16, device=DEV)
    y_eager, xs_eager, _ = ops.layer_forward(x, wq, ws, b)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):               # the two separate passes (cooperative launches are not captured)
        ops.act_absmax(x, absmax_bits=absmax)
        ops.act_quantize(x, absmax, x_scale=xs, xq=xq)
        ops.causalconv3d_w8a8(xq, xs, wq, ws, b, out=y)
    for rep in range(4):
        y.zero_()
        xs.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), f"replay {rep}"
        assert xs.item() == xs_eager.item()
        other = ops.causalconv3d_w8a8(xq, xs, wq, ws, None)      # eager work between replays
        torch.cuda.synchronize()
        del other


def test_layer_causality_end_to_end(ops):
    """The GPU layer (absmax, quantize, conv): future frames changed under the
    tensor maximum leave earlier frames' outputs bit-identical, with and without
    a cache."""
    g = torch.Generator().manual_seed(380)
    N, T, H, W, C = 1, 6, 33, 40, 192
    x = torch.randn(N, T, H, W, C, generator=g)
    x[0, 0, 3, 4, 5] = 9.0
    x2 = x.clone()
    t0 = 2
    x2[:, t0 + 1:] = (torch.rand(N, T - t0 - 1, H, W, C, generator=g) * 2 - 1) * 8.5
    w = torch.randn(C, C, 3, 3, 3, generator=g) * 0.03
    b = torch.randn(C, generator=g) * 0.01
    wq, ws = ops.quantize_weights(w.to(DEV))
    bd = b.to(DEV)
    cache = torch.randint(-127, 128, (N, 2, H, W, C), generator=g, dtype=torch.int8).to(DEV)
    for c in (None, cache):
        y1, s1, _ = ops.layer_forward(to_dev_bits(_bits_of(x)).view(N, T, H, W, C), wq, ws, bd, c)
        y2, s2, _ = ops.layer_forward(to_dev_bits(_bits_of(x2)).view(N, T, H, W, C), wq, ws, bd, c)
        torch.cuda.synchronize()
        assert f32_bits(s1.item()) == f32_bits(s2.item())
        assert torch.equal(y1[:, :t0 + 1].view(torch.int16), y2[:, :t0 + 1].view(torch.int16))
        assert not torch.equal(y1[:, t0 + 1:].view(torch.int16), y2[:, t0 + 1:].view(torch.int16))


def test_init_loads_the_code_and_changes_nothing(ops):
    """qvae_init (optional set-up) succeeds, may be repeated, and the calls
    after it give the same results as before."""
    ci, wq, ws, s, xq, cache = _small_inputs((1, 2, 9, 21, 64, 96, (3, 3, 3), True), 390)
    args = (torch.from_numpy(xq).to(DEV), torch.tensor([s], device=DEV),
            torch.from_numpy(pack_weight_codes(wq)).to(DEV), torch.from_numpy(ws).to(DEV),
            torch.from_numpy(ci.b).to(DEV), torch.from_numpy(cache).to(DEV))
    y0 = ops.causalconv3d_w8a8(*args)
    ops.init()
    ops.init()
    y1 = ops.causalconv3d_w8a8(*args)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


def test_binding_rejects_mismatched_buffers(ops):
    """Caller-supplied outputs and per-channel vectors are checked (device,
    dtype, shape or length) before the C call: the kernels size their stores
    from the dimensions, not from the tensors."""
    N, T, H, W, C = 1, 2, 8, 16, 64
    x = torch.zeros((N, T, H, W, C), dtype=torch.bfloat16, device=DEV)
    xq = torch.zeros((N, T, H, W, C), dtype=torch.int8, device=DEV)
    wq, ws = ops.quantize_weights(torch.ones((C, C, 3, 3, 3), device=DEV) * 0.01)
    am = torch.zeros((ops.ABSMAX_WORDS,), dtype=torch.int32, device=DEV)
    xs = torch.ones((1,), dtype=torch.float32, device=DEV)
    short_y = torch.empty((N, T, H, W - 1, C), dtype=torch.bfloat16, device=DEV)
    f32_y = torch.empty((N, T, H, W, C), dtype=torch.float32, device=DEV)
    bad_calls = [
        lambda: ops.causalconv3d_w8a8_qin(x, am, wq, ws, out=short_y),
        lambda: ops.causalconv3d_w8a8_qin(x, am, wq, ws, out=f32_y),
        lambda: ops.causalconv3d_w8a8_qin(x, am, wq, ws, x_scale=torch.ones(1)),            # host scale
        lambda: ops.causalconv3d_w8a8_qin(x, am, wq, ws[:C - 1]),
        lambda: ops.causalconv3d_w8a8_acc32(xq, wq, out=torch.empty((N, T, H, W, C), dtype=torch.int16,
                                                                    device=DEV)),
        lambda: ops.causalconv3d_w8a8_acc32(xq, wq, out=torch.empty((N, T, H, W, C - 32), dtype=torch.int32,
                                                                    device=DEV)),
        lambda: ops.causalconv3d_w8a8(xq, xs, wq, ws, torch.zeros(C - 1, device=DEV)),       # short bias
        lambda: ops.causalconv3d_w8a8(xq, xs, wq, ws[:C // 2]),                              # short w_scale
        lambda: ops.causalconv3d_w8a8(xq, torch.ones(1), wq, ws),                            # host x_scale
        lambda: ops.act_quantize(x, am, xq=torch.empty((N, T, H, W, C - 1), dtype=torch.int8, device=DEV)),
        lambda: ops.act_absmax_quant(x, xq=torch.empty((N, T, H, W, C), dtype=torch.uint8, device=DEV)),
    ]
    for i, call in enumerate(bad_calls):
        with pytest.raises(ValueError):
            call()
            pytest.fail(f"call {i} was accepted")
