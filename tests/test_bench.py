"""bench.py contract on the CPU: the one-GPU message for --gpus N > 1, and the
algorithmic work it divides by (conv ops with structurally zero front-pad taps
excluded, bytes per launch), checked against hand-derived counts."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
    assert r.stdout.strip() == ""


def _spec(**kw):
    from w8a8_int8_quantized_act_amd.workloads import ConvSpec
    return ConvSpec("t", **kw)


@pytest.mark.parametrize("kw,cache,ops", [
    # 3x3x3, T=1 with a 2-frame cache: all 27 taps are data
    (dict(N=1, Cin=384, Cout=384, T=1, H=128, W=128), True, 2 * 384 * 384 * 27 * 128 * 128),
    # T=1 without a cache: only the last temporal tap touches data
    (dict(N=1, Cin=96, Cout=96, T=1, H=1024, W=1024), False, 2 * 96 * 96 * 9 * 1024 * 1024),
    # T=4 front padding: frames see 1, 2, 3, 3 temporal taps
    (dict(N=1, Cin=96, Cout=96, T=4, H=32, W=32), False, 2 * 96 * 96 * 9 * 32 * 32 * (1 + 2 + 3 + 3)),
    # 1x1x1: one tap per frame
    (dict(N=1, Cin=384, Cout=192, T=8, H=90, W=160, k=(1, 1, 1)), False, 2 * 384 * 192 * 90 * 160 * 8),
])
def test_layer_counts(kw, cache, ops):
    import bench
    c = bench.layer_counts(_spec(**kw), cache)
    assert c["ops"] == ops
    s = _spec(**kw)
    kt = s.k[0]
    hw = s.H * s.W
    expect_bytes = (s.N * s.T * hw * s.Cin + (s.N * (kt - 1) * hw * s.Cin if cache else 0)
                    + s.Cout * s.Cin * kt * s.k[1] * s.k[2] + 8 * s.Cout + 2 * s.Cout * s.N * s.T * hw)
    assert c["conv_bytes"] == expect_bytes
    assert c["absmax_bytes"] == 2 * s.numel and c["quant_bytes"] == 3 * s.numel


def test_workload_op_counts_in_gop():
    # the algorithmic GOP of every workload layer (rounded as the profiles print them)
    import bench
    from w8a8_int8_quantized_act_amd import workloads as wl
    expect = {"single_96_t4_32": [1.53], "latent_384_128_cache": [130.46],
              "sweep_1024": [43.49, 173.95, 173.95, 173.95], "sweep_840x1256": [43.75, 175.02, 175.02, 175.02],
              "video_384_t8_chunked": [802.63]}
    for key, gops in expect.items():
        got = [round(bench.layer_counts(s, s.zero_cache)["ops"] / 1e9, 2) for s in wl.WORKLOADS[key].convs]
        assert got == gops, key


def test_zero_share_of_k():
    import bench
    assert bench.zero_share_of_k(1, 3, True) == 2 / 3          # latent layer: two cache taps of three
    assert bench.zero_share_of_k(4, 3, True) == 3 / 12         # frames 0 and 1 read 2 and 1 cache taps
    assert bench.zero_share_of_k(8, 3, False) == 0.0           # no cache: padding taps are skipped
    assert bench.zero_share_of_k(1, 1, True) == 0.0            # a 1x1x1 conv has no temporal taps to pad


def test_chunked_step_launches():
    """The chunked decode step: 4 chunk convs of 2 frames (chunk 0 front-padded:
    its frames see 1 and 2 temporal taps; chunks 1-3 read the previous chunk's
    2 frames as cache: 3 taps each), then the 1x1x1 projection over all 8 frames."""
    import bench
    from w8a8_int8_quantized_act_amd import workloads as wl
    spec = wl.WORKLOADS["video_384_t8_chunked"].convs[0]
    ls = bench.chunk_launches(spec)
    assert [L["name"] for L in ls] == ["chunk0", "chunk1", "chunk2", "chunk3", "proj"]
    assert [L["frame0"] for L in ls] == [0, 2, 4, 6, 0]
    assert [L["cache_frame0"] for L in ls] == [None, 0, 2, 4, None]
    per_tap_frame = 2 * 384 * 384 * 9 * 90 * 160
    assert [L["ops"] for L in ls[:4]] == [3 * per_tap_frame] + [6 * per_tap_frame] * 3
    assert ls[4]["ops"] == 2 * 384 * 192 * 90 * 160 * 8
    assert [round(L["ops"] / 1e9, 2) for L in ls] == [114.66, 229.32, 229.32, 229.32, 16.99]
    px = 90 * 160
    w3 = 384 * 384 * 27
    assert ls[0]["conv_bytes"] == 2 * px * 384 + w3 + 8 * 384 + 2 * 384 * 2 * px
    assert ls[1]["conv_bytes"] == 4 * px * 384 + w3 + 8 * 384 + 2 * 384 * 2 * px
    assert ls[4]["conv_bytes"] == 8 * px * 384 + 384 * 192 + 8 * 192 + 2 * 192 * 8 * px
    # the whole step: the 3x3x3 conv over 8 frames plus the projection
    assert sum(L["ops"] for L in ls[:4]) == bench.layer_counts(spec, False)["ops"]
