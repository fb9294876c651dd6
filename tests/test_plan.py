"""Layer selection (host logic of the library), pinned to the numbers the page
prints: ComfyUI-Qwen-VAE-Triton v0.2.0, section "Three presets explained" --
28 patched Conv3d layers, 15 / 22 / 26 of them in W8A8 under Conservative /
Balanced / Aggressive, and decoder.upsamples.14.residual.2 and .6 always
native (tests/golden/presets.json)."""
import json
import os

import pytest

from w8a8_int8_quantized_act_amd import decoder, ops

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "presets.json")))


@pytest.fixture(scope="module")
def layers():
    if not os.path.exists(ops.LIB_PATH):
        from w8a8_int8_quantized_act_amd import build
        build.build()
    return decoder.residual_convs(1024, 1024)


def test_layer_table_has_the_pages_count(layers):
    assert len(layers) == GOLDEN["patched_layers"]
    assert len({L.name for L in layers}) == len(layers)
    for name in GOLDEN["native_under_aggressive"]:
        assert name in {L.name for L in layers}


@pytest.mark.parametrize("preset", ["conservative", "balanced", "aggressive"])
def test_preset_counts_match_the_page(layers, preset):
    plan = decoder.plan(preset, layers)
    assert sum(plan.values()) == GOLDEN["w8a8_layers"][preset]


def test_exclusions_and_levels(layers):
    agg = decoder.plan("aggressive", layers)
    assert sorted(n for n, q in agg.items() if not q) == sorted(GOLDEN["native_under_aggressive"])
    bal = decoder.plan("balanced", layers)
    keep = GOLDEN["balanced_keeps_native_channels"]
    assert all(not bal[L.name] for L in layers if L.Cin == keep and L.Cout == keep)
    assert all(bal[L.name] for L in layers if L.Cin > keep and L.Cout > keep)
    con = decoder.plan("conservative", layers)
    top = max(L.Cout for L in layers)
    assert all(con[L.name] == (L.Cin == top and L.Cout == top) for L in layers)
    # nested: every layer a milder preset quantizes, a stronger one does too
    for L in layers:
        assert con[L.name] <= bal[L.name] <= agg[L.name]
    assert not any(decoder.plan("native", layers).values())


def test_counts_do_not_depend_on_the_resolution():
    for h, w in [(512, 512), (928, 1664), (1328, 1328)]:
        L = decoder.residual_convs(h, w)
        assert [sum(decoder.plan(p, L).values()) for p in ("conservative", "balanced", "aggressive")] == [15, 22, 26]


def test_selection_rules_at_the_boundary(layers):
    sel = ops.select_layer
    assert sel("aggressive", "first_stage_model.decoder.upsamples.0.residual.2", 384, 384)   # any prefix
    assert not sel("aggressive", "first_stage_model.decoder.upsamples.14.residual.6", 96, 96)
    assert not sel("aggressive", "decoder.upsamples.0.shortcut", 192, 384, (1, 1, 1))
    assert not sel("aggressive", "decoder.upsamples.3.resample.1", 384, 768, (3, 1, 1))
    assert not sel("aggressive", "decoder.conv1", 16, 384)
    assert not sel("aggressive", "encoder.downsamples.0.residual.2", 96, 96)          # decoder only
    assert not sel("aggressive", "decoder.middle.0.residual.2", 384, 380)             # not in 32s
    assert not sel("aggressive", "decoder.xupsamples.14.residual.2x", 96, 96)
    assert sel("aggressive", "decoder.xupsamples.14.residual.2", 96, 96)              # only the named layers
    L = ops.lib()
    assert L.qvae_select_layer(4, b"decoder.middle.0.residual.2", 384, 384, 3, 3, 3, 384) == ops.EINVAL
    assert L.qvae_select_layer(3, None, 384, 384, 3, 3, 3, 384) == ops.EINVAL
    assert L.qvae_select_layer(3, b"decoder.middle.0.residual.2", 384, 384, 3, 3, 3, 0) == ops.EINVAL
