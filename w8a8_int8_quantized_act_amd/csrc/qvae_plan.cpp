// qvae_plan.cpp -- which decoder layers a preset runs in W8A8 (host code only).
//
// Page "ComfyUI-Qwen-VAE-Triton v0.2.0", section "Three presets explained":
// the patch covers 28 Conv3d layers of the Qwen VAE decoder.  Conservative
// quantizes only the decoder's highest channel level (15 of the 28);
// Balanced the two highest levels (22), keeping the bottom 96-channel level
// native; Aggressive every eligible layer (26) except the two that the fixed
// exclusion rule keeps native, decoder.upsamples.14.residual.2 and .6.
//
// Readings (where the page names counts, not rules): the 28 are the two
// 3x3x3 convolutions of every residual block of the decoder (module names
// ending in ".residual.2" and ".residual.6"); the decoder's first and last
// convolutions, the 1x1x1 shortcut and the temporal up-sampling convs are not
// among them.  "Highest channel level" is Cin = Cout = the decoder's widest
// channel count; "two highest levels" is Cin and Cout at least half of it.
// With the Wan / Qwen-Image decoder (widest level 384) these rules give
// exactly the page's 15, 22 and 26.
#include <string.h>

#include "qvae.h"

namespace {

bool ends_with(const char *s, size_t n, const char *suffix)
{
    const size_t m = strlen(suffix);
    return n >= m && memcmp(s + n - m, suffix, m) == 0;
}

// suffix match on a whole dotted component: "x.decoder.a.b" matches
// "decoder.a.b", "xdecoder.a.b" does not
bool ends_with_name(const char *s, size_t n, const char *suffix)
{
    const size_t m = strlen(suffix);
    if (!ends_with(s, n, suffix)) return false;
    return n == m || s[n - m - 1] == '.';
}

bool in_decoder(const char *s)
{
    return strncmp(s, "decoder.", 8) == 0 || strstr(s, ".decoder.") != nullptr;
}

}  // namespace

extern "C" int qvae_select_layer(int preset, const char *name, int Cin, int Cout, int kt, int kh, int kw,
                                 int top_channels)
{
    if (!name || Cin <= 0 || Cout <= 0 || kt <= 0 || kh <= 0 || kw <= 0 || top_channels <= 0) return QVAE_EINVAL;
    if (preset < QVAE_PRESET_NATIVE || preset > QVAE_PRESET_AGGRESSIVE) return QVAE_EINVAL;
    if (preset == QVAE_PRESET_NATIVE) return 0;
    const size_t n = strlen(name);
    const bool residual_conv =
        in_decoder(name) && (ends_with(name, n, ".residual.2") || ends_with(name, n, ".residual.6"));
    // what the W8A8 convolution runs: 3x3x3, channel counts in 32s
    const bool supported = kt == 3 && kh == 3 && kw == 3 && Cin % 32 == 0 && Cout % 32 == 0;
    if (!residual_conv || !supported) return 0;
    if (ends_with_name(name, n, "decoder.upsamples.14.residual.2") ||
        ends_with_name(name, n, "decoder.upsamples.14.residual.6"))
        return 0;
    switch (preset) {
    case QVAE_PRESET_CONSERVATIVE: return Cin == top_channels && Cout == top_channels;
    case QVAE_PRESET_BALANCED: return 2 * Cin >= top_channels && 2 * Cout >= top_channels;
    default: return 1;
    }
}
