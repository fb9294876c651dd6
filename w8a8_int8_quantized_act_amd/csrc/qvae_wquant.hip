// qvae_wquant.hip -- per-output-channel symmetric INT8 weight quantization.
//
// Scheme (page "ComfyUI-Qwen-VAE-Triton v0.2.0", section "Three presets
// explained"): symmetric INT8 weights, one scale per output channel, weight
// clip ratio 1.0.  s[co] = fl(clip * max |w[co,...]|) / 127 over every
// (ci, kt, kh, kw) of the channel; q = clamp(rne(w / s[co]), -127, 127).
// Any clip ratio in (0, 1] is accepted.
//
// Runs once per layer at load time.  One workgroup per output channel: a
// max-reduction over the channel (non-negative floats compare like their bit
// patterns, so the DPP integer max applies), then every lane quantizes and
// scatters into the layout the convolution consumes: MFMA fragments of 32
// output channels x 32 input channels, one contiguous kilobyte each, in the
// order the K loop walks them,
//   wq[co/32][i][ci/32][j*kw + l][lane][byte],  lane = 32*((ci%32)/16) + co%32,
//   byte = ci % 16,
// so a wave fetches one fragment with one fully coalesced 16-byte-per-lane load.
#include "qvae_internal.h"

namespace qvae {

constexpr int kWqThreads = 256;

__global__ __launch_bounds__(kWqThreads) void k_quantize_weights(const float *__restrict__ w, int Cin,
                                                                 int kt, int kh, int kw,
                                                                 float clip_ratio,
                                                                 int8_t *__restrict__ wq,
                                                                 float *__restrict__ w_scale)
{
    const int co = blockIdx.x;
    const int taps = kt * kh * kw;
    const int64_t per_co = (int64_t)Cin * taps;
    const float *wc = w + (int64_t)co * per_co;

    uint32_t m = 0;
    for (int64_t e = threadIdx.x; e < per_co; e += kWqThreads) m = max(m, __float_as_uint(fabsf(wc[e])));
    m = wave_max_u32(m);
    __shared__ uint32_t part[kWqThreads / 64];
    __shared__ float s_sh;
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b = part[0];
#pragma unroll
        for (int k = 1; k < kWqThreads / 64; ++k) b = max(b, part[k]);
        float s = (clip_ratio * __uint_as_float(b)) / 127.0f;
        s_sh = s;
        w_scale[co] = s;
    }
    __syncthreads();
    const float s = s_sh;
    const bool s_pos = s > 0.0f;

    // source order [ci][i][j][l]; destination: packed fragments (see above)
    const int khw = kh * kw;
    const int S = Cin >> 5;
    const int cb = co >> 5, row = co & 31;
    for (int64_t e = threadIdx.x; e < per_co; e += kWqThreads) {
        const int ci = (int)(e / taps);
        const int tap = (int)(e - (int64_t)ci * taps);
        const int i = tap / khw, sp = tap - i * khw;
        const int sl = ci >> 5, c = ci & 31;
        const int lane = (c >> 4) * 32 + row;
        int q = 0;
        if (s_pos) {
            float v = wc[e] / s;   // correctly rounded division
            v = fminf(fmaxf(__builtin_rintf(v), -127.0f), 127.0f);
            q = (int)v;
        }
        const int64_t dst = ((((int64_t)cb * kt + i) * S + sl) * khw + sp) * 1024 + lane * 16 + (c & 15);
        wq[dst] = (int8_t)q;
    }
}

// Native-precision weights for the layers left unquantized: bf16 values in
// the same fragment order, a fragment holding 32 output x 16 input channels
// (one kilobyte, 16 bytes per lane):
//   wp[co/32][i][ci/16][j*kw + l][lane][e],  lane = 32*((ci%16)/8) + co%32,
//   e = ci % 8.
// One thread per weight, a pure permutation (no arithmetic).
__global__ __launch_bounds__(kWqThreads) void k_pack_weights_bf16(const uint16_t *__restrict__ w, int Cin, int kt,
                                                                  int kh, int kw, int64_t total,
                                                                  uint16_t *__restrict__ wp)
{
    const int64_t e = (int64_t)blockIdx.x * kWqThreads + threadIdx.x;
    if (e >= total) return;
    const int taps = kt * kh * kw, khw = kh * kw;
    const int64_t per_co = (int64_t)Cin * taps;
    const int co = (int)(e / per_co);
    const int64_t r = e - (int64_t)co * per_co;
    const int ci = (int)(r / taps);
    const int tap = (int)(r - (int64_t)ci * taps);
    const int i = tap / khw, sp = tap - i * khw;
    const int S = Cin >> 4;
    const int cb = co >> 5, row = co & 31;
    const int sl = ci >> 4, c = ci & 15;
    const int lane = (c >> 3) * 32 + row;
    const int64_t dst = ((((int64_t)cb * kt + i) * S + sl) * khw + sp) * 512 + lane * 8 + (c & 7);
    wp[dst] = w[e];
}

int preload_wquant()
{
    hipFuncAttributes attr;
    return hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(&k_quantize_weights)) == hipSuccess
               ? QVAE_OK
               : QVAE_ELAUNCH;
}

}  // namespace qvae

using namespace qvae;

extern "C" int qvae_pack_weights_bf16(const uint16_t *w, int Cout, int Cin, int kt, int kh, int kw, uint16_t *wp,
                                      void *stream)
{
    if (force_fail(false)) return QVAE_EFORCED;
    if (!w || !wp || Cout <= 0 || Cin <= 0 || kt <= 0 || kh <= 0 || kw <= 0) return QVAE_EINVAL;
    if ((kt != 1 && kt != 3) || (kh != 1 && kh != 3) || (kw != 1 && kw != 3)) return QVAE_EUNSUPPORTED;
    if (Cout % 32 != 0 || Cin % 16 != 0) return QVAE_EUNSUPPORTED;
    if (!aligned16(wp)) return QVAE_EINVAL;
    const int64_t total = (int64_t)Cout * Cin * kt * kh * kw;
    if ((total + kWqThreads - 1) / kWqThreads > 0x7FFFFFFF) return QVAE_EUNSUPPORTED;
    hipLaunchKernelGGL(k_pack_weights_bf16, dim3((unsigned)((total + kWqThreads - 1) / kWqThreads)),
                       dim3(kWqThreads), 0, as_stream(stream), w, Cin, kt, kh, kw, total, wp);
    return launch_status();
}

extern "C" int qvae_quantize_weights(const float *w, int Cout, int Cin, int kt, int kh, int kw,
                                     float clip_ratio, int8_t *wq, float *w_scale, void *stream)
{
    if (force_fail(true)) return QVAE_EFORCED;
    if (!w || !wq || !w_scale || Cout <= 0 || Cin <= 0 || kt <= 0 || kh <= 0 || kw <= 0)
        return QVAE_EINVAL;
    if (!(clip_ratio > 0.0f)) return QVAE_EINVAL;         // zero, negative or NaN
    if (clip_ratio > 1.0f) return QVAE_EUNSUPPORTED;
    if ((kt != 1 && kt != 3) || (kh != 1 && kh != 3) || (kw != 1 && kw != 3)) return QVAE_EUNSUPPORTED;
    if (Cout % 32 != 0 || Cin % 32 != 0) return QVAE_EUNSUPPORTED;
    if (!aligned16(wq)) return QVAE_EINVAL;
    hipLaunchKernelGGL(k_quantize_weights, dim3(Cout), dim3(kWqThreads), 0, as_stream(stream), w, Cin,
                       kt, kh, kw, clip_ratio, wq, w_scale);
    return launch_status();
}

extern "C" int qvae_version(void) { return (0 << 16) | 3; }

extern "C" int qvae_init(void)
{
    (void)device_cus();
    const int r[] = {preload_act(), preload_wquant(), preload_conv(), preload_norm(), setup_scratch()};
    for (int v : r)
        if (v != QVAE_OK) return v;
    return QVAE_OK;
}

extern "C" const char *qvae_strerror(int status)
{
    switch (status) {
    case QVAE_OK: return "ok";
    case QVAE_EINVAL: return "invalid argument (null pointer, non-positive size or misaligned buffer)";
    case QVAE_EUNSUPPORTED: return "unsupported configuration";
    case QVAE_ELAUNCH: return "kernel launch failed";
    case QVAE_EFORCED: return "failure forced by QVAE_FORCE_FAIL";
    default: return "unknown status";
    }
}
