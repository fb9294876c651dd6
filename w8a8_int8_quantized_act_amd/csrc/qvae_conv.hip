// qvae_conv.hip -- W8A8 causal 3-D convolution as an implicit GEMM on CDNA4
// INT8 matrix cores (gfx950).
//
// What it computes (page "ComfyUI-Qwen-VAE-Triton v0.2.0": intro paragraph,
// the implicit-GEMM kernel for the VAE decoder's CausalConv3d; section "Three
// presets explained", scheme paragraph: INT8 x INT8 products, INT32
// accumulation, FP32 rescale, output in the activation precision):
//
//   acc[n,t,h,w,co] = sum_{i,j,l,ci} wq[co,i,j,l,ci] * X(n, t-(kt-1)+i, h-ph+j, w-pw+l, ci)
//   y = bf16_rne(fma(float(acc), fl(s_x * s_w[co]), bias[co]))
//
// X reads the int8 input, the int8 cache of the kt-1 previous frames when a
// frame index is negative and a cache is given, and zero otherwise (causal
// front padding); out-of-image pixels are zero.  Symmetric quantization has no
// zero point, so padding is the integer 0.
//
// GEMM view: rows = output channels (A = weights, K-contiguous per channel),
// columns = output pixels (B = activations, channels-last so K = Cin is
// contiguous per pixel), K = valid temporal taps x kh x kw x Cin.  Nothing is
// materialised: a workgroup owns a TH x TW pixel tile of one frame and BCO
// output channels; the K loop runs over "stages" = (valid temporal tap i,
// 32-channel slice c).  Per stage the workgroup stages in LDS
//   - the activation halo (TH+kh-1) x (TW+kw-1) pixels x 32 channels of the
//     frame that tap i reads (zero outside the image), and
//   - the weights of all kh*kw spatial taps for tap i and slice c,
// then every wave runs kh*kw x MB x NB v_mfma_i32_32x32x32_i8 on shifted
// windows of the halo.  Frames that are structurally zero (front padding
// without a cache) are skipped, not multiplied.  Stages are double-buffered:
// the global loads of stage s+1 are in flight while stage s computes.
//
// MFMA 32x32x32 i8 operands: lane L supplies 16 bytes of row/column (L % 32)
// for K-half (L / 32); A and B use the same lane/byte -> k assignment, so the
// product covers all 32 k of the slice whatever order the hardware sums them
// in (integer sums are exact).  The INT32 result: lane L holds column L % 32
// and, in register r, row 8*(r/4) + 4*(L/32) + r%4 -- four consecutive output
// channels per register quad, so the epilogue writes 4 bf16 (8 bytes) per
// store along the channels-last output.
#include "qvae_internal.h"

namespace qvae {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

struct ConvArgs {
    const int8_t *xq;
    const int8_t *cache;
    const int8_t *wq;
    const float *x_scale;
    const float *w_scale;
    const float *bias;
    void *out;
    int N, T, H, W, Cin, Cout, kt;
    int tiles_w, tiles_h, co_tiles;
};

// Halo pixels are stored with a 48-byte pitch (32 data bytes + 16 unused):
// 3 is odd, so any 8 (or 16) consecutive pixels read by consecutive lanes hit
// distinct 16-byte bank groups.
constexpr int kHaloPitch = 48;

// Weight rows are 32 bytes; the two 16-byte halves of row r are swapped when
// bit 2 xor bit 3 of r is set, which spreads 8 (or 16) consecutive aligned
// rows over distinct bank groups.
__device__ __forceinline__ int wswz(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }

template <int WM, int WN, int MB, int NB, int TH, int TW, int KH, int KW>
struct Tile {
    static constexpr int NT = WM * WN * 64;
    static constexpr int BCO = WM * MB * 32;
    static constexpr int BPX = WN * NB * 32;
    static_assert(TH * TW == BPX, "pixel tile must match the wave layout");
    static_assert(32 % TW == 0 || TW % 32 == 0, "a 32-column MFMA block must tile rows evenly");
    static constexpr int HH = TH + KH - 1;
    static constexpr int HWD = TW + KW - 1;
    static constexpr int HALO_CHUNKS = HH * HWD * 2;        // 16-byte chunks per stage
    static constexpr int W_CHUNKS = KH * KW * BCO * 2;
    static constexpr int HALO_BYTES = HH * HWD * kHaloPitch;
    static constexpr int W_BYTES = KH * KW * BCO * 32;
    static constexpr int BUF_BYTES = HALO_BYTES + W_BYTES;
    static constexpr int HALO_PT = (HALO_CHUNKS + NT - 1) / NT;
    static constexpr int W_PT = (W_CHUNKS + NT - 1) / NT;
};

template <int WM, int WN, int MB, int NB, int TH, int TW, int KH, int KW, bool ACC32>
__global__ __launch_bounds__(WM *WN * 64) void k_conv_igemm(ConvArgs a)
{
    using TL = Tile<WM, WN, MB, NB, TH, TW, KH, KW>;
    constexpr int NT = TL::NT;
    constexpr int PH = (KH - 1) / 2, PW = (KW - 1) / 2;
    __shared__ __attribute__((aligned(16))) char smem[2 * TL::BUF_BYTES];

    const int tid = threadIdx.x;
    // ---- which tile: output-channel tile fastest, so with an even number of
    // channel tiles each XCD (workgroups are dealt round-robin over 8 XCDs)
    // keeps to the same weight slice in its L2.
    int b = blockIdx.x;
    const int cot = b % a.co_tiles;
    b /= a.co_tiles;
    const int twi = b % a.tiles_w;
    b /= a.tiles_w;
    const int thi = b % a.tiles_h;
    b /= a.tiles_h;
    const int t = b % a.T;
    const int n = b / a.T;
    const int h0 = thi * TH, w0 = twi * TW, co0 = cot * TL::BCO;
    const int H = a.H, W = a.W, Cin = a.Cin, kt = a.kt;

    // valid temporal taps: frame t-(kt-1)+i exists, or comes from the cache
    const int i_lo = a.cache ? 0 : max(0, kt - 1 - t);
    const int nslices = Cin >> 5;
    const int nst = (kt - i_lo) * nslices;

    // ---- per-thread load descriptors (stage independent parts)
    int h_off[TL::HALO_PT];    // byte offset inside a frame (+ half), -1 = zero / idle
    int h_lds[TL::HALO_PT];
#pragma unroll
    for (int k = 0; k < TL::HALO_PT; ++k) {
        const int u = tid + k * NT;
        h_off[k] = -1;
        h_lds[k] = -1;
        if (u < TL::HALO_CHUNKS) {
            const int q = u >> 1, half = u & 1;
            const int hh = q / TL::HWD, ww = q - hh * TL::HWD;
            const int gh = h0 - PH + hh, gw = w0 - PW + ww;
            h_lds[k] = q * kHaloPitch + half * 16;
            if (gh >= 0 && gh < H && gw >= 0 && gw < W) h_off[k] = (gh * W + gw) * Cin + half * 16;
        }
    }
    int w_off[TL::W_PT];       // byte offset into wq for temporal tap 0, slice 0
    int w_lds[TL::W_PT];
    const int wrow = kt * KH * KW * Cin;   // bytes per output channel
#pragma unroll
    for (int k = 0; k < TL::W_PT; ++k) {
        const int u = tid + k * NT;
        w_lds[k] = -1;
        w_off[k] = 0;
        if (u < TL::W_CHUNKS) {
            const int tap = u / (TL::BCO * 2);
            const int rem = u - tap * (TL::BCO * 2);
            const int co = rem >> 1, half = rem & 1;
            w_off[k] = (co0 + co) * wrow + tap * Cin + half * 16;
            w_lds[k] = (tap * TL::BCO + co) * 32 + ((half ^ wswz(co)) * 16);
        }
    }

    const size_t frame_bytes = (size_t)H * W * Cin;
    auto frame_ptr = [&](int i) -> const int8_t * {
        const int tau = t - (kt - 1) + i;
        if (tau >= 0) return a.xq + ((size_t)n * a.T + tau) * frame_bytes;
        return a.cache + ((size_t)n * (kt - 1) + (kt - 1 + tau)) * frame_bytes;
    };

    v4i hreg[TL::HALO_PT];
    v4i wreg[TL::W_PT];
    auto load_stage = [&](int s) {
        const int i = i_lo + s / nslices;
        const int c = s - (s / nslices) * nslices;
        const int8_t *fp = frame_ptr(i) + c * 32;
        const int8_t *wp = a.wq + i * KH * KW * Cin + c * 32;
#pragma unroll
        for (int k = 0; k < TL::HALO_PT; ++k) {
            hreg[k] = v4i{0, 0, 0, 0};
            if (h_off[k] >= 0) hreg[k] = *reinterpret_cast<const v4i *>(fp + h_off[k]);
        }
#pragma unroll
        for (int k = 0; k < TL::W_PT; ++k) {
            if (w_lds[k] >= 0) wreg[k] = *reinterpret_cast<const v4i *>(wp + w_off[k]);
        }
    };
    auto store_stage = [&](int buf) {
        char *xs = smem + buf * TL::BUF_BYTES;
        char *ws = xs + TL::HALO_BYTES;
#pragma unroll
        for (int k = 0; k < TL::HALO_PT; ++k)
            if (h_lds[k] >= 0) *reinterpret_cast<v4i *>(xs + h_lds[k]) = hreg[k];
#pragma unroll
        for (int k = 0; k < TL::W_PT; ++k)
            if (w_lds[k] >= 0) *reinterpret_cast<v4i *>(ws + w_lds[k]) = wreg[k];
    };

    // ---- per-lane fragment addresses
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int lrow = lane & 31, lhalf = lane >> 5;
    int a_off[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int co = wm * MB * 32 + mb * 32 + lrow;
        a_off[mb] = co * 32 + ((lhalf ^ wswz(co)) * 16);
    }
    int b_q0[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int p = (wn * NB + nb) * 32 + lrow;
        const int pr = p / TW, pc = p - pr * TW;
        b_q0[nb] = (pr * TL::HWD + pc) * kHaloPitch + lhalf * 16;
    }

    v16i acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = v16i{};

    if (nst > 0) {
        load_stage(0);
        store_stage(0);
    }
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        const int buf = s & 1;
        if (s + 1 < nst) load_stage(s + 1);
        const char *xs = smem + buf * TL::BUF_BYTES;
        const char *ws = xs + TL::HALO_BYTES;
#pragma unroll
        for (int j = 0; j < KH; ++j) {
#pragma unroll
            for (int l = 0; l < KW; ++l) {
                const int tap = j * KW + l;
                v4i av[MB], bv[NB];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    av[mb] = *reinterpret_cast<const v4i *>(ws + tap * TL::BCO * 32 + a_off[mb]);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    bv[nb] = *reinterpret_cast<const v4i *>(xs + b_q0[nb] + (j * TL::HWD + l) * kHaloPitch);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[mb], bv[nb], acc[mb][nb], 0, 0, 0);
            }
        }
        if (s + 1 < nst) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds pixel (column) lrow of each 32-pixel block and
    // output channels 8*g + 4*lhalf + {0..3} of each 32-channel block.
    const size_t pix_base = ((size_t)n * a.T + t) * H;
    float sx = 0.0f;
    if (!ACC32) sx = *a.x_scale;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int co = co0 + wm * MB * 32 + mb * 32 + g * 8 + lhalf * 4;
            float m[4], bb[4];
            if (!ACC32) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    m[e] = sx * a.w_scale[co + e];
                    bb[e] = a.bias ? a.bias[co + e] : 0.0f;
                }
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int p = (wn * NB + nb) * 32 + lrow;
                const int pr = p / TW, pc = p - pr * TW;
                const int gh = h0 + pr, gw = w0 + pc;
                if (gh < H && gw < W) {
                    const size_t o = ((pix_base + gh) * W + gw) * (size_t)a.Cout + co;
                    if (ACC32) {
                        v4i v = {acc[mb][nb][g * 4 + 0], acc[mb][nb][g * 4 + 1], acc[mb][nb][g * 4 + 2],
                                 acc[mb][nb][g * 4 + 3]};
                        *reinterpret_cast<v4i *>(static_cast<int32_t *>(a.out) + o) = v;
                    } else {
                        uint32_t h[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float y = __builtin_fmaf((float)acc[mb][nb][g * 4 + e], m[e], bb[e]);
                            h[e] = float_to_bf16_bits(y);
                        }
                        uint2 v = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
                        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + o) = v;
                    }
                }
            }
        }
    }
}

// ---- host side ------------------------------------------------------------

template <int WM, int WN, int MB, int NB, int TH, int TW, int KH, int KW>
static int launch_tile(const ConvArgs &base, bool acc32, hipStream_t st)
{
    using TL = Tile<WM, WN, MB, NB, TH, TW, KH, KW>;
    ConvArgs a = base;
    a.tiles_w = (a.W + TW - 1) / TW;
    a.tiles_h = (a.H + TH - 1) / TH;
    a.co_tiles = a.Cout / TL::BCO;
    const int64_t blocks = (int64_t)a.co_tiles * a.tiles_w * a.tiles_h * a.T * a.N;
    if (blocks <= 0 || blocks > 0x7FFFFFFF) return QVAE_EUNSUPPORTED;
    if (acc32)
        hipLaunchKernelGGL((k_conv_igemm<WM, WN, MB, NB, TH, TW, KH, KW, true>), dim3((unsigned)blocks),
                           dim3(TL::NT), 0, st, a);
    else
        hipLaunchKernelGGL((k_conv_igemm<WM, WN, MB, NB, TH, TW, KH, KW, false>), dim3((unsigned)blocks),
                           dim3(TL::NT), 0, st, a);
    return launch_status();
}

template <int KH, int KW>
static int launch_spatial(const ConvArgs &a, bool acc32, hipStream_t st)
{
    if (a.Cout % 192 == 0) return launch_tile<2, 2, 3, 2, 8, 16, KH, KW>(a, acc32, st);
    if (a.Cout % 96 == 0) return launch_tile<1, 4, 3, 2, 16, 16, KH, KW>(a, acc32, st);
    if (a.Cout % 64 == 0) return launch_tile<2, 2, 1, 2, 8, 16, KH, KW>(a, acc32, st);
    return launch_tile<1, 4, 1, 2, 16, 16, KH, KW>(a, acc32, st);
}

static int conv_validate(const int8_t *xq, const int8_t *wq, const void *out, int N, int T, int H, int W,
                         int Cin, int Cout, int kt, int kh, int kw, const int8_t *cache)
{
    if (!xq || !wq || !out) return QVAE_EINVAL;
    if (N <= 0 || T <= 0 || H <= 0 || W <= 0 || Cin <= 0 || Cout <= 0 || kt <= 0 || kh <= 0 || kw <= 0)
        return QVAE_EINVAL;
    if (!aligned16(xq) || !aligned16(out) || (cache && !aligned16(cache))) return QVAE_EINVAL;
    if (Cin % 32 != 0 || Cout % 32 != 0) return QVAE_EUNSUPPORTED;
    if (kt != 1 && kt != 3) return QVAE_EUNSUPPORTED;
    if (!((kh == 1 && kw == 1) || (kh == 3 && kw == 3))) return QVAE_EUNSUPPORTED;
    // |acc| <= 127^2 * K must stay inside int32
    const int64_t K = (int64_t)Cin * kt * kh * kw;
    if (K * 127 * 127 >= ((int64_t)1 << 31)) return QVAE_EUNSUPPORTED;
    // byte offsets inside one frame and one weight row are 32-bit
    if ((int64_t)H * W * Cin >= ((int64_t)1 << 31)) return QVAE_EUNSUPPORTED;
    if ((int64_t)Cout * K >= ((int64_t)1 << 31)) return QVAE_EUNSUPPORTED;
    return QVAE_OK;
}

static int conv_dispatch(const ConvArgs &a, int kh, bool acc32, hipStream_t st)
{
    if (kh == 3) return launch_spatial<3, 3>(a, acc32, st);
    return launch_spatial<1, 1>(a, acc32, st);
}

}  // namespace qvae

using namespace qvae;

extern "C" int qvae_causalconv3d_w8a8(const int8_t *xq, const float *x_scale, const int8_t *cache,
                                      const int8_t *wq, const float *w_scale, const float *bias, int N,
                                      int T, int H, int W, int Cin, int Cout, int kt, int kh, int kw,
                                      uint16_t *y, void *stream)
{
    if (force_fail()) return QVAE_EFORCED;
    if (!x_scale || !w_scale) return QVAE_EINVAL;
    int rc = conv_validate(xq, wq, y, N, T, H, W, Cin, Cout, kt, kh, kw, cache);
    if (rc != QVAE_OK) return rc;
    ConvArgs a{};
    a.xq = xq;
    a.cache = (kt > 1) ? cache : nullptr;
    a.wq = wq;
    a.x_scale = x_scale;
    a.w_scale = w_scale;
    a.bias = bias;
    a.out = y;
    a.N = N, a.T = T, a.H = H, a.W = W, a.Cin = Cin, a.Cout = Cout, a.kt = kt;
    return conv_dispatch(a, kh, false, as_stream(stream));
}

extern "C" int qvae_causalconv3d_w8a8_acc32(const int8_t *xq, const int8_t *cache, const int8_t *wq, int N,
                                            int T, int H, int W, int Cin, int Cout, int kt, int kh, int kw,
                                            int32_t *acc, void *stream)
{
    if (force_fail()) return QVAE_EFORCED;
    int rc = conv_validate(xq, wq, acc, N, T, H, W, Cin, Cout, kt, kh, kw, cache);
    if (rc != QVAE_OK) return rc;
    ConvArgs a{};
    a.xq = xq;
    a.cache = (kt > 1) ? cache : nullptr;
    a.wq = wq;
    a.out = acc;
    a.N = N, a.T = T, a.H = H, a.W = W, a.Cin = Cin, a.Cout = Cout, a.kt = kt;
    return conv_dispatch(a, kh, true, as_stream(stream));
}
