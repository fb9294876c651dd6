// qvae_norm.hip -- the norm + SiLU pass in front of a decoder residual conv,
// with the activation maximum of its output fused in (gfx950).
//
// Why it is here: the W8A8 activation quantizer needs the maximum of the
// conv's input before it can emit a single code (page "ComfyUI-Qwen-VAE-Triton
// v0.2.0", section "Three presets explained": dynamic symmetric INT8
// activations).  In the decoder that input is SiLU(RMSNorm(x)), produced by a
// pass that reads x and writes the bf16 result anyway; letting that pass also
// leave the partial maxima of its output removes the quantizer's own absmax
// pass (a read of the whole tensor).  The absorption of the preceding RMSNorm
// by the activation quantizer is the prologue fusion of ComfyUI's INT8
// linear kernels (page "Doubling LLM token rates in ComfyUI" (ComfyUI
// v0.45.0), section "Optimizing linear kernels"); that the VAE's residual
// convs sit behind norm and SiLU is a reading of the residual-block layer
// names the presets use.
//
// What it computes: h = bf16_rne(SiLU(x * gamma / sqrt(mean(x^2) + eps))), per
// pixel of C channels (channels-last), held to one bf16 ulp of that value
// taken exactly.  The binary32 sequence below is this kernel's own choice
// (the exp in particular), not part of the definition:
//   ss  = 0;  ss = fma(x_c, x_c, ss) for c = 0, 1, ..., C-1 (in this order)
//   r   = 1 / sqrt(ss / C + eps)
//   n_c = (x_c * r) * gamma_c
//   h_c = bf16_rne(n_c / (1 + E(-n_c)))
// with E(y) ~ exp(y) by Cody-Waite range reduction and a Taylor polynomial:
//   y' = min(max(y, -104), 89);  k = rint(y' * log2(e));
//   r' = fma(k, -ln2_hi, y');  r' = fma(k, -ln2_lo, r');
//   p = Horner(1, 1, 1/2!, ..., 1/6!) at r' (fma at each step);  E = ldexp(p, k)
// (|r'| <= ln2/2 + tiny; the truncation error r'^7/7! is below 2^-27 and E is
// within a few units in the last place of exp).
//
// The quotient.  n / d (d = 1 + E) must be the correctly rounded binary32
// quotient, but only its bf16 rounding is stored.  The pass computes
//   c = rcp(d) (hardware reciprocal, within 1 ulp),  q0 = n * c,
//   q = fma(-fma(d, q0, -n), c, q0)
// which is fl(n/d + eta) with |eta| a tiny fraction of an ulp of n/d (q0 is
// within a few ulps of n/d, and the correction multiplies that error by
// about the reciprocal's relative error), so q is the correctly rounded
// quotient or, when n/d lies within |eta| of a midpoint between two floats,
// its neighbour.  A neighbour changes the bf16 result only if q's low 16 bits
// are 0x7FFF, 0x8000 or 0x8001 (next to the bf16 round-to-even boundary).
// A group of 8 values with such a quotient, or with |n| > 64 (where d grows
// past the range the argument needs, up to infinity), is recomputed with the
// correctly rounded division, so h equals bf16_rne(fl(n / d)) exactly for
// this sequence's n and d; values with n < -64 take n e^n instead (the
// quotient's denominator overflows there while the value does not, see
// silu_neg_tail).  The binary32 steps are within a few parts in 2^24
// of the exact quantity, so h is the exact value rounded to bf16 or, when that
// value lies that close to a bf16 rounding boundary, its neighbour.
//
// Layout of one pass.  A workgroup is 4 independent waves; a wave takes
// chunks of P consecutive pixels (P*C*2 contiguous bytes), stages them in its
// own LDS slice (coalesced 16-byte loads, issued one chunk ahead into
// registers; pixel rows padded to 2C+16 bytes so the row-per-lane reads below
// are conflict-free), lets lane p sum pixel p's
// squares in channel order and leave its r, then processes the chunk's
// 16-byte groups in memory order: 8 values of one pixel per lane, one 16-byte
// store of bf16 results, a packed 16-bit running maximum of |h|.  Every
// workgroup writes one partial maximum (the quantize pass reduces them).
#include "qvae_internal.h"

namespace qvae {

typedef int v4i_n __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_n __attribute__((ext_vector_type(4)));
typedef float f2_n __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_n __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_n __attribute__((ext_vector_type(2)));

constexpr int kNormThreads = 256;
constexpr int kNormWaves = kNormThreads / 64;
constexpr int kNormMaxLoads = 16;   // 16-byte loads per lane per chunk: P * C / 8 <= 1024 (see norm_chunk_pixels)

// exp(y) = p * 2^k by the steps in the header (all binary32): the mantissa
// part p (in [0.7, 1.42]) and the exponent k
__device__ __forceinline__ float exp_cw_parts(float y, int &k)
{
    constexpr float kLog2e = 0x1.715476p+0f;
    constexpr float kLn2Hi = 0x1.62e4p-1f;         // 8 significant bits: k * kLn2Hi is exact
    constexpr float kLn2Lo = 0x1.7f7d1cp-20f;      // ln 2 - kLn2Hi
    y = fminf(fmaxf(y, -104.0f), 89.0f);
    const float kf = __builtin_rintf(y * kLog2e);
    float r = __builtin_fmaf(kf, -kLn2Hi, y);
    r = __builtin_fmaf(kf, -kLn2Lo, r);
    float p = 0x1.6c16c2p-10f;                     // 1/6!
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);      // 1/5!
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);      // 1/4!
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);      // 1/3!
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    k = (int)kf;
    return p;
}

__device__ __forceinline__ float exp_cw(float y)
{
    int k;
    const float p = exp_cw_parts(y, k);
    return __builtin_amdgcn_ldexpf(p, k);
}

// SiLU(n) for n < -64, where n / (1 + exp(-n)) would overflow the
// denominator below n = -88.7 and return -0 for values that are still
// (sub)normal floats down to n ~ -103: n e^n / (1 + e^n) equals n e^n to
// binary32 precision (e^n < 2^-92), formed as ldexp(n * p, k) with
// e^n = p 2^k, so the one rounding into the subnormal range comes last
// (denormals are kept, not flushed).
__device__ __forceinline__ float silu_neg_tail(float n)
{
    int k;
    const float p = exp_cw_parts(n, k);
    return __builtin_amdgcn_ldexpf(n * p, k);
}


// LDS written by some lanes of a wave and read by others of the same wave
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

template <int P, bool OUTMAX>
__global__ __launch_bounds__(kNormThreads) void k_rmsnorm_silu(const uint16_t *__restrict__ x, int64_t npix, int C,
                                                               const float *__restrict__ gamma, float eps,
                                                               uint16_t *__restrict__ h, uint32_t *__restrict__ partials)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pitch = 2 * C + 16;
    const int G = C >> 3;                                    // 16-byte groups per pixel
    const int gamma_bytes = (C * 4 + 15) & ~15;
    float *s_gamma = reinterpret_cast<float *>(smem);
    char *s_x = smem + gamma_bytes + wave * (P * pitch + P * 4);
    float *s_r = reinterpret_cast<float *>(s_x + P * pitch);
    for (int c = tid; c < C; c += kNormThreads) s_gamma[c] = gamma[c];
    __syncthreads();

    const int64_t nchunks = (npix + P - 1) / P;
    const int64_t cstride = (int64_t)gridDim.x * kNormWaves;
    const float fC = (float)C;
    const int nld = (P * G + 63) / 64;                       // 16-byte loads per lane per chunk
    const int dq = 64 / G, dg = 64 - (64 / G) * G;          // (pixel, group) step of 64 groups
    uint32_t ymax = 0;
    // The next chunk of this wave is loaded into registers while the current
    // one is processed (its loads are waited for only when it is staged).
    v4i_n pf[kNormMaxLoads];
    auto load_chunk = [&](int64_t c) {
        const int64_t q0 = c * P;
        const int nq = (int)(npix - q0 < P ? npix - q0 : P);
        const __amdgpu_buffer_rsrc_t rin = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(x) + q0 * C, 0, nq * C * 2, 0x00020000);   // pixels past the end read 0
#pragma unroll
        for (int k = 0; k < kNormMaxLoads; ++k)
            if (k < nld)
                pf[k] = __builtin_bit_cast(v4i_n, __builtin_amdgcn_raw_buffer_load_b128(rin, (lane + 64 * k) * 16, 0, 0));
    };
    int64_t ch = (int64_t)blockIdx.x * kNormWaves + wave;
    if (ch < nchunks) load_chunk(ch);
    for (; ch < nchunks; ch += cstride) {
        const int64_t p0 = ch * P;
        const int np = (int)(npix - p0 < P ? npix - p0 : P);
        const int bytes = np * C * 2;
        // stage the chunk (16-byte pieces in memory order), then start the next one's loads
#pragma unroll
        for (int k = 0; k < kNormMaxLoads; ++k) {
            const int u = lane + 64 * k;
            if (k < nld && u < P * G) {
                const int p = u / G, g = u - p * G;
                *reinterpret_cast<v4i_n *>(s_x + p * pitch + g * 16) = pf[k];
            }
        }
        wave_lds_sync();
        if (ch + cstride < nchunks) load_chunk(ch + cstride);
        // one lane per pixel: the sum of squares in channel order
        if (lane < P) {
            const char *row = s_x + lane * pitch;
            float ss = 0.0f;
            for (int g = 0; g < G; ++g) {
                const v4i_n v = *reinterpret_cast<const v4i_n *>(row + g * 16);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t w = (uint32_t)v[k >> 1];
                    const float xv = __uint_as_float((k & 1) ? (w & 0xFFFF0000u) : (w << 16));
                    ss = __builtin_fmaf(xv, xv, ss);
                }
            }
            const float d = __builtin_sqrtf(ss / fC + eps);
            s_r[lane] = 1.0f / d;
        }
        wave_lds_sync();
        const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc(h + p0 * C, 0, bytes, 0x00020000);
        // group u = lane + 64 i is (pixel p, 16-byte group g) = (u / G, u % G),
        // stepped without a division per group
        int p = lane / G, g = lane - (lane / G) * G;
        for (int u = lane; u < np * G; u += 64) {
            const v4i_n v = *reinterpret_cast<const v4i_n *>(s_x + p * pitch + g * 16);
            const float r = s_r[p];
            float nv[8], dv[8], qv[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t w = (uint32_t)v[k];
                const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xFFFF0000u);
                nv[2 * k] = (x0 * r) * s_gamma[g * 8 + 2 * k];
                nv[2 * k + 1] = (x1 * r) * s_gamma[g * 8 + 2 * k + 1];
            }
            float namax = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                dv[k] = 1.0f + exp_cw(-nv[k]);
                const float c = __builtin_amdgcn_rcpf(dv[k]);
                const float q0 = nv[k] * c;
                // the residual n - d q0 is formed as -(d q0 - n): for n = -0 it
                // is then -0 and q keeps n's sign (-0 + -0), as n / d does
                qv[k] = __builtin_fmaf(-__builtin_fmaf(dv[k], q0, -nv[k]), c, q0);
                namax = __builtin_fmaxf(namax, __builtin_fabsf(nv[k]));
            }
            // low 16 bits of each quotient minus 0x7FFF (mod 2^16), two per register
            u16x2_n near = u16x2_n{0xFFFF, 0xFFFF};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const u16x2_n lo = __builtin_bit_cast(
                    u16x2_n, __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, qv[2 * k + 1]),
                                                   __builtin_bit_cast(uint32_t, qv[2 * k]), 0x05040100u));
                near = __builtin_elementwise_min(near, lo + u16x2_n{0x8001, 0x8001});
            }
            if (!(namax <= 64.0f) || near.x <= 2 || near.y <= 2) {
#pragma unroll
                for (int k = 0; k < 8; ++k) qv[k] = (nv[k] < -64.0f) ? silu_neg_tail(nv[k]) : nv[k] / dv[k];
            }
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                o[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_n{qv[2 * k], qv[2 * k + 1]}, bf2_n));
                if constexpr (OUTMAX) ymax = pk_absmax(ymax, o[k]);
            }
            // non-temporal: measured 4-8 % faster for this pass than the default policy
            __builtin_amdgcn_raw_buffer_store_b128(u32x4_n{o[0], o[1], o[2], o[3]}, rout, u * 16, 0, 2);
            p += dq;
            g += dg;
            if (g >= G) {
                g -= G;
                ++p;
            }
        }
        wave_lds_sync();   // the next chunk overwrites this wave's slice
    }

    if constexpr (OUTMAX) {
        __shared__ uint32_t s_red[kNormWaves];
        const uint32_t m = wave_max_u32(max(ymax & 0xFFFFu, ymax >> 16));
        if (lane == 0) s_red[wave] = m;
        __syncthreads();
        if (tid == 0) {
            uint32_t b = s_red[0];
            for (int k = 1; k < kNormWaves; ++k) b = max(b, s_red[k]);
            partials[blockIdx.x] = b;
        }
        if (blockIdx.x == 0)
            for (int k = gridDim.x + tid; k < kAbsmaxParts; k += kNormThreads) partials[k] = 0;
    }
}

// pixels per wave chunk for a channel count: the workgroup's LDS (gamma + 4
// slices of P rows of 2C+16 bytes + P factors) stays within 64 KB
static int norm_chunk_pixels(int C)
{
    auto lds = [C](int P) { return ((C * 4 + 15) & ~15) + kNormWaves * (P * (2 * C + 16) + P * 4); };
    for (int P : {64, 32, 16})
        if (lds(P) <= 65536 && P * (C / 8) <= 64 * kNormMaxLoads) return P;
    return 0;
}

static int norm_launch(const uint16_t *x, int64_t npix, int C, const float *gamma, float eps, uint16_t *h,
                       uint32_t *partials, hipStream_t st)
{
    const int P = norm_chunk_pixels(C);
    if (P == 0) return QVAE_EUNSUPPORTED;
    const size_t lds = ((C * 4 + 15) & ~15) + kNormWaves * ((size_t)P * (2 * C + 16) + P * 4);
    const int64_t nchunks = (npix + P - 1) / P;
    int64_t want = (nchunks + kNormWaves - 1) / kNormWaves;
    const int64_t cap = partials ? kAbsmaxParts : (int64_t)device_cus() * 8;
    const int grid = (int)(want < 1 ? 1 : (want > cap ? cap : want));
#define QVAE_NORM_LAUNCH(PP)                                                                              \
    if (partials)                                                                                         \
        hipLaunchKernelGGL((k_rmsnorm_silu<PP, true>), dim3(grid), dim3(kNormThreads), lds, st, x, npix, C, \
                           gamma, eps, h, partials);                                                      \
    else                                                                                                  \
        hipLaunchKernelGGL((k_rmsnorm_silu<PP, false>), dim3(grid), dim3(kNormThreads), lds, st, x, npix, C, \
                           gamma, eps, h, partials);
    if (P == 64) {
        QVAE_NORM_LAUNCH(64)
    } else if (P == 32) {
        QVAE_NORM_LAUNCH(32)
    } else {
        QVAE_NORM_LAUNCH(16)
    }
#undef QVAE_NORM_LAUNCH
    return launch_status();
}

static int norm_validate(const uint16_t *x, int64_t npix, int C, const float *gamma, float eps, const uint16_t *h)
{
    if (!x || !gamma || !h || npix <= 0 || C <= 0) return QVAE_EINVAL;
    if (!(eps > 0.0f) || eps > 3.0e38f) return QVAE_EINVAL;   // zero, negative, NaN or infinite
    if (!aligned16(x) || !aligned16(h)) return QVAE_EINVAL;
    if (C % 8 != 0 || norm_chunk_pixels(C) == 0) return QVAE_EUNSUPPORTED;
    return QVAE_OK;
}


int preload_norm()
{
    hipFuncAttributes attr;
    return hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(&k_rmsnorm_silu<64, false>)) == hipSuccess ? QVAE_OK
                                                                                                   : QVAE_ELAUNCH;
}

}  // namespace qvae

using namespace qvae;

extern "C" int qvae_rmsnorm_silu(const uint16_t *x, int64_t npix, int C, const float *gamma, float eps,
                                 uint16_t *h, void *stream)
{
    if (force_fail(false)) return QVAE_EFORCED;
    const int rc = norm_validate(x, npix, C, gamma, eps, h);
    if (rc != QVAE_OK) return rc;
    return norm_launch(x, npix, C, gamma, eps, h, nullptr, as_stream(stream));
}

extern "C" int qvae_rmsnorm_silu_absmax(const uint16_t *x, int64_t npix, int C, const float *gamma, float eps,
                                        uint16_t *h, uint32_t *h_absmax, void *stream)
{
    if (force_fail(true)) return QVAE_EFORCED;
    if (!h_absmax) return QVAE_EINVAL;
    const int rc = norm_validate(x, npix, C, gamma, eps, h);
    if (rc != QVAE_OK) return rc;
    return norm_launch(x, npix, C, gamma, eps, h, h_absmax + 1, as_stream(stream));
}
