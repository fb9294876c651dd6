/*
 * qvae_oracle.c -- plain, slow CPU oracle for the W8A8 CausalConv3d path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * What it computes, and where that is defined (all on the page
 * "ComfyUI-Qwen-VAE-Triton v0.2.0: Triton W8A8 kernel accelerates the Qwen
 * Image VAE decoder", sd114.wiki):
 *   - intro paragraph: the kernel is an implicit-GEMM W8A8 kernel for the
 *     CausalConv3d layers of the Qwen-Image / Wan VAE decoder;
 *   - section "Three presets explained" (三个预设详解), scheme paragraph:
 *     symmetric INT8 weights with one scale per output channel, dynamic
 *     symmetric INT8 activations, INT8 x INT8 products accumulated in INT32,
 *     an FP32 rescale, and output kept in the activation's precision;
 *   - same section, fixed-parameter paragraph: activation clip ratio 1.0,
 *     weight clip ratio 1.0, channels_last layout;
 *   - same section, the presets: the layers a preset leaves out keep the
 *     VAE's native precision (here a bf16 convolution, computed exactly).
 * The page leaves open the activation-scale granularity, rounding, clamp range,
 * division form, epilogue order and the causal padding; the readings taken
 * here (per-tensor absmax/127, round-half-to-even, clamp to +-127, IEEE
 * float32 division x/s, y = fma(float(acc), s_x*s_w, bias), bf16
 * round-to-nearest-even, kt-1 zero front frames or an explicit int8 cache of
 * the previous kt-1 frames) are listed with their reasons in the design notes.
 *
 * Every floating-point step of the W8A8 path below is a single IEEE binary32
 * operation (compile with -ffp-contract=off, no fast-math); integer sums are
 * exact in int64.  The native-precision conv and the RMSNorm + SiLU prologue,
 * whose results are held to a tolerance rather than bit for bit, are computed
 * in binary64 and rounded once.  Nothing is blocked, fused or reordered beyond
 * the definitions.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EOVERFLOW 1  /* an accumulator left the int32 range */
#define ORACLE_EARG 2

/* ---- bf16 <-> binary32 ---------------------------------------------------
 * bf16 is the upper half of a binary32.  Widening is exact.  Narrowing is
 * round-to-nearest, ties-to-even, written out from that definition on the 16
 * discarded bits (finite inputs only). */
float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t kept = u >> 16;          /* truncated result                    */
    uint32_t dropped = u & 0xFFFFu;   /* the part that is rounded away       */
    if (dropped > 0x8000u) {
        kept += 1;                    /* more than half an ulp: round up     */
    } else if (dropped == 0x8000u) {
        if (kept & 1u) kept += 1;     /* exactly half: go to the even one    */
    }
    return (uint16_t)kept;
}

/* ---- round half to even, then clamp to the symmetric int8 range ---------- */
static int32_t round_half_even(float v)
{
    /* |v| <= 2^23 here, so floor and the difference below are exact. */
    float fl = floorf(v);
    float frac = v - fl;
    int32_t r = (int32_t)fl;
    if (frac > 0.5f) {
        r += 1;
    } else if (frac == 0.5f) {
        if (r % 2 != 0) r += 1;       /* tie: pick the even neighbour        */
    }
    return r;
}

static int8_t quantize_one(float v, float s)
{
    if (s == 0.0f) return 0;          /* all-zero tensor or channel          */
    float t = v / s;                  /* one correctly rounded division      */
    int32_t r;
    if (t >= 128.0f) {
        r = 127;                      /* beyond the range: clamp (and keep   */
    } else if (t <= -128.0f) {        /* the float -> int step in range)     */
        r = -127;
    } else {
        r = round_half_even(t);
        if (r > 127) r = 127;
        if (r < -127) r = -127;
    }
    return (int8_t)r;
}

/* Scale from an absolute maximum: s = fl(fl(clip * a) / 127). */
float oracle_scale_from_absmax(float absmax, float clip_ratio)
{
    float c = clip_ratio * absmax;
    return c / 127.0f;
}

/* ---- weights: one scale per output channel -------------------------------
 * w  : float32 [Cout][Cin][kt][kh][kw]   (the usual Conv3d weight layout)
 * wq : int8    [Cout][kt][kh][kw][Cin]   (channels-last along K)
 * s_w: float32 [Cout]
 * The maximum runs over every element of the output channel, temporal taps
 * included. */
int oracle_quantize_weights(const float *w, int Cout, int Cin, int kt, int kh,
                            int kw, float clip_ratio, int8_t *wq, float *s_w)
{
    if (!w || !wq || !s_w || Cout <= 0 || Cin <= 0 || kt <= 0 || kh <= 0 ||
        kw <= 0)
        return ORACLE_EARG;
    const int64_t per_co = (int64_t)Cin * kt * kh * kw;
    for (int co = 0; co < Cout; ++co) {
        const float *wc = w + (int64_t)co * per_co;
        float a = 0.0f;
        for (int64_t e = 0; e < per_co; ++e) {
            float m = fabsf(wc[e]);
            if (m > a) a = m;
        }
        float s = oracle_scale_from_absmax(a, clip_ratio);
        s_w[co] = s;
        for (int ci = 0; ci < Cin; ++ci)
            for (int i = 0; i < kt; ++i)
                for (int j = 0; j < kh; ++j)
                    for (int l = 0; l < kw; ++l) {
                        int64_t src = (((int64_t)ci * kt + i) * kh + j) * kw + l;
                        int64_t dst =
                            ((((int64_t)co * kt + i) * kh + j) * kw + l) * Cin + ci;
                        wq[dst] = quantize_one(wc[src], s);
                    }
    }
    return ORACLE_OK;
}

/* ---- activations: one dynamic scale for the whole tensor ----------------- */
float oracle_act_absmax(const uint16_t *x, int64_t n)
{
    float a = 0.0f;
    for (int64_t e = 0; e < n; ++e) {
        float m = fabsf(oracle_bf16_to_f32(x[e]));
        if (m > a) a = m;
    }
    return a;
}

void oracle_act_quantize(const uint16_t *x, int64_t n, float s, int8_t *q)
{
    for (int64_t e = 0; e < n; ++e) q[e] = quantize_one(oracle_bf16_to_f32(x[e]), s);
}

/* ---- the causal 3-D convolution over int8 codes ---------------------------
 * xq   : int8 [N][T][H][W][Cin]
 * cache: int8 [N][kt-1][H][W][Cin] (oldest frame first) or NULL
 * wq   : int8 [Cout][kt][kh][kw][Cin]
 * acc  : int32 [Cout] for the one output position (n, t, h, w)
 *
 * acc[co] = sum over (i, j, l, ci) of wq[co,i,j,l,ci] * X(n, t-(kt-1)+i,
 *           h-(kh-1)/2+j, w-(kw-1)/2+l, ci), where a frame index below zero
 * reads the cache slot kt-1+frame when a cache is given and is zero
 * otherwise, and a spatial index outside the image is zero.  Stride 1. */
static int conv_one_position(const int8_t *xq, const int8_t *cache,
                             const int8_t *wq, int N, int T, int H, int W,
                             int Cin, int Cout, int kt, int kh, int kw, int n,
                             int t, int h, int w, int32_t *acc)
{
    (void)N;
    const int ph = (kh - 1) / 2, pw = (kw - 1) / 2;
    for (int co = 0; co < Cout; ++co) {
        int64_t sum = 0;
        for (int i = 0; i < kt; ++i) {
            int tau = t - (kt - 1) + i;
            const int8_t *frame;
            if (tau >= 0) {
                frame = xq + ((int64_t)n * T + tau) * H * W * Cin;
            } else if (cache) {
                frame = cache + ((int64_t)n * (kt - 1) + (kt - 1 + tau)) * H * W * Cin;
            } else {
                continue;                 /* zero front padding              */
            }
            for (int j = 0; j < kh; ++j) {
                int hh = h - ph + j;
                if (hh < 0 || hh >= H) continue;
                for (int l = 0; l < kw; ++l) {
                    int ww = w - pw + l;
                    if (ww < 0 || ww >= W) continue;
                    const int8_t *xp = frame + ((int64_t)hh * W + ww) * Cin;
                    const int8_t *wp =
                        wq + ((((int64_t)co * kt + i) * kh + j) * kw + l) * Cin;
                    for (int ci = 0; ci < Cin; ++ci)
                        sum += (int64_t)wp[ci] * (int64_t)xp[ci];
                }
            }
        }
        if (sum > INT32_MAX || sum < INT32_MIN) return ORACLE_EOVERFLOW;
        acc[co] = (int32_t)sum;
    }
    return ORACLE_OK;
}

/* Accumulators for a list of output positions.  pos holds flattened indices
 * ((n*T + t)*H + h)*W + w; acc is [npos][Cout]. */
int oracle_conv_acc_positions(const int8_t *xq, const int8_t *cache,
                              const int8_t *wq, int N, int T, int H, int W,
                              int Cin, int Cout, int kt, int kh, int kw,
                              const int64_t *pos, int64_t npos, int32_t *acc)
{
    if (!xq || !wq || !acc || N <= 0 || T <= 0 || H <= 0 || W <= 0 ||
        Cin <= 0 || Cout <= 0 || kt <= 0 || kh <= 0 || kw <= 0 || npos < 0)
        return ORACLE_EARG;
    const int64_t total = (int64_t)N * T * H * W;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npos; ++p) {
        int64_t q = pos ? pos[p] : p;
        if (q < 0 || q >= total) {
#pragma omp atomic write
            status = ORACLE_EARG;
            continue;
        }
        int w = (int)(q % W);
        int h = (int)((q / W) % H);
        int t = (int)((q / ((int64_t)W * H)) % T);
        int n = (int)(q / ((int64_t)W * H * T));
        int rc = conv_one_position(xq, cache, wq, N, T, H, W, Cin, Cout, kt, kh,
                                   kw, n, t, h, w, acc + p * Cout);
        if (rc != ORACLE_OK) {
#pragma omp atomic write
            status = rc;
        }
    }
    return status;
}

/* Every output position, in order: acc is [N][T][H][W][Cout]. */
int oracle_conv_acc(const int8_t *xq, const int8_t *cache, const int8_t *wq,
                    int N, int T, int H, int W, int Cin, int Cout, int kt,
                    int kh, int kw, int32_t *acc)
{
    return oracle_conv_acc_positions(xq, cache, wq, N, T, H, W, Cin, Cout, kt,
                                     kh, kw, NULL, (int64_t)N * T * H * W, acc);
}

/* ---- FP32 rescale and bf16 output ---------------------------------------
 * m[co] = fl(s_x * s_w[co]);  y32 = fma(float(acc), m[co], bias[co]);
 * y = bf16 round-to-nearest-even of y32.  bias may be NULL (zero). */
void oracle_epilogue(const int32_t *acc, int64_t npos, int Cout, float s_x,
                     const float *s_w, const float *bias, uint16_t *y)
{
    for (int64_t p = 0; p < npos; ++p)
        for (int co = 0; co < Cout; ++co) {
            float m = s_x * s_w[co];
            float a = (float)acc[p * Cout + co];
            float b = bias ? bias[co] : 0.0f;
            float y32 = fmaf(a, m, b);
            y[p * Cout + co] = oracle_f32_to_bf16(y32);
        }
}

/* Same rescale, kept in float32 (the value the bf16 tolerance is measured
 * against). */
void oracle_epilogue_f32(const int32_t *acc, int64_t npos, int Cout, float s_x,
                         const float *s_w, const float *bias, float *y32)
{
    for (int64_t p = 0; p < npos; ++p)
        for (int co = 0; co < Cout; ++co) {
            float m = s_x * s_w[co];
            float a = (float)acc[p * Cout + co];
            float b = bias ? bias[co] : 0.0f;
            y32[p * Cout + co] = fmaf(a, m, b);
        }
}

/* ---- native-precision conv, for the layers a preset leaves unquantized ----
 * Same preset section of the page: the layers outside the chosen set keep
 * the VAE's own precision.  x bf16 [N][T][H][W][Cin], cache bf16
 * [N][kt-1][H][W][Cin] or NULL, w bf16 [Cout][Cin][kt][kh][kw] (the usual
 * Conv3d weight layout), bias float32 [Cout] or NULL.  For each listed output
 * position and channel:
 *   z   = sum over (i, j, l, ci) of x * w, plus bias   (the exact value: each
 *         product of two bf16 numbers is exact in binary64, and the binary64
 *         sum of K products is within K * 2^-53 of the exact sum)
 *   mag = sum of |x * w|, plus |bias|                 (scales the rounding
 *         error a float32 accumulation may make)
 * Frame and padding rules are those of the INT8 convolution above. */
int oracle_conv_bf16_positions(const uint16_t *x, const uint16_t *cache,
                               const uint16_t *w, const float *bias, int N,
                               int T, int H, int W, int Cin, int Cout, int kt,
                               int kh, int kw, const int64_t *pos, int64_t npos,
                               double *z, double *mag)
{
    if (!x || !w || !z || !mag || N <= 0 || T <= 0 || H <= 0 || W <= 0 ||
        Cin <= 0 || Cout <= 0 || kt <= 0 || kh <= 0 || kw <= 0 || npos < 0)
        return ORACLE_EARG;
    const int64_t total = (int64_t)N * T * H * W;
    const int ph = (kh - 1) / 2, pw = (kw - 1) / 2;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npos; ++p) {
        int64_t q = pos ? pos[p] : p;
        if (q < 0 || q >= total) {
#pragma omp atomic write
            status = ORACLE_EARG;
            continue;
        }
        int wo = (int)(q % W);
        int h = (int)((q / W) % H);
        int t = (int)((q / ((int64_t)W * H)) % T);
        int n = (int)(q / ((int64_t)W * H * T));
        for (int co = 0; co < Cout; ++co) {
            double sum = 0.0, abs_sum = 0.0;
            for (int i = 0; i < kt; ++i) {
                int tau = t - (kt - 1) + i;
                const uint16_t *frame;
                if (tau >= 0) {
                    frame = x + ((int64_t)n * T + tau) * H * W * Cin;
                } else if (cache) {
                    frame = cache + ((int64_t)n * (kt - 1) + (kt - 1 + tau)) * H * W * Cin;
                } else {
                    continue;             /* zero front padding              */
                }
                for (int j = 0; j < kh; ++j) {
                    int hh = h - ph + j;
                    if (hh < 0 || hh >= H) continue;
                    for (int l = 0; l < kw; ++l) {
                        int ww = wo - pw + l;
                        if (ww < 0 || ww >= W) continue;
                        const uint16_t *xp = frame + ((int64_t)hh * W + ww) * Cin;
                        for (int ci = 0; ci < Cin; ++ci) {
                            int64_t widx = ((((int64_t)co * Cin + ci) * kt + i) * kh + j) * kw + l;
                            double prod = (double)oracle_bf16_to_f32(xp[ci]) *
                                          (double)oracle_bf16_to_f32(w[widx]);
                            sum += prod;
                            abs_sum += fabs(prod);
                        }
                    }
                }
            }
            double b = bias ? (double)bias[co] : 0.0;
            z[p * Cout + co] = sum + b;
            mag[p * Cout + co] = abs_sum + fabs(b);
        }
    }
    return status;
}

/* ---- bf16 from binary64 ---------------------------------------------------
 * Round a finite binary64 value to bf16 once, to nearest with ties to even:
 * bf16 keeps 8 significant bits, so the rounding quantum of d is 2^(e-8)
 * where 2^(e-1) <= |d| < 2^e (never finer than bf16's subnormal step
 * 2^-133).  Scaling by a power of two is exact, rint() rounds half to even
 * in the default rounding mode, and the rounded value has at most 8
 * significant bits, so it is exact in binary32 and its upper half is the
 * bf16 pattern (a value that rounds past the largest bf16 becomes inf). */
uint16_t oracle_bf16_from_f64(double d)
{
    if (d == 0.0) return signbit(d) ? 0x8000u : 0x0000u;
    int e;
    (void)frexp(d, &e);                     /* |d| = m * 2^e, 0.5 <= m < 1       */
    int qe = e - 8;
    if (qe < -133) qe = -133;
    double r = ldexp(rint(ldexp(d, -qe)), qe);
    float f = (float)r;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* ---- RMSNorm + SiLU in front of a residual conv ---------------------------
 * The activation the quantizer sees in a decoder residual block is
 * SiLU(RMSNorm(x)) (the absorption of a preceding RMSNorm by the activation
 * quantizer: page "Doubling LLM token rates in ComfyUI" (ComfyUI v0.45.0),
 * section "Optimizing linear kernels"; the norm-SiLU-conv order of the VAE's
 * residual blocks is a reading).  Per pixel of C channels, by the definition,
 * in binary64 (libm's exp and sqrt), rounded to bf16 once at the end:
 *   n_c = x_c * gamma_c / sqrt(mean_c(x_c^2) + eps)
 *   h_c = bf16_rne(n_c / (1 + exp(-n_c)))
 * The GPU pass computes the same quantity in binary32 with its own exp; it is
 * held to one bf16 ulp of this value, not to its operation sequence. */
int oracle_rmsnorm_silu(const uint16_t *x, int64_t npix, int C, const float *gamma,
                        float eps, uint16_t *h)
{
    if (!x || !gamma || !h || npix <= 0 || C <= 0 || !(eps > 0.0f)) return ORACLE_EARG;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npix; ++p) {
        const uint16_t *xp = x + p * C;
        double ss = 0.0;
        for (int c = 0; c < C; ++c) {
            double v = (double)oracle_bf16_to_f32(xp[c]);
            ss += v * v;
        }
        double rms = sqrt(ss / (double)C + (double)eps);
        for (int c = 0; c < C; ++c) {
            double n = (double)oracle_bf16_to_f32(xp[c]) * (double)gamma[c] / rms;
            h[p * C + c] = oracle_bf16_from_f64(n / (1.0 + exp(-n)));
        }
    }
    return ORACLE_OK;
}

/* ---- the whole layer, end to end (used for CPU timing) -------------------
 * x bf16 [N][T][H][W][Cin] -> y bf16 [N][T][H][W][Cout] for the positions in
 * pos (all positions when pos is NULL and npos = N*T*H*W).  xq and acc are
 * caller-provided work buffers (numel of x, and npos*Cout). */
int oracle_layer(const uint16_t *x, const int8_t *cache, const int8_t *wq,
                 const float *s_w, const float *bias, int N, int T, int H,
                 int W, int Cin, int Cout, int kt, int kh, int kw,
                 float clip_ratio, const int64_t *pos, int64_t npos,
                 int8_t *xq, int32_t *acc, uint16_t *y, float *s_x_out)
{
    const int64_t numel = (int64_t)N * T * H * W * Cin;
    float a = oracle_act_absmax(x, numel);
    float s_x = oracle_scale_from_absmax(a, clip_ratio);
    oracle_act_quantize(x, numel, s_x, xq);
    int rc = oracle_conv_acc_positions(xq, cache, wq, N, T, H, W, Cin, Cout, kt,
                                       kh, kw, pos, npos, acc);
    if (rc != ORACLE_OK) return rc;
    oracle_epilogue(acc, npos, Cout, s_x, s_w, bias, y);
    if (s_x_out) *s_x_out = s_x;
    return ORACLE_OK;
}
