/*
 * qvae.h -- C ABI of the W8A8 INT8 CausalConv3d library for AMD Instinct
 * MI355X (gfx950).
 *
 * The method (page "ComfyUI-Qwen-VAE-Triton v0.2.0: Triton W8A8 kernel
 * accelerates the Qwen Image VAE decoder", sd114.wiki):
 *   - intro paragraph: an implicit-GEMM W8A8 kernel for the CausalConv3d
 *     layers of the Qwen-Image / Wan VAE decoder;
 *   - section "Three presets explained", scheme paragraph: symmetric INT8
 *     weights with one scale per output channel, dynamic symmetric INT8
 *     activations, INT8 x INT8 products with INT32 accumulation, FP32
 *     rescale, output in the activation's precision;
 *   - same section, fixed-parameter paragraph: clip ratio 1.0 for activations
 *     and weights, channels_last layout, automatic fallback to native
 *     precision on error;
 *   - same section, the preset list and the exclusion rule: which of the
 *     decoder's 28 patched Conv3d layers run in W8A8, the others staying in
 *     native precision (qvae_select_layer, qvae_causalconv3d_bf16).
 * Around the convolution: the RMSNorm + SiLU pass that feeds a decoder
 * residual conv, with the activation maximum fused in (qvae_rmsnorm_silu*;
 * page "Doubling LLM token rates in ComfyUI", section "Optimizing linear
 * kernels": activation quantization absorbing the preceding RMSNorm).
 * Readings where the page is silent: the activation scale is one scale per
 * tensor, s = fl(clip * absmax) / 127; codes are round-half-to-even of the
 * IEEE float32 quotient x / s, clamped to [-127, 127] (0 when s == 0); the
 * epilogue is y = bf16_rne(fma(float(acc), fl(s_x * s_w[co]), bias[co]));
 * causality is kt-1 zero front frames, or an explicit int8 cache of the
 * kt-1 previous frames quantized with the same scale.
 *
 * Conventions for every call:
 *   - pointers are DEVICE pointers (memory from hipMalloc / a torch CUDA
 *     tensor) unless stated otherwise; the caller allocates and frees every
 *     buffer, the library allocates nothing and keeps no per-call state
 *     (except qvae_act_absmax_quant_noalloc's static scratch array);
 *   - calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronize with the host;
 *   - layouts are channels-last: activations [N][T][H][W][C], contiguous;
 *   - x, xq, wq, wp, h, y, acc and cache must be 16-byte aligned;
 *   - the return value is a status code (QVAE_OK = 0, negative on error);
 *     arguments are validated before anything is launched; the library never
 *     aborts or throws; on a non-zero status the caller is expected to fall
 *     back to its native-precision path;
 *   - setting the environment variable QVAE_FORCE_FAIL=1 makes every call
 *     that launches work return QVAE_EFORCED without launching anything;
 *     QVAE_FORCE_FAIL=w8a8 does so only for the W8A8 calls (the quantizers
 *     and the INT8 convolutions), so a caller's per-layer fallback to the
 *     native-precision convolution runs instead (the page's "disable" A/B);
 *   - concurrent calls on different streams are safe as long as their output
 *     buffers do not alias (qvae_act_absmax_quant_noalloc: not on one GPU).
 */
#ifndef QVAE_H
#define QVAE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QVAE_OK 0
#define QVAE_EINVAL (-1)       /* null pointer, bad size, misaligned buffer   */
#define QVAE_EUNSUPPORTED (-2) /* valid but outside the supported set          */
#define QVAE_ELAUNCH (-3)      /* the HIP runtime reported a launch error      */
#define QVAE_EFORCED (-4)      /* failure forced by QVAE_FORCE_FAIL            */

/* Library version, (major << 16) | minor. */
int qvae_version(void);

/* Human-readable text for a status code (static storage, never NULL). */
const char *qvae_strerror(int status);

/*
 * Weight quantization, once per layer at load time (scheme paragraph:
 * symmetric INT8 weights, one scale per output channel; fixed parameters:
 * weight clip ratio 1.0).
 *   w        float32 [Cout][Cin][kt][kh][kw]  (the usual Conv3d weight layout)
 *   wq       int8, Cout*Cin*kt*kh*kw bytes, out, 16-byte aligned, packed in
 *            the order the convolution's matrix-core loop consumes it:
 *              wq[cb][i][s][j*kw + l][L][b] = q(co = 32*cb + L%32, i, j, l,
 *                                              ci = 32*s + 16*(L/32) + b)
 *            for cb < Cout/32, s < Cin/32, L < 64, b < 16 (each [L][b] block
 *            is one 1 KB operand fragment of 32 output x 32 input channels)
 *   w_scale  float32 [Cout]                   out
 * w_scale[co] = fl(clip * max |w[co,...]|) / 127, the maximum taken over
 * every (ci, kt, kh, kw); q = clamp(rne(w / w_scale[co]), -127, 127), 0 for
 * an all-zero channel.  The page fixes clip 1.0; a smaller ratio clips the
 * channel's outliers to +-127.
 * clip_ratio <= 0 or NaN is QVAE_EINVAL.
 * Supported: 0 < clip_ratio <= 1, Cout % 32 == 0, Cin % 32 == 0,
 * kt, kh, kw in {1, 3}.
 */
int qvae_quantize_weights(const float *w, int Cout, int Cin, int kt, int kh,
                          int kw, float clip_ratio, int8_t *wq,
                          float *w_scale, void *stream);

/* Words of the activation-maximum buffer (see qvae_act_absmax). */
#define QVAE_ABSMAX_WORDS 513

/*
 * Dynamic activation absmax, first of the two passes of the activation
 * quantizer (scheme paragraph: dynamic symmetric INT8 activations; the scale
 * is per tensor).
 *   x       bf16 bit patterns, numel elements (any layout)
 *   absmax  uint32 [QVAE_ABSMAX_WORDS], caller-allocated device buffer: this
 *           pass writes per-workgroup partial maxima of |x| (as bf16 bit
 *           patterns) into words 1.. (all of them: 0 where no workgroup
 *           reports); qvae_act_quantize reduces them and stores the bf16 bit
 *           pattern of max |x| (0..0x7F7F) in word 0.
 * Inputs must be finite.  numel >= 1.  Pass the same x and numel to the
 * following qvae_act_quantize.
 */
int qvae_act_absmax(const uint16_t *x, int64_t numel, uint32_t *absmax,
                    void *stream);

/*
 * Activation quantization, second pass, with the scale derived on the device
 * from the partial maxima of qvae_act_absmax (fixed parameters: activation
 * clip ratio 1.0; a smaller ratio clips outliers to +-127).
 *   absmax   in: partial maxima (from qvae_act_absmax on x, or from
 *            qvae_causalconv3d_w8a8_absmax that produced x);
 *            out: word 0 = bf16 bit pattern of max |x|
 *   x_scale  float32 [1] out: s = fl(clip * max |x|) / 127
 *   xq       int8 [numel] out: clamp(rne(x / s), -127, 127), 0 when s == 0
 * clip_ratio <= 0 or NaN is QVAE_EINVAL.  Supported: 0 < clip_ratio <= 1.
 */
int qvae_act_quantize(const uint16_t *x, int64_t numel, float clip_ratio,
                      uint32_t *absmax, float *x_scale, int8_t *xq,
                      void *stream);

/* qvae_act_absmax followed by qvae_act_quantize on the same stream (two
 * launches, no host synchronization); same clip_ratio rules. */
int qvae_act_absmax_quant(const uint16_t *x, int64_t numel, float clip_ratio,
                          uint32_t *absmax, float *x_scale, int8_t *xq,
                          void *stream);

/*
 * qvae_act_absmax_quant for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same two passes, the same codes, scale and maximum, but
 * the QVAE_ABSMAX_WORDS activation-maximum words live in a static device
 * array of the library instead of a caller's workspace (2052 bytes, one copy
 * per GPU, held until the process ends).  The caller still passes x, x_scale
 * and xq.  Allocates nothing on any call (the array's device address is
 * looked up once per device, by qvae_init or by the first call on that
 * device).  The array carries no state a call relies on; any numel that
 * qvae_act_absmax_quant accepts is accepted (the partial maxima never need
 * more than the array's 512 slots).  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (on different streams) race and may
 * return wrong scales; serialize them.  Same arguments and errors as
 * qvae_act_absmax_quant, minus `absmax`; QVAE_ELAUNCH if the runtime cannot
 * give the array's address.
 */
int qvae_act_absmax_quant_noalloc(const uint16_t *x, int64_t numel, float clip_ratio,
                                  float *x_scale, int8_t *xq, void *stream);

/*
 * The norm + SiLU pass in front of a decoder residual conv, h = SiLU(RMSNorm(x))
 * over the channels of every pixel (the absorption of a preceding RMSNorm by
 * the activation quantizer: page "Doubling LLM token rates in ComfyUI"
 * (ComfyUI v0.45.0), section "Optimizing linear kernels"; that the VAE's
 * residual convs sit behind norm and SiLU is a reading).  Per pixel:
 *   n_c = x_c * gamma[c] / sqrt(mean_c(x_c^2) + eps)
 *   h_c = bf16(n_c / (1 + exp(-n_c)))
 * computed in binary32 (a sequential sum of squares, an exp by Cody-Waite
 * range reduction and a polynomial, the correctly rounded quotient) and
 * rounded to nearest even: each h_c is the exact value rounded to bf16 or,
 * next to a bf16 rounding boundary, its neighbour (within one bf16 ulp).
 *   x      bf16 bit patterns [npix][C] (channels-last; npix = N*T*H*W)
 *   gamma  float32 [C]
 *   eps    > 0 (finite)
 *   h      bf16 bit patterns [npix][C] out
 * Supported: C % 8 == 0, 8 <= C <= 480.  eps <= 0, NaN or infinite: QVAE_EINVAL.
 */
int qvae_rmsnorm_silu(const uint16_t *x, int64_t npix, int C, const float *gamma, float eps, uint16_t *h,
                      void *stream);

/*
 * qvae_rmsnorm_silu that also leaves the partial maxima of |h| in an
 * activation-maximum buffer (words 1..; word 0 untouched), exactly as
 * qvae_act_absmax would for h: qvae_act_quantize(h, h_absmax, ...) then
 * quantizes h for the W8A8 conv without an absmax pass.  A W8A8 call
 * (QVAE_FORCE_FAIL=w8a8 fails it); h_absmax == NULL is QVAE_EINVAL.
 */
int qvae_rmsnorm_silu_absmax(const uint16_t *x, int64_t npix, int C, const float *gamma, float eps,
                             uint16_t *h, uint32_t *h_absmax, void *stream);

/*
 * W8A8 causal 3-D convolution as an implicit GEMM (intro paragraph: the
 * implicit-GEMM kernel for CausalConv3d; scheme paragraph: INT8 x INT8 with
 * INT32 accumulation, FP32 rescale, output in the activation precision).
 *   xq       int8 [N][T][H][W][Cin]
 *   x_scale  float32 [1] (device; from qvae_act_quantize)
 *   cache    int8 [N][kt-1][H][W][Cin], the kt-1 frames before frame 0, oldest
 *            first, quantized with the same x_scale; NULL = zero front frames
 *   wq, w_scale  from qvae_quantize_weights (wq in its packed layout)
 *   bias     float32 [Cout] or NULL (zero)
 *   y        bf16 bit patterns [N][T][H][W][Cout] out
 * y[n,t,h,w,co] = bf16_rne(fma(float(acc), fl(x_scale * w_scale[co]),
 * bias[co])) with acc = sum over (i, j, l, ci) of
 * q(co,i,j,l,ci) * X(n, t-(kt-1)+i, h-(kh-1)/2+j, w-(kw-1)/2+l, ci), where
 * frames before 0 come from the cache (or are zero) and out-of-image pixels
 * are zero.  Stride 1, dilation 1, "same" spatial padding.
 * Supported: Cin % 32 == 0, Cout % 32 == 0, kt in {1, 3}, (kh, kw) in
 * {(1, 1), (3, 3)}, 127^2 * Cin * kt * kh * kw < 2^31.
 */
int qvae_causalconv3d_w8a8(const int8_t *xq, const float *x_scale,
                           const int8_t *cache, const int8_t *wq,
                           const float *w_scale, const float *bias, int N,
                           int T, int H, int W, int Cin, int Cout, int kt,
                           int kh, int kw, uint16_t *y, void *stream);

/*
 * qvae_causalconv3d_w8a8 that also produces the activation maximum of its own
 * output, for the next layer's quantizer (the absmax pass fused into the
 * producing layer's epilogue):
 *   y_absmax  uint32 [QVAE_ABSMAX_WORDS], caller-allocated device buffer, out:
 *             words 1.. hold partial maxima of |y| over the output's pixels
 *             inside the image (bf16 bit patterns), exactly as qvae_act_absmax
 *             leaves them for y; word 0 is not touched.  Passing this buffer
 *             and y to qvae_act_quantize quantizes y without its absmax pass.
 * Same arguments, support and errors as qvae_causalconv3d_w8a8 otherwise;
 * y_absmax == NULL is QVAE_EINVAL.
 */
int qvae_causalconv3d_w8a8_absmax(const int8_t *xq, const float *x_scale,
                                  const int8_t *cache, const int8_t *wq,
                                  const float *w_scale, const float *bias,
                                  int N, int T, int H, int W, int Cin,
                                  int Cout, int kt, int kh, int kw,
                                  uint16_t *y, uint32_t *y_absmax,
                                  void *stream);

/*
 * Layer selection (section "Three presets explained": the patch covers 28
 * Conv3d layers of the decoder; Conservative quantizes the highest channel
 * level, 15 layers; Balanced the two highest levels, 22, keeping the 96-channel
 * level native; Aggressive every eligible layer, 26, except the two the fixed
 * rule keeps native, decoder.upsamples.14.residual.2 and .6).
 */
#define QVAE_PRESET_NATIVE 0        /* no layer quantized                     */
#define QVAE_PRESET_CONSERVATIVE 1
#define QVAE_PRESET_BALANCED 2
#define QVAE_PRESET_AGGRESSIVE 3

/*
 * 1 if the preset runs the named Conv3d layer in W8A8, 0 if it keeps it in
 * native precision, QVAE_EINVAL for a NULL name, a non-positive size or an
 * unknown preset.  Host only (no device work, never forced to fail).
 *   name          the layer's module name, e.g. "decoder.middle.0.residual.2"
 *                 (any prefix before "decoder." is allowed)
 *   Cin, Cout, kt, kh, kw   the layer's shape
 *   top_channels  the decoder's widest channel count (384 for the Wan /
 *                 Qwen-Image VAE)
 * Eligible: a decoder residual-block conv (name ending in ".residual.2" or
 * ".residual.6") of 3x3x3 with Cin and Cout multiples of 32.  Conservative:
 * eligible with Cin = Cout = top_channels.  Balanced: eligible with Cin and
 * Cout >= top_channels / 2.  Aggressive: eligible.  The two excluded layers are
 * native under every preset.
 */
int qvae_select_layer(int preset, const char *name, int Cin, int Cout, int kt, int kh, int kw,
                      int top_channels);

/*
 * Native-precision weights for the layers left unquantized: a permutation of
 * the bf16 weights into the order the convolution's matrix-core loop reads.
 *   w   bf16 bit patterns [Cout][Cin][kt][kh][kw]
 *   wp  bf16 bit patterns, Cout*Cin*kt*kh*kw values, out, 16-byte aligned:
 *         wp[cb][i][s][j*kw + l][L][e] = w(co = 32*cb + L%32,
 *                                          ci = 16*s + 8*(L/32) + e, i, j, l)
 *       for cb < Cout/32, s < Cin/16, L < 64, e < 8 (1 KB per fragment of 32
 *       output x 16 input channels)
 * Supported: Cout % 32 == 0, Cin % 16 == 0, kt, kh, kw in {1, 3}.
 */
int qvae_pack_weights_bf16(const uint16_t *w, int Cout, int Cin, int kt, int kh, int kw, uint16_t *wp,
                           void *stream);

/*
 * Native-precision causal 3-D convolution (the layers a preset keeps in the
 * VAE's own precision): bf16 x bf16 products, FP32 accumulation,
 *   y[n,t,h,w,co] = bf16_rne(fl32(sum over (i, j, l, ci) of w * X) + bias[co])
 * with X, the frame rules and the padding of qvae_causalconv3d_w8a8; the FP32
 * sum is formed in the matrix cores' order (not a fixed sequential order).
 *   x      bf16 bit patterns [N][T][H][W][Cin]
 *   cache  bf16 bit patterns [N][kt-1][H][W][Cin] (the kt-1 frames before
 *          frame 0, oldest first) or NULL = zero front frames
 *   wp     from qvae_pack_weights_bf16
 *   bias   float32 [Cout] or NULL (zero)
 *   y      bf16 bit patterns [N][T][H][W][Cout] out
 * Supported: Cin % 16 == 0, Cout % 32 == 0, kt in {1, 3}, (kh, kw) in
 * {(1, 1), (3, 3)}.
 */
int qvae_causalconv3d_bf16(const uint16_t *x, const uint16_t *cache, const uint16_t *wp, const float *bias,
                           int N, int T, int H, int W, int Cin, int Cout, int kt, int kh, int kw, uint16_t *y,
                           void *stream);

/*
 * qvae_causalconv3d_w8a8 on bf16 input: the conv quantizes x (and the cache)
 * itself as it stages them, so no quantize pass runs in between (the
 * activation quantizer absorbed into its consumer).  Codes, scale and output
 * are exactly those of qvae_act_quantize on x (and on the cache, with the same
 * scale) followed by qvae_causalconv3d_w8a8.
 *   x         bf16 bit patterns [N][T][H][W][Cin]
 *   cache     bf16 bit patterns [N][kt-1][H][W][Cin] (the kt-1 frames before
 *             frame 0, oldest first) or NULL = zero front frames
 *   x_absmax  activation-maximum buffer (QVAE_ABSMAX_WORDS words) whose words
 *             1.. hold partial maxima of |x| and of the cache (from
 *             qvae_act_absmax, qvae_causalconv3d_w8a8_absmax or
 *             qvae_rmsnorm_silu_absmax over the tensor they belong to); word 0
 *             is written with the maximum
 *   clip_ratio  0 < clip_ratio <= 1, as for qvae_act_quantize
 *   x_scale   float32 [1] out (the scale used), or NULL
 *   y         bf16 bit patterns [N][T][H][W][Cout] out
 * Same support as qvae_causalconv3d_w8a8; x_absmax == NULL or clip_ratio <= 0 /
 * NaN is QVAE_EINVAL.
 */
int qvae_causalconv3d_w8a8_qin(const uint16_t *x, const uint16_t *cache, uint32_t *x_absmax, float clip_ratio,
                               const int8_t *wq, const float *w_scale, const float *bias, int N, int T, int H,
                               int W, int Cin, int Cout, int kt, int kh, int kw, float *x_scale, uint16_t *y,
                               void *stream);

/*
 * Same contraction, writing the raw INT32 accumulators instead of the
 * epilogue (a verification export):
 *   acc  int32 [N][T][H][W][Cout] out
 */
int qvae_causalconv3d_w8a8_acc32(const int8_t *xq, const int8_t *cache,
                                 const int8_t *wq, int N, int T, int H, int W,
                                 int Cin, int Cout, int kt, int kh, int kw,
                                 int32_t *acc, void *stream);

/*
 * Optional set-up: loads the library's GPU code for the current device and
 * queries the device once, so that no later call pays for it (otherwise each
 * source file's kernels are loaded on the first launch of one of them).
 * Launches nothing and allocates nothing; calls work the same without it.
 * Returns QVAE_OK, or QVAE_ELAUNCH if the runtime cannot provide the code.
 */
int qvae_init(void);


#ifdef __cplusplus
}
#endif

#endif /* QVAE_H */
