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
// GEMM view: rows = output channels (A = weights), columns = output pixels
// (B = activations, channels-last so K = Cin is contiguous per pixel),
// K = valid temporal taps x kh x kw x Cin.  Nothing is materialised.
//
// Work split.  A workgroup owns BCO output channels and works through TH x TW
// pixel tiles of one frame at a time (one tile, or several in a row when the
// layer has more tiles than resident workgroups).  Each wave owns MB x NB
// blocks of 32x32 outputs (MB*32 channels x NB*32 pixels) and, when WK = 2,
// half of the K range (its own group of 32-channel slices in every stage);
// the two K halves are summed through LDS before the epilogue (INT32 sums are
// exact in any order).
//
// K loop.  A "stage" = one valid temporal tap i and SL 32-channel slices.
// Per stage the workgroup stages in LDS only the activation halo
// (TH+kh-1) x (TW+kw-1) pixels x 32 channels per slice, zero outside the
// image; it is reused by all kh*kw spatial taps (shifted windows) and by
// every wave.  Weights bypass LDS: they are pre-packed in MFMA fragment order
// (one contiguous 1 KB fragment per 32 channels x 32 K), so each wave loads
// its own fragments straight from L2 into VGPRs, PD k-steps ahead of use.
// Frames that are structurally zero (front padding without a cache) are
// skipped, not multiplied.  Halo stages are double-buffered: the global loads
// of stage s+1 (of the next tile, after a tile's last stage) are in flight
// while stage s computes.
//
// MFMA 32x32x32 i8 operands: lane L supplies 16 bytes of row/column (L % 32)
// for K-half (L / 32); A and B use the same lane/byte -> k assignment, so the
// product covers all 32 k of the slice whatever order the hardware sums them
// in.  The INT32 result: lane L holds column L % 32 and, in register r, row
// 8*(r/4) + 4*(L/32) + r%4 -- four consecutive output channels per register
// quad.  The 16x16x64 i8 shape (used by the large 3x3 tiles, see ConvCfg):
// lane L supplies 16 bytes of row/column (L % 16) for k-group (L / 16), again
// the same assignment for A and B; lane L holds column L % 16 and rows
// 4*(L/16) + {0..3} of the INT32 result.  The epilogue rescales them and
// transposes each 32-pixel block through LDS, so every lane stores 16
// contiguous bytes of the channels-last output; on request it also reduces
// the maximum of |y| into one partial slot per workgroup (the next layer's
// activation maximum).
//
// The same kernel, compiled with bf16 operands, is the native-precision conv
// of the layers a preset leaves unquantized (same section, the preset list):
// y = bf16_rne(fl32(sum of bf16 x bf16 products) + bias[co]), the sum in the
// matrix cores' FP32 accumulation order.  Everything above moves bytes, so
// that variant only swaps the matrix instruction (32x32x16 bf16, the same 16
// bytes per lane and operand) and the epilogue's rescale.
#include <type_traits>
#include <utility>

#include "qvae_internal.h"

namespace qvae {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// What a launch computes (one kernel instantiation each):
//   kModePlain  W8A8, bf16 output (with the output maximum when y_absmax is set)
//   kModeAcc32  W8A8, raw INT32 accumulators
//   kModeBf16   bf16 x bf16 products, FP32 accumulation, y = bf16_rne(acc + bias)
//               (the native-precision conv for the layers left unquantized)
//   kModeQin    W8A8 from bf16 input: the conv quantizes x (and the cache) as it
//               stages the halo, with the scale it reduces from the partial
//               maxima of x in its prologue (no separate quantize pass)
constexpr int kModePlain = 0, kModeAcc32 = 1, kModeBf16 = 2, kModeQin = 3;

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>): the index
// is a compile-time constant in every call, so arrays it selects from stay in
// registers whatever the surrounding loops look like to the optimizer
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// (fields in the order the prologue needs them, so its first scalar loads
// fetch them together)
struct ConvArgs {
    const int8_t *wq;       // packed [Cout/32][kt][Cin/32][kh*kw][64 lanes][16 bytes]
    const float *x_scale;
    const float *w_scale;
    const float *bias;
    const int8_t *xq;
    const int8_t *cache;
    void *out;
    uint32_t *y_absmax;     // partial-maximum slots of the output's |y|, or NULL
    int co_tiles, T, H, W, Cin, Cout, kt, N;
    int tiles_w, tiles_h;
    uint32_t *x_absmax;     // input-quantizing conv: activation-maximum buffer of x (words 1.. read, word 0 written)
    float *x_scale_out;     // input-quantizing conv: the scale it used, or NULL
    float clip;             // input-quantizing conv: clip ratio
};

// Cache policy of the output stores: non-temporal (the output is not read
// again by this kernel; measured 1-8 % faster than the default policy, most on
// the store-heavy 96-channel layers, outputs identical).
constexpr int kStoreNT = 2;

// Halo pixels are stored with a 48-byte pitch (32 data bytes + 16 unused):
// 3 is odd, so 16 consecutive pixels read by 16 consecutive lanes hit 16
// distinct 16-byte bank groups.  (Measured with the LDS bank-conflict
// counter: the 32x32 tiles' B reads, 32 pixels in lanes 0-31 and the same
// pixels' second 16 bytes in lanes 32-63, are conflict-free; for the 16x16
// tiles see SLICE_BYTES and b_q0.)
constexpr int kHaloPitch = 48;

// (QCFG: the input-quantizing conv's configuration, see M16 and HD; ACC32_:
// the INT32-output conv's, see PD; the launch-side quantities, threads and
// LDS bytes, depend on neither)
template <int WCO, int WPX, int WK, int MB, int NB, int TH, int TW, int KH, int KW, int SPW_, bool QCFG = false,
          bool ACC32_ = false>
struct ConvCfg {
    static constexpr int NW = WCO * WPX * WK;
    static constexpr int NT = NW * 64;
    static constexpr int BCO = WCO * MB * 32;
    static constexpr int BPX = WPX * NB * 32;
    static_assert(TH * TW == BPX, "pixel tile must match the wave layout");
    static_assert(TW == 16 || TW == 32, "a 32-pixel MFMA block covers two rows of 16 or one row of 32");
    static constexpr int KHW = KH * KW;
    static constexpr int SPW = SPW_;                         // slices per wave per stage
    static constexpr int SL = WK * SPW;                      // slices staged per stage
    // Matrix instruction shape.  The 3x3 kernels with two slices per wave and
    // stage and the large wave tiles (3 x 4 or 3 x 3 blocks, at least 4 waves) use the
    // 16x16 tiles with 64-deep K (16x16x64 INT8, 16x16x32 bf16: the same 16
    // bytes per lane and operand): one k-step spans both slices of one spatial
    // tap, and each 32x32 block of the wave tile is four 16x16 accumulator
    // blocks.  Under the chip's power limit these sustain ~13-16 % more INT8
    // ops per second than the 32x32x32 shape on nonzero operands (same tile,
    // same operand bytes per op).  The other kernels keep 32x32 tiles with one
    // slice per k-step: their smaller tiles give a one-step weight prefetch too
    // little time, and the two-wave tiles run out of registers (as does the
    // input-quantizing conv, whose quantizer needs registers in the K loop).
    static constexpr bool M16 = !QCFG && SPW == 2 && KHW > 1 && MB * NB >= 9 && NW >= 4;
    static constexpr int MA = M16 ? 2 * MB : MB;             // accumulator blocks along the channels
    static constexpr int NA = M16 ? 2 * NB : NB;             // accumulator blocks along the pixels
    static constexpr int KS = M16 ? KHW : KHW * SPW;         // k-steps per wave per stage
    // weight prefetch distance in k-steps.  A 16x16 k-step is 48 MFMAs, enough
    // for an L2 hit but not for a weight row that the pass before the conv
    // pushed out of L2.  The 16x16 tiles with the registers for a three-step
    // ring take it (4-5 % off their launches, none spilled): the split-K tile
    // and the 96 x 96 wave tile, the latter not in its INT32-output form.  The
    // 96 x 128 single-K tile spills with three slots and keeps one.
    static constexpr int PD = M16 ? ((WK > 1 || (NB == 3 && !ACC32_)) ? 3 : 1)
                                  : (KS % 3 == 0) ? 3 : (KS % 2 == 0) ? 2 : 1;
    static_assert(KS % PD == 0, "ring slots must repeat per stage");
    // (unspread halo: all chunks stored in the last step; PD for the input-quantizing conv, see HD)
    static constexpr int HALO_STORE_STEP = (QCFG && PD < KS) ? PD : KS - 1;
    static constexpr int HH = TH + KH - 1;
    static constexpr int HWD = TW + KW - 1;
    // one 32-channel slice of the halo.  32x32 tiles: slices 32 bytes apart
    // modulo 128, so the chunks of one pixel written by consecutive lanes
    // spread over banks.  16x16 tiles: slices a multiple of 256 bytes apart,
    // which with the lane groups of their B reads (see b_q0) makes those
    // reads conflict-free (measured with the LDS bank-conflict counter: any
    // other distance modulo 256, or the other assignment of lane groups to
    // slices, costs every such read twice the LDS cycles)
    static constexpr int SLICE_BYTES = M16 ? (HH * HWD * kHaloPitch + 16 + 255) / 256 * 256
                                           : (HH * HWD * kHaloPitch + 127) / 128 * 128 + 32;
    // the padding after slice 0's pixels, never read: the halo stores of lanes
    // without a chunk go there so the store loop needs no branch
    static constexpr int HALO_PAD = HH * HWD * kHaloPitch;
    static_assert(HALO_PAD + 16 <= SLICE_BYTES, "padding holds one 16-byte chunk");
    static constexpr int BUF_BYTES = SL * SLICE_BYTES;
    static constexpr int HALO_CHUNKS = SL * HH * HWD * 2;
    static constexpr int HALO_PT = (HALO_CHUNKS + NT - 1) / NT;
    // steps between loading a halo chunk of the next stage and storing it to
    // LDS: as many as the stage allows (the last chunk is stored in the last
    // step), so each load has most of a stage to arrive.  The input-quantizing
    // conv stores (and codes) each chunk PD steps after its load: its chunks
    // take twice the registers, and holding them longer costs it spills.
    static constexpr int HD = (!QCFG && KS - HALO_PT > PD) ? KS - HALO_PT : PD;
    static constexpr int ACC_BYTES = MB * NB * 16 * 64 * 4;  // one wave's accumulators
    // split K: each wave exports the half of its blocks its partner finishes
    static constexpr int XB = ACC_BYTES / 2;
    static constexpr int RED_BYTES = (WK > 1) ? WCO * WPX * 2 * XB : 0;
    static_assert(WK == 1 || NB % 2 == 0, "split K shares the pixel blocks between the two halves");
    // per-channel rescale factors fl(s_x * s_w[co]) and biases of the tile
    static constexpr int FAC_BYTES = 2 * BCO * 4;
    // LDS layout, elem = output bytes per value:
    //   WK = 1: [halo buffer 0][halo buffer 1][epilogue staging, a slice per wave][factors]
    //           separate regions: a workgroup that runs several tiles holds the
    //           next tile's first halo in a buffer while it finishes this one
    //   WK = 2: [halo buffers and split-K export slices, overlapped][factors]
    //           (one tile per workgroup; the exports start after the last stage)
    static constexpr int epi_wave_bytes(int elem) { return 32 * (MB * 32 * elem + 16); }
    static constexpr int work_bytes(int elem)
    {
        return WK > 1 ? ((2 * BUF_BYTES > RED_BYTES) ? 2 * BUF_BYTES : RED_BYTES)
                      : 2 * BUF_BYTES + WCO * WPX * epi_wave_bytes(elem);
    }
    static constexpr int lds_bytes(int elem) { return work_bytes(elem) + FAC_BYTES; }
};

// ACC32: write the raw INT32 accumulators instead of the epilogue.  OUTMAX:
// also reduce the maximum of |y| into a.y_absmax (one partial per workgroup).
// BF: bf16 operands (the kernel moves bytes: a.Cin is the bytes per pixel,
// 2 x the channels, so a 32-byte slice holds 16 channels and one 16-byte lane
// fragment feeds the bf16 matrix instruction exactly as it feeds the INT8
// one), FP32 accumulators, y = bf16_rne(fma(acc, 1, bias)).
// QIN: the input (and the cache) are bf16; every halo chunk of 16 channels is
// loaded as 32 bytes and quantized to codes before it is staged, exactly as
// the quantize pass would code it, with the scale s = fl(clip * max|x|) / 127
// reduced from x's partial maxima in the prologue.
template <int WCO, int WPX, int WK, int MB, int NB, int TH, int TW, int KH, int KW, int SPW, bool ACC32, bool OUTMAX,
          bool BF, bool QIN>
__global__ __launch_bounds__(WCO *WPX *WK * 64, (WK == 1 && MB * NB < 9) ? 2 : 1) void k_conv_igemm(ConvArgs a)
{
    static_assert(!(BF && (ACC32 || OUTMAX)), "the bf16 conv has the plain epilogue only");
    static_assert(!(QIN && (ACC32 || OUTMAX || BF)), "the input-quantizing conv has the plain epilogue only");
    constexpr int XB = QIN ? 2 : 1;   // bytes per input value in global memory
    using C = ConvCfg<WCO, WPX, WK, MB, NB, TH, TW, KH, KW, SPW, QIN, ACC32>;
    constexpr bool M16 = C::M16;
    constexpr int MA = C::MA, NA = C::NA;
    // one accumulator block: 32x32 (16 values per lane) or 16x16 (4 per lane)
    using AccV = std::conditional_t<M16, std::conditional_t<BF, v4f, v4i>, std::conditional_t<BF, v16f, v16i>>;
    constexpr int NT = C::NT;
    constexpr int PH = (KH - 1) / 2, PW = (KW - 1) / 2;
    constexpr int ELEM = ACC32 ? 4 : 2;                  // output bytes per value
    constexpr int WORK = C::work_bytes(ELEM);
    // Tiles per workgroup (see the launch): split K runs one (0).  Otherwise a
    // workgroup runs several, and the last stage of a tile prefetches the next
    // tile's first halo and, for the large wave tiles, its weight ring too (2).
    // The small tiles (1) reload the ring after the epilogue instead: holding
    // it across the epilogue would cost them their second workgroup per CU.
    constexpr int PERSIST = WK > 1 ? 0 : (MB * NB >= 9 ? 2 : 1);
    __shared__ __attribute__((aligned(16))) char smem[C::lds_bytes(ELEM)];

    const int tid = threadIdx.x;
    // all arguments in scalar registers before anything else: one batch of
    // scalar loads and one wait, instead of a wait at each first use
    asm volatile("" ::"s"(a.wq), "s"(a.x_scale), "s"(a.w_scale), "s"(a.bias), "s"(a.xq), "s"(a.cache), "s"(a.out),
                 "s"(a.co_tiles), "s"(a.T), "s"(a.H), "s"(a.W), "s"(a.Cin), "s"(a.Cout), "s"(a.kt), "s"(a.N),
                 "s"(a.tiles_w), "s"(a.tiles_h), "s"(a.y_absmax));
    if constexpr (QIN) asm volatile("" ::"s"(a.x_absmax), "s"(a.x_scale_out), "s"(a.clip));
    // ---- tiles.  Pixel tiles are numbered pt = column + tiles_w * (row +
    // tiles_h * (t + T * n)).  Workgroup b runs channel tile b % co_tiles and
    // pixel tiles b / co_tiles + k * (gridDim.x / co_tiles), k = 0, 1, ...
    // (the grid is a multiple of co_tiles; with split K, or when one round of
    // workgroups covers the frame, each runs one tile).  The channel tile is
    // fastest in the workgroup index, so with an even number of channel tiles
    // each XCD (workgroups are dealt round-robin over 8 XCDs) keeps to the
    // same weight slice in its L2.
    const int cot = blockIdx.x % a.co_tiles;
    const int pstride = gridDim.x / a.co_tiles;
    const int nptiles = a.tiles_w * a.tiles_h * a.T * a.N;
    const int co0 = cot * C::BCO;
    const int H = a.H, W = a.W, Cin = a.Cin, kt = a.kt;
    const int S = Cin >> 5;                       // 32-channel slices (a multiple of SL)
    const int nsp = S / C::SL;                    // stages per temporal tap
    struct Tile {
        int h0, w0, t, n;
        int i_lo;   // first temporal tap: frame t-(kt-1)+i exists, or comes from the cache
        int nst;    // K stages
    };
    auto decode = [&](int ptile) {
        Tile tl;
        const int tw = ptile % a.tiles_w;
        int r = ptile / a.tiles_w;
        const int th = r % a.tiles_h;
        r /= a.tiles_h;
        tl.t = r % a.T;
        tl.n = r / a.T;
        tl.h0 = th * TH;
        tl.w0 = tw * TW;
        tl.i_lo = a.cache ? 0 : max(0, kt - 1 - tl.t);
        tl.nst = (kt - tl.i_lo) * nsp;
        return tl;
    };
    int pt = blockIdx.x / a.co_tiles;
    Tile cur = decode(pt);

    // ---- wave roles (wave-uniform: keep them in scalar registers so every
    // branch on them is a scalar branch and the unrolled K loop stays
    // straight-line code)
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wk = wave / (WCO * WPX);
    const int wr = wave - wk * (WCO * WPX);
    const int wco = wr % WCO, wpx = wr / WCO;
    const int lrow = lane & 31, lhalf = lane >> 5;

    // weights: fragment (co block cb, tap i, slice s, spatial tap) at
    // ((((cb * kt + i) * S + s) * KHW + tap) * 64 + lane) * 16.  Within one
    // stage a wave walks KS consecutive fragments, so the k-step e of stage st
    // is at wstage(tile, st) + e * 1 KB.
    // The loads are raw buffer loads from this wave's weight slab: the
    // offset of a fragment is wave-uniform (a scalar operand) and the lane's
    // 16 bytes are a constant vector offset, so a load needs no address
    // arithmetic.
    // With 16x16 tiles, lane (r, g) = (lane % 16, lane / 16) of the operand of
    // channels 16 h .. 16 h + 15 of a 32-channel block takes the 16 bytes that
    // lane r + 16 h + 32 (g / 2) holds in the fragment of slice g % 2 (KHW
    // fragments further on): row r + 16 h, the same k values.  The k value
    // behind each (lane group, byte) is the same function for A and B (the B
    // reads below pair it the same way), so the product covers the 64 k of the
    // two slices exactly once whatever order the instruction sums them in.
    const int cb_stride = kt * S * C::KHW * 1024;          // bytes per 32-channel block (< 2^23)
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(a.wq) + (size_t)(co0 / 32 + wco * MB) * cb_stride, 0, MB * cb_stride, 0x00020000);
    const int wlane = M16 ? (((lane >> 4) & 1) * C::KHW * 1024 + ((lane & 15) + 32 * (lane >> 5)) * 16) : lane * 16;
    auto wstage = [&](const Tile &tl, int st) -> int {
        const int it = st / nsp;
        const int p = st - it * nsp;
        return (((tl.i_lo + it) * S + p * C::SL + wk * C::SPW) * C::KHW) * 1024;
    };
    // operand row m of the ring (32-channel block m, or 16-channel half m % 2
    // of block m / 2) for the k-step at fragment offset off
    auto load_wf = [&](int off, int m) -> v4i {
        if constexpr (M16)
            return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(wrs, wlane + (m & 1) * 256,
                                                                                 off + (m >> 1) * cb_stride, 0));
        else
            return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(wrs, wlane, off + m * cb_stride, 0));
    };
    v4i wreg[C::PD][MA];

    // ---- prologue loads: the epilogue's factors (a few words, issued first
    // so their latency hides under the rest), then the first stage's halo,
    // then the weight ring.  The factor products are formed only after the
    // halo's wait, so no load waits for another.  The factors and biases of this
    // tile's channels go to LDS with the first halo.
    constexpr int FPT = (C::BCO + NT - 1) / NT;
    float *s_fac = reinterpret_cast<float *>(smem + WORK);
    float f_ws[FPT], f_b[FPT];
    float sx = 0.0f;
    uint32_t qmax = 0;   // QIN: this thread's share of x's partial maxima
    if constexpr (QIN) {
        for (int k = tid; k < kAbsmaxParts; k += NT) qmax = max(qmax, a.x_absmax[1 + k]);
    }
    if constexpr (!ACC32) {
        sx = (BF || QIN) ? 1.0f : *a.x_scale;
#pragma unroll
        for (int k = 0; k < FPT; ++k) {
            const int c = tid + k * NT;
            f_ws[k] = 0.0f;
            f_b[k] = 0.0f;
            if (c < C::BCO) {
                f_ws[k] = BF ? 1.0f : a.w_scale[co0 + c];
                if (a.bias) f_b[k] = a.bias[co0 + c];
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    int wcur = wstage(cur, 0);

    // ---- halo load descriptors (stage independent parts).  Chunk u covers
    // pixel q = u / (2*SL) and 16 bytes c = u % (2*SL) of its SL slices, so
    // consecutive lanes read each pixel's 32*SL contiguous bytes together.
    // The loads are raw buffer loads: a pixel outside the image gets an
    // offset past the buffer's size, and the hardware returns zeros for it,
    // so neither the loads nor the LDS stores branch per lane.
    constexpr uint32_t kOutside = 0x80000000u;   // >= any frame size (frames are < 2^31 bytes)
    uint32_t h_off[C::HALO_PT];   // byte offset from the stage's slice base, kOutside = zero pixel
    int h_lds[C::HALO_PT];        // LDS byte offset inside a stage buffer (idle lanes: slice padding)
    auto set_hoff = [&](const Tile &tl) {
#pragma unroll
        for (int k = 0; k < C::HALO_PT; ++k) {
            const int u = tid + k * NT;
            h_off[k] = kOutside;
            if (u < C::HALO_CHUNKS) {
                const int q = u / (2 * C::SL), c = u - q * (2 * C::SL);
                const int hh = q / C::HWD, ww = q - hh * C::HWD;
                const int gh = tl.h0 - PH + hh, gw = tl.w0 - PW + ww;
                if (gh >= 0 && gh < H && gw >= 0 && gw < W) h_off[k] = (uint32_t)(((gh * W + gw) * Cin + c * 16) * XB);
            }
        }
    };
#pragma unroll
    for (int k = 0; k < C::HALO_PT; ++k) {
        const int u = tid + k * NT;
        h_lds[k] = C::HALO_PAD;
        if (u < C::HALO_CHUNKS) {
            const int q = u / (2 * C::SL), c = u - q * (2 * C::SL);
            h_lds[k] = (c >> 1) * C::SLICE_BYTES + q * kHaloPitch + (c & 1) * 16;
        }
    }
    const size_t frame_bytes = (size_t)H * W * Cin * XB;   // bytes of one input frame in global memory
    auto frame_ptr = [&](const Tile &tl, int i) -> const int8_t * {
        const int tau = tl.t - (kt - 1) + i;
        if (tau >= 0) return a.xq + ((size_t)tl.n * a.T + tau) * frame_bytes;
        return a.cache + ((size_t)tl.n * (kt - 1) + (kt - 1 + tau)) * frame_bytes;
    };
    v4i hreg[C::HALO_PT];
    v4i hreg2[QIN ? C::HALO_PT : 1];   // QIN: the second 16 bytes (channels 8..15) of each bf16 chunk
    auto halo_rsrc = [&](const Tile &tl, int st) {
        const int it = st / nsp;
        const int p = st - it * nsp;
        const int8_t *fps = frame_ptr(tl, tl.i_lo + it) + p * C::SL * 32 * XB;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(fps), 0,
                                                 (int)(frame_bytes - (size_t)p * C::SL * 32 * XB), 0x00020000);
    };
    auto load_chunk = [&](__amdgpu_buffer_rsrc_t rs, int k) {
        hreg[k] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)h_off[k], 0, 0));
        if constexpr (QIN)   // (an out-of-image pixel's offset + 16 is still past the buffer)
            hreg2[k] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(h_off[k] + 16), 0, 0));
    };
    // QIN: the scale of x and the quantizer's constants (set in the prologue)
    float q_s = 0.0f, q_r = 0.0f;
    bool q_zero = true, q_exact = false;
    auto quant_half = [&](v4i v) -> uint2 {
        return q_zero ? make_uint2(0u, 0u) : quant8(__builtin_bit_cast(u32x4, v), q_s, q_r, q_exact);
    };
    auto store_codes_lds = [&](int buf, int k, uint2 c0, uint2 c1) {
        *reinterpret_cast<v4i *>(smem + buf * C::BUF_BYTES + h_lds[k]) = v4i{(int)c0.x, (int)c0.y, (int)c1.x, (int)c1.y};
    };
    auto store_chunk = [&](int buf, int k) {
        v4i v = hreg[k];
        if constexpr (QIN) {
            v = v4i{0, 0, 0, 0};
            if (!q_zero) {
                const uint2 c0 = quant8(__builtin_bit_cast(u32x4, hreg[k]), q_s, q_r, q_exact);
                const uint2 c1 = quant8(__builtin_bit_cast(u32x4, hreg2[k]), q_s, q_r, q_exact);
                v = v4i{(int)c0.x, (int)c0.y, (int)c1.x, (int)c1.y};
            }
        }
        *reinterpret_cast<v4i *>(smem + buf * C::BUF_BYTES + h_lds[k]) = v;
    };
    auto load_halo = [&](const Tile &tl, int st) {
        const __amdgpu_buffer_rsrc_t rs = halo_rsrc(tl, st);
#pragma unroll
        for (int k = 0; k < C::HALO_PT; ++k) load_chunk(rs, k);
    };
    auto store_halo = [&](int buf) {
#pragma unroll
        for (int k = 0; k < C::HALO_PT; ++k) store_chunk(buf, k);
    };

    set_hoff(cur);
    load_halo(cur, 0);
    __builtin_amdgcn_sched_barrier(0);
    // the weight ring after the first halo: loads complete in issue order, so
    // the halo's LDS stores and the barrier before the first stage wait for
    // the halo alone and the ring's rows stay in flight until their MFMAs
#pragma unroll
    for (int e = 0; e < C::PD; ++e)
#pragma unroll
        for (int m = 0; m < MA; ++m) wreg[e][m] = load_wf(wcur + e * 1024, m);
    __builtin_amdgcn_sched_barrier(0);

    // QIN: the tensor maximum from the partial maxima (while the first halo is
    // in flight), then the scale the quantize pass would derive from it
    if constexpr (QIN) {
        __shared__ uint32_t s_qmax[C::NW];
        const uint32_t m = wave_max_u32(qmax);
        if (lane == 0) s_qmax[wave] = m;
        lds_barrier();
        uint32_t mbits = s_qmax[0];
#pragma unroll
        for (int k = 1; k < C::NW; ++k) mbits = max(mbits, s_qmax[k]);
        const float amax = bf16_bits_to_float(mbits);
        q_s = (a.clip * amax) / 127.0f;
        q_r = 1.0f / q_s;
        q_zero = !(q_s > 0.0f);
        q_exact = !(q_r < __builtin_inff());
        sx = q_s;
        if (blockIdx.x == 0 && tid == 0) {
            a.x_absmax[0] = mbits;
            if (a.x_scale_out) *a.x_scale_out = q_s;
        }
    }

    // B fragment base offsets (pixel of lane, within the stage buffer).  32x32
    // tiles: lane (lrow, lhalf) reads 16 bytes lhalf of pixel lrow of the block.
    // 16x16 tiles: lane (r, g) reads 16 bytes g / 2 of slice g % 2 of pixel r,
    // the k values the weight operand's lane group g holds (lanes 0-15 and
    // 16-31 read the two slices at the same bank offsets, lanes 32-63 the same
    // pixels 16 bytes further on).
    int b_q0[NA];
#pragma unroll
    for (int nb = 0; nb < NA; ++nb) {
        if constexpr (M16) {
            const int p = (wpx * NA + nb) * 16 + (lane & 15);
            const int pr = p / TW, pc = p - pr * TW;
            b_q0[nb] = (pr * C::HWD + pc) * kHaloPitch + (lane >> 5) * 16 +
                       (((lane >> 4) & 1) + wk * C::SPW) * C::SLICE_BYTES;
        } else {
            const int p = (wpx * NB + nb) * 32 + lrow;
            const int pr = p / TW, pc = p - pr * TW;
            b_q0[nb] = (pr * C::HWD + pc) * kHaloPitch + lhalf * 16 + wk * C::SPW * C::SLICE_BYTES;
        }
    }

    AccV acc[MA][NA];
#pragma unroll
    for (int mb = 0; mb < MA; ++mb)
#pragma unroll
        for (int nb = 0; nb < NA; ++nb) acc[mb][nb] = AccV{};

    store_halo(0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!ACC32) {
#pragma unroll
        for (int k = 0; k < FPT; ++k) {
            const int c = tid + k * NT;
            if (c < C::BCO) {
                s_fac[c] = sx * f_ws[k];
                s_fac[C::BCO + c] = f_b[k];
            }
        }
    }
    lds_barrier();

    // B fragments of k-step e of the stage held in buffer xs
    auto read_b1 = [&](const char *xs, int e, int nb) -> v4i {
        const int sp = e / C::KHW, tap = e % C::KHW;
        const int j = tap / KW, l = tap % KW;
        return *reinterpret_cast<const v4i *>(xs + sp * C::SLICE_BYTES + (j * C::HWD + l) * kHaloPitch + b_q0[nb]);
    };
    auto read_b = [&](const char *xs, int e, v4i (&bv)[NA]) {
        const int sp = e / C::KHW, tap = e % C::KHW;
        const int j = tap / KW, l = tap % KW;
        const char *xsl = xs + sp * C::SLICE_BYTES + (j * C::HWD + l) * kHaloPitch;
#pragma unroll
        for (int nb = 0; nb < NA; ++nb) bv[nb] = *reinterpret_cast<const v4i *>(xsl + b_q0[nb]);
    };

    // One stage on the halo in buffer buf.  MORE > 0: a next stage exists (in
    // this tile or the workgroup's next one) and its halo (buffer resource rsn,
    // lane offsets h_off) goes to the other buffer; MORE = 2: its weights (ring
    // offset wnext) also enter the ring in the last PD k-steps.  The very last
    // stage is an instantiation without either, so the epilogue never waits
    // for prefetches nobody uses.  When the stage has enough k-steps, halo
    // chunk k of the next stage is loaded in step k and stored to the other
    // buffer in step k + HD (HD = KS - HALO_PT: the last chunk in the last
    // step, so each load has most of the stage to arrive; measured 1-4 %
    // faster than storing PD steps after the load), one instruction per step
    // between two MFMAs; otherwise all chunks are loaded at the start and
    // stored in the last step.
    constexpr bool SPREAD = C::HALO_PT + C::PD <= C::KS;
    auto run_stage = [&](int buf, int wnext, __amdgpu_buffer_rsrc_t rsn, auto more_c) __attribute__((always_inline)) {
        constexpr int MORE = decltype(more_c)::value;
        if constexpr (!SPREAD && MORE > 0) {
#pragma unroll
            for (int k = 0; k < C::HALO_PT; ++k) load_chunk(rsn, k);
        }
        const char *xs = smem + buf * C::BUF_BYTES;
        v4i bcur[NA], bnext[NA];
        read_b(xs, 0, bcur);
        // Each k-step issues its MB x NB MFMAs with one memory instruction
        // after each of the first few: the LDS read of the next step's B
        // fragment nb after MFMA nb, and the reload of weight ring slot row
        // mb (PD steps ahead) right after the last MFMA that reads it.  A
        // wave has one MFMA in flight at a time, so a memory instruction
        // issued between two MFMAs costs nothing, while a cluster of them
        // stalls the matrix pipe.  The scheduling barriers pin this order (the
        // scheduler would otherwise sink the prefetches down to their use
        // and expose their latency).
#pragma unroll
        for (int e = 0; e < C::KS; ++e) {
            const int slot = e % C::PD;
            uint2 qc0 = make_uint2(0u, 0u);   // QIN: first half of the chunk being staged this step
            const bool wload = e + C::PD < C::KS || MORE == 2;
            const int wsrc = (e + C::PD < C::KS) ? wcur + (e + C::PD) * 1024 : wnext + (e + C::PD - C::KS) * 1024;
#pragma unroll
            for (int mb = 0; mb < MA; ++mb)
#pragma unroll
                for (int nb = 0; nb < NA; ++nb) {
                    constexpr int last = MA * NA - 1;
                    const int i = mb * NA + nb;
                    if constexpr (M16 && BF)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wreg[slot][mb]),
                                                                              __builtin_bit_cast(bf16x8_t, bcur[nb]),
                                                                              acc[mb][nb], 0, 0, 0);
                    else if constexpr (M16)
                        acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wreg[slot][mb], bcur[nb], acc[mb][nb], 0, 0, 0);
                    else if constexpr (BF)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, wreg[slot][mb]),
                                                                              __builtin_bit_cast(bf16x8_t, bcur[nb]),
                                                                              acc[mb][nb], 0, 0, 0);
                    else
                        acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wreg[slot][mb], bcur[nb], acc[mb][nb], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (i < NA && e + 1 < C::KS) bnext[i] = read_b1(xs, e + 1, i);
#pragma unroll
                    for (int m2 = 0; m2 < MA; ++m2) {
                        const int at = (m2 == 0) ? (NA < last ? NA : last) : (m2 + 1) * NA - 1;
                        if (i == at && wload) wreg[slot][m2] = load_wf(wsrc, m2);
                    }
                    if constexpr (SPREAD && MORE > 0) {
                        // halo chunk e goes out right after weight row 0, so
                        // the wait for weight row 1 of the same step (PD steps
                        // later) covers it and its store needs no extra wait
                        constexpr int hl = NA < last ? NA : last;
                        constexpr int hs = NA + 1 < last ? NA + 1 : last;
                        if (i == hl && e < C::HALO_PT) load_chunk(rsn, e);
                        if constexpr (QIN) {
                            // the two 8-value halves of the chunk are quantized in two
                            // consecutive MFMA slots, so neither burst stalls the matrix pipe long
                            constexpr int hs2 = hs + 1 <= last ? hs + 1 : hs;
                            if (e >= C::HD && e - C::HD < C::HALO_PT) {
                                if (i == hs) qc0 = quant_half(hreg[e - C::HD]);
                                if (i == hs2) store_codes_lds(buf ^ 1, e - C::HD, qc0, quant_half(hreg2[e - C::HD]));
                            }
                        } else {
                            if (i == hs && e >= C::HD && e - C::HD < C::HALO_PT) store_chunk(buf ^ 1, e - C::HD);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            // Without spreading, the next stage's halo (loaded at the start of
            // this stage) goes to the other buffer in the last step; nobody
            // reads that buffer after the previous stage's barrier.
            if constexpr (!SPREAD && MORE > 0) {
                if (e == C::HALO_STORE_STEP) store_halo(buf ^ 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (e + 1 < C::KS) {
#pragma unroll
                for (int nb = 0; nb < NA; ++nb) bcur[nb] = bnext[nb];
            }
        }
        lds_barrier();
        wcur = wnext;
    };
    // ---- the workgroup's tiles: stages run back to back across tile
    // boundaries (the last stage of a tile prefetches the next tile's first
    // halo and weights), the epilogue of a tile runs while that halo waits in
    // its buffer.
    uint32_t ymax = 0;   // packed running maximum of |y| (bf16 bits) over this lane's outputs
    auto epilogue = [&](const Tile &tl) __attribute__((always_inline)) {
        // 16x16 tiles: accumulators in units of register quads (below); 32x32
        // tiles: the per-(block, register group) form, kept apart so that its
        // register allocation is the one the 32x32 kernels were tuned with
        if constexpr (M16) {
            // ---- split K: each half finishes half of the pixel blocks.  Wave wk
            // exports to LDS the blocks the other half finishes; after the barrier it
            // reads the other half's export of its own blocks into registers and adds
            // it while rescaling (INT32 sums, exact in any order; FP32 sums of the
            // bf16 conv add the same two partials whichever wave finishes).
            constexpr int HB = (WK > 1) ? NB / 2 : NB;           // 32-pixel blocks this wave finishes
            // A lane's accumulators of one 32-pixel block come in UNITS pieces of 4
            // values: 32x32 tiles, unit u = (mb, g) = (u / 4, u % 4) holds channels
            // 32 mb + 8 g + 4 lhalf + {0..3} of pixel lrow; 16x16 tiles, unit u =
            // (m, hf) = (u / 2, u % 2) is the lane's register quad of the 16x16
            // block (m, 2 j + hf): channels 16 m + 4 (lane / 16) + {0..3} of pixel
            // 16 hf + lane % 16 of the 32-pixel block j.
            constexpr int UNITS = 4 * MB;
            // (every lambda that touches the accumulators is forced inline: one left
            // out of line takes their address, and they then live in scratch memory)
            auto unit_acc = [&](auto wkc, auto jc, auto uc) __attribute__((always_inline)) -> v4i {
                constexpr int WKC = decltype(wkc)::value, j = decltype(jc)::value, u = decltype(uc)::value;
                if constexpr (M16) {
                    return __builtin_bit_cast(v4i, acc[u >> 1][WKC * 2 * HB + 2 * j + (u & 1)]);
                } else {
                    const v16i x = __builtin_bit_cast(v16i, acc[u >> 2][WKC * HB + j]);
                    constexpr int g = u & 3;
                    return v4i{x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
                }
            };
            v4i part[(WK > 1) ? MB * HB * 4 : 1];
            if constexpr (WK > 1) {
                int4 *exp_mine = reinterpret_cast<int4 *>(smem + (wr * 2 + wk) * C::XB);
                const int4 *exp_other = reinterpret_cast<const int4 *>(smem + (wr * 2 + (1 - wk)) * C::XB);
                // The exported block is picked by value (a select on the wave-uniform
                // wk), not by branching on wk: the optimizer merges two branches that
                // differ only in a constant block index into one with a variable
                // index, and a variable index sends the accumulators to scratch memory.
                static_for<HB>([&](auto jc) __attribute__((always_inline)) {
                    static_for<UNITS>([&](auto uc) __attribute__((always_inline)) {
                        constexpr int j = decltype(jc)::value, u = decltype(uc)::value;
                        const v4i a0 = unit_acc(std::integral_constant<int, 0>{}, jc, uc);
                        const v4i a1 = unit_acc(std::integral_constant<int, 1>{}, jc, uc);
                        const v4i v = (wk == 0) ? a1 : a0;   // the partner's half
                        exp_mine[(j * UNITS + u) * 64 + lane] = make_int4(v[0], v[1], v[2], v[3]);
                    });
                });
                lds_barrier();
    #pragma unroll
                for (int q = 0; q < MB * HB * 4; ++q) {
                    const int4 u = exp_other[q * 64 + lane];
                    part[q] = v4i{u.x, u.y, u.z, u.w};
                }
            }

            // ---- epilogue.  A lane holds four consecutive output channels of a
            // pixel per accumulator unit (the unit map above).  Each 32-pixel
            // block is rescaled (one FP32 fma with the
            // per-channel factor and bias, then bf16 round-to-nearest-even with the
            // packed convert), written to the wave's LDS staging rows
            // [pixel][channel], then read back row-wise so every lane stores 16
            // contiguous bytes and consecutive lanes continue along the channels-last
            // output row.  The stores are raw buffer stores relative to the tile's
            // first output: a pixel outside the image gets an offset past the
            // buffer's size and the hardware drops it, so no lane branches.
            constexpr int ROWB = MB * 32 * ELEM;                 // one pixel's channels of this wave
            constexpr int EPITCH = ROWB + 16;                    // odd multiple of 16 bytes
            constexpr int CHUNKS = 32 * ROWB / 16;               // 16-byte pieces per block
            static_assert(CHUNKS % 64 == 0, "whole chunks per lane");
            static_assert(32 * EPITCH <= C::epi_wave_bytes(ELEM), "staging rows fit the wave's LDS slice");
            static_assert(WK == 1 || 32 * EPITCH <= C::XB, "staging rows fit the partner's export slice");
            // staging: with split K the partner's export slice (this wave has read it
            // into registers and nobody else touches it); otherwise a slice per wave
            char *stage = smem + (WK > 1 ? (wr * 2 + (1 - wk)) * C::XB : 2 * C::BUF_BYTES + wr * C::epi_wave_bytes(ELEM));

            const int cw0 = co0 + wco * MB * 32;                 // first channel of this wave
            const size_t tile_first = ((((size_t)tl.n * a.T + tl.t) * H + tl.h0) * W + tl.w0) * (size_t)a.Cout + cw0;
            const size_t out_total = (size_t)a.N * a.T * H * W * (size_t)a.Cout;
            const size_t left = (out_total - tile_first) * ELEM;
            const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
                static_cast<char *>(a.out) + tile_first * ELEM, 0, (int)(left < kOutside ? left : kOutside), 0x00020000);
            const uint32_t row_bytes = (uint32_t)W * (uint32_t)a.Cout * ELEM;
            typedef float f4 __attribute__((ext_vector_type(4)));
            typedef float f2 __attribute__((ext_vector_type(2)));
            typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
            // this lane's per-channel factors and biases: read from LDS once for the
            // large wave tiles (registers to spare after the K loop), else at each
            // use (small tiles keep two waves per SIMD; with the output maximum a
            // workgroup running several tiles has no registers left for them)
            constexpr bool HOIST = !ACC32 && (WK > 1 || (!OUTMAX && MB * NB >= 9));
            // the first channel of unit u (relative to the wave's first channel) and
            // the pixel row it sits in within the 32-pixel block
            auto unit_col = [&](int u) __attribute__((always_inline)) { return M16 ? (u >> 1) * 16 + 4 * (lane >> 4) : (u >> 2) * 32 + (u & 3) * 8 + lhalf * 4; };
            auto unit_px = [&](int u) __attribute__((always_inline)) { return M16 ? (u & 1) * 16 + (lane & 15) : lrow; };
            // distinct factor quads: one per unit (32x32), one per 16-channel row (16x16)
            constexpr int NF = M16 ? MA : UNITS;
            auto unit_f = [&](int u) __attribute__((always_inline)) { return M16 ? (u >> 1) : u; };
            f4 fm[HOIST ? NF : 1], fb[HOIST ? NF : 1];
            if constexpr (HOIST) {
    #pragma unroll
                for (int k = 0; k < NF; ++k) {
                    const int col = wco * MB * 32 + unit_col(M16 ? 2 * k : k);
                    fm[k] = *reinterpret_cast<const f4 *>(s_fac + col);
                    fb[k] = *reinterpret_cast<const f4 *>(s_fac + C::BCO + col);
                }
            }
            // block j (0 <= j < HB) of this wave's share; WKC = its K half (0 without split K)
            auto finish_block = [&](auto wkc, auto jc) __attribute__((always_inline)) {
                constexpr int WKC = decltype(wkc)::value;
                constexpr int j = decltype(jc)::value;
                // the pixels this lane holds in the matrix layout (row lrow of the
                // block; 16x16 tiles: rows lane % 16 and 16 + lane % 16): only
                // outputs inside the image count towards the output maximum
                bool px_in[M16 ? 2 : 1] = {};
                if constexpr (OUTMAX) {
    #pragma unroll
                    for (int hf = 0; hf < (M16 ? 2 : 1); ++hf) {
                        const int pl = (wpx * NB + WKC * HB + j) * 32 + unit_px(hf);
                        const int plr = pl / TW;
                        px_in[hf] = tl.h0 + plr < H && tl.w0 + (pl - plr * TW) < W;
                    }
                }
                static_for<UNITS>([&](auto uc) __attribute__((always_inline)) {
                    constexpr int u = decltype(uc)::value;
                    v4i v = unit_acc(wkc, jc, uc);
                    f4 vf{};
                    if constexpr (BF) {
                        vf = __builtin_bit_cast(f4, v);
                        if constexpr (WK > 1) vf += __builtin_bit_cast(f4, part[j * UNITS + u]);
                    } else {
                        if constexpr (WK > 1) v += part[j * UNITS + u];
                    }
                    char *dst = stage + unit_px(u) * EPITCH + unit_col(u) * ELEM;
                    if constexpr (ACC32) {
                        *reinterpret_cast<v4i *>(dst) = v;
                    } else {
                        f4 y;
    #pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float av = BF ? vf[e] : (float)v[e];
                            if constexpr (HOIST) {
                                y[e] = __builtin_fmaf(av, fm[unit_f(u)][e], fb[unit_f(u)][e]);
                            } else {
                                const int col = wco * MB * 32 + unit_col(u) + e;
                                y[e] = __builtin_fmaf(av, s_fac[col], s_fac[C::BCO + col]);
                            }
                        }
                        const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{y[0], y[1]}, bf2));
                        const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{y[2], y[3]}, bf2));
                        *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
                        if constexpr (OUTMAX) {
                            if (px_in[M16 ? (u & 1) : 0]) ymax = pk_absmax(pk_absmax(ymax, lo), hi);
                        }
                    }
                });
    #pragma unroll
                for (int k = 0; k < CHUNKS / 64; ++k) {
                    const int c = k * 64 + lane;
                    const int px = c / (ROWB / 16);
                    const int off = (c - px * (ROWB / 16)) * 16;
                    const v4i v = *reinterpret_cast<const v4i *>(stage + px * EPITCH + off);
                    const int p = (wpx * NB + WKC * HB + j) * 32 + px;
                    const int pr = p / TW, pc = p - pr * TW;
                    const bool inside = tl.h0 + pr < H && tl.w0 + pc < W;
                    const uint32_t o = inside ? pr * row_bytes + (uint32_t)(pc * a.Cout * ELEM + off) : kOutside;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), orsrc, (int)o, 0, kStoreNT);
                }
            };
            auto finish_all = [&](auto wkc) __attribute__((always_inline)) { static_for<HB>([&](auto jc) __attribute__((always_inline)) { finish_block(wkc, jc); }); };
            if (WK > 1 && wk == 1)
                finish_all(std::integral_constant<int, 1>{});
            else
                finish_all(std::integral_constant<int, 0>{});
        } else {
            // ---- split K: each half finishes half of the pixel blocks.  Wave wk
            // exports to LDS the blocks the other half finishes; after the barrier it
            // reads the other half's export of its own blocks into registers and adds
            // it while rescaling (INT32 sums, exact in any order; FP32 sums of the
            // bf16 conv add the same two partials whichever wave finishes).
            constexpr int HB = (WK > 1) ? NB / 2 : NB;           // blocks this wave finishes
            v4i part[(WK > 1) ? MB * HB * 4 : 1];
            if constexpr (WK > 1) {
                int4 *exp_mine = reinterpret_cast<int4 *>(smem + (wr * 2 + wk) * C::XB);
                const int4 *exp_other = reinterpret_cast<const int4 *>(smem + (wr * 2 + (1 - wk)) * C::XB);
                auto xport = [&](auto wkc) {
                    constexpr int other = 1 - decltype(wkc)::value;
                    static_for<MB>([&](auto mbc) {
                        static_for<HB>([&](auto jc) {
                            constexpr int mb = decltype(mbc)::value, j = decltype(jc)::value;
                            const v16i v = __builtin_bit_cast(v16i, acc[mb][other * HB + j]);
    #pragma unroll
                            for (int g = 0; g < 4; ++g)
                                exp_mine[((mb * HB + j) * 4 + g) * 64 + lane] =
                                    make_int4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
                        });
                    });
                };
                if (wk == 0)
                    xport(std::integral_constant<int, 0>{});
                else
                    xport(std::integral_constant<int, 1>{});
                lds_barrier();
    #pragma unroll
                for (int q = 0; q < MB * HB * 4; ++q) {
                    const int4 u = exp_other[q * 64 + lane];
                    part[q] = v4i{u.x, u.y, u.z, u.w};
                }
            }

            // ---- epilogue.  Lane (lrow, lhalf) holds pixel lrow of each 32-pixel
            // block and output channels 8*g + 4*lhalf + {0..3} of each 32-channel
            // block.  Each 32-pixel block is rescaled (one FP32 fma with the
            // per-channel factor and bias, then bf16 round-to-nearest-even with the
            // packed convert), written to the wave's LDS staging rows
            // [pixel][channel], then read back row-wise so every lane stores 16
            // contiguous bytes and consecutive lanes continue along the channels-last
            // output row.  The stores are raw buffer stores relative to the tile's
            // first output: a pixel outside the image gets an offset past the
            // buffer's size and the hardware drops it, so no lane branches.
            constexpr int ROWB = MB * 32 * ELEM;                 // one pixel's channels of this wave
            constexpr int EPITCH = ROWB + 16;                    // odd multiple of 16 bytes
            constexpr int CHUNKS = 32 * ROWB / 16;               // 16-byte pieces per block
            static_assert(CHUNKS % 64 == 0, "whole chunks per lane");
            static_assert(32 * EPITCH <= C::epi_wave_bytes(ELEM), "staging rows fit the wave's LDS slice");
            static_assert(WK == 1 || 32 * EPITCH <= C::XB, "staging rows fit the partner's export slice");
            // staging: with split K the partner's export slice (this wave has read it
            // into registers and nobody else touches it); otherwise a slice per wave
            char *stage = smem + (WK > 1 ? (wr * 2 + (1 - wk)) * C::XB : 2 * C::BUF_BYTES + wr * C::epi_wave_bytes(ELEM));

            const int cw0 = co0 + wco * MB * 32;                 // first channel of this wave
            const size_t tile_first = ((((size_t)tl.n * a.T + tl.t) * H + tl.h0) * W + tl.w0) * (size_t)a.Cout + cw0;
            const size_t out_total = (size_t)a.N * a.T * H * W * (size_t)a.Cout;
            const size_t left = (out_total - tile_first) * ELEM;
            const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
                static_cast<char *>(a.out) + tile_first * ELEM, 0, (int)(left < kOutside ? left : kOutside), 0x00020000);
            const uint32_t row_bytes = (uint32_t)W * (uint32_t)a.Cout * ELEM;
            typedef float f4 __attribute__((ext_vector_type(4)));
            typedef float f2 __attribute__((ext_vector_type(2)));
            typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
            // this lane's per-channel factors and biases: read from LDS once for the
            // large wave tiles (registers to spare after the K loop), else at each
            // use (small tiles keep two waves per SIMD; with the output maximum a
            // workgroup running several tiles has no registers left for them)
            constexpr bool HOIST = !ACC32 && (WK > 1 || (!OUTMAX && MB * NB >= 9));
            f4 fm[HOIST ? MB : 1][4], fb[HOIST ? MB : 1][4];
            if constexpr (HOIST) {
    #pragma unroll
                for (int mb = 0; mb < MB; ++mb)
    #pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int col = wco * MB * 32 + mb * 32 + g * 8 + lhalf * 4;
                        fm[mb][g] = *reinterpret_cast<const f4 *>(s_fac + col);
                        fb[mb][g] = *reinterpret_cast<const f4 *>(s_fac + C::BCO + col);
                    }
            }
            // block j (0 <= j < HB) of this wave's share; WKC = its K half (0 without split K)
            auto finish_block = [&](auto wkc, auto jc) {
                constexpr int WKC = decltype(wkc)::value;
                constexpr int j = decltype(jc)::value;
                // the pixel this lane holds in the MFMA layout (row lrow of the block):
                // only outputs inside the image count towards the output maximum
                bool px_in = false;
                if constexpr (OUTMAX) {
                    const int pl = (wpx * NB + WKC * HB + j) * 32 + lrow;
                    const int plr = pl / TW;
                    px_in = tl.h0 + plr < H && tl.w0 + (pl - plr * TW) < W;
                }
    #pragma unroll
                for (int mb = 0; mb < MB; ++mb)
    #pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const v16i x = __builtin_bit_cast(v16i, acc[mb][WKC * HB + j]);
                        v4i v = v4i{x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
                        f4 vf{};
                        if constexpr (BF) {
                            vf = __builtin_bit_cast(f4, v);
                            if constexpr (WK > 1) vf += __builtin_bit_cast(f4, part[(mb * HB + j) * 4 + g]);
                        } else {
                            if constexpr (WK > 1) v += part[(mb * HB + j) * 4 + g];
                        }
                        char *dst = stage + lrow * EPITCH + (mb * 32 + g * 8 + lhalf * 4) * ELEM;
                        if constexpr (ACC32) {
                            *reinterpret_cast<v4i *>(dst) = v;
                        } else {
                            f4 y;
    #pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float av = BF ? vf[e] : (float)v[e];
                                if constexpr (HOIST) {
                                    y[e] = __builtin_fmaf(av, fm[mb][g][e], fb[mb][g][e]);
                                } else {
                                    const int col = wco * MB * 32 + mb * 32 + g * 8 + lhalf * 4 + e;
                                    y[e] = __builtin_fmaf(av, s_fac[col], s_fac[C::BCO + col]);
                                }
                            }
                            const uint32_t lo =
                                __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{y[0], y[1]}, bf2));
                            const uint32_t hi =
                                __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{y[2], y[3]}, bf2));
                            *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
                            if constexpr (OUTMAX) {
                                if (px_in) ymax = pk_absmax(pk_absmax(ymax, lo), hi);
                            }
                        }
                    }
    #pragma unroll
                for (int k = 0; k < CHUNKS / 64; ++k) {
                    const int c = k * 64 + lane;
                    const int px = c / (ROWB / 16);
                    const int off = (c - px * (ROWB / 16)) * 16;
                    const v4i v = *reinterpret_cast<const v4i *>(stage + px * EPITCH + off);
                    const int p = (wpx * NB + WKC * HB + j) * 32 + px;
                    const int pr = p / TW, pc = p - pr * TW;
                    const bool inside = tl.h0 + pr < H && tl.w0 + pc < W;
                    const uint32_t o = inside ? pr * row_bytes + (uint32_t)(pc * a.Cout * ELEM + off) : kOutside;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), orsrc, (int)o, 0, kStoreNT);
                }
            };
            auto finish_all = [&](auto wkc) { static_for<HB>([&](auto jc) { finish_block(wkc, jc); }); };
            if (WK > 1 && wk == 1)
                finish_all(std::integral_constant<int, 1>{});
            else
                finish_all(std::integral_constant<int, 0>{});
        }
    };
    int gs = 0;   // stages run by this workgroup (buffer parity)
    for (;;) {
        for (int st = 0; st + 1 < cur.nst; ++st, ++gs)
            run_stage(gs & 1, wstage(cur, st + 1), halo_rsrc(cur, st + 1), std::integral_constant<int, 2>{});
        // the tile's last stage: prefetch the workgroup's next tile, if any
        if constexpr (PERSIST > 0) {
            const int ptn = pt + pstride;
            if (ptn < nptiles) {
                const Tile nxt = decode(ptn);
                set_hoff(nxt);   // this stage's halo loads are the next tile's
                run_stage(gs & 1, wstage(nxt, 0), halo_rsrc(nxt, 0), std::integral_constant<int, PERSIST>{});
                ++gs;
                epilogue(cur);
                cur = nxt;
                pt = ptn;
#pragma unroll
                for (int mb = 0; mb < MA; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NA; ++nb) acc[mb][nb] = AccV{};
                if constexpr (PERSIST == 1) {
                    wcur = wstage(cur, 0);
#pragma unroll
                    for (int e = 0; e < C::PD; ++e)
#pragma unroll
                        for (int m = 0; m < MA; ++m) wreg[e][m] = load_wf(wcur + e * 1024, m);
                }
                continue;
            }
        }
        run_stage(gs & 1, wcur, halo_rsrc(cur, cur.nst - 1), std::integral_constant<int, 0>{});
        epilogue(cur);
        break;
    }

    // the workgroup's maximum of |y| into its partial slot (the output
    // maximum the next layer's quantize pass reduces; slots 0..511, the grid
    // has at most 512 workgroups when it is asked for)
    if constexpr (OUTMAX) {
        if (a.y_absmax) {
            __shared__ uint32_t s_red[NT / 64];
            const uint32_t m = wave_max_u32(max(ymax & 0xFFFFu, ymax >> 16));
            if (lane == 0) s_red[wave] = m;
            lds_barrier();
            if (tid == 0) {
                uint32_t b = s_red[0];
                for (int k = 1; k < NT / 64; ++k) b = max(b, s_red[k]);
                a.y_absmax[blockIdx.x] = b;
            }
            if (blockIdx.x == 0)
                for (int k = gridDim.x + tid; k < kAbsmaxParts; k += NT) a.y_absmax[k] = 0;
        }
    }
}


// ---- host side ------------------------------------------------------------

// The kernel instantiation of one launch mode (the output maximum is a mode
// of its own only for the W8A8 epilogue).
template <int WCO, int WPX, int WK, int MB, int NB, int TH, int TW, int KH, int KW, int SPW>
static const void *conv_kernel(int mode, bool outmax)
{
    if (mode == kModeAcc32)
        return reinterpret_cast<const void *>(
            &k_conv_igemm<WCO, WPX, WK, MB, NB, TH, TW, KH, KW, SPW, true, false, false, false>);
    if (mode == kModeBf16)
        return reinterpret_cast<const void *>(
            &k_conv_igemm<WCO, WPX, WK, MB, NB, TH, TW, KH, KW, SPW, false, false, true, false>);
    if (mode == kModeQin)
        return reinterpret_cast<const void *>(
            &k_conv_igemm<WCO, WPX, WK, MB, NB, TH, TW, KH, KW, SPW, false, false, false, true>);
    if (outmax)
        return reinterpret_cast<const void *>(
            &k_conv_igemm<WCO, WPX, WK, MB, NB, TH, TW, KH, KW, SPW, false, true, false, false>);
    return reinterpret_cast<const void *>(
        &k_conv_igemm<WCO, WPX, WK, MB, NB, TH, TW, KH, KW, SPW, false, false, false, false>);
}

// Workgroups of one instantiation that fit on a CU at once (registers, LDS,
// waves), asked of the runtime once per instantiation and device (the
// answer depends on the device's resources).
template <int WCO, int WPX, int WK, int MB, int NB, int TH, int TW, int KH, int KW, int SPW>
static int resident_per_cu(int mode, bool outmax)
{
    using C = ConvCfg<WCO, WPX, WK, MB, NB, TH, TW, KH, KW, SPW>;
    static std::atomic<int> occ[kMaxDevices][5];   // 0 = not yet queried
    const int v = (mode == kModePlain && outmax) ? 4 : mode;
    const int dev = current_device();
    const bool slot = dev >= 0 && dev < kMaxDevices;
    if (slot) {
        const int o = occ[dev][v].load(std::memory_order_relaxed);
        if (o > 0) return o;
    }
    int n = 0;
    const void *f = conv_kernel<WCO, WPX, WK, MB, NB, TH, TW, KH, KW, SPW>(mode, outmax);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, C::NT, 0) != hipSuccess || n < 1) n = 1;
    if (slot) occ[dev][v].store(n, std::memory_order_relaxed);
    return n;
}

template <int WCO, int WPX, int WK, int MB, int NB, int TH, int TW, int KH, int KW, int SPW>
static int launch_cfg(const ConvArgs &base, int mode, hipStream_t st)
{
    using C = ConvCfg<WCO, WPX, WK, MB, NB, TH, TW, KH, KW, SPW>;
    ConvArgs a = base;
    if ((a.Cin / 32) % C::SL != 0) return QVAE_EUNSUPPORTED;   // (the dispatcher never asks)
    a.tiles_w = (a.W + TW - 1) / TW;
    a.tiles_h = (a.H + TH - 1) / TH;
    a.co_tiles = a.Cout / C::BCO;
    const int64_t nptiles = (int64_t)a.tiles_w * a.tiles_h * a.T * a.N;
    if (nptiles * a.co_tiles > 0x7FFFFFFF) return QVAE_EUNSUPPORTED;
    const bool outmax = a.y_absmax != nullptr;
    int64_t grid = nptiles * a.co_tiles;
    if (WK == 1) {
        // more tiles than resident workgroups: each workgroup runs several
        // tiles in a row (the grid stays a multiple of the channel tiles)
        const int64_t per = (int64_t)device_cus() *
                            resident_per_cu<WCO, WPX, WK, MB, NB, TH, TW, KH, KW, SPW>(mode, outmax) / a.co_tiles;
        if (per >= 1 && nptiles > per) grid = per * a.co_tiles;
        // one partial slot per workgroup for the output maximum
        if (outmax && grid > kAbsmaxParts) grid = (kAbsmaxParts / a.co_tiles) * a.co_tiles;
    }
    if (outmax && (grid > kAbsmaxParts || grid < 1)) return QVAE_EUNSUPPORTED;
    const void *f = conv_kernel<WCO, WPX, WK, MB, NB, TH, TW, KH, KW, SPW>(mode, outmax);
    void *args[] = {&a};
    (void)hipLaunchKernel(f, dim3((unsigned)grid), dim3(C::NT), args, 0, st);   // a failure is reported below
    return launch_status();
}

static int64_t px_tiles(const ConvArgs &a, int th, int tw)
{
    return (int64_t)((a.H + th - 1) / th) * ((a.W + tw - 1) / tw) * a.T * a.N;
}

// Tile choice: the largest per-wave tile (3 x 4 blocks of 32x32 = 96 channels
// x 128 pixels) whenever the channel count allows; split K inside the
// workgroup when there are too few pixel tiles to give every CU a
// workgroup, but only while the split-K workgroups fit in one round of
// resident workgroups (a second round would pay the fixed prologue and
// epilogue again, and the full-K tiles then finish in one round anyway).
// For 384 channels with full K, 6x16-pixel tiles (3 x 3 blocks per wave)
// replace the 8x16 ones when fewer rounds of smaller tiles finish sooner
// (384 @105x157: 140 tiles of 8x16 leave 116 CUs idle, 180 of 6x16 fewer).
// 1x1 kernels stage two slices per wave per stage when the slice count allows
// it, so a stage still holds more than one k-step.
template <int KH, int KW, int SPW>
static int launch_spatial(const ConvArgs &a, int mode, hipStream_t st)
{
    const int64_t cus = device_cus();
    const int S = a.Cin / 32;
    const bool k2 = S % (2 * SPW) == 0;   // the K range splits into two equal halves
    const bool outmax = a.y_absmax != nullptr;
    if (a.Cout % 96 == 0) {
        if (a.Cout % 384 == 0) {
            const int64_t full = px_tiles(a, 8, 16) * (a.Cout / 384);
            const int64_t split = px_tiles(a, 8, 16) * (a.Cout / 192);
            if (full >= cus || !k2 ||
                split > cus * resident_per_cu<2, 1, 2, 3, 4, 8, 16, KH, KW, SPW>(mode, outmax)) {
                if constexpr (KH * KW > 1) {
                    // 6x16 tiles (96 x 96 per wave) when they finish sooner: rounds of
                    // resident workgroups times the tile's pixels, the smaller tile
                    // taken as 8 % less efficient per pixel (less operand reuse)
                    const int64_t t6 = px_tiles(a, 6, 16) * (a.Cout / 384);
                    const int64_t s8 = cus * resident_per_cu<4, 1, 1, 3, 4, 8, 16, KH, KW, SPW>(mode, outmax);
                    const int64_t s6 = cus * resident_per_cu<4, 1, 1, 3, 3, 6, 16, KH, KW, SPW>(mode, outmax);
                    const int64_t r8 = (full + s8 - 1) / s8, r6 = (t6 + s6 - 1) / s6;
                    if (r6 * 96 * 108 < r8 * 128 * 100) return launch_cfg<4, 1, 1, 3, 3, 6, 16, KH, KW, SPW>(a, mode, st);
                }
                return launch_cfg<4, 1, 1, 3, 4, 8, 16, KH, KW, SPW>(a, mode, st);
            }
        }
        if (a.Cout % 192 == 0) {
            const int64_t full = px_tiles(a, 16, 16) * (a.Cout / 192);
            const int64_t split = px_tiles(a, 8, 16) * (a.Cout / 192);
            if (full >= cus || !k2 ||
                split > cus * resident_per_cu<2, 1, 2, 3, 4, 8, 16, KH, KW, SPW>(mode, outmax))
                return launch_cfg<2, 2, 1, 3, 4, 16, 16, KH, KW, SPW>(a, mode, st);
            return launch_cfg<2, 1, 2, 3, 4, 8, 16, KH, KW, SPW>(a, mode, st);
        }
        const int64_t full = px_tiles(a, 16, 16) * (a.Cout / 96);
        const bool split_fits =
            k2 && px_tiles(a, 8, 16) * (a.Cout / 96) <= cus * resident_per_cu<1, 1, 2, 3, 4, 8, 16, KH, KW, SPW>(mode, outmax);
        if constexpr (KH * KW > 1) {
            // 96 channels: memory-bound; 96x64 wave tiles keep two workgroups
            // per CU so one's loads and stores overlap the other's MFMAs.  The
            // bf16 conv (twice the operand bytes per MFMA) does better with
            // 96x128 wave tiles, which halve the weight loads per pixel, once the
            // frame has a tile for every CU.
            if (mode == kModeBf16 && full >= cus) return launch_cfg<1, 2, 1, 3, 4, 16, 16, KH, KW, SPW>(a, mode, st);
            if (full >= cus || !split_fits) return launch_cfg<1, 4, 1, 3, 2, 16, 16, KH, KW, SPW>(a, mode, st);
        } else {
            if (full >= cus || !split_fits) return launch_cfg<1, 2, 1, 3, 4, 16, 16, KH, KW, SPW>(a, mode, st);
        }
        return launch_cfg<1, 1, 2, 3, 4, 8, 16, KH, KW, SPW>(a, mode, st);
    }
    return launch_cfg<1, 2, 1, 1, 4, 16, 16, KH, KW, SPW>(a, mode, st);
}

// Shape checks shared by both operand types; cin_bytes = bytes per input
// pixel (Cin for int8, 2 Cin for bf16), out_elem = bytes per output value.
static int conv_validate(const void *x, const void *w, const void *out, int N, int T, int H, int W, int Cin,
                         int Cout, int kt, int kh, int kw, const void *cache, int64_t cin_bytes, int out_elem)
{
    if (!x || !w || !out) return QVAE_EINVAL;
    if (N <= 0 || T <= 0 || H <= 0 || W <= 0 || Cin <= 0 || Cout <= 0 || kt <= 0 || kh <= 0 || kw <= 0)
        return QVAE_EINVAL;
    if (!aligned16(x) || !aligned16(w) || !aligned16(out) || (cache && !aligned16(cache))) return QVAE_EINVAL;
    if (cin_bytes % 32 != 0 || Cout % 32 != 0) return QVAE_EUNSUPPORTED;
    if (kt != 1 && kt != 3) return QVAE_EUNSUPPORTED;
    if (!((kh == 1 && kw == 1) || (kh == 3 && kw == 3))) return QVAE_EUNSUPPORTED;
    // byte offsets inside one frame are 32-bit
    if ((int64_t)H * W * cin_bytes >= ((int64_t)1 << 31)) return QVAE_EUNSUPPORTED;
    // output byte offsets inside one pixel tile (at most 32 rows) are 32-bit
    if ((int64_t)32 * W * Cout * out_elem >= ((int64_t)1 << 31)) return QVAE_EUNSUPPORTED;
    return QVAE_OK;
}

static int conv_validate_w8a8(const int8_t *xq, const int8_t *wq, const void *out, int N, int T, int H, int W,
                              int Cin, int Cout, int kt, int kh, int kw, const int8_t *cache)
{
    int rc = conv_validate(xq, wq, out, N, T, H, W, Cin, Cout, kt, kh, kw, cache, Cin, 4);
    if (rc != QVAE_OK) return rc;
    // |acc| <= 127^2 * K must stay inside int32
    const int64_t K = (int64_t)Cin * kt * kh * kw;
    if (K * 127 * 127 >= ((int64_t)1 << 31)) return QVAE_EUNSUPPORTED;
    return QVAE_OK;
}

static int conv_dispatch(const ConvArgs &a, int kh, int mode, hipStream_t st)
{
    // two 32-byte slices per wave and stage when the slice count is even:
    // half the stages (barriers) and 64 contiguous bytes per halo pixel load
    if (kh == 3 && (a.Cin / 32) % 2 == 0) return launch_spatial<3, 3, 2>(a, mode, st);
    if (kh == 3) return launch_spatial<3, 3, 1>(a, mode, st);
    if ((a.Cin / 32) % 2 == 0) return launch_spatial<1, 1, 2>(a, mode, st);
    return launch_spatial<1, 1, 1>(a, mode, st);
}

// (the plain W8A8 instantiation of the 384-channel tile: any kernel of this
// file makes the runtime load the file's whole code object)
int preload_conv()
{
    hipFuncAttributes attr;
    const void *f = conv_kernel<4, 1, 1, 3, 4, 8, 16, 3, 3, 2>(kModePlain, false);
    return hipFuncGetAttributes(&attr, f) == hipSuccess ? QVAE_OK : QVAE_ELAUNCH;
}

}  // namespace qvae

using namespace qvae;

extern "C" int qvae_causalconv3d_w8a8(const int8_t *xq, const float *x_scale, const int8_t *cache,
                                      const int8_t *wq, const float *w_scale, const float *bias, int N,
                                      int T, int H, int W, int Cin, int Cout, int kt, int kh, int kw,
                                      uint16_t *y, void *stream)
{
    if (force_fail(true)) return QVAE_EFORCED;
    if (!x_scale || !w_scale) return QVAE_EINVAL;
    int rc = conv_validate_w8a8(xq, wq, y, N, T, H, W, Cin, Cout, kt, kh, kw, cache);
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
    return conv_dispatch(a, kh, kModePlain, as_stream(stream));
}

extern "C" int qvae_causalconv3d_w8a8_absmax(const int8_t *xq, const float *x_scale, const int8_t *cache,
                                             const int8_t *wq, const float *w_scale, const float *bias, int N,
                                             int T, int H, int W, int Cin, int Cout, int kt, int kh, int kw,
                                             uint16_t *y, uint32_t *y_absmax, void *stream)
{
    if (force_fail(true)) return QVAE_EFORCED;
    if (!x_scale || !w_scale || !y_absmax) return QVAE_EINVAL;
    int rc = conv_validate_w8a8(xq, wq, y, N, T, H, W, Cin, Cout, kt, kh, kw, cache);
    if (rc != QVAE_OK) return rc;
    ConvArgs a{};
    a.xq = xq;
    a.cache = (kt > 1) ? cache : nullptr;
    a.wq = wq;
    a.x_scale = x_scale;
    a.w_scale = w_scale;
    a.bias = bias;
    a.out = y;
    a.y_absmax = y_absmax + 1;
    a.N = N, a.T = T, a.H = H, a.W = W, a.Cin = Cin, a.Cout = Cout, a.kt = kt;
    return conv_dispatch(a, kh, kModePlain, as_stream(stream));
}

extern "C" int qvae_causalconv3d_w8a8_acc32(const int8_t *xq, const int8_t *cache, const int8_t *wq, int N,
                                            int T, int H, int W, int Cin, int Cout, int kt, int kh, int kw,
                                            int32_t *acc, void *stream)
{
    if (force_fail(true)) return QVAE_EFORCED;
    int rc = conv_validate_w8a8(xq, wq, acc, N, T, H, W, Cin, Cout, kt, kh, kw, cache);
    if (rc != QVAE_OK) return rc;
    ConvArgs a{};
    a.xq = xq;
    a.cache = (kt > 1) ? cache : nullptr;
    a.wq = wq;
    a.out = acc;
    a.N = N, a.T = T, a.H = H, a.W = W, a.Cin = Cin, a.Cout = Cout, a.kt = kt;
    return conv_dispatch(a, kh, kModeAcc32, as_stream(stream));
}

extern "C" int qvae_causalconv3d_bf16(const uint16_t *x, const uint16_t *cache, const uint16_t *wp,
                                      const float *bias, int N, int T, int H, int W, int Cin, int Cout, int kt,
                                      int kh, int kw, uint16_t *y, void *stream)
{
    if (force_fail(false)) return QVAE_EFORCED;
    int rc = conv_validate(x, wp, y, N, T, H, W, Cin, Cout, kt, kh, kw, cache, 2 * (int64_t)Cin, 2);
    if (rc != QVAE_OK) return rc;
    ConvArgs a{};
    a.xq = reinterpret_cast<const int8_t *>(x);
    a.cache = (kt > 1) ? reinterpret_cast<const int8_t *>(cache) : nullptr;
    a.wq = reinterpret_cast<const int8_t *>(wp);
    a.bias = bias;
    a.out = y;
    a.N = N, a.T = T, a.H = H, a.W = W, a.Cin = 2 * Cin, a.Cout = Cout, a.kt = kt;
    return conv_dispatch(a, kh, kModeBf16, as_stream(stream));
}

extern "C" int qvae_causalconv3d_w8a8_qin(const uint16_t *x, const uint16_t *cache, uint32_t *x_absmax,
                                          float clip_ratio, const int8_t *wq, const float *w_scale,
                                          const float *bias, int N, int T, int H, int W, int Cin, int Cout, int kt,
                                          int kh, int kw, float *x_scale, uint16_t *y, void *stream)
{
    if (force_fail(true)) return QVAE_EFORCED;
    if (!x_absmax || !w_scale) return QVAE_EINVAL;
    if (!(clip_ratio > 0.0f)) return QVAE_EINVAL;
    if (clip_ratio > 1.0f) return QVAE_EUNSUPPORTED;
    int rc = conv_validate(x, wq, y, N, T, H, W, Cin, Cout, kt, kh, kw, cache, 2 * (int64_t)Cin, 4);
    if (rc != QVAE_OK) return rc;
    if (Cin % 32 != 0) return QVAE_EUNSUPPORTED;
    const int64_t K = (int64_t)Cin * kt * kh * kw;
    if (K * 127 * 127 >= ((int64_t)1 << 31)) return QVAE_EUNSUPPORTED;
    ConvArgs a{};
    a.xq = reinterpret_cast<const int8_t *>(x);
    a.cache = (kt > 1) ? reinterpret_cast<const int8_t *>(cache) : nullptr;
    a.wq = wq;
    a.w_scale = w_scale;
    a.bias = bias;
    a.out = y;
    a.x_absmax = x_absmax;
    a.x_scale_out = x_scale;
    a.clip = clip_ratio;
    a.N = N, a.T = T, a.H = H, a.W = W, a.Cin = Cin, a.Cout = Cout, a.kt = kt;
    return conv_dispatch(a, kh, kModeQin, as_stream(stream));
}
