// qvae_act.hip -- dynamic per-tensor INT8 activation quantization on gfx950.
//
// Scheme (page "ComfyUI-Qwen-VAE-Triton v0.2.0", section "Three presets
// explained"): activations are dynamically, symmetrically quantized to INT8
// with clip ratio 1.0.  One scale per tensor: s = fl(clip * absmax) / 127 and
// q = clamp(rne(x / s), -127, 127).  Any clip ratio in (0, 1] is accepted;
// below 1 the clamp is what maps the clipped outliers to +-127.
//
// Two HBM-bound passes.  The scale is a grid-wide dependency, so the max is
// reduced first (pass 1) and every quantize workgroup derives the same scale
// from the reduced maxima (pass 2); the scale never visits the host.
//
//   pass 1  k_absmax    16-byte loads of bf16, integer max of |x| bit patterns
//                       (for finite bf16, |a| < |b| iff (a & 0x7FFF) <
//                       (b & 0x7FFF) as integers), packed 2x16-bit max, DPP
//                       wave reduction, LDS workgroup reduction; each
//                       workgroup writes its own partial maximum (no atomics:
//                       hundreds of same-address atomics serialize in L2 and
//                       cost more than the whole pass).
//   pass 2  k_quantize  every workgroup reduces the 512 partial slots (2 KB
//                       from L2; slots no producer owns are 0), derives s, and quantizes: 16 bytes of bf16 in,
//                       8 int8 codes out per lane and load, four loads in
//                       flight.  Workgroup 0 publishes the maximum and the
//                       scale.
//
// The codes come from quant8 (qvae_internal.h): a multiply by fl(1/s) where
// that provably rounds like the IEEE binary32 quotient x / s, the correctly
// rounded division otherwise.  The conv that quantizes its own bf16 input uses
// the same routine, so the two produce the same codes.
#include "qvae_internal.h"

namespace qvae {

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

constexpr int kAbsmaxThreads = 256;
constexpr int kAbsmaxUnroll = 8;   // 16-byte loads in flight per lane
static_assert(kAbsmaxParts == QVAE_ABSMAX_WORDS - 1, "one word for the maximum, the rest partials");

// Number of workgroups (= partial maxima) of the absmax pass for numel.
static int absmax_blocks(int64_t numel)
{
    // at least one 16-byte vector per lane, all CUs busy for mid-sized tensors
    const int64_t n16 = numel / 8;
    int64_t want = (n16 + kAbsmaxThreads - 1) / kAbsmaxThreads;
    if (want < 1) want = 1;
    if (want > kAbsmaxParts) want = kAbsmaxParts;
    return (int)want;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t m, uint32_t *part /* [blockDim/64] LDS */)
{
    m = wave_max_u32(m);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) part[wave] = m;
    lds_barrier();   // (LDS only: global loads in flight need not land first)
    uint32_t b = part[0];
    for (int k = 1; k < (int)(blockDim.x >> 6); ++k) b = max(b, part[k]);
    return b;
}

__global__ __launch_bounds__(kAbsmaxThreads) void k_absmax(const u32x4 *__restrict__ x16, int64_t n16,
                                                          const uint16_t *__restrict__ tail, int ntail,
                                                          uint32_t *__restrict__ partials)
{
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * kAbsmaxThreads;
    int64_t i = (int64_t)blockIdx.x * kAbsmaxThreads + threadIdx.x;
    // every pass issues all of its (in-range) loads before it uses any, the
    // last, partial pass included: one memory round trip per pass
    for (; i < n16; i += kAbsmaxUnroll * stride) {
        u32x4 v[kAbsmaxUnroll];
#pragma unroll
        for (int u = 0; u < kAbsmaxUnroll; ++u)
            v[u] = (i + u * stride < n16) ? __builtin_nontemporal_load(&x16[i + u * stride]) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < kAbsmaxUnroll; ++u) {
            m = pk_absmax(m, v[u].x);
            m = pk_absmax(m, v[u].y);
            m = pk_absmax(m, v[u].z);
            m = pk_absmax(m, v[u].w);
        }
    }
    if (blockIdx.x == 0 && (int)threadIdx.x < ntail) m = pk_absmax(m, tail[threadIdx.x]);
    m = max(m & 0xFFFFu, m >> 16);
    __shared__ uint32_t part[kAbsmaxThreads / 64];
    const uint32_t b = block_max_u32(m, part);
    if (threadIdx.x == 0) partials[blockIdx.x] = b;
    // every partial slot holds a valid maximum: the ones no workgroup owns are 0
    if (blockIdx.x == 0)
        for (int k = gridDim.x + threadIdx.x; k < kAbsmaxParts; k += kAbsmaxThreads) partials[k] = 0;
}

// 8 codes.  NT: non-temporal (the pass alone runs 2-10 % faster that way);
// otherwise the default policy, which leaves the codes in the last-level cache
// for the conv that reads them next (see kCachedCodesMin).
template <bool NT>
__device__ __forceinline__ void store_codes(uint2 *dst, uint2 v)
{
    typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
    if constexpr (NT)
        __builtin_nontemporal_store(u32x2_t{v.x, v.y}, reinterpret_cast<u32x2_t *>(dst));
    else
        *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{v.x, v.y};
}

constexpr int kQuantThreads = 256;
constexpr int kQuantUnroll = 4;   // 16-byte loads in flight per lane

// From this many elements on, the codes are stored with the default cache
// policy: the consumer's reads then hit the last-level cache, which outweighs
// the slower pass (measured with the codes' consumer, the conv, right after:
// layer steps at 25, 50 and 100 M elements 1, 4 and 8 % faster, the chunked
// decode step at 44 M ~2 % faster; at 6.3 M elements the step is ~2.5 % faster
// with non-temporal stores, so smaller tensors keep them).
constexpr int64_t kCachedCodesMin = 16 << 20;

// Each lane: 8 bf16 per 16-byte load -> 8 codes per 8-byte store; a wave's
// load instruction covers 1 KB of contiguous input.
template <bool NT>
__global__ __launch_bounds__(kQuantThreads) void k_quantize(const u32x4 *__restrict__ x16,
                                                           int64_t n16,   // groups of 8 elements
                                                           const uint16_t *__restrict__ x,
                                                           int64_t numel,
                                                           float clip_ratio,
                                                           uint32_t *__restrict__ absmax,
                                                           float *__restrict__ x_scale,
                                                           uint2 *__restrict__ q8,
                                                           int8_t *__restrict__ q)
{
    const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
    int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    // The partial maxima (written by the absmax pass, or by the producing
    // convolution's epilogue; unused slots are 0) are loaded first, then the
    // first unrolled pass over x.  Every wave reduces all partials itself (no
    // workgroup barrier, whose fence would wait for the x loads too), so the
    // reduction waits only for the partials (loads complete in order) and x's
    // HBM latency overlaps it (at small sizes the grid covers the tensor in
    // this one pass).
    static_assert(kAbsmaxParts % 64 == 0, "whole partial slots per lane");
    const int lane = threadIdx.x & 63;
    uint32_t pv[kAbsmaxParts / 64];
#pragma unroll
    for (int k = 0; k < kAbsmaxParts / 64; ++k) pv[k] = absmax[1 + lane + k * 64];
    const int64_t i0 = i;
    // (raw buffer loads: a group past the end reads as zero, so no lane
    // branches and the wait for the partials can leave these in flight; the
    // first pass's offsets are below 4 x 2048 x 256 x 16 bytes)
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4 *>(x16), 0, (int)(n16 * 16 < 0x7FFFFFF0 ? n16 * 16 : 0x7FFFFFF0), 0x00020000);
    u32x4 v0[kQuantUnroll];
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u)
        v0[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (int)((i + u * stride) * 16), 0, 2));
    uint32_t mp = 0;
#pragma unroll
    for (int k = 0; k < kAbsmaxParts / 64; ++k) mp = max(mp, pv[k]);
    const uint32_t mbits = wave_max_u32(mp);
    const float a = bf16_bits_to_float(mbits);
    const float s = (clip_ratio * a) / 127.0f;
    const float r = 1.0f / s;
    const bool zero = !(s > 0.0f);
    const bool exact_only = !(r < __builtin_inff());
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        absmax[0] = mbits;
        *x_scale = s;
    }

    if (zero) {
        for (i = i0; i < n16; i += stride) q8[i] = make_uint2(0u, 0u);
    } else {
        // as in the absmax pass, every pass (the last, partial one included)
        // issues all its loads before its first store
#pragma unroll
        for (int u = 0; u < kQuantUnroll; ++u)
            if (i + u * stride < n16) store_codes<NT>(&q8[i + u * stride], quant8(v0[u], s, r, exact_only));
        for (i += kQuantUnroll * stride; i < n16; i += kQuantUnroll * stride) {
            u32x4 v[kQuantUnroll];
#pragma unroll
            for (int u = 0; u < kQuantUnroll; ++u)
                v[u] = (i + u * stride < n16) ? __builtin_nontemporal_load(&x16[i + u * stride]) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < kQuantUnroll; ++u)
                if (i + u * stride < n16) store_codes<NT>(&q8[i + u * stride], quant8(v[u], s, r, exact_only));
        }
    }
    // the last numel % 8 elements, one per lane of workgroup 0
    if (blockIdx.x == 0) {
        const int64_t e = n16 * 8 + threadIdx.x;
        if (e < numel) q[e] = zero ? 0 : (int8_t)quant_code_exact(bf16_bits_to_float(x[e]), s);
    }
}


// ---- the allocation-free entry point's scratch ------------------------------
// qvae_act_absmax_quant_noalloc keeps its activation-maximum words (the same
// QVAE_ABSMAX_WORDS words a caller's workspace holds for
// qvae_act_absmax_quant) in this file-scope device array.  Every GPU the
// library runs on holds its own copy, at its own address, until the process
// ends.  On the host the name only stands in for the symbol; kernels get the
// device address that hipGetSymbolAddress returns for the current device,
// looked up once per device and kept here.  Nothing needs clearing between
// calls: the absmax pass writes all of the partial words (0 where it has
// nothing) and the quantize pass writes word 0.
static __device__ __align__(256) uint32_t scratch[QVAE_ABSMAX_WORDS];

static std::atomic<uint32_t *> g_scratch[kMaxDevices];   // per device id; nullptr = not looked up yet

// The current device's copy of scratch, or nullptr if the runtime cannot give it.
static uint32_t *scratch_on_device()
{
    const int dev = current_device();
    const bool slot = dev >= 0 && dev < kMaxDevices;
    if (slot) {
        uint32_t *p = g_scratch[dev].load(std::memory_order_acquire);
        if (p) return p;
    }
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (slot) g_scratch[dev].store(static_cast<uint32_t *>(p), std::memory_order_release);
    return static_cast<uint32_t *>(p);
}

int setup_scratch() { return scratch_on_device() ? QVAE_OK : QVAE_ELAUNCH; }

int preload_act()
{
    hipFuncAttributes attr;
    return hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(&k_absmax)) == hipSuccess ? QVAE_OK
                                                                                                   : QVAE_ELAUNCH;
}

}  // namespace qvae

using namespace qvae;

extern "C" int qvae_act_absmax(const uint16_t *x, int64_t numel, uint32_t *absmax, void *stream)
{
    if (force_fail(true)) return QVAE_EFORCED;
    if (!x || !absmax || numel <= 0) return QVAE_EINVAL;
    if (!aligned16(x)) return QVAE_EINVAL;
    const int64_t n16 = numel / 8;
    const int ntail = (int)(numel - n16 * 8);
    hipLaunchKernelGGL(k_absmax, dim3(absmax_blocks(numel)), dim3(kAbsmaxThreads), 0, as_stream(stream),
                       reinterpret_cast<const u32x4 *>(x), n16, x + n16 * 8, ntail, absmax + 1);
    return launch_status();
}

extern "C" int qvae_act_quantize(const uint16_t *x, int64_t numel, float clip_ratio, uint32_t *absmax,
                                 float *x_scale, int8_t *xq, void *stream)
{
    if (force_fail(true)) return QVAE_EFORCED;
    if (!x || !absmax || !x_scale || !xq || numel <= 0) return QVAE_EINVAL;
    if (!aligned16(x) || !aligned16(xq)) return QVAE_EINVAL;
    if (!(clip_ratio > 0.0f)) return QVAE_EINVAL;         // zero, negative or NaN
    if (clip_ratio > 1.0f) return QVAE_EUNSUPPORTED;
    const int64_t n16 = numel / 8;
    // enough workgroups for every lane to have kQuantUnroll loads in flight,
    // at most 8 per CU (one grid-stride sweep of the tensor per unrolled pass)
    int64_t want = (n16 + (int64_t)kQuantThreads * kQuantUnroll - 1) / ((int64_t)kQuantThreads * kQuantUnroll);
    const int64_t cap = (int64_t)device_cus() * 8;
    const int blocks = (int)(want < 1 ? 1 : (want > cap ? cap : want));
    hipLaunchKernelGGL(numel >= kCachedCodesMin ? k_quantize<false> : k_quantize<true>, dim3(blocks),
                       dim3(kQuantThreads), 0, as_stream(stream),
                       reinterpret_cast<const u32x4 *>(x), n16, x, numel, clip_ratio, absmax, x_scale,
                       reinterpret_cast<uint2 *>(xq), xq);
    return launch_status();
}

extern "C" int qvae_act_absmax_quant(const uint16_t *x, int64_t numel, float clip_ratio, uint32_t *absmax,
                                     float *x_scale, int8_t *xq, void *stream)
{
    if (force_fail(true)) return QVAE_EFORCED;
    if (!x || !absmax || !x_scale || !xq || numel <= 0) return QVAE_EINVAL;
    if (!aligned16(x) || !aligned16(xq)) return QVAE_EINVAL;
    if (!(clip_ratio > 0.0f)) return QVAE_EINVAL;         // zero, negative or NaN
    if (clip_ratio > 1.0f) return QVAE_EUNSUPPORTED;
    int rc = qvae_act_absmax(x, numel, absmax, stream);
    if (rc != QVAE_OK) return rc;
    return qvae_act_quantize(x, numel, clip_ratio, absmax, x_scale, xq, stream);
}

extern "C" int qvae_act_absmax_quant_noalloc(const uint16_t *x, int64_t numel, float clip_ratio, float *x_scale,
                                             int8_t *xq, void *stream)
{
    if (force_fail(true)) return QVAE_EFORCED;
    if (!x || !x_scale || !xq || numel <= 0) return QVAE_EINVAL;
    if (!aligned16(x) || !aligned16(xq)) return QVAE_EINVAL;
    if (!(clip_ratio > 0.0f)) return QVAE_EINVAL;         // zero, negative or NaN
    if (clip_ratio > 1.0f) return QVAE_EUNSUPPORTED;
    uint32_t *ws = scratch_on_device();
    if (!ws) return QVAE_ELAUNCH;
    return qvae_act_absmax_quant(x, numel, clip_ratio, ws, x_scale, xq, stream);
}
