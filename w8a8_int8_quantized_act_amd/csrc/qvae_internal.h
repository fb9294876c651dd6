// qvae_internal.h -- helpers shared by the HIP sources of libqvae (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <atomic>
#include <stdlib.h>

#include "qvae.h"

namespace qvae {

// Every entry point starts with this: the fallback test hook.
// QVAE_FORCE_FAIL=1 fails every call; QVAE_FORCE_FAIL=w8a8 fails only the
// W8A8 calls (quantizers and the INT8 conv), so a caller's per-layer fallback
// to the native-precision conv runs instead.
inline bool force_fail(bool w8a8)
{
    const char *v = getenv("QVAE_FORCE_FAIL");
    if (!v) return false;
    if (v[0] == '1' && v[1] == 0) return true;
    return w8a8 && v[0] == 'w' && v[1] == '8' && v[2] == 'a' && v[3] == '8' && v[4] == 0;
}

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Map the state after a launch to a status code (never throws or aborts).
inline int launch_status()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? QVAE_OK : QVAE_ELAUNCH;
}

// Per-device caches: one slot per device id below kMaxDevices (larger ids are
// queried on every call).  Slots are atomics, so concurrent first calls on
// different threads each store the same value without a data race.
constexpr int kMaxDevices = 64;

// The current device's id, or -1 if the runtime cannot say.
inline int current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    return dev;
}

// Compute units of the current device (queried once per device; 256 on MI355X).
inline int device_cus()
{
    static std::atomic<int> cache[kMaxDevices];   // 0 = not yet queried
    const int dev = current_device();
    const bool slot = dev >= 0 && dev < kMaxDevices;
    if (slot) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int n = 0;
    if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (slot) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Load this translation unit's GPU code for the current device now instead of
// at its first launch (each source file's kernels form a code object of its
// own); QVAE_OK or QVAE_ELAUNCH.  Used by qvae_init.
int preload_act();
int preload_wquant();
int preload_conv();
int preload_norm();
// Look up the current device's copy of the allocation-free entry point's
// scratch array (qvae_act.hip); QVAE_OK or QVAE_ELAUNCH.  Used by qvae_init.
int setup_scratch();

// ---- device helpers -------------------------------------------------------

// bf16 bit pattern -> float (exact widening).
__device__ __forceinline__ float bf16_bits_to_float(uint32_t h)
{
    return __uint_as_float(h << 16);
}

// float -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global load of the wave (vmcnt(0)), which would drain the
// weight prefetches in flight; the K loop only communicates through LDS.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Maximum of an unsigned value over the 64 lanes of a wavefront: DPP
// exchanges inside each row of 16 lanes, then the four row results are read
// with readlane.  Every lane returns the wave maximum.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// Packed 2x16-bit unsigned max of the magnitudes held in one 32-bit word
// (two bf16 bit patterns: for finite bf16, |a| < |b| iff (a & 0x7FFF) <
// (b & 0x7FFF) as integers).
__device__ __forceinline__ uint32_t pk_absmax(uint32_t acc, uint32_t w)
{
    typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
    const ushort2_t a = __builtin_bit_cast(ushort2_t, acc);
    const ushort2_t b = __builtin_bit_cast(ushort2_t, w & 0x7FFF7FFFu);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

// ---- the activation quantizer's codes (shared by the quantize pass and the
// conv that quantizes its own bf16 input) ------------------------------------
//
// The quotient x / s is the IEEE binary32 one.  The fast path computes
// t = x * r with r = fl(1 / s) and keeps rne(t) when t is far from a rounding
// boundary: |fl(x*r) - x/s| <= |x/s| * (2^-23 + 2^-46) and
// |fl(x/s) - x/s| <= |x/s| * 2^-24, so when t is more than |t| * 2^-20 away from
// every half-integer, t and fl(x/s) round to the same integer.  Otherwise (and
// whenever 1/s is not finite) the group is redone with the correctly rounded
// division.  A scale of 0 is the caller's case (every code 0).

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One activation code by the definition: clamp(rne(fl(x / s)), -127, 127).
__device__ __forceinline__ int quant_code_exact(float x, float s)
{
    const float n = __builtin_rintf(x / s);
    return (int)fminf(fmaxf(n, -127.0f), 127.0f);
}

// Fast path for 8 bf16 values (one 16-byte load) -> 8 codes (two words).
//   t  = med3(x * r, -127, 127)     clamping first is exact: the code of any
//                                   |x/s| >= 127 is +-127 either way, and a
//                                   clamped t sits 0.5 from every boundary
//   m  = t + 1.5 * 2^23             rounds t to an integer (round to nearest
//                                   even); the low byte of m's bits is the
//                                   two's-complement code
//   d  = |t - (m - 1.5 * 2^23)| - 0.5   minus the distance to the nearest half-integer
//   f  = |d| - |t| * 2^-20           negative when t is too close to a rounding
//                                   boundary for fl(x * r) to stand in for fl(x / s)
// The smallest f of the 8 values is returned in fmin; the caller redoes the
// whole group exactly when it is not positive.
__device__ __forceinline__ uint2 quant8_fast(u32x4 v, float r, float &fmin)
{
    constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23
    uint32_t code[8];
    float f = 1.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t w = v[k >> 1];
        const float x = __builtin_bit_cast(float, (k & 1) ? (w & 0xFFFF0000u) : (w << 16));
        const float t = __builtin_amdgcn_fmed3f(x * r, -127.0f, 127.0f);
        const float m = t + kMagic;
        const float d = fabsf(t - (m - kMagic)) - 0.5f;
        f = fminf(f, __builtin_fmaf(fabsf(t), -0x1p-20f, fabsf(d)));
        code[k] = __builtin_bit_cast(uint32_t, m);
    }
    fmin = f;
    // byte 0 of each word -> packed: sel 0x00/0x04 pick byte 0 of the second/first operand, 0x0C gives zero
    const uint32_t lo01 = __builtin_amdgcn_perm(code[1], code[0], 0x0C0C0400u);
    const uint32_t lo23 = __builtin_amdgcn_perm(code[3], code[2], 0x0C0C0400u);
    const uint32_t hi01 = __builtin_amdgcn_perm(code[5], code[4], 0x0C0C0400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(code[7], code[6], 0x0C0C0400u);
    return make_uint2(__builtin_amdgcn_perm(lo23, lo01, 0x05040100u), __builtin_amdgcn_perm(hi23, hi01, 0x05040100u));
}

__device__ __forceinline__ uint2 quant8_exact(u32x4 v, float s)
{
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t w = v[k >> 1];
        const float x = __builtin_bit_cast(float, (k & 1) ? (w & 0xFFFF0000u) : (w << 16));
        o[k >> 2] |= (uint32_t)(quant_code_exact(x, s) & 0xFF) << (8 * (k & 3));
    }
    return make_uint2(o[0], o[1]);
}

__device__ __forceinline__ uint2 quant8(u32x4 v, float s, float r, bool exact_only)
{
    float fmin;
    uint2 o = quant8_fast(v, r, fmin);
    if (exact_only || !(fmin > 0.0f)) o = quant8_exact(v, s);
    return o;
}

// Partial-maximum slots of an activation-maximum buffer (words 1.. of the
// QVAE_ABSMAX_WORDS words): every producer writes all of them, 0 where it
// has nothing, and the quantize pass reduces all of them.
constexpr int kAbsmaxParts = 512;

}  // namespace qvae
