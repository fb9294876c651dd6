// qvae_internal.h -- helpers shared by the HIP sources of libqvae (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
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

// Compute units of the current device (queried once; 256 on MI355X).
inline int device_cus()
{
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
        else
            cus = 256;
    }
    return cus;
}

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

// Partial-maximum slots of an activation-maximum buffer (words 1.. of the
// QVAE_ABSMAX_WORDS words): every producer writes all of them, 0 where it
// has nothing, and the quantize pass reduces all of them.
constexpr int kAbsmaxParts = 512;

}  // namespace qvae
