// qvae_probe.hip -- matrix-core rate probe (gfx950): a measurement aid for
// the roofline of the convolution, not part of the method.
//
// Every lane loads its operands once (14 16-byte values from a caller table)
// and then issues nothing but matrix instructions of one shape, cycling
// through those operands, for `iters` rounds.  With no memory traffic and no
// other instructions in the loop, the launch time (measured by the caller)
// gives the rate the matrix cores sustain for that shape on those operand
// values.  On MI355X that rate depends on the values themselves: the chip is
// power-limited under dense matrix load, and nonzero operands draw more than
// zeros; the INT8 convolution's achievable rate is bounded by it.
//
// Per round and wave (one wave per SIMD at 256 threads per workgroup):
//   shape 0  INT8 32x32x32: 2 x 12 instructions on 12 accumulator blocks
//            (3 A x 4 B operands per half-round), 24 x 65536 ops
//   shape 1  INT8 16x16x64: 32 instructions on 32 blocks (4 A x 8 B), 32 x 32768 ops
//   shape 2  bf16 32x32x16: as shape 0 with bf16 operands, 24 x 32768 flops
//   shape 3  bf16 16x16x32: as shape 1 with bf16 operands, 32 x 16384 flops
// The 16x16 loops use inline assembly for the instruction alone (no memory
// access in it; accumulators pinned to the accumulation registers): with the
// builtin the compiler shuffles those registers between iterations.
#include <type_traits>

#include "qvae_internal.h"

namespace qvae {

typedef int p_v4i __attribute__((ext_vector_type(4)));
typedef int p_v16i __attribute__((ext_vector_type(16)));
typedef float p_v4f __attribute__((ext_vector_type(4)));
typedef float p_v16f __attribute__((ext_vector_type(16)));
typedef __bf16 p_bf8 __attribute__((ext_vector_type(8)));

constexpr int kProbeRows = 14;     // operand rows: 6 A + 8 B
constexpr int kProbeLanes = 4096;  // entries per row (a lane takes entry gid % 4096)
constexpr int kProbeThreads = 256;

template <int SHAPE>
__global__ __launch_bounds__(kProbeThreads) void k_probe_mfma(const p_v4i *__restrict__ tab, int iters,
                                                              int *__restrict__ out)
{
    const int gid = blockIdx.x * kProbeThreads + threadIdx.x;
    const int g = gid % kProbeLanes;
    p_v4i a[6], b[8];
#pragma unroll
    for (int k = 0; k < 6; ++k) a[k] = tab[k * kProbeLanes + g];
#pragma unroll
    for (int k = 0; k < 8; ++k) b[k] = tab[(6 + k) * kProbeLanes + g];
    int sum = 0;
    if constexpr (SHAPE == 0 || SHAPE == 2) {
        using Acc = std::conditional_t<SHAPE == 0, p_v16i, p_v16f>;
        Acc acc[12];
#pragma unroll
        for (int k = 0; k < 12; ++k) acc[k] = Acc{};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int m = 0; m < 3; ++m)
#pragma unroll
                    for (int n = 0; n < 4; ++n) {
                        if constexpr (SHAPE == 0)
                            acc[m * 4 + n] =
                                __builtin_amdgcn_mfma_i32_32x32x32_i8(a[m + 3 * p], b[n + 4 * p], acc[m * 4 + n], 0, 0, 0);
                        else
                            acc[m * 4 + n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(p_bf8, a[m + 3 * p]), __builtin_bit_cast(p_bf8, b[n + 4 * p]),
                                acc[m * 4 + n], 0, 0, 0);
                    }
        }
#pragma unroll
        for (int k = 0; k < 12; ++k)
#pragma unroll
            for (int j = 0; j < 16; ++j) sum += (int)acc[k][j];
    } else {
        using Acc = std::conditional_t<SHAPE == 1, p_v4i, p_v4f>;
        Acc acc[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) acc[k] = Acc{};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int n = 0; n < 8; ++n) {
                    if constexpr (SHAPE == 1)
                        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc[m * 8 + n]) : "v"(a[m]), "v"(b[n]));
                    else
                        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[m * 8 + n]) : "v"(a[m]), "v"(b[n]));
                }
        }
        // The compiler does not see into the assembly: give the last matrix
        // instructions' results their latency before the accumulators are read.
        // (Both statements name every accumulator as an operand, so no read of
        // one can be scheduled before the wait.)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]), "+a"(acc[5]), "+a"(acc[6]), "+a"(acc[7]), "+a"(acc[8]), "+a"(acc[9]), "+a"(acc[10]), "+a"(acc[11]), "+a"(acc[12]), "+a"(acc[13]), "+a"(acc[14]), "+a"(acc[15]));
        asm volatile("" : "+a"(acc[16]), "+a"(acc[17]), "+a"(acc[18]), "+a"(acc[19]), "+a"(acc[20]), "+a"(acc[21]), "+a"(acc[22]), "+a"(acc[23]), "+a"(acc[24]), "+a"(acc[25]), "+a"(acc[26]), "+a"(acc[27]), "+a"(acc[28]), "+a"(acc[29]), "+a"(acc[30]), "+a"(acc[31]));
#pragma unroll
        for (int k = 0; k < 32; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) sum += (int)acc[k][j];
    }
    out[gid] = sum;
}


int preload_probe()
{
    hipFuncAttributes attr;
    return hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(&k_probe_mfma<0>)) == hipSuccess ? QVAE_OK
                                                                                                   : QVAE_ELAUNCH;
}

}  // namespace qvae

using namespace qvae;

extern "C" int qvae_probe_mfma(int shape, const int32_t *operands, int iters, int blocks, int32_t *out, void *stream)
{
    if (force_fail(false)) return QVAE_EFORCED;
    if (!operands || !out || iters < 1 || blocks < 1 || blocks > 4096) return QVAE_EINVAL;
    if (!aligned16(operands)) return QVAE_EINVAL;
    const p_v4i *tab = reinterpret_cast<const p_v4i *>(operands);
    int *o = reinterpret_cast<int *>(out);
    const dim3 grid((unsigned)blocks), block(kProbeThreads);
    switch (shape) {
    case 0: hipLaunchKernelGGL(k_probe_mfma<0>, grid, block, 0, as_stream(stream), tab, iters, o); break;
    case 1: hipLaunchKernelGGL(k_probe_mfma<1>, grid, block, 0, as_stream(stream), tab, iters, o); break;
    case 2: hipLaunchKernelGGL(k_probe_mfma<2>, grid, block, 0, as_stream(stream), tab, iters, o); break;
    case 3: hipLaunchKernelGGL(k_probe_mfma<3>, grid, block, 0, as_stream(stream), tab, iters, o); break;
    default: return QVAE_EINVAL;
    }
    return launch_status();
}
