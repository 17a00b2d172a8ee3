// Measurement aid of librns_gemm, not a step of the exact product: the int8
// matrix-core rate the device sustains on given operand bytes with no memory
// traffic, against which the products' share of the dense peak can be read.
#include "rns_device.h"

namespace rns {

// One wave per SIMD, 16 chains of v_mfma_i32_32x32x32_i8 in the accumulator
// registers (as a 128 x 128 sub-tile of a product would hold them), 32 MFMAs
// per iteration: 16 on one set of fragments, 16 on a second set.  Each
// thread reads its 8 fragments (128 bytes) once; between iterations every
// fragment is XORed with another, so operands with random bytes stay random
// and the multiplier inputs keep switching as in a product, while zero
// operands stay zero.  No memory traffic and no LDS inside the loop: the
// rate is what the matrix cores sustain on such data at the clock the chip
// then runs.  out[thread] receives the sum of the thread's accumulators.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_probe_kernel(const v4i *__restrict__ src, int iters, int *__restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    v4i fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        fa[i] = src[t * 8 + i];
        fb[i] = src[t * 8 + 4 + i];
    }
    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = v16i{0};
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[j], fa[i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; i++) fa[i] ^= fb[(i + 1) & 3];
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[j], fb[i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; i++) fb[i] ^= fa[(i + 3) & 3];
    }
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) sum += acc[i][j][e];
    out[t] = sum;
}

int launch_mfma_probe(const int8_t *src, int workgroups, int iters, int32_t *out, hipStream_t s) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0, s, (const v4i *)src, iters,
                       (int *)out);
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

}  // namespace rns
