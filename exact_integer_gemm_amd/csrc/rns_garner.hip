// K3 of the exact residue GEMM on gfx950: balanced Garner mixed-radix
// digits -> signed int64 limbs (exact-solve, "Method"; enclosure-gemm,
// "Method"), and the zero fill of C for K = 0.
#include "rns_device.h"

namespace rns {

// ============================================================================
// K3: Garner reconstruction
// ============================================================================
// One thread per output entry.  NB (a multiple of 8, >= n) bounds the fully
// unrolled digit loops, so every digit and partial sum lives in registers.
// Slots k >= n are padding that the tables make inert (q = 1, all constants
// zero), so the loops carry no guards.  Slot 0 holds the even modulus (2 or
// 256) when the plan has one; its digit is taken in (-q/2, q/2], which puts
// the mixed-radix value in (-P/2, P/2].
//
// acc[k] starts at y_k * Q_k^-1 and loses v_j * (Q_j Q_k^-1 mod q_k) for every
// earlier digit j; |acc| <= 128 + 54 * 128 * 125 < 2^20 keeps the rounding
// step exact.
// The value X = sum_k v_k Q_k is gathered in 16-bit chunks t[c] (signed,
// |t[c]| < 54 * 125 * 2^16 < 2^29) and carried into limbs at the end.
template <int NB>
__global__ __launch_bounds__(256) void garner_kernel(GarnerConsts gc, const int8_t *__restrict__ y,
                                                     int64_t y_plane, int64_t y_pitch, int64_t M,
                                                     int64_t N, int64_t *__restrict__ C, int c_limbs) {
    constexpr int CB = garner_chunks(NB - 1);   // chunks of the widest Q_k
    const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (e >= M * N) return;
    const int64_t i = e / N, j = e - i * N;
    const int8_t *yp = y + i * y_pitch + j;

    int acc[NB];
#pragma unroll
    for (int k = 0; k < NB; k++) acc[k] = (int)yp[gc.plane[k] * y_plane] * (int)gc.tri[tri_index(k, k)];
    int t[CB + 1];
#pragma unroll
    for (int c = 0; c <= CB; c++) t[c] = 0;

#pragma unroll
    for (int k = 0; k < NB; k++) {
        int v;
        if (k == 0 && gc.q[0] == 2) v = acc[0] & 1;
        else if (k == 0 && gc.q[0] == 256) v = ((acc[0] + 127) & 255) - 127;   // digit in [-127, 128]
        else v = reduce_exact(acc[k], gc.q[k], gc.inv[k]);
#pragma unroll
        for (int kk = k + 1; kk < NB; kk++) acc[kk] -= __mul24(v, (int)gc.tri[tri_index(k, kk)]);
#pragma unroll
        for (int c = 0; c < garner_chunks(k); c++)
            t[c] += __mul24(v, (int)gc.q16[garner_chunk_offset(k) + c]);
    }

    // carry the signed chunks into 16-bit digits; the final carry is the sign
    int carry = 0;
    uint32_t words[2 * RNS_MAX_OUT_LIMBS];
#pragma unroll
    for (int w = 0; w < 2 * RNS_MAX_OUT_LIMBS; w++) {
        uint32_t half16[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int c = 2 * w + h;
            const int s = (c <= CB ? t[c] : 0) + carry;
            half16[h] = (uint32_t)s & 0xffffu;
            carry = s >> 16;
        }
        words[w] = half16[0] | (half16[1] << 16);
    }
    int64_t *out = C + e * c_limbs;
#pragma unroll
    for (int l = 0; l < RNS_MAX_OUT_LIMBS; l++)
        if (l < c_limbs) out[l] = (int64_t)(((uint64_t)words[2 * l + 1] << 32) | words[2 * l]);
}

int launch_garner(const GarnerConsts &g, const int8_t *y, int64_t y_plane, int64_t y_pitch,
                  int64_t M, int64_t N, int64_t *C, int32_t c_limbs, hipStream_t s) {
    const int64_t total = M * N;
    if (total == 0) return RNS_OK;
    const int64_t grid = (total + 255) / 256;
    if (grid > 0x7fffffff) return RNS_E_ARG;
    const int nb = (g.n + 7) / 8 * 8;
    dim3 gd((unsigned)grid), bd(256);
    switch (nb) {
        case 8: hipLaunchKernelGGL(garner_kernel<8>, gd, bd, 0, s, g, y, y_plane, y_pitch, M, N, C, c_limbs); break;
        case 16: hipLaunchKernelGGL(garner_kernel<16>, gd, bd, 0, s, g, y, y_plane, y_pitch, M, N, C, c_limbs); break;
        case 24: hipLaunchKernelGGL(garner_kernel<24>, gd, bd, 0, s, g, y, y_plane, y_pitch, M, N, C, c_limbs); break;
        case 32: hipLaunchKernelGGL(garner_kernel<32>, gd, bd, 0, s, g, y, y_plane, y_pitch, M, N, C, c_limbs); break;
        case 40: hipLaunchKernelGGL(garner_kernel<40>, gd, bd, 0, s, g, y, y_plane, y_pitch, M, N, C, c_limbs); break;
        case 48: hipLaunchKernelGGL(garner_kernel<48>, gd, bd, 0, s, g, y, y_plane, y_pitch, M, N, C, c_limbs); break;
        default: hipLaunchKernelGGL(garner_kernel<56>, gd, bd, 0, s, g, y, y_plane, y_pitch, M, N, C, c_limbs); break;
    }
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

// ============================================================================
// zero fill of C (K = 0)
// ============================================================================
__global__ void zero_kernel(int64_t *C, int64_t count) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        C[i] = 0;
}

int launch_zero(int64_t *C, int64_t count, hipStream_t s) {
    if (count == 0) return RNS_OK;
    int64_t grid = (count + 255) / 256;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)grid), dim3(256), 0, s, C, count);
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

}  // namespace rns
