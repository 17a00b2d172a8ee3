// Floating-point front and back end of the exact product on gfx950
// (enclosure-gemm, "Method"): exponent-field reductions that plan the scale
// of an operand, the scaling of binary64 entries into two's-complement
// integer limbs, and the outward rounding of the exact integer product to an
// IEEE pair.  Integer and bit operations only: no floating-point instruction
// takes part (enclosure-gemm, "Method": IEEE values are read and written as
// bit patterns, no rounding mode is consulted).
#include <climits>

#include "rns_device.h"
#include "../../include/rns_enclose.h"

namespace rns {

constexpr int kStatsBlocks = 1024;     // 4 per CU: enough loads in flight to stream X
constexpr int kStatsThreads = 256;
static_assert(kStatsBlocks * 4 * 4 <= RNS_FP_STATS_WS_BYTES, "stats workspace");

// A finite binary64 value is m * 2^e2 with m < 2^53 (the hidden bit for
// normal numbers, none for subnormals, whose exponent is that of the
// smallest normal).
struct Fp64Fields {
    bool neg, zero, finite;
    uint64_t m;
    int e2;
};

__device__ __forceinline__ Fp64Fields fp64_fields(uint64_t b) {
    Fp64Fields f;
    const uint64_t a = b & 0x7fffffffffffffffull;
    const int ef = (int)(a >> 52);
    const uint64_t frac = a & ((1ull << 52) - 1);
    f.neg = (b >> 63) != 0;
    f.zero = a == 0;
    f.finite = ef != 0x7ff;
    f.m = ef ? (frac | (1ull << 52)) : frac;
    f.e2 = ef ? ef - 1075 : -1074;
    return f;
}

// ---- planner reductions ----------------------------------------------------
// Block b reduces a grid-stride share of X into partial[4b .. 4b+3]
// (max msb, min lsb, any nonzero, any non-finite); one block then reduces the
// partials.  Two kernels, no atomics.
__device__ __forceinline__ void block_reduce4(int (&v)[4], int (*sh)[kStatsThreads]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < 4; k++) sh[k][t] = v[k];
    __syncthreads();
    for (int s = kStatsThreads / 2; s > 0; s >>= 1) {
        if (t < s) {
            sh[0][t] = max(sh[0][t], sh[0][t + s]);
            sh[1][t] = min(sh[1][t], sh[1][t + s]);
            sh[2][t] |= sh[2][t + s];
            sh[3][t] |= sh[3][t + s];
        }
        __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < 4; k++) v[k] = sh[k][0];
}

__global__ __launch_bounds__(kStatsThreads) void fp_stats_kernel(const uint64_t *__restrict__ x, int64_t count,
                                                                 int *__restrict__ partial) {
    __shared__ int sh[4][kStatsThreads];
    int v[4] = {INT_MIN, INT_MAX, 0, 0};
    auto take = [&](uint64_t b) {
        const Fp64Fields f = fp64_fields(b);
        if (!f.finite) {
            v[3] = 1;
        } else if (!f.zero) {
            v[2] = 1;
            v[0] = max(v[0], f.e2 + 63 - __clzll((long long)f.m));
            v[1] = min(v[1], f.e2 + __ffsll((long long)f.m) - 1);
        }
    };
    // four loads in flight per thread, then the tail one by one
    const int64_t stride = (int64_t)gridDim.x * kStatsThreads;
    int64_t i = (int64_t)blockIdx.x * kStatsThreads + threadIdx.x;
    for (; i + 3 * stride < count; i += 4 * stride) {
        uint64_t b[4];
#pragma unroll
        for (int u = 0; u < 4; u++) b[u] = x[i + u * stride];
#pragma unroll
        for (int u = 0; u < 4; u++) take(b[u]);
    }
    for (; i < count; i += stride) take(x[i]);
    block_reduce4(v, sh);
    if (threadIdx.x == 0) {
        int4 *o = reinterpret_cast<int4 *>(partial) + blockIdx.x;
        *o = make_int4(v[0], v[1], v[2], v[3]);
    }
}

__global__ __launch_bounds__(kStatsThreads) void fp_stats_final_kernel(const int *__restrict__ partial, int blocks,
                                                                       rns_fp_stats_t *__restrict__ out) {
    __shared__ int sh[4][kStatsThreads];
    int v[4] = {INT_MIN, INT_MAX, 0, 0};
    for (int b = threadIdx.x; b < blocks; b += kStatsThreads) {
        const int4 p = reinterpret_cast<const int4 *>(partial)[b];
        v[0] = max(v[0], p.x);
        v[1] = min(v[1], p.y);
        v[2] |= p.z;
        v[3] |= p.w;
    }
    block_reduce4(v, sh);
    if (threadIdx.x == 0) {
        rns_fp_stats_t s;
        s.max_msb = v[0];
        s.min_lsb = v[1];
        s.nonzero = v[2];
        s.nonfinite = v[3];
        *out = s;
    }
}

// ---- scaling into integer limbs ------------------------------------------------
template <int L>
__global__ __launch_bounds__(256) void fp64_to_limbs_kernel(const uint64_t *__restrict__ x, int64_t count, int F,
                                                            int64_t *__restrict__ out) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
        uint64_t limb[L];
        fp64_floor_scaled<L>(x[i], F, limb);
        int64_t *o = out + i * L;
#pragma unroll
        for (int l = 0; l < L; l++) o[l] = (int64_t)limb[l];
    }
}

// ---- outward rounding ------------------------------------------------------------
// (lo, hi) of S * 2^-q.  With t the index of the leading bit of |S|, the value
// has exponent E = t - q.  Its grid step in the format is 2^(e - mb) with
// e = max(E, emin) (mb = significand bits after the point), i.e. bit
// s = e - mb + q of |S|: g = |S| >> s is the truncated significand and any
// set bit below s makes the value inexact.  The encoding of the truncation is
// ((e + bias - 1) << mb) + g for normal and subnormal values alike, and the
// next encoding is the next value away from zero (up to infinity).  E above
// emax saturates the truncation to the largest finite value.
template <bool F32>
__global__ __launch_bounds__(256) void round_outward_kernel(const int64_t *__restrict__ S, int64_t count, int lc,
                                                            int q, void *__restrict__ lo_out,
                                                            void *__restrict__ hi_out) {
    constexpr int mb = F32 ? 23 : 52;
    constexpr int emin = F32 ? -126 : -1022;
    constexpr int emax = F32 ? 127 : 1023;
    constexpr int bias = emax;
    constexpr uint64_t sign_bit = F32 ? (1ull << 31) : (1ull << 63);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
        const int64_t *s = S + i * lc;
        uint64_t mag[RNS_MAX_OUT_LIMBS];
        const uint64_t top = (uint64_t)s[lc - 1];
        const bool neg = (int64_t)top < 0;
        uint64_t carry = neg ? 1 : 0;
        int ti = -1;
#pragma unroll
        for (int l = 0; l < RNS_MAX_OUT_LIMBS; l++) {
            uint64_t w = l < lc ? (uint64_t)s[l] : (neg ? ~0ull : 0ull);
            if (neg) {
                w = ~w + carry;
                carry = (carry && w == 0) ? 1 : 0;
            }
            mag[l] = w;
            if (w) ti = l;
        }
        uint64_t lo_bits = 0, hi_bits = 0;
        if (ti >= 0) {
            uint64_t mtop = 0;
#pragma unroll
            for (int l = 0; l < RNS_MAX_OUT_LIMBS; l++)
                if (l == ti) mtop = mag[l];
            const int t = ti * 64 + 63 - __clzll((long long)mtop);
            const int E = t - q;
            uint64_t trunc;
            bool inexact;
            if (E > emax) {
                trunc = ((uint64_t)(2 * bias) << mb) | ((1ull << mb) - 1);
                inexact = true;
            } else {
                const int e = E > emin ? E : emin;
                const int sh = e - mb + q;
                uint64_t g = 0;
                inexact = false;
                if (sh >= 0) {
                    const int li = sh >> 6, off = sh & 63;
#pragma unroll
                    for (int l = 0; l < RNS_MAX_OUT_LIMBS; l++) {
                        if (l == li) {
                            g |= mag[l] >> off;
                            if (off && (mag[l] & ((1ull << off) - 1))) inexact = true;
                        }
                        if (l == li + 1 && off) g |= mag[l] << (64 - off);
                        if (l < li && mag[l]) inexact = true;
                    }
                } else {
                    g = mag[0] << -sh;      // |S| < 2^(mb+1) here: exact
                }
                trunc = ((uint64_t)(e + bias - 1) << mb) + g;
            }
            const uint64_t away = trunc + (inexact ? 1 : 0);
            lo_bits = neg ? (away | sign_bit) : trunc;
            hi_bits = neg ? (trunc | sign_bit) : away;
        }
        if (F32) {
            static_cast<uint32_t *>(lo_out)[i] = (uint32_t)lo_bits;
            static_cast<uint32_t *>(hi_out)[i] = (uint32_t)hi_bits;
        } else {
            static_cast<uint64_t *>(lo_out)[i] = lo_bits;
            static_cast<uint64_t *>(hi_out)[i] = hi_bits;
        }
    }
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t *__restrict__ p, int64_t words) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

static unsigned grid_for(int64_t count) {
    const int64_t g = (count + 255) / 256;
    return (unsigned)(g < 4096 ? (g < 1 ? 1 : g) : 4096);
}

}  // namespace rns

using namespace rns;

namespace {

// limbs holding a two's-complement value v with |v| < 2^bits
int limbs_for_bits(int bits) { return (bits + 1 + 63) / 64; }

int64_t round_up256(int64_t x) { return (x + 255) / 256 * 256; }

// The exact product S, then rns_gemm's workspace (the split reads the
// binary64 operands directly, so no integer copy of them is kept).
struct EncloseLayout {
    int64_t s_off, gemm_off, gemm_bytes, total;
};

int enclose_layout(const rns_enclose_plan_t *ep, int64_t M, int64_t N, int64_t K, EncloseLayout *L) {
    size_t gb = 0;
    const int rc = rns_workspace_size(&ep->plan, M, N, K, 0, &gb);
    if (rc != RNS_OK) return rc;
    int64_t off = 0;
    L->s_off = off;
    off = round_up256(off + M * N * ep->c_limbs * 8);
    L->gemm_off = off;
    L->gemm_bytes = (int64_t)gb;
    L->total = off + (int64_t)gb;
    return RNS_OK;
}

bool plan_ok(const rns_enclose_plan_t *ep) {
    return ep && (ep->out_format == 64 || ep->out_format == 32) && ep->a_limbs >= 1 &&
           ep->a_limbs <= RNS_MAX_IN_LIMBS && ep->b_limbs >= 1 && ep->b_limbs <= RNS_MAX_IN_LIMBS &&
           ep->c_limbs >= ep->plan.out_limbs_min && ep->c_limbs <= RNS_MAX_OUT_LIMBS &&
           ep->plan.n_primes >= 1 && ep->plan.n_primes <= RNS_MAX_PRIMES;
}

}  // namespace

extern "C" {

int rns_fp64_stats(const double *X, int64_t count, rns_fp_stats_t *stats, void *ws, size_t ws_bytes,
                   hipStream_t stream) {
    if (!stats || !ws || count < 0 || (count > 0 && !X) || reinterpret_cast<uintptr_t>(ws) % 16) return RNS_E_ARG;
    if (ws_bytes < RNS_FP_STATS_WS_BYTES) return RNS_E_WORKSPACE;
    int blocks = (int)((count + kStatsThreads - 1) / kStatsThreads);
    if (blocks > kStatsBlocks) blocks = kStatsBlocks;
    if (blocks < 1) blocks = 1;
    int *partial = static_cast<int *>(ws);
    hipLaunchKernelGGL(fp_stats_kernel, dim3(blocks), dim3(kStatsThreads), 0, stream,
                       reinterpret_cast<const uint64_t *>(X), count, partial);
    if (hipGetLastError() != hipSuccess) return RNS_E_HIP;
    hipLaunchKernelGGL(fp_stats_final_kernel, dim3(1), dim3(kStatsThreads), 0, stream, partial, blocks, stats);
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

int rns_enclose_plan(int64_t K, const rns_fp_stats_t *a, const rns_fp_stats_t *b, int32_t out_format,
                     rns_enclose_plan_t *out) {
    if (!a || !b || !out || (out_format != 64 && out_format != 32)) return RNS_E_ARG;
    if (K < 0 || K > RNS_K_MAX) return RNS_E_K;
    if (a->nonfinite || b->nonfinite) return RNS_E_NONFINITE;
    rns_enclose_plan_t ep{};
    ep.out_format = out_format;
    ep.zero = (!a->nonzero || !b->nonzero || K == 0) ? 1 : 0;
    if (ep.zero) {
        ep.fa = ep.fb = 0;
        ep.a_bits = ep.b_bits = 0;
    } else {
        // coarsest lossless scales: the lowest set bit of the finest entry lands on bit 0
        ep.fa = -a->min_lsb;
        ep.fb = -b->min_lsb;
        ep.a_bits = a->max_msb - a->min_lsb + 1;
        ep.b_bits = b->max_msb - b->min_lsb + 1;
    }
    ep.a_limbs = limbs_for_bits(ep.a_bits);
    ep.b_limbs = limbs_for_bits(ep.b_bits);
    if (ep.a_limbs > RNS_MAX_IN_LIMBS || ep.b_limbs > RNS_MAX_IN_LIMBS || ep.a_bits > 255 || ep.b_bits > 255)
        return RNS_E_CAPACITY;
    // the primes below 256 first; past their 334.9 bits, the prime-power
    // moduli (362.8 bits, K <= 2^17 - 1)
    int rc = rns_plan(K, ep.a_bits, ep.b_bits, &ep.plan);
    if (rc == RNS_E_CAPACITY && K <= RNS_K_MAX - 1)
        rc = rns_plan_moduli(K, ep.a_bits, ep.b_bits, RNS_MODULI_PRIME_POWERS, &ep.plan);
    if (rc != RNS_OK) return rc;
    ep.c_limbs = ep.plan.out_limbs_min;
    ep.q = ep.fa + ep.fb;
    *out = ep;
    return RNS_OK;
}

int rns_enclose_workspace_size(const rns_enclose_plan_t *ep, int64_t M, int64_t N, int64_t K, size_t *bytes) {
    if (!plan_ok(ep) || !bytes || M < 0 || N < 0 || K < 0) return RNS_E_ARG;
    EncloseLayout L;
    const int rc = enclose_layout(ep, M, N, K, &L);
    if (rc != RNS_OK) return rc;
    *bytes = (size_t)L.total;
    return RNS_OK;
}

int rns_fp64_to_limbs(const double *X, int64_t count, int32_t F, int32_t limbs, int64_t *out,
                      hipStream_t stream) {
    if (count < 0 || limbs < 1 || limbs > RNS_MAX_IN_LIMBS || (count > 0 && (!X || !out))) return RNS_E_ARG;
    if (count == 0) return RNS_OK;
    const dim3 g(grid_for(count)), b(256);
    const uint64_t *x = reinterpret_cast<const uint64_t *>(X);
    switch (limbs) {
        case 1: hipLaunchKernelGGL(fp64_to_limbs_kernel<1>, g, b, 0, stream, x, count, F, out); break;
        case 2: hipLaunchKernelGGL(fp64_to_limbs_kernel<2>, g, b, 0, stream, x, count, F, out); break;
        case 3: hipLaunchKernelGGL(fp64_to_limbs_kernel<3>, g, b, 0, stream, x, count, F, out); break;
        default: hipLaunchKernelGGL(fp64_to_limbs_kernel<4>, g, b, 0, stream, x, count, F, out); break;
    }
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

int rns_round_outward(const int64_t *S, int64_t count, int32_t s_limbs, int32_t q, int32_t out_format,
                      void *lo, void *hi, hipStream_t stream) {
    if (count < 0 || s_limbs < 1 || s_limbs > RNS_MAX_OUT_LIMBS || (out_format != 64 && out_format != 32) ||
        (count > 0 && (!S || !lo || !hi)))
        return RNS_E_ARG;
    if (count == 0) return RNS_OK;
    const dim3 g(grid_for(count)), b(256);
    if (out_format == 32)
        hipLaunchKernelGGL(round_outward_kernel<true>, g, b, 0, stream, S, count, s_limbs, q, lo, hi);
    else
        hipLaunchKernelGGL(round_outward_kernel<false>, g, b, 0, stream, S, count, s_limbs, q, lo, hi);
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

static int mm_enclose(const rns_enclose_plan_t *ep, int64_t M, int64_t N, int64_t K, const double *A,
                      const double *B, int b_rows_n, void *lo, void *hi, void *ws, size_t ws_bytes,
                      hipStream_t stream) {
    if (!plan_ok(ep) || M < 0 || N < 0 || K < 0) return RNS_E_ARG;
    if (K > ep->plan.k_max && !(K == 0)) return RNS_E_K;
    if (M == 0 || N == 0) return RNS_OK;
    if (!lo || !hi || !ws || (K > 0 && (!A || !B))) return RNS_E_ARG;
    if (ep->zero) {
        // an all-zero operand or K == 0: the exact product is 0, (+0.0, +0.0)
        const int64_t words = M * N * (ep->out_format / 32);
        hipLaunchKernelGGL(zero_words_kernel, dim3(grid_for(words)), dim3(256), 0, stream,
                           static_cast<uint32_t *>(lo), words);
        if (hipGetLastError() != hipSuccess) return RNS_E_HIP;
        hipLaunchKernelGGL(zero_words_kernel, dim3(grid_for(words)), dim3(256), 0, stream,
                           static_cast<uint32_t *>(hi), words);
        return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
    }
    EncloseLayout L;
    int rc = enclose_layout(ep, M, N, K, &L);
    if (rc != RNS_OK) return rc;
    if ((int64_t)ws_bytes < L.total) return RNS_E_WORKSPACE;
    int8_t *base = static_cast<int8_t *>(ws);
    int64_t *Si = reinterpret_cast<int64_t *>(base + L.s_off);
    if ((rc = gemm_fp64_scaled(&ep->plan, M, N, K, A, ep->a_limbs, B, ep->b_limbs,
                               Fp64Scales{ep->fa, ep->fb, b_rows_n}, Si, ep->c_limbs, base + L.gemm_off,
                               (size_t)L.gemm_bytes, stream)) != RNS_OK)
        return rc;
    return rns_round_outward(Si, M * N, ep->c_limbs, ep->q, ep->out_format, lo, hi, stream);
}

int rns_mm_enclose(const rns_enclose_plan_t *ep, int64_t M, int64_t N, int64_t K, const double *A,
                   const double *B, void *lo, void *hi, void *ws, size_t ws_bytes, hipStream_t stream) {
    return mm_enclose(ep, M, N, K, A, B, 0, lo, hi, ws, ws_bytes, stream);
}

int rns_mm_enclose_nt(const rns_enclose_plan_t *ep, int64_t M, int64_t N, int64_t K, const double *A,
                      const double *Bt, void *lo, void *hi, void *ws, size_t ws_bytes, hipStream_t stream) {
    return mm_enclose(ep, M, N, K, A, Bt, 1, lo, hi, ws, ws_bytes, stream);
}

}  // extern "C"
