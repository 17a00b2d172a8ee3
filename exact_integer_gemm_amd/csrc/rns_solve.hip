// The GPU part of the exact rational solve (exact-solve, "Method"): the
// batched modular inverse by Gauss-Jordan elimination over every prime at
// once, and the Dixon lift (the batched residue product of rns_gemm plus the
// residual update in one limb).
#include "rns_device.h"
#include "../../include/rns_solve.h"

namespace rns {

// Per-prime constants of the elimination: q and the Barrett multiplier
// floor(2^32 / q).
struct GjConsts {
    int32_t n_primes;
    uint32_t q[kMaxPrimes];
    uint32_t mq[kMaxPrimes];
};

// t mod q for t < 2^32: qh = floor(t * floor(2^32/q) / 2^32) is floor(t/q) or
// one less (Barrett), so one conditional subtraction finishes it.
__device__ __forceinline__ uint32_t barrett(uint32_t t, uint32_t q, uint32_t mq) {
    const uint32_t r = t - __umulhi(t, mq) * q;
    return r >= q ? r - q : r;
}

__global__ __launch_bounds__(64) void zero_i32_kernel(int32_t *__restrict__ p, int64_t count) {
    for (int64_t i = threadIdx.x; i < count; i += 64) p[i] = 0;
}

// ---- [A mod q | I] for every prime ----------------------------------------------
// The augmented matrices are bytes (residues in [0, q)), [E][n][pitch] with
// pitch = 2n rounded up to 16 (the padding stays zero).  A signed 64-bit x is
// reduced from its two 32-bit halves: u = x mod 2^64 = hi 2^32 + lo, and a
// negative x is u - 2^64.
__global__ __launch_bounds__(256) void gj_init_kernel(GjConsts gc, const int64_t *__restrict__ A, int64_t n,
                                                      int64_t pitch, uint8_t *__restrict__ W) {
    const int64_t plane = n * pitch;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < n * pitch;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t i = idx / pitch, j = idx - i * pitch;
        const bool left = j < n;
        const int64_t x = left ? A[i * n + j] : 0;
        const uint64_t u = (uint64_t)x;
        const uint32_t hi = (uint32_t)(u >> 32), lo = (uint32_t)u;
        for (int e = 0; e < gc.n_primes; e++) {
            const uint32_t q = gc.q[e], mq = gc.mq[e];
            uint8_t v;
            if (left) {
                const uint32_t c32 = barrett(barrett(1u << 31, q, mq) * 2, q, mq);   // 2^32 mod q
                uint32_t r = barrett(barrett(hi, q, mq) * c32 + barrett(lo, q, mq), q, mq);
                if (x < 0) {
                    // subtract 2^64 mod q = (2^32 mod q)^2 mod q
                    const uint32_t c64 = barrett(c32 * c32, q, mq);
                    r = barrett(r + q - c64, q, mq);
                }
                v = (uint8_t)r;
            } else {
                v = (j - n == i) ? 1 : 0;      // identity; zero in the padding
            }
            W[e * plane + idx] = v;
        }
    }
}

// ---- one elimination step k, pivot part (one block per prime) ---------------------
// Finds the first row p >= k with a nonzero entry in column k, keeps column k
// of every row (the multipliers, before the swap), writes the pivot row
// scaled by the inverse of its pivot into prow (zero below column k), then
// moves row k into row p.  No pivot: the prime is marked singular and skipped
// from then on.
__global__ __launch_bounds__(256) void gj_pivot_kernel(GjConsts gc, uint8_t *__restrict__ W, int64_t n,
                                                       int64_t pitch, int64_t k, uint8_t *__restrict__ prow,
                                                       uint8_t *__restrict__ mcol, int32_t *__restrict__ pivrow,
                                                       int32_t *__restrict__ singular) {
    const int e = blockIdx.x;
    const int t = threadIdx.x;
    if (singular[e]) return;                 // uniform over the block
    const uint32_t q = gc.q[e], mq = gc.mq[e];
    uint8_t *Wm = W + (int64_t)e * n * pitch;
    __shared__ int64_t best_sh[256];
    __shared__ uint32_t inv_sh;
    int64_t best = n;
    for (int64_t i = k + t; i < n; i += 256)
        if (Wm[i * pitch + k]) { best = i; break; }
    best_sh[t] = best;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (t < s) best_sh[t] = min(best_sh[t], best_sh[t + s]);
        __syncthreads();
    }
    const int64_t p = best_sh[0];
    if (p == n) {
        if (t == 0) {
            singular[e] = 1;
            pivrow[e] = -1;
        }
        return;
    }
    if (t == 0) {
        // pivot^(q-2) mod q
        uint32_t b = Wm[p * pitch + k], r = 1, ex = q - 2;
        while (ex) {
            if (ex & 1) r = barrett(r * b, q, mq);
            b = barrett(b * b, q, mq);
            ex >>= 1;
        }
        inv_sh = r;
    }
    __syncthreads();
    const uint32_t inv = inv_sh;
    for (int64_t i = t; i < n; i += 256) mcol[(int64_t)e * n + i] = Wm[i * pitch + k];
    const int64_t k16 = k & ~(int64_t)15;
    for (int64_t j = k16 + t; j < pitch; j += 256)
        prow[(int64_t)e * pitch + j] = (j < k) ? 0 : (uint8_t)barrett(Wm[p * pitch + j] * inv, q, mq);
    __syncthreads();
    if (p != k)
        for (int64_t j = k16 + t; j < pitch; j += 256) Wm[p * pitch + j] = Wm[k * pitch + j];
    if (t == 0) pivrow[e] = (int32_t)p;
}

// ---- one elimination step k, update part (one wave per row of one prime) ----------
// Row k becomes the scaled pivot row; every other row i loses m_i times it,
// where m_i is its column-k entry (for row p, which now holds the old row k,
// the old row k's entry).  Columns below k16 are untouched: the pivot row is
// zero there.  16 bytes per lane per pass.
__global__ __launch_bounds__(64) void gj_update_kernel(GjConsts gc, uint8_t *__restrict__ W, int64_t n,
                                                       int64_t pitch, int64_t k, const uint8_t *__restrict__ prow,
                                                       const uint8_t *__restrict__ mcol,
                                                       const int32_t *__restrict__ pivrow,
                                                       const int32_t *__restrict__ singular) {
    const int64_t row = blockIdx.x;          // e * n + i
    const int e = (int)(row / n);
    const int64_t i = row - (int64_t)e * n;
    if (singular[e]) return;
    const int64_t p = pivrow[e];
    const uint32_t q = gc.q[e], mq = gc.mq[e];
    const uint32_t qq = q * q;
    const uint32_t m = (i == p) ? mcol[(int64_t)e * n + k] : mcol[(int64_t)e * n + i];
    if (i != k && m == 0) return;
    uint8_t *Wr = W + (int64_t)e * n * pitch + i * pitch;
    const uint8_t *pr = prow + (int64_t)e * pitch;
    const int64_t k16 = k & ~(int64_t)15;
    for (int64_t j = k16 + 16 * threadIdx.x; j < pitch; j += 16 * 64) {
        const v4u pv = *(const v4u *)(pr + j);
        if (i == k) {
            *(v4u *)(Wr + j) = pv;
            continue;
        }
        const v4u wv = *(const v4u *)(Wr + j);
        v4u out;
#pragma unroll
        for (int w = 0; w < 4; w++) {
            uint32_t o = 0;
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const uint32_t a = (wv[w] >> (8 * b)) & 0xffu, c = (pv[w] >> (8 * b)) & 0xffu;
                o |= barrett(a + qq - m * c, q, mq) << (8 * b);
            }
            out[w] = o;
        }
        *(v4u *)(Wr + j) = out;
    }
}

// ---- the inverses as balanced int8 planes ---------------------------------------
struct PlaneSelect {
    int32_t n_sel;
    int32_t src[kMaxPrimes];   // source prime index of each output plane
    int32_t q[kMaxPrimes];
};

__global__ __launch_bounds__(256) void gj_planes_kernel(PlaneSelect ps, const uint8_t *__restrict__ W, int64_t n,
                                                        int64_t pitch, int8_t *__restrict__ out) {
    const int64_t per = n * n;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < ps.n_sel * per;
         idx += (int64_t)gridDim.x * 256) {
        const int t = (int)(idx / per);
        const int64_t rc = idx - (int64_t)t * per;
        const int64_t i = rc / n, j = rc - i * n;
        const int q = ps.q[t];
        const int v = W[(int64_t)ps.src[t] * n * pitch + i * pitch + n + j];
        out[idx] = (int8_t)(v > q / 2 ? v - q : v);
    }
}

// ---- the residual update of the lift ----------------------------------------------
// r_i <- (r_i - A x_i) * P^-1 mod 2^64 for one row of A per block; only the low
// limb of the digit x_i enters A x_i mod 2^64.  The true quotient is below
// 2^63 in magnitude (n * max|A| < 2^63), so the low 64 bits are the value.
constexpr int kLiftCols = 16;

__global__ __launch_bounds__(256) void lift_residual_kernel(const int64_t *__restrict__ A, int64_t n,
                                                            const int64_t *__restrict__ x, int64_t c, int dl,
                                                            int64_t *__restrict__ r, uint64_t p_inv) {
    const int64_t i = blockIdx.x;
    const int t = threadIdx.x;
    __shared__ uint64_t part[kLiftCols][256 / 64];
    for (int64_t c0 = 0; c0 < c; c0 += kLiftCols) {
        uint64_t s[kLiftCols];
#pragma unroll
        for (int cc = 0; cc < kLiftCols; cc++) s[cc] = 0;
        for (int64_t kk = t; kk < n; kk += 256) {
            const uint64_t a = (uint64_t)A[i * n + kk];
            const int64_t *xr = x + (kk * c + c0) * dl;
#pragma unroll
            for (int cc = 0; cc < kLiftCols; cc++)
                if (c0 + cc < c) s[cc] += a * (uint64_t)xr[(int64_t)cc * dl];
        }
        // wave sums, then the four waves
#pragma unroll
        for (int cc = 0; cc < kLiftCols; cc++) {
            uint64_t v = s[cc];
            for (int off = 32; off > 0; off >>= 1) {
                const uint32_t lo = __shfl_xor((uint32_t)v, off), hi = __shfl_xor((uint32_t)(v >> 32), off);
                v += ((uint64_t)hi << 32) | lo;
            }
            if ((t & 63) == 0) part[cc][t >> 6] = v;
        }
        __syncthreads();
        if (t < kLiftCols && c0 + t < c) {
            const uint64_t sum = part[t][0] + part[t][1] + part[t][2] + part[t][3];
            int64_t *rp = r + i * c + c0 + t;
            *rp = (int64_t)(((uint64_t)*rp - sum) * p_inv);
        }
        __syncthreads();
    }
}

}  // namespace rns

using namespace rns;

namespace {

int64_t pad16(int64_t x) { return (x + 15) / 16 * 16; }
int64_t pad256(int64_t x) { return (x + 255) / 256 * 256; }

struct InvLayout {
    int64_t pitch, w_off, prow_off, mcol_off, piv_off, total;
};

InvLayout inv_layout(int32_t E, int64_t n) {
    InvLayout L;
    L.pitch = pad16(2 * n);
    int64_t off = 0;
    L.w_off = off;
    off = pad256(off + (int64_t)E * n * L.pitch);
    L.prow_off = off;
    off = pad256(off + (int64_t)E * L.pitch);
    L.mcol_off = off;
    off = pad256(off + (int64_t)E * n);
    L.piv_off = off;
    off = pad256(off + (int64_t)E * 4);
    L.total = off;
    return L;
}

bool small_prime(int q) {
    if (q < 2 || q > 255) return false;
    for (int d = 2; d * d <= q; d++)
        if (q % d == 0) return false;
    return true;
}

bool primes_ok(const int32_t *primes, int32_t E) {
    if (!primes || E < 1 || E > kMaxPrimes) return false;
    for (int a = 0; a < E; a++) {
        if (!small_prime(primes[a])) return false;
        for (int b = 0; b < a; b++)
            if (primes[a] == primes[b]) return false;
    }
    return true;
}

GjConsts gj_consts(const int32_t *primes, int32_t E) {
    GjConsts gc{};
    gc.n_primes = E;
    for (int e = 0; e < E; e++) {
        gc.q[e] = (uint32_t)primes[e];
        gc.mq[e] = (uint32_t)((1ull << 32) / (uint64_t)primes[e]);
    }
    return gc;
}

unsigned grid_for(int64_t count) {
    const int64_t g = (count + 255) / 256;
    return (unsigned)(g < 8192 ? (g < 1 ? 1 : g) : 8192);
}

}  // namespace

extern "C" {

int rns_inverse_workspace_size(int32_t n_primes, int64_t n, size_t *bytes) {
    if (!bytes || n_primes < 1 || n_primes > kMaxPrimes || n < 1) return RNS_E_ARG;
    *bytes = (size_t)inv_layout(n_primes, n).total;
    return RNS_OK;
}

int rns_batched_inverse(const int32_t *primes, int32_t n_primes, int64_t n, const int64_t *A, int32_t *singular,
                        void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!primes_ok(primes, n_primes) || n < 1 || !A || !singular || !ws) return RNS_E_ARG;
    if (n > RNS_K_MAX) return RNS_E_K;
    if ((int64_t)n_primes * n > 0x7fffffff) return RNS_E_ARG;
    const InvLayout L = inv_layout(n_primes, n);
    if ((int64_t)ws_bytes < L.total) return RNS_E_WORKSPACE;
    uint8_t *base = static_cast<uint8_t *>(ws);
    uint8_t *W = base + L.w_off, *prow = base + L.prow_off, *mcol = base + L.mcol_off;
    int32_t *piv = reinterpret_cast<int32_t *>(base + L.piv_off);
    const GjConsts gc = gj_consts(primes, n_primes);
    hipLaunchKernelGGL(gj_init_kernel, dim3(grid_for(n * L.pitch)), dim3(256), 0, stream, gc, A, n, L.pitch, W);
    if (hipGetLastError() != hipSuccess) return RNS_E_HIP;
    // singular flags start at 0 (a fill kernel: no memset node in a captured graph)
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(64), 0, stream, singular, (int64_t)n_primes);
    if (hipGetLastError() != hipSuccess) return RNS_E_HIP;
    for (int64_t k = 0; k < n; k++) {
        hipLaunchKernelGGL(gj_pivot_kernel, dim3(n_primes), dim3(256), 0, stream, gc, W, n, L.pitch, k, prow, mcol,
                           piv, singular);
        hipLaunchKernelGGL(gj_update_kernel, dim3((unsigned)(n_primes * n)), dim3(64), 0, stream, gc, W, n,
                           L.pitch, k, prow, mcol, piv, singular);
    }
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

int rns_inverse_planes(const int32_t *primes, int32_t n_primes, int64_t n, const int32_t *select, int32_t n_sel,
                       int8_t *planes, const void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!primes_ok(primes, n_primes) || n < 1 || !select || n_sel < 0 || n_sel > n_primes || !ws) return RNS_E_ARG;
    if (n_sel == 0) return RNS_OK;
    if (!planes) return RNS_E_ARG;
    const InvLayout L = inv_layout(n_primes, n);
    if ((int64_t)ws_bytes < L.total) return RNS_E_WORKSPACE;
    PlaneSelect ps{};
    ps.n_sel = n_sel;
    for (int t = 0; t < n_sel; t++) {
        if (select[t] < 0 || select[t] >= n_primes) return RNS_E_ARG;
        ps.src[t] = select[t];
        ps.q[t] = primes[select[t]];
    }
    const uint8_t *W = static_cast<const uint8_t *>(ws) + L.w_off;
    hipLaunchKernelGGL(gj_planes_kernel, dim3(grid_for((int64_t)n_sel * n * n)), dim3(256), 0, stream, ps, W, n,
                       L.pitch, planes);
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

int rns_plan_from_moduli(const int32_t *moduli, int32_t n, int64_t k_max, rns_plan_t *out) {
    if (!moduli || !out || n < 1 || n > kMaxPrimes || k_max < 1 || k_max > RNS_K_MAX) return RNS_E_ARG;
    return plan_from_moduli(moduli, n, k_max, out);
}

int rns_lift_workspace_size(const rns_plan_t *plan, int64_t n, int64_t c, size_t *bytes) {
    if (!plan || !bytes || n < 1 || c < 1) return RNS_E_ARG;
    size_t g = 0;
    const int rc = rns_workspace_size(plan, n, c, n, 1, &g);
    if (rc != RNS_OK) return rc;
    *bytes = (size_t)pad256(n * c * 8) + g;
    return RNS_OK;
}

int rns_dixon_lift(const rns_plan_t *plan, int64_t n, int64_t c, const int8_t *Binv, const int64_t *A,
                   const int64_t *b, int32_t steps, int64_t *digits, int32_t d_limbs, void *ws, size_t ws_bytes,
                   hipStream_t stream) {
    if (!plan || n < 1 || c < 1 || steps < 0 || !Binv || !A || !b || !ws || (steps > 0 && !digits))
        return RNS_E_ARG;
    if (n > plan->k_max) return RNS_E_K;
    for (int j = 0; j < plan->n_primes; j++)
        if (plan->primes[j] % 2 == 0) return RNS_E_ARG;    // P must be odd
    if (d_limbs < plan->out_limbs_min || d_limbs > RNS_MAX_OUT_LIMBS) return RNS_E_OUT_LIMBS;
    size_t need = 0;
    int rc = rns_lift_workspace_size(plan, n, c, &need);
    if (rc != RNS_OK) return rc;
    if (ws_bytes < need) return RNS_E_WORKSPACE;
    if (n * c > 0x7fffffff) return RNS_E_ARG;
    // P^-1 mod 2^64 by Newton's iteration (P odd: P*P = 1 mod 8 to start)
    uint64_t P = 1;
    for (int j = 0; j < plan->n_primes; j++) P *= (uint64_t)plan->primes[j];
    uint64_t inv = P;
    for (int it = 0; it < 6; it++) inv *= 2 - P * inv;
    int64_t *r = static_cast<int64_t *>(ws);
    int8_t *gws = static_cast<int8_t *>(ws) + pad256(n * c * 8);
    const size_t gbytes = ws_bytes - (size_t)pad256(n * c * 8);
    if (hipMemcpyAsync(r, b, (size_t)(n * c * 8), hipMemcpyDeviceToDevice, stream) != hipSuccess) return RNS_E_HIP;
    for (int s = 0; s < steps; s++) {
        int64_t *xs = digits + (int64_t)s * n * c * d_limbs;
        rc = rns_gemm_batched_residue(plan, n, c, n, Binv, r, 1, xs, d_limbs, gws, gbytes, stream);
        if (rc != RNS_OK) return rc;
        hipLaunchKernelGGL(lift_residual_kernel, dim3((unsigned)n), dim3(256), 0, stream, A, n, xs, c, d_limbs, r,
                           inv);
        if (hipGetLastError() != hipSuccess) return RNS_E_HIP;
    }
    return RNS_OK;
}

}  // extern "C"
