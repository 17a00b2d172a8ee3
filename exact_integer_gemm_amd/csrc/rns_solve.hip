// The GPU part of the exact rational solve (exact-solve, "Method"): the
// batched modular inverse by Gauss-Jordan elimination over every prime at
// once, and the Dixon lift (the batched residue product of rns_gemm plus the
// residual update in one limb).
#include <algorithm>
#include <cstring>
#include <vector>

#include "rns_device.h"
#include "../../include/rns_solve.h"

namespace rns {

// Per-prime constants of the elimination: q and the Barrett multiplier
// floor(2^32 / q).
struct GjConsts {
    int32_t n_primes;
    uint32_t q[kMaxPrimes];
    uint32_t mq[kMaxPrimes];
    float inv[kMaxPrimes];     // fl(1/q) in binary32
};

// t mod q for t < 2^32: qh = floor(t * floor(2^32/q) / 2^32) is floor(t/q) or
// one less (Barrett), so one conditional subtraction finishes it.
__device__ __forceinline__ uint32_t barrett(uint32_t t, uint32_t q, uint32_t mq) {
    const uint32_t r = t - __umulhi(t, mq) * q;
    return r >= q ? r - q : r;
}

// t mod q in [0, q) for |t| < 2^22, with full-rate operations only (Barrett's
// 32-bit high and low products are quarter-rate): the nearest integer k to
// t/q by one binary32 rounding step (fma with 1.5 * 2^23; |t/q| * 2^-24 <
// 1/(4q) keeps it exact, t/q being at least 1/(2q) from a half-integer), then
// t - q k in [-(q-1)/2, (q-1)/2] by a 24-bit multiply-add, then + q if negative.
__device__ __forceinline__ uint32_t mod_q(int t, int q, float inv) {
    const int k = __float_as_int(__builtin_fmaf((float)t, inv, kRoundMagic32)) - 0x4b400000;
    const int r = __mul24(k, -q) + t;
    return (uint32_t)(r < 0 ? r + q : r);
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
    const uint32_t q = gc.q[e];
    const float qf = gc.inv[e];
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
                o |= mod_q((int)a - (int)(m * c), (int)q, qf) << (8 * b);
            }
            out[w] = o;
        }
        *(v4u *)(Wr + j) = out;
    }
}

// ---- blocked elimination: a panel of B columns in LDS, then one rank-B update --------
// Gauss-Jordan on the B panel columns, with every row operation also applied to
// a companion block Y (unit column j placed at the pivot row when step j
// begins), leaves Y = X + S^T, where the panel's whole transformation is
// T = (I + X S) Pi: Pi the row interchanges, S the selection of the B pivot
// rows kb..kb+B-1 of Pi W.  So the rest of the matrix is updated at once as
//   W'[i][c] = W[perm(i)][c] + sum_j X[i][j] * W[perm(kb + j)][c]  (mod q),
// a product of depth B done with byte dot products.  The rows the update reads
// in another row's place (the pivot rows, and rows moved by an interchange,
// whose old contents all come from rows kb..kb+B-1) are copied out first, so
// the update runs in place.

// bytes of a (value in [0, q)) row as balanced int8 packed in a dword
__device__ __forceinline__ uint32_t balanced4(uint32_t w, uint32_t q) {
    uint32_t o = 0;
#pragma unroll
    for (int b = 0; b < 4; b++) {
        const uint32_t v = (w >> (8 * b)) & 0xffu;
        o |= ((v > q / 2 ? v - q : v) & 0xffu) << (8 * b);
    }
    return o;
}

template <int B, int NMAX>
__global__ __launch_bounds__(1024) void gj_panel_kernel(GjConsts gc, const uint8_t *__restrict__ W, int64_t n,
                                                        int64_t pitch, int64_t kb, int bw, int8_t *__restrict__ Xb,
                                                        int8_t *__restrict__ Rb, uint8_t *__restrict__ Oc,
                                                        int32_t *__restrict__ perm, int32_t *__restrict__ singular) {
    constexpr int S = 2 * B + 4;        // LDS row: B panel bytes, B bytes of Y, 4 bytes of padding
    constexpr int WD = B / 4 + 1;       // dwords of the window a step touches
    __shared__ uint32_t rows[NMAX * S / 4];
    __shared__ int16_t pl[NMAX];
    __shared__ int32_t piv_sh[2];
    __shared__ uint32_t ftab[256][WD];  // the pivot row's window times every multiplier f, mod q
    __shared__ uint8_t inv_tab[256];     // inverses mod q (Fermat), once per launch
    const int e = blockIdx.x;
    if (singular[e]) return;
    const int t = threadIdx.x;
    const uint32_t q = gc.q[e], mq = gc.mq[e];
    const float qf = gc.inv[e];
    const uint8_t *We = W + (int64_t)e * n * pitch;
    uint8_t *lb = reinterpret_cast<uint8_t *>(rows);

    // the panel columns of every row; Y and the padding start at zero
    for (int64_t it = t; it < n * (S / 4); it += 1024) {
        const int64_t i = it / (S / 4);
        const int d = (int)(it - i * (S / 4));
        uint32_t v = 0;
        if (4 * d < bw) {
            v = *reinterpret_cast<const uint32_t *>(We + i * pitch + kb + 4 * d);
            const int keep = bw - 4 * d;                   // bytes of this dword inside the panel
            if (keep < 4) v &= (1u << (8 * keep)) - 1u;
        }
        rows[it] = v;
    }
    for (int64_t i = t; i < n; i += 1024) pl[i] = (int16_t)i;
    if (t < 2) piv_sh[t] = (int32_t)n;
    if (t > 0 && t < (int)q) {
        uint32_t inv = 1, base = (uint32_t)t, ex = q - 2;
        while (ex) {
            if (ex & 1) inv = barrett(inv * base, q, mq);
            base = barrett(base * base, q, mq);
            ex >>= 1;
        }
        inv_tab[t] = (uint8_t)inv;
    }
    __syncthreads();

    for (int j = 0; j < bw; j++) {
        const int64_t r0 = kb + j;
        // the first row at or below r0 with a nonzero entry in column j: each
        // wave finds its first by a ballot over rows r0 + 1024 it + t, and
        // one lane per wave meets the others in an LDS minimum
        for (int64_t base = r0; base < n; base += 1024) {
            const int64_t i = base + t;
            const uint64_t m = __ballot(i < n && lb[i * S + j] != 0);
            if (m) {
                if ((t & 63) == 0) atomicMin(&piv_sh[j & 1], (int32_t)(base + (t & ~63) + __ffsll((long long)m) - 1));
                break;
            }
        }
        if (t == 0) piv_sh[(j + 1) & 1] = (int32_t)n;      // read last at step j - 1, before the barrier above
        __syncthreads();
        const int64_t p = piv_sh[j & 1];
        if (p >= n) {
            if (t == 0) singular[e] = 1;
            return;
        }
        // interchange rows r0 and p, put Y's unit in column j, scale by the pivot's inverse
        if (t < S / 4) {
            const uint32_t inv = inv_tab[lb[p * S + j]];
            uint32_t x = rows[p * (S / 4) + t];
            const uint32_t y = rows[r0 * (S / 4) + t];
            if (t == (B + j) / 4) x |= 1u << (8 * ((B + j) % 4));
            uint32_t o = 0;
#pragma unroll
            for (int b = 0; b < 4; b++) o |= mod_q((int)(((x >> (8 * b)) & 0xffu) * inv), (int)q, qf) << (8 * b);
            if (p != r0) rows[p * (S / 4) + t] = y;
            rows[r0 * (S / 4) + t] = o;
            if (t == 0 && p != r0) {
                const int16_t s = pl[p];
                pl[p] = pl[r0];
                pl[r0] = s;
            }
        }
        __syncthreads();
        // f times the pivot row's window, for every f < q: the elimination then subtracts bytes
        const int d0 = (j + 1) / 4;
        for (int it = t; it < (int)q * WD; it += 1024) {
            const int f = it / WD, dd = it - f * WD;
            const uint32_t pv = d0 + dd < S / 4 ? rows[r0 * (S / 4) + d0 + dd] : 0u;
            uint32_t o = 0;
#pragma unroll
            for (int b = 0; b < 4; b++)
                o |= mod_q(f * (int)((pv >> (8 * b)) & 0xffu), (int)q, qf) << (8 * b);
            ftab[f][dd] = o;
        }
        __syncthreads();
        // eliminate column j from every other row over the window j+1 .. B+j: per byte a - f c mod q
        // with a and f c in [0, q), two bytes at a time in 16-bit lanes (256 + a - f c, then + q
        // where bit 8 is clear, i.e. where a < f c)
        // One thread per row (n <= NMAX: 32-bit indices): the row's multiplier f is read once and a
        // row with f = 0 is skipped whole.  The window's WD dwords all lie inside the row (d0 + WD <=
        // S / 4, the last one the zero padding at j >= B - 4).
        const uint32_t qq = q | (q << 16);
        const int keep = j + 1 - 4 * d0;                     // bytes of dword d0 left of column j + 1
        const uint32_t km = keep > 0 ? (1u << (8 * keep)) - 1u : 0u;   // keep <= 3
        for (int i = t; i < (int)n; i += 1024) {
            if (i == r0) continue;
            const uint32_t f = lb[i * S + j];
            if (!f) continue;
            uint32_t *row = rows + i * (S / 4) + d0;
            const uint32_t *ft = ftab[f];
#pragma unroll
            for (int dd = 0; dd < WD; dd++) {
                const uint32_t fc = ft[dd], wv = row[dd];
                uint32_t x = ((wv & 0x00ff00ffu) | 0x01000100u) - (fc & 0x00ff00ffu);
                uint32_t y = (((wv >> 8) & 0x00ff00ffu) | 0x01000100u) - ((fc >> 8) & 0x00ff00ffu);
                const uint32_t mx = (~x >> 8) & 0x00010001u, my = (~y >> 8) & 0x00010001u;
                x = (x + (((mx << 8) - mx) & qq)) & 0x00ff00ffu;
                y = (y + (((my << 8) - my) & qq)) & 0x00ff00ffu;
                uint32_t o = x | (y << 8);
                // bytes of columns <= j are left as they were (the window starts in their dword)
                if (dd == 0) o = (o & ~km) | (wv & km);
                row[dd] = o;
            }
        }
        __syncthreads();
    }

    // X = Y - S^T as balanced int8 [n][B] (columns bw.. zero); the permutation
    int8_t *Xe = Xb + (int64_t)e * n * B;
    for (int64_t it = t; it < n * (B / 4); it += 1024) {
        const int64_t i = it / (B / 4);
        const int d = (int)(it - i * (B / 4));
        uint32_t y = rows[i * (S / 4) + B / 4 + d];
        const int64_t jj = i - kb;                      // the unit sits at row kb + jj, column jj
        if (jj >= 4 * d && jj < 4 * d + 4 && jj < bw) {
            const int b = (int)(jj - 4 * d);
            const uint32_t v = (y >> (8 * b)) & 0xffu;
            y = (y & ~(0xffu << (8 * b))) | ((v == 0 ? q - 1 : v - 1) << (8 * b));
        }
        if (4 * d + 4 > bw) y &= (4 * d >= bw) ? 0u : (1u << (8 * (bw - 4 * d))) - 1u;
        reinterpret_cast<uint32_t *>(Xe)[it] = balanced4(y, q);
    }
    for (int64_t i = t; i < n; i += 1024) perm[(int64_t)e * n + i] = pl[i];
    // copies of the rows the update reads in another row's place, columns cs..pitch
    const int64_t cs = (kb + bw) & ~(int64_t)15;
    const int64_t cw = (pitch - cs) / 4;
    int8_t *Re = Rb + (int64_t)e * B * pitch;
    uint8_t *Oe = Oc + (int64_t)e * B * pitch;
    for (int64_t it = t; it < (int64_t)bw * cw; it += 1024) {
        const int64_t jr = it / cw;
        const int64_t c = cs + 4 * (it - jr * cw);
        const uint32_t src = *reinterpret_cast<const uint32_t *>(We + (int64_t)pl[kb + jr] * pitch + c);
        *reinterpret_cast<uint32_t *>(Re + jr * pitch + c) = balanced4(src, q);
        *reinterpret_cast<uint32_t *>(Oe + jr * pitch + c) =
            *reinterpret_cast<const uint32_t *>(We + (kb + jr) * pitch + c);
    }
    for (int64_t it = t; it < (int64_t)(B - bw) * cw; it += 1024) {      // rows bw..B of R: zero
        const int64_t jr = bw + it / cw;
        const int64_t c = cs + 4 * (it % cw);
        *reinterpret_cast<uint32_t *>(Re + jr * pitch + c) = 0u;
    }
}

// W[i][c] <- W[perm(i)][c] + sum_j X[i][j] R[j][c] (mod q) for columns c >= cs:
// 64 rows x 256 columns per block of 256 threads, 8 rows x 8 columns each (a
// wave covers two row groups, 256 contiguous bytes of each row).  The eight
// source words are fetched first, so that their latency overlaps the product.
template <int B>
__global__ __launch_bounds__(256) void gj_block_update_kernel(GjConsts gc, uint8_t *__restrict__ W, int64_t n,
                                                              int64_t pitch, int64_t kb, int bw, int64_t cs,
                                                              int64_t row_tiles, int64_t col_tiles,
                                                              const int8_t *__restrict__ Xb,
                                                              const int8_t *__restrict__ Rb,
                                                              const uint8_t *__restrict__ Oc,
                                                              const int32_t *__restrict__ perm,
                                                              const int32_t *__restrict__ singular) {
    constexpr int KC = B / 4;           // dword chunks of the depth
    __shared__ uint32_t xs[64][KC];
    __shared__ uint32_t rt[KC][256];
    const int64_t per = row_tiles * col_tiles;
    const int e = (int)(blockIdx.x / per);
    if (singular[e]) return;
    const int64_t tile = blockIdx.x - (int64_t)e * per;
    // row tiles fastest: the blocks an XCD runs together share a column tile, so its R^T comes
    // from that XCD's L2
    const int64_t i0 = (tile % row_tiles) * 64;
    const int64_t c0 = cs + (tile / row_tiles) * 256;
    const int t = threadIdx.x, cg = t & 31, rg = t >> 5;
    const uint32_t q = gc.q[e];
    const float qf = gc.inv[e];
    const int8_t *Xe = Xb + (int64_t)e * n * B;
    const int8_t *Re = Rb + (int64_t)e * B * pitch;
    uint8_t *We = W + (int64_t)e * n * pitch;
    const uint8_t *Oe = Oc + (int64_t)e * B * pitch;
    const int64_t c = c0 + 8 * cg;
    const bool col_ok = c < pitch;

    uint64_t src[8];
    uint32_t piv = 0;                   // bit r: row r's source is a pivot row (balanced bytes)
    // a row's own words are fetched together with its permutation entry, not after it: only the
    // few rows that traded places with a pivot row (at most B per panel) then read their copy
    // (in-bounds addresses for every lane, so the loads need no branch)
    int32_t pis[8];
    uint64_t own[8];
    const int64_t cl = col_ok ? c : 0;
#pragma unroll
    for (int r = 0; r < 8; r++) {
        const int64_t i = i0 + 8 * rg + r;
        const int64_t ic = i < n ? i : n - 1;
        pis[r] = perm[(int64_t)e * n + ic];
        own[r] = *reinterpret_cast<const uint64_t *>(We + ic * pitch + cl);
    }
#pragma unroll
    for (int r = 0; r < 8; r++) {
        const int64_t i = i0 + 8 * rg + r;
        src[r] = 0;
        if (i < n && col_ok) {
            if (i >= kb && i < kb + bw) {
                src[r] = *reinterpret_cast<const uint64_t *>(Re + (i - kb) * pitch + c);
                piv |= 1u << r;
            } else {
                src[r] = pis[r] == i ? own[r] : *reinterpret_cast<const uint64_t *>(Oe + (pis[r] - kb) * pitch + c);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 8; r++) asm volatile("" ::"v"(own[r]));   // the own loads stay unconditional
    for (int it = t; it < 64 * KC; it += 256) {
        const int r = it / KC, d = it - r * KC;
        xs[r][d] = (i0 + r < n) ? reinterpret_cast<const uint32_t *>(Xe + (i0 + r) * B)[d] : 0u;
    }
    // R^T: four depth rows of this thread's eight columns, transposed in registers
    for (int jc = rg; jc < KC; jc += 8) {
        uint64_t r4[4];
#pragma unroll
        for (int k = 0; k < 4; k++)
            r4[k] = col_ok ? *reinterpret_cast<const uint64_t *>(Re + (int64_t)(4 * jc + k) * pitch + c) : 0ull;
#pragma unroll
        for (int k = 0; k < 8; k++) {           // column k: byte r is depth row 4 jc + r
            uint32_t v = 0;
#pragma unroll
            for (int r = 0; r < 4; r++) v |= (uint32_t)((r4[r] >> (8 * k)) & 0xffu) << (8 * r);
            rt[jc][8 * cg + k] = v;
        }
    }
    __syncthreads();
    int acc[8][8];
#pragma unroll
    for (int r = 0; r < 8; r++)
#pragma unroll
        for (int k = 0; k < 8; k++) acc[r][k] = 0;
#pragma unroll
    for (int jc = 0; jc < KC; jc++) {
        const v4u r0 = *reinterpret_cast<const v4u *>(&rt[jc][8 * cg]);
        const v4u r1 = *reinterpret_cast<const v4u *>(&rt[jc][8 * cg + 4]);
#pragma unroll
        for (int r = 0; r < 8; r++) {
            const int x = (int)xs[8 * rg + r][jc];
#pragma unroll
            for (int k = 0; k < 4; k++) {
                acc[r][k] = __builtin_amdgcn_sdot4(x, (int)r0[k], acc[r][k], false);
                acc[r][k + 4] = __builtin_amdgcn_sdot4(x, (int)r1[k], acc[r][k + 4], false);
            }
        }
    }
    if (!col_ok) return;
#pragma unroll
    for (int r = 0; r < 8; r++) {
        const int64_t i = i0 + 8 * rg + r;
        if (i >= n) break;
        const bool sgn = (piv >> r) & 1u;
        uint64_t o = 0;
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const uint32_t sb = (uint32_t)(src[r] >> (8 * k)) & 0xffu;
            const int sv = sgn ? (int)(int8_t)sb : (int)sb;
            o |= (uint64_t)mod_q(acc[r][k] + sv, (int)q, qf) << (8 * k);
        }
        *reinterpret_cast<uint64_t *>(We + i * pitch + c) = o;
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

// ---- fused lift step (n a multiple of 16, at most kFusedCols right-hand sides) ----
// One wave per row i of B = A^-1 mod P.  Digit kernel: the wave's lanes split
// the columns k in 16-byte runs and form, for every prime at once, the dot
// products of row i of the inverse plane with the residues of r mod that
// prime (`v_dot4_i32_i8`); the partial sums meet in LDS, lane e reduces prime
// e's sum mod q_e, and the wave rebuilds the digit by the rounded-quotient CRT
// (X = sum_e u_e M_e - r P, u_e = y_e (M_e^-1 mod q_e) balanced, r the nearest
// integer to sum_e u_e / q_e, one exact correction by P), written as the
// digit's limbs and, apart, its low limb.  Update kernel: r <- (r - A x_low)
// P^-1 mod 2^64 with the wave's row sum, then the new residues of r mod every
// prime for the next digit.  Two launches per step in place of the split, the
// per-prime product, the CRT and the residual update.
constexpr int kFusedCols = 4;
constexpr int kLiftChunks = 11;       // 32-bit chunks of P: up to 352 bits

struct LiftConsts {
    int32_t E;                        // moduli
    int32_t nch;                      // chunks of P in use
    int32_t q[kMaxPrimes];
    int32_t w[kMaxPrimes];            // (P / q)^-1 mod q, balanced
    uint32_t M[kMaxPrimes][kLiftChunks];   // P / q, little-endian chunks
    uint32_t P[kLiftChunks];
};

// the balanced residue of a signed 64-bit value mod q (odd q < 256)
__device__ __forceinline__ int residue_i64(int64_t v, int q) {
    const double inv = 1.0 / (double)q;
    const int hi = (int)(v >> 32);
    const uint32_t lo = (uint32_t)v;
    const int rh = hi - q * (int)__builtin_rint((double)hi * inv);
    const int rl = (int)((double)lo - (double)q * __builtin_rint((double)lo * inv));
    const int two16 = (1 << 16) % q, two32 = (two16 * two16) % q;
    const int t = rh * two32 + rl;                       // |t| < 2^16
    return t - q * (int)__builtin_rintf((float)t / (float)q);
}

template <int W>
__global__ __launch_bounds__(256) void lift_digit_kernel(LiftConsts lc, const int8_t *__restrict__ Binv, int64_t n,
                                                         int64_t c, const int8_t *__restrict__ rres, int64_t npad,
                                                         int64_t *__restrict__ digits, int dl,
                                                         int64_t *__restrict__ xlow) {
    constexpr int R = 4 / W;                               // rows per block
    __shared__ int32_t part[R][64][kMaxPrimes + 1];
    __shared__ int32_t uu[R][kMaxPrimes];
    __shared__ float fs[R][kMaxPrimes];
    __shared__ int64_t ss[R][kLiftChunks];
    const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int rw = wv / W, ww = wv % W;                    // the wave's row in the block, its place in the row
    const int64_t i = (int64_t)blockIdx.x * R + rw;
    const bool row_ok = i < n;
    const bool lead = ww == 0;                             // the row's first wave finishes the digit
    const int E = lc.E;
    const int64_t runs = npad / 16;
    for (int64_t cc = 0; cc < c; cc++) {
        // the row's W waves take alternate batches of eight moduli: 8 partial sums and 16 loads in
        // flight per lane
        for (int e0 = 8 * ww; e0 < E; e0 += 8 * W) {
            int acc[8];
#pragma unroll
            for (int u = 0; u < 8; u++) acc[u] = 0;
            if (row_ok) {
                for (int64_t run = l; run < runs; run += 64) {
#pragma unroll
                    for (int u = 0; u < 8; u++) {
                        const int e = e0 + u;
                        if (e < E) {
                            const v4i a = *(const v4i *)(Binv + ((int64_t)e * n + i) * n + 16 * run);
                            const v4i x = *(const v4i *)(rres + ((int64_t)e * c + cc) * npad + 16 * run);
                            int s = acc[u];
#pragma unroll
                            for (int w4 = 0; w4 < 4; w4++) s = __builtin_amdgcn_sdot4(a[w4], x[w4], s, false);
                            acc[u] = s;
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 8; u++)
                if (e0 + u < E) part[rw][l][e0 + u] = acc[u];
        }
        __syncthreads();
        if (lead && l < E) {
            int64_t t = 0;                                  // |t| < 2^31 (n <= 2^17, |entries| < 128)
            for (int j = 0; j < 64; j++) t += part[rw][j][l];
            const int q = lc.q[l];
            const int y = (int)(t - (int64_t)q * (int64_t)__builtin_rint((double)t / (double)q));
            const int yw = y * lc.w[l];                      // |yw| < 2^14
            const int u = yw - q * (int)__builtin_rintf((float)yw / (float)q);
            uu[rw][l] = u;
            fs[rw][l] = (float)u / (float)q;
        }
        __syncthreads();
        if (lead && l < lc.nch) {
            int64_t s = 0;                                  // |s| < 2^45
            for (int e = 0; e < E; e++) s += (int64_t)uu[rw][e] * (int64_t)lc.M[e][l];
            ss[rw][l] = s;
        }
        __syncthreads();
        if (lead && l == 0 && row_ok) {
            float f = 0.0f;
            for (int e = 0; e < E; e++) f += fs[rw][e];
            const int64_t r = (int64_t)__builtin_rintf(f);
            // X = sum - r P in 32-bit chunks with a sign word
            uint32_t x[kLiftChunks];
            int64_t carry = 0;
            for (int j = 0; j < kLiftChunks; j++) {
                const int64_t v = (j < lc.nch ? ss[rw][j] - r * (int64_t)lc.P[j] : 0) + carry;
                x[j] = (uint32_t)v;
                carry = v >> 32;
            }
            // one exact correction: X > P/2 <=> 2X - P > 0; X < -P/2 <=> 2X + P < 0 (P odd)
            for (int pass = 0; pass < 2; pass++) {
                int64_t bm = 0, bp = 0;
                uint32_t nzm = 0;
                for (int j = 0; j < kLiftChunks; j++) {
                    const uint32_t two = (x[j] << 1) | (j ? x[j - 1] >> 31 : 0u);
                    const int64_t dm = (int64_t)two - (int64_t)lc.P[j] + bm;
                    const int64_t dp = (int64_t)two + (int64_t)lc.P[j] + bp;
                    nzm |= (uint32_t)dm;
                    bm = dm >> 32;
                    bp = dp >> 32;
                }
                const int64_t top2 = 2 * carry + (int64_t)(x[kLiftChunks - 1] >> 31);
                const bool above = top2 + bm > 0 || (top2 + bm == 0 && nzm != 0);
                const bool below = top2 + bp < 0;
                if (!above && !below) break;
                int64_t c2 = 0;
                for (int j = 0; j < kLiftChunks; j++) {
                    c2 += (int64_t)x[j] + (above ? -(int64_t)lc.P[j] : (int64_t)lc.P[j]);
                    x[j] = (uint32_t)c2;
                    c2 >>= 32;
                }
                carry += c2;
            }
            int64_t *dst = digits + (i * c + cc) * dl;
            const uint32_t sgn = (uint32_t)carry;
            for (int li = 0; li < dl; li++) {
                const uint32_t lo = 2 * li < kLiftChunks ? x[2 * li] : sgn;
                const uint32_t hi = 2 * li + 1 < kLiftChunks ? x[2 * li + 1] : sgn;
                dst[li] = (int64_t)(((uint64_t)hi << 32) | lo);
            }
            xlow[cc * n + i] = (int64_t)(((uint64_t)x[1] << 32) | x[0]);
        }
        __syncthreads();
    }
}

// r <- (r - A x_low) P^-1 mod 2^64 per row (first: r <- b), then the residues of
// the new r mod every modulus into rres[e][cc][i].
template <int W>
__global__ __launch_bounds__(256) void lift_update_kernel(LiftConsts lc, const int64_t *__restrict__ A, int64_t n,
                                                          int64_t c, const int64_t *__restrict__ xlow,
                                                          int64_t *__restrict__ r, uint64_t p_inv,
                                                          int8_t *__restrict__ rres, int64_t npad, int first,
                                                          const int64_t *__restrict__ b) {
    constexpr int R = 4 / W;                              // rows per block; W waves share a row's k range
    __shared__ uint64_t part[4];
    const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int rw = wv / W, ww = wv % W;
    const int64_t i = (int64_t)blockIdx.x * R + rw;
    const bool row_ok = i < n;
    for (int64_t cc = 0; cc < c; cc++) {
        uint64_t s = 0;
        if (!first && row_ok) {
            const int64_t *Ai = A + i * n;
            const int64_t *xc = xlow + cc * n;
            int64_t k = (int64_t)ww * 64 + l;
            // four products in flight per lane
            for (; k + 3 * 64 * W < n; k += 4 * 64 * W) {
                const uint64_t a0 = (uint64_t)Ai[k], a1 = (uint64_t)Ai[k + 64 * W];
                const uint64_t a2 = (uint64_t)Ai[k + 128 * W], a3 = (uint64_t)Ai[k + 192 * W];
                const uint64_t x0 = (uint64_t)xc[k], x1 = (uint64_t)xc[k + 64 * W];
                const uint64_t x2 = (uint64_t)xc[k + 128 * W], x3 = (uint64_t)xc[k + 192 * W];
                s += a0 * x0 + a1 * x1 + a2 * x2 + a3 * x3;
            }
            for (; k < n; k += 64 * W) s += (uint64_t)Ai[k] * (uint64_t)xc[k];
            for (int off = 32; off > 0; off >>= 1) {
                const uint32_t lo = __shfl_xor((uint32_t)s, off), hi = __shfl_xor((uint32_t)(s >> 32), off);
                s += ((uint64_t)hi << 32) | lo;
            }
        }
        if (W > 1) {
            if (l == 0) part[wv] = s;
            __syncthreads();
            if (ww == 0)
                for (int w2 = 1; w2 < W; w2++) s += part[wv + w2];
            __syncthreads();
        }
        if (ww == 0 && row_ok) {
            const int64_t v = first ? b[i * c + cc] : (int64_t)(((uint64_t)r[i * c + cc] - s) * p_inv);
            if (l == 0) r[i * c + cc] = v;
            if (l < lc.E) rres[((int64_t)l * c + cc) * npad + i] = (int8_t)residue_i64(v, lc.q[l]);
        }
    }
}

// ---- p-adic values as binary chunks (the radix conversion of the host stage) ----
// X = sum_s d_s P^s for every component is the product of the digits with the
// table pow[t][s] = chunk t of P^s, formed exactly by the residue GEMM: with
// d = d_lo + 2^192 d_hi (d_lo the low three limbs, unsigned; d_hi the rest,
// signed), C_lo = pow d_lo and C_hi = pow d_hi give X = sum_t (C_lo[t] +
// 2^192 C_hi[t]) 2^(32 t), and 2^192 is six chunks.  The pieces landing on
// each chunk are summed in parallel, and a carry pass per component writes X's
// 32-bit chunks.

// digits [m][count][dl] -> lo [m][count][lo_store], hi [m][count][dl - 3]
__global__ __launch_bounds__(256) void digit_halves_kernel(const int64_t *__restrict__ digits, int64_t total, int dl,
                                                           int lo_store, int64_t *__restrict__ lo,
                                                           int64_t *__restrict__ hi) {
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t *d = digits + e * dl;
        if (dl <= 3) {
            for (int l = 0; l < dl; l++) lo[e * lo_store + l] = d[l];
        } else {
            for (int l = 0; l < 3; l++) lo[e * lo_store + l] = d[l];
            lo[e * lo_store + 3] = 0;
            for (int l = 3; l < dl; l++) hi[e * (dl - 3) + l - 3] = d[l];
        }
    }
}

// ---- chunk arithmetic: big integers per component as 32-bit chunks ----
// A source of pieces: entries src[t][idx] of `limbs` int64 limbs (two's
// complement), each worth 2^(32 (t + shift)) times its value, added with `sign`.
struct PieceSrc {
    const int64_t *p;
    int limbs, shift, sign;
    int64_t rows;
};

struct SumArgs {
    PieceSrc src[2];
    int nsrc;
    const int64_t *base;       // optional chunk values base[u][idx] (rows base_rows), added as they are
    int64_t base_rows;
    int64_t bias_u;            // 2^31 is added at chunk bias_u (-1: none)
    int64_t T, count, Tp, cp;  // chunks and components; W is [Tp][cp], zero beyond [T][count]
};

// W[u][idx] = base[u] + the sum of the 32-bit pieces landing on chunk u:
// piece j of an entry at row t lands on t + shift + j (the top piece signed,
// the others unsigned).  The value is sum_u W[u] 2^(32 u), with no carries yet.
// One thread per (u, component).
__global__ __launch_bounds__(256) void chunk_sums_kernel(SumArgs a, int64_t *__restrict__ W) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= a.cp) return;
    for (int64_t u = blockIdx.y; u < a.Tp; u += gridDim.y) {
        int64_t w = 0;
        if (idx < a.count && u < a.T) {
            if (a.base && u < a.base_rows) w = a.base[u * a.count + idx];
            if (u == a.bias_u) w += (int64_t)1 << 31;
            for (int si = 0; si < a.nsrc; si++) {
                const PieceSrc &ps = a.src[si];
                int64_t v = 0;
                for (int j = 0; j < 2 * ps.limbs; j++) {
                    const int64_t t = u - ps.shift - j;
                    if (t < 0) break;
                    if (t >= ps.rows) continue;
                    const uint32_t *pc = reinterpret_cast<const uint32_t *>(ps.p + (t * a.count + idx) * ps.limbs);
                    v += j == 2 * ps.limbs - 1 ? (int64_t)(int32_t)pc[j] : (int64_t)pc[j];
                }
                w += ps.sign < 0 ? -v : v;
            }
        }
        W[u * a.cp + idx] = w;
    }
}

// The carry pass over W: chunk_u = (W[u] + carry) mod 2^32, carry = the
// arithmetic shift by 32.  One lane per component walks its chunks in order;
// its loads run 16 chunks ahead (unconditional: W's zero padding covers
// every position up to 16 past the last 64-chunk block).  Chunks at u >= T
// are dropped: the value fits T chunks.  Output either as uint32 [count][T]
// (the chunks gather in LDS and leave 64 at a time per component, 256
// contiguous bytes) or, with out64, as int64 [T][count] chunk values, the top
// one signed (the operand layout of a following product).
constexpr int kCarryAhead = 16;

__global__ __launch_bounds__(64) void chunk_carry_kernel(const int64_t *__restrict__ W, int64_t T, int64_t count,
                                                         int64_t cp, uint32_t *__restrict__ out,
                                                         int64_t *__restrict__ out64) {
    __shared__ uint32_t tile[64][65];
    const int lane = threadIdx.x;
    const int64_t idx0 = (int64_t)blockIdx.x * 64, idx = idx0 + lane;
    const int64_t *wl = W + idx;
    int64_t carry = 0;
    int64_t ra[kCarryAhead], rb[kCarryAhead];
#define CHUNK_LOAD(r, tb)                                                      \
    _Pragma("unroll") for (int k = 0; k < kCarryAhead; k++) r[k] = wl[((tb) + k) * cp];
#define CHUNK_CARRY(r, off)                                                    \
    _Pragma("unroll") for (int k = 0; k < kCarryAhead; k++) {                  \
        const int64_t s_ = r[k] + carry;                                       \
        tile[lane][(off) + k] = (uint32_t)s_;                                  \
        carry = s_ >> 32;                                                      \
    }
    CHUNK_LOAD(ra, 0)
    for (int64_t t0 = 0; t0 < T; t0 += 64) {
        CHUNK_LOAD(rb, t0 + 16)
        CHUNK_CARRY(ra, 0)
        CHUNK_LOAD(ra, t0 + 32)
        CHUNK_CARRY(rb, 16)
        CHUNK_LOAD(rb, t0 + 48)
        CHUNK_CARRY(ra, 32)
        CHUNK_LOAD(ra, t0 + 64)
        CHUNK_CARRY(rb, 48)
        if (out64) {
            if (idx < count)
                for (int k = 0; k < 64 && t0 + k < T; k++) {
                    const uint32_t ch = tile[lane][k];
                    out64[(t0 + k) * count + idx] = t0 + k == T - 1 ? (int64_t)(int32_t)ch : (int64_t)ch;
                }
        } else {
            __syncthreads();
            const int64_t t = t0 + lane;
            for (int c = 0; c < 64; c++)
                if (idx0 + c < count && t < T) out[(idx0 + c) * T + t] = tile[c][lane];
            __syncthreads();
        }
    }
#undef CHUNK_LOAD
#undef CHUNK_CARRY
}

// Toeplitz matrix of a chunk vector: out[r][t] = c[r + r0 - t] inside 0..Tc-1,
// else 0 ([rows][cols] int64), so out . x is the product c x restricted to
// the chunk positions r0 .. r0 + rows - 1.
__global__ __launch_bounds__(256) void toeplitz_kernel(const int64_t *__restrict__ c, int64_t Tc, int64_t rows,
                                                       int64_t cols, int64_t r0, int64_t *__restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= cols) return;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        const int64_t d = r + r0 - t;
        out[r * cols + t] = d >= 0 && d < Tc ? c[d] : 0;
    }
}

// The bound test of the numerators: ok = |w| <= B for w in Tw two's-complement
// chunks and B >= 0 in TB chunks, without carries: with v = w (w >= 0) or the
// bitwise complement of w (w < 0, then |w| <= B <=> v < B), the highest chunk
// where v and B differ decides.  One wave per component; w leaves as w_limbs
// int64 limbs when ok, zeros otherwise.
__global__ __launch_bounds__(256) void chunk_bound_kernel(const uint32_t *__restrict__ w, int64_t Tw, int64_t count,
                                                          const uint32_t *__restrict__ B, int64_t TB,
                                                          int64_t *__restrict__ num, int w_limbs,
                                                          int32_t *__restrict__ ok, int32_t *__restrict__ used) {
    const int l = threadIdx.x & 63;
    const int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (idx >= count) return;                             // no barriers below
    const uint32_t *wi = w + idx * Tw;
    const bool neg = (int32_t)wi[Tw - 1] < 0;
    const uint32_t fill = neg ? ~0u : 0u;
    const int64_t len = Tw > TB ? Tw : TB;
    int64_t key = -1;                                     // 2 * (highest differing chunk) + (v < B there)
    int64_t top = -1;                                     // the highest chunk of w that is not sign fill
    for (int64_t i = l; i < len; i += 64) {
        const uint32_t wv = i < Tw ? wi[i] : fill;
        const uint32_t v = neg ? ~wv : wv;
        const uint32_t b = i < TB ? B[i] : 0u;
        if (v != b) key = 2 * i + (v < b ? 1 : 0);
        if (v != 0) top = i;
    }
    for (int off = 32; off > 0; off >>= 1) {
        const int64_t o = __shfl_xor(key, off), ot = __shfl_xor(top, off);
        key = o > key ? o : key;
        top = ot > top ? ot : top;
    }
    const bool good = key < 0 ? !neg : (key & 1) != 0;
    if (l == 0) {
        ok[idx] = good ? 1 : 0;
        // limbs that hold w with its sign: the chunks up to top, and one more for the sign bit
        const int64_t lim = (top + 2) / 2 + 1;
        used[idx] = good ? (int32_t)(lim < w_limbs ? lim : w_limbs) : 0;
    }
    for (int li = l; li < w_limbs; li += 64) {
        const int64_t c0 = 2 * (int64_t)li, c1 = c0 + 1;
        const uint32_t lo = c0 < Tw ? wi[c0] : fill, hi = c1 < Tw ? wi[c1] : fill;
        num[idx * w_limbs + li] = good ? (int64_t)(((uint64_t)hi << 32) | lo) : 0;
    }
}

}  // namespace rns

using namespace rns;

namespace {

int64_t pad16(int64_t x) { return (x + 15) / 16 * 16; }
int64_t pad256(int64_t x) { return (x + 255) / 256 * 256; }

// Panel width of the blocked elimination: the panel and its companion block
// of n rows sit in LDS (n * (2B + 4) bytes plus the permutation).  Above
// 4096 rows the elimination runs unblocked, one step per launch pair.
int panel_width(int64_t n) { return n <= 2048 ? 32 : (n <= 4096 ? 16 : 0); }

struct InvLayout {
    int64_t pitch, w_off, prow_off, mcol_off, piv_off;
    int B;                                   // panel width (0: unblocked)
    int64_t xb_off, rb_off, oc_off, perm_off, total;
};

InvLayout inv_layout(int32_t E, int64_t n) {
    InvLayout L;
    L.pitch = pad16(2 * n);
    L.B = panel_width(n);
    int64_t off = 0;
    L.w_off = off;
    off = pad256(off + (int64_t)E * n * L.pitch);
    L.prow_off = off;
    off = pad256(off + (int64_t)E * L.pitch);
    L.mcol_off = off;
    off = pad256(off + (int64_t)E * n);
    L.piv_off = off;
    off = pad256(off + (int64_t)E * 4);
    L.xb_off = off;                          // X: [E][n][B] int8
    off = pad256(off + (int64_t)E * n * L.B);
    L.rb_off = off;                          // pivot rows: [E][B][pitch] int8
    off = pad256(off + (int64_t)E * L.B * L.pitch);
    L.oc_off = off;                          // old rows kb..kb+B-1: [E][B][pitch]
    off = pad256(off + (int64_t)E * L.B * L.pitch);
    L.perm_off = off;                        // [E][n] int32
    off = pad256(off + (L.B ? (int64_t)E * n * 4 : 0));
    L.total = off;
    return L;
}

template <int B, int NMAX>
int blocked_inverse(const GjConsts &gc, int32_t E, int64_t n, const InvLayout &L, uint8_t *base, int32_t *singular,
                    hipStream_t stream) {
    uint8_t *W = base + L.w_off;
    int8_t *Xb = reinterpret_cast<int8_t *>(base + L.xb_off);
    int8_t *Rb = reinterpret_cast<int8_t *>(base + L.rb_off);
    uint8_t *Oc = base + L.oc_off;
    int32_t *perm = reinterpret_cast<int32_t *>(base + L.perm_off);
    const int64_t row_tiles = (n + 63) / 64;
    for (int64_t kb = 0; kb < n; kb += B) {
        const int bw = (int)(n - kb < B ? n - kb : B);
        hipLaunchKernelGGL((gj_panel_kernel<B, NMAX>), dim3((unsigned)E), dim3(1024), 0, stream, gc, W, n, L.pitch, kb,
                           bw, Xb, Rb, Oc, perm, singular);
        const int64_t cs = (kb + bw) & ~(int64_t)15;
        const int64_t col_tiles = (L.pitch - cs + 255) / 256;
        hipLaunchKernelGGL((gj_block_update_kernel<B>), dim3((unsigned)(E * row_tiles * col_tiles)), dim3(256), 0,
                           stream, gc, W, n, L.pitch, kb, bw, cs, row_tiles, col_tiles, Xb, Rb, Oc, perm, singular);
    }
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
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
        gc.inv[e] = 1.0f / (float)primes[e];
    }
    return gc;
}

// The constants of the fused lift step: q, (P/q)^-1 mod q (balanced) and the
// 32-bit chunks of P/q and P.  False when P needs more than kLiftChunks chunks.
bool lift_consts(const rns_plan_t &pl, LiftConsts &lc) {
    std::memset(&lc, 0, sizeof(lc));
    const int E = pl.n_primes;
    lc.E = E;
    auto mul = [](std::vector<uint32_t> &v, uint32_t m) {
        uint64_t carry = 0;
        for (auto &x : v) {
            const uint64_t t = (uint64_t)x * m + carry;
            x = (uint32_t)t;
            carry = t >> 32;
        }
        if (carry) v.push_back((uint32_t)carry);
    };
    std::vector<uint32_t> P{1u};
    for (int e = 0; e < E; e++) mul(P, (uint32_t)pl.primes[e]);
    if ((int)P.size() > kLiftChunks) return false;
    lc.nch = (int)P.size();
    for (int j = 0; j < lc.nch; j++) lc.P[j] = P[j];
    for (int e = 0; e < E; e++) {
        const int q = pl.primes[e];
        std::vector<uint32_t> M{1u};
        int64_t m_mod = 1;
        for (int f = 0; f < E; f++)
            if (f != e) {
                mul(M, (uint32_t)pl.primes[f]);
                m_mod = m_mod * pl.primes[f] % q;
            }
        for (int j = 0; j < (int)M.size() && j < kLiftChunks; j++) lc.M[e][j] = M[j];
        int64_t inv = 1;
        {
            // m_mod^-1 mod q by extended Euclid (q need not be prime)
            int64_t a = m_mod, bq = q, x0 = 1, x1 = 0;
            while (bq) {
                const int64_t t = a / bq;
                int64_t tmp = a - t * bq; a = bq; bq = tmp;
                tmp = x0 - t * x1; x0 = x1; x1 = tmp;
            }
            inv = ((x0 % q) + q) % q;
        }
        lc.q[e] = q;
        lc.w[e] = (int32_t)(inv > q / 2 ? inv - q : inv);
    }
    return true;
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
    if (L.B == 32) return blocked_inverse<32, 2048>(gc, n_primes, n, L, base, singular, stream);
    if (L.B == 16) return blocked_inverse<16, 4096>(gc, n_primes, n, L, base, singular, stream);
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

// plans and buffers of rns_padic_chunks
struct ChunkLayout {
    rns_plan_t lo, hi;
    int has_hi, lo_store, hi_limbs;
    int64_t lo_off, hi_off, clo_off, chi_off, w_off, g_off, total;
    int64_t wT, wc;                          // rows and columns of W, padded
    size_t g_bytes;
};

// W rows and columns for a carry pass over T chunks of count components:
// zero padding for the read-ahead
static int64_t carry_rows(int64_t T) { return (T + 63) / 64 * 64 + kCarryAhead; }
static int64_t carry_cols(int64_t count) { return (count + 63) / 64 * 64; }

// chunk sums into W, then the carry pass into out (uint32 [count][T]) or out64 (int64 [T][count])
static int carry_chunks(const SumArgs &sa, int64_t *W, uint32_t *out, int64_t *out64, hipStream_t stream) {
    const unsigned gy = (unsigned)(sa.Tp < 65535 ? sa.Tp : 65535);
    hipLaunchKernelGGL(chunk_sums_kernel, dim3((unsigned)((sa.cp + 255) / 256), gy), dim3(256), 0, stream, sa, W);
    if (hipGetLastError() != hipSuccess) return RNS_E_HIP;
    hipLaunchKernelGGL(chunk_carry_kernel, dim3((unsigned)(sa.cp / 64)), dim3(64), 0, stream, W, sa.T, sa.count,
                       sa.cp, out, out64);
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

static int chunk_layout(int64_t T, int32_t m, int64_t count, int32_t dl, int32_t P_bits, ChunkLayout &L) {
    if (T < 1 || m < 1 || count < 1 || dl < 1 || dl > RNS_MAX_OUT_LIMBS || P_bits < 2 || P_bits > 64 * dl)
        return RNS_E_ARG;
    if (m > RNS_K_MAX) return RNS_E_K;
    L.has_hi = dl > 3;
    L.lo_store = L.has_hi ? 4 : dl;
    L.hi_limbs = L.has_hi ? dl - 3 : 0;
    // pow chunks < 2^32; the low digit parts < 2^192, the high parts <= 2^(P_bits - 192)
    int rc = rns_plan(m, 32, L.has_hi ? 192 : P_bits, &L.lo);
    if (rc != RNS_OK) return rc;
    size_t glo = 0, ghi = 0;
    rc = rns_workspace_size(&L.lo, T, count, m, 0, &glo);
    if (rc != RNS_OK) return rc;
    if (L.has_hi) {
        rc = rns_plan(m, 32, P_bits > 192 ? P_bits - 192 : 1, &L.hi);
        if (rc != RNS_OK) return rc;
        rc = rns_workspace_size(&L.hi, T, count, m, 0, &ghi);
        if (rc != RNS_OK) return rc;
    }
    int64_t off = 0;
    L.lo_off = off;
    off = pad256(off + (int64_t)m * count * L.lo_store * 8);
    L.hi_off = off;
    off = pad256(off + (int64_t)m * count * L.hi_limbs * 8);
    L.clo_off = off;
    off = pad256(off + T * count * L.lo.out_limbs_min * 8);
    L.chi_off = off;
    off = pad256(off + (L.has_hi ? T * count * L.hi.out_limbs_min * 8 : 0));
    // W: [Tp][cp] with zero padding for the carry pass's read-ahead
    L.wT = carry_rows(T);
    L.wc = carry_cols(count);
    L.w_off = off;
    off = pad256(off + L.wT * L.wc * 8);
    L.g_off = off;
    L.g_bytes = glo > ghi ? glo : ghi;
    L.total = off + (int64_t)L.g_bytes;
    return RNS_OK;
}

// The Barrett step on chunks: Y = D X ([TY][count], TY = T + TD), a = the
// rows of Y from s1c, P1 = a mu + 2^(32 k2c - 1) ([TP1][count], TP1 = Ta +
// Tmu), q = the rows of P1 from k2c, and (Y - q Pm) mod 2^(32 Tw).  Three
// exact residue products with Toeplitz matrices of the constants' chunks.
struct ModmulLayout {
    int64_t TY, Ta, TP1, Tq;
    rns_plan_t py, p1, pz;
    int64_t toep_off, c_off, y_off, p1_off, w_off, g_off, total;
    int64_t wT, wc;
    size_t g_bytes;
};

static int modmul_layout(int64_t T, int64_t count, int64_t TD, int64_t Tmu, int64_t TP, int64_t s1c, int64_t k2c,
                         int64_t Tw, ModmulLayout &L) {
    if (T < 1 || count < 1 || TD < 1 || Tmu < 1 || TP < 1 || Tw < 1 || s1c < 0 || k2c < 1) return RNS_E_ARG;
    L.TY = T + TD;
    if (s1c >= L.TY || Tw > L.TY) return RNS_E_ARG;
    L.Ta = L.TY - s1c;
    L.TP1 = L.Ta + Tmu;
    if (k2c >= L.TP1) return RNS_E_ARG;
    L.Tq = L.TP1 - k2c;
    if (L.TY * count > ((int64_t)1 << 40) || L.TP1 * count > ((int64_t)1 << 40)) return RNS_E_ARG;
    // chunk entries: constants in [0, 2^32), operands' chunks of magnitude at most 2^32
    int rc = rns_plan(T, 32, 32, &L.py);
    if (rc == RNS_OK) rc = rns_plan(L.Ta, 32, 32, &L.p1);
    if (rc == RNS_OK) rc = rns_plan(L.Tq, 32, 32, &L.pz);
    if (rc != RNS_OK) return rc;
    size_t g0 = 0, g1 = 0, g2 = 0;
    rc = rns_workspace_size(&L.py, L.TY, count, T, 0, &g0);
    if (rc == RNS_OK) rc = rns_workspace_size(&L.p1, L.TP1, count, L.Ta, 0, &g1);
    if (rc == RNS_OK) rc = rns_workspace_size(&L.pz, Tw, count, L.Tq, 0, &g2);
    if (rc != RNS_OK) return rc;
    const int64_t toep = std::max(L.TY * T, std::max(L.TP1 * L.Ta, Tw * L.Tq));
    const int64_t cbytes = std::max(L.TY * L.py.out_limbs_min, std::max(L.TP1 * L.p1.out_limbs_min,
                                                                          Tw * L.pz.out_limbs_min)) * count * 8;
    L.wT = carry_rows(std::max(L.TY, L.TP1));
    L.wc = carry_cols(count);
    int64_t off = 0;
    L.toep_off = off;
    off = pad256(off + toep * 8);
    L.c_off = off;
    off = pad256(off + cbytes);
    L.y_off = off;
    off = pad256(off + L.TY * count * 8);
    L.p1_off = off;
    off = pad256(off + L.TP1 * count * 8);
    L.w_off = off;
    off = pad256(off + L.wT * L.wc * 8);
    L.g_off = off;
    L.g_bytes = std::max(g0, std::max(g1, g2));
    L.total = off + (int64_t)L.g_bytes;
    return RNS_OK;
}

static int launch_toeplitz(const int64_t *c, int64_t Tc, int64_t rows, int64_t cols, int64_t *out,
                           hipStream_t stream) {
    const unsigned gy = (unsigned)(rows < 65535 ? rows : 65535);
    hipLaunchKernelGGL(toeplitz_kernel, dim3((unsigned)((cols + 255) / 256), gy), dim3(256), 0, stream, c, Tc, rows,
                       cols, (int64_t)0, out);
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
    if (steps > 0 && c <= kFusedCols && n % 16 == 0) {
        LiftConsts lc;
        if (lift_consts(*plan, lc)) {
            const int64_t r_bytes = pad256(n * c * 8), x_bytes = pad256(n * c * 8);
            const int64_t need_fused = r_bytes + x_bytes + (int64_t)lc.E * c * n;
            if ((int64_t)ws_bytes >= need_fused) {
                uint8_t *base = static_cast<uint8_t *>(ws);
                int64_t *r = reinterpret_cast<int64_t *>(base);
                int64_t *xlow = reinterpret_cast<int64_t *>(base + r_bytes);
                int8_t *rres = reinterpret_cast<int8_t *>(base + r_bytes + x_bytes);
                // each row's work spread over W waves: W = 4 up to 1024 rows and 2 up to 2048 (4n waves,
                // all resident at once); above, one wave per row
                const int W = n <= 1024 ? 4 : (n <= 2048 ? 2 : 1);
                const unsigned grid = (unsigned)((n * W + 3) / 4);
                auto update = [&](int first) {
                    if (W == 4)
                        hipLaunchKernelGGL(lift_update_kernel<4>, dim3(grid), dim3(256), 0, stream, lc, A, n, c, xlow,
                                           r, inv, rres, n, first, b);
                    else if (W == 2)
                        hipLaunchKernelGGL(lift_update_kernel<2>, dim3(grid), dim3(256), 0, stream, lc, A, n, c, xlow,
                                           r, inv, rres, n, first, b);
                    else
                        hipLaunchKernelGGL(lift_update_kernel<1>, dim3(grid), dim3(256), 0, stream, lc, A, n, c, xlow,
                                           r, inv, rres, n, first, b);
                };
                update(1);
                for (int st = 0; st < steps; st++) {
                    int64_t *xs = digits + (int64_t)st * n * c * d_limbs;
                    if (W == 4)
                        hipLaunchKernelGGL(lift_digit_kernel<4>, dim3(grid), dim3(256), 0, stream, lc, Binv, n, c,
                                           rres, n, xs, d_limbs, xlow);
                    else if (W == 2)
                        hipLaunchKernelGGL(lift_digit_kernel<2>, dim3(grid), dim3(256), 0, stream, lc, Binv, n, c,
                                           rres, n, xs, d_limbs, xlow);
                    else
                        hipLaunchKernelGGL(lift_digit_kernel<1>, dim3(grid), dim3(256), 0, stream, lc, Binv, n, c,
                                           rres, n, xs, d_limbs, xlow);
                    update(0);
                }
                return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
            }
        }
    }
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

int rns_padic_chunks_workspace_size(int64_t T, int32_t m, int64_t count, int32_t d_limbs, int32_t P_bits,
                                    size_t *bytes) {
    if (!bytes) return RNS_E_ARG;
    ChunkLayout L;
    const int rc = chunk_layout(T, m, count, d_limbs, P_bits, L);
    if (rc != RNS_OK) return rc;
    *bytes = (size_t)L.total;
    return RNS_OK;
}

int rns_padic_chunks(const int64_t *pow, int64_t T, int32_t m, const int64_t *digits, int64_t count, int32_t d_limbs,
                     int32_t P_bits, int32_t layout, void *out, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!pow || !digits || !out || !ws || (layout != 0 && layout != 1)) return RNS_E_ARG;
    ChunkLayout L;
    int rc = chunk_layout(T, m, count, d_limbs, P_bits, L);
    if (rc != RNS_OK) return rc;
    if ((int64_t)ws_bytes < L.total) return RNS_E_WORKSPACE;
    if (T * count > ((int64_t)1 << 40)) return RNS_E_ARG;
    uint8_t *base = static_cast<uint8_t *>(ws);
    int64_t *lo = reinterpret_cast<int64_t *>(base + L.lo_off);
    int64_t *hi = reinterpret_cast<int64_t *>(base + L.hi_off);
    int64_t *clo = reinterpret_cast<int64_t *>(base + L.clo_off);
    int64_t *chi = reinterpret_cast<int64_t *>(base + L.chi_off);
    void *g = base + L.g_off;
    hipLaunchKernelGGL(digit_halves_kernel, dim3(grid_for((int64_t)m * count)), dim3(256), 0, stream, digits,
                       (int64_t)m * count, d_limbs, L.lo_store, lo, hi);
    if (hipGetLastError() != hipSuccess) return RNS_E_HIP;
    // C^T = pow [T][m] . digits [m][count]: one exact product per half of the digits
    rc = rns_gemm(&L.lo, T, count, m, pow, 1, lo, L.lo_store, clo, L.lo.out_limbs_min, g, L.g_bytes, stream);
    if (rc != RNS_OK) return rc;
    if (L.has_hi) {
        rc = rns_gemm(&L.hi, T, count, m, pow, 1, hi, L.hi_limbs, chi, L.hi.out_limbs_min, g, L.g_bytes, stream);
        if (rc != RNS_OK) return rc;
    }
    int64_t *W = reinterpret_cast<int64_t *>(base + L.w_off);
    SumArgs sa{};
    sa.src[0] = PieceSrc{clo, L.lo.out_limbs_min, 0, 1, T};
    if (L.has_hi) sa.src[1] = PieceSrc{chi, L.hi.out_limbs_min, 6, 1, T};
    sa.nsrc = L.has_hi ? 2 : 1;
    sa.bias_u = -1;
    sa.T = T;
    sa.count = count;
    sa.Tp = L.wT;
    sa.cp = L.wc;
    return carry_chunks(sa, W, layout ? nullptr : static_cast<uint32_t *>(out),
                        layout ? static_cast<int64_t *>(out) : nullptr, stream);
}


int rns_chunk_modmul_workspace_size(int64_t T, int64_t count, int64_t TD, int64_t Tmu, int64_t TP, int64_t s1c,
                                    int64_t k2c, int64_t Tw, size_t *bytes) {
    if (!bytes) return RNS_E_ARG;
    ModmulLayout L;
    const int rc = modmul_layout(T, count, TD, Tmu, TP, s1c, k2c, Tw, L);
    if (rc != RNS_OK) return rc;
    *bytes = (size_t)L.total;
    return RNS_OK;
}

int rns_chunk_modmul(const int64_t *X, int64_t T, int64_t count, const int64_t *Dc, int64_t TD, const int64_t *muc,
                     int64_t Tmu, const int64_t *Pmc, int64_t TP, int64_t s1c, int64_t k2c, int64_t Tw,
                     uint32_t *out, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!X || !Dc || !muc || !Pmc || !out || !ws) return RNS_E_ARG;
    ModmulLayout L;
    int rc = modmul_layout(T, count, TD, Tmu, TP, s1c, k2c, Tw, L);
    if (rc != RNS_OK) return rc;
    if ((int64_t)ws_bytes < L.total) return RNS_E_WORKSPACE;
    uint8_t *base = static_cast<uint8_t *>(ws);
    int64_t *toep = reinterpret_cast<int64_t *>(base + L.toep_off);
    int64_t *C = reinterpret_cast<int64_t *>(base + L.c_off);
    int64_t *Y = reinterpret_cast<int64_t *>(base + L.y_off);
    int64_t *P1 = reinterpret_cast<int64_t *>(base + L.p1_off);
    int64_t *W = reinterpret_cast<int64_t *>(base + L.w_off);
    void *g = base + L.g_off;
    SumArgs sa{};
    sa.nsrc = 1;
    sa.bias_u = -1;
    sa.count = count;
    sa.cp = L.wc;
    // Y = D X
    rc = launch_toeplitz(Dc, TD, L.TY, T, toep, stream);
    if (rc == RNS_OK) rc = rns_gemm(&L.py, L.TY, count, T, toep, 1, X, 1, C, L.py.out_limbs_min, g, L.g_bytes, stream);
    if (rc != RNS_OK) return rc;
    sa.src[0] = PieceSrc{C, L.py.out_limbs_min, 0, 1, L.TY};
    sa.T = L.TY;
    sa.Tp = carry_rows(L.TY);
    rc = carry_chunks(sa, W, nullptr, Y, stream);
    if (rc != RNS_OK) return rc;
    // P1 = a mu + 2^(32 k2c - 1), a = floor(Y / 2^(32 s1c))
    rc = launch_toeplitz(muc, Tmu, L.TP1, L.Ta, toep, stream);
    if (rc == RNS_OK)
        rc = rns_gemm(&L.p1, L.TP1, count, L.Ta, toep, 1, Y + s1c * count, 1, C, L.p1.out_limbs_min, g, L.g_bytes,
                      stream);
    if (rc != RNS_OK) return rc;
    sa.src[0] = PieceSrc{C, L.p1.out_limbs_min, 0, 1, L.TP1};
    sa.T = L.TP1;
    sa.Tp = carry_rows(L.TP1);
    sa.bias_u = k2c - 1;
    rc = carry_chunks(sa, W, nullptr, P1, stream);
    if (rc != RNS_OK) return rc;
    // (Y - q Pm) mod 2^(32 Tw), q = floor(P1 / 2^(32 k2c))
    rc = launch_toeplitz(Pmc, TP, Tw, L.Tq, toep, stream);
    if (rc == RNS_OK)
        rc = rns_gemm(&L.pz, Tw, count, L.Tq, toep, 1, P1 + k2c * count, 1, C, L.pz.out_limbs_min, g, L.g_bytes,
                      stream);
    if (rc != RNS_OK) return rc;
    sa.src[0] = PieceSrc{C, L.pz.out_limbs_min, 0, -1, Tw};
    sa.base = Y;
    sa.base_rows = L.TY;
    sa.bias_u = -1;
    sa.T = Tw;
    sa.Tp = carry_rows(Tw);
    return carry_chunks(sa, W, out, nullptr, stream);
}


int rns_chunk_bound(const uint32_t *w, int64_t Tw, int64_t count, const uint32_t *B, int64_t TB, int64_t *num,
                    int32_t w_limbs, int32_t *ok, int32_t *used, hipStream_t stream) {
    if (!w || !B || !num || !ok || !used || Tw < 1 || count < 0 || TB < 1 || w_limbs < 1) return RNS_E_ARG;
    if (count == 0) return RNS_OK;
    hipLaunchKernelGGL(chunk_bound_kernel, dim3((unsigned)((count + 3) / 4)), dim3(256), 0, stream, w, Tw, count, B,
                       TB, num, w_limbs, ok, used);
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

}  // extern "C"
