// K3 of the exact residue GEMM on gfx950, default form: the centered CRT
// value by rounded quotient (Ozaki Scheme II paper, §3.5.2: the GPU
// reconstruction takes the centered representative by rounding to nearest),
// with the sum over primes on the matrix cores.
//
// For an entry with residues y_k (the int8 bytes of the product planes):
//   e_k = w_k M_k, w_k = M_k^-1 mod q_k balanced    (M_k = P / q_k, |e_k| <= P/2)
//   r   = nearest integer to sum_k y_k w_k / q_k     (fixed point, error < 2^-19)
//   X'  = sum_k y_k e_k - r P
// X' is congruent to the product entry X mod P and, when r is the true
// nearest integer, equal to it.  No residue is reduced per entry: the
// multiplier w_k is folded into the constant e_k.  X' is formed in balanced
// base-256 chunks by one int8 MFMA: the entry's slots (y_0 .. y_{n-1},
// -r_lo, -r_hi; r = r_lo + 256 r_hi, r_lo in [-127, 128]) against the digits
// of (e_0 .. e_{n-1}, P, 256 P);
// |chunk sum| <= 56 * 128 * 128 < 2^20.
//
// A wave takes 32 entries.  Lane (l32, h) holds entry l32 and slots
// 16h .. 16h + 15 of each 32-slot K step: exactly the second-operand
// fragment of v_mfma_i32_32x32x32_i8, whose result gives lane (l32, h) the
// chunk sums 8*gq + 4h + e (gq, e < 4) of its entry.  The two halves trade
// their 16-bit pairs of chunks and each carries the whole value into 32-bit
// words; each then stores half of the entry's limbs.
#include "rns_device.h"

namespace rns {

// The value x of the lane in the other half-wave (lane l xor 32), by
// v_permlane32_swap: swapping x with itself gives the lower half-wave the
// upper half's values in the second result and vice versa in the first.
__device__ __forceinline__ uint32_t partner_u32(uint32_t x, int h) {
    const auto s = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return h ? s[0] : s[1];
}

// pair_stores: C is 16-byte aligned and c_limbs is even, so the two limbs
// of a lane leave as one 16-byte store
// OFF32: every Y byte lies within 2^32 of y, so addresses are 32-bit offsets
// from the (uniform) base.
template <int KS, int NB, bool OFF32, bool ROWS>
__global__ __launch_bounds__(256) void crt_kernel(CrtConsts cc, CrtDigits cd,
                                                  const int8_t *__restrict__ y, int64_t y_plane,
                                                  int64_t y_pitch, int64_t M, int64_t N,
                                                  int64_t *__restrict__ C, int c_limbs, int pair_stores) {
    constexpr bool rows_mode = ROWS;
    constexpr int W = 8 * NB;                 // 32-bit words of X'
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, l32 = lane & 31;

    // first-operand fragments of the digits: block (ks, nb), lane (c32, h),
    // byte b = digit 32*nb + c32 of the constant of slot 32*ks + 16*h + b.
    // The block first transposes the digit table (a kernel argument) into
    // LDS, digit-major, so that each fragment is one 16-byte LDS read.
    __shared__ v4i dT[kCrtDigits][kCrtSlots / 16];
    {
        int8_t *t = (int8_t *)&dT[0][0];
        for (int i = threadIdx.x; i < kCrtDigits * kCrtSlots; i += blockDim.x) {
            const int c = i / kCrtSlots, k = i - c * kCrtSlots;
            t[i] = k < kCrtSlots - 8 ? cd.d[k][c] : (int8_t)0;
        }
    }
    __syncthreads();
    v4i dig[KS][NB];
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
            const int c = 32 * nb + l32;
            dig[ks][nb] = c < kCrtDigits ? dT[c][2 * ks + h] : v4i{0, 0, 0, 0};
        }

    // this lane's slot constants: the fixed-point weights and plane offsets
    int shi[KS][16], slo[KS][16], plane[KS][16];
    uint32_t poff[KS][16];
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
#pragma unroll
        for (int b = 0; b < 16; b++) {
            const int k0 = 32 * ks + b, k1 = k0 + 16;
            shi[ks][b] = h ? cc.chi[k1] : cc.chi[k0];
            slo[ks][b] = h ? cc.clo[k1] : cc.clo[k0];
            const int k = h ? k1 : k0;
            plane[ks][b] = k < cc.n ? k : cc.n - 1;   // other slots read a valid plane, weight 0
            poff[ks][b] = OFF32 ? (uint32_t)(plane[ks][b] * y_plane) : 0u;
        }

    // rows mode (wide rows): a wave takes 32 consecutive columns of one row at
    // a time, and the row and column group advance by the grid stride without
    // a division per step.  Otherwise 32 consecutive entries of the flattened
    // output, the row found by one division (32-bit when the count allows).
    const int64_t total = M * N;
    const int64_t cgs = rows_mode ? (N + 31) >> 5 : 1;        // column groups per row
    const int64_t groups = rows_mode ? M * cgs : (total + 31) >> 5;
    const int64_t stride = (int64_t)gridDim.x * 4;
    const int64_t g0 = (int64_t)blockIdx.x * 4 + wave;
    int64_t row = g0 / cgs, cg = g0 - row * cgs;
    const int64_t drow = stride / cgs, dcg = stride - drow * cgs;
    const bool small = total < (1ll << 32);
    for (int64_t grp = g0; grp < groups; grp += stride) {
        bool ok;
        int64_t i, j;
        if (rows_mode) {
            const int64_t jj = cg * 32 + l32;
            ok = jj < N;
            j = ok ? jj : N - 1;
            i = row;
            row += drow;
            cg += dcg;
            if (cg >= cgs) {
                cg -= cgs;
                row++;
            }
        } else {
            const int64_t e0 = grp * 32 + l32;
            ok = e0 < total;
            const int64_t ee = ok ? e0 : total - 1;
            i = small ? (int64_t)((uint32_t)ee / (uint32_t)N) : ee / N;
            j = ee - i * N;
        }
        const int64_t e = i * N + j;
        const int8_t *yp = y + i * y_pitch + j;
        const uint32_t yo = OFF32 ? (uint32_t)(i * y_pitch + j) : 0u;

        // the slots' bytes, and the fixed-point sum of y_k c_k in two 16-bit halves
        // of c_k (|sum y chi| < 2^27, |sum y clo| < 2^29 per half-wave)
        int ahi = 0, alo = 0;
        v4i ua[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            int byte[16];
#pragma unroll
            for (int b = 0; b < 16; b++) {
                const int yv = OFF32 ? (int)y[yo + poff[ks][b]] : (int)yp[plane[ks][b] * y_plane];
                ahi = __mul24(yv, shi[ks][b]) + ahi;
                alo = __mul24(yv, slo[ks][b]) + alo;
                byte[b] = yv;
            }
#pragma unroll
            for (int wd = 0; wd < 4; wd++)
                ua[ks][wd] = (int)pack4(byte[4 * wd], byte[4 * wd + 1], byte[4 * wd + 2], byte[4 * wd + 3]);
        }
        ahi += (int)partner_u32((uint32_t)ahi, h);
        alo += (int)partner_u32((uint32_t)alo, h);
        // F / 2^31 is within 2^-19 of S / P; r = floor(F / 2^31 + 1/2)
        const int64_t F = ((int64_t)ahi << 16) + alo;
        const int64_t r64 = (F + (1ll << 30)) >> 31;
        const int64_t fr = F - (r64 << 31);        // in [-2^30, 2^30)
        const bool near_half = fr < -(1ll << 30) + (1ll << 21) || fr >= (1ll << 30) - (1ll << 21);
        const int r = (int)r64;
        const int rlo = ((r + 127) & 255) - 127;  // r = rlo + 256 rhi, rlo in [-127, 128]:
        const int rhi = (r - rlo) >> 8;           // -rlo and -rhi fit int8
        // slots n and n + 1 carry -rlo and -rhi (their bytes were read from a
        // valid plane with weight zero); a slot's K step, half-wave, word and
        // byte are uniform
#pragma unroll
        for (int t = 0; t < 2; t++) {
            const int k = cc.n + t, val = t ? -rhi : -rlo;
            const int ks_k = k >> 5, h_k = (k >> 4) & 1, x_k = (k >> 2) & 3, sh = 8 * (k & 3);
#pragma unroll
            for (int ks = 0; ks < KS; ks++)
#pragma unroll
                for (int x = 0; x < 4; x++)
                    if (ks == ks_k && x == x_k && h == h_k)
                        ua[ks][x] = (int)(((uint32_t)ua[ks][x] & ~(0xffu << sh)) | ((uint32_t)(val & 0xff) << sh));
        }

        v16i acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
            acc[nb] = v16i{0};
#pragma unroll
            for (int ks = 0; ks < KS; ks++)
                acc[nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(dig[ks][nb], ua[ks], acc[nb], 0, 0, 0);
        }

        // Lane (l32, h) holds the chunk sums a[4 gq + e] of digits
        // 32 nb + 8 gq + 4 h + e (|a| < 2^20).  Their pairs lo = a0 + 2^8 a1
        // and hi = a2 + 2^8 a3 (|.| < 2^29) are the 16-bit places 2 w and
        // 2 w + 1 of X' for word w = 8 nb + 2 gq + h.  v_permlane32_swap of a
        // value with itself hands every lane both half-waves' values: the
        // first result is the lower half's (word 8 nb + 2 gq), the second the
        // upper half's (word 8 nb + 2 gq + 1).  Every lane then carries the
        // whole value through 2 W places of 16 bits in 32-bit arithmetic.
        int part[2 * W];
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
#pragma unroll
            for (int gq = 0; gq < 4; gq++) {
                const v16i &a = acc[nb];
                const int lo = a[4 * gq] + (a[4 * gq + 1] << 8);
                const int hi = a[4 * gq + 2] + (a[4 * gq + 3] << 8);
                const auto sl = __builtin_amdgcn_permlane32_swap((uint32_t)lo, (uint32_t)lo, false, false);
                const auto sh = __builtin_amdgcn_permlane32_swap((uint32_t)hi, (uint32_t)hi, false, false);
                const int w0 = 8 * nb + 2 * gq;
                part[2 * w0] = (int)sl[0];
                part[2 * w0 + 1] = (int)sh[0];
                part[2 * w0 + 2] = (int)sl[1];
                part[2 * w0 + 3] = (int)sh[1];
            }
        uint32_t wv[W];
        int c16 = 0;
#pragma unroll
        for (int w = 0; w < W; w++) {
            const int t0 = part[2 * w] + c16;
            const int t1 = part[2 * w + 1] + (t0 >> 16);
            c16 = t1 >> 16;
            wv[w] = __builtin_amdgcn_perm((uint32_t)t1, (uint32_t)t0, 0x05040100u);   // low halves of t0, t1
        }
        int64_t carry = c16;
        // carry is now the sign word (0 or -1): X' = wv + carry * 2^(32 W)

        if (near_half) {
            // exact: X' > P/2 <=> 2X' - P > 0;  X' <= -P/2 <=> 2X' + P <= 0
            int64_t bm = 0, bp = 0;
            uint32_t nzm = 0, nzp = 0;
#pragma unroll
            for (int w = 0; w < W; w++) {
                const uint32_t two = (wv[w] << 1) | (w ? (wv[w - 1] >> 31) : 0u);
                const uint32_t pw = w < 16 ? cc.P[w] : 0u;
                const int64_t dm = (int64_t)two - pw + bm;
                const int64_t dp = (int64_t)two + pw + bp;
                nzm |= (uint32_t)dm;
                nzp |= (uint32_t)dp;
                bm = dm >> 32;
                bp = dp >> 32;
            }
            const int64_t top2 = 2 * carry + (int64_t)(wv[W - 1] >> 31);
            const int64_t tm = top2 + bm, tp = top2 + bp;
            const bool above = tm > 0 || (tm == 0 && nzm != 0);
            const bool below = tp < 0 || (tp == 0 && nzp == 0);
            if (above || below) {
                int64_t c2 = 0;
#pragma unroll
                for (int w = 0; w < W; w++) {
                    const int64_t pw = w < 16 ? (int64_t)cc.P[w] : 0;
                    c2 += (int64_t)wv[w] + (above ? -pw : pw);
                    wv[w] = (uint32_t)c2;
                    c2 >>= 32;
                }
                carry += c2;
            }
        }

        if (ok) {
            // lane (l32, h) writes limbs 4t + 2h and 4t + 2h + 1 of its entry
            int64_t *ce = C + e * c_limbs;
            const uint32_t sign = (uint32_t)carry;
#pragma unroll
            for (int t = 0; t < RNS_MAX_OUT_LIMBS / 4; t++) {
                uint32_t wd[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int i0 = 8 * t + i, i1 = 8 * t + 4 + i;
                    const uint32_t a0 = i0 < W ? wv[i0] : sign, a1 = i1 < W ? wv[i1] : sign;
                    wd[i] = h ? a1 : a0;
                }
                const int l = 4 * t + 2 * h;
                if (pair_stores) {
                    if (l < c_limbs) *(v4u *)(ce + l) = v4u{wd[0], wd[1], wd[2], wd[3]};
                } else {
                    if (l < c_limbs) ce[l] = (int64_t)(((uint64_t)wd[1] << 32) | wd[0]);
                    if (l + 1 < c_limbs) ce[l + 1] = (int64_t)(((uint64_t)wd[3] << 32) | wd[2]);
                }
            }
        }
    }
}

// Quad form (rows mode, or N a multiple of 4): a wave takes 128 entries,
// four consecutive ones per lane pair.  Lane (l32, h) reads, for each of its
// 16 slots per K step, the 4-byte word of entries 4 l32 .. 4 l32 + 3 of one
// plane; a 4 x 4 byte transpose of four such words gives four slots of each
// of the four entries, so one load serves four entries.  The fixed-point sum
// of y_k c_k runs on the matrix cores as well: a first product against the
// balanced base-256 digits of c_k (rows 0-3, repeated in rows 4-7 so that
// both half-waves receive them) leaves F in four partial sums
// (|partial| <= 64 * 128 * 128 < 2^20).
template <int KS, int NB, bool OFF32, bool ROWS, int G>
__global__ __launch_bounds__(256, 2) void crt4_kernel(CrtConsts cc, CrtDigits cd,
                                                   const int8_t *__restrict__ y, int64_t y_plane,
                                                   int64_t y_pitch, int64_t M, int64_t N,
                                                   int64_t *__restrict__ C, int c_limbs, int pair_stores) {
    constexpr int W = 8 * NB;                 // 32-bit words of X'
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, l32 = lane & 31;

    __shared__ v4i dT[kCrtDigits][kCrtSlots / 16];
    // each wave's 128 output entries, as they lie in C, in 16-byte units
    // (unit u at u ^ ((u >> 4) & 15): conflict-free for the entry-strided
    // writes and the contiguous reads)
    __shared__ v4u outs[4][128 * RNS_MAX_OUT_LIMBS / 2];
    {
        int8_t *t = (int8_t *)&dT[0][0];
        for (int i = threadIdx.x; i < kCrtDigits * kCrtSlots; i += blockDim.x) {
            const int c = i / kCrtSlots, k = i - c * kCrtSlots;
            t[i] = k < kCrtSlots - 8 ? cd.d[k][c] : (int8_t)0;
        }
    }
    __syncthreads();
    v4i dig[KS][NB];
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
            const int c = 32 * nb + l32;
            dig[ks][nb] = c < kCrtDigits ? dT[c][2 * ks + h] : v4i{0, 0, 0, 0};
        }
    // fixed-point fragments: row l32 < 8 holds digit l32 % 4 of c_k for the lane's slots
    v4i fx[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int b = 0; b < 16; b++) {
            const int k = 32 * ks + 16 * h + b;
            const uint32_t byte = l32 < 8 ? (cc.cb[k] >> (8 * (l32 & 3))) & 0xffu : 0u;
            wd[b >> 2] |= byte << (8 * (b & 3));
        }
        fx[ks] = v4i{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
    }
    // the lane's slot planes (slots past the moduli read the last plane; their weights are zero)
    int plane[KS][16];
    uint32_t poff[KS][16];
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
#pragma unroll
        for (int b = 0; b < 16; b++) {
            const int k = 32 * ks + 16 * h + b;
            plane[ks][b] = k < cc.n ? k : cc.n - 1;
            poff[ks][b] = OFF32 ? (uint32_t)(plane[ks][b] * y_plane) : 0u;
        }

    const int64_t total = M * N;
    const int64_t cgs = ROWS ? (N + 127) >> 7 : 1;            // 128-column groups per row
    const int64_t groups = ROWS ? M * cgs : (total + 127) >> 7;
    const int64_t stride = (int64_t)gridDim.x * 4;
    const int64_t g0 = (int64_t)blockIdx.x * 4 + wave;
    int64_t row = g0 / cgs, cg = g0 - row * cgs;
    const int64_t drow = stride / cgs, dcg = stride - drow * cgs;
    for (int64_t grp = g0; grp < groups; grp += stride) {
        int64_t i, j0, lim;                   // entries j0 + m < lim (columns, or flat indices) are real
        int64_t base;                         // the group's first entry (flat); `count` of them are real
        int count;
        if (ROWS) {
            i = row;
            j0 = cg * 128 + 4 * l32;          // within the plane's row pitch (a multiple of 128)
            lim = N;
            base = i * N + cg * 128;
            count = (int)min((int64_t)128, N - cg * 128);
            row += drow;
            cg += dcg;
            if (cg >= cgs) {
                cg -= cgs;
                row++;
            }
        } else {
            // N is a multiple of 4: a quad of flat indices lies in one row
            const int64_t f0 = grp * 128 + 4 * l32;
            const int64_t ff = f0 < total ? f0 : total - 4;
            i = ff / N;
            j0 = ff - i * N;
            lim = f0 < total ? j0 + (total - f0) : 0;
            base = grp * 128;
            count = (int)min((int64_t)128, total - base);
        }
        uint32_t q[KS][16];
        const uint32_t yo = OFF32 ? (uint32_t)(i * y_pitch + j0) : 0u;
        const int8_t *yp = y + i * y_pitch + j0;
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
#pragma unroll
            for (int b = 0; b < 16; b++)
                q[ks][b] = OFF32 ? *(const uint32_t *)(y + (yo + poff[ks][b]))
                                 : *(const uint32_t *)(yp + (int64_t)plane[ks][b] * y_plane);
        // 4 x 4 byte transposes: ua[m][ks] word wd = slots 4 wd .. 4 wd + 3 of entry m
        v4i ua[4][KS];
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
#pragma unroll
            for (int wd = 0; wd < 4; wd++) {
                const uint32_t *qq = &q[ks][4 * wd];
                const uint32_t a = __builtin_amdgcn_perm(qq[1], qq[0], 0x05010400u);
                const uint32_t b = __builtin_amdgcn_perm(qq[3], qq[2], 0x05010400u);
                const uint32_t c = __builtin_amdgcn_perm(qq[1], qq[0], 0x07030602u);
                const uint32_t d = __builtin_amdgcn_perm(qq[3], qq[2], 0x07030602u);
                ua[0][ks][wd] = (int)__builtin_amdgcn_perm(b, a, 0x05040100u);
                ua[1][ks][wd] = (int)__builtin_amdgcn_perm(b, a, 0x07060302u);
                ua[2][ks][wd] = (int)__builtin_amdgcn_perm(d, c, 0x05040100u);
                ua[3][ks][wd] = (int)__builtin_amdgcn_perm(d, c, 0x07060302u);
            }

        // the four entries of each lane in groups of G, each group in stages
        // so that the matrix-core products of one entry run while the others'
        // scalar work issues: the group's quotient products, then their
        // quotients and -r slots, then its value products, then carries and
        // stores.  G = 4 hides the most latency; G = 2 holds half as many
        // accumulators, which leaves room for 4 waves per SIMD instead of 3.
#pragma unroll
        for (int m0 = 0; m0 < 4; m0 += G) {
            v16i fsq[4];
#pragma unroll
            for (int m = m0; m < m0 + G; m++) {
                // F = sum_k y_k c_k from the four digit sums
                fsq[m] = v16i{0};
#pragma unroll
                for (int ks = 0; ks < KS; ks++)
                    fsq[m] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fx[ks], ua[m][ks], fsq[m], 0, 0, 0);
            }
            v4i um[4][KS];
            bool nhm[4];
#pragma unroll
            for (int m = m0; m < m0 + G; m++) {
                const v16i &fs = fsq[m];
                const int64_t F = (int64_t)fs[0] + (int64_t)fs[1] * 256 + (int64_t)fs[2] * 65536 +
                                  (int64_t)fs[3] * 16777216;
                // F / 2^31 is within 2^-19 of S / P; r = floor(F / 2^31 + 1/2)
                const int64_t r64 = (F + (1ll << 30)) >> 31;
                const int64_t fr = F - r64 * (1ll << 31);
                const bool near_half = fr < -(1ll << 30) + (1ll << 21) || fr >= (1ll << 30) - (1ll << 21);
                const int r = (int)r64;
                const int rlo = ((r + 127) & 255) - 127;
                const int rhi = (r - rlo) >> 8;
                nhm[m] = near_half;
                v4i (&u)[KS] = um[m];
#pragma unroll
                for (int ks = 0; ks < KS; ks++) u[ks] = ua[m][ks];
#pragma unroll
                for (int t = 0; t < 2; t++) {
                    const int k = cc.n + t, val = t ? -rhi : -rlo;
                    const int ks_k = k >> 5, h_k = (k >> 4) & 1, x_k = (k >> 2) & 3, sh = 8 * (k & 3);
#pragma unroll
                    for (int ks = 0; ks < KS; ks++)
#pragma unroll
                        for (int x = 0; x < 4; x++)
                            if (ks == ks_k && x == x_k && h == h_k)
                                u[ks][x] = (int)(((uint32_t)u[ks][x] & ~(0xffu << sh)) | ((uint32_t)(val & 0xff) << sh));
                }
            }
            v16i accm[4][NB];
#pragma unroll
            for (int m = m0; m < m0 + G; m++)
#pragma unroll
                for (int nb = 0; nb < NB; nb++) {
                    accm[m][nb] = v16i{0};
#pragma unroll
                    for (int ks = 0; ks < KS; ks++)
                        accm[m][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(dig[ks][nb], um[m][ks], accm[m][nb], 0, 0, 0);
                }
#pragma unroll
            for (int m = m0; m < m0 + G; m++) {
                const v16i (&acc)[NB] = accm[m];
                const bool near_half = nhm[m];
                int part[2 * W];
#pragma unroll
                for (int nb = 0; nb < NB; nb++)
#pragma unroll
                    for (int gq = 0; gq < 4; gq++) {
                        const v16i &a = acc[nb];
                        const int lo = a[4 * gq] + (a[4 * gq + 1] << 8);
                        const int hi = a[4 * gq + 2] + (a[4 * gq + 3] << 8);
                        const auto sl = __builtin_amdgcn_permlane32_swap((uint32_t)lo, (uint32_t)lo, false, false);
                        const auto sh = __builtin_amdgcn_permlane32_swap((uint32_t)hi, (uint32_t)hi, false, false);
                        const int w0 = 8 * nb + 2 * gq;
                        part[2 * w0] = (int)sl[0];
                        part[2 * w0 + 1] = (int)sh[0];
                        part[2 * w0 + 2] = (int)sl[1];
                        part[2 * w0 + 3] = (int)sh[1];
                    }
                uint32_t wv[W];
                int c16 = 0;
#pragma unroll
                for (int w = 0; w < W; w++) {
                    const int t0 = part[2 * w] + c16;
                    const int t1 = part[2 * w + 1] + (t0 >> 16);
                    c16 = t1 >> 16;
                    wv[w] = __builtin_amdgcn_perm((uint32_t)t1, (uint32_t)t0, 0x05040100u);
                }
                int64_t carry = c16;
                if (near_half) {
                    int64_t bm = 0, bp = 0;
                    uint32_t nzm = 0, nzp = 0;
#pragma unroll
                    for (int w = 0; w < W; w++) {
                        const uint32_t two = (wv[w] << 1) | (w ? (wv[w - 1] >> 31) : 0u);
                        const uint32_t pw = w < 16 ? cc.P[w] : 0u;
                        const int64_t dm = (int64_t)two - pw + bm;
                        const int64_t dp = (int64_t)two + pw + bp;
                        nzm |= (uint32_t)dm;
                        nzp |= (uint32_t)dp;
                        bm = dm >> 32;
                        bp = dp >> 32;
                    }
                    const int64_t top2 = 2 * carry + (int64_t)(wv[W - 1] >> 31);
                    const int64_t tm = top2 + bm, tp = top2 + bp;
                    const bool above = tm > 0 || (tm == 0 && nzm != 0);
                    const bool below = tp < 0 || (tp == 0 && nzp == 0);
                    if (above || below) {
                        int64_t c2 = 0;
#pragma unroll
                        for (int w = 0; w < W; w++) {
                            const int64_t pw = w < 16 ? (int64_t)cc.P[w] : 0;
                            c2 += (int64_t)wv[w] + (above ? -pw : pw);
                            wv[w] = (uint32_t)c2;
                            c2 >>= 32;
                        }
                        carry += c2;
                    }
                }
                const uint32_t sign = (uint32_t)carry;
#pragma unroll
                for (int t = 0; t < RNS_MAX_OUT_LIMBS / 4; t++) {
                    uint32_t wd[4];
#pragma unroll
                    for (int ii = 0; ii < 4; ii++) {
                        const int i0 = 8 * t + ii, i1 = 8 * t + 4 + ii;
                        const uint32_t a0 = i0 < W ? wv[i0] : sign, a1 = i1 < W ? wv[i1] : sign;
                        wd[ii] = h ? a1 : a0;
                    }
                    const int l = 4 * t + 2 * h;
                    if (pair_stores) {
                        // into the wave's staging area: entry 4 l32 + m, limbs l, l + 1
                        const int u = (4 * l32 + m) * (c_limbs >> 1) + (l >> 1);
                        if (l < c_limbs) outs[wave][u ^ ((u >> 4) & 15)] = v4u{wd[0], wd[1], wd[2], wd[3]};
                    } else if (j0 + m < lim) {
                        int64_t *ce = C + (i * N + j0 + m) * c_limbs;
                        if (l < c_limbs) ce[l] = (int64_t)(((uint64_t)wd[1] << 32) | wd[0]);
                        if (l + 1 < c_limbs) ce[l + 1] = (int64_t)(((uint64_t)wd[3] << 32) | wd[2]);
                    }
                }
            }
        }
        if (pair_stores) {
            // the group's entries leave in 1 KiB runs (2 c_limbs of them): lane x
            // of run r stores unit 64 r + x (entry (64 r + x) / (c_limbs / 2)) if
            // that entry is real
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
            const int upe = c_limbs >> 1;     // units per entry
            v4u *cu = (v4u *)(C + base * c_limbs);
            // nothing in the path reads C back: the stores carry the
            // non-temporal hint (square 19.8 -> 18.8 us, wide 63.2 -> 62.5 us)
#pragma unroll
            for (int r = 0; r < RNS_MAX_OUT_LIMBS; r++) {
                const int u = 64 * r + lane;
                if (r < 2 * upe && u < count * upe)
                    __builtin_nontemporal_store(outs[wave][u ^ ((u >> 4) & 15)], cu + u);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        }
    }
}

// Workgroups of `kernel` (256 threads) resident on the device at once,
// cached per kernel: grid-stride launches take no more, so that no
// workgroup waits for a second round while others finish.
template <typename Kern>
static int64_t crt_resident_blocks(Kern kernel) {
    static const int64_t cached = [&] {
        int dev = 0, cus = 0, per = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 1;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, 256, 0) != hipSuccess || per < 1) per = 1;
        return (int64_t)cus * per;
    }();
    return cached;
}

template <int KS, int NB, bool OFF32, bool ROWS, int G>
static void launch_crt4(int64_t groups, const CrtConsts &c, const CrtDigits &d, const int8_t *y, int64_t y_plane,
                        int64_t y_pitch, int64_t M, int64_t N, int64_t *C, int32_t c_limbs, int pairs,
                        hipStream_t s) {
    auto kernel = crt4_kernel<KS, NB, OFF32, ROWS, G>;
    const int64_t cap = crt_resident_blocks(kernel);
    int64_t grid = (groups + 3) / 4;
    if (grid > cap) grid = cap;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), 0, s, c, d, y, y_plane, y_pitch, M, N, C, c_limbs,
                       pairs);
}

int launch_crt(const CrtConsts &c, const CrtDigits &d, int ksteps, int nblocks,
               const int8_t *y, int64_t y_plane, int64_t y_pitch, int64_t M, int64_t N, int64_t *C,
               int32_t c_limbs, hipStream_t s) {
    const int64_t total = M * N;
    if (total == 0) return RNS_OK;
    if (c.n < 1 || c.n + 2 > 32 * ksteps || ksteps < 1 || ksteps > 2 || nblocks < 1 || nblocks > 2)
        return RNS_E_ARG;
    const int pairs = (reinterpret_cast<uintptr_t>(C) % 16 == 0 && c_limbs % 2 == 0) ? 1 : 0;
    // the Y planes span y_plane * n bytes from y
    const bool off32 = (uint64_t)y_plane * (uint64_t)c.n < (1ull << 32);
    // quad form: rows mode when whole 128-column groups waste little (N a
    // multiple of 128, or N >= 1024), else flat when N is a multiple of 4
    // (the row pitch of the planes is a multiple of 128, so a quad never
    // leaves its row).  Below 1024 groups of 128 entries (4 per compute
    // unit) the byte form's four times as many waves hide latency better.
    if ((N % 128 == 0 || N >= 1024 || N % 4 == 0) && total >= 1024 * 128) {
        const int rows4 = (N % 128 == 0 || N >= 1024) ? 1 : 0;
        if (!rows4 && N % 4) return RNS_E_ARG;
        const int64_t groups4 = rows4 ? M * ((N + 127) / 128) : (total + 127) / 128;
#define RNS_CRT4_LAUNCH(KS, NB, G)                                                                          \
    do {                                                                                                      \
        if (off32 && rows4)                                                                                   \
            launch_crt4<KS, NB, true, true, G>(groups4, c, d, y, y_plane, y_pitch, M, N, C, c_limbs, pairs, s);  \
        else if (off32)                                                                                       \
            launch_crt4<KS, NB, true, false, G>(groups4, c, d, y, y_plane, y_pitch, M, N, C, c_limbs, pairs, s); \
        else if (rows4)                                                                                       \
            launch_crt4<KS, NB, false, true, G>(groups4, c, d, y, y_plane, y_pitch, M, N, C, c_limbs, pairs, s); \
        else                                                                                                  \
            launch_crt4<KS, NB, false, false, G>(groups4, c, d, y, y_plane, y_pitch, M, N, C, c_limbs, pairs,  \
                                                 s);                                                          \
    } while (0)
        // one K step and one digit block: with few bytes per entry (square,
        // 10 primes and 2 limbs: 26) the latency the four-entry stages hide
        // counts most; with many (wide, 29 primes and 4 limbs: 61) the extra
        // waves of pairs keep more loads in flight
        if (ksteps == 1 && nblocks == 1 && c.n + 8 * c_limbs < 40)
            RNS_CRT4_LAUNCH(1, 1, 4);
        else if (ksteps == 1 && nblocks == 1)
            RNS_CRT4_LAUNCH(1, 1, 2);
        else if (ksteps == 1)
            RNS_CRT4_LAUNCH(1, 2, 2);
        else if (nblocks == 1)
            RNS_CRT4_LAUNCH(2, 1, 2);
        else
            RNS_CRT4_LAUNCH(2, 2, 2);
#undef RNS_CRT4_LAUNCH
        return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
    }
    // rows mode when whole 32-column groups waste little: N a multiple of 32, or N >= 256
    const int rows = (N % 32 == 0 || N >= 256) ? 1 : 0;
    const int64_t groups = rows ? M * ((N + 31) / 32) : (total + 31) / 32;
    int64_t grid = (groups + 3) / 4;
    if (grid > 1536) grid = 1536;             // grid-stride: each wave amortises its set-up
    const dim3 g((unsigned)grid), b(256);
#define RNS_CRT_LAUNCH(KS, NB)                                                                              \
    do {                                                                                                    \
        if (off32 && rows)                                                                                  \
            hipLaunchKernelGGL((crt_kernel<KS, NB, true, true>), g, b, 0, s, c, d, y, y_plane, y_pitch, M, N, \
                               C, c_limbs, pairs);                                                          \
        else if (off32)                                                                                     \
            hipLaunchKernelGGL((crt_kernel<KS, NB, true, false>), g, b, 0, s, c, d, y, y_plane, y_pitch, M,  \
                               N, C, c_limbs, pairs);                                                       \
        else if (rows)                                                                                      \
            hipLaunchKernelGGL((crt_kernel<KS, NB, false, true>), g, b, 0, s, c, d, y, y_plane, y_pitch, M,  \
                               N, C, c_limbs, pairs);                                                       \
        else                                                                                                \
            hipLaunchKernelGGL((crt_kernel<KS, NB, false, false>), g, b, 0, s, c, d, y, y_plane, y_pitch, M, \
                               N, C, c_limbs, pairs);                                                       \
    } while (0)
    if (ksteps == 1 && nblocks == 1)
        RNS_CRT_LAUNCH(1, 1);
    else if (ksteps == 1)
        RNS_CRT_LAUNCH(1, 2);
    else if (nblocks == 1)
        RNS_CRT_LAUNCH(2, 1);
    else
        RNS_CRT_LAUNCH(2, 2);
#undef RNS_CRT_LAUNCH
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

}  // namespace rns
