// The batched-residue lift step for skinny right-hand sides in one kernel
// (exact-solve, "Method": each lift step applies every prime's inverse plane
// to the residual as one batched INT8 product, and the CRT assembles the
// wide digit).
//
// X = CRT_j (A_j @ r mod q_j) for A_j the caller's int8 plane j ([n][M][K],
// row-major, read as an integer matrix mod q_j) and r the int64 right-hand
// side [K][N], N <= 16, without a separate residue split or reconstruction
// launch.  The products run on the raw bytes of r rather than on its
// residues, which are the same for every modulus: with the top bit of every
// byte but the top one flipped, r = sum_b a_b 256^b + c_1 (a_b the bytes as
// int8, c_1 = 128 (1 + 256 + ... + 256^6)), so
//   A_j r = sum_b 256^b P_b + c_1 s,   P_b = A_j a_b,  s = A_j 1 (row sums),
// nine int8 products whose right-hand sides do not depend on j.  So one MFMA
// (v_mfma_i32_16x16x64_i8) may mix rows of different moduli: a workgroup
// takes four output rows for all n moduli, product row 4 j + x (modulus j,
// row x), against the 16 columns of each byte of r and a column of ones
// (|P_b| <= K 128 128 <= 2^30 for K <= 2^16).  Then per entry
//   y = sum_b (256^b mod q) P_b + (c_1 mod q) s     (|y| < 2^41, exact in binary64)
// and one rounding step gives its balanced residue.  The workgroup holds all
// n residues of its 64 entries and reconstructs them itself with the
// rounded-quotient CRT of rns_crt.hip (same constants, same arithmetic).
//
// Operand k-order: lane l of an MFMA operand holds row (or column) l % 16 and
// the 16 bytes k = 64 kc + 16 (l / 16) + t, t < 16, of the 64-wide chunk kc
// -- the same k for both operands, so the dot products pair every A byte
// with the byte of r at the same k whatever order the instruction adds them
// in.  The accumulators hold entry (4 (l / 16) + e, l % 16) in element e of
// lane l.
#include "rns_device.h"

namespace rns {

constexpr int kLsRows = 4;                          // output rows per workgroup
constexpr int kLsWaves = 8;
constexpr int kLsNB = 9;                            // byte blocks 0..7 of r, then the row sums
constexpr int kLsPhase = 16;                        // 64-wide K chunks of r held in LDS at once
constexpr int kLsRowPitch = 64 * kLsPhase + 16;     // LDS bytes per (column, byte) row: a phase of k, + 16
constexpr int kLsColPitch = 8 * kLsRowPitch + 16;   // LDS bytes per column (its eight byte rows), + 16
constexpr int kLsPre = 4;                           // K chunks of A in flight per wave
constexpr int kLsW = 12;                            // doubles per modulus: 256^b mod q (8), c_1, q, 1/q, pad

struct LiftArgs {
    const int8_t *a;                // planes [n][M][K]
    const int64_t *r;               // [K][N]
    int64_t *C;                     // [M][N][c_limbs]
    uint32_t *status;               // the workspace's status header
    int32_t M, N, K, KC, c_limbs, pair_stores;
};

// the digit table is read as 32-bit words: it starts 4-byte aligned in the kernel arguments
static_assert(sizeof(LiftArgs) % 8 == 0 && sizeof(StepConsts) % 4 == 0, "argument offsets");
static_assert((kCrtSlots - 8) * kCrtDigits % 4 == 0, "whole words of digits");
static_assert(kLsPhase % kLsPre == 0 && kLsRowPitch % 16 == 0 && kLsColPitch % 16 == 0,
              "phases of whole loop groups, aligned rows");
// the 16 columns of a fragment read fall in distinct groups of four banks
static_assert((kLsColPitch / 4) % 64 % 8 == 4, "column pitch: an odd multiple of 16 bytes modulo 256");
// one base register per lane reaches all eight byte rows of a column within a
// phase through the 16-bit offset of an LDS instruction
static_assert(8 * kLsRowPitch < 65536, "byte rows within the offset range");

// 4 x 4 byte transpose: out[m] byte i = in[i] byte m
__device__ __forceinline__ void transpose4(const uint32_t (&in)[4], uint32_t (&out)[4]) {
    const uint32_t a = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);
    const uint32_t b = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
    const uint32_t c = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);
    const uint32_t d = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
    out[0] = __builtin_amdgcn_perm(b, a, 0x05040100u);
    out[1] = __builtin_amdgcn_perm(b, a, 0x07060302u);
    out[2] = __builtin_amdgcn_perm(d, c, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(d, c, 0x07060302u);
}

// r's bytes for up to kLsPhase chunks are staged in LDS at once ([column][byte][k]:
// kLsRowPitch bytes per row, kLsColPitch per column), so the products run with no
// barrier inside a phase: one phase for K <= 1024, a new staging per further 1024.
template <int MBW, int KS, int NB>
__global__ __launch_bounds__(64 * kLsWaves) void lift_step_kernel(LiftArgs g, StepConsts lc, CrtDigits cd) {
    constexpr int W = 8 * NB;                        // 32-bit words of X'
    __shared__ __align__(16) uint8_t rT[16 * kLsColPitch];     // r's bytes of a phase: [column][b][k]
    __shared__ __align__(16) int8_t Yl[kLsRows * 16][64];      // residues: [entry][modulus]
    __shared__ v4i dT[kCrtDigits][kCrtSlots / 16];              // CRT digits, digit-major
    __shared__ __align__(16) double wt[kMaxPrimes][kLsW];      // per-modulus weights
    __shared__ v4i fxl[2][2][4];                                // fixed-point fragments

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31, g16 = lane >> 4, c16 = lane & 15;
    const int n = lc.n, M = g.M, N = g.N, K = g.K, KC = g.KC;
    const int MB = (4 * n + 15) >> 4;                // 16-row blocks of (modulus, row) pairs
    const int i0 = blockIdx.x * kLsRows;

    // r: thread t stages column t % 16, k = 64 c + 4 ((t / 16) % 16) + u (u < 4) of
    // the phase's chunks c = 2 x + t / 256 (x < kLsPhase / 2).  A k past K reads row
    // K - 1 and a column past N column N - 1 (no branch); both are zeroed when
    // staged.  K is a multiple of 16, so a thread's four k are all below K or all
    // past it.  The top bit of bytes 0..6 is flipped.
    const int sc = tid & 15, sk = 4 * ((tid >> 4) & 15), spar = tid >> 8;
    const uint32_t rrow = 8u * (uint32_t)N;
    const uint32_t rcol = 8u * (uint32_t)min(sc, N - 1);
    const uint32_t rcmask = sc < N ? 0xffffffffu : 0u;
    const char *rbase = (const char *)g.r;
    constexpr int kRx = kLsPhase / 2;                // chunk pairs per phase
    uint2 rv[kRx][4];
    // (x0, x1): the chunk pairs x0 <= x < x1 of phase ph
    auto rload = [&](int ph, int x0, int x1) {
#pragma unroll
        for (int x = x0; x < x1; x++) {
            const int k0 = 64 * (ph * kLsPhase + 2 * x + spar) + sk;
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const uint32_t kk = (uint32_t)min(k0 + u, K - 1);
                rv[x][u] = *(const uint2 *)(rbase + (__umul24(kk, rrow) + rcol));
            }
        }
    };
    auto rstage = [&](int ph, int x0, int x1) {
#pragma unroll
        for (int x = x0; x < x1; x++) {
            const int c = 2 * x + spar;
            const uint32_t m = 64 * (ph * kLsPhase + c) + sk < K ? rcmask : 0u;
            uint32_t lo[4], hi[4], wl[4], wh[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                lo[u] = (rv[x][u].x ^ 0x80808080u) & m;
                hi[u] = (rv[x][u].y ^ 0x00808080u) & m;
            }
            transpose4(lo, wl);
            transpose4(hi, wh);
#pragma unroll
            for (int b = 0; b < 4; b++) {
                *(uint32_t *)&rT[sc * kLsColPitch + b * kLsRowPitch + 64 * c + sk] = wl[b];
                *(uint32_t *)&rT[sc * kLsColPitch + (b + 4) * kLsRowPitch + 64 * c + sk] = wh[b];
            }
        }
    };

    // this lane's A rows: block m = wave + 8 i, product row 16 m + c16 = 4 j + x
    const int8_t *arow[MBW];
#pragma unroll
    for (int i = 0; i < MBW; i++) {
        const int mi = 16 * (wave + kLsWaves * i) + c16;
        const int j = min(mi >> 2, n - 1);
        const int row = min(i0 + (mi & 3), M - 1);
        arow[i] = g.a + ((int64_t)j * M + row) * K + 16 * g16;
    }
    // unconditional loads: a chunk past the last re-reads the last, and a lane
    // group past K re-reads the row's last 16 bytes (r's bytes there are zero)
    auto aload = [&](int i, int kc) {
        const int off = min(min(kc, KC - 1) * 64, K - 16 - 16 * g16);
        return *(const v4i *)(arow[i] + off);
    };

    // The loads go out first: r's first phase, the constants, then A kLsPre
    // chunks ahead of its use.  The chunk count is rounded up to whole groups
    // of kLsPre (chunks past KC have zero bytes of r and no ones), so the
    // unrolled loop has no early exit and the counter waits stay exact.
    const int KCR = (KC + kLsPre - 1) / kLsPre * kLsPre;
    rload(0, 0, kRx);
    constexpr int kWords = (kCrtSlots - 8) * kCrtDigits / 4;
    uint32_t cwd[2], ctb[2] = {0u, 0u}, cfx = 0u;
    int cq = 3, cc1 = 0;
    {
        const uint32_t *src = (const uint32_t *)&cd.d[0][0];
#pragma unroll
        for (int x = 0; x < 2; x++) cwd[x] = src[min(tid + 512 * x, kWords - 1)];
        if (tid < n) {
            ctb[0] = lc.tb[tid][0];
            ctb[1] = lc.tb[tid][1];
            cq = lc.q[tid];
            cc1 = lc.c1[tid];
        }
        if (tid < 64) cfx = (&lc.fx[0][0][0][0])[tid];
    }
    v4i abuf[kLsPre][MBW];
#pragma unroll
    for (int p = 0; p < kLsPre; p++)
#pragma unroll
        for (int i = 0; i < MBW; i++) abuf[p][i] = aload(i, p);
    if (blockIdx.x == 0 && tid == 0) {
        g.status[0] = 0u;                            // no bound is checked: no blocks, no flags
        g.status[1] = kStatusCheck;
    }

    // constants into LDS while A is in flight: the CRT digits (the slot-major
    // table's words scattered digit-major), the weights of modulus tid, the
    // fixed-point fragments, zero residues past the moduli.  (The values are
    // only used from here on, so no wait for them is hoisted above the loads of A.)
    asm volatile("" : "+v"(cwd[0]), "+v"(cwd[1]), "+v"(ctb[0]), "+v"(ctb[1]), "+v"(cq), "+v"(cc1), "+v"(cfx));
    rstage(0, 0, kRx);
    {
        int8_t *t = (int8_t *)&dT[0][0];
#pragma unroll
        for (int x = 0; x < 2; x++) {
            const int w = tid + 512 * x;
            if (w < kWords)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int i = 4 * w + e, k = i / kCrtDigits, c = i - k * kCrtDigits;
                    t[c * kCrtSlots + k] = (int8_t)(cwd[x] >> (8 * e));
                }
        }
        if (tid < kCrtDigits * 8) t[(tid >> 3) * kCrtSlots + kCrtSlots - 8 + (tid & 7)] = 0;
        if (tid < n) {
#pragma unroll
            for (int b = 0; b < 8; b++) wt[tid][b] = (double)(int8_t)(ctb[b >> 2] >> (8 * (b & 3)));
            wt[tid][8] = (double)cc1;
            wt[tid][9] = (double)cq;
            wt[tid][10] = 1.0 / (double)cq;
            wt[tid][11] = 0.0;
        }
        if (tid < 64) ((uint32_t *)&fxl[0][0][0])[tid] = cfx;
        ((uint32_t *)&Yl[0][0])[tid] = 0u;
        ((uint32_t *)&Yl[0][0])[tid + 512] = 0u;
    }
    auto lds_barrier = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
    lds_barrier();

    v4i acc[MBW][kLsNB];
#pragma unroll
    for (int i = 0; i < MBW; i++)
#pragma unroll
        for (int nb = 0; nb < kLsNB; nb++) acc[i][nb] = v4i{0, 0, 0, 0};

    // one group of kLsPre chunks from kc0 (within a staged phase, no barrier)
    auto group = [&](int kc0) {
        const int lc0 = kc0 % kLsPhase;
#pragma unroll
        for (int p = 0; p < kLsPre; p++) {
            const int kc = kc0 + p;
            v4i bf[8];
#pragma unroll
            for (int b = 0; b < 8; b++)
                bf[b] = *(const v4i *)&rT[c16 * kLsColPitch + b * kLsRowPitch + 64 * (lc0 + p) + 16 * g16];
            // the row-sum column: ones for k < K (K is a multiple of 16)
            const int one = K - (64 * kc + 16 * g16) > 0 ? 0x01010101 : 0;
            const v4i ones = v4i{one, one, one, one};
            // the products read abuf[p] before the load of chunk kc + kLsPre
            // replaces it, so the loop carries A in fixed registers
#pragma unroll
            for (int i = 0; i < MBW; i++) {
#pragma unroll
                for (int nb = 0; nb < 8; nb++)
                    acc[i][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(abuf[p][i], bf[nb], acc[i][nb], 0, 0, 0);
                acc[i][8] = __builtin_amdgcn_mfma_i32_16x16x64_i8(abuf[p][i], ones, acc[i][8], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < MBW; i++) abuf[p][i] = aload(i, kc + kLsPre);
        }
    };
    // per phase of r: staged (after a barrier: every wave is done with the
    // last phase), then its groups of chunks with no barrier
    for (int c0 = 0; c0 < KCR; c0 += kLsPhase) {
        if (c0 > 0) {
            const int ph = c0 / kLsPhase;
            rload(ph, 0, kRx);
            lds_barrier();
            rstage(ph, 0, kRx);
            lds_barrier();
        }
        const int c1 = min(c0 + kLsPhase, KCR);
        for (int kc0 = c0; kc0 < c1; kc0 += kLsPre) group(kc0);
    }

    // residues: element e of lane (g16, c16) in block m is product row
    // 16 m + 4 g16 + e, i.e. modulus j = 4 m + g16, row e, column c16
#pragma unroll
    for (int i = 0; i < MBW; i++) {
        const int m = wave + kLsWaves * i;
        const int j = 4 * m + g16;
        if (m >= MB || j >= n) continue;
        double w[kLsW];
#pragma unroll
        for (int x = 0; x < kLsW; x += 2) {
            const auto v = *(const double2 *)&wt[j][x];
            w[x] = v.x;
            w[x + 1] = v.y;
        }
#pragma unroll
        for (int e = 0; e < 4; e++) {
            double y = w[8] * (double)acc[i][8][e];
#pragma unroll
            for (int b = 0; b < 8; b++) y = __builtin_fma(w[b], (double)acc[i][b][e], y);
            // |y| < 2^41: y w[10] is within 2^-12 of y / q, so the rounding
            // to an integer (the 1.5 * 2^52 sum) gives round(y / q)
            const double kq = __builtin_fma(y, w[10], kRoundMagic) - kRoundMagic;
            Yl[e * 16 + c16][j] = (int8_t)(int)__builtin_fma(-w[9], kq, y);
        }
    }
    __syncthreads();

    // the CRT of the workgroup's 64 entries: wave cw < 2 takes entries
    // 32 cw + l32 (row 2 cw + l32 / 16, column l32 % 16)
    if (wave >= 2) return;
    const int ent = 32 * wave + l32;
    v4i dig[KS][NB], fx[KS], ua[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
            const int c = 32 * nb + l32;
            dig[ks][nb] = c < kCrtDigits ? dT[c][2 * ks + h] : v4i{0, 0, 0, 0};
        }
        fx[ks] = l32 < 8 ? fxl[ks][h][l32 & 3] : v4i{0, 0, 0, 0};
        ua[ks] = *(const v4i *)&Yl[ent][32 * ks + 16 * h];
    }
    // F = sum_k y_k c_k from the four digit sums (rows 0-3, repeated in 4-7)
    v16i fs = v16i{0};
#pragma unroll
    for (int ks = 0; ks < KS; ks++) fs = __builtin_amdgcn_mfma_i32_32x32x32_i8(fx[ks], ua[ks], fs, 0, 0, 0);
    const int64_t F = (int64_t)fs[0] + (int64_t)fs[1] * 256 + (int64_t)fs[2] * 65536 + (int64_t)fs[3] * 16777216;
    const int64_t r64 = (F + (1ll << 30)) >> 31;
    const int64_t fr = F - r64 * (1ll << 31);
    const bool near_half = fr < -(1ll << 30) + (1ll << 21) || fr >= (1ll << 30) - (1ll << 21);
    const int r = (int)r64;
    const int rlo = ((r + 127) & 255) - 127;
    const int rhi = (r - rlo) >> 8;
#pragma unroll
    for (int t = 0; t < 2; t++) {
        const int k = n + t, val = t ? -rhi : -rlo;
        const int ks_k = k >> 5, h_k = (k >> 4) & 1, x_k = (k >> 2) & 3, sh = 8 * (k & 3);
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
#pragma unroll
            for (int x = 0; x < 4; x++)
                if (ks == ks_k && x == x_k && h == h_k)
                    ua[ks][x] = (int)(((uint32_t)ua[ks][x] & ~(0xffu << sh)) | ((uint32_t)(val & 0xff) << sh));
    }
    v16i accd[NB];
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
        accd[nb] = v16i{0};
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            accd[nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(dig[ks][nb], ua[ks], accd[nb], 0, 0, 0);
    }
    int part[2 * W];
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
        for (int gq = 0; gq < 4; gq++) {
            const v16i &a = accd[nb];
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
    int c16c = 0;
#pragma unroll
    for (int w = 0; w < W; w++) {
        const int t0 = part[2 * w] + c16c;
        const int t1 = part[2 * w + 1] + (t0 >> 16);
        c16c = t1 >> 16;
        wv[w] = __builtin_amdgcn_perm((uint32_t)t1, (uint32_t)t0, 0x05040100u);
    }
    int64_t carry = c16c;
    if (near_half) {
        int64_t bm = 0, bp = 0;
        uint32_t nzm = 0, nzp = 0;
#pragma unroll
        for (int w = 0; w < W; w++) {
            const uint32_t two = (wv[w] << 1) | (w ? (wv[w - 1] >> 31) : 0u);
            const uint32_t pw = w < 16 ? lc.P[w] : 0u;
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
                const int64_t pw = w < 16 ? (int64_t)lc.P[w] : 0;
                c2 += (int64_t)wv[w] + (above ? -pw : pw);
                wv[w] = (uint32_t)c2;
                c2 >>= 32;
            }
            carry += c2;
        }
    }
    const int row = i0 + (ent >> 4), col = ent & 15;
    if (row < M && col < N) {
        int64_t *ce = g.C + ((int64_t)row * N + col) * g.c_limbs;
        const uint32_t sign = (uint32_t)carry;
#pragma unroll
        for (int t = 0; t < RNS_MAX_OUT_LIMBS / 4; t++) {
            uint32_t wd[4];
#pragma unroll
            for (int ii = 0; ii < 4; ii++) {
                const int ia = 8 * t + ii, ib = 8 * t + 4 + ii;
                const uint32_t a0 = ia < W ? wv[ia] : sign, a1 = ib < W ? wv[ib] : sign;
                wd[ii] = h ? a1 : a0;
            }
            const int l = 4 * t + 2 * h;
            if (g.pair_stores) {
                if (l < g.c_limbs) *(v4u *)(ce + l) = v4u{wd[0], wd[1], wd[2], wd[3]};
            } else {
                if (l < g.c_limbs) ce[l] = (int64_t)(((uint64_t)wd[1] << 32) | wd[0]);
                if (l + 1 < g.c_limbs) ce[l + 1] = (int64_t)(((uint64_t)wd[3] << 32) | wd[2]);
            }
        }
    }
}

int launch_lift_step(const StepConsts &lc, const CrtDigits &cd, int ksteps, int nblocks, const int8_t *a,
                     const int64_t *r, int64_t M, int64_t N, int64_t K, int64_t *C, int32_t c_limbs,
                     uint32_t *status, hipStream_t s) {
    const int n = lc.n;
    if (n < 1 || n > kMaxPrimes || M < 1 || N < 1 || N > 16 || K < 16 || K % 16 || K > RNS_LIFT_K_MAX ||
        M > (1 << 30) || (reinterpret_cast<uintptr_t>(a) & 15) || !r || !C || !status || c_limbs < 1 ||
        c_limbs > RNS_MAX_OUT_LIMBS || ksteps < 1 || ksteps > 2 || nblocks < 1 || nblocks > 2 ||
        n + 2 > 32 * ksteps)
        return RNS_E_ARG;
    LiftArgs g{};
    g.a = a;
    g.r = r;
    g.C = C;
    g.status = status;
    g.M = (int32_t)M;
    g.N = (int32_t)N;
    g.K = (int32_t)K;
    g.KC = (int32_t)((K + 63) / 64);
    g.c_limbs = c_limbs;
    g.pair_stores = (reinterpret_cast<uintptr_t>(C) % 16 == 0 && c_limbs % 2 == 0) ? 1 : 0;
    const int mb = (4 * n + 15) / 16, mbw = (mb + kLsWaves - 1) / kLsWaves;
    const dim3 grid((unsigned)((M + kLsRows - 1) / kLsRows)), block(64 * kLsWaves);
#define RNS_LS(MBW_, KS_, NB_) hipLaunchKernelGGL((lift_step_kernel<MBW_, KS_, NB_>), grid, block, 0, s, g, lc, cd)
    if (mbw == 1) {
        if (ksteps == 1) { if (nblocks == 1) RNS_LS(1, 1, 1); else RNS_LS(1, 1, 2); }
        else { if (nblocks == 1) RNS_LS(1, 2, 1); else RNS_LS(1, 2, 2); }
    } else {
        if (ksteps == 1) { if (nblocks == 1) RNS_LS(2, 1, 1); else RNS_LS(2, 1, 2); }
        else { if (nblocks == 1) RNS_LS(2, 2, 1); else RNS_LS(2, 2, 2); }
    }
#undef RNS_LS
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

}  // namespace rns
