/*
 * Schoolbook exact integer GEMM over multi-limb two's-complement operands.
 *
 * TEST INFRASTRUCTURE ONLY: built and loaded by the test suite, the smoke
 * check and the cpu_baseline leg of the benchmark; never by the product path.
 * It shares no source, header or table with the HIP library.
 *
 * What it computes is the plain definition that the residue method reaches
 * exactly (Ozaki Scheme II paper, §3.1: the integer products are exact and
 * there is a single reconstruction at the end):
 *
 *     C[i][j] = sum_k A[i][k] * B[k][j]        over the integers.
 *
 * Operand format (enclosure-gemm, "Method": two's-complement integers of up
 * to four int64 limbs): element-major, limb-minor, little-endian limbs; lower
 * limbs are unsigned, the top limb is signed.
 *
 *   A: int64 [M][K][la]    B: int64 [K][N][lb]    C: int64 [M][N][lc]
 *
 * Each product is formed from the operands' magnitudes by the schoolbook
 * 64x64->128 rule and added to (or subtracted from) a two's-complement
 * accumulator of la+lb+1 limbs, which cannot overflow for K <= 2^17.
 * Rows of C are independent and are shared among OpenMP threads.
 *
 * Returns 0, or 1 when some C[i][j] does not fit lc limbs (that entry is then
 * written truncated), or 2 on bad arguments.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MAXL 8

typedef unsigned __int128 u128;

/* magnitude (l limbs, unsigned) and sign of an l-limb two's-complement value */
static int magnitude(const int64_t *x, int l, uint64_t *mag)
{
    int neg = x[l - 1] < 0;
    if (!neg) {
        for (int i = 0; i < l; i++) mag[i] = (uint64_t)x[i];
        return 0;
    }
    /* two's-complement negation: invert every limb, then add one */
    uint64_t carry = 1;
    for (int i = 0; i < l; i++) {
        uint64_t v = ~(uint64_t)x[i];
        mag[i] = v + carry;
        carry = (carry && mag[i] == 0) ? 1 : 0;
    }
    return 1;
}

/* acc (w limbs, two's complement) += sign * p (np limbs, unsigned) */
static void accumulate(uint64_t *acc, int w, const uint64_t *p, int np, int negative)
{
    if (!negative) {
        uint64_t carry = 0;
        for (int i = 0; i < w; i++) {
            uint64_t pi = i < np ? p[i] : 0;
            u128 s = (u128)acc[i] + pi + carry;
            acc[i] = (uint64_t)s;
            carry = (uint64_t)(s >> 64);
        }
    } else {
        uint64_t borrow = 0;
        for (int i = 0; i < w; i++) {
            uint64_t pi = i < np ? p[i] : 0;
            u128 d = (u128)acc[i] - pi - borrow;
            acc[i] = (uint64_t)d;
            borrow = (uint64_t)(d >> 64) ? 1 : 0;
        }
    }
}

int oracle_gemm(int64_t M, int64_t N, int64_t K,
                const int64_t *A, int la, const int64_t *B, int lb,
                int64_t *C, int lc)
{
    if (M < 0 || N < 0 || K < 0 || la < 1 || lb < 1 || lc < 1 ||
        la > MAXL || lb > MAXL || lc > 2 * MAXL + 1)
        return 2;
    if (M == 0 || N == 0) return 0;

    /* B transposed to [N][K][lb] so that the k loop walks memory in order;
     * only the storage changes, not the arithmetic. */
    int64_t *Bt = (int64_t *)malloc((size_t)(N * K * lb + 1) * sizeof(int64_t));
    if (!Bt) return 2;
    for (int64_t k = 0; k < K; k++)
        for (int64_t j = 0; j < N; j++)
            memcpy(Bt + (j * K + k) * lb, B + (k * N + j) * lb, (size_t)lb * sizeof(int64_t));

    const int w = la + lb + 1;
    int overflow = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : overflow)
    for (int64_t i = 0; i < M; i++) {
        uint64_t ma[MAXL], mb[MAXL], p[2 * MAXL], acc[2 * MAXL + 1];
        for (int64_t j = 0; j < N; j++) {
            memset(acc, 0, sizeof(acc));
            for (int64_t k = 0; k < K; k++) {
                int sa = magnitude(A + (i * K + k) * la, la, ma);
                int sb = magnitude(Bt + (j * K + k) * lb, lb, mb);
                /* schoolbook product of the magnitudes */
                memset(p, 0, sizeof(uint64_t) * (size_t)(la + lb));
                for (int x = 0; x < la; x++) {
                    uint64_t carry = 0;
                    for (int y = 0; y < lb; y++) {
                        u128 t = (u128)ma[x] * mb[y] + p[x + y] + carry;
                        p[x + y] = (uint64_t)t;
                        carry = (uint64_t)(t >> 64);
                    }
                    p[x + lb] = carry;
                }
                accumulate(acc, w, p, la + lb, sa ^ sb);
            }
            /* the value fits lc limbs iff every limb above lc-1 is the sign
             * extension of limb lc-1 */
            int64_t *c = C + (i * N + j) * lc;
            for (int l = 0; l < lc; l++)
                c[l] = (int64_t)(l < w ? acc[l] : ((int64_t)acc[w - 1] < 0 ? ~0ull : 0ull));
            uint64_t ext = ((int64_t)c[lc - 1] < 0) ? ~0ull : 0ull;
            for (int l = lc; l < w; l++)
                if (acc[l] != ext) overflow = 1;
        }
    }
    free(Bt);
    return overflow;
}
