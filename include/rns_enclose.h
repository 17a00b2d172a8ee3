/*
 * rns_enclose.h -- floating-point front and back end of the exact product:
 * a pair (lo, hi) of IEEE matrices with lo <= A @ B <= hi entrywise, where
 * A @ B is evaluated in exact real arithmetic (enclosure-gemm).
 *
 * The method (enclosure-gemm, "Method"): each operand is scaled by a power of
 * two into two's-complement integers of up to four int64 limbs; the integer
 * product is computed exactly by rns_gemm (residues mod primes below 256, one
 * INT8 product per prime, one reconstruction); the exact integer S and its
 * binary exponent Q are then rounded outward once, by bit manipulation
 * (enclosure-gemm, "Method": the top significand bits of S, the remainder
 * deciding between lo == hi and one representable step apart; overflow
 * saturates to the largest finite value inward and to infinity outward; the
 * encoding is contiguous across the subnormal boundary).
 *
 * Scaling.  Every binary64 value is a rational x = odd * 2^t.  The scale of an
 * operand is its coarsest lossless one, F = -min t over its nonzero entries,
 * so x * 2^F is an integer for every entry and the integer product times
 * 2^-(F_A + F_B) is the real product.  Operands whose exponent spread does not
 * fit the 256-bit fixed point, or whose product does not fit the residue
 * range, are rejected (RNS_E_CAPACITY): this library returns only the tight
 * bracket of the lossless regime.
 *
 * Conventions are those of rns_gemm.h: device pointers owned by the caller,
 * asynchronous launches on the caller's stream, 0 on success and a negative
 * RNS_E_* code on failure with nothing written.  Matrices are row-major and
 * contiguous: A is double [M][K], B is double [K][N], lo and hi are [M][N]
 * of the output format.  binary32 operands are passed as their (exact)
 * binary64 values with out_format 32.
 */
#ifndef RNS_ENCLOSE_H
#define RNS_ENCLOSE_H

#include "rns_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* An operand had an infinite or NaN entry (enclosure-gemm, "Requirements and
 * limits": non-finite operands raise rather than propagate). */
#define RNS_E_NONFINITE (-7)

/* Device workspace of rns_fp64_stats, in bytes. */
#define RNS_FP_STATS_WS_BYTES 16384

/* The exponent-field reductions that plan one operand (enclosure-gemm,
 * "Method": planning an operand reads reductions over its exponent field). */
typedef struct rns_fp_stats {
    int32_t max_msb;     /* largest exponent of a leading bit, over nonzero finite entries */
    int32_t min_lsb;     /* smallest exponent of a lowest set bit, over the same entries */
    int32_t nonzero;     /* 1 if some entry is finite and nonzero */
    int32_t nonfinite;   /* 1 if some entry is infinite or NaN */
} rns_fp_stats_t;

/*
 * rns_fp64_stats -- the reductions above over `count` doubles X (device),
 * written to *stats (a DEVICE pointer).  ws: device workspace of at least
 * RNS_FP_STATS_WS_BYTES.  Two kernels on `stream`, no synchronisation.
 * count == 0 gives {INT32_MIN, INT32_MAX, 0, 0}.
 * Returns RNS_OK, RNS_E_ARG, RNS_E_WORKSPACE or RNS_E_HIP.
 */
int rns_fp64_stats(const double *X, int64_t count, rns_fp_stats_t *stats,
                   void *ws, size_t ws_bytes, hipStream_t stream);

/* A plan for one enclosure product.  Plain data, filled by rns_enclose_plan. */
typedef struct rns_enclose_plan {
    rns_plan_t plan;     /* the residue plan of the integer product */
    int32_t fa, fb;      /* A_int = A * 2^fa, B_int = B * 2^fb, both exact */
    int32_t a_bits, b_bits;   /* |A_int| < 2^a_bits, |B_int| < 2^b_bits */
    int32_t a_limbs, b_limbs; /* int64 limbs of the integer operands (1..4) */
    int32_t c_limbs;     /* limbs of the exact integer product S */
    int32_t q;           /* A @ B == S * 2^-q */
    int32_t out_format;  /* 64: binary64 lo/hi, 32: binary32 lo/hi */
    int32_t zero;        /* 1 when an operand is all zero (the product is 0) */
} rns_enclose_plan_t;

/*
 * rns_enclose_plan -- plan A @ B from host copies of both operands' stats.
 * K in 0..2^17, out_format 64 or 32.  The residue plan takes the primes below
 * 256 when they suffice, else the prime-power moduli (rns_gemm.h; up to 362.8
 * bits, K <= 2^17 - 1).  Returns RNS_OK, RNS_E_ARG, RNS_E_K, RNS_E_NONFINITE,
 * or RNS_E_CAPACITY when the scaled operands need more than four limbs or
 * their product exceeds the range of all 54 prime powers.
 */
int rns_enclose_plan(int64_t K, const rns_fp_stats_t *a, const rns_fp_stats_t *b,
                     int32_t out_format, rns_enclose_plan_t *out);

/*
 * rns_enclose_workspace_size -- device bytes needed by rns_mm_enclose: the
 * exact integer product plus rns_gemm's workspace.  Returns RNS_OK,
 * RNS_E_ARG or RNS_E_K.
 */
int rns_enclose_workspace_size(const rns_enclose_plan_t *ep, int64_t M, int64_t N, int64_t K,
                               size_t *bytes);

/*
 * rns_mm_enclose -- lo, hi (device, [M][N] of double or float by
 * ep->out_format) with lo <= A @ B <= hi exactly, lo the largest and hi the
 * smallest such format values; lo == hi when the product is representable.
 * An exact zero gives +0.0 in both.  ep must come from rns_enclose_plan on
 * the stats of these very operands.  The steps of rns_gemm on `stream`, with
 * the residue split reading the binary64 entries and scaling them into
 * integer limbs itself, then the outward rounding.
 * Returns RNS_OK, RNS_E_ARG, RNS_E_K, RNS_E_WORKSPACE or RNS_E_HIP.
 */
int rns_mm_enclose(const rns_enclose_plan_t *ep, int64_t M, int64_t N, int64_t K,
                   const double *A, const double *B, void *lo, void *hi,
                   void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * rns_mm_enclose_nt -- the same for A @ Bt^T with Bt given as double [N][K]
 * row-major (no transposed copy is made; enclosure-gemm, "Usage").  Stats
 * and plan as for rns_mm_enclose, with Bt's stats standing for B's.
 */
int rns_mm_enclose_nt(const rns_enclose_plan_t *ep, int64_t M, int64_t N, int64_t K,
                      const double *A, const double *Bt, void *lo, void *hi,
                      void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * rns_fp64_to_limbs -- floor(X * 2^F) for `count` doubles as `limbs` int64
 * limbs each (device [count][limbs], two's complement).  The caller
 * guarantees |floor(X * 2^F)| < 2^(64 limbs - 1).  limbs in 1..4.
 * Returns RNS_OK, RNS_E_ARG or RNS_E_HIP.
 */
int rns_fp64_to_limbs(const double *X, int64_t count, int32_t F, int32_t limbs,
                      int64_t *out, hipStream_t stream);

/*
 * rns_round_outward -- (lo, hi) of S * 2^-q entrywise for `count` integers S
 * of s_limbs limbs (device [count][s_limbs]), out_format 64 or 32, by bit
 * manipulation only.  s_limbs in 1..8.  Returns RNS_OK, RNS_E_ARG or
 * RNS_E_HIP.
 */
int rns_round_outward(const int64_t *S, int64_t count, int32_t s_limbs, int32_t q,
                      int32_t out_format, void *lo, void *hi, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RNS_ENCLOSE_H */
