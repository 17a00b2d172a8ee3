/*
 * rns_solve.h -- the GPU part of the exact rational solve A x = b by Dixon
 * p-adic lifting on the residue engine (exact-solve).
 *
 * The method (exact-solve, "Method"): with B = A^-1 mod P for a squarefree
 * product P of primes below 256, r_0 = b, x_i = B r_i mod P and
 * r_{i+1} = (r_i - A x_i) / P, the digits x_i give x mod P^m, from which the
 * rational solution is reconstructed once P^m exceeds twice the Hadamard
 * bound on numerator and denominator.  The parts:
 *   - the batched modular inverse: A^-1 mod q_j for every prime by
 *     Gauss-Jordan elimination of the augmented matrix [A | I], in panels of
 *     columns (a panel kernel per prime, then a rank-update of the rest;
 *     up to 4096 rows) or one step per launch pair above, reductions by
 *     exact floating-point rounding steps or Barrett;
 *   - the lift: per step, x_i = B r_i mod P from one INT8 product per prime
 *     and the wide digit by the CRT, and the residual update in one limb as
 *     (r_i - A x_i) * P^-1 mod 2^64 (P odd).  For n a multiple of 16 and at
 *     most 4 right-hand sides a step is two kernels (every prime's dot
 *     products and the digit in one, the update and the next residues in the
 *     other); otherwise it runs through rns_gemm_batched_residue;
 *   - the reconstruction's bulk work (exact-solve, "Method", where it is a CPU
 *     stage): the p-adic values in binary (rns_padic_chunks), the one
 *     modular multiply per numerator (rns_chunk_modmul) and the bound test
 *     (rns_chunk_bound), as exact residue products and chunk passes.
 * The host stage (a component's rational reconstruction by the extended
 * Euclidean algorithm, tables, and the same multiply on host threads) is
 * declared at the end of this header.
 *
 * Conventions of rns_gemm.h: device pointers owned by the caller,
 * asynchronous launches on the caller's stream, 0 on success and a negative
 * RNS_E_* code on failure with nothing written.  A is int64 [n][n], b and r
 * int64 [n][c], row-major.  Range (exact-solve, "Requirements and limits"):
 * n * max|A_ij| < 2^63 keeps the residual in one signed limb; n <= 2^17.
 */
#ifndef RNS_SOLVE_H
#define RNS_SOLVE_H

#include "rns_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Errors of the host stage, beside those of rns_gemm.h. */
#define RNS_E_RECONSTRUCT (-8) /* no fraction within the bounds matches the residue */
#define RNS_E_HOSTLIB (-9)     /* the host big-integer library (libgmp.so.10) is not available */

/*
 * rns_inverse_workspace_size -- device bytes of rns_batched_inverse for
 * n_primes primes and an n x n matrix: the augmented matrices as bytes
 * ([n_primes][n][2n], residues in [0, q)) plus per-step pivot rows and
 * columns.  Returns RNS_OK or RNS_E_ARG.
 */
int rns_inverse_workspace_size(int32_t n_primes, int64_t n, size_t *bytes);

/*
 * rns_batched_inverse -- Gauss-Jordan elimination of [A mod q_j | I] for every
 * prime q_j = primes[j] (host array of n_primes distinct primes below 256).
 * A: device int64 [n][n].  singular: device int32 [n_primes], set to 1 where
 * A is singular mod q_j (that prime's inverse is then unspecified), else 0.
 * The inverses stay in ws for rns_inverse_planes.  2n + 2 launches.
 * Returns RNS_OK, RNS_E_ARG, RNS_E_K (n > 2^17), RNS_E_WORKSPACE or RNS_E_HIP.
 */
int rns_batched_inverse(const int32_t *primes, int32_t n_primes, int64_t n, const int64_t *A,
                        int32_t *singular, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * rns_inverse_planes -- the balanced int8 residue planes of the inverses left
 * in ws by rns_batched_inverse (same primes, n, ws): plane t of `planes`
 * (device int8 [n_sel][n][n]) is A^-1 mod primes[select[t]], select a host
 * array of n_sel indices.  The planes are in the layout of A_res of
 * rns_gemm_batched_residue.  Returns RNS_OK, RNS_E_ARG or RNS_E_HIP.
 */
int rns_inverse_planes(const int32_t *primes, int32_t n_primes, int64_t n, const int32_t *select,
                       int32_t n_sel, int8_t *planes, const void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * rns_plan_from_moduli -- a plan over the given moduli (host array, any
 * order, distinct prime powers up to 256), with no operand bound and the
 * given k_max (1..2^17, 2^17 - 1 with 256).  For the lift: the primes for
 * which A is invertible.  Returns RNS_OK or RNS_E_ARG.
 */
int rns_plan_from_moduli(const int32_t *moduli, int32_t n, int64_t k_max, rns_plan_t *out);

/*
 * rns_lift_workspace_size -- device bytes of rns_dixon_lift: the residual and
 * the batched-residue product's workspace.  Returns RNS_OK, RNS_E_ARG or
 * RNS_E_K.
 */
int rns_lift_workspace_size(const rns_plan_t *plan, int64_t n, int64_t c, size_t *bytes);

/*
 * rns_dixon_lift -- `steps` Dixon steps from r_0 = b.
 * plan: odd primes only (P odd), k_max >= n.  Binv: device int8
 * [plan->n_primes][n][n], the balanced residues of A^-1 mod each prime in
 * plan order (rns_inverse_planes).  digits: device int64
 * [steps][n][c][d_limbs], d_limbs >= plan->out_limbs_min: digit i is the
 * balanced representative of B r_i mod P.  Both step forms give the same
 * digits; ws (rns_lift_workspace_size bytes) holds the residual and the
 * step's scratch.  Returns RNS_OK, RNS_E_ARG (also for an even modulus),
 * RNS_E_K, RNS_E_OUT_LIMBS, RNS_E_WORKSPACE or RNS_E_HIP.
 */
int rns_dixon_lift(const rns_plan_t *plan, int64_t n, int64_t c, const int8_t *Binv, const int64_t *A,
                   const int64_t *b, int32_t steps, int64_t *digits, int32_t d_limbs,
                   void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * rns_padic_chunks_workspace_size -- device bytes of rns_padic_chunks.
 * Returns RNS_OK, RNS_E_ARG or RNS_E_K.
 */
int rns_padic_chunks_workspace_size(int64_t T, int32_t m, int64_t count, int32_t d_limbs, int32_t P_bits,
                                    size_t *bytes);

/*
 * rns_padic_chunks -- the p-adic values X_idx = sum_{s < m} digits[s][idx] P^s
 * of every component, as T little-endian 32-bit two's-complement chunks:
 * layout 0: out is device uint32 [count][T]; layout 1: out is device int64
 * [T][count], each chunk's value (the top chunk signed, the others in
 * [0, 2^32)), the operand layout of rns_chunk_modmul.  digits: device int64 [m][count][d_limbs]
 * (rns_dixon_lift's output, |digit| < 2^(P_bits - 1)); pow: device int64
 * [T][m], pow[t][s] = chunk t of P^s (in [0, 2^32)), built by the caller.
 * 32 T must exceed the bit length of P^m (then |X| <= (P^m - 1)/2 fits).
 * The sum is two exact residue products (the digits' low three limbs and
 * the rest) and one carry pass: the radix conversion of the host stage on
 * the GPU.  Returns RNS_OK, RNS_E_ARG, RNS_E_K (m > 2^17), RNS_E_WORKSPACE or
 * RNS_E_HIP.
 */
int rns_padic_chunks(const int64_t *pow, int64_t T, int32_t m, const int64_t *digits, int64_t count, int32_t d_limbs,
                     int32_t P_bits, int32_t layout, void *out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * rns_chunk_modmul_workspace_size -- device bytes of rns_chunk_modmul.
 * Returns RNS_OK, RNS_E_ARG or RNS_E_K.
 */
int rns_chunk_modmul_workspace_size(int64_t T, int64_t count, int64_t TD, int64_t Tmu, int64_t TP, int64_t s1c,
                                    int64_t k2c, int64_t Tw, size_t *bytes);

/*
 * rns_chunk_modmul -- the one modular multiply per numerator (exact-solve,
 * "Method": the numerators are D x mod P^m for the common denominator D) as a
 * Barrett step on the GPU, for every component at once.  With the
 * non-negative integers D, mu and Pm given by their 32-bit chunks (device
 * int64 vectors Dc[TD], muc[Tmu], Pmc[TP], values in [0, 2^32)) and X_idx the
 * signed integer of the chunks X[0..T)[idx] (device int64 [T][count], layout
 * 1 of rns_padic_chunks), it writes
 *   Y = D X,  a = floor(Y / 2^(32 s1c)),
 *   q = floor((a mu + 2^(32 k2c - 1)) / 2^(32 k2c)),
 *   out[idx] = (Y - q Pm) mod 2^(32 Tw)   (device uint32 [count][Tw], two's complement).
 * With mu = floor(2^(32 (s1c + k2c)) / Pm), 2^(32 s1c) <= Pm 2^-G and
 * |a| <= 2^(32 k2c - G) for G >= 2, |Y / Pm - q| < 1/2 + 2^(1 - G): the result
 * is D X mod Pm up to one correction by +-Pm, which the caller makes (and Tw
 * chunks must hold Pm in two's complement).  Three exact residue products
 * with Toeplitz matrices of the constants' chunks and three carry passes.
 * Requires Tw <= T + TD, s1c < T + TD, k2c < T + TD - s1c + Tmu, and the
 * contraction lengths T, T + TD - s1c and T + TD - s1c + Tmu - k2c at most
 * 2^17.  Returns RNS_OK, RNS_E_ARG, RNS_E_K, RNS_E_WORKSPACE or RNS_E_HIP.
 */
int rns_chunk_modmul(const int64_t *X, int64_t T, int64_t count, const int64_t *Dc, int64_t TD, const int64_t *muc,
                     int64_t Tmu, const int64_t *Pmc, int64_t TP, int64_t s1c, int64_t k2c, int64_t Tw,
                     uint32_t *out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * rns_chunk_bound -- the bound test of the numerators (exact-solve, "Method":
 * a numerator over the common denominator is accepted when it lies within
 * the bound): ok[idx] = 1 and num[idx] = w_idx as w_limbs int64 two's-complement
 * limbs when |w_idx| <= B, else ok[idx] = 0 and num[idx] = 0.  w: device
 * uint32 [count][Tw] two's complement (rns_chunk_modmul's output); B: device
 * uint32 [TB], a non-negative integer; num: device int64 [count][w_limbs]
 * (w_limbs must hold B plus a sign); ok: device int32 [count]; used: device
 * int32 [count], the limbs that hold an accepted w with its sign (at most
 * w_limbs; 0 when not accepted), so a caller may copy fewer.  For
 * rns_chunk_modmul's output with G >= 63 (|w| < (1/2 + 2^-62) Pm, w congruent
 * to D X) and Pm > 2 B (1 + 2^-60), |w| <= B holds exactly when it holds for
 * the balanced residue of D X mod Pm, and then the two are equal: no
 * correction by +-Pm is needed.  Returns RNS_OK, RNS_E_ARG or RNS_E_HIP.
 */
int rns_chunk_bound(const uint32_t *w, int64_t Tw, int64_t count, const uint32_t *B, int64_t TB, int64_t *num,
                    int32_t w_limbs, int32_t *ok, int32_t *used, hipStream_t stream);

/*
 * ---- host stage (exact-solve, "Method": the final rational reconstruction is
 * a CPU stage: a common denominator, then one modular multiply per numerator).
 * Host pointers only; no device memory is touched.  Big integers cross as
 * little-endian uint64 magnitudes (unsigned) or two's-complement int64 limbs
 * with a signed top limb (signed).  Big-integer arithmetic is GMP's, opened at
 * first use from libgmp.so.10; without it these calls return RNS_E_HOSTLIB.
 */

/* rns_host_bigint_available -- 1 when libgmp.so.10 could be opened, else 0. */
int rns_host_bigint_available(void);

/*
 * rns_padic_numerators -- for each t < n_index, the component idx = index[t]:
 *   X = sum_{s < steps} digits[s][idx] * P^s   (digits: host int64
 *       [steps][count][d_limbs], two's complement, the layout rns_dixon_lift
 *       writes for [n][c] components),
 *   w = D * X mod P^steps, taken in (-P^steps/2, P^steps/2),
 * and ok[t] = 1 with num[t] = w (int64 [n_index][w_limbs], two's complement)
 * when |w| <= bound, else ok[t] = 0 and num[t] = 0.  With D = 1 and bound =
 * (P^steps - 1)/2 every X is returned as is.  Accepting |w| <= bound is the
 * common-denominator test: if X = a/e (mod P^steps) with |D a| <= bound and
 * P^steps > bound * (e + 1), an accepted w satisfies |w e - D a| < P^steps
 * and w e = D a (mod P^steps), so w e = D a exactly.  P: odd, > 1 (magnitude, p_limbs); D > 0 (den_limbs); bound
 * (b_limbs) must satisfy bound < 2^(64 w_limbs - 1).  threads = 0 uses up to
 * 16 host threads.  Returns RNS_OK, RNS_E_ARG, RNS_E_OUT_LIMBS (bound too
 * wide for w_limbs) or RNS_E_HOSTLIB.
 */
int rns_padic_numerators(const int64_t *digits, int32_t steps, int64_t count, int32_t d_limbs,
                         const int64_t *index, int64_t n_index, const uint64_t *P, int32_t p_limbs,
                         const uint64_t *D, int32_t den_limbs, const uint64_t *bound, int32_t b_limbs,
                         int64_t *num, int32_t w_limbs, int32_t *ok, int32_t threads);

/*
 * rns_pow_table -- the table of rns_padic_chunks on the host: out[t][s] =
 * 32-bit chunk t of P^s for s < m, t < T (host int64 [T][m]; P a magnitude of
 * p_limbs limbs).  Returns RNS_OK, RNS_E_ARG (also when P^(m-1) does not fit
 * T chunks) or RNS_E_HOSTLIB.
 */
int rns_pow_table(const uint64_t *P, int32_t p_limbs, int32_t m, int64_t T, int64_t *out);

/*
 * rns_pow2_quotient -- q = floor(2^e / d) for a magnitude d > 0 (d_limbs
 * limbs), written as q_limbs limbs: the reciprocal of rns_chunk_modmul's
 * Barrett step.  Returns RNS_OK, RNS_E_ARG, RNS_E_OUT_LIMBS (q does not fit)
 * or RNS_E_HOSTLIB.
 */
int rns_pow2_quotient(int64_t e, const uint64_t *d, int32_t d_limbs, uint64_t *q, int32_t q_limbs);

/*
 * rns_reduce_fractions -- N_i / D in lowest terms for every i: with
 * g = gcd(|N_i|, D), num_out[i] = N_i / g (int64 [count][limbs], two's
 * complement, the layout of num) and den_out[i] = D / g (uint64
 * [count][d_limbs] magnitudes); up to 16 host threads (or `threads`).
 * Returns RNS_OK, RNS_E_ARG, RNS_E_OUT_LIMBS or RNS_E_HOSTLIB.
 */
int rns_reduce_fractions(const int64_t *num, int64_t count, int32_t limbs, const uint64_t *D, int32_t d_limbs,
                         int64_t *num_out, uint64_t *den_out, int32_t threads);

/*
 * rns_chunk_numerators -- rns_padic_numerators with the p-adic values given
 * as binary chunks (host uint32 [count][T], little-endian two's complement,
 * rns_padic_chunks's output) and P^steps as the modulus.  Returns RNS_OK,
 * RNS_E_ARG, RNS_E_OUT_LIMBS or RNS_E_HOSTLIB.
 */
int rns_chunk_numerators(const uint32_t *chunks, int64_t T, int64_t count, const int64_t *index, int64_t n_index,
                         const uint64_t *P, int32_t p_limbs, int32_t steps, const uint64_t *D, int32_t den_limbs,
                         const uint64_t *bound, int32_t b_limbs, int64_t *num, int32_t w_limbs, int32_t *ok,
                         int32_t threads);

/*
 * rns_rational_reconstruct -- the fraction N/d with |N| <= Nb, 0 < d <= Db and
 * N = d * u (mod M), from the remainder sequence of the extended Euclidean
 * algorithm on (M, u mod M), stopped at the first remainder not above Nb; it
 * is unique when M > 2 * Nb * Db.  u, M (> 0), Nb, Db: magnitudes.  Writes N
 * (two's complement, num_limbs) and d (magnitude, den_limbs), not necessarily
 * in lowest terms.  Returns RNS_OK, RNS_E_ARG, RNS_E_RECONSTRUCT (no such
 * fraction), RNS_E_OUT_LIMBS or RNS_E_HOSTLIB.
 */
int rns_rational_reconstruct(const uint64_t *u, int32_t u_limbs, const uint64_t *M, int32_t m_limbs,
                             const uint64_t *Nb, int32_t nb_limbs, const uint64_t *Db, int32_t db_limbs,
                             int64_t *num, int32_t num_limbs, uint64_t *den, int32_t den_limbs);

#ifdef __cplusplus
}
#endif

#endif /* RNS_SOLVE_H */
