/*
 * rns_gemm.h -- exact integer matrix product computed in residues (gfx950).
 *
 * The product C = A @ B of signed multi-limb integer matrices is computed
 * exactly: every operand entry is reduced to balanced residues modulo primes
 * below 256, one INT8 matrix product per prime is accumulated in int32 and
 * reduced mod that prime, and the exact signed result is rebuilt from its
 * residues by the centered CRT with a rounded quotient (Ozaki Scheme II
 * paper, §3.5.2), with balanced Garner mixed-radix reconstruction
 * (exact-solve, "Method"; enclosure-gemm, "Method") available as
 * rns_reconstruct_garner for the same result (Ozaki Scheme II paper, §3.1:
 * the integer products are exact and the result is reconstructed once).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Integers.  An integer of L limbs is L int64 words, little-endian two's
 *   complement: limbs 0..L-2 are read unsigned, limb L-1 is signed
 *   (enclosure-gemm, "Method": two's-complement integers of up to four int64
 *   limbs).  Matrices are row-major and contiguous with the limbs innermost:
 *   A is [M][K][a_limbs], B is [K][N][b_limbs], C is [M][N][c_limbs].
 * Memory.  Pointers named A, B, C, A_res and ws are DEVICE pointers, owned by
 *   the caller (e.g. allocated through PyTorch).  The library never allocates
 *   or frees device memory.  rns_plan_t is a plain host struct owned by the
 *   caller; it needs no release.
 * Streams.  Every launch is asynchronous on the caller's stream; no entry
 *   point synchronises except rns_status.  Concurrent calls are safe when
 *   they use distinct workspaces.
 * Errors.  0 is success, negative values are failures (RNS_E_*).  All
 *   arguments are validated on the host before anything is launched, so on a
 *   validation error nothing is written.  rns_error_string names a code.
 * Sizes.  M == 0 or N == 0 is a no-op.  K == 0 writes zeros to C.
 */
#ifndef RNS_GEMM_H
#define RNS_GEMM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* There are 54 primes below 256 (2, 3, 5, ..., 251); their product P is a
 * 335-bit number (enclosure-gemm, "Requirements and limits"). */
#define RNS_MAX_PRIMES 54
/* int32 accumulation of products of balanced residues (|r| <= 125) is exact
 * for K <= 2^17 (exact-solve, "Requirements and limits"; enclosure-gemm,
 * "Requirements and limits"). */
#define RNS_K_MAX (1 << 17)
/* operand limbs: up to four (a 256-bit fixed point, enclosure-gemm, "Method") */
#define RNS_MAX_IN_LIMBS 4
/* output limbs: the 54-prime range needs 6 (the pages' signed 384 bits) */
#define RNS_MAX_OUT_LIMBS 8

enum rns_status_code {
    RNS_OK = 0,
    RNS_E_ARG = -1,        /* null pointer, negative size, limbs out of range, bad plan */
    RNS_E_K = -2,          /* K > 2^17, or K above the K the plan was made for */
    RNS_E_CAPACITY = -3,   /* the bound 2*K*2^(a_bits+b_bits) is not below P of all 54 primes */
    RNS_E_OUT_LIMBS = -4,  /* c_limbs < plan->out_limbs_min or > RNS_MAX_OUT_LIMBS */
    RNS_E_WORKSPACE = -5,  /* ws_bytes smaller than rns_workspace_size reports */
    RNS_E_HIP = -6,        /* a HIP launch or copy failed */
    RNS_E_SCRATCH = -10    /* rns_gemm_noalloc: the workspace exceeds RNS_NOALLOC_SCRATCH_BYTES */
};

/* Bits of the status word read by rns_status. */
#define RNS_FLAG_A_RANGE 1u   /* some |A| entry exceeded 2^a_bits */
#define RNS_FLAG_B_RANGE 2u   /* some |B| entry exceeded 2^b_bits */

/* A prime plan.  Plain data, filled by rns_plan or rns_plan_n. */
typedef struct rns_plan {
    int32_t n_primes;        /* primes used, 1..54 */
    int32_t out_limbs_min;   /* limbs that hold every value of (-P/2, P/2] */
    int32_t a_bits;          /* declared |A| <= 2^a_bits; -1 when no bound is declared */
    int32_t b_bits;          /* declared |B| <= 2^b_bits; -1 when no bound is declared */
    int64_t k_max;           /* largest K the plan is valid for */
    double  log2_P;          /* log2 of the product P of the primes used */
    int32_t primes[RNS_MAX_PRIMES];  /* the primes used, largest first; rest 0 */
} rns_plan_t;

/*
 * rns_plan -- choose the primes for |A| <= 2^a_bits, |B| <= 2^b_bits and
 * contraction length K.
 *
 * The entries of C obey |C| <= K * 2^(a_bits+b_bits).  The plan takes the
 * fewest primes, largest first (251, 241, 239, ...), whose product P strictly
 * exceeds 2*K*2^(a_bits+b_bits), so that the balanced representative of C mod P
 * is C itself (exact-solve, "Method": the precision must exceed twice the
 * bound).  Accepts every case of the pages' budget
 * a_bits + b_bits + ceil(log2 K) <= 332 (enclosure-gemm, "Requirements and
 * limits"); the exact limit here is P of all 54 primes > 2*K*2^(a_bits+b_bits).
 *
 * K in 0..2^17 (K = 0 is planned as K = 1); a_bits, b_bits in 0..255.
 * Returns RNS_OK, RNS_E_ARG (null out, bits out of range), RNS_E_K (K out of
 * range) or RNS_E_CAPACITY.  On success out->k_max = max(K, 1).
 */
int rns_plan(int64_t K, int32_t a_bits, int32_t b_bits, rns_plan_t *out);

/*
 * rns_plan_n -- a plan of the n_primes largest primes below 256 (54 = all of
 * them), with no operand bound.  The result of a GEMM under this plan is, by
 * definition, the balanced representative in (-P/2, P/2] of the product mod
 * P: this is the base-P digit of the lift step (exact-solve, "Method").  When
 * P contains 2 (n_primes == 54) the range is (-P/2, P/2]; otherwise it is
 * [-(P-1)/2, (P-1)/2].  k_max = 2^17.  Returns RNS_OK or RNS_E_ARG.
 */
int rns_plan_n(int32_t n_primes, rns_plan_t *out);

/*
 * Moduli of a plan.  RNS_MODULI_PRIMES: the 54 primes below 256 (P up to
 * 2^334.9).  RNS_MODULI_PRIME_POWERS: for each of those primes its largest
 * power not above 256 -- 256, 251, 243, 241, ..., 169, ..., 125, 121, ...,
 * 49, ..., 17 -- whose product is lcm(1..256), about 2^362.8: the INT8 CRT
 * capacity of the Ozaki Scheme II paper (§1.2, §4.2.2).  The moduli are
 * pairwise coprime; residues mod 256 are the int8 values themselves, in
 * [-128, 127], so K <= 2^17 - 1 keeps the int32 accumulation exact
 * (2^17 * 128^2 would reach 2^31).  The other moduli keep their balanced
 * residues (|r| <= 125).  The field `primes` of a plan lists its moduli.
 */
#define RNS_MODULI_PRIMES 0
#define RNS_MODULI_PRIME_POWERS 1

/*
 * rns_plan_moduli -- rns_plan over either modulus set: the fewest moduli,
 * largest first, whose product exceeds 2*K*2^(a_bits+b_bits).  K in 0..2^17
 * (0..2^17-1 for prime powers).  rns_plan(K, a, b, out) is
 * rns_plan_moduli(K, a, b, RNS_MODULI_PRIMES, out).  Returns as rns_plan,
 * and RNS_E_ARG for an unknown kind.
 */
int rns_plan_moduli(int64_t K, int32_t a_bits, int32_t b_bits, int32_t kind, rns_plan_t *out);

/*
 * rns_plan_n_moduli -- rns_plan_n over either modulus set (k_max = 2^17, or
 * 2^17 - 1 for prime powers).  With all 54 prime powers the representative
 * range is (-P/2, P/2] for P = lcm(1..256).  Returns RNS_OK or RNS_E_ARG.
 */
int rns_plan_n_moduli(int32_t n, int32_t kind, rns_plan_t *out);

/*
 * rns_workspace_size -- device workspace bytes needed by rns_gemm
 * (batched_residue == 0) or rns_gemm_batched_residue (batched_residue != 0)
 * for this plan and shape.  The workspace holds the residue planes of both
 * operands and of the product (about n*(M*K + N*K + M*N) bytes plus tile
 * padding; cf. enclosure-gemm, "Requirements and limits" on working memory),
 * a small status area and, when the large 256 x 256 tiling is chosen, a
 * 16 MiB area for the partial residues of tiles that are split over K to
 * balance the last round over the compute units.  Writes the size to *bytes.
 * Returns RNS_OK, RNS_E_ARG or RNS_E_K.
 */
int rns_workspace_size(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                       int32_t batched_residue, size_t *bytes);

/*
 * rns_gemm -- C = A @ B exactly.
 *
 * A: device int64 [M][K][a_limbs], B: device int64 [K][N][b_limbs],
 * C: device int64 [M][N][c_limbs] (written in full, sign-extended),
 * a_limbs, b_limbs in 1..4, c_limbs in plan->out_limbs_min..8,
 * ws: device workspace of ws_bytes >= rns_workspace_size(plan, M, N, K, 0).
 *
 * Three kernels run on `stream`: the residue split of A and B into int8
 * planes, the prime-batched INT8 MFMA product with a fused mod-q epilogue,
 * and the reconstruction: the centered CRT by rounded quotient (Ozaki Scheme
 * II paper, §3.5.2; described under rns_reconstruct below), whose output is
 * bit for bit the one balanced Garner gives (rns_reconstruct_garner).  The
 * result equals the integer product whenever
 * the operands respect the plan's declared bounds; if an entry exceeds its
 * bound, a flag is recorded for rns_status and C is unspecified.
 * Returns RNS_OK, RNS_E_ARG, RNS_E_K (K > plan->k_max), RNS_E_OUT_LIMBS,
 * RNS_E_WORKSPACE or RNS_E_HIP.
 */
int rns_gemm(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
             const int64_t *A, int32_t a_limbs,
             const int64_t *B, int32_t b_limbs,
             int64_t *C, int32_t c_limbs,
             void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * rns_gemm_batched_residue -- the lift-step shape (exact-solve, "Method": each
 * step's inverse mod q_j applied to the residual is one INT8 GEMM per prime,
 * run as one batched product, and the CRT assembles the wide digit).
 *
 * A_res: device int8 [n_primes][M][K]; plane j is read as an integer matrix
 *   mod plan->primes[j] (any int8 value is accepted; |a| <= 128 keeps the
 *   int32 accumulation exact for K <= 2^17).
 * B: device int64 [K][N][b_limbs], reduced per prime by the split kernel.
 * C: device int64 [M][N][c_limbs]: the unique X in the plan's representative
 *   range with X = A_res[j] @ B (mod primes[j]) for every j.
 * When N <= 16, b_limbs == 1, K is a multiple of 16 up to 2^16, the plan
 * declares no bound for B (b_bits < 0 or >= 63) and A_res is 16-byte
 * aligned, the whole call is one kernel: the products run on the bytes of
 * B, which every prime shares, and each workgroup reconstructs its own
 * entries; the workspace then holds only the status header (zero blocks)
 * afterwards, not residue planes.  Otherwise the three stage kernels run.
 * Returns as rns_gemm.
 */
int rns_gemm_batched_residue(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                             const int8_t *A_res,
                             const int64_t *B, int32_t b_limbs,
                             int64_t *C, int32_t c_limbs,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Stage calls.  rns_gemm is exactly rns_split, then rns_residue_products,
 * then rns_reconstruct on the same workspace and stream; the stages are
 * exposed for callers that time them separately or keep the residue planes
 * (for instance a lift that splits its residual once per step).  Arguments
 * mean what they mean for rns_gemm / rns_gemm_batched_residue, and each
 * stage validates them the same way.
 *
 * rns_split            -- kernel 1: the balanced int8 residue planes of A
 *                         (skipped when A == NULL: the batched-residue
 *                         variant) and of B, written into ws.
 * rns_residue_products -- kernel 2: Y_j = (A_j @ B_j) mod q_j, balanced, for
 *                         every prime; A_j from ws, or from A_res when it is
 *                         not NULL (batched-residue variant).
 * rns_reconstruct      -- kernel 3: C from the Y planes, the centered CRT
 *                         value by rounded quotient (Ozaki Scheme II paper,
 *                         §3.5.2: the centered representative by rounding to
 *                         nearest): with M_j = P / q_j, w_j = M_j^-1 mod q_j
 *                         (balanced) and the basis e_j = w_j M_j,
 *                         X = sum_j y_j e_j - r P with r the nearest integer
 *                         to sum_j y_j w_j / q_j (the y_j as stored, no
 *                         per-entry reduction), the sum over primes formed
 *                         on the matrix cores; where the
 *                         binary32 estimate of r is near a half-integer the
 *                         result is compared with P/2 exactly and moved by one
 *                         period, so C is the same exact value as Garner's.
 *                         batched_residue selects the workspace layout of that
 *                         variant.  K == 0 writes zeros.
 * rns_reconstruct_garner -- the same C by balanced Garner mixed-radix digits
 *                         (exact-solve, "Method"; enclosure-gemm, "Method":
 *                         balanced-Garner digits assembled in signed
 *                         arithmetic), one thread per entry; the O(n^2) digit
 *                         recurrence (Ozaki Scheme II paper, §1.1).  Same
 *                         arguments, layout and errors as rns_reconstruct.
 */
int rns_split(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
              const int64_t *A, int32_t a_limbs, const int64_t *B, int32_t b_limbs,
              void *ws, size_t ws_bytes, hipStream_t stream);
int rns_residue_products(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                         const int8_t *A_res, void *ws, size_t ws_bytes, hipStream_t stream);
int rns_reconstruct(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                    int32_t batched_residue, int64_t *C, int32_t c_limbs,
                    void *ws, size_t ws_bytes, hipStream_t stream);
int rns_reconstruct_garner(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                           int32_t batched_residue, int64_t *C, int32_t c_limbs,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * rns_gemm_noalloc -- rns_gemm for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, checks, result and errors as rns_gemm, minus
 * the workspace: the library uses a fixed array of RNS_NOALLOC_SCRATCH_BYTES
 * (64 MiB) that every GPU it runs on holds until the process ends.  The call
 * allocates nothing.  Shapes whose rns_workspace_size exceeds the array are
 * rejected with RNS_E_SCRATCH before anything is launched.  All calls on one
 * GPU share that GPU's array and leave their data in it: calls that overlap
 * on one GPU (other streams, other host threads) race and must be ordered by
 * the caller.  rns_status does not apply to these calls.
 */
#define RNS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int rns_gemm_noalloc(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                     const int64_t *A, int32_t a_limbs,
                     const int64_t *B, int32_t b_limbs,
                     int64_t *C, int32_t c_limbs, hipStream_t stream);

/*
 * rns_status -- synchronises `stream`, then reports in *flags the
 * RNS_FLAG_* bits recorded by the last rns_gemm / rns_gemm_batched_residue
 * call that used workspace `ws` (0: every operand entry met its declared
 * bound).  Returns RNS_OK, RNS_E_ARG or RNS_E_HIP.
 */
int rns_status(const void *ws, hipStream_t stream, uint32_t *flags);

/*
 * rns_workspace_layout -- where the residue planes live inside the
 * workspace, for inspection by tests and for callers that reuse the planes.
 * Plane j of an operand is the balanced residue of every entry mod
 * plan->primes[j], stored as int8.  Operand planes are K-blocked in blocks
 * of k_block (64) entries, so that a 64-wide K step of a row tile is one
 * contiguous run of whole cache lines:
 *   A planes at a_off, a_plane bytes apart:  [k_pad / k_block][m_pad][k_block]  (row m, column k of A)
 *   B planes at b_off, b_plane bytes apart:  [k_pad / k_block][n_pad][k_block]  (column n, row k of B)
 * A plane pitch is its m_pad * k_pad (n_pad * k_pad) bytes, plus 4 KiB when
 * that is a multiple of 64 KiB: with equal power-of-two strides the same
 * offset of every plane would share cache sets and memory channels.
 * Product planes are row-major with a row pitch of y_pitch bytes (an odd
 * multiple of 128, which spreads a tile's rows over the L2 channels):
 *   Y planes at y_off: [n][m_pad][y_pitch], entries 0..n_pad-1 of each row
 *   (the balanced residue of (A_j @ B_j) mod q_j).
 * Entries beyond M, N or K inside m_pad, n_pad, k_pad are zero.  In the
 * batched-residue variant A planes are absent (a_off = -1) when the caller's
 * A_res is used in place.
 */
typedef struct rns_layout {
    int64_t m_pad, n_pad, k_pad;
    int64_t k_block, y_pitch;
    int64_t a_off, b_off, y_off;
    int64_t status_off;
    int64_t total_bytes;
    int32_t tile_config;     /* which GEMM tiling was chosen */
    int64_t a_plane, b_plane;   /* bytes from one residue plane to the next */
} rns_layout_t;

int rns_workspace_layout(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                         int32_t batched_residue, rns_layout_t *out);

/* Measurement aid, not a step of the product: the int8 matrix-core rate the
 * device sustains on given operand bytes, against which the products'
 * roofline fraction can be read (the dense peak assumes the full clock; the
 * clock falls under the power limit by how much the operand bits switch).
 * `workgroups` workgroups of four waves (one per SIMD) each run `iters`
 * iterations of 32 v_mfma_i32_32x32x32_i8 on fragments read once from
 * `src` (device, 16-byte aligned, at least workgroups * 32 KiB; thread t
 * reads bytes 128 t .. 128 t + 127) and XORed with one another between
 * iterations, with 16 accumulator chains per wave and no memory traffic in
 * the loop: 2 * 32^3 * 32 * iters * 4 * workgroups int8 ops.  out (device,
 * workgroups * 256 int32) receives each thread's accumulator sum.
 * Asynchronous on `stream`; RNS_E_ARG for a null or short buffer or a count
 * below 1. */
int rns_probe_int8_mfma(const void *src, size_t src_bytes, int32_t workgroups, int32_t iters, int32_t *out,
                        hipStream_t stream);

/* A constant string naming an RNS_* code. */
const char *rns_error_string(int code);

#ifdef __cplusplus
}
#endif
#endif /* RNS_GEMM_H */
