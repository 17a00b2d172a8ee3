/*
 * rns_sliced.h -- exact integer products beyond the residue capacity, by
 * slicing the operands (Ozaki Scheme II paper, §5.1 and §5.2: more slices
 * trade additional GEMMs for a smaller range per product).
 *
 * One product of the residue engine is exact while 2 * K * max|A| * max|B|
 * stays below the product of the moduli (2^334.9 for the primes below 256).
 * Wider operands are cut at limb boundaries, A = sum_i A_i 2^(64 sa i) and
 * B = sum_j B_j 2^(64 sb j): the lower slices are the raw limbs read
 * unsigned, the top slice the remaining limbs with the sign.  Each slice
 * product A_i B_j is one exact rns_gemm with sa + sb <= 4 limbs of range, and
 *   C = sum_{i,j} (A_i B_j) 2^(64 (sa i + sb j))
 * is accumulated in two's complement by one more kernel.
 *
 * Conventions of rns_gemm.h (device pointers owned by the caller, launches
 * asynchronous on the caller's stream, 0 or a negative RNS_E_* code, nothing
 * written on a validation error).  A is int64 [M][K][a_limbs], B int64
 * [K][N][b_limbs], C int64 [M][N][c_limbs].
 */
#ifndef RNS_SLICED_H
#define RNS_SLICED_H

#include "rns_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* operand limbs of a sliced product, and the widest output */
#define RNS_SLICED_MAX_IN_LIMBS 8
#define RNS_SLICED_MAX_OUT_LIMBS 18

typedef struct {
    rns_plan_t slice;       /* the plan of one slice product (K, 64 sa and 64 sb bits) */
    int32_t a_limbs, b_limbs;
    int32_t sa, sb;         /* slice widths in limbs; sa + sb <= 4 */
    int32_t na, nb;         /* slices of A and of B: na * nb slice products */
    int32_t part_limbs;     /* limbs of one slice product */
    int32_t out_limbs_min;  /* limbs holding every |C| <= K 2^(64 a_limbs - 1) 2^(64 b_limbs - 1) */
} rns_sliced_plan_t;

/*
 * rns_sliced_plan -- slice widths for operands of a_limbs and b_limbs limbs
 * (1..RNS_SLICED_MAX_IN_LIMBS, any values) and contraction length K
 * (1..2^17): sa + sb = 4 limbs with sa, sb as even as the operands allow.
 * Returns RNS_OK, RNS_E_ARG or RNS_E_K.
 */
int rns_sliced_plan(int64_t K, int32_t a_limbs, int32_t b_limbs, rns_sliced_plan_t *out);

/*
 * rns_sliced_workspace_size -- device bytes for rns_gemm_sliced: the slices
 * of A and B (one limb wider than the slice), the slice products, and the
 * workspace of one slice product.  Returns RNS_OK, RNS_E_ARG or RNS_E_K.
 */
int rns_sliced_workspace_size(const rns_sliced_plan_t *plan, int64_t M, int64_t N, int64_t K, size_t *bytes);

/*
 * rns_gemm_sliced -- C = A @ B exactly, for the plan's operand limbs.
 * c_limbs in [plan->out_limbs_min, RNS_SLICED_MAX_OUT_LIMBS].  Returns RNS_OK,
 * RNS_E_ARG, RNS_E_K (K above the plan's), RNS_E_OUT_LIMBS, RNS_E_WORKSPACE
 * or RNS_E_HIP.  M == 0 or N == 0 is a no-op; K == 0 writes zeros.
 */
int rns_gemm_sliced(const rns_sliced_plan_t *plan, int64_t M, int64_t N, int64_t K, const int64_t *A,
                    const int64_t *B, int64_t *C, int32_t c_limbs, void *ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RNS_SLICED_H */
