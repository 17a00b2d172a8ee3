// Internal definitions shared by the host code and the gfx950 kernels of
// librns_gemm.  Nothing here is part of the public C ABI (include/rns_gemm.h).
//
// The per-prime constant tables travel to the kernels by value, as kernel
// arguments: they are read with uniform (scalar) loads, need no device
// allocation and no host->device copy, and stay valid under stream capture.
#pragma once

#include <stdint.h>

#include "../../include/rns_gemm.h"

namespace rns {

constexpr int kMaxPrimes = RNS_MAX_PRIMES;   // 54
constexpr int kGarnerSlots = 56;             // kMaxPrimes rounded up to 8
constexpr int kTriEntries = kGarnerSlots * (kGarnerSlots + 1) / 2;

// 1.5 * 2^52: adding it to a double |x| < 2^51 rounds x to the nearest
// integer j and leaves j in the low 32 bits of the bit pattern (two's
// complement), because the low 32 bits of 1.5 * 2^52 are zero.
constexpr double kRoundMagic = 6755399441055744.0;
// 1.5 * 2^23, the binary32 counterpart (for |x| < 2^22)
constexpr float kRoundMagic32 = 12582912.0f;

// ---- residue split (kernel 1) ---------------------------------------------
// An L-limb entry x is sum_b a_b 256^b + c_L over its bytes, with a_b the
// byte minus 128 (the top byte: its signed value) and c_L = 128 (1 + 256 +
// ... + 256^(8L-2)).  So x mod q = sum_b a_b t_b + c_L mod q with
// t_b = 256^b mod q: an INT8 dot product on the matrix cores.
constexpr int kSplitBytes = 8 * RNS_MAX_IN_LIMBS;   // 32 byte positions
struct SplitConsts {
    alignas(16) uint32_t t[kMaxPrimes][kSplitBytes / 4];   // balanced t_b as packed int8, b = 0 .. 31
    int32_t start[2][kMaxPrimes];   // accumulator start for A (0) and B (1): c_L mod q plus a
                                    // multiple of q that keeps every sum positive
    int32_t q[kMaxPrimes];
    float inv[kMaxPrimes];          // binary32 1/q; for q a power of two the float just below
                                    // it, so that a sum = q/2 (mod q) gives +q/2
    int32_t n;
};
// |sum_b a_b t_b| <= 32 * 128 * 127 < 2^19: the start adds at least this much.
constexpr int32_t kSplitSumBias = 1 << 19;

// ---- mod-q epilogue of the residue product (kernel 2) ----------------------
// The int32 accumulator s itself goes through the binary64 rounding step.
struct EpiConsts {
    int32_t q[kMaxPrimes];
    double inv[kMaxPrimes];
};

// ---- Garner reconstruction (kernel 3) --------------------------------------
// Slot k of the Garner order holds prime q_k; Q_k = q_0 * ... * q_{k-1}.
// Digits: v_k = ( y_k * Q_k^-1  -  sum_{j<k} v_j * (Q_j * Q_k^-1 mod q_k) ) mod q_k,
// balanced.  tri[T(j,k)] holds Q_j * Q_k^-1 mod q_k (balanced) for j < k and
// Q_k^-1 mod q_k for j == k, with T(j,k) = j*(2S - j + 1)/2 + (k - j),
// S = kGarnerSlots.  The value is X = sum_k v_k Q_k, formed from the 16-bit
// chunks of each Q_k.  Q_k < 256^k has at most garner_chunks(k) = k/2 + 1
// chunks; slot k's chunks start at garner_chunk_offset(k) in q16 (unused
// chunks are zero).  Slots k >= n are padding: q = 1, inv = 1, zero tables.
__host__ __device__ constexpr int garner_chunks(int k) { return k / 2 + 1; }
__host__ __device__ constexpr int garner_chunk_offset(int k) {
    // sum_{j<k} (j/2 + 1)
    return (k / 2) * (k / 2 - 1) + (k % 2) * (k / 2) + k;
}
constexpr int kMaxQChunks = garner_chunk_offset(kGarnerSlots);   // 812

struct GarnerConsts {
    int32_t n;
    uint8_t plane[kGarnerSlots];   // Garner slot -> residue plane index
    uint16_t q[kGarnerSlots];      // moduli up to 256
    double inv[kGarnerSlots];
    int8_t tri[kTriEntries];
    uint16_t q16[kMaxQChunks];
};

__host__ __device__ constexpr int tri_index(int j, int k) {
    return j * (2 * kGarnerSlots - j + 1) / 2 + (k - j);
}

// ---- CRT by rounded quotient (kernel 3, default) -----------------------------
// Ozaki Scheme II paper, §3.5.2: the centered representative is taken by
// rounding to nearest.  With M_k = P / q_k and w_k = M_k^-1 mod q_k
// (balanced, |w_k| <= q_k / 2), the CRT basis element e_k = w_k M_k is 1 mod
// q_k and 0 mod the other moduli, and |e_k| <= P / 2.  So for any
// representatives y_k of the residues (the int8 bytes as stored),
// S = sum_k y_k e_k = X (mod P) and S / P = sum_k y_k w_k / q_k exactly;
// X = S - r P with r the nearest integer to that sum.  No residue is reduced
// per entry: the multiplier w_k lives in the constant e_k.  r comes from a
// fixed-point sum: c_k = round(w_k 2^31 / q_k), so sum_k y_k c_k / 2^31 is
// within n * 128 / 2^32 < 2^-19 of S / P; where it lies within 2^-10 of a
// half-integer the result is compared with P/2 exactly and moved by one
// period if needed.  One INT8 MFMA per 32 entries forms S - r P in balanced
// base-256 chunks: the entries' slots (y_0 .. y_{n-1}, -r_lo, -r_hi) times
// the balanced base-256 digits of (e_0 .. e_{n-1}, P, 256 P), where
// r = r_lo + 256 r_hi with r_lo in [-127, 128] (so -r_lo fits a byte).
constexpr int kCrtSlots = 64;        // n moduli + the two -r slots, padded to two K steps of 32
constexpr int kCrtDigits = 48;       // balanced base-256 digits kept per constant (256 P < 2^384)

struct CrtConsts {
    int32_t n;                       // moduli; slots n and n + 1 hold -r_lo and -r_hi
    int32_t chi[kCrtSlots];          // c_k = chi 2^16 + clo, clo in [0, 2^16); zero past slot n - 1
    int32_t clo[kCrtSlots];
    uint32_t cb[kCrtSlots];          // c_k as four balanced base-256 digits (packed int8, low first)
    uint32_t P[16];                  // P, little-endian 32-bit words
};
// Balanced base-256 digits of e_0 .. e_{n-1}, P (slot n) and 256 P (slot
// n + 1); the kernel takes them as an argument and lays out its MFMA
// fragments itself.
struct CrtDigits {
    int8_t d[kCrtSlots - 8][kCrtDigits];   // slots 0 .. 55 (n + 2 <= 56)
};

// ---- residue plane layout ----------------------------------------------------
// A and B^T planes are K-blocked: [n][k_pad / 64][rows][64] int8, so the
// 64-wide K step of a tile is one contiguous run of whole cache lines.
constexpr int kKBlock = 64;

// ---- GEMM tilings ----------------------------------------------------------
enum TileConfig : int32_t {
    kTileBig = 0,      // 256 x 256 x 64, eight waves of 128 x 64 in ping-pong, LDS ring fed by DMA
    kTileSmall = 1,    // 64 x 64 x 64, four waves of 32 x 32
    kTileSkinny = 2,   // 128 x 32 x 64, four waves of 32 x 32 stacked along M
};

struct TileShape { int bm, bn, bk; };

// Large tiling: tiles past the last whole round over the compute units are
// split over K; each part leaves its 256 x 256 residues in a slot of
// kTailUnitBytes, and a second kernel adds up the parts of each tile.
constexpr int kTailUnitsMax = 256;
constexpr int64_t kTailUnitBytes = 256 * 256;

__host__ __device__ constexpr TileShape tile_shape(int cfg) {
    return cfg == kTileBig ? TileShape{256, 256, 64}
         : cfg == kTileSmall ? TileShape{64, 64, 64}
         : TileShape{128, 32, 64};
}

// ---- launchers (rns_split.hip, rns_gemm.hip, rns_garner.hip) ------------------
struct SplitOperand {
    const int64_t *x;      // [rows][cols][limbs] for A, [K][N][limbs] for B
    int8_t *planes;        // n planes of [k_pad / 64][r_pad][64], `plane` bytes apart
    int64_t plane;
    int64_t rows;          // A: M        B: N  (plane rows)
    int64_t k;             // K
    int64_t r_pad, k_pad;  // padded plane rows (multiple of 16); K padded to whole K blocks
    int32_t limbs;
    int32_t bits;          // declared bound, or -1 for no check
    int32_t transposed;    // 0: A ([rows][K]), 1: B ([K][rows])
    int32_t fp64;          // 1: x holds binary64 values (one word per entry), read as
                           //    `limbs` limbs of floor(x * 2^scale)
    int32_t scale;
};

int launch_split(const SplitOperand *a, const SplitOperand *b, const SplitConsts &c,
                 uint32_t *status, int64_t status_slots, hipStream_t s);

// A plan over explicit moduli (validated like any plan), no operand bound.
int plan_from_moduli(const int32_t *moduli, int n, int64_t k_max, rns_plan_t *out);

// Binary64 operands read by the split as floor(A * 2^fa), floor(B * 2^fb).
struct Fp64Scales {
    int32_t fa, fb;
    int32_t b_rows_n;      // 1: B is given as B^T, [N][K] row-major
};
// rns_gemm on binary64 operands A [M][K], B [K][N], scaled into a_limbs /
// b_limbs limbs inside the split (same checks, layout and errors as rns_gemm).
int gemm_fp64_scaled(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                     const double *A, int32_t a_limbs, const double *B, int32_t b_limbs,
                     const Fp64Scales &scales, int64_t *C, int32_t c_limbs,
                     void *ws, size_t ws_bytes, hipStream_t stream);
int launch_repack_residues(const int8_t *src, int64_t n, int64_t M, int64_t K,
                           int8_t *dst, int64_t m_pad, int64_t k_pad, int64_t plane, hipStream_t s);
int launch_gemm(int cfg, int n, const int8_t *a, const int8_t *b, int8_t *y,
                int64_t m_pad, int64_t n_pad, int64_t k_pad,
                int64_t a_plane, int64_t b_plane, int64_t y_plane,
                int64_t a_row, int64_t a_kstep, int64_t b_row, int64_t b_kstep, int64_t y_pitch,
                int8_t *partial, const EpiConsts &c, hipStream_t s);
int launch_mfma_probe(const int8_t *src, int workgroups, int iters, int32_t *out, hipStream_t s);
int launch_garner(const GarnerConsts &g, const int8_t *y, int64_t y_plane, int64_t y_pitch,
                  int64_t M, int64_t N, int64_t *C, int32_t c_limbs, hipStream_t s);
int launch_zero(int64_t *C, int64_t count, hipStream_t s);
// The whole batched step for N <= 16 one-limb right-hand sides without a
// bound to check (K a multiple of 16, up to RNS_LIFT_K_MAX; a 16-byte aligned):
// the products on r's bytes and the reconstruction in one kernel, C written
// directly (no residue planes in the workspace) and a status header of zero
// blocks.  K <= 2^16 keeps every int32 byte product within 2^30.
#define RNS_LIFT_K_MAX 65536
// Its per-plan constants: the moduli, 256^b mod q_j (b < 8, balanced int8,
// packed four to a word), c_1 mod q_j (c_1 = 128 (1 + 256 + ... + 256^6)),
// P, and the reconstruction's fixed-point weights c_k (CrtConsts::cb) as
// MFMA fragments: fx[ks][h][d] holds digit d of c_k for slots
// k = 32 ks + 16 h .. 32 ks + 16 h + 15, one byte each.
struct StepConsts {
    uint32_t tb[kMaxPrimes][2];
    uint32_t fx[2][2][4][4];
    uint32_t P[16];
    uint16_t q[kMaxPrimes];
    uint8_t c1[kMaxPrimes];
    int32_t n;
};
int launch_lift_step(const StepConsts &lc, const CrtDigits &cd, int ksteps, int nblocks, const int8_t *a,
                     const int64_t *r, int64_t M, int64_t N, int64_t K, int64_t *C, int32_t c_limbs,
                     uint32_t *status, hipStream_t s);
// ksteps / nblocks: MFMA K steps (slots n + 1 in 32s) and N blocks (digits in 32s)
int launch_crt(const CrtConsts &c, const CrtDigits &d, int ksteps, int nblocks,
               const int8_t *y, int64_t y_plane, int64_t y_pitch, int64_t M, int64_t N, int64_t *C,
               int32_t c_limbs, hipStream_t s);

// Status area written by the split kernel: word 0 = number of split blocks,
// word 1 = that number XOR kStatusCheck, then one flag word per block.
constexpr int kStatusHeader = 2;
constexpr uint32_t kStatusCheck = 0x52534e53u;
// status slots written by the split kernel: one word per block plus the header
int64_t split_status_slots(const SplitOperand *a, const SplitOperand *b, int n_primes);

}  // namespace rns
