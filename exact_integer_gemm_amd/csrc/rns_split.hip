// K1 of the exact residue GEMM on gfx950: int64-limb operands -> balanced
// int8 residue planes, one per prime (enclosure-gemm, "Method": the residue
// split), and the repack of caller-given residue planes.
//
// The split runs on the matrix cores.  Write an L-limb entry x in bytes x_b
// (little-endian two's complement) and let a_b = x_b - 128 for every byte but
// the top one, whose signed value is a_b itself; then
//     x = sum_b a_b 256^b + c_L,   c_L = 128 (1 + 256 + ... + 256^(8L-2)),
// so  x = sum_b a_b t_b + c_L (mod q)  with t_b = 256^b mod q (balanced):
// a dot product of signed bytes.  The bytes a_b are the entry's bytes with
// bit 7 flipped (all but the top one), so the first operand of
// v_mfma_i32_32x32x32_i8 is the loaded entry XOR a constant, and its
// second operand holds the t_b of 32 moduli.  The accumulator starts at
// c_L mod q plus a multiple of q above 32 * 128 * 127, which keeps every sum
// t in (0, 2^21); one binary32 rounding step then reduces t mod q.
//
// Two packings of the 32 byte positions of one product (lane (row, h) of the
// first operand holds 16 of them; the same 16 positions are lane (col, h) of
// the second operand, whatever their order inside the instruction):
//   pair   (L <= 2): lane (row, h) holds entry 32 h + row of a 64-entry group;
//          column c holds the t_b of modulus c % 16 in half c / 16 and zeros
//          in the other half.  Column c then gives entry 32 (c / 16) + row mod
//          modulus c % 16: 64 entries x 16 moduli per product.
//   single (L = 3, 4): lane (row, h) holds bytes 16 h .. 16 h + 15 of entry
//          row; column c holds t_{16 h + j} of modulus c: 32 entries x 32
//          moduli per product.
// Result lane (c, hh) holds rows 8 g + 4 hh + e (g, e < 4) of column c.
#include "rns_device.h"

namespace rns {

// ============================================================================
// K1: residue split
// ============================================================================
constexpr int kSplitThreads = 256;                 // four waves
constexpr int kSplitWaves = kSplitThreads / 64;
constexpr int kRowsPair = 8;                       // plane rows per wave, pair packing
constexpr int kRowsSingle = 4;                     // plane rows per wave, single packing

typedef uint64_t u64;

struct SplitStatus {
    uint32_t *status;      // [kStatusHeader + total] words
    int64_t work;          // row path: wave units; column path: workgroup tiles
    int32_t first;         // this launch's first status word (after the header)
    int32_t total;         // status words of every launch of the split
    uint32_t flag_bit;     // RNS_FLAG_* recorded for an out-of-bound entry
    int32_t b_start;       // 1: the operand takes start_b (the B offsets)
};

// |x| <= 2^bits for an L-limb value, bits >= 0.  For x < 0 use ~x = -x-1:
// |x| <= 2^bits  <=>  ~x < 2^bits.  For x >= 0: x < 2^bits or x == 2^bits.
template <int L>
__device__ __forceinline__ bool within_bound(const uint64_t (&x)[L], int bits) {
    const bool neg = (int64_t)x[L - 1] < 0;
    bool below = true, is_pow = !neg;
#pragma unroll
    for (int l = 0; l < L; l++) {
        uint64_t v = neg ? ~x[l] : x[l];
        int lo = 64 * l;
        // bits of this limb at positions >= bits must be zero for v < 2^bits
        uint64_t mask_ge = bits <= lo ? ~0ull : (bits >= lo + 64 ? 0ull : (~0ull << (bits - lo)));
        if (v & mask_ge) below = false;
        // v == 2^bits
        uint64_t want = (bits >= lo && bits < lo + 64) ? (1ull << (bits - lo)) : 0ull;
        if (v != want) is_pow = false;
    }
    return below || is_pow;
}

// The first-operand bytes of limb l of an L-limb entry: bit 7 of every byte
// flipped but for the entry's top byte; limbs past the entry are zero.
template <int L>
__device__ __forceinline__ u64 operand_limb(u64 x, int l) {
    return l < L - 1 ? x ^ 0x8080808080808080ull : l == L - 1 ? x ^ 0x0080808080808080ull : 0ull;
}

__device__ __forceinline__ v4i as_v4i(u64 lo, u64 hi) {
    return v4i{(int)(uint32_t)lo, (int)(uint32_t)(lo >> 32), (int)(uint32_t)hi, (int)(uint32_t)(hi >> 32)};
}

typedef unsigned long long u64x2 __attribute__((ext_vector_type(2), aligned(8)));

// W consecutive words from an 8-byte aligned address, in 16-byte loads.
// Every entry is read once, so the loads carry the non-temporal hint (on
// the wide workload, measured with one launch per operand: 160 us with it,
// 165 us without).
template <int W>
__device__ __forceinline__ void load_words(const int64_t *p, u64 (&w)[W]) {
    if constexpr (W % 2 == 0) {
#pragma unroll
        for (int i = 0; i < W / 2; i++) {
            const u64x2 v = __builtin_nontemporal_load((const u64x2 *)p + i);
            w[2 * i] = v.x;
            w[2 * i + 1] = v.y;
        }
    } else {
        __builtin_memcpy(w, p, sizeof(w));
    }
}

// The limbs of an entry from its loaded words (binary64: floor(x * 2^scale));
// an entry outside the operand (ok false) is zero.
template <int L, bool FP, int W>
__device__ __forceinline__ void entry_limbs(const u64 (&xs)[W], bool ok, int scale, u64 (&x)[L]) {
    if constexpr (FP) {
        fp64_floor_scaled<L>(ok ? xs[0] : 0ull, scale, x);
    } else {
#pragma unroll
        for (int l = 0; l < L; l++) x[l] = ok ? xs[l] : 0ull;
    }
}

// The per-modulus constants of one operand, staged in LDS once per
// workgroup: the columns of every block of moduli read them from there.
struct SplitLds {
    v4i t[kMaxPrimes][2];      // t_b, b = 0 .. 31
    int32_t start[kMaxPrimes];
    int32_t q[kMaxPrimes];
    float inv[kMaxPrimes];
};
constexpr int kTWords = kMaxPrimes * kSplitBytes / 4;
constexpr int kLdsWords = kTWords + 3 * kMaxPrimes;     // the image without its tail padding
constexpr int kLdsLoads = (kLdsWords + kSplitThreads - 1) / kSplitThreads;
static_assert(sizeof(SplitLds) >= 4 * kLdsWords && offsetof(SplitLds, inv) == 4 * (kTWords + 2 * kMaxPrimes),
              "LDS image layout");

// Each thread reads its share of the constants (word w of the LDS image)
// from the kernel arguments; issued before the entry loads, written to LDS
// after them.
struct TableWords {
    uint32_t v[kLdsLoads];
};

__device__ __forceinline__ TableWords table_load(const SplitConsts &c, int sidx) {
    TableWords tw;
#pragma unroll
    for (int j = 0; j < kLdsLoads; j++) {
        int w = (int)threadIdx.x + kSplitThreads * j;
        w = w < kLdsWords ? w : kLdsWords - 1;
        const uint32_t *src = w < kTWords ? &c.t[0][0] + w
                            : w < kTWords + kMaxPrimes ? (const uint32_t *)&c.start[sidx][w - kTWords]
                            : w < kTWords + 2 * kMaxPrimes ? (const uint32_t *)&c.q[w - kTWords - kMaxPrimes]
                            : (const uint32_t *)&c.inv[w - kTWords - 2 * kMaxPrimes];
        tw.v[j] = *src;
    }
    return tw;
}

__device__ __forceinline__ void table_commit(const TableWords &tw, SplitLds &lds) {
#pragma unroll
    for (int j = 0; j < kLdsLoads; j++) {
        const int w = (int)threadIdx.x + kSplitThreads * j;
        if (w < kLdsWords) reinterpret_cast<uint32_t *>(&lds)[w] = tw.v[j];
    }
    __syncthreads();
}

// The second operand and the per-column constants of one block of moduli.
// A column past the last modulus repeats the last one.
struct Column {
    v4i t;         // t_b bytes of this lane's half (zero where the lane holds none)
    v16i start;    // accumulator start
    int q;
    float inv;
    int p;         // modulus index
};

template <bool PAIR>
__device__ __forceinline__ Column column(const SplitLds &lds, int n, int blk, int lane) {
    Column col;
    const int h = lane >> 5, c32 = lane & 31;
    int p, half;
    bool sel;
    if constexpr (PAIR) {
        p = 16 * blk + (c32 & 15);
        half = 0;
        sel = (c32 >> 4) == h;
    } else {
        p = 32 * blk + c32;
        half = h;
        sel = true;
    }
    col.p = p < n ? p : n - 1;
    const v4i t = lds.t[col.p][half];
    col.t = sel ? t : v4i{0, 0, 0, 0};
    const int s0 = lds.start[col.p];
#pragma unroll
    for (int e = 0; e < 16; e++) col.start[e] = s0;
    col.q = lds.q[col.p];
    col.inv = lds.inv[col.p];
    return col;
}

// The 16 sums of a lane reduced mod q and packed: word g holds rows 8 g + 4 hh .. + 3.
__device__ __forceinline__ void reduce_pack(const v16i &acc, int q, float inv, uint32_t (&w)[4]) {
#pragma unroll
    for (int g = 0; g < 4; g++)
        w[g] = pack4(reduce_low_byte_f32(acc[4 * g], q, inv), reduce_low_byte_f32(acc[4 * g + 1], q, inv),
                     reduce_low_byte_f32(acc[4 * g + 2], q, inv), reduce_low_byte_f32(acc[4 * g + 3], q, inv));
}

// The half-waves trade words so that every lane holds 16 consecutive rows:
// the lower lane rows 0 .. 15 (its own 0-3 and 8-11, its partner's 4-7 and
// 12-15), the upper lane rows 16 .. 31.
__device__ __forceinline__ v4u rows16(const uint32_t (&w)[4]) {
    const auto a = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
    return v4u{a[0], a[1], b[0], b[1]};
}

// The lane's half (limbs 2 h, 2 h + 1) of an entry of L = 3 or 4 limbs, and
// the whole entry by trading halves with the partner lane (for the bound check).
template <int L>
__device__ __forceinline__ void whole_entry(u64 p0, u64 p1, u64 (&x)[L]) {
    uint32_t v[4] = {(uint32_t)p0, (uint32_t)(p0 >> 32), (uint32_t)p1, (uint32_t)(p1 >> 32)};
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const auto s = __builtin_amdgcn_permlane32_swap(v[i], v[i], false, false);
        lo[i] = s[0];
        hi[i] = s[1];
    }
    u64 all[4] = {lo[0] | (u64)lo[1] << 32, lo[2] | (u64)lo[3] << 32, hi[0] | (u64)hi[1] << 32,
                  hi[2] | (u64)hi[3] << 32};
#pragma unroll
    for (int l = 0; l < L; l++) x[l] = all[l];
}

// The words one thread loads for an entry: binary64, one word; integer
// entries on the row path with the pair packing and on the column path, the
// L limbs; on the row path with the single packing, the lane's limbs 2 h and
// 2 h + 1 (the second read again from limb 2 h where it lies past the entry,
// and dropped later).
template <int L, bool FP, bool PART>
struct EntryWords {
    static constexpr int W = FP ? 1 : (PART ? 2 : L);
};

template <int L, bool FP, bool PART>
__device__ __forceinline__ void load_entry(const int64_t *x, int64_t e, int h,
                                           u64 (&w)[EntryWords<L, FP, PART>::W]) {
    if constexpr (FP) {
        w[0] = (u64)x[e];
    } else if constexpr (!PART) {
        load_words<L>(x + e * L, w);
    } else {
        w[0] = (u64)x[e * L + 2 * h];
        w[1] = (u64)x[e * L + (2 * h + 1 < L ? 2 * h + 1 : 2 * h)];
    }
}

// The lane's first-operand fragment of an entry on the row path; sets flag
// when the entry lies outside the declared bound.
template <int L, bool FP, bool PAIR>
__device__ __forceinline__ v4i fragment(const u64 (&w)[EntryWords<L, FP, !PAIR>::W], bool ok,
                                        const SplitOperand &op, int h, uint32_t &flag) {
    if constexpr (PAIR) {
        u64 x[L];
        entry_limbs<L, FP>(w, ok, op.scale, x);
        if (op.bits >= 0 && !within_bound<L>(x, op.bits)) flag = 1;
        return as_v4i(operand_limb<L>(x[0], 0), L > 1 ? operand_limb<L>(x[L > 1 ? 1 : 0], 1) : 0ull);
    } else if constexpr (FP) {
        u64 x[L];
        entry_limbs<L, true>(w, ok, op.scale, x);
        if (op.bits >= 0 && !within_bound<L>(x, op.bits)) flag = 1;
        const u64 p0 = h ? x[2] : x[0];
        const u64 p1 = h ? (L > 3 ? x[L - 1] : 0ull) : x[1];
        return as_v4i(operand_limb<L>(p0, 2 * h), operand_limb<L>(p1, 2 * h + 1));
    } else {
        const u64 p0 = ok ? w[0] : 0ull;
        const u64 p1 = (ok && 2 * h + 1 < L) ? w[1] : 0ull;
        if (op.bits >= 0) {
            u64 x[L];
            whole_entry<L>(p0, p1, x);
            if (!within_bound<L>(x, op.bits)) flag = 1;
        }
        return as_v4i(operand_limb<L>(p0, 2 * h), operand_limb<L>(p1, 2 * h + 1));
    }
}

// Workgroup barrier ordering LDS only: pending global stores keep flowing.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Output staging: the results of one block of moduli for one wave unit
// (R plane rows of one K block: PB contiguous bytes of each plane) pass
// through LDS, so that each store writes 256 or 512 contiguous bytes of
// one or a few planes rather than 64 bytes of each of 16 planes.  Rows of a
// modulus sit PB + 16 bytes apart: the 16-byte pieces that lanes of one
// modulus column write land in distinct banks.
template <bool PAIR>
struct OutStage {
    static constexpr int P = PAIR ? 16 : 32;                        // moduli per block
    static constexpr int PB = (PAIR ? kRowsPair : kRowsSingle) * kKBlock;   // bytes per modulus
    static constexpr int PITCH = PB + 16;
    static constexpr int BYTES = P * PITCH;
};
constexpr int kOutStageBytes = OutStage<true>::BYTES > OutStage<false>::BYTES ? OutStage<true>::BYTES
                                                                               : OutStage<false>::BYTES;

// The products of F first-operand fragments against NB blocks of moduli.
// Fragment f's 16-byte result of lane (c, hh) lies off[f] + 32 s + 16 hh
// bytes into the unit's PB bytes of its modulus (s = c / 16 in the pair
// packing, else 0); the product of the next fragment is issued before the
// current one is reduced.  Every lane stores: a column past the last modulus
// repeats the last one, writing the same bytes to the same place as the
// column that owns it.
template <bool PAIR, int NB, int F>
__device__ __forceinline__ void products(const v4i (&a)[F], const SplitLds &lds, int n, int lane, int8_t *unit_dst,
                                         int64_t plane, const int (&off)[F], uint8_t *ostage) {
    using O = OutStage<PAIR>;
    const int cs = PAIR ? 32 * ((lane >> 4) & 1) + 16 * (lane >> 5) : 16 * (lane >> 5);
#pragma unroll
    for (int blk = 0; blk < NB; blk++) {
        const Column col = column<PAIR>(lds, n, blk, lane);
        uint8_t *mine = ostage + (PAIR ? (lane & 15) : (lane & 31)) * O::PITCH + cs;
        v16i acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0], col.t, col.start, 0, 0, 0);
#pragma unroll
        for (int f = 0; f < F; f++) {
            const v16i cur = acc;
            if (f + 1 < F)
                acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[f + 1 < F ? f + 1 : f], col.t, col.start, 0, 0, 0);
            uint32_t w[4];
            reduce_pack(cur, col.q, col.inv, w);
            *(v4u *)(mine + off[f]) = rows16(w);
        }
        // LDS operations of a wave complete in order; this keeps the
        // compiler from moving the reads above the writes
        asm volatile("" ::: "memory");
        // store j: 16-byte piece ch = 64 j + lane, modulus ch / (PB / 16) of the block
#pragma unroll
        for (int j = 0; j < O::P * O::PB / 1024; j++) {
            const int ch = 64 * j + lane;
            const int pl = ch / (O::PB / 16), piece = ch % (O::PB / 16);
            int p = O::P * blk + pl;
            p = p < n ? p : n - 1;
            const v4u v = *(const v4u *)(ostage + pl * O::PITCH + piece * 16);
            *(v4u *)(unit_dst + (int64_t)p * plane + piece * 16) = v;
        }
        asm volatile("" ::: "memory");
    }
}

// Row path (the operand is [rows][K]: A, or B given as B^T).  A wave unit
// is R plane rows of one K block, 64 consecutive entries of a row per load;
// waves run through the units with the grid's stride and load the next unit
// while the current one is in the matrix cores.
//   fragment f: pair, row r0 + f, entry k = 64 kb + lane;
//               single, row r0 + f / 2, entry k = 64 kb + 32 (f % 2) + lane % 32.
template <int L, bool FP, int NB>
__device__ void split_rows(const SplitOperand &op, const SplitConsts &c, int sidx, SplitLds &lds,
                           uint8_t *ostage, int64_t units, uint32_t &flag, int64_t bid, int64_t nblk) {
    constexpr bool PAIR = L <= 2;
    constexpr int R = PAIR ? kRowsPair : kRowsSingle;
    constexpr int F = PAIR ? R : 2 * R;
    constexpr int W = EntryWords<L, FP, !PAIR>::W;
    const int lane = threadIdx.x & 63, h = lane >> 5;
    const int64_t groups = op.r_pad / R;
    const int64_t stride = nblk * kSplitWaves;
    int64_t unit = bid * kSplitWaves + (threadIdx.x >> 6);

    // all loads are unconditional: an entry outside the operand (or of a
    // unit past the end) reads entry 0 and is then taken as zero
    u64 xs[F][W];
    bool ok[F];
    auto load_unit = [&](int64_t u, bool valid) {
        const int64_t kb = u / groups, r0 = (u - kb * groups) * R;
#pragma unroll
        for (int f = 0; f < F; f++) {
            const int64_t r = r0 + (PAIR ? f : f >> 1);
            const int64_t k = kb * kKBlock + (PAIR ? lane : 32 * (f & 1) + (lane & 31));
            ok[f] = valid && r < op.rows && k < op.k;
            load_entry<L, FP, !PAIR>(op.x, ok[f] ? r * op.k + k : 0, h, xs[f]);
        }
    };
    const TableWords tw = table_load(c, sidx);
    load_unit(unit < units ? unit : 0, unit < units);
    table_commit(tw, lds);

    const int64_t plane = op.plane;
    int off[F];
#pragma unroll
    for (int f = 0; f < F; f++) off[f] = PAIR ? f * kKBlock : (f >> 1) * kKBlock + 32 * (f & 1);
    auto body = [&](int64_t u) {
        v4i a[F];
#pragma unroll
        for (int f = 0; f < F; f++) a[f] = fragment<L, FP, PAIR>(xs[f], ok[f], op, h, flag);
        const int64_t kb = u / groups, r0 = (u - kb * groups) * R;
        const int64_t next = u + stride;
        load_unit(next < units ? next : u, next < units);
        int8_t *dst = op.planes + kb * (op.r_pad * kKBlock) + r0 * kKBlock;
        products<PAIR, NB, F>(a, lds, c.n, lane, dst, plane, off, ostage);
    };
    // The first unit runs outside the loop, so that every wait for a unit's
    // loads follows the previous unit's stores alike and counts them exactly.
    if (unit < units) {
        body(unit);
        for (unit += stride; unit < units; unit += stride) body(unit);
    }
}

// Column path (the operand is [K][rows]: B).  A workgroup tile is NT plane
// rows of one K block; its 64 NT entries are loaded NT consecutive plane
// rows at a time, turned into operand bytes and staged in LDS by plane row,
// and each wave then reads the fragments of its NT / 4 rows as on the row
// path.  Workgroups run through the tiles with the grid's stride and load
// the next tile while the current one is in the matrix cores.
template <bool PAIR>
struct ColsTile {
    static constexpr int NT = PAIR ? 32 : 16;          // plane rows per tile
    static constexpr int ES = PAIR ? 16 : 32;          // staged bytes per entry
    static constexpr int PITCH = 64 * ES + 16;         // LDS bytes per plane row
    static constexpr int EPT = 64 * NT / kSplitThreads;   // entries per thread
    static constexpr int BYTES = NT * PITCH;
};
constexpr int kColsLdsBytes = ColsTile<true>::BYTES > ColsTile<false>::BYTES ? ColsTile<true>::BYTES
                                                                               : ColsTile<false>::BYTES;

template <int L, bool FP, int NB>
__device__ void split_cols(const SplitOperand &op, const SplitConsts &c, int sidx, SplitLds &lds,
                           uint8_t *stage, uint8_t *ostage, int64_t tiles, uint32_t &flag, int64_t bid,
                           int64_t nblk) {
    constexpr bool PAIR = L <= 2;
    using T = ColsTile<PAIR>;
    constexpr int F = 8;                               // fragments per wave and tile
    constexpr int W = EntryWords<L, FP, false>::W;
    const int lane = threadIdx.x & 63, h = lane >> 5, wave = threadIdx.x >> 6;
    const int64_t nts = (op.r_pad + T::NT - 1) / T::NT;

    // thread entry j of a tile: i = thread + 256 j, plane row n0 + i % NT, k = 64 kb + i / NT
    u64 xs[T::EPT][W];
    bool ok[T::EPT];
    auto load_tile = [&](int64_t t, bool valid) {
        const int64_t kb = t / nts, n0 = (t - kb * nts) * T::NT;
#pragma unroll
        for (int j = 0; j < T::EPT; j++) {
            const int i = (int)threadIdx.x + kSplitThreads * j;
            const int64_t n = n0 + i % T::NT, k = kb * kKBlock + i / T::NT;
            ok[j] = valid && n < op.rows && k < op.k;
            load_entry<L, FP, false>(op.x, ok[j] ? k * op.rows + n : 0, h, xs[j]);
        }
    };
    int64_t tile = bid;
    const TableWords tw = table_load(c, sidx);
    load_tile(tile < tiles ? tile : 0, tile < tiles);
    table_commit(tw, lds);

    const int64_t plane = op.plane;
    auto body = [&](int64_t t, bool first) {
        // operand bytes of the loaded entries into LDS, [plane row][k]
        if (!first) lds_barrier();      // every wave has read the previous tile
#pragma unroll
        for (int j = 0; j < T::EPT; j++) {
            u64 x[L];
            entry_limbs<L, FP>(xs[j], ok[j], op.scale, x);
            if (op.bits >= 0 && !within_bound<L>(x, op.bits)) flag = 1;
            const int i = (int)threadIdx.x + kSplitThreads * j;
            uint8_t *p = stage + (i % T::NT) * T::PITCH + (i / T::NT) * T::ES;
            *(v4i *)p = as_v4i(operand_limb<L>(x[0], 0), L > 1 ? operand_limb<L>(x[L > 1 ? 1 : 0], 1) : 0ull);
            if constexpr (!PAIR)
                *(v4i *)(p + 16) = as_v4i(operand_limb<L>(x[2 < L ? 2 : 0], 2),
                                          L > 3 ? operand_limb<L>(x[L - 1], 3) : 0ull);
        }
        lds_barrier();

        // Wave w takes plane rows n0 + RW w' .. + RW - 1 (RW = NT / 4): fragment
        // f is, pair, row n0 + RW w' + f, entry k = lane; single, row
        // n0 + RW w' + f / 2, bytes 16 h of entry 32 (f % 2) + lane % 32.  A
        // tile reaches past the plane only by whole waves (plane rows come in
        // 16s): such a wave repeats one that lies inside (w' = w - a for the
        // a waves inside), writing the same bytes to the same place.
        constexpr int RW = T::NT / kSplitWaves;
        const int64_t kb = t / nts, n0 = (t - kb * nts) * T::NT;
        const int inside = (int)((op.r_pad - n0) / RW);
        const int wv = wave < inside ? wave : wave - inside;
        v4i a[F];
        int off[F];
#pragma unroll
        for (int f = 0; f < F; f++) {
            const int rl = RW * wv + (PAIR ? f : f >> 1);
            const int eo = PAIR ? lane * 16 : (32 * (f & 1) + (lane & 31)) * 32 + 16 * h;
            a[f] = *(const v4i *)(stage + rl * T::PITCH + eo);
            off[f] = (PAIR ? f : f >> 1) * kKBlock + (PAIR ? 0 : 32 * (f & 1));
        }
        const int64_t next = t + nblk;
        load_tile(next < tiles ? next : t, next < tiles);
        int8_t *dst = op.planes + kb * (op.r_pad * kKBlock) + (n0 + RW * wv) * kKBlock;
        products<PAIR, NB, F>(a, lds, c.n, lane, dst, plane, off, ostage);
    };
    // the first tile runs outside the loop (exact waits, as on the row path)
    if (tile < tiles) {
        body(tile, true);
        for (tile += nblk; tile < tiles; tile += nblk) body(tile, false);
    }
}

// One status word per block, written unconditionally (no clearing pass);
// the first block of the first launch also writes the header: the block
// count of the whole split and its check word.  Every thread of the block
// calls it (the flag is reduced over the block).
__device__ __forceinline__ void write_status(const SplitStatus &st, uint32_t flag, int64_t bid) {
    const bool any = __syncthreads_or(flag != 0);
    if (threadIdx.x == 0) {
        st.status[kStatusHeader + st.first + bid] = any ? st.flag_bit : 0u;
        if (st.first == 0 && bid == 0) {
            st.status[0] = (uint32_t)st.total;
            st.status[1] = (uint32_t)st.total ^ kStatusCheck;
        }
    }
}

template <int L, bool FP, bool COLS, int NB>
__global__ __launch_bounds__(kSplitThreads, 2) void split_kernel(SplitOperand op, SplitConsts c, SplitStatus st) {
    __shared__ SplitLds lds;
    __shared__ __align__(16) uint8_t ostage[kSplitWaves][kOutStageBytes];
    uint8_t *mine = ostage[threadIdx.x >> 6];
    uint32_t flag = 0;
    if constexpr (COLS) {
        __shared__ __align__(16) uint8_t stage[kColsLdsBytes];
        split_cols<L, FP, NB>(op, c, st.b_start, lds, stage, mine, st.work, flag, blockIdx.x, gridDim.x);
    } else {
        split_rows<L, FP, NB>(op, c, st.b_start, lds, mine, st.work, flag, blockIdx.x, gridDim.x);
    }
    write_status(st, flag, blockIdx.x);
}

// Both operands in one launch, for shapes whose two grids fit on the device
// at once: blocks below ga run A on the row path, the others B on the column
// path (integer entries of L limbs both).  One launch instead of two, and
// the two operands' blocks run side by side.
template <int L, int NB>
__global__ __launch_bounds__(kSplitThreads, 2) void split_ab_kernel(SplitOperand a, SplitOperand b, SplitConsts c,
                                                                    SplitStatus sa, SplitStatus sb, int32_t ga) {
    __shared__ SplitLds lds;
    __shared__ __align__(16) uint8_t ostage[kSplitWaves][kOutStageBytes];
    __shared__ __align__(16) uint8_t stage[kColsLdsBytes];
    uint8_t *mine = ostage[threadIdx.x >> 6];
    uint32_t flag = 0;
    const int64_t bid = blockIdx.x;
    if (bid < ga) {
        split_rows<L, false, NB>(a, c, sa.b_start, lds, mine, sa.work, flag, bid, ga);
        write_status(sa, flag, bid);
    } else {
        split_cols<L, false, NB>(b, c, sb.b_start, lds, stage, mine, sb.work, flag, bid - ga,
                                 (int64_t)gridDim.x - ga);
        write_status(sb, flag, bid - ga);
    }
}

// Work of one operand: row path, wave units; column path, workgroup tiles.
static int64_t split_work(const SplitOperand &op, bool pair, bool cols) {
    const int64_t kblocks = op.k_pad / kKBlock;
    if (cols) {
        const int64_t nt = pair ? ColsTile<true>::NT : ColsTile<false>::NT;
        return (op.r_pad + nt - 1) / nt * kblocks;
    }
    return op.r_pad / (pair ? kRowsPair : kRowsSingle) * kblocks;
}

// blocks the work asks for (before the cap at what the device holds at once)
static int64_t split_blocks(const SplitOperand &op, bool pair, bool cols) {
    const int64_t w = split_work(op, pair, cols);
    return cols ? w : (w + kSplitWaves - 1) / kSplitWaves;
}

// blocks of one operand for any limb count and either path
static int64_t split_blocks_max(const SplitOperand &op) {
    int64_t m = 0;
    for (int pair = 0; pair < 2; pair++)
        for (int cols = 0; cols < 2; cols++) {
            const int64_t b = split_blocks(op, pair != 0, cols != 0);
            m = b > m ? b : m;
        }
    return m;
}

int64_t split_status_slots(const SplitOperand *a, const SplitOperand *b, int) {
    return kStatusHeader + (a ? split_blocks_max(*a) : 0) + split_blocks_max(*b);
}

// Resident blocks of a kernel on the current device (compute units times
// blocks per unit), found once per kernel.
template <typename Kern>
static int64_t resident_blocks(Kern kernel) {
    static const int64_t cached = [&] {
        int dev = 0, cus = 0, per = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 1;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, kSplitThreads, 0) != hipSuccess || per < 1)
            per = 1;
        return (int64_t)cus * per;
    }();
    return cached;
}

template <int L, bool FP, bool COLS, int NB>
static int64_t launch_one(const SplitOperand &op, const SplitConsts &c, SplitStatus st, int64_t blocks,
                          bool dry, hipStream_t s) {
    auto kernel = split_kernel<L, FP, COLS, NB>;
    const int64_t cap = resident_blocks(kernel);
    const int64_t grid = blocks < cap ? blocks : cap;
    if (!dry) hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kSplitThreads), 0, s, op, c, st);
    return grid;
}

template <int L, bool FP, bool COLS>
static int64_t launch_nb(int nb, const SplitOperand &op, const SplitConsts &c, const SplitStatus &st,
                         int64_t blocks, bool dry, hipStream_t s) {
    switch (nb) {
        case 1: return launch_one<L, FP, COLS, 1>(op, c, st, blocks, dry, s);
        case 2: return launch_one<L, FP, COLS, 2>(op, c, st, blocks, dry, s);
        case 3: if constexpr (L <= 2) return launch_one<L, FP, COLS, 3>(op, c, st, blocks, dry, s); else return -1;
        case 4: if constexpr (L <= 2) return launch_one<L, FP, COLS, 4>(op, c, st, blocks, dry, s); else return -1;
        default: return -1;
    }
}

template <bool FP, bool COLS>
static int64_t launch_kind(int nb, const SplitOperand &op, const SplitConsts &c, const SplitStatus &st,
                           int64_t blocks, bool dry, hipStream_t s) {
    switch (op.limbs) {
        case 1: return launch_nb<1, FP, COLS>(nb, op, c, st, blocks, dry, s);
        case 2: return launch_nb<2, FP, COLS>(nb, op, c, st, blocks, dry, s);
        case 3: return launch_nb<3, FP, COLS>(nb, op, c, st, blocks, dry, s);
        default: return launch_nb<4, FP, COLS>(nb, op, c, st, blocks, dry, s);
    }
}

// The grid of one operand's launch (dry) or the launch itself.
static int64_t launch_operand(const SplitOperand &op, const SplitConsts &c, const SplitStatus &st, bool dry,
                              hipStream_t s) {
    const bool pair = op.limbs <= 2, cols = op.transposed != 0;
    const int per = pair ? 16 : 32;
    const int nb = (c.n + per - 1) / per;
    const int64_t blocks = split_blocks(op, pair, cols);
    if (op.fp64)
        return cols ? launch_kind<true, true>(nb, op, c, st, blocks, dry, s)
                    : launch_kind<true, false>(nb, op, c, st, blocks, dry, s);
    return cols ? launch_kind<false, true>(nb, op, c, st, blocks, dry, s)
                : launch_kind<false, false>(nb, op, c, st, blocks, dry, s);
}

// The fused launch of both operands (split_ab_kernel), or -1 where no
// instance exists.  dry: only the resident-block count of that instance.
template <int L, int NB>
static int64_t launch_ab_one(const SplitOperand &a, const SplitOperand &b, const SplitConsts &c,
                             const SplitStatus &sa, const SplitStatus &sb, int64_t ga, int64_t gb, bool dry,
                             hipStream_t s) {
    auto kernel = split_ab_kernel<L, NB>;
    if (dry) return resident_blocks(kernel);
    hipLaunchKernelGGL(kernel, dim3((unsigned)(ga + gb)), dim3(kSplitThreads), 0, s, a, b, c, sa, sb, (int32_t)ga);
    return ga + gb;
}
template <int L>
static int64_t launch_ab_nb(int nb, const SplitOperand &a, const SplitOperand &b, const SplitConsts &c,
                            const SplitStatus &sa, const SplitStatus &sb, int64_t ga, int64_t gb, bool dry,
                            hipStream_t s) {
    switch (nb) {
        case 1: return launch_ab_one<L, 1>(a, b, c, sa, sb, ga, gb, dry, s);
        case 2: return launch_ab_one<L, 2>(a, b, c, sa, sb, ga, gb, dry, s);
        case 3: if constexpr (L <= 2) return launch_ab_one<L, 3>(a, b, c, sa, sb, ga, gb, dry, s); else return -1;
        case 4: if constexpr (L <= 2) return launch_ab_one<L, 4>(a, b, c, sa, sb, ga, gb, dry, s); else return -1;
        default: return -1;
    }
}
static int64_t launch_ab(const SplitOperand &a, const SplitOperand &b, const SplitConsts &c, const SplitStatus &sa,
                         const SplitStatus &sb, int64_t ga, int64_t gb, bool dry, hipStream_t s) {
    const int nb = (c.n + (a.limbs <= 2 ? 16 : 32) - 1) / (a.limbs <= 2 ? 16 : 32);
    switch (a.limbs) {
        case 1: return launch_ab_nb<1>(nb, a, b, c, sa, sb, ga, gb, dry, s);
        case 2: return launch_ab_nb<2>(nb, a, b, c, sa, sb, ga, gb, dry, s);
        case 3: return launch_ab_nb<3>(nb, a, b, c, sa, sb, ga, gb, dry, s);
        default: return launch_ab_nb<4>(nb, a, b, c, sa, sb, ga, gb, dry, s);
    }
}

int launch_split(const SplitOperand *a, const SplitOperand *b, const SplitConsts &c,
                 uint32_t *status, int64_t status_slots, hipStream_t s) {
    if (c.n < 1 || c.n > kMaxPrimes) return RNS_E_ARG;
    const SplitOperand *ops[2] = {a, b};
    int64_t grid[2] = {0, 0};
    SplitStatus st[2] = {};
    for (int i = 0; i < 2; i++) {
        if (!ops[i]) continue;
        const SplitOperand &op = *ops[i];
        // the paths assume whole 16-row groups and whole K blocks
        if (op.limbs < 1 || op.limbs > RNS_MAX_IN_LIMBS || op.r_pad % 16 || op.k_pad % kKBlock ||
            op.rows > op.r_pad || op.k > op.k_pad || op.rows < 0 || op.k < 0 ||
            op.plane < op.r_pad * op.k_pad)
            return RNS_E_ARG;
        st[i].status = status;
        st[i].work = split_work(op, op.limbs <= 2, op.transposed != 0);
        st[i].flag_bit = i == 0 ? RNS_FLAG_A_RANGE : RNS_FLAG_B_RANGE;
        st[i].b_start = i;
        if (st[i].work > 0) grid[i] = launch_operand(op, c, st[i], true, s);
        if (grid[i] < 0) return RNS_E_ARG;
    }
    const int64_t total = grid[0] + grid[1];
    if (total <= 0) return RNS_OK;
    if (total + kStatusHeader > status_slots || total > 0x7fffffff) return RNS_E_ARG;
    // Both operands in one launch when A (row path) and B (column path, B
    // given as [K][N]) have integer entries of the same limb count: the
    // blocks (at most the fused kernel's resident ones) are shared in
    // proportion to the work, and each walks its operand's units with the
    // stride of its share.  Small shapes lose one launch and its gap; on the
    // wide workload (2048 x 4096 entries each, 2 limbs, 29 primes) the two
    // access patterns running side by side and the single tail take the
    // split from 157-160 us to 144-148 us.
    if (grid[0] > 0 && grid[1] > 0 && !a->fp64 && !b->fp64 && a->limbs == b->limbs && !a->transposed &&
        b->transposed) {
        const bool pair = a->limbs <= 2;
        const int64_t ba = split_blocks(*a, pair, false), bb = split_blocks(*b, pair, true);
        const int64_t cap = launch_ab(*a, *b, c, st[0], st[1], 0, 0, true, s);
        if (cap > 1) {
            int64_t ga = ba, gb = bb;
            if (ba + bb > cap) {
                ga = ba * cap / (ba + bb);
                ga = ga < 1 ? 1 : (ga > ba ? ba : ga);
                gb = cap - ga;
                gb = gb < 1 ? 1 : (gb > bb ? bb : gb);
            }
            if (ga + gb + kStatusHeader > status_slots) return RNS_E_ARG;
            st[0].first = 0;
            st[1].first = (int32_t)ga;
            st[0].total = st[1].total = (int32_t)(ga + gb);
            if (launch_ab(*a, *b, c, st[0], st[1], ga, gb, false, s) < 0) return RNS_E_ARG;
            return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
        }
    }
    int64_t first = 0;
    for (int i = 0; i < 2; i++) {
        if (grid[i] == 0) continue;
        st[i].first = (int32_t)first;
        st[i].total = (int32_t)total;
        launch_operand(*ops[i], c, st[i], false, s);
        if (hipGetLastError() != hipSuccess) return RNS_E_HIP;
        first += grid[i];
    }
    return RNS_OK;
}

// ============================================================================
// repack of caller-given residue planes into the padded tile layout
// ============================================================================
__global__ void repack_kernel(const int8_t *src, int64_t n, int64_t M, int64_t K,
                              int8_t *dst, int64_t m_pad, int64_t k_pad, int64_t plane) {
    const int64_t total = n * m_pad * k_pad;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = i / (m_pad * k_pad);
        const int64_t rem = i - p * m_pad * k_pad;
        const int64_t m = rem / k_pad, k = rem - m * k_pad;
        dst[p * plane + (k / kKBlock) * (m_pad * kKBlock) + m * kKBlock + k % kKBlock] =
            (m < M && k < K) ? src[(p * M + m) * K + k] : (int8_t)0;
    }
}

int launch_repack_residues(const int8_t *src, int64_t n, int64_t M, int64_t K,
                           int8_t *dst, int64_t m_pad, int64_t k_pad, int64_t plane, hipStream_t s) {
    const int64_t total = n * m_pad * k_pad;
    if (total == 0) return RNS_OK;
    int64_t grid = (total + 255) / 256;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(repack_kernel, dim3((unsigned)grid), dim3(256), 0, s, src, n, M, K, dst, m_pad,
                       k_pad, plane);
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

}  // namespace rns
