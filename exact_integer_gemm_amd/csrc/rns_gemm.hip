// K2 of the exact residue GEMM on gfx950: one INT8 MFMA product per prime
// with int32 accumulation and a fused reduction mod q (exact-solve, "Method":
// one INT8 GEMM per prime, batched; exact for K <= 2^17).
#include "rns_device.h"

namespace rns {

// ============================================================================
// K2: prime-batched INT8 MFMA product with fused mod-q epilogue
// ============================================================================
// Operands are K-contiguous int8 planes: A [Mp][Kp] and B^T [Np][Kp] per prime.
// A block computes one BM x BN tile of one prime.  Tiles of BK bytes of K are
// staged through LDS (double buffered, one barrier per step) as 16-byte
// chunks, XOR-swizzled so that fragment reads are free of bank conflicts
// (see swz).  Each wave owns a (BM/WM) x (BN/WN) sub-tile built from
// v_mfma_i32_32x32x32_i8; the operand fragments of the next 32-wide K slice
// are read from LDS while the MFMAs of the current one run.  The MFMA is fed
// B^T as its first operand so that each lane's accumulators hold four
// consecutive output columns of one row, which pack into one 32-bit store.
//
// Block order: the hardware hands consecutive workgroups to the 8 XCDs in
// turn, so workgroup i is remapped to tile (i % 8) * G/8 + i / 8: each XCD
// works through a contiguous run of tiles of the same prime, whose A rows
// and B columns its own L2 then serves to all of them.
struct GemmArgs {
    const int8_t *a;
    const int8_t *b;
    int8_t *y;
    int64_t a_plane, b_plane, y_plane;   // bytes between planes
    int64_t a_row, a_kstep;              // A: bytes between rows, between K steps of BK
    int64_t b_row, b_kstep;              // B^T: the same
    int64_t y_pitch;                     // Y: bytes between rows
    int32_t kt;                          // K steps of BK bytes
    int32_t tiles_m, tiles_n;
    // Large tiling only: the first full_tiles workgroups each run a whole
    // tile; each later workgroup runs 1/split of the K steps of one of the
    // remaining tiles and leaves its residues in `partial` (kTailUnitBytes
    // per workgroup), which gemm_tail4_kernel combines.
    int32_t full_tiles, split;
    int8_t *partial;
    int32_t tiles;                       // all tiles of all primes
};

// ds_read_b128 is served 32 lanes at a time from 64 banks of 4 bytes: a
// group is conflict-free when every 16-byte bank slot (address / 16 mod 16)
// is hit by exactly two of its lanes.  A fragment read has 32 consecutive
// rows at one logical chunk, so the physical chunk is XORed with bits of the
// row that, together with the row's own slot offset, spread the 32 rows
// evenly: for 64-byte rows the slot is 4 * (row & 3) + chunk, for 128-byte
// rows 8 * (row & 1) + chunk.
template <int CH>
__device__ __forceinline__ int swz(int row) {
    if constexpr (CH == 4) return (row >> 2) & 3;
    else return (row ^ (row >> 3)) & 7;
}

template <int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g, EpiConsts ec) {
    constexpr int NT = 256;
    static_assert(WM * WN * 64 == NT, "four waves");
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int CH = BK / 16;
    constexpr int KK = BK / 32;
    constexpr int A_CHUNKS = BM * CH, B_CHUNKS = BN * CH;
    constexpr int LA = (A_CHUNKS + NT - 1) / NT, LB = (B_CHUNKS + NT - 1) / NT;
    static_assert(FM >= 1 && FN >= 1 && KK % 2 == 0, "tile shape");

    __shared__ v4i lds[2][A_CHUNKS + B_CHUNKS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = wave / WN, wn = wave % WN;
    const int half = lane >> 5, l32 = lane & 31;

    // XCD-aware workgroup -> tile map (a bijection on [0, G))
    const int G = gridDim.x;
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int tile = xcd * (G >> 3) + min(xcd, G & 7) + idx;
    const int per_prime = g.tiles_m * g.tiles_n;
    const int p = tile / per_prime;
    const int t = tile - p * per_prime;
    const int tm = t / g.tiles_n, tn = t - tm * g.tiles_n;

    const int8_t *Ap = g.a + p * g.a_plane + (int64_t)(tm * BM) * g.a_row;
    const int8_t *Bp = g.b + p * g.b_plane + (int64_t)(tn * BN) * g.b_row;

    v4i ra[LA], rb[LB];
    auto load_global = [&](int kt) {
        const int8_t *As = Ap + kt * g.a_kstep, *Bs = Bp + kt * g.b_kstep;
#pragma unroll
        for (int i = 0; i < LA; i++) {
            const int c = tid + i * NT;
            if (A_CHUNKS % NT == 0 || c < A_CHUNKS)
                ra[i] = *(const v4i *)(As + (int64_t)(c / CH) * g.a_row + (c % CH) * 16);
        }
#pragma unroll
        for (int i = 0; i < LB; i++) {
            const int c = tid + i * NT;
            if (B_CHUNKS % NT == 0 || c < B_CHUNKS)
                rb[i] = *(const v4i *)(Bs + (int64_t)(c / CH) * g.b_row + (c % CH) * 16);
        }
    };
    auto store_lds = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LA; i++) {
            const int c = tid + i * NT;
            if (A_CHUNKS % NT == 0 || c < A_CHUNKS) {
                const int row = c / CH, col = c % CH;
                lds[buf][row * CH + (col ^ swz<CH>(row))] = ra[i];
            }
        }
#pragma unroll
        for (int i = 0; i < LB; i++) {
            const int c = tid + i * NT;
            if (B_CHUNKS % NT == 0 || c < B_CHUNKS) {
                const int row = c / CH, col = c % CH;
                lds[buf][A_CHUNKS + row * CH + (col ^ swz<CH>(row))] = rb[i];
            }
        }
    };
    auto read_frags = [&](int buf, int kk, v4i (&af)[FM], v4i (&bf)[FN]) {
        const int chunk = kk * 2 + half;
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int row = wm * TM + i * 32 + l32;
            af[i] = lds[buf][row * CH + (chunk ^ swz<CH>(row))];
        }
#pragma unroll
        for (int j = 0; j < FN; j++) {
            const int row = wn * TN + j * 32 + l32;
            bf[j] = lds[buf][A_CHUNKS + row * CH + (chunk ^ swz<CH>(row))];
        }
    };

    v16i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) acc[i][j] = v16i{0};

    v4i af[2][FM], bf[2][FN];
    const int KT = g.kt;
    if (KT > 0) {
        load_global(0);
        store_lds(0);
    }
    __syncthreads();
    if (KT > 0) read_frags(0, 0, af[0], bf[0]);
    for (int kt = 0; kt < KT; kt++) {
        const int buf = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) load_global(kt + 1);
#pragma unroll
        for (int kk = 0; kk < KK; kk++) {
            const int cur = kk & 1;
            if (kk + 1 < KK) read_frags(buf, kk + 1, af[cur ^ 1], bf[cur ^ 1]);
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[cur][j], af[cur][i],
                                                                      acc[i][j], 0, 0, 0);
        }
        if (more) store_lds(buf ^ 1);
        __syncthreads();
        if (more) read_frags(buf ^ 1, 0, af[0], bf[0]);
    }

    // epilogue: balanced residue mod q of every accumulator, as int8
    const int q = ec.q[p];
    const double inv = ec.inv[p];
    int8_t *Yp = g.y + p * g.y_plane;
#pragma unroll
    for (int i = 0; i < FM; i++) {
        const int64_t m = tm * BM + wm * TM + i * 32 + l32;
#pragma unroll
        for (int j = 0; j < FN; j++) {
#pragma unroll
            for (int gq = 0; gq < 4; gq++) {
                const int n = tn * BN + wn * TN + j * 32 + 8 * gq + 4 * half;
                int r[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int s = acc[i][j][4 * gq + e];
                    r[e] = q == 2 ? (s & 1) : reduce_low_byte(s, q, inv);
                }
                *(uint32_t *)(Yp + m * g.y_pitch + n) = pack4(r[0], r[1], r[2], r[3]);
            }
        }
    }
}

// ---- large-tile output ---------------------------------------------------------
// A 256 x 256 tile is held by NW waves (8: sub-tiles of 128 x 64, 4: sub-tiles
// of 128 x 128), wave w at (wm, wn) = (w % 2, w / 2), as 4 x FN MFMA
// accumulators (FN = 16 / NW): acc[i][j][4 * gq + e] is row wm*128 + i*32 +
// l32, column wn*32*FN + j*32 + 8*gq + 4*half + e.  The balanced residues mod
// q go through LDS (row pitch kOutPitch) so that the tile leaves in whole
// 16-byte row chunks.  `out` must hold 256 * kOutPitch bytes.
constexpr int kOutPitch = 256 + 16;

template <int NW>
__device__ __forceinline__ void store_big_tile(v16i (&acc)[4][16 / NW], int q, double inv, int8_t *out,
                                               int8_t *Yp, int64_t y_pitch, int tid) {
    constexpr int FN = 16 / NW;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1, half = lane >> 5, l32 = lane & 31;
    if (q == 2) {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < FN; j++)
#pragma unroll
                for (int gq = 0; gq < 4; gq++) {
                    const int row = wm * 128 + i * 32 + l32;
                    const int col = wn * 32 * FN + j * 32 + 8 * gq + 4 * half;
                    const v16i &a = acc[i][j];
                    *(uint32_t *)(out + row * kOutPitch + col) =
                        pack4(a[4 * gq] & 1, a[4 * gq + 1] & 1, a[4 * gq + 2] & 1, a[4 * gq + 3] & 1);
                }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < FN; j++)
#pragma unroll
                for (int gq = 0; gq < 4; gq++) {
                    const int row = wm * 128 + i * 32 + l32;
                    const int col = wn * 32 * FN + j * 32 + 8 * gq + 4 * half;
                    const v16i &a = acc[i][j];
                    *(uint32_t *)(out + row * kOutPitch + col) =
                        pack4(reduce_low_byte(a[4 * gq], q, inv), reduce_low_byte(a[4 * gq + 1], q, inv),
                              reduce_low_byte(a[4 * gq + 2], q, inv), reduce_low_byte(a[4 * gq + 3], q, inv));
                }
    }
    __syncthreads();
    // 256 rows x 256 bytes: 16 lanes per row, 4 * NW rows per pass
#pragma unroll
    for (int pass = 0; pass < 64 / NW; pass++) {
        const int row = pass * 4 * NW + (tid >> 4);
        const int c = (tid & 15) * 16;
        *(v4i *)(Yp + (int64_t)row * y_pitch + c) = *(const v4i *)(out + row * kOutPitch + c);
    }
}

// A part of a split tile leaves its residues for gemm_tail4_kernel: thread
// tid's 64 * FN values as 4 * FN runs of 16 bytes, run c = i * FN + j at
// [c][tid][16] of the part's kTailUnitBytes slot.
// For q = 2 the rounding step leaves s - 2 round(s / 2) in {-1, 0, 1}, whose
// low bit is the residue: `keep` masks each byte to it.
__device__ __forceinline__ uint32_t residue_keep_mask(int q) { return q == 2 ? 0x01010101u : 0xffffffffu; }

template <int NW>
__device__ __forceinline__ void store_part(v16i (&acc)[4][16 / NW], int q, double inv, int8_t *slot,
                                           int tid) {
    constexpr int FN = 16 / NW;
    const uint32_t keep = residue_keep_mask(q);
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) {
            const v16i &a = acc[i][j];
            uint32_t w[4];
#pragma unroll
            for (int gq = 0; gq < 4; gq++)
                w[gq] = pack4(reduce_low_byte(a[4 * gq], q, inv), reduce_low_byte(a[4 * gq + 1], q, inv),
                              reduce_low_byte(a[4 * gq + 2], q, inv), reduce_low_byte(a[4 * gq + 3], q, inv)) &
                        keep;
            *(v4u *)(slot + ((i * FN + j) * 64 * NW + tid) * 16) = v4u{w[0], w[1], w[2], w[3]};
            __builtin_amdgcn_sched_barrier(0);          // one block at a time: bounded registers
        }
}

// ---- the large-tile variant: 8 waves in ping-pong ----------------------------
// 256 x 256 tiles, BK = 64, 512 threads: two waves per SIMD (waves w and w+4
// share SIMD w % 4).  Each wave owns a 128 x 64 sub-tile (8 accumulator
// chains).  The waves form two groups that alternate between a memory phase
// (reading the fragments of a K step from LDS) and a compute phase (16 MFMAs
// on those fragments, with this wave's share of the direct global->LDS loads
// of a later K step slotted between them), one group in each phase at any
// time, so that one wave per SIMD always has MFMAs to issue while its partner
// waits on LDS.  Phases end at a plain s_barrier; ordering is by explicit
// counter waits: in its memory phase for step j a wave waits (vmcnt) for its
// own loads of step j + 1 and (lgkmcnt) for its fragment reads, so after the
// next barrier step j + 1 is complete in LDS and step j - 1's stage is no
// longer read.  The LDS holds an S-stage ring; step j + S - 1 is requested
// during the compute phase of step j, into the stage of step j - 1.
template <int S>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmArgs g, EpiConsts ec) {
    constexpr int BM = 256, BN = 256, BK = 64, CH = BK / 16;
    constexpr int FM = 4, FN = 2;                  // 128 x 64 per wave
    constexpr int STAGE = (BM + BN) * CH;          // 2048 chunks = 32 KB
    constexpr int DPW = STAGE / 512;               // 4 loads per wave per step
    constexpr int D = S - 1;                       // prefetch distance in steps
    static_assert(S >= 2 && S <= 4 && S * STAGE * 16 <= 160 * 1024, "LDS ring");
    static_assert(BM * kOutPitch <= S * STAGE * 16, "output staging fits the ring");

    __shared__ v4i lds[S][STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int group = wave >> 2;
    const int wm = wave & 1, wn = wave >> 1;       // 2 x 4 waves over the tile
    const int half = lane >> 5, l32 = lane & 31;

    // Whole tiles: workgroup b runs on XCD b % 8 (round-robin dispatch), so
    // each XCD gets one contiguous range of tiles and its L2 serves tiles
    // that share operand rows.  Split tiles: unit u runs part u % split.
    int tile, unit = -1, part = 0, k_first = 0, KT = g.kt;
    if ((int)blockIdx.x < g.full_tiles) {
        const int G = g.full_tiles;
        const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
        tile = xcd * (G >> 3) + min(xcd, G & 7) + idx;
    } else {
        unit = blockIdx.x - g.full_tiles;
        const int t = unit / g.split;
        part = unit - t * g.split;
        tile = g.full_tiles + t;
        KT = g.kt / g.split;
        k_first = part * KT;
    }
    const int per_prime = g.tiles_m * g.tiles_n;
    const int p = tile / per_prime;
    const int t = tile - p * per_prime;
    const int tm = t / g.tiles_n, tn = t - tm * g.tiles_n;
    const int8_t *Ap = g.a + p * g.a_plane + (int64_t)(tm * BM) * g.a_row + k_first * g.a_kstep;
    const int8_t *Bp = g.b + p * g.b_plane + (int64_t)(tn * BN) * g.b_row + k_first * g.b_kstep;

    // Load j of this wave fills LDS slots [(j*8 + wave)*64, +64) of a stage:
    // loads 0, 1 carry A rows, loads 2, 3 B rows.
    const int8_t *src[DPW];
#pragma unroll
    for (int j = 0; j < DPW; j++) {
        const int s = (j * 8 + wave) * 64 + lane;
        const int row = s / CH;
        const int c = (s % CH) ^ swz<CH>(row);
        src[j] = row < BM ? Ap + (int64_t)row * g.a_row + c * 16
                          : Bp + (int64_t)(row - BM) * g.b_row + c * 16;
    }
    auto issue = [&](int step) {
        v4i *dst = lds[step % S];
#pragma unroll
        for (int j = 0; j < DPW; j++)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(
                    src[j] + step * (j < DPW / 2 ? g.a_kstep : g.b_kstep)),
                (__attribute__((address_space(3))) void *)(dst + (j * 8 + wave) * 64), 16, 0, 0);
    };
    // s_waitcnt vmcnt(4 * n), other counters untouched (gfx9 encoding: vmcnt
    // in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8): at most n later steps
    // of this wave's loads may still be pending
    auto wait_steps = [&](int n) {
        if (n <= 0) __builtin_amdgcn_s_waitcnt(0x0f70);
        else if (n == 1) __builtin_amdgcn_s_waitcnt(0x0f74);
        else __builtin_amdgcn_s_waitcnt(0x0f78);
    };
    auto read_frags = [&](int stage, int kk, v4i (&af)[FM], v4i (&bf)[FN]) {
        const int chunk = kk * 2 + half;
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int row = wm * 128 + i * 32 + l32;
            af[i] = lds[stage][row * CH + (chunk ^ swz<CH>(row))];
        }
#pragma unroll
        for (int j = 0; j < FN; j++) {
            const int row = BM + wn * 64 + j * 32 + l32;
            bf[j] = lds[stage][row * CH + (chunk ^ swz<CH>(row))];
        }
    };

    v16i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) acc[i][j] = v16i{0};
    v4i af0[FM], bf0[FN], af1[FM], bf1[FN];

    // memory phase for step j: request step j + D, read the fragments of step
    // j, then wait for own loads of step j + 1 and for the fragments
    auto memory = [&](int j) {
        read_frags(j % S, 0, af0, bf0);
        read_frags(j % S, 1, af1, bf1);
        wait_steps(min(j + D - 1, KT - 1) - (j + 1));
        __builtin_amdgcn_s_waitcnt(0xc07f);        // lgkmcnt(0)
    };
    auto compute = [&](int jj) {
        const bool more = jj + D < KT;
        const int step = jj + D;
        v4i *dst = lds[step % S];
#pragma unroll
        for (int i = 0; i < FM; i++) {
#pragma unroll
            for (int j = 0; j < FN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf0[j], af0[i], acc[i][j], 0, 0, 0);
            if (more)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void *)(
                        src[i] + step * (i < DPW / 2 ? g.a_kstep : g.b_kstep)),
                    (__attribute__((address_space(3))) void *)(dst + (i * 8 + wave) * 64), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf1[j], af1[i], acc[i][j], 0, 0, 0);
    };

    if (KT > 0) {
#pragma unroll
        for (int s = 0; s < D; s++)
            if (s < KT) issue(s);
        wait_steps(min(D - 1, KT - 1));            // own loads of step 0 done
        __builtin_amdgcn_s_barrier();               // step 0 visible
        // Every wave runs memory(j), barrier, compute, barrier.  Group 1
        // starts one barrier late (and group 0 ends one barrier late), so
        // the compute phase of one group coincides with the memory phase of
        // the other.
        // sched_barrier(0) keeps the compiler from moving instructions
        // across a phase boundary.
        if (group == 1) __builtin_amdgcn_s_barrier();
        for (int j = 0; j < KT; j++) {
            memory(j);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            compute(j);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
        if (group == 0) __builtin_amdgcn_s_barrier();
    }

    __builtin_amdgcn_s_waitcnt(0x0f70);             // vmcnt(0): no load may still target LDS
    __syncthreads();
    const int q = ec.q[p];
    const double inv = ec.inv[p];

    if (unit >= 0) {
        store_part<8>(acc, q, inv, g.partial + (int64_t)unit * kTailUnitBytes, tid);
        return;
    }
    store_big_tile<8>(acc, q, inv, (int8_t *)&lds[0][0],
                      g.y + p * g.y_plane + (int64_t)(tm * BM) * g.y_pitch + tn * BN, g.y_pitch, tid);
}

// ---- the persistent variant ---------------------------------------------------
// gemm_pp_kernel's ping-pong with one workgroup per compute unit (G of them, G
// a multiple of 8), each running a fixed list of items: the whole tiles b, b +
// G, b + 2G, ... in the same XCD-aware order (G = 0 mod 8 keeps every item of
// workgroup b on XCD b % 8), then K part b of the split tiles, if there is
// one.  The LDS ring and the direct loads run on across items: a workgroup
// counts its K steps globally, and the first steps of its next item are
// requested during the last compute phases of the current one, so no item
// starts by waiting for operands.  Each wave reduces and stores its own
// 128 x 64 sub-tile right after its last compute phase of an item (no LDS, no
// barrier), while the other group's waves keep the matrix cores busy; the
// first compute phase of the next item starts its chains from zero.
template <int S>
__global__ __launch_bounds__(512) void gemm_ps_kernel(GemmArgs g, EpiConsts ec) {
    constexpr int BM = 256, BN = 256, BK = 64, CH = BK / 16;
    constexpr int FM = 4, FN = 2;                  // 128 x 64 per wave
    constexpr int STAGE = (BM + BN) * CH;          // 2048 chunks = 32 KB
    constexpr int DPW = STAGE / 512;               // 4 loads per wave per step
    constexpr int D = S - 1;                       // prefetch distance in steps
    constexpr int NST = FM * FN;                   // stores per wave per item
    static_assert(S >= 2 && S <= 4 && S * STAGE * 16 <= 160 * 1024, "LDS ring");
    static_assert(DPW == FM, "one direct load after each of the first FM MFMA rows");

    __shared__ v4i lds[S][STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int group = wave >> 2;
    const int wm = wave & 1, wn = wave >> 1;
    const int half = lane >> 5, l32 = lane & 31;

    const int G = gridDim.x, b = blockIdx.x;
    const int nfull = b < g.full_tiles ? (g.full_tiles - 1 - b) / G + 1 : 0;
    const bool has_part = b < (g.tiles - g.full_tiles) * g.split;
    const int kt_part = g.kt / g.split;
    const int items = nfull + (has_part ? 1 : 0);
    const int KT = nfull * g.kt + (has_part ? kt_part : 0);
    const int per_prime = g.tiles_m * g.tiles_n;

    // item -> prime, tile row and column, first K step
    auto locate = [&](int item, int &p, int &tm, int &tn, int &k_first) {
        int tile;
        k_first = 0;
        if (item < nfull) {
            const int F = g.full_tiles, v = b + item * G;
            const int xcd = v & 7, idx = v >> 3;
            tile = xcd * (F >> 3) + min(xcd, F & 7) + idx;
        } else {
            tile = g.full_tiles + b / g.split;
            k_first = (b % g.split) * kt_part;
        }
        p = tile / per_prime;
        const int t = tile - p * per_prime;
        tm = t / g.tiles_n;
        tn = t - tm * g.tiles_n;
    };

    // Load j of this wave fills LDS slots [(j*8 + wave)*64, +64) of a stage:
    // loads 0, 1 carry A rows, loads 2, 3 B rows; off[j] is this lane's byte
    // offset from the tile's first row at the current K step.
    uint32_t off[DPW];
#pragma unroll
    for (int j = 0; j < DPW; j++) {
        const int s = (j * 8 + wave) * 64 + lane;
        const int row = s / CH;
        const int c = (s % CH) ^ swz<CH>(row);
        off[j] = row < BM ? (uint32_t)(row * g.a_row + c * 16) : (uint32_t)((row - BM) * g.b_row + c * 16);
    }
    // the load cursor: item and remaining steps of the next step to request
    int d_item = 0, d_left = 0;
    const int8_t *dA = g.a, *dB = g.b;
    auto d_start = [&](int item) {
        int p, tm, tn, kf;
        locate(item, p, tm, tn, kf);
        dA = g.a + p * g.a_plane + (int64_t)(tm * BM) * g.a_row + kf * g.a_kstep;
        dB = g.b + p * g.b_plane + (int64_t)(tn * BN) * g.b_row + kf * g.b_kstep;
        d_left = item < nfull ? g.kt : kt_part;
    };
    auto d_load = [&](int j, v4i *dst) {
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void *)((j < DPW / 2 ? dA : dB) + off[j]),
            (__attribute__((address_space(3))) void *)(dst + (j * 8 + wave) * 64), 16, 0, 0);
    };
    auto d_advance = [&]() {
        dA += g.a_kstep;
        dB += g.b_kstep;
        if (--d_left == 0 && ++d_item < items) d_start(d_item);
    };
    // s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding: vmcnt in
    // bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).  Vector memory
    // operations, the direct loads and the output stores alike, complete in
    // the order they were issued.
    auto wait_vm = [&](int n) {
        switch (n) {
            case 0: __builtin_amdgcn_s_waitcnt(0x0f70); break;
            case 4: __builtin_amdgcn_s_waitcnt(0x0f74); break;
            case 8: __builtin_amdgcn_s_waitcnt(0x0f78); break;
            case 12: __builtin_amdgcn_s_waitcnt(0x0f7c); break;
            default: __builtin_amdgcn_s_waitcnt(0x4f70); break;   // 16
        }
    };
    auto read_frags = [&](int stage, int kk, v4i (&af)[FM], v4i (&bf)[FN]) {
        const int chunk = kk * 2 + half;
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int row = wm * 128 + i * 32 + l32;
            af[i] = lds[stage][row * CH + (chunk ^ swz<CH>(row))];
        }
#pragma unroll
        for (int j = 0; j < FN; j++) {
            const int row = BM + wn * 64 + j * 32 + l32;
            bf[j] = lds[stage][row * CH + (chunk ^ swz<CH>(row))];
        }
    };

    v16i acc[FM][FN];
    v4i af0[FM], bf0[FN], af1[FM], bf1[FN];

    // memory phase for global step j: read the fragments of step j, then wait
    // for the fragments and for own loads of step j + 1, behind which n later
    // steps of loads may stay pending (and, in the first D - 1 steps of an
    // item, the previous item's output stores)
    auto pending = [&](int j) { return max(min(j + D - 1, KT - 1) - (j + 1), 0); };
    auto memory = [&](int j, int n, bool after_store) {
        read_frags(j % S, 0, af0, bf0);
        read_frags(j % S, 1, af1, bf1);
        wait_vm(4 * n + (after_store ? NST : 0));
        __builtin_amdgcn_s_waitcnt(0xc07f);        // lgkmcnt(0)
    };
    // compute phase for global step j: 16 MFMAs, the loads of step j + D
    // between them; FIRST starts the chains from zero; CHECK: step j + D may
    // be past the end or in the next item
    auto compute = [&](auto first, auto check, int jj) {
        constexpr bool FIRST = decltype(first)::value, CHECK = decltype(check)::value;
        const bool more = !CHECK || jj + D < KT;
        v4i *dst = lds[(jj + D) % S];
#pragma unroll
        for (int i = 0; i < FM; i++) {
#pragma unroll
            for (int j = 0; j < FN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf0[j], af0[i], FIRST ? v16i{0} : acc[i][j],
                                                                  0, 0, 0);
            if (more) d_load(i, dst);
        }
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf1[j], af1[i], acc[i][j], 0, 0, 0);
        if (more) {
            dA += g.a_kstep;
            dB += g.b_kstep;
            --d_left;
            if (CHECK && d_left == 0 && ++d_item < items) d_start(d_item);
        }
    };
    // one K step: memory phase, barrier, compute phase, barrier
    auto step = [&](auto first, auto check, int j, int n, bool after_store) {
        memory(j, n, after_store);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        compute(first, check, j);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // The lane index, read afresh where an item ends: values derived from it
    // there are not kept live (or spilled) across the whole item loop.
    auto lane_now = []() {
        int l;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
        return l;
    };
    // this wave's 128 x 64 sub-tile of item `item`: balanced residues mod q;
    // the two half-waves swap 4-byte runs so that each lane stores 16 bytes
    // of one row
    auto store_tile = [&](int item) {
        int p, tm, tn, kf;
        locate(item, p, tm, tn, kf);
        const int q = ec.q[p];
        const double inv = ec.inv[p];
        const uint32_t keep = residue_keep_mask(q);
        // a uniform base per accumulator block plus this lane's 32-bit offset
        const int ln = lane_now();
        const uint32_t yl = (uint32_t)((wm * 128 + (ln & 31)) * g.y_pitch + wn * 64 + 16 * (ln >> 5));
        int8_t *Yt = g.y + p * g.y_plane + (int64_t)(tm * BM) * g.y_pitch + tn * BN;
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++) {
                const v16i &a = acc[i][j];
                uint32_t w[4];
#pragma unroll
                for (int gq = 0; gq < 4; gq++)
                    w[gq] = pack4(reduce_low_byte(a[4 * gq], q, inv), reduce_low_byte(a[4 * gq + 1], q, inv),
                                  reduce_low_byte(a[4 * gq + 2], q, inv), reduce_low_byte(a[4 * gq + 3], q, inv)) &
                            keep;
                // w[gq] holds columns 8gq + 4 half .. + 3.  v_permlane32_swap
                // trades the upper half-wave of its first operand for the
                // lower half-wave of its second: lane (l32, 0) gets columns
                // 0 .. 15, lane (l32, 1) columns 16 .. 31.
                const auto s02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
                const auto s13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
                int8_t *Yb = Yt + (int64_t)(i * 32) * g.y_pitch + j * 32;
                *(v4u *)(Yb + yl) = v4u{s02[0], s02[1], s13[0], s13[1]};
                __builtin_amdgcn_sched_barrier(0);      // one block at a time: bounded registers
            }
    };
    auto epilogue = [&](int item) {
        int p, tm, tn, kf;
        locate(item, p, tm, tn, kf);
        if (item >= nfull)
            store_part<8>(acc, ec.q[p], ec.inv[p], g.partial + (int64_t)b * kTailUnitBytes, wave * 64 + lane_now());
        else
            store_tile(item);
    };

    if (KT == 0) return;
    d_start(0);
#pragma unroll
    for (int s = 0; s < D; s++)
        if (s < KT) {
            v4i *dst = lds[s % S];
#pragma unroll
            for (int j = 0; j < DPW; j++) d_load(j, dst);
            d_advance();
        }
    wait_vm(4 * min(D - 1, KT - 1));               // own loads of step 0 done
    __builtin_amdgcn_s_barrier();                   // step 0 visible
    // As in gemm_pp_kernel: group 1 runs one barrier behind group 0, so the
    // compute phase of one group coincides with the memory phase (and the
    // item epilogue) of the other.
    if (group == 1) __builtin_amdgcn_s_barrier();
    const std::true_type yes;
    const std::false_type no;
    int gs = 0;                                     // global K step
    for (int item = 0; item < items; item++) {
        const int len = item < nfull ? g.kt : kt_part;
        const bool after = item > 0;
        // the first D - 1 steps may wait behind the previous item's stores;
        // the loads of the last D + 1 steps may reach into the next item
        int j = 0;
        step(yes, yes, gs, pending(gs), after);
        for (j = 1, gs++; j < len && j < D - 1; j++, gs++) step(no, yes, gs, pending(gs), after);
        for (; j < len - D - 1; j++, gs++) step(no, no, gs, D - 2, false);
        for (; j < len; j++, gs++) step(no, yes, gs, pending(gs), false);
        epilogue(item);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (group == 0) __builtin_amdgcn_s_barrier();
}

// The split tiles: the residues the `split` parts of a tile left in their
// slots are added up (|sum| <= split * 128, exact in int32), reduced again
// mod q and stored like the product kernel stores a tile; NW matches the
// product kernel's wave count (the slots' layout).  Four workgroups per
// split tile, so the combine spreads over four times as many compute units:
// workgroup 4 t + i takes accumulator row block i of tile full_tiles + t
// (rows wm * 128 + 32 i + l32, all 256 columns: two runs of each part's
// slot).  Its 64 rows go through LDS and leave in 16-byte row chunks.
template <int NW>
__global__ __launch_bounds__(64 * NW) void gemm_tail4_kernel(GemmArgs g, EpiConsts ec) {
    constexpr int FN = 16 / NW;
    __shared__ v4i out[64 * kOutPitch / 16];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1, half = lane >> 5, l32 = lane & 31;
    const int t = blockIdx.x >> 2, i = blockIdx.x & 3;
    const int tile = g.full_tiles + t;
    const int per_prime = g.tiles_m * g.tiles_n;
    const int p = tile / per_prime;
    const int tt = tile - p * per_prime;
    const int tm = tt / g.tiles_n, tn = tt - tm * g.tiles_n;
    v16i acc[FN];
#pragma unroll
    for (int j = 0; j < FN; j++) acc[j] = v16i{0};
    const int8_t *slots = g.partial + (int64_t)t * g.split * kTailUnitBytes;
    for (int o = 0; o < g.split; o++) {
#pragma unroll
        for (int j = 0; j < FN; j++) {
            const v4i v = *(const v4i *)(slots + (int64_t)o * kTailUnitBytes + ((i * FN + j) * 64 * NW + tid) * 16);
#pragma unroll
            for (int e = 0; e < 16; e++) acc[j][e] += (int)(int8_t)(v[e >> 2] >> (8 * (e & 3)));
        }
    }
    const int q = ec.q[p];
    const double inv = ec.inv[p];
    const uint32_t keep = residue_keep_mask(q);
    int8_t *ob = (int8_t *)out;
#pragma unroll
    for (int j = 0; j < FN; j++)
#pragma unroll
        for (int gq = 0; gq < 4; gq++) {
            const int row = wm * 32 + l32;                       // local row
            const int col = wn * 32 * FN + j * 32 + 8 * gq + 4 * half;
            const v16i &a = acc[j];
            *(uint32_t *)(ob + row * kOutPitch + col) =
                pack4(reduce_low_byte(a[4 * gq], q, inv), reduce_low_byte(a[4 * gq + 1], q, inv),
                      reduce_low_byte(a[4 * gq + 2], q, inv), reduce_low_byte(a[4 * gq + 3], q, inv)) & keep;
        }
    __syncthreads();
    // 64 rows x 256 bytes: 16 lanes per row, 4 * NW rows per pass; local row
    // r is row (r / 32) * 128 + 32 i + r % 32 of the tile
    int8_t *Yp = g.y + p * g.y_plane + (int64_t)(tm * 256) * g.y_pitch + tn * 256;
#pragma unroll
    for (int pass = 0; pass < 16 / NW; pass++) {
        const int r = pass * 4 * NW + (tid >> 4);
        const int c = (tid & 15) * 16;
        const int row = (r >> 5) * 128 + 32 * i + (r & 31);
        *(v4i *)(Yp + (int64_t)row * g.y_pitch + c) = *(const v4i *)(ob + r * kOutPitch + c);
    }
}

// Compute units of the current device (cached per device).
static int device_cus() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev < 64) cached[dev] = cus;
    return cus;
}

int tail_split(int64_t tiles, int kt, int cus, int *split) {
    // Tiles beyond the last whole round over the compute units would leave
    // most units idle while they run; split each of them over K into as
    // many parts (a power of two, at least 4 K steps each) as still fit in
    // one round.  Returns the number of tiles that run whole.
    *split = 1;
    if (cus <= 0 || tiles < cus) return (int)tiles;
    const int64_t tail = tiles % cus;
    if (tail == 0) return (int)tiles;
    int sp = 1;
    while (tail * sp * 2 <= cus && tail * sp * 2 <= kTailUnitsMax && kt % (sp * 2) == 0 &&
           kt / (sp * 2) >= 4)
        sp *= 2;
    if (sp == 1) return (int)tiles;
    *split = sp;
    return (int)(tiles - tail);
}

int launch_gemm(int cfg, int n, const int8_t *a, const int8_t *b, int8_t *y,
                int64_t m_pad, int64_t n_pad, int64_t k_pad,
                int64_t a_plane, int64_t b_plane, int64_t y_plane,
                int64_t a_row, int64_t a_kstep, int64_t b_row, int64_t b_kstep, int64_t y_pitch,
                int8_t *partial, const EpiConsts &c, hipStream_t s) {
    const TileShape ts = tile_shape(cfg);
    GemmArgs g{a, b, y, a_plane, b_plane, y_plane, a_row, a_kstep, b_row, b_kstep, y_pitch,
               (int32_t)(k_pad / ts.bk), (int32_t)(m_pad / ts.bm), (int32_t)(n_pad / ts.bn),
               0, 1, partial};
    const int64_t tiles = (int64_t)n * g.tiles_m * g.tiles_n;
    if (tiles == 0) return RNS_OK;
    if (tiles > 0x7fffffff || m_pad > 0x7fffffff || n_pad > 0x7fffffff) return RNS_E_ARG;
    int64_t grid = tiles;
    g.tiles = (int32_t)tiles;
    g.full_tiles = (int32_t)tiles;
    const int cus = device_cus();
    if (cfg == kTileBig && partial) {
        int sp = 1;
        g.full_tiles = tail_split(tiles, g.kt, cus, &sp);
        g.split = sp;
        grid = g.full_tiles + (tiles - g.full_tiles) * sp;
        if (grid - g.full_tiles > kTailUnitsMax || (sp > 1 && g.kt % sp)) return RNS_E_ARG;
    }
    // One persistent workgroup per compute unit once there is more than a
    // round of tiles (its per-lane load offsets are 32-bit); a single round
    // runs as before, one tile per workgroup.
    const bool persistent = cfg == kTileBig && cus >= 8 && cus % 8 == 0 && tiles > cus &&
                            256 * a_row < (int64_t)1 << 32 && 256 * b_row < (int64_t)1 << 32;
    switch (cfg) {
        case kTileBig:
            if (persistent)
                hipLaunchKernelGGL((gemm_ps_kernel<4>), dim3((unsigned)cus), dim3(512), 0, s, g, c);
            else
                hipLaunchKernelGGL((gemm_pp_kernel<4>), dim3((unsigned)grid), dim3(512), 0, s, g, c);
            if (g.split > 1) {
                if (hipGetLastError() != hipSuccess) return RNS_E_HIP;
                hipLaunchKernelGGL((gemm_tail4_kernel<8>), dim3((unsigned)(4 * (tiles - g.full_tiles))), dim3(512),
                                   0, s, g, c);
            }
            break;
        case kTileSmall:
            hipLaunchKernelGGL((gemm_kernel<64, 64, 64, 2, 2>), dim3((unsigned)grid), dim3(256), 0, s, g, c);
            break;
        default:
            hipLaunchKernelGGL((gemm_kernel<128, 32, 64, 4, 1>), dim3((unsigned)grid), dim3(256), 0, s, g, c);
            break;
    }
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

}  // namespace rns
