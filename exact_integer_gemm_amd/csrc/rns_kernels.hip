// gfx950 kernels of the exact residue GEMM.
//
//   K1 split   : int64-limb operands -> balanced int8 residue planes, one per
//                prime (enclosure-gemm, "Method": the residue split).
//   K2 gemm    : one INT8 MFMA product per prime with int32 accumulation and a
//                fused reduction mod q (exact-solve, "Method": one INT8 GEMM per
//                prime, batched; exact for K <= 2^17).
//   K3 garner  : balanced Garner mixed-radix digits -> signed int64 limbs
//                (exact-solve, "Method"; enclosure-gemm, "Method").
//
// Every reduction mod q is one exact rounding step: t - q * round(t / q) is
// the balanced residue of t for odd q.  round(t / q) is formed from fl(1/q) by
// a fused multiply-add with 1.5 * 2^52 (binary64, any int32 t: the relative
// error 2^-53 moves t/q by less than 2^-22, while t/q stays at least 1/(2q)
// from every half-integer) or with 1.5 * 2^23 (binary32, |t| < 2^22), which
// leaves the rounded quotient in the low bits of the result.  q = 2 is
// handled separately (the low bit).
#include <hip/hip_runtime.h>

#include "rns_internal.h"

namespace rns {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// The residue split reduces values |t| < 2^22, for which binary32 suffices:
// fl(1/q) moves t/q by less than 1/(4q), and adding 1.5 * 2^23 in the fused
// multiply-add leaves 0x400000 + round(t/q) in the low 24 bits of the result,
// which __mul24 reads as a signed 24-bit value.  The result is t - q *
// round(t/q) - q * 2^22, exact in its low byte (q * 2^22 = 0 mod 256).
__device__ __forceinline__ int reduce_low_byte_f32(int t, int q, float inv) {
    return __mul24(__float_as_int(__builtin_fmaf((float)t, inv, kRoundMagic32)), -q) + t;
}

// round(t / q) as a 32-bit integer, for |t| < 2^31 and odd q (exact).
__device__ __forceinline__ int round_div(int t, double inv) {
    const double g = __builtin_fma((double)t, inv, kRoundMagic);
    return (int)(uint32_t)__double_as_longlong(g);
}

// t - q * round(t / q): the balanced residue of t, exact for |t| < 2^23 and odd q.
__device__ __forceinline__ int reduce_exact(int t, int q, double inv) {
    return __mul24(round_div(t, inv), -q) + t;
}

// The same expression for any |t| < 2^31: the 24-bit product wraps, but
// only mod 2^24, so the low byte (the int8 residue that is stored) is exact.
__device__ __forceinline__ int reduce_low_byte(int t, int q, double inv) {
    return __mul24(round_div(t, inv), -q) + t;
}

__device__ __forceinline__ uint32_t pack4(int b0, int b1, int b2, int b3) {
    // low bytes of four ints -> one word (byte 0 = b0)
    uint32_t lo = __builtin_amdgcn_perm((uint32_t)b1, (uint32_t)b0, 0x0c0c0400u);
    uint32_t hi = __builtin_amdgcn_perm((uint32_t)b3, (uint32_t)b2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// ============================================================================
// K1: residue split
// ============================================================================
// One thread handles a run of 16 consecutive k of one plane row (a row of A,
// or a column of B), so each prime's 16 residues leave as one 16-byte store
// into the K-blocked plane.
constexpr int kSplitThreads = 256;
constexpr int kRun = 16;

struct SplitArgs {
    SplitOperand op[2];
    int64_t tasks[2];      // r_pad * (k_pad / 16) per operand
    int32_t blocks0;       // blocks that serve operand 0
    uint32_t flag_bit[2];  // RNS_FLAG_* recorded for an out-of-bound entry of each operand
    uint32_t *status;      // [2 + gridDim.x] words
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

template <int L>
__device__ void split_run(const SplitOperand &op, const SplitConsts &c, const int32_t *h,
                          int64_t task, uint32_t &flag) {
    // 64 consecutive tasks (one wave) cover one K block (64 k) of 16 plane
    // rows: lane / 4 picks the row, lane % 4 the run of 16 k.  The wave's
    // stores then fill 1 KB of the K-blocked plane contiguously.
    const int64_t lane = task & 63, wv = task >> 6;
    const int64_t groups = op.r_pad / 16;
    const int64_t kb = wv / groups, rg = wv - kb * groups;
    const int64_t r = rg * 16 + (lane >> 2);
    const int64_t k0 = kb * kKBlock + (lane & 3) * kRun;
    const bool row_ok = r < op.rows;

    // U = x + 2^(64L-1) as 2L little-endian 32-bit words, per element
    uint32_t u[kRun][2 * L];
    uint32_t lowbit = 0;   // bit e: x_e is odd (residue mod 2)
#pragma unroll
    for (int e = 0; e < kRun; e++) {
        const int64_t k = k0 + e;
        uint64_t x[L];
        const bool ok = row_ok && k < op.k;
        const int64_t idx = op.transposed ? (k * op.rows + r) : (r * op.k + k);
#pragma unroll
        for (int l = 0; l < L; l++) x[l] = ok ? (uint64_t)op.x[idx * L + l] : 0ull;
        if (op.bits >= 0 && !within_bound<L>(x, op.bits)) flag = 1;
        lowbit |= (uint32_t)(x[0] & 1u) << e;
#pragma unroll
        for (int l = 0; l < L; l++) {
            uint64_t v = x[l] ^ (l == L - 1 ? (1ull << 63) : 0ull);
            u[e][2 * l] = (uint32_t)v;
            u[e][2 * l + 1] = (uint32_t)(v >> 32);
        }
    }

    int8_t *dst = op.planes + kb * (op.r_pad * kKBlock) + r * kKBlock + (lane & 3) * kRun;
    const int64_t plane = op.r_pad * op.k_pad;
    for (int p = 0; p < c.n; p++) {
        const int q = c.q[p];
        uint32_t word[4];
        if (q == 2) {
#pragma unroll
            for (int w = 0; w < 4; w++) {
                uint32_t b = (lowbit >> (4 * w)) & 0xFu;
                // spread 4 bits into the low bit of 4 bytes
                word[w] = (b & 1u) | ((b & 2u) << 7) | ((b & 4u) << 14) | ((b & 8u) << 21);
            }
        } else {
            const float inv = c.inv[p];
            const int hp = h[p];
            int res[kRun];
#pragma unroll
            for (int e = 0; e < kRun; e++) {
                uint32_t t = (uint32_t)(-hp);
#pragma unroll
                for (int w = 0; w < 2 * L; w++)
                    t = __builtin_amdgcn_udot4(u[e][w], c.w[p][w], t, false);
                res[e] = reduce_low_byte_f32((int)t, q, inv);
            }
#pragma unroll
            for (int w = 0; w < 4; w++)
                word[w] = pack4(res[4 * w], res[4 * w + 1], res[4 * w + 2], res[4 * w + 3]);
        }
        v4u out = {word[0], word[1], word[2], word[3]};
        *(v4u *)(dst + p * plane) = out;
    }
}

__global__ __launch_bounds__(kSplitThreads) void split_kernel(SplitArgs args, SplitConsts c) {
    const int which = (int)blockIdx.x < args.blocks0 ? 0 : 1;
    const int64_t block = which == 0 ? blockIdx.x : blockIdx.x - args.blocks0;
    const int64_t task = block * kSplitThreads + threadIdx.x;
    const SplitOperand &op = args.op[which];
    const int32_t *h = which == 0 ? c.h_a : c.h_b;
    uint32_t flag = 0;
    if (task < args.tasks[which]) {
        switch (op.limbs) {
            case 1: split_run<1>(op, c, h, task, flag); break;
            case 2: split_run<2>(op, c, h, task, flag); break;
            case 3: split_run<3>(op, c, h, task, flag); break;
            default: split_run<4>(op, c, h, task, flag); break;
        }
    }
    // one status word per block, written unconditionally (no clearing pass);
    // block 0 also writes the header: the block count and its check word
    const bool any = __syncthreads_or(flag != 0);
    if (threadIdx.x == 0) {
        args.status[kStatusHeader + blockIdx.x] =
            any ? args.flag_bit[which] : 0u;
        if (blockIdx.x == 0) {
            args.status[0] = gridDim.x;
            args.status[1] = gridDim.x ^ kStatusCheck;
        }
    }
}

int64_t split_status_slots(const SplitOperand *a, const SplitOperand *b) {
    int64_t ta = a ? a->r_pad * (a->k_pad / kRun) : 0;
    int64_t tb = b->r_pad * (b->k_pad / kRun);
    return kStatusHeader + (ta + kSplitThreads - 1) / kSplitThreads +
           (tb + kSplitThreads - 1) / kSplitThreads;
}

int launch_split(const SplitOperand *a, const SplitOperand *b, const SplitConsts &c,
                 uint32_t *status, int64_t status_slots, hipStream_t s) {
    SplitArgs args{};
    // operand 0 is A when present, else B alone
    const SplitOperand *ops[2] = {a ? a : b, a ? b : nullptr};
    int64_t blocks[2] = {0, 0};
    for (int i = 0; i < 2; i++) {
        if (!ops[i]) continue;
        args.op[i] = *ops[i];
        args.tasks[i] = ops[i]->r_pad * (ops[i]->k_pad / kRun);
        blocks[i] = (args.tasks[i] + kSplitThreads - 1) / kSplitThreads;
    }
    const int64_t grid = blocks[0] + blocks[1];
    if (grid <= 0) return RNS_OK;
    if (grid + kStatusHeader > status_slots || grid > 0x7fffffff) return RNS_E_ARG;
    args.blocks0 = (int32_t)blocks[0];
    args.flag_bit[0] = a ? RNS_FLAG_A_RANGE : RNS_FLAG_B_RANGE;
    args.flag_bit[1] = RNS_FLAG_B_RANGE;
    args.status = status;
    SplitConsts cc = c;
    if (!a) {
        // operand 0 is B: its offset constant lives in h_a's place
        for (int p = 0; p < kMaxPrimes; p++) cc.h_a[p] = c.h_b[p];
    }
    hipLaunchKernelGGL(split_kernel, dim3((unsigned)grid), dim3(kSplitThreads), 0, s, args, cc);
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

// ============================================================================
// repack of caller-given residue planes into the padded tile layout
// ============================================================================
__global__ void repack_kernel(const int8_t *src, int64_t n, int64_t M, int64_t K,
                              int8_t *dst, int64_t m_pad, int64_t k_pad) {
    const int64_t total = n * m_pad * k_pad;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = i / (m_pad * k_pad);
        const int64_t rem = i - p * m_pad * k_pad;
        const int64_t m = rem / k_pad, k = rem - m * k_pad;
        dst[p * m_pad * k_pad + (k / kKBlock) * (m_pad * kKBlock) + m * kKBlock + k % kKBlock] =
            (m < M && k < K) ? src[(p * M + m) * K + k] : (int8_t)0;
    }
}

int launch_repack_residues(const int8_t *src, int64_t n, int64_t M, int64_t K,
                           int8_t *dst, int64_t m_pad, int64_t k_pad, hipStream_t s) {
    const int64_t total = n * m_pad * k_pad;
    if (total == 0) return RNS_OK;
    int64_t grid = (total + 255) / 256;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(repack_kernel, dim3((unsigned)grid), dim3(256), 0, s, src, n, M, K, dst, m_pad,
                       k_pad);
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

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
    constexpr int OUT_PITCH = BN + 16;             // bytes per LDS row of the output tile
    static_assert(S >= 2 && S <= 4 && S * STAGE * 16 <= 160 * 1024, "LDS ring");
    static_assert(BM * OUT_PITCH <= S * STAGE * 16, "output staging fits the ring");

    __shared__ v4i lds[S][STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int group = wave >> 2;
    const int wm = wave & 1, wn = wave >> 1;       // 2 x 4 waves over the tile
    const int half = lane >> 5, l32 = lane & 31;

    const int G = gridDim.x;
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int tile = xcd * (G >> 3) + min(xcd, G & 7) + idx;
    const int per_prime = g.tiles_m * g.tiles_n;
    const int p = tile / per_prime;
    const int t = tile - p * per_prime;
    const int tm = t / g.tiles_n, tn = t - tm * g.tiles_n;
    const int8_t *Ap = g.a + p * g.a_plane + (int64_t)(tm * BM) * g.a_row;
    const int8_t *Bp = g.b + p * g.b_plane + (int64_t)(tn * BN) * g.b_row;

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
    const int KT = g.kt;
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

    // epilogue: residues mod q as int8, staged through LDS (row pitch
    // OUT_PITCH bytes) so that the tile leaves in whole 16-byte row chunks
    __builtin_amdgcn_s_waitcnt(0x0f70);             // vmcnt(0): no load may still target LDS
    __syncthreads();
    int8_t *out = (int8_t *)&lds[0][0];
    const int q = ec.q[p];
    const double inv = ec.inv[p];
    if (q == 2) {
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++)
#pragma unroll
                for (int gq = 0; gq < 4; gq++) {
                    const int row = wm * 128 + i * 32 + l32;
                    const int col = wn * 64 + j * 32 + 8 * gq + 4 * half;
                    const v16i &a = acc[i][j];
                    *(uint32_t *)(out + row * OUT_PITCH + col) =
                        pack4(a[4 * gq] & 1, a[4 * gq + 1] & 1, a[4 * gq + 2] & 1, a[4 * gq + 3] & 1);
                }
    } else {
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++)
#pragma unroll
                for (int gq = 0; gq < 4; gq++) {
                    const int row = wm * 128 + i * 32 + l32;
                    const int col = wn * 64 + j * 32 + 8 * gq + 4 * half;
                    const v16i &a = acc[i][j];
                    *(uint32_t *)(out + row * OUT_PITCH + col) =
                        pack4(reduce_low_byte(a[4 * gq], q, inv), reduce_low_byte(a[4 * gq + 1], q, inv),
                              reduce_low_byte(a[4 * gq + 2], q, inv), reduce_low_byte(a[4 * gq + 3], q, inv));
                }
    }
    __syncthreads();
    int8_t *Yp = g.y + p * g.y_plane + (int64_t)(tm * BM) * g.y_pitch + tn * BN;
    // 256 rows x 256 bytes: 16 lanes per row, 32 rows per pass of 512 threads
#pragma unroll
    for (int pass = 0; pass < BM / 32; pass++) {
        const int row = pass * 32 + (tid >> 4);
        const int c = (tid & 15) * 16;
        *(v4i *)(Yp + (int64_t)row * g.y_pitch + c) = *(const v4i *)(out + row * OUT_PITCH + c);
    }
}

int launch_gemm(int cfg, int n, const int8_t *a, const int8_t *b, int8_t *y,
                int64_t m_pad, int64_t n_pad, int64_t k_pad,
                int64_t a_plane, int64_t b_plane, int64_t y_plane,
                int64_t a_row, int64_t a_kstep, int64_t b_row, int64_t b_kstep, int64_t y_pitch,
                const EpiConsts &c, hipStream_t s) {
    const TileShape ts = tile_shape(cfg);
    GemmArgs g{a, b, y, a_plane, b_plane, y_plane, a_row, a_kstep, b_row, b_kstep, y_pitch,
               (int32_t)(k_pad / ts.bk), (int32_t)(m_pad / ts.bm), (int32_t)(n_pad / ts.bn)};
    const int64_t grid = (int64_t)n * g.tiles_m * g.tiles_n;
    if (grid == 0) return RNS_OK;
    if (grid > 0x7fffffff || m_pad > 0x7fffffff || n_pad > 0x7fffffff) return RNS_E_ARG;
    switch (cfg) {
        case kTileBig:
            hipLaunchKernelGGL((gemm_pp_kernel<4>), dim3((unsigned)grid), dim3(512), 0, s, g, c);
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

// ============================================================================
// K3: Garner reconstruction
// ============================================================================
// One thread per output entry.  NB (a multiple of 8, >= n) bounds the fully
// unrolled digit loops, so every digit and partial sum lives in registers.
// Slots k >= n are padding that the tables make inert (q = 1, all constants
// zero), so the loops carry no guards.  Slot 0 holds the prime 2 when the
// plan has it.
//
// acc[k] starts at y_k * Q_k^-1 and loses v_j * (Q_j Q_k^-1 mod q_k) for every
// earlier digit j; |acc| <= 54 * 125^2 < 2^20 keeps the rounding step exact.
// The value X = sum_k v_k Q_k is gathered in 16-bit chunks t[c] (signed,
// |t[c]| < 54 * 125 * 2^16 < 2^29) and carried into limbs at the end.
template <int NB>
__global__ __launch_bounds__(256) void garner_kernel(GarnerConsts gc, const int8_t *__restrict__ y,
                                                     int64_t y_plane, int64_t y_pitch, int64_t M,
                                                     int64_t N, int64_t *__restrict__ C, int c_limbs) {
    constexpr int CB = garner_chunks(NB - 1);   // chunks of the widest Q_k
    const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (e >= M * N) return;
    const int64_t i = e / N, j = e - i * N;
    const int8_t *yp = y + i * y_pitch + j;

    int acc[NB];
#pragma unroll
    for (int k = 0; k < NB; k++) acc[k] = (int)yp[gc.plane[k] * y_plane] * (int)gc.tri[tri_index(k, k)];
    int t[CB + 1];
#pragma unroll
    for (int c = 0; c <= CB; c++) t[c] = 0;

#pragma unroll
    for (int k = 0; k < NB; k++) {
        int v;
        if (k == 0 && gc.q[0] == 2) v = acc[0] & 1;
        else v = reduce_exact(acc[k], gc.q[k], gc.inv[k]);
#pragma unroll
        for (int kk = k + 1; kk < NB; kk++) acc[kk] -= __mul24(v, (int)gc.tri[tri_index(k, kk)]);
#pragma unroll
        for (int c = 0; c < garner_chunks(k); c++)
            t[c] += __mul24(v, (int)gc.q16[garner_chunk_offset(k) + c]);
    }

    // carry the signed chunks into 16-bit digits; the final carry is the sign
    int carry = 0;
    uint32_t words[2 * RNS_MAX_OUT_LIMBS];
#pragma unroll
    for (int w = 0; w < 2 * RNS_MAX_OUT_LIMBS; w++) {
        uint32_t half16[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int c = 2 * w + h;
            const int s = (c <= CB ? t[c] : 0) + carry;
            half16[h] = (uint32_t)s & 0xffffu;
            carry = s >> 16;
        }
        words[w] = half16[0] | (half16[1] << 16);
    }
    int64_t *out = C + e * c_limbs;
#pragma unroll
    for (int l = 0; l < RNS_MAX_OUT_LIMBS; l++)
        if (l < c_limbs) out[l] = (int64_t)(((uint64_t)words[2 * l + 1] << 32) | words[2 * l]);
}

int launch_garner(const GarnerConsts &g, const int8_t *y, int64_t y_plane, int64_t y_pitch,
                  int64_t M, int64_t N, int64_t *C, int32_t c_limbs, hipStream_t s) {
    const int64_t total = M * N;
    if (total == 0) return RNS_OK;
    const int64_t grid = (total + 255) / 256;
    if (grid > 0x7fffffff) return RNS_E_ARG;
    const int nb = (g.n + 7) / 8 * 8;
    dim3 gd((unsigned)grid), bd(256);
    switch (nb) {
        case 8: hipLaunchKernelGGL(garner_kernel<8>, gd, bd, 0, s, g, y, y_plane, y_pitch, M, N, C, c_limbs); break;
        case 16: hipLaunchKernelGGL(garner_kernel<16>, gd, bd, 0, s, g, y, y_plane, y_pitch, M, N, C, c_limbs); break;
        case 24: hipLaunchKernelGGL(garner_kernel<24>, gd, bd, 0, s, g, y, y_plane, y_pitch, M, N, C, c_limbs); break;
        case 32: hipLaunchKernelGGL(garner_kernel<32>, gd, bd, 0, s, g, y, y_plane, y_pitch, M, N, C, c_limbs); break;
        case 40: hipLaunchKernelGGL(garner_kernel<40>, gd, bd, 0, s, g, y, y_plane, y_pitch, M, N, C, c_limbs); break;
        case 48: hipLaunchKernelGGL(garner_kernel<48>, gd, bd, 0, s, g, y, y_plane, y_pitch, M, N, C, c_limbs); break;
        default: hipLaunchKernelGGL(garner_kernel<56>, gd, bd, 0, s, g, y, y_plane, y_pitch, M, N, C, c_limbs); break;
    }
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

// ============================================================================
// zero fill of C (K = 0)
// ============================================================================
__global__ void zero_kernel(int64_t *C, int64_t count) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        C[i] = 0;
}

int launch_zero(int64_t *C, int64_t count, hipStream_t s) {
    if (count == 0) return RNS_OK;
    int64_t grid = (count + 255) / 256;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)grid), dim3(256), 0, s, C, count);
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

}  // namespace rns
