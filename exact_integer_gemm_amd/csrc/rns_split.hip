// K1 of the exact residue GEMM on gfx950: int64-limb operands -> balanced
// int8 residue planes, one per prime (enclosure-gemm, "Method": the residue
// split), and the repack of caller-given residue planes.
#include "rns_device.h"

namespace rns {

// ============================================================================
// K1: residue split
// ============================================================================
// One thread handles a run of 16 consecutive k of one plane row (a row of A,
// or a column of B), so each prime's 16 residues leave as one 16-byte store
// into the K-blocked plane.
constexpr int kSplitThreads = 256;
constexpr int kRun = 16;

// Small problems (a few hundred blocks or fewer) would leave most compute
// units idle while each thread loops over every prime; their grid repeats
// the task blocks for groups of primes instead (the entries are loaded once
// per group).
constexpr int64_t kSplitTargetBlocks = 1024;

struct SplitArgs {
    SplitOperand op[2];
    int64_t tasks[2];      // r_pad * (k_pad / 16) per operand
    int32_t blocks0;       // task blocks that serve operand 0
    int32_t task_blocks;   // task blocks of both operands
    int32_t prime_groups;  // the grid is prime_groups x task_blocks
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

template <int L, bool FP>
__device__ void split_run(const SplitOperand &op, const SplitConsts &c, const int32_t *h,
                          int64_t task, int p_begin, int p_end, uint32_t &flag) {
    // 64 consecutive tasks (one wave) cover one K block (64 k) of 16 plane
    // rows: lane / 4 picks the row, lane % 4 the run of 16 k.  The wave's
    // stores then fill 1 KB of the K-blocked plane contiguously.
    const int64_t lane = task & 63, wv = task >> 6;
    const int64_t groups = op.r_pad / 16;
    const int64_t kb = wv / groups, rg = wv - kb * groups;
    const int64_t r = rg * 16 + (lane >> 2);
    const int64_t k0 = kb * kKBlock + (lane & 3) * kRun;
    const bool row_ok = r < op.rows;

    // All 16 L limbs are requested before any is used: a padding entry reads
    // entry 0 (the operand is not empty when there are tasks) and is then
    // replaced by zero, so no load sits behind a branch and a wait.
    // (binary64 operands: one word per entry, scaled into L limbs here)
    constexpr int W = FP ? 1 : L;
    uint64_t xs[kRun][W];
#pragma unroll
    for (int e = 0; e < kRun; e++) {
        const int64_t k = k0 + e;
        const bool ok = row_ok && k < op.k;
        const int64_t idx = !ok ? 0 : op.transposed ? (k * op.rows + r) : (r * op.k + k);
#pragma unroll
        for (int l = 0; l < W; l++) xs[e][l] = (uint64_t)op.x[idx * W + l];
    }
    // U = x + 2^(64L-1) as 2L little-endian 32-bit words, per element
    uint32_t u[kRun][2 * L];
    uint32_t lowbit = 0;   // bit e: x_e is odd (residue mod 2)
#pragma unroll
    for (int e = 0; e < kRun; e++) {
        const int64_t k = k0 + e;
        const bool ok = row_ok && k < op.k;
        uint64_t x[L];
        if constexpr (FP) {
            fp64_floor_scaled<L>(ok ? xs[e][0] : 0ull, op.scale, x);
        } else {
#pragma unroll
            for (int l = 0; l < L; l++) x[l] = ok ? xs[e][l] : 0ull;
        }
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
    for (int p = p_begin; p < p_end; p++) {
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

// FP: both operands are binary64 (one kernel per operand kind keeps the
// register allocation of each path separate)
template <bool FP>
__global__ __launch_bounds__(kSplitThreads) void split_kernel(SplitArgs args, SplitConsts c) {
    const int tb = (int)blockIdx.x % args.task_blocks, pg = (int)blockIdx.x / args.task_blocks;
    const int p_begin = pg * c.n / args.prime_groups, p_end = (pg + 1) * c.n / args.prime_groups;
    const int which = tb < args.blocks0 ? 0 : 1;
    const int64_t block = which == 0 ? tb : tb - args.blocks0;
    const int64_t task = block * kSplitThreads + threadIdx.x;
    const SplitOperand &op = args.op[which];
    const int32_t *h = which == 0 ? c.h_a : c.h_b;
    uint32_t flag = 0;
    if (task < args.tasks[which]) {
        switch (op.limbs) {
            case 1: split_run<1, FP>(op, c, h, task, p_begin, p_end, flag); break;
            case 2: split_run<2, FP>(op, c, h, task, p_begin, p_end, flag); break;
            case 3: split_run<3, FP>(op, c, h, task, p_begin, p_end, flag); break;
            default: split_run<4, FP>(op, c, h, task, p_begin, p_end, flag); break;
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

static int split_prime_groups(int64_t task_blocks, int n) {
    if (task_blocks <= 0 || task_blocks >= kSplitTargetBlocks / 2) return 1;
    const int64_t g = (kSplitTargetBlocks + task_blocks - 1) / task_blocks;
    return (int)(g < n ? g : n);
}

int64_t split_status_slots(const SplitOperand *a, const SplitOperand *b, int n) {
    int64_t ta = a ? a->r_pad * (a->k_pad / kRun) : 0;
    int64_t tb = b->r_pad * (b->k_pad / kRun);
    const int64_t blocks = (ta + kSplitThreads - 1) / kSplitThreads + (tb + kSplitThreads - 1) / kSplitThreads;
    return kStatusHeader + blocks * split_prime_groups(blocks, n);
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
    const int64_t task_blocks = blocks[0] + blocks[1];
    if (task_blocks <= 0) return RNS_OK;
    if (c.n < 1 || c.n > kMaxPrimes) return RNS_E_ARG;
    const int groups = split_prime_groups(task_blocks, c.n);
    const int64_t grid = task_blocks * groups;
    if (grid + kStatusHeader > status_slots || grid > 0x7fffffff) return RNS_E_ARG;
    args.blocks0 = (int32_t)blocks[0];
    args.task_blocks = (int32_t)task_blocks;
    args.prime_groups = groups;
    args.flag_bit[0] = a ? RNS_FLAG_A_RANGE : RNS_FLAG_B_RANGE;
    args.flag_bit[1] = RNS_FLAG_B_RANGE;
    args.status = status;
    SplitConsts cc = c;
    if (!a) {
        // operand 0 is B: its offset constant lives in h_a's place
        for (int p = 0; p < kMaxPrimes; p++) cc.h_a[p] = c.h_b[p];
    }
    const bool fp = ops[0]->fp64 != 0;
    if (ops[1] && (ops[1]->fp64 != 0) != fp) return RNS_E_ARG;
    if (fp)
        hipLaunchKernelGGL(split_kernel<true>, dim3((unsigned)grid), dim3(kSplitThreads), 0, s, args, cc);
    else
        hipLaunchKernelGGL(split_kernel<false>, dim3((unsigned)grid), dim3(kSplitThreads), 0, s, args, cc);
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

}  // namespace rns
