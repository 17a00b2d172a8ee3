// The batched-residue product for skinny right-hand sides, fused with the
// residue split of that right-hand side (exact-solve, "Method": each lift
// step applies every prime's inverse plane to the residual as one batched
// INT8 product; the CRT of the wide digit follows).
//
// Y_j = (A_j @ (r mod q_j)) mod q_j, balanced, for every prime j, where A_j
// is the caller's int8 plane j ([n][M][K], row-major, read as an integer
// matrix mod q_j) and r is the int64 right-hand side [K][N] with N <= 16.
// The product is memory-bound (K bytes of A per 2*16*K operations), so each
// plane is streamed from HBM exactly once, straight into the operand
// registers of v_mfma_i32_16x16x64_i8, while the small right-hand side is
// reduced mod q_j into small int8 planes that the product kernel's
// workgroups copy into LDS.
//
// Two kernels.  skinny_split_kernel reduces r mod every prime into int8
// planes laid out as the products' MFMA operand wants them: rr[j][kc][g][c]
// holds the 16 residues of r[64 kc + 16 g + t][c], t < 16 (zero past K and
// past N), for the KC = ceil(K / 64) chunks.  skinny_kernel: workgroup
// (j, b) owns rows 64 b .. 64 b + 63 of plane j, four waves of 16 rows (one
// MFMA block each).  The product is latency-bound at this size, so every
// load of a wave is issued at once: its row chunks (up to kSkRound of them
// per round) and its share of rr[j], which the workgroup copies into LDS;
// small LDS and register footprints keep several workgroups resident per
// compute unit, which overlaps their memory latencies.
//
// Operand k-order: lane l of an MFMA operand holds row (or column) l % 16 and
// the 16 bytes k = 64 kc + 16 (l / 16) + t, t < 16, of the 64-wide chunk kc
// -- the same k for both operands, so the dot products pair every A byte
// with the r residue of the same k whatever order the instruction adds them
// in.  The accumulators hold entry (4 (l / 16) + e, l % 16) in element e of
// lane l.
#include "rns_device.h"

namespace rns {

constexpr int kSkRows = 64;           // rows of a plane per workgroup
constexpr int kSkWaves = 4;           // 16 rows per wave
constexpr int kSkRound = 16;          // 64-wide K chunks per wave loaded at once

// The balanced residue of a signed 64-bit value x mod q (q <= 256), exact.
// With U = x + 2^63 (the top bit flipped; unsigned) and its bytes u_b,
// x = sum_b u_b 256^b - 2^63, so x = t (mod q) for
// t = sum_b u_b (256^b mod q) - (2^63 mod q), two four-byte dot products
// against the packed constants wl (bytes 0..3) and wh (bytes 4..7);
// 0 <= t + h < 8 * 255 * 256 < 2^21, so one binary32 rounding step balances it.
struct ResidueConsts {
    uint32_t wl, wh;                  // packed 256^b mod q, b = 0..3 and 4..7
    int32_t h;                        // 2^63 mod q
    float inv;                        // fl(1/q)
};
struct ResidueTables {
    ResidueConsts c[kMaxPrimes];
};
__device__ __forceinline__ int residue_i64(int64_t x, int q, const ResidueConsts &c) {
    const uint32_t lo = (uint32_t)x, hi = (uint32_t)((uint64_t)x >> 32) ^ 0x80000000u;
    const int t = (int)__builtin_amdgcn_udot4(hi, c.wh, __builtin_amdgcn_udot4(lo, c.wl, 0u, false), false) - c.h;
    const int k = __float_as_int(__builtin_fmaf((float)t, c.inv, kRoundMagic32)) - 0x4b400000;
    return __mul24(k, -q) + t;
}

struct SkinnyArgs {
    const int8_t *a;                  // planes [n][M][K]
    const int64_t *r;                 // right-hand side [K][N]
    int8_t *rr;                       // residue planes of r [n][KC][4][16][16]
    int8_t *y;                        // product planes [n][.][y_pitch]
    uint32_t *status;                 // the workspace's status header
    int64_t y_plane, y_pitch;
    int32_t n, M, N, K, KC;
    int32_t row_blocks;
};

// thread (quad, column, prime): four consecutive k of one column, one 32-bit
// word of the residue plane
__global__ __launch_bounds__(256) void skinny_split_kernel(SkinnyArgs g, EpiConsts ec, ResidueTables rt) {
    const int nq = g.KC * 16;                         // quads per column
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_prime = (int64_t)nq * 16;
    const int j = (int)(id / per_prime);
    const int rem = (int)(id - (int64_t)j * per_prime);
    const int quad = rem >> 4, c = rem & 15;
    if (id == 0) {
        // no bound is checked on this path: a header of zero blocks (no flags)
        g.status[0] = 0u;
        g.status[1] = kStatusCheck;
    }
    if (j >= g.n) return;
    const int q = ec.q[j];
    const ResidueConsts rc = rt.c[j];
    const int k0 = 4 * quad;
    const int cc = min(c, g.N - 1);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int k = k0 + i;
        const int64_t x = g.r[(uint32_t)(min(k, g.K - 1) * g.N + cc)];
        const int res = residue_i64(x, q, rc);
        word |= (uint32_t)((k < g.K && c < g.N) ? (res & 0xff) : 0) << (8 * i);
    }
    const int kc = k0 >> 6, grp = (k0 >> 4) & 3, t = k0 & 15;
    uint32_t *dst = (uint32_t *)(g.rr + (int64_t)j * g.KC * 1024);
    dst[(((kc * 4 + grp) * 16 + c) * 16 + t) >> 2] = word;
}

// KCP: 64-wide chunks of K, padded (a multiple of kSkRound, or less than it)
template <int KCP>
__global__ __launch_bounds__(64 * kSkWaves) void skinny_kernel(SkinnyArgs g, EpiConsts ec) {
    constexpr int R = KCP < kSkRound ? KCP : kSkRound;         // chunks per round
    static_assert(KCP % R == 0, "whole rounds");
    constexpr int kPieces = KCP * 64 / (64 * kSkWaves);       // 16-byte pieces of rr per thread
    static_assert(kPieces * 64 * kSkWaves == KCP * 64, "rr pieces spread evenly");
    __shared__ v4i rl[KCP][4][16];                             // residues of r mod q_j: [chunk][lane group][column]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = blockIdx.x / g.row_blocks, rb = blockIdx.x - j * g.row_blocks;
    const int q = ec.q[j];
    const double inv = ec.inv[j];
    const int KC = g.KC;                               // chunks holding data (K is a multiple of 16)

    // this lane's A row (clamped into the plane; rows past M are computed and dropped)
    const int row = min(rb * kSkRows + wave * 16 + (lane & 15), g.M - 1);
    const int8_t *pa = g.a + (int64_t)j * g.M * g.K + (int64_t)row * g.K + 16 * (lane >> 4);
    // Loads are unconditional, so that the counter waits stay exact: a chunk
    // past the last re-reads the last, and within the last chunk a lane group
    // past K re-reads the row's last 16 bytes; the zero residues of those k
    // cancel whatever they read.
    auto load = [&](int kc) {
        const int off = min(min(kc, KC - 1) * 64, g.K - 16 - 16 * (lane >> 4));
        return *(const v4i *)(pa + off);
    };

    // rr[j] pieces first (a piece past KC chunks re-reads one of them and is
    // replaced by zero), then the first round of row chunks
    const v4i *src = (const v4i *)(g.rr + (int64_t)j * KC * 1024);
    v4i rv[kPieces];
#pragma unroll
    for (int i = 0; i < kPieces; i++) {
        const int piece = tid + i * 64 * kSkWaves;
        rv[i] = src[piece < KC * 64 ? piece : piece % (KC * 64)];
    }
    v4i abuf[R];
#pragma unroll
    for (int c = 0; c < R; c++) abuf[c] = load(c);
    __builtin_amdgcn_s_waitcnt(0x0f70 | (R & 15) | ((R >> 4) << 14));   // rr pieces in; row chunks may pend
#pragma unroll
    for (int i = 0; i < kPieces; i++) {
        const int piece = tid + i * 64 * kSkWaves;
        (&rl[0][0][0])[piece] = piece < KC * 64 ? rv[i] : v4i{0, 0, 0, 0};
    }
    __syncthreads();

    v4i acc = {0, 0, 0, 0};
#pragma unroll
    for (int r0 = 0; r0 < KCP; r0 += R) {
#pragma unroll
        for (int c = 0; c < R; c++) {
            const v4i bv = rl[r0 + c][lane >> 4][lane & 15];
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(abuf[c], bv, acc, 0, 0, 0);
            if (r0 + R < KCP) abuf[c] = load(r0 + R + c);
        }
    }

    // balanced residues mod q, one byte per entry (q = 2: the low bit)
    const int col = lane & 15;
    if (col < g.N) {
        int8_t *yp = g.y + (int64_t)j * g.y_plane + col;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int rw = rb * kSkRows + wave * 16 + 4 * (lane >> 4) + e;
            if (rw < g.M) {
                const int s = acc[e];
                yp[(int64_t)rw * g.y_pitch] = (int8_t)(q == 2 ? (s & 1) : reduce_low_byte(s, q, inv));
            }
        }
    }
}

int64_t skinny_rr_bytes(int n, int64_t K) { return (int64_t)n * ((K + 63) / 64) * 1024; }

int launch_skinny(int n, const int8_t *a, const int64_t *r, int64_t M, int64_t N, int64_t K, int8_t *rr,
                  int8_t *y, int64_t y_plane, int64_t y_pitch, uint32_t *status, const EpiConsts &c,
                  hipStream_t s) {
    if (n < 1 || n > kMaxPrimes || M < 1 || N < 1 || N > 16 || K < 16 || K % 16 || K > RNS_SKINNY_K_MAX ||
        M > (1 << 24) || (reinterpret_cast<uintptr_t>(a) & 15) || (reinterpret_cast<uintptr_t>(rr) & 15))
        return RNS_E_ARG;
    const int64_t row_blocks = (M + kSkRows - 1) / kSkRows;
    const int64_t grid = row_blocks * n;
    if (grid > 0x7fffffff || (int64_t)n * M * K > ((int64_t)1 << 40)) return RNS_E_ARG;
    const int64_t kc = (K + 63) / 64;
    SkinnyArgs g{a, r, rr, y, status, y_plane, y_pitch, (int32_t)n, (int32_t)M, (int32_t)N, (int32_t)K, (int32_t)kc,
                 (int32_t)row_blocks};
    // per prime: the packed byte weights 256^b mod q, 2^63 mod q and fl(1/q)
    ResidueTables rt;
    for (int jj = 0; jj < n; jj++) {
        const uint32_t q = (uint32_t)c.q[jj];
        uint32_t p = 1, w[2] = {0, 0};
        for (int b = 0; b < 8; b++) {
            w[b >> 2] |= (p % q) << (8 * (b & 3));
            p = (p * 256u) % q;
        }
        rt.c[jj].wl = w[0];
        rt.c[jj].wh = w[1];
        rt.c[jj].h = (int32_t)((((w[1] >> 24) & 0xffu) * 128u) % q);   // 2^63 = 256^7 * 128
        rt.c[jj].inv = 1.0f / (float)q;
    }
    const int64_t split_threads = (int64_t)n * kc * 16 * 16;
    hipLaunchKernelGGL(skinny_split_kernel, dim3((unsigned)((split_threads + 255) / 256)), dim3(256), 0, s, g, c, rt);
    if (hipGetLastError() != hipSuccess) return RNS_E_HIP;
    const dim3 gr((unsigned)grid), bl(64 * kSkWaves);
    if (kc <= 4)
        hipLaunchKernelGGL((skinny_kernel<4>), gr, bl, 0, s, g, c);
    else if (kc <= 8)
        hipLaunchKernelGGL((skinny_kernel<8>), gr, bl, 0, s, g, c);
    else if (kc <= 16)
        hipLaunchKernelGGL((skinny_kernel<16>), gr, bl, 0, s, g, c);
    else if (kc <= 32)
        hipLaunchKernelGGL((skinny_kernel<32>), gr, bl, 0, s, g, c);
    else
        hipLaunchKernelGGL((skinny_kernel<64>), gr, bl, 0, s, g, c);
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

}  // namespace rns
