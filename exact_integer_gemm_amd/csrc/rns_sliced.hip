// Exact integer products beyond the residue capacity by operand slices
// (Ozaki Scheme II paper, §5.1 and §5.2): limb-aligned slices of A and B, one
// exact residue product per pair of slices, and their shifted two's-complement
// sum.
#include "rns_device.h"
#include "../../include/rns_sliced.h"

namespace rns {

// Slice i of every entry, as s + 1 limbs: the lower slices are the raw limbs
// i s .. i s + s - 1 read unsigned (a zero limb on top), the top slice the
// remaining limbs with the entry's sign carried into the limbs above them.
__global__ __launch_bounds__(256) void slice_kernel(const int64_t *__restrict__ X, int64_t count, int L, int s,
                                                    int ns, int64_t *__restrict__ out) {
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < count; e += (int64_t)gridDim.x * 256) {
        const int64_t *x = X + e * L;
        const int64_t sign = x[L - 1] < 0 ? -1 : 0;
        for (int i = 0; i < ns; i++) {
            int64_t *o = out + ((int64_t)i * count + e) * (s + 1);
            for (int t = 0; t <= s; t++) {
                const int l = i * s + t;
                o[t] = (t < s && l < L) ? x[l] : (i == ns - 1 ? sign : 0);
            }
        }
    }
}

// C = sum_{i,j} part_ij 2^(64 (sa i + sb j)), limb by limb with carries;
// every part is sign-extended across the limbs above it.
__global__ __launch_bounds__(256) void sliced_accumulate_kernel(const int64_t *__restrict__ parts, int na, int nb,
                                                                int sa, int sb, int pl, int64_t count,
                                                                int64_t *__restrict__ C, int cl) {
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < count; e += (int64_t)gridDim.x * 256) {
        uint64_t acc[RNS_SLICED_MAX_OUT_LIMBS];
#pragma unroll
        for (int t = 0; t < RNS_SLICED_MAX_OUT_LIMBS; t++) acc[t] = 0;
        for (int i = 0; i < na; i++)
            for (int j = 0; j < nb; j++) {
                const int off = sa * i + sb * j;
                const int64_t *p = parts + ((int64_t)(i * nb + j) * count + e) * pl;
                const uint64_t sign = p[pl - 1] < 0 ? ~0ull : 0ull;
                uint64_t carry = 0;
#pragma unroll
                for (int t = 0; t < RNS_SLICED_MAX_OUT_LIMBS; t++) {
                    if (t < off || t >= cl) continue;
                    const uint64_t add = t - off < pl ? (uint64_t)p[t - off] : sign;
                    const uint64_t s1 = acc[t] + add;
                    const uint64_t c1 = s1 < add ? 1ull : 0ull;
                    const uint64_t s2 = s1 + carry;
                    const uint64_t c2 = s2 < s1 ? 1ull : 0ull;
                    acc[t] = s2;
                    carry = c1 | c2;
                }
            }
        int64_t *c = C + e * cl;
#pragma unroll
        for (int t = 0; t < RNS_SLICED_MAX_OUT_LIMBS; t++)
            if (t < cl) c[t] = (int64_t)acc[t];
    }
}

}  // namespace rns

using namespace rns;

namespace {

int64_t pad256(int64_t x) { return (x + 255) / 256 * 256; }

unsigned grid_of(int64_t count) {
    const int64_t g = (count + 255) / 256;
    return (unsigned)(g < 1 ? 1 : (g > 8192 ? 8192 : g));
}

struct SlicedLayout {
    int64_t a_off, b_off, p_off, g_off, total;
    size_t g_bytes;
};

int sliced_layout(const rns_sliced_plan_t &p, int64_t M, int64_t N, int64_t K, SlicedLayout &L) {
    size_t g = 0;
    const int rc = rns_workspace_size(&p.slice, M, N, K, 0, &g);
    if (rc != RNS_OK) return rc;
    int64_t off = 0;
    L.a_off = off;
    off = pad256(off + (int64_t)p.na * M * K * (p.sa + 1) * 8);
    L.b_off = off;
    off = pad256(off + (int64_t)p.nb * K * N * (p.sb + 1) * 8);
    L.p_off = off;
    off = pad256(off + (int64_t)p.na * p.nb * M * N * p.part_limbs * 8);
    L.g_off = off;
    L.g_bytes = g;
    L.total = off + (int64_t)g;
    return RNS_OK;
}

bool plan_ok(const rns_sliced_plan_t *p) {
    return p && p->a_limbs >= 1 && p->a_limbs <= RNS_SLICED_MAX_IN_LIMBS && p->b_limbs >= 1 &&
           p->b_limbs <= RNS_SLICED_MAX_IN_LIMBS && p->sa >= 1 && p->sb >= 1 && p->sa + p->sb <= 4 &&
           p->na == (p->a_limbs + p->sa - 1) / p->sa && p->nb == (p->b_limbs + p->sb - 1) / p->sb &&
           p->part_limbs >= p->slice.out_limbs_min && p->part_limbs <= RNS_MAX_OUT_LIMBS &&
           p->out_limbs_min >= 1 && p->out_limbs_min <= RNS_SLICED_MAX_OUT_LIMBS;
}

}  // namespace

extern "C" {

int rns_sliced_plan(int64_t K, int32_t a_limbs, int32_t b_limbs, rns_sliced_plan_t *out) {
    if (!out || K < 0 || a_limbs < 1 || a_limbs > RNS_SLICED_MAX_IN_LIMBS || b_limbs < 1 ||
        b_limbs > RNS_SLICED_MAX_IN_LIMBS)
        return RNS_E_ARG;
    if (K > RNS_K_MAX) return RNS_E_K;
    rns_sliced_plan_t p{};
    p.a_limbs = a_limbs;
    p.b_limbs = b_limbs;
    // sa + sb = 4 limbs of range per slice product: 2 * K * 2^256 <= 2^274 fits the 54 primes
    if (a_limbs >= 2 && b_limbs >= 2) {
        p.sa = 2;
        p.sb = 2;
    } else if (a_limbs == 1) {
        p.sa = 1;
        p.sb = b_limbs < 3 ? b_limbs : 3;
    } else {
        p.sb = 1;
        p.sa = a_limbs < 3 ? a_limbs : 3;
    }
    p.na = (a_limbs + p.sa - 1) / p.sa;
    p.nb = (b_limbs + p.sb - 1) / p.sb;
    // lower slices are below 2^(64 s), the top slice at most 2^(64 s - 1) in magnitude
    int rc = rns_plan(K, 64 * p.sa, 64 * p.sb, &p.slice);
    if (rc != RNS_OK) return rc;
    p.part_limbs = p.slice.out_limbs_min;
    // |C| <= K 2^(64 a_limbs - 1) 2^(64 b_limbs - 1), plus a sign bit
    int lg = 0;
    while ((1ll << lg) < (K < 1 ? 1 : K)) lg++;
    const int bits = 64 * (a_limbs + b_limbs) - 2 + lg + 1;
    p.out_limbs_min = (bits + 63) / 64;
    *out = p;
    return RNS_OK;
}

int rns_sliced_workspace_size(const rns_sliced_plan_t *plan, int64_t M, int64_t N, int64_t K, size_t *bytes) {
    if (!plan_ok(plan) || !bytes || M < 0 || N < 0 || K < 0) return RNS_E_ARG;
    if (K > plan->slice.k_max) return RNS_E_K;
    SlicedLayout L;
    const int rc = sliced_layout(*plan, M, N, K, L);
    if (rc != RNS_OK) return rc;
    *bytes = (size_t)L.total;
    return RNS_OK;
}

int rns_gemm_sliced(const rns_sliced_plan_t *plan, int64_t M, int64_t N, int64_t K, const int64_t *A,
                    const int64_t *B, int64_t *C, int32_t c_limbs, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!plan_ok(plan) || M < 0 || N < 0 || K < 0) return RNS_E_ARG;
    if (K > plan->slice.k_max) return RNS_E_K;
    if (c_limbs < plan->out_limbs_min || c_limbs > RNS_SLICED_MAX_OUT_LIMBS) return RNS_E_OUT_LIMBS;
    if (M == 0 || N == 0) return RNS_OK;
    if (!C) return RNS_E_ARG;
    if (K == 0) return launch_zero(C, M * N * c_limbs, stream);
    if (!A || !B || !ws) return RNS_E_ARG;
    SlicedLayout L;
    int rc = sliced_layout(*plan, M, N, K, L);
    if (rc != RNS_OK) return rc;
    if ((int64_t)ws_bytes < L.total) return RNS_E_WORKSPACE;
    uint8_t *base = static_cast<uint8_t *>(ws);
    int64_t *As = reinterpret_cast<int64_t *>(base + L.a_off);
    int64_t *Bs = reinterpret_cast<int64_t *>(base + L.b_off);
    int64_t *parts = reinterpret_cast<int64_t *>(base + L.p_off);
    void *g = base + L.g_off;
    const int sa = plan->sa, sb = plan->sb, na = plan->na, nb = plan->nb, pl = plan->part_limbs;
    hipLaunchKernelGGL(slice_kernel, dim3(grid_of(M * K)), dim3(256), 0, stream, A, M * K, plan->a_limbs, sa, na, As);
    hipLaunchKernelGGL(slice_kernel, dim3(grid_of(K * N)), dim3(256), 0, stream, B, K * N, plan->b_limbs, sb, nb, Bs);
    if (hipGetLastError() != hipSuccess) return RNS_E_HIP;
    for (int i = 0; i < na; i++)
        for (int j = 0; j < nb; j++) {
            rc = rns_gemm(&plan->slice, M, N, K, As + (int64_t)i * M * K * (sa + 1), sa + 1,
                          Bs + (int64_t)j * K * N * (sb + 1), sb + 1, parts + (int64_t)(i * nb + j) * M * N * pl, pl,
                          g, L.g_bytes, stream);
            if (rc != RNS_OK) return rc;
        }
    hipLaunchKernelGGL(sliced_accumulate_kernel, dim3(grid_of(M * N)), dim3(256), 0, stream, parts, na, nb, sa, sb, pl,
                       M * N, C, c_limbs);
    return hipGetLastError() == hipSuccess ? RNS_OK : RNS_E_HIP;
}

}  // extern "C"
