// Host-only stand-ins for the launchers that live in the .hip sources, so that
// the library's host code (plans, layouts, argument checks, the per-plan
// constant tables, the host big-integer stage) links into a plain g++ build
// under AddressSanitizer and UndefinedBehaviorSanitizer.  Every launch
// "succeeds" without touching memory; the pointers it receives are checked
// only for the alignment and ordering the real launchers rely on.
#include <cstdio>
#include <cstdlib>

#include "../../exact_integer_gemm_amd/csrc/rns_internal.h"

namespace rns {

static void require(bool ok, const char *what) {
    if (!ok) {
        std::fprintf(stderr, "stub launcher: %s\n", what);
        std::abort();
    }
}

int launch_split(const SplitOperand *a, const SplitOperand *b, const SplitConsts &c, uint32_t *status,
                 int64_t status_slots, hipStream_t) {
    require(b != nullptr && status != nullptr && status_slots > kStatusHeader, "split arguments");
    require(c.n >= 1 && c.n <= kMaxPrimes, "split constants");
    for (const SplitOperand *op : {a, b})
        if (op) require(op->plane >= op->r_pad * op->k_pad && op->rows <= op->r_pad && op->k <= op->k_pad,
                        "split operand shape");
    return RNS_OK;
}

int64_t split_status_slots(const SplitOperand *a, const SplitOperand *b, int) {
    return kStatusHeader + (a ? a->r_pad * (a->k_pad / kKBlock) : 0) + b->r_pad * (b->k_pad / kKBlock);
}

int launch_repack_residues(const int8_t *, int64_t n, int64_t M, int64_t K, int8_t *, int64_t m_pad, int64_t k_pad,
                           int64_t plane, hipStream_t) {
    require(n >= 1 && M <= m_pad && K <= k_pad && plane >= m_pad * k_pad, "repack shape");
    return RNS_OK;
}

int launch_gemm(int cfg, int n, const int8_t *, const int8_t *, int8_t *, int64_t m_pad, int64_t n_pad,
                int64_t k_pad, int64_t a_plane, int64_t b_plane, int64_t, int64_t, int64_t, int64_t, int64_t,
                int64_t, int8_t *, const EpiConsts &, hipStream_t) {
    const TileShape ts = tile_shape(cfg);
    require(n >= 1 && m_pad % ts.bm == 0 && n_pad % ts.bn == 0 && k_pad % ts.bk == 0, "gemm tiles");
    require(a_plane > 0 && b_plane >= n_pad * k_pad, "gemm planes");
    return RNS_OK;
}

int launch_garner(const GarnerConsts &g, const int8_t *, int64_t, int64_t, int64_t M, int64_t N, int64_t *,
                  int32_t c_limbs, hipStream_t) {
    require(g.n >= 1 && M >= 0 && N >= 0 && c_limbs >= 1, "garner arguments");
    return RNS_OK;
}

int launch_mfma_probe(const int8_t *src, int workgroups, int iters, int32_t *out, hipStream_t) {
    require(src != nullptr && out != nullptr && workgroups >= 1 && iters >= 1, "probe arguments");
    require(reinterpret_cast<uintptr_t>(src) % 16 == 0, "probe source alignment");
    return RNS_OK;
}

int launch_zero(int64_t *, int64_t count, hipStream_t) {
    require(count >= 0, "zero count");
    return RNS_OK;
}

int launch_lift_step(const StepConsts &lc, const CrtDigits &, int ksteps, int nblocks, const int8_t *a,
                     const int64_t *r, int64_t M, int64_t N, int64_t K, int64_t *C, int32_t c_limbs,
                     uint32_t *status, hipStream_t) {
    require(lc.n >= 1 && a && r && C && M >= 1 && N >= 1 && N <= 16 && K % 16 == 0 && K <= RNS_LIFT_K_MAX &&
                status != nullptr && lc.n + 2 <= 32 * ksteps && nblocks >= 1 && nblocks <= 2 && c_limbs >= 1,
            "lift step arguments");
    for (int j = 0; j < lc.n; j++) require(lc.q[j] >= 2 && lc.q[j] <= 256 && lc.c1[j] < lc.q[j], "lift tables");
    return RNS_OK;
}

int launch_crt(const CrtConsts &c, const CrtDigits &, int ksteps, int nblocks, const int8_t *, int64_t, int64_t,
               int64_t, int64_t, int64_t *, int32_t c_limbs, hipStream_t) {
    require(c.n + 2 <= 32 * ksteps && nblocks >= 1 && nblocks <= 2 && c_limbs >= 1, "crt arguments");
    return RNS_OK;
}

}  // namespace rns
