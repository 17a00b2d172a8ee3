// The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
// plans, workspace layouts, argument checks and the per-plan constant tables
// (every entry point down to its launches, which are host stand-ins here), and
// the host big-integer stage of the exact solve against 128-bit arithmetic.
// Exit status 0 when every check holds.
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <random>
#include <vector>

#include "../../include/rns_gemm.h"
#include "../../include/rns_solve.h"

static int fails = 0;
#define CHECK(c)                                                            \
    do {                                                                    \
        if (!(c)) {                                                         \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            fails++;                                                        \
        }                                                                   \
    } while (0)

typedef __int128 i128;

static i128 gcd128(i128 a, i128 b) {
    if (a < 0) a = -a;
    if (b < 0) b = -b;
    while (b) { i128 t = a % b; a = b; b = t; }
    return a;
}

// pointers the host code only computes with (the launches are stand-ins)
static void *fake(uintptr_t a) { return reinterpret_cast<void *>(a); }

static void plans() {
    rns_plan_t p;
    for (int64_t K : {1, 64, 1024, 4096, 131072, 131073})
        for (int a : {-1, 0, 20, 31, 52, 63, 100, 127, 160})
            for (int b : {-1, 0, 31, 64, 100, 160}) {
                const int rc = rns_plan(K, a, b, &p);
                CHECK(rc == RNS_OK || rc == RNS_E_CAPACITY || rc == RNS_E_K || rc == RNS_E_ARG);
                if (rc == RNS_OK) CHECK(p.n_primes >= 1 && p.n_primes <= RNS_MAX_PRIMES && p.out_limbs_min >= 1);
            }
    for (int n = -1; n <= RNS_MAX_PRIMES + 1; n++)
        for (int kind : {RNS_MODULI_PRIMES, RNS_MODULI_PRIME_POWERS, 7}) {
            const int rc = rns_plan_n_moduli(n, kind, &p);
            CHECK((rc == RNS_OK) == (n >= 1 && n <= RNS_MAX_PRIMES && kind != 7));
        }
    CHECK(rns_plan(64, 20, 20, nullptr) == RNS_E_ARG);
    for (int code = -12; code <= 1; code++) CHECK(rns_error_string(code) != nullptr);
}

// every stage on fake device pointers: layouts, argument checks, tables
static void calls(const rns_plan_t &p, int64_t M, int64_t N, int64_t K, int la, int lb, bool batched) {
    size_t ws = 0;
    const int rc = rns_workspace_size(&p, M, N, K, batched, &ws);
    if (rc != RNS_OK) return;
    rns_layout_t L;
    CHECK(rns_workspace_layout(&p, M, N, K, batched, &L) == RNS_OK);
    if (M && N && K) {
        CHECK((size_t)L.total_bytes == ws && L.b_off >= 0 && L.y_off > L.b_off && L.b_plane >= L.n_pad * L.k_pad);
        CHECK(batched ? true : L.a_plane >= L.m_pad * L.k_pad);
    }
    void *W = fake(1 << 20), *A = fake(1 << 21), *B = fake(1 << 22), *C = fake(1 << 23);
    const int lc = p.out_limbs_min;
    if (!batched) {
        CHECK(rns_gemm(&p, M, N, K, (const int64_t *)A, la, (const int64_t *)B, lb, (int64_t *)C, lc, W, ws,
                       nullptr) == RNS_OK);
        CHECK(rns_split(&p, M, N, K, (const int64_t *)A, la, (const int64_t *)B, lb, W, ws, nullptr) == RNS_OK);
        CHECK(rns_residue_products(&p, M, N, K, nullptr, W, ws, nullptr) == RNS_OK);
        // errors, before anything is launched
        CHECK(rns_gemm(&p, M, N, K, (const int64_t *)A, 0, (const int64_t *)B, lb, (int64_t *)C, lc, W, ws,
                       nullptr) == RNS_E_ARG);
        CHECK(rns_gemm(&p, M, N, K, (const int64_t *)A, la, (const int64_t *)B, lb, (int64_t *)C, lc, W,
                       ws ? ws - 1 : 0, nullptr) != RNS_OK || !(M && N && K));
    } else {
        CHECK(rns_gemm_batched_residue(&p, M, N, K, (const int8_t *)A, (const int64_t *)B, lb, (int64_t *)C, lc,
                                       W, ws, nullptr) == RNS_OK);
        CHECK(rns_split(&p, M, N, K, nullptr, 0, (const int64_t *)B, lb, W, ws, nullptr) == RNS_OK);
        CHECK(rns_residue_products(&p, M, N, K, (const int8_t *)A, W, ws, nullptr) == RNS_OK);
    }
    CHECK(rns_reconstruct(&p, M, N, K, batched, (int64_t *)C, lc, W, ws, nullptr) == RNS_OK);
    CHECK(rns_reconstruct_garner(&p, M, N, K, batched, (int64_t *)C, lc, W, ws, nullptr) == RNS_OK);
    CHECK(rns_reconstruct(&p, M, N, K, batched, (int64_t *)C, lc - 1, W, ws, nullptr) == RNS_E_OUT_LIMBS ||
          lc == 1 || !(M && N));
    CHECK(rns_gemm(nullptr, M, N, K, (const int64_t *)A, la, (const int64_t *)B, lb, (int64_t *)C, lc, W, ws,
                   nullptr) == RNS_E_ARG);
    CHECK(rns_gemm(&p, -1, N, K, (const int64_t *)A, la, (const int64_t *)B, lb, (int64_t *)C, lc, W, ws,
                   nullptr) == RNS_E_ARG);
}

static void stages() {
    rns_plan_t p;
    struct S { int64_t M, N, K; int la, lb, a, b; };
    const S shapes[] = {{1, 1, 1, 1, 1, 10, 10}, {64, 64, 64, 1, 1, 20, 20}, {65, 70, 130, 2, 3, 90, 150},
                        {2048, 2048, 4096, 2, 2, 100, 100}, {513, 260, 129, 4, 4, 150, 160},
                        {17, 5, 4096, 1, 2, 60, 90}, {0, 5, 7, 1, 1, 10, 10}, {3, 3, 0, 1, 1, 10, 10}};
    for (const S &s : shapes) {
        if (rns_plan(s.K > 0 ? s.K : 1, s.a, s.b, &p) != RNS_OK) continue;
        calls(p, s.M, s.N, s.K, s.la, s.lb, false);
    }
    for (int n : {1, 6, 20, 54})
        for (int kind : {RNS_MODULI_PRIMES, RNS_MODULI_PRIME_POWERS}) {
            if (rns_plan_n_moduli(n, kind, &p) != RNS_OK) continue;
            calls(p, 1024, 16, 1024, 0, 1, true);     // the skinny path
            calls(p, 300, 7, 48, 0, 1, true);
            calls(p, 257, 300, 129, 0, 2, true);     // the general path
        }
}

// the host big-integer stage against 128-bit integers
static void bigint() {
    if (!rns_host_bigint_available()) {
        std::fprintf(stderr, "libgmp.so.10 not available: host big-integer checks skipped\n");
        return;
    }
    std::mt19937_64 rng(7);
    // rational reconstruction: M a product of odd primes below 2^62, N/d with |N|, d below 2^28
    const uint64_t M = 4611686018427387847ull;      // prime below 2^62
    for (int t = 0; t < 2000; t++) {
        int64_t a = (int64_t)(rng() % (1ull << 28)) - (1ll << 27);
        uint64_t d = 1 + rng() % ((1ull << 28) - 1);
        // u = a / d mod M by Fermat: d^(M-2)
        i128 base = d % M, e = M - 2, inv = 1;
        while (e > 0) {
            if (e & 1) inv = inv * base % M;
            base = base * base % M;
            e >>= 1;
        }
        i128 u = ((i128)(a % (int64_t)M + (int64_t)M) % M) * inv % M;
        uint64_t uu = (uint64_t)u, mm = M, nb = 1ull << 28, db = 1ull << 28;
        int64_t num = 0;
        uint64_t den = 0;
        const int rc = rns_rational_reconstruct(&uu, 1, &mm, 1, &nb, 1, &db, 1, &num, 1, &den, 1);
        CHECK(rc == RNS_OK);
        if (rc == RNS_OK) CHECK((i128)num * d == (i128)a * den);
    }
    // lowest terms: N_i / D with 128-bit N_i
    for (int t = 0; t < 200; t++) {
        const uint64_t D = (1 + rng() % 1000000) * (1ull << (rng() % 20));
        const int count = 64;
        std::vector<int64_t> num(2 * count), out(2 * count);
        std::vector<uint64_t> den(count);
        std::vector<i128> val(count);
        for (int i = 0; i < count; i++) {
            i128 v = (i128)(int64_t)(rng() >> (rng() % 64)) * (int64_t)(1 + rng() % 4096);
            if (i % 7 == 0) v = 0;
            if (i % 11 == 0) v = (i128)D * (int64_t)(rng() % 1000);
            val[i] = v;
            num[2 * i] = (int64_t)(uint64_t)v;
            num[2 * i + 1] = (int64_t)(v >> 64);
        }
        CHECK(rns_reduce_fractions(num.data(), count, 2, &D, 1, out.data(), den.data(), 0) == RNS_OK);
        for (int i = 0; i < count; i++) {
            const i128 n2 = (i128)(uint64_t)out[2 * i] + (i128)out[2 * i + 1] * ((i128)1 << 64);
            CHECK(den[i] > 0 && n2 * (i128)D == val[i] * (i128)den[i] && gcd128(n2, den[i]) == 1);
        }
    }
    // powers and quotients
    const uint64_t P = 1000003ull * 999983ull;
    std::vector<int64_t> tab(8 * 3);
    CHECK(rns_pow_table(&P, 1, 3, 8, tab.data()) == RNS_OK);
    i128 acc = 0;
    for (int t = 3; t >= 0; t--) acc = (acc << 32) | (uint32_t)tab[t * 3 + 2];
    CHECK(acc == (i128)P * P);
    uint64_t q[2] = {0, 0}, dd = 1000003ull;
    CHECK(rns_pow2_quotient(100, &dd, 1, q, 2) == RNS_OK);
    const i128 qq = (i128)q[0] | ((i128)q[1] << 64);
    CHECK(qq * dd <= ((i128)1 << 100) && (qq + 1) * dd > ((i128)1 << 100));
    CHECK(rns_reduce_fractions(nullptr, 1, 1, &dd, 1, nullptr, nullptr, 0) == RNS_E_ARG);
}

// the measurement aid's argument checks, then one accepted call (the stand-in
// launcher checks what it receives)
static void probe() {
    alignas(16) static int8_t src[2 * 256 * 128];
    static int32_t out[2 * 256];
    int ok = rns_probe_int8_mfma(src, sizeof src, 2, 3, out, nullptr) == RNS_OK;
    ok &= rns_probe_int8_mfma(src, sizeof src - 1, 2, 3, out, nullptr) == RNS_E_ARG;
    ok &= rns_probe_int8_mfma(src + 1, sizeof src - 1, 1, 3, out, nullptr) == RNS_E_ARG;
    ok &= rns_probe_int8_mfma(nullptr, sizeof src, 1, 3, out, nullptr) == RNS_E_ARG;
    ok &= rns_probe_int8_mfma(src, sizeof src, 1, 0, out, nullptr) == RNS_E_ARG;
    if (!ok) {
        std::fprintf(stderr, "probe argument checks\n");
        fails++;
    }
}

int main() {
    plans();
    stages();
    probe();
    bigint();
    if (fails) std::fprintf(stderr, "%d checks failed\n", fails);
    else std::printf("host checks passed\n");
    return fails ? 1 : 0;
}
