// rns_ratrec.cpp -- the host stage of the exact solve (exact-solve, "Method":
// the final rational reconstruction runs on the CPU): the p-adic value of the
// lift digits, the numerators over a common denominator, and rational
// reconstruction by the extended Euclidean algorithm.
//
// Big integers go through GMP, opened at first use from the system's
// libgmp.so.10 (its documented mpz interface, declared below).  Components are
// spread over host threads; GMP is reentrant and the shared values are only
// read.  No device memory is touched here.
#include <dlfcn.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <thread>
#include <vector>

#include "../../include/rns_solve.h"

namespace {

// ---- GMP, opened at run time ------------------------------------------------------
struct Mpz {
    int alloc;
    int size;  // |size| limbs, sign of the value
    uint64_t *d;
};
using mpz_ptr = Mpz *;
using mpz_srcptr = const Mpz *;

struct Gmp {
    void (*init)(mpz_ptr);
    void (*clear)(mpz_ptr);
    void (*import_)(mpz_ptr, size_t, int, size_t, int, size_t, const void *);
    void *(*export_)(void *, size_t *, int, size_t, int, size_t, mpz_srcptr);
    void (*mul)(mpz_ptr, mpz_srcptr, mpz_srcptr);
    void (*add)(mpz_ptr, mpz_srcptr, mpz_srcptr);
    void (*sub)(mpz_ptr, mpz_srcptr, mpz_srcptr);
    void (*submul)(mpz_ptr, mpz_srcptr, mpz_srcptr);
    void (*fdiv_r)(mpz_ptr, mpz_srcptr, mpz_srcptr);
    void (*tdiv_qr)(mpz_ptr, mpz_ptr, mpz_srcptr, mpz_srcptr);
    int (*cmp)(mpz_srcptr, mpz_srcptr);
    int (*cmpabs)(mpz_srcptr, mpz_srcptr);
    void (*set)(mpz_ptr, mpz_srcptr);
    void (*set_ui)(mpz_ptr, unsigned long);
    void (*neg)(mpz_ptr, mpz_srcptr);
    void (*swap)(mpz_ptr, mpz_ptr);
    void (*fdiv_q_2exp)(mpz_ptr, mpz_srcptr, unsigned long);
    size_t (*sizeinbase)(mpz_srcptr, int);
    void (*mul_si)(mpz_ptr, mpz_srcptr, long);
    void (*addmul_ui)(mpz_ptr, mpz_srcptr, unsigned long);
    void (*submul_ui)(mpz_ptr, mpz_srcptr, unsigned long);
    void (*mul_2exp)(mpz_ptr, mpz_srcptr, unsigned long);
    void (*tdiv_q)(mpz_ptr, mpz_srcptr, mpz_srcptr);
    void (*gcd)(mpz_ptr, mpz_srcptr, mpz_srcptr);
    void (*divexact)(mpz_ptr, mpz_srcptr, mpz_srcptr);
    bool ok = false;
};

const Gmp *gmp() {
    static Gmp g;
    static std::once_flag once;
    std::call_once(once, [] {
        void *h = dlopen("libgmp.so.10", RTLD_NOW | RTLD_LOCAL);
        if (!h) return;
        bool all = true;
        auto get = [&](auto &fn, const char *name) {
            fn = reinterpret_cast<std::remove_reference_t<decltype(fn)>>(dlsym(h, name));
            all = all && fn != nullptr;
        };
        get(g.init, "__gmpz_init");
        get(g.clear, "__gmpz_clear");
        get(g.import_, "__gmpz_import");
        get(g.export_, "__gmpz_export");
        get(g.mul, "__gmpz_mul");
        get(g.add, "__gmpz_add");
        get(g.sub, "__gmpz_sub");
        get(g.submul, "__gmpz_submul");
        get(g.fdiv_r, "__gmpz_fdiv_r");
        get(g.tdiv_qr, "__gmpz_tdiv_qr");
        get(g.cmp, "__gmpz_cmp");
        get(g.cmpabs, "__gmpz_cmpabs");
        get(g.set, "__gmpz_set");
        get(g.set_ui, "__gmpz_set_ui");
        get(g.neg, "__gmpz_neg");
        get(g.swap, "__gmpz_swap");
        get(g.fdiv_q_2exp, "__gmpz_fdiv_q_2exp");
        get(g.sizeinbase, "__gmpz_sizeinbase");
        get(g.mul_si, "__gmpz_mul_si");
        get(g.addmul_ui, "__gmpz_addmul_ui");
        get(g.submul_ui, "__gmpz_submul_ui");
        get(g.mul_2exp, "__gmpz_mul_2exp");
        get(g.tdiv_q, "__gmpz_tdiv_q");
        get(g.gcd, "__gmpz_gcd");
        get(g.divexact, "__gmpz_divexact");
        g.ok = all;
    });
    return g.ok ? &g : nullptr;
}

// An mpz that clears itself.
struct Z {
    Mpz v;
    const Gmp *g;
    explicit Z(const Gmp *g_) : g(g_) { g->init(&v); }
    ~Z() { g->clear(&v); }
    Z(const Z &) = delete;
    Z &operator=(const Z &) = delete;
    mpz_ptr operator&() { return &v; }
    mpz_srcptr c() const { return &v; }
};

int sign(mpz_srcptr x) { return x->size > 0 ? 1 : (x->size < 0 ? -1 : 0); }

// magnitude limbs (least significant first) -> x
void from_mag(const Gmp *g, mpz_ptr x, const uint64_t *mag, int32_t n) {
    g->import_(x, (size_t)n, -1, sizeof(uint64_t), 0, 0, mag);
}

// two's-complement int64 limbs (top limb signed) -> x
void from_twos(const Gmp *g, mpz_ptr x, const int64_t *l, int32_t n, uint64_t *tmp) {
    const bool neg = l[n - 1] < 0;
    uint64_t carry = 1;
    for (int32_t i = 0; i < n; i++) {
        const uint64_t w = (uint64_t)l[i];
        if (neg) {
            const uint64_t t = ~w + carry;
            carry = (carry && t == 0) ? 1 : 0;
            tmp[i] = t;
        } else {
            tmp[i] = w;
        }
    }
    from_mag(g, x, tmp, n);
    if (neg) g->neg(x, x);
}

// |x| < 2^(64n - 1) is required (checked by the callers' bounds); x -> n limbs.
bool to_twos(const Gmp *g, int64_t *out, int32_t n, mpz_srcptr x) {
    std::memset(out, 0, sizeof(int64_t) * (size_t)n);
    if (sign(x) == 0) return true;
    if (g->sizeinbase(x, 2) >= (size_t)64 * (size_t)n) return false;
    size_t cnt = 0;
    g->export_(out, &cnt, -1, sizeof(uint64_t), 0, 0, x);
    if (sign(x) < 0) {
        uint64_t carry = 1;
        for (int32_t i = 0; i < n; i++) {
            const uint64_t t = ~(uint64_t)out[i] + carry;
            carry = (carry && t == 0) ? 1 : 0;
            out[i] = (int64_t)t;
        }
    }
    return true;
}

bool to_mag(const Gmp *g, uint64_t *out, int32_t n, mpz_srcptr x) {
    std::memset(out, 0, sizeof(uint64_t) * (size_t)n);
    if (sign(x) == 0) return true;
    if (g->sizeinbase(x, 2) > (size_t)64 * (size_t)n) return false;
    size_t cnt = 0;
    g->export_(out, &cnt, -1, sizeof(uint64_t), 0, 0, x);
    return true;
}

// floor(|x| / 2^h) for a value known to be below 2^(h + 63), from the limbs
uint64_t top_bits(mpz_srcptr x, size_t h) {
    const size_t n = (size_t)(x->size < 0 ? -x->size : x->size);
    const size_t w = h / 64, b = h % 64;
    const uint64_t lo = w < n ? x->d[w] : 0, hi = w + 1 < n ? x->d[w + 1] : 0;
    return b ? (lo >> b) | (hi << (64 - b)) : lo;
}

// dst = a * x + b * y with single-word signed cofactors
void lincomb(const Gmp *g, mpz_ptr dst, int64_t a, mpz_srcptr x, int64_t b, mpz_srcptr y) {
    g->mul_si(dst, x, (long)a);
    if (b >= 0)
        g->addmul_ui(dst, y, (unsigned long)b);
    else
        g->submul_ui(dst, y, (unsigned long)(-(b + 1)) + 1ul);
}

bool mag_positive(const uint64_t *m, int32_t n) {
    for (int32_t i = 0; i < n; i++)
        if (m[i]) return true;
    return false;
}

}  // namespace

extern "C" {

int rns_host_bigint_available(void) { return gmp() ? 1 : 0; }

}  // extern "C"

namespace {

// w = D X mod P^m in (-P^m/2, P^m/2) and the common-denominator test |w| <= bound,
// shared by the two sources of X.  Barrett reduction by P^m for y = D X with
// |X| <= (P^m - 1)/2 < 2^(L-1): the quotient is below 2^kd (kd = bits of D), and
// mu = floor(2^(L+kd+1) / P^m) has kd + 2 bits, so the estimate
// floor(floor(|y| / 2^(L-1)) mu / 2^(kd+2)) is at most the quotient and a few short.
struct Numerators {
    const Gmp *g;
    Z Pz, Dz, Bz, Pm, half, mu;
    unsigned long L = 0, kd = 0;
    std::vector<Mpz> pw;     // P^(2^j), j <= levels
    explicit Numerators(const Gmp *g_) : g(g_), Pz(g_), Dz(g_), Bz(g_), Pm(g_), half(g_), mu(g_) {}
    ~Numerators() {
        for (auto &z : pw) g->clear(&z);
    }
    void setup(const uint64_t *P, int32_t p_limbs, int32_t steps, const uint64_t *D, int32_t den_limbs,
               const uint64_t *bound, int32_t b_limbs) {
        from_mag(g, &Pz, P, p_limbs);
        from_mag(g, &Dz, D, den_limbs);
        from_mag(g, &Bz, bound, b_limbs);
        int levels = 0;
        while ((1LL << levels) < steps) levels++;
        pw.resize((size_t)levels + 1);
        for (auto &z : pw) g->init(&z);
        g->set(&pw[0], Pz.c());
        for (int j = 1; j <= levels; j++) g->mul(&pw[j], &pw[j - 1], &pw[j - 1]);
        g->set_ui(&Pm, 1);
        for (int j = 0; j <= levels; j++)
            if ((steps >> j) & 1) g->mul(&Pm, Pm.c(), &pw[j]);
        g->fdiv_q_2exp(&half, Pm.c(), 1);  // (P^m - 1) / 2, P odd
        L = (unsigned long)g->sizeinbase(Pm.c(), 2);
        kd = (unsigned long)g->sizeinbase(Dz.c(), 2);
        g->set_ui(&mu, 1);
        g->mul_2exp(&mu, mu.c(), L + kd + 1);
        g->tdiv_q(&mu, mu.c(), Pm.c());
    }
    // X is overwritten
    void finish(mpz_ptr X, Z &tmp, Z &w, int64_t *out, int32_t w_limbs, int32_t *okp) const {
        const bool neg = sign(X) < 0;
        if (neg) g->neg(X, X);
        g->mul(&w, Dz.c(), X);                   // |y|
        g->fdiv_q_2exp(&tmp, w.c(), L - 1);
        g->mul(&tmp, tmp.c(), mu.c());
        g->fdiv_q_2exp(&tmp, tmp.c(), kd + 2);
        g->mul(&tmp, tmp.c(), Pm.c());
        g->sub(&w, w.c(), tmp.c());
        while (g->cmp(w.c(), Pm.c()) >= 0) g->sub(&w, w.c(), Pm.c());
        if (neg && sign(w.c()) != 0) g->sub(&w, Pm.c(), w.c());
        if (g->cmp(w.c(), half.c()) > 0) g->sub(&w, w.c(), Pm.c());
        if (g->cmpabs(w.c(), Bz.c()) <= 0) {
            to_twos(g, out, w_limbs, w.c());       // fits: |w| <= bound < 2^(64 w_limbs - 1)
            *okp = 1;
        } else {
            std::memset(out, 0, sizeof(int64_t) * (size_t)w_limbs);
            *okp = 0;
        }
    }
};

// Up to 16 host threads (or `threads`) take the components from a counter.
template <class Work>
void run_threads(int threads, int64_t items, Work work) {
    int nt = threads ? threads : (int)std::min<unsigned>(std::max(1u, std::thread::hardware_concurrency()), 16u);
    nt = (int)std::max<int64_t>(1, std::min<int64_t>(nt, items));
    std::vector<std::thread> pool;
    for (int i = 1; i < nt; i++) {
        try {
            pool.emplace_back(work);
        } catch (...) {          // no more threads to be had: the ones running share the rest
            break;
        }
    }
    work();
    for (auto &th : pool) th.join();
}

int check_common(int32_t steps, int64_t count, int64_t n_index, int32_t p_limbs, int32_t den_limbs, int32_t b_limbs,
                 int32_t w_limbs, int32_t threads, const int64_t *index, const uint64_t *P, const uint64_t *D,
                 const uint64_t *bound, const void *src, int64_t *num, int32_t *ok) {
    if (steps < 1 || count < 0 || n_index < 0 || p_limbs < 1 || den_limbs < 1 || b_limbs < 1 || w_limbs < 1 ||
        threads < 0)
        return RNS_E_ARG;
    if (!P || !D || !bound || (n_index > 0 && (!src || !index || !num || !ok))) return RNS_E_ARG;
    for (int64_t t = 0; t < n_index; t++)
        if (index[t] < 0 || index[t] >= count) return RNS_E_ARG;
    if (!mag_positive(D, den_limbs) || !(P[0] & 1) || (p_limbs == 1 && P[0] < 3)) return RNS_E_ARG;
    return RNS_OK;
}

}  // namespace

extern "C" {

int rns_padic_numerators(const int64_t *digits, int32_t steps, int64_t count, int32_t d_limbs,
                         const int64_t *index, int64_t n_index, const uint64_t *P, int32_t p_limbs,
                         const uint64_t *D, int32_t den_limbs, const uint64_t *bound, int32_t b_limbs,
                         int64_t *num, int32_t w_limbs, int32_t *ok, int32_t threads) {
    if (d_limbs < 1 || d_limbs > 64) return RNS_E_ARG;
    int rc = check_common(steps, count, n_index, p_limbs, den_limbs, b_limbs, w_limbs, threads, index, P, D, bound,
                          digits, num, ok);
    if (rc != RNS_OK) return rc;
    const Gmp *g = gmp();
    if (!g) return RNS_E_HOSTLIB;
    Numerators nm(g);
    nm.setup(P, p_limbs, steps, D, den_limbs, bound, b_limbs);
    if (g->sizeinbase(nm.Bz.c(), 2) >= (size_t)64 * (size_t)w_limbs) return RNS_E_OUT_LIMBS;
    if (n_index == 0) return RNS_OK;
    std::atomic<int64_t> next{0};
    run_threads(threads, n_index, [&]() {
        std::vector<Mpz> v((size_t)steps);
        for (auto &z : v) g->init(&z);
        Z tmp(g), w(g);
        std::vector<uint64_t> scratch((size_t)d_limbs);
        for (;;) {
            const int64_t t = next.fetch_add(1);
            if (t >= n_index) break;
            const int64_t idx = index[t];
            for (int32_t s = 0; s < steps; s++)
                from_twos(g, &v[s], digits + ((int64_t)s * count + idx) * d_limbs, d_limbs, scratch.data());
            // X = sum_s x_s P^s: adjacent pairs joined level by level
            int64_t n = steps;
            for (int j = 0; n > 1; j++) {
                for (int64_t i = 0; i < n / 2; i++) {
                    g->mul(&tmp, &v[2 * i + 1], &nm.pw[j]);
                    g->add(&v[i], &v[2 * i], tmp.c());
                }
                if (n & 1) g->swap(&v[n / 2], &v[n - 1]);
                n = (n + 1) / 2;
            }
            nm.finish(&v[0], tmp, w, num + t * w_limbs, w_limbs, ok + t);
        }
        for (auto &z : v) g->clear(&z);
    });
    return RNS_OK;
}

int rns_chunk_numerators(const uint32_t *chunks, int64_t T, int64_t count, const int64_t *index, int64_t n_index,
                         const uint64_t *P, int32_t p_limbs, int32_t steps, const uint64_t *D, int32_t den_limbs,
                         const uint64_t *bound, int32_t b_limbs, int64_t *num, int32_t w_limbs, int32_t *ok,
                         int32_t threads) {
    if (T < 1) return RNS_E_ARG;
    int rc = check_common(steps, count, n_index, p_limbs, den_limbs, b_limbs, w_limbs, threads, index, P, D, bound,
                          chunks, num, ok);
    if (rc != RNS_OK) return rc;
    const Gmp *g = gmp();
    if (!g) return RNS_E_HOSTLIB;
    Numerators nm(g);
    nm.setup(P, p_limbs, steps, D, den_limbs, bound, b_limbs);
    if (g->sizeinbase(nm.Bz.c(), 2) >= (size_t)64 * (size_t)w_limbs) return RNS_E_OUT_LIMBS;
    if (n_index == 0) return RNS_OK;
    std::atomic<int64_t> next{0};
    run_threads(threads, n_index, [&]() {
        Z X(g), tmp(g), w(g), top(g);
        for (;;) {
            const int64_t t = next.fetch_add(1);
            if (t >= n_index) break;
            const uint32_t *c = chunks + index[t] * T;
            // T chunks, two's complement: the unsigned value, less 2^(32 T) when the top bit is set
            g->import_(&X, (size_t)T, -1, sizeof(uint32_t), 0, 0, c);
            if (c[T - 1] >> 31) {
                g->set_ui(&top, 1);
                g->mul_2exp(&top, top.c(), (unsigned long)(32 * T));
                g->sub(&X, X.c(), top.c());
            }
            nm.finish(&X, tmp, w, num + t * w_limbs, w_limbs, ok + t);
        }
    });
    return RNS_OK;
}

int rns_rational_reconstruct(const uint64_t *u, int32_t u_limbs, const uint64_t *M, int32_t m_limbs,
                             const uint64_t *Nb, int32_t nb_limbs, const uint64_t *Db, int32_t db_limbs,
                             int64_t *num, int32_t num_limbs, uint64_t *den, int32_t den_limbs) {
    if (!u || !M || !Nb || !Db || !num || !den || u_limbs < 1 || m_limbs < 1 || nb_limbs < 1 || db_limbs < 1 ||
        num_limbs < 1 || den_limbs < 1)
        return RNS_E_ARG;
    if (!mag_positive(M, m_limbs)) return RNS_E_ARG;
    const Gmp *g = gmp();
    if (!g) return RNS_E_HOSTLIB;
    Z Mz(g), uz(g), Nz(g), Dz(g), r0(g), r1(g), t0(g), t1(g), q(g), r(g), chk(g);
    from_mag(g, &Mz, M, m_limbs);
    from_mag(g, &uz, u, u_limbs);
    from_mag(g, &Nz, Nb, nb_limbs);
    from_mag(g, &Dz, Db, db_limbs);
    g->fdiv_r(&uz, uz.c(), Mz.c());
    // r_i = t_i u (mod M) along the remainder sequence of (M, u); stop at the
    // first remainder within the numerator bound
    g->set(&r0, Mz.c());
    g->set(&r1, uz.c());
    g->set_ui(&t0, 0);
    g->set_ui(&t1, 1);
    auto euclid_step = [&]() {
        g->tdiv_qr(&q, &r, r0.c(), r1.c());
        g->swap(&r0, &r1);
        g->swap(&r1, &r);
        g->submul(&t0, q.c(), t1.c());  // t0 - q t1
        g->swap(&t0, &t1);
    };
    // Lehmer's method (Knuth, TAOCP vol. 2, 4.5.2, Algorithm L) while the remainders are far above
    // the bound: Euclid on the leading 62 bits yields the next quotients, exactly where the two
    // bracketing single-word quotients agree, as one 2x2 cofactor matrix applied at once.  A batch
    // shrinks r1 by at most 64 bits (its matrix entries are below 2^62), so it cannot step past
    // the first remainder within the bound.
    const size_t nb_bits = g->sizeinbase(Nz.c(), 2);
    Z u0(g), u1(g), v0(g), v1(g);
    while (sign(r1.c()) != 0 && g->sizeinbase(r1.c(), 2) > nb_bits + 70) {
        const size_t h = g->sizeinbase(r0.c(), 2) - 62;
        int64_t x = (int64_t)top_bits(r0.c(), h), y = (int64_t)top_bits(r1.c(), h);
        int64_t A = 1, B = 0, C = 0, D = 1;
        for (;;) {
            if (y + C <= 0 || y + D <= 0 || x + A < 0 || x + B < 0) break;
            const int64_t q1 = (x + A) / (y + C), q2 = (x + B) / (y + D);
            if (q1 != q2) break;
            const __int128 nC = (__int128)A - (__int128)q1 * C, nD = (__int128)B - (__int128)q1 * D;
            if (nC > ((__int128)1 << 62) || nC < -((__int128)1 << 62) || nD > ((__int128)1 << 62) ||
                nD < -((__int128)1 << 62))
                break;
            A = C;
            C = (int64_t)nC;
            B = D;
            D = (int64_t)nD;
            const int64_t ny = x - q1 * y;
            x = y;
            y = ny;
        }
        if (B == 0) {
            euclid_step();
            continue;
        }
        lincomb(g, &u0, A, r0.c(), B, r1.c());
        lincomb(g, &u1, C, r0.c(), D, r1.c());
        lincomb(g, &v0, A, t0.c(), B, t1.c());
        lincomb(g, &v1, C, t0.c(), D, t1.c());
        g->swap(&r0, &u0);
        g->swap(&r1, &u1);
        g->swap(&t0, &v0);
        g->swap(&t1, &v1);
    }
    while (g->cmp(r1.c(), Nz.c()) > 0) euclid_step();
    if (sign(t1.c()) == 0 || g->cmpabs(t1.c(), Dz.c()) > 0) return RNS_E_RECONSTRUCT;
    g->mul(&chk, t1.c(), uz.c());
    g->sub(&chk, r1.c(), chk.c());
    g->fdiv_r(&chk, chk.c(), Mz.c());
    if (sign(chk.c()) != 0) return RNS_E_RECONSTRUCT;
    if (sign(t1.c()) < 0) {
        g->neg(&t1, t1.c());
        g->neg(&r1, r1.c());
    }
    if (!to_twos(g, num, num_limbs, r1.c()) || !to_mag(g, den, den_limbs, t1.c())) return RNS_E_OUT_LIMBS;
    return RNS_OK;
}

int rns_pow_table(const uint64_t *P, int32_t p_limbs, int32_t m, int64_t T, int64_t *out) {
    if (!P || !out || p_limbs < 1 || m < 1 || T < 1) return RNS_E_ARG;
    const Gmp *g = gmp();
    if (!g) return RNS_E_HOSTLIB;
    Z Pz(g), v(g);
    from_mag(g, &Pz, P, p_limbs);
    g->set_ui(&v, 1);
    // the powers' chunks power by power, then written out transposed in 64 x 64 blocks (a column
    // of out is m * 8 bytes apart, so writing it power by power touches a new line per chunk)
    // (exported as native 64-bit words, GMP's fast path, and split into chunks here)
    const size_t T64 = ((size_t)T + 1) / 2;
    std::vector<uint64_t> words((size_t)m * T64, 0u);
    for (int32_t s = 0; s < m; s++) {
        if (g->sizeinbase(v.c(), 2) > (size_t)32 * (size_t)T) return RNS_E_ARG;
        size_t cnt = 0;
        g->export_(words.data() + (size_t)s * T64, &cnt, -1, sizeof(uint64_t), 0, 0, v.c());
        g->mul(&v, v.c(), Pz.c());
    }
    for (int64_t t0 = 0; t0 < T; t0 += 64)
        for (int32_t s0 = 0; s0 < m; s0 += 64)
            for (int64_t t = t0; t < std::min<int64_t>(t0 + 64, T); t++)
                for (int32_t s = s0; s < std::min<int32_t>(s0 + 64, m); s++)
                    out[t * m + s] = (int64_t)((words[(size_t)s * T64 + (size_t)(t >> 1)] >> (32 * (t & 1))) &
                                               0xffffffffull);
    return RNS_OK;
}

int rns_pow2_quotient(int64_t e, const uint64_t *d, int32_t d_limbs, uint64_t *q, int32_t q_limbs) {
    if (!d || !q || e < 0 || d_limbs < 1 || q_limbs < 1 || !mag_positive(d, d_limbs)) return RNS_E_ARG;
    const Gmp *g = gmp();
    if (!g) return RNS_E_HOSTLIB;
    Z dz(g), qz(g);
    from_mag(g, &dz, d, d_limbs);
    g->set_ui(&qz, 1);
    g->mul_2exp(&qz, qz.c(), (unsigned long)e);
    g->tdiv_q(&qz, qz.c(), dz.c());
    if (g->sizeinbase(qz.c(), 2) > (size_t)64 * (size_t)q_limbs) return RNS_E_OUT_LIMBS;
    std::memset(q, 0, sizeof(uint64_t) * (size_t)q_limbs);
    size_t cnt = 0;
    g->export_(q, &cnt, -1, sizeof(uint64_t), 0, 0, qz.c());
    return RNS_OK;
}


int rns_reduce_fractions(const int64_t *num, int64_t count, int32_t limbs, const uint64_t *D, int32_t d_limbs,
                         int64_t *num_out, uint64_t *den_out, int32_t threads) {
    if (count < 0 || limbs < 1 || d_limbs < 1 || threads < 0 || !D || !mag_positive(D, d_limbs) ||
        (count > 0 && (!num || !num_out || !den_out)))
        return RNS_E_ARG;
    const Gmp *g = gmp();
    if (!g) return RNS_E_HOSTLIB;
    std::atomic<int64_t> next{0};
    std::atomic<int> fail{0};
    run_threads(threads, count, [&] {
        Z Dz(g), x(g), gz(g), t(g);
        std::vector<uint64_t> tmp((size_t)limbs);
        from_mag(g, &Dz, D, d_limbs);
        for (int64_t i = next++; i < count; i = next++) {
            from_twos(g, &x, num + i * limbs, limbs, tmp.data());
            g->gcd(&gz, x.c(), Dz.c());                  // gcd(|N|, D) > 0 since D > 0
            g->divexact(&t, x.c(), gz.c());
            to_twos(g, num_out + i * limbs, limbs, t.c());
            g->divexact(&t, Dz.c(), gz.c());
            if (g->sizeinbase(t.c(), 2) > (size_t)64 * (size_t)d_limbs) {
                fail = 1;
                continue;
            }
            std::memset(den_out + i * d_limbs, 0, sizeof(uint64_t) * (size_t)d_limbs);
            size_t cnt = 0;
            g->export_(den_out + i * d_limbs, &cnt, -1, sizeof(uint64_t), 0, 0, t.c());
        }
    });
    return fail ? RNS_E_OUT_LIMBS : RNS_OK;
}

}  // extern "C"
