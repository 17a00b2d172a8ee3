// Host side of librns_gemm: prime plans, per-prime constant tables, workspace
// layout, argument validation and the C ABI declared in include/rns_gemm.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "rns_internal.h"

namespace rns {
namespace {

// ---- the moduli, largest first ----------------------------------------------
// kind RNS_MODULI_PRIMES: the primes below 256.  kind RNS_MODULI_PRIME_POWERS:
// for each of those primes its largest power not above 256 (256, 243, 169,
// 125, 121, 49 and the primes from 17 up), the factors of lcm(1..256).
bool is_prime(int x) {
    if (x < 2) return false;
    for (int d = 2; d * d <= x; d++)
        if (x % d == 0) return false;
    return true;
}
struct ModuliTable {
    int p[kMaxPrimes];
    explicit ModuliTable(bool powers) {
        int cnt = 0;
        for (int x = 255; x >= 2; x--) {
            if (!is_prime(x)) continue;
            int q = x;
            if (powers)
                while (q * x <= 256) q *= x;
            p[cnt++] = q;
        }
        std::sort(p, p + cnt, [](int a, int b) { return a > b; });
    }
};
const ModuliTable &moduli(int kind) {
    static const ModuliTable primes(false), powers(true);
    return kind == RNS_MODULI_PRIME_POWERS ? powers : primes;
}

// ---- a minimal unsigned big integer (little-endian 32-bit words) ----------
struct Big {
    std::vector<uint32_t> w;
    explicit Big(uint64_t v = 0) {
        if (v) { w.push_back((uint32_t)v); if (v >> 32) w.push_back((uint32_t)(v >> 32)); }
    }
    void mul_small(uint32_t m) {
        uint64_t carry = 0;
        for (auto &x : w) {
            uint64_t t = (uint64_t)x * m + carry;
            x = (uint32_t)t;
            carry = t >> 32;
        }
        if (carry) w.push_back((uint32_t)carry);
    }
    void shl(int bits) {
        const int words = bits / 32, r = bits % 32;
        if (w.empty()) return;
        std::vector<uint32_t> o(w.size() + words + 1, 0);
        for (size_t i = 0; i < w.size(); i++) {
            uint64_t v = (uint64_t)w[i] << r;
            o[i + words] |= (uint32_t)v;
            o[i + words + 1] |= (uint32_t)(v >> 32);
        }
        w = o;
        trim();
    }
    void trim() { while (!w.empty() && w.back() == 0) w.pop_back(); }
    int bit_length() const {
        if (w.empty()) return 0;
        int b = 32 * (int)(w.size() - 1);
        uint32_t top = w.back();
        while (top) { b++; top >>= 1; }
        return b;
    }
    uint16_t chunk16(int c) const {
        const int wi = c / 2;
        if (wi >= (int)w.size()) return 0;
        return (uint16_t)((c & 1) ? (w[wi] >> 16) : (w[wi] & 0xffff));
    }
    // strict comparison a > b
    static bool greater(Big a, Big b) {
        a.trim(); b.trim();
        if (a.w.size() != b.w.size()) return a.w.size() > b.w.size();
        for (size_t i = a.w.size(); i-- > 0;)
            if (a.w[i] != b.w[i]) return a.w[i] > b.w[i];
        return false;
    }
};

int64_t powmod(int64_t b, int64_t e, int64_t m) {
    int64_t r = 1 % m;
    b %= m;
    if (b < 0) b += m;
    while (e > 0) {
        if (e & 1) r = r * b % m;
        b = b * b % m;
        e >>= 1;
    }
    return r;
}
int64_t inv_mod(int64_t a, int64_t q) {   // gcd(a, q) = 1 (extended Euclid)
    int64_t r0 = q, r1 = ((a % q) + q) % q, t0 = 0, t1 = 1;
    while (r1 != 0) {
        const int64_t k = r0 / r1;
        int64_t r = r0 - k * r1; r0 = r1; r1 = r;
        int64_t t = t0 - k * t1; t0 = t1; t1 = t;
    }
    return ((t0 % q) + q) % q;
}
int balanced(int64_t x, int64_t q) {
    int64_t r = x % q;
    if (r < 0) r += q;
    return (int)(r > q / 2 ? r - q : r);
}

void fill_common(rns_plan_t *out, int n, int kind) {
    Big P(1);
    double l2 = 0;
    for (int i = 0; i < kMaxPrimes; i++) out->primes[i] = 0;
    for (int i = 0; i < n; i++) {
        const int q = moduli(kind).p[i];
        out->primes[i] = q;
        P.mul_small((uint32_t)q);
        l2 += std::log2((double)q);
    }
    out->n_primes = n;
    out->log2_P = l2;
    out->out_limbs_min = (P.bit_length() + 63) / 64;
}

// the prime of a prime power q <= 256, or 0 when q is not one
int prime_of(int q) {
    for (int d = 2; d <= q; d++)
        if (q % d == 0) {
            int r = q;
            while (r % d == 0) r /= d;
            return (r == 1 && is_prime(d)) ? d : 0;
        }
    return 0;
}

bool plan_ok(const rns_plan_t *p) {
    if (!p || p->n_primes < 1 || p->n_primes > kMaxPrimes) return false;
    if (p->k_max < 1 || p->k_max > RNS_K_MAX) return false;
    if (p->out_limbs_min < 1 || p->out_limbs_min > RNS_MAX_OUT_LIMBS) return false;
    // the moduli must be prime powers up to 256 over distinct primes (so
    // pairwise coprime), in any order; 256 (residues down to -128) needs
    // K <= 2^17 - 1 for exact int32 accumulation
    bool seen[257] = {false};
    for (int i = 0; i < p->n_primes; i++) {
        const int q = p->primes[i];
        if (q < 2 || q > 256) return false;
        const int pr = prime_of(q);
        if (!pr || seen[pr]) return false;
        seen[pr] = true;
        if (q == 256 && p->k_max > RNS_K_MAX - 1) return false;
    }
    return true;
}

// ---- tables -------------------------------------------------------------------
void build_split(const rns_plan_t &pl, int la, int lb, SplitConsts &c) {
    std::memset(&c, 0, sizeof(c));
    c.n = pl.n_primes;
    const int limbs[2] = {la > 0 ? la : 1, lb};
    for (int j = 0; j < pl.n_primes; j++) {
        const int q = pl.primes[j];
        c.q[j] = q;
        float inv = 1.0f / (float)q;
        if (q % 2 == 0) inv = std::nextafterf(inv, 0.0f);   // q is a power of two
        c.inv[j] = inv;
        for (int b = 0; b < kSplitBytes; b++) {
            const int64_t v = powmod(256, b, q);              // in [0, q)
            const int64_t t = v > q / 2 ? v - q : v;          // balanced, |t| <= 127
            c.t[j][b / 4] |= (uint32_t)(uint8_t)(int8_t)t << (8 * (b % 4));
        }
        for (int o = 0; o < 2; o++) {
            int64_t sum = 0;                                  // 1 + 256 + ... + 256^(8L-2) mod q
            for (int b = 0; b < 8 * limbs[o] - 1; b++) sum = (sum + powmod(256, b, q)) % q;
            const int64_t cl = 128 * sum % q;
            c.start[o][j] = (int32_t)(cl + (int64_t)q * ((kSplitSumBias + q - 1) / q));
        }
    }
}

void build_epi(const rns_plan_t &pl, EpiConsts &c) {
    std::memset(&c, 0, sizeof(c));
    for (int j = 0; j < pl.n_primes; j++) {
        const int q = pl.primes[j];
        c.q[j] = q;
        c.inv[j] = 1.0 / (double)q;
    }
}

// Garner order: 2 first when present (so that balanced mixed-radix digits land
// in (-P/2, P/2] for even P), then the plan order.
void build_garner(const rns_plan_t &pl, GarnerConsts &g) {
    std::memset(&g, 0, sizeof(g));
    const int n = pl.n_primes;
    g.n = n;
    int slot = 0;
    for (int j = 0; j < n; j++)
        if (pl.primes[j] % 2 == 0) g.plane[slot++] = (uint8_t)j;
    for (int j = 0; j < n; j++)
        if (pl.primes[j] % 2 != 0) g.plane[slot++] = (uint8_t)j;
    for (int k = 0; k < kGarnerSlots; k++) {
        if (k < n) {
            g.q[k] = (uint16_t)pl.primes[g.plane[k]];
            g.inv[k] = 1.0 / (double)g.q[k];
        } else {
            // inert padding slot: reads plane of slot 0, multiplies it by 0
            g.plane[k] = g.plane[0];
            g.q[k] = 1;
            g.inv[k] = 1.0;
        }
    }
    // Q_j mod q_k for j <= k, by running products
    for (int k = 0; k < n; k++) {
        const int64_t qk = g.q[k];
        int64_t Qj = 1 % qk;   // Q_0 = 1
        std::vector<int64_t> Qmod(k + 1);
        for (int j = 0; j <= k; j++) {
            Qmod[j] = Qj;
            Qj = Qj * g.q[j] % qk;
        }
        const int64_t Qk_inv = inv_mod(Qmod[k], qk);
        g.tri[tri_index(k, k)] = (int8_t)balanced(Qk_inv, qk);
        for (int j = 0; j < k; j++)
            g.tri[tri_index(j, k)] = (int8_t)balanced(Qmod[j] * Qk_inv, qk);
    }
    // 16-bit chunks of every Q_k
    Big Q(1);
    for (int k = 0; k < n; k++) {
        const int nb = (Q.bit_length() + 15) / 16;
        for (int c = 0; c < nb && c < garner_chunks(k); c++)
            g.q16[garner_chunk_offset(k) + c] = Q.chunk16(c);
        Q.mul_small(g.q[k]);
    }
}

// CRT by rounded quotient: per slot the fixed-point weight c_k = round(w_k
// 2^31 / q_k), P's words, and the balanced base-256 digits of every basis
// element e_k = w_k M_k (signed), of P and of 256 P.  Returns the MFMA K
// steps and N blocks through *ksteps, *nblocks.
// balanced base-256 digits of +-v (out[i] in [-128, 127], sum out[i] 256^i);
// returns the digits in use
int signed_digits(const Big &v, bool neg, int8_t *out) {
    int carry = 0, last = 0;
    const int nbytes = 4 * (int)v.w.size();
    for (int ci = 0; ci < kCrtDigits; ci++) {
        int byte = ci < nbytes ? (int)((v.w[ci / 4] >> (8 * (ci % 4))) & 0xffu) : 0;
        if (neg) byte = -byte;
        byte += carry;                       // in [-256, 256]
        carry = 0;
        while (byte >= 128) { byte -= 256; carry++; }
        while (byte < -128) { byte += 256; carry--; }
        out[ci] = (int8_t)byte;
        if (byte) last = ci + 1;
    }
    return last;
}
int64_t floor_div(int64_t a, int64_t b) {   // b > 0
    return a >= 0 ? a / b : -((-a + b - 1) / b);
}
void build_crt(const rns_plan_t &pl, CrtConsts &c, CrtDigits &d, int *ksteps, int *nblocks) {
    const int n = pl.n_primes;
    std::memset(&c, 0, sizeof(c));
    std::memset(&d, 0, sizeof(d));
    c.n = n;
    Big P(1);
    for (int k = 0; k < n; k++) P.mul_small((uint32_t)pl.primes[k]);
    int used = 0;
    for (int k = 0; k < n; k++) {
        const int q = pl.primes[k];
        Big Mk(1);
        int64_t Mk_mod = 1;
        for (int j = 0; j < n; j++)
            if (j != k) {
                Mk.mul_small((uint32_t)pl.primes[j]);
                Mk_mod = Mk_mod * pl.primes[j] % q;
            }
        const int w = balanced(inv_mod(Mk_mod, q), q);
        const int64_t cfix = floor_div((int64_t)w * (INT64_C(1) << 32) + q, 2 * (int64_t)q);   // round(w 2^31 / q)
        c.chi[k] = (int32_t)(cfix >> 16);
        c.clo[k] = (int32_t)(cfix & 0xffff);
        int64_t rest = cfix;                          // |c_k| <= 2^30: four balanced digits
        for (int i = 0; i < 4; i++) {
            const int64_t dgt = ((rest % 256) + 256 + 128) % 256 - 128;
            c.cb[k] |= (uint32_t)(uint8_t)(int8_t)dgt << (8 * i);
            rest = (rest - dgt) / 256;
        }
        Big E = Mk;
        E.mul_small((uint32_t)(w < 0 ? -w : w));
        used = std::max(used, signed_digits(E, w < 0, d.d[k]));
    }
    used = std::max(used, signed_digits(P, false, d.d[n]));
    Big P256 = P;
    P256.mul_small(256u);
    used = std::max(used, signed_digits(P256, false, d.d[n + 1]));
    for (int i = 0; i < 16; i++) c.P[i] = i < (int)P.w.size() ? P.w[i] : 0u;
    *ksteps = (n + 2 + 31) / 32;
    *nblocks = (used + 31) / 32;
}

// ---- table cache ---------------------------------------------------------------
// The constant tables depend only on the plan's moduli (and, for the split,
// on the operand limb counts).  Building them costs tens of microseconds of
// host time (big-integer products for the CRT, modular powers for the
// split), as much as a whole small product on the GPU, so each host thread
// keeps the tables of its last few plans.
struct TableKey {
    int32_t n = 0, x0 = 0, x1 = 0;
    int32_t q[kMaxPrimes] = {};
    bool operator==(const TableKey &o) const {
        return n == o.n && x0 == o.x0 && x1 == o.x1 && std::memcmp(q, o.q, sizeof(int32_t) * n) == 0;
    }
};
TableKey table_key(const rns_plan_t &pl, int x0 = 0, int x1 = 0) {
    TableKey k;
    k.n = pl.n_primes;
    k.x0 = x0;
    k.x1 = x1;
    for (int i = 0; i < pl.n_primes; i++) k.q[i] = pl.primes[i];
    return k;
}
template <class V, int N = 8>
struct TableCache {
    TableKey key[N];
    V val[N];
    bool used[N] = {};
    int next = 0;
    template <class Build>
    const V &get(const TableKey &k, Build build) {
        for (int i = 0; i < N; i++)
            if (used[i] && key[i] == k) return val[i];
        const int i = next;
        next = (next + 1) % N;
        build(val[i]);
        key[i] = k;
        used[i] = true;
        return val[i];
    }
};
struct CrtTables {
    CrtConsts c;
    CrtDigits d;
    int ksteps, nblocks;
};
const SplitConsts &split_tables(const rns_plan_t &pl, int la, int lb) {
    static thread_local TableCache<SplitConsts> cache;
    return cache.get(table_key(pl, la, lb), [&](SplitConsts &v) { build_split(pl, la, lb, v); });
}
const EpiConsts &epi_tables(const rns_plan_t &pl) {
    static thread_local TableCache<EpiConsts> cache;
    return cache.get(table_key(pl), [&](EpiConsts &v) { build_epi(pl, v); });
}
const CrtTables &crt_tables(const rns_plan_t &pl) {
    static thread_local TableCache<CrtTables> cache;
    return cache.get(table_key(pl), [&](CrtTables &v) { build_crt(pl, v.c, v.d, &v.ksteps, &v.nblocks); });
}
// The fused lift step's constants: 256^b mod q (b < 8) balanced, c_1 mod q,
// and the reconstruction's fixed-point weights and P.
void build_step(const rns_plan_t &pl, const CrtConsts &c, StepConsts &v) {
    std::memset(&v, 0, sizeof v);
    v.n = pl.n_primes;
    for (int j = 0; j < pl.n_primes; j++) {
        const int q = pl.primes[j];
        int p = 1 % q, sum = 0;
        for (int b = 0; b < 8; b++) {
            const int bal = p > q / 2 ? p - q : p;
            v.tb[j][b >> 2] |= (uint32_t)(uint8_t)(int8_t)bal << (8 * (b & 3));
            if (b < 7) sum = (sum + p) % q;
            p = p * 256 % q;
        }
        v.q[j] = (uint16_t)q;
        v.c1[j] = (uint8_t)(128 * sum % q);
    }
    for (int k = 0; k < kCrtSlots; k++)
        for (int d = 0; d < 4; d++) {
            const int b = k & 15;
            v.fx[k >> 5][(k >> 4) & 1][d][b >> 2] |= ((c.cb[k] >> (8 * d)) & 0xffu) << (8 * (b & 3));
        }
    std::memcpy(v.P, c.P, sizeof v.P);
}
struct StepTables {
    StepConsts c;
    CrtDigits d;
    int ksteps, nblocks;
};
const StepTables &step_tables(const rns_plan_t &pl) {
    static thread_local TableCache<StepTables> cache;
    return cache.get(table_key(pl), [&](StepTables &v) {
        const CrtTables &ct = crt_tables(pl);
        build_step(pl, ct.c, v.c);
        v.d = ct.d;
        v.ksteps = ct.ksteps;
        v.nblocks = ct.nblocks;
    });
}
const GarnerConsts &garner_tables(const rns_plan_t &pl) {
    static thread_local TableCache<GarnerConsts, 4> cache;
    return cache.get(table_key(pl), [&](GarnerConsts &v) { build_garner(pl, v); });
}

// ---- layout ------------------------------------------------------------------
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// The 256 x 256 tiles run at well over twice the rate of the 64 x 64 ones per
// compute unit, so they win from half a round of tiles over the 256 units up
// (square 1024^3 with 10 primes: 160 tiles, products 26.7 -> 18.6 us).
int choose_tile(int n, int64_t M, int64_t N) {
    if (N <= 32) return kTileSkinny;
    const int64_t big_tiles = (int64_t)n * ((M + 255) / 256) * ((N + 255) / 256);
    if (M >= 256 && N >= 256 && big_tiles >= 128) return kTileBig;
    return kTileSmall;
}

// Row pitch of the product planes: at least `bytes`, a whole number of
// 128-byte lines, and an odd number of them, so that the same column of
// consecutive rows falls into different L2 channels (a power-of-two pitch
// sends a whole tile's rows to one channel).
int64_t plane_pitch(int64_t bytes) {
    int64_t p = round_up(bytes < 1 ? 1 : bytes, 128);
    if ((p / 128) % 2 == 0) p += 128;
    return p;
}

// Pitch of the operand residue planes: their bytes, plus 4 KiB when those
// are a multiple of 64 KiB, so that the same offset of consecutive planes
// does not fall into the same cache sets and memory channels.
int64_t operand_plane_pitch(int64_t bytes) {
    return bytes % 65536 == 0 ? bytes + 4096 : bytes;
}

struct Layout {
    rns_layout_t pub;
    int64_t status_slots;
    bool a_in_place;
    int64_t partial_off;   // split-tile residues (large tiling only, else -1)
};

Layout make_layout(const rns_plan_t &pl, int64_t M, int64_t N, int64_t K, bool batched) {
    Layout L{};
    const int n = pl.n_primes;
    const int cfg = choose_tile(n, M, N);
    const TileShape ts = tile_shape(cfg);
    L.pub.tile_config = cfg;
    L.pub.m_pad = round_up(M, ts.bm);
    L.pub.n_pad = round_up(N, ts.bn);
    L.pub.k_pad = round_up(K, ts.bk);
    L.pub.k_block = kKBlock;
    L.pub.y_pitch = plane_pitch(L.pub.n_pad);
    // the caller's residue planes ([n][M][K], pitch K) serve in place when
    // they already cover whole tiles
    L.a_in_place = batched && L.pub.m_pad == M && L.pub.k_pad == K;

    SplitOperand a{}, b{};
    a.r_pad = L.pub.m_pad; a.k_pad = L.pub.k_pad;
    b.r_pad = L.pub.n_pad; b.k_pad = L.pub.k_pad;
    L.status_slots = split_status_slots(batched ? nullptr : &a, &b, n);

    int64_t off = 0;
    auto take = [&](int64_t bytes) { int64_t o = off; off = round_up(off + bytes, 256); return o; };
    L.pub.status_off = take(L.status_slots * 4);
    L.pub.a_plane = L.a_in_place ? L.pub.m_pad * L.pub.k_pad : operand_plane_pitch(L.pub.m_pad * L.pub.k_pad);
    L.pub.b_plane = operand_plane_pitch(L.pub.n_pad * L.pub.k_pad);
    L.pub.a_off = L.a_in_place ? -1 : take((int64_t)n * L.pub.a_plane);
    L.pub.b_off = take((int64_t)n * L.pub.b_plane);
    L.pub.y_off = take((int64_t)n * L.pub.m_pad * L.pub.y_pitch);
    L.partial_off = cfg == kTileBig ? take(kTailUnitsMax * kTailUnitBytes) : -1;
    L.pub.total_bytes = off;
    return L;
}

int validate(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K) {
    if (!plan_ok(plan)) return RNS_E_ARG;
    if (M < 0 || N < 0 || K < 0) return RNS_E_ARG;
    if (K > RNS_K_MAX || K > plan->k_max) return RNS_E_K;
    // index arithmetic inside the kernels is 32-bit on padded row/column counts
    if (M > (1ll << 30) || N > (1ll << 30)) return RNS_E_ARG;
    return RNS_OK;
}

// Shape, pointer and size checks shared by the stage calls.  Returns the
// layout through *L when the call has work to do (rc == RNS_OK, *work = true).
int prepare(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K, bool batched,
            void *ws, size_t ws_bytes, Layout *L, bool *work) {
    *work = false;
    int rc = validate(plan, M, N, K);
    if (rc) return rc;
    if (M == 0 || N == 0 || K == 0) return RNS_OK;
    if (!ws) return RNS_E_ARG;
    *L = make_layout(*plan, M, N, K, batched);
    if (ws_bytes < (size_t)L->pub.total_bytes) return RNS_E_WORKSPACE;
    *work = true;
    return RNS_OK;
}

int stage_split(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                const int64_t *A, int32_t a_limbs, const int64_t *B, int32_t b_limbs,
                void *ws, size_t ws_bytes, hipStream_t stream, const Fp64Scales *fp = nullptr) {
    const bool batched = A == nullptr;
    if (!batched && (a_limbs < 1 || a_limbs > RNS_MAX_IN_LIMBS)) return RNS_E_ARG;
    if (b_limbs < 1 || b_limbs > RNS_MAX_IN_LIMBS) return RNS_E_ARG;
    Layout L;
    bool work;
    int rc = prepare(plan, M, N, K, batched, ws, ws_bytes, &L, &work);
    if (rc || !work) return rc;
    if (!B) return RNS_E_ARG;
    int8_t *base = (int8_t *)ws;
    const SplitConsts &sc = split_tables(*plan, batched ? 1 : a_limbs, b_limbs);
    SplitOperand sa{}, sb{};
    if (!batched) {
        sa.x = A; sa.planes = base + L.pub.a_off; sa.plane = L.pub.a_plane; sa.rows = M; sa.k = K;
        sa.r_pad = L.pub.m_pad; sa.k_pad = L.pub.k_pad; sa.limbs = a_limbs;
        sa.bits = (plan->a_bits >= 0 && plan->a_bits < 64 * a_limbs - 1) ? plan->a_bits : -1;
        sa.transposed = 0;
        if (fp) { sa.fp64 = 1; sa.scale = fp->fa; }
    }
    sb.x = B; sb.planes = base + L.pub.b_off; sb.plane = L.pub.b_plane; sb.rows = N; sb.k = K;
    sb.r_pad = L.pub.n_pad; sb.k_pad = L.pub.k_pad; sb.limbs = b_limbs;
    sb.bits = (plan->b_bits >= 0 && plan->b_bits < 64 * b_limbs - 1) ? plan->b_bits : -1;
    sb.transposed = 1;
    if (fp) {
        sb.fp64 = 1;
        sb.scale = fp->fb;
        if (fp->b_rows_n) sb.transposed = 0;   // B^T [N][K]: plane rows are its rows
    }
    return launch_split(batched ? nullptr : &sa, &sb, sc, (uint32_t *)(base + L.pub.status_off),
                        L.status_slots, stream);
}

int stage_products(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K, const int8_t *A_res,
                   void *ws, size_t ws_bytes, hipStream_t stream) {
    const bool batched = A_res != nullptr;
    Layout L;
    bool work;
    int rc = prepare(plan, M, N, K, batched, ws, ws_bytes, &L, &work);
    if (rc || !work) return rc;
    int8_t *base = (int8_t *)ws;
    const int n = plan->n_primes;
    const int8_t *apl = base + L.pub.a_off;
    int64_t a_row = kKBlock, a_kstep = L.pub.m_pad * kKBlock;   // K-blocked planes
    if (batched) {
        if (L.a_in_place) {
            apl = A_res;                      // the caller's row-major [n][M][K]
            a_row = K;
            a_kstep = kKBlock;
        } else {
            rc = launch_repack_residues(A_res, n, M, K, base + L.pub.a_off, L.pub.m_pad,
                                        L.pub.k_pad, L.pub.a_plane, stream);
            if (rc) return rc;
        }
    }
    const EpiConsts &ec = epi_tables(*plan);
    return launch_gemm(L.pub.tile_config, n, apl, base + L.pub.b_off, base + L.pub.y_off,
                       L.pub.m_pad, L.pub.n_pad, L.pub.k_pad, L.pub.a_plane,
                       L.pub.b_plane, L.pub.m_pad * L.pub.y_pitch,
                       a_row, a_kstep, kKBlock, L.pub.n_pad * kKBlock, L.pub.y_pitch,
                       L.partial_off >= 0 ? base + L.partial_off : nullptr, ec, stream);
}

enum Recon { kReconCrt = 0, kReconGarner = 1 };

int stage_reconstruct(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K, bool batched,
                      int64_t *C, int32_t c_limbs, void *ws, size_t ws_bytes, hipStream_t stream,
                      int method = kReconCrt) {
    int rc = validate(plan, M, N, K);
    if (rc) return rc;
    if (c_limbs < plan->out_limbs_min || c_limbs > RNS_MAX_OUT_LIMBS) return RNS_E_OUT_LIMBS;
    if (M == 0 || N == 0) return RNS_OK;
    if (!C) return RNS_E_ARG;
    if (K == 0) return launch_zero(C, M * N * c_limbs, stream);
    Layout L;
    bool work;
    rc = prepare(plan, M, N, K, batched, ws, ws_bytes, &L, &work);
    if (rc || !work) return rc;
    if (method == kReconGarner) {
        const GarnerConsts &gc = garner_tables(*plan);
        return launch_garner(gc, (const int8_t *)ws + L.pub.y_off, L.pub.m_pad * L.pub.y_pitch,
                             L.pub.y_pitch, M, N, C, c_limbs, stream);
    }
    const CrtTables &ct = crt_tables(*plan);
    return launch_crt(ct.c, ct.d, ct.ksteps, ct.nblocks, (const int8_t *)ws + L.pub.y_off,
                      L.pub.m_pad * L.pub.y_pitch, L.pub.y_pitch, M, N, C, c_limbs, stream);
}

// Full product: every argument is checked before the first launch.
int run(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
        const int64_t *A, int32_t a_limbs, const int8_t *A_res,
        const int64_t *B, int32_t b_limbs, int64_t *C, int32_t c_limbs,
        void *ws, size_t ws_bytes, hipStream_t stream, const Fp64Scales *fp = nullptr) {
    const bool batched = A_res != nullptr;
    int rc = validate(plan, M, N, K);
    if (rc) return rc;
    if (!batched && (a_limbs < 1 || a_limbs > RNS_MAX_IN_LIMBS)) return RNS_E_ARG;
    if (b_limbs < 1 || b_limbs > RNS_MAX_IN_LIMBS) return RNS_E_ARG;
    if (c_limbs < plan->out_limbs_min || c_limbs > RNS_MAX_OUT_LIMBS) return RNS_E_OUT_LIMBS;
    if (M == 0 || N == 0) return RNS_OK;
    if (!C) return RNS_E_ARG;
    // K == 0: the operands are empty (their pointers may be null); C = 0
    if (K == 0) return launch_zero(C, M * N * c_limbs, stream);
    if (!B || (!batched && !A) || !ws) return RNS_E_ARG;
    const Layout L = make_layout(*plan, M, N, K, batched);
    if (ws_bytes < (size_t)L.pub.total_bytes) return RNS_E_WORKSPACE;
    if (batched && b_limbs == 1 && N <= 16 && K >= 16 && K % 16 == 0 && K <= RNS_LIFT_K_MAX &&
        (plan->b_bits < 0 || plan->b_bits >= 63) && reinterpret_cast<uintptr_t>(A_res) % 16 == 0) {
        // skinny right-hand side without a bound to check: one kernel
        const StepTables &lt = step_tables(*plan);
        return launch_lift_step(lt.c, lt.d, lt.ksteps, lt.nblocks, A_res, B, M, N, K, C, c_limbs,
                                reinterpret_cast<uint32_t *>((int8_t *)ws + L.pub.status_off), stream);
    }
    rc = stage_split(plan, M, N, K, batched ? nullptr : A, a_limbs, B, b_limbs, ws, ws_bytes, stream, fp);
    if (rc) return rc;
    rc = stage_products(plan, M, N, K, A_res, ws, ws_bytes, stream);
    if (rc) return rc;
    return stage_reconstruct(plan, M, N, K, batched, C, c_limbs, ws, ws_bytes, stream);
}

}  // namespace

int plan_from_moduli(const int32_t *moduli, int n, int64_t k_max, rns_plan_t *out) {
    rns_plan_t pl{};
    Big P(1);
    double l2 = 0;
    for (int i = 0; i < n; i++) {
        if (moduli[i] < 2 || moduli[i] > 256) return RNS_E_ARG;
        pl.primes[i] = moduli[i];
        P.mul_small((uint32_t)moduli[i]);
        l2 += std::log2((double)moduli[i]);
    }
    pl.n_primes = n;
    pl.log2_P = l2;
    pl.out_limbs_min = (P.bit_length() + 63) / 64;
    pl.a_bits = -1;
    pl.b_bits = -1;
    pl.k_max = k_max;
    if (!plan_ok(&pl)) return RNS_E_ARG;
    *out = pl;
    return RNS_OK;
}

int gemm_fp64_scaled(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                     const double *A, int32_t a_limbs, const double *B, int32_t b_limbs,
                     const Fp64Scales &scales, int64_t *C, int32_t c_limbs,
                     void *ws, size_t ws_bytes, hipStream_t stream) {
    // the split reads each binary64 operand as one 64-bit word per entry
    return run(plan, M, N, K, reinterpret_cast<const int64_t *>(A), a_limbs, nullptr,
               reinterpret_cast<const int64_t *>(B), b_limbs, C, c_limbs, ws, ws_bytes, stream, &scales);
}

}  // namespace rns

using namespace rns;

extern "C" {

int rns_plan_moduli(int64_t K, int32_t a_bits, int32_t b_bits, int32_t kind, rns_plan_t *out) {
    if (!out || (kind != RNS_MODULI_PRIMES && kind != RNS_MODULI_PRIME_POWERS)) return RNS_E_ARG;
    if (a_bits < 0 || b_bits < 0 || a_bits > 255 || b_bits > 255) return RNS_E_ARG;
    const int64_t kmax = kind == RNS_MODULI_PRIME_POWERS ? RNS_K_MAX - 1 : RNS_K_MAX;
    if (K < 0 || K > kmax) return RNS_E_K;
    const int64_t Kb = K < 1 ? 1 : K;
    Big bound((uint64_t)Kb);
    bound.shl(a_bits + b_bits + 1);          // 2 * K * 2^(a+b)
    Big P(1);
    for (int n = 1; n <= kMaxPrimes; n++) {
        P.mul_small((uint32_t)moduli(kind).p[n - 1]);
        if (Big::greater(P, bound)) {
            fill_common(out, n, kind);
            out->a_bits = a_bits;
            out->b_bits = b_bits;
            out->k_max = Kb;
            return RNS_OK;
        }
    }
    return RNS_E_CAPACITY;
}

int rns_probe_int8_mfma(const void *src, size_t src_bytes, int32_t workgroups, int32_t iters, int32_t *out,
                        hipStream_t stream) {
    if (!src || !out || workgroups < 1 || workgroups > (1 << 20) || iters < 1) return RNS_E_ARG;
    if (src_bytes < (size_t)workgroups * 256 * 128 || reinterpret_cast<uintptr_t>(src) % 16) return RNS_E_ARG;
    return launch_mfma_probe((const int8_t *)src, workgroups, iters, out, stream);
}

int rns_plan(int64_t K, int32_t a_bits, int32_t b_bits, rns_plan_t *out) {
    return rns_plan_moduli(K, a_bits, b_bits, RNS_MODULI_PRIMES, out);
}

int rns_plan_n_moduli(int32_t n, int32_t kind, rns_plan_t *out) {
    if (!out || n < 1 || n > kMaxPrimes || (kind != RNS_MODULI_PRIMES && kind != RNS_MODULI_PRIME_POWERS))
        return RNS_E_ARG;
    fill_common(out, n, kind);
    out->a_bits = -1;
    out->b_bits = -1;
    out->k_max = kind == RNS_MODULI_PRIME_POWERS ? RNS_K_MAX - 1 : RNS_K_MAX;
    return RNS_OK;
}

int rns_plan_n(int32_t n_primes, rns_plan_t *out) {
    return rns_plan_n_moduli(n_primes, RNS_MODULI_PRIMES, out);
}

int rns_workspace_layout(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                         int32_t batched_residue, rns_layout_t *out) {
    if (!out) return RNS_E_ARG;
    int rc = validate(plan, M, N, K);
    if (rc) return rc;
    *out = make_layout(*plan, M, N, K, batched_residue != 0).pub;
    return RNS_OK;
}

int rns_workspace_size(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                       int32_t batched_residue, size_t *bytes) {
    if (!bytes) return RNS_E_ARG;
    rns_layout_t l;
    int rc = rns_workspace_layout(plan, M, N, K, batched_residue, &l);
    if (rc) return rc;
    *bytes = (size_t)l.total_bytes;
    return RNS_OK;
}

int rns_gemm(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
             const int64_t *A, int32_t a_limbs, const int64_t *B, int32_t b_limbs,
             int64_t *C, int32_t c_limbs, void *ws, size_t ws_bytes, hipStream_t stream) {
    return run(plan, M, N, K, A, a_limbs, nullptr, B, b_limbs, C, c_limbs, ws, ws_bytes, stream);
}

int rns_gemm_batched_residue(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                             const int8_t *A_res, const int64_t *B, int32_t b_limbs,
                             int64_t *C, int32_t c_limbs, void *ws, size_t ws_bytes,
                             hipStream_t stream) {
    if (!A_res && M > 0 && N > 0 && K > 0) return RNS_E_ARG;
    if (!A_res) {
        // nothing to read: validate and handle the degenerate sizes only
        int rc = validate(plan, M, N, K);
        if (rc) return rc;
        if (b_limbs < 1 || b_limbs > RNS_MAX_IN_LIMBS) return RNS_E_ARG;
        if (c_limbs < plan->out_limbs_min || c_limbs > RNS_MAX_OUT_LIMBS) return RNS_E_OUT_LIMBS;
        if (M == 0 || N == 0) return RNS_OK;
        if (!C) return RNS_E_ARG;
        return launch_zero(C, M * N * c_limbs, stream);
    }
    return run(plan, M, N, K, nullptr, 1, A_res, B, b_limbs, C, c_limbs, ws, ws_bytes, stream);
}

int rns_split(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
              const int64_t *A, int32_t a_limbs, const int64_t *B, int32_t b_limbs,
              void *ws, size_t ws_bytes, hipStream_t stream) {
    return stage_split(plan, M, N, K, A, a_limbs, B, b_limbs, ws, ws_bytes, stream);
}

int rns_residue_products(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                         const int8_t *A_res, void *ws, size_t ws_bytes, hipStream_t stream) {
    return stage_products(plan, M, N, K, A_res, ws, ws_bytes, stream);
}

int rns_reconstruct(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                    int32_t batched_residue, int64_t *C, int32_t c_limbs,
                    void *ws, size_t ws_bytes, hipStream_t stream) {
    return stage_reconstruct(plan, M, N, K, batched_residue != 0, C, c_limbs, ws, ws_bytes, stream);
}

int rns_reconstruct_garner(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                           int32_t batched_residue, int64_t *C, int32_t c_limbs,
                           void *ws, size_t ws_bytes, hipStream_t stream) {
    return stage_reconstruct(plan, M, N, K, batched_residue != 0, C, c_limbs, ws, ws_bytes, stream,
                             kReconGarner);
}

int rns_status(const void *ws, hipStream_t stream, uint32_t *flags) {
    if (!ws || !flags) return RNS_E_ARG;
    if (hipStreamSynchronize(stream) != hipSuccess) return RNS_E_HIP;
    uint32_t head[kStatusHeader] = {0, 0};
    if (hipMemcpy(head, ws, sizeof(head), hipMemcpyDeviceToHost) != hipSuccess) return RNS_E_HIP;
    const uint32_t nblocks = head[0];
    // a workspace that no completed call has written fails the check word
    if ((head[0] ^ kStatusCheck) != head[1] || nblocks > (1u << 30)) return RNS_E_ARG;
    std::vector<uint32_t> words(nblocks);
    if (nblocks && hipMemcpy(words.data(), (const uint32_t *)ws + kStatusHeader,
                             4 * (size_t)nblocks, hipMemcpyDeviceToHost) != hipSuccess)
        return RNS_E_HIP;
    uint32_t f = 0;
    for (uint32_t w : words) f |= w;
    *flags = f;
    return RNS_OK;
}

const char *rns_error_string(int code) {
    switch (code) {
        case RNS_OK: return "success";
        case RNS_E_ARG: return "invalid argument";
        case RNS_E_K: return "K exceeds 2^17 or the plan's K";
        case RNS_E_CAPACITY: return "bound exceeds the product of the primes below 256";
        case RNS_E_OUT_LIMBS: return "too few (or too many) output limbs";
        case RNS_E_WORKSPACE: return "workspace too small";
        case RNS_E_HIP: return "HIP launch or copy failed";
        case -7: return "non-finite operand";
        case -8: return "no fraction within the bounds matches the residue";
        case -9: return "the host big-integer library (libgmp.so.10) is not available";
        case RNS_E_SCRATCH: return "workspace exceeds the fixed scratch array of rns_gemm_noalloc";
        default: return "unknown error code";
    }
}

}  // extern "C"
