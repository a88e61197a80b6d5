// tables.cpp -- host-side number theory for Ozaki Scheme II.
//
// [Q] = Qiita article "8ビットの整数で53ビットの倍精度を組み立てる。中国剰余定理を
// GPUに載せたOzaki Scheme II"; [G] = "Improved Scaling for Fast Mode of Ozaki
// Scheme II" (technical summary).
//
// Everything here runs once per number of moduli N and is cached. Exact
// integers up to 256 bits are held in a fixed array of 32-bit limbs.
#include "tables.h"

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

namespace oz2 {
namespace {

// Unsigned 256-bit integer, little-endian 32-bit limbs.
struct U256 {
    uint32_t d[8] = {};

    static U256 from(uint64_t v) {
        U256 r;
        r.d[0] = (uint32_t)v;
        r.d[1] = (uint32_t)(v >> 32);
        return r;
    }
    bool is_zero() const {
        for (uint32_t x : d)
            if (x) return false;
        return true;
    }
    U256 mul_small(uint32_t f) const {
        U256 r;
        uint64_t carry = 0;
        for (int i = 0; i < 8; ++i) {
            uint64_t t = (uint64_t)d[i] * f + carry;
            r.d[i] = (uint32_t)t;
            carry = t >> 32;
        }
        return r;  // callers stay below 2^256
    }
    // *this / f, remainder in *rem
    U256 div_small(uint32_t f, uint32_t *rem) const {
        U256 q;
        uint64_t r = 0;
        for (int i = 7; i >= 0; --i) {
            uint64_t cur = (r << 32) | d[i];
            q.d[i] = (uint32_t)(cur / f);
            r = cur % f;
        }
        if (rem) *rem = (uint32_t)r;
        return q;
    }
    uint32_t mod_small(uint32_t f) const {
        uint32_t r;
        div_small(f, &r);
        return r;
    }
    U256 add_small(uint32_t a) const {
        U256 r = *this;
        uint64_t carry = a;
        for (int i = 0; i < 8 && carry; ++i) {
            uint64_t t = (uint64_t)r.d[i] + carry;
            r.d[i] = (uint32_t)t;
            carry = t >> 32;
        }
        return r;
    }
    U256 sub_one() const {  // *this - 1, *this > 0
        U256 r = *this;
        for (int i = 0; i < 8; ++i) {
            if (r.d[i]--) break;
        }
        return r;
    }
    int bit_length() const {
        for (int i = 7; i >= 0; --i)
            if (d[i]) return 32 * i + 32 - __builtin_clz(d[i]);
        return 0;
    }
    // bits [lo, lo + cnt) as an integer, cnt <= 64
    uint64_t bits(int lo, int cnt) const {
        uint64_t v = 0;
        for (int b = cnt - 1; b >= 0; --b) {
            int pos = lo + b;
            uint64_t bit = pos < 256 ? (d[pos / 32] >> (pos % 32)) & 1u : 0u;
            v = (v << 1) | bit;
        }
        return v;
    }
};

int gcd_int(int a, int b) {
    while (b) {
        int t = a % b;
        a = b;
        b = t;
    }
    return a;
}

// x^-1 mod p by the extended Euclidean algorithm (the procedure [Q] section
// 秦九韶の大衍求一術 describes as Qin Jiushao's 大衍求一術).
int64_t inverse_mod(int64_t x, int64_t p) {
    int64_t r0 = p, r1 = x % p, s0 = 0, s1 = 1;
    while (r1 != 0) {
        int64_t q = r0 / r1;
        int64_t r2 = r0 - q * r1;
        r0 = r1;
        r1 = r2;
        int64_t s2 = s0 - q * s1;
        s0 = s1;
        s1 = s2;
    }
    // r0 == gcd == 1 and s0 * x == 1 mod p
    int64_t v = s0 % p;
    return v < 0 ? v + p : v;
}

// The 40-bit pieces of v as doubles (exact).
void chunks40(const U256 &v, double *out) {
    for (int t = 0; t < kChunks; ++t) out[t] = (double)v.bits(kChunkBits * t, kChunkBits);
}

// P'_prop = 0.5 * log2((P-1)/2) rounded down to a double ([G] section Methodik,
// the constant of the proposed exponent). log2 of the integer is taken from its
// bit length plus log2 of its leading 64 bits in extended precision.
// (P is even, so (P-1)/2 is not an integer: use log2(P-1) - 1.)
double scaling_constant(const U256 &P) {
    U256 q = P.sub_one();
    int L = q.bit_length();
    int shift = L > 64 ? L - 64 : 0;
    uint64_t top = q.bits(shift, 64);
    long double lg = (long double)shift + log2l((long double)top) - 1.0L;
    long double half = lg * 0.5L;
    double d = (double)half;
    if ((long double)d > half) d = std::nextafter(d, -INFINITY);
    return d;
}

void build(Tables &t, int n) {
    t.n = n;
    greedy_moduli(n, t.moduli);
    U256 P = U256::from(1);
    for (int l = 0; l < n; ++l) P = P.mul_small((uint32_t)t.moduli[l]);

    t.Pp = scaling_constant(P);

    // split constants: p, 1/p and 2^42 mod p (symmetric)
    t.split.n = n;
    for (int l = 0; l < n; ++l) {
        int p = t.moduli[l];
        t.split.p[l] = (double)p;
        t.split.pinv[l] = 1.0 / (double)p;
        int64_t c = 1;
        for (int b = 0; b < 42; ++b) c = (c * 2) % p;
        if (c > (p - 1) / 2) c -= p;
        t.split.c42[l] = (double)c;
        t.mod.p[l] = (double)p;
        t.mod.pinv[l] = 1.0 / (double)p;
    }

    // CRT weights ([Q] section 秦九韶の大衍求一術): M_l = P / p_l (衍数),
    // G_l = M_l mod p_l (奇数), K_l = G_l^-1 mod p_l (乗率), W_l = M_l K_l (用数).
    t.crt.n = n;
    int limbs = (P.bit_length() + 31) / 32;
    t.weight_limbs = limbs;
    for (int l = 0; l < n; ++l) {
        uint32_t r;
        U256 M = P.div_small((uint32_t)t.moduli[l], &r);
        uint32_t G = M.mod_small((uint32_t)t.moduli[l]);
        uint32_t K = (uint32_t)inverse_mod(G, t.moduli[l]);
        U256 W = M.mul_small(K);
        std::memcpy(t.weight[l], W.d, sizeof(W.d));
        chunks40(W, t.crt.w[l]);
        // signed base-256 digits, least significant first: X = sum_v d_v 256^v,
        // d_v in [-128, 127]; returns the digit count
        auto digits = [](U256 rest, int8_t *out, int stride, int max_digits) {
            int v = 0;
            for (; !rest.is_zero(); ++v) {
                if (v >= max_digits) std::abort();  // cannot happen for P < 2^159
                uint32_t low = rest.d[0] & 0xffu;
                int d = low >= 128 ? (int)low - 256 : (int)low;
                rest = rest.div_small(256, nullptr);
                if (d < 0) rest = rest.add_small(1);
                out[v * stride] = (int8_t)d;
            }
            return v;
        };
        const int nd = digits(W, &t.crt.digit[0][l], 32, kMaxDigits);
        if (nd > t.crt.nd) t.crt.nd = nd;
        // P - W_l = M_l (p_l - K_l), congruent to -W_l mod P: its digits stand
        // in for a negative weight in the complex reconstruction
        const int nnd = digits(M.mul_small((uint32_t)t.moduli[l] - K), &t.crt.ndigit[0][l], 32, kMaxDigits);
        if (nnd > t.crt.nnd) t.crt.nnd = nnd;
    }
    chunks40(P, t.crt.P);
    U256 H = P.div_small(2, nullptr);
    chunks40(H, t.crt.H);
    // RN(2^120 / P): P as a long double is exact to 64 bits, far more than needed.
    long double Pld = 0.0L;
    for (int i = 7; i >= 0; --i) Pld = Pld * 4294967296.0L + (long double)P.d[i];
    t.crt.pinv120 = (double)(ldexpl(1.0L, 120) / Pld);
    t.crt.pinv128 = (double)(ldexpl(1.0L, 128) / Pld);
    t.crt.pinv96 = (double)(ldexpl(1.0L, 96) / Pld);
    t.crt.pinv64 = (double)(ldexpl(1.0L, 64) / Pld);
    t.crt.pinv32 = (double)(ldexpl(1.0L, 32) / Pld);
    {
        const int by_digits = (t.crt.nd + 3) / 4, by_p = (P.bit_length() + 31) / 32;
        t.crt.np32 = by_digits > by_p ? by_digits : by_p;
        if (t.crt.np32 < 2) t.crt.np32 = 2;
    }
    for (int c = 0; c < kChunks32; ++c) {  // 32-bit pieces (P < 2^160)
        t.crt.P32[c] = (double)P.d[c];
        t.crt.H32[c] = (double)H.d[c];
    }

    // check against the next modulus of the table ([Q] section
    // 時計の針で見る定理の中身: an integer outside (-P/2, P/2] comes back as
    // another one; one more clock tells the two apart)
    if (n < kMaxModuli) {
        int32_t next[kMaxModuli];
        greedy_moduli(n + 1, next);
        const int pc = next[n];
        t.check.n = n;
        t.check.pc = pc;
        t.check.pm = (int)P.mod_small((uint32_t)pc);
        for (int l = 0; l < n; ++l) {
            U256 W;
            std::memcpy(W.d, t.weight[l], sizeof(W.d));
            t.check.wm[l] = (int)W.mod_small((uint32_t)pc);
            uint32_t r;
            const U256 M = P.div_small((uint32_t)t.moduli[l], &r);
            const int64_t K = inverse_mod(M.mod_small((uint32_t)t.moduli[l]), t.moduli[l]);
            t.check.kp[l] = (double)K / (double)t.moduli[l];
        }
    }
}

std::mutex g_mu;
Tables g_tables[kMaxModuli + 1];
bool g_built[kMaxModuli + 1];

}  // namespace

bool greedy_moduli(int n, int32_t *out) {
    if (n < 1 || n > kMaxModuli) return false;
    int cnt = 0;
    for (int x = 256; x >= 2 && cnt < n; --x) {
        bool ok = true;
        for (int i = 0; i < cnt; ++i)
            if (gcd_int(x, out[i]) != 1) {
                ok = false;
                break;
            }
        if (ok) out[cnt++] = x;
    }
    return cnt == n;
}

const Tables *get_tables(int n) {
    if (n < 2 || n > kMaxModuli) return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_built[n]) {
        build(g_tables[n], n);
        g_built[n] = true;
    }
    return &g_tables[n];
}

}  // namespace oz2
