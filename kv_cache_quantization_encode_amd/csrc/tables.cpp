// Host-side construction of the codec tables (pure C++, no HIP).
//
//  - Lloyd-Max levels/boundaries of N(0,1) for 1..4 bits, float64
//    (quidproquo.cc, "TurboQuant+ KV cache compression", Stage 1: the optimal
//    Gaussian codebook is precomputed with Lloyd's algorithm).
//  - Random sign diagonal D and Gaussian QJL matrix S from one seed
//    (chenxutan.com, "TurboQuant+ deep dive", 2.3: a fixed-seed matrix shared
//    by encoder and decoder).  Generator: splitmix64 in counter form
//    (Steele, Lea & Flood, 2014): state_i = seed + i * 0x9E3779B97F4A7C15,
//    output = two xor-shift-multiply rounds.  Counters 1..d give the signs
//    (top bit set -> -1); counters d+1.. feed Box-Muller (1958) in pairs,
//    filling S row-major; each draw is rounded to fp16 (round to nearest even).
//  - Device-friendly rearrangements of S for the MFMA fragments.
#include "internal.h"

#include <cmath>
#include <cstring>

namespace tq {

static uint64_t splitmix64_at(uint64_t seed, uint64_t counter) {
    uint64_t z = seed + counter * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// IEEE binary64 -> binary16, round to nearest, ties to even, computed from the
// bit pattern so that no intermediate float32 rounding takes place.
uint16_t double_to_half_rne(double v) {
    uint64_t b;
    std::memcpy(&b, &v, 8);
    const uint16_t sign = uint16_t((b >> 48) & 0x8000u);
    const int exp = int((b >> 52) & 0x7FF);
    const uint64_t frac = b & ((1ull << 52) - 1);
    if (exp == 0x7FF) return uint16_t(sign | 0x7C00u | (frac ? 0x200u : 0u));
    if (exp == 0) return sign;  // double subnormals are far below half's range
    const int e = exp - 1023;
    const uint64_t m = (1ull << 52) | frac;  // 53 significant bits
    if (e > 15) return uint16_t(sign | 0x7C00u);
    if (e >= -14) {
        uint64_t hm = m >> 42;
        const uint64_t rem = m & ((1ull << 42) - 1), half = 1ull << 41;
        if (rem > half || (rem == half && (hm & 1))) ++hm;
        int he = e + 15;
        if (hm == (1ull << 11)) { hm >>= 1; ++he; }
        if (he >= 31) return uint16_t(sign | 0x7C00u);
        return uint16_t(sign | (he << 10) | (hm & 0x3FF));
    }
    // half subnormal: units of 2^-24
    const int shift = 28 - e;  // value = m * 2^(e-52) = (m >> shift) units
    if (shift > 53) return sign;
    uint64_t hm = m >> shift;
    const uint64_t rem = m & ((1ull << shift) - 1), half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (hm & 1))) ++hm;
    return uint16_t(sign | hm);
}

double half_to_double(uint16_t h) {
    const int s = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x3FF;
    double v;
    if (e == 0) v = std::ldexp(double(f), -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = std::ldexp(double(f | 0x400), e - 25);
    return s ? -v : v;
}

// Standard normal density and the probability of (lo, hi), taking the upper
// tail where both ends are non-negative so that no precision is lost there.
static double npdf(double t) {
    if (std::isinf(t)) return 0.0;
    return std::exp(-0.5 * t * t) * 0.39894228040143267794;
}
static double upper_tail(double t) {  // P(Z > t)
    if (t == INFINITY) return 0.0;
    if (t == -INFINITY) return 1.0;
    return 0.5 * std::erfc(t * 0.70710678118654752440);
}
static double cell_mass(double lo, double hi) {
    if (lo >= 0.0) return upper_tail(lo) - upper_tail(hi);
    return upper_tail(-hi) - upper_tail(-lo);  // P(lo<Z<hi) = P(-hi<Z<-lo)
}

void lloyd_max_gaussian(int bits, double *levels, double *bounds) {
    const int L = 1 << bits;
    double c[16], nc[16], t[15];
    // start from evenly spaced levels over [-2, 2]; Lloyd's fixed point for a
    // log-concave density is unique, so the start only sets the iteration count
    for (int k = 0; k < L; ++k) c[k] = -2.0 + 4.0 * (k + 0.5) / L;
    for (int it = 0; it < 1000000; ++it) {
        for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
        for (int k = 0; k < L; ++k) {
            const double lo = k == 0 ? -INFINITY : t[k - 1];
            const double hi = k == L - 1 ? INFINITY : t[k];
            nc[k] = (npdf(lo) - npdf(hi)) / cell_mass(lo, hi);
        }
        double delta = 0.0;
        for (int k = 0; k < L; ++k) {
            const double sym = 0.5 * (nc[k] - nc[L - 1 - k]);
            delta = std::fmax(delta, std::fabs(sym - c[k]));
            c[k] = sym;
        }
        if (delta < 1e-14) break;
    }
    for (int k = 0; k < L; ++k) levels[k] = c[k];
    for (int k = 0; k + 1 < L; ++k) bounds[k] = 0.5 * (c[k] + c[k + 1]);
}

void random_tables(int d, int m, uint64_t seed, float *signs, uint16_t *S) {
    for (int i = 0; i < d; ++i) {
        const uint64_t w = splitmix64_at(seed, uint64_t(i) + 1);
        signs[i] = (w >> 63) ? -1.0f : 1.0f;
    }
    const double two_pi = 6.28318530717958647692;
    const int n = m * d;
    for (int j = 0; j < n / 2; ++j) {
        const uint64_t w1 = splitmix64_at(seed, uint64_t(d) + 1 + 2 * uint64_t(j));
        const uint64_t w2 = splitmix64_at(seed, uint64_t(d) + 2 + 2 * uint64_t(j));
        const double u1 = (double(w1 >> 11) + 0.5) * 0x1.0p-53;
        const double u2 = double(w2 >> 11) * 0x1.0p-53;
        const double r = std::sqrt(-2.0 * std::log(u1));
        S[2 * j] = double_to_half_rne(r * std::cos(two_pi * u2));
        S[2 * j + 1] = double_to_half_rne(r * std::sin(two_pi * u2));
    }
}

bool build_device_tables(int d, int m, uint64_t seed, DevTables *t) {
    std::memset(t, 0, sizeof(DevTables));
    for (int b = 1; b <= 4; ++b) {
        double lv[16], bd[15];
        lloyd_max_gaussian(b, lv, bd);
        for (int k = 0; k < (1 << b); ++k) t->levels[b - 1][k] = float(lv[k]);
        for (int k = 0; k + 1 < (1 << b); ++k) t->bounds[b - 1][k] = float(bd[k]);
        for (int k = (1 << b) - 1; k < 16; ++k) t->bounds[b - 1][k] = INFINITY;
    }
    random_tables(d, m, seed, t->signs, t->S);
    for (int r = 0; r < m; ++r)
        for (int c = 0; c < d; ++c) t->ST[c * m + r] = t->S[r * d + c];
    // xor masks that flip the sign bits of packed fp16 pairs in the encoder's
    // load layout: lane quarter q holds coordinates 8q + (r&7) + 32(r>>3) in
    // register r, pair p = registers 2p, 2p+1
    for (int q = 0; q < 4; ++q)
        for (int p = 0; p < 16; ++p) {
            const int c0 = 8 * q + ((2 * p) & 7) + 32 * ((2 * p) >> 3);
            uint32_t msk = 0;
            if (t->signs[c0] < 0) msk |= 0x8000u;
            if (t->signs[c0 + 1] < 0) msk |= 0x80000000u;
            t->sign_pair_xor[q][p] = msk;
        }
    // Quantiser buckets: bucket j (0..96) is [-12.125 + 0.25 j, -11.875 + 0.25 j),
    // the outer two open-ended.  Every Lloyd-Max boundary of 1..4 bits lies at
    // least 0.02 from an edge and no bucket holds two boundaries, so
    // idx = base_j + (z >= thr_j) even when rounding moves a z next to an edge
    // into the neighbouring bucket.
    for (int b = 1; b <= 4; ++b) {
        double lv[16], bd[15];
        lloyd_max_gaussian(b, lv, bd);
        const int L = 1 << b;
        for (int j = 0; j < kBuckets; ++j) {
            QBucket qb{INFINITY, 0u, 0.0f, 0.0f};
            const double lo = j == 0 ? -INFINITY : -12.125 + 0.25 * j;
            const double hi = j == kBuckets - 1 ? INFINITY : -11.875 + 0.25 * j;
            int base = 0, inside = 0;
            double thr = INFINITY;
            for (int k = 0; k + 1 < L; ++k) {
                if (bd[k] < lo) ++base;
                else if (bd[k] < hi) { ++inside; thr = bd[k]; }
            }
            if (inside > 1) return false;  // cannot happen for these codebooks
            qb.thr = float(thr);
            qb.base = uint32_t(base);
            qb.c_lo = float(lv[base]);
            qb.c_hi = float(lv[base + 1 < L ? base + 1 : base]);
            t->qlut[b - 1][j] = qb;
        }
    }
    // Encode QJL fragments (A operand of a 16x16x32 MFMA, rows = projections).
    // Fragment f = mb*4 + s; lane l = 16*q + i supplies the eight fp16 values
    //   S[32*(i/4) + 4*mb + i%4][32*q + 8*s + j],  j = 0..7,
    // so that output row 4*q + j' of block mb is projection 32*q + 4*mb + j'.
    for (int mb = 0; mb < 8; ++mb)
        for (int s = 0; s < 4; ++s)
            for (int l = 0; l < 64; ++l) {
                const int i = l & 15, q = l >> 4;
                const int row = 32 * (i >> 2) + 4 * mb + (i & 3);
                for (int j = 0; j < 8; ++j)
                    t->S_enc[((mb * 4 + s) * 64 + l) * 8 + j] = t->S[row * d + 32 * q + 8 * s + j];
            }
    // Dequant fragments for S^T (rows = coordinates, k = projections):
    //   lane l = 16*q + i, fragment cb*4 + s:  S[32*q + 8*s + j][32*(i/4) + 4*cb + i%4].
    for (int cb = 0; cb < 8; ++cb)
        for (int s = 0; s < 4; ++s)
            for (int l = 0; l < 64; ++l) {
                const int i = l & 15, q = l >> 4;
                const int col = 32 * (i >> 2) + 4 * cb + (i & 3);
                for (int j = 0; j < 8; ++j)
                    t->St_dec[((cb * 4 + s) * 64 + l) * 8 + j] = t->S[(32 * q + 8 * s + j) * d + col];
            }
    return true;
}

}  // namespace tq
