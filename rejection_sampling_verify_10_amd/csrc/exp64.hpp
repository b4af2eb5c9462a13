// Exponentials in fp64 for the final draws, which need every weight to fp64
// accuracy (a boundary of the inverse CDF lies within 1e-5 of u*S in about 8% of
// draws over a wide distribution).
#pragma once

#include <math.h>

#include "common.hpp"

namespace sv {

namespace {

// exp(x) for x <= 0 in fp64 by Tang's table-driven method (ACM TOMS 15(2),
// 1989), with 256 table entries.  The caller passes y = x * 256/ln2 (folded
// into one fma with the temperature and the row maximum); with N = round(y)
// and f = y - N (exact), exp(x) = 2^(N div 256) * 2^((N mod 256)/256) * e^(f ln2/256),
// |f ln2/256| <= 0.00136, and e^t - 1 is its Taylor series to t^4 (truncation
// < 4e-17 relative).  tbl[k] = 2^(k/256).  y below -800*256/ln2 gives 0 (as exp
// does in double); y = -inf is such an argument.
//
// The constants arrive as kernel arguments: they then sit in scalar registers
// and feed v_fma_f64 directly, instead of being rebuilt in vector registers
// for every element.
struct ExpConsts {
    double scale;        // 256 / ln 2
    double floor;        // -800 * scale
    double b1, b2, b3, b4;   // (ln2/256)^k / k!
};
inline ExpConsts exp_consts() {
    ExpConsts k;
    k.scale = 0x1.71547652b82fep+8;
    k.floor = -800.0 * k.scale;
    k.b1 = 0x1.62e42fefa39efp-9;
    k.b2 = 0x1.ebfbdff82c58fp-19;
    k.b3 = 0x1.c6b08d704a0c0p-29;
    k.b4 = 0x1.3b2ab6fba4e77p-39;
    return k;
}
constexpr int kTableSize = 256;

__device__ __forceinline__ double exp_scaled(double y, const double* tbl, const ExpConsts& k) {
    y = fmax(y, k.floor);
    const double n = __builtin_rint(y);
    const int N = static_cast<int>(n);
    const double f = y - n;
    double p = fma(f, k.b4, k.b3);
    p = fma(p, f, k.b2);
    p = fma(p, f, k.b1);
    p *= f;                                                  // e^(f ln2/256) - 1
    const double t = tbl[N & (kTableSize - 1)];
    return ldexp(fma(t, p, t), N >> 8);
}

// y for exp((z - m)/T): one fma per element with k1 = scale/T, mk1 = -m*k1.
struct ExpArg {
    double k1, mk1;
};
__device__ __forceinline__ ExpArg exp_arg(double m, double invT, const ExpConsts& k) {
    const double k1 = invT * k.scale;
    return ExpArg{k1, -m * k1};
}
__device__ __forceinline__ double exp_of(float z, const ExpArg& g, const double* tbl, const ExpConsts& k) {
    return exp_scaled(fma(static_cast<double>(z), g.k1, g.mk1), tbl, k);
}

// q^(1/T) for a float32 q > 0 in fp64, as 2^(log2(q)/T): the logarithm by Tang's
// table-driven method (ACM TOMS 16(4), 1990), the power of two by exp_scaled.
// With q = 2^e * m, m in [1, 2), and c_j = 1 + j/128 the table point nearest m
// (j = 0..128), log2 q = e - log2(inv_j) + log2(1 + r), where inv_j is the fp64
// value of 1/c_j and r = m*inv_j - 1 (one fma; |r| <= 1/256).  Using log2 of the
// stored inv_j rather than of c_j cancels the rounding of inv_j exactly.
// ln(1 + r) is its Taylor series to r^6 (truncation < 2e-18).  Relative error
// about 3e-15 where the result exceeds 1e-6 of the largest weight (the rounding
// of the scaled argument, as in exp_of), up to 1e-13 for results below that;
// q = 2^e gives 2^(e/T) to the last bit of exp_scaled (r = 0).
constexpr int kLogTab = 129;
struct LogEntry {
    double inv;       // 1 / (1 + j/128), rounded
    double lg;        // -log2(inv)
};
__device__ __forceinline__ void build_log_table(LogEntry* lt) {
    for (int j = threadIdx.x; j < kLogTab; j += blockDim.x) {
        const double inv = 1.0 / (1.0 + static_cast<double>(j) * (1.0 / 128));
        lt[j] = LogEntry{inv, -log2(inv)};
    }
}
// y = A*log2(q) + ... in exp_scaled's units: A = 256/T, B = A/ln2.
struct PowArg {
    double A, B;
};
__device__ __forceinline__ PowArg pow_arg(double invT, const ExpConsts& k) {
    return PowArg{256.0 * invT, invT * k.scale};
}
__device__ __forceinline__ double pow_q(float q, const PowArg& pa, const LogEntry* lt, const double* tbl,
                                        const ExpConsts& k) {
    const double d = static_cast<double>(q);
    const int hi = __double2hiint(d), lo = __double2loint(d);
    const int e = ((hi >> 20) & 0x7ff) - 1023;
    const int j = (((hi >> 12) & 0xff) + 1) >> 1;
    const double m = __hiloint2double((hi & 0x000fffff) | 0x3ff00000, lo);
    const LogEntry c = lt[j];
    const double r = fma(m, c.inv, -1.0);
    double t = fma(r, -1.0 / 6, 1.0 / 5);
    t = fma(t, r, -0.25);
    t = fma(t, r, 1.0 / 3);
    t = fma(t, r, -0.5);
    t *= r;
    const double l1p = fma(t, r, r);                        // ln(1 + r)
    return exp_scaled(fma(pa.A, static_cast<double>(e) + c.lg, pa.B * l1p), tbl, k);
}

// bfloat16 logits take few distinct values: the pass looks exp((z - m)/T) up in
// a per-row LDS table holding exp_of of every bf16 value with 2^-20 <= |z| < 256
// (28 binades of 128 values per sign), so the result is the one exp_of gives.
// Entry of bit pattern h: sign(h)*kTabSpan + (h & 0x7fff) - kTabLo.  Values
// outside the table (smaller, larger, zero, inf, NaN) take exp_of.
constexpr uint32_t kTabLo = 0x3580u;                 // bf16 bits of 2^-20
constexpr uint32_t kTabSpan = 0x0e00u;               // bits of 256 minus kTabLo
constexpr int kTabSize = 2 * static_cast<int>(kTabSpan);
constexpr size_t kTabBytes = kTabSize * sizeof(double);

__device__ __forceinline__ void build_exp_table(double* etab, const ExpArg& g, const double* tbl, const ExpConsts& k) {
    for (int t = threadIdx.x; t < kTabSize; t += blockDim.x) {
        const uint32_t h = t < static_cast<int>(kTabSpan) ? kTabLo + t : 0x8000u + kTabLo + (t - kTabSpan);
        etab[t] = exp_of(__uint_as_float(h << 16), g, tbl, k);
    }
}

// exp_of of the 8 bf16 logits of r, from the table where it holds them.
template <typename R8>
__device__ __forceinline__ void exp8_table(const R8& r, const double* etab, const ExpArg& g, const double* tbl,
                                           const ExpConsts& k, double ex[8]) {
    bool out = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t w = r.z[0][e >> 1];
        const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xffffu);
        const uint32_t off = (h & 0x7fffu) - kTabLo;
        const bool in = off < kTabSpan;
        out |= !in;
        ex[e] = etab[(in ? off : 0u) + ((h & 0x8000u) ? kTabSpan : 0u)];
    }
    if (__ballot(out)) {            // wave-uniform: rows with logits outside the table
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t w = r.z[0][e >> 1];
            const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xffffu);
            if ((h & 0x7fffu) - kTabLo >= kTabSpan) ex[e] = exp_of(r.zf(e), g, tbl, k);
        }
    }
}

}  // namespace

}  // namespace sv
