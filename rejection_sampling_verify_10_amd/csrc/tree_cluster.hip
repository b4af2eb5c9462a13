// Sampling verification of a draft tree with each batch row's walk shared by a
// cluster of G workgroups.
//
// The method is the one of tree_sample.hip ("投机解码与 EAGLE", the EAGLE part:
// a rejected branch makes the verifier try the others; "064 · 投机解码",
// section 三, and "EAGLE-2: Faster Inference of Language Models with Dynamic
// Draft Trees", section 2.1, for the single test and the residual): from the
// root c with P = p'_c and Q = q'_c the children of c are tried in increasing
// node order, child n accepted iff u[n] < min(1, P(x_n)/Q(x_n)); a rejection
// replaces P by max(0, P - Q)/S (kept when S = 0); an accepted child becomes c;
// where no child is accepted, or at a leaf, a token is drawn from P with u[0]
// by index-ascending inverse CDF.  After rejections at c,
//     P(v) = max(0, P_0(v) - cq Q(v)) / D,
// each rejection of mass S > 0 adding D to cq and multiplying D by S (the
// recursion unrolled).
//
// A batch row's vocabulary is split into G contiguous slices, one per member
// workgroup of 512 threads; a member holds its slice of the current node's rows in registers.
// Every quantity the walk needs is a sum or a maximum over the vocabulary, so
// per node a member computes its slice's part (the row maximum and
// sum_v exp((z_v - m_g)/T) against its own maximum m_g, the draft power sum),
// per rejection the slice's residual mass, and at the end the slice's draw
// weight; the members exchange these parts through device words and combine
// them in member order, so every member holds the same values and takes the
// same decisions.  Member 0 draws: it rescans the slice that holds u[0] times
// the total weight (the members' totals tile it in order) and writes the row's
// outputs.  Everything is fp64: exp((z - m)/T) by Tang's table-driven
// exponential, q^(1/T) by the table-driven power.
//
// Exchange words: per (batch row, round, member) 8 words of 64 bits, each the
// round number plus one in its high half and 32 bits of the member's part in
// its low half, so a word is valid by itself (8-byte accesses are single-copy
// atomic) and a zero word is not yet written.  A member writes its words, then
// polls the other members' words of the same round.  The last member of a row
// to finish zeroes the row's words, so every call finds them zero.  Members of
// a row are G <= 8 consecutive workgroups, so they sit on different XCDs, and
// each XCD dispatches its workgroups in grid order: on every XCD the rows
// dispatched form a prefix, and every row below the shortest prefix has all
// its members running, so it finishes and makes room.  A wait that passes the
// spin limit ends the row as timed out.

#include <math.h>

#include "common.hpp"
#include "exp64.hpp"
#include "internal.hpp"
#include "lists.hpp"

namespace sv {

namespace {

constexpr int kTcThreads = 512;
constexpr int kTcWaves = kTcThreads / kWave;
constexpr int kTcMaxNodes = 64;

struct TcSmem {
    double tbl[kTableSize];
    LogEntry lt[kLogTab];
    double red[kTcWaves];
    double red2[kTcWaves];
    int ired[kTcWaves];
    uint32_t ex[kTcMaxG * kTcWords];     // the round's parts: member g's piece k at [g * kTcWords + k]
    uint32_t out[kTcWords];              // this member's pieces of the round
    float mg[kTcMaxG];                   // every member's slice maximum at the current node
    double wtot[kTcMaxG];                // every member's share of P's mass, times tot_inv below
    int timed_out;
    int last;
    int par[kTcMaxNodes];
    int fch[kTcMaxNodes];
    int nsib[kTcMaxNodes];
    int path[kTcMaxNodes];
    int toks[kTcMaxNodes];
    int ntok[kTcMaxNodes];               // the batch row's node tokens and uniforms
    float nu[kTcMaxNodes];
    float gz[kTcMaxNodes];               // z[x_n] and q[x_n] of the current node's children n
    float gq[kTcMaxNodes];
};

__device__ __forceinline__ uint32_t lo32(double v) { return static_cast<uint32_t>(__double_as_longlong(v)); }
__device__ __forceinline__ uint32_t hi32(double v) {
    return static_cast<uint32_t>(static_cast<unsigned long long>(__double_as_longlong(v)) >> 32);
}
__device__ __forceinline__ double dbl(uint32_t lo, uint32_t hi) {
    return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

__device__ __forceinline__ double tc_block_sum(double v, TcSmem& sm) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) sm.red[threadIdx.x / kWave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kTcWaves; ++w) t += sm.red[w];
    return t;
}
__device__ __forceinline__ void tc_block_sum2(double& a, double& b, TcSmem& sm) {
    a = wave_sum(a);
    b = wave_sum(b);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) {
        sm.red[threadIdx.x / kWave] = a;
        sm.red2[threadIdx.x / kWave] = b;
    }
    __syncthreads();
    a = 0.0;
    b = 0.0;
#pragma unroll
    for (int w = 0; w < kTcWaves; ++w) {
        a += sm.red[w];
        b += sm.red2[w];
    }
}
__device__ __forceinline__ int tc_block_or(int v, TcSmem& sm) {
    v = __ballot(v != 0) != 0ull;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) sm.ired[threadIdx.x / kWave] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < kTcWaves; ++w) t |= sm.ired[w];
    return t;
}
__device__ __forceinline__ int tc_block_max(int v, TcSmem& sm) {
    v = wave_max_int(v);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) sm.ired[threadIdx.x / kWave] = v;
    __syncthreads();
    int t = sm.ired[0];
#pragma unroll
    for (int w = 1; w < kTcWaves; ++w) t = max(t, sm.ired[w]);
    return t;
}
__device__ __forceinline__ float tc_block_maxf(float v, TcSmem& sm) {
    v = wave_max(v);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) sm.red[threadIdx.x / kWave] = static_cast<double>(v);
    __syncthreads();
    float t = static_cast<float>(sm.red[0]);
#pragma unroll
    for (int w = 1; w < kTcWaves; ++w) t = fmaxf(t, static_cast<float>(sm.red[w]));
    return t;
}

// One exchange round: this member's 8 pieces (sm.out, set by thread 0 before
// the call) out, every member's pieces into sm.ex.  Returns false when the wait
// passed the spin limit (block-uniform).
__device__ __forceinline__ bool tc_exchange(const TcArgs& a, unsigned long long* rw, int G, int g, int round,
                                            TcSmem& sm) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const unsigned long long mark = static_cast<unsigned long long>(round + 1) << 32;
    __syncthreads();                       // sm.out written; sm.ex of the previous round read by all
    if (tid < kWave) {
        const int n = G * kTcWords;
        unsigned long long* p = rw + static_cast<long>(round) * G * kTcWords + lane;
        if (lane >= g * kTcWords && lane < (g + 1) * kTcWords) st_agent64(p, mark | sm.out[lane - g * kTcWords]);
        unsigned long long w = 0ull;
        bool have = lane >= n;
        int spins = 0;
        bool late = false;
        for (;;) {
            if (!have) {
                w = ld_agent64(p);
                have = (w & 0xffffffff00000000ull) == mark;
            }
            if (__ballot(!have) == 0ull) break;
            if (++spins > a.spin_limit) { late = true; break; }
            __builtin_amdgcn_s_sleep(2);
        }
        if (lane < n) sm.ex[lane] = static_cast<uint32_t>(w);
        if (lane == 0) sm.timed_out = late ? 1 : 0;
    }
    __syncthreads();
    return sm.timed_out == 0;
}

// The weights of the current node in fp64: e_v = exp((z_v - m_g)/T) against the
// member's own maximum (scaled by sc = exp((m_g - m)/T) to the row maximum), the
// draft weight y_v (q, or q^(1/T)), Q_v = y_v / Sq.
template <bool TR>
struct TcDist {
    double sc, invZ, invSq, cq, invD;
    bool plain;
    __device__ __forceinline__ double P(double e, double Q) const {
        return fmax(e * sc * invZ - cq * Q, 0.0) * invD;
    }
};

template <int DT, bool TR, int NG>
__global__ __launch_bounds__(kTcThreads, 1) void tree_cluster_kernel(TcArgs a, ExpConsts ek) {
    __shared__ TcSmem sm;
    const TreeSampleArgs& t = a.t;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = wave_id();
    const int G = a.G;
    const int b = blockIdx.x / G, g = blockIdx.x - b * G;
    const int N = t.N, V = t.V;
    const long esz = Elem<DT>::kBytes;
    for (int i = tid; i < kTableSize; i += kTcThreads) sm.tbl[i] = exp2(static_cast<double>(i) * (1.0 / kTableSize));
    if (TR) build_log_table(sm.lt);
    const PowArg pa = pow_arg(t.invT, ek);
    const int32_t* tok = t.node_tokens + static_cast<long>(b) * N;
    const float* ub = t.u + static_cast<long>(b) * N;
    const char* zbase = static_cast<const char*>(t.logits) + static_cast<long>(b) * N * V * esz;
    const float* qbase = t.q + static_cast<long>(b) * N * V;
    unsigned long long* rw = a.words + static_cast<long>(b) * a.R * G * kTcWords;

    // The tree (static, or the batch row's own, checked and linked), E2 and E5.
    int bad = 0;
    if (t.parents_rows) {
        if (tid < N) {
            const int p = t.parents_rows[static_cast<long>(b) * N + tid];
            bad |= tid == 0 ? p != -1 : (p < 0 || p >= tid);
            sm.par[tid] = p;
        }
        __syncthreads();
        if (tid == 0) {
            for (int n = 0; n < N; ++n) sm.fch[n] = sm.nsib[n] = -1;
            for (int n = N - 1; n >= 1; --n) {
                const int p = sm.par[n];
                if (p < 0 || p >= n) continue;
                sm.nsib[n] = sm.fch[p];
                sm.fch[p] = n;
            }
        }
    } else if (tid < N) {
        sm.par[tid] = t.parent[tid];
        sm.fch[tid] = t.first_child[tid];
        sm.nsib[tid] = t.next_sibling[tid];
    }
    if (tid < N) {
        const float uv = ub[tid];
        const int tv = tok[tid];
        bad |= !u_ok(uv);
        if (tid > 0) bad |= (tv < 0 || tv >= V);
        sm.nu[tid] = uv;
        sm.ntok[tid] = tv;
    }
    int err = tc_block_or(bad, sm);
    bool late = false;

    // This member's slice [s0, s1): groups of 8 elements, thread tid holding
    // groups tid, tid + kTcThreads, ... (NG of them) of the slice.
    const int s0 = min(V, g * a.L), s1 = min(V, s0 + a.L);
    auto gidx = [&](int k) { return s0 + (tid + k * kTcThreads) * 8; };
    auto load_z = [&](const char* row, float (&z)[NG][8]) {
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            const int i0 = gidx(k);
            if (i0 < s1) {
                if (DT == 1) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(row + static_cast<long>(i0) * 2);
#pragma unroll
                    for (int e = 0; e < 8; ++e) z[k][e] = Elem<1>::get(v, e);
                } else {
                    const u32x4* p = reinterpret_cast<const u32x4*>(row + static_cast<long>(i0) * 4);
                    const u32x4 v0 = p[0], v1 = p[1];
#pragma unroll
                    for (int e = 0; e < 4; ++e) { z[k][e] = __uint_as_float(v0[e]); z[k][4 + e] = __uint_as_float(v1[e]); }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) z[k][e] = -INFINITY;
            }
        }
    };
    auto load_q = [&](const float* row, float (&q)[NG][8]) {
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            const int i0 = gidx(k);
            if (i0 < s1) {
                const u32x4* p = reinterpret_cast<const u32x4*>(row + i0);
                const u32x4 v0 = p[0], v1 = p[1];
#pragma unroll
                for (int e = 0; e < 4; ++e) { q[k][e] = __uint_as_float(v0[e]); q[k][4 + e] = __uint_as_float(v1[e]); }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) q[k][e] = 0.f;
            }
        }
    };
    auto dw = [&](float qv) -> double {      // draft weight: q, or q^(1/T); 0 for q <= 0
        if (!(qv > 0.f)) return 0.0;
        return TR ? pow_q(qv, pa, sm.lt, sm.tbl, ek) : static_cast<double>(qv);
    };

    // a round's pieces: two 32-bit values and two doubles
    auto post = [&](uint32_t p0, uint32_t p1, double d0, double d1) {
        if (tid == 0) {
            sm.out[0] = p0;
            sm.out[1] = p1;
            sm.out[2] = lo32(d0);
            sm.out[3] = hi32(d0);
            sm.out[4] = lo32(d1);
            sm.out[5] = hi32(d1);
            sm.out[6] = 0u;
            sm.out[7] = 0u;
        }
    };
    float z[NG][8], zn[NG][8], q[NG][8];
    double ev[NG][8];                    // exp((z - m_g)/T) of the slice
    bool have_q = false, have_next = false;
    int c = 0, d = 0, round = 0;
    float m = 0.f;
    TcDist<TR> ds{};
    double Zrow = 1.0, Sq = 1.0, Dk = 1.0, tot_inv = 1.0;
    if (tid == 0) sm.path[0] = 0;

    while (!err) {
        const char* zr = zbase + static_cast<long>(c) * V * esz;
        const float* qr = qbase + static_cast<long>(c) * V;
        const int first = sm.fch[c];
        // Loads: the node's slice (unless prefetched), its draft slice when the node
        // has children (a rejection reads it; its validity is checked then), the
        // children's z[x_n] and q[x_n] (lanes of wave 0, stored after the exchange
        // so that their latency overlaps the slice's arithmetic), then the first
        // child's slice, the likeliest next node.
        if (have_next) {
#pragma unroll
            for (int k = 0; k < NG; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) z[k][e] = zn[k][e];
        } else {
            load_z(zr, z);
        }
        have_q = first >= 0;
        if (have_q) load_q(qr, q);
        float gzr = 0.f, gqr = 0.f;
        const bool gl = wid == 0 && lane > 0 && lane < N && sm.par[lane] == c;
        if (gl) {
            const int x = sm.ntok[lane];
            gzr = Elem<DT>::scalar(zr, x);
            gqr = qr[x];
        }
        if (first >= 0) load_z(zbase + static_cast<long>(first) * V * esz, zn);

        // The slice's maximum, +inf when the slice holds NaN or +inf (E1); its
        // exponential sum against that maximum; the draft's power sum, NaN when a
        // value is NaN, negative or +inf (E3).
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < NG; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = maximum3(mx, z[k][e], z[k][e]);
        const float mg = tc_block_maxf(mx == mx ? mx : INFINITY, sm);
        double Zg = 0.0, Sqg = 0.0;
        if (mg > -INFINITY && mg < INFINITY) {
            const ExpArg ga = exp_arg(static_cast<double>(mg), t.invT, ek);
#pragma unroll
            for (int k = 0; k < NG; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ev[k][e] = exp_of(z[k][e], ga, sm.tbl, ek);
                    Zg += ev[k][e];
                }
        } else {
#pragma unroll
            for (int k = 0; k < NG; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) ev[k][e] = 0.0;
        }
        if (TR && first >= 0) {
            int qb = 0;
#pragma unroll
            for (int k = 0; k < NG; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    qb |= !q_ok(q[k][e]);
                    Sqg += dw(q[k][e]);
                }
            if (qb) Sqg = NAN;
        }
        tc_block_sum2(Zg, Sqg, sm);
        post(0u, __float_as_uint(mg), Zg, Sqg);
        if (!tc_exchange(a, rw, G, g, round++, sm)) { late = true; break; }
        if (gl) {
            sm.gz[lane] = gzr;
            sm.gq[lane] = gqr;
        }
        // Combine: lane h of every wave takes member h's part, then wave reductions,
        // the same in every member.
        {
            const bool hl = lane < G;
            const float mh = hl ? __uint_as_float(sm.ex[lane * kTcWords + 1]) : -INFINITY;
            m = wave_max(mh);
            if (!(m > -INFINITY) || !(m < INFINITY)) { err = 1; break; }            // E1
            const ExpArg gm = exp_arg(static_cast<double>(m), t.invT, ek);
            double zp = 0.0, sp = 0.0;
            if (hl) {
                if (mh > -INFINITY)
                    zp = dbl(sm.ex[lane * kTcWords + 2], sm.ex[lane * kTcWords + 3]) * exp_of(mh, gm, sm.tbl, ek);
                sp = dbl(sm.ex[lane * kTcWords + 4], sm.ex[lane * kTcWords + 5]);
            }
            Zrow = wave_sum(zp);
            Sq = TR ? wave_sum(sp) : 1.0;
            ds.sc = bcast(mg > -INFINITY ? exp_of(mg, gm, sm.tbl, ek) : 0.0, 0);
            // member h's share of P = e/Z: zp_h / Z (read by the draw after a barrier)
            if (wid == 0 && hl) sm.wtot[lane] = zp;
            tot_inv = 1.0 / Zrow;
        }
        if (first < 0) break;                                                      // a leaf: the draw is here
        if (TR && (!(Sq > 0.0) || !(Sq < INFINITY))) { err = 1; break; }           // E3 (NaN), E4
        ds.invZ = 1.0 / Zrow;
        ds.invSq = 1.0 / Sq;
        ds.cq = 0.0;
        ds.invD = 1.0;
        Dk = 1.0;
        __syncthreads();                   // sm.gz, sm.gq

        // The children in node order; the tests are the same in every member.
        int accepted = -1;
        bool q_checked = TR;
        const ExpArg gm = exp_arg(static_cast<double>(m), t.invT, ek);
        for (int n = first; n >= 0; n = sm.nsib[n]) {
            const float zx = sm.gz[n], qx = sm.gq[n];
            if (!TR && !q_ok(qx)) { err = 1; break; }                               // E3
            const double Qx = TR ? dw(qx) * ds.invSq : static_cast<double>(qx);
            const double Px = fmax(exp_of(zx, gm, sm.tbl, ek) * ds.invZ - ds.cq * Qx, 0.0) * ds.invD;
            double ratio;
            if (Qx > 0.0) ratio = Px / Qx;
            else ratio = Px > 0.0 ? INFINITY : 0.0;
            const double thr = ratio < 1.0 ? ratio : 1.0;
            if (static_cast<double>(sm.nu[n]) < thr) { accepted = n; break; }
            // Rejected: the slice's residual mass sum_v max(0, P(v) - Q(v)), NaN when an
            // untransformed draft row read for the first time holds a bad value (E3).
            double Sg = 0.0;
            int qb = 0;
#pragma unroll
            for (int k = 0; k < NG; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (!q_checked) qb |= !q_ok(q[k][e]);
                    const double Qv = TR ? dw(q[k][e]) * ds.invSq : static_cast<double>(q[k][e]);
                    Sg += fmax(ds.P(ev[k][e], Qv) - Qv, 0.0);
                }
            if (qb) Sg = NAN;
            Sg = tc_block_sum(Sg, sm);
            post(0u, 0u, Sg, 0.0);
            if (!tc_exchange(a, rw, G, g, round++, sm)) { late = true; break; }
            const double Sh = lane < G ? dbl(sm.ex[lane * kTcWords + 2], sm.ex[lane * kTcWords + 3]) : 0.0;
            const double S = wave_sum(Sh);
            if (S != S) { err = 1; break; }                                         // E3
            q_checked = true;
            if (S > 0.0) {
                ds.cq += Dk;
                Dk *= S;
                ds.invD = 1.0 / Dk;
                // the new P's shares: member h's residual mass over S
                if (wid == 0 && lane < G) sm.wtot[lane] = Sh;
                tot_inv = 1.0 / S;
            }
        }
        if (late || err) break;
        have_next = accepted >= 0 && accepted == first;
        if (accepted < 0) break;
        ++d;
        c = accepted;
        if (tid == 0) {
            sm.path[d] = c;
            sm.toks[d - 1] = sm.ntok[c];
        }
        __syncthreads();
    }

    // The draw at c from P (after the rejections there).  Every member knows each
    // member's share of P's mass from the last exchange (zp_h / Z, or S_h / S after
    // a rejection), and the shares tile [0, W) in member order; the member whose
    // part holds u[0]*W finds the token among its own weights and hands it to
    // member 0 in one more round.
    int y = -1;
    if (!err && !late) {
        __syncthreads();                     // sm.wtot
        const bool res = have_q && ds.cq > 0.0;
        if (sm.fch[c] < 0) {                 // a leaf: no rejection, P = e/Z
            ds.invZ = 1.0 / Zrow;
            ds.cq = 0.0;
            ds.invD = 1.0;
        }
        double W = 0.0, base = 0.0;
        int hold = -1, lasth = -1;
        for (int h = 0; h < G; ++h) W += sm.wtot[h] * tot_inv;
        const double target = static_cast<double>(sm.nu[0]) * W;
        double acc = 0.0;
        for (int h = 0; h < G; ++h) {
            const double wh = sm.wtot[h] * tot_inv;
            const double nx = acc + wh;
            if (hold < 0 && wh > 0.0 && acc <= target && target < nx) { hold = h; base = acc; }
            if (wh > 0.0) lasth = h;
            acc = nx;
        }
        if (hold < 0) {                      // rounding (or no mass): the last member with mass, its end
            hold = lasth >= 0 ? lasth : 0;
            base = INFINITY;
        }
        int found = -1;
        if (g == hold) {
            double w[NG][8];
            int lp = -1;
#pragma unroll
            for (int k = 0; k < NG; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const double Qv = res ? (TR ? dw(q[k][e]) * ds.invSq : static_cast<double>(q[k][e])) : 0.0;
                    w[k][e] = ds.P(ev[k][e], Qv);
                    if (w[k][e] > 0.0) lp = gidx(k) + e;
                }
            // index order within the slice: every thread's first group, then every
            // thread's second; parts tiled by shuffled inclusive sums
            double lo = base;
#pragma unroll
            for (int k = 0; k < NG; ++k) {
                double sk = 0.0;
#pragma unroll
                for (int e = 0; e < 8; ++e) sk += w[k][e];
                const double incl = wave_inclusive_scan(sk);
                double excl = __shfl_up(incl, 1, kWave);
                if (lane == 0) excl = 0.0;
                __syncthreads();
                if (lane == kWave - 1) sm.red[wid] = incl;
                __syncthreads();
                double wb = 0.0, tot = 0.0;
                for (int x = 0; x < kTcWaves; ++x) {
                    if (x == wid) wb = tot;
                    tot += sm.red[x];
                }
                const double tlo = lo + wb + excl, thi = lo + wb + incl;
                if (found < 0 && tlo <= target && target < thi) {
                    double cacc = tlo;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        cacc += w[k][e];
                        if (found < 0 && w[k][e] > 0.0 && target < cacc) found = gidx(k) + e;
                    }
                    if (found < 0)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (w[k][e] > 0.0) found = gidx(k) + e;
                }
                lo = lo + tot;
            }
            found = tc_block_max(found, sm);
            // u[0]*W past this scan's end (rounding): the slice's last weighted index
            if (found < 0) found = tc_block_max(lp, sm);
        }
        post(static_cast<uint32_t>(found), 0u, 0.0, 0.0);
        if (!tc_exchange(a, rw, G, g, round++, sm)) late = true;
        else y = static_cast<int>(sm.ex[hold * kTcWords]);
    }

    // Member 0 writes the row: path, accepted tokens and the drawn one, -1 padded.
    if (g == 0) {
        const long ob = static_cast<long>(b) * (t.D + 1);
        for (int i = tid; i <= t.D; i += kTcThreads) {
            const bool ok = !err && !late && i <= d;
            t.out_path[ob + i] = ok ? sm.path[i] : -1;
            t.out_tokens[ob + i] = ok ? (i < d ? sm.toks[i] : y) : -1;
        }
        if (tid == 0) t.out_accept_len[b] = late ? kTimedOut : (err ? -1 : d);
    }
    // The last member of the row to finish zeroes its words.
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(a.done + b, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        sm.last = prev == static_cast<unsigned>(G - 1) ? 1 : 0;
    }
    __syncthreads();
    if (sm.last) {
        const int nw = a.R * G * kTcWords;
        for (int i = tid; i < nw; i += kTcThreads) st_agent64(rw + i, 0ull);
        if (tid == 0) __hip_atomic_store(a.done + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int DT, bool TR>
hipError_t tc_launch_ng(const TcArgs& a, int ng, hipStream_t s, Timing tm) {
    const dim3 grid(static_cast<unsigned>(a.t.B * a.G));
    if (ng == 1) launch_timed(tm, tree_cluster_kernel<DT, TR, 1>, grid, dim3(kTcThreads), 0, s, a, exp_consts());
    else launch_timed(tm, tree_cluster_kernel<DT, TR, TR ? 1 : 2>, grid, dim3(kTcThreads), 0, s, a, exp_consts());
    return hipGetLastError();
}

}  // namespace

int tree_cluster_members(int B) {
    if (B < 1) return 0;
    int G = 256 / B;
    return G > kTcMaxG ? kTcMaxG : G;
}

// A slice of at most two groups of 8 elements per thread (one when the draft is
// transformed): the registers the kernel holds without spilling.
bool tree_cluster_fits(int B, int N, int V, const void* logits, int dtype, const float* q, bool transformed) {
    const int G = tree_cluster_members(B);
    if (G < 2 || N > kTcMaxNodes || V % 8 != 0) return false;
    if (!vec_ok(logits, V, dtype == 1 ? 2 : 4) || !vec_ok(q, V, 4)) return false;
    const long L = ((static_cast<long>(V) + G - 1) / G + 7) / 8 * 8;
    return L <= (transformed ? 1L : 2L) * kTcThreads * 8;
}

hipError_t launch_tree_cluster(TcArgs a, hipStream_t s, Timing tm) {
    a.L = ((a.t.V + a.G - 1) / a.G + 7) / 8 * 8;
    const int ng = (a.L / 8 + kTcThreads - 1) / kTcThreads;
    if (ng < 1 || ng > (a.t.transformed ? 1 : 2) || a.G < 2 || a.G > kTcMaxG || a.t.N > kTcMaxNodes) return hipErrorInvalidValue;
    if (a.t.dtype == 1) return a.t.transformed ? tc_launch_ng<1, true>(a, ng, s, tm) : tc_launch_ng<1, false>(a, ng, s, tm);
    return a.t.transformed ? tc_launch_ng<0, true>(a, ng, s, tm) : tc_launch_ng<0, false>(a, ng, s, tm);
}

}  // namespace sv
