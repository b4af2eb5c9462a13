// Sampling verification of a static draft tree: one workgroup per batch row
// walks down from the root.
//
// "投机解码与 EAGLE", the EAGLE part: with a tree of drafts a rejected token
// does not end the step, the other branches are tried.  "EAGLE-2: Faster
// Inference of Language Models with Dynamic Draft Trees", section 2.1, and
// "064 · 投机解码", section 三, give the single test (accept with probability
// min(1, p/q)) and the residual norm(max(0, p - q)).  The pages give no rule
// for several branches; the reading taken applies that test once per
// sibling.  At the current node c, P = p'_c (the target row of c under the
// temperature) and Q = q'_c (the draft distribution at c, from which c's
// children were drawn).  Children are tried in increasing node order: child n
// is accepted iff u[n] < min(1, P(x_n)/Q(x_n)) (q' = 0 accepts iff P > 0); a
// rejection replaces P by max(0, P - Q)/S, S its mass (P is kept when S = 0);
// an acceptance moves to n.  When no child is accepted, or c is a leaf, the
// token is drawn from P with u[0]: the first index, ascending, whose inclusive
// prefix of P exceeds u[0]*sum P (rounding fallback: the last index with
// P > 0).
//
// Two precisions.  The tests along the walk take fp32 probabilities (one
// v_exp_f32 per element, sums accumulated in fp64), as the chain's ratio tests
// do: a test's outcome moves only where u lies within ~1e-6 of its threshold.
// The final draw needs every weight to fp64 accuracy (a boundary of the inverse
// CDF lies within 1e-5 of u*S for a good share of draws over a wide
// distribution), so at the node where the walk stops the normalisers and the
// residual masses are recomputed in fp64 (bf16 logits: one LDS table lookup of
// an fp64 exponential per element), the last of those passes also leaving the
// per-segment sums of the draw's weights; the draw then rescans one
// 512-element segment.
//
// Rows.  A logit row of at most 64 KiB is copied into LDS when the walk
// reaches its node (every load issued at once) and every pass reads it from
// there; while a node is being tested, its first child's row -- the likeliest
// next node -- is loaded into registers and parked in a second LDS buffer.
// The draft row is streamed, each tile's loads issued one tile ahead.  Longer
// rows are streamed (from L2 after the first pass).

#include <math.h>

#include "common.hpp"
#include "exp64.hpp"
#include "internal.hpp"
#include "lists.hpp"

namespace sv {

namespace {

constexpr int kTsThreads = 1024;
constexpr int kTsWaves = kTsThreads / kWave;
constexpr int kTsTile = 8 * kTsThreads;                     // elements per tile: 8 per thread
constexpr int kTsMaxTiles = (kMaxV + kTsTile - 1) / kTsTile;
constexpr int kTsParts = kTsMaxTiles * kTsWaves;            // one 512-element segment per (tile, wave)
constexpr int kTsMaxNodes = 64;
constexpr int kTsRowBytes = 64 * 1024;                      // largest LDS-held logit row
constexpr int kTsRowVecs = kTsRowBytes / 16 / kTsThreads;   // its 16-byte vectors per thread
constexpr float kLog2e = 1.4426950408889634f;

constexpr int kTsFastRej = 3;                               // rejections the one-pass final stage takes
constexpr int kTsListCap = 256;                             // its undecided elements
constexpr double kTsBracket = 1e-4;                         // relative bracket around the walk's fp32 points

// A value every lane holds alike, moved to scalar registers.
__device__ __forceinline__ double uniform_d(double v) {
    const long long bits = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readfirstlane(static_cast<int>(bits));
    const int hi = __builtin_amdgcn_readfirstlane(static_cast<int>(bits >> 32));
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}

// Segment-sum slots the LDS layout provides (two arrays of this many doubles).
template <int DT, bool LROW> constexpr int ts_parts_cap() {
    return LROW ? kTsRowBytes / Elem<DT>::kBytes / kTsTile * kTsWaves : kTsParts;
}

struct TsSmem {
    double tbl[kTableSize];          // 2^(k/256) for the fp64 exponential
    double red[kTsWaves];
    double redn[kTsWaves][2 + 2 * kTsFastRej];
    int li_v[kTsListCap];            // undecided elements of the one-pass final stage: index,
    int li_j[kTsListCap];            //   evaluation point, e_v and the draft weight y_v
    double li_e[kTsListCap];
    double li_y[kTsListCap];
    int n_list;
    int fast_ok;
    double lam_last;                 // the exact point of the draw's residual
    int last_list;                   // the largest listed index with a positive draw weight
    float fred[kTsWaves];
    int ired[kTsWaves];
    float sinv32[kTsMaxNodes];       // walk (fp32): 1/S of each rejection at the current node
    int kept32[kTsMaxNodes];         //   1: that rejection left P as it was (S = 0)
    double sinv[kTsMaxNodes];        // final node (fp64): the same
    int kept[kTsMaxNodes];
    int path[kTsMaxNodes];
    int toks[kTsMaxNodes];
    float gz[kTsMaxNodes];           // z[x_n] and q[x_n] of the current node's children n
    float gq[kTsMaxNodes];
    int par[kTsMaxNodes];            // the batch row's tree: parent, first child, next sibling (-1: none)
    int fch[kTsMaxNodes];
    int nsib[kTsMaxNodes];
    int dec;                         // thread 0's decision: 0 reject, 1 accept, 2 error
    int seg;                         // draw: segment holding u*S, -1 for the fallback
    double base;                     // draw: weight before that segment
};

// Eight consecutive logits from i0 (a multiple of 8), widened; -inf past V.
template <int DT, bool VEC>
__device__ __forceinline__ void ts_load_z(const char* row, int i0, int V, float z[8]) {
    using E = Elem<DT>;
    if (VEC) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row + static_cast<long>(i0) * E::kBytes);
        if (i0 >= V) {
#pragma unroll
            for (int e = 0; e < 8; ++e) z[e] = -INFINITY;
            return;
        }
        if (DT == 1) {
            const u32x4 v = p[0];
#pragma unroll
            for (int e = 0; e < 8; ++e) z[e] = E::get(v, e);
        } else {
            const u32x4 v0 = p[0], v1 = p[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) { z[e] = __uint_as_float(v0[e]); z[4 + e] = __uint_as_float(v1[e]); }
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (i0 + e < V) ? E::scalar(row, i0 + e) : -INFINITY;
}

// Eight consecutive draft probabilities from i0; 0 past V.
template <bool VEC>
__device__ __forceinline__ void ts_load_q(const float* row, int i0, int V, float q[8]) {
    if (VEC) {
        if (i0 >= V) {
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = 0.f;
            return;
        }
        const u32x4* p = reinterpret_cast<const u32x4*>(row + i0);
        const u32x4 v0 = p[0], v1 = p[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) { q[e] = __uint_as_float(v0[e]); q[4 + e] = __uint_as_float(v1[e]); }
        return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = (i0 + e < V) ? row[i0 + e] : 0.f;
}

__device__ __forceinline__ double ts_block_sum(double v, TsSmem& sm) {
    v = wave_sum(v);
    if ((threadIdx.x & (kWave - 1)) == 0) sm.red[threadIdx.x / kWave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kTsWaves; ++w) t += sm.red[w];
    __syncthreads();
    return t;
}

__device__ __forceinline__ int ts_block_or(int v, TsSmem& sm) {
    v = __ballot(v != 0) != 0ull;
    if ((threadIdx.x & (kWave - 1)) == 0) sm.ired[threadIdx.x / kWave] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < kTsWaves; ++w) t |= sm.ired[w];
    __syncthreads();
    return t;
}

__device__ __forceinline__ int ts_block_max(int v, TsSmem& sm) {
    v = wave_max_int(v);
    if ((threadIdx.x & (kWave - 1)) == 0) sm.ired[threadIdx.x / kWave] = v;
    __syncthreads();
    int t = sm.ired[0];
#pragma unroll
    for (int w = 1; w < kTsWaves; ++w) t = max(t, sm.ired[w]);
    __syncthreads();
    return t;
}

// The current node's logit row: from an LDS copy (LROW) or streamed.
template <int DT, bool VEC, bool LROW>
struct NodeRow {
    static constexpr bool kVec = VEC;
    const u32x4* zs;      // LDS copy (LROW)
    const char* zr;
    const float* qr;
    int V;

    __device__ __forceinline__ void get_z(int t, float out[8]) const {
        const int i0 = t * kTsTile + 8 * static_cast<int>(threadIdx.x);
        if constexpr (LROW) {
            if (i0 >= V) {
#pragma unroll
                for (int e = 0; e < 8; ++e) out[e] = -INFINITY;
                return;
            }
            if (DT == 1) {
                const u32x4 v = zs[i0 / 8];
#pragma unroll
                for (int e = 0; e < 8; ++e) out[e] = Elem<1>::get(v, e);
            } else {
                const u32x4 v0 = zs[i0 / 4], v1 = zs[i0 / 4 + 1];
#pragma unroll
                for (int e = 0; e < 4; ++e) { out[e] = __uint_as_float(v0[e]); out[4 + e] = __uint_as_float(v1[e]); }
            }
        } else {
            ts_load_z<DT, VEC>(zr, i0, V, out);
        }
    }
};

// A row of at most kTsRowBytes (nvec 16-byte vectors): thread t's vectors t,
// t + 1024, ... are loaded into v, then stored to an LDS buffer.
__device__ __forceinline__ void row_issue(const char* row, int nvec, u32x4 (&v)[kTsRowVecs]) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row);
#pragma unroll
    for (int k = 0; k < kTsRowVecs; ++k) {
        const int j = k * kTsThreads + static_cast<int>(threadIdx.x);
        v[k] = p[j < nvec ? j : 0];
    }
}
__device__ __forceinline__ void row_park(u32x4* dst, int nvec, const u32x4 (&v)[kTsRowVecs]) {
#pragma unroll
    for (int k = 0; k < kTsRowVecs; ++k) {
        const int j = k * kTsThreads + static_cast<int>(threadIdx.x);
        if (j < nvec) dst[j] = v[k];
    }
}

// f(t, i0, z[8], q[8]) over the tiles in index order (q only when with_q).
template <class Row, class F>
__device__ __forceinline__ void for_tiles(const Row& r, int ntiles, bool with_q, F&& f) {
    const int lo = 8 * static_cast<int>(threadIdx.x);
    if constexpr (!Row::kVec) {
        for (int t = 0; t < ntiles; ++t) {
            const int i0 = t * kTsTile + lo;
            float z[8], q[8];
            if (with_q) ts_load_q<false>(r.qr, i0, r.V, q);
            r.get_z(t, z);
            f(t, i0, z, q);
        }
        return;
    }
    float qn[8];
    if (with_q) ts_load_q<true>(r.qr, lo, r.V, qn);
    for (int t = 0; t < ntiles; ++t) {
        const int i0 = t * kTsTile + lo;
        float z[8], q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = qn[e];
        if (with_q && t + 1 < ntiles) ts_load_q<true>(r.qr, i0 + kTsTile, r.V, qn);
        r.get_z(t, z);
        f(t, i0, z, q);
    }
}

// The walk's fp32 view of the current node.  After rejections at the node,
// P(v) = max(0, P_0(v) - cq Q(v)) * invD: each rejection with mass S > 0 adds
// D to cq and multiplies D by S (a rejection with S = 0 changes nothing), which
// is the residual recursion max(0, P - Q)/S unrolled.
template <bool TR>
struct Dist32 {
    float m, k32;          // row maximum, log2(e)/T
    float invT;
    float invZ, invSq;
    float cq, invD;
    __device__ __forceinline__ float e_of(float z) const { return __builtin_amdgcn_exp2f((z - m) * k32); }
    __device__ __forceinline__ float w_of(float q) const {
        if (!TR) return q;
        return q > 0.f ? __builtin_amdgcn_exp2f(__builtin_amdgcn_logf(q) * invT) : 0.f;
    }
    __device__ __forceinline__ float Q_of(float q) const { return TR ? w_of(q) * invSq : q; }
    __device__ __forceinline__ float P_of(float e, float Q) const { return fmaxf(e * invZ - cq * Q, 0.f) * invD; }
};

// The final node's fp64 view.
template <int DT, bool TR>
struct Dist64 {
    const double* etab;    // bf16: exp((z - m)/T) of every tabulated logit value
    const double* tbl;
    ExpArg g;
    ExpConsts ek;
    double invZ, qk1, invSq;
    const double* sinv;
    const int* kept;

    __device__ __forceinline__ double e_of(float z) const {
        if (DT == 1) {
            const uint32_t h = __float_as_uint(z) >> 16;
            const uint32_t off = (h & 0x7fffu) - kTabLo;
            if (off < kTabSpan) return etab[off + ((h & 0x8000u) ? kTabSpan : 0u)];
        }
        return exp_of(z, g, tbl, ek);
    }
    __device__ __forceinline__ double w_of(float q) const {
        if (!TR) return static_cast<double>(q);
        return q > 0.f ? exp_scaled(log(static_cast<double>(q)) * qk1, tbl, ek) : 0.0;
    }
    __device__ __forceinline__ double Q_of(float q) const { return TR ? w_of(q) * invSq : static_cast<double>(q); }
    __device__ __forceinline__ double P_of(double e, double Q, int upto) const {
        double P = e * invZ;
        for (int j = 0; j < upto; ++j) P = kept[j] ? P : fmax(P - Q, 0.0) * sinv[j];
        return P;
    }
};

template <int DT, bool VEC, bool TR, bool LROW>
__global__ __launch_bounds__(kTsThreads, 1) void tree_sample_kernel(TreeSampleArgs a, ExpConsts ek) {
    extern __shared__ double dyn[];
    __shared__ TsSmem sm;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = wave_id();
    const int b = blockIdx.x, N = a.N, V = a.V;
    const long esz = Elem<DT>::kBytes;
    const int ntiles = (V + kTsTile - 1) / kTsTile;
    const int nvec = static_cast<int>(static_cast<long>(V) * esz / 16);
    for (int t = tid; t < kTableSize; t += kTsThreads) sm.tbl[t] = exp2(static_cast<double>(t) * (1.0 / kTableSize));
    const int32_t* tok = a.node_tokens + static_cast<long>(b) * N;
    const float* ub = a.u + static_cast<long>(b) * N;
    const char* zbase = static_cast<const char*>(a.logits) + static_cast<long>(b) * N * V * esz;
    const float* qbase = a.q + static_cast<long>(b) * N * V;

    // The tree: the static one of the arguments, or the batch row's own, checked
    // (parents[0] = -1, 0 <= parents[n] < n) and linked here.
    int bad = 0;
    if (a.parents_rows) {
        if (tid < N) {
            const int p = a.parents_rows[static_cast<long>(b) * N + tid];
            bad |= tid == 0 ? p != -1 : (p < 0 || p >= tid);
            sm.par[tid] = p;
        }
        __syncthreads();
        if (tid == 0) {
            // pushing children in decreasing node order leaves each list increasing
            for (int n = 0; n < N; ++n) sm.fch[n] = sm.nsib[n] = -1;
            for (int n = N - 1; n >= 1; --n) {
                const int p = sm.par[n];
                if (p < 0 || p >= n) continue;                  // (an error row)
                sm.nsib[n] = sm.fch[p];
                sm.fch[p] = n;
            }
        }
    } else if (tid < N) {
        sm.par[tid] = a.parent[tid];
        sm.fch[tid] = a.first_child[tid];
        sm.nsib[tid] = a.next_sibling[tid];
    }
    // E2 (every node token) and E5 (every uniform).
    if (tid < N) {
        bad |= !u_ok(ub[tid]);
        if (tid > 0) bad |= (tok[tid] < 0 || tok[tid] >= V);
    }
    int err = ts_block_or(bad, sm);

    // LDS: two row buffers (LROW; the final node's fp64 table goes into the one
    // not holding its row) or the table alone.
    u32x4* buf_cur = reinterpret_cast<u32x4*>(dyn);
    u32x4* buf_next = buf_cur + kTsRowBytes / 16;
    bool have_next = false;

    Dist32<TR> d32;
    d32.k32 = kLog2e * static_cast<float>(a.invT);
    d32.invT = static_cast<float>(a.invT);
    NodeRow<DT, VEC, LROW> row;
    row.V = V;
    row.zs = buf_cur;
    int c = 0, d = 0, nrej = 0;
    float m = 0.f;
    double Zw = 1.0, Sqw = 1.0;      // the walk's normalisers at the current node (fp32 terms)
    if (tid == 0) sm.path[0] = 0;
    while (!err) {
        const char* zr = zbase + static_cast<long>(c) * V * esz;
        const float* qr = qbase + static_cast<long>(c) * V;
        row.zr = zr;
        row.qr = qr;
        const int first = sm.fch[c];
        // Loads, in this order: the node's row unless parked already, the tested
        // children's z[x_n] and q[x_n] (lanes of wave 0), then the first child's
        // row.  The memory counter retires in order, so waiting for one set never
        // waits for a later one.
        u32x4 cur[kTsRowVecs], pf[kTsRowVecs];
        if constexpr (LROW) {
            if (have_next) {
                u32x4* t = buf_cur;
                buf_cur = buf_next;
                buf_next = t;
            } else {
                row_issue(zr, nvec, cur);
            }
        }
        float gz = 0.f, gq = 0.f;
        const bool gl = wid == 0 && lane > 0 && lane < N && sm.par[lane] == c;
        if (gl) {
            const int x = tok[lane];
            gz = Elem<DT>::scalar(zr, x);
            gq = qr[x];
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (LROW) {
            if (first >= 0) row_issue(zbase + static_cast<long>(first) * V * esz, nvec, pf);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (LROW) {
            if (!have_next) row_park(buf_cur, nvec, cur);
        }
        if (gl) {
            sm.gz[lane] = gz;
            sm.gq[lane] = gq;
        }
        have_next = false;
        row.zs = buf_cur;
        __syncthreads();

        // Row maximum; E1 for NaN, +inf or a row of -inf only.
        float mx = -INFINITY;
        for_tiles(row, ntiles, false, [&](int, int, const float* z, const float*) {
            mx = maximum3(maximum3(mx, z[0], z[1]), maximum3(z[2], z[3], z[4]), maximum3(z[5], z[6], z[7]));
        });
        const unsigned long long rbw = __ballot(!(mx < INFINITY));     // NaN (propagated) or +inf
        mx = wave_max(mx);
        if (lane == 0) {
            sm.fred[wid] = mx;
            sm.ired[wid] = rbw != 0ull;
        }
        __syncthreads();
        m = sm.fred[0];
        int rb = sm.ired[0];
#pragma unroll
        for (int w = 1; w < kTsWaves; ++w) {
            m = fmaxf(m, sm.fred[w]);
            rb |= sm.ired[w];
        }
        __syncthreads();
        if (rb || m == -INFINITY) { err = 1; break; }
        nrej = 0;
        if (first < 0) break;                                           // a leaf: the draw is here

        // The walk's tests in fp32: normalisers, then the children in node order.
        d32.m = m;
        double Z = 0.0, Sq = 0.0;
        int qb = 0;
        for_tiles(row, ntiles, TR, [&](int, int, const float* z, const float* q) {
            float s = 0.f, sq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                s += d32.e_of(z[e]);
                if (TR) {
                    qb |= !q_ok(q[e]);
                    sq += d32.w_of(q[e]);
                }
            }
            Z += static_cast<double>(s);
            if (TR) Sq += static_cast<double>(sq);
        });
        if constexpr (LROW) {
            // park the first child's row (its loads have had the passes above to land);
            // the barriers below order these stores before the next node reads them
            if (first >= 0) row_park(buf_next, nvec, pf);
        }
        Z = ts_block_sum(Z, sm);
        if (TR) {
            Sq = ts_block_sum(Sq, sm);
            qb = ts_block_or(qb, sm);
            if (qb || !(Sq > 0.0)) { err = 1; break; }                  // E3, E4
        }
        d32.invZ = static_cast<float>(1.0 / Z);
        d32.invSq = TR ? static_cast<float>(1.0 / Sq) : 1.f;
        d32.cq = 0.f;
        d32.invD = 1.f;
        double Dw = 1.0;                 // D of the closed form, kept in fp64
        Zw = Z;
        Sqw = TR ? Sq : 1.0;
        int accepted = -1, q_checked = 0;
        for (int n = first; n >= 0; n = sm.nsib[n]) {
            if (tid == 0) {
                const float zx = sm.gz[n];
                const float qx = sm.gq[n];
                int dec = 0;
                if (!TR && !q_ok(qx)) {
                    dec = 2;                                                 // E3
                } else {
                    const float Qx = d32.Q_of(qx);
                    const float Px = d32.P_of(d32.e_of(zx), Qx);
                    float ratio;
                    if (Qx > 0.f) ratio = Px / Qx;
                    else ratio = Px > 0.f ? INFINITY : 0.f;
                    const float thr = ratio < 1.f ? ratio : 1.f;
                    dec = ub[n] < thr ? 1 : 0;
                }
                sm.dec = dec;
            }
            __syncthreads();
            const int dec = sm.dec;
            __syncthreads();
            if (dec == 2) { err = 1; break; }
            if (dec == 1) { accepted = n; break; }
            // Rejected: S = sum_v max(0, P(v) - Q(v)); an untransformed draft row is
            // checked whole the first time a residual reads it (E3).
            const bool check_q = !TR && !q_checked;
            double S = 0.0;
            qb = 0;
            for_tiles(row, ntiles, true, [&](int, int, const float* z, const float* q) {
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (check_q) qb |= !q_ok(q[e]);
                    const float Qv = d32.Q_of(q[e]);
                    s += fmaxf(d32.P_of(d32.e_of(z[e]), Qv) - Qv, 0.f);
                }
                S += static_cast<double>(s);
            });
            S = ts_block_sum(S, sm);
            if (check_q) {
                q_checked = 1;
                if (ts_block_or(qb, sm)) { err = 1; break; }
            }
            if (tid == 0) {
                sm.kept32[nrej] = !(S > 0.0);
                sm.sinv32[nrej] = S > 0.0 ? static_cast<float>(1.0 / S) : 1.f;
            }
            if (S > 0.0) {                   // (S is the same in every thread)
                d32.cq += static_cast<float>(Dw);
                Dw *= S;
                d32.invD = static_cast<float>(1.0 / Dw);
            }
            __syncthreads();
            ++nrej;
        }
        if constexpr (LROW) have_next = !err && first >= 0 && accepted == first;
        if (err || accepted < 0) break;
        ++d;
        c = accepted;
        if (tid == 0) {
            sm.path[d] = c;
            sm.toks[d - 1] = tok[c];
        }
    }

    // The final node c, nrej = R rejections there, in fp64.  Without a kept step,
    // after j rejections P_j(v) = max(0, P_0(v) - c_j Q_v) / D_j with c_0 = 0,
    // D_0 = 1, c_{j+1} = c_j + D_j, D_{j+1} = D_j S_j, so every residual mass is a
    // hinge sum of the node's first distribution:
    //     S_j = sum_v max(0, e_v - lam_j y_v) / (Z D_j),   lam_j = (c_j + D_j) Z / Sq
    // (e_v = exp((z_v - m)/T), y_v the draft weight, Sq its sum; Sq = 1 untransformed).
    // The walk's fp32 S's give each lam_j to ~1e-6, so one pass sorts every element
    // against lam_j (1 -+ kTsBracket): above (sum e_v and y_v), below (nothing), or
    // between (listed).  The exact lam_j then follow in order from those sums, each
    // checked to lie inside its bracket.  The same pass leaves the segment sums of the
    // draw's weights: e_v (no rejection) or max(0, e_v - lam_{R-1} y_v).  A kept
    // step, more than kTsFastRej rejections, a full list or a point outside its
    // bracket take the multi-pass route instead (one fp64 pass per S_j).
    int y = -1;
    if (!err) {
        __syncthreads();                 // every thread is done with the walk's LDS rows
        double* etab = LROW ? reinterpret_cast<double*>(buf_next) : dyn;
        double* partE = dyn + (LROW ? 2 * kTsRowBytes / 8 : (DT == 1 ? kTabBytes / 8 : 0));
        double* partY = partE + ts_parts_cap<DT, LROW>();
        const float* qr = qbase + static_cast<long>(c) * V;
        const int R = nrej;
        Dist64<DT, TR> d64;
        d64.etab = etab;
        d64.tbl = sm.tbl;
        d64.ek = ek;
        d64.g = exp_arg(static_cast<double>(m), a.invT, ek);
        d64.qk1 = a.invT * ek.scale;
        d64.sinv = sm.sinv;
        d64.kept = sm.kept;
        if (tid == 0) {
            sm.n_list = 0;
            sm.last_list = -1;
        }
        if (DT == 1) build_exp_table(etab, d64.g, sm.tbl, ek);
        __syncthreads();
        const bool with_q = R > 0;
        const int nparts = ntiles * kTsWaves;
        auto seg_sum = [&](double* part, int t, double v) {
            v = wave_sum(v);
            if (lane == 0) part[t * kTsWaves + wid] = v;
        };
        // The walk's points and their brackets (every thread computes the same).
        bool fast = a.onepass && R <= kTsFastRej;
        double lamLo[kTsFastRej], lamHi[kTsFastRej];
        {
            double cc = 0.0, DD = 1.0;
#pragma unroll
            for (int j = 0; j < kTsFastRej; ++j) {
                lamLo[j] = lamHi[j] = 0.0;
                if (j < R) {
                    fast = fast && !sm.kept32[j];
                    const double lam = (cc + DD) * Zw / Sqw;
                    lamLo[j] = uniform_d(lam * (1.0 - kTsBracket));
                    lamHi[j] = uniform_d(lam * (1.0 + kTsBracket));
                    cc += DD;
                    DD *= 1.0 / static_cast<double>(sm.sinv32[j]);
                }
            }
        }
        int mode = 0;            // draw weights: 0 e_v, 1 the hinge max(0, e_v - lam y_v), 2 and 3 the
        int last = -1;           // multi-pass route's residual and kept P
        if (fast) {
            double Zs = 0.0, Sqs = 0.0, Ej[kTsFastRej], Yj[kTsFastRej];
#pragma unroll
            for (int j = 0; j < kTsFastRej; ++j) Ej[j] = Yj[j] = 0.0;
            for_tiles(row, ntiles, with_q, [&](int t, int i0, const float* z, const float* q) {
                double sE = 0.0, sY = 0.0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const double ev = d64.e_of(z[e]);
                    Zs += ev;
                    if (R == 0) {
                        sE += ev;
                        if (ev > 0.0) last = i0 + e;
                        continue;
                    }
                    const double yv = d64.w_of(q[e]);
                    Sqs += yv;
#pragma unroll
                    for (int j = 0; j < kTsFastRej; ++j) {
                        if (j >= R) continue;
                        const bool pos = ev > lamHi[j] * yv;
                        Ej[j] += pos ? ev : 0.0;
                        Yj[j] += pos ? yv : 0.0;
                        if (j == R - 1) {
                            sE += pos ? ev : 0.0;
                            sY += pos ? yv : 0.0;
                            last = pos ? i0 + e : last;
                        }
                        const bool und = !pos && ev > lamLo[j] * yv;
                        if (__ballot(und)) {             // rare: a few elements per row
                            if (und) {
                                const int k = atomicAdd(&sm.n_list, 1);
                                if (k < kTsListCap) {
                                    sm.li_v[k] = i0 + e;
                                    sm.li_j[k] = j;
                                    sm.li_e[k] = ev;
                                    sm.li_y[k] = yv;
                                }
                            }
                        }
                    }
                }
                seg_sum(partE, t, sE);
                if (R > 0) seg_sum(partY, t, sY);
            });
            // block sums of Z, Sq and the per-point sums in one exchange
            {
                double v[2 + 2 * kTsFastRej];
                v[0] = Zs;
                v[1] = Sqs;
#pragma unroll
                for (int j = 0; j < kTsFastRej; ++j) {
                    v[2 + 2 * j] = Ej[j];
                    v[3 + 2 * j] = Yj[j];
                }
#pragma unroll
                for (int k = 0; k < 2 + 2 * kTsFastRej; ++k) {
                    const double w = wave_sum(v[k]);
                    if (lane == 0) sm.redn[wid][k] = w;
                }
            }
            last = ts_block_max(last, sm);       // (its barriers also publish redn, the list and the parts)
            if (wid == 0) {
                // lane k sums value k over the waves; every lane then holds all of them
                double tk = 0.0;
                if (lane < 2 + 2 * kTsFastRej)
                    for (int w = 0; w < kTsWaves; ++w) tk += sm.redn[w][lane];
                double tot[2 + 2 * kTsFastRej];
#pragma unroll
                for (int k = 0; k < 2 + 2 * kTsFastRej; ++k) tot[k] = bcast(tk, k);
                const double Z = tot[0];
                const double Sq = TR && R > 0 ? tot[1] : 1.0;
                const int nl = sm.n_list;
                int ok = nl <= kTsListCap;
                double cc = 0.0, DD = 1.0, lam = 0.0;
#pragma unroll
                for (int j = 0; j < kTsFastRej; ++j) {
                    if (j >= R || !ok) continue;
                    lam = (cc + DD) * Z / Sq;
                    ok = lam >= lamLo[j] && lam <= lamHi[j];
                    double G = tot[2 + 2 * j] - lam * tot[3 + 2 * j];
                    for (int k = 0; k < nl; ++k)
                        if (sm.li_j[k] == j) G += fmax(sm.li_e[k] - lam * sm.li_y[k], 0.0);
                    const double S = G / (Z * DD);
                    ok = ok && S > 0.0;
                    cc += DD;
                    DD *= S;
                }
                int ll = -1;
                if (ok && R > 0) {
                    for (int k = 0; k < nl; ++k)
                        if (sm.li_j[k] == R - 1 && sm.li_e[k] - lam * sm.li_y[k] > 0.0) ll = max(ll, sm.li_v[k]);
                }
                if (lane == 0) {
                    sm.fast_ok = ok;
                    sm.lam_last = lam;
                    sm.last_list = ll;
                }
            }
            __syncthreads();
            fast = sm.fast_ok != 0;
            if (fast && R > 0) {
                // the draw's segment sums at the exact point, then the listed elements
                const double lam = sm.lam_last;
                for (int p = tid; p < nparts; p += kTsThreads) partE[p] = partE[p] - lam * partY[p];
                __syncthreads();
                if (tid == 0) {
                    const int nl = sm.n_list;
                    for (int k = 0; k < nl; ++k) {
                        if (sm.li_j[k] != R - 1) continue;
                        const int v = sm.li_v[k];
                        partE[(v / kTsTile) * kTsWaves + (v % kTsTile) / 8 / kWave] +=
                            fmax(sm.li_e[k] - lam * sm.li_y[k], 0.0);
                    }
                }
                last = max(last, sm.last_list);
                mode = 1;
            }
        }
        if (!fast) {
            // Multi-pass route: the normalisers, then one pass per rejection.
            mode = R == 0 ? 0 : 2;
            last = -1;
            double Z = 0.0, Sq = 0.0;
            for_tiles(row, ntiles, TR && R > 0, [&](int t, int i0, const float* z, const float* q) {
                double s = 0.0, sq = 0.0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const double ev = d64.e_of(z[e]);
                    s += ev;
                    if (ev > 0.0) last = i0 + e;
                    if (TR && R > 0) sq += d64.w_of(q[e]);
                }
                Z += s;
                Sq += sq;
                if (R == 0) seg_sum(partE, t, s);
            });
            Z = ts_block_sum(Z, sm);
            if (TR && R > 0) Sq = ts_block_sum(Sq, sm);
            d64.invZ = 1.0 / Z;
            d64.invSq = TR && R > 0 ? 1.0 / Sq : 1.0;
            for (int j = 0; j < R; ++j) {
                const bool lastj = j == R - 1;
                if (lastj) last = -1;
                double S = 0.0;
                for_tiles(row, ntiles, true, [&](int t, int i0, const float* z, const float* q) {
                    double s = 0.0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const double Qv = d64.Q_of(q[e]);
                        const double r = fmax(d64.P_of(d64.e_of(z[e]), Qv, j) - Qv, 0.0);
                        s += r;
                        if (lastj && r > 0.0) last = i0 + e;
                    }
                    S += s;
                    if (lastj) seg_sum(partE, t, s);
                });
                S = ts_block_sum(S, sm);
                if (tid == 0) {
                    sm.kept[j] = !(S > 0.0);
                    sm.sinv[j] = S > 0.0 ? 1.0 / S : 1.0;
                }
                __syncthreads();
            }
            if (R > 0 && sm.kept[R - 1]) {
                mode = 3;
                last = -1;
                for_tiles(row, ntiles, true, [&](int t, int i0, const float* z, const float* q) {
                    double s = 0.0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const double P = d64.P_of(d64.e_of(z[e]), d64.Q_of(q[e]), R);
                        s += P;
                        if (P > 0.0) last = i0 + e;
                    }
                    seg_sum(partE, t, s);
                });
            }
        }
        last = ts_block_max(last, sm);       // (its barrier also publishes the parts)
        if (wid == 0) {
            // Lane l sums a run of consecutive segments; an inclusive scan of the
            // runs, then a serial walk inside the run that crosses u*S.
            const int per = (nparts + kWave - 1) / kWave;
            double run = 0.0;
            for (int j = 0; j < per; ++j) {
                const int p = lane * per + j;
                if (p < nparts) run += partE[p];
            }
            const double incl = wave_inclusive_scan(run);
            const double S = bcast(incl, kWave - 1);
            const double target = static_cast<double>(ub[0]) * S;
            const unsigned long long hit = __ballot(target < incl);
            int seg = -1;
            double base = 0.0;
            if (hit) {
                const int l = __ffsll(static_cast<long long>(hit)) - 1;
                double acc = bcast(incl - run, l);
                for (int j = 0; j < per; ++j) {
                    const int p = l * per + j;
                    if (p >= nparts) break;
                    const double nxt = acc + partE[p];
                    if (target < nxt) { seg = p; break; }
                    acc = nxt;
                }
                base = acc;
            }
            if (lane == 0) {
                sm.seg = seg;
                sm.base = base;
                sm.red[0] = target;
            }
        }
        __syncthreads();
        const int seg = sm.seg;
        if (seg < 0) {
            y = last;                                   // rounding fallback
        } else if (wid == seg % kTsWaves) {
            const int ts = seg / kTsWaves;
            const int i0 = ts * kTsTile + 8 * tid;
            const double target = sm.red[0];
            const double lam = sm.lam_last;
            float z[8], q[8];
            row.get_z(ts, z);
            if (with_q) ts_load_q<VEC>(qr, i0, V, q);
            double w[8], s = 0.0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double ev = d64.e_of(z[e]);
                if (mode == 0) {
                    w[e] = ev;
                } else if (mode == 1) {
                    w[e] = fmax(ev - lam * d64.w_of(q[e]), 0.0);
                } else {
                    const double Qv = d64.Q_of(q[e]);
                    w[e] = mode == 2 ? fmax(d64.P_of(ev, Qv, R - 1) - Qv, 0.0) : d64.P_of(ev, Qv, R);
                }
                s += w[e];
            }
            const double incl = sm.base + wave_inclusive_scan(s);
            const unsigned long long hit = __ballot(target < incl);
            int yy;
            if (hit) {
                const int l = __ffsll(static_cast<long long>(hit)) - 1;
                int pick = -1;
                if (lane == l) {
                    double acc = incl - s;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        acc += w[e];
                        if (pick < 0 && w[e] > 0.0 && target < acc) pick = i0 + e;
                    }
                    if (pick < 0) {                      // rounding inside the lane: its last positive
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (w[e] > 0.0) pick = i0 + e;
                    }
                }
                yy = bcast(pick, l);
            } else {
                // rounding between the segment sums and this scan: the segment's last positive
                int lp = -1;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (w[e] > 0.0) lp = i0 + e;
                yy = wave_max_int(lp);
            }
            if (lane == 0) sm.seg = yy;
        }
        __syncthreads();
        if (seg >= 0) y = sm.seg;
    }

    // Outputs: path, accepted tokens and the drawn one, -1 padded.
    const long ob = static_cast<long>(b) * (a.D + 1);
    for (int t = tid; t <= a.D; t += kTsThreads) {
        const bool ok = !err && t <= d;
        a.out_path[ob + t] = ok ? sm.path[t] : -1;
        a.out_tokens[ob + t] = ok ? (t < d ? sm.toks[t] : y) : -1;
    }
    if (tid == 0) a.out_accept_len[b] = err ? -1 : d;
}

template <int DT, bool VEC, bool TR, bool LROW>
hipError_t ts_launch(const TreeSampleArgs& a, hipStream_t s, Timing t) {
    // LDS row buffers (or the fp64 table), then two arrays of segment sums
    const unsigned parts = ts_parts_cap<DT, LROW>();
    const unsigned lds = (LROW ? 2u * kTsRowBytes : (DT == 1 ? static_cast<unsigned>(kTabBytes) : 0u)) +
                         2u * parts * static_cast<unsigned>(sizeof(double));
    launch_timed(t, tree_sample_kernel<DT, VEC, TR, LROW>, dim3(a.B), dim3(kTsThreads), lds, s, a, exp_consts());
    return hipGetLastError();
}

template <int DT>
hipError_t ts_dispatch(const TreeSampleArgs& a, hipStream_t s, Timing t) {
    // 16-byte vectors: 8 elements per load need V a multiple of 8 and aligned rows.
    const bool vec = a.V % 8 == 0 && vec_ok(a.logits, a.V, Elem<DT>::kBytes) && vec_ok(a.q, a.V, 4);
    const bool lrow = vec && static_cast<long>(a.V) * Elem<DT>::kBytes <= kTsRowBytes;
    if (a.transformed) {
        if (lrow) return ts_launch<DT, true, true, true>(a, s, t);
        return vec ? ts_launch<DT, true, true, false>(a, s, t) : ts_launch<DT, false, true, false>(a, s, t);
    }
    if (lrow) return ts_launch<DT, true, false, true>(a, s, t);
    return vec ? ts_launch<DT, true, false, false>(a, s, t) : ts_launch<DT, false, false, false>(a, s, t);
}

static_assert(kTabBytes <= kTsRowBytes, "the final node's fp64 table fits the spare row buffer");

}  // namespace

hipError_t launch_tree_sample(const TreeSampleArgs& a, hipStream_t s, Timing t) {
    if (a.N > kTsMaxNodes || a.V > kMaxV) return hipErrorInvalidValue;
    return a.dtype == 1 ? ts_dispatch<1>(a, s, t) : ts_dispatch<0>(a, s, t);
}

}  // namespace sv
