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
// Every probability is fp64 (a draw over a wide distribution needs every weight
// to fp64 accuracy).  The passes over a row recompute P(v) from the logit
// (one table-driven fp64 exponential: the bf16 logits of a row take few
// distinct values, looked up in an LDS table built per node) and the chain of
// residual normalisers, instead of storing intermediate rows: the only
// memory traffic is the rows themselves, re-read from L2 after the first pass.
// Passes at node c: the row maximum (and E1 flags), the normalisers Z (and Sq
// when the draft is transformed), one pass per rejected sibling (its S), and
// for the final draw one pass of per-segment sums plus the rescan of the
// segment that holds u*S.

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

struct TsSmem {
    double tbl[kTableSize];          // 2^(k/256) for the fp64 exponential
    double part[kTsParts];           // segment sums of the draw pass, in index order
    double red[kTsWaves];
    float fred[kTsWaves];
    int ired[kTsWaves];
    double sinv[kTsMaxNodes];        // 1/S of each rejection at the current node (1 when kept)
    int kept[kTsMaxNodes];           // 1: that rejection left P as it was (S = 0)
    int path[kTsMaxNodes];
    int toks[kTsMaxNodes];
    int dec;                         // thread 0's decision: 0 reject, 1 accept, 2 error
    int seg;                         // draw: segment holding u*S, -1 for the fallback
    double base;                     // draw: mass before that segment
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

// Everything a pass needs to turn one (logit, draft probability) pair into the
// current P(v) and Q(v).
template <int DT, bool TR>
struct NodeDist {
    const double* etab;    // bf16: exp of every tabulated logit value at this node
    const double* tbl;
    ExpArg g;
    ExpConsts ek;
    double invZ;           // 1 / sum_v exp((z_v - m)/T)
    double qk1;            // transformed draft: invT * 256/ln2
    double invSq;          // transformed draft: 1 / sum_v q_v^(1/T)
    int nrej;              // rejections so far at this node
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
    // q^(1/T) in fp64 (0 stays 0); as given when the draft is untransformed.
    __device__ __forceinline__ double w_of(float q) const {
        if (!TR) return static_cast<double>(q);
        return q > 0.f ? exp_scaled(log(static_cast<double>(q)) * qk1, tbl, ek) : 0.0;
    }
    __device__ __forceinline__ double Q_of(float q) const { return TR ? w_of(q) * invSq : static_cast<double>(q); }
    // P(v) after the first `upto` rejections at this node.
    __device__ __forceinline__ double P_of(double e, double Q, int upto) const {
        double P = e * invZ;
        for (int j = 0; j < upto; ++j) P = kept[j] ? P : fmax(P - Q, 0.0) * sinv[j];
        return P;
    }
};

template <int DT, bool VEC, bool TR>
__global__ __launch_bounds__(kTsThreads, 1) void tree_sample_kernel(TreeSampleArgs a, ExpConsts ek) {
    extern __shared__ double etab[];
    __shared__ TsSmem sm;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = wave_id();
    const int b = blockIdx.x, N = a.N, V = a.V;
    const long esz = Elem<DT>::kBytes;
    const int ntiles = (V + kTsTile - 1) / kTsTile;
    for (int t = tid; t < kTableSize; t += kTsThreads) sm.tbl[t] = exp2(static_cast<double>(t) * (1.0 / kTableSize));
    const int32_t* tok = a.node_tokens + static_cast<long>(b) * N;
    const float* ub = a.u + static_cast<long>(b) * N;

    // E2 (every node token) and E5 (every uniform).
    int bad = 0;
    if (tid < N) {
        bad |= !u_ok(ub[tid]);
        if (tid > 0) bad |= (tok[tid] < 0 || tok[tid] >= V);
    }
    int err = ts_block_or(bad, sm);

    int c = 0, d = 0;
    if (tid == 0) sm.path[0] = 0;
    NodeDist<DT, TR> nd;
    nd.etab = etab;
    nd.tbl = sm.tbl;
    nd.ek = ek;
    nd.qk1 = a.invT * ek.scale;
    nd.sinv = sm.sinv;
    nd.kept = sm.kept;
    const char* zr = nullptr;
    const float* qr = nullptr;
    while (!err) {
        zr = static_cast<const char*>(a.logits) + (static_cast<long>(b) * N + c) * V * esz;
        qr = a.q + (static_cast<long>(b) * N + c) * V;
        // Row maximum; E1 for NaN, +inf or a row of -inf only.
        float m = -INFINITY;
        int rb = 0;
        for (int t = 0; t < ntiles; ++t) {
            float z[8];
            ts_load_z<DT, VEC>(zr, t * kTsTile + 8 * tid, V, z);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                rb |= (z[e] != z[e]) || z[e] == INFINITY;
                m = fmaxf(m, z[e]);
            }
        }
        m = wave_max(m);
        if (lane == 0) sm.fred[wid] = m;
        rb = ts_block_or(rb, sm);
        m = sm.fred[0];
#pragma unroll
        for (int w = 1; w < kTsWaves; ++w) m = fmaxf(m, sm.fred[w]);
        if (rb || m == -INFINITY) { err = 1; break; }
        nd.g = exp_arg(static_cast<double>(m), a.invT, ek);
        if (DT == 1) {
            build_exp_table(etab, nd.g, sm.tbl, ek);
            __syncthreads();
        }
        // Normalisers: Z of the target row, Sq of a transformed draft row (with E3).
        const int first = a.first_child[c];
        const bool need_q = TR && first >= 0;
        double Z = 0.0, Sq = 0.0;
        int qb = 0;
        for (int t = 0; t < ntiles; ++t) {
            const int i0 = t * kTsTile + 8 * tid;
            float z[8], q[8];
            ts_load_z<DT, VEC>(zr, i0, V, z);
            if (need_q) ts_load_q<VEC>(qr, i0, V, q);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                Z += nd.e_of(z[e]);
                if (need_q) {
                    qb |= !q_ok(q[e]);
                    Sq += nd.w_of(q[e]);
                }
            }
        }
        Z = ts_block_sum(Z, sm);
        if (need_q) {
            Sq = ts_block_sum(Sq, sm);
            qb = ts_block_or(qb, sm);
            if (qb || !(Sq > 0.0)) { err = 1; break; }                               // E3, E4
        }
        nd.invZ = 1.0 / Z;
        nd.invSq = need_q ? 1.0 / Sq : 1.0;
        nd.nrej = 0;
        // Children in node order, each one round of the chain's test.
        int accepted = -1, q_checked = 0;
        for (int n = first; n >= 0; n = a.next_sibling[n]) {
            if (tid == 0) {
                const int x = tok[n];
                const float zx = Elem<DT>::scalar(zr, x);
                const float qx = qr[x];
                int dec = 0;
                if (!TR && !q_ok(qx)) {
                    dec = 2;                                                             // E3
                } else {
                    const double Qx = nd.Q_of(qx);
                    const double Px = nd.P_of(nd.e_of(zx), Qx, nd.nrej);
                    double ratio;
                    if (Qx > 0.0) ratio = Px / Qx;
                    else ratio = Px > 0.0 ? INFINITY : 0.0;
                    const double thr = ratio < 1.0 ? ratio : 1.0;
                    dec = static_cast<double>(ub[n]) < thr ? 1 : 0;
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
            for (int t = 0; t < ntiles; ++t) {
                const int i0 = t * kTsTile + 8 * tid;
                float z[8], q[8];
                ts_load_z<DT, VEC>(zr, i0, V, z);
                ts_load_q<VEC>(qr, i0, V, q);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (check_q) qb |= !q_ok(q[e]);
                    const double Qv = nd.Q_of(q[e]);
                    S += fmax(nd.P_of(nd.e_of(z[e]), Qv, nd.nrej) - Qv, 0.0);
                }
            }
            S = ts_block_sum(S, sm);
            if (check_q) {
                q_checked = 1;
                if (ts_block_or(qb, sm)) { err = 1; break; }
            }
            if (tid == 0) {
                sm.kept[nd.nrej] = !(S > 0.0);
                sm.sinv[nd.nrej] = S > 0.0 ? 1.0 / S : 1.0;
            }
            __syncthreads();
            ++nd.nrej;
        }
        if (err || accepted < 0) break;
        ++d;
        c = accepted;
        if (tid == 0) {
            sm.path[d] = c;
            sm.toks[d - 1] = tok[c];
        }
    }

    // Final draw from P at node c with u[0]: segment sums in index order, the
    // segment holding u*S, then that segment rescanned by the wave that owns it.
    int y = -1;
    if (!err) {
        int last = -1;
        for (int t = 0; t < ntiles; ++t) {
            const int i0 = t * kTsTile + 8 * tid;
            float z[8], q[8];
            ts_load_z<DT, VEC>(zr, i0, V, z);
            if (nd.nrej > 0) ts_load_q<VEC>(qr, i0, V, q);
            double s = 0.0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double Qv = nd.nrej > 0 ? nd.Q_of(q[e]) : 0.0;
                const double P = nd.P_of(nd.e_of(z[e]), Qv, nd.nrej);
                s += P;
                if (P > 0.0) last = i0 + e;
            }
            s = wave_sum(s);
            if (lane == 0) sm.part[t * kTsWaves + wid] = s;
        }
        last = ts_block_max(last, sm);       // (its barrier also publishes sm.part)
        const int nparts = ntiles * kTsWaves;
        if (wid == 0) {
            // Lane l sums a run of consecutive segments; an inclusive scan of the
            // runs, then a serial walk inside the run that crosses u*S.
            const int per = (nparts + kWave - 1) / kWave;
            double run = 0.0;
            for (int j = 0; j < per; ++j) {
                const int p = lane * per + j;
                if (p < nparts) run += sm.part[p];
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
                    const double nxt = acc + sm.part[p];
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
            const int t = seg / kTsWaves;
            const int i0 = t * kTsTile + 8 * tid;
            float z[8], q[8];
            ts_load_z<DT, VEC>(zr, i0, V, z);
            if (nd.nrej > 0) ts_load_q<VEC>(qr, i0, V, q);
            double P[8], s = 0.0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double Qv = nd.nrej > 0 ? nd.Q_of(q[e]) : 0.0;
                P[e] = nd.P_of(nd.e_of(z[e]), Qv, nd.nrej);
                s += P[e];
            }
            const double target = sm.red[0];
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
                        acc += P[e];
                        if (pick < 0 && P[e] > 0.0 && target < acc) pick = i0 + e;
                    }
                    if (pick < 0) {                      // rounding inside the lane: its last positive
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (P[e] > 0.0) pick = i0 + e;
                    }
                }
                yy = bcast(pick, l);
            } else {
                // rounding between the segment sums and this scan: the segment's last positive
                int lp = -1;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (P[e] > 0.0) lp = i0 + e;
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

template <int DT, bool VEC, bool TR>
hipError_t ts_launch(const TreeSampleArgs& a, hipStream_t s, Timing t) {
    const unsigned lds = DT == 1 ? static_cast<unsigned>(kTabBytes) : 0u;
    launch_timed(t, tree_sample_kernel<DT, VEC, TR>, dim3(a.B), dim3(kTsThreads), lds, s, a, exp_consts());
    return hipGetLastError();
}

template <int DT>
hipError_t ts_dispatch(const TreeSampleArgs& a, hipStream_t s, Timing t) {
    // 16-byte vectors: 8 elements per load need V a multiple of 8 and aligned rows.
    const bool vec = a.V % 8 == 0 && vec_ok(a.logits, a.V, Elem<DT>::kBytes) && vec_ok(a.q, a.V, 4);
    if (a.transformed) return vec ? ts_launch<DT, true, true>(a, s, t) : ts_launch<DT, false, true>(a, s, t);
    return vec ? ts_launch<DT, true, false>(a, s, t) : ts_launch<DT, false, false>(a, s, t);
}

}  // namespace

hipError_t launch_tree_sample(const TreeSampleArgs& a, hipStream_t s, Timing t) {
    if (a.N > kTsMaxNodes || a.V > kMaxV) return hipErrorInvalidValue;
    return a.dtype == 1 ? ts_dispatch<1>(a, s, t) : ts_dispatch<0>(a, s, t);
}

}  // namespace sv
