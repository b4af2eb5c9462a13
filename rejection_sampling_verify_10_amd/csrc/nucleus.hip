// Chain verification with the nucleus (top-p) transform on whole rows (top-k off).
//
// "064 · 投机解码", section 二: the sampling transforms are part of p and q, so
// the nucleus applies to both the target and the draft distributions.  After
// the temperature, a row keeps the shortest prefix of its tokens in probability
// order (lower index first among equal probabilities) whose mass reaches
// top_p, renormalised; a token of zero probability is never kept.
//
// nucleus_row_kernel finds that cut for every target and draft row, one
// workgroup of 1024 threads per row, in fp64:
//   1. the normaliser: Z = sum exp((z - m)/T) (m the row maximum) for a target
//      row, S = sum w, w = q^(1/T), for a draft row;
//   2. the boundary value by a radix select on the value's order key (bits
//      31..20, then 19..10, then 9..0): per level a histogram of the elements
//      that share the key prefix found so far, holding their count and their
//      probability mass in 62-bit fixed point (integer sums: exact whatever the
//      order of the atomic adds), and the bin where the mass taken from the top
//      reaches top_p;
//   3. the number n of elements of the boundary value that the cut keeps (they
//      are kept in index order), the index of the last of them, and the kept
//      mass P in fp64.
// A token i is then kept when its key exceeds the boundary key, or equals it
// with i at or before that index; its nucleus probability is p_i / P.
//
// nucleus_chain_kernel runs the ratio tests left to right from these rows'
// cuts and draws the emitted token by inverse CDF in index order (u_K) from the
// residual max(0, p'_j - q'_j) at the first rejection j, from p'_j when that
// residual has no mass, or from p'_K when every draft token passed; weights and
// sums in fp64 (one table-driven exponential per element, the draft's power in
// fp64), the draw's chunk sums first, then the rescan of the chunk holding u*W.

#include <math.h>

#include "common.hpp"
#include "exp64.hpp"
#include "internal.hpp"
#include "lists.hpp"

namespace sv {

namespace {

constexpr int kNT = 1024;                       // threads of a row's workgroup
constexpr int kNW = kNT / kWave;
constexpr int kLevels = 3;
__host__ __device__ constexpr int level_shift(int l) { return l == 0 ? 20 : (l == 1 ? 10 : 0); }
__host__ __device__ constexpr int level_bins(int l) { return l == 0 ? 4096 : 1024; }
constexpr int kMaxBins = 4096;

// Probability p in [0, 1] as a 62-bit fixed-point integer (rounded).
__device__ __forceinline__ unsigned long long fixp(double p) {
    return static_cast<unsigned long long>(p * 4611686018427387904.0 + 0.5);
}

struct NucSmem {
    uint32_t cnt[kMaxBins];
    unsigned long long mass[kMaxBins];
    double tbl[kTableSize];
    double red[kNW];
    unsigned long long ured[kNW];
    uint32_t bad;
    float fred[kNW];
    int ired[kNW];
    // the radix select
    uint32_t prefix;
    int bin;
    unsigned long long above;   // fixed-point mass of the elements above the prefix
    unsigned long long goal;    // top_p in fixed point, capped by the row's total
    int tie_last;
};

__device__ __forceinline__ double block_sum_d(double v, NucSmem& sm) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) sm.red[threadIdx.x / kWave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kNW; ++w) t += sm.red[w];
    return t;
}

// A row's values and their unnormalised weights: exp((z - m)/T) for a target
// row, q^(1/T) for a draft row (q as given at T == 1; 0 for q <= 0).
template <int DT, bool DRAFT>
struct RowView {
    const char* row;
    int V;
    double invT;
    bool plain;
    ExpArg g;
    const double* tbl;
    ExpConsts ek;
    __device__ __forceinline__ double weight(float v) const {
        if (DRAFT) {
            if (!(v > 0.f)) return 0.0;
            return plain ? static_cast<double>(v) : pow(static_cast<double>(v), invT);
        }
        return exp_of(v, g, tbl, ek);
    }
    // f(i, v) for the elements of this thread, chunk by chunk: with VEC thread t
    // takes the 16-byte vector t of each chunk of kNT vectors (so its elements
    // within a chunk are contiguous and follow those of thread t - 1); else one
    // element per thread per chunk.  Every thread runs the same chunks; f may
    // return true to end the loop after the current chunk (a block-uniform
    // decision, taken through `stop`).
    template <bool VEC, typename F>
    __device__ __forceinline__ void each(F f) const {
        constexpr int EPV = DRAFT ? 4 : Elem<DT>::kPerVec;
        if constexpr (VEC) {
            const int nvec = V / EPV;
            const u32x4* rv = reinterpret_cast<const u32x4*>(row);
            for (int c = 0; c < nvec; c += kNT) {
                const int g = c + static_cast<int>(threadIdx.x);
                if (g < nvec) {
                    const u32x4 w = load_stream(rv + g);
#pragma unroll
                    for (int e = 0; e < EPV; ++e)
                        f(g * EPV + e, DRAFT ? __uint_as_float(w[e]) : Elem<DT>::get(w, e));
                }
            }
        } else {
            for (int i = threadIdx.x; i < V; i += kNT)
                f(i, DRAFT ? reinterpret_cast<const float*>(row)[i] : Elem<DT>::scalar(row, i));
        }
    }
};

// The cut of target row r (DRAFT false) or draft row r.
template <int DT, bool DRAFT, bool VEC>
__device__ void nucleus_row(const NucleusArgs& a, const ExpConsts& ek, int r, NucleusRow* outp, NucSmem& sm) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = wave_id();
    const int V = a.V;
    const char* rowp = static_cast<const char*>(DRAFT ? static_cast<const void*>(a.q) : a.logits) +
                       static_cast<long>(r) * V * (DRAFT ? 4 : Elem<DT>::kBytes);
    for (int t = tid; t < kTableSize; t += kNT) sm.tbl[t] = exp2(static_cast<double>(t) * (1.0 / kTableSize));
    if (tid == 0) { sm.bad = 0u; sm.tie_last = -1; }
    __syncthreads();
    RowView<DT, DRAFT> rv{rowp, V, a.invT, a.plain != 0, ExpArg{0.0, 0.0}, sm.tbl, ek};
    NucleusRow out{};

    // 1. the row's validity, maximum (targets) and normaliser
    float mx = -INFINITY;
    bool bad = false;
    rv.template each<VEC>([&](int, float v) {
        if (DRAFT) bad |= !q_ok(v);
        else bad |= !(v < INFINITY);                 // NaN or +inf (E1)
        mx = fmaxf(mx, v);
    });
    mx = wave_max(mx);
    if (lane == 0) sm.fred[wid] = mx;
    if (__ballot(bad) && lane == 0) atomicOr(&sm.bad, 1u);
    __syncthreads();
    float M = sm.fred[0];
#pragma unroll
    for (int w = 1; w < kNW; ++w) M = fmaxf(M, sm.fred[w]);
    bad = sm.bad != 0u || (!DRAFT && M == -INFINITY);    // only -inf (E1)
    if (!DRAFT) rv.g = exp_arg(static_cast<double>(M), a.invT, ek);
    double norm = 0.0;
    if (!bad) {
        double s = 0.0;
        rv.template each<VEC>([&](int, float v) { s += rv.weight(v); });
        norm = block_sum_d(s, sm);
        if (!(norm > 0.0 && norm < INFINITY)) bad = true;     // E4 (drafts), or an overflow
    }
    if (bad) {
        if (tid == 0) {
            out.flags = 1u;
            outp[r] = out;
        }
        return;
    }
    const double invN = 1.0 / norm;

    // 2. radix select of the boundary key.  Tokens of probability below
    // tau = (1 - top_p) / (2V) hold less than (1 - top_p)/2 together, so the mass
    // taken from the top reaches top_p before them: they are left out (their
    // value lies below the boundary).  A value threshold skips their weights.
    const unsigned long long target = max(fixp(static_cast<double>(a.top_p)), 1ull);   // at least the top token
    const double tau = (1.0 - static_cast<double>(a.top_p)) / (2.0 * V);
    float vskip;                                  // values strictly below it have p < tau
    if (DRAFT) {
        const double qt = a.plain ? tau * norm : pow(tau * norm, 1.0 / a.invT);
        vskip = static_cast<float>(qt * (1.0 - 1e-9));
    } else {
        vskip = static_cast<float>(static_cast<double>(M) + log(tau * norm) / a.invT - 1e-6 * (1.0 + fabs(M)));
    }
    if (!(tau > 0.0)) vskip = -INFINITY;
    if (tid == 0) { sm.prefix = 0u; sm.above = 0ull; sm.goal = target; }
    int last_cnt = 0;
    for (int l = 0; l < kLevels; ++l) {
        const int sh = level_shift(l), nb = level_bins(l);
        const int psh = sh + (l == 0 ? 12 : 10);           // bits above this level
        for (int t = tid; t < nb; t += kNT) { sm.cnt[t] = 0u; sm.mass[t] = 0ull; }
        __syncthreads();
        const uint32_t prefix = sm.prefix;
        rv.template each<VEC>([&](int, float v) {
            if (!(v >= vskip)) return;
            const uint32_t key = order_key(v);
            if (l > 0 && (key >> psh) != prefix) return;
            const double p = rv.weight(v) * invN;
            if (!(p > 0.0)) return;
            const int bin = static_cast<int>((key >> sh) & static_cast<uint32_t>(nb - 1));
            atomicAdd(&sm.cnt[bin], 1u);
            atomicAdd(&sm.mass[bin], fixp(p));
        });
        __syncthreads();
        // Bins from the top: thread t holds bins nb-1-per*t .. nb-per-per*t.
        const int per = (nb + kNT - 1) / kNT;
        unsigned long long mine = 0ull;
        for (int e = 0; e < per; ++e) {
            const int bin = nb - 1 - (tid * per + e);
            if (bin >= 0) mine += sm.mass[bin];
        }
        // exclusive sums from the top, by waves of 64 threads (a sequential pass over
        // the wave totals, then lane scans): integers, so exact in any order
        unsigned long long incl = mine;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const unsigned long long tv = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += tv;
        }
        if (lane == kWave - 1) sm.ured[wid] = incl;
        __syncthreads();
        unsigned long long before = sm.above;
        for (int w = 0; w < wid; ++w) before += sm.ured[w];
        before += incl - mine;
        unsigned long long total = sm.above;
        for (int w = 0; w < kNW; ++w) total += sm.ured[w];
        // the mass can fall just short of top_p by rounding: then the cut keeps every
        // element of positive mass, whose lowest bin is found the same way
        const unsigned long long tgt = sm.goal < total ? sm.goal : total;
        int found = -1;
        unsigned long long above = 0ull;
        if (before < tgt && before + mine >= tgt) {
            unsigned long long c = before;
            for (int e = 0; e < per; ++e) {
                const int bin = nb - 1 - (tid * per + e);
                if (bin < 0) break;
                const unsigned long long mb = sm.mass[bin];
                if (c + mb >= tgt && mb > 0ull) { found = bin; above = c; break; }
                c += mb;
            }
        }
        __syncthreads();
        if (found >= 0) {
            sm.bin = found;
            sm.above = above;
            sm.goal = tgt;
        }
        __syncthreads();
        const int b = sm.bin;
        last_cnt = static_cast<int>(sm.cnt[b]);
        __syncthreads();
        if (tid == 0) sm.prefix = (prefix << (l == 0 ? 12 : 10)) | static_cast<uint32_t>(b);
        __syncthreads();
    }
    const uint32_t bkey = sm.prefix;
    const unsigned long long above = sm.above, goal = sm.goal;
    const float bval = order_value(bkey);
    const double pb = rv.weight(bval) * invN;
    const unsigned long long mb = fixp(pb);
    long long n = last_cnt;
    if (mb > 0ull) {
        const unsigned long long need = goal > above ? goal - above : 1ull;
        n = static_cast<long long>((need + mb - 1ull) / mb);
        n = n < 1 ? 1 : (n > last_cnt ? last_cnt : n);
    }

    // 3. The last kept element of the boundary value in index order (a scan of tie
    // counts, ended once it is found; every one of them when all are kept), and
    // the kept mass: the elements above the boundary from their exact fixed-point
    // sum, plus n times the boundary probability.
    if (n >= last_cnt) {
        if (tid == 0) sm.tie_last = V;
    } else {
        long long seen = 0;                       // boundary elements before this chunk
        constexpr int EPT = VEC ? (DRAFT ? 4 : Elem<DT>::kPerVec) : 1;
        const int step = kNT * EPT;
        for (int base = 0; base < V; base += step) {
            const int i0 = base + tid * EPT;
            int ties = 0;
            for (int e = 0; e < EPT; ++e) {
                const int i = i0 + e;
                if (i < V && order_key(DRAFT ? reinterpret_cast<const float*>(rowp)[i]
                                             : Elem<DT>::scalar(rowp, i)) == bkey)
                    ++ties;
            }
            int incl = ties;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const int tv = __shfl_up(incl, o, kWave);
                if (lane >= o) incl += tv;
            }
            __syncthreads();
            if (lane == kWave - 1) sm.ired[wid] = incl;
            __syncthreads();
            long long rank = seen + incl - ties;
            for (int w = 0; w < wid; ++w) rank += sm.ired[w];
            long long chunk_ties = 0;
            for (int w = 0; w < kNW; ++w) chunk_ties += sm.ired[w];
            if (ties > 0 && rank < n && rank + ties >= n) {
                long long rr = rank;
                for (int e = 0; e < EPT; ++e) {
                    const int i = i0 + e;
                    if (i >= V) break;
                    if (order_key(DRAFT ? reinterpret_cast<const float*>(rowp)[i] : Elem<DT>::scalar(rowp, i)) ==
                            bkey &&
                        ++rr == n) {
                        sm.tie_last = i;
                        break;
                    }
                }
            }
            seen += chunk_ties;
            if (seen >= n) break;                 // block-uniform: every thread has the same `seen`
        }
    }
    __syncthreads();
    if (tid == 0) {
        out.m = M;
        out.key = bkey;
        out.tie_last = sm.tie_last;
        out.flags = 0u;
        out.norm = norm;
        out.kept = static_cast<double>(above) * 0x1p-62 + static_cast<double>(n) * pb;
        outp[r] = out;
    }
}

// One launch for every row of a call: the rows_t target rows first, then the
// draft rows.
template <int DT, bool VEC>
__global__ __launch_bounds__(kNT, 1) void nucleus_row_kernel(NucleusArgs a, ExpConsts ek) {
    __shared__ NucSmem sm;
    const int r = blockIdx.x;
    if (r < a.rows_t) nucleus_row<DT, false, VEC>(a, ek, r, a.out_t, sm);
    else nucleus_row<0, true, VEC>(a, ek, r - a.rows_t, a.out_d, sm);
}

// ---- the chain ----

constexpr int kCT = 256;                          // threads of a batch row's workgroup
constexpr int kCW = kCT / kWave;
constexpr int kCE = 8;                            // contiguous elements per thread per chunk
constexpr int kCChunk = kCT * kCE;
constexpr int kCMaxChunks = (kMaxV + kCChunk - 1) / kCChunk;

struct ChainSmem {
    double tbl[kTableSize];
    double part[kCMaxChunks];
    double red[kCW];
    int ired[kCW];
    int j, err, chunk, fallback;
    double before;
};

__device__ __forceinline__ double csum(double v, ChainSmem& sm) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) sm.red[threadIdx.x / kWave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kCW; ++w) t += sm.red[w];
    return t;
}

// Kept by the nucleus of a row whose cut is c: a larger key, or the boundary key
// at or before the last kept index.
__device__ __forceinline__ bool kept_by(const NucleusRow& c, uint32_t key, int i) {
    return key > c.key || (key == c.key && i <= c.tie_last);
}

template <int DT>
__global__ __launch_bounds__(kCT) void nucleus_chain_kernel(NucleusChainArgs na, ExpConsts ek) {
    __shared__ ChainSmem sm;
    const ChainArgs& a = na.ch;
    const int b = blockIdx.x;
    const int K = a.K, V = a.V;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = wave_id();
    const long rbase = static_cast<long>(b) * (K + 1);
    float* diag = a.out_diag ? a.out_diag + static_cast<long>(b) * (2 * K + 2) : nullptr;
    const char* zb = static_cast<const char*>(a.logits) + rbase * V * Elem<DT>::kBytes;
    const bool plain = na.plain != 0;
    for (int t = tid; t < kTableSize; t += kCT) sm.tbl[t] = exp2(static_cast<double>(t) * (1.0 / kTableSize));
    __syncthreads();

    // Ratio tests from the rows' cuts, lanes k = 0..K of wave 0, as the
    // left-to-right walk sees them: position k consults target row k (E1), then,
    // for k < K, draft row k (E3, E4) and the test.
    if (tid < kWave) {
        const int k = lane;
        bool inputs_bad = false, rows_bad = false, rej = false;
        double pk = NAN, qk = NAN;
        if (k <= K) {
            inputs_bad |= !u_ok(a.u[rbase + k]);
            rows_bad |= na.trow[rbase + k].flags != 0u;
        }
        if (k < K) {
            const int x = a.x[static_cast<long>(b) * K + k];
            inputs_bad |= (x < 0 || x >= V);
            const NucleusRow dr = na.drow[static_cast<long>(b) * K + k];
            rows_bad |= dr.flags != 0u;
            if (x >= 0 && x < V && !rows_bad) {
                const NucleusRow tr = na.trow[rbase + k];
                const float z = Elem<DT>::scalar(zb + static_cast<long>(k) * V * Elem<DT>::kBytes, x);
                const double e = exp_of(z, exp_arg(static_cast<double>(tr.m), a.invT, ek), sm.tbl, ek);
                // p_i exactly as the row's cut formed it (times the normaliser's inverse),
                // so that a nucleus of one token has p' = 1 exactly
                pk = kept_by(tr, order_key(z), x) ? (e * (1.0 / tr.norm)) / tr.kept : 0.0;
                const float qv = a.q[(static_cast<long>(b) * K + k) * V + x];
                double w = 0.0;
                if (qv > 0.f) w = plain ? static_cast<double>(qv) : pow(static_cast<double>(qv), a.invT);
                qk = kept_by(dr, order_key(qv), x) ? (w * (1.0 / dr.norm)) / dr.kept : 0.0;
                double ratio;
                if (qk > 0.0) ratio = pk / qk;
                else ratio = pk > 0.0 ? INFINITY : 0.0;
                const double thr = ratio < 1.0 ? ratio : 1.0;
                rej = !(static_cast<double>(a.u[rbase + k]) < thr);
            }
        }
        const unsigned long long stop = __ballot(k <= K && (rows_bad || (k < K && rej)));
        const int j = stop ? __ffsll(static_cast<long long>(stop)) - 1 : K;
        const bool err = __ballot(inputs_bad) != 0ull || (stop && bcast(static_cast<int>(rows_bad), j) != 0);
        if (diag && k < K) {
            diag[k] = (err || k > j) ? NAN : static_cast<float>(pk);
            diag[K + k] = (err || k > j) ? NAN : static_cast<float>(qk);
        }
        if (lane == 0) { sm.j = j; sm.err = err; }
    }
    __syncthreads();
    const int j = sm.j;
    if (sm.err) {
        for (int t = tid; t <= K; t += kCT) a.out_tokens[rbase + t] = -1;
        if (tid == 0) a.out_accept_len[b] = -1;
        if (diag)
            for (int t = tid; t < 2 * K + 2; t += kCT) diag[t] = NAN;
        return;
    }

    // The draw: residual max(0, p'_j - q'_j) at a rejection, p'_K after the last position.
    const bool res = j < K;
    const NucleusRow tr = na.trow[rbase + j];
    const NucleusRow dr = res ? na.drow[static_cast<long>(b) * K + j] : NucleusRow{};
    const char* zr = zb + static_cast<long>(j) * V * Elem<DT>::kBytes;
    const float* qr = a.q + (static_cast<long>(b) * K + (res ? j : 0)) * V;
    const ExpArg g = exp_arg(static_cast<double>(tr.m), a.invT, ek);
    bool residual = res;
    const double tinv = 1.0 / tr.norm, dinv = res ? 1.0 / dr.norm : 0.0;
    auto weight = [&](int i) -> double {
        const float z = Elem<DT>::scalar(zr, i);
        const double p = kept_by(tr, order_key(z), i) ? (exp_of(z, g, sm.tbl, ek) * tinv) / tr.kept : 0.0;
        if (!residual) return p;
        const float qv = qr[i];
        double w = 0.0;
        if (qv > 0.f && kept_by(dr, order_key(qv), i))
            w = ((plain ? static_cast<double>(qv) : pow(static_cast<double>(qv), a.invT)) * dinv) / dr.kept;
        const double d = p - w;
        return d > 0.0 ? d : 0.0;
    };
    const int C = (V + kCChunk - 1) / kCChunk;
    auto chunk_sums = [&]() {
        for (int c = 0; c < C; ++c) {
            double s = 0.0;
            const int i0 = c * kCChunk + tid * kCE;
            for (int e = 0; e < kCE; ++e)
                if (i0 + e < V) s += weight(i0 + e);
            s = csum(s, sm);
            if (tid == 0) sm.part[c] = s;
        }
        __syncthreads();
        double W = 0.0;
        for (int c = 0; c < C; ++c) W += sm.part[c];
        return W;
    };
    double W = chunk_sums();
    const double S = W;
    if (residual && !(W > 0.0)) {
        residual = false;                 // zero residual: the draw falls back to p'_j
        __syncthreads();
        W = chunk_sums();
    }
    const double target = static_cast<double>(a.u[rbase + K]) * W;
    if (tid == 0) {
        double before = 0.0;
        int chunk = -1, last = 0;
        for (int c = 0; c < C; ++c) {
            const double pc = sm.part[c];
            if (target < before + pc) { chunk = c; break; }
            before += pc;
            if (pc > 0.0) last = c;
        }
        sm.fallback = chunk < 0;          // rounding: u*W at or past the total
        sm.chunk = chunk < 0 ? last : chunk;
        sm.before = before;
    }
    __syncthreads();
    // Thread t holds elements [t*kCE, t*kCE + kCE) of the chunk: its sum, the
    // exclusive sums of the threads before it, then the crossing.
    const int i0 = sm.chunk * kCChunk + tid * kCE;
    double s = 0.0, wlast = 0.0;
    int lastpos = -1;
    for (int e = 0; e < kCE; ++e) {
        if (i0 + e >= V) break;
        const double w = weight(i0 + e);
        s += w;
        if (w > 0.0) { lastpos = i0 + e; wlast = w; }
    }
    double incl = s;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) sm.red[wid] = incl;
    __syncthreads();
    double cum = sm.before;
    for (int x = 0; x < wid; ++x) cum += sm.red[x];
    cum += incl - s;
    int found = 0x7fffffff;
    double wfound = 0.0;
    if (!sm.fallback && target < cum + s) {
        for (int e = 0; e < kCE; ++e) {
            if (i0 + e >= V) break;
            const double w = weight(i0 + e);
            cum += w;
            if (w > 0.0 && target < cum) { found = i0 + e; wfound = w; break; }
        }
    }
    int y = wave_min_int(found);
    const int lp = wave_max_int(lastpos);
    __syncthreads();
    if (lane == 0) { sm.ired[wid] = y; sm.red[wid] = static_cast<double>(lp); }
    __syncthreads();
    y = sm.ired[0];
    int lpb = static_cast<int>(sm.red[0]);
#pragma unroll
    for (int x = 1; x < kCW; ++x) { y = min(y, sm.ired[x]); lpb = max(lpb, static_cast<int>(sm.red[x])); }
    const bool crossed = y != 0x7fffffff;
    if (!crossed) y = lpb;
    const double my = crossed ? (found == y ? wfound : 0.0) : (lastpos == y ? wlast : 0.0);
    const double wy = csum(my, sm);
    for (int t = tid; t <= K; t += kCT) {
        int tok = -1;
        if (t < j) tok = a.x[static_cast<long>(b) * K + t];
        else if (t == j) tok = y;
        a.out_tokens[rbase + t] = tok;
    }
    if (tid == 0) {
        a.out_accept_len[b] = j;
        if (diag) {
            diag[2 * K] = static_cast<float>(residual ? S : 1.0);
            diag[2 * K + 1] = static_cast<float>(wy / W);
        }
    }
}

}  // namespace

hipError_t launch_nucleus_rows(const NucleusArgs& a, hipStream_t s, Timing t) {
    const int rows = a.rows_t + a.rows_d;
    if (rows <= 0) return hipSuccess;
    const ExpConsts ek = exp_consts();
    // 16-byte loads when every target and draft row starts 16-byte aligned
    const bool vec = vec_ok(a.logits, a.V, a.dtype == 1 ? 2 : 4) && vec_ok(a.q, a.V, 4);
    if (a.dtype == 1) {
        if (vec) launch_timed(t, nucleus_row_kernel<1, true>, dim3(rows), dim3(kNT), 0, s, a, ek);
        else launch_timed(t, nucleus_row_kernel<1, false>, dim3(rows), dim3(kNT), 0, s, a, ek);
    } else {
        if (vec) launch_timed(t, nucleus_row_kernel<0, true>, dim3(rows), dim3(kNT), 0, s, a, ek);
        else launch_timed(t, nucleus_row_kernel<0, false>, dim3(rows), dim3(kNT), 0, s, a, ek);
    }
    return hipGetLastError();
}

hipError_t launch_nucleus_chain(const NucleusChainArgs& a, hipStream_t s, Timing t) {
    const ExpConsts ek = exp_consts();
    if (a.ch.dtype == 1) launch_timed(t, nucleus_chain_kernel<1>, dim3(a.ch.B), dim3(kCT), 0, s, a, ek);
    else launch_timed(t, nucleus_chain_kernel<0>, dim3(a.ch.B), dim3(kCT), 0, s, a, ek);
    return hipGetLastError();
}

}  // namespace sv
