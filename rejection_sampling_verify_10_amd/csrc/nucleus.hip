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
//      row, S = sum w, w = q^(1/T), for a draft row (one pass with the row's
//      validity);
//   2. the boundary value by a radix select on the value's order key (bits
//      31..21, then 20..10, then 9..0): per level a histogram of the elements
//      that share the key prefix found so far, holding their count and their
//      probability mass in 62-bit fixed point (integer sums: exact whatever the
//      order of the atomic adds), and the bin where the mass taken from the top
//      reaches top_p.  The first level also lists its elements' values in
//      LDS, so that the later levels read the list, not the row;
//   3. the number n of elements of the boundary value that the cut keeps (they
//      are kept in index order), the index of the last of them, and the kept
//      mass P in fp64.
// A token i is then kept when its key exceeds the boundary key, or equals it
// with i at or before that index; its nucleus probability is p_i / P.
//
// nucleus_chain_kernel runs the ratio tests left to right from these rows'
// cuts and draws the emitted token by inverse CDF in index order (u_K) from the
// residual max(0, p'_j - q'_j) at the first rejection j, from p'_j when that
// residual has no mass, or from p'_K when every draft token passed.  Only the
// target's kept tokens carry weight; each thread sums the weights of a
// contiguous index range in fp64, a block scan places u*W in one range, and
// that thread finds the token.
//
// Weights are fp64 in both kernels and formed by the same code: exp_of (Tang's
// table-driven exponential; for bfloat16 rows looked up from a per-row table of
// its values) and pow_q (a table-driven power).

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
__host__ __device__ constexpr int level_shift(int l) { return l == 0 ? 21 : (l == 1 ? 10 : 0); }
__host__ __device__ constexpr int level_bits(int l) { return l == 2 ? 10 : 11; }
constexpr int kMaxBins = 2048;
// The first level lists its elements' values in LDS: target rows share the
// space with their exponential table, draft rows (no table) have all of it.
constexpr int kCandBytes = 32768;
constexpr int kCandCapT = kCandBytes / 4;
constexpr int kCandCapD = (kCandBytes + static_cast<int>(kTabBytes)) / 4;
// 16-byte loads per thread in flight in each pass over a row, as many as the
// pass's registers allow without spilling (1024 threads: at most 128 VGPRs)
constexpr int kBatchPow = 8;      // draft rows: validity and the power sum
constexpr int kBatchMax = 16;     // target rows: validity and the maximum
constexpr int kBatchTab = 8;      // target rows: the exponential sum
constexpr int kBatchList = 8;     // the first level's listing pass
constexpr int kBatchOneD = 4;     // one pass: draft rows
constexpr int kBatchOneT = 4;     // one pass: target rows

// Probability p in [0, 1] as a 62-bit fixed-point integer (rounded).
__device__ __forceinline__ unsigned long long fixp(double p) {
    return static_cast<unsigned long long>(p * 4611686018427387904.0 + 0.5);
}

struct NucSmem {
    uint32_t cnt[kMaxBins];
    unsigned long long mass[kMaxBins];
    double tbl[kTableSize];
    LogEntry lt[kLogTab];
    // target rows: [kTabSize] exp_of of every tabulated bfloat16 value, then the
    // listed values; draft rows: the listed values
    double region[kTabSize + kCandBytes / 8];
    double red[kNW];
    unsigned long long ured[kNW];
    float fred[kNW];
    float fmax[kNW];
    int ired[kNW];
    uint32_t bad;
    uint32_t ncand;
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

// Unnormalised weight of a target value: exp((z - m)/T), from the row's table
// where it holds z (bfloat16 rows), else exp_of; both give exp_of's value.
template <int DT>
__device__ __forceinline__ double target_w(float z, const ExpArg& g, const double* etab, const double* tbl,
                                           const ExpConsts& ek) {
    if (DT == 1 && etab) {
        const uint32_t h = __float_as_uint(z) >> 16;
        const uint32_t off = (h & 0x7fffu) - kTabLo;
        if (off < kTabSpan) return etab[off + ((h & 0x8000u) ? kTabSpan : 0u)];
    }
    return exp_of(z, g, tbl, ek);
}
// Unnormalised weight of a draft value: q^(1/T), q itself when plain, 0 for q <= 0.
__device__ __forceinline__ double draft_w(float q, bool plain, const PowArg& pa, const LogEntry* lt,
                                          const double* tbl, const ExpConsts& ek) {
    if (!(q > 0.f)) return 0.0;
    return plain ? static_cast<double>(q) : pow_q(q, pa, lt, tbl, ek);
}

// A row's values and their unnormalised weights.
template <int DT, bool DRAFT>
struct RowView {
    const char* row;
    int V;
    bool plain;
    ExpArg g;
    PowArg pa;
    const double* etab;          // null until built
    const double* tbl;
    const LogEntry* lt;
    ExpConsts ek;
    __device__ __forceinline__ double weight(float v) const {
        if (DRAFT) return draft_w(v, plain, pa, lt, tbl, ek);
        return target_w<DT>(v, g, etab, tbl, ek);
    }
    // f(i, v) for the elements of this thread, chunk by chunk: with VEC thread t
    // takes the 16-byte vector t of each chunk of kNT vectors (so its elements
    // within a chunk are contiguous and follow those of thread t - 1), loading
    // kBatch chunks' vectors before it uses them (a row is a few such batches, and
    // one load in flight per thread would leave the pass waiting on latency);
    // else one element per thread per chunk.  Every thread runs the same chunks.
    template <bool VEC, int kBatch, typename F>
    __device__ __forceinline__ void each(F f) const {
        constexpr int EPV = DRAFT ? 4 : Elem<DT>::kPerVec;
        if constexpr (VEC) {
            const int nvec = V / EPV;
            const u32x4* rv = reinterpret_cast<const u32x4*>(row);
            for (int c = 0; c < nvec; c += kBatch * kNT) {
                u32x4 w[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int g = c + u * kNT + static_cast<int>(threadIdx.x);
                    if (g < nvec) w[u] = load_stream(rv + g);
                }
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int g = c + u * kNT + static_cast<int>(threadIdx.x);
                    if (g < nvec) {
#pragma unroll
                        for (int e = 0; e < EPV; ++e)
                            f(g * EPV + e, DRAFT ? __uint_as_float(w[u][e]) : Elem<DT>::get(w[u], e));
                    }
                }
            }
        } else {
            for (int i = threadIdx.x; i < V; i += kNT)
                f(i, DRAFT ? reinterpret_cast<const float*>(row)[i] : Elem<DT>::scalar(row, i));
        }
    }
    // f(i, v) for the elements v of this thread with v >= lo only, in the order
    // each() visits them: a batch's elements are compared first (a bit mask),
    // then the few that pass are taken out of the loaded vectors one by one, so
    // that the rare work is not unrolled over the whole batch.
    template <bool VEC, int kBatch, typename F>
    __device__ __forceinline__ void each_at_least(float lo, F f) const {
        constexpr int EPV = DRAFT ? 4 : Elem<DT>::kPerVec;
        static_assert(kBatch * EPV <= 64, "one bit per element of a batch");
        if constexpr (VEC) {
            const int nvec = V / EPV;
            const u32x4* rv = reinterpret_cast<const u32x4*>(row);
            for (int c = 0; c < nvec; c += kBatch * kNT) {
                u32x4 w[kBatch];
                unsigned long long mask = 0ull;
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int g = c + u * kNT + static_cast<int>(threadIdx.x);
                    if (g < nvec) {
                        w[u] = load_stream(rv + g);
#pragma unroll
                        for (int e = 0; e < EPV; ++e) {
                            const float v = DRAFT ? __uint_as_float(w[u][e]) : Elem<DT>::get(w[u], e);
                            if (v >= lo) mask |= 1ull << (u * EPV + e);
                        }
                    }
                }
                while (mask) {
                    const int bit = __ffsll(static_cast<long long>(mask)) - 1;
                    mask &= mask - 1ull;
                    const int u = bit / EPV, e = bit - u * EPV;
                    u32x4 x = w[0];
#pragma unroll
                    for (int t = 1; t < kBatch; ++t) x = (u == t) ? w[t] : x;
                    float v;
                    if (DRAFT || DT == 0) {
                        const uint32_t b01 = (e & 1) ? x[1] : x[0], b23 = (e & 1) ? x[3] : x[2];
                        v = __uint_as_float((e & 2) ? b23 : b01);
                    } else {
                        const uint32_t b01 = (e & 2) ? x[1] : x[0], b23 = (e & 2) ? x[3] : x[2];
                        const uint32_t word = (e & 4) ? b23 : b01;
                        v = (e & 1) ? bf16_hi(word) : bf16_lo(word);
                    }
                    f((c + u * kNT + static_cast<int>(threadIdx.x)) * EPV + e, v);
                }
            }
        } else {
            for (int i = threadIdx.x; i < V; i += kNT) {
                const float v = DRAFT ? reinterpret_cast<const float*>(row)[i] : Elem<DT>::scalar(row, i);
                if (v >= lo) f(i, v);
            }
        }
    }
};

// The cut of target row r (DRAFT false) or draft row r.
template <int DT, bool DRAFT, bool VEC>
__device__ __forceinline__ void nucleus_row(const NucleusArgs& a, const ExpConsts& ek, int r, NucleusRow* outp, NucSmem& sm) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = wave_id();
    const int V = a.V;
    const char* rowp = static_cast<const char*>(DRAFT ? static_cast<const void*>(a.q) : a.logits) +
                       static_cast<long>(r) * V * (DRAFT ? 4 : Elem<DT>::kBytes);
    for (int t = tid; t < kTableSize; t += kNT) sm.tbl[t] = exp2(static_cast<double>(t) * (1.0 / kTableSize));
    if (DRAFT && !a.plain) build_log_table(sm.lt);
    if (tid == 0) { sm.bad = 0u; sm.tie_last = -1; sm.ncand = 0u; }
    __syncthreads();
    RowView<DT, DRAFT> rv{rowp, V, a.plain != 0, ExpArg{0.0, 0.0}, pow_arg(a.invT, ek), nullptr, sm.tbl, sm.lt, ek};
    NucleusRow out{};

    // Tokens of probability below tau = (1 - top_p) / (2V) hold less than
    // (1 - top_p)/2 together, so the mass taken from the top reaches top_p before
    // them: they lie below the boundary, and a value threshold (vskip, below)
    // leaves them out of the select without computing their weight.
    const double tau = (1.0 - static_cast<double>(a.top_p)) / (2.0 * V);
    float* const cand = reinterpret_cast<float*>(DRAFT ? sm.region : sm.region + kTabSize);
    const int cap = DRAFT ? kCandCapD : kCandCapT;
    uint32_t npre = 0u;          // target rows: values listed by the normaliser's pass

    // 1. the row's validity and normaliser, and the list of values that may lie
    // above the boundary.
    bool bad = false, done = false, listed = false;
    double norm = 0.0;
    float M = 0.f;               // target rows: the reference value of the weights
    float vpre = -INFINITY;      // values below it lie below the boundary
    auto list = [&](float v) {   // few values are listed: one LDS atomic each
        const uint32_t slot = atomicAdd(&sm.ncand, 1u);
        if (slot < static_cast<uint32_t>(cap)) cand[slot] = v;
    };
    if constexpr (VEC) {
        // One pass over the row, its loads one batch ahead of the arithmetic.
        // The first batch (the first kB vectors of every thread) gives a target
        // row's reference value x1, its largest (weights w = exp((z - x1)/T)), and
        // the batch's weight sum S0: the row's sum is at least S0, so a value whose
        // weight is below tau * S0 has p < tau.  The pass lists the others.
        constexpr int EPV = DRAFT ? 4 : Elem<DT>::kPerVec;
        constexpr int kB = DRAFT ? kBatchOneD : kBatchOneT;
        const int nvec = V / EPV;
        const u32x4* rvp = reinterpret_cast<const u32x4*>(rowp);
        auto val = [&](const u32x4& x, int e) { return DRAFT ? __uint_as_float(x[e]) : Elem<DT>::get(x, e); };
        auto load = [&](u32x4 (&w)[kB], int c) {
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const int g = c + u * kNT + tid;
                if (g < nvec) w[u] = load_stream(rvp + g);
            }
        };
        u32x4 w[kB], nx[kB];
        load(w, 0);
        float x1 = 0.f;
        float mx = -INFINITY;
        if (!DRAFT) {
#pragma unroll
            for (int u = 0; u < kB; ++u)
                if (u * kNT + tid < nvec) {
#pragma unroll
                    for (int e = 0; e < EPV; ++e) mx = fmaxf(mx, val(w[u], e));
                }
            const float wm = wave_max(mx);
            if (lane == 0) sm.fred[wid] = wm;
            __syncthreads();
            x1 = sm.fred[0];
#pragma unroll
            for (int q = 1; q < kNW; ++q) x1 = fmaxf(x1, sm.fred[q]);
        }
        // a target row whose first batch holds no value above -inf takes the
        // general route (block-uniform)
        if (DRAFT || x1 > -INFINITY) {
            if (!DRAFT) {
                M = x1;
                rv.g = exp_arg(static_cast<double>(M), a.invT, ek);
                if (DT == 1) {
                    build_exp_table(sm.region, rv.g, sm.tbl, ek);
                    __syncthreads();
                    rv.etab = sm.region;
                }
            }
            const int step = kB * kNT;
            if (step < nvec) load(nx, step);
            // the batch's weights, validity and (targets) maximum
            auto sum_batch = [&](const u32x4 (&b)[kB], int c) {
                double s = 0.0;
#pragma unroll
                for (int u = 0; u < kB; ++u)
                    if (c + u * kNT + tid < nvec) {
#pragma unroll
                        for (int e = 0; e < EPV; ++e) {
                            const float v = val(b[u], e);
                            bad |= DRAFT ? !q_ok(v) : !(v < INFINITY);      // E3 / E1 (NaN or +inf)
                            if (!DRAFT) mx = fmaxf(mx, v);
                            s += rv.weight(v);
                        }
                    }
                return s;
            };
            // list the batch's values v >= vpre: one LDS atomic per wave
            auto list_batch = [&](const u32x4 (&b)[kB], int c) {
                unsigned long long mask = 0ull;
#pragma unroll
                for (int u = 0; u < kB; ++u)
                    if (c + u * kNT + tid < nvec) {
#pragma unroll
                        for (int e = 0; e < EPV; ++e)
                            if (val(b[u], e) >= vpre) mask |= 1ull << (u * EPV + e);
                    }
                const int cnt = __popcll(mask);
                int incl = cnt;
#pragma unroll
                for (int o = 1; o < kWave; o <<= 1) {
                    const int t = __shfl_up(incl, o, kWave);
                    if (lane >= o) incl += t;
                }
                const int total = bcast(incl, kWave - 1);
                if (total == 0) return;                          // wave-uniform
                uint32_t base = 0u;
                if (lane == kWave - 1) base = atomicAdd(&sm.ncand, static_cast<uint32_t>(total));
                uint32_t slot = static_cast<uint32_t>(bcast(static_cast<int>(base), kWave - 1) + incl - cnt);
                if (mask) {
                    // the marked values in batch order (static register indices)
#pragma unroll
                    for (int u = 0; u < kB; ++u)
#pragma unroll
                        for (int e = 0; e < EPV; ++e)
                            if ((mask >> (u * EPV + e)) & 1ull) {
                                if (slot < static_cast<uint32_t>(cap)) cand[slot] = val(b[u], e);
                                ++slot;
                            }
                }
            };
            double s = sum_batch(w, 0);
            const double s0 = block_sum_d(s, sm);
            if (tau > 0.0 && s0 > 0.0 && s0 < INFINITY) {
                if (DRAFT) {
                    // q^(1/T) >= tau * S0  <=>  q >= (tau * S0)^T
                    const double qt = a.plain ? tau * s0 : pow(tau * s0, 1.0 / a.invT);
                    vpre = static_cast<float>(qt * (1.0 - 1e-9));
                } else {
                    vpre = static_cast<float>(static_cast<double>(M) + log(tau * s0) / a.invT -
                                              1e-6 * (1.0 + fabs(M)));
                }
            }
            list_batch(w, 0);
            for (int c = step; c < nvec; c += step) {
#pragma unroll
                for (int u = 0; u < kB; ++u) w[u] = nx[u];
                if (c + step < nvec) load(nx, c + step);
                s += sum_batch(w, c);
                list_batch(w, c);
            }
            if (__ballot(bad) && lane == 0) atomicOr(&sm.bad, 1u);
            if (!DRAFT) {
                mx = wave_max(mx);
                if (lane == 0) sm.fmax[wid] = mx;
            }
            norm = block_sum_d(s, sm);             // its barriers publish sm.bad, sm.fmax, sm.ncand
            bad = sm.bad != 0u;
            npre = sm.ncand;
            done = listed = true;
            if (!DRAFT && !bad) {
                float mrow = sm.fmax[0];
#pragma unroll
                for (int q = 1; q < kNW; ++q) mrow = fmaxf(mrow, sm.fmax[q]);
                // weights far above 1 could overflow the sum: the general route, with
                // the row's maximum as the reference (rare)
                if (!(norm < INFINITY) || (static_cast<double>(mrow) - static_cast<double>(M)) * a.invT > 600.0)
                    done = listed = false;
            }
            __syncthreads();                       // sm.ncand and sm.bad read by all
            if (!done) {
                if (tid == 0) { sm.ncand = 0u; sm.bad = 0u; }
                __syncthreads();
                bad = false;
                npre = 0u;
                rv.etab = nullptr;
            }
        }
    }
    if (!done && DRAFT) {
        double s = 0.0;
        rv.template each<VEC, kBatchPow>([&](int, float v) {
            bad |= !q_ok(v);
            s += rv.weight(v);
        });
        if (__ballot(bad) && lane == 0) atomicOr(&sm.bad, 1u);
        norm = block_sum_d(s, sm);                 // its barriers publish sm.bad
        bad = sm.bad != 0u;
    } else if (!done) {
        float mx = -INFINITY;
        rv.template each<VEC, kBatchMax>([&](int, float v) {
            bad |= !(v < INFINITY);                // NaN or +inf (E1)
            mx = fmaxf(mx, v);
        });
        mx = wave_max(mx);
        if (lane == 0) sm.fred[wid] = mx;
        if (__ballot(bad) && lane == 0) atomicOr(&sm.bad, 1u);
        __syncthreads();
        M = sm.fred[0];
#pragma unroll
        for (int w = 1; w < kNW; ++w) M = fmaxf(M, sm.fred[w]);
        bad = sm.bad != 0u || M == -INFINITY;      // only -inf (E1)
        if (!bad) {
            rv.g = exp_arg(static_cast<double>(M), a.invT, ek);
            if (DT == 1) {
                build_exp_table(sm.region, rv.g, sm.tbl, ek);
                __syncthreads();
                rv.etab = sm.region;
            }
            // With the row maximum as the reference the largest weight is 1, so
            // Z >= 1 and every value v with p >= tau has weight >= tau: v >= vpre.
            vpre = tau > 0.0 ? static_cast<float>(static_cast<double>(M) + log(tau) / a.invT -
                                                  1e-6 * (1.0 + fabs(M)))
                             : -INFINITY;
            double s = 0.0;
            rv.template each<VEC, kBatchTab>([&](int, float v) {
                s += rv.weight(v);
                if (v >= vpre) list(v);
            });
            norm = block_sum_d(s, sm);             // its barriers publish sm.ncand
            npre = sm.ncand;
            listed = true;
            __syncthreads();
        }
    }
    if (!bad && !(norm > 0.0 && norm < INFINITY)) bad = true;     // E4 (drafts), or an overflow
    if (bad) {
        if (tid == 0) {
            out.flags = 1u;
            outp[r] = out;
        }
        return;
    }
    const double invN = 1.0 / norm;

    // 2. radix select of the boundary key.
    const unsigned long long target = max(fixp(static_cast<double>(a.top_p)), 1ull);   // at least the top token
    float vskip;                                  // values strictly below it have p < tau
    if (DRAFT) {
        const double qt = a.plain ? tau * norm : pow(tau * norm, 1.0 / a.invT);
        vskip = static_cast<float>(qt * (1.0 - 1e-9));
    } else {
        vskip = static_cast<float>(static_cast<double>(M) + log(tau * norm) / a.invT - 1e-6 * (1.0 + fabs(M)));
    }
    if (!(tau > 0.0)) vskip = -INFINITY;
    // vpre is a valid threshold too; the larger one keeps the list a superset
    if (listed) vskip = fmaxf(vskip, vpre);
    // rows whose listed values fit: the first level reads the list
    const bool prelisted = listed && npre <= static_cast<uint32_t>(cap);
    if (tid == 0) { sm.prefix = 0u; sm.above = 0ull; sm.goal = target; }
    int last_cnt = 0;
    uint32_t ncand = 0u;
    for (int l = 0; l < kLevels; ++l) {
        const int sh = level_shift(l), nb = 1 << level_bits(l);
        const int psh = sh + level_bits(l);                   // bits above this level
        for (int t = tid; t < nb; t += kNT) { sm.cnt[t] = 0u; sm.mass[t] = 0ull; }
        if (l == 0 && !prelisted && tid == 0) sm.ncand = 0u;    // listed again by the row pass
        __syncthreads();
        const uint32_t prefix = sm.prefix;
        auto add = [&](uint32_t key, double p) {
            const int bin = static_cast<int>((key >> sh) & static_cast<uint32_t>(nb - 1));
            atomicAdd(&sm.cnt[bin], 1u);
            atomicAdd(&sm.mass[bin], fixp(p));
        };
        if (l == 0 && prelisted) {
            for (int c = tid; c < static_cast<int>(npre); c += kNT) {
                const float v = cand[c];
                if (!(v >= vskip)) continue;
                const double p = rv.weight(v) * invN;
                if (p > 0.0) add(order_key(v), p);
            }
        } else if (l == 0) {
            rv.template each_at_least<VEC, kBatchList>(vskip, [&](int, float v) {
                const double p = rv.weight(v) * invN;
                if (!(p > 0.0)) return;
                add(order_key(v), p);
                // list the element (few pass the threshold: one LDS atomic each)
                const uint32_t slot = atomicAdd(&sm.ncand, 1u);
                if (slot < static_cast<uint32_t>(cap)) cand[slot] = v;
            });
        } else {
            auto level = [&](float v) {
                if (!(v >= vskip)) return;
                const uint32_t key = order_key(v);
                if ((key >> psh) != prefix) return;
                const double p = rv.weight(v) * invN;
                if (p > 0.0) add(key, p);
            };
            if (ncand <= static_cast<uint32_t>(cap)) {
                for (int c = tid; c < static_cast<int>(ncand); c += kNT) level(cand[c]);
            } else {
                rv.template each_at_least<VEC, kBatchList>(vskip, [&](int, float v) { level(v); });
            }
        }
        __syncthreads();
        if (l == 0) ncand = sm.ncand;
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
        if (tid == 0) sm.prefix = (prefix << level_bits(l)) | static_cast<uint32_t>(b);
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

// One launch for every row of a call: the rows_d draft rows first (the longer
// ones: fp32, and a power per element), then the target rows.
template <int DT, bool VEC>
__global__ __launch_bounds__(kNT, 1) void nucleus_row_kernel(NucleusArgs a, ExpConsts ek) {
    __shared__ NucSmem sm;
    const int r = blockIdx.x;
    if (r < a.rows_d) nucleus_row<0, true, VEC>(a, ek, r, a.out_d, sm);
    else nucleus_row<DT, false, VEC>(a, ek, r - a.rows_d, a.out_t, sm);
}

// ---- the chain ----

constexpr int kCT = 1024;                         // threads of a batch row's workgroup
constexpr int kCW = kCT / kWave;

struct ChainSmem {
    double tbl[kTableSize];
    LogEntry lt[kLogTab];
    double red[kCW];
    int ired[kCW];
    int j, err, y;
    double wy;
};

// Kept by the nucleus of a row whose cut is c: a larger key, or the boundary key
// at or before the last kept index.
__device__ __forceinline__ bool kept_by(const NucleusRow& c, uint32_t key, int i) {
    return key > c.key || (key == c.key && i <= c.tie_last);
}

// Bounds of this thread's part of the block's inclusive scan of s (thread
// order): [lo, hi), with the parts of consecutive threads sharing their bound
// bit for bit (the lower bound is the previous thread's upper bound, by shuffle),
// so the parts tile [0, total) exactly; total is the last upper bound.
__device__ __forceinline__ void block_scan_bounds(double s, ChainSmem& sm, double& lo, double& hi, double& total) {
    const int lane = threadIdx.x & (kWave - 1), wid = wave_id();
    const double incl = wave_inclusive_scan(s);
    double excl = __shfl_up(incl, 1, kWave);
    if (lane == 0) excl = 0.0;
    __syncthreads();
    if (lane == kWave - 1) sm.red[wid] = incl;
    __syncthreads();
    double base = 0.0, t = 0.0;
    for (int w = 0; w < kCW; ++w) {
        if (w == wid) base = t;
        t += sm.red[w];
    }
    lo = base + excl;
    hi = base + incl;
    total = t;
}

template <int DT, bool VEC>
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
    const PowArg pa = pow_arg(a.invT, ek);
    for (int t = tid; t < kTableSize; t += kCT) sm.tbl[t] = exp2(static_cast<double>(t) * (1.0 / kTableSize));
    if (!plain) build_log_table(sm.lt);
    if (tid == 0) { sm.y = kNoIndex; sm.wy = 0.0; }
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
                const double w = draft_w(qv, plain, pa, sm.lt, sm.tbl, ek);
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
    auto weight = [&](int i, float z) -> double {
        if (!kept_by(tr, order_key(z), i)) return 0.0;
        const double p = (exp_of(z, g, sm.tbl, ek) * tinv) / tr.kept;
        if (!residual) return p;
        const float qv = qr[i];
        double w = 0.0;
        if (qv > 0.f && kept_by(dr, order_key(qv), i)) w = (draft_w(qv, plain, pa, sm.lt, sm.tbl, ek) * dinv) / dr.kept;
        const double d = p - w;
        return d > 0.0 ? d : 0.0;
    };
    // Thread t owns indices [t*L, t*L + L) (whole 16-byte vectors with VEC).
    constexpr int EPV = Elem<DT>::kPerVec;
    int L = (V + kCT - 1) / kCT;
    if (VEC) L = (L + EPV - 1) / EPV * EPV;
    const int i0 = min(V, tid * L), i1 = min(V, i0 + L);
    auto range = [&](auto f) {
        if constexpr (VEC) {
            const u32x4* rv = reinterpret_cast<const u32x4*>(zr);
            for (int i = i0; i < i1; i += 8 * EPV) {
                u32x4 w[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (i + u * EPV < i1) w[u] = rv[(i + u * EPV) / EPV];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (i + u * EPV < i1) {
#pragma unroll
                        for (int e = 0; e < EPV; ++e)
                            if (f(i + u * EPV + e, Elem<DT>::get(w[u], e))) return;
                    }
            }
        } else {
            for (int i = i0; i < i1; ++i)
                if (f(i, Elem<DT>::scalar(zr, i))) return;
        }
    };
    double s = 0.0;
    int lastpos = -1;
    auto sum_pass = [&]() {
        s = 0.0;
        lastpos = -1;
        range([&](int i, float z) {
            const double w = weight(i, z);
            s += w;
            if (w > 0.0) lastpos = i;
            return false;
        });
    };
    sum_pass();
    double lo, hi, W;
    block_scan_bounds(s, sm, lo, hi, W);
    const double S = W;
    if (residual && !(W > 0.0)) {
        residual = false;                 // zero residual: the draw falls back to p'_j
        sum_pass();
        block_scan_bounds(s, sm, lo, hi, W);
    }
    const double target = static_cast<double>(a.u[rbase + K]) * W;
    if (lo <= target && target < hi) {
        // the one thread whose part holds u*W: its first token whose running sum
        // passes it (its last weighted token if rounding leaves none)
        double c = lo, wf = 0.0;
        int found = -1, lp = -1;
        double wl = 0.0;
        range([&](int i, float z) {
            const double w = weight(i, z);
            if (!(w > 0.0)) return false;
            c += w;
            lp = i;
            wl = w;
            if (target < c) { found = i; wf = w; return true; }
            return false;
        });
        if (found < 0) { found = lp; wf = wl; }
        if (found >= 0) { sm.y = found; sm.wy = wf; }
    }
    // no part holds it (W not positive): the last weighted token
    int lp = wave_max_int(lastpos);
    if (lane == 0) sm.ired[wid] = lp;
    __syncthreads();
    int y = sm.y;
    double wy = sm.wy;
    if (y == kNoIndex) {
        lp = sm.ired[0];
#pragma unroll
        for (int x = 1; x < kCW; ++x) lp = max(lp, sm.ired[x]);
        y = lp;
        wy = 0.0;
    }
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
    const bool vec = vec_ok(a.ch.logits, a.ch.V, a.ch.dtype == 1 ? 2 : 4);
    if (a.ch.dtype == 1) {
        if (vec) launch_timed(t, nucleus_chain_kernel<1, true>, dim3(a.ch.B), dim3(kCT), 0, s, a, ek);
        else launch_timed(t, nucleus_chain_kernel<1, false>, dim3(a.ch.B), dim3(kCT), 0, s, a, ek);
    } else {
        if (vec) launch_timed(t, nucleus_chain_kernel<0, true>, dim3(a.ch.B), dim3(kCT), 0, s, a, ek);
        else launch_timed(t, nucleus_chain_kernel<0, false>, dim3(a.ch.B), dim3(kCT), 0, s, a, ek);
    }
    return hipGetLastError();
}

}  // namespace sv
