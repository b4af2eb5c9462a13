// Final draw of the dense chain path (no top-k): the residual draw at the first
// rejection j, or the bonus draw from p'_K.
//
// "064 · 投机解码", section 三: at the first rejection j the emitted token is
// drawn from r = max(0, p'_j - q'_j) / sum max(0, p'_j - q'_j); when all K
// drafts pass, from p'_K.  "Việc giải mã giả định và EAGLE-3", step 2 of its
// residual routine: a residual with zero mass falls back to p'_j.  The draw is
// an inverse CDF over token indices in ascending order driven by u_K:
// y = min{ i : u_K * S < C_i }, C the inclusive prefix of the weights, S their
// total; if rounding leaves no such i, the last index with positive weight.
//
// About 8% of draws on a wide (perplexity ~180) target distribution have a
// CDF boundary within 1e-5 of u*S, so the draw is computed in fp64 end to end
// (one table-driven fp64 exponential per element, fp64 weights and sums).
//
// One pass over row j, although the residual needs the exact normaliser
// Zp = sum_i e_i (e_i = exp((z_i - m)/T)) before any weight is known: the row
// statistics give Zp' (fp32 terms, within ~1e-6).  With iz = 1/Zp' and
// d_i = e_i*iz - w_i (w_i = q'_i, the draft weight), the pass sums per chunk
// of 8 elements per thread
//     E = sum e_i,   R = sum max(0, d_i),   P = sum_{d_i > 0} w_i,
// and lists the elements with |d_i| within a relative delta of zero
// ("undecided").  For every other element the sign of e_i/Zp - w_i equals
// that of d_i as long as Zp lies in Zp'(1 -+ delta), and there the residual is
// rho*d_i + (rho - 1)*w_i with rho = Zp'/Zp, so the chunk's residual mass is
//     rho*R + (rho - 1)*P + (exact share of the listed elements),
// with Zp = sum E known after the pass.  P only scales a term of relative size
// delta, so its terms are fp32.  The bracket is checked afterwards (else, and
// when the list overflowed, a second pass recomputes the chunk sums exactly),
// so the result never depends on the accuracy of Zp'.  A transformed draft
// (T != 1) brackets its normaliser Zq the same way.
//
// One workgroup per batch entry.  dense_walk_kernel (T == 1) walks the
// positions, computing each target row's statistics just before its test;
// dense_row_kernel (transformed drafts) takes all rows' statistics from
// rowstats_kernel and runs the K ratio tests in one wave (lanes k = 0..K).  The
// workgroup then streams row j chunk by chunk, loading the next chunks while it
// computes chunk c, keeps the chunk sums in LDS, and finishes with the draw:
// the chunk holding u*S, rescanned element by element.

//
// This file is compiled twice (dense_walk.hip, dense_tr.hip), each translation
// unit holding one of the two kernels; SV_DENSE_THREADS sets the block size (a
// 1024-thread walk, a whole CU per batch row, measured slower than 512).

#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "exp64.hpp"
#include "internal.hpp"
#include "lists.hpp"

#ifndef SV_SPLIT_TAB_CHUNKS
#define SV_SPLIT_TAB_CHUNKS 3
#endif
#ifndef SV_DENSE_THREADS
#error "define SV_DENSE_THREADS before including dense_impl.hpp"
#endif

namespace sv {

namespace {

constexpr int kThreads = SV_DENSE_THREADS;
constexpr int kDenseChunk = 8 * kThreads;           // elements per chunk: 8 per thread
constexpr int kWaves = kThreads / kWave;
constexpr int kEPT = kDenseChunk / kThreads;        // 8 elements per thread per chunk
constexpr int kSub = kEPT / 8;                      // 8-element groups per thread
constexpr int kMaxChunks = (kMaxV + kDenseChunk - 1) / kDenseChunk;
constexpr int kListCap = 64;                        // undecided elements per row
// Register buffers of the streaming pass: three (two chunks in flight) where the
// registers allow four waves per SIMD, else two.
template <bool VEC, bool TR> constexpr int ring_depth() { return (VEC && !TR) ? 3 : 2; }
// Waves per SIMD the registers must allow: a 1024-thread workgroup is four per SIMD.
template <bool VEC, bool TR> constexpr int min_waves() {
    return kThreads >= 1024 ? kThreads / kWave / 4 : ((VEC && !TR) ? 4 : 2);
}

// Eight consecutive logits from i0 (a multiple of 8); -inf past V.  With VEC
// the row is 16-byte aligned and V a multiple of the vector length, so each
// vector lies wholly inside or wholly past the row.
template <int DT, bool VEC, bool NT>
__device__ __forceinline__ void load8_z(const char* row, int i0, int V, float out[8]) {
    using E = Elem<DT>;
    if (VEC) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row + static_cast<long>(i0) * E::kBytes);
        constexpr uint32_t ninf = DT == 1 ? 0xff80ff80u : 0xff800000u;
        const u32x4 pad = u32x4{ninf, ninf, ninf, ninf};
        if (DT == 1) {
            const u32x4 v = (i0 < V) ? (NT ? load_stream(p) : p[0]) : pad;
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] = E::get(v, e);
        } else {
            const u32x4 a = (i0 < V) ? (NT ? load_stream(p) : p[0]) : pad;
            const u32x4 b = (i0 + 4 < V) ? (NT ? load_stream(p + 1) : p[1]) : pad;
#pragma unroll
            for (int e = 0; e < 4; ++e) { out[e] = __uint_as_float(a[e]); out[4 + e] = __uint_as_float(b[e]); }
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (i0 + e < V) ? E::scalar(row, i0 + e) : -INFINITY;
}

// Eight consecutive draft probabilities from i0; 0 past V.
template <bool VEC, bool NT>
__device__ __forceinline__ void load8_q(const float* row, int i0, int V, float out[8]) {
    if (VEC) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row + i0);
        const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
        const u32x4 a = (i0 < V) ? (NT ? load_stream(p) : p[0]) : zero;
        const u32x4 b = (i0 + 4 < V) ? (NT ? load_stream(p + 1) : p[1]) : zero;
#pragma unroll
        for (int e = 0; e < 4; ++e) { out[e] = __uint_as_float(a[e]); out[4 + e] = __uint_as_float(b[e]); }
        return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (i0 + e < V) ? row[i0 + e] : 0.f;
}

// The same eight elements kept packed as loaded (bf16 pairs or fp32 words): half
// the registers of the widened values for bf16.  kZW vectors hold 8 logits.
template <int DT> struct Raw8 {
    static constexpr int kZW = DT == 1 ? 1 : 2;
    u32x4 z[kZW];
    u32x4 q[2];
    __device__ __forceinline__ float zf(int e) const {
        return DT == 1 ? Elem<1>::get(z[0], e) : __uint_as_float(z[e >> 2][e & 3]);
    }
    __device__ __forceinline__ float qf(int e) const { return __uint_as_float(q[e >> 2][e & 3]); }
    // The same for an index known only at run time (selects, no register indexing).
    __device__ __forceinline__ static uint32_t pick4(const u32x4& v, int i) {
        const uint32_t lo = (i & 1) ? v[1] : v[0], hi = (i & 1) ? v[3] : v[2];
        return (i & 2) ? hi : lo;
    }
    __device__ __forceinline__ float zf_at(int e) const {
        if (DT == 1) {
            const uint32_t w = pick4(z[0], e >> 1);
            return (e & 1) ? bf16_hi(w) : bf16_lo(w);
        }
        return __uint_as_float((e & 4) ? pick4(z[kZW - 1], e & 3) : pick4(z[0], e & 3));
    }
    __device__ __forceinline__ float qf_at(int e) const {
        return __uint_as_float((e & 4) ? pick4(q[1], e & 3) : pick4(q[0], e & 3));
    }
};
// GUARD: the vectors may lie past the row's end.  Loads are then issued from a
// clamped (valid) address and replaced by padding, so that no load sits behind a
// branch and the wait for one buffer does not also wait for the other.
template <int DT, bool VEC, bool GUARD>
__device__ __forceinline__ void load8_raw(const char* zrow, const float* qrow, bool with_q, int i0, int V,
                                          Raw8<DT>& r) {
    constexpr uint32_t ninf = DT == 1 ? 0xff80ff80u : 0xff800000u;
    const u32x4 pad = u32x4{ninf, ninf, ninf, ninf};
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
    if (VEC) {
        const u32x4* pz = reinterpret_cast<const u32x4*>(zrow);
        const u32x4* pq = reinterpret_cast<const u32x4*>(qrow);
        constexpr int zv = 8 / Raw8<DT>::kZW;              // elements per z vector
        if (!GUARD) {
#pragma unroll
            for (int w = 0; w < Raw8<DT>::kZW; ++w) r.z[w] = load_stream(pz + (i0 + w * zv) / zv);
            if (with_q) {
                r.q[0] = load_stream(pq + i0 / 4);
                r.q[1] = load_stream(pq + i0 / 4 + 1);
            }
            return;
        }
#pragma unroll
        for (int w = 0; w < Raw8<DT>::kZW; ++w) {
            const int i = i0 + w * zv;
            const u32x4 v = load_stream(pz + (i < V ? i : 0) / zv);
            r.z[w] = i < V ? v : pad;
        }
        if (with_q) {
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                const int i = i0 + 4 * w;
                const u32x4 v = load_stream(pq + (i < V ? i : 0) / 4);
                r.q[w] = i < V ? v : zero;
            }
        }
        return;
    }
    float z[8], q[8];
    load8_z<DT, false, false>(zrow, i0, V, z);
    if (DT == 1) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            r.z[0][w] = (__float_as_uint(z[2 * w]) >> 16) | (__float_as_uint(z[2 * w + 1]) & 0xffff0000u);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) r.z[e >> 2][e & 3] = __float_as_uint(z[e]);
    }
    if (with_q) {
        load8_q<false, false>(qrow, i0, V, q);
#pragma unroll
        for (int e = 0; e < 8; ++e) r.q[e >> 2][e & 3] = __float_as_uint(q[e]);
    }
}

// Ratio tests of one batch row from the row statistics, lanes k = 0..K of a
// wave, as the left-to-right walk sees them: j = the first position whose rows
// are unusable (E1, E3 at x_k, E4: an error) or whose draft token is rejected,
// K if none; invalid tokens or uniforms (E2, E5) are errors wherever they are.
// Writes p'_k(x_k) and q'_k(x_k) for k <= j to diag when given (NaN past j).
template <bool TR>
__device__ __forceinline__ void first_reject(const ChainArgs& a, int b, float* diag, int& j_out, bool& err_out) {
    const int K = a.K, V = a.V;
    const int k = threadIdx.x & (kWave - 1);
    const long rbase = static_cast<long>(b) * (K + 1);
    bool rows_bad = false, inputs_bad = false, rej = false;
    double pk = NAN, qk = NAN;
    if (k <= K) {
        rows_bad |= (a.st.flags[rbase + k] != 0u);
        inputs_bad |= !u_ok(a.u[rbase + k]);
    }
    if (k < K) {
        const int x = a.x[static_cast<long>(b) * K + k];
        inputs_bad |= (x < 0 || x >= V);
        if (x >= 0 && x < V) {
            const float qx = a.q[(static_cast<long>(b) * K + k) * V + x];
            rows_bad |= !q_ok(qx);
            if (TR) rows_bad |= (a.qflags[static_cast<long>(b) * K + k] != 0u);
            const double zx = static_cast<double>(a.st.zx[rbase + k]);
            pk = exp((zx - static_cast<double>(a.st.m[rbase + k])) * a.invT) / a.st.Z[rbase + k];
            qk = static_cast<double>(qx);
            if (TR) qk = (qx > 0.f) ? pow(qk, a.invT) / a.qsum[static_cast<long>(b) * K + k] : 0.0;
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
    j_out = j;
    err_out = err;
}

__device__ __forceinline__ double block_sum(double v, double* red) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += red[w];
    return t;
}

// Draft weight w_i: q_i, or q_i^(1/T) when the draft is transformed (0 stays 0), by
// the table-driven fp64 power (Tang's logarithm and exponential, within 3e-15 of the
// exact power wherever the weight exceeds 1e-6 of the largest): every weight of a row,
// in the pass and in the rescan, comes from this one function.
// The power's logarithm table lives outside RowSmem, at namespace scope, so that
// only the kernels of transformed drafts (the ones that read it) are given its LDS.
__shared__ LogEntry dense_log_tab[kLogTab];
struct PowCtx {
    PowArg pa;
    const LogEntry* lt;
    const double* tbl;
    ExpConsts ek;
};
template <bool TR>
__device__ __forceinline__ double draft_w(float q, const PowCtx& pw) {
    if (!TR) return static_cast<double>(q);
    return q > 0.f ? pow_q(q, pw.pa, pw.lt, pw.tbl, pw.ek) : 0.0;
}

// True when Z lies strictly inside Zapprox(1 -+ delta), with room for rounding.
__device__ __forceinline__ bool in_bracket(double Z, double Zapprox, double delta) {
    return Z > Zapprox * (1.0 - delta) * (1.0 + 1e-12) && Z < Zapprox * (1.0 + delta) * (1.0 - 1e-12);
}

// Inclusive sums within each 16-lane row (DPP row shifts, zero fill): lane 16r+15
// ends with the sum of row r.
__device__ __forceinline__ double row_scan(double v) {
    auto step = [&](auto ctrl_tag) {
        constexpr int kCtrl = decltype(ctrl_tag)::value;
        const long long bits = __double_as_longlong(v);
        const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(bits), kCtrl, 0xF, 0xF, true);
        const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(bits >> 32), kCtrl, 0xF, 0xF, true);
        v += __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
    };
    step(std::integral_constant<int, 0x111>{});   // row_shr:1
    step(std::integral_constant<int, 0x112>{});   // row_shr:2
    step(std::integral_constant<int, 0x114>{});   // row_shr:4
    step(std::integral_constant<int, 0x118>{});   // row_shr:8
    return v;
}
__device__ __forceinline__ float row_scan(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, true));
    return v;
}
// Chunk partials live in dynamic LDS, summed in slot order after the pass: 4 row
// sums per wave (32 slots per chunk) while C <= 128 (48 KiB), else one wave sum per
// wave (8 slots; longer rows, fewer slots, the same 48 KiB bound).
constexpr int kRowSlots = kWaves * 4;
__host__ __device__ inline int dense_slots(int C) { return C <= 128 ? kRowSlots : kWaves; }
inline size_t dense_dyn_lds(int C, bool tab) {
    return (tab ? kTabBytes : 0) + static_cast<size_t>(C) * dense_slots(C) * (sizeof(double) + sizeof(float));
}
// The exponential table is used for bf16 rows of up to 48 chunks: two workgroups
// share a CU's 160 KiB of LDS up to 47 chunks (42 with a transformed draft, whose
// kernels also hold the power's logarithm table), one beyond.
constexpr int kTabMaxChunks = 48;
// A slice of the split draw builds the table when it has at least this many chunks.
constexpr int kSplitTabChunks = SV_SPLIT_TAB_CHUNKS;

struct RowSmem {
    float wq[kWave];                   // walk: q[x_k], lane k
    float wz[kWave];                   //       z[x_k]
    float wu[kWave];                   //       u_k
    float wmax[kWaves];                //       per-wave row maxima
    double tbl[kTableSize];
    double part[kMaxChunks];           // chunk weights of the draw
    int32_t li[kListCap];              // undecided elements
    double le[kListCap], lw[kListCap];
    double red[kWaves];
    int ired[kWaves];
    int n_list, j, err, chunk, fallback;
    uint32_t qbad;
    uint32_t zbad;                     // the bonus row holds NaN or +inf
    double before;
};

// Exact chunk sums of a draw row by a pass of its own (the slow path: a
// normaliser outside its bracket or an overflowing list): sm.part[c] = the sum
// of e_i (resid false) or of max(0, e_i/Zp - w_i/Zq) (true) over chunk c.
template <int DT, bool VEC, bool TR>
__device__ __forceinline__ void exact_chunk_sums(const ChainArgs& a, const char* zr, const float* qr, int C, ExpArg g,
                                              const double* tbl, ExpConsts ek, bool resid, double invZp,
                                              double invZq, RowSmem& sm) {
    const int tid = threadIdx.x, V = a.V;
    const PowCtx pw{pow_arg(a.invT, ek), dense_log_tab, tbl, ek};
#pragma unroll 1
    for (int c = 0; c < C; ++c) {
        double sc = 0.0;
#pragma unroll 1
        for (int s = 0; s < kSub; ++s) {
            const int i0 = c * kDenseChunk + (s * kThreads + tid) * 8;
            float z[8], q[8];
            load8_z<DT, VEC, false>(zr, i0, V, z);
            if (resid) load8_q<VEC, false>(qr, i0, V, q);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double ex = exp_of(z[e], g, tbl, ek);
                if (resid) {
                    const double rr = ex * invZp - draft_w<TR>(q[e], pw) * invZq;
                    sc += rr > 0.0 ? rr : 0.0;
                } else {
                    sc += ex;
                }
            }
        }
        sc = block_sum(sc, sm.red);
        if (tid == 0) sm.part[c] = sc;
    }
    __syncthreads();
}

// The draw of batch row b from its chunk weights sm.part[0..C) (total W): the
// chunk holding u_K*W, rescanned element by element (weights e_i (residual false)
// or max(0, e_i/Zp - w_i/Zq)), then the row's outputs.  S: the residual mass
// reported in diag (residual rows).
template <int DT, bool VEC, bool TR>
__device__ __forceinline__ void draw_emit(const ChainArgs& a, int b, int j, const char* zr, const float* qr, int C,
                                          ExpArg g, const double* tbl, const ExpConsts& ek, bool residual, double W,
                                          double S, double invZp, double invZq, RowSmem& sm) {
    const int K = a.K, V = a.V;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = wave_id();
    const long rbase = static_cast<long>(b) * (K + 1);
    float* diag = a.out_diag ? a.out_diag + static_cast<long>(b) * (2 * K + 2) : nullptr;
    const double target = static_cast<double>(a.u[rbase + K]) * W;
    const PowCtx pw{pow_arg(a.invT, ek), dense_log_tab, tbl, ek};
    if (tid == 0) {
        double before = 0.0;
        int chunk = -1, last = 0;
        for (int c = 0; c < C; ++c) {
            const double pc = sm.part[c];
            if (target < before + pc) { chunk = c; break; }
            before += pc;
            if (pc > 0.0) last = c;
        }
        sm.fallback = chunk < 0;     // rounding: u*W at or past the total
        sm.chunk = chunk < 0 ? last : chunk;
        sm.before = before;
    }
    __syncthreads();
    const int chunk = sm.chunk;
    const bool fallback = sm.fallback != 0;

    // Weights of 8 consecutive elements from i0: exp (p' draw) or residual.
    auto weights8 = [&](int i0, double wt[8]) {
        float z[8], q[8];
        load8_z<DT, VEC, false>(zr, i0, V, z);
        if (residual) load8_q<VEC, false>(qr, i0, V, q);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double ex = exp_of(z[e], g, tbl, ek);
            double w = ex;
            if (residual) {
                w = ex * invZp - draft_w<TR>(q[e], pw) * invZq;
                w = w > 0.0 ? w : 0.0;
            }
            wt[e] = (i0 + e < V) ? w : 0.0;
        }
    };
    // Thread t holds elements [t*8, t*8 + 8) of the chunk.  Two passes
    // (recomputing beats holding 16 doubles): thread sums, then the crossing.
    const int i0 = chunk * kDenseChunk + tid * kEPT;
    double s = 0.0, wlast = 0.0;
    int lastpos = -1;
#pragma unroll 1
    for (int sub = 0; sub < kSub; ++sub) {
        double wt[8];
        weights8(i0 + 8 * sub, wt);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s += wt[e];
            if (wt[e] > 0.0) { lastpos = i0 + 8 * sub + e; wlast = wt[e]; }
        }
    }
    double incl = s;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    __syncthreads();
    if (lane == kWave - 1) sm.red[wid] = incl;
    __syncthreads();
    double cum = sm.before;
    for (int x = 0; x < wid; ++x) cum += sm.red[x];
    cum += incl - s;
    int found = 0x7fffffff;
    double wfound = 0.0;
    // Threads whose span ends past u*W rescan; the smallest crossing wins.
    if (!fallback && target < cum + s) {
#pragma unroll 1
        for (int sub = 0; sub < kSub && found == 0x7fffffff; ++sub) {
            double wt[8];
            weights8(i0 + 8 * sub, wt);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                cum += wt[e];
                if (found == 0x7fffffff && wt[e] > 0.0 && target < cum) { found = i0 + 8 * sub + e; wfound = wt[e]; }
            }
        }
    }
    // Smallest crossing index; if rounding left none in the chunk, its last positive index.
    int y = wave_min_int(found);
    const int lp = wave_max_int(lastpos);
    __syncthreads();
    if (lane == 0) { sm.ired[wid] = y; sm.red[wid] = static_cast<double>(lp); }
    __syncthreads();
    y = sm.ired[0];
    int lpb = static_cast<int>(sm.red[0]);
#pragma unroll
    for (int x = 1; x < kWaves; ++x) { y = min(y, sm.ired[x]); lpb = max(lpb, static_cast<int>(sm.red[x])); }
    const bool crossed = y != 0x7fffffff;
    if (!crossed) y = lpb;
    const double my = crossed ? (found == y ? wfound : 0.0) : (lastpos == y ? wlast : 0.0);
    const double wy = block_sum(my, sm.red);

    for (int t = tid; t <= K; t += kThreads) {
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

// The draw of batch row b from row j (j < K: the residual max(0, p'_j - q'_j);
// j = K: p'_K), around the row statistics' maximum m_j and normaliser Zp_row.
struct DrawCtx {
    int j, C, C_full, nslots;
    bool res;
    const char* zr;
    const float* qr;
    long qrow;
    ExpArg g;
    double Zp_ap, Zq_ap, iz, iq, tol2;
};
template <int DT, bool TR>
__device__ __forceinline__ DrawCtx draw_ctx(const ChainArgs& a, int b, int j, double bracket, const ExpConsts& ek,
                                            float m_j, double Zp_row) {
    const int K = a.K, V = a.V;
    DrawCtx d;
    d.j = j;
    d.C = (V + kDenseChunk - 1) / kDenseChunk;
    d.C_full = V / kDenseChunk;                      // chunks wholly inside the row
    d.nslots = dense_slots(d.C);
    d.res = j < K;
    const long zrow = static_cast<long>(b) * (K + 1) + j;
    d.qrow = static_cast<long>(b) * K + (d.res ? j : 0);
    d.zr = static_cast<const char*>(a.logits) + zrow * V * Elem<DT>::kBytes;
    d.qr = a.q + d.qrow * V;
    d.g = exp_arg(static_cast<double>(m_j), a.invT, ek);
    d.Zp_ap = Zp_row;
    d.Zq_ap = (TR && d.res) ? a.qsum[d.qrow] : 1.0;
    d.iz = 1.0 / d.Zp_ap;
    d.iq = TR ? 1.0 / d.Zq_ap : 1.0;
    // |d| > tol*(e*iz + w') (w' = w*iq, tol >= delta/(1 - delta) plus rounding room)
    // fixes the sign of the residual over the brackets; since e*iz = d + w' this
    // holds whenever |d| > tol2*w'.
    const double tol = bracket * (1.0 + 2.0 * bracket) + 1e-12;
    d.tol2 = 2.0 * tol / (1.0 - tol);
    return d;
}

// The draw's pass over chunks [c_begin, c_end) of row j: per chunk the slot partials
// pr (R on residual rows, else E) and pp (P) at [c][slot]; per thread se_tot (sum
// e, residual rows), sq_tot (sum w, transformed draft), zmax / zbad (bonus rows);
// undecided elements into sm's list, a bad draft value into sm.qbad.
template <int DT, bool VEC, bool TR, bool TAB>
__device__ __forceinline__ void draw_pass(const ChainArgs& a, const DrawCtx& d, int c_begin, int c_end,
                                          const double* etab, const double* tbl, const ExpConsts& ek, double* pr,
                                          float* pp, RowSmem& sm, double& se_tot, double& sq_tot, float& zmax,
                                          bool& zbad) {
    const int V = a.V;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = wave_id();
    const int C = d.C, C_full = d.C_full, nslots = d.nslots;
    const bool res = d.res;
    const char* zr = d.zr;
    const float* qr = d.qr;
    const ExpArg g = d.g;
    const double iz = d.iz, iq = d.iq, tol2 = d.tol2;
    const PowCtx pw{pow_arg(a.invT, ek), dense_log_tab, tbl, ek};
    auto body = [&](auto res_tag) {
        constexpr bool RES = decltype(res_tag)::value;
        using Buf = Raw8<DT>[kSub];
        auto load = [&](int c, Buf& rb, auto guard_tag) {
            constexpr bool GUARD = decltype(guard_tag)::value;
#pragma unroll
            for (int s = 0; s < kSub; ++s)
                load8_raw<DT, VEC, GUARD>(zr, qr, RES, c * kDenseChunk + (s * kThreads + tid) * 8, V, rb[s]);
        };
        auto compute = [&](int c, Buf& rb) {
            double se = 0.0, sr = 0.0;
            float sp = 0.f, qmin = 0.f, qmax = 0.f;
            bool und = false;
#pragma unroll
            for (int s = 0; s < kSub; ++s) {
                if (RES) {
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        qmin = minimum3(qmin, rb[s].qf(e), rb[s].qf(e + 1));
                        qmax = maximum3(qmax, rb[s].qf(e), rb[s].qf(e + 1));
                    }
                }
                double ext[8];
                if constexpr (TAB) exp8_table(rb[s], etab, g, tbl, ek, ext);
                // (without the table the transformed draft's loop is unrolled only by
                // two, to keep two copies of the power function: its element index is a
                // run-time value, read through selects rather than by indexing the
                // registers; with the table it is unrolled whole, as ext[] must be)
                auto one = [&](int e) {
                    const float zf = TR ? rb[s].zf_at(e) : rb[s].zf(e);
                    const double ex = TAB ? ext[e] : exp_of(zf, g, tbl, ek);
                    se += ex;
                    if (!RES) {
                        zmax = fmaxf(zmax, zf);
                        zbad |= !(zf < INFINITY);
                    }
                    if (RES) {
                        const float qv = TR ? rb[s].qf_at(e) : rb[s].qf(e);
                        const double w = draft_w<TR>(qv, pw);
                        if (TR) sq_tot += w;
                        const double wq = TR ? w * iq : w;
                        const double dd = fma(ex, iz, -wq);
                        sr += fmax(dd, 0.0);
                        sp += dd > 0.0 ? (TR ? static_cast<float>(w) : qv) : 0.f;
                        und |= fabs(dd) <= tol2 * wq;
                    }
                };
                if (TR && !TAB) {
                    // two elements per turn: two independent fp64 chains in flight
#pragma unroll 1
                    for (int e = 0; e < 8; e += 2) {
                        one(e);
                        one(e + 1);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) one(e);
                }
            }
            if (RES) {
                if (__ballot(!(qmin >= 0.f && qmax < INFINITY)) && lane == 0) atomicOr(&sm.qbad, 1u);
                // Undecided elements are rare (about one per row): list them in a
                // wave-uniform branch.  Untransformed drafts recompute the thread's
                // elements from the registers (a branch holding loads would make
                // the compiler wait for every prefetch in flight); transformed
                // ones re-read them, keeping a single copy of the power function.
                if constexpr (!TR) {
                    if (__ballot(und)) {
#pragma unroll
                        for (int s2 = 0; s2 < kSub; ++s2) {
#pragma unroll 1
                            for (int e = 0; e < 8; ++e) {
                                const int i = c * kDenseChunk + (s2 * kThreads + tid) * 8 + e;
                                const double ex = exp_of(rb[s2].zf_at(e), g, tbl, ek);
                                const double w = static_cast<double>(rb[s2].qf_at(e));
                                const double dd = fma(ex, iz, -w);
                                if (und && i < V && fabs(dd) <= tol2 * w) {
                                    const int p = atomicAdd(&sm.n_list, 1);
                                    if (p < kListCap) { sm.li[p] = i; sm.le[p] = ex; sm.lw[p] = w; }
                                }
                            }
                        }
                    }
                } else if (__ballot(und) && und) {
#pragma unroll 1
                    for (int k = 0; k < kEPT; ++k) {
                        const int i = c * kDenseChunk + ((k >> 3) * kThreads + tid) * 8 + (k & 7);
                        if (i >= V) break;
                        const double ex = exp_of(Elem<DT>::scalar(zr, i), g, tbl, ek);
                        const double w = draft_w<TR>(qr[i], pw);
                        const double wq = TR ? w * iq : w;
                        const double dd = fma(ex, iz, -wq);
                        if (fabs(dd) <= tol2 * wq) {
                            const int p = atomicAdd(&sm.n_list, 1);
                            if (p < kListCap) { sm.li[p] = i; sm.le[p] = ex; sm.lw[p] = w; }
                        }
                    }
                }
            }
            // Per chunk the residual rows need R and P; E only as a row total (kept per
            // lane).  The bonus rows need E per chunk.
            if (RES) se_tot += se;
            double v = RES ? sr : se;
            if (nslots == kRowSlots) {
                const int slot = c * kRowSlots + wid * 4 + (lane >> 4);
                v = row_scan(v);
                if (RES) sp = row_scan(sp);
                if ((lane & 15) == 15) {
                    pr[slot] = v;
                    if (RES) pp[slot] = sp;
                }
            } else {
                v = wave_sum(v);
                if (RES) sp = wave_sum(sp);
                if (lane == 0) {
                    pr[c * kWaves + wid] = v;
                    if (RES) pp[c * kWaves + wid] = sp;
                }
            }
        };
        // Full chunks: a ring of kRing register buffers keeps chunks c+1 .. c+kRing-1
        // in flight while chunk c is computed.  The loads are unconditional (indices
        // clamped to the last full chunk; the surplus loads are discarded) so that
        // the wait for one buffer does not also wait for the others.  The partial
        // last chunk comes after.
        constexpr int kRing = ring_depth<VEC, TR>();
        Buf ring[kRing];
        const int f_end = min(c_end, C_full);          // full chunks of the range: [c_begin, f_end)
        if (c_begin < f_end) {
#pragma unroll
            for (int r = 0; r < kRing - 1; ++r) load(min(c_begin + r, f_end - 1), ring[r], std::false_type{});
        }
#pragma unroll 1
        for (int c = c_begin; c < f_end; c += kRing) {
#pragma unroll
            for (int st = 0; st < kRing; ++st) {
                load(min(c + st + kRing - 1, f_end - 1), ring[(st + kRing - 1) % kRing], std::false_type{});
                __builtin_amdgcn_sched_barrier(0);     // keep the prefetch ahead of the compute
                if (st == 0 || c + st < f_end) compute(c + st, ring[st]);
            }
        }
        if (C_full < C && c_end == C) {
            load(C_full, ring[0], std::true_type{});
            compute(C_full, ring[0]);
        }
    };
    if (res) body(std::true_type{});
    else body(std::false_type{});
    __syncthreads();
}

// Everything after the pass: the bracket check (or exact sums), the chunk weights and
// the draw.  pr / pp hold every chunk's slot partials; se_tot, sq_tot, zmax, zbad are
// this thread's parts of the pass's sums.
template <int DT, bool VEC, bool TR>
__device__ __forceinline__ void draw_finish(const ChainArgs& a, int b, const DrawCtx& d, double bracket,
                                            const ExpConsts& ek, RowSmem& sm, const double* pr, const float* pp,
                                            float m_j, double se_tot, double sq_tot, float zmax, bool zbad) {
    const int K = a.K;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = wave_id();
    const int j = d.j, C = d.C, nslots = d.nslots;
    const bool res = d.res;
    const char* zr = d.zr;
    const float* qr = d.qr;
    const long qrow = d.qrow;
    const double* tbl = sm.tbl;
    const ExpArg g = d.g;
    const double Zp_ap = d.Zp_ap, Zq_ap = d.Zq_ap, iz = d.iz, iq = d.iq, tol2 = d.tol2;
    (void)tol2;
    (void)qrow;
    const long rbase = static_cast<long>(b) * (K + 1);
    float* diag = a.out_diag ? a.out_diag + static_cast<long>(b) * (2 * K + 2) : nullptr;
    auto fail_row = [&]() {
        for (int t = tid; t <= K; t += kThreads) a.out_tokens[rbase + t] = -1;
        if (tid == 0) a.out_accept_len[b] = -1;
        if (diag)
            for (int t = tid; t < 2 * K + 2; t += kThreads) diag[t] = NAN;
    };


    double Zp = 0.0, Zq = 1.0, S = 0.0;
    bool residual = false;
    ExpArg gd = g;                          // the draw's exponents
    if (!res) {
        // The bonus row's validity (E1) and maximum: the walk leaves row K to this pass.
        {
            const float wz = wave_max(zmax);
            if (lane == 0) sm.wmax[wid] = wz;
            if (__ballot(zbad) && lane == 0) atomicOr(&sm.zbad, 1u);
        }
        __syncthreads();
        float zm = sm.wmax[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) zm = fmaxf(zm, sm.wmax[w]);
        if (sm.zbad || zm == -INFINITY) { fail_row(); return; }
        for (int c = tid; c < C; c += kThreads) {
            double e = 0.0;
#pragma unroll
            for (int w = 0; w < nslots; ++w) e += pr[c * nslots + w];
            sm.part[c] = e;
        }
        __syncthreads();
        for (int c = 0; c < C; ++c) Zp += sm.part[c];
        if (!(Zp > 0.0 && Zp < INFINITY) || fabs((static_cast<double>(zm) - m_j) * a.invT) > 600.0) {
            // exponents too far from the reference (overflow or underflow risk): again
            // against the row's own maximum
            gd = exp_arg(static_cast<double>(zm), a.invT, ek);
            __syncthreads();
            exact_chunk_sums<DT, VEC, TR>(a, zr, qr, C, gd, tbl, ek, false, 0.0, 0.0, sm);
            Zp = 0.0;
            for (int c = 0; c < C; ++c) Zp += sm.part[c];
        }
    } else {
        Zp = block_sum(se_tot, sm.red);
        if (TR) Zq = block_sum(sq_tot, sm.red);      // exact normaliser of the transformed draft
        if (sm.qbad || (TR && !(Zq > 0.0))) { fail_row(); return; }
        const double invZp = 1.0 / Zp, invZq = 1.0 / Zq;
        const bool exact_ok = sm.n_list <= kListCap && in_bracket(Zp, Zp_ap, bracket) &&
                              (!TR || in_bracket(Zq, Zq_ap, bracket));
        if (exact_ok) {
            // over d > 0 the residual e/Zp - w/Zq is rho*d + kap*w, rho = Zp'/Zp
            const double rho = Zp_ap * invZp;
            const double kap = TR ? rho * iq - invZq : (Zp_ap - Zp) * invZp;
            const int n = sm.n_list;
            for (int c = tid; c < C; c += kThreads) {
                double r = 0.0;
                float psum = 0.f;
                for (int w = 0; w < nslots; ++w) { r += pr[c * nslots + w]; psum += pp[c * nslots + w]; }
                double pc = rho * r + kap * static_cast<double>(psum);
                for (int t = 0; t < n; ++t) {
                    if (sm.li[t] / kDenseChunk != c) continue;
                    const double e = sm.le[t], w = sm.lw[t];
                    const double wq = TR ? w * iq : w;
                    const double dd = fma(e, iz, -wq);
                    const double rr = e * invZp - w * invZq;
                    pc += (rr > 0.0 ? rr : 0.0) - (dd > 0.0 ? rho * dd + kap * w : 0.0);
                }
                sm.part[c] = pc > 0.0 ? pc : 0.0;
            }
            __syncthreads();
        } else {
            // A normaliser outside its bracket or the list overflowed: never expected,
            // always correct.
            exact_chunk_sums<DT, VEC, TR>(a, zr, qr, C, g, tbl, ek, true, invZp, invZq, sm);
        }
        for (int c = 0; c < C; ++c) S += sm.part[c];
        __syncthreads();
        residual = S > 0.0;
        if (!residual) {
            // zero residual: the draw falls back to p'_j, whose chunk sums this pass skipped
            exact_chunk_sums<DT, VEC, TR>(a, zr, qr, C, g, tbl, ek, false, 0.0, 0.0, sm);
            Zp = 0.0;
            for (int c = 0; c < C; ++c) Zp += sm.part[c];
        }
    }
    const double invZp = 1.0 / Zp, invZq = 1.0 / Zq;

    draw_emit<DT, VEC, TR>(a, b, j, zr, qr, C, gd, tbl, ek, residual, residual ? S : Zp, S, invZp, invZq, sm);
}


// The final draw of batch row b (one workgroup): sm.j / sm.err set, sm.tbl
// built, sm.n_list = sm.qbad = 0, all visible after a barrier; (m_j, Zp_ap):
// the maximum and approximate normaliser of target row j.
template <int DT, bool VEC, bool TR, bool TAB>
__device__ __forceinline__ void final_draw(const ChainArgs& a, int b, double bracket, const ExpConsts& ek,
                                           RowSmem& sm, double* dyn_lds, float m_j, double Zp_row) {
    static_assert(!TAB || DT == 1, "the exponential table is for bf16 logits");
    const int K = a.K;
    const int tid = threadIdx.x;
    if (sm.err) {
        const long rbase = static_cast<long>(b) * (K + 1);
        float* diag = a.out_diag ? a.out_diag + static_cast<long>(b) * (2 * K + 2) : nullptr;
        for (int t = tid; t <= K; t += kThreads) a.out_tokens[rbase + t] = -1;
        if (tid == 0) a.out_accept_len[b] = -1;
        if (diag)
            for (int t = tid; t < 2 * K + 2; t += kThreads) diag[t] = NAN;
        return;
    }
    const DrawCtx d = draw_ctx<DT, TR>(a, b, sm.j, bracket, ek, m_j, Zp_row);
    double* etab = dyn_lds;                          // TAB: [kTabSize] exponentials
    double* pr = dyn_lds + (TAB ? kTabSize : 0);     // [C][nslots]: R (residual rows) or E
    float* pp = reinterpret_cast<float*>(pr + static_cast<long>(d.C) * d.nslots);        // [C][nslots]: P
    if constexpr (TAB) {
        build_exp_table(etab, d.g, sm.tbl, ek);
        __syncthreads();
    }
    double se_tot = 0.0, sq_tot = 0.0;
    float zmax = -INFINITY;
    bool zbad = false;
    draw_pass<DT, VEC, TR, TAB>(a, d, 0, d.C, etab, sm.tbl, ek, pr, pp, sm, se_tot, sq_tot, zmax, zbad);
    draw_finish<DT, VEC, TR>(a, b, d, bracket, ek, sm, pr, pp, m_j, se_tot, sq_tot, zmax, zbad);
}

template <bool TR = false>
__device__ __forceinline__ void init_draw_smem(RowSmem& sm) {
    for (int t = threadIdx.x; t < kTableSize; t += kThreads) sm.tbl[t] = exp2(static_cast<double>(t) * (1.0 / kTableSize));
    if (TR) build_log_table(dense_log_tab);
    if (threadIdx.x == 0) { sm.n_list = 0; sm.qbad = 0; sm.zbad = 0; }
}

// All rows' statistics precomputed (rowstats_kernel): ratio tests in one wave,
// then the final draw.
template <int DT, bool VEC, bool TR, bool TAB>
__global__ __launch_bounds__(kThreads, (min_waves<VEC, TR>())) void dense_row_kernel(ChainArgs a, double bracket,
                                                                                     ExpConsts ek) {
    __shared__ RowSmem sm;
    extern __shared__ double dyn_lds[];
    const int b = blockIdx.x;
    if (threadIdx.x < kWave) {
        int j;
        bool err;
        first_reject<TR>(a, b, a.out_diag ? a.out_diag + static_cast<long>(b) * (2 * a.K + 2) : nullptr, j, err);
        if (threadIdx.x == 0) { sm.j = j; sm.err = err; }
    }
    init_draw_smem<TR>(sm);
    __syncthreads();
    const long zrow = static_cast<long>(b) * (a.K + 1) + sm.j;
    final_draw<DT, VEC, TR, TAB>(a, b, bracket, ek, sm, dyn_lds, a.st.m[zrow], a.st.Z[zrow]);
}

// ---- the draw split over several workgroups per batch row (all-rows route) ----
//
// With the statistics of every row precomputed, a batch row's draw is one pass
// over its row j plus a short finish; a small batch then leaves most CUs idle while
// B workgroups draw.  The split: slice s of S workgroups of the row runs the ratio
// tests itself (a few gathers), takes chunks [s*P, (s+1)*P) of the pass and stores
// their slot partials and its own sums and undecided elements; a second launch, one
// workgroup per row, gathers them and finishes exactly as the single workgroup does.

struct SliceRec {
    double E, Q;            // sums of e (residual rows) and of the draft weights (transformed)
    float zmax;             // bonus rows: the slice's maximum logit
    uint32_t flags;         // bit 0: a bad draft value; bit 1: a NaN or +inf logit
    int n;                  // undecided elements found (more than kListCap: overflow)
    int32_t li[kListCap];
    double le[kListCap], lw[kListCap];
};
__host__ __device__ inline int split_chunks(int V) { return (V + kDenseChunk - 1) / kDenseChunk; }

template <int DT, bool VEC, bool TR, bool TAB>
__global__ __launch_bounds__(kThreads, (min_waves<VEC, TR>())) void draw_part_kernel(ChainArgs a, double bracket,
                                                                                     ExpConsts ek) {
    __shared__ RowSmem sm;
    extern __shared__ double dyn_lds[];
    const int s = blockIdx.x, b = blockIdx.y, S = a.split_S;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = wave_id();
    if (tid < kWave) {
        int j;
        bool err;
        first_reject<TR>(a, b, nullptr, j, err);
        if (tid == 0) { sm.j = j; sm.err = err; }
    }
    init_draw_smem<TR>(sm);
    __syncthreads();
    if (sm.err) return;                              // the finish writes the error row
    const long zrow = static_cast<long>(b) * (a.K + 1) + sm.j;
    const DrawCtx d = draw_ctx<DT, TR>(a, b, sm.j, bracket, ek, a.st.m[zrow], a.st.Z[zrow]);
    const int per = (d.C + S - 1) / S;
    const int c0 = min(d.C, s * per), c1 = min(d.C, c0 + per);
    double* pr = a.split_pr + static_cast<long>(b) * d.C * d.nslots;
    float* pp = a.split_pp + static_cast<long>(b) * d.C * d.nslots;
    double se = 0.0, sq = 0.0;
    float zmax = -INFINITY;
    bool zbad = false;
    const double* etab = nullptr;
    if constexpr (TAB) {
        build_exp_table(dyn_lds, d.g, sm.tbl, ek);
        __syncthreads();
        etab = dyn_lds;
    }
    if (c0 < c1) draw_pass<DT, VEC, TR, TAB>(a, d, c0, c1, etab, sm.tbl, ek, pr, pp, sm, se, sq, zmax, zbad);
    se = block_sum(se, sm.red);
    if (TR) sq = block_sum(sq, sm.red);
    const float wz = wave_max(zmax);
    const bool wb = __ballot(zbad) != 0ull;
    __syncthreads();
    if (lane == 0) { sm.wmax[wid] = wz; if (wb) atomicOr(&sm.zbad, 1u); }
    __syncthreads();
    SliceRec* rec = reinterpret_cast<SliceRec*>(a.split_rec) + static_cast<long>(b) * kSplitMax + s;
    const int n = sm.n_list;
    if (tid == 0) {
        float zm = sm.wmax[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) zm = fmaxf(zm, sm.wmax[w]);
        rec->E = se;
        rec->Q = sq;
        rec->zmax = zm;
        rec->flags = (sm.qbad ? 1u : 0u) | (sm.zbad ? 2u : 0u);
        rec->n = n;
    }
    for (int t = tid; t < min(n, kListCap); t += kThreads) {
        rec->li[t] = sm.li[t];
        rec->le[t] = sm.le[t];
        rec->lw[t] = sm.lw[t];
    }
}

template <int DT, bool VEC, bool TR>
__global__ __launch_bounds__(kThreads, (min_waves<VEC, TR>())) void draw_combine_kernel(ChainArgs a, double bracket,
                                                                                        ExpConsts ek) {
    __shared__ RowSmem sm;
    extern __shared__ double dyn_lds[];
    const int b = blockIdx.x, S = a.split_S;
    const int K = a.K, tid = threadIdx.x;
    float* diag = a.out_diag ? a.out_diag + static_cast<long>(b) * (2 * K + 2) : nullptr;
    if (tid < kWave) {
        int j;
        bool err;
        first_reject<TR>(a, b, diag, j, err);
        if (tid == 0) { sm.j = j; sm.err = err; }
    }
    init_draw_smem<TR>(sm);
    __syncthreads();
    if (sm.err) {
        const long rbase = static_cast<long>(b) * (K + 1);
        for (int t = tid; t <= K; t += kThreads) a.out_tokens[rbase + t] = -1;
        if (tid == 0) a.out_accept_len[b] = -1;
        if (diag)
            for (int t = tid; t < 2 * K + 2; t += kThreads) diag[t] = NAN;
        return;
    }
    const long zrow = static_cast<long>(b) * (K + 1) + sm.j;
    const float m_j = a.st.m[zrow];
    const DrawCtx d = draw_ctx<DT, TR>(a, b, sm.j, bracket, ek, m_j, a.st.Z[zrow]);
    const int ns = d.C * d.nslots;
    double* pr = dyn_lds;
    float* pp = reinterpret_cast<float*>(pr + ns);
    const double* gpr = a.split_pr + static_cast<long>(b) * ns;
    const float* gpp = a.split_pp + static_cast<long>(b) * ns;
    for (int t = tid; t < ns; t += kThreads) {
        pr[t] = gpr[t];
        pp[t] = gpp[t];
    }
    const SliceRec* rec = reinterpret_cast<const SliceRec*>(a.split_rec) + static_cast<long>(b) * kSplitMax;
    // every slice's sums as one thread's part; the lists in slice order
    const double se = tid < S ? rec[tid].E : 0.0;
    const double sq = tid < S ? rec[tid].Q : 0.0;
    const float zmax = tid < S ? rec[tid].zmax : -INFINITY;
    const bool zbad = tid < S && (rec[tid].flags & 2u) != 0u;
    if (tid < S && (rec[tid].flags & 1u)) atomicOr(&sm.qbad, 1u);
    if (tid == 0) {
        int n = 0;
        for (int s = 0; s < S; ++s) n += rec[s].n;
        sm.n_list = n;
    }
    __syncthreads();
    if (sm.n_list <= kListCap && tid < S) {
        int off = 0;
        for (int s = 0; s < tid; ++s) off += rec[s].n;
        for (int t = 0; t < rec[tid].n; ++t) {
            sm.li[off + t] = rec[tid].li[t];
            sm.le[off + t] = rec[tid].le[t];
            sm.lw[off + t] = rec[tid].lw[t];
        }
    }
    __syncthreads();
    draw_finish<DT, VEC, TR>(a, b, d, bracket, ek, sm, pr, pp, m_j, se, sq, zmax, zbad);
}

// ---- the walk: statistics of target rows 0, 1, ... until the first rejection ----

constexpr int kWalkUnroll = 4;   // vectors per thread per tile
constexpr int kWalkTile = kThreads * kWalkUnroll;

// Workgroup barrier for LDS traffic only: it waits for the wave's LDS operations
// but not for its global loads, so a prefetch stays in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Per-thread part of a row's statistics: fp32 exponentials against a running
// maximum (the numerics of rowstats_kernel).
template <int DT>
struct RowAcc {
    float m = -INFINITY;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    __device__ __forceinline__ void add(const u32x4 (&v)[kWalkUnroll], float scale) {
        using E = Elem<DT>;
        float tmax = m;
#pragma unroll
        for (int u = 0; u < kWalkUnroll; ++u)
#pragma unroll
            for (int e = 0; e < E::kPerVec; ++e) tmax = fmaxf(tmax, E::get(v[u], e));
        if (tmax > m) {
            const float f = __builtin_amdgcn_exp2f((m - tmax) * scale);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] *= f;
            m = tmax;
        }
        if (m != -INFINITY) {
#pragma unroll
            for (int u = 0; u < kWalkUnroll; ++u)
#pragma unroll
                for (int e = 0; e < E::kPerVec; ++e) acc[u & 3] += __builtin_amdgcn_exp2f((E::get(v[u], e) - m) * scale);
        } else {
            // everything so far is -inf (or padding): only a NaN matters
#pragma unroll
            for (int u = 0; u < kWalkUnroll; ++u)
#pragma unroll
                for (int e = 0; e < E::kPerVec; ++e)
                    if (E::get(v[u], e) != E::get(v[u], e)) acc[0] = NAN;
        }
    }
};

// Row maximum M and Z' from the per-thread parts (every thread returns them):
// partials rescaled to M and summed in fp64.  LDS barriers only.
template <int DT>
__device__ __forceinline__ void row_reduce(const RowAcc<DT>& ra, double invT, RowSmem& sm, float& M, double& Z) {
    const int lane = threadIdx.x & (kWave - 1), wid = wave_id();
    const float s = (ra.acc[0] + ra.acc[1]) + (ra.acc[2] + ra.acc[3]);
    const float wm = wave_max(ra.m);
    if (lane == 0) sm.wmax[wid] = wm;
    lds_barrier();
    M = sm.wmax[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm.wmax[w]);
    double c = static_cast<double>(s) * exp((static_cast<double>(ra.m) - static_cast<double>(M)) * invT);
    c = wave_sum(c);
    if (lane == 0) sm.red[wid] = c;
    lds_barrier();
    Z = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) Z += sm.red[w];
    lds_barrier();                 // the slots are reused by the next row
}

// The walk of batch row b with the draft used as given (T == 1, no top-k), one
// workgroup: the positions left to right ("064 · 投机解码", section 三), reading
// target row k only once x_0..x_{k-1} are accepted: its statistics, then test k
// from the gathered z[x_k] and q[x_k].  Returns the first rejection j (K if
// none), the error flag and the maximum and normaliser of target row j.  The
// rows are one stream of tiles: the tile after the last of row k (the first of
// row k+1) is in flight while row k is reduced and tested, and is dropped if the
// walk stops.  sm.tbl must be built (init_draw_smem) before the call.
template <int DT, bool VEC>
__device__ __forceinline__ void walk_positions(const ChainArgs& a, int b, RowSmem& sm, int& j_out, bool& err_out,
                                               float& mj_out, double& zj_out) {
    using E = Elem<DT>;
    const int K = a.K, V = a.V;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const long rbase = static_cast<long>(b) * (K + 1);
    float* diag = a.out_diag ? a.out_diag + static_cast<long>(b) * (2 * K + 2) : nullptr;
    const char* zbase = static_cast<const char*>(a.logits) + rbase * V * E::kBytes;
    // Tokens and uniforms are checked up front (E2, E5 count anywhere); lane k
    // gathers q[x_k] and z[x_k].
    if (tid < kWave) {
        bool bad = false;
        float qx = NAN, uk = 0.f, zx = 0.f;
        if (lane <= K) {
            uk = a.u[rbase + lane];
            bad |= !u_ok(uk);
        }
        if (lane < K) {
            const int x = a.x[static_cast<long>(b) * K + lane];
            bad |= (x < 0 || x >= V);
            if (x >= 0 && x < V) {
                qx = a.q[(static_cast<long>(b) * K + lane) * V + x];
                zx = E::scalar(zbase + static_cast<long>(lane) * V * E::kBytes, x);
            }
        }
        sm.wq[lane] = qx;
        sm.wz[lane] = zx;
        sm.wu[lane] = uk;
        bad = __ballot(bad) != 0ull;
        if (lane == 0) sm.err = bad;
    }
    __syncthreads();
    const float scale = static_cast<float>(1.4426950408889634 * a.invT);
    bool err = sm.err != 0;
    int j = K;
    float mj = 0.f;
    double Zj = 1.0;
    // Test k from M, Z of row k: returns true when the walk stops there.
    auto test = [&](int k, float M, double Z) -> bool {
        mj = M;
        Zj = Z;
        if (!(Z >= 1.0 && Z < INFINITY)) { err = true; return true; }                  // E1
        if (k == K) return true;
        const float qx = sm.wq[k];
        if (!q_ok(qx)) { err = true; return true; }                                     // E3
        const double pk = exp((static_cast<double>(sm.wz[k]) - static_cast<double>(M)) * a.invT) / Z;
        const double qk = static_cast<double>(qx);
        double ratio;
        if (qk > 0.0) ratio = pk / qk;
        else ratio = pk > 0.0 ? INFINITY : 0.0;
        const double thr = ratio < 1.0 ? ratio : 1.0;
        if (diag && tid == 0) {
            diag[k] = static_cast<float>(pk);
            diag[K + k] = static_cast<float>(qk);
        }
        if (!(static_cast<double>(sm.wu[k]) < thr)) { j = k; return true; }
        return false;
    };
    if (!err) {
        if constexpr (VEC) {
            const int nvec = V / E::kPerVec;
            const int T_row = (nvec + kWalkTile - 1) / kWalkTile;     // tiles per row, the last maybe partial
            const bool partial = nvec % kWalkTile != 0;
            constexpr uint32_t ninf = DT == 1 ? 0xff80ff80u : 0xff800000u;
            // tile t of row k; indices past the row are clamped to a valid vector
            auto load = [&](int k, int t, u32x4 (&v)[kWalkUnroll]) {
                const u32x4* rv = reinterpret_cast<const u32x4*>(zbase + static_cast<long>(k) * V * E::kBytes);
#pragma unroll
                for (int u = 0; u < kWalkUnroll; ++u) {
                    const int i = t * kWalkTile + u * kThreads + tid;
                    v[u] = load_stream(rv + (i < nvec ? i : nvec - 1));
                }
            };
            int k = 0, t = 0;
            RowAcc<DT> ra;
            // One tile: prefetch the next one (the next row's first after the last),
            // add this one, and at a row's end reduce and test.  Returns true to stop.
            auto step = [&](u32x4 (&cur)[kWalkUnroll], u32x4 (&nxt)[kWalkUnroll]) -> bool {
                const bool last = t == T_row - 1;
                load(last ? min(k + 1, K) : k, last ? 0 : t + 1, nxt);
                __builtin_amdgcn_sched_barrier(0);
                if (last && partial) {
#pragma unroll
                    for (int u = 0; u < kWalkUnroll; ++u)
                        if (t * kWalkTile + u * kThreads + tid >= nvec) cur[u] = u32x4{ninf, ninf, ninf, ninf};
                }
                ra.add(cur, scale);
                if (!last) {
                    ++t;
                    return false;
                }
                float M;
                double Z;
                row_reduce<DT>(ra, a.invT, sm, M, Z);
                if (test(k, M, Z)) return true;
                ++k;
                if (k == K) {
                    // Every draft token passed: row K feeds only the bonus draw, whose fp64
                    // pass takes the row's validity and maximum itself.  Its exponents are
                    // taken against row K-1's maximum (mj), a common factor of every weight
                    // that cancels in the draw.
                    j = K;
                    return true;
                }
                t = 0;
                ra = RowAcc<DT>();
                return false;
            };
            u32x4 va[kWalkUnroll], vb[kWalkUnroll];
            load(0, 0, va);
#pragma unroll 1
            for (;;) {
                if (step(va, vb)) break;
                if (step(vb, va)) break;
            }
        } else {
#pragma unroll 1
            for (int k = 0; k <= K; ++k) {
                const char* row = zbase + static_cast<long>(k) * V * E::kBytes;
                RowAcc<DT> ra;
                for (int base = 0; base < V; base += kThreads * kWalkUnroll * E::kPerVec) {
                    u32x4 v[kWalkUnroll];
#pragma unroll
                    for (int u = 0; u < kWalkUnroll; ++u) {
                        const long i0 = base + static_cast<long>(u * kThreads + tid) * E::kPerVec;
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            if (DT == 1) {
                                const uint32_t lo = i0 + 2 * w < V ? static_cast<const uint16_t*>(static_cast<const void*>(row))[i0 + 2 * w] : 0xff80u;
                                const uint32_t hi = i0 + 2 * w + 1 < V ? static_cast<const uint16_t*>(static_cast<const void*>(row))[i0 + 2 * w + 1] : 0xff80u;
                                v[u][w] = lo | (hi << 16);
                            } else {
                                v[u][w] = i0 + w < V ? reinterpret_cast<const uint32_t*>(row)[i0 + w] : 0xff800000u;
                            }
                        }
                    }
                    ra.add(v, scale);
                }
                float M;
                double Z;
                row_reduce<DT>(ra, a.invT, sm, M, Z);
                if (test(k, M, Z)) break;
            }
        }
    }
    if (diag && !err)
        for (int t = j + 1 + tid; t < K; t += kThreads) { diag[t] = NAN; diag[K + t] = NAN; }
    j_out = j;
    err_out = err;
    mj_out = mj;
    zj_out = Zj;
}

// Chain verification with the draft used as given (T == 1, no top-k): one
// workgroup per batch row walks the positions (walk_positions), then draws the
// emitted token as dense_row_kernel does.
template <int DT, bool VEC, bool TAB>
__global__ __launch_bounds__(kThreads, (min_waves<VEC, false>())) void dense_walk_kernel(ChainArgs a, double bracket,
                                                                                         ExpConsts ek) {
    __shared__ RowSmem sm;
    extern __shared__ double dyn_lds[];
    const int b = blockIdx.x;
    // The walks are the launch's critical path; a workgroup drawing its row
    // shares the CU with one still walking: the walk takes issue precedence.
    __builtin_amdgcn_s_setprio(2);
    init_draw_smem(sm);
    int j;
    bool err;
    float mj;
    double Zj;
    walk_positions<DT, VEC>(a, b, sm, j, err, mj, Zj);
    __builtin_amdgcn_s_setprio(0);
    if (threadIdx.x == 0) { sm.j = j; sm.err = err; }
    __syncthreads();
    final_draw<DT, VEC, false, TAB>(a, b, bracket, ek, sm, dyn_lds, mj, Zj);
}

#if SV_DENSE_TR
template <int DT, bool VEC, bool TR>
hipError_t dense_launch(const ChainArgs& a, double bracket, hipStream_t s, Timing t) {
    const int C = (a.V + kDenseChunk - 1) / kDenseChunk;
    if (a.split_S > 1) {
        // bf16 slices of at least kSplitTabChunks chunks tabulate the exponentials first
        bool tab = false;
        if constexpr (DT == 1 && VEC) {
            if ((C + a.split_S - 1) / a.split_S >= kSplitTabChunks) {
                tab = true;
                launch_timed(t, draw_part_kernel<DT, VEC, TR, true>, dim3(a.split_S, a.B), dim3(kThreads),
                             static_cast<unsigned>(kTabBytes), s, a, bracket, exp_consts());
            }
        }
        if (!tab)
            launch_timed(t, draw_part_kernel<DT, VEC, TR, false>, dim3(a.split_S, a.B), dim3(kThreads), 0u, s, a,
                         bracket, exp_consts());
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const size_t lds = static_cast<size_t>(C) * dense_slots(C) * (sizeof(double) + sizeof(float));
        launch_timed(Timing{}, draw_combine_kernel<DT, VEC, TR>, dim3(a.B), dim3(kThreads), static_cast<unsigned>(lds),
                     s, a, bracket, exp_consts());
        return hipGetLastError();
    }
    if constexpr (DT == 1 && VEC) {
        if (C <= kTabMaxChunks) {
            launch_timed(t, dense_row_kernel<DT, VEC, TR, true>, dim3(a.B), dim3(kThreads),
                         static_cast<unsigned>(dense_dyn_lds(C, true)), s, a, bracket, exp_consts());
            return hipGetLastError();
        }
    }
    launch_timed(t, dense_row_kernel<DT, VEC, TR, false>, dim3(a.B), dim3(kThreads),
                 static_cast<unsigned>(dense_dyn_lds(C, false)), s, a, bracket, exp_consts());
    return hipGetLastError();
}
#endif

#if SV_DENSE_WALK
template <int DT, bool VEC>
hipError_t walk_launch(const ChainArgs& a, double bracket, hipStream_t s, Timing t) {
    const int C = (a.V + kDenseChunk - 1) / kDenseChunk;
    if constexpr (DT == 1 && VEC) {
        if (C <= kTabMaxChunks) {
            launch_timed(t, dense_walk_kernel<DT, VEC, true>, dim3(a.B), dim3(kThreads),
                         static_cast<unsigned>(dense_dyn_lds(C, true)), s, a, bracket, exp_consts());
            return hipGetLastError();
        }
    }
    launch_timed(t, dense_walk_kernel<DT, VEC, false>, dim3(a.B), dim3(kThreads),
                 static_cast<unsigned>(dense_dyn_lds(C, false)), s, a, bracket, exp_consts());
    return hipGetLastError();
}
#endif

}  // namespace

#if SV_DENSE_WALK
hipError_t launch_chain_walk(const ChainArgs& a, double bracket, hipStream_t s, Timing t) {
    const int esz = a.dtype ? 2 : 4;
    const bool vec = vec_ok(a.logits, a.V, esz) && vec_ok(a.q, a.V, 4);
    if (a.dtype == 1) return vec ? walk_launch<1, true>(a, bracket, s, t) : walk_launch<1, false>(a, bracket, s, t);
    return vec ? walk_launch<0, true>(a, bracket, s, t) : walk_launch<0, false>(a, bracket, s, t);
}
#endif

#if SV_DENSE_TR
size_t dense_split_bytes(int B, int V) {
    const int C = split_chunks(V);
    const size_t per = static_cast<size_t>(C) * dense_slots(C) * (sizeof(double) + sizeof(float)) +
                       kSplitMax * sizeof(SliceRec);
    return static_cast<size_t>(B) * per + 2 * 256;
}
void dense_split_plan(ChainArgs& a, unsigned char* base, int B, int V, int S) {
    const int C = split_chunks(V);
    const size_t slots = static_cast<size_t>(C) * dense_slots(C);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        off = (off + 255) & ~static_cast<size_t>(255);
        unsigned char* p = base + off;
        off += bytes;
        return p;
    };
    a.split_pr = reinterpret_cast<double*>(take(static_cast<size_t>(B) * slots * sizeof(double)));
    a.split_pp = reinterpret_cast<float*>(take(static_cast<size_t>(B) * slots * sizeof(float)));
    a.split_rec = take(static_cast<size_t>(B) * kSplitMax * sizeof(SliceRec));
    a.split_S = S;
}
// Enough slices to put about two workgroups on every CU, at least one chunk each;
// two per row for untransformed batches of 65 to 192 rows.
// Measured (K = 8, V = 128256; µs per call, split / one workgroup per row): T = 1:
// B = 32 48.0 / 60.2, B = 64 62.8 / 72.7, B = 96 79.3 (S = 2) / 83.1,
// B = 128 91.2 (S = 2) / 95.7;
// transformed (T = 0.7): B = 64 (K = 7) 118.8 / 178.6, B = 128 219.3 / 259.9,
// B = 192 322 (S = 2) to 315 (S = 8) / 328, B = 256 397-420 / 398.
// Larger batches keep one workgroup per row (their draws already fill the GPU).
int dense_split_slices(int B, int V, bool transformed, int forced) {
    if (forced <= 0 && B > (transformed ? 160 : 192)) return 1;
    const int C = split_chunks(V);
    int S = forced > 0 ? forced : (!transformed && B > 64) ? 2 : (512 + B - 1) / B;
    if (S > C) S = C;
    if (S > kSplitMax) S = kSplitMax;
    return S < 1 ? 1 : S;
}

hipError_t launch_chain_dense(const ChainArgs& a, double bracket, hipStream_t s, Timing t) {
    const int esz = a.dtype ? 2 : 4;
    const bool vec = vec_ok(a.logits, a.V, esz) && vec_ok(a.q, a.V, 4);
    if (a.transformed) {
        if (a.dtype == 1) return vec ? dense_launch<1, true, true>(a, bracket, s, t) : dense_launch<1, false, true>(a, bracket, s, t);
        return vec ? dense_launch<0, true, true>(a, bracket, s, t) : dense_launch<0, false, true>(a, bracket, s, t);
    }
    if (a.dtype == 1) return vec ? dense_launch<1, true, false>(a, bracket, s, t) : dense_launch<1, false, false>(a, bracket, s, t);
    return vec ? dense_launch<0, true, false>(a, bracket, s, t) : dense_launch<0, false, false>(a, bracket, s, t);
}
#endif

}  // namespace sv
