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
// CDF boundary within 1e-5 of u*S, so the row is recomputed in fp64 end to end:
// one fp64 exponential per element (a table-driven exponential, below), fp64
// weights and sums.  The one row per batch entry is split into chunks of 8192
// elements spread over the whole chip, in three launches:
//   dense_sum_kernel       per chunk: sum_i exp((z_i - m)/T) (and, when the
//                          draft is transformed, sum_i q_i^(1/T)) in fp64;
//   dense_residual_kernel  per chunk (rows with a rejection): sum of the
//                          residual weights given the exact row normalisers;
//                          invalid draft probabilities flag the chunk (E3);
//   dense_draw_kernel      per batch entry: picks the chunk holding u*S from
//                          the chunk sums, rescans that chunk element by
//                          element and writes the outputs.
// Every kernel derives the first rejection j from the row statistics itself
// (one wave, K+1 lanes), so no kernel waits for another workgroup.

#include <math.h>

#include "common.hpp"
#include "internal.hpp"
#include "lists.hpp"

namespace sv {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kEPT = kDenseChunk / kThreads;        // 32 elements per thread per chunk
constexpr int kSub = kEPT / 8;                      // 8-element groups per thread

// exp(x) for x <= 0 in fp64, by Tang's table-driven method (ACM TOMS 15(2),
// 1989): x = N ln2/64 + r with N = round(64 x / ln2) and |r| <= ln2/128, so
// exp(x) = 2^(N div 64) * 2^((N mod 64)/64) * exp(r); exp(r) - 1 is its Taylor
// series to r^6 (truncation < 3e-20 relative).  tbl[t] = 2^(t/64).  Arguments
// below -800 give 0 (as exp does in double); x = -inf is such an argument.
__device__ __forceinline__ double exp_nonpos(double x, const double* tbl) {
    constexpr double kInvStep = 92.33248261689366;           // 64 / ln 2
    constexpr double kStepHi = 0x1.62e42fefa39efp-7;         // ln 2 / 64, leading part
    constexpr double kStepLo = 0x1.abc9e3b39803fp-62;        // ln 2 / 64 - kStepHi
    x = fmax(x, -800.0);
    const double n = __builtin_rint(x * kInvStep);
    const int N = static_cast<int>(n);
    double r = fma(-n, kStepHi, x);
    r = fma(-n, kStepLo, r);
    double p = fma(r, 1.0 / 720.0, 1.0 / 120.0);
    p = fma(r, p, 1.0 / 24.0);
    p = fma(r, p, 1.0 / 6.0);
    p = fma(r, p, 0.5);
    p = fma(r, p, 1.0);
    p *= r;                                                  // exp(r) - 1
    const double t = tbl[N & 63];
    return ldexp(fma(t, p, t), N >> 6);
}

__device__ __forceinline__ void fill_exp_table(double* tbl) {
    if (threadIdx.x < 64) tbl[threadIdx.x] = exp2(static_cast<double>(threadIdx.x) * (1.0 / 64.0));
}

// Eight consecutive logits from i0 (a multiple of 8); -inf past V.
template <int DT, bool VEC, bool NT>
__device__ __forceinline__ void load8_z(const char* row, int i0, int V, float out[8]) {
    using E = Elem<DT>;
    if (VEC && i0 + 8 <= V) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row + static_cast<long>(i0) * E::kBytes);
        if (DT == 1) {
            const u32x4 v = NT ? load_stream(p) : p[0];
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] = E::get(v, e);
        } else {
            const u32x4 a = NT ? load_stream(p) : p[0];
            const u32x4 b = NT ? load_stream(p + 1) : p[1];
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
    if (VEC && i0 + 8 <= V) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row + i0);
        const u32x4 a = NT ? load_stream(p) : p[0];
        const u32x4 b = NT ? load_stream(p + 1) : p[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) { out[e] = __uint_as_float(a[e]); out[4 + e] = __uint_as_float(b[e]); }
        return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (i0 + e < V) ? row[i0 + e] : 0.f;
}

// Ratio tests of batch row b from the row statistics (lanes k = 0..K of wave 0):
// sets *j (first rejection, K if none) and *err (E1..E5); writes p'_k(x_k) and
// q'_k(x_k) to diag when given.  Call from the whole of wave 0.
template <bool TR>
__device__ __forceinline__ void first_reject(const ChainArgs& a, int b, float* diag, int* j_out, int* err_out) {
    const int K = a.K, V = a.V;
    const int k = threadIdx.x;
    const long rbase = static_cast<long>(b) * (K + 1);
    bool bad = false, rej = false;
    double pk = NAN, qk = NAN;
    if (k <= K) {
        bad |= (a.st.flags[rbase + k] != 0u);
        bad |= !u_ok(a.u[rbase + k]);
    }
    if (k < K) {
        const int x = a.x[static_cast<long>(b) * K + k];
        bad |= (x < 0 || x >= V);
        if (x >= 0 && x < V) {
            const float qx = a.q[(static_cast<long>(b) * K + k) * V + x];
            bad |= !q_ok(qx);
            if (TR) bad |= (a.qflags[static_cast<long>(b) * K + k] != 0u);
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
    const unsigned long long bm = __ballot(bad);
    const unsigned long long rm = __ballot(rej && k < K);
    if (diag && k < K) {
        diag[k] = bm ? NAN : static_cast<float>(pk);
        diag[K + k] = bm ? NAN : static_cast<float>(qk);
    }
    if (k == 0) {
        *j_out = rm ? __ffsll(static_cast<long long>(rm)) - 1 : K;
        *err_out = bm != 0ull;
    }
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

// Sum over a batch row's chunks, in chunk order (the same order in every kernel).
__device__ __forceinline__ double chunk_total(const double* part, long base, int C) {
    double s = 0.0;
    for (int c = 0; c < C; ++c) s += part[base + c];
    return s;
}

template <int DT, bool VEC, bool TR>
__global__ __launch_bounds__(kThreads) void dense_sum_kernel(ChainArgs a, DenseParts d) {
    __shared__ double tbl[64];
    __shared__ double red[2][kWaves];
    __shared__ int s_j, s_err;
    const long blk = blockIdx.x;
    const int b = static_cast<int>(blk / d.C);
    const int c = static_cast<int>(blk - static_cast<long>(b) * d.C);
    fill_exp_table(tbl);
    if (threadIdx.x < kWave) first_reject<TR>(a, b, nullptr, &s_j, &s_err);
    __syncthreads();
    if (s_err) return;
    const int j = s_j, K = a.K, V = a.V;
    const long zrow = static_cast<long>(b) * (K + 1) + j;
    const char* zr = static_cast<const char*>(a.logits) + zrow * V * Elem<DT>::kBytes;
    const double m = static_cast<double>(a.st.m[zrow]);
    const int start = c * kDenseChunk;
    float z[kSub][8];
#pragma unroll
    for (int g = 0; g < kSub; ++g) load8_z<DT, VEC, true>(zr, start + (g * kThreads + threadIdx.x) * 8, V, z[g]);
    double acc = 0.0;
#pragma unroll
    for (int g = 0; g < kSub; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += exp_nonpos((static_cast<double>(z[g][e]) - m) * a.invT, tbl);
    double accq = 0.0;
    if (TR && j < K) {
        const float* qr = a.q + (static_cast<long>(b) * K + j) * V;
#pragma unroll 1
        for (int g = 0; g < kSub; ++g) {
            float q[8];
            load8_q<VEC, true>(qr, start + (g * kThreads + threadIdx.x) * 8, V, q);
#pragma unroll 1
            for (int e = 0; e < 8; ++e)
                if (q[e] > 0.f) accq += pow(static_cast<double>(q[e]), a.invT);
        }
    }
    acc = block_sum(acc, red[0]);
    if (TR) accq = block_sum(accq, red[1]);
    if (threadIdx.x == 0) {
        d.pe[blk] = acc;
        if (TR) d.pq[blk] = accq;
    }
}

// Residual weight max(0, e_i/Zp - q'_i), q'_i = q_i or (TR) q_i^(1/T)/Zq.
template <bool TR>
__device__ __forceinline__ double residual_w(double e, float q, double invZp, double invT, double invZq) {
    double qq = static_cast<double>(q);
    if (TR) qq = (q > 0.f) ? pow(qq, invT) * invZq : 0.0;
    const double r = e * invZp - qq;
    return r > 0.0 ? r : 0.0;
}

template <int DT, bool VEC, bool TR>
__global__ __launch_bounds__(kThreads) void dense_residual_kernel(ChainArgs a, DenseParts d) {
    __shared__ double tbl[64];
    __shared__ double red[kWaves];
    __shared__ int s_j, s_err;
    const long blk = blockIdx.x;
    const int b = static_cast<int>(blk / d.C);
    const int c = static_cast<int>(blk - static_cast<long>(b) * d.C);
    fill_exp_table(tbl);
    if (threadIdx.x < kWave) first_reject<TR>(a, b, nullptr, &s_j, &s_err);
    __syncthreads();
    const int j = s_j, K = a.K, V = a.V;
    if (s_err || j == K) return;
    const long zrow = static_cast<long>(b) * (K + 1) + j;
    const char* zr = static_cast<const char*>(a.logits) + zrow * V * Elem<DT>::kBytes;
    const float* qr = a.q + (static_cast<long>(b) * K + j) * V;
    const double m = static_cast<double>(a.st.m[zrow]);
    const long pbase = static_cast<long>(b) * d.C;
    const double invZp = 1.0 / chunk_total(d.pe, pbase, d.C);
    const double invZq = TR ? 1.0 / chunk_total(d.pq, pbase, d.C) : 1.0;
    const int start = c * kDenseChunk;
    float z[kSub][8], q[kSub][8];
#pragma unroll
    for (int g = 0; g < kSub; ++g) {
        const int i0 = start + (g * kThreads + threadIdx.x) * 8;
        load8_z<DT, VEC, true>(zr, i0, V, z[g]);
        load8_q<VEC, true>(qr, i0, V, q[g]);
    }
    double acc = 0.0;
    bool bad = false;
    auto one = [&](int g, int e) {
        const int i = start + (g * kThreads + threadIdx.x) * 8 + e;
        bad |= (i < V) && !q_ok(q[g][e]);
        const double ex = exp_nonpos((static_cast<double>(z[g][e]) - m) * a.invT, tbl);
        acc += residual_w<TR>(ex, q[g][e], invZp, a.invT, invZq);
    };
    if constexpr (TR) {
        // q^(1/T) in fp64 is long: one element at a time keeps the registers in check.
#pragma unroll
        for (int g = 0; g < kSub; ++g)
#pragma unroll 1
            for (int e = 0; e < 8; ++e) one(g, e);
    } else {
#pragma unroll
        for (int g = 0; g < kSub; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) one(g, e);
    }
    const unsigned long long bb = __ballot(bad);
    acc = block_sum(acc, red);
    __shared__ uint32_t s_bad;
    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0 && bb) atomicOr(&s_bad, 1u);
    __syncthreads();
    if (threadIdx.x == 0) {
        d.pr[blk] = acc;
        d.pflag[blk] = s_bad;
    }
}

template <int DT, bool VEC, bool TR>
__global__ __launch_bounds__(kThreads, 2) void dense_draw_kernel(ChainArgs a, DenseParts d) {
    __shared__ double tbl[64];
    __shared__ double red[kWaves];
    __shared__ int ired[kWaves];
    __shared__ int s_j, s_err, s_chunk, s_fallback;
    __shared__ double s_before;
    const int b = blockIdx.x;
    const int K = a.K, V = a.V, C = d.C;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
    const long rbase = static_cast<long>(b) * (K + 1);
    float* diag = a.out_diag ? a.out_diag + static_cast<long>(b) * (2 * K + 2) : nullptr;
    fill_exp_table(tbl);
    if (tid < kWave) first_reject<TR>(a, b, diag, &s_j, &s_err);
    __syncthreads();
    const int j = s_j;
    const long pbase = static_cast<long>(b) * C;
    bool err = s_err != 0;
    double Zp = 1.0, Zq = 1.0, S = 0.0;
    if (!err) {
        Zp = chunk_total(d.pe, pbase, C);
        if (j < K) {
            S = chunk_total(d.pr, pbase, C);
            for (int c = 0; c < C; ++c) err |= d.pflag[pbase + c] != 0u;
            if (TR) {
                Zq = chunk_total(d.pq, pbase, C);
                err |= !(Zq > 0.0);
            }
        }
    }
    if (err) {
        for (int t = tid; t <= K; t += kThreads) a.out_tokens[rbase + t] = -1;
        if (tid == 0) a.out_accept_len[b] = -1;
        if (diag)
            for (int t = tid; t < 2 * K + 2; t += kThreads) diag[t] = NAN;
        return;
    }
    const bool residual = j < K && S > 0.0;
    const double W = residual ? S : Zp;
    const double* part = residual ? d.pr : d.pe;
    const double target = static_cast<double>(a.u[rbase + K]) * W;
    if (tid == 0) {
        double before = 0.0;
        int chunk = -1, last = 0;
        for (int c = 0; c < C; ++c) {
            const double pc = part[pbase + c];
            if (target < before + pc) { chunk = c; break; }
            before += pc;
            if (pc > 0.0) last = c;
        }
        s_fallback = chunk < 0;
        if (chunk < 0) {        // rounding: u*W at or past the total
            chunk = last;
            before = 0.0;       // unused
        }
        s_chunk = chunk;
        s_before = before;
    }
    __syncthreads();
    const int chunk = s_chunk;
    const bool fallback = s_fallback != 0;

    // Rescan the chunk: thread t holds elements [t*32, t*32 + 32) of it.
    const long zrow = rbase + j;
    const char* zr = static_cast<const char*>(a.logits) + zrow * V * Elem<DT>::kBytes;
    const float* qr = residual ? a.q + (static_cast<long>(b) * K + j) * V : nullptr;
    const double m = static_cast<double>(a.st.m[zrow]);
    const double invZp = 1.0 / Zp, invZq = 1.0 / Zq;
    const int i0 = chunk * kDenseChunk + tid * kEPT;
    // Two passes over the thread's 32 elements (recomputing beats holding 32
    // doubles): thread sums, then the crossing after the block's prefix.
    auto weights8 = [&](int g, double wt[8]) {
        float z[8], q[8];
        load8_z<DT, VEC, false>(zr, i0 + 8 * g, V, z);
        if (residual) load8_q<VEC, false>(qr, i0 + 8 * g, V, q);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double ex = exp_nonpos((static_cast<double>(z[e]) - m) * a.invT, tbl);
            wt[e] = residual ? residual_w<TR>(ex, q[e], invZp, a.invT, invZq) : ex;
            if (i0 + 8 * g + e >= V) wt[e] = 0.0;
        }
    };
    double s = 0.0, wlast = 0.0;
    int lastpos = -1;
#pragma unroll 1
    for (int g = 0; g < kSub; ++g) {
        double wt[8];
        weights8(g, wt);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s += wt[e];
            if (wt[e] > 0.0) { lastpos = i0 + 8 * g + e; wlast = wt[e]; }
        }
    }
    // Exclusive prefix of the thread sums in index order.
    double incl = s;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) red[wid] = incl;
    __syncthreads();
    double cum = s_before;
    for (int x = 0; x < wid; ++x) cum += red[x];
    cum += incl - s;
    int found = 0x7fffffff;
    double wfound = 0.0;
    // Threads whose span ends past u*W rescan; the smallest crossing wins.
    if (!fallback && target < cum + s) {
#pragma unroll 1
        for (int g = 0; g < kSub && found == 0x7fffffff; ++g) {
            double wt[8];
            weights8(g, wt);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                cum += wt[e];
                if (found == 0x7fffffff && wt[e] > 0.0 && target < cum) { found = i0 + 8 * g + e; wfound = wt[e]; }
            }
        }
    }
    // Smallest crossing index; if rounding left none in the chunk, its last positive index.
    int y = wave_min_int(found);
    const int lp = wave_max_int(lastpos);
    __syncthreads();
    if (lane == 0) { ired[wid] = y; red[wid] = static_cast<double>(lp); }
    __syncthreads();
    y = ired[0];
    int lpb = static_cast<int>(red[0]);
#pragma unroll
    for (int x = 1; x < kWaves; ++x) { y = min(y, ired[x]); lpb = max(lpb, static_cast<int>(red[x])); }
    const bool crossed = y != 0x7fffffff;
    if (!crossed) y = lpb;
    const double my = crossed ? (found == y ? wfound : 0.0) : (lastpos == y ? wlast : 0.0);
    const double wy = block_sum(my, red);

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

template <int DT, bool VEC, bool TR>
hipError_t dense_launch(const ChainArgs& a, const DenseParts& d, unsigned chunks, hipStream_t s) {
    hipLaunchKernelGGL((dense_sum_kernel<DT, VEC, TR>), dim3(chunks), dim3(kThreads), 0, s, a, d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dense_residual_kernel<DT, VEC, TR>), dim3(chunks), dim3(kThreads), 0, s, a, d);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dense_draw_kernel<DT, VEC, TR>), dim3(a.B), dim3(kThreads), 0, s, a, d);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chain_dense(const ChainArgs& a, const DenseParts& d, hipStream_t s) {
    const int esz = a.dtype ? 2 : 4;
    const bool vec = vec_ok(a.logits, a.V, esz) && vec_ok(a.q, a.V, 4);
    const unsigned chunks = static_cast<unsigned>(static_cast<long>(a.B) * d.C);
    if (a.dtype == 1) {
        if (vec) return a.transformed ? dense_launch<1, true, true>(a, d, chunks, s) : dense_launch<1, true, false>(a, d, chunks, s);
        return a.transformed ? dense_launch<1, false, true>(a, d, chunks, s) : dense_launch<1, false, false>(a, d, chunks, s);
    }
    if (vec) return a.transformed ? dense_launch<0, true, true>(a, d, chunks, s) : dense_launch<0, true, false>(a, d, chunks, s);
    return a.transformed ? dense_launch<0, false, true>(a, d, chunks, s) : dense_launch<0, false, false>(a, d, chunks, s);
}

}  // namespace sv
