// Per-batch-row verification: ratio tests, first-rejection scan, final draw.
//
// The loop follows "064 · 投机解码", section 三: for positions k = 0, 1, ...
// accept x_k iff u_k < min(1, p'_k(x_k) / q'_k(x_k)) (acceptance a(x) of
// section 二); at the first rejection j draw one token from
// r = max(0, p'_j - q'_j) normalised (zero mass: from p'_j, as the residual
// routine of "Việc giải mã giả định và EAGLE-3", step 2, does); if nothing is
// rejected draw the bonus token from p'_K.  The draw is an inverse CDF over
// token indices in ascending order driven by u_K.
//
// The K tests are independent of each other, so they run in parallel lanes
// and the first rejection is a ballot.  This file holds the greedy chain, the
// static tree and the acceptance rate; the top-k chain finishes inside its
// selection launch (chain_finish.hpp) and the dense path is in dense_impl.hpp.

#include "common.hpp"
#include "internal.hpp"
#include "lists.hpp"

namespace sv {

namespace {

// Greedy chain: argmax comparisons only, walking positions left to right.  A
// row's flags count only if the walk reaches it; every token is range-checked.
__global__ void chain_greedy_kernel(ChainArgs a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.B) return;
    const int K = a.K, V = a.V;
    const long rbase = static_cast<long>(b) * (K + 1);
    float* diag = a.out_diag ? a.out_diag + static_cast<long>(b) * (2 * K + 2) : nullptr;
    bool bad = false;
    for (int k = 0; k < K; ++k) {
        const int x = a.x[static_cast<long>(b) * K + k];
        bad |= (x < 0 || x >= V);
    }
    int j = K;
    if (!bad) {
        for (int k = 0; k <= K; ++k) {
            if (a.st.flags[rbase + k] != 0u) { bad = true; break; }
            if (k == K) break;
            if (a.x[static_cast<long>(b) * K + k] != a.st.arg[rbase + k]) { j = k; break; }
        }
    }
    if (bad) {
        for (int t = 0; t <= K; ++t) a.out_tokens[rbase + t] = -1;
        a.out_accept_len[b] = -1;
        if (diag) for (int t = 0; t < 2 * K + 2; ++t) diag[t] = NAN;
        return;
    }
    if (diag) {
        for (int k = 0; k < K; ++k) {
            diag[k] = k < j ? 1.f : (k == j ? 0.f : NAN);
            diag[K + k] = NAN;
        }
    }
    for (int t = 0; t <= K; ++t)
        a.out_tokens[rbase + t] = t < j ? a.x[static_cast<long>(b) * K + t] : (t == j ? a.st.arg[rbase + j] : -1);
    a.out_accept_len[b] = j;
    if (diag) { diag[2 * K] = 1.f; diag[2 * K + 1] = 1.f; }
}

// Tree, greedy: one wave per batch entry, one lane per node.  The tree is the
// static one of the arguments, or the batch row's own (parents_rows), checked
// here: parents[0] = -1 and 0 <= parents[n] < n, else the row is an error.
__global__ __launch_bounds__(kWave) void tree_kernel(TreeArgs a) {
    __shared__ int sp[kWave];
    const int b = blockIdx.x;
    const int n = threadIdx.x;
    const int N = a.N, D = a.D;
    const bool node = n < N;
    const long base = static_cast<long>(b) * N;
    bool bad = false;
    if (a.parents_rows) {
        int p = node ? a.parents_rows[base + n] : -1;
        bad = node && (n == 0 ? p != -1 : (p < 0 || p >= n));
        sp[n] = bad ? -1 : p;
    } else {
        sp[n] = node ? a.parents[n] : -1;
    }
    __syncthreads();
    const int par = sp[n];
    int depth = 0;
    for (int p = par; p >= 0; p = sp[p]) ++depth;
    const int g = node ? a.st.arg[base + n] : -1;
    const int tok = (node && n > 0) ? a.node_tokens[base + n] : -1;
    bad |= node && a.st.flags[base + n] != 0u;
    bad |= node && n > 0 && (tok < 0 || tok >= a.V);
    int32_t* op = a.out_path + static_cast<long>(b) * (D + 1);
    int32_t* ot = a.out_tokens + static_cast<long>(b) * (D + 1);
    if (__ballot(bad)) {
        for (int t = n; t <= D; t += kWave) { op[t] = -1; ot[t] = -1; }
        if (n == 0) a.out_accept_len[b] = -1;
        return;
    }
    bool acc = (n == 0);
    for (int d = 1; d <= D; ++d) {
        const int ps = par < 0 ? 0 : par;
        const bool ap = __shfl(static_cast<int>(acc), ps, kWave) != 0;
        const int gp = __shfl(g, ps, kWave);
        if (node && depth == d) acc = ap && tok == gp;
    }
    // Deepest accepted node, lowest index on ties.
    int key = (node && acc) ? (depth << 8) | (255 - n) : -1;
    key = wave_max_int(key);
    const int best = 255 - (key & 255);
    const int dbest = key >> 8;
    const int gbest = __shfl(g, best, kWave);
    // Path root..best, then the accepted tokens and the bonus argmax.
    __shared__ int path[kWave];
    if (n == 0) {
        int cur = best;
        for (int t = dbest; t >= 0; --t) { path[t] = cur; cur = cur > 0 ? sp[cur] : 0; }
    }
    __syncthreads();
    if (n <= D) {
        op[n] = n <= dbest ? path[n] : -1;
        ot[n] = n < dbest ? a.node_tokens[base + path[n + 1]] : (n == dbest ? gbest : -1);
    }
    if (n == 0) a.out_accept_len[b] = dbest;
}

// alpha = sum_i min(p'_i, q'_i) over dense rows (fp32 terms, fp64 sums), from
// precomputed row statistics: the route for rows too long for the one-pass
// kernel (alpha.hip) or not 16-byte aligned, hence element loads.
template <int DT>
__global__ __launch_bounds__(256) void alpha_dense_kernel(AlphaArgs a) {
    __shared__ double red[4];
    __shared__ uint32_t fred[4];
    const int r = blockIdx.x;                      // b*K + k
    const int b = r / a.K, k = r - b * a.K;
    const long zrow = static_cast<long>(b) * (a.K + 1) + k;
    const char* zr = static_cast<const char*>(a.logits) + zrow * a.V * Elem<DT>::kBytes;
    const float* qr = a.q + static_cast<long>(r) * a.V;
    const float m = a.st.m[r];
    const float invZ = static_cast<float>(1.0 / a.st.Z[r]);
    const float invQ = a.transformed ? static_cast<float>(1.0 / a.qsum[r]) : 1.f;
    double acc = 0.0;
    uint32_t bad = 0;
    for (int i = threadIdx.x; i < a.V; i += 256) {
        const float z = Elem<DT>::scalar(zr, i);
        const float q = qr[i];
        bad |= !q_ok(q);
        const float p = __builtin_amdgcn_exp2f((z - m) * a.scale) * invZ;
        float qq = q;
        if (a.transformed) qq = (q > 0.f) ? __builtin_amdgcn_exp2f(__builtin_amdgcn_logf(q) * a.invT) * invQ : 0.f;
        acc += static_cast<double>(fminf(p, qq));
    }
    acc = wave_sum(acc);
    bad = wave_or(bad);
    if ((threadIdx.x & 63) == 0) { red[threadIdx.x / 64] = acc; fred[threadIdx.x / 64] = bad; }
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = red[0] + red[1] + red[2] + red[3];
        uint32_t f = fred[0] | fred[1] | fred[2] | fred[3] | a.st.flags[r];
        if (a.transformed) f |= a.qflags[r];
        a.out_alpha[r] = f ? NAN : static_cast<float>(s);
    }
}

// ---- top-k acceptance rate (the chain finish is fused into the selection launch) ----

// alpha over the kept sets: one workgroup of two waves per (b, k).
__global__ __launch_bounds__(2 * kWave) void alpha_topk_kernel(AlphaArgs a) {
    __shared__ int32_t sidx[kWave];
    __shared__ double sp[kWave];
    __shared__ int32_t skd, sok;
    const int lane = threadIdx.x & (kWave - 1), wid = wave_id();
    const long r = blockIdx.x;                                  // b*K + k
    const int b = static_cast<int>(r / a.K), k = static_cast<int>(r - static_cast<long>(b) * a.K);
    int it = kNoIndex, kt = 0;
    double pt = 0.0;
    bool ok = false;
    if (wid == 0) ok = position_row(a.tk, b, k, false, it, pt, kt);
    else {
        int id, kd;
        double pd;
        const bool okd = position_row(a.tk, b, k, true, id, pd, kd);
        sidx[lane] = id;
        sp[lane] = pd;
        if (lane == 0) { skd = kd; sok = okd; }
    }
    __syncthreads();
    if (wid != 0) return;
    const double q = lane < kt ? lds_lookup(sidx, sp, skd, it) : 0.0;
    const double s = wave_sum(lane < kt ? fmin(pt, q) : 0.0);
    if (lane == 0) a.out_alpha[r] = (ok && sok) ? static_cast<float>(s) : NAN;
}

__global__ void alpha_greedy_kernel(AlphaArgs a) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= a.B * a.K) return;
    const bool bad = a.st.flags[r] != 0u || a.qst.flags[r] != 0u;
    a.out_alpha[r] = bad ? NAN : (a.st.arg[r] == a.qst.arg[r] ? 1.f : 0.f);
}

}  // namespace

hipError_t launch_chain_greedy(const ChainArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(chain_greedy_kernel, dim3((a.B + 63) / 64), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_tree(const TreeArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(tree_kernel, dim3(a.B), dim3(kWave), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_alpha_dense(const AlphaArgs& a, hipStream_t s) {
    const int R = a.B * a.K;
    if (a.dtype == 1) hipLaunchKernelGGL(alpha_dense_kernel<1>, dim3(R), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(alpha_dense_kernel<0>, dim3(R), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_alpha_topk(const AlphaArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(alpha_topk_kernel, dim3(a.B * a.K), dim3(2 * kWave), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_alpha_greedy(const AlphaArgs& a, hipStream_t s) {
    const int R = a.B * a.K;
    hipLaunchKernelGGL(alpha_greedy_kernel, dim3((R + 63) / 64), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace sv
