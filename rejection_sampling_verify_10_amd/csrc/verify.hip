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
// Dense rows: the K tests are independent of each other, so they run in
// parallel lanes and the first rejection is a ballot.  The final draw touches
// one target row (and one draft row) per batch entry; it is recomputed in fp64
// so that its CDF boundaries sit ~1e-16 from the exact ones: pass A sums
// exp((z - m)/T) per 4096-element tile, pass B (residual only) sums
// max(0, p' - q') per tile, then the tile holding u*S is rescanned element by
// element.

#include "common.hpp"
#include "internal.hpp"
#include "lists.hpp"

namespace sv {

namespace {

constexpr int kDrawThreads = 512;
constexpr int kDrawWaves = kDrawThreads / kWave;
constexpr int kEPT = 8;                                   // elements per thread per tile
constexpr int kTile = kDrawThreads * kEPT;                // 4096
constexpr int kMaxTiles = (kMaxV + kTile - 1) / kTile;


// Loads 8 consecutive logits starting at i0 (multiple of 8); -inf beyond V.
template <int DT, bool VEC>
__device__ __forceinline__ void load8_logits(const char* row, int i0, int V, float out[kEPT]) {
    using E = Elem<DT>;
    if (VEC && DT == 1) {
        if (i0 + 8 <= V) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(row + static_cast<long>(i0) * 2);
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] = E::get(v, e);
            return;
        }
    }
    if (VEC && DT == 0) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row + static_cast<long>(i0) * 4);
        if (i0 + 8 <= V) {
            const u32x4 a = p[0], b = p[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) { out[e] = __uint_as_float(a[e]); out[4 + e] = __uint_as_float(b[e]); }
            return;
        }
    }
#pragma unroll
    for (int e = 0; e < kEPT; ++e) out[e] = (i0 + e < V) ? E::scalar(row, i0 + e) : -INFINITY;
}

template <bool VEC>
__device__ __forceinline__ void load8_probs(const float* row, int i0, int V, float out[kEPT]) {
    if (VEC && i0 + 8 <= V) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row + i0);
        const u32x4 a = p[0], b = p[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) { out[e] = __uint_as_float(a[e]); out[4 + e] = __uint_as_float(b[e]); }
        return;
    }
#pragma unroll
    for (int e = 0; e < kEPT; ++e) out[e] = (i0 + e < V) ? row[i0 + e] : 0.f;
}

struct DrawSmem {
    double wsum[kMaxTiles][kDrawWaves];
    double tsum[kMaxTiles];
    double red[kDrawWaves];
    int ired[kDrawWaves];
    int j, err, tile, y, tail, bad;
    double zp, zq, total, target, before;
};

__device__ __forceinline__ double block_sum_d(double v, DrawSmem& sm) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) sm.red[threadIdx.x / kWave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kDrawWaves; ++w) t += sm.red[w];
    return t;
}

__device__ __forceinline__ int block_min_i(int v, DrawSmem& sm) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, xshfl(v, o));
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) sm.ired[threadIdx.x / kWave] = v;
    __syncthreads();
    int t = sm.ired[0];
#pragma unroll
    for (int w = 1; w < kDrawWaves; ++w) t = min(t, sm.ired[w]);
    return t;
}

__device__ __forceinline__ int block_max_i(int v, DrawSmem& sm) { return -block_min_i(-v, sm); }

// Weight of element i in the final-draw distribution.
//   mode 0: e_i = exp((z_i - m)/T)            (bonus, or zero-residual fallback)
//   mode 1: max(0, e_i/Zp - q'_i)             (residual)
struct DrawRow {
    const char* z;
    const float* q;
    int V;
    double m, invT, inv_zp, inv_zq;
    int transformed;
};

template <int DT, bool VEC>
__device__ __forceinline__ void tile_weights(const DrawRow& r, int mode, int i0, double w[kEPT], bool& bad) {
    float z[kEPT];
    load8_logits<DT, VEC>(r.z, i0, r.V, z);
    if (mode == 0) {
#pragma unroll
        for (int e = 0; e < kEPT; ++e) w[e] = exp((static_cast<double>(z[e]) - r.m) * r.invT);
        return;
    }
    float q[kEPT];
    load8_probs<VEC>(r.q, i0, r.V, q);
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
        bad |= (i0 + e < r.V) && !q_ok(q[e]);
        const double p = exp((static_cast<double>(z[e]) - r.m) * r.invT) * r.inv_zp;
        double qq = static_cast<double>(q[e]);
        if (r.transformed) qq = (q[e] > 0.f) ? pow(qq, r.invT) * r.inv_zq : 0.0;
        const double d = p - qq;
        w[e] = d > 0.0 ? d : 0.0;
    }
}

// Per-tile sums of the weights (mode) into sm.tsum; returns the total.  *qbad
// becomes true (block-uniformly) when a draft probability read is invalid (E3).
template <int DT, bool VEC>
__device__ double tile_sums(const DrawRow& r, int mode, int ntiles, DrawSmem& sm, bool* qbad) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    bool bad = false;
    if (threadIdx.x == 0) sm.bad = 0;
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        double w[kEPT];
        tile_weights<DT, VEC>(r, mode, t * kTile + threadIdx.x * kEPT, w, bad);
        double s = 0.0;
#pragma unroll
        for (int e = 0; e < kEPT; ++e) s += w[e];
        s = wave_sum(s);
        if (lane == 0) sm.wsum[t][wid] = s;
    }
    if (__ballot(bad) && lane == 0) atomicOr(&sm.bad, 1);
    __syncthreads();
    for (int t = threadIdx.x; t < ntiles; t += kDrawThreads) {
        double s = 0.0;
#pragma unroll
        for (int w = 0; w < kDrawWaves; ++w) s += sm.wsum[t][w];
        sm.tsum[t] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double tot = 0.0;
        for (int t = 0; t < ntiles; ++t) tot += sm.tsum[t];
        sm.total = tot;
    }
    __syncthreads();
    if (qbad) *qbad = sm.bad != 0;
    return sm.total;
}

// Inverse CDF: smallest index i with target < C_i, C the index-ascending
// inclusive prefix of the weights; rounding fallback = last positive weight.
template <int DT, bool VEC>
__device__ int draw_from(const DrawRow& r, int mode, int ntiles, double target, DrawSmem& sm, double* wy) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    if (threadIdx.x == 0) {
        double before = 0.0;
        int tile = -1, tail = -1;
        for (int t = 0; t < ntiles; ++t) {
            if (sm.tsum[t] > 0.0) tail = t;
            if (tile < 0 && target < before + sm.tsum[t]) { tile = t; break; }
            before += sm.tsum[t];
        }
        if (tile < 0) {
            for (int t = ntiles - 1; t >= 0; --t) if (sm.tsum[t] > 0.0) { tail = t; break; }
        }
        sm.tile = tile;
        sm.tail = tail;
        sm.before = before;
    }
    __syncthreads();
    const int tile = sm.tile;
    const int t_use = tile >= 0 ? tile : (sm.tail >= 0 ? sm.tail : 0);
    double w[kEPT];
    const int i0 = t_use * kTile + threadIdx.x * kEPT;
    bool unused = false;
    tile_weights<DT, VEC>(r, mode, i0, w, unused);
    int found = 0x7fffffff;
    int lastpos = -1;
#pragma unroll
    for (int e = 0; e < kEPT; ++e) if (w[e] > 0.0 && i0 + e < r.V) lastpos = i0 + e;
    if (tile >= 0) {
        double s = 0.0;
#pragma unroll
        for (int e = 0; e < kEPT; ++e) s += w[e];
        // exclusive scan of the thread sums across the block
        double incl = s;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            double t = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += t;
        }
        if (lane == kWave - 1) sm.red[wid] = incl;
        __syncthreads();
        double base = sm.before;
        for (int x = 0; x < wid; ++x) base += sm.red[x];
        double c = base + incl - s;
#pragma unroll
        for (int e = 0; e < kEPT; ++e) {
            c += w[e];
            if (found == 0x7fffffff && target < c && w[e] > 0.0) found = i0 + e;
        }
    }
    int y = block_min_i(found, sm);
    if (y == 0x7fffffff) y = block_max_i(lastpos, sm);
    // weight of the drawn token
    double my = 0.0;
#pragma unroll
    for (int e = 0; e < kEPT; ++e) if (i0 + e == y) my = w[e];
    *wy = block_sum_d(my, sm);
    return y;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kDrawThreads) void chain_dense_kernel(ChainArgs a) {
    __shared__ DrawSmem sm;
    const int b = blockIdx.x;
    const int K = a.K, V = a.V;
    const int tid = threadIdx.x;
    const long rbase = static_cast<long>(b) * (K + 1);
    float* diag = a.out_diag ? a.out_diag + static_cast<long>(b) * (2 * K + 2) : nullptr;

    if (tid < kWave) {
        const int k = tid;
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
                if (a.transformed) bad |= (a.qflags[static_cast<long>(b) * K + k] != 0u);
                const double zx = static_cast<double>(a.st.zx[rbase + k]);
                pk = exp((zx - static_cast<double>(a.st.m[rbase + k])) * a.invT) / a.st.Z[rbase + k];
                qk = static_cast<double>(qx);
                if (a.transformed)
                    qk = (qx > 0.f) ? pow(qk, a.invT) / a.qsum[static_cast<long>(b) * K + k] : 0.0;
                double ratio;
                if (qk > 0.0) ratio = pk / qk;
                else ratio = pk > 0.0 ? INFINITY : 0.0;
                const double thr = ratio < 1.0 ? ratio : 1.0;
                rej = !(static_cast<double>(a.u[rbase + k]) < thr);
            }
        }
        const unsigned long long bm = __ballot(bad);
        const unsigned long long rm = __ballot(rej && k < K);
        const int j = rm ? __ffsll(static_cast<long long>(rm)) - 1 : K;
        if (diag && k < K) {
            diag[k] = bm ? NAN : static_cast<float>(pk);
            diag[K + k] = bm ? NAN : static_cast<float>(qk);
        }
        if (tid == 0) {
            sm.j = j;
            sm.err = bm != 0ull;
        }
    }
    __syncthreads();
    const int j = sm.j;
    if (sm.err) {
        for (int t = tid; t <= K; t += kDrawThreads) a.out_tokens[rbase + t] = -1;
        if (tid == 0) {
            a.out_accept_len[b] = -1;
            if (diag) { diag[2 * K] = NAN; diag[2 * K + 1] = NAN; }
        }
        return;
    }

    const long zrow = rbase + j;
    DrawRow r;
    r.z = static_cast<const char*>(a.logits) + zrow * V * Elem<DT>::kBytes;
    r.q = (j < K) ? a.q + (static_cast<long>(b) * K + j) * V : nullptr;
    r.V = V;
    r.m = static_cast<double>(a.st.m[zrow]);
    r.invT = a.invT;
    r.transformed = a.transformed;
    const int ntiles = (V + kTile - 1) / kTile;

    // Pass A: exact normaliser of p'_j.
    const double zp = tile_sums<DT, VEC>(r, 0, ntiles, sm, nullptr);
    r.inv_zp = 1.0 / zp;
    r.inv_zq = 1.0;
    int mode = 0;
    double W = zp;
    bool qbad = false;
    if (j < K) {
        if (a.transformed) {
            // Exact normaliser of q'_j = q_j^(1/T) / sum q_j^(1/T) (top-k is off here).
            double zq = 0.0;
            bool badq = false;
            for (int i = tid; i < V; i += kDrawThreads) {
                const float v = r.q[i];
                badq |= !q_ok(v);
                if (v > 0.f) zq += pow(static_cast<double>(v), a.invT);
            }
            const unsigned long long bq = __ballot(badq);
            if ((tid & (kWave - 1)) == 0) sm.ired[tid / kWave] = bq != 0ull;
            zq = block_sum_d(zq, sm);
            for (int w = 0; w < kDrawWaves; ++w) qbad |= sm.ired[w] != 0;
            qbad |= !(zq > 0.0);
            r.inv_zq = 1.0 / zq;
        }
        __syncthreads();
        bool badb = false;
        const double S = tile_sums<DT, VEC>(r, 1, ntiles, sm, &badb);
        qbad |= badb;
        if (!qbad) {
            if (S > 0.0) {
                mode = 1;
                W = S;
            } else {
                __syncthreads();
                tile_sums<DT, VEC>(r, 0, ntiles, sm, nullptr);   // restore the p' tile sums
            }
        }
    }
    if (qbad) {
        for (int t = tid; t <= K; t += kDrawThreads) a.out_tokens[rbase + t] = -1;
        if (tid == 0) {
            a.out_accept_len[b] = -1;
            if (diag)
                for (int k = 0; k < 2 * K + 2; ++k) diag[k] = NAN;
        }
        return;
    }
    const double target = static_cast<double>(a.u[rbase + K]) * W;
    double wy;
    const int y = draw_from<DT, VEC>(r, mode, ntiles, target, sm, &wy);

    for (int t = tid; t <= K; t += kDrawThreads) {
        int tok = -1;
        if (t < j) tok = a.x[static_cast<long>(b) * K + t];
        else if (t == j) tok = y;
        a.out_tokens[rbase + t] = tok;
    }
    if (tid == 0) {
        a.out_accept_len[b] = j;
        if (diag) {
            diag[2 * K] = static_cast<float>(mode == 1 ? W : W / zp);
            diag[2 * K + 1] = static_cast<float>(wy / W);
        }
    }
}

// Greedy chain: argmax comparisons only.
__global__ void chain_greedy_kernel(ChainArgs a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.B) return;
    const int K = a.K, V = a.V;
    const long rbase = static_cast<long>(b) * (K + 1);
    float* diag = a.out_diag ? a.out_diag + static_cast<long>(b) * (2 * K + 2) : nullptr;
    bool bad = false;
    for (int k = 0; k <= K; ++k) bad |= a.st.flags[rbase + k] != 0u;
    for (int k = 0; k < K; ++k) {
        const int x = a.x[static_cast<long>(b) * K + k];
        bad |= (x < 0 || x >= V);
    }
    if (bad) {
        for (int t = 0; t <= K; ++t) a.out_tokens[rbase + t] = -1;
        a.out_accept_len[b] = -1;
        if (diag) for (int t = 0; t < 2 * K + 2; ++t) diag[t] = NAN;
        return;
    }
    int j = K;
    for (int k = 0; k < K; ++k) {
        const bool match = a.x[static_cast<long>(b) * K + k] == a.st.arg[rbase + k];
        if (diag) { diag[k] = match ? 1.f : 0.f; diag[K + k] = NAN; }
        if (!match && j == K) j = k;
    }
    for (int t = 0; t <= K; ++t)
        a.out_tokens[rbase + t] = t < j ? a.x[static_cast<long>(b) * K + t] : (t == j ? a.st.arg[rbase + j] : -1);
    a.out_accept_len[b] = j;
    if (diag) { diag[2 * K] = 1.f; diag[2 * K + 1] = 1.f; }
}

// Static tree, greedy: one wave per batch entry, one lane per node.
__global__ __launch_bounds__(kWave) void tree_kernel(TreeArgs a) {
    const int b = blockIdx.x;
    const int n = threadIdx.x;
    const int N = a.N, D = a.D;
    const bool node = n < N;
    const long base = static_cast<long>(b) * N;
    const int par = node ? a.parents[n] : -1;
    int depth = 0;
    for (int p = par; p >= 0; p = a.parents[p]) ++depth;
    const int g = node ? a.st.arg[base + n] : -1;
    const int tok = (node && n > 0) ? a.node_tokens[base + n] : -1;
    bool bad = node && a.st.flags[base + n] != 0u;
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
        for (int t = dbest; t >= 0; --t) { path[t] = cur; cur = cur > 0 ? a.parents[cur] : 0; }
    }
    __syncthreads();
    if (n <= D) {
        op[n] = n <= dbest ? path[n] : -1;
        ot[n] = n < dbest ? a.node_tokens[base + path[n + 1]] : (n == dbest ? gbest : -1);
    }
    if (n == 0) a.out_accept_len[b] = dbest;
}

// alpha = sum_i min(p'_i, q'_i) over dense rows (fp32 terms, fp64 sums).
template <int DT, bool VEC>
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

// ---- top-k path: merge the chunk lists of each position, test, draw, combine ----

// Kept distribution of row (b, k): target (draft = false) or draft.
__device__ __forceinline__ bool position_row(const TopkLists& t, int b, int k, bool draft, int& idx, double& p,
                                             int& kk) {
    const long unit0 = t.unit_base(b, k) + (draft ? t.Ct : 0);
    float v;
    int i;
    uint32_t flags = 0;
    const int tot = merge_global_lists(t, unit0, draft ? t.Cd : t.Ct, v, i, flags);
    kk = tot < t.top_k ? tot : t.top_k;
    return kept_distribution(v, i, kk, flags == 0u, draft, t.invT, draft && t.draft_identity, idx, p);
}

// One workgroup of two waves per position (b, k): wave 0 merges target row k's
// chunk lists, wave 1 draft row k's, in parallel; wave 0 then runs test k and
// draws the token that would be emitted if k were the first rejection (the bonus
// token for k = K).  One position per workgroup spreads the work over the chip.
__global__ __launch_bounds__(2 * kWave) void chain_topk_position_kernel(ChainArgs a) {
    __shared__ int32_t sidx[kWave];
    __shared__ double sp[kWave];
    __shared__ int32_t skd, sok;
    const int K = a.K, V = a.V;
    const int b = blockIdx.x / (K + 1), k = blockIdx.x - b * (K + 1);
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const long rbase = static_cast<long>(b) * (K + 1);
    const TopkLists& t = a.tk;
    int it = kNoIndex, kt = 0;
    double pt = 0.0;
    bool ok = false;
    if (wid == 0) {
        ok = position_row(t, b, k, false, it, pt, kt);
    } else if (k < K) {
        int id, kd;
        double pd;
        const bool okd = position_row(t, b, k, true, id, pd, kd);
        sidx[lane] = id;
        sp[lane] = pd;
        if (lane == 0) { skd = kd; sok = okd; }
    }
    __syncthreads();
    if (wid != 0) return;
    const float uK = a.u[rbase + K];
    ok = ok && u_ok(a.u[rbase + k]) && u_ok(uK);
    double r = pt, px = 0.0, qx = 0.0;
    bool accept = false;
    if (k < K) {
        const int x = a.x[static_cast<long>(b) * K + k];
        ok = ok && sok && x >= 0 && x < V;
        px = lane_lookup(it, pt, x);
        qx = lds_lookup(sidx, sp, skd, x);
        double ratio;
        if (qx > 0.0) ratio = px / qx;
        else ratio = px > 0.0 ? INFINITY : 0.0;
        const double thr = ratio < 1.0 ? ratio : 1.0;
        accept = static_cast<double>(a.u[rbase + k]) < thr;
        const double q = lane < kt ? lds_lookup(sidx, sp, skd, it) : 0.0;
        r = lane < kt ? fmax(pt - q, 0.0) : 0.0;
    }
    double S = wave_sum(r);
    if (!(S > 0.0)) {                       // zero residual: draw from p'_k
        r = pt;
        S = wave_sum(pt);
    }
    const int src = lane_draw(r, lane < kt, static_cast<double>(uK) * S);
    const int y = bcast(it, src);
    const double ry = bcast(r, src);
    if (lane == 0) {
        PosRecord rc;
        rc.accept = accept;
        rc.y = y;
        rc.bad = !ok;
        rc.pad = 0;
        rc.pk = static_cast<float>(px);
        rc.qk = static_cast<float>(qx);
        rc.S = static_cast<float>(S);
        rc.py = static_cast<float>(ry / S);
        a.rec[rbase + k] = rc;
    }
}

// Per batch row: first rejection j from the position records, emitted tokens
// x_0..x_{j-1}, y_j, accept_len = j.  One wave per batch row.
__global__ __launch_bounds__(4 * kWave) void chain_topk_combine_kernel(ChainArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int b = blockIdx.x * 4 + threadIdx.x / kWave;
    if (b >= a.B) return;
    const int K = a.K;
    const long rb = static_cast<long>(b) * (K + 1);
    bool bad = false;
    for (int k = lane; k <= K; k += kWave) bad |= a.rec[rb + k].bad != 0;
    const bool err = __ballot(bad) != 0ull;
    int j = K;
    for (int base = 0; base < K; base += kWave) {
        const int k = base + lane;
        const unsigned long long rm = __ballot(k < K && !a.rec[rb + k].accept);
        if (rm) { j = base + __ffsll(static_cast<long long>(rm)) - 1; break; }
    }
    float* diag = a.out_diag ? a.out_diag + static_cast<long>(b) * (2 * K + 2) : nullptr;
    for (int k = lane; k <= K; k += kWave) {
        int tok = -1;
        if (!err) tok = k < j ? a.x[static_cast<long>(b) * K + k] : (k == j ? a.rec[rb + j].y : -1);
        a.out_tokens[rb + k] = tok;
        if (diag && k < K) {
            diag[k] = err ? NAN : a.rec[rb + k].pk;
            diag[K + k] = err ? NAN : a.rec[rb + k].qk;
        }
    }
    if (lane == 0) {
        a.out_accept_len[b] = err ? -1 : j;
        if (diag) {
            diag[2 * K] = err ? NAN : a.rec[rb + j].S;
            diag[2 * K + 1] = err ? NAN : a.rec[rb + j].py;
        }
    }
}

// alpha over the kept sets: one workgroup of two waves per (b, k).
__global__ __launch_bounds__(2 * kWave) void alpha_topk_kernel(AlphaArgs a) {
    __shared__ int32_t sidx[kWave];
    __shared__ double sp[kWave];
    __shared__ int32_t skd, sok;
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
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

hipError_t launch_chain_dense(const ChainArgs& a, hipStream_t s) {
    const int esz = a.dtype ? 2 : 4;
    const bool vec = vec_ok(a.logits, a.V, esz) && vec_ok(a.q, a.V, 4);
    if (a.dtype == 1) {
        if (vec) hipLaunchKernelGGL((chain_dense_kernel<1, true>), dim3(a.B), dim3(kDrawThreads), 0, s, a);
        else hipLaunchKernelGGL((chain_dense_kernel<1, false>), dim3(a.B), dim3(kDrawThreads), 0, s, a);
    } else {
        if (vec) hipLaunchKernelGGL((chain_dense_kernel<0, true>), dim3(a.B), dim3(kDrawThreads), 0, s, a);
        else hipLaunchKernelGGL((chain_dense_kernel<0, false>), dim3(a.B), dim3(kDrawThreads), 0, s, a);
    }
    return hipGetLastError();
}

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
    if (a.dtype == 1) hipLaunchKernelGGL((alpha_dense_kernel<1, false>), dim3(R), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((alpha_dense_kernel<0, false>), dim3(R), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_chain_topk(const ChainArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(chain_topk_position_kernel, dim3(a.B * (a.K + 1)), dim3(2 * kWave), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chain_topk_combine_kernel, dim3((a.B + 3) / 4), dim3(4 * kWave), 0, s, a);
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
