// EAGLE-2 draft-tree construction: one expansion layer's finish and the
// reranking ("EAGLE-2: Faster Inference of Language Models with Dynamic Draft
// Trees", section 4).
//
// Expansion (section 4.1): the nodes being expanded get their draft rows' most
// probable tokens as children, and a child's value is its parent's value times
// the token's probability (the value of a node is the product of the
// confidences along its path).  The vocabulary-wide part, the top_k of every
// draft row, is the top-k selection kernel's (draft rows only, per-chunk
// sorted lists); tree_expand_kernel merges each row's chunk lists, forms the
// float32 products and keeps the k_next children of highest value.
//
// Reranking (section 4.2): the m nodes of highest value over the whole tree,
// the shallower node first among equal values (which keeps the selection a
// connected tree), flattened in that order after the root, with each token's
// ancestor mask.  tree_rerank_kernel sorts the candidates' 64-bit keys
// (value descending, depth, index) with a bitonic network in LDS.
//
// Orderings are decided on the float32 values themselves (the products are one
// float32 multiply each), the lower index first among equal keys.

#include "common.hpp"
#include "internal.hpp"
#include "lists.hpp"

namespace sv {

namespace {

constexpr int kExThreads = 1024;
constexpr int kExWaves = kExThreads / kWave;

__global__ __launch_bounds__(kExThreads) void tree_expand_kernel(TreeExpandArgs a) {
    __shared__ float cv[kExpandMax];
    __shared__ int bad_s;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = wave_id();
    const int b = blockIdx.x, E = a.E, K = a.K, EK = E * K;
    if (tid == 0) bad_s = 0;
    __syncthreads();
    // One wave per expanded node: merge its draft row's chunk lists (lane l ends
    // with the l-th most probable token), then the children's values.
    int bad = 0;
    for (int e = wid; e < E; e += kExWaves) {
        const long unit0 = a.tk.unit_base(b, e);
        float v;
        int i;
        uint32_t flags = 0;
        merge_global_lists(a.tk, unit0, a.tk.Cd, v, i, flags);
        const float nv = a.node_values[static_cast<long>(b) * E + e];
        // E3-like: NaN or negative probabilities (chunk flags), +inf (the top entry),
        // a node value that is not a finite non-negative number
        const bool row_bad = flags != 0u || !(bcast(v, 0) < INFINITY) || !q_ok(nv);
        bad |= row_bad;
        if (lane < K) {
            const float val = (nv * v) + 0.f;             // one float32 product (+0: no negative zero)
            const long o = (static_cast<long>(b) * E + e) * K + lane;
            a.out_tokens[o] = i;
            a.out_values[o] = val;
            cv[e * K + lane] = val;
        }
    }
    if (lane == 0 && bad) atomicOr(&bad_s, 1);
    __syncthreads();
    const bool err = bad_s != 0;
    // The next layer: child t's rank among the E*K children (value descending, lower
    // flat index first); ranks below k_next are written out.
    for (int t = tid; t < EK; t += kExThreads) {
        const float vt = cv[t];
        int rank = 0;
        for (int s = 0; s < EK; ++s) {
            const float vs = cv[s];
            rank += (vs > vt) || (vs == vt && s < t);
        }
        if (!err && rank < a.k_next) a.out_next[static_cast<long>(b) * a.k_next + rank] = t;
    }
    if (err) {
        for (int t = tid; t < EK; t += kExThreads) {
            a.out_tokens[static_cast<long>(b) * EK + t] = -1;
            a.out_values[static_cast<long>(b) * EK + t] = NAN;
        }
        for (int t = tid; t < a.k_next; t += kExThreads) a.out_next[static_cast<long>(b) * a.k_next + t] = -1;
    }
}

constexpr int kRrThreads = 1024;

__global__ __launch_bounds__(kRrThreads) void tree_rerank_kernel(TreeRerankArgs a) {
    __shared__ unsigned long long key[kRerankMax];
    __shared__ int nxt[2][kRerankMax];
    __shared__ int dst[2][kRerankMax];
    __shared__ int pos[kRerankMax];
    __shared__ int bad_s;
    const int tid = threadIdx.x, b = blockIdx.x, M = a.M, m = a.m;
    const int32_t* par = a.parents + static_cast<long>(b) * M;
    const float* val = a.values + static_cast<long>(b) * M;
    if (tid == 0) bad_s = 0;
    int p = -1;
    float v = 0.f;
    if (tid < M) {
        p = par[tid];
        v = val[tid] + 0.f;
        if (p < -1 || p >= tid || v != v) atomicOr(&bad_s, 1);
        if (p < -1 || p >= tid) p = -1;                 // (an error row; keeps the jumps in range)
    }
    nxt[0][tid] = p;
    dst[0][tid] = 1;
    pos[tid] = 0;
    __syncthreads();
    // Depths by pointer jumping: after round r every node knows its distance to
    // its 2^r-th ancestor (or to the root).
    int cur = 0;
    for (int r = 0; (1 << r) < M; ++r) {
        const int n = nxt[cur][tid];
        nxt[cur ^ 1][tid] = n < 0 ? -1 : nxt[cur][n];
        dst[cur ^ 1][tid] = dst[cur][tid] + (n < 0 ? 0 : dst[cur][n]);
        cur ^= 1;
        __syncthreads();
    }
    const int depth = dst[cur][tid];
    // keys: (value descending, depth, index) ascending; padding last
    key[tid] = tid < M ? (static_cast<unsigned long long>(~order_key(v)) << 32) |
                             (static_cast<unsigned long long>(depth) << 11) | static_cast<unsigned>(tid)
                       : ~0ull;
    __syncthreads();
    for (int k = 2; k <= kRrThreads; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            const int o = tid ^ j;
            if (o > tid) {
                const unsigned long long x = key[tid], y = key[o];
                const bool up = (tid & k) == 0;
                if ((x > y) == up) {
                    key[tid] = y;
                    key[o] = x;
                }
            }
            __syncthreads();
        }
    }
    // the first m keys are the kept nodes, in flattened order
    if (tid < m) pos[static_cast<int>(key[tid] & 0x7ffu)] = tid + 1;
    __syncthreads();
    int err = bad_s;
    int node = -1, ppos = -1;
    if (tid < m) {
        node = static_cast<int>(key[tid] & 0x7ffu);
        const int pn = par[node];
        ppos = pn < 0 ? 0 : pos[pn];
        if (!err && ppos == 0 && pn >= 0) atomicOr(&bad_s, 1);     // parent not kept
    }
    __syncthreads();
    err = bad_s;
    uint8_t* mk = a.out_mask + static_cast<long>(b) * (m + 1) * (m + 1);
    for (long t = tid; t < static_cast<long>(m + 1) * (m + 1); t += kRrThreads) mk[t] = 0;
    if (tid < m) {
        a.out_nodes[static_cast<long>(b) * m + tid] = err ? -1 : node;
        a.out_parent_pos[static_cast<long>(b) * m + tid] = err ? -1 : ppos;
    }
    __syncthreads();              // the mask's zeros land before its ones
    if (!err) {
        if (tid == 0) mk[0] = 1;
        if (tid < m) {
            uint8_t* row = mk + static_cast<long>(tid + 1) * (m + 1);
            row[0] = 1;
            for (int i = node; i >= 0; i = par[i]) row[pos[i]] = 1;
        }
    }
}

}  // namespace

hipError_t launch_tree_expand(const TreeExpandArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(tree_expand_kernel, dim3(a.B), dim3(kExThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_tree_rerank(const TreeRerankArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(tree_rerank_kernel, dim3(a.B), dim3(kRrThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace sv
