// Kernel argument blocks and launchers shared by the library's translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

// Events that timestamp one kernel launch (taken from the dispatch itself, not
// from markers queued around it), or none.
struct Timing {
    hipEvent_t start = nullptr, stop = nullptr;
};

template <typename... Params, typename... Args>
inline void launch_timed(const Timing& t, void (*kernel)(Params...), dim3 grid, dim3 block, unsigned shmem,
                         hipStream_t s, Args... args) {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, t.start, t.stop, 0u, args...);
}

// Per-row statistics of a logit row (dense path, greedy path).
struct RowStats {
    float* m;          // [R] row maximum of the raw logits
    double* Z;         // [R] sum_i exp((z_i - m)/T) (softmax mode)
    int32_t* arg;      // [R] argmax, lowest index on ties (argmax mode)
    float* zx;         // [R] raw logit at the gathered draft token (NaN if none / out of range)
    uint32_t* flags;   // [R] kFlagInvalid when the row is unusable
};

struct RowStatsArgs {
    const void* base;      // rows of V elements (dtype)
    int dtype;             // 0 f32, 1 bf16
    int V;
    int rows_per_batch;    // rows processed per batch entry
    int batch_stride;      // rows between batch entries in memory
    int R;                 // total rows processed (= B * rows_per_batch)
    int argmax_mode;       // 1: argmax + NaN detection only
    float scale;           // log2(e) / T
    double invT;           // 1 / T
    const int32_t* gather_tokens;  // [B][gather_K] or null
    int gather_K;
    RowStats out;
};

struct PowerSumArgs {       // sum_i q_i^(1/T) per draft row (transformed dense mode)
    const float* q;
    int V;
    int R;
    float invT;
    double* S;              // [R]
    uint32_t* flags;        // [R]
};

// Sorted per-chunk top-k lists (topk.hip).  Units are ordered by batch row b,
// then position k; position k owns Ct target chunks followed, when k has a
// draft row, by Cd draft chunks: unit_base(b, k) = b*Ub + k*(Ct + Cd).
struct TopkLists {
    float* vals;            // [units][kTopkMax], entries past cnt are ignored
    int32_t* idx;
    int32_t* cnt;           // [units]
    uint32_t* flags;
    unsigned long long* words;   // chain calls: [units][kTopkMax] list words, zero between calls
    int Ct, Cd;             // chunks per target / draft row
    int chunk_t, chunk_d;   // elements per target / draft chunk
    long Ub;                // units per batch row
    int top_k;
    float top_p;            // nucleus cut after top-k (chain finish; 1 = off)
    int draft_identity;     // T == 1: q^(1/T) = q exactly
    double invT;
    uint32_t tag;           // chain calls: this call's tag in the list and record words
    int spin_limit;         // chain calls: polls before a finisher gives up on missing words
    __host__ __device__ long unit_base(int b, int k) const {
        return static_cast<long>(b) * Ub + static_cast<long>(k) * (Ct + Cd);
    }
};

// One launch of the top-k selection: B batch rows of P positions (K+1 for a
// chain, K for the acceptance rate); positions k < K carry a draft row.
struct TopkChunkArgs {
    const void* target;     // logits [B][K+1][V] (dtype)
    const float* draft;     // [B][K][V]
    int dtype;
    int B, K, V, P;
    TopkLists l;
};

struct ChainArgs {
    const void* logits;
    int dtype;
    const float* q;
    const int32_t* x;
    const float* u;
    int B, K, V;
    double T, invT;
    int transformed;        // dense path: T != 1
    RowStats st;            // dense / greedy statistics for rows b*(K+1)+k
    const double* qsum;     // dense transformed: [B*K] sum q^(1/T) (fp32-accurate)
    const uint32_t* qflags;
    TopkLists tk;           // top-k path
    unsigned long long* recw;   // top-k chain: [B][K+1][kRecWords] position record words, zero between calls
    // dense all-rows route with each batch row's draw split over split_S workgroups
    // (0: one workgroup draws), their partial sums in the workspace
    double* split_pr;           // [B][chunks][slots]
    float* split_pp;            // [B][chunks][slots]
    unsigned char* split_rec;   // [B][kSplitMax] slice records
    int split_S;
    int32_t* out_tokens;
    int32_t* out_accept_len;
    float* out_diag;
};

// The nucleus (top-p) cut of a dense row (nucleus.hip): tokens whose order key
// exceeds `key`, or equals it at an index <= tie_last, are kept; their nucleus
// probability is (weight / norm) / kept.
struct NucleusRow {
    float m;            // target rows: the maximum logit
    uint32_t key;       // order key of the boundary value
    int32_t tie_last;   // last kept index among the boundary value's elements
    uint32_t flags;     // nonzero: the row is unusable (E1 target; E3, E4 draft)
    double norm;        // target: sum exp((z - m)/T); draft: sum q^(1/T)
    double kept;        // the kept probability mass
};
struct NucleusArgs {
    const void* logits;     // target rows [rows_t][V] (dtype)
    const float* q;         // draft rows [rows_d][V]
    int rows_t, rows_d;
    int dtype;
    int V;
    double invT;
    int plain;              // draft used as given (T == 1)
    float top_p;
    NucleusRow* out_t;      // [rows_t]
    NucleusRow* out_d;      // [rows_d]
};
struct NucleusChainArgs {
    ChainArgs ch;
    const NucleusRow* trow;     // [B][K+1]
    const NucleusRow* drow;     // [B][K]
    int plain;
};
hipError_t launch_nucleus_rows(const NucleusArgs& a, hipStream_t s, Timing t = {});
hipError_t launch_nucleus_chain(const NucleusChainArgs& a, hipStream_t s, Timing t = {});

// A top-k chain in one launch (topk.hip): B*Ub selection units, then the
// finisher workgroups, finish_groups(K) per batch row (chain_finish.hpp).
constexpr int kRecWords = 5;    // 64-bit words of a position record
constexpr int kTimedOut = -2;   // accept_len of a row whose hand-over words did not arrive in time
constexpr int kDefaultSpinLimit = 1 << 16;
struct TopkChainArgs {
    TopkChunkArgs sel;
    ChainArgs ch;
};


// LM head fused with the selection (lmhead.hip): logits = hidden @ W^T never
// leave the GEMM's registers; per (row, unit of 128 columns) the epilogue keeps
// candidates, and a merge writes each row's exact top-k as one list into the
// hand-over words of a top-k chain launch (targets pre-listed: Ct = 1), or its
// argmax for the greedy chain.
struct LMHeadArgs {
    const uint16_t* hidden;     // [R][H] bf16 bits, R = B*(K+1)
    const uint16_t* weight;     // [V][H] bf16 bits
    int R, V, H, K;
    int units;                  // ceil(V / 128)
    int top_k;
    unsigned long long* cand;   // [R][units][4] keys (top-k) or [R][units] (greedy)
    uint32_t* cflag;            // [R][units]: a NaN logit in the unit
    int32_t* greedy_arg;        // greedy: [R] argmax, else null
    uint32_t* greedy_flags;     // greedy: [R]
    unsigned long long* words;  // top-k: the chain's list words
    TopkLists tk;               // top-k: the chain's unit layout and tag
};

struct TreeArgs {
    const int32_t* node_tokens;
    int B, N, V, D;             // per-row trees: D = N - 1 (the output stride is N)
    int16_t parents[64];
    const int32_t* parents_rows;    // [B][N] device: a tree per batch row (parents unused), or null
    RowStats st;
    int32_t* out_path;
    int32_t* out_tokens;
    int32_t* out_accept_len;
};

// Sampling verification of a static tree (tree_sample.hip): one workgroup per
// batch row.  Children of a node, in increasing node order, are linked by
// first_child / next_sibling (-1 ends a list).
struct TreeSampleArgs {
    const void* logits;     // [B][N][V] (dtype)
    int dtype;
    const float* q;         // [B][N][V]: row n = the draft distribution at node n
    const int32_t* node_tokens;   // [B][N]
    const float* u;         // [B][N]: u[n] tests node n, u[0] drives the final draw
    int B, N, V, D;
    double invT;
    int transformed;        // T != 1: q'(v) = q_v^(1/T) / sum
    int onepass;            // 0: the drawing node's residual masses always take one pass each
    int8_t parent[64];      // parent[0] = -1
    int8_t first_child[64];
    int8_t next_sibling[64];
    const int32_t* parents_rows;    // [B][N] device: a tree per batch row (the arrays above unused;
                                    // D = N - 1), or null
    int32_t* out_path;
    int32_t* out_tokens;
    int32_t* out_accept_len;
};

// The sampled tree with each batch row's walk shared by a cluster of G
// workgroups (tree_cluster.hip), exchanging per-slice sums through words.
constexpr int kTcMaxG = 8;       // members per batch row
constexpr int kTcWords = 8;      // 64-bit words per (batch row, round, member)
struct TcArgs {
    TreeSampleArgs t;
    unsigned long long* words;   // [B][R][G][kTcWords], zero before and after a call
    unsigned* done;              // [B] members finished, zero before and after a call
    int G;                       // members per batch row
    int L;                       // elements per member slice (set by the launcher)
    int R;                       // exchange rounds per batch row (2N + 2)
    int spin_limit;              // polls before a wait gives up
};
int tree_cluster_members(int B);   // G for a batch of B rows (< 2: no cluster)
bool tree_cluster_fits(int B, int N, int V, const void* logits, int dtype, const float* q, bool transformed);
hipError_t launch_tree_cluster(TcArgs a, hipStream_t s, Timing t = {});

// EAGLE-2 draft-tree construction (eagle2.hip).
constexpr int kExpandMax = 1024;    // children of one expansion layer (E * K)
constexpr int kRerankMax = 1024;    // candidate nodes of one reranking
struct TreeExpandArgs {
    const float* node_values;   // [B][E]
    int B, E, K, k_next;
    TopkLists tk;               // the draft rows' per-chunk lists (draft units only)
    int32_t* out_tokens;        // [B][E][K]
    float* out_values;          // [B][E][K]
    int32_t* out_next;          // [B][k_next]
};
struct TreeRerankArgs {
    const int32_t* parents;     // [B][M]
    const float* values;        // [B][M]
    int B, M, m;
    int32_t* out_nodes;         // [B][m]
    int32_t* out_parent_pos;    // [B][m]
    uint8_t* out_mask;          // [B][m+1][m+1]
};

// KV commit of an accepted tree path (kv_commit.hip).
struct KVCommitArgs {
    uint8_t* kv;                    // row (plane, b, s) at plane*plane_stride + b*batch_stride + s*pos_stride
    long long plane_stride, batch_stride, pos_stride;
    int planes, B, row_bytes;
    int capacity;                   // positions 0 .. capacity-1 exist in every (plane, b) row
    const int32_t* prefix;          // [B]
    const int32_t* path;            // [B][path_stride]
    int path_stride, N;
    const int32_t* accept_len;      // [B]
    int32_t* new_len;               // [B]
};

struct AlphaArgs {
    const void* logits;
    int dtype;
    const float* q;
    int B, K, V;
    float scale;            // log2(e)/T
    float invT;
    double T;
    int transformed;
    RowStats st;            // target rows (b, k<K), dense or argmax
    RowStats qst;           // greedy: argmax of draft rows
    const double* qsum;
    const uint32_t* qflags;
    TopkLists tk;
    float* out_alpha;
};

// True when every row of V elements of `esz` bytes starting at `p` can be read
// with aligned 16-byte vector loads.
inline bool vec_ok(const void* p, int V, int esz) {
    return (reinterpret_cast<uintptr_t>(p) % 16 == 0) && ((static_cast<long>(V) * esz) % 16 == 0);
}

hipError_t launch_rowstats(const RowStatsArgs& a, hipStream_t s, Timing t = {});
hipError_t launch_power_sums(const PowerSumArgs& a, hipStream_t s);
hipError_t launch_topk_chunks(const TopkChunkArgs& a, hipStream_t s, Timing t = {});
hipError_t launch_chain_topk(const TopkChainArgs& a, hipStream_t s, Timing t = {});   // selection + finish
hipError_t launch_alpha_topk(const AlphaArgs& a, hipStream_t s);
// bracket: relative half-width of the brackets put around the row statistics'
// normalisers (any value gives the same result; it sets how often the slow path runs)
hipError_t launch_chain_dense(const ChainArgs& a, double bracket, hipStream_t s, Timing t = {});   // statistics precomputed
// The dense draw split over several workgroups per batch row: at most kSplitMax slices
// of a row; the workspace bytes of the split for B batch rows of V, and the slice count
// the launch uses (1: no split; forced > 0 asks for that many, clamped to the row's
// chunks and kSplitMax).
constexpr int kSplitMax = 16;
size_t dense_split_bytes(int B, int V);
int dense_split_slices(int B, int V, bool transformed, int forced = 0);
// Points a's split fields into `base` (dense_split_bytes(B, V) bytes) for S slices.
void dense_split_plan(ChainArgs& a, unsigned char* base, int B, int V, int S);
// T == 1 without top-k: the whole chain (row statistics of the rows the walk
// reaches, tests, final draw) in one launch.
hipError_t launch_chain_walk(const ChainArgs& a, double bracket, hipStream_t s, Timing t = {});
hipError_t launch_chain_greedy(const ChainArgs& a, hipStream_t s);
hipError_t launch_tree(const TreeArgs& a, hipStream_t s);
hipError_t launch_tree_sample(const TreeSampleArgs& a, hipStream_t s, Timing t = {});
hipError_t launch_tree_expand(const TreeExpandArgs& a, hipStream_t s);
hipError_t launch_tree_rerank(const TreeRerankArgs& a, hipStream_t s);
hipError_t launch_kv_commit(const KVCommitArgs& a, hipStream_t s, Timing t = {});
hipError_t launch_alpha_dense(const AlphaArgs& a, hipStream_t s);
// Dense acceptance rate in one pass per row (alpha.hip), for rows that fit its registers.
bool alpha_rows_fit(const AlphaArgs& a);
hipError_t launch_alpha_rows(const AlphaArgs& a, hipStream_t s, Timing t = {});
hipError_t launch_alpha_greedy(const AlphaArgs& a, hipStream_t s);
hipError_t launch_lmhead(const LMHeadArgs& a, hipStream_t s, Timing t = {});   // tiles + merge
int lmhead_units(int V);
hipError_t launch_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t s);
hipError_t launch_read_probe(const void* src, size_t bytes, void* sink, hipStream_t s);
hipError_t launch_zero_fill(void* dst, size_t bytes, hipStream_t s);

// Chunking of a row for the top-k selection kernel: chunks of at most
// kChunkBytes, equal sizes rounded up to whole 16-byte vectors.
constexpr int kChunkBytes = 112 * 1024;
constexpr int kMaxV = 1 << 20;
static_assert((static_cast<long>(kMaxV) * 4 + kChunkBytes - 1) / kChunkBytes <= 64,
              "a row's chunk lists are merged one count per lane");
inline void topk_chunking(int V, int esz, int* nchunks, int* chunk_elems) {
    const int per_vec = 16 / esz;
    const long bytes = static_cast<long>(V) * esz;
    int c = static_cast<int>((bytes + kChunkBytes - 1) / kChunkBytes);
    if (c < 1) c = 1;
    int e;
    for (;; ++c) {      // equal chunks of whole vectors, each within kChunkBytes
        e = (V + c - 1) / c;
        e = (e + per_vec - 1) / per_vec * per_vec;
        if (static_cast<long>(e) * esz <= kChunkBytes) break;
    }
    *nchunks = (V + e - 1) / e;
    *chunk_elems = e;
}

}  // namespace sv
