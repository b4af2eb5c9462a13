// Kernel argument blocks and launchers shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

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

struct TopkChunkArgs {
    const void* target;     // [Rt][V] dtype
    const float* draft;     // [Rd][V] f32 (may be null when Rd == 0)
    int dtype;
    int V;
    int top_k;
    int Rt, Ct, chunk_t;    // target rows, chunks per target row, elements per target chunk
    int Rd, Cd, chunk_d;
    int target_rows_per_batch, target_batch_stride;   // maps row index -> memory row
    float* vals;            // [units][kTopkMax]
    int32_t* idx;           // [units][kTopkMax]
    int32_t* cnt;           // [units]
    uint32_t* flags;        // [units]
};

struct TopkRowsArgs {
    const float* chunk_vals;
    const int32_t* chunk_idx;
    const int32_t* chunk_cnt;
    const uint32_t* chunk_flags;
    int Rt, Ct, Rd, Cd;
    int top_k;
    double invT;
    int draft_identity;     // T == 1: q^(1/T) = q exactly
    int32_t* row_idx;       // [rows][kTopkMax], index-ascending
    double* row_p;          // [rows][kTopkMax]
    int32_t* row_cnt;       // [rows]
    uint32_t* row_flags;    // [rows]
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
    // top-k path
    const int32_t* row_idx;
    const double* row_p;
    const int32_t* row_cnt;
    const uint32_t* row_flags;
    int32_t* out_tokens;
    int32_t* out_accept_len;
    float* out_diag;
};

struct TreeArgs {
    const int32_t* node_tokens;
    int B, N, V, D;
    int16_t parents[64];
    RowStats st;
    int32_t* out_path;
    int32_t* out_tokens;
    int32_t* out_accept_len;
};

struct AlphaArgs {
    const void* logits;
    int dtype;
    const float* q;
    int B, K, V;
    float scale;            // log2(e)/T
    float invT;
    int transformed;
    RowStats st;            // target rows (b, k<K), dense or argmax
    RowStats qst;           // greedy: argmax of draft rows
    const double* qsum;
    const uint32_t* qflags;
    const int32_t* row_idx;
    const double* row_p;
    const int32_t* row_cnt;
    const uint32_t* row_flags;
    float* out_alpha;
};

// True when every row of V elements of `esz` bytes starting at `p` can be read
// with aligned 16-byte vector loads.
inline bool vec_ok(const void* p, int V, int esz) {
    return (reinterpret_cast<uintptr_t>(p) % 16 == 0) && ((static_cast<long>(V) * esz) % 16 == 0);
}

hipError_t launch_rowstats(const RowStatsArgs& a, hipStream_t s);
hipError_t launch_power_sums(const PowerSumArgs& a, hipStream_t s);
hipError_t launch_topk_chunks(const TopkChunkArgs& a, hipStream_t s);
hipError_t launch_topk_rows(const TopkRowsArgs& a, hipStream_t s);
hipError_t launch_chain_dense(const ChainArgs& a, hipStream_t s);
hipError_t launch_chain_topk(const ChainArgs& a, hipStream_t s);
hipError_t launch_chain_greedy(const ChainArgs& a, hipStream_t s);
hipError_t launch_tree(const TreeArgs& a, hipStream_t s);
hipError_t launch_alpha_dense(const AlphaArgs& a, hipStream_t s);
hipError_t launch_alpha_topk(const AlphaArgs& a, hipStream_t s);
hipError_t launch_alpha_greedy(const AlphaArgs& a, hipStream_t s);
hipError_t launch_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t s);

// Chunking of a row for the top-k selection kernel: chunks of at most
// kChunkBytes, equal sizes rounded up to whole 16-byte vectors.
constexpr int kChunkBytes = 64 * 1024;
constexpr int kMaxV = 1 << 20;
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
