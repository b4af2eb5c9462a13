// C ABI entry points: argument checks, workspace carving, launch sequencing.
// Every call only enqueues kernels on the caller's stream.

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/spec_verify.h"
#include "common.hpp"
#include "internal.hpp"

using namespace sv;

// Device scratch of spec_verify_chain_noalloc (see ScratchSlot below).
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

namespace {

static_assert(SPEC_TOPK_MAX == kTopkMax, "top-k list width");
static_assert(SPEC_MAX_V == kMaxV, "vocabulary limit");

// Tags the hand-over words of each top-k chain call (9 bits of them are used),
// so that a finisher never merges a word an earlier call left in its slot.
std::atomic<uint32_t> g_chain_calls{0};

// Polls before a top-k chain finisher gives up on words that have not arrived;
// SPEC_VERIFY_SPIN_LIMIT (a non-negative integer) lowers it, for tests that
// force the give-up path.
int spin_limit() {
    const char* env = getenv("SPEC_VERIFY_SPIN_LIMIT");
    if (env && *env) {
        const long v = atol(env);
        if (v >= 0 && v <= kDefaultSpinLimit) return static_cast<int>(v);
    }
    return kDefaultSpinLimit;
}

thread_local hipEvent_t t_prof_start = nullptr;
thread_local hipEvent_t t_prof_stop = nullptr;

// The pending profiling request of this thread, consumed by the call that
// constructs it and handed to its dominant kernel's launch.
struct ProfileScope {
    Timing t;
    ProfileScope() {
        t.start = t_prof_start;
        t.stop = t_prof_stop;
        t_prof_start = t_prof_stop = nullptr;
    }
    Timing timing() const { return t; }
};

// Bump allocator over the caller's workspace (or a size counter when base is null).
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <typename T> T* take(size_t n) {
        off = (off + 255) & ~static_cast<size_t>(255);
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += n * sizeof(T);
        return p;
    }
};

bool topk_active(int top_k, int V) { return top_k > 0 && top_k < V; }
int esz_of(int dtype) { return dtype == SPEC_BF16 ? 2 : 4; }
bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

RowStats carve_rowstats(Carver& c, size_t R) {
    RowStats st;
    st.m = c.take<float>(R);
    st.Z = c.take<double>(R);
    st.arg = c.take<int32_t>(R);
    st.zx = c.take<float>(R);
    st.flags = c.take<uint32_t>(R);
    return st;
}

// Chunk lists for B batch rows of P positions, K of which carry a draft row:
// list words for a chain (handed to its finisher workgroups within the launch,
// zero between calls), value / index arrays for a separate merge kernel.
TopkLists carve_topk(Carver& c, int dtype, int V, int B, int P, int K, int top_k, float T, bool words) {
    TopkLists t{};
    topk_chunking(V, esz_of(dtype), &t.Ct, &t.chunk_t);
    topk_chunking(V, 4, &t.Cd, &t.chunk_d);
    t.Ub = static_cast<long>(P) * t.Ct + static_cast<long>(K) * t.Cd;
    const size_t units = static_cast<size_t>(B) * t.Ub;
    if (words) {
        t.words = c.take<unsigned long long>(units * kTopkMax);
    } else {
        t.vals = c.take<float>(units * kTopkMax);
        t.idx = c.take<int32_t>(units * kTopkMax);
        t.cnt = c.take<int32_t>(units);
        t.flags = c.take<uint32_t>(units);
    }
    t.top_k = top_k;
    t.top_p = 1.f;
    t.draft_identity = (T == 1.f) ? 1 : 0;
    t.invT = T > 0.f ? 1.0 / static_cast<double>(T) : 0.0;
    return t;
}

// Per-chunk lists of E draft rows per batch row, no target rows (tree expansion).
TopkLists carve_draft_lists(Carver& c, int V, int B, int E, int top_k) {
    TopkLists t{};
    t.Ct = 0;
    t.chunk_t = 0;
    topk_chunking(V, 4, &t.Cd, &t.chunk_d);
    t.Ub = static_cast<long>(E) * t.Cd;
    const size_t units = static_cast<size_t>(B) * t.Ub;
    t.vals = c.take<float>(units * kTopkMax);
    t.idx = c.take<int32_t>(units * kTopkMax);
    t.cnt = c.take<int32_t>(units);
    t.flags = c.take<uint32_t>(units);
    t.top_k = top_k;
    t.draft_identity = 1;
    t.invT = 1.0;
    return t;
}

TopkChunkArgs topk_chunk_args(const void* target, const float* draft, int dtype, int B, int K, int V, int P,
                              const TopkLists& t) {
    TopkChunkArgs a{};
    a.target = target;
    a.draft = draft;
    a.dtype = dtype;
    a.B = B;
    a.K = K;
    a.V = V;
    a.P = P;
    a.l = t;
    return a;
}

// A row's chunk lists are merged one count per lane: at most 64 chunks.
bool topk_shape_ok(int dtype, int V) {
    int c1, e1, c2, e2;
    topk_chunking(V, esz_of(dtype), &c1, &e1);
    topk_chunking(V, 4, &c2, &e2);
    return c1 <= 64 && c2 <= 64;      // a row's chunk lists are merged one count per lane
}

int check_common(const void* logits, int dtype, int B, int K, int V, float T) {
    if (!logits) return SPEC_EINVAL;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EINVAL;
    if (B < 1 || K < 1 || V < 1) return SPEC_EINVAL;
    if (!(T >= 0.f) || isinf(T)) return SPEC_EINVAL;
    if (!aligned(logits, esz_of(dtype))) return SPEC_EINVAL;
    if (K > SPEC_MAX_K || V > SPEC_MAX_V) return SPEC_EUNSUPPORTED;
    if (static_cast<long>(B) * (K + 1) > (1L << 30)) return SPEC_EUNSUPPORTED;
    return SPEC_OK;
}

int check_workspace(void* ws, size_t have, size_t need) {
    if (need == 0) return SPEC_OK;
    if (!ws || !aligned(ws, 256) || have < need) return SPEC_EWORKSPACE;
    return SPEC_OK;
}

// Plans the chain call into `c`; returns the workspace size.
struct ChainPlan {
    int mode;   // 0 dense, 1 top-k, 2 greedy
    RowStats st;
    NucleusRow* nt;             // dense with a nucleus: the target rows' cuts [B][K+1]
    NucleusRow* nd;             //                        the draft rows' cuts [B][K]
    double* qsum;
    uint32_t* qflags;
    TopkLists tk;
    unsigned long long* recw;
    unsigned char* split;       // dense: the split draw's partial sums (dense_split_bytes)
};

// Relative half-width of the brackets the dense draw puts around the row
// normalisers it takes from the row statistics (fp32 terms: within ~1e-6; the
// draft power sums of a transformed draft: within ~1e-5).  Any width gives the
// same result (a normaliser outside its bracket makes the draw recompute the
// row exactly); it only sets how often that slow path runs.  The environment
// variable SPEC_VERIFY_DENSE_BRACKET overrides it (0 forces the slow path).
double dense_bracket(bool transformed) {
    const char* env = getenv("SPEC_VERIFY_DENSE_BRACKET");
    if (env && *env) {
        const double v = atof(env);
        if (v >= 0.0 && v < 0.5) return v;
    }
    return transformed ? 3e-5 : 4e-6;
}

// Dense chains with the draft used as given (T == 1): the walk (one workgroup per
// batch row reads target rows only up to the first rejection) or every row's
// statistics at once followed by the tests and the draw.  The walk reads fewer
// bytes but its rows are sequential; a small batch does not fill the GPU with
// walks.  SPEC_VERIFY_DENSE_PATH=walk|rows overrides the choice.
bool dense_walks(int B, int K, int V) {
    const char* env = getenv("SPEC_VERIFY_DENSE_PATH");
    if (env && !strcmp(env, "walk")) return true;
    if (env && !strcmp(env, "rows")) return false;
    // Measured crossover (K = 8, V = 128256, the all-rows draw split): the all-rows
    // route is faster at B = 128 (90.7 against 107.0 us), the walk from B = 160
    // (111.9 against 115.0 us; B = 256: 118.5 against 149.3).  Short rows (V = 1000)
    // favour the walk's single launch.
    return static_cast<long>(B) * (K + 1) > 1344 || V < 4096;
}

ChainPlan plan_chain(Carver& c, int B, int K, int V, int dtype, float T, int top_k) {
    ChainPlan p{};
    const size_t Rt = static_cast<size_t>(B) * (K + 1), Rd = static_cast<size_t>(B) * K;
    if (T == 0.f) {
        p.mode = 2;
        p.st = carve_rowstats(c, Rt);
    } else if (topk_active(top_k, V)) {
        p.mode = 1;
        p.tk = carve_topk(c, dtype, V, B, K + 1, K, top_k, T, true);
        p.recw = c.take<unsigned long long>(Rt * kRecWords);
    } else {
        p.mode = 0;
        p.st = carve_rowstats(c, Rt);
        if (T != 1.f) {
            p.qsum = c.take<double>(Rd);
            p.qflags = c.take<uint32_t>(Rd);
        }
        p.nt = c.take<NucleusRow>(Rt);
        p.nd = c.take<NucleusRow>(Rd);
        p.split = c.take<unsigned char>(dense_split_bytes(B, V));
    }
    return p;
}

// The all-rows route's draw split over several workgroups per batch row (rows of
// the split's partial sums carved from `split`).  The environment variable
// SPEC_VERIFY_DENSE_SPLIT overrides the slice count: 0 keeps one workgroup per batch
// row, N >= 2 asks for N slices at any batch size (clamped to the row's chunks and
// to 16).
void plan_dense_split(ChainArgs& ca, unsigned char* split, int B, int V) {
    const char* env = getenv("SPEC_VERIFY_DENSE_SPLIT");
    const int forced = env ? atoi(env) : 0;
    const int S = (env && forced == 0 && !strcmp(env, "0")) ? 1
                                                            : dense_split_slices(B, V, ca.transformed != 0, forced);
    if (S > 1) dense_split_plan(ca, split, B, V, S);
}

// The fused LM-head chain: per-unit candidates, then the top-k chain's lists
// with the target rows pre-listed (one list per row) or the greedy statistics.
struct FusedPlan {
    bool greedy;
    unsigned long long* cand;
    uint32_t* cflag;
    RowStats st;
    TopkLists tk;
    unsigned long long* recw;
};

FusedPlan plan_fused(Carver& c, int B, int K, int V, float T, int top_k) {
    FusedPlan p{};
    const size_t R = static_cast<size_t>(B) * (K + 1);
    const size_t units = static_cast<size_t>(lmhead_units(V));
    p.greedy = T == 0.f;
    p.cand = c.take<unsigned long long>(R * units * (p.greedy ? 1 : 4));
    p.cflag = c.take<uint32_t>(R * units);
    if (p.greedy) {
        p.st = carve_rowstats(c, R);
    } else {
        p.tk.Ct = 1;                   // the target row's list, written by the merge
        p.tk.chunk_t = V;
        topk_chunking(V, 4, &p.tk.Cd, &p.tk.chunk_d);
        p.tk.Ub = static_cast<long>(K + 1) * p.tk.Ct + static_cast<long>(K) * p.tk.Cd;
        p.tk.words = c.take<unsigned long long>(static_cast<size_t>(B) * p.tk.Ub * kTopkMax);
        p.tk.top_k = top_k;
        p.tk.top_p = 1.f;
        p.tk.draft_identity = (T == 1.f) ? 1 : 0;
        p.tk.invT = 1.0 / static_cast<double>(T);
        p.recw = c.take<unsigned long long>(R * kRecWords);
    }
    return p;
}

struct AlphaPlan {
    int mode;   // 0 dense, 1 top-k, 2 greedy
    RowStats st, qst;
    double* qsum;
    uint32_t* qflags;
    TopkLists tk;
};

AlphaPlan plan_alpha(Carver& c, int B, int K, int V, int dtype, float T, int top_k) {
    AlphaPlan p{};
    const size_t R = static_cast<size_t>(B) * K;
    if (T == 0.f) {
        p.mode = 2;
        p.st = carve_rowstats(c, R);
        p.qst = carve_rowstats(c, R);
    } else if (topk_active(top_k, V)) {
        p.mode = 1;
        p.tk = carve_topk(c, dtype, V, B, K, K, top_k, T, false);
    } else {
        p.mode = 0;
        p.st = carve_rowstats(c, R);
        if (T != 1.f) {
            p.qsum = c.take<double>(R);
            p.qflags = c.take<uint32_t>(R);
        }
    }
    return p;
}

RowStatsArgs rowstats_args(const void* base, int dtype, int V, int rows_per_batch, int batch_stride, int B,
                           bool argmax, float T, const int32_t* gather, int gather_K, const RowStats& out) {
    RowStatsArgs a{};
    a.base = base;
    a.dtype = dtype;
    a.V = V;
    a.rows_per_batch = rows_per_batch;
    a.batch_stride = batch_stride;
    a.R = B * rows_per_batch;
    a.argmax_mode = argmax ? 1 : 0;
    a.scale = argmax ? 0.f : static_cast<float>(1.4426950408889634 / static_cast<double>(T));
    a.invT = argmax ? 0.0 : 1.0 / static_cast<double>(T);
    a.gather_tokens = gather;
    a.gather_K = gather_K;
    a.out = out;
    return a;
}

// ---- device scratch of spec_verify_chain_noalloc (for callers that cannot
// allocate).  Each GPU the library runs on holds its own copy of this array
// until the process ends.  In host code `scratch` only names the symbol: its
// device address comes from hipGetSymbolAddress, once per device, with that
// device current, and only that address is ever handed to a kernel or a fill.
constexpr size_t kScratchBytes = SPEC_NOALLOC_SCRATCH_BYTES;

constexpr int kScratchDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;           // the device address of `scratch` on this device
    hipError_t err = hipSuccess;
    std::atomic<bool> zeroed{false};   // no call other than a top-k chain has written it since it was zeroed
};
ScratchSlot g_scratch[kScratchDevices];

#define SV_TRY(expr)                                  \
    do {                                              \
        if ((expr) != hipSuccess) return SPEC_ELAUNCH; \
    } while (0)

}  // namespace

extern "C" {

const char* spec_error_string(int code) {
    switch (code) {
        case SPEC_OK: return "ok";
        case SPEC_EINVAL: return "invalid argument";
        case SPEC_EWORKSPACE: return "workspace missing, misaligned or too small";
        case SPEC_ELAUNCH: return "kernel launch failed";
        case SPEC_EUNSUPPORTED: return "outside the limits of this build";
        case SPEC_ESCRATCH: return "the call needs more device scratch than the no-allocation entry point holds";
        default: return "unknown error";
    }
}

size_t spec_chain_workspace_bytes(int B, int K, int V, spec_dtype_t dtype, float temperature, int top_k) {
    if (B < 1 || K < 1 || K > SPEC_MAX_K || V < 1 || V > SPEC_MAX_V) return 0;
    if ((dtype != SPEC_F32 && dtype != SPEC_BF16) || !(temperature >= 0.f) || isinf(temperature)) return 0;
    Carver c(nullptr);
    plan_chain(c, B, K, V, dtype, temperature, top_k);
    return (c.off + 255) & ~static_cast<size_t>(255);
}

size_t spec_tree_workspace_bytes(int B, int N, int V, spec_dtype_t dtype) {
    if (B < 1 || N < 1 || N > SPEC_MAX_NODES || V < 1 || V > SPEC_MAX_V) return 0;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return 0;
    Carver c(nullptr);
    carve_rowstats(c, static_cast<size_t>(B) * N);
    return (c.off + 255) & ~static_cast<size_t>(255);
}

size_t spec_accept_rate_workspace_bytes(int B, int K, int V, spec_dtype_t dtype, float temperature, int top_k) {
    if (B < 1 || K < 1 || K > SPEC_MAX_K || V < 1 || V > SPEC_MAX_V) return 0;
    if ((dtype != SPEC_F32 && dtype != SPEC_BF16) || !(temperature >= 0.f) || isinf(temperature)) return 0;
    Carver c(nullptr);
    plan_alpha(c, B, K, V, dtype, temperature, top_k);
    return (c.off + 255) & ~static_cast<size_t>(255);
}

size_t spec_workspace_bytes(int B, int K_or_N, int V, int top_k) {
    if (B < 1 || K_or_N < 1 || V < 1 || V > SPEC_MAX_V) return 0;
    size_t need = 0;
    const spec_dtype_t dtypes[2] = {SPEC_F32, SPEC_BF16};
    // temperature 0 (greedy), 1 (draft as given) and any other value (transformed
    // draft) select the three workspace layouts; 0.5 stands for the last
    const float temps[3] = {0.f, 1.f, 0.5f};
    for (spec_dtype_t dt : dtypes) {
        if (K_or_N <= SPEC_MAX_K) {
            for (float T : temps) {
                const size_t c = spec_chain_workspace_bytes(B, K_or_N, V, dt, T, top_k);
                const size_t a = spec_accept_rate_workspace_bytes(B, K_or_N, V, dt, T, top_k);
                need = c > need ? c : need;
                need = a > need ? a : need;
            }
        }
        const size_t t = spec_tree_workspace_bytes(B, K_or_N, V, dt);
        need = t > need ? t : need;
    }
    return need;
}

static int chain_call(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                      const int32_t* draft_tokens, const float* uniforms, int B, int K, int V,
                      float temperature, int top_k, float top_p, int32_t* out_tokens, int32_t* out_accept_len,
                      float* out_diag, void* workspace, size_t workspace_bytes, void* hip_stream);

int spec_verify_chain(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                      const int32_t* draft_tokens, const float* uniforms, int B, int K, int V,
                      float temperature, int top_k, int32_t* out_tokens, int32_t* out_accept_len,
                      float* out_diag, void* workspace, size_t workspace_bytes, void* hip_stream) {
    return chain_call(target_logits, dtype, draft_probs, draft_tokens, uniforms, B, K, V, temperature, top_k, 1.f,
                      out_tokens, out_accept_len, out_diag, workspace, workspace_bytes, hip_stream);
}

int spec_verify_chain_topp(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                           const int32_t* draft_tokens, const float* uniforms, int B, int K, int V,
                           float temperature, int top_k, float top_p, int32_t* out_tokens,
                           int32_t* out_accept_len, float* out_diag, void* workspace, size_t workspace_bytes,
                           void* hip_stream) {
    if (!(top_p > 0.f && top_p <= 1.f)) return SPEC_EINVAL;
    return chain_call(target_logits, dtype, draft_probs, draft_tokens, uniforms, B, K, V, temperature, top_k, top_p,
                      out_tokens, out_accept_len, out_diag, workspace, workspace_bytes, hip_stream);
}

static int chain_check(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                       const int32_t* draft_tokens, const float* uniforms, int B, int K, int V, float temperature,
                       int top_k, float top_p, int32_t* out_tokens, int32_t* out_accept_len, float* out_diag,
                       size_t* need);

int spec_verify_chain_noalloc(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                              const int32_t* draft_tokens, const float* uniforms, int B, int K, int V,
                              float temperature, int top_k, int32_t* out_tokens, int32_t* out_accept_len,
                              float* out_diag, void* hip_stream) {
    size_t need = 0;
    int rc = chain_check(target_logits, dtype, draft_probs, draft_tokens, uniforms, B, K, V, temperature, top_k,
                         1.f, out_tokens, out_accept_len, out_diag, &need);
    if (rc) return rc;
    if (need > kScratchBytes) return SPEC_ESCRATCH;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return SPEC_ELAUNCH;
    ScratchSlot& slot = g_scratch[dev];
    std::call_once(slot.once, [&slot] {
        slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
        if (slot.err == hipSuccess && slot.ptr == nullptr) slot.err = hipErrorInvalidSymbol;
    });
    if (slot.err != hipSuccess) return SPEC_ELAUNCH;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    // A top-k chain call needs the words it uses to be zero and leaves them zero;
    // every other call leaves scratch data behind.  The array is zero-filled (a
    // fill kernel on the caller's stream, no memset node) before its first top-k
    // chain call and again after any other call used it.
    const bool topk = temperature != 0.f && topk_active(top_k, V);
    if (topk) {
        if (!slot.zeroed.load(std::memory_order_acquire)) {
            if (launch_zero_fill(slot.ptr, kScratchBytes, s) != hipSuccess) return SPEC_ELAUNCH;
            slot.zeroed.store(true, std::memory_order_release);
        }
    } else if (need > 0) {
        slot.zeroed.store(false, std::memory_order_release);
    }
    return chain_call(target_logits, dtype, draft_probs, draft_tokens, uniforms, B, K, V, temperature, top_k, 1.f,
                      out_tokens, out_accept_len, out_diag, slot.ptr, kScratchBytes, hip_stream);
}

// Host checks of a chain call's arguments (workspace aside); the workspace size
// it needs goes to *need.
static int chain_check(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                       const int32_t* draft_tokens, const float* uniforms, int B, int K, int V, float temperature,
                       int top_k, float top_p, int32_t* out_tokens, int32_t* out_accept_len, float* out_diag,
                       size_t* need) {
    int rc = check_common(target_logits, dtype, B, K, V, temperature);
    if (rc) return rc;
    const bool greedy = temperature == 0.f;
    if (!draft_tokens || !out_tokens || !out_accept_len) return SPEC_EINVAL;
    if (!greedy && (!draft_probs || !uniforms)) return SPEC_EINVAL;
    if (!aligned(draft_tokens, 4) || !aligned(out_tokens, 4) || !aligned(out_accept_len, 4)) return SPEC_EINVAL;
    if ((draft_probs && !aligned(draft_probs, 4)) || (uniforms && !aligned(uniforms, 4)) ||
        (out_diag && !aligned(out_diag, 4)))
        return SPEC_EINVAL;
    if (!greedy && topk_active(top_k, V)) {
        if (top_k > SPEC_TOPK_MAX || !topk_shape_ok(dtype, V)) return SPEC_EUNSUPPORTED;
    }
    // the nucleus needs a temperature (greedy decoding has no distribution to cut)
    if (top_p < 1.f && greedy) return SPEC_EUNSUPPORTED;
    *need = spec_chain_workspace_bytes(B, K, V, dtype, temperature, top_k);
    return SPEC_OK;
}

static int chain_call(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                      const int32_t* draft_tokens, const float* uniforms, int B, int K, int V,
                      float temperature, int top_k, float top_p, int32_t* out_tokens, int32_t* out_accept_len,
                      float* out_diag, void* workspace, size_t workspace_bytes, void* hip_stream) {
    size_t need = 0;
    int rc = chain_check(target_logits, dtype, draft_probs, draft_tokens, uniforms, B, K, V, temperature, top_k,
                         top_p, out_tokens, out_accept_len, out_diag, &need);
    if (rc) return rc;
    rc = check_workspace(workspace, workspace_bytes, need);
    if (rc) return rc;
    const bool greedy = temperature == 0.f;

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    ProfileScope prof;
    Carver c(workspace);
    ChainPlan p = plan_chain(c, B, K, V, dtype, temperature, top_k);

    ChainArgs ca{};
    ca.logits = target_logits;
    ca.dtype = dtype;
    ca.q = draft_probs;
    ca.x = draft_tokens;
    ca.u = uniforms;
    ca.B = B;
    ca.K = K;
    ca.V = V;
    ca.T = temperature;
    ca.invT = greedy ? 0.0 : 1.0 / static_cast<double>(temperature);
    ca.transformed = (!greedy && temperature != 1.f) ? 1 : 0;
    ca.out_tokens = out_tokens;
    ca.out_accept_len = out_accept_len;
    ca.out_diag = out_diag;

    if (p.mode == 2) {
        ca.st = p.st;
        RowStatsArgs ra = rowstats_args(target_logits, dtype, V, K + 1, K + 1, B, true, 0.f, nullptr, 0, p.st);
        SV_TRY(launch_rowstats(ra, s, prof.timing()));
        SV_TRY(launch_chain_greedy(ca, s));
    } else if (p.mode == 1) {
        p.tk.top_p = top_p;
        p.tk.tag = g_chain_calls.fetch_add(1, std::memory_order_relaxed) + 1u;
        p.tk.spin_limit = spin_limit();
        ca.tk = p.tk;
        ca.recw = p.recw;
        TopkChainArgs fa{};
        fa.sel = topk_chunk_args(target_logits, draft_probs, dtype, B, K, V, K + 1, p.tk);
        fa.ch = ca;
        SV_TRY(launch_chain_topk(fa, s, prof.timing()));
    } else if (top_p < 1.f) {
        // the nucleus on whole rows: every row's cut, then the tests and the draw
        NucleusArgs na{};
        na.logits = target_logits;
        na.q = draft_probs;
        na.dtype = dtype;
        na.V = V;
        na.invT = ca.invT;
        na.plain = temperature == 1.f ? 1 : 0;
        na.top_p = top_p;
        na.rows_t = B * (K + 1);
        na.rows_d = B * K;
        na.out_t = p.nt;
        na.out_d = p.nd;
        SV_TRY(launch_nucleus_rows(na, s, prof.timing()));
        NucleusChainArgs nc{};
        nc.ch = ca;
        nc.trow = p.nt;
        nc.drow = p.nd;
        nc.plain = na.plain;
        SV_TRY(launch_nucleus_chain(nc, s));
    } else if (!ca.transformed && dense_walks(B, K, V)) {
        SV_TRY(launch_chain_walk(ca, dense_bracket(false), s, prof.timing()));
    } else if (!ca.transformed) {
        // every target row's statistics at once, then the tests and the draw per batch row
        ca.st = p.st;
        plan_dense_split(ca, p.split, B, V);
        RowStatsArgs ra =
            rowstats_args(target_logits, dtype, V, K + 1, K + 1, B, false, temperature, draft_tokens, K, p.st);
        SV_TRY(launch_rowstats(ra, s));
        SV_TRY(launch_chain_dense(ca, dense_bracket(false), s, prof.timing()));
    } else {
        ca.st = p.st;
        RowStatsArgs ra =
            rowstats_args(target_logits, dtype, V, K + 1, K + 1, B, false, temperature, draft_tokens, K, p.st);
        SV_TRY(launch_rowstats(ra, s, prof.timing()));
        PowerSumArgs pa{draft_probs, V, B * K, static_cast<float>(1.0 / temperature), p.qsum, p.qflags};
        SV_TRY(launch_power_sums(pa, s));
        ca.qsum = p.qsum;
        ca.qflags = p.qflags;
        plan_dense_split(ca, p.split, B, V);
        SV_TRY(launch_chain_dense(ca, dense_bracket(true), s));
    }
    return SPEC_OK;
}

size_t spec_chain_fused_workspace_bytes(int B, int K, int V, int H, float temperature, int top_k) {
    if (B < 1 || K < 1 || K > SPEC_MAX_K || V < 1 || V > SPEC_MAX_V || H < 64 || H % 64 != 0) return 0;
    if (!(temperature >= 0.f) || isinf(temperature)) return 0;
    if (temperature != 0.f && !(topk_active(top_k, V) && top_k <= SPEC_TOPK_MAX)) return 0;
    Carver c(nullptr);
    plan_fused(c, B, K, V, temperature, top_k);
    return (c.off + 255) & ~static_cast<size_t>(255);
}

int spec_verify_chain_fused(const void* hidden, const void* head_weight, const float* draft_probs,
                            const int32_t* draft_tokens, const float* uniforms, int B, int K, int V, int H,
                            float temperature, int top_k, int32_t* out_tokens, int32_t* out_accept_len,
                            float* out_diag, void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (!hidden || !head_weight || !draft_tokens || !out_tokens || !out_accept_len) return SPEC_EINVAL;
    if (B < 1 || K < 1 || V < 1 || H < 1 || !(temperature >= 0.f) || isinf(temperature)) return SPEC_EINVAL;
    const bool greedy = temperature == 0.f;
    if (!greedy && (!draft_probs || !uniforms)) return SPEC_EINVAL;
    if (K > SPEC_MAX_K || V > SPEC_MAX_V || H % 64 != 0) return SPEC_EUNSUPPORTED;
    // 32-bit element offsets into the head and the hidden states
    if (static_cast<long>(V) * H >= (1L << 31) || static_cast<long>(B) * (K + 1) * H >= (1L << 31))
        return SPEC_EUNSUPPORTED;
    if (static_cast<long>(B) * (K + 1) > (1L << 24)) return SPEC_EUNSUPPORTED;
    // the fused call serves the modes whose selection fits in the GEMM's epilogue:
    // greedy and top-k; the dense draw needs whole logit rows
    if (!greedy && !(topk_active(top_k, V) && top_k <= SPEC_TOPK_MAX)) return SPEC_EUNSUPPORTED;
    if (!greedy && !topk_shape_ok(SPEC_F32, V)) return SPEC_EUNSUPPORTED;
    if (!aligned(hidden, 16) || !aligned(head_weight, 16) || !aligned(draft_tokens, 4) || !aligned(out_tokens, 4) ||
        !aligned(out_accept_len, 4) || (draft_probs && !aligned(draft_probs, 4)) || (uniforms && !aligned(uniforms, 4)) ||
        (out_diag && !aligned(out_diag, 4)))
        return SPEC_EINVAL;
    const size_t need = spec_chain_fused_workspace_bytes(B, K, V, H, temperature, top_k);
    int rc = check_workspace(workspace, workspace_bytes, need);
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    ProfileScope prof;
    Carver c(workspace);
    FusedPlan p = plan_fused(c, B, K, V, temperature, top_k);

    LMHeadArgs la{};
    la.hidden = static_cast<const uint16_t*>(hidden);
    la.weight = static_cast<const uint16_t*>(head_weight);
    la.R = B * (K + 1);
    la.V = V;
    la.H = H;
    la.K = K;
    la.units = lmhead_units(V);
    la.top_k = greedy ? 1 : top_k;
    la.cand = p.cand;
    la.cflag = p.cflag;

    ChainArgs ca{};
    ca.logits = nullptr;
    ca.dtype = SPEC_F32;
    ca.q = draft_probs;
    ca.x = draft_tokens;
    ca.u = uniforms;
    ca.B = B;
    ca.K = K;
    ca.V = V;
    ca.T = temperature;
    ca.invT = greedy ? 0.0 : 1.0 / static_cast<double>(temperature);
    ca.out_tokens = out_tokens;
    ca.out_accept_len = out_accept_len;
    ca.out_diag = out_diag;
    if (greedy) {
        la.greedy_arg = p.st.arg;
        la.greedy_flags = p.st.flags;
        SV_TRY(launch_lmhead(la, s, prof.timing()));
        ca.st = p.st;
        SV_TRY(launch_chain_greedy(ca, s));
    } else {
        p.tk.tag = g_chain_calls.fetch_add(1, std::memory_order_relaxed) + 1u;
        p.tk.spin_limit = spin_limit();
        la.words = p.tk.words;
        la.tk = p.tk;
        SV_TRY(launch_lmhead(la, s, prof.timing()));
        ca.tk = p.tk;
        ca.recw = p.recw;
        TopkChainArgs fa{};
        fa.sel = topk_chunk_args(nullptr, draft_probs, SPEC_F32, B, K, V, K + 1, p.tk);
        fa.ch = ca;
        SV_TRY(launch_chain_topk(fa, s));
    }
    return SPEC_OK;
}

int spec_verify_tree_greedy(const void* target_logits, spec_dtype_t dtype, const int32_t* node_tokens,
                            const int32_t* parents_host, int B, int N, int V, int32_t* out_path,
                            int32_t* out_tokens, int32_t* out_accept_len, void* workspace,
                            size_t workspace_bytes, void* hip_stream) {
    if (!target_logits || !node_tokens || !parents_host || !out_path || !out_tokens || !out_accept_len)
        return SPEC_EINVAL;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EINVAL;
    if (B < 1 || N < 1 || V < 1) return SPEC_EINVAL;
    if (N > SPEC_MAX_NODES || V > SPEC_MAX_V) return SPEC_EUNSUPPORTED;
    if (!aligned(target_logits, esz_of(dtype)) || !aligned(node_tokens, 4) || !aligned(out_path, 4) ||
        !aligned(out_tokens, 4) || !aligned(out_accept_len, 4))
        return SPEC_EINVAL;
    TreeArgs ta{};
    if (parents_host[0] != -1) return SPEC_EINVAL;
    int depth[SPEC_MAX_NODES];
    depth[0] = 0;
    int D = 0;
    ta.parents[0] = -1;
    for (int n = 1; n < N; ++n) {
        const int p = parents_host[n];
        if (p < 0 || p >= n) return SPEC_EINVAL;
        depth[n] = depth[p] + 1;
        if (depth[n] > D) D = depth[n];
        ta.parents[n] = static_cast<int16_t>(p);
    }
    const size_t need = spec_tree_workspace_bytes(B, N, V, dtype);
    int rc = check_workspace(workspace, workspace_bytes, need);
    if (rc) return rc;

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    ProfileScope prof;
    Carver c(workspace);
    RowStats st = carve_rowstats(c, static_cast<size_t>(B) * N);
    RowStatsArgs ra = rowstats_args(target_logits, dtype, V, N, N, B, true, 0.f, nullptr, 0, st);
    SV_TRY(launch_rowstats(ra, s, prof.timing()));
    ta.node_tokens = node_tokens;
    ta.B = B;
    ta.N = N;
    ta.V = V;
    ta.D = D;
    ta.st = st;
    ta.out_path = out_path;
    ta.out_tokens = out_tokens;
    ta.out_accept_len = out_accept_len;
    SV_TRY(launch_tree(ta, s));
    return SPEC_OK;
}

// Both tree-sample entry points: a static tree (host parents) or one per batch row (device).
static int tree_sample_call(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                            const int32_t* node_tokens, const float* uniforms, const int32_t* parents_host,
                            const int32_t* parents_rows, int B, int N, int V, float temperature, int top_k,
                            int32_t* out_path, int32_t* out_tokens, int32_t* out_accept_len, void* workspace,
                            size_t workspace_bytes, bool with_ws, void* hip_stream);

// Exchange words of the clustered walk: [B][2N+2][G][kTcWords] words, then [B] counters.
struct TcPlan {
    unsigned long long* words;
    unsigned* done;
    int G, R;
};
static TcPlan plan_tree_cluster(Carver& c, int B, int N) {
    TcPlan p{};
    p.G = tree_cluster_members(B);
    p.R = 2 * N + 2;
    if (p.G < 2) return p;
    p.words = c.take<unsigned long long>(static_cast<size_t>(B) * p.R * p.G * kTcWords);
    p.done = c.take<unsigned>(static_cast<size_t>(B));
    return p;
}

size_t spec_tree_sample_workspace_bytes(int B, int N) {
    if (B < 1 || N < 1 || N > SPEC_MAX_NODES) return 0;
    Carver c(nullptr);
    plan_tree_cluster(c, B, N);
    return (c.off + 255) & ~static_cast<size_t>(255);
}

int spec_verify_tree_sample(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                            const int32_t* node_tokens, const float* uniforms, const int32_t* parents_host,
                            int B, int N, int V, float temperature, int top_k, int32_t* out_path,
                            int32_t* out_tokens, int32_t* out_accept_len, void* hip_stream) {
    if (!parents_host) return SPEC_EINVAL;
    return tree_sample_call(target_logits, dtype, draft_probs, node_tokens, uniforms, parents_host, nullptr, B, N,
                            V, temperature, top_k, out_path, out_tokens, out_accept_len, nullptr, 0, false, hip_stream);
}

int spec_verify_tree_sample_ws(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                               const int32_t* node_tokens, const float* uniforms, const int32_t* parents_host,
                               int B, int N, int V, float temperature, int top_k, int32_t* out_path,
                               int32_t* out_tokens, int32_t* out_accept_len, void* workspace, size_t workspace_bytes,
                               void* hip_stream) {
    if (!parents_host) return SPEC_EINVAL;
    return tree_sample_call(target_logits, dtype, draft_probs, node_tokens, uniforms, parents_host, nullptr, B, N,
                            V, temperature, top_k, out_path, out_tokens, out_accept_len, workspace, workspace_bytes,
                            true, hip_stream);
}

int spec_verify_tree_sample_rows(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                                 const int32_t* node_tokens, const float* uniforms, const int32_t* parents,
                                 int B, int N, int V, float temperature, int top_k, int32_t* out_path,
                                 int32_t* out_tokens, int32_t* out_accept_len, void* hip_stream) {
    if (!parents || !aligned(parents, 4)) return SPEC_EINVAL;
    return tree_sample_call(target_logits, dtype, draft_probs, node_tokens, uniforms, nullptr, parents, B, N, V,
                            temperature, top_k, out_path, out_tokens, out_accept_len, nullptr, 0, false, hip_stream);
}

int spec_verify_tree_sample_rows_ws(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                                    const int32_t* node_tokens, const float* uniforms, const int32_t* parents, int B,
                                    int N, int V, float temperature, int top_k, int32_t* out_path,
                                    int32_t* out_tokens, int32_t* out_accept_len, void* workspace,
                                    size_t workspace_bytes, void* hip_stream) {
    if (!parents || !aligned(parents, 4)) return SPEC_EINVAL;
    return tree_sample_call(target_logits, dtype, draft_probs, node_tokens, uniforms, nullptr, parents, B, N, V,
                            temperature, top_k, out_path, out_tokens, out_accept_len, workspace, workspace_bytes,
                            true, hip_stream);
}

static int tree_sample_call(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                            const int32_t* node_tokens, const float* uniforms, const int32_t* parents_host,
                            const int32_t* parents_rows, int B, int N, int V, float temperature, int top_k,
                            int32_t* out_path, int32_t* out_tokens, int32_t* out_accept_len, void* workspace,
                            size_t workspace_bytes, bool with_ws, void* hip_stream) {
    if (!target_logits || !draft_probs || !node_tokens || !uniforms || !out_path || !out_tokens ||
        !out_accept_len)
        return SPEC_EINVAL;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EINVAL;
    if (B < 1 || N < 1 || V < 1 || !(temperature > 0.f) || isinf(temperature)) return SPEC_EINVAL;
    if (N > SPEC_MAX_NODES || V > SPEC_MAX_V || topk_active(top_k, V)) return SPEC_EUNSUPPORTED;
    if (!aligned(target_logits, esz_of(dtype)) || !aligned(draft_probs, 4) || !aligned(node_tokens, 4) ||
        !aligned(uniforms, 4) || !aligned(out_path, 4) || !aligned(out_tokens, 4) || !aligned(out_accept_len, 4))
        return SPEC_EINVAL;
    TreeSampleArgs ta{};
    int D = N - 1;                     // per-row trees: outputs of N entries per batch row
    if (parents_host) {
        if (parents_host[0] != -1) return SPEC_EINVAL;
        int depth[SPEC_MAX_NODES];
        int last_child[SPEC_MAX_NODES];
        depth[0] = 0;
        D = 0;
        for (int n = 0; n < N; ++n) {
            ta.parent[n] = static_cast<int8_t>(parents_host[n] < 0 ? -1 : parents_host[n]);
            ta.first_child[n] = -1;
            ta.next_sibling[n] = -1;
            last_child[n] = -1;
        }
        for (int n = 1; n < N; ++n) {
            const int p = parents_host[n];
            if (p < 0 || p >= n) return SPEC_EINVAL;
            depth[n] = depth[p] + 1;
            if (depth[n] > D) D = depth[n];
            // children are appended in increasing node order
            if (last_child[p] < 0) ta.first_child[p] = static_cast<int8_t>(n);
            else ta.next_sibling[last_child[p]] = static_cast<int8_t>(n);
            last_child[p] = n;
        }
    }
    ta.parents_rows = parents_rows;
    ta.logits = target_logits;
    ta.dtype = dtype;
    ta.q = draft_probs;
    ta.node_tokens = node_tokens;
    ta.u = uniforms;
    ta.B = B;
    ta.N = N;
    ta.V = V;
    ta.D = D;
    ta.invT = 1.0 / static_cast<double>(temperature);
    ta.transformed = temperature != 1.f ? 1 : 0;
    const char* env = getenv("SPEC_VERIFY_TREE_ONEPASS");
    ta.onepass = (env && env[0] == '0') ? 0 : 1;
    ta.out_path = out_path;
    ta.out_tokens = out_tokens;
    ta.out_accept_len = out_accept_len;
    ProfileScope prof;
    if (with_ws) {
        const int rc = check_workspace(workspace, workspace_bytes, spec_tree_sample_workspace_bytes(B, N));
        if (rc) return rc;
        if (tree_cluster_fits(B, N, V, target_logits, dtype, draft_probs, ta.transformed != 0)) {
            // each batch row's walk shared by a cluster of workgroups
            Carver c(workspace);
            const TcPlan p = plan_tree_cluster(c, B, N);
            TcArgs ca{};
            ca.t = ta;
            ca.words = p.words;
            ca.done = p.done;
            ca.G = p.G;
            ca.R = p.R;
            ca.spin_limit = spin_limit();
            SV_TRY(launch_tree_cluster(ca, static_cast<hipStream_t>(hip_stream), prof.timing()));
            return SPEC_OK;
        }
    }
    SV_TRY(launch_tree_sample(ta, static_cast<hipStream_t>(hip_stream), prof.timing()));
    return SPEC_OK;
}

size_t spec_tree_expand_workspace_bytes(int B, int E, int V, int top_k) {
    if (B < 1 || E < 1 || V < 1 || V > SPEC_MAX_V || top_k < 1 || top_k > SPEC_TOPK_MAX) return 0;
    Carver c(nullptr);
    carve_draft_lists(c, V, B, E, top_k);
    return (c.off + 255) & ~static_cast<size_t>(255);
}

int spec_tree_expand(const float* draft_probs, const float* node_values, int B, int E, int V, int top_k,
                     int k_next, int32_t* out_child_tokens, float* out_child_values, int32_t* out_next,
                     void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (!draft_probs || !node_values || !out_child_tokens || !out_child_values || !out_next) return SPEC_EINVAL;
    if (B < 1 || E < 1 || V < 1 || top_k < 1 || top_k > V || k_next < 1 ||
        static_cast<long>(k_next) > static_cast<long>(E) * top_k)
        return SPEC_EINVAL;
    if (V > SPEC_MAX_V || top_k > SPEC_TOPK_MAX || static_cast<long>(E) * top_k > SPEC_EXPAND_MAX)
        return SPEC_EUNSUPPORTED;
    if (!aligned(draft_probs, 4) || !aligned(node_values, 4) || !aligned(out_child_tokens, 4) ||
        !aligned(out_child_values, 4) || !aligned(out_next, 4))
        return SPEC_EINVAL;
    const size_t need = spec_tree_expand_workspace_bytes(B, E, V, top_k);
    int rc = check_workspace(workspace, workspace_bytes, need);
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    ProfileScope prof;
    Carver c(workspace);
    TreeExpandArgs ea{};
    ea.tk = carve_draft_lists(c, V, B, E, top_k);
    // the draft rows only: E positions, each with a draft row and no target row
    SV_TRY(launch_topk_chunks(topk_chunk_args(nullptr, draft_probs, SPEC_F32, B, E, V, E, ea.tk), s, prof.timing()));
    ea.node_values = node_values;
    ea.B = B;
    ea.E = E;
    ea.K = top_k;
    ea.k_next = k_next;
    ea.out_tokens = out_child_tokens;
    ea.out_values = out_child_values;
    ea.out_next = out_next;
    SV_TRY(launch_tree_expand(ea, s));
    return SPEC_OK;
}

int spec_tree_rerank(const int32_t* parents, const float* values, int B, int M, int m, int32_t* out_nodes,
                     int32_t* out_parent_pos, uint8_t* out_mask, void* hip_stream) {
    if (!parents || !values || !out_nodes || !out_parent_pos || !out_mask) return SPEC_EINVAL;
    if (B < 1 || M < 1 || m < 1 || m > M) return SPEC_EINVAL;
    if (M > SPEC_RERANK_MAX) return SPEC_EUNSUPPORTED;
    if (!aligned(parents, 4) || !aligned(values, 4) || !aligned(out_nodes, 4) || !aligned(out_parent_pos, 4))
        return SPEC_EINVAL;
    TreeRerankArgs ra{};
    ra.parents = parents;
    ra.values = values;
    ra.B = B;
    ra.M = M;
    ra.m = m;
    ra.out_nodes = out_nodes;
    ra.out_parent_pos = out_parent_pos;
    ra.out_mask = out_mask;
    SV_TRY(launch_tree_rerank(ra, static_cast<hipStream_t>(hip_stream)));
    return SPEC_OK;
}

int spec_verify_tree_greedy_rows(const void* target_logits, spec_dtype_t dtype, const int32_t* node_tokens,
                                 const int32_t* parents, int B, int N, int V, int32_t* out_path,
                                 int32_t* out_tokens, int32_t* out_accept_len, void* workspace,
                                 size_t workspace_bytes, void* hip_stream) {
    if (!target_logits || !node_tokens || !parents || !out_path || !out_tokens || !out_accept_len)
        return SPEC_EINVAL;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EINVAL;
    if (B < 1 || N < 1 || V < 1) return SPEC_EINVAL;
    if (N > SPEC_MAX_NODES || V > SPEC_MAX_V) return SPEC_EUNSUPPORTED;
    if (!aligned(target_logits, esz_of(dtype)) || !aligned(node_tokens, 4) || !aligned(parents, 4) ||
        !aligned(out_path, 4) || !aligned(out_tokens, 4) || !aligned(out_accept_len, 4))
        return SPEC_EINVAL;
    const size_t need = spec_tree_workspace_bytes(B, N, V, dtype);
    int rc = check_workspace(workspace, workspace_bytes, need);
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    ProfileScope prof;
    Carver c(workspace);
    RowStats st = carve_rowstats(c, static_cast<size_t>(B) * N);
    RowStatsArgs ra = rowstats_args(target_logits, dtype, V, N, N, B, true, 0.f, nullptr, 0, st);
    SV_TRY(launch_rowstats(ra, s, prof.timing()));
    TreeArgs ta{};
    ta.node_tokens = node_tokens;
    ta.B = B;
    ta.N = N;
    ta.V = V;
    ta.D = N - 1;
    ta.parents_rows = parents;
    ta.st = st;
    ta.out_path = out_path;
    ta.out_tokens = out_tokens;
    ta.out_accept_len = out_accept_len;
    SV_TRY(launch_tree(ta, s));
    return SPEC_OK;
}

int spec_kv_commit(void* kv, int planes, long long plane_stride, int B, long long batch_stride,
                   long long pos_stride, int row_bytes, int capacity, const int32_t* prefix, const int32_t* path,
                   int path_stride, int N, const int32_t* accept_len, int32_t* out_len, void* hip_stream) {
    if (!kv || !prefix || !path || !accept_len || !out_len) return SPEC_EINVAL;
    if (planes < 1 || B < 1 || row_bytes < 1 || path_stride < 1 || N < 1 || plane_stride < 0 || batch_stride < 0 ||
        pos_stride < row_bytes || capacity < 1)
        return SPEC_EINVAL;
    // planes or batch rows that share memory would be moved by several workgroups at once
    if ((planes > 1 && plane_stride == 0) || (B > 1 && batch_stride == 0)) return SPEC_EINVAL;
    if (B > 65535 || path_stride > SPEC_MAX_NODES) return SPEC_EUNSUPPORTED;
    if (!aligned(prefix, 4) || !aligned(path, 4) || !aligned(accept_len, 4) || !aligned(out_len, 4))
        return SPEC_EINVAL;
    KVCommitArgs ka{};
    ka.kv = static_cast<uint8_t*>(kv);
    ka.plane_stride = plane_stride;
    ka.batch_stride = batch_stride;
    ka.pos_stride = pos_stride;
    ka.planes = planes;
    ka.B = B;
    ka.row_bytes = row_bytes;
    ka.capacity = capacity;
    ka.prefix = prefix;
    ka.path = path;
    ka.path_stride = path_stride;
    ka.N = N;
    ka.accept_len = accept_len;
    ka.new_len = out_len;
    ProfileScope prof;
    SV_TRY(launch_kv_commit(ka, static_cast<hipStream_t>(hip_stream), prof.timing()));
    return SPEC_OK;
}

int spec_accept_rate(const void* target_logits, spec_dtype_t dtype, const float* draft_probs, int B, int K,
                     int V, float temperature, int top_k, float* out_alpha, void* workspace,
                     size_t workspace_bytes, void* hip_stream) {
    int rc = check_common(target_logits, dtype, B, K, V, temperature);
    if (rc) return rc;
    if (!draft_probs || !out_alpha || !aligned(draft_probs, 4) || !aligned(out_alpha, 4)) return SPEC_EINVAL;
    const bool greedy = temperature == 0.f;
    if (!greedy && topk_active(top_k, V)) {
        if (top_k > SPEC_TOPK_MAX || !topk_shape_ok(dtype, V)) return SPEC_EUNSUPPORTED;
    }
    const size_t need = spec_accept_rate_workspace_bytes(B, K, V, dtype, temperature, top_k);
    rc = check_workspace(workspace, workspace_bytes, need);
    if (rc) return rc;

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    ProfileScope prof;
    Carver c(workspace);
    AlphaPlan p = plan_alpha(c, B, K, V, dtype, temperature, top_k);
    AlphaArgs aa{};
    aa.logits = target_logits;
    aa.dtype = dtype;
    aa.q = draft_probs;
    aa.B = B;
    aa.K = K;
    aa.V = V;
    aa.scale = greedy ? 0.f : static_cast<float>(1.4426950408889634 / static_cast<double>(temperature));
    aa.invT = greedy ? 0.f : static_cast<float>(1.0 / static_cast<double>(temperature));
    aa.T = temperature;
    aa.transformed = (!greedy && temperature != 1.f) ? 1 : 0;
    aa.out_alpha = out_alpha;
    if (p.mode == 2) {
        SV_TRY(launch_rowstats(rowstats_args(target_logits, dtype, V, K, K + 1, B, true, 0.f, nullptr, 0, p.st), s,
                               prof.timing()));
        SV_TRY(launch_rowstats(rowstats_args(draft_probs, SPEC_F32, V, K, K, B, true, 0.f, nullptr, 0, p.qst), s));
        aa.st = p.st;
        aa.qst = p.qst;
        SV_TRY(launch_alpha_greedy(aa, s));
    } else if (p.mode == 1) {
        TopkChunkArgs ta = topk_chunk_args(target_logits, draft_probs, dtype, B, K, V, K, p.tk);
        SV_TRY(launch_topk_chunks(ta, s, prof.timing()));
        aa.tk = p.tk;
        SV_TRY(launch_alpha_topk(aa, s));
    } else if (alpha_rows_fit(aa)) {
        // every target and draft row read once, in one launch
        SV_TRY(launch_alpha_rows(aa, s, prof.timing()));
    } else {
        SV_TRY(launch_rowstats(
            rowstats_args(target_logits, dtype, V, K, K + 1, B, false, temperature, nullptr, 0, p.st), s, prof.timing()));
        aa.st = p.st;
        if (aa.transformed) {
            PowerSumArgs pa{draft_probs, V, B * K, static_cast<float>(1.0 / temperature), p.qsum, p.qflags};
            SV_TRY(launch_power_sums(pa, s));
            aa.qsum = p.qsum;
            aa.qflags = p.qflags;
        }
        SV_TRY(launch_alpha_dense(aa, s));
    }
    return SPEC_OK;
}

int spec_profile_events(void* start_event, void* stop_event) {
    t_prof_start = static_cast<hipEvent_t>(start_event);
    t_prof_stop = static_cast<hipEvent_t>(stop_event);
    return SPEC_OK;
}

int spec_workspace_init(void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (!workspace || !aligned(workspace, 256) || workspace_bytes % 4 != 0) return SPEC_EINVAL;
    if (launch_zero_fill(workspace, workspace_bytes, static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return SPEC_ELAUNCH;
    return SPEC_OK;
}

int spec_copy_probe(const void* src, void* dst, size_t bytes, void* hip_stream) {
    if (!src || !dst || bytes % 16 != 0 || !aligned(src, 16) || !aligned(dst, 16)) return SPEC_EINVAL;
    if (launch_copy_probe(src, dst, bytes, static_cast<hipStream_t>(hip_stream)) != hipSuccess) return SPEC_ELAUNCH;
    return SPEC_OK;
}

int spec_read_probe(const void* src, size_t bytes, void* sink, void* hip_stream) {
    if (!src || !sink || bytes % 16 != 0 || !aligned(src, 16) || !aligned(sink, 4)) return SPEC_EINVAL;
    if (launch_read_probe(src, bytes, sink, static_cast<hipStream_t>(hip_stream)) != hipSuccess) return SPEC_ELAUNCH;
    return SPEC_OK;
}

}  // extern "C"
