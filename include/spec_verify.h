/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) library for the verification
 * step of speculative decoding.
 *
 * The method (p = target, q = draft):
 *   - "投机解码与 EAGLE", section 二 (exactness rule; temperature-0 greedy rule);
 *   - "064 · 投机解码：小模型先起草，大模型怎样并行验收而不改变分布",
 *     section 二 (acceptance a(x) = min(1, p(x)/q(x)); residual
 *     r(x) = max(0, p(x) - q(x)) / sum max(0, p - q); p and q must carry the
 *     temperature / top-k transforms; acceptance rate alpha = sum min(p, q)),
 *     section 三 (the per-position loop: test, stop at the first rejection
 *     and draw from the residual, or draw a bonus token from p_{K+1});
 *   - "EAGLE-2: Faster Inference of Language Models with Dynamic Draft
 *     Trees", section 2.1 (same rule), section 2.2 (tree drafts verified in one
 *     pass; the longest accepted branch wins).
 *
 * Conventions shared by every entry point
 *   - All array arguments except `parents_host` are DEVICE pointers, row-major
 *     and contiguous.  Every buffer is owned by the caller; the library
 *     allocates nothing and keeps no pointer after returning.  Calls on
 *     different streams may run concurrently as long as they use different
 *     workspaces.  The library's own state is: a process-wide atomic counter
 *     that gives every top-k chain call its tag (see the hand-over below),
 *     the per-thread request of spec_profile_events, and the device scratch
 *     of spec_verify_chain_noalloc (one array per GPU, looked up on first use).
 *   - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without synchronising.  Inputs must stay valid and
 *     outputs must not be read until the stream has reached the call.
 *   - `workspace` is device scratch of at least the size reported by the
 *     matching *_workspace_bytes function (or spec_workspace_bytes, which
 *     covers every call of a shape), 256-byte aligned.  It must be
 *     zero-filled before its first use (spec_workspace_init, or any zeroing
 *     allocation).  A top-k chain call (temperature > 0, 0 < top_k < V)
 *     needs the part it uses to be zero and leaves it zero (the hand-over
 *     words one call writes are cleared by the same call), so a series of
 *     such calls needs zeroing once.  Every other call leaves scratch data
 *     behind: before a top-k chain call that follows a call of another kind
 *     on the same workspace, zero it again.  A workspace serves one call at a
 *     time: calls that may overlap need separate workspaces.
 *   - Hand-over inside a top-k chain launch: the finisher workgroups of a
 *     batch row wait, with a bounded poll, for the words the selection
 *     workgroups of the same launch store.  Finishers come after every
 *     selection workgroup in the grid, and the GPU dispatches a launch's
 *     workgroups in grid order within each XCD, so a finisher only waits for
 *     workgroups that are running or done; progress relies on that order.
 *     If words still have not arrived after about 0.1 s (another process
 *     holding the GPU's compute units), the row gets accept_len =
 *     SPEC_ROW_TIMED_OUT and -1 tokens, and the launch still ends.  Words
 *     carry the call's tag, so a word a late workgroup stores after its
 *     call gave up is ignored by later calls.  A graph replay reuses the tag
 *     of the captured call: after a replay that reports a timed-out row, zero
 *     the workspace before the next replay.
 *   - Logit rows are bfloat16 (SPEC_BF16, raw bits) or float32 (SPEC_F32).
 *     Draft probabilities are float32.  Uniforms are float32 in [0, 1).
 *   - Host-detectable argument errors return a negative code and launch
 *     nothing.  Bad DATA never aborts a call: the affected batch row gets
 *     accept_len = -1 and all its output tokens (and path entries) = -1,
 *     under these rules:
 *       E1 a target row that is consulted contains NaN, or (sampling mode)
 *          +inf, or only -inf values;
 *       E2 a draft / node token outside [0, V) (every token is checked);
 *       E3 a draft probability that is consulted is NaN, negative or +inf;
 *       E4 a transformed draft row that is consulted keeps zero mass;
 *       E5 a uniform outside [0, 1) (sampling mode; every uniform is checked).
 *     A chain consults position k only when x_0..x_{k-1} were all accepted
 *     (the left-to-right walk of the method): target rows 0..j, and for the
 *     draft, q[x_k] for k <= j (T == 1, no top-k) or whole rows 0..j (any
 *     other transform), plus row j itself for a residual draw; j = first
 *     rejection (K if none).  A greedy tree consults every node row; a
 *     sampled tree the rows of the nodes its walk visits.
 *   - Environment: SPEC_VERIFY_DENSE_BRACKET (a number in [0, 0.5)) sets the
 *     relative width of the bracket the dense final draw (temperature > 0,
 *     top-k off) puts around the normalisers taken from its row statistics.
 *     Results do not depend on it; a normaliser outside its bracket only makes
 *     the draw recompute that row exactly (0 forces that path, for tests).
 *     Read on every call; unset or invalid values leave the built-in width.
 *     SPEC_VERIFY_TREE_ONEPASS = 0 makes spec_verify_tree_sample compute the
 *     residual masses of the node it draws at with one pass each, instead of
 *     one pass for all of them (the same results; for tests).
 *     SPEC_VERIFY_DENSE_PATH = walk | rows picks the route of a chain with
 *     temperature 1 and top-k off: the walk (one workgroup per batch row reads
 *     target rows only up to the first rejection) or every row's statistics
 *     first; by default the walk when B*(K+1) > 1344 or V < 4096.  Results
 *     are the same either way.
 *     SPEC_VERIFY_DENSE_SPLIT sets how many workgroups share each batch row's
 *     draw on the every-row-first route (temperature > 0, top-k off): 0 keeps
 *     one per row, N >= 2 asks for N (at most 16 and the row's 4096-token
 *     chunks) at any batch size; unset, the library splits batches of up to
 *     192 rows (160 with a transformed draft).  Results are the same.
 *     SPEC_VERIFY_SPIN_LIMIT (an integer in [0, 65536]) lowers the number of
 *     polls a top-k chain finisher, or a member of a sampled tree's cluster
 *     (spec_verify_tree_sample_ws), makes before it gives up (tests of the
 *     timed-out path); read on every call.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of logit rows.  A plain integer, so that a value outside the two
 * below is an argument error the library reports (SPEC_EINVAL), not an
 * out-of-range enumeration. */
typedef int32_t spec_dtype_t;
enum { SPEC_F32 = 0, SPEC_BF16 = 1 };

enum {
    SPEC_OK = 0,
    SPEC_EINVAL = -1,        /* bad sizes, pointers, dtype, temperature, parents */
    SPEC_EWORKSPACE = -2,    /* workspace missing, misaligned or too small */
    SPEC_ELAUNCH = -3,       /* a kernel launch failed (hipGetLastError) */
    SPEC_EUNSUPPORTED = -4,  /* valid request outside this build's limits */
    SPEC_ESCRATCH = -5       /* spec_verify_chain_noalloc: more scratch needed than it holds */
};

/* accept_len of a batch row whose top-k chain hand-over timed out (see above). */
#define SPEC_ROW_TIMED_OUT (-2)

/* Limits of this build: K <= SPEC_MAX_K draft positions, N <= SPEC_MAX_NODES
 * tree nodes, top_k <= SPEC_TOPK_MAX when top-k is active, V < 2^24 and V <=
 * SPEC_MAX_V. */
#define SPEC_MAX_K 63
#define SPEC_MAX_NODES 64
#define SPEC_TOPK_MAX 64
#define SPEC_MAX_V (1 << 20)
#define SPEC_EXPAND_MAX 1024     /* children of one expansion layer, E * top_k */
#define SPEC_RERANK_MAX 1024     /* candidate nodes of one reranking */

/* Human-readable text for a return code (static storage). */
const char* spec_error_string(int code);

/* One workspace size (bytes) that serves every spec_verify_chain,
 * spec_verify_chain_topp and spec_accept_rate call with B batch rows and K =
 * K_or_N draft positions, and every spec_verify_tree_greedy(_rows) call with
 * N = K_or_N tree nodes, over V tokens with this top_k, whatever the dtype and
 * temperature; 0 if no such call is valid (B, K_or_N or V below 1, V above
 * SPEC_MAX_V).  It is the largest of the per-call sizes below. */
size_t spec_workspace_bytes(int B, int K_or_N, int V, int top_k);

/* Workspace sizes (bytes) for the calls below with the same arguments; 0 if the
 * arguments are invalid.  Sizes depend only on the arguments. */
size_t spec_chain_workspace_bytes(int B, int K, int V, spec_dtype_t dtype, float temperature, int top_k);
size_t spec_tree_workspace_bytes(int B, int N, int V, spec_dtype_t dtype);
size_t spec_accept_rate_workspace_bytes(int B, int K, int V, spec_dtype_t dtype, float temperature, int top_k);
size_t spec_tree_expand_workspace_bytes(int B, int E, int V, int top_k);

/*
 * spec_verify_chain -- batched verification of B drafted chains of K tokens.
 * "064 · 投机解码", section 二 (the test min(1, p/q), the residual
 * norm(max(0, p - q)), p and q carrying the temperature and top-k) and section
 * 三 (the left-to-right loop, the residual draw at the first rejection, the
 * bonus draw from p_{K+1}); "投机解码与 EAGLE", section 二 (greedy mode);
 * "Việc giải mã giả định và EAGLE-3", step 2 of the residual routine (zero
 * residual mass: draw from the target).
 *
 * For each batch row b (independently):
 *   p'_k = softmax(z_k / T) over the top_k largest logits of row k (all V when
 *          top-k is off), zero elsewhere; k = 0..K.
 *   q'_k = q_k as given when T == 1 and top-k is off; otherwise q_k^(1/T)
 *          renormalised over the top_k largest entries of q_k.
 *   Test k = 0, 1, ...: accept x_k iff u_k < min(1, p'_k(x_k) / q'_k(x_k))
 *   (q'_k(x_k) = 0: accept iff p'_k(x_k) > 0); stop at the first rejection j.
 *   Final draw with u_K: at j < K from r = max(0, p'_j - q'_j) (if r has zero
 *   mass, from p'_j), at j = K from p'_K; the token is the smallest index i
 *   with u_K * S < C_i (C the inclusive prefix sum of r in index order, S its
 *   total).
 *   Top-k sets are exact: k entries, larger value first, lower index on ties.
 * Greedy mode (temperature == 0): accept while x_k equals the argmax of row k
 * (lowest index on ties), then emit the argmax of the first mismatching row
 * (or of row K); draft_probs and uniforms are not read (may be NULL).
 *
 *   target_logits [B][K+1][V]  dtype                   device, read
 *   draft_probs   [B][K][V]    float32                 device, read (rows sum to ~1)
 *   draft_tokens  [B][K]       int32                   device, read
 *   uniforms      [B][K+1]     float32 in [0,1)        device, read
 *   temperature   >= 0, finite (0 = greedy); top_k <= 0 or >= V disables top-k
 *   out_tokens    [B][K+1]     int32                   device, written: x_0..x_{j-1}, y, then -1
 *   out_accept_len[B]          int32                   device, written: j in [0,K], -1 on error,
 *                                                      SPEC_ROW_TIMED_OUT (top-k mode only, see above)
 *   out_diag      [B][2K+2]    float32, may be NULL    device, written:
 *                 [k] = p'_k(x_k), [K+k] = q'_k(x_k) for the tested
 *                 positions k <= j, k < K (NaN for k > j; greedy: [k] = 1 if
 *                 x_k matched, else 0, and [K+k] = NaN),
 *                 [2K] = mass of the final-draw distribution before
 *                 normalisation (residual mass, or 1 for p'), [2K+1] = the
 *                 drawn token's probability under it.
 * Returns SPEC_OK or a negative code.
 */
int spec_verify_chain(const void* target_logits, spec_dtype_t dtype,
                      const float* draft_probs, const int32_t* draft_tokens,
                      const float* uniforms, int B, int K, int V,
                      float temperature, int top_k,
                      int32_t* out_tokens, int32_t* out_accept_len, float* out_diag,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * spec_verify_chain_topp -- spec_verify_chain with a nucleus (top-p) transform
 * on both distributions ("064 · 投机解码", section 二: the sampling transforms
 * are part of p and q).  After the temperature and top-k, each row keeps the
 * shortest prefix of its kept tokens, in value order (lower index first on
 * ties), whose probability mass reaches top_p, renormalised; a token of zero
 * probability is never kept.  0 < top_p <= 1 (1: spec_verify_chain); top_p < 1
 * needs temperature > 0 (SPEC_EUNSUPPORTED otherwise).  With top-k on, the cut
 * runs over the kept top-k entries; with top-k off, over whole rows (every
 * target and draft row's cut is found first, by a radix select on the values
 * with the masses summed exactly in fixed point, then the tests and the
 * residual draw run in fp64).  The cut is decided on fp64 probabilities.
 * Everything else, workspace included, is as for spec_verify_chain.
 */
int spec_verify_chain_topp(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                           const int32_t* draft_tokens, const float* uniforms, int B, int K, int V,
                           float temperature, int top_k, float top_p, int32_t* out_tokens,
                           int32_t* out_accept_len, float* out_diag, void* workspace, size_t workspace_bytes,
                           void* hip_stream);

/*
 * spec_verify_chain_noalloc -- spec_verify_chain for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and kernels, no
 * workspace: the call uses a device array of SPEC_NOALLOC_SCRATCH_BYTES that
 * the library holds on each GPU it runs on until the process ends, and calls
 * no hipMalloc, hipFree or other allocating routine.  A call whose workspace
 * (spec_chain_workspace_bytes) would exceed that size returns SPEC_ESCRATCH
 * and launches nothing.  The first call on a device looks the array up (with
 * that device current); the array is zero-filled by a fill kernel on the
 * call's stream before a top-k call whenever another kind of call used it
 * since; that decision is taken when a call is issued, so a graph that
 * captured a top-k call replays without it: between its replays, run no call
 * that leaves scratch behind.  Every call on a GPU shares that GPU's array: calls that may overlap
 * (different streams, or several host threads, without ordering between them)
 * race and give undefined results; order them on one stream.
 */
#define SPEC_NOALLOC_SCRATCH_BYTES (32u << 20)
int spec_verify_chain_noalloc(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                              const int32_t* draft_tokens, const float* uniforms, int B, int K, int V,
                              float temperature, int top_k, int32_t* out_tokens, int32_t* out_accept_len,
                              float* out_diag, void* hip_stream);

/*
 * spec_verify_chain_fused -- spec_verify_chain with the target's LM head in
 * front of it, so that the logits never reach memory ("064 · 投机解码", section
 * 三: one target pass yields the K+1 distributions the verification consumes;
 * "Việc giải mã giả định và EAGLE-3": decoding is bound by memory bandwidth).
 * The logits are z[b][k][v] = sum_h hidden[b][k][h] * head_weight[v][h]
 * (bfloat16 operands, fp32 accumulation on the matrix cores); the verification
 * is then exactly spec_verify_chain's on those logits, for the two modes whose
 * selection runs in the GEMM's epilogue: greedy (temperature == 0) and top-k
 * (temperature > 0, 0 < top_k < V, top_k <= SPEC_TOPK_MAX).  Without top-k the
 * residual draw needs whole logit rows: SPEC_EUNSUPPORTED.
 *
 *   hidden        [B][K+1][H]  bfloat16 (raw bits)     device, read; 16-byte aligned
 *   head_weight   [V][H]       bfloat16 (raw bits)     device, read; 16-byte aligned (no bias)
 *   H             hidden size, a multiple of 64 (V*H and B*(K+1)*H below 2^31)
 *   draft_probs, draft_tokens, uniforms, temperature, top_k, out_tokens,
 *   out_accept_len, out_diag: as for spec_verify_chain (the logit rows are the
 *   fp32 logits above; a NaN logit makes its row unusable, E1).
 *   workspace     spec_chain_fused_workspace_bytes(B, K, V, H, temperature, top_k)
 *                 bytes, 256-byte aligned, zero-filled before its first use; a
 *                 top-k call leaves its hand-over words zero, as a top-k chain does,
 *                 and a greedy call leaves scratch behind (zero the workspace before
 *                 a top-k call that follows one on it).
 * Precision: the verification is exact on the fp32 logits the matrix cores
 * produce; they differ from exact logits by the rounding of fp32 accumulation
 * over H/16 steps (a few 1e-6 at |z| ~ 20, H = 4096).
 */
size_t spec_chain_fused_workspace_bytes(int B, int K, int V, int H, float temperature, int top_k);
int spec_verify_chain_fused(const void* hidden, const void* head_weight, const float* draft_probs,
                            const int32_t* draft_tokens, const float* uniforms, int B, int K, int V, int H,
                            float temperature, int top_k, int32_t* out_tokens, int32_t* out_accept_len,
                            float* out_diag, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * spec_verify_tree_greedy -- greedy verification of a static draft tree.
 * "EAGLE-2: Faster Inference of Language Models with Dynamic Draft Trees",
 * section 2.2 (every branch of the draft tree verified in one target pass, the
 * longest accepted branch kept); "投机解码与 EAGLE", section 二 (temperature 0:
 * a draft token is accepted when it is the target's argmax) and its EAGLE part
 * (tree drafts).
 *
 * Node 0 is the root; parents_host[0] = -1 and 0 <= parents_host[n] < n
 * (nodes in topological, e.g. breadth-first, order).  Row n of the logits is
 * the target's next-token distribution after the path to node n.  Node n > 0 is
 * accepted iff its parent is accepted and node_tokens[b][n] equals the argmax
 * of the parent's row (lowest index on ties).  The result is the deepest
 * accepted node n* (lowest node index on ties), its root-to-n* path and the
 * bonus token argmax(row n*).  D = the tree's maximum depth.
 *
 *   target_logits [B][N][V]    dtype                   device, read
 *   node_tokens   [B][N]       int32                   device, read ([b][0] ignored)
 *   parents_host  [N]          int32                   HOST, read during the call only
 *   out_path      [B][D+1]     int32                   device, written: node ids root..n*, then -1
 *   out_tokens    [B][D+1]     int32                   device, written: accepted tokens, bonus, then -1
 *   out_accept_len[B]          int32                   device, written: depth of n*, -1 on error
 */
int spec_verify_tree_greedy(const void* target_logits, spec_dtype_t dtype,
                            const int32_t* node_tokens, const int32_t* parents_host,
                            int B, int N, int V,
                            int32_t* out_path, int32_t* out_tokens, int32_t* out_accept_len,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * spec_verify_tree_sample -- sampling verification of a static draft tree
 * ("投机解码与 EAGLE", the EAGLE part: a rejected branch makes the verifier try
 * the others; "064 · 投机解码", section 三, and "EAGLE-2: Faster Inference of
 * Language Models with Dynamic Draft Trees", section 2.1, for the single test
 * and the residual).
 *
 * Tree layout as in spec_verify_tree_greedy.  Row n of the logits is the
 * target's distribution after the path to node n; row n of draft_probs is the
 * draft model's distribution at node n, from which node n's children were
 * drawn (independently of one another; rows of leaves are not read).
 * p'_n and q'_n carry the temperature as in spec_verify_chain (T == 1: q as
 * given).  For each batch row, from the root c = 0 with P = p'_c and Q = q'_c:
 * the children of c are tried in increasing node order; child n is accepted
 * iff u[n] < min(1, P(x_n)/Q(x_n)) (Q = 0 accepts iff P > 0), which emits x_n
 * and moves to n; a rejection replaces P by max(0, P - Q)/S, S its mass (P is
 * kept when S = 0), and the next child is tried.  When no child is accepted,
 * or c is a leaf, a token is drawn from P with u[0] (index-ascending inverse
 * CDF: the first y with u[0]*sum P < prefix_y, as in spec_verify_chain).
 * This reading (the pages give no rule for several branches) keeps the
 * emitted tokens distributed as the target's when children are independent
 * draws from q'.  Computed in fp64.  The walk consults the target rows of the
 * nodes it visits and, for a visited node with children, its draft row:
 * q[x_n] of the tested children (T == 1), the whole row when T != 1 or once a
 * residual is formed (E1, E3, E4); E2 and E5 cover every token and uniform.
 *
 *   target_logits [B][N][V]    dtype                   device, read
 *   draft_probs   [B][N][V]    float32                 device, read
 *   node_tokens   [B][N]       int32                   device, read ([b][0] ignored)
 *   uniforms      [B][N]       float32                 device, read (u[n]: node n's test; u[0]: the draw)
 *   parents_host  [N]          int32                   HOST, read during the call only
 *   temperature   > 0 (greedy trees: spec_verify_tree_greedy); top_k must be
 *                 off (<= 0 or >= V) in this build, else SPEC_EUNSUPPORTED
 *   out_path      [B][D+1]     int32                   device, written: node ids root..last accepted, then -1
 *   out_tokens    [B][D+1]     int32                   device, written: accepted tokens, the drawn one, then -1
 *   out_accept_len[B]          int32                   device, written: depth reached, -1 on error
 * Needs no workspace.
 */
int spec_verify_tree_sample(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                            const int32_t* node_tokens, const float* uniforms, const int32_t* parents_host,
                            int B, int N, int V, float temperature, int top_k,
                            int32_t* out_path, int32_t* out_tokens, int32_t* out_accept_len,
                            void* hip_stream);

/*
 * Per-row trees (a dynamic draft tree differs from one batch row to the next,
 * e.g. the output of spec_tree_rerank with the root at position 0):
 * spec_verify_tree_greedy_rows and spec_verify_tree_sample_rows are the two
 * calls above with `parents` a DEVICE array [B][N] (row b: parents[b][0] = -1,
 * 0 <= parents[b][n] < n; a row that breaks this is an error row, accept_len
 * -1) instead of parents_host, and out_path / out_tokens of N entries per batch
 * row ([B][N], -1 padded).  Everything else is as above; the greedy call takes
 * the workspace of spec_tree_workspace_bytes(B, N, V, dtype).
 */
int spec_verify_tree_greedy_rows(const void* target_logits, spec_dtype_t dtype, const int32_t* node_tokens,
                                 const int32_t* parents, int B, int N, int V, int32_t* out_path,
                                 int32_t* out_tokens, int32_t* out_accept_len, void* workspace,
                                 size_t workspace_bytes, void* hip_stream);
int spec_verify_tree_sample_rows(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                                 const int32_t* node_tokens, const float* uniforms, const int32_t* parents,
                                 int B, int N, int V, float temperature, int top_k, int32_t* out_path,
                                 int32_t* out_tokens, int32_t* out_accept_len, void* hip_stream);

/*
 * spec_verify_tree_sample_ws, spec_verify_tree_sample_rows_ws -- the two
 * sampled-tree calls above (same method, pages and arguments), given a
 * workspace of spec_tree_sample_workspace_bytes(B, N) bytes (256-byte
 * aligned; SPEC_EWORKSPACE if smaller).  With it, a batch of B <= 128 rows
 * shares each row's walk among min(8, 256/B) workgroups, each summing a slice
 * of the vocabulary, which exchange their sums through the workspace; this
 * needs V a multiple of 8, 16-byte aligned rows and V <= 8192 * min(8, 256/B)
 * (4096 * min(8, 256/B) when temperature != 1), else (and for B > 128, where
 * the size is 0) the call runs as without one.
 * Same results as the calls above, up to the rounding order of the sums.
 *
 * The workspace must be zero-filled before its first use; every call leaves
 * it zero, so it can be reused, including by replays of a captured graph.
 * Calls that overlap on one workspace race.  The members of a batch row wait
 * for one another's words.  A row's members are consecutive workgroups, so they
 * sit on different XCDs, and each XCD dispatches its workgroups in grid order:
 * on every XCD the rows already dispatched form a prefix, and every row below
 * the shortest prefix has all its members running and finishes, so progress
 * relies on that order, as the top-k chain's hand-over does.  A wait that
 * exceeds the spin limit (SPEC_VERIFY_SPIN_LIMIT, above) gives up: that batch
 * row's accept_len is SPEC_ROW_TIMED_OUT and its outputs -1.
 */
size_t spec_tree_sample_workspace_bytes(int B, int N);
int spec_verify_tree_sample_ws(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                               const int32_t* node_tokens, const float* uniforms, const int32_t* parents_host,
                               int B, int N, int V, float temperature, int top_k, int32_t* out_path,
                               int32_t* out_tokens, int32_t* out_accept_len, void* workspace, size_t workspace_bytes,
                               void* hip_stream);
int spec_verify_tree_sample_rows_ws(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                                    const int32_t* node_tokens, const float* uniforms, const int32_t* parents, int B,
                                    int N, int V, float temperature, int top_k, int32_t* out_path,
                                    int32_t* out_tokens, int32_t* out_accept_len, void* workspace,
                                    size_t workspace_bytes, void* hip_stream);

/*
 * EAGLE-2 draft-tree construction ("EAGLE-2: Faster Inference of Language
 * Models with Dynamic Draft Trees", section 4).  A node's value is the product
 * of the draft model's confidences along its path (section 4.1).  Values and
 * their products are float32, and every ordering is decided on those float32
 * numbers, the lower index first among equal keys.
 *
 * spec_tree_expand -- one expansion layer (section 4.1).  For each batch row,
 * each of the E nodes being expanded gets its draft row's top_k most probable
 * tokens as children (larger probability first, lower token index on ties);
 * a child's value is the node's value times the token's probability (one
 * float32 multiply); out_next lists the k_next children of highest value (flat
 * index e*top_k + i), the lower flat index first among equal values -- the
 * nodes to expand next.
 *
 *   draft_probs      [B][E][V]        float32   device, read: the draft distribution at each expanded node
 *   node_values      [B][E]           float32   device, read: the expanded nodes' values
 *   out_child_tokens [B][E][top_k]    int32     device, written
 *   out_child_values [B][E][top_k]    float32   device, written
 *   out_next         [B][k_next]      int32     device, written
 *   1 <= top_k <= min(V, SPEC_TOPK_MAX), 1 <= k_next <= E*top_k <= SPEC_EXPAND_MAX.
 *   workspace: spec_tree_expand_workspace_bytes(B, E, V, top_k) bytes (leaves
 *   scratch behind, like the other non-top-k-chain calls).
 * A batch row whose draft rows hold a NaN, negative or +inf probability, or
 * whose node value is not a finite non-negative number, gets -1 tokens and
 * next indices and NaN values.
 */
int spec_tree_expand(const float* draft_probs, const float* node_values, int B, int E, int V, int top_k,
                     int k_next, int32_t* out_child_tokens, float* out_child_values, int32_t* out_next,
                     void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * spec_tree_rerank -- reranking (section 4.2).  For each batch row, M
 * candidate nodes (the root excluded) with parent indices (-1: a child of the
 * root; otherwise below the node's own index) and values.  The m nodes first
 * in (value descending, depth ascending, index ascending) are kept -- the
 * shallower node wins among equal values, so with values that never grow
 * along a path the kept nodes form a connected tree -- and flattened in that
 * order after the root (position 0).
 *
 *   parents        [B][M]           int32     device, read
 *   values         [B][M]           float32   device, read
 *   out_nodes      [B][m]           int32     device, written: candidate index at position p + 1
 *   out_parent_pos [B][m]           int32     device, written: the parent's position (0 = root)
 *   out_mask       [B][m+1][m+1]    uint8     device, written: 1 where the column is the row's
 *                                             own position or an ancestor's (the attention mask)
 *   1 <= m <= M <= SPEC_RERANK_MAX.  Needs no workspace.
 * A batch row with a parent index out of range, a NaN value, or a kept node
 * whose parent is not kept gets -1 outputs and an all-zero mask.
 */
int spec_tree_rerank(const int32_t* parents, const float* values, int B, int M, int m, int32_t* out_nodes,
                     int32_t* out_parent_pos, uint8_t* out_mask, void* hip_stream);

/*
 * spec_kv_commit -- KV commit of an accepted tree path ("Việc giải mã giả
 * định và EAGLE-3", KV cache rollback: write the draft's entries to scratch,
 * commit on acceptance).  The verifier appended the N tree nodes' KV rows at
 * positions prefix[b] + n; the accepted path path[b][0..d] (d = accept_len[b],
 * the out_path / out_accept_len of a tree verification) moves to positions
 * prefix[b] + 0..d in every plane, in place, and out_len[b] = prefix[b] + d + 1.
 * Rows move in increasing order; as the path increases from node 0, no row is
 * overwritten before it is read.
 *
 *   kv          device, read and written: row (plane, b, s) at byte offset
 *               plane*plane_stride + b*batch_stride + s*pos_stride, row_bytes
 *               long (e.g. planes = layers x {K, V}, a row = heads x head_dim);
 *               16-byte aligned layouts move with 16-byte accesses
 *   capacity    positions s = 0 .. capacity-1 that exist in every (plane, b)
 *               row of the cache (>= 1)
 *   prefix      [B] int32 device; path [B][path_stride] int32 device;
 *   accept_len  [B] int32 device; out_len [B] int32 device, written
 *   N           tree nodes (path entries must be below N)
 * A row with accept_len < 0, a negative prefix, a path that is not node 0
 * followed by increasing node indices below N, or a path whose last (largest)
 * node lies past the cache (prefix[b] + path[b][d] >= capacity) moves nothing
 * and gets out_len -1; the check covers every row the move would touch before
 * any byte of the batch row moves.
 * Rows must not overlap: pos_stride >= row_bytes, and no two (plane, b,
 * position) rows may share bytes (a zero plane_stride with planes > 1, or a
 * zero batch_stride with B > 1, is SPEC_EINVAL; other overlaps are the
 * caller's to avoid and give undefined contents).  B <= 65535 and
 * path_stride <= SPEC_MAX_NODES (a path is at most one tree's nodes), else
 * SPEC_EUNSUPPORTED.
 */
int spec_kv_commit(void* kv, int planes, long long plane_stride, int B, long long batch_stride,
                   long long pos_stride, int row_bytes, int capacity, const int32_t* prefix, const int32_t* path,
                   int path_stride, int N, const int32_t* accept_len, int32_t* out_len, void* hip_stream);

/*
 * spec_accept_rate -- "064 · 投机解码", section 二: the chance that one drafted
 * token is accepted is the overlap of the two distributions,
 * alpha[b][k] = sum_i min(p'_k(i), q'_k(i)) for k < K, with
 * p' and q' transformed as in spec_verify_chain (rows 0..K-1 of the logits are
 * read; row K is not).  Greedy (temperature == 0): 1 if the argmax of target
 * row k equals the argmax of draft row k, else 0.  An invalid row gives NaN.
 *
 *   target_logits [B][K+1][V], draft_probs [B][K][V] (device, read)
 *   out_alpha     [B][K]       float32                 device, written
 */
int spec_accept_rate(const void* target_logits, spec_dtype_t dtype, const float* draft_probs,
                     int B, int K, int V, float temperature, int top_k,
                     float* out_alpha, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Zero-fills `workspace_bytes` (a multiple of 4) of a 256-byte aligned workspace
 * with a fill kernel on hip_stream (no memset node, so it may be captured). */
int spec_workspace_init(void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Instrumentation.
 *
 * spec_profile_events (the library's one per-thread state): the next
 * verification call made BY THIS HOST THREAD
 * launches its dominant (vocabulary-streaming) kernel with `start_event` and
 * `stop_event` attached to the dispatch (hipExtLaunchKernel), so that they hold
 * that kernel's own start and end times; both are hipEvent_t created by the
 * caller.  The request is consumed by that call.
 *
 * spec_copy_probe: plain device-to-device copy of `bytes` (multiple of 16,
 * 16-byte aligned pointers) by a streaming kernel, for calibrating hardware
 * byte counters against a known traffic.
 *
 * spec_read_probe: reads `bytes` (multiple of 16, 16-byte aligned) of device
 * memory once with the same 16-byte non-temporal loads as the verification
 * kernels and writes nothing but, at most, one word to `sink` (4 bytes of device
 * memory, contents meaningless): the achievable streaming-read bandwidth.
 */
int spec_profile_events(void* start_event, void* stop_event);
int spec_copy_probe(const void* src, void* dst, size_t bytes, void* hip_stream);
int spec_read_probe(const void* src, size_t bytes, void* sink, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
