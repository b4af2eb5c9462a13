/*
 * spec_oracle.c -- CPU oracle for the verification step of speculative decoding.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The product path (the HIP
 * library and its Python binding) never calls it, and it shares no code,
 * header, table or helper with that path.
 *
 * Everything is plain and slow on purpose: full-vocabulary fp64 arrays, a
 * full sort for top-k, sequential index-ascending sums.  Each function states
 * the passage it follows.  Sources (cited by page title and section):
 *   [LEV]  "064 · 投机解码：小模型先起草，大模型怎样并行验收而不改变分布" (notes on
 *          Leviathan, Kalman, Matias, ICML 2023): section 二 (a(x), r(x),
 *          alpha = sum min(p,q) = 1 - TV, the two-token example, the note that
 *          p and q carry the sampling transforms), section 三 (the per-position
 *          loop: test, residual draw, bonus draw).
 *   [EAG]  "投机解码与 EAGLE": section 二 (the exactness rule, the greedy
 *          rule for temperature 0, E[tokens]); the EAGLE part (tree drafts,
 *          longest accepted branch).
 *   [E2]   "EAGLE-2: Faster Inference of Language Models with Dynamic Draft
 *          Trees": section 2.1 (acceptance min(1, p/p_hat), residual
 *          norm(max(0, p - p_hat)), discard the rest).
 *   [P10]  "Việc giải mã giả định và EAGLE-3": step 2 (residual with the
 *          zero-sum fallback to the target distribution).
 *
 * Notation: p = target, q = draft (as in [LEV] and [EAG]).
 *
 * Readings taken where the pages leave a step open (all listed with reasons
 * in the design notes of the repository):
 *   - strict "u < min(1, ratio)";
 *   - test k consumes u[k]; the single final draw (residual or bonus)
 *     consumes u[K];
 *   - the final draw is an inverse CDF over token indices in ascending order:
 *     y = min{ i : u*S < C_i }, C_i the inclusive prefix sum of r; if no i
 *     qualifies (rounding) y is the largest i with r_i > 0;
 *   - zero residual mass: draw from the target distribution ([P10]);
 *   - q(x) = 0 for the drafted token: accept iff p(x) > 0;
 *   - top-k keeps exactly k entries, ordered by value descending and index
 *     ascending; temperature on a draft given as probabilities is
 *     q^(1/T) renormalised over its own top-k;
 *   - with T = 1 and no top-k the draft probabilities are used as given;
 *   - greedy (T = 0) ties go to the lowest index; the tree's "longest path"
 *     is the deepest accepted node, lowest node index on ties.
 *
 * Error rules (a batch row with an error gets accept_len = -1 and -1 tokens):
 *   E1 a target row the walk consults holds NaN, or (sampling mode) +inf or
 *      only -inf values;
 *   E2 a draft / node token lies outside [0, V) (all of them are checked);
 *   E3 a draft probability that is read is NaN, negative or +inf;
 *   E4 a transformed draft row the walk consults keeps zero mass;
 *   E5 a uniform outside [0, 1) (sampling mode; all of them are checked).
 * The chain walk consults position k only when every earlier draft token was
 * accepted ([LEV] section 3): target rows 0..j and the draft rows / entries of
 * positions 0..j, j the first rejection (K if none).  Greedy tree nodes are
 * verified together: every node row is consulted.  The sampled tree walks from
 * the root and consults the rows of the nodes it visits.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2      /* fp64 logit rows, e.g. the logits oracle_lm_head_logits forms */

/* Deliberate-mistake switch used only by the tests that show the pins bite:
 * 0 = the method as stated; 1 = on rejection re-sample from p instead of the
 * residual (the "naive" variant of [LEV] section 二); 2 = bonus token drawn
 * from p_{K-1} instead of p_K; 3 = ratio written q/p instead of p/q;
 * 4 = in the sampled tree, a rejected sibling leaves P as it was;
 * 5 = the draw's margin left in units of mass (not divided by S);
 * 6 = a test's margin measured against the ratio instead of min(1, ratio). */
static int g_variant = 0;
void oracle_set_variant(int v) { g_variant = v; }

/* Threads of the OpenMP loops over batch rows (the benchmark times one and all). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static size_t logit_size(int dtype) { return dtype == ORC_BF16 ? 2 : dtype == ORC_F64 ? 8 : 4; }

static double load_logit(const void* row, int dtype, int i) {
    if (dtype == ORC_F64) return ((const double*)row)[i];
    if (dtype == ORC_BF16) {
        uint32_t bits = ((uint32_t)((const uint16_t*)row)[i]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float*)row)[i];
}

/* Ordering used by top-k: larger value first, then smaller index. */
typedef struct { double v; int i; } vi_t;
static int cmp_desc_then_index(const void* a, const void* b) {
    const vi_t* x = (const vi_t*)a;
    const vi_t* y = (const vi_t*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->i > y->i) - (x->i < y->i);
}

static int topk_enabled(int top_k, int V) { return top_k > 0 && top_k < V; }

/* Marks the top_k entries of vals (value desc, index asc) in keep[]. */
static void mark_topk(const double* vals, int V, int top_k, unsigned char* keep) {
    vi_t* tmp = (vi_t*)malloc(sizeof(vi_t) * (size_t)V);
    for (int i = 0; i < V; ++i) { tmp[i].v = vals[i]; tmp[i].i = i; }
    qsort(tmp, (size_t)V, sizeof(vi_t), cmp_desc_then_index);
    memset(keep, 0, (size_t)V);
    for (int t = 0; t < top_k; ++t) keep[tmp[t].i] = 1;
    free(tmp);
}

/* Index of the largest value, lowest index among equals; -1 if a NaN is present.
 * [EAG] section 二, greedy rule. */
int oracle_argmax_row(const void* row, int dtype, int V) {
    int best = 0;
    double bv = load_logit(row, dtype, 0);
    if (isnan(bv)) return -1;
    for (int i = 1; i < V; ++i) {
        double v = load_logit(row, dtype, i);
        if (isnan(v)) return -1;
        if (v > bv) { bv = v; best = i; }
    }
    return best;
}

int oracle_argmax_f32(const float* row, int V) { return oracle_argmax_row(row, ORC_F32, V); }

/* Nucleus (top-p) cut of a distribution dist[0..V) in place: order the tokens
 * by probability (larger first, lower index on ties), keep the shortest prefix
 * whose mass reaches top_p, zero the rest and renormalise ([LEV] section 二:
 * the sampling transforms travel with p and q).  top_p >= 1 keeps everything. */
static void nucleus_cut(double* dist, int V, double top_p) {
    if (!(top_p < 1.0)) return;
    vi_t* tmp = (vi_t*)malloc(sizeof(vi_t) * (size_t)V);
    for (int i = 0; i < V; ++i) { tmp[i].v = dist[i]; tmp[i].i = i; }
    qsort(tmp, (size_t)V, sizeof(vi_t), cmp_desc_then_index);
    double cum = 0.0;
    int keep = 0;
    while (keep < V && cum < top_p && tmp[keep].v > 0.0) { cum += tmp[keep].v; ++keep; }
    for (int t = keep; t < V; ++t) dist[tmp[t].i] = 0.0;
    double s = 0.0;
    for (int i = 0; i < V; ++i) s += dist[i];
    for (int i = 0; i < V; ++i) dist[i] /= s;
    free(tmp);
}

/* Target distribution p' of one logit row under temperature T > 0 and top-k:
 * x = z/T, keep set S (all, or the top_k of x), p'_i = exp(x_i - m) / sum_S exp(x_j - m)
 * on S and 0 elsewhere ([LEV] section 二: p must already carry the temperature and
 * truncation).  Returns 0, or 1 when the row is invalid (E1). */
int oracle_target_dist_p(const void* row, int dtype, int V, double T, int top_k, double top_p, double* p);
int oracle_target_dist(const void* row, int dtype, int V, double T, int top_k, double* p) {
    return oracle_target_dist_p(row, dtype, V, T, top_k, 1.0, p);
}
/* The same, then the nucleus cut at top_p. */
int oracle_target_dist_p(const void* row, int dtype, int V, double T, int top_k, double top_p, double* p) {
    if (V <= 0 || !(T > 0.0)) return 1;
    double* x = (double*)malloc(sizeof(double) * (size_t)V);
    unsigned char* keep = (unsigned char*)malloc((size_t)V);
    int bad = 0;
    double m = -INFINITY;
    for (int i = 0; i < V; ++i) {
        double z = load_logit(row, dtype, i);
        if (isnan(z) || z == INFINITY) bad = 1;
        x[i] = z / T;
    }
    if (!bad) {
        if (topk_enabled(top_k, V)) mark_topk(x, V, top_k, keep);
        else memset(keep, 1, (size_t)V);
        for (int i = 0; i < V; ++i)
            if (keep[i] && x[i] > m) m = x[i];
        if (m == -INFINITY) bad = 1;
    }
    if (!bad) {
        double Z = 0.0;
        for (int i = 0; i < V; ++i) {
            p[i] = keep[i] ? exp(x[i] - m) : 0.0;
            Z += p[i];
        }
        for (int i = 0; i < V; ++i) p[i] /= Z;
        nucleus_cut(p, V, top_p);
    }
    free(x);
    free(keep);
    return bad;
}

/* Draft distribution q' of one row of draft probabilities.
 * T == 1 and no top-k: q as given.  Otherwise w_i = q_i^(1/T), keep the top_k of w,
 * q' = w / sum_kept w ([LEV] section 二; temperature applied to both p and q).
 * Returns 0, or 1 when invalid (E3, E4). */
int oracle_draft_dist_p(const float* q, int V, double T, int top_k, double top_p, double* out);
int oracle_draft_dist(const float* q, int V, double T, int top_k, double* out) {
    return oracle_draft_dist_p(q, V, T, top_k, 1.0, out);
}
/* The same, then the nucleus cut at top_p (a transformed draft whenever top_p < 1). */
int oracle_draft_dist_p(const float* q, int V, double T, int top_k, double top_p, double* out) {
    if (V <= 0 || !(T > 0.0)) return 1;
    for (int i = 0; i < V; ++i) {
        double v = (double)q[i];
        if (isnan(v) || v < 0.0 || v == INFINITY) return 1;
    }
    if (T == 1.0 && !topk_enabled(top_k, V) && !(top_p < 1.0)) {
        for (int i = 0; i < V; ++i) out[i] = (double)q[i];
        return 0;
    }
    double* w = (double*)malloc(sizeof(double) * (size_t)V);
    unsigned char* keep = (unsigned char*)malloc((size_t)V);
    for (int i = 0; i < V; ++i) w[i] = (q[i] > 0.0f) ? pow((double)q[i], 1.0 / T) : 0.0;
    if (topk_enabled(top_k, V)) mark_topk(w, V, top_k, keep);
    else memset(keep, 1, (size_t)V);
    double s = 0.0;
    for (int i = 0; i < V; ++i) s += keep[i] ? w[i] : 0.0;
    int bad = !(s > 0.0);
    if (!bad) {
        for (int i = 0; i < V; ++i) out[i] = keep[i] ? w[i] / s : 0.0;
        nucleus_cut(out, V, top_p);
    }
    free(w);
    free(keep);
    return bad;
}

/* Logits of an LM head with no bias: z[r][v] = sum_h hidden[r][h] * W[v][h], both
 * operands bfloat16 (raw bits), every product exact in fp64 and the sum taken in
 * fp64 in index order.  This is the target pass that yields the distributions
 * p[1..gamma+1] the verification consumes ("064 · 投机解码", section 三), done
 * here so that the verification can be checked from hidden states and head
 * weights.  hidden [R][H], W [V][H] row-major, z [R][V]. */
int oracle_lm_head_logits(const uint16_t* hidden, const uint16_t* W, int R, int V, int H, double* z) {
    if (R <= 0 || V <= 0 || H <= 0) return -1;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < R; ++r) {
        const uint16_t* hr = hidden + (size_t)r * H;
        for (int v = 0; v < V; ++v) {
            const uint16_t* wv = W + (size_t)v * H;
            double s = 0.0;
            for (int h = 0; h < H; ++h) s += load_logit(hr, ORC_BF16, h) * load_logit(wv, ORC_BF16, h);
            z[(size_t)r * V + v] = s;
        }
    }
    return 0;
}

/* Inverse-CDF draw over r[0..V) with total S (index-ascending). */
static int draw_index(const double* r, int V, double S, double u, double* margin) {
    double t = u * S, c = 0.0, prev = 0.0;
    for (int i = 0; i < V; ++i) {
        prev = c;
        c += r[i];
        if (t < c) {
            double a = t - prev, b = c - t;
            *margin = (a < b ? a : b) / (g_variant == 5 ? 1.0 : S);
            return i;
        }
    }
    for (int i = V - 1; i >= 0; --i)
        if (r[i] > 0.0) { *margin = 0.0; return i; }
    *margin = 0.0;
    return V - 1;
}

static int u_ok(float u) { return u >= 0.0f && u < 1.0f; }
static int q_ok(float v) { return !(isnan(v) || v < 0.0f || v == INFINITY); }

/*
 * Chain verification for B independent rows ([LEV] section 三; [EAG] section 二;
 * [E2] section 2.1).  Layouts (row-major):
 *   logits [B][K+1][V] (bf16 bits or f32), q [B][K][V] f32, x [B][K] i32, u [B][K+1] f32.
 * Outputs: tokens [B][K+1] (-1 padded), accept_len [B] (-1 on error),
 *   pk, qk [B][K]: p'_k(x_k), q'_k(x_k) for the positions tested, k <= j
 *   (NaN past the first rejection and on error);
 *   S [B]: mass of the final-draw distribution before normalising; py [B]: r_y/S;
 *   m_test [B][K]: |u_k - min(1, ratio_k)| for tests performed (NaN otherwise);
 *   m_draw [B]: distance of u*S to the nearest edge of the chosen cell, over S.
 * Greedy mode (T == 0): argmax comparisons; pk = 1 if x_k is the argmax else 0,
 * qk = NaN, S = py = 1, margins = +inf (the decisions are exact).
 */
int oracle_verify_chain_p(const void* logits, int dtype, const float* q, const int32_t* x,
                          const float* u, int B, int K, int V, double T, int top_k, double top_p,
                          int32_t* tokens, int32_t* accept_len, double* pk, double* qk,
                          double* S_out, double* py_out, double* m_test, double* m_draw);
int oracle_verify_chain(const void* logits, int dtype, const float* q, const int32_t* x,
                        const float* u, int B, int K, int V, double T, int top_k,
                        int32_t* tokens, int32_t* accept_len, double* pk, double* qk,
                        double* S_out, double* py_out, double* m_test, double* m_draw) {
    return oracle_verify_chain_p(logits, dtype, q, x, u, B, K, V, T, top_k, 1.0, tokens, accept_len, pk, qk,
                                 S_out, py_out, m_test, m_draw);
}
/* The same with a nucleus cut at top_p (0 < top_p <= 1) on both distributions,
 * after the temperature and top-k. */
int oracle_verify_chain_p(const void* logits, int dtype, const float* q, const int32_t* x,
                          const float* u, int B, int K, int V, double T, int top_k, double top_p,
                          int32_t* tokens, int32_t* accept_len, double* pk, double* qk,
                          double* S_out, double* py_out, double* m_test, double* m_draw) {
    if (B <= 0 || K <= 0 || V <= 0 || !(T >= 0.0) || isinf(T) || !(top_p > 0.0)) return -1;
    const size_t esz = logit_size(dtype);
    const int greedy = (T == 0.0);
    const int transformed = !(T == 1.0 && !topk_enabled(top_k, V) && !(top_p < 1.0));
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        const char* zb = (const char*)logits + (size_t)b * (K + 1) * V * esz;
        const float* qb = q + (size_t)b * K * V;
        const int32_t* xb = x + (size_t)b * K;
        const float* ub = u + (size_t)b * (K + 1);
        int32_t* tb = tokens + (size_t)b * (K + 1);
        double *pkb = pk + (size_t)b * K, *qkb = qk + (size_t)b * K, *mtb = m_test + (size_t)b * K;
        for (int k = 0; k <= K; ++k) tb[k] = -1;
        for (int k = 0; k < K; ++k) { pkb[k] = NAN; qkb[k] = NAN; mtb[k] = NAN; }
        S_out[b] = NAN; py_out[b] = NAN; m_draw[b] = NAN;
        accept_len[b] = -1;
        int err = 0;
        for (int k = 0; k < K; ++k) if (xb[k] < 0 || xb[k] >= V) err = 1;   /* E2 */
        /* The walk of [LEV] section 3: position k is examined only after every
         * earlier draft token was accepted, so the rows of positions past the
         * first rejection are never consulted (nor checked for E1 / E3 / E4). */
        if (greedy) {
            if (err) continue;
            int j = K, gj = -1;
            for (int k = 0; k <= K; ++k) {
                const int g = oracle_argmax_row(zb + (size_t)k * V * esz, dtype, V);
                if (g < 0) { err = 1; break; }                                   /* E1 */
                if (k == K) { gj = g; break; }
                pkb[k] = (xb[k] == g) ? 1.0 : 0.0;
                mtb[k] = INFINITY;
                if (xb[k] != g) { j = k; gj = g; break; }
            }
            if (err) {
                for (int k = 0; k < K; ++k) { pkb[k] = NAN; mtb[k] = NAN; }
                continue;
            }
            for (int k = 0; k < j; ++k) tb[k] = xb[k];
            tb[j] = gj;
            accept_len[b] = j;
            S_out[b] = 1.0; py_out[b] = 1.0; m_draw[b] = INFINITY;
            continue;
        }
        for (int k = 0; k <= K; ++k) if (!u_ok(ub[k])) err = 1;                  /* E5 */
        if (err) continue;
        double* p = (double*)malloc(sizeof(double) * (size_t)(K + 1) * V);
        double* qq = (double*)malloc(sizeof(double) * (size_t)V * (transformed ? K : 1));
        double* r = (double*)malloc(sizeof(double) * (size_t)V);
        /* Ratio tests left to right, stop at the first rejection. */
        int j = K;
        for (int k = 0; k <= K; ++k) {
            if (oracle_target_dist_p(zb + (size_t)k * V * esz, dtype, V, T, top_k, top_p, p + (size_t)k * V)) {
                err = 1;                                                           /* E1 */
                break;
            }
            if (k == K) break;
            if (transformed) {
                if (oracle_draft_dist_p(qb + (size_t)k * V, V, T, top_k, top_p, qq + (size_t)k * V)) {
                    err = 1;                                                       /* E3, E4 */
                    break;
                }
            } else if (!q_ok(qb[(size_t)k * V + xb[k]])) {
                err = 1;                                                           /* E3 */
                break;
            }
            pkb[k] = p[(size_t)k * V + xb[k]];
            qkb[k] = transformed ? qq[(size_t)k * V + xb[k]] : (double)qb[(size_t)k * V + xb[k]];
            double a = pkb[k], c = qkb[k], ratio;
            if (g_variant == 3) { double t = a; a = c; c = t; }
            if (c > 0.0) ratio = a / c;
            else ratio = a > 0.0 ? INFINITY : 0.0;
            double thr = ratio < 1.0 ? ratio : 1.0;
            mtb[k] = fabs((double)ub[k] - (g_variant == 6 ? ratio : thr));
            if (!((double)ub[k] < thr)) { j = k; break; }
        }
        if (!err) {
            /* Final draw with u[K]: residual at the rejected position, else bonus. */
            const double* pj = p + (size_t)j * V;
            double S = 0.0;
            if (j < K && g_variant != 1) {
                const float* qrow = qb + (size_t)j * V;
                if (!transformed)
                    for (int i = 0; i < V; ++i) if (!q_ok(qrow[i])) err = 1;      /* E3 */
                for (int i = 0; i < V && !err; ++i) {
                    double qi = transformed ? qq[(size_t)j * V + i] : (double)qrow[i];
                    double d = pj[i] - qi;
                    r[i] = d > 0.0 ? d : 0.0;
                    S += r[i];
                }
                if (!err && !(S > 0.0)) {                                         /* [P10] */
                    S = 0.0;
                    for (int i = 0; i < V; ++i) { r[i] = pj[i]; S += r[i]; }
                }
            } else {
                const double* src = (j == K && g_variant == 2) ? p + (size_t)(K - 1) * V : pj;
                for (int i = 0; i < V; ++i) { r[i] = src[i]; S += r[i]; }
            }
            if (!err) {
                double md;
                int y = draw_index(r, V, S, (double)ub[K], &md);
                for (int k = 0; k < j; ++k) tb[k] = xb[k];
                tb[j] = y;
                accept_len[b] = j;
                S_out[b] = S;
                py_out[b] = r[y] / S;
                m_draw[b] = md;
            }
        }
        if (err)
            for (int k = 0; k < K; ++k) { pkb[k] = NAN; qkb[k] = NAN; mtb[k] = NAN; }
        free(p);
        free(qq);
        free(r);
    }
    return 0;
}

/*
 * Greedy verification of a static draft tree ([EAG] greedy rule and tree drafts;
 * [E2] section 2.2 verification stage).  logits [B][N][V]: row n is the target's
 * distribution after the path to node n; node_tokens [B][N] (entry 0 ignored);
 * parents [N] with parents[0] = -1 and 0 <= parents[i] < i.  Node n (n > 0) is
 * accepted iff its parent is accepted and its token equals the argmax of the
 * parent's row.  The chosen node is the deepest accepted node (lowest index on
 * ties); the output is its path and the bonus argmax of its own row.
 * out_path, out_tokens [B][D+1] (-1 padded), accept_len [B] = depth (-1 on error).
 */
int oracle_verify_tree_greedy(const void* logits, int dtype, const int32_t* node_tokens,
                              const int32_t* parents, int B, int N, int V,
                              int32_t* out_path, int32_t* out_tokens, int32_t* accept_len) {
    if (B <= 0 || N <= 0 || V <= 0 || parents[0] != -1) return -1;
    int D = 0;
    int* depth = (int*)malloc(sizeof(int) * (size_t)N);
    depth[0] = 0;
    for (int n = 1; n < N; ++n) {
        if (parents[n] < 0 || parents[n] >= n) { free(depth); return -1; }
        depth[n] = depth[parents[n]] + 1;
        if (depth[n] > D) D = depth[n];
    }
    const size_t esz = logit_size(dtype);
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        const char* zb = (const char*)logits + (size_t)b * N * V * esz;
        const int32_t* tk = node_tokens + (size_t)b * N;
        int32_t* op = out_path + (size_t)b * (D + 1);
        int32_t* ot = out_tokens + (size_t)b * (D + 1);
        for (int d = 0; d <= D; ++d) { op[d] = -1; ot[d] = -1; }
        accept_len[b] = -1;
        int* g = (int*)malloc(sizeof(int) * (size_t)N);
        unsigned char* acc = (unsigned char*)malloc((size_t)N);
        int err = 0;
        for (int n = 1; n < N; ++n) if (tk[n] < 0 || tk[n] >= V) err = 1;        /* E2 */
        for (int n = 0; n < N && !err; ++n) {
            g[n] = oracle_argmax_row(zb + (size_t)n * V * esz, dtype, V);
            if (g[n] < 0) err = 1;                                                 /* E1 */
        }
        if (!err) {
            int best = 0;
            acc[0] = 1;
            for (int n = 1; n < N; ++n) {
                acc[n] = acc[parents[n]] && tk[n] == g[parents[n]];
                if (acc[n] && depth[n] > depth[best]) best = n;
            }
            int d = depth[best];
            for (int n = best, t = d; t >= 0; n = parents[n], --t) op[t] = n;
            for (int t = 1; t <= d; ++t) ot[t - 1] = tk[op[t]];
            ot[d] = g[best];
            accept_len[b] = d;
        }
        free(g);
        free(acc);
    }
    free(depth);
    return 0;
}

/*
 * Acceptance rate alpha[b][k] = sum_i min(p'_k(i), q'_k(i)) for k < K ([LEV]
 * section 二: the overlap mass of the two transformed distributions).
 * Greedy (T == 0): 1 if the argmax of the target row equals the argmax of the
 * draft row, else 0.  NaN for an invalid row.
 */
int oracle_accept_rate(const void* logits, int dtype, const float* q, int B, int K, int V,
                       double T, int top_k, double* alpha) {
    if (B <= 0 || K <= 0 || V <= 0 || !(T >= 0.0) || isinf(T)) return -1;
    const size_t esz = logit_size(dtype);
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int b = 0; b < B; ++b) {
        for (int k = 0; k < K; ++k) {
            const char* zrow = (const char*)logits + ((size_t)b * (K + 1) + k) * V * esz;
            const float* qrow = q + ((size_t)b * K + k) * V;
            double* out = alpha + (size_t)b * K + k;
            if (T == 0.0) {
                int gp = oracle_argmax_row(zrow, dtype, V);
                int gq = oracle_argmax_f32(qrow, V);
                *out = (gp < 0 || gq < 0) ? NAN : (gp == gq ? 1.0 : 0.0);
                continue;
            }
            double* p = (double*)malloc(sizeof(double) * (size_t)V);
            double* qq = (double*)malloc(sizeof(double) * (size_t)V);
            if (oracle_target_dist(zrow, dtype, V, T, top_k, p) ||
                oracle_draft_dist(qrow, V, T, top_k, qq)) {
                *out = NAN;
            } else {
                double s = 0.0;
                for (int i = 0; i < V; ++i) s += p[i] < qq[i] ? p[i] : qq[i];
                *out = s;
            }
            free(p);
            free(qq);
        }
    }
    return 0;
}

/*
 * Sampling verification of a static draft tree.  [EAG], the EAGLE part: with a
 * tree of drafts, a rejected token does not end the step, the other branches
 * are tried; [E2] section 2.1 and [LEV] section 三 give the single test
 * (accept with probability min(1, p/q)) and the residual norm(max(0, p - q)).
 *
 * The pages give no rule for several branches; the reading taken here applies
 * the chain's rule once per sibling.  At the current node c (the root first)
 * P = p'_c, the target distribution of c's row, and Q = q'_c, the draft
 * distribution at c from which c's children were drawn.  The children are
 * tried in increasing node order: child n is accepted iff u[n] < min(1,
 * P(x_n)/Q(x_n)) (the same q'=0 rule as the chain); an acceptance emits x_n and
 * moves to n; a rejection replaces P by max(0, P - Q)/sum (P is kept when that
 * has zero mass) and the next child is tried.  When no child is accepted, or c
 * is a leaf, the token is drawn from P with u[0] (index-ascending inverse CDF,
 * as in the chain).  With the children of c drawn independently from q'_c each
 * round is one step of the chain's method, so the emitted tokens follow the
 * target's law.
 *
 * Layouts: logits [B][N][V]; q [B][N][V] (row n: the draft distribution at
 * node n; rows of leaves are never read); node_tokens [B][N] (entry 0
 * ignored); u [B][N] (u[n], n >= 1: the test of node n; u[0]: the final draw);
 * parents [N], parents[0] = -1, 0 <= parents[n] < n.  T > 0.
 * Outputs: path and tokens [B][D+1] (-1 padded), accept_len [B] = depth of the
 * last accepted node (-1 on error); m_test [B][N]: |u[n] - min(1, ratio)| for
 * the tests performed (NaN otherwise); m_draw [B] as in the chain.
 * Errors: E2 (every node token), E5 (every uniform), E1 for the rows of the
 * nodes the walk visits, E3 / E4 for the draft rows it consults: the whole row
 * when transformed or when a residual is formed, else the entries gathered.
 */
int oracle_verify_tree_sample(const void* logits, int dtype, const float* q, const int32_t* node_tokens,
                              const float* u, const int32_t* parents, int B, int N, int V, double T,
                              int top_k, int32_t* out_path, int32_t* out_tokens, int32_t* accept_len,
                              double* m_test, double* m_draw) {
    if (B <= 0 || N <= 0 || V <= 0 || !(T > 0.0) || isinf(T) || parents[0] != -1) return -1;
    int D = 0;
    int* depth = (int*)malloc(sizeof(int) * (size_t)N);
    depth[0] = 0;
    for (int n = 1; n < N; ++n) {
        if (parents[n] < 0 || parents[n] >= n) { free(depth); return -1; }
        depth[n] = depth[parents[n]] + 1;
        if (depth[n] > D) D = depth[n];
    }
    const size_t esz = logit_size(dtype);
    const int transformed = !(T == 1.0 && !topk_enabled(top_k, V));
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        const char* zb = (const char*)logits + (size_t)b * N * V * esz;
        const float* qb = q + (size_t)b * N * V;
        const int32_t* tk = node_tokens + (size_t)b * N;
        const float* ub = u + (size_t)b * N;
        int32_t* op = out_path + (size_t)b * (D + 1);
        int32_t* ot = out_tokens + (size_t)b * (D + 1);
        double* mt = m_test + (size_t)b * N;
        for (int d = 0; d <= D; ++d) { op[d] = -1; ot[d] = -1; }
        for (int n = 0; n < N; ++n) mt[n] = NAN;
        accept_len[b] = -1;
        m_draw[b] = NAN;
        int err = 0;
        for (int n = 1; n < N; ++n) if (tk[n] < 0 || tk[n] >= V) err = 1;        /* E2 */
        for (int n = 0; n < N; ++n) if (!u_ok(ub[n])) err = 1;                    /* E5 */
        if (err) continue;
        double* P = (double*)malloc(sizeof(double) * (size_t)V);
        double* Q = (double*)malloc(sizeof(double) * (size_t)V);
        int c = 0, d = 0;
        op[0] = 0;
        for (;;) {
            if (oracle_target_dist(zb + (size_t)c * V * esz, dtype, V, T, top_k, P)) { err = 1; break; }  /* E1 */
            const float* qrow = qb + (size_t)c * V;
            int accepted = -1, have_q = 0;
            for (int n = c + 1; n < N && !err; ++n) {
                if (parents[n] != c) continue;
                if (!have_q && transformed) {
                    if (oracle_draft_dist(qrow, V, T, top_k, Q)) { err = 1; break; }       /* E3, E4 */
                    have_q = 1;
                }
                const int x = tk[n];
                if (!have_q && !q_ok(qrow[x])) { err = 1; break; }                           /* E3 */
                const double a = P[x], cq = have_q ? Q[x] : (double)qrow[x];
                double ratio;
                if (cq > 0.0) ratio = a / cq;
                else ratio = a > 0.0 ? INFINITY : 0.0;
                const double thr = ratio < 1.0 ? ratio : 1.0;
                mt[n] = fabs((double)ub[n] - thr);
                if ((double)ub[n] < thr) { accepted = n; break; }
                if (g_variant == 4) continue;   /* planted mistake: the next sibling sees P again */
                /* Rejected: the next sibling (or the final draw) sees the residual. */
                if (!have_q) {
                    for (int i = 0; i < V; ++i) if (!q_ok(qrow[i])) err = 1;                 /* E3 */
                    if (err) break;
                    for (int i = 0; i < V; ++i) Q[i] = (double)qrow[i];
                    have_q = 1;
                }
                double S = 0.0;
                for (int i = 0; i < V; ++i) { const double r = P[i] - Q[i]; S += r > 0.0 ? r : 0.0; }
                if (S > 0.0)                                                                 /* [P10] */
                    for (int i = 0; i < V; ++i) { const double r = P[i] - Q[i]; P[i] = (r > 0.0 ? r : 0.0) / S; }
            }
            if (err || accepted < 0) break;
            ot[d] = tk[accepted];
            c = accepted;
            op[++d] = c;
        }
        if (!err) {
            double S = 0.0, md;
            for (int i = 0; i < V; ++i) S += P[i];
            ot[d] = draw_index(P, V, S, (double)ub[0], &md);
            accept_len[b] = d;
            m_draw[b] = md;
        } else {
            for (int t = 0; t <= D; ++t) { op[t] = -1; ot[t] = -1; }
            for (int n = 0; n < N; ++n) mt[n] = NAN;
        }
        free(P);
        free(Q);
    }
    free(depth);
    return 0;
}

/*
 * EAGLE-2 draft-tree construction ([E2] section 4).  The value of a node is the
 * product of the draft model's confidences along its path from the root
 * (section 4.1; the printed formula is lost, the text states it); the
 * expansion phase feeds the top-k nodes of the newest layer, by value, to the
 * draft model, and each of them gets the draft's top-k tokens as children
 * (section 4.1); the reranking phase keeps the m nodes of highest value over
 * the whole tree, the shallower node first among equal values, which keeps the
 * selection a connected tree, flattens it and masks each token to its ancestors
 * (section 4.2).
 *
 * Readings (the pages fix none of these): values and their products are
 * float32 (value_child = value_parent * q(token), one float32 multiply), so
 * both implementations take every ordering decision on the same numbers; a
 * node's children are its draft row's top_k tokens by probability, larger
 * first, lower index on ties; among equal keys the lower index wins; the
 * selection is flattened in its ranking order (parents come first: a child's
 * value never exceeds its parent's and ties go to the shallower node).
 */

typedef struct { float v; int i; } fi_t;
static int cmp_fdesc_then_index(const void* a, const void* b) {
    const fi_t* x = (const fi_t*)a;
    const fi_t* y = (const fi_t*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->i > y->i) - (x->i < y->i);
}

/*
 * One expansion layer for B batch rows.  q [B][E][V]: the draft distribution at
 * each of the E nodes being expanded; node_value [B][E].  Outputs:
 * child_token [B][E][K] (the row's K most probable tokens), child_value
 * [B][E][K] (node value times the token's probability, in float32), next
 * [B][k_next] (flat indices e*K + i of the k_next children of highest value,
 * lower flat index first among equals).  A row with a NaN, negative or +inf
 * probability, or a node value that is NaN, negative or +inf, is an error: its
 * outputs are all -1 (values NaN).
 */
int oracle_tree_expand(const float* q, const float* node_value, int B, int E, int V, int K, int k_next,
                       int32_t* child_token, float* child_value, int32_t* next) {
    if (B <= 0 || E <= 0 || V <= 0 || K <= 0 || K > V || k_next <= 0 || k_next > E * K) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        int err = 0;
        fi_t* row = (fi_t*)malloc(sizeof(fi_t) * (size_t)V);
        fi_t* kids = (fi_t*)malloc(sizeof(fi_t) * (size_t)E * K);
        for (int e = 0; e < E && !err; ++e) {
            const float* qr = q + ((size_t)b * E + e) * V;
            const float nv = node_value[(size_t)b * E + e];
            if (!q_ok(nv)) err = 1;
            for (int i = 0; i < V; ++i) {
                if (!q_ok(qr[i])) err = 1;
                row[i].v = qr[i];
                row[i].i = i;
            }
            if (err) break;
            qsort(row, (size_t)V, sizeof(fi_t), cmp_fdesc_then_index);
            for (int t = 0; t < K; ++t) {
                const size_t o = ((size_t)b * E + e) * K + t;
                child_token[o] = row[t].i;
                volatile float prod = nv * row[t].v;          /* one float32 rounding */
                child_value[o] = prod;
                kids[e * K + t].v = prod;
                kids[e * K + t].i = e * K + t;
            }
        }
        if (err) {
            for (int o = 0; o < E * K; ++o) {
                child_token[(size_t)b * E * K + o] = -1;
                child_value[(size_t)b * E * K + o] = NAN;
            }
            for (int t = 0; t < k_next; ++t) next[(size_t)b * k_next + t] = -1;
        } else {
            qsort(kids, (size_t)E * K, sizeof(fi_t), cmp_fdesc_then_index);
            for (int t = 0; t < k_next; ++t) next[(size_t)b * k_next + t] = kids[t].i;
        }
        free(row);
        free(kids);
    }
    return 0;
}

typedef struct { float v; int d; int i; } fdi_t;
static int cmp_rerank(const void* a, const void* b) {
    const fdi_t* x = (const fdi_t*)a;
    const fdi_t* y = (const fdi_t*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    if (x->d != y->d) return x->d < y->d ? -1 : 1;
    return (x->i > y->i) - (x->i < y->i);
}

/*
 * Reranking for B batch rows of M candidate nodes (the root excluded).
 * parent [B][M]: the parent's candidate index, -1 for a child of the root,
 * else < the node's own index; value [B][M] (float32).  Keeps the m nodes
 * first in the order (value descending, depth ascending, index ascending) and
 * flattens them in that order after the root (position 0).  Outputs:
 * node [B][m] (candidate index at flattened position p + 1), parent_pos [B][m]
 * (the flattened position of its parent, 0 for the root), mask [B][m+1][m+1]
 * (1 where the column is the row's own position or one of its ancestors').
 * Errors (outputs -1, mask 0): a parent index out of range or not below the
 * node's, a NaN value, or a kept node whose parent is not kept (values that
 * grow along a path).
 */
int oracle_tree_rerank(const int32_t* parent, const float* value, int B, int M, int m,
                       int32_t* node, int32_t* parent_pos, uint8_t* mask) {
    if (B <= 0 || M <= 0 || m <= 0 || m > M) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        const int32_t* pr = parent + (size_t)b * M;
        const float* vr = value + (size_t)b * M;
        int32_t* on = node + (size_t)b * m;
        int32_t* op = parent_pos + (size_t)b * m;
        uint8_t* mk = mask + (size_t)b * (m + 1) * (m + 1);
        int err = 0;
        fdi_t* key = (fdi_t*)malloc(sizeof(fdi_t) * (size_t)M);
        int* depth = (int*)malloc(sizeof(int) * (size_t)M);
        int* pos = (int*)malloc(sizeof(int) * (size_t)M);
        for (int i = 0; i < M; ++i) {
            if (pr[i] < -1 || pr[i] >= i || isnan(vr[i])) { err = 1; break; }
            depth[i] = pr[i] < 0 ? 1 : depth[pr[i]] + 1;
            key[i].v = vr[i];
            key[i].d = depth[i];
            key[i].i = i;
            pos[i] = -1;
        }
        memset(mk, 0, (size_t)(m + 1) * (m + 1));
        if (!err) {
            qsort(key, (size_t)M, sizeof(fdi_t), cmp_rerank);
            for (int p = 0; p < m; ++p) pos[key[p].i] = p + 1;
            for (int p = 0; p < m && !err; ++p) {
                const int i = key[p].i;
                on[p] = i;
                op[p] = pr[i] < 0 ? 0 : pos[pr[i]];
                if (op[p] < 0) err = 1;                       /* parent not kept */
            }
        }
        if (!err) {
            mk[0] = 1;
            for (int p = 0; p < m; ++p) {
                uint8_t* r = mk + (size_t)(p + 1) * (m + 1);
                r[0] = 1;
                for (int i = on[p]; i >= 0; i = pr[i]) r[pos[i]] = 1;
            }
        } else {
            for (int p = 0; p < m; ++p) { on[p] = -1; op[p] = -1; }
            memset(mk, 0, (size_t)(m + 1) * (m + 1));
        }
        free(key);
        free(depth);
        free(pos);
    }
    return 0;
}

/*
 * KV commit after a tree verification ("Việc giải mã giả định và EAGLE-3",
 * KV cache rollback: write the draft's entries to scratch and commit on
 * acceptance, or keep a logical length and cut on rejection).  The verifier
 * appended the N tree nodes' rows at positions prefix[b] + n; the accepted
 * path root..n* (path[b][0..d], d = accept_len[b]) is moved to positions
 * prefix[b] + 0..d in every plane, and the new logical length is
 * prefix[b] + d + 1.  Layout: row (plane, b, s) at byte offset
 * plane*plane_stride + b*batch_stride + s*pos_stride, row_bytes long.  Rows are
 * moved in increasing t; since path is increasing and path[t] >= t, a row is
 * never overwritten before it is read.  Positions 0 .. capacity-1 exist in every
 * (plane, b) row.  A row with accept_len < 0, a negative prefix, a path that is
 * not 0 followed by increasing node indices below N, or a path reaching past the
 * capacity (prefix + path[t] >= capacity), moves nothing and gets new length -1.
 */
int oracle_kv_commit(uint8_t* kv, int planes, long long plane_stride, int B, long long batch_stride,
                     long long pos_stride, int row_bytes, int capacity, const int32_t* prefix, const int32_t* path,
                     int path_stride, int N, const int32_t* accept_len, int32_t* new_len) {
    if (planes <= 0 || B <= 0 || row_bytes <= 0 || N <= 0 || path_stride <= 0 || capacity <= 0) return -1;
    for (int b = 0; b < B; ++b) {
        const int d = accept_len[b];
        const int32_t* pb = path + (size_t)b * path_stride;
        int ok = d >= 0 && d < path_stride && d < N && prefix[b] >= 0 && pb[0] == 0;
        for (int t = 1; ok && t <= d; ++t) ok = pb[t] > pb[t - 1] && pb[t] < N;
        /* every row read (prefix + path[t]) and written (prefix + t <= prefix + path[t])
         * must exist in the cache */
        for (int t = 0; ok && t <= d; ++t) ok = (long long)prefix[b] + pb[t] < (long long)capacity;
        if (!ok) { new_len[b] = -1; continue; }
        for (int pl = 0; pl < planes; ++pl) {
            uint8_t* base = kv + (size_t)pl * plane_stride + (size_t)b * batch_stride;
            for (int t = 1; t <= d; ++t)
                memmove(base + (size_t)(prefix[b] + t) * pos_stride, base + (size_t)(prefix[b] + pb[t]) * pos_stride,
                        (size_t)row_bytes);
        }
        new_len[b] = prefix[b] + d + 1;
    }
    return 0;
}
