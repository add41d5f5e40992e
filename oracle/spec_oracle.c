/*
 * Plain fp64 CPU oracle of the speculative-sampling verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library; the two are checked against
 * each other, never built from each other.
 *
 * Notation follows the pages: p is the target distribution, q the draft
 * distribution (the French lesson "Décodage spéculatif et Eagle", section "Le
 * concept", and the forum post "Speculative Decoding: от идеи до SOTA", §2).
 * The Arabic lesson "Speculative decoding: draft, verify, repeat" swaps the two
 * letters; its formulas are read with the letters exchanged back.
 *
 * Everything is computed in double precision with scalar loops in index order.
 * Sequences (rows, trees) are independent: with OpenMP they are spread over
 * threads, and each one's arithmetic is exactly the single-threaded one, so
 * the results are bitwise the same at any thread count.
 * bf16 inputs are widened exactly (bf16 bits become the top half of an fp32,
 * which is then converted to double); fp32 inputs and the caller's uniforms are
 * promoted to double.  Build with -ffp-contract=off and without fast-math so
 * that every operation is the plain IEEE one written here.
 *
 * Readings of the pages that are not spelled out there (each listed in the
 * design notes):
 *   - acceptance is the strict test u < P/Q (French lesson, "La règle de
 *     l'exactitude"; forum post §3 writes it as accepting with probability
 *     min(1, P/Q), which is the same event because u < 1);
 *   - Q == 0 accepts iff P > 0 (the Arabic lesson's step 1 treats a zero draft
 *     probability as an infinite ratio; a token the target gives zero mass is
 *     not accepted);
 *   - sampling a distribution w is the inverse CDF with one uniform: the
 *     smallest i whose running sum C_i exceeds u * sum(w), strictly;
 *   - if a rejection meets an all-zero residual (possible only through
 *     rounding), the replacement is drawn from p at that position;
 *   - one uniform per drafted position for the accept test and one uniform per
 *     sequence for whichever draw (residual or bonus) ends the step.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_OK = 0, OR_BAD_ARG = 1, OR_NO_MEMORY = 2 };

/* Threads the parallel loops over sequences use (0 or less: OpenMP's default). */
void oracle_set_threads(int n)
{
    omp_set_num_threads(n > 0 ? n : omp_get_num_procs());
}

int oracle_get_threads(void)
{
    return omp_get_max_threads();
}

/* One logit, widened to double.  bf16 is the upper 16 bits of an IEEE fp32. */
static double logit_at(const void *base, int dtype, size_t idx)
{
    if (dtype == OR_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[idx];
}

/* Row `row` of a [rows][V] logit array, widened into out[V]. */
static void load_row(const void *base, int dtype, size_t row, int V, double *out)
{
    for (int i = 0; i < V; ++i)
        out[i] = logit_at(base, dtype, row * (size_t)V + (size_t)i);
}

/*
 * p = softmax(l / T): m is the largest logit, e_i = exp((l_i - m) / T)
 * (exp(-inf) = 0), Z the sum of e_i in index order, p_i = e_i / Z.
 * French lesson, code of "Faites-le": softmax(q_draft(state) / temperature);
 * the same temperature is handed to the target's forward.
 */
static void softmax_T(const double *l, int V, double T, double *p)
{
    double m = -INFINITY;
    for (int i = 0; i < V; ++i)
        if (l[i] > m)
            m = l[i];
    double Z = 0.0;
    for (int i = 0; i < V; ++i) {
        p[i] = exp((l[i] - m) / T);
        Z += p[i];
    }
    for (int i = 0; i < V; ++i)
        p[i] = p[i] / Z;
}

/*
 * Inverse CDF with threshold tau = u * sum(w): the smallest i with
 * C_i = w_0 + ... + w_i > tau.  A zero-weight index is never returned because
 * the comparison is strict.  If rounding lets the loop run out, the largest
 * index with positive weight is returned.
 */
static int invcdf(const double *w, int V, double tau)
{
    double C = 0.0;
    for (int i = 0; i < V; ++i) {
        C += w[i];
        if (C > tau)
            return i;
    }
    for (int i = V - 1; i >= 0; --i)
        if (w[i] > 0.0)
            return i;
    return -1;
}

/* Sum of w in index order. */
static double total(const double *w, int V)
{
    double s = 0.0;
    for (int i = 0; i < V; ++i)
        s += w[i];
    return s;
}

/*
 * Accept/reject of one drafted token (French lesson, "La règle de
 * l'exactitude"; forum post §3, acceptance rule).  P = p(x), Q = q(x).
 */
static int accepts(double P, double Q, double u)
{
    if (Q > 0.0)
        return u < P / Q;
    return P > 0.0;
}

/*
 * Replacement draw after the first rejection: w = max(0, p - q),
 * S = sum(w), token = invcdf(w, u * S)  (French lesson, "La règle de
 * l'exactitude", residual (p - q)+ / ||(p - q)+||_1; forum post §3,
 * resampling rule).  An all-zero residual falls back to p.
 * `w` is scratch of length V; *S_out receives the mass actually sampled.
 */
static int residual_draw(const double *p, const double *q, int V, double u,
                         double *w, double *S_out)
{
    for (int i = 0; i < V; ++i) {
        double d = p[i] - q[i];
        w[i] = d > 0.0 ? d : 0.0;
    }
    double S = total(w, V);
    if (S > 0.0) {
        *S_out = S;
        return invcdf(w, V, u * S);
    }
    double Sp = total(p, V);
    *S_out = Sp;
    return invcdf(p, V, u * Sp);
}

/* Bonus draw when every drafted token is accepted: token = invcdf(p, u * sum p). */
static int bonus_draw(const double *p, int V, double u, double *S_out)
{
    double S = total(p, V);
    *S_out = S;
    return invcdf(p, V, u * S);
}

/*
 * One sequence of the chain verify at temperature T > 0.
 *   target: rows 0..K of the target's logits, draft: rows 0..K-1 of the
 *   draft's logits, x: the K drafted tokens, ua: K accept uniforms,
 *   us: the one residual-or-bonus uniform.
 * Row k of the target scores drafted token k; row K is the bonus row
 * (French lesson, step 2 of the procedure, "K+1 positions").
 * Outputs: tokens[0..K] (first j+1 valid, rest -1), *j_out, and optionally
 * diag[k][4] = {P_k, Q_k, ratio_k, S at k == j else 0}.
 */
static int chain_one(const void *target, const void *draft, int dtype,
                     size_t seq, const int32_t *x, const double *ua, double us,
                     int K, int V, double T, int32_t *tokens, int32_t *j_out,
                     double *diag)
{
    double *buf = (double *)malloc(sizeof(double) * (size_t)V * 4);
    if (!buf)
        return OR_NO_MEMORY;
    double *l = buf, *p = buf + V, *q = buf + 2 * (size_t)V, *w = buf + 3 * (size_t)V;

    if (diag)
        for (int k = 0; k < 4 * (K + 1); ++k)
            diag[k] = 0.0;

    /*
     * Positions 0..K-1 left to right: P = p_k(x_k), Q = q_k(x_k); the first
     * rejection draws the replacement and stops.  With diag requested, the
     * remaining positions' P and Q are still evaluated (and only reported).
     */
    int j = K;
    for (int k = 0; k < K && (j == K || diag); ++k) {
        load_row(target, dtype, seq * (size_t)(K + 1) + (size_t)k, V, l);
        softmax_T(l, V, T, p);
        load_row(draft, dtype, seq * (size_t)K + (size_t)k, V, l);
        softmax_T(l, V, T, q);
        double P = p[x[k]], Q = q[x[k]];
        if (diag) {
            diag[4 * k + 0] = P;
            diag[4 * k + 1] = Q;
            diag[4 * k + 2] = Q > 0.0 ? P / Q : (P > 0.0 ? INFINITY : 0.0);
        }
        if (j < K)
            continue;
        if (accepts(P, Q, ua[k])) {
            tokens[k] = x[k];
        } else {
            j = k;
            double S;
            tokens[k] = residual_draw(p, q, V, us, w, &S);
            if (diag)
                diag[4 * k + 3] = S;
        }
    }
    if (j == K) {
        load_row(target, dtype, seq * (size_t)(K + 1) + (size_t)K, V, l);
        softmax_T(l, V, T, p);
        double S;
        tokens[K] = bonus_draw(p, V, us, &S);
        if (diag)
            diag[4 * K + 3] = S;
    }
    for (int k = j + 1; k <= K; ++k)
        tokens[k] = -1;
    *j_out = j;
    free(buf);
    return OR_OK;
}

static int chain_args_ok(const void *target, const void *draft, int dtype,
                         const int32_t *x, int B, int K, int V, double T)
{
    if (B < 0 || K < 0 || V < 1 || !(T > 0.0) || isinf(T))
        return 0;
    if (dtype != OR_F32 && dtype != OR_BF16)
        return 0;
    if (B > 0 && (!target || (K > 0 && (!draft || !x))))
        return 0;
    for (size_t i = 0; i < (size_t)B * (size_t)K; ++i)
        if (x[i] < 0 || x[i] >= V)
            return 0;
    return 1;
}

/*
 * Chain verify over B sequences with double-precision uniforms.
 *   target [B][K+1][V], draft [B][K][V], x [B][K], ua [B][K], us [B]
 *   out_tokens [B][K+1], out_accepted [B], out_diag nullable [B][K+1][4].
 */
int oracle_verify_chain_f64u(const void *target, const void *draft, int dtype,
                             const int32_t *x, const double *ua, const double *us,
                             int B, int K, int V, double T, int32_t *out_tokens,
                             int32_t *out_accepted, double *out_diag)
{
    if (!chain_args_ok(target, draft, dtype, x, B, K, V, T))
        return OR_BAD_ARG;
    int rc = OR_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        int r = chain_one(target, draft, dtype, (size_t)b, x + (size_t)b * K,
                          ua + (size_t)b * K, us[b], K, V, T,
                          out_tokens + (size_t)b * (K + 1), out_accepted + b,
                          out_diag ? out_diag + (size_t)b * 4 * (K + 1) : NULL);
        if (r != OR_OK) {
#pragma omp critical
            rc = r;
        }
    }
    return rc;
}

/* Same, with the float32 uniforms the GPU library takes. */
int oracle_verify_chain(const void *target, const void *draft, int dtype,
                        const int32_t *x, const float *ua, const float *us,
                        int B, int K, int V, double T, int32_t *out_tokens,
                        int32_t *out_accepted, double *out_diag)
{
    if (!chain_args_ok(target, draft, dtype, x, B, K, V, T))
        return OR_BAD_ARG;
    double *u = (double *)malloc(sizeof(double) * ((size_t)B * (size_t)K + (size_t)B + 1));
    if (!u)
        return OR_NO_MEMORY;
    for (size_t i = 0; i < (size_t)B * (size_t)K; ++i)
        u[i] = (double)ua[i];
    for (int b = 0; b < B; ++b)
        u[(size_t)B * K + b] = (double)us[b];
    int rc = oracle_verify_chain_f64u(target, draft, dtype, x, u, u + (size_t)B * K,
                                      B, K, V, T, out_tokens, out_accepted, out_diag);
    free(u);
    return rc;
}

/*
 * Weights the final draw of a sequence samples from, as doubles in out_w[V]:
 * with a draft row, w = max(0, p - q) (the residual); without one
 * (draft_row == NULL), w = p (the bonus row).  Returns sum(w), or -1 on bad
 * arguments.  Used by the tests to locate CDF boundaries.
 */
double oracle_draw_weights(const void *target_row, const void *draft_row, int dtype,
                           int V, double T, double *out_w)
{
    if (!target_row || !out_w || V < 1 || !(T > 0.0) || (dtype != OR_F32 && dtype != OR_BF16))
        return -1.0;
    double *buf = (double *)malloc(sizeof(double) * (size_t)V * 3);
    if (!buf)
        return -1.0;
    double *l = buf, *p = buf + V, *q = buf + 2 * (size_t)V;
    load_row(target_row, dtype, 0, V, l);
    softmax_T(l, V, T, p);
    if (draft_row) {
        load_row(draft_row, dtype, 0, V, l);
        softmax_T(l, V, T, q);
        for (int i = 0; i < V; ++i) {
            double d = p[i] - q[i];
            out_w[i] = d > 0.0 ? d : 0.0;
        }
    } else {
        for (int i = 0; i < V; ++i)
            out_w[i] = p[i];
    }
    free(buf);
    return total(out_w, V);
}

/* softmax(l / T) of one logit row into out_p[V] (double).  0 on success. */
int oracle_softmax_row(const void *row, int dtype, int V, double T, double *out_p)
{
    if (!row || !out_p || V < 1 || !(T > 0.0) || (dtype != OR_F32 && dtype != OR_BF16))
        return OR_BAD_ARG;
    double *l = (double *)malloc(sizeof(double) * (size_t)V);
    if (!l)
        return OR_NO_MEMORY;
    load_row(row, dtype, 0, V, l);
    softmax_T(l, V, T, out_p);
    free(l);
    return OR_OK;
}

/*
 * Residual draw on given distributions (double p[V], q[V]) with uniform u:
 * the step the chain verify takes at its first rejection, exposed so the
 * all-zero-residual fallback can be exercised directly.
 */
int oracle_residual_draw(const double *p, const double *q, int V, double u, double *S_out)
{
    if (!p || !q || V < 1)
        return -1;
    double *w = (double *)malloc(sizeof(double) * (size_t)V);
    if (!w)
        return -1;
    double S;
    int t = residual_draw(p, q, V, u, w, &S);
    if (S_out)
        *S_out = S;
    free(w);
    return t;
}

/*
 * Acceptance rate of one (target, draft) row pair: sum_i min(p_i, q_i), the
 * probability that a token drawn from q is accepted (forum post §3: summing
 * q(x) min(1, p(x)/q(x)) over x gives the total of min(p, q)).
 */
double oracle_acceptance_rate(const void *target_row, const void *draft_row, int dtype,
                              int V, double T)
{
    if (!target_row || !draft_row || V < 1 || !(T > 0.0))
        return -1.0;
    double *buf = (double *)malloc(sizeof(double) * (size_t)V * 3);
    if (!buf)
        return -1.0;
    double *l = buf, *p = buf + V, *q = buf + 2 * (size_t)V;
    load_row(target_row, dtype, 0, V, l);
    softmax_T(l, V, T, p);
    load_row(draft_row, dtype, 0, V, l);
    softmax_T(l, V, T, q);
    double a = 0.0;
    for (int i = 0; i < V; ++i)
        a += p[i] < q[i] ? p[i] : q[i];
    free(buf);
    return a;
}

/*
 * argmax of one row of raw logits; ties go to the lowest index.  Values are
 * compared as numbers, so -0.0 and +0.0 tie.  Temperature plays no part
 * because softmax is monotone.
 */
static int row_argmax(const void *base, int dtype, size_t row, int V)
{
    int best = 0;
    double bv = logit_at(base, dtype, row * (size_t)V);
    for (int i = 1; i < V; ++i) {
        double v = logit_at(base, dtype, row * (size_t)V + (size_t)i);
        if (v > bv) {
            bv = v;
            best = i;
        }
    }
    return best;
}

int oracle_row_argmax(const void *row, int dtype, int V)
{
    if (!row || V < 1 || (dtype != OR_F32 && dtype != OR_BF16))
        return -1;
    return row_argmax(row, dtype, 0, V);
}

/*
 * Greedy chain verify, T = 0 (French lesson, "La règle de l'exactitude",
 * greedy case): a_k = argmax of target row k; accept drafted token k while it
 * equals a_k; at the first mismatch j emit a_j and stop; if all K match emit
 * the bonus a_K.
 *   target [B][K+1][V], x [B][K] -> out_tokens [B][K+1] (-1 padded), out_accepted [B].
 */
int oracle_verify_greedy(const void *target, int dtype, const int32_t *x, int B, int K,
                         int V, int32_t *out_tokens, int32_t *out_accepted)
{
    if (B < 0 || K < 0 || V < 1 || (dtype != OR_F32 && dtype != OR_BF16))
        return OR_BAD_ARG;
    if (B > 0 && (!target || !out_tokens || !out_accepted || (K > 0 && !x)))
        return OR_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        int32_t *out = out_tokens + (size_t)b * (K + 1);
        int j = K;
        for (int k = 0; k < K; ++k) {
            int a = row_argmax(target, dtype, (size_t)b * (K + 1) + (size_t)k, V);
            if (x[(size_t)b * K + k] == a) {
                out[k] = a;
            } else {
                out[k] = a;
                j = k;
                break;
            }
        }
        if (j == K)
            out[K] = row_argmax(target, dtype, (size_t)b * (K + 1) + (size_t)K, V);
        for (int k = j + 1; k <= K; ++k)
            out[k] = -1;
        out_accepted[b] = j;
    }
    return OR_OK;
}

/*
 * Greedy verify on a static candidate tree, T = 0 (French lesson, "Vérifie
 * l'attention des arbres" and the EAGLE section: one target pass scores every
 * candidate path, the longest accepted branch wins).
 *   node_logits [B][N][V]: row v is the target's distribution after the path
 *     root..v;  node_tokens [B][N]: token of node v (column 0, the root, unused);
 *   parents [N]: parents[0] = -1, 0 <= parents[v] < v.
 * Node v (v > 0) matches iff its token equals the argmax of its parent's row;
 * a node is accepted iff it and all its ancestors match.  The deepest accepted
 * node wins, the lowest node index among equally deep ones.  Output:
 *   out_path [B][D+1]: node ids root..best then -1 (nullable),
 *   out_tokens [B][D+1]: tokens of path[1..d] then the argmax at best, then -1,
 *   out_depth [B]: d.  D is the deepest node's depth.
 */
int oracle_verify_tree_greedy(const void *node_logits, int dtype, const int32_t *node_tokens,
                              const int32_t *parents, int B, int N, int V,
                              int32_t *out_tokens, int32_t *out_path, int32_t *out_depth)
{
    if (B < 0 || N < 1 || V < 1 || !parents || (dtype != OR_F32 && dtype != OR_BF16))
        return OR_BAD_ARG;
    if (parents[0] != -1)
        return OR_BAD_ARG;
    for (int v = 1; v < N; ++v)
        if (parents[v] < 0 || parents[v] >= v)
            return OR_BAD_ARG;
    if (B > 0 && (!node_logits || !node_tokens || !out_tokens || !out_depth))
        return OR_BAD_ARG;

    int *depth = (int *)malloc(sizeof(int) * (size_t)N);
    if (!depth)
        return OR_NO_MEMORY;
    int D = 0;
    depth[0] = 0;
    for (int v = 1; v < N; ++v) {
        depth[v] = depth[parents[v]] + 1;
        if (depth[v] > D)
            D = depth[v];
    }
    int rc = OR_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        int *ok = (int *)malloc(sizeof(int) * (size_t)N * 3);
        if (!ok) {
#pragma omp critical
            rc = OR_NO_MEMORY;
            continue;
        }
        int *amax = ok + N, *path = ok + 2 * N;
        for (int v = 0; v < N; ++v)
            amax[v] = row_argmax(node_logits, dtype, (size_t)b * N + (size_t)v, V);
        ok[0] = 1;
        for (int v = 1; v < N; ++v)
            ok[v] = ok[parents[v]] && node_tokens[(size_t)b * N + v] == amax[parents[v]];
        int best = 0;
        for (int v = 1; v < N; ++v)
            if (ok[v] && depth[v] > depth[best])
                best = v;
        int d = depth[best];
        for (int v = best, i = d; i >= 0; --i) {
            path[i] = v;
            v = parents[v];
        }
        int32_t *ot = out_tokens + (size_t)b * (D + 1);
        for (int i = 0; i < d; ++i)
            ot[i] = node_tokens[(size_t)b * N + path[i + 1]];
        ot[d] = amax[best];
        for (int i = d + 1; i <= D; ++i)
            ot[i] = -1;
        if (out_path) {
            int32_t *op = out_path + (size_t)b * (D + 1);
            for (int i = 0; i <= D; ++i)
                op[i] = i <= d ? path[i] : -1;
        }
        out_depth[b] = d;
        free(ok);
    }
    free(depth);
    return rc;
}

/*
 * Greedy verify on per-sequence candidate trees, T = 0 (French lesson, EAGLE
 * section: the second version of EAGLE shapes each step's tree to the draft's
 * confidence, wider where it is unsure; forum post §6).  The verify rule is the
 * static tree's, applied to each sequence's own tree:
 *   node_logits [B][Nmax][V], node_tokens [B][Nmax], parents [B][Nmax] and
 *   node_count [B]: sequence b has nodes 0..n-1 with n = node_count[b],
 *   1 <= n <= Nmax, parents[b][0] = -1 and 0 <= parents[b][v] < v; rows and
 *   tokens at v >= n are padding and are not read.
 * Node v (0 < v < n) matches iff its token equals the argmax of its parent's
 * row; a node is accepted iff it and all its ancestors match; the deepest
 * accepted node wins, the lowest node index among equally deep ones.  Output,
 * each row padded with -1 to Nmax entries:
 *   out_path [B][Nmax]: node ids root..best (nullable),
 *   out_tokens [B][Nmax]: tokens of path[1..d], then the argmax at best,
 *   out_depth [B]: d.
 */
int oracle_verify_tree_greedy_dyn(const void *node_logits, int dtype, const int32_t *node_tokens,
                                  const int32_t *parents, const int32_t *node_count, int B,
                                  int Nmax, int V, int32_t *out_tokens, int32_t *out_path,
                                  int32_t *out_depth)
{
    if (B < 0 || Nmax < 1 || V < 1 || (dtype != OR_F32 && dtype != OR_BF16))
        return OR_BAD_ARG;
    if (B > 0 && (!node_logits || !node_tokens || !parents || !node_count || !out_tokens ||
                  !out_depth))
        return OR_BAD_ARG;
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parents + (size_t)b * Nmax;
        const int n = node_count[b];
        if (n < 1 || n > Nmax || par[0] != -1)
            return OR_BAD_ARG;
        for (int v = 1; v < n; ++v)
            if (par[v] < 0 || par[v] >= v)
                return OR_BAD_ARG;
    }
    int rc = OR_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        int *dep = (int *)malloc(sizeof(int) * (size_t)Nmax * 4);
        if (!dep) {
#pragma omp critical
            rc = OR_NO_MEMORY;
            continue;
        }
        int *acc = dep + Nmax, *am = dep + 2 * Nmax, *route = dep + 3 * Nmax;
        const int32_t *par = parents + (size_t)b * Nmax;
        const int32_t *tok = node_tokens + (size_t)b * Nmax;
        const int n = node_count[b];
        dep[0] = 0;
        for (int v = 1; v < n; ++v)
            dep[v] = dep[par[v]] + 1;
        for (int v = 0; v < n; ++v)
            am[v] = row_argmax(node_logits, dtype, (size_t)b * Nmax + (size_t)v, V);
        acc[0] = 1;
        for (int v = 1; v < n; ++v)
            acc[v] = acc[par[v]] && tok[v] == am[par[v]];
        int top = 0;
        for (int v = 1; v < n; ++v)
            if (acc[v] && dep[v] > dep[top])
                top = v;
        const int d = dep[top];
        for (int v = top, i = d; i >= 0; --i) {
            route[i] = v;
            v = par[v];
        }
        int32_t *ot = out_tokens + (size_t)b * Nmax;
        for (int i = 0; i < Nmax; ++i)
            ot[i] = i < d ? tok[route[i + 1]] : (i == d ? am[top] : -1);
        if (out_path) {
            int32_t *op = out_path + (size_t)b * Nmax;
            for (int i = 0; i < Nmax; ++i)
                op[i] = i <= d ? route[i] : -1;
        }
        out_depth[b] = d;
        free(dep);
    }
    return rc;
}

/*
 * Top-k of draft rows, the expansion step of an EAGLE-style tree drafter
 * (French lesson, EAGLE section: a tree of 4 to 8 candidates per depth, and
 * its exercise: the draft proposes its top branches at each depth).
 *   logits [rows][V]; 1 <= k <= 8, k <= V.
 *   out_idx [rows][k]: the k entries of largest value, by value descending and
 *     then index ascending (so -0.0 ties +0.0 and the lower index comes first);
 *   out_val [rows][k] (nullable): their logits, as stored (bf16 widened).
 * k rounds per row, each taking the best entry not yet taken.
 */
int oracle_topk(const void *logits, int dtype, int rows, int V, int k, int32_t *out_idx,
                float *out_val)
{
    if (rows < 0 || V < 1 || k < 1 || k > 8 || k > V || (dtype != OR_F32 && dtype != OR_BF16))
        return OR_BAD_ARG;
    if (rows > 0 && (!logits || !out_idx))
        return OR_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; ++r) {
        int taken[8];
        for (int q = 0; q < k; ++q) {
            int best = -1;
            double bv = 0.0;
            for (int i = 0; i < V; ++i) {
                int used = 0;
                for (int t = 0; t < q; ++t)
                    used |= taken[t] == i;
                if (used)
                    continue;
                double v = logit_at(logits, dtype, (size_t)r * (size_t)V + (size_t)i);
                if (best < 0 || v > bv) {
                    bv = v;
                    best = i;
                }
            }
            taken[q] = best;
            out_idx[(size_t)r * k + q] = best;
            if (out_val)
                out_val[(size_t)r * k + q] = (float)bv;
        }
    }
    return OR_OK;
}

/*
 * KV commit after verify (the Arabic lesson, section on rolling the KV cache
 * back, and its key-terms entry "KV rollback": the verifier's forward writes
 * the drafted positions' keys and values to a scratch buffer first; the ones
 * the verify accepts are committed to the cache and the rest discarded; its
 * exercises check that after a rejection the cache reads the prefix followed
 * by the accepted drafts).  Byte copies only, no arithmetic.
 *
 *   scratch [planes][B][N][row_bytes]  keys / values the forward wrote, one row
 *                                      per scratch position (a chain's drafts, or
 *                                      a tree's nodes);
 *   cache   [planes][B][S][row_bytes]  the per-sequence cache, slots 0..len-1 in use;
 *   path    [B][P] or NULL             scratch row of the i-th committed entry
 *                                      (NULL: row i);
 *   count   [B]                        entries to commit;
 *   len     [B]                        slots in use before the commit;
 *   new_len [B]                        slots in use after it.
 * Sequence b is committed iff 0 <= count[b] <= P (P = N when path is NULL),
 * 0 <= len[b], len[b] + count[b] <= S and every path[b][i], i < count[b], lies
 * in [0, N).  Then for every plane, cache slot len[b] + i receives scratch row
 * path[b][i] for i < count[b], and new_len[b] = len[b] + count[b].  Otherwise
 * nothing of b is written and new_len[b] = len[b].
 */
int oracle_kv_commit(const void *scratch, void *cache, int planes, int B, int N, int S,
                     int64_t row_bytes, const int32_t *path, int P, const int32_t *count,
                     const int32_t *len, int32_t *new_len)
{
    if (planes < 0 || B < 0 || N < 0 || S < 0 || row_bytes < 0 || (path && P < 0))
        return OR_BAD_ARG;
    if (B > 0 && (!count || !len || !new_len))
        return OR_BAD_ARG;
    if (!path)
        P = N;
    const unsigned char *src = (const unsigned char *)scratch;
    unsigned char *dst = (unsigned char *)cache;
    for (int b = 0; b < B; ++b) {
        int c = count[b], L = len[b];
        int ok = c >= 0 && c <= P && L >= 0 && (int64_t)L + c <= S;
        for (int i = 0; ok && i < c; ++i) {
            int r = path ? path[(size_t)b * P + i] : i;
            if (r < 0 || r >= N)
                ok = 0;
        }
        if (!ok) {
            new_len[b] = L;
            continue;
        }
        for (int l = 0; l < planes; ++l)
            for (int i = 0; i < c; ++i) {
                int r = path ? path[(size_t)b * P + i] : i;
                size_t from = (((size_t)l * B + b) * N + r) * (size_t)row_bytes;
                size_t to = (((size_t)l * B + b) * S + L + i) * (size_t)row_bytes;
                memcpy(dst + to, src + from, (size_t)row_bytes);
            }
        new_len[b] = L + c;
    }
    return OR_OK;
}

/*
 * Tree attention mask (the French lesson, section on verifying a tree with
 * attention: one forward over the tree where each token attends only to its
 * ancestors; the forum post §10 adds that this needs custom masks and
 * position ids).
 *
 *   parents    [B][N]  parents[b][0] is the root's entry; node v > 0 is
 *                      attached when 0 <= parents[b][v] < v and its parent is
 *                      attached (the root always is);
 *   node_count [B] or NULL (all N): nodes v >= node_count[b] are padding
 *                      (node_count is clamped to [1, N]);
 *   mask  [B][N][W] uint32, W = ceil(N / 32): for an attached node v, bit j
 *                      (word j / 32, bit j % 32) is set iff j == v or j is an
 *                      ancestor of v; rows of other nodes are all zero;
 *   depth [B][N] int32: the number of ancestors of an attached node, -1 for
 *                      the others (a position id is the cache length plus it).
 * Each node walks to the root through its parent entries, one step at a time.
 */
int oracle_tree_mask(const int32_t *parents, const int32_t *node_count, int B, int N,
                     uint32_t *mask, int32_t *depth)
{
    if (B < 0 || N < 1 || (B > 0 && (!parents || !mask || !depth)))
        return OR_BAD_ARG;
    int W = (N + 31) / 32;
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parents + (size_t)b * N;
        int n = node_count ? node_count[b] : N;
        if (n < 1)
            n = 1;
        if (n > N)
            n = N;
        for (int v = 0; v < N; ++v) {
            uint32_t *row = mask + ((size_t)b * N + v) * W;
            for (int w = 0; w < W; ++w)
                row[w] = 0;
            depth[(size_t)b * N + v] = -1;
            if (v >= n)
                continue;
            int cur = v, steps = 0, attached = 1;
            row[cur / 32] |= 1u << (cur % 32);
            while (cur != 0) {
                int p = par[cur];
                if (p < 0 || p >= cur) {
                    attached = 0;
                    break;
                }
                cur = p;
                row[cur / 32] |= 1u << (cur % 32);
                ++steps;
            }
            if (!attached) {
                for (int w = 0; w < W; ++w)
                    row[w] = 0;
                continue;
            }
            depth[(size_t)b * N + v] = steps;
        }
    }
    return OR_OK;
}
