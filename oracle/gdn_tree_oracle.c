/*
 * Test infrastructure, not part of the product path. Only the tests, the smoke check and the
 * benchmark's CPU baseline load this library.
 *
 * The oracle for tree-structured verification of one Gated DeltaNet layer: a plain, slow fp64
 * CPU implementation that runs the gated delta rule along every node's root path, forking the
 * parent's full d_k x d_v state at every node. It contains no triangular solve, no pseudo-value
 * algebra, no blocking and no reordering: each node's output is the recurrence's own output.
 *
 * Sources (the canopy project page, projects.dotslasha.me/p/canopy.md):
 *  - "Science background / The gated delta rule": for a token with query q, key k, value v,
 *    decay alpha and write strength beta, the state is first decayed (S~ = alpha S), the
 *    pseudo-value is u = beta (v - S~^T k), the new state is S = S~ + k u^T and the output is
 *    o = S^T q, read from the updated state. The state has shape d_k x d_v.
 *  - "The tree closed form": nodes are numbered so that every parent precedes its child, node 0
 *    is a root, S0 is the committed state before the tree, l_i = log alpha_i + l_parent(i) with
 *    the root's parent contributing 0, A(i) is the set of strict ancestors and path(i) adds i.
 *  - "M1: Oracle and tree generators": the oracle visits nodes in index order, starts a root
 *    from S0 and every other node from its parent's state, and records every node's state and
 *    output; the pseudo-value u of node i is row i of U.
 *  - Commit ("What the commit kernel stores", "M5"): the committed state for an accepted node a
 *    is the state the recurrence reaches at a, i.e. after the accepted root path's tokens.
 *
 * Layouts (row-major, C order): q, k [B,T,H,dk]; v [B,T,H,dv]; alpha, beta [B,T,H];
 * S0 [B,H,dk,dv]; parent [B,T] int32; O, U [B,T,H,dv]; ell [B,T,H].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the OpenMP thread count of later calls (n >= 1); used to time the oracle on one core. */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* 0 if every node satisfies -1 <= parent[i] < i, else 1 + the first node that does not.
 * (Parents precede children; node 0 is therefore a root.) */
int oracle_tree_check(int T, const int32_t *parent) {
    for (int i = 0; i < T; ++i)
        if (parent[i] < -1 || parent[i] >= i) return 1 + i;
    return 0;
}

/* Brute-force tree structure by walking parent pointers.
 * depth[b,i] = |A(i)| (root 0). mask[b,i,w] bit (j % 32) of word j / 32 is set iff j is in
 * path(i) (ancestors and i itself), words = ceil(T/32). status[b] = oracle_tree_check. */
void oracle_tree_structure(int B, int T, const int32_t *parent, int32_t *depth,
                           uint32_t *mask, int32_t *status) {
    const int W = (T + 31) / 32;
    for (int b = 0; b < B; ++b) {
        const int32_t *p = parent + (size_t)b * T;
        status[b] = oracle_tree_check(T, p);
        for (int i = 0; i < T; ++i) {
            uint32_t *row = mask + ((size_t)b * T + i) * W;
            for (int w = 0; w < W; ++w) row[w] = 0u;
            depth[(size_t)b * T + i] = 0;
            if (status[b] != 0) continue;
            int n = i, count = 0;
            while (n >= 0) {
                row[n / 32] |= 1u << (n % 32);
                n = p[n];
                ++count;
            }
            depth[(size_t)b * T + i] = count - 1;
        }
    }
}

/* One step of the gated delta rule on a dk x dv state, in place:
 * S <- alpha S; u = beta (v - S^T k); S <- S + k u^T. Writes u. */
static void gdn_step(int dk, int dv, double *S, const double *k, const double *v,
                     double alpha, double beta, double *u) {
    for (int a = 0; a < dk * dv; ++a) S[a] *= alpha;
    for (int c = 0; c < dv; ++c) {
        double stk = 0.0;
        for (int r = 0; r < dk; ++r) stk += S[(size_t)r * dv + c] * k[r];
        u[c] = beta * (v[c] - stk);
    }
    for (int r = 0; r < dk; ++r)
        for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] += k[r] * u[c];
}

/* Every node's output, pseudo-value and log cumulative decay, by the per-path recurrence.
 * accept[b] (may be NULL): a node whose state is copied to S_accept[b] (S0 if accept[b] < 0).
 * S_all (may be NULL): every node's state [B,T,H,dk,dv]. Sequences whose tree fails
 * oracle_tree_check get NaN outputs. */
void oracle_gdn_tree(int B, int H, int T, int dk, int dv, const int32_t *parent,
                     const double *q, const double *k, const double *v, const double *alpha,
                     const double *beta, const double *S0, double *O, double *U, double *ell,
                     const int32_t *accept, double *S_accept, double *S_all) {
    const size_t SS = (size_t)dk * dv;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < (long)B * H; ++bh) {
        const int b = (int)(bh / H), h = (int)(bh % H);
        const int32_t *p = parent + (size_t)b * T;
        const double *s0 = S0 + (size_t)bh * SS;
        const int bad = oracle_tree_check(T, p);
        double *S = (double *)malloc(sizeof(double) * SS * (size_t)(T > 0 ? T : 1));
        for (int i = 0; i < T; ++i) {
            const size_t node = ((size_t)b * T + i) * H + h; /* index of (b, i, h) */
            double *o = O + node * dv, *u = U + node * dv;
            if (bad) {
                for (int c = 0; c < dv; ++c) o[c] = u[c] = NAN;
                ell[node] = NAN;
                continue;
            }
            double *Si = S + (size_t)i * SS;
            const double *Sp = p[i] < 0 ? s0 : S + (size_t)p[i] * SS;
            memcpy(Si, Sp, sizeof(double) * SS); /* fork the parent's state */
            gdn_step(dk, dv, Si, k + node * dk, v + node * dv, alpha[node], beta[node], u);
            const double *qi = q + node * dk;
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int r = 0; r < dk; ++r) acc += Si[(size_t)r * dv + c] * qi[r];
                o[c] = acc;
            }
            const double lp = p[i] < 0 ? 0.0 : ell[((size_t)b * T + p[i]) * H + h];
            ell[node] = log(alpha[node]) + lp;
            if (S_all) memcpy(S_all + node * SS, Si, sizeof(double) * SS);
        }
        if (S_accept) {
            double *dst = S_accept + (size_t)bh * SS;
            const int a = accept ? accept[b] : -1;
            if (bad)
                for (size_t x = 0; x < SS; ++x) dst[x] = NAN;
            else
                memcpy(dst, (a < 0 || a >= T) ? s0 : S + (size_t)a * SS, sizeof(double) * SS);
        }
        free(S);
    }
}

/* The committed state for an accepted root path: the recurrence run from S0 over the path's
 * tokens only. path [B,T] root-first node ids, path_len [B]. A valid path has 0 <= path_len <= T,
 * starts at a root and every next node is a child of the previous one (only the path's own
 * parent links are checked). status[b] = 0 if valid, -1 if path_len is out of range, else
 * 1 + the first position whose node breaks the chain; S_new[b] is then NaN.
 * path_len 0 returns S0. */
void oracle_commit(int B, int H, int T, int dk, int dv, const int32_t *parent,
                   const int32_t *path, const int32_t *path_len, const double *k,
                   const double *v, const double *alpha, const double *beta, const double *S0,
                   double *S_new, int32_t *status) {
    const size_t SS = (size_t)dk * dv;
    for (int b = 0; b < B; ++b) {
        const int32_t *p = parent + (size_t)b * T;
        const int32_t *pa = path + (size_t)b * T;
        const int m = path_len[b];
        int st = (m < 0 || m > T) ? -1 : 0;
        for (int t = 0; st == 0 && t < m; ++t) {
            const int n = pa[t];
            if (n < 0 || n >= T || p[n] != (t == 0 ? -1 : pa[t - 1])) st = 1 + t;
        }
        status[b] = st;
#pragma omp parallel for schedule(dynamic, 1)
        for (int h = 0; h < H; ++h) {
            const size_t bh = (size_t)b * H + h;
            double *S = S_new + bh * SS;
            if (st != 0) {
                for (size_t x = 0; x < SS; ++x) S[x] = NAN;
                continue;
            }
            memcpy(S, S0 + bh * SS, sizeof(double) * SS);
            double *u = (double *)malloc(sizeof(double) * (size_t)(dv > 0 ? dv : 1));
            for (int t = 0; t < m; ++t) {
                const size_t node = ((size_t)b * T + pa[t]) * H + h;
                gdn_step(dk, dv, S, k + node * dk, v + node * dv, alpha[node], beta[node], u);
            }
            free(u);
        }
    }
}
