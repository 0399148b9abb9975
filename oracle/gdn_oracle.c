/*
 * gdn_oracle.c -- plain fp64 CPU oracle for Gated DeltaNet tree verification
 * and accepted-path persistence.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is loaded by the test suite, by the
 * smoke check and by the CPU-baseline leg of the benchmark, never by the GPU
 * library; it shares no code, header or constant with it.
 *
 * What it computes.  The GreenGames page ("TL;DR", "Why the experiment
 * exists") builds its decoder around a Gated DeltaNet kernel that keeps a
 * recurrent ("SSM") state per layer next to the KV cache; the pages never
 * write the recurrence down.  The reading taken here is the gated delta rule:
 * one token with key k (length D_k), value v (length D_v), decay a and write
 * strength b turns the D_v x D_k state S into
 *
 *         S' = a * S * (I - b k k^T) + b * v k^T ,      output o = S' q .
 *
 * In a draft tree every node holds one token; node n's state is the rule
 * applied to its parent's state (the committed state S0 for a root), so a
 * node's state is the plain sequential recurrence over the tokens on its
 * root-to-node path.  That is the DDTree idea on the magik.net page ("The
 * Broader Context": verify a whole tree of drafts in one target forward) and
 * the persist kernel on the GreenGames page ("Key wins"): after acceptance,
 * the accepted node's state becomes the new committed state.
 *
 * Everything is fp64 with straightforward loops; the only reassociation is
 * S (I - b k k^T) = S - b (S k) k^T, evaluated row by row.  Inputs arrive as
 * fp64 (exact widening of their bf16/fp32 storage).  Layouts (row-major):
 *   q, k   [n][hk][dk]      v   [n][hv][dv]      a, b  [n][hv]
 *   S0     [hv][dv][dk]     out [n][hv][dv]      value head h reads key head
 *   h / (hv / hk) (contiguous grouping).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* out = a * S (I - b k k^T) + b v k^T   (S, out: dv x dk; out may not alias S) */
static void gated_delta_rule(int dv, int dk, const double *S, const double *k,
                             const double *v, double a, double b, double *out)
{
    for (int i = 0; i < dv; ++i) {
        const double *Si = S + (size_t)i * dk;
        double sk = 0.0; /* (S k)_i */
        for (int j = 0; j < dk; ++j)
            sk += Si[j] * k[j];
        double *Oi = out + (size_t)i * dk;
        for (int j = 0; j < dk; ++j)
            Oi[j] = a * (Si[j] - b * sk * k[j]) + b * v[i] * k[j];
    }
}

/* y = S x */
static void state_times(int dv, int dk, const double *S, const double *x, double *y)
{
    for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j)
            acc += S[(size_t)i * dk + j] * x[j];
        y[i] = acc;
    }
}

/*
 * Sequential recurrence over L tokens, all value heads.
 * q/out may be NULL (state only).  S_final (nullable) gets the state after
 * the last token, [hv][dv][dk].
 */
int oracle_chain(int L, int hk, int hv, int dk, int dv,
                 const double *q, const double *k, const double *v,
                 const double *a, const double *b,
                 const double *S0, double *out, double *S_final)
{
    if (L < 0 || hk <= 0 || hv <= 0 || hv % hk != 0 || dk <= 0 || dv <= 0)
        return -1;
    const int group = hv / hk;
    const size_t ss = (size_t)dv * dk;
    int err = 0;
#pragma omp parallel for schedule(dynamic)
    for (int h = 0; h < hv; ++h) {
        const int g = h / group;
        double *cur = malloc(ss * sizeof(double));
        double *nxt = malloc(ss * sizeof(double));
        if (!cur || !nxt) {
            err = -2;
            free(cur);
            free(nxt);
            continue;
        }
        memcpy(cur, S0 + (size_t)h * ss, ss * sizeof(double));
        for (int t = 0; t < L; ++t) {
            const double *kt = k + ((size_t)t * hk + g) * dk;
            const double *vt = v + ((size_t)t * hv + h) * dv;
            gated_delta_rule(dv, dk, cur, kt, vt, a[(size_t)t * hv + h], b[(size_t)t * hv + h], nxt);
            double *tmp = cur;
            cur = nxt;
            nxt = tmp;
            if (q && out)
                state_times(dv, dk, cur, q + ((size_t)t * hk + g) * dk, out + ((size_t)t * hv + h) * dv);
        }
        if (S_final)
            memcpy(S_final + (size_t)h * ss, cur, ss * sizeof(double));
        free(cur);
        free(nxt);
    }
    return err;
}

/* depth of node i (root = 1); -1 if the walk does not end within n steps */
static int node_depth(int n, const int32_t *parent, int i)
{
    int d = 0;
    while (i != -1) {
        if (i < 0 || i >= n || ++d > n)
            return -1;
        i = parent[i];
    }
    return d;
}

/*
 * Tree verify for one sequence of n nodes (parent: local ids, -1 = root; the
 * tree must be valid).  Nodes are visited in increasing depth (then id) and
 * every node's full state is kept, so each state is computed from its
 * parent's stored state.  out [n][hv][dv]; node_states (nullable)
 * [n][hv][dv][dk].
 */
int oracle_tree(int n, const int32_t *parent, int hk, int hv, int dk, int dv,
                const double *q, const double *k, const double *v,
                const double *a, const double *b, const double *S0,
                double *out, double *node_states)
{
    if (n < 0 || hk <= 0 || hv <= 0 || hv % hk != 0)
        return -1;
    if (n == 0)
        return 0;
    int *depth = malloc((size_t)n * sizeof(int));
    int *visit = malloc((size_t)n * sizeof(int));
    if (!depth || !visit) {
        free(depth);
        free(visit);
        return -2;
    }
    int maxd = 0;
    for (int i = 0; i < n; ++i) {
        depth[i] = node_depth(n, parent, i);
        if (depth[i] < 0) {
            free(depth);
            free(visit);
            return -3;
        }
        if (depth[i] > maxd)
            maxd = depth[i];
    }
    int cnt = 0;
    for (int d = 1; d <= maxd; ++d)
        for (int i = 0; i < n; ++i)
            if (depth[i] == d)
                visit[cnt++] = i;

    const int group = hv / hk;
    const size_t ss = (size_t)dv * dk;
    int err = 0;
#pragma omp parallel for schedule(dynamic)
    for (int h = 0; h < hv; ++h) {
        const int g = h / group;
        double *st = malloc((size_t)n * ss * sizeof(double));
        if (!st) {
            err = -2;
            continue;
        }
        for (int c = 0; c < n; ++c) {
            const int i = visit[c];
            const double *par = parent[i] < 0 ? S0 + (size_t)h * ss : st + (size_t)parent[i] * ss;
            gated_delta_rule(dv, dk, par, k + ((size_t)i * hk + g) * dk, v + ((size_t)i * hv + h) * dv,
                             a[(size_t)i * hv + h], b[(size_t)i * hv + h], st + (size_t)i * ss);
            state_times(dv, dk, st + (size_t)i * ss, q + ((size_t)i * hk + g) * dk,
                        out + ((size_t)i * hv + h) * dv);
            if (node_states)
                memcpy(node_states + ((size_t)i * hv + h) * ss, st + (size_t)i * ss, ss * sizeof(double));
        }
        free(st);
    }
    free(depth);
    free(visit);
    return err;
}

/*
 * Persist for one sequence: walk parent pointers from the accepted node m up
 * to its root, then replay the rule over that path from S0, root first.
 * path_out (nullable, capacity n) receives the path root-first; returns the
 * path length, or a negative value for a bad m / tree.
 */
int oracle_accept_state(int n, const int32_t *parent, int m, int hk, int hv, int dk, int dv,
                        const double *k, const double *v, const double *a, const double *b,
                        const double *S0, double *S_out, int32_t *path_out)
{
    if (m < 0 || m >= n || hk <= 0 || hv <= 0 || hv % hk != 0)
        return -1;
    int len = node_depth(n, parent, m);
    if (len < 0)
        return -3;
    int32_t *path = malloc((size_t)len * sizeof(int32_t));
    if (!path)
        return -2;
    for (int i = m, pos = len - 1; i != -1; i = parent[i], --pos)
        path[pos] = i;
    if (path_out)
        memcpy(path_out, path, (size_t)len * sizeof(int32_t));

    const int group = hv / hk;
    const size_t ss = (size_t)dv * dk;
    int err = 0;
#pragma omp parallel for schedule(dynamic)
    for (int h = 0; h < hv; ++h) {
        const int g = h / group;
        double *cur = malloc(ss * sizeof(double));
        double *nxt = malloc(ss * sizeof(double));
        if (!cur || !nxt) {
            err = -2;
            free(cur);
            free(nxt);
            continue;
        }
        memcpy(cur, S0 + (size_t)h * ss, ss * sizeof(double));
        for (int p = 0; p < len; ++p) {
            const int i = path[p];
            gated_delta_rule(dv, dk, cur, k + ((size_t)i * hk + g) * dk, v + ((size_t)i * hv + h) * dv,
                             a[(size_t)i * hv + h], b[(size_t)i * hv + h], nxt);
            double *tmp = cur;
            cur = nxt;
            nxt = tmp;
        }
        memcpy(S_out + (size_t)h * ss, cur, ss * sizeof(double));
        free(cur);
        free(nxt);
    }
    free(path);
    return err < 0 ? err : len;
}

/* number of OpenMP threads the oracle runs with (1 without OpenMP) */
int oracle_num_threads(void)
{
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            t = omp_get_num_threads();
#endif
        }
    }
    return t;
}

/* Threads the loops above use from now on (the CPU baseline times one thread
   and all of them); n < 1 restores the OpenMP default. */
void oracle_set_threads(int n)
{
    static int dflt = 0;
    if (dflt == 0)
        dflt = omp_get_max_threads();
    omp_set_num_threads(n >= 1 ? n : dflt);
}
