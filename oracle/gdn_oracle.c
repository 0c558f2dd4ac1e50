/*
 * gdn_oracle.c - plain fp64 CPU oracle for tree-structured gated-delta-rule
 * (GDN) verification, accepted-path commit, and the ancestry-gathered causal
 * conv1d that feeds it.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP library, and it never reads a value
 * produced by the HIP library.
 *
 * Everything here is the plain definition, computed node by node in double
 * precision, with no blocking, fusion or reordering:
 *
 *  - The gated delta rule, S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,
 *    o_t = S_t q_t, with the state a d_v x d_k matrix
 *    (TreeWY: Speculative Verification for Gated DeltaNet Hybrids, Sec. 1).
 *  - Its three-step form: decay the state, take the delta correction against
 *    the decayed state, add the outer-product write, then read out
 *    (Bole review, Sec. 1, Eq. (1); there the state is stored transposed).
 *  - On a draft tree a node starts from its parent's state, never from the
 *    previous packed row (Bole review, Sec. 3.1; GDN Tree-Scan review,
 *    "Background" and the packed-buffer example).
 *  - The shared descriptor: parent indices, depth, logical-to-physical rows
 *    (LumoTree, Sec. III-A and III-C).
 *  - Commit replays the accepted root-to-frontier path from the committed
 *    state and publishes the result in place (LumoTree, Sec. IV-B and V-A;
 *    Bole review, Algorithm 2 step 8: nothing accepted leaves the state alone).
 *  - Convolution windows come from the node's ancestors, then from the prior
 *    convolution history, taps applied oldest to newest, unused history kept
 *    as padding (LumoTree, Sec. V-C).
 *
 * Where the pages are silent this file reads them as follows: parent -1
 * means "child of the committed state"; q/k normalisation (when asked for)
 * is x / sqrt(sum x^2 + 1e-6); gates a, b are given post-activation; no
 * 1/sqrt(d_k) query scale; value head h reads qk head floor(h * Hqk / Hv).
 *
 * Parity pins live in tests/test_oracle_pins.py and tests/test_oracle_bruteforce.py.
 *
 * ORA_MUTATION (compile-time, default 0) plants one deliberate mistake; the
 * test suite builds such variants in a temporary directory to show that the
 * pins catch each of them.  The default build contains none.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORA_MUTATION
#define ORA_MUTATION 0
#endif

/* Error bits, one per kind of malformed input.  Same meaning as the bits in
 * the library header, written down again here on purpose (no shared header). */
#define EV_PARENT 1 /* parent[i] outside [-1, i-1] */
#define EV_ROW 2    /* node_row outside [0, R) or not injective */
#define EV_STATE 4  /* state_idx outside [0, P) (commit: or shared by two requests) */
#define EV_PATH 8   /* accepted path not a parent chain from a root-level node */

int ora_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the parallel loops that follow (n < 1: leave as is). */
void ora_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------- */
/* Descriptor: validation, depth, strict-ancestor mask, conv tap sources.     */
/* ------------------------------------------------------------------------- */
int ora_desc_build(int T, int N, int R, int W, const int32_t *parent,
                   const int32_t *node_row, int32_t *depth, uint64_t *anc,
                   int32_t *conv_src, int32_t *status)
{
    const int H = W - 1; /* taps taken from predecessors / history slots */
    int all = 0;
    for (int t = 0; t < T; t++) {
        const int32_t *par = parent + (size_t)t * N;
        const int32_t *row = node_row + (size_t)t * N;
        int32_t *dep = depth + (size_t)t * N;
        uint64_t *an = anc + (size_t)t * N;
        int32_t *src = (H > 0) ? conv_src + (size_t)t * N * H : NULL;
        int st = 0;
        for (int i = 0; i < N; i++) {
            if (par[i] < -1 || par[i] >= i)
                st |= EV_PARENT;
            if (row[i] < 0 || row[i] >= R)
                st |= EV_ROW;
            for (int j = 0; j < i; j++)
                if (row[j] == row[i])
                    st |= EV_ROW;
        }
        status[t] = st;
        all |= st;
        if (st) {
            memset(dep, 0, sizeof(int32_t) * N);
            memset(an, 0, sizeof(uint64_t) * N);
            if (src)
                memset(src, 0, sizeof(int32_t) * N * H);
            continue;
        }
        for (int i = 0; i < N; i++) {
            int p = par[i];
            /* depth = number of nodes on the root-to-i path (1 for a child of
             * the committed state); anc = set of strict ancestors */
            dep[i] = (p < 0) ? 1 : dep[p] + 1;
            an[i] = (p < 0) ? 0 : (an[p] | (1ull << p));
        }
        for (int i = 0; i < N && H > 0; i++) {
            /* m-th predecessor, most recent first: parent, grandparent, ...;
             * past the root-level node, history slots H-1, H-2, ... */
            int cur = par[i];
            int slot = H - 1;
            for (int m = 0; m < H; m++) {
                int32_t v;
                if (cur >= 0) {
#if ORA_MUTATION == 5
                    v = row[i > 0 ? i - 1 : 0]; /* planted: previous packed row */
#else
                    v = row[cur];
#endif
                    cur = par[cur];
                } else {
                    v = -(slot + 1);
                    slot--;
                }
                /* stored oldest -> newest: position H-1 is the parent */
                src[(size_t)i * H + (H - 1 - m)] = v;
            }
        }
    }
    return all;
}

/* ------------------------------------------------------------------------- */
/* Ancestry-gathered causal conv1d over the tree.                             */
/* ------------------------------------------------------------------------- */
int ora_conv(int B, int N, int R, int C, int W, int shared,
             const int32_t *node_row, const int32_t *conv_src,
             const int32_t *status, const double *x, const double *hist, int P,
             const int32_t *state_idx, const double *w, const double *bias,
             int act, double *y)
{
    const int H = W - 1;
    int err = 0;
    for (int b = 0; b < B; b++) {
        const int t = shared ? 0 : b;
        if (status[t])
            continue;
        const int s = state_idx[b];
        if (s < 0 || s >= P) {
            err |= EV_STATE;
            continue;
        }
        for (int i = 0; i < N; i++) {
            const int row = node_row[(size_t)t * N + i];
            const int32_t *src = (H > 0) ? conv_src + ((size_t)t * N + i) * H : NULL;
            for (int c = 0; c < C; c++) {
                double z = 0.0;
                for (int tap = 0; tap < H; tap++) { /* oldest tap first */
#if ORA_MUTATION == 6
                    const int32_t sv = src[H - 1 - tap]; /* planted: taps reversed */
#else
                    const int32_t sv = src[tap];
#endif
                    const double xv = (sv >= 0)
                        ? x[((size_t)b * R + sv) * C + c]
                        : hist[((size_t)s * H + (size_t)(-sv - 1)) * C + c];
                    z += w[(size_t)c * W + tap] * xv;
                }
                z += w[(size_t)c * W + H] * x[((size_t)b * R + row) * C + c];
                if (bias)
                    z += bias[c];
                if (act == 1)
                    z = z / (1.0 + exp(-z)); /* SiLU */
                y[((size_t)b * R + row) * C + c] = z;
            }
        }
    }
    return err;
}

/* x <- x / sqrt(sum x^2 + 1e-6) */
static void l2norm(double *x, int D)
{
    double ss = 0.0;
    for (int c = 0; c < D; c++)
        ss += x[c] * x[c];
#if ORA_MUTATION == 8
    const double inv = 1.0 / (sqrt(ss) + 1e-6); /* planted: floor outside the root */
#else
    const double inv = 1.0 / sqrt(ss + 1e-6);
#endif
    for (int c = 0; c < D; c++)
        x[c] *= inv;
}

/* One gated-delta update of a d x d state, then the readout.
 *   St = a * Sp                      (decay)
 *   u  = b * (v - St k)              (delta correction against the decayed state)
 *   S  = St + u k^T                  (outer-product write)
 *   o  = S q                         (readout after the update; q may be NULL)
 * Sp and S may be the same buffer. */
static void gdn_update(double *S, const double *Sp, double a, double b,
                       const double *k, const double *v, const double *q,
                       double *u, double *o, int D)
{
    for (size_t e = 0; e < (size_t)D * D; e++)
#if ORA_MUTATION == 2
        S[e] = Sp[e]; /* planted: decay dropped */
#else
        S[e] = a * Sp[e];
#endif
    for (int r = 0; r < D; r++) {
        double pred = 0.0;
        for (int c = 0; c < D; c++)
#if ORA_MUTATION == 4
            pred += S[(size_t)c * D + r] * k[c]; /* planted: transposed state */
#else
            pred += S[(size_t)r * D + c] * k[c];
#endif
#if ORA_MUTATION == 3
        u[r] = b * (v[r] + pred); /* planted: sign of the correction */
#else
        u[r] = b * (v[r] - pred);
#endif
    }
    for (int r = 0; r < D; r++)
        for (int c = 0; c < D; c++)
            S[(size_t)r * D + c] += u[r] * k[c];
    if (q)
        for (int r = 0; r < D; r++) {
            double acc = 0.0;
            for (int c = 0; c < D; c++)
                acc += S[(size_t)r * D + c] * q[c];
            o[r] = acc;
        }
}

/* ------------------------------------------------------------------------- */
/* Tree verify: every node's output, each node from its parent's state.       */
/* ------------------------------------------------------------------------- */
int ora_verify(int B, int N, int R, int shared, const int32_t *parent,
               const int32_t *node_row, const int32_t *status, const double *q,
               const double *k, const double *v, const double *alpha,
               const double *beta, const double *pool, int P,
               const int32_t *state_idx, int Hqk, int Hv, int D, int norm,
               double *out, double *states, double *u_out)
{
    int err = 0;
    char *ok = (char *)calloc((size_t)B, 1);
    for (int b = 0; b < B; b++) {
        const int t = shared ? 0 : b;
        if (status[t])
            continue;
        if (state_idx[b] < 0 || state_idx[b] >= P) {
            err |= EV_STATE;
            continue;
        }
        ok[b] = 1;
    }
#pragma omp parallel for schedule(dynamic)
    for (long bh = 0; bh < (long)B * Hv; bh++) {
        const int b = (int)(bh / Hv), h = (int)(bh % Hv);
        if (!ok[b])
            continue;
        const int t = shared ? 0 : b;
        const int g = (int)(((long)h * Hqk) / Hv);
        const size_t DD = (size_t)D * D;
        double *S = (double *)malloc(sizeof(double) * DD * N);
        double *kv = (double *)malloc(sizeof(double) * D);
        double *qv = (double *)malloc(sizeof(double) * D);
        double *u = (double *)malloc(sizeof(double) * D);
        double *o = (double *)malloc(sizeof(double) * D);
        const double *S0 = pool + ((size_t)state_idx[b] * Hv + h) * DD;
        for (int i = 0; i < N; i++) {
            const int row = node_row[(size_t)t * N + i];
#if ORA_MUTATION == 1
            const int p = i - 1; /* planted: previous packed node as parent */
#else
            const int p = parent[(size_t)t * N + i];
#endif
            const double *Sp = (p < 0) ? S0 : S + (size_t)p * DD;
            const size_t qk_off = (((size_t)b * R + row) * Hqk + g) * D;
            const size_t v_off = (((size_t)b * R + row) * Hv + h) * D;
            const size_t gate = ((size_t)b * R + row) * Hv + h;
            memcpy(kv, k + qk_off, sizeof(double) * D);
            memcpy(qv, q + qk_off, sizeof(double) * D);
            if (norm) {
                l2norm(kv, D);
                l2norm(qv, D);
            }
            gdn_update(S + (size_t)i * DD, Sp, alpha[gate], beta[gate], kv,
                       v + v_off, qv, u, o, D);
            memcpy(out + v_off, o, sizeof(double) * D);
            if (u_out) { /* the node's delta correction u_i (Bole review, Lemma 2) */
#if ORA_MUTATION == 10
                for (int r = 0; r < D; r++) /* planted: u before the write strength */
                    u_out[v_off + r] = u[r] / beta[gate];
#else
                memcpy(u_out + v_off, u, sizeof(double) * D);
#endif
            }
            if (states)
                memcpy(states + (((size_t)b * N + i) * Hv + h) * DD,
                       S + (size_t)i * DD, sizeof(double) * DD);
        }
        free(S);
        free(kv);
        free(qv);
        free(u);
        free(o);
    }
    free(ok);
    return err;
}

/* ------------------------------------------------------------------------- */
/* Commit: replay the accepted path from the committed state, in place, and   */
/* publish the matching conv history.                                         */
/* ------------------------------------------------------------------------- */
int ora_commit(int B, int N, int R, int shared, const int32_t *parent,
               const int32_t *node_row, const int32_t *status,
               const int32_t *path, const int32_t *path_len, int Lmax,
               const double *k, const double *v, const double *alpha,
               const double *beta, double *pool, int P,
               const int32_t *state_idx, int Hqk, int Hv, int D, int norm,
               const double *x, double *hist, int C, int W)
{
    int err = 0;
    char *ok = (char *)calloc((size_t)B, 1);
    for (int b = 0; b < B; b++) {
        const int t = shared ? 0 : b;
        if (status[t])
            continue;
        int bad = 0;
        const int s = state_idx[b];
        if (s < 0 || s >= P) {
            bad |= EV_STATE;
        } else {
            for (int b2 = 0; b2 < B; b2++)
                if (b2 != b && state_idx[b2] == s)
                    bad |= EV_STATE;
        }
        const int L = path_len[b];
        if (L < 0 || L > Lmax) {
            bad |= EV_PATH;
        } else {
            for (int j = 0; j < L; j++) {
                const int nd = path[(size_t)b * Lmax + j];
                if (nd < 0 || nd >= N) {
                    bad |= EV_PATH;
                    break;
                }
                const int want = (j == 0) ? -1 : path[(size_t)b * Lmax + j - 1];
                if (parent[(size_t)t * N + nd] != want) {
                    bad |= EV_PATH;
                    break;
                }
            }
        }
        err |= bad;
        ok[b] = (bad == 0);
    }
#pragma omp parallel for schedule(dynamic)
    for (long bh = 0; bh < (long)B * Hv; bh++) {
        const int b = (int)(bh / Hv), h = (int)(bh % Hv);
        if (!ok[b])
            continue;
        const int t = shared ? 0 : b;
        const int g = (int)(((long)h * Hqk) / Hv);
        const size_t DD = (size_t)D * D;
        double *S = pool + ((size_t)state_idx[b] * Hv + h) * DD;
        double *kv = (double *)malloc(sizeof(double) * D);
        double *u = (double *)malloc(sizeof(double) * D);
        const int L = path_len[b];
#if ORA_MUTATION == 7
        const int Lrun = (L > 0) ? L - 1 : 0; /* planted: frontier step dropped */
#else
        const int Lrun = L;
#endif
        for (int j = 0; j < Lrun; j++) {
            const int nd = path[(size_t)b * Lmax + j];
            const int row = node_row[(size_t)t * N + nd];
            const size_t qk_off = (((size_t)b * R + row) * Hqk + g) * D;
            const size_t v_off = (((size_t)b * R + row) * Hv + h) * D;
            const size_t gate = ((size_t)b * R + row) * Hv + h;
            memcpy(kv, k + qk_off, sizeof(double) * D);
            if (norm)
                l2norm(kv, D);
            gdn_update(S, S, alpha[gate], beta[gate], kv, v + v_off, NULL, u,
                       NULL, D);
        }
        free(kv);
        free(u);
    }
    /* conv history: last W-1 entries of old history followed by the accepted
     * rows' conv inputs */
    const int H = W - 1;
    if (x && hist && H > 0) {
        double *seq = (double *)malloc(sizeof(double) * (size_t)(H + Lmax));
        for (int b = 0; b < B; b++) {
            if (!ok[b])
                continue;
            const int t = shared ? 0 : b;
            const int s = state_idx[b];
            const int L = path_len[b];
            for (int c = 0; c < C; c++) {
                int n = 0;
                for (int m = 0; m < H; m++)
                    seq[n++] = hist[((size_t)s * H + m) * C + c];
                for (int j = 0; j < L; j++) {
                    const int row = node_row[(size_t)t * N + path[(size_t)b * Lmax + j]];
                    seq[n++] = x[((size_t)b * R + row) * C + c];
                }
                for (int m = 0; m < H; m++)
#if ORA_MUTATION == 9
                    hist[((size_t)s * H + m) * C + c] = seq[n - 1 - m]; /* planted: newest first */
#else
                    hist[((size_t)s * H + m) * C + c] = seq[n - H + m];
#endif
            }
        }
        free(seq);
    }
    free(ok);
    return err;
}
