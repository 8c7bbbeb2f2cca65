/*
 * fp64 CPU oracle for the key-only-gated linear-attention (GLA) forward pass
 * of GTR (Gated Token Recurrence).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * What it computes is the plain definition, one token at a time, in double
 * precision, with no chunking, blocking or reordering:
 *
 *   Source: x-techcon article on GTR ("视觉AI看得越细，还能又快又准吗？..."),
 *   section 架构 (Architecture):
 *     - the layer keeps a state matrix S (d_k x d_v);
 *     - at each new scan position it FIRST keeps part of the old state,
 *       scaled per key dimension by a gate alpha_t that is generated from the
 *       input, and THEN adds the current key/value outer product;
 *     - the gate acts on key dimensions only; the value-side decay is 1;
 *     - the query of the current position reads its output from the UPDATED
 *       state.
 *   The article's displayed update formula did not survive extraction; the
 *   reading used here is the one that these sentences fix:
 *       S_t = diag(alpha_t) S_{t-1} + k_t^T v_t ,   o_t = q_t S_t ,  S_{-1} = 0
 *   with alpha_t = exp(log_gate_t) taken element-wise over the d_k key dims.
 *   No softmax and no q.k scale are applied (none is described).
 *
 *   Same article, section 架构: consecutive layers scan the patch grid
 *   left-to-right, right-to-left, top-to-bottom and bottom-to-top, and each
 *   layer hands on its outputs in grid arrangement.  Reading used here
 *   (the article gives no index formula):
 *     direction 0, L->R : row-major order, rows top to bottom;
 *     direction 1, R->L : the L->R sequence reversed (starts bottom-right);
 *     direction 2, T->B : column-major order, columns left to right;
 *     direction 3, B->T : the T->B sequence reversed.
 *   "Restored" means each output is written back at its own grid position.
 *
 * Layout: q, k, log_gate are [B][H][grid_h][grid_w][d_k]; v and out are
 * [B][H][grid_h][grid_w][d_v]; all dense row-major doubles.  Optional s0
 * ([B][H][d_k][d_v], NULL means zero) is the state before the first token;
 * optional s_final (same shape, NULL means not wanted) receives the state
 * after the last token.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Grid index (row-major r*grid_w + c) of scan position t; -1 if out of range. */
long gla_oracle_scan_index(long t, long grid_h, long grid_w, int direction)
{
    long n_tok = grid_h * grid_w;
    if (t < 0 || t >= n_tok || grid_h <= 0 || grid_w <= 0) return -1;
    switch (direction) {
    case 0: return t;                                   /* L->R */
    case 1: return n_tok - 1 - t;                       /* R->L */
    case 2: {                                           /* T->B */
        long col = t / grid_h, row = t % grid_h;
        return row * grid_w + col;
    }
    case 3: {                                           /* B->T */
        long u = n_tok - 1 - t;
        long col = u / grid_h, row = u % grid_h;
        return row * grid_w + col;
    }
    default: return -1;
    }
}

/*
 * Returns the number of OpenMP threads used (>= 1), or a negative value on a
 * bad argument: -1 null pointer, -2 non-positive size, -3 bad direction,
 * -4 out of memory.  n_threads <= 0 means the OpenMP default.
 */
int gla_oracle_f64(const double *q, const double *k, const double *v,
                   const double *log_gate, double *out,
                   int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                   int direction, const double *s0, double *s_final,
                   int n_threads)
{
    if (!q || !k || !v || !log_gate || !out) return -1;
    if (B <= 0 || H <= 0 || grid_h <= 0 || grid_w <= 0 || d_k <= 0 || d_v <= 0)
        return -2;
    if (direction < 0 || direction > 3) return -3;

    const long n_tok = (long)grid_h * grid_w;
    const long n_seq = (long)B * H;
    int used = 1;
    int failed = 0;
#ifdef _OPENMP
    if (n_threads <= 0) n_threads = omp_get_max_threads();
    if (n_threads > n_seq) n_threads = (int)n_seq;
    if (n_threads < 1) n_threads = 1;
#else
    n_threads = 1;
#endif

#pragma omp parallel num_threads(n_threads)
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double *S = (double *)malloc(sizeof(double) * (size_t)d_k * d_v);
        double *alpha = (double *)malloc(sizeof(double) * (size_t)d_k);
        if (!S || !alpha) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long bh = 0; bh < n_seq; ++bh) {
            if (!S || !alpha) continue;
            const double *qs = q + bh * n_tok * d_k;
            const double *ks = k + bh * n_tok * d_k;
            const double *gs = log_gate + bh * n_tok * d_k;
            const double *vs = v + bh * n_tok * d_v;
            double *os = out + bh * n_tok * d_v;

            if (s0) memcpy(S, s0 + bh * (long)d_k * d_v, sizeof(double) * (size_t)d_k * d_v);
            else memset(S, 0, sizeof(double) * (size_t)d_k * d_v);

            for (long t = 0; t < n_tok; ++t) {
                const long n = gla_oracle_scan_index(t, grid_h, grid_w, direction);
                const double *qt = qs + n * d_k;
                const double *kt = ks + n * d_k;
                const double *gt = gs + n * d_k;
                const double *vt = vs + n * d_v;
                /* decay first (per key dimension), then write k_t^T v_t */
                for (int i = 0; i < d_k; ++i) alpha[i] = exp(gt[i]);
                for (int i = 0; i < d_k; ++i) {
                    double *row = S + (long)i * d_v;
                    for (int j = 0; j < d_v; ++j)
                        row[j] = alpha[i] * row[j] + kt[i] * vt[j];
                }
                /* read with the query from the updated state: o_t = q_t S_t */
                double *ot = os + n * d_v;
                for (int j = 0; j < d_v; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < d_k; ++i) acc += qt[i] * S[(long)i * d_v + j];
                    ot[j] = acc;
                }
            }
            if (s_final)
                memcpy(s_final + bh * (long)d_k * d_v, S, sizeof(double) * (size_t)d_k * d_v);
        }
        free(S);
        free(alpha);
    }
    if (failed) return -4;
    return used;
}

/*
 * Backward pass of the same recurrence, by the chain rule applied to it one
 * token at a time (no chunking, no identities): given dout = dL/dout and,
 * optionally, ds_final = dL/dS_final, it returns dq, dk, dv, dlog_gate and,
 * optionally, ds0 = dL/ds0.
 *
 *   forward sweep:  S_t = diag(alpha_t) S_{t-1} + k_t^T v_t,  keeping every S_{t-1};
 *                   dq_t = S_t dout_t^T                     (o_t = q_t S_t)
 *   reverse sweep:  G = ds_final (or 0);  for t = N-1 .. 0:
 *                     G      += q_t^T dout_t                 (G = dL/dS_t)
 *                     dk_t    = G v_t^T,  dv_t = k_t G       (from k_t^T v_t)
 *                     dlog_gate_t[i] = alpha_t[i] sum_j G[i,j] S_{t-1}[i,j]
 *                     G       = diag(alpha_t) G              (dL/dS_{t-1})
 *                   ds0 = G.
 *
 * Layouts as the forward pass; dq, dk, dlog_gate like q, dv like v.  Each
 * thread keeps the N states of one sequence (N * d_k * d_v doubles).  Returns
 * the thread count, or -1 null pointer, -2 bad size, -3 bad direction, -4 out
 * of memory.
 */
int gla_oracle_bwd_f64(const double *q, const double *k, const double *v,
                       const double *log_gate, const double *dout, const double *s0,
                       const double *ds_final, double *dq, double *dk, double *dv,
                       double *dlog_gate, double *ds0, int B, int H, int grid_h, int grid_w,
                       int d_k, int d_v, int direction, int n_threads)
{
    if (!q || !k || !v || !log_gate || !dout || !dq || !dk || !dv || !dlog_gate) return -1;
    if (B <= 0 || H <= 0 || grid_h <= 0 || grid_w <= 0 || d_k <= 0 || d_v <= 0)
        return -2;
    if (direction < 0 || direction > 3) return -3;

    const long n_tok = (long)grid_h * grid_w;
    const long n_seq = (long)B * H;
    const long kv = (long)d_k * d_v;
    int used = 1;
    int failed = 0;
#ifdef _OPENMP
    if (n_threads <= 0) n_threads = omp_get_max_threads();
    if (n_threads > n_seq) n_threads = (int)n_seq;
    if (n_threads < 1) n_threads = 1;
#else
    n_threads = 1;
#endif

#pragma omp parallel num_threads(n_threads)
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double *prev = (double *)malloc(sizeof(double) * (size_t)(n_tok * kv));  /* S_{t-1}, all t */
        double *S = (double *)malloc(sizeof(double) * (size_t)kv);
        double *G = (double *)malloc(sizeof(double) * (size_t)kv);
        if (!prev || !S || !G) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long bh = 0; bh < n_seq; ++bh) {
            if (!prev || !S || !G) continue;
            const double *qs = q + bh * n_tok * d_k, *ks = k + bh * n_tok * d_k;
            const double *gs = log_gate + bh * n_tok * d_k;
            const double *vs = v + bh * n_tok * d_v, *dos = dout + bh * n_tok * d_v;
            double *dqs = dq + bh * n_tok * d_k, *dks = dk + bh * n_tok * d_k;
            double *dvs = dv + bh * n_tok * d_v, *dgs = dlog_gate + bh * n_tok * d_k;

            if (s0) memcpy(S, s0 + bh * kv, sizeof(double) * (size_t)kv);
            else memset(S, 0, sizeof(double) * (size_t)kv);
            for (long t = 0; t < n_tok; ++t) {
                const long n = gla_oracle_scan_index(t, grid_h, grid_w, direction);
                memcpy(prev + t * kv, S, sizeof(double) * (size_t)kv);
                for (int i = 0; i < d_k; ++i) {
                    const double a = exp(gs[n * d_k + i]);
                    for (int j = 0; j < d_v; ++j)
                        S[(long)i * d_v + j] = a * S[(long)i * d_v + j] + ks[n * d_k + i] * vs[n * d_v + j];
                }
                for (int i = 0; i < d_k; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < d_v; ++j) acc += S[(long)i * d_v + j] * dos[n * d_v + j];
                    dqs[n * d_k + i] = acc;
                }
            }

            if (ds_final) memcpy(G, ds_final + bh * kv, sizeof(double) * (size_t)kv);
            else memset(G, 0, sizeof(double) * (size_t)kv);
            for (long t = n_tok - 1; t >= 0; --t) {
                const long n = gla_oracle_scan_index(t, grid_h, grid_w, direction);
                const double *Sp = prev + t * kv;
                for (int i = 0; i < d_k; ++i)
                    for (int j = 0; j < d_v; ++j)
                        G[(long)i * d_v + j] += qs[n * d_k + i] * dos[n * d_v + j];
                for (int i = 0; i < d_k; ++i) {
                    double acc = 0.0, da = 0.0;
                    for (int j = 0; j < d_v; ++j) {
                        acc += G[(long)i * d_v + j] * vs[n * d_v + j];
                        da += G[(long)i * d_v + j] * Sp[(long)i * d_v + j];
                    }
                    dks[n * d_k + i] = acc;
                    dgs[n * d_k + i] = exp(gs[n * d_k + i]) * da;
                }
                for (int j = 0; j < d_v; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < d_k; ++i) acc += ks[n * d_k + i] * G[(long)i * d_v + j];
                    dvs[n * d_v + j] = acc;
                }
                for (int i = 0; i < d_k; ++i) {
                    const double a = exp(gs[n * d_k + i]);
                    for (int j = 0; j < d_v; ++j) G[(long)i * d_v + j] *= a;
                }
            }
            if (ds0) memcpy(ds0 + bh * kv, G, sizeof(double) * (size_t)kv);
        }
        free(prev);
        free(S);
        free(G);
    }
    if (failed) return -4;
    return used;
}
