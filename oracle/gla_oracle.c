/*
 * gla_oracle.c -- plain, slow, fp64 CPU oracle for the DiG token mixer:
 * the Gated Linear Attention (GLA) forward scanned in one SREM direction and
 * its reverse-mode derivative,
 * the 3x3 depthwise conv of the SREM block with its direction remap, and
 * the adaLN modulation that feeds the block.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
 * Python binding) may include, link, load or call this file.  Only the tests,
 * the smoke check and the CPU-baseline leg of the benchmark use it.  It shares
 * no code, header, table or constant with the GPU path.
 *
 * Every value is computed in IEEE fp64, token by token, with no chunking,
 * blocking, factorisation or reordering beyond the plain definitions below.
 * Inputs arrive as fp64 arrays (bf16 and fp32 inputs convert to fp64 exactly).
 *
 * Sources (web pages; cited by title and section):
 *  [DiG-notes]  "DiG: Scalable and Efficient Diffusion Models with Gated Linear
 *               Attention", Paper-Notes (CVPR 2025): sections 关键设计 / SREM
 *               (scan-direction control, transpose + flip, 3x3 DWConv2d with
 *               identity init), 关键设计 / DiG Block设计 (block order: adaLN ->
 *               GLA -> adaLN -> FFN -> reshape to 2D -> DWConv2d -> direction
 *               change), 关键设计 / 硬件友好的效率设计 (chunk-wise GLA).
 *  [GLA-issue]  "DiG: Scalable and Efficient Diffusion Models with Gated Linear
 *               Attention", diffusers issue #20: description bullets (per-head
 *               head_dim x head_dim recurrent state; data-dependent forget gate
 *               on that state) and the draft recurrence (gate applied over the
 *               key rows of the state, current token written before the read,
 *               readout q . state, zero initial state).  Its feature map, its
 *               sigmoid(q*k) gate and its normaliser are NOT part of the
 *               operator computed here.
 *  [DiT-notes]  "Scalable Diffusion Models with Transformers" notes, section
 *               3.2 DiT Block 设计 (adaLN: scale and shift regressed from the
 *               conditioning; adaLN-Zero identity-at-init convention).
 *  [ZigMa-notes] "ZigMa: A DiT-style Zigzag Mamba Diffusion Model",
 *               Paper-Notes (ECCV 2024), 关键设计 / 异构逐层扫描 (arrange ->
 *               scan -> arrange back, one scan order per layer).
 *
 * Readings where the pages leave a step open are stated at each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Scan directions, in the order [DiG-notes] SREM lists them. */
enum { OR_L2R = 0, OR_R2L = 1, OR_T2B = 2, OR_B2T = 3 };

/*
 * Canonical grid index visited at scan position p.
 *
 * The canonical order is the row-major order of the (gh x gw) token grid.
 * [DiG-notes] SREM names four scans (left->right, right->left, top->bottom,
 * bottom->top) obtained with a transpose of the 2D token matrix and a flip of
 * the sequence.  Reading: the flip reverses the whole sequence, so
 *   left->right : row-major order;
 *   right->left : row-major order reversed;
 *   top->bottom : column-major order (row-major order of the transpose);
 *   bottom->top : column-major order reversed.
 * Returns -1 for an unknown direction.
 */
int64_t oracle_scan_index(int dir, int64_t gh, int64_t gw, int64_t p)
{
    const int64_t T = gh * gw;
    int64_t r, c, s;
    if (p < 0 || p >= T) return -1;
    switch (dir) {
    case OR_L2R:
        return p;
    case OR_R2L:
        return T - 1 - p;
    case OR_T2B:
        c = p / gh;          /* column being walked */
        r = p - c * gh;      /* row inside that column */
        return r * gw + c;
    case OR_B2T:
        s = T - 1 - p;
        c = s / gh;
        r = s - c * gh;
        return r * gw + c;
    default:
        return -1;
    }
}

/* Fill perm[p] = canonical index of scan position p, for p in [0, T). */
int oracle_scan_perm(int dir, int64_t gh, int64_t gw, int64_t *perm)
{
    const int64_t T = gh * gw;
    for (int64_t p = 0; p < T; ++p) {
        perm[p] = oracle_scan_index(dir, gh, gw, p);
        if (perm[p] < 0) return -1;
    }
    return 0;
}

/*
 * GLA forward, token by token, per (batch, head).
 *
 * Layouts (contiguous, fp64):
 *   q, k, log_alpha : [B, T, H, dk]   canonical token order
 *   v               : [B, T, H, dv]   canonical token order
 *   s0 (nullable)   : [B, H, dk, dv]  initial state; NULL means zero
 *   o               : [B, T, H, dv]   written in SCAN order (position p)
 *   s_final (nullable): [B, H, dk, dv] state after the last scanned token
 *
 * For each (b, h), with S := s0[b, h] (dk x dv), and for p = 0 .. T-1 with
 * n = canonical index at scan position p:
 *   a_i      = exp(log_alpha[b, n, h, i])                (forget gate)
 *   S_ij    := a_i * S_ij + k[b, n, h, i] * v[b, n, h, j] (decay, then write)
 *   o[b,p,h,j] = sum_i q[b, n, h, i] * S_ij               (inclusive readout)
 * This is the recurrence of [GLA-issue] (state of head_dim x head_dim, gate
 * over the key rows, write before read, q . state readout, zero start) with
 * the per-key-channel gate supplied as an input in log space, and without the
 * draft's feature map and normaliser.  [DiG-notes] 硬件友好的效率设计 states
 * that the chunk-wise form computes the same thing, so no chunks appear here.
 *
 * nthreads <= 0 means "let OpenMP decide".  Returns 0, or -1 on bad args.
 */
static int gla_fwd_perm(const double *q, const double *k, const double *v,
                        const double *log_alpha, int64_t B, int64_t T, int64_t H,
                        int64_t dk, int64_t dv, int64_t *perm,
                        const double *s0, double *o, double *s_final, int nthreads);

int oracle_gla_fwd(const double *q, const double *k, const double *v,
                   const double *log_alpha, int64_t B, int64_t T, int64_t H,
                   int64_t dk, int64_t dv, int64_t gh, int64_t gw, int dir,
                   const double *s0, double *o, double *s_final, int nthreads)
{
    if (B <= 0 || T <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (gh <= 0 || gw <= 0 || gh * gw != T) return -1;
    if (dir < OR_L2R || dir > OR_B2T) return -1;

    int64_t *perm = (int64_t *)malloc((size_t)T * sizeof(int64_t));
    if (!perm) return -1;
    oracle_scan_perm(dir, gh, gw, perm);
    return gla_fwd_perm(q, k, v, log_alpha, B, T, H, dk, dv, perm, s0, o, s_final, nthreads);
}

/* A scan order given as a table: order[p] = canonical index of the token at
 * scan position p, a permutation of 0..T-1 (ZigMa notes, 关键设计 / Zigzag
 * 扫描方案: any space-filling order; DiG notes: the four SREM orders are the
 * special cases).  Same recurrence and outputs as oracle_gla_fwd. */
static int copy_order(const int64_t *order, int64_t T, int64_t **perm)
{
    char *seen = (char *)calloc((size_t)T, 1);
    *perm = (int64_t *)malloc((size_t)T * sizeof(int64_t));
    if (!seen || !*perm) { free(seen); free(*perm); return -1; }
    for (int64_t p = 0; p < T; ++p) {
        const int64_t n = order[p];
        if (n < 0 || n >= T || seen[n]) { free(seen); free(*perm); return -1; }
        seen[n] = 1;
        (*perm)[p] = n;
    }
    free(seen);
    return 0;
}

int oracle_gla_fwd_order(const double *q, const double *k, const double *v,
                         const double *log_alpha, int64_t B, int64_t T, int64_t H,
                         int64_t dk, int64_t dv, const int64_t *order,
                         const double *s0, double *o, double *s_final, int nthreads)
{
    if (B <= 0 || T <= 0 || H <= 0 || dk <= 0 || dv <= 0 || !order) return -1;
    int64_t *perm;
    if (copy_order(order, T, &perm)) return -1;
    return gla_fwd_perm(q, k, v, log_alpha, B, T, H, dk, dv, perm, s0, o, s_final, nthreads);
}

/* Takes ownership of perm (freed on return). */
static int gla_fwd_perm(const double *q, const double *k, const double *v,
                        const double *log_alpha, int64_t B, int64_t T, int64_t H,
                        int64_t dk, int64_t dv, int64_t *perm,
                        const double *s0, double *o, double *s_final, int nthreads)
{

    const int64_t units = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t u = 0; u < units; ++u) {
        const int64_t b = u / H, h = u % H;
        double *S = (double *)malloc((size_t)(dk * dv) * sizeof(double));
        double *a = (double *)malloc((size_t)dk * sizeof(double));
        if (!S || !a) {
            failed = 1;
            free(S);
            free(a);
            continue;
        }
        if (s0)
            memcpy(S, s0 + (b * H + h) * dk * dv, (size_t)(dk * dv) * sizeof(double));
        else
            memset(S, 0, (size_t)(dk * dv) * sizeof(double));

        for (int64_t p = 0; p < T; ++p) {
            const int64_t n = perm[p];
            const double *qn = q + ((b * T + n) * H + h) * dk;
            const double *kn = k + ((b * T + n) * H + h) * dk;
            const double *gn = log_alpha + ((b * T + n) * H + h) * dk;
            const double *vn = v + ((b * T + n) * H + h) * dv;
            double *op = o + ((b * T + p) * H + h) * dv;

            for (int64_t i = 0; i < dk; ++i) a[i] = exp(gn[i]);
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j)
                    S[i * dv + j] = a[i] * S[i * dv + j] + kn[i] * vn[j];
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < dk; ++i) acc += qn[i] * S[i * dv + j];
                op[j] = acc;
            }
        }
        if (s_final)
            memcpy(s_final + (b * H + h) * dk * dv, S, (size_t)(dk * dv) * sizeof(double));
        free(S);
        free(a);
    }
    free(perm);
    return failed ? -1 : 0;
}

/*
 * GLA backward, token by token, per (batch, head): the gradients of
 *   L = sum_{p,j} do[b,p,h,j] * o[b,p,h,j] + sum_{i,j} ds_final[b,h,i,j] * S_final[i,j]
 * with respect to q, k, v, log_alpha and s0, for the forward above.
 *
 * Layouts as in oracle_gla_fwd; do is in SCAN order like o, ds_final is
 * [B, H, dk, dv] (NULL means zero); dq, dk_out, dlog_alpha are [B, T, H, dk]
 * and dv_out [B, T, H, dv] in canonical token order; ds0 (nullable) is
 * [B, H, dk, dv].
 *
 * Reading: the pages train the model with this operator but print no
 * backward; this is the plain reverse-mode derivative of the recurrence.
 * With S_p the state after scan position p (n its canonical token, a its
 * gate exp(log_alpha)) and G_p = dL/dS_p,
 *   G_{T-1} = ds_final + q^T do_{T-1},  G_p = q_n^T do_p + diag(a_{p+1}) G_{p+1}
 *   dq_n[i]        = sum_j S_p[i,j] do_p[j]
 *   dk_n[i]        = sum_j G_p[i,j] v_n[j]
 *   dv_n[j]        = sum_i k_n[i] G_p[i,j]
 *   dlog_alpha_n[i] = a_n[i] * sum_j G_p[i,j] S_{p-1}[i,j]
 *   ds0            = diag(a_0) G_0
 * The states S_p are those of the forward, recomputed in blocks of about
 * sqrt(T) positions from states stored at block starts (the same operations
 * in the same order, so the same values) to keep memory at O(sqrt(T) d^2).
 */
static int gla_bwd_perm(const double *q, const double *k, const double *v,
                        const double *log_alpha, int64_t B, int64_t T, int64_t H,
                        int64_t dk, int64_t dv, int64_t *perm,
                        const double *s0, const double *do_scan, const double *ds_final,
                        double *dq, double *dk_out, double *dv_out, double *dlog_alpha,
                        double *ds0, int nthreads);

int oracle_gla_bwd(const double *q, const double *k, const double *v,
                   const double *log_alpha, int64_t B, int64_t T, int64_t H,
                   int64_t dk, int64_t dv, int64_t gh, int64_t gw, int dir,
                   const double *s0, const double *do_scan, const double *ds_final,
                   double *dq, double *dk_out, double *dv_out, double *dlog_alpha,
                   double *ds0, int nthreads)
{
    if (B <= 0 || T <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (gh <= 0 || gw <= 0 || gh * gw != T) return -1;
    if (dir < OR_L2R || dir > OR_B2T) return -1;

    int64_t *perm = (int64_t *)malloc((size_t)T * sizeof(int64_t));
    if (!perm) return -1;
    oracle_scan_perm(dir, gh, gw, perm);
    return gla_bwd_perm(q, k, v, log_alpha, B, T, H, dk, dv, perm, s0, do_scan, ds_final, dq, dk_out,
                        dv_out, dlog_alpha, ds0, nthreads);
}

/* The backward over a scan order given as a table (a permutation, as for
 * oracle_gla_fwd_order); do_scan in that order. */
int oracle_gla_bwd_order(const double *q, const double *k, const double *v,
                         const double *log_alpha, int64_t B, int64_t T, int64_t H,
                         int64_t dk, int64_t dv, const int64_t *order,
                         const double *s0, const double *do_scan, const double *ds_final,
                         double *dq, double *dk_out, double *dv_out, double *dlog_alpha,
                         double *ds0, int nthreads)
{
    if (B <= 0 || T <= 0 || H <= 0 || dk <= 0 || dv <= 0 || !order) return -1;
    int64_t *perm;
    if (copy_order(order, T, &perm)) return -1;
    return gla_bwd_perm(q, k, v, log_alpha, B, T, H, dk, dv, perm, s0, do_scan, ds_final, dq, dk_out,
                        dv_out, dlog_alpha, ds0, nthreads);
}

/* Takes ownership of perm (freed on return). */
static int gla_bwd_perm(const double *q, const double *k, const double *v,
                        const double *log_alpha, int64_t B, int64_t T, int64_t H,
                        int64_t dk, int64_t dv, int64_t *perm,
                        const double *s0, const double *do_scan, const double *ds_final,
                        double *dq, double *dk_out, double *dv_out, double *dlog_alpha,
                        double *ds0, int nthreads)
{

    int64_t K = 1;
    while (K * K < T) ++K;                 /* block length ~ sqrt(T) */
    const int64_t nblk = (T + K - 1) / K;
    const int64_t dd = dk * dv;
    const int64_t units = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t u = 0; u < units; ++u) {
        const int64_t b = u / H, h = u % H;
        double *start = (double *)malloc((size_t)(nblk * dd) * sizeof(double)); /* state before each block */
        double *blk = (double *)malloc((size_t)(K * dd) * sizeof(double));      /* states after each position */
        double *S = (double *)malloc((size_t)dd * sizeof(double));
        double *G = (double *)malloc((size_t)dd * sizeof(double));
        double *a = (double *)malloc((size_t)dk * sizeof(double));
        if (!start || !blk || !S || !G || !a) {
            failed = 1;
            free(start); free(blk); free(S); free(G); free(a);
            continue;
        }
#define TOK(arr, n, d) ((arr) + ((b * T + (n)) * H + h) * (d))
        /* forward: the state entering every block */
        if (s0)
            memcpy(S, s0 + (b * H + h) * dd, (size_t)dd * sizeof(double));
        else
            memset(S, 0, (size_t)dd * sizeof(double));
        for (int64_t p = 0; p < T; ++p) {
            if (p % K == 0) memcpy(start + (p / K) * dd, S, (size_t)dd * sizeof(double));
            const int64_t n = perm[p];
            const double *kn = TOK(k, n, dk), *gn = TOK(log_alpha, n, dk), *vn = TOK(v, n, dv);
            for (int64_t i = 0; i < dk; ++i) a[i] = exp(gn[i]);
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j)
                    S[i * dv + j] = a[i] * S[i * dv + j] + kn[i] * vn[j];
        }
        /* backward, block by block from the end */
        if (ds_final)
            memcpy(G, ds_final + (b * H + h) * dd, (size_t)dd * sizeof(double));
        else
            memset(G, 0, (size_t)dd * sizeof(double));
        for (int64_t c = nblk - 1; c >= 0; --c) {
            const int64_t p0 = c * K, p1 = (p0 + K < T) ? p0 + K : T;
            memcpy(S, start + c * dd, (size_t)dd * sizeof(double));
            for (int64_t p = p0; p < p1; ++p) {      /* recompute S_p, p in the block */
                const int64_t n = perm[p];
                const double *kn = TOK(k, n, dk), *gn = TOK(log_alpha, n, dk), *vn = TOK(v, n, dv);
                for (int64_t i = 0; i < dk; ++i) a[i] = exp(gn[i]);
                for (int64_t i = 0; i < dk; ++i)
                    for (int64_t j = 0; j < dv; ++j)
                        S[i * dv + j] = a[i] * S[i * dv + j] + kn[i] * vn[j];
                memcpy(blk + (p - p0) * dd, S, (size_t)dd * sizeof(double));
            }
            for (int64_t p = p1 - 1; p >= p0; --p) {
                const int64_t n = perm[p];
                const double *qn = TOK(q, n, dk), *kn = TOK(k, n, dk), *gn = TOK(log_alpha, n, dk);
                const double *vn = TOK(v, n, dv);
                const double *dop = do_scan + ((b * T + p) * H + h) * dv;
                const double *Sp = blk + (p - p0) * dd;
                const double *Sprev = (p > p0) ? blk + (p - 1 - p0) * dd : start + c * dd;
                for (int64_t i = 0; i < dk; ++i)
                    for (int64_t j = 0; j < dv; ++j) G[i * dv + j] += qn[i] * dop[j];
                double *dqn = TOK(dq, n, dk), *dkn = TOK(dk_out, n, dk), *dgn = TOK(dlog_alpha, n, dk);
                double *dvn = TOK(dv_out, n, dv);
                for (int64_t i = 0; i < dk; ++i) {
                    double sq = 0.0, sk = 0.0, sg = 0.0;
                    for (int64_t j = 0; j < dv; ++j) {
                        sq += Sp[i * dv + j] * dop[j];
                        sk += G[i * dv + j] * vn[j];
                        sg += G[i * dv + j] * Sprev[i * dv + j];
                    }
                    dqn[i] = sq;
                    dkn[i] = sk;
                    dgn[i] = exp(gn[i]) * sg;
                }
                for (int64_t j = 0; j < dv; ++j) {
                    double sv = 0.0;
                    for (int64_t i = 0; i < dk; ++i) sv += kn[i] * G[i * dv + j];
                    dvn[j] = sv;
                }
                for (int64_t i = 0; i < dk; ++i) {
                    const double ai = exp(gn[i]);
                    for (int64_t j = 0; j < dv; ++j) G[i * dv + j] *= ai;
                }
            }
        }
        if (ds0) memcpy(ds0 + (b * H + h) * dd, G, (size_t)dd * sizeof(double));
#undef TOK
        free(start); free(blk); free(S); free(G); free(a);
    }
    free(perm);
    return failed ? -1 : 0;
}

/*
 * SREM 3x3 depthwise conv with the direction remap to canonical order.
 *
 *   x : [B, T, C]  the mixer output in SCAN order of direction `dir`
 *   w : [C, 3, 3]  one 3x3 kernel per channel
 *   y : [B, T, C]  CANONICAL (row-major grid) order
 *
 * [DiG-notes] DiG Block设计 step (4) reshapes the sequence to 2D and applies a
 * DWConv2d; step (5) changes the scan direction.  Readings: the reshape is of
 * the scan-ordered sequence into its scan frame, (R, Q) = (gh, gw) for the
 * row scans and (gw, gh) for the column scans, X[r][c] = x[r*Q + c]; the conv
 * is a cross-correlation with zero padding 1, stride 1 and no bias
 *   Y[r][c] = sum_{a,e in 0..2} w[ch][a][e] * X[r+a-1][c+e-1];
 * the direction change is the exact permutation back to canonical order,
 * y[canon(p)] = Y[p / Q][p % Q], the arrange-back step of [ZigMa-notes].
 */
int oracle_srem_dwconv(const double *x, int64_t B, int64_t T, int64_t C,
                       const double *w, int64_t gh, int64_t gw, int dir,
                       double *y, int nthreads)
{
    if (B <= 0 || T <= 0 || C <= 0 || gh <= 0 || gw <= 0 || gh * gw != T) return -1;
    if (dir < OR_L2R || dir > OR_B2T) return -1;
    const int64_t R = (dir == OR_L2R || dir == OR_R2L) ? gh : gw;
    const int64_t Q = (dir == OR_L2R || dir == OR_R2L) ? gw : gh;
    int64_t *perm = (int64_t *)malloc((size_t)T * sizeof(int64_t));
    if (!perm) return -1;
    oracle_scan_perm(dir, gh, gw, perm);
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t bp = 0; bp < B * T; ++bp) {
        const int64_t b = bp / T, p = bp % T;
        const int64_t r = p / Q, c = p % Q;
        double *yo = y + (b * T + perm[p]) * C;
        for (int64_t ch = 0; ch < C; ++ch) {
            double acc = 0.0;
            for (int a = 0; a < 3; ++a) {
                const int64_t rr = r + a - 1;
                if (rr < 0 || rr >= R) continue;
                for (int e = 0; e < 3; ++e) {
                    const int64_t cc = c + e - 1;
                    if (cc < 0 || cc >= Q) continue;
                    acc += w[ch * 9 + a * 3 + e] * x[(b * T + rr * Q + cc) * C + ch];
                }
            }
            yo[ch] = acc;
        }
    }
    free(perm);
    return 0;
}

/*
 * Exact permutation between two scan orders of the same grid:
 * x is in scan order `from`, y in scan order `to`; the token at canonical
 * index n moves from position inv_from(n) to position inv_to(n).
 * ([DiG-notes] SREM transpose + flip; [ZigMa-notes] arrange / arrange back.)
 */
int oracle_remap(const double *x, int64_t B, int64_t C, int64_t gh, int64_t gw,
                 int from, int to, double *y)
{
    const int64_t T = gh * gw;
    if (B <= 0 || C <= 0 || gh <= 0 || gw <= 0) return -1;
    if (from < OR_L2R || from > OR_B2T || to < OR_L2R || to > OR_B2T) return -1;
    int64_t *pf = (int64_t *)malloc((size_t)T * sizeof(int64_t));
    int64_t *inv = (int64_t *)malloc((size_t)T * sizeof(int64_t));
    if (!pf || !inv) {
        free(pf);
        free(inv);
        return -1;
    }
    oracle_scan_perm(from, gh, gw, pf);
    for (int64_t p = 0; p < T; ++p) inv[pf[p]] = p;   /* canonical -> from-position */
    for (int64_t b = 0; b < B; ++b)
        for (int64_t p2 = 0; p2 < T; ++p2) {
            const int64_t n = oracle_scan_index(to, gh, gw, p2);
            memcpy(y + (b * T + p2) * C, x + (b * T + inv[n]) * C, (size_t)C * sizeof(double));
        }
    free(pf);
    free(inv);
    return 0;
}

/*
 * adaLN modulation of each token, over its C channels:
 *   y = ((x - mean) / sqrt(var + eps) * (1 + scale) + shift) * out_scale
 * with the population variance.  [DiG-notes] DiG Block设计 step (2) (adaLN
 * before the GLA); [DiT-notes] 3.2 (adaLN regresses the norm's scale and
 * shift; adaLN-Zero starts from the identity, hence the 1 + scale form).
 * out_scale is the fixed 1/sqrt(head_dim) pre-scaling of the synthetic q/k/v.
 */
int oracle_adaln_modulate(const double *x, int64_t N, int64_t C,
                          const double *scale, const double *shift, double eps,
                          double out_scale, double *y, int nthreads)
{
    if (N <= 0 || C <= 0) return -1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t n = 0; n < N; ++n) {
        const double *xr = x + n * C;
        double *yr = y + n * C;
        double mean = 0.0, var = 0.0;
        for (int64_t c = 0; c < C; ++c) mean += xr[c];
        mean /= (double)C;
        for (int64_t c = 0; c < C; ++c) var += (xr[c] - mean) * (xr[c] - mean);
        var /= (double)C;
        const double inv = 1.0 / sqrt(var + eps);
        for (int64_t c = 0; c < C; ++c)
            yr[c] = ((xr[c] - mean) * inv * (1.0 + scale[c]) + shift[c]) * out_scale;
    }
    return 0;
}

/* Number of OpenMP threads the oracle would use by default (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
