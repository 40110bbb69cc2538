/*
 * fp64 CPU oracle for exact scaled-dot-product attention, forward and backward.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU path shares no
 * code with it, and nothing in the GPU path may call it.
 *
 * What it computes is standard attention as the pages define it: "FlashAttention:
 * making attention fast by respecting the memory hierarchy" (groundtruth.day,
 * paragraph on what attention costs) describes the full N-by-N grid of scores,
 * the softmax over each row of that grid and the multiplication by the values;
 * the michaelc-yu summary of Dao et al. ("What FlashAttention targets") states
 * that the method must give the same outputs as this naive formulation. This
 * file is that naive formulation, one query row (or, in the backward, one key
 * column) at a time, in double precision, with no tiling, no online softmax
 * and no reordering beyond the definition:
 *
 *   S_ij  = scale * q_i . k_j                 (causal: only j <= i is kept)
 *   m_i   = max_j S_ij,  l_i = sum_j exp(S_ij - m_i)
 *   P_ij  = exp(S_ij - m_i) / l_i,  lse_i = m_i + ln l_i   (natural log)
 *   O_i   = sum_j P_ij v_j
 *
 * The pages name the backward only as recomputation from saved softmax
 * statistics (michaelc-yu summary, "Backward / recomputation"); the gradient
 * itself is the chain rule through the definition above, with the softmax
 * Jacobian dP_ij/dS_ik = P_ij (delta_jk - P_ik):
 *
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_j P_ij dP_ij            (also returned: dO_i . O_i, equal in exact arithmetic)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 *
 * Masked pairs (causal, j > i) have P_ij = 0 exactly and contribute nothing.
 * All tensors are contiguous [B,H,N,d] (lse and D: [B,H,N]) fp64.
 *
 * Block-sparse attention (the michaelc-yu summary of Dao et al. names a
 * block-sparse extension of the method without defining it): the plainest
 * reading is the same definition with more pairs masked. A block mask M of
 * nb x nb bytes per head splits queries and keys into blocks of bs rows;
 * pair (i, j) is kept iff M[i / bs][j / bs] != 0 (and j <= i when causal).
 * A query row with no kept pair has P_i = 0, O_i = 0, lse_i = -inf and no
 * gradient (D_i = 0, dQ_i = 0, and it adds nothing to dK or dV).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

int oracle_num_threads(void) { return omp_get_max_threads(); }

static double dot(const double* a, const double* b, int d)
{
    double s = 0.0;
    for (int c = 0; c < d; ++c) s += a[c] * b[c];
    return s;
}

/* The keys a head may pair: causal flag and, for block-sparse attention, the
 * head's block mask (NULL: every block). */
typedef struct {
    int causal;
    int offset;            /* causal: query i sees keys j <= i + offset */
    const uint8_t* blocks; /* nb x nb, row = query block, column = key block */
    int nb, bs;
} Visibility;

/* Is pair (query i, key j) kept? */
static int visible(const Visibility* vis, int i, int j)
{
    if (vis->causal && j > i + vis->offset) return 0;
    return vis->blocks == NULL || vis->blocks[(size_t)(i / vis->bs) * vis->nb + j / vis->bs] != 0;
}

/*
 * One query row of the forward: fills p[0..N) with the probabilities P_i.
 * (zero where masked), o_i[0..d) with O_i and *lse_i with lse_i.
 * Q, K, V point at one head ([N,d] each).
 */
static void forward_row(const double* Q, const double* K, const double* V, int N, int d,
                        double scale, const Visibility* vis, int i, double* p, double* o_i, double* lse_i)
{
    double m = -INFINITY;
    int kept = 0;
    for (int j = 0; j < N; ++j) {
        if (!visible(vis, i, j)) { p[j] = 0.0; continue; }
        p[j] = scale * dot(Q + (size_t)i * d, K + (size_t)j * d, d);
        if (p[j] > m) m = p[j];
        ++kept;
    }
    for (int c = 0; c < d; ++c) o_i[c] = 0.0;
    if (kept == 0) { /* no key to attend to */
        *lse_i = -INFINITY;
        return;
    }
    double l = 0.0;
    for (int j = 0; j < N; ++j) {
        if (!visible(vis, i, j)) continue;
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    for (int j = 0; j < N; ++j) if (visible(vis, i, j)) p[j] /= l;
    for (int j = 0; j < N; ++j)
        if (visible(vis, i, j))
            for (int c = 0; c < d; ++c) o_i[c] += p[j] * V[(size_t)j * d + c];
    *lse_i = m + log(l);
}

/* Visibility of head bh: mask bytes of head bh start mask_stride * bh bytes after
 * mask (stride 0: one mask for every head). */
static Visibility head_visibility(int causal, const uint8_t* mask, int nb, int bs, int64_t mask_stride, int64_t bh)
{
    Visibility v;
    v.causal = causal;
    v.offset = 0;
    v.blocks = mask ? mask + mask_stride * bh : NULL;
    v.nb = nb;
    v.bs = bs;
    return v;
}

/* Forward for every row of every head; mask NULL for dense attention. */
void oracle_fwd_masked(const double* q, const double* k, const double* v, int B, int H, int N, int d,
                       double scale, int causal, const uint8_t* mask, int nb, int bs, int64_t mask_stride,
                       double* o, double* lse)
{
    const int64_t rows = (int64_t)B * H * N;
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < rows; ++r) {
            const int64_t bh = r / N;
            const int i = (int)(r % N);
            const size_t head = (size_t)bh * N * d;
            const Visibility vis = head_visibility(causal, mask, nb, bs, mask_stride, bh);
            forward_row(q + head, k + head, v + head, N, d, scale, &vis, i, p,
                        o + (size_t)r * d, lse + r);
        }
        free(p);
    }
}

void oracle_fwd(const double* q, const double* k, const double* v, int B, int H, int N, int d,
                double scale, int causal, double* o, double* lse)
{
    oracle_fwd_masked(q, k, v, B, H, N, d, scale, causal, NULL, 0, 1, 0, o, lse);
}

/*
 * Forward with Nq queries against Nk keys per head (attention over a key/value
 * cache): q, o are [B,H,Nq,d], k, v [B,H,Nk,d], lse [B,H,Nq]. The queries are
 * the last Nq positions of the sequence, so with causal masking query t sees
 * keys j <= t + (Nk - Nq).
 */
void oracle_fwd_kv(const double* q, const double* k, const double* v, int B, int H, int Nq, int Nk, int d,
                   double scale, int causal, double* o, double* lse)
{
    const int64_t rows = (int64_t)B * H * Nq;
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)Nk);
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < rows; ++r) {
            const int64_t bh = r / Nq;
            const int t = (int)(r % Nq);
            Visibility vis = head_visibility(causal, NULL, 0, 1, 0, bh);
            vis.offset = Nk - Nq;
            const size_t kv_head = (size_t)bh * Nk * d;
            forward_row(q + (size_t)bh * Nq * d, k + kv_head, v + kv_head, Nk, d, scale, &vis, t, p,
                        o + (size_t)r * d, lse + r);
        }
        free(p);
    }
}

/*
 * Forward for a list of rows only. rows[t] is the flat row index (b*H + h)*N + i;
 * o_rows is [nrows, d] and lse_rows [nrows].
 */
void oracle_fwd_rows(const double* q, const double* k, const double* v, int B, int H, int N, int d,
                     double scale, int causal, int64_t nrows, const int64_t* rows,
                     double* o_rows, double* lse_rows)
{
    (void)B; (void)H;
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nrows; ++t) {
            const int64_t bh = rows[t] / N;
            const int i = (int)(rows[t] % N);
            const size_t head = (size_t)bh * N * d;
            const Visibility vis = head_visibility(causal, NULL, 0, 1, 0, bh);
            forward_row(q + head, k + head, v + head, N, d, scale, &vis, i, p,
                        o_rows + (size_t)t * d, lse_rows + t);
        }
        free(p);
    }
}

/*
 * Forward and backward for every head, Nq queries against Nk keys (q, o, dout,
 * dq: [B,H,Nq,d]; k, v, dk, dv: [B,H,Nk,d]; lse, D_pdp, D_odo: [B,H,Nq]).
 * Causal masking keeps j <= i + offset.
 * Outputs: o, lse (as the forward), dq, dk, dv, D_pdp (sum_j P_ij dP_ij) and
 * D_odo (dO_i . O_i).
 *
 * Pass 1 runs over query rows: P_i, O_i, lse_i, dP_i, D_i, dS_i and dQ_i.
 * Pass 2 runs over key columns: with lse_i and D_i of every row known, it forms
 * column j of P, dP and dS (P_ij = exp(S_ij - lse_i), the same value as pass 1's
 * exp(S_ij - m_i) / l_i) and sums dV_j and dK_j.
 */
static void bwd_heads(const double* q, const double* k, const double* v, const double* dout,
                      int B, int H, int Nq, int Nk, int d, double scale, int causal, int offset,
                      const uint8_t* mask, int nb, int bs, int64_t mask_stride,
                      double* o, double* lse, double* dq, double* dk, double* dv,
                      double* D_pdp, double* D_odo)
{
    const int64_t rows = (int64_t)B * H * Nq, cols = (int64_t)B * H * Nk;
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)Nk);
        double* dp = (double*)malloc(sizeof(double) * (size_t)Nk);
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < rows; ++r) {
            const int64_t bh = r / Nq;
            const int i = (int)(r % Nq);
            const size_t qh = (size_t)bh * Nq * d, kh = (size_t)bh * Nk * d;
            const double *Q = q + qh, *K = k + kh, *V = v + kh, *dO = dout + qh;
            Visibility vis = head_visibility(causal, mask, nb, bs, mask_stride, bh);
            vis.offset = offset;
            forward_row(Q, K, V, Nk, d, scale, &vis, i, p, o + (size_t)r * d, lse + r);
            double Dp = 0.0;
            for (int j = 0; j < Nk; ++j) {
                if (!visible(&vis, i, j)) continue;
                dp[j] = dot(dO + (size_t)i * d, V + (size_t)j * d, d);
                Dp += p[j] * dp[j];
            }
            D_pdp[r] = Dp;
            D_odo[r] = dot(dO + (size_t)i * d, o + (size_t)r * d, d);
            double* dq_i = dq + (size_t)r * d;
            for (int c = 0; c < d; ++c) dq_i[c] = 0.0;
            for (int j = 0; j < Nk; ++j) {
                if (!visible(&vis, i, j)) continue;
                const double ds = p[j] * (dp[j] - Dp);
                for (int c = 0; c < d; ++c) dq_i[c] += ds * K[(size_t)j * d + c];
            }
            for (int c = 0; c < d; ++c) dq_i[c] *= scale;
        }
        free(p);
        free(dp);
    }
    /* pass 2: one key column at a time */
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t r = 0; r < cols; ++r) {
        const int64_t bh = r / Nk;
        const int j = (int)(r % Nk);
        const size_t kh = (size_t)bh * Nk * d, qh = (size_t)bh * Nq * d;
        const double *Q = q + qh, *K = k + kh, *V = v + kh, *dO = dout + qh;
        const double* lse_h = lse + (size_t)bh * Nq;
        const double* D_h = D_pdp + (size_t)bh * Nq;
        double* dk_j = dk + (size_t)r * d;
        double* dv_j = dv + (size_t)r * d;
        for (int c = 0; c < d; ++c) { dk_j[c] = 0.0; dv_j[c] = 0.0; }
        Visibility vis = head_visibility(causal, mask, nb, bs, mask_stride, bh);
        vis.offset = offset;   /* pass 2 */
        for (int i = 0; i < Nq; ++i) {
            if (!visible(&vis, i, j)) continue;   /* query i does not attend to key j */
            const double pij = exp(scale * dot(Q + (size_t)i * d, K + (size_t)j * d, d) - lse_h[i]);
            const double dpij = dot(dO + (size_t)i * d, V + (size_t)j * d, d);
            const double ds = pij * (dpij - D_h[i]);
            for (int c = 0; c < d; ++c) {
                dv_j[c] += pij * dO[(size_t)i * d + c];
                dk_j[c] += ds * Q[(size_t)i * d + c];
            }
        }
        for (int c = 0; c < d; ++c) dk_j[c] *= scale;
    }
}

/* Forward and backward over N x N heads; mask NULL for dense attention. */
void oracle_bwd_masked(const double* q, const double* k, const double* v, const double* dout,
                       int B, int H, int N, int d, double scale, int causal,
                       const uint8_t* mask, int nb, int bs, int64_t mask_stride,
                       double* o, double* lse, double* dq, double* dk, double* dv,
                       double* D_pdp, double* D_odo)
{
    bwd_heads(q, k, v, dout, B, H, N, N, d, scale, causal, 0, mask, nb, bs, mask_stride, o, lse, dq, dk, dv,
              D_pdp, D_odo);
}

/*
 * Forward and backward of Nq queries, the last positions of their sequence,
 * over Nk keys (causal: query t sees keys j <= t + Nk - Nq, as oracle_fwd_kv).
 */
void oracle_bwd_kv(const double* q, const double* k, const double* v, const double* dout,
                   int B, int H, int Nq, int Nk, int d, double scale, int causal,
                   double* o, double* lse, double* dq, double* dk, double* dv,
                   double* D_pdp, double* D_odo)
{
    bwd_heads(q, k, v, dout, B, H, Nq, Nk, d, scale, causal, Nk - Nq /* causal offset */, NULL, 0, 1, 0,
              o, lse, dq, dk, dv, D_pdp, D_odo);
}

void oracle_bwd(const double* q, const double* k, const double* v, const double* dout,
                int B, int H, int N, int d, double scale, int causal,
                double* o, double* lse, double* dq, double* dk, double* dv,
                double* D_pdp, double* D_odo)
{
    oracle_bwd_masked(q, k, v, dout, B, H, N, d, scale, causal, NULL, 0, 1, 0, o, lse, dq, dk, dv, D_pdp, D_odo);
}
