/*
 * attn_oracle.c -- plain fp64 CPU reference for attention and its gradient.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never calls it and shares no code, header or constant with it.
 *
 * What it computes (per sequence s and query head h, KV head g = h / (H/Hk)):
 *
 *   S_ij  = scale * sum_d Q_id K_jd                       (scores)
 *   S_ij <- c * tanh(S_ij / c)                 (only with softcap c > 0)
 *   visible(i,j) = (!causal || j <= i + Lk - Lq)          (bottom-right causal)
 *                  && (wr < 0 || j <= i + Lk - Lq + wr)   (local window, right)
 *                  && (wl < 0 || j >= i + Lk - Lq - wl)   (local window, left)
 *   LSE_i = log sum_{visible j} exp(S_ij)                 (-inf if none visible)
 *   P_ij  = exp(S_ij - LSE_i) if visible else 0           (softmax)
 *   M_ij  = Z_ij / (1 - p)      (dropout with probability p; 1 without)
 *   O_i   = sum_j P_ij M_ij V_j
 *
 *   backward of f = sum(dO * O):
 *   dP_ij = sum_d dO_id V_jd
 *   dS_i  = J_i (M_i * dP_i),   J_i = diag(P_i) - P_i P_i^T   (softmax Jacobian)
 *   dS_ij <- dS_ij * (1 - (S_ij / c)^2)       (softcap: d/dx c tanh(x/c))
 *   dQ_i  = scale * sum_j dS_ij K_j
 *   dK_j  = scale * sum_{h in group g} sum_i dS^(h)_ij Q^(h)_i
 *   dV_j  =         sum_{h in group g} sum_i P^(h)_ij M^(h)_ij dO^(h)_i
 *
 *   Dropout keep bits Z (0 or 1) come from Philox4x32-10 (Salmon, Moraes,
 *   Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011),
 *   written here from that definition: for sequence b, query head h of H,
 *   query row i and key j (local indices), the counter is
 *   (j / 4, i, b * H + h, offset mod 2^32) and the key (seed mod 2^32,
 *   (seed / 2^32) xor (offset / 2^32)); word j mod 4 of the output is the
 *   element's random u, and Z = (u >= floor(p * 2^32)).
 *
 * Passages followed (page titles as listed in the design notes):
 *   - sm90 backward kernel page (FlashAttentionBackwardSm90), mma_one_m_block:
 *     the five products S = Q K^T, dP = dO V^T, dV += P^T dO, dQ = dS K,
 *     dK += dS^T Q, the pointwise P = exp(S - LSE) and dS = P (dP - rowsum);
 *     epilogue_dKV for the single final softmax_scale on dK.
 *   - Triton FA2 teaching page, backward dQ kernel: dq is multiplied by the
 *     softmax scale once at the end.
 *   - GQA/MQA page, causal block bound: the key limit of query row i is
 *     i + seqlen_k - seqlen_q (bottom-right alignment); backward GQA section:
 *     dK/dV of the query heads are summed over each head group.
 *   - Backward call-trace page, GQA reduce: the group sum over the H/Hk heads;
 *     mha_bwd's window_size_left / window_size_right arguments, read as a
 *     band around the bottom-right diagonal (query i sees keys
 *     i + Lk - Lq - wl .. i + Lk - Lq + wr; a negative size leaves that
 *     side unbounded), the plainest reading of names the pages do not
 *     define further; its softcap argument (a kernel variant switched on by
 *     softcap > 0), read as the usual logit soft-capping c * tanh(x / c) of
 *     the scaled score x, with the gradient through it by the chain rule.
 *   - Triton FA2 teaching page, dropout_mask and the forward inner loop:
 *     elements dropped by a Philox draw keyed by the seed, at a counter
 *     derived from the element's position and the offset, and the kept ones
 *     scaled by 1 / (1 - p); the page's comparison is read as the drop test
 *     (u below p * 2^32 is dropped, so that the scale keeps the expectation),
 *     and the counter layout above is this library's own (the page's call is
 *     garbled).  Backward call-trace page: the backward replays the
 *     forward's rng_state (seed, offset).
 *
 * Two backward evaluations are provided and tested against each other:
 *   oracle_backward_explicit -- materialises P, dP and each row's Jacobian
 *                               J_i (O(Lk^2) per row; small inputs only);
 *   oracle_backward          -- the same Jacobian-vector product written as
 *                               dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik), row
 *                               pass for dQ, key pass for dK/dV; any size.
 * Neither uses the GPU's rowsum(dO * O) shortcut; that identity is checked by
 * the tests, not assumed.
 *
 * Layouts: tokens-major packed rows.  q, dout, out, dq: [total_q][H][D];
 * k, v, dk, dv: [total_k][Hk][D]; lse, dj: [total_q][H].  Sequence s owns
 * rows cu_q[s] .. cu_q[s+1]-1 (and cu_k likewise).  A dense batch of B
 * sequences of equal length is the special case cu_q = {0, Sq, 2Sq, ...}.
 * All inputs are fp64 (bf16 values upcast exactly by the caller).
 *
 * Optional `mask` (only with nseq == 1): additive [Lq][Lk] matrix of 0 / -inf
 * applied to every head on top of the causal rule; used by the tests to show
 * that the causal rule equals an explicit -inf mask.
 *
 * Optional `drop_base` (nullable): {b0, h0, hc}, the place of this call's
 * sequences and heads in a larger call whose dropout bits it replays:
 * sequence b and head h here draw the bits of sequence b + b0 and head
 * h + h0 of hc heads there (h0 + H <= hc).  Used to evaluate one sampled
 * (sequence, head group) of a large dropout run alone.
 *
 * Return value: 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- Philox4x32-10 (SC 2011 paper): ten rounds of two 32x32->64 products
 * with the multipliers 0xD2511F53 and 0xCD9E8D57, the key bumped by the Weyl
 * constants 0x9E3779B9 and 0xBB67AE85 between rounds. ---- */
static void philox_round(uint32_t c[4], const uint32_t k[2])
{
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k[0];
    const uint32_t n2 = hi0 ^ c[3] ^ k[1];
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
}

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int r = 0; r < 10; r++) {
        if (r > 0) {
            k[0] += 0x9E3779B9u;
            k[1] += 0xBB67AE85u;
        }
        philox_round(c, k);
    }
    for (int w = 0; w < 4; w++)
        out[w] = c[w];
}

/* Dropout parameters of one call: p = 0 means none.  The counter names the
 * element's sequence and query head within the whole attention call; a call
 * that evaluates part of it (one sequence, one group of heads) gives that
 * part's place: sequence b of the part is sequence b + b0 of the whole, head h
 * is head h + h0 of hc heads (b0 = h0 = 0, hc = the part's own H when no base
 * is given). */
typedef struct {
    double p;
    uint64_t seed, offset;
    int64_t b0, h0, hc;
} drop_t;

static int bad_base(const int64_t *base, int H)
{
    return base && (base[0] < 0 || base[1] < 0 || base[2] < base[1] + H);
}

static drop_t make_drop(double p, uint64_t seed, uint64_t offset, const int64_t *base)
{
    drop_t dr = {p, seed, offset, 0, 0, 0};
    if (base) {
        dr.b0 = base[0];
        dr.h0 = base[1];
        dr.hc = base[2];
    }
    return dr;
}

/* Keep bit Z of element (b, h, i, j), H query heads. */
static int drop_keep(const drop_t *dr, int b, int h, int H, int i, int j)
{
    if (dr->p <= 0.0)
        return 1;
    const int64_t hc = dr->hc > 0 ? dr->hc : H;
    const uint32_t ctr[4] = {(uint32_t)j >> 2, (uint32_t)i,
                             (uint32_t)((b + dr->b0) * hc + h + dr->h0), (uint32_t)dr->offset};
    const uint32_t key[2] = {(uint32_t)dr->seed,
                             (uint32_t)(dr->seed >> 32) ^ (uint32_t)(dr->offset >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    const uint32_t thr = (uint32_t)floor(dr->p * 4294967296.0);
    return out[j & 3] >= thr;
}

/* Dropout multiplier M_ij = Z_ij / (1 - p) (1 without dropout). */
static double drop_mult(const drop_t *dr, int b, int h, int H, int i, int j)
{
    if (dr->p <= 0.0)
        return 1.0;
    return drop_keep(dr, b, h, H, i, j) ? 1.0 / (1.0 - dr->p) : 0.0;
}

/* The keep bits of one (sequence, head) as a [Lq][Lk] byte matrix. */
int oracle_dropout_mask(double p, uint64_t seed, uint64_t offset, int b, int h, int H,
                        int Lq, int Lk, uint8_t *mask)
{
    if (!(p >= 0.0 && p < 1.0) || Lq < 0 || Lk < 0 || H <= 0)
        return -1;
    const drop_t dr = make_drop(p, seed, offset, NULL);
    for (int i = 0; i < Lq; i++)
        for (int j = 0; j < Lk; j++)
            mask[(size_t)i * Lk + j] = (uint8_t)drop_keep(&dr, b, h, H, i, j);
    return 0;
}

/* Dot product over the head dimension.  Fixed summation order: four
 * interleaved partial sums (d = 0,4,8.. / 1,5,9.. / ...) added as
 * (p0 + p1) + (p2 + p3), then the tail in ascending d.  Every dot product in
 * this file goes through here, so all evaluations of one score agree bit for
 * bit. */
static double dot(const double *a, const double *b, int D)
{
    double p0 = 0.0, p1 = 0.0, p2 = 0.0, p3 = 0.0;
    int d = 0;
    for (; d + 4 <= D; d += 4) {
        p0 += a[d] * b[d];
        p1 += a[d + 1] * b[d + 1];
        p2 += a[d + 2] * b[d + 2];
        p3 += a[d + 3] * b[d + 3];
    }
    double acc = (p0 + p1) + (p2 + p3);
    for (; d < D; d++)
        acc += a[d] * b[d];
    return acc;
}

/* One score S_ij (soft-capped when softcap > 0), or -inf when the pair is
 * not visible. */
static double score(const double *qi, const double *kj, int D, double scale,
                    int i, int j, int Lq, int Lk, int causal, int wl, int wr,
                    double softcap, const double *mask_row)
{
    const int64_t diag = (int64_t)i + Lk - Lq;   /* bottom-right diagonal key of row i */
    if (causal && (int64_t)j > diag)
        return -INFINITY;
    if (wr >= 0 && (int64_t)j > diag + wr)
        return -INFINITY;
    if (wl >= 0 && (int64_t)j < diag - wl)
        return -INFINITY;
    if (mask_row && mask_row[j] == -INFINITY)
        return -INFINITY;
    double s = scale * dot(qi, kj, D);
    if (softcap > 0.0)
        s = softcap * tanh(s / softcap);
    if (mask_row)
        s += mask_row[j];
    return s;
}

/* Derivative of the capped score with respect to the uncapped one, from the
 * capped value s = c tanh(x / c): 1 - tanh^2 = 1 - (s / c)^2 (1 without a
 * cap).  The explicit masks add only 0, so s is the capped score itself. */
static double cap_grad(double s, double softcap)
{
    if (softcap > 0.0) {
        const double t = s / softcap;
        return 1.0 - t * t;
    }
    return 1.0;
}

/* Natural-log log-sum-exp of one row of scores (-inf if all are -inf). */
static double row_lse(const double *s, int Lk)
{
    double m = -INFINITY;
    for (int j = 0; j < Lk; j++)
        if (s[j] > m)
            m = s[j];
    if (m == -INFINITY)
        return -INFINITY;
    double l = 0.0;
    for (int j = 0; j < Lk; j++)
        l += exp(s[j] - m);
    return m + log(l);
}

static int check_common(int nseq, const int64_t *cu_q, const int64_t *cu_k,
                        int H, int Hk, int D, const double *mask)
{
    if (nseq < 0 || H <= 0 || Hk <= 0 || D <= 0 || H % Hk != 0)
        return -1;
    if (!cu_q || !cu_k)
        return -1;
    if (mask && nseq != 1)
        return -1;
    for (int s = 0; s < nseq; s++)
        if (cu_q[s + 1] < cu_q[s] || cu_k[s + 1] < cu_k[s])
            return -1;
    return 0;
}

static int max_len(int nseq, const int64_t *cu)
{
    int64_t m = 0;
    for (int s = 0; s < nseq; s++)
        if (cu[s + 1] - cu[s] > m)
            m = cu[s + 1] - cu[s];
    return (int)m;
}

/* Forward: O and LSE for every (row, head). */
int oracle_forward(int nseq, const int64_t *cu_q, const int64_t *cu_k,
                   int H, int Hk, int D, double scale, int causal, int wl, int wr,
                   double softcap, double drop_p, uint64_t drop_seed, uint64_t drop_offset,
                   const int64_t *drop_base, const double *mask,
                   const double *q, const double *k, const double *v,
                   double *out, double *lse)
{
    if (check_common(nseq, cu_q, cu_k, H, Hk, D, mask) || !(drop_p >= 0.0 && drop_p < 1.0) ||
        bad_base(drop_base, H))
        return -1;
    const drop_t dr = make_drop(drop_p, drop_seed, drop_offset, drop_base);
    const int G = H / Hk;
    const int Lk_max = max_len(nseq, cu_k);
    const int64_t nunits = (int64_t)nseq * H;
    int failed = 0;

#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Lk_max + 1));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < nunits; u++) {
            if (!s)
                continue;
            const int b = (int)(u / H), h = (int)(u % H), g = h / G;
            const int64_t q0 = cu_q[b], k0 = cu_k[b];
            const int Lq = (int)(cu_q[b + 1] - q0), Lk = (int)(cu_k[b + 1] - k0);
            for (int i = 0; i < Lq; i++) {
                const double *qi = q + ((q0 + i) * H + h) * D;
                const double *mrow = mask ? mask + (int64_t)i * Lk : NULL;
                for (int j = 0; j < Lk; j++)
                    s[j] = score(qi, k + ((k0 + j) * Hk + g) * D, D, scale,
                                 i, j, Lq, Lk, causal, wl, wr, softcap, mrow);
                const double L = row_lse(s, Lk);
                double *o = out + ((q0 + i) * H + h) * D;
                for (int d = 0; d < D; d++)
                    o[d] = 0.0;
                lse[(q0 + i) * H + h] = L;
                if (L == -INFINITY)
                    continue;
                for (int j = 0; j < Lk; j++) {
                    if (s[j] == -INFINITY)
                        continue;
                    const double p = exp(s[j] - L) * drop_mult(&dr, b, h, H, i, j);
                    const double *vj = v + ((k0 + j) * Hk + g) * D;
                    for (int d = 0; d < D; d++)
                        o[d] += p * vj[d];
                }
            }
        }
        free(s);
    }
    return failed ? -2 : 0;
}

/* D^O diagnostic: sum_d dO_id * O_id for every (row, head), O as given. */
int oracle_rowdot(int64_t total_q, int H, int D, const double *dout,
                  const double *out, double *res)
{
    if (total_q < 0 || H <= 0 || D <= 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < total_q * H; r++) {
        res[r] = dot(dout + r * D, out + r * D, D);
    }
    return 0;
}

/* Sum the per-query-head gradients of one KV head in ascending head order:
 * dst[row][g] = sum_{h = gG}^{gG+G-1} src[row][h]. */
static void group_sum(int64_t total_k, int H, int Hk, int D,
                      const double *src, double *dst)
{
    const int G = H / Hk;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < total_k; r++)
        for (int g = 0; g < Hk; g++) {
            double *o = dst + (r * Hk + g) * D;
            for (int d = 0; d < D; d++)
                o[d] = 0.0;
            for (int h = g * G; h < (g + 1) * G; h++) {
                const double *x = src + (r * H + h) * D;
                for (int d = 0; d < D; d++)
                    o[d] += x[d];
            }
        }
}

/*
 * Explicit-Jacobian backward.  For every (sequence, head) it materialises
 * P and dP (Lq x Lk), and for every row the Lk x Lk Jacobian of the softmax,
 * then forms dS = J dP row by row and the three products with plain loops.
 * ds_out (nullable, nseq == 1 only): [H][Lq][Lk].  dj_out (nullable):
 * sum_k P_ik dP_ik per (row, head).
 */
int oracle_backward_explicit(int nseq, const int64_t *cu_q, const int64_t *cu_k,
                             int H, int Hk, int D, double scale, int causal, int wl, int wr,
                             double softcap, double drop_p, uint64_t drop_seed,
                             uint64_t drop_offset, const int64_t *drop_base,
                             const double *mask,
                             const double *q, const double *k, const double *v,
                             const double *dout,
                             double *dq, double *dk, double *dv,
                             double *ds_out, double *dj_out)
{
    if (check_common(nseq, cu_q, cu_k, H, Hk, D, mask) || !(drop_p >= 0.0 && drop_p < 1.0) ||
        bad_base(drop_base, H))
        return -1;
    const drop_t dr = make_drop(drop_p, drop_seed, drop_offset, drop_base);
    if (ds_out && nseq != 1)
        return -1;
    const int G = H / Hk;
    const int64_t total_k = cu_k[nseq];
    const int64_t nunits = (int64_t)nseq * H;
    /* per-query-head dK, dV before the group sum: [total_k][H][D] */
    double *dkh = (double *)calloc((size_t)(total_k * H * D) + 1, sizeof(double));
    double *dvh = (double *)calloc((size_t)(total_k * H * D) + 1, sizeof(double));
    if (!dkh || !dvh) {
        free(dkh);
        free(dvh);
        return -2;
    }
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < nunits; u++) {
        const int b = (int)(u / H), h = (int)(u % H), g = h / G;
        const int64_t q0 = cu_q[b], k0 = cu_k[b];
        const int Lq = (int)(cu_q[b + 1] - q0), Lk = (int)(cu_k[b + 1] - k0);
        const size_t n = (size_t)Lq * Lk + 1;
        double *S = (double *)malloc(n * sizeof(double));
        double *P = (double *)malloc(n * sizeof(double));
        double *dP = (double *)malloc(n * sizeof(double));
        double *dS = (double *)malloc(n * sizeof(double));
        double *J = (double *)malloc(((size_t)Lk * Lk + 1) * sizeof(double));
        if (!S || !P || !dP || !dS || !J) {
#pragma omp atomic write
            failed = 1;
            free(S); free(P); free(dP); free(dS); free(J);
            continue;
        }
#define QP(i) (q + ((q0 + (i)) * H + h) * D)
#define DOP(i) (dout + ((q0 + (i)) * H + h) * D)
#define KP(j) (k + ((k0 + (j)) * Hk + g) * D)
#define VP(j) (v + ((k0 + (j)) * Hk + g) * D)
        /* scores and softmax */
        for (int i = 0; i < Lq; i++) {
            const double *mrow = mask ? mask + (int64_t)i * Lk : NULL;
            for (int j = 0; j < Lk; j++)
                S[(size_t)i * Lk + j] = score(QP(i), KP(j), D, scale, i, j, Lq, Lk,
                                              causal, wl, wr, softcap, mrow);
            const double L = row_lse(S + (size_t)i * Lk, Lk);
            for (int j = 0; j < Lk; j++) {
                const double sij = S[(size_t)i * Lk + j];
                P[(size_t)i * Lk + j] = (L == -INFINITY || sij == -INFINITY) ? 0.0 : exp(sij - L);
            }
        }
        /* dP = dO V^T, times the dropout multiplier (the gradient with
         * respect to P of O = (P * M) V) */
        for (int i = 0; i < Lq; i++)
            for (int j = 0; j < Lk; j++) {
                dP[(size_t)i * Lk + j] = dot(DOP(i), VP(j), D) * drop_mult(&dr, b, h, H, i, j);
            }
        /* dS_i = J_i dP_i with J_i = diag(P_i) - P_i P_i^T, then through the
         * soft cap (invisible pairs have P = 0 and so dS = 0 already) */
        for (int i = 0; i < Lq; i++) {
            const double *Pi = P + (size_t)i * Lk;
            for (int j = 0; j < Lk; j++)
                for (int c = 0; c < Lk; c++)
                    J[(size_t)j * Lk + c] = (j == c ? Pi[j] : 0.0) - Pi[j] * Pi[c];
            for (int j = 0; j < Lk; j++) {
                double acc = 0.0;
                for (int c = 0; c < Lk; c++)
                    acc += J[(size_t)j * Lk + c] * dP[(size_t)i * Lk + c];
                const double sij = S[(size_t)i * Lk + j];
                dS[(size_t)i * Lk + j] = sij == -INFINITY ? acc : acc * cap_grad(sij, softcap);
            }
            if (dj_out) {
                double acc = 0.0;
                for (int c = 0; c < Lk; c++)
                    acc += Pi[c] * dP[(size_t)i * Lk + c];
                dj_out[(q0 + i) * H + h] = acc;
            }
        }
        /* dQ = scale * dS K */
        for (int i = 0; i < Lq; i++) {
            double *o = dq + ((q0 + i) * H + h) * D;
            for (int d = 0; d < D; d++) {
                double acc = 0.0;
                for (int j = 0; j < Lk; j++)
                    acc += dS[(size_t)i * Lk + j] * KP(j)[d];
                o[d] = scale * acc;
            }
        }
        /* dK^(h) = scale * dS^T Q,  dV^(h) = P^T dO */
        for (int j = 0; j < Lk; j++) {
            double *ok = dkh + ((k0 + j) * H + h) * D;
            double *ov = dvh + ((k0 + j) * H + h) * D;
            for (int d = 0; d < D; d++) {
                double acck = 0.0, accv = 0.0;
                for (int i = 0; i < Lq; i++) {
                    acck += dS[(size_t)i * Lk + j] * QP(i)[d];
                    accv += P[(size_t)i * Lk + j] * drop_mult(&dr, b, h, H, i, j) * DOP(i)[d];
                }
                ok[d] = scale * acck;
                ov[d] = accv;
            }
        }
        if (ds_out)
            memcpy(ds_out + (size_t)h * Lq * Lk, dS, (size_t)Lq * Lk * sizeof(double));
#undef QP
#undef DOP
#undef KP
#undef VP
        free(S); free(P); free(dP); free(dS); free(J);
    }
    if (!failed) {
        group_sum(total_k, H, Hk, D, dkh, dk);
        group_sum(total_k, H, Hk, D, dvh, dv);
    }
    free(dkh);
    free(dvh);
    return failed ? -2 : 0;
}

/*
 * Contracted backward for any size.  The softmax Jacobian-vector product is
 * written out as dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik), which is J_i dP_i
 * expanded.  Row pass (one task per query row and head): scores, LSE, P, dP,
 * the row contraction D^J_i, dS and dQ_i.  Key pass (one task per key row and
 * KV head): for each query head of the group in ascending order, the column
 * sums over query rows of dS_ij Q_i and P_ij dO_i, with P and dS recomputed
 * from the same scores, the row pass's LSE_i and D^J_i; the per-head results
 * are then added in ascending head order.
 * dj_out, lse_out (nullable): D^J and LSE per (row, head).
 */
int oracle_backward(int nseq, const int64_t *cu_q, const int64_t *cu_k,
                    int H, int Hk, int D, double scale, int causal, int wl, int wr,
                    double softcap, double drop_p, uint64_t drop_seed, uint64_t drop_offset,
                    const int64_t *drop_base, const double *mask,
                    const double *q, const double *k, const double *v,
                    const double *dout,
                    double *dq, double *dk, double *dv,
                    double *dj_out, double *lse_out)
{
    if (check_common(nseq, cu_q, cu_k, H, Hk, D, mask) || !(drop_p >= 0.0 && drop_p < 1.0) ||
        bad_base(drop_base, H))
        return -1;
    const drop_t dr = make_drop(drop_p, drop_seed, drop_offset, drop_base);
    const int G = H / Hk;
    const int64_t total_q = cu_q[nseq];
    const int Lk_max = max_len(nseq, cu_k);
    double *LSE = (double *)malloc(sizeof(double) * (size_t)(total_q * H + 1));
    double *DJ = (double *)malloc(sizeof(double) * (size_t)(total_q * H + 1));
    /* row -> sequence map for the row pass */
    int *seq_of_row = (int *)malloc(sizeof(int) * (size_t)(total_q + 1));
    if (!LSE || !DJ || !seq_of_row) {
        free(LSE); free(DJ); free(seq_of_row);
        return -2;
    }
    for (int s = 0; s < nseq; s++)
        for (int64_t r = cu_q[s]; r < cu_q[s + 1]; r++)
            seq_of_row[r] = s;
    int failed = 0;

    /* ---- row pass: LSE, P, dP, D^J, dS, dQ ---- */
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Lk_max + 1));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(Lk_max + 1));
        double *cg = (double *)malloc(sizeof(double) * (size_t)(Lk_max + 1));
        if (!s || !dp || !cg) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < total_q * H; t++) {
            if (!s || !dp || !cg)
                continue;
            const int64_t r = t / H;
            const int h = (int)(t % H), g = h / G, b = seq_of_row[r];
            const int64_t q0 = cu_q[b], k0 = cu_k[b];
            const int Lq = (int)(cu_q[b + 1] - q0), Lk = (int)(cu_k[b + 1] - k0);
            const int i = (int)(r - q0);
            const double *qi = q + (r * H + h) * D;
            const double *doi = dout + (r * H + h) * D;
            const double *mrow = mask ? mask + (int64_t)i * Lk : NULL;
            for (int j = 0; j < Lk; j++)
                s[j] = score(qi, k + ((k0 + j) * Hk + g) * D, D, scale, i, j, Lq, Lk,
                             causal, wl, wr, softcap, mrow);
            const double L = row_lse(s, Lk);
            LSE[r * H + h] = L;
            double *o = dq + (r * H + h) * D;
            for (int d = 0; d < D; d++)
                o[d] = 0.0;
            double dj = 0.0;
            if (L != -INFINITY) {
                for (int j = 0; j < Lk; j++) {
                    if (s[j] == -INFINITY) {
                        s[j] = 0.0; /* P_ij = 0 */
                        dp[j] = 0.0;
                        cg[j] = 0.0;
                        continue;
                    }
                    cg[j] = cap_grad(s[j], softcap);
                    s[j] = exp(s[j] - L); /* s now holds P_ij */
                    const double *vj = v + ((k0 + j) * Hk + g) * D;
                    dp[j] = dot(doi, vj, D) * drop_mult(&dr, b, h, H, i, j);   /* M_ij dP_ij */
                }
                for (int j = 0; j < Lk; j++)
                    dj += s[j] * dp[j];
                for (int j = 0; j < Lk; j++) {
                    if (s[j] == 0.0)
                        continue;
                    const double dsij = s[j] * (dp[j] - dj) * cg[j];
                    const double *kj = k + ((k0 + j) * Hk + g) * D;
                    for (int d = 0; d < D; d++)
                        o[d] += dsij * kj[d];
                }
                for (int d = 0; d < D; d++)
                    o[d] *= scale;
            }
            DJ[r * H + h] = dj;
        }
        free(s);
        free(dp);
        free(cg);
    }

    /* ---- key pass: dK, dV ---- */
    const int64_t total_k = cu_k[nseq];
    int *seq_of_key = (int *)malloc(sizeof(int) * (size_t)(total_k + 1));
    if (!seq_of_key)
        failed = 1;
    else
        for (int s2 = 0; s2 < nseq; s2++)
            for (int64_t r = cu_k[s2]; r < cu_k[s2 + 1]; r++)
                seq_of_key[r] = s2;
    if (!failed) {
#pragma omp parallel
        {
            double *acck = (double *)malloc(sizeof(double) * (size_t)D);
            double *accv = (double *)malloc(sizeof(double) * (size_t)D);
            if (!acck || !accv) {
#pragma omp atomic write
                failed = 1;
            }
#pragma omp for schedule(dynamic, 16)
            for (int64_t t = 0; t < total_k * Hk; t++) {
                if (!acck || !accv)
                    continue;
                const int64_t rk = t / Hk;
                const int g = (int)(t % Hk), b = seq_of_key[rk];
                const int64_t q0 = cu_q[b], k0 = cu_k[b];
                const int Lq = (int)(cu_q[b + 1] - q0), Lk = (int)(cu_k[b + 1] - k0);
                const int j = (int)(rk - k0);
                const double *kj = k + (rk * Hk + g) * D;
                const double *vj = v + (rk * Hk + g) * D;
                double *ok = dk + (rk * Hk + g) * D;
                double *ov = dv + (rk * Hk + g) * D;
                for (int d = 0; d < D; d++) {
                    ok[d] = 0.0;
                    ov[d] = 0.0;
                }
                for (int h = g * G; h < (g + 1) * G; h++) {
                    for (int d = 0; d < D; d++) {
                        acck[d] = 0.0;
                        accv[d] = 0.0;
                    }
                    for (int i = 0; i < Lq; i++) {
                        const int64_t r = q0 + i;
                        const double L = LSE[r * H + h];
                        if (L == -INFINITY)
                            continue;
                        const double *qi = q + (r * H + h) * D;
                        const double *mrow = mask ? mask + (int64_t)i * Lk : NULL;
                        const double sij = score(qi, kj, D, scale, i, j, Lq, Lk, causal, wl, wr,
                                                 softcap, mrow);
                        if (sij == -INFINITY)
                            continue;
                        const double p = exp(sij - L);
                        const double m = drop_mult(&dr, b, h, H, i, j);
                        const double *doi = dout + (r * H + h) * D;
                        const double dpij = dot(doi, vj, D) * m;
                        const double dsij = p * (dpij - DJ[r * H + h]) * cap_grad(sij, softcap);
                        for (int d = 0; d < D; d++) {
                            acck[d] += dsij * qi[d];
                            accv[d] += p * m * doi[d];
                        }
                    }
                    for (int d = 0; d < D; d++) {
                        ok[d] += scale * acck[d];
                        ov[d] += accv[d];
                    }
                }
            }
            free(acck);
            free(accv);
        }
    }
    if (!failed) {
        if (dj_out)
            memcpy(dj_out, DJ, sizeof(double) * (size_t)(total_q * H));
        if (lse_out)
            memcpy(lse_out, LSE, sizeof(double) * (size_t)(total_q * H));
    }
    free(LSE);
    free(DJ);
    free(seq_of_row);
    free(seq_of_key);
    return failed ? -2 : 0;
}

/* Number of OpenMP threads a parallel region of this library would use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
