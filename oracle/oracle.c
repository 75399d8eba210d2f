/*
 * oracle.c -- plain fp64 CPU oracle for exact masked row-softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header or constant with the HIP library.
 *
 * Sources (cited by page title and the named definition/algorithm/theorem):
 *  [AM]  alphabetamath.cc, "Exact tiled attention and memory-aware
 *        differentiation": Definition "Stable summary of an attention key block",
 *        Algorithm "Exact tiled softmax attention with block-recomputed
 *        vector-Jacobian products", Theorem "Tiled attention and its recomputed
 *        reverse pass are exact" (proof steps 1.1-7.1).
 *  [AI]  igniting.github.io, "The Arithmetic of Intelligence", chapter 12,
 *        section "Streaming softmax" (the running max / running sum update).
 *  [NS]  harperz9.github.io, Night School "Fused attention", section
 *        "Forget one step" (the broken-rescale control).
 *  [WT]  webturing.com.tr Principia, "Bellek Duvarinin Fizigi: Standart
 *        Attention'dan FlashAttention'a", section on the KV cache, long context
 *        and approximate attention (decode-shaped rows against a key cache).
 *
 * Conventions (readings of the pages, also listed in the design notes):
 *  - Rows and keys are 0-based here; the pages index from 1.
 *  - Allowed-key sets A_i: mask 0 = all keys; 1 = causal, j <= i (the diagonal
 *    is allowed); 2 = sliding window of W keys ending at the diagonal,
 *    max(0, i-W+1) <= j <= i, with W >= 1.  Every such A_i is nonempty, so
 *    the all-masked row the exactness theorem leaves undefined never occurs.
 *  - Layout: head-major, row-major, contiguous: Q,K [nh][n][d], V,G,Y [nh][n][dv].
 *  - All arithmetic is IEEE double; the exponential base is e.
 *
 * Functions with a pin (see the tests): every exported function is pinned by
 * the page's worked examples, closed forms, invariants, finite differences or
 * a brute-force evaluation.  No function here is "parity unpinned".
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL 1
#define OR_ENOMEM 2

/* Membership of key j in A_i, read on demand as the Algorithm of [AM] allows. */
static int in_allowed(int mask, int64_t window, int64_t i, int64_t j)
{
    if (mask == 0) return 1;
    if (mask == 1) return j <= i;
    return j <= i && j >= i - window + 1;
}

static int check_args(int64_t nh, int64_t n, int64_t d, int64_t dv, int mask, int64_t window)
{
    if (nh < 0 || n < 0 || d < 1 || dv < 1) return OR_EINVAL;
    if (mask < 0 || mask > 2) return OR_EINVAL;
    if (mask == 2 && window < 1) return OR_EINVAL;
    return OR_OK;
}

/* Score s_ij = c * sum_r Q_ir K_jr  ([AM] Definition, "Stable summary"). */
static double score(const double *qi, const double *kj, int64_t d, double c)
{
    double acc = 0.0;
    for (int64_t r = 0; r < d; r++) acc += qi[r] * kj[r];
    return c * acc;
}

/*
 * Dropout on the attention weights (an extension: [AM] Algorithm, reverse
 * procedure, and Remark on rounding: the base algorithm has none, and an
 * extension must replay the same realized mask in its reverse pass).  Reading:
 * inverted dropout on the normalized weights, Y_i = sum_j p_ij D_ij V_j with
 * D_ij = keep_ij * 256 / (256 - thr), the statistics m_i, l_i (and LSE) those
 * of the undropped softmax.  The realized mask is a function of the indices,
 * so the reverse pass regenerates it:
 *   row key   r_i    = XXH32(le32(seed_hi) | le32(bh) | le32(i), seed_lo)
 *   group     u_ij   = XXH32(le32(j >> 2), r_i)
 *   keep_ij          = byte (j & 3) of u_ij (little-endian) >= thr
 * with XXH32 the 32-bit xxHash function (its published specification, short
 * inputs) and thr in 0..255 (drop probability thr / 256).  bh is the flat head
 * index b * H + h.
 */
typedef struct {
    uint64_t seed;
    int thr;
    int64_t bh0; /* head index of the first head passed in */
} drop_t;

static uint32_t rotl32(uint32_t x, int r) { return (x << r) | (x >> (32 - r)); }

/* XXH32 of a message of nwords (< 4) little-endian 32-bit words. */
static uint32_t xxh32_words(const uint32_t *w, int nwords, uint32_t seed)
{
    const uint32_t P1 = 0x9E3779B1u, P2 = 0x85EBCA77u, P3 = 0xC2B2AE3Du, P4 = 0x27D4EB2Fu,
                   P5 = 0x165667B1u;
    (void)P1;
    uint32_t h = seed + P5 + (uint32_t)(4 * nwords);
    for (int k = 0; k < nwords; k++) {
        h += w[k] * P3;
        h = rotl32(h, 17) * P4;
    }
    h ^= h >> 15;
    h *= P2;
    h ^= h >> 13;
    h *= P3;
    h ^= h >> 16;
    return h;
}

static uint32_t drop_row_key(const drop_t *dr, int64_t h, int64_t i)
{
    const uint32_t w[3] = {(uint32_t)(dr->seed >> 32), (uint32_t)(dr->bh0 + h), (uint32_t)i};
    return xxh32_words(w, 3, (uint32_t)dr->seed);
}

/* D_ij: 0 for a dropped weight, 256 / (256 - thr) for a kept one. */
static double drop_factor(const drop_t *dr, uint32_t row_key, int64_t j)
{
    if (dr == NULL) return 1.0;
    const uint32_t g = (uint32_t)(j >> 2);
    const uint32_t u = xxh32_words(&g, 1, row_key);
    const int byte = (int)((u >> (8 * (j & 3))) & 0xFFu);
    return byte >= dr->thr ? 256.0 / (256.0 - dr->thr) : 0.0;
}

int oracle_xxh32_words(const uint32_t *w, int nwords, uint32_t seed, uint32_t *out)
{
    if (nwords < 0 || nwords > 3) return OR_EINVAL;
    *out = xxh32_words(w, nwords, seed);
    return OR_OK;
}

/* keep_ij of the mask above (1 kept, 0 dropped). */
int oracle_dropout_keep(uint64_t seed, int thr, int64_t bh, int64_t i, int64_t j, int *keep)
{
    if (thr < 0 || thr > 255 || bh < 0 || i < 0 || j < 0) return OR_EINVAL;
    drop_t dr = {seed, thr, 0};
    *keep = drop_factor(&dr, drop_row_key(&dr, bh, i), j) != 0.0;
    return OR_OK;
}

/*
 * One row of the dense definition ([AM] Theorem "Tiled attention ... are exact",
 * the displayed dense masked attention row, with the max shift of step 2.1):
 *   m_i = max_{j in A_i} s_ij,  l_i = sum_{j in A_i} e^{s_ij - m_i},
 *   Y_i = sum_{j in A_i} (e^{s_ij - m_i} / l_i) V_j,
 * for the query vector qi sitting at row position i (A_i is the mask's set for
 * position i over keys 0..n-1), with the dropout factors D_ij in the value sum
 * when dr != NULL (head bh).  srow is caller scratch of length n.
 */
static void dense_row_at(const double *qi, const double *K, const double *V, int64_t n,
                         int64_t d, int64_t dv, double c, int mask, int64_t window, int64_t i,
                         const drop_t *dr, int64_t bh, double *srow, double *y, double *m_out,
                         double *l_out)
{
    const uint32_t rk = dr ? drop_row_key(dr, bh, i) : 0u;
    double m = -INFINITY;
    for (int64_t j = 0; j < n; j++) {
        if (!in_allowed(mask, window, i, j)) continue;
        srow[j] = score(qi, K + j * d, d, c);
        if (srow[j] > m) m = srow[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n; j++) {
        if (!in_allowed(mask, window, i, j)) continue;
        l += exp(srow[j] - m);
    }
    for (int64_t a = 0; a < dv; a++) y[a] = 0.0;
    for (int64_t j = 0; j < n; j++) {
        if (!in_allowed(mask, window, i, j)) continue;
        double p = exp(srow[j] - m) / l * drop_factor(dr, rk, j);
        const double *vj = V + j * dv;
        for (int64_t a = 0; a < dv; a++) y[a] += p * vj[a];
    }
    *m_out = m;
    *l_out = l;
}

/* Row i of the dense definition with its own query vector Q_i. */
static void dense_row(const double *Q, const double *K, const double *V, int64_t n, int64_t d,
                      int64_t dv, double c, int mask, int64_t window, int64_t i,
                      const drop_t *dr, int64_t bh, double *srow, double *y, double *m_out,
                      double *l_out)
{
    dense_row_at(Q + i * d, K, V, n, d, dv, c, mask, window, i, dr, bh, srow, y, m_out, l_out);
}

/*
 * Dense forward on nh independent heads.  rows (length nrows) selects which
 * query rows to evaluate (rows are independent in the definition); rows == NULL
 * means every row, in order.  Outputs are [nh][nrows][dv] for Y and [nh][nrows]
 * for M (row max), L (normaliser l) and LSE = m + ln l (natural log).
 * Any of M, L, LSE may be NULL.
 */
static int fwd_core(int64_t nh, int64_t n, int64_t d, int64_t dv, const double *Q,
                    const double *K, const double *V, double c, int mask, int64_t window,
                    const drop_t *dr, const int64_t *rows, int64_t nrows, double *Y, double *M,
                    double *L, double *LSE)
{
    if (check_args(nh, n, d, dv, mask, window)) return OR_EINVAL;
    if (rows == NULL) nrows = n;
    for (int64_t r = 0; rows != NULL && r < nrows; r++)
        if (rows[r] < 0 || rows[r] >= n) return OR_EINVAL;
    int failed = 0;
#pragma omp parallel
    {
        double *srow = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        if (srow == NULL) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for collapse(2) schedule(dynamic, 4)
        for (int64_t h = 0; h < nh; h++) {
            for (int64_t r = 0; r < nrows; r++) {
                if (srow == NULL) continue;
                int64_t i = rows ? rows[r] : r;
                const double *Qh = Q + h * n * d, *Kh = K + h * n * d, *Vh = V + h * n * dv;
                double m, l;
                dense_row(Qh, Kh, Vh, n, d, dv, c, mask, window, i, dr, h, srow,
                          Y + (h * nrows + r) * dv, &m, &l);
                if (M) M[h * nrows + r] = m;
                if (L) L[h * nrows + r] = l;
                if (LSE) LSE[h * nrows + r] = m + log(l);
            }
        }
        free(srow);
    }
    return failed ? OR_ENOMEM : OR_OK;
}

int oracle_fwd(int64_t nh, int64_t n, int64_t d, int64_t dv, const double *Q, const double *K,
               const double *V, double c, int mask, int64_t window, const int64_t *rows,
               int64_t nrows, double *Y, double *M, double *L, double *LSE)
{
    return fwd_core(nh, n, d, dv, Q, K, V, c, mask, window, NULL, rows, nrows, Y, M, L, LSE);
}

/* The dense forward with the dropout above; head h of the nh passed in is
 * head bh = bh0 + h of the mask. */
int oracle_fwd_drop(int64_t nh, int64_t n, int64_t d, int64_t dv, const double *Q,
                    const double *K, const double *V, double c, int mask, int64_t window,
                    uint64_t seed, int thr, int64_t bh0, double *Y, double *LSE)
{
    if (thr < 0 || thr > 255 || bh0 < 0) return OR_EINVAL;
    drop_t dr = {seed, thr, bh0};
    return fwd_core(nh, n, d, dv, Q, K, V, c, mask, window, &dr, NULL, n, Y, NULL, NULL, LSE);
}

/*
 * Decode-shaped forward: nq new query rows per head against a cache of nk keys
 * (1 <= nq <= nk), the rows being the LAST nq positions of the sequence, so row
 * i sits at position p_i = nk - nq + i and its allowed set is the mask's set
 * for position p_i over keys 0..nk-1 (the KV-cache setting of [WT], section on
 * the KV cache and long context, where every new token attends to the cached
 * keys and values of all earlier tokens; [AI] on verifying several new
 * positions in one pass).  H query heads share Hkv key/value heads: query head
 * h reads key/value head h / (H / Hkv) (H a multiple of Hkv; Hkv = H is one
 * head each).  Every row is the dense definition above at position p_i.
 * Layout: Q [B][H][nq][d], K [B][Hkv][nk][d], V [B][Hkv][nk][dv];
 * outputs Y [B][H][nq][dv] and LSE [B][H][nq] (LSE may be NULL).
 */
int oracle_decode(int64_t B, int64_t H, int64_t Hkv, int64_t nq, int64_t nk, int64_t d,
                  int64_t dv, const double *Q, const double *K, const double *V, double c,
                  int mask, int64_t window, double *Y, double *LSE)
{
    if (B < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || nq < 1 || nk < nq) return OR_EINVAL;
    if (check_args(B * H, nk, d, dv, mask, window)) return OR_EINVAL;
    const int64_t G = H / Hkv;
    int failed = 0;
#pragma omp parallel
    {
        double *srow = (double *)malloc(sizeof(double) * (size_t)nk);
        if (srow == NULL) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int64_t b = 0; b < B; b++) {
            for (int64_t h = 0; h < H; h++) {
                for (int64_t i = 0; i < nq; i++) {
                    if (srow == NULL) continue;
                    const int64_t hk = h / G;
                    const double *qi = Q + ((b * H + h) * nq + i) * d;
                    const double *Kh = K + (b * Hkv + hk) * nk * d;
                    const double *Vh = V + (b * Hkv + hk) * nk * dv;
                    const int64_t row = (b * H + h) * nq + i;
                    double m, l;
                    dense_row_at(qi, Kh, Vh, nk, d, dv, c, mask, window, nk - nq + i, NULL, 0,
                                 srow, Y + row * dv, &m, &l);
                    if (LSE) LSE[row] = m + log(l);
                }
            }
        }
        free(srow);
    }
    return failed ? OR_ENOMEM : OR_OK;
}

/*
 * Analytic vector-Jacobian product of Phi = sum_{i,a} G_ia Y_ia, the reverse
 * procedure of [AM] Algorithm written per output element (proof steps 4.1-6.1):
 *   p_ij     = e^{s_ij - m_i} / l_i                        (frozen m_i, l_i)
 *   delta_i  = sum_a G_ia Y_ia
 *   gamma_ij = p_ij (sum_a G_ia V_ja - delta_i)
 *   dQ_i     = c sum_{j in A_i} gamma_ij K_j
 *   dK_j     = c sum_{i : j in A_i} gamma_ij Q_i
 *   dV_j     = sum_{i : j in A_i} p_ij G_i
 * Y, M, L come from the dense forward above.  Optional outputs Yout [nh][n][dv],
 * Dout (delta) and LSEout [nh][n] may be NULL.
 */
static int bwd_core(int64_t nh, int64_t n, int64_t d, int64_t dv, const double *Q,
                    const double *K, const double *V, const double *G, double c, int mask,
                    int64_t window, const drop_t *dr, double *dQ, double *dK, double *dV,
                    double *Yout, double *Dout, double *LSEout)
{
    if (check_args(nh, n, d, dv, mask, window)) return OR_EINVAL;
    size_t rows_total = (size_t)(nh * n);
    double *Y = (double *)malloc(sizeof(double) * (rows_total * dv + 1));
    double *M = (double *)malloc(sizeof(double) * (rows_total + 1));
    double *L = (double *)malloc(sizeof(double) * (rows_total + 1));
    double *D = (double *)malloc(sizeof(double) * (rows_total + 1));
    if (!Y || !M || !L || !D) {
        free(Y); free(M); free(L); free(D);
        return OR_ENOMEM;
    }
    int rc = fwd_core(nh, n, d, dv, Q, K, V, c, mask, window, dr, NULL, n, Y, M, L, NULL);
    if (rc) {
        free(Y); free(M); free(L); free(D);
        return rc;
    }

    /* delta_i = sum_a G_ia Y_ia */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < (int64_t)rows_total; t++) {
        double acc = 0.0;
        for (int64_t a = 0; a < dv; a++) acc += G[t * dv + a] * Y[t * dv + a];
        D[t] = acc;
    }

    /* dQ_i: one query row at a time. */
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int64_t h = 0; h < nh; h++) {
        for (int64_t i = 0; i < n; i++) {
            const double *Qh = Q + h * n * d, *Kh = K + h * n * d, *Vh = V + h * n * dv;
            const double *gi = G + (h * n + i) * dv;
            double m = M[h * n + i], l = L[h * n + i], delta = D[h * n + i];
            const uint32_t rk = dr ? drop_row_key(dr, h, i) : 0u;
            double *dqi = dQ + (h * n + i) * d;
            for (int64_t r = 0; r < d; r++) dqi[r] = 0.0;
            for (int64_t j = 0; j < n; j++) {
                if (!in_allowed(mask, window, i, j)) continue;
                double p = exp(score(Qh + i * d, Kh + j * d, d, c) - m) / l;
                double gv = 0.0;
                for (int64_t a = 0; a < dv; a++) gv += gi[a] * Vh[j * dv + a];
                double gamma = p * (drop_factor(dr, rk, j) * gv - delta);
                for (int64_t r = 0; r < d; r++) dqi[r] += c * gamma * Kh[j * d + r];
            }
        }
    }

    /* dK_j and dV_j: one key row at a time, summing over the queries that see it. */
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int64_t h = 0; h < nh; h++) {
        for (int64_t j = 0; j < n; j++) {
            const double *Qh = Q + h * n * d, *Kh = K + h * n * d, *Vh = V + h * n * dv;
            double *dkj = dK + (h * n + j) * d;
            double *dvj = dV + (h * n + j) * dv;
            for (int64_t r = 0; r < d; r++) dkj[r] = 0.0;
            for (int64_t a = 0; a < dv; a++) dvj[a] = 0.0;
            for (int64_t i = 0; i < n; i++) {
                if (!in_allowed(mask, window, i, j)) continue;
                const double *gi = G + (h * n + i) * dv;
                double m = M[h * n + i], l = L[h * n + i], delta = D[h * n + i];
                double p = exp(score(Qh + i * d, Kh + j * d, d, c) - m) / l;
                const double dij = dr ? drop_factor(dr, drop_row_key(dr, h, i), j) : 1.0;
                double gv = 0.0;
                for (int64_t a = 0; a < dv; a++) gv += gi[a] * Vh[j * dv + a];
                double gamma = p * (dij * gv - delta);
                for (int64_t r = 0; r < d; r++) dkj[r] += c * gamma * Qh[i * d + r];
                for (int64_t a = 0; a < dv; a++) dvj[a] += p * dij * gi[a];
            }
        }
    }

    if (Yout) memcpy(Yout, Y, sizeof(double) * rows_total * dv);
    if (Dout) memcpy(Dout, D, sizeof(double) * rows_total);
    if (LSEout)
        for (size_t t = 0; t < rows_total; t++) LSEout[t] = M[t] + log(L[t]);
    free(Y); free(M); free(L); free(D);
    return OR_OK;
}

int oracle_bwd(int64_t nh, int64_t n, int64_t d, int64_t dv, const double *Q, const double *K,
               const double *V, const double *G, double c, int mask, int64_t window, double *dQ,
               double *dK, double *dV, double *Yout, double *Dout, double *LSEout)
{
    return bwd_core(nh, n, d, dv, Q, K, V, G, c, mask, window, NULL, dQ, dK, dV, Yout, Dout,
                    LSEout);
}

/*
 * VJP of Phi = sum G * Y for the forward with dropout, the same realized mask
 * replayed ([AM]'s requirement): with D_ij the factors above,
 *   delta_i  = sum_a G_ia Y_ia                 (Y with dropout)
 *   gamma_ij = p_ij (D_ij sum_a G_ia V_ja - delta_i)
 *   dQ_i = c sum_j gamma_ij K_j,  dK_j = c sum_i gamma_ij Q_i,
 *   dV_j = sum_i p_ij D_ij G_i.
 */
int oracle_bwd_drop(int64_t nh, int64_t n, int64_t d, int64_t dv, const double *Q,
                    const double *K, const double *V, const double *G, double c, int mask,
                    int64_t window, uint64_t seed, int thr, int64_t bh0, double *dQ, double *dK,
                    double *dV, double *Yout, double *Dout, double *LSEout)
{
    if (thr < 0 || thr > 255 || bh0 < 0) return OR_EINVAL;
    drop_t dr = {seed, thr, bh0};
    return bwd_core(nh, n, d, dv, Q, K, V, G, c, mask, window, &dr, dQ, dK, dV, Yout, Dout,
                    LSEout);
}

/*
 * Summary Sigma(S) = (m, l, z) of one nonempty block ([AM] Definition "Stable
 * summary of an attention key block"): from the block's k scores s[] and its k
 * value rows Vrows [k][dv],
 *   m = max s,  l = sum e^{s - m},  z = sum e^{s - m} v.
 */
int oracle_summary(int64_t k, int64_t dv, const double *s, const double *Vrows, double *m_out,
                   double *l_out, double *z)
{
    if (k < 1 || dv < 0) return OR_EINVAL;
    double m = -INFINITY;
    for (int64_t t = 0; t < k; t++)
        if (s[t] > m) m = s[t];
    double l = 0.0;
    for (int64_t a = 0; a < dv; a++) z[a] = 0.0;
    for (int64_t t = 0; t < k; t++) {
        double w = exp(s[t] - m);
        l += w;
        for (int64_t a = 0; a < dv; a++) z[a] += w * Vrows[t * dv + a];
    }
    *m_out = m;
    *l_out = l;
    return OR_OK;
}

/*
 * Merge Sigma(S) * Sigma(T) of two disjoint nonempty summaries ([AM] Definition):
 *   m' = max(m_S, m_T), l' = e^{m_S-m'} l_S + e^{m_T-m'} l_T, z' likewise.
 * broken != 0 plants the mistake of [NS] "Forget one step": the running state
 * (S, the left operand) is not shrunk, i.e. e^{m_S - m'} is replaced by 1.
 * Output may alias either input.
 */
int oracle_merge(int64_t dv, double mS, double lS, const double *zS, double mT, double lT,
                 const double *zT, int broken, double *m_out, double *l_out, double *z_out)
{
    if (dv < 0) return OR_EINVAL;
    double mp = mS > mT ? mS : mT;
    double aS = broken ? 1.0 : exp(mS - mp);
    double aT = exp(mT - mp);
    for (int64_t a = 0; a < dv; a++) z_out[a] = aS * zS[a] + aT * zT[a];
    *l_out = aS * lS + aT * lT;
    *m_out = mp;
    return OR_OK;
}

/*
 * The forward procedure of [AM] Algorithm, in exact order, with key-block size
 * b: for each row start from the empty state; for t = 1..ceil(n/b) form
 * I = J_t cap A_i; skip an empty I; otherwise copy Sigma(I) into an empty
 * state or merge it in with the merge above; finally Y_i = z_i / l_i and the
 * row statistics m_i, l_i are retained.  broken is passed to the merge.
 * Used by the tests to pin the exactness theorem (result independent of b and
 * equal to the dense rows) and the [NS] control.
 */
int oracle_fwd_tiled(int64_t nh, int64_t n, int64_t d, int64_t dv, const double *Q, const double *K,
                     const double *V, double c, int mask, int64_t window, int64_t b, int broken,
                     double *Y, double *M, double *L)
{
    if (check_args(nh, n, d, dv, mask, window) || b < 1) return OR_EINVAL;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)b);
        double *vrows = (double *)malloc(sizeof(double) * (size_t)(b * dv));
        double *zb = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!s || !vrows || !zb) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for collapse(2) schedule(dynamic, 4)
        for (int64_t h = 0; h < nh; h++) {
            for (int64_t i = 0; i < n; i++) {
                if (!s || !vrows || !zb) continue;
                const double *Qh = Q + h * n * d, *Kh = K + h * n * d, *Vh = V + h * n * dv;
                double *z = Y + (h * n + i) * dv;
                int empty = 1; /* the state "bottom" */
                double m = 0.0, l = 0.0;
                int64_t nblocks = (n + b - 1) / b;
                for (int64_t t = 0; t < nblocks; t++) {
                    int64_t k = 0;
                    for (int64_t j = t * b; j < (t + 1) * b && j < n; j++) {
                        if (!in_allowed(mask, window, i, j)) continue;
                        s[k] = score(Qh + i * d, Kh + j * d, d, c);
                        memcpy(vrows + k * dv, Vh + j * dv, sizeof(double) * (size_t)dv);
                        k++;
                    }
                    if (k == 0) continue; /* I is empty: leave the state unchanged */
                    double mb, lb;
                    oracle_summary(k, dv, s, vrows, &mb, &lb, zb);
                    if (empty) {
                        m = mb;
                        l = lb;
                        memcpy(z, zb, sizeof(double) * (size_t)dv);
                        empty = 0;
                    } else {
                        oracle_merge(dv, m, l, z, mb, lb, zb, broken, &m, &l, z);
                    }
                }
                for (int64_t a = 0; a < dv; a++) z[a] /= l;
                if (M) M[h * n + i] = m;
                if (L) L[h * n + i] = l;
            }
        }
        free(s);
        free(vrows);
        free(zb);
    }
    return failed ? OR_ENOMEM : OR_OK;
}

/*
 * Block-scaled FP8 inputs for the scores (an extension; webturing.com.tr
 * Principia, "Bellek Duvarinin Fizigi", FlashAttention-3 section: FP8 with
 * block-wise scaling and "incoherent processing", random sign multipliers,
 * to hold the precision loss down).  Reading:
 *   1. incoherent processing: x' = H (s * x), s a caller-given vector of
 *      +-1 (the random draw is an input), H the unnormalized Sylvester
 *      Walsh-Hadamard matrix of order d (H H^T = d I), so that for Q and K
 *      rotated with the same s, Q' K'^T = d Q K^T;
 *   2. block scaling (the OCP microscaling layout): each block of 32
 *      consecutive values of a row gets a power-of-two scale 2^e, e the
 *      smallest integer with max |x'| <= 448 * 2^e (448 the largest e4m3
 *      value; at least -127, and 0 for an all-zero block), stored as the
 *      byte e + 127, so no value saturates; the values are stored as the FP8
 *      e4m3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 *      infinities, largest 448) nearest to x' / 2^e, ties to even.
 * The quantized codes are integers decided by floating point, so they are
 * computed here in the precision the GPU kernel uses: float32, with the
 * transform taken as butterfly stages of span 1, 2, 4, ..., d/2 (each pair
 * (a, b) becomes (a + b, a - b), rounded to float32).
 */

/* Value of an FP8 e4m3 code (exact). */
double oracle_e4m3_decode(uint8_t c)
{
    const int sign = c >> 7, ex = (c >> 3) & 15, man = c & 7;
    if (ex == 15 && man == 7) return NAN;
    const double mag = ex == 0 ? ldexp((double)man, -9) : ldexp(8.0 + man, ex - 10);
    return sign ? -mag : mag;
}

/* The e4m3 code nearest to x (|x| <= 448, finite), ties to even code; the
 * sign bit is x's own (so -0 and negatives that round to zero give 0x80). */
uint8_t oracle_e4m3_encode(double x)
{
    const uint8_t sign = signbit(x) ? 0x80 : 0;
    const double a = fabs(x);
    /* candidate codes are monotone in value for 0..126: binary search the neighbours */
    int lo = 0, hi = 126;
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (oracle_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid;
    }
    if (oracle_e4m3_decode((uint8_t)hi) <= a) lo = hi; /* a >= 448 */
    int best = lo;
    if (lo < 126) {
        const double dl = a - oracle_e4m3_decode((uint8_t)lo);
        const double dh = oracle_e4m3_decode((uint8_t)(lo + 1)) - a;
        if (dh < dl || (dh == dl && ((lo + 1) & 1) == 0)) best = lo + 1;
    }
    return (uint8_t)(sign | best);
}

/* In-place unnormalized Walsh-Hadamard transform of n = 2^k floats, in the
 * stage order stated above. */
static void fwht_f32(float *x, int64_t n)
{
    for (int64_t span = 1; span < n; span <<= 1)
        for (int64_t i = 0; i < n; i += 2 * span)
            for (int64_t j = i; j < i + span; j++) {
                const float a = x[j], b = x[j + span];
                x[j] = a + b;
                x[j + span] = a - b;
            }
}

/* Exposed for the pins: the float32 transform of one vector. */
int oracle_fwht_f32(int64_t n, float *x)
{
    if (n < 1 || (n & (n - 1))) return OR_EINVAL;
    fwht_f32(x, n);
    return OR_OK;
}

/* Smallest e >= -127 with amax <= 448 * 2^e (amax finite; 0 for amax = 0). */
static int mx_exponent(float amax)
{
    if (amax == 0.0f) return 0;
    int ex;
    const double mant = frexp((double)amax, &ex); /* amax = mant 2^ex, mant in [0.5, 1) */
    const int e = mant <= 0.875 ? ex - 9 : ex - 8;
    return e < -127 ? -127 : e;
}

/*
 * Quantize rows x [rows][d] with the incoherent processing and block scaling
 * above.  signs [d] in {+1, -1} (NULL: no rotation, i.e. s = 1 and H = I; a
 * rotation needs d a power of two).  Outputs codes [rows][d] and scale bytes
 * [rows][ceil(d / 32)]; a last, shorter block takes its maximum over the
 * values it has.
 */
int oracle_mx_quant(int64_t rows, int64_t d, const double *x, const int8_t *signs, uint8_t *codes,
                    uint8_t *scales)
{
    if (rows < 0 || d < 1 || (signs && (d & (d - 1)))) return OR_EINVAL;
    const int64_t nb = (d + 31) / 32;
    int failed = 0;
#pragma omp parallel
    {
        float *v = (float *)malloc(sizeof(float) * (size_t)d);
        if (!v) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; r++) {
            if (!v) continue;
            for (int64_t k = 0; k < d; k++) {
                v[k] = (float)x[r * d + k];
                if (signs) v[k] = signs[k] < 0 ? -v[k] : v[k];
            }
            if (signs) fwht_f32(v, d);
            for (int64_t b = 0; b < nb; b++) {
                const int64_t k1 = b * 32 + 32 < d ? b * 32 + 32 : d;
                float amax = 0.0f;
                for (int64_t k = b * 32; k < k1; k++) amax = fmaxf(amax, fabsf(v[k]));
                const int e = mx_exponent(amax);
                scales[r * nb + b] = (uint8_t)(e + 127);
                for (int64_t k = b * 32; k < k1; k++)
                    codes[r * d + k] = oracle_e4m3_encode(ldexp((double)v[k], -e));
            }
        }
        free(v);
    }
    return failed ? OR_ENOMEM : OR_OK;
}

/* Values of block-scaled codes: x[r][k] = value(code) * 2^(scale byte - 127). */
int oracle_mx_dequant(int64_t rows, int64_t d, const uint8_t *codes, const uint8_t *scales,
                      double *x)
{
    if (rows < 0 || d < 1) return OR_EINVAL;
    const int64_t nb = (d + 31) / 32;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < d; k++)
            x[r * d + k] = ldexp(oracle_e4m3_decode(codes[r * d + k]),
                                 (int)scales[r * nb + k / 32] - 127);
    return OR_OK;
}

/* Number of OpenMP threads the oracle would use (reported by the benchmark). */
int oracle_num_threads(void)
{
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        t = omp_get_num_threads();
    }
    return t;
}
