/*
 * Lighthouse attention: plain CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU path and must never be used as a
 * fallback for it.
 *
 * Source: "Long Context Pre-Training with Lighthouse Attention" (Peng, Ghosh,
 * Quesnelle; arXiv 2605.06554), as mirrored on the pages
 *   P1  bittide.aicompass.dev article (translation of the arXiv HTML):
 *       Sec. 1 (Introduction), Fig. 1, Sec. 3, Sec. 3.1 / Eq. (1), Fig. 2;
 *   P3  alphasignal.ai summary ("Pyramid Pool" bullet);
 *   P4  aibriefing.imbch.dev summary ("three key points").
 * Everything is fp64 except the selection scores, which are fp32 in a fixed
 * reduction order so that the selected index set is reproducible bit for bit.
 *
 * Readings taken where the pages leave a step open:
 *   R1 score of an entry = ||q||^2 + ||k||^2 of its leaves (no sqrt: monotone),
 *      coarser levels take the max over their p children (Fig. 2 "l2 norm +
 *      max-pool").  The other readings of what the norm is taken of (Sec. 1
 *      "bidirectional"; Fig. 2 "qk scores kq") are score modes: 1 = ||k||^2,
 *      2 = ||q||^2, 3 = ||q||^2 * ||k||^2 (ranks as ||q|| ||k||; one fp32
 *      multiply of the two fixed-order sums);
 *   R2 selection is top-down: K entries per level and per head, ordered by
 *      (score descending, index ascending); a selected entry is replaced by
 *      its p children, an unselected candidate is kept as it is, so the kept
 *      entries partition [0, N) (Fig. 2 "bitonic argsort + tree-prune");
 *   R3 kept entries are ordered by their first token to form the causal
 *      sub-sequence (Fig. 1 caption; P4 "hole-free causal sequence");
 *   R4 attention on the sub-sequence is Eq. (1) with scale 1/sqrt(d) and the
 *      ordinary lower-triangular mask;
 *   R5 scatter copies each output to the p^l tokens its entry covers
 *      (Sec. 3 stage (iv)); the gradient of the mean-pool divides by p^l.
 *   R2' the other reading of "parent kept" (select mode 1): a selected entry
 *      stays in the sequence next to its p children, so every candidate of
 *      every level is kept and the entries overlap; they are ordered by first
 *      token, the coarser entry first where two start together; a token's
 *      output is the sum of the outputs of the entries that cover it, and
 *      the adjoints sum likewise.
 *
 * dtype codes: 0 = bf16 (raw uint16 bit patterns), 1 = fp32.
 * Tensors q, k, v, dO, O, dq, dk, dv are [N][H][d] (token-major); the
 * sub-sequence tensors are [H][S][d]; scores are [H][n_l] per level.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define LHO_OK 0
#define LHO_ERR_ARG (-1)
#define LHO_ERR_MEM (-2)

/* ---------------------------------------------------------------- helpers */

static int64_t ipow(int64_t b, int e) {
    int64_t r = 1;
    for (int i = 0; i < e; ++i) r *= b;
    return r;
}

/* Exact conversion of one stored element to fp32. */
static float load_f32(const void* x, int dtype, int64_t i) {
    if (dtype == 0) {
        uint32_t b = (uint32_t)((const uint16_t*)x)[i] << 16;
        float f;
        memcpy(&f, &b, sizeof f);
        return f;
    }
    return ((const float*)x)[i];
}

static int check_shape(int N, int H, int d, int dtype, int p, int L, int K) {
    if (N <= 0 || H <= 0 || p < 2 || L < 1 || K < 0) return LHO_ERR_ARG;
    if (dtype != 0 && dtype != 1) return LHO_ERR_ARG;
    if (d < 8 || d % 8 != 0) return LHO_ERR_ARG;
    int G = d / 8;
    if (G & (G - 1)) return LHO_ERR_ARG;      /* groups combine by a power-of-two butterfly */
    int64_t top = ipow(p, L - 1);
    if (top > N || N % top != 0) return LHO_ERR_ARG;
    return LHO_OK;
}

/* ------------------------------------------------------- sub-sequence size */

/* Number of kept entries S for (N, p, L, K) under reading R2: start with all
 * N/p^(L-1) top entries; each of the min(K, #candidates) selections at a
 * level replaces one entry by p children. */
int64_t lho_subseq_len_sel(int N, int p, int L, int K, int select_mode) {
    if (N <= 0 || p < 2 || L < 1 || K < 0 || select_mode < 0 || select_mode > 1) return -1;
    int64_t top = ipow(p, L - 1);
    if (top > N || N % top != 0) return -1;
    int64_t n = N / top, S = n, cand = n;
    for (int l = L - 1; l >= 1; --l) {
        int64_t sel = cand < K ? cand : K;
        /* partition: a selected entry gives way to its p children; parent kept: it stays */
        S += sel * (select_mode ? p : p - 1);
        cand = sel * p;
    }
    return S;
}

int64_t lho_subseq_len(int N, int p, int L, int K) { return lho_subseq_len_sel(N, p, L, K, 0); }

/* ------------------------------------------------------------- pyramid (O1) */

/* Mean of the p children one level down, recursively (Sec. 3 stage (i),
 * Fig. 2 step 1: level l averages p^l tokens).  `scratch` holds (lev)*d
 * doubles for the recursion. */
static void pooled_row(const void* x, int dtype, int H, int d, int h, int p,
                       int lev, int64_t j, double* out, double* scratch) {
    if (lev == 0) {
        int64_t base = (j * H + h) * (int64_t)d;
        for (int e = 0; e < d; ++e) out[e] = (double)load_f32(x, dtype, base + e);
        return;
    }
    double* child = scratch;
    for (int e = 0; e < d; ++e) out[e] = 0.0;
    for (int c = 0; c < p; ++c) {
        pooled_row(x, dtype, H, d, h, p, lev - 1, (int64_t)p * j + c, child, scratch + d);
        for (int e = 0; e < d; ++e) out[e] += child[e];
    }
    for (int e = 0; e < d; ++e) out[e] /= (double)p;
}

/* Full pyramid, levels 1..L-1, each [N/p^l][H][d] fp64, concatenated. */
int lho_pyramid(const void* x, int N, int H, int d, int dtype, int p, int L, double* out) {
    int rc = check_shape(N, H, d, dtype, p, L, 0);
    if (rc) return rc;
    int64_t off = 0;
    double* scratch = (double*)malloc(sizeof(double) * (size_t)d * (size_t)(L + 1));
    if (!scratch) return LHO_ERR_MEM;
    for (int l = 1; l < L; ++l) {
        int64_t n = N / ipow(p, l);
        for (int64_t j = 0; j < n; ++j)
            for (int h = 0; h < H; ++h)
                pooled_row(x, dtype, H, d, h, p, l, j, out + off + (j * H + h) * (int64_t)d, scratch);
        off += n * H * (int64_t)d;
    }
    free(scratch);
    return LHO_OK;
}

/* --------------------------------------------------------------- scores (O2, O3) */

/* Sum of squares of d exact fp32 values in the fixed order of reading R1:
 * groups of 8 consecutive elements, each accumulated by fmaf from +0 in
 * element order, then the d/8 group sums combined by a xor butterfly
 * (a_g <- a_g + a_(g^off) for off = G/2 .. 1); the result is a_0. */
static float ssq_fixed_order(const float* x, int d) {
    int G = d / 8;
    float a[64], b[64];
    for (int g = 0; g < G; ++g) {
        float acc = 0.0f;
        for (int e = 0; e < 8; ++e) acc = fmaf(x[8 * g + e], x[8 * g + e], acc);
        a[g] = acc;
    }
    for (int off = G / 2; off >= 1; off /= 2) {
        for (int g = 0; g < G; ++g) b[g] = a[g] + a[g ^ off];
        for (int g = 0; g < G; ++g) a[g] = b[g];
    }
    return a[0];
}

/* Leaf score from the two fixed-order sums of squares, by score mode (R1). */
static float leaf_score(float sq, float sk, int mode) {
    switch (mode) {
        case 1: return sk;
        case 2: return sq;
        case 3: return sq * sk;
        default: return sq + sk;
    }
}

static void head_leaf_scores(const void* q, const void* k, int N, int H, int d, int dtype, int mode, int h,
                             float* s0) {
    float xq[512], xk[512];
    for (int64_t t = 0; t < N; ++t) {
        int64_t base = (t * H + h) * (int64_t)d;
        for (int e = 0; e < d; ++e) {
            xq[e] = load_f32(q, dtype, base + e);
            xk[e] = load_f32(k, dtype, base + e);
        }
        s0[t] = leaf_score(ssq_fixed_order(xq, d), ssq_fixed_order(xk, d), mode);
    }
}

/* Same quantity in fp64 with plain sums, for the near-tie report only. */
static void head_leaf_scores64(const void* q, const void* k, int N, int H, int d, int dtype, int mode, int h,
                               double* s0) {
    for (int64_t t = 0; t < N; ++t) {
        int64_t base = (t * H + h) * (int64_t)d;
        double aq = 0.0, ak = 0.0;
        for (int e = 0; e < d; ++e) {
            double a = load_f32(q, dtype, base + e), b = load_f32(k, dtype, base + e);
            aq += a * a;
            ak += b * b;
        }
        s0[t] = mode == 1 ? ak : mode == 2 ? aq : mode == 3 ? aq * ak : aq + ak;
    }
}

/* Leaf scores for every head: s0 is [H][N]. */
int lho_leaf_scores(const void* q, const void* k, int N, int H, int d, int dtype, int mode, float* s0) {
    int rc = check_shape(N, H, d, dtype, 2, 1, 0);
    if (rc) return rc;
    if (d > 512 || mode < 0 || mode > 3) return LHO_ERR_ARG;
    for (int h = 0; h < H; ++h) head_leaf_scores(q, k, N, H, d, dtype, mode, h, s0 + (int64_t)h * N);
    return LHO_OK;
}

/* Score of a level-l entry = max of its p children (Fig. 2 step 2). */
static void max_pool_levels_f32(float** lev, int N, int p, int L) {
    for (int l = 1; l < L; ++l) {
        int64_t n = N / ipow(p, l);
        for (int64_t j = 0; j < n; ++j) {
            float m = lev[l - 1][(int64_t)p * j];
            for (int c = 1; c < p; ++c) {
                float v = lev[l - 1][(int64_t)p * j + c];
                if (v > m) m = v;
            }
            lev[l][j] = m;
        }
    }
}

static void max_pool_levels_f64(double** lev, int N, int p, int L) {
    for (int l = 1; l < L; ++l) {
        int64_t n = N / ipow(p, l);
        for (int64_t j = 0; j < n; ++j) {
            double m = lev[l - 1][(int64_t)p * j];
            for (int c = 1; c < p; ++c) {
                double v = lev[l - 1][(int64_t)p * j + c];
                if (v > m) m = v;
            }
            lev[l][j] = m;
        }
    }
}

/* ----------------------------------------------------------- selection (O4, O5) */

typedef struct {
    uint32_t bits;   /* fp32 score bit pattern; scores are >= +0 so this orders them */
    int64_t idx;
} key_t_;

static int key_cmp(const void* pa, const void* pb) {
    const key_t_* a = (const key_t_*)pa;
    const key_t_* b = (const key_t_*)pb;
    if (a->bits != b->bits) return a->bits > b->bits ? -1 : 1;   /* larger score first */
    if (a->idx != b->idx) return a->idx < b->idx ? -1 : 1;       /* then lower index   */
    return 0;
}

static int i64_cmp(const void* pa, const void* pb) {
    int64_t a = *(const int64_t*)pa, b = *(const int64_t*)pb;
    return a < b ? -1 : (a > b ? 1 : 0);
}

typedef struct {
    int64_t start;
    int level;
} entry_t;

static int entry_cmp(const void* pa, const void* pb) {
    const entry_t* a = (const entry_t*)pa;
    const entry_t* b = (const entry_t*)pb;
    if (a->start != b->start) return a->start < b->start ? -1 : 1;
    return a->level > b->level ? -1 : (a->level < b->level ? 1 : 0);   /* coarser first (R2') */
}

static uint32_t f32_bits(float f) {
    uint32_t b;
    memcpy(&b, &f, sizeof b);
    return b;
}

/* Top-down tree selection for one head (reading R2), then ordering by start
 * (reading R3).  lev[l] holds the fp32 scores of level l.  Writes S entries
 * to start/level and returns S (or -1 on allocation failure).  lev64 (may be
 * NULL) gives fp64 scores for the near-tie count. */
static int64_t head_select(float** lev, double** lev64, int N, int p, int L, int K, int select_mode,
                           int32_t* start_out, int8_t* level_out, int* near_ties) {
    int64_t n_top = N / ipow(p, L - 1);
    int64_t cap = n_top > (int64_t)K * p ? n_top : (int64_t)K * p;
    int64_t S_max = lho_subseq_len_sel(N, p, L, K, select_mode);
    int64_t* cand = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    int64_t* next = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (size_t)(K + 1));
    key_t_* keys = (key_t_*)malloc(sizeof(key_t_) * (size_t)cap);
    entry_t* E = (entry_t*)malloc(sizeof(entry_t) * (size_t)S_max);
    if (!cand || !next || !sel || !keys || !E) {
        free(cand); free(next); free(sel); free(keys); free(E);
        return -1;
    }
    int64_t ncand = n_top, nE = 0;
    for (int64_t j = 0; j < n_top; ++j) cand[j] = j;
    for (int l = L - 1; l >= 1; --l) {
        for (int64_t c = 0; c < ncand; ++c) {
            keys[c].bits = f32_bits(lev[l][cand[c]]);
            keys[c].idx = cand[c];
        }
        qsort(keys, (size_t)ncand, sizeof(key_t_), key_cmp);
        int64_t nsel = ncand < K ? ncand : K;
        if (near_ties && lev64 && nsel > 0 && nsel < ncand) {
            double a = lev64[l][keys[nsel - 1].idx], b = lev64[l][keys[nsel].idx];
            if (fabs(a - b) <= 1e-6 * fabs(a)) ++*near_ties;
        }
        for (int64_t s = 0; s < nsel; ++s) sel[s] = keys[s].idx;
        qsort(sel, (size_t)nsel, sizeof(int64_t), i64_cmp);
        /* candidates not selected are kept at this level (cand is ascending);
           with the parent kept (R2') the selected ones are kept as well */
        int64_t s = 0;
        for (int64_t c = 0; c < ncand; ++c) {
            if (s < nsel && sel[s] == cand[c]) {
                ++s;
                if (!select_mode) continue;
            }
            E[nE].start = cand[c] * ipow(p, l);
            E[nE].level = l;
            ++nE;
        }
        /* children of the selected entries become the next candidates */
        int64_t nn = 0;
        for (int64_t i = 0; i < nsel; ++i)
            for (int c = 0; c < p; ++c) next[nn++] = sel[i] * p + c;
        int64_t* tmp = cand; cand = next; next = tmp;
        ncand = nn;
    }
    for (int64_t c = 0; c < ncand; ++c) {        /* level 0: every candidate is kept */
        E[nE].start = cand[c];
        E[nE].level = 0;
        ++nE;
    }
    qsort(E, (size_t)nE, sizeof(entry_t), entry_cmp);
    for (int64_t i = 0; i < nE; ++i) {
        start_out[i] = (int32_t)E[i].start;
        level_out[i] = (int8_t)E[i].level;
    }
    free(cand); free(next); free(sel); free(keys); free(E);
    return nE;
}

/* ------------------------------------------------------------ attention (O6, O8) */

/* The logits s_ij = Q_i . K_j / sqrt(d) of query i for every visible key
 * j <= i (the causal mask of Eq. (1)), their maximum and the sum of
 * exp(s_ij - max). */
static void row_logits(int64_t i, int d, const double* Q, const double* K, double* logit, double* m_out,
                       double* sum_out) {
    double scale = 1.0 / sqrt((double)d);
    double m = -INFINITY;
    for (int64_t j = 0; j <= i; ++j) {
        double acc = 0.0;
        for (int e = 0; e < d; ++e) acc += Q[i * d + e] * K[j * d + e];
        logit[j] = acc * scale;
        if (logit[j] > m) m = logit[j];
    }
    double sum = 0.0;
    for (int64_t j = 0; j <= i; ++j) sum += exp(logit[j] - m);
    *m_out = m;
    *sum_out = sum;
}

/* Eq. (1) for query row i of one head: O_i = sum_j softmax_j(s_ij) V_j (a
 * two-pass softmax) and lse_i. */
static void attn_fwd_row(int64_t i, int d, const double* Q, const double* K, const double* V, double* O,
                         double* lse, double* logit) {
    double m, sum;
    row_logits(i, d, Q, K, logit, &m, &sum);
    for (int e = 0; e < d; ++e) O[i * d + e] = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
        double w = exp(logit[j] - m) / sum;
        for (int e = 0; e < d; ++e) O[i * d + e] += w * V[j * d + e];
    }
    if (lse) lse[i] = m + log(sum);
}

/* Gradient of the above: P = softmax, dV = P^T dO, dP = dO V^T,
 * dS = P o (dP - rowsum(dO o O)), dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d).
 *
 * cond (may be NULL) receives, for the tolerance of finite-precision
 * comparisons only, 8 arrays of S*d.  The first four are the sums of absolute
 * values of the terms each output is made of (O, dQ, dK, dV).  With
 * A_ij = sum |dO_i||V_j|, B_i = sum |dO_i||O_i| and w_ij = P_ij (A_ij + B_i):
 *   cO_i = sum_j P_ij |V_j|,  cdQ_i = sum_j w_ij |K_j| / sqrt(d),
 *   cdK_j = sum_i w_ij |Q_i| / sqrt(d),  cdV_j = sum_i P_ij |dO_i|.
 * A computation in precision u with length-n dot products has error of order
 * n u times these sums (the standard forward error bound of a dot product).
 * The last four bound, to first order, how far each output moves when every
 * logit s_ij is perturbed by at most Lam_ij = sum_e |Q_ie K_je| / sqrt(d) (the
 * size of the rounding error of a dot product computed in precision 1, scaled
 * by u for precision u) and, separately, the log-sum-exp of each row by at
 * most |lse_i| (its own rounding where it is stored apart from the logits and
 * read back by the gradient).  With M_i = sum_k P_ik Lam_ik + |lse_i|,
 * a_ij = |dP_ij - D_i| and R_i = sum_k P_ik Lam_ik a_ik, such a perturbation
 * moves the gradient's weights P_ij = exp(s_ij - lse_i) by at most
 * P_ij (Lam_ij + M_i), O_i (normalised by its own sum) by at most
 * sum_j P_ij Lam_ij |V_j - O_i| (dO_i/ds_ij = P_ij (V_j - O_i)),
 * D_i = dO_i . O_i by at most R_i, and dS_ij by at most
 * W_ij = P_ij ((Lam_ij + M_i) a_ij + R_i), so:
 *   lO_i = sum_j P_ij Lam_ij |V_j - O_i|,  ldQ_i = sum_j W_ij |K_j| / sqrt(d),
 *   ldK_j = sum_i W_ij |Q_i| / sqrt(d),  ldV_j = sum_i P_ij (Lam_ij + M_i) |dO_i|.
 * Where logits are large (heavy-tailed rows) these dominate the first four. */
/* The gradient is computed in two passes, each a loop over independent rows:
 * the query side (attn_bwd_query_row: dQ_i, the row's statistics, and P_ij,
 * dS_ij for j <= i, stored row by row in packed lower-triangular arrays at
 * tri(i) + j) and the key side (attn_bwd_key_row: dK_j and dV_j, adding the
 * stored P_ij and dS_ij over i >= j in increasing i).  Every sum is taken in
 * the same order as one loop over i then j would take it.  rs[i] holds m,
 * sum, D, B, M, R of row i; cz the 8 condition arrays of the head (or NULL)
 * and, with them, wt[3] the packed per-pair weights w_ij, W_ij and
 * P_ij (Lam_ij + M_i) that the key side needs; lam, adp: scratch. */
static int64_t tri(int64_t i) { return i * (i + 1) / 2; }
enum { RS_M, RS_SUM, RS_D, RS_B, RS_LM, RS_R, RS_N };

static void attn_bwd_query_row(int64_t i, int d, const double* Q, const double* K, const double* V,
                               const double* O, const double* dO, double* dQ, double* rs, double* Pt,
                               double* dSt, double* logit, double* lam, double* adp, double* const* cz,
                               double* const* wt) {
    double scale = 1.0 / sqrt((double)d);
    double m, sum;
    row_logits(i, d, Q, K, logit, &m, &sum);
    double D = 0.0, B = 0.0;
    for (int e = 0; e < d; ++e) {
        D += dO[i * d + e] * O[i * d + e];
        B += fabs(dO[i * d + e] * O[i * d + e]);
    }
    double M = fabs(m + log(sum)), R = 0.0;   /* |lse_i| + sum_k P_ik Lam_ik */
    if (cz) {
        for (int64_t j = 0; j <= i; ++j) {
            double P = exp(logit[j] - m) / sum, la = 0.0, dP = 0.0;
            for (int e = 0; e < d; ++e) {
                la += fabs(Q[i * d + e] * K[j * d + e]);
                dP += dO[i * d + e] * V[j * d + e];
            }
            lam[j] = la * scale;
            adp[j] = fabs(dP - D);
            M += P * lam[j];
            R += P * lam[j] * adp[j];
        }
    }
    for (int e = 0; e < d; ++e) dQ[i * d + e] = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
        double P = exp(logit[j] - m) / sum;
        double dP = 0.0, A = 0.0;
        for (int e = 0; e < d; ++e) {
            dP += dO[i * d + e] * V[j * d + e];
            A += fabs(dO[i * d + e] * V[j * d + e]);
        }
        double dS = P * (dP - D);
        Pt[tri(i) + j] = P;
        dSt[tri(i) + j] = dS;
        for (int e = 0; e < d; ++e) dQ[i * d + e] += dS * K[j * d + e] * scale;
        if (cz) {
            double w = P * (A + B);
            double wl = P * ((lam[j] + M) * adp[j] + R);
            wt[0][tri(i) + j] = w;
            wt[1][tri(i) + j] = wl;
            wt[2][tri(i) + j] = P * (lam[j] + M);
            for (int e = 0; e < d; ++e) {
                cz[0][i * d + e] += P * fabs(V[j * d + e]);
                cz[1][i * d + e] += w * fabs(K[j * d + e]) * scale;
                cz[4][i * d + e] += P * lam[j] * fabs(V[j * d + e] - O[i * d + e]);
                cz[5][i * d + e] += wl * fabs(K[j * d + e]) * scale;
            }
        }
    }
    double* r = rs + i * RS_N;
    r[RS_M] = m; r[RS_SUM] = sum; r[RS_D] = D; r[RS_B] = B; r[RS_LM] = M; r[RS_R] = R;
}

static void attn_bwd_key_row(int64_t j, int64_t S, int d, const double* Q, const double* dO, const double* Pt,
                             const double* dSt, double* dK, double* dV, double* const* cz,
                             const double* const* wt) {
    double scale = 1.0 / sqrt((double)d);
    for (int e = 0; e < d; ++e) dK[j * d + e] = dV[j * d + e] = 0.0;
    for (int64_t i = j; i < S; ++i) {
        double P = Pt[tri(i) + j], dS = dSt[tri(i) + j];
        for (int e = 0; e < d; ++e) {
            dK[j * d + e] += dS * Q[i * d + e] * scale;
            dV[j * d + e] += P * dO[i * d + e];
        }
        if (cz) {
            double w = wt[0][tri(i) + j], wl = wt[1][tri(i) + j], plm = wt[2][tri(i) + j];
            for (int e = 0; e < d; ++e) {
                cz[2][j * d + e] += w * fabs(Q[i * d + e]) * scale;
                cz[3][j * d + e] += P * fabs(dO[i * d + e]);
                cz[6][j * d + e] += wl * fabs(Q[i * d + e]) * scale;
                cz[7][j * d + e] += plm * fabs(dO[i * d + e]);
            }
        }
    }
}

/* ------------------------------------------------------------- per-head work */

typedef struct {
    const void *q, *k, *v, *dout;
    int N, H, d, dtype, p, L, K;
    int64_t S;
    int score_mode;   /* R1 and its alternatives, see leaf_score */
    int select_mode;  /* 0: partition (R2), 1: parent kept (R2') */
} ctx_t;

/* Scores, levels and the selection for head h.  Returns 0 or an error. */
static int head_scores_select(const ctx_t* c, int h, float* levels_out, int32_t* st, int8_t* lv,
                              int* near_ties) {
    int L = c->L;
    float** lev = (float**)calloc((size_t)L, sizeof(float*));
    double** lev64 = near_ties ? (double**)calloc((size_t)L, sizeof(double*)) : NULL;
    int rc = LHO_OK;
    if (!lev || (near_ties && !lev64)) { rc = LHO_ERR_MEM; goto done; }
    for (int l = 0; l < L; ++l) {
        lev[l] = (float*)malloc(sizeof(float) * (size_t)(c->N / ipow(c->p, l)));
        if (!lev[l]) { rc = LHO_ERR_MEM; goto done; }
        if (lev64) {
            lev64[l] = (double*)malloc(sizeof(double) * (size_t)(c->N / ipow(c->p, l)));
            if (!lev64[l]) { rc = LHO_ERR_MEM; goto done; }
        }
    }
    head_leaf_scores(c->q, c->k, c->N, c->H, c->d, c->dtype, c->score_mode, h, lev[0]);
    max_pool_levels_f32(lev, c->N, c->p, L);
    if (lev64) {
        head_leaf_scores64(c->q, c->k, c->N, c->H, c->d, c->dtype, c->score_mode, h, lev64[0]);
        max_pool_levels_f64(lev64, c->N, c->p, L);
    }
    if (levels_out) {
        /* level l of head h lives at H*sum_{l'<l} n_l' + h*n_l */
        int64_t off = 0;
        for (int l = 0; l < L; ++l) {
            int64_t n = c->N / ipow(c->p, l);
            memcpy(levels_out + off + (int64_t)h * n, lev[l], sizeof(float) * (size_t)n);
            off += n * c->H;
        }
    }
    if (st) {
        int64_t S = head_select(lev, lev64, c->N, c->p, L, c->K, c->select_mode, st, lv, near_ties);
        if (S != c->S) rc = LHO_ERR_MEM;
    }
done:
    if (lev) for (int l = 0; l < L; ++l) free(lev[l]);
    if (lev64) for (int l = 0; l < L; ++l) free(lev64[l]);
    free(lev);
    free(lev64);
    return rc;
}

/* Gather (O5): row i of the sub-sequence is the level-l_i pyramid entry that
 * starts at token start_i. */
static void head_gather(const ctx_t* c, const void* x, int h, const int32_t* st, const int8_t* lv,
                        double* out, double* scratch) {
    for (int64_t i = 0; i < c->S; ++i) {
        int l = lv[i];
        int64_t j = st[i] / ipow(c->p, l);
        pooled_row(x, c->dtype, c->H, c->d, h, c->p, l, j, out + i * c->d, scratch);
    }
}

/* ----------------------------------------------------------------- public API */

/*
 * Forward pass (Fig. 1 forward path).  Output pointers may be NULL.
 *   score_mode: 0 = ||q||^2 + ||k||^2 (R1), 1 = ||k||^2, 2 = ||q||^2,
 *       3 = ||q||^2 * ||k||^2
 *   score_levels [sum_l H*N/p^l] fp32, level-major then [H][n_l]
 *   sel_start, sel_level [H][S]: written unless given_sel != 0, in which case
 *       they are read (the selection is frozen; used for finite differences)
 *   Qt, Kt, Vt, Ot [H][S][d], lse [H][S]
 *   O [N][H][d]
 *   near_ties [H]: count of selection boundaries whose fp64 scores are within
 *       1e-6 relative (reported, not an error)
 */
int lho_forward(const void* q, const void* k, const void* v, int N, int H, int d, int dtype,
                int p, int L, int K, int score_mode, int select_mode, int given_sel, float* score_levels,
                int32_t* sel_start, int8_t* sel_level, double* Qt, double* Kt, double* Vt,
                double* Ot, double* lse, double* O, int* near_ties, int nthreads) {
    int rc = check_shape(N, H, d, dtype, p, L, K);
    if (rc) return rc;
    if (d > 512 || !sel_start || !sel_level) return LHO_ERR_ARG;
    if (score_mode < 0 || score_mode > 3 || select_mode < 0 || select_mode > 1) return LHO_ERR_ARG;
    ctx_t c = {q, k, v, NULL, N, H, d, dtype, p, L, K, lho_subseq_len_sel(N, p, L, K, select_mode), score_mode,
               select_mode};
    int64_t S = c.S;
    size_t sd = (size_t)(S * d);
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int need_attn = Ot || lse || O;
    int need_rows = Qt || Kt || Vt || need_attn;
    /* every head's gathered rows, output rows and lse, for the row-parallel attention */
    double* Qa = need_rows ? (double*)malloc(sizeof(double) * sd * (size_t)H) : NULL;
    double* Ka = need_rows ? (double*)malloc(sizeof(double) * sd * (size_t)H) : NULL;
    double* Va = need_rows ? (double*)malloc(sizeof(double) * sd * (size_t)H) : NULL;
    double* Oa = need_attn ? (double*)malloc(sizeof(double) * sd * (size_t)H) : NULL;
    double* la = need_attn ? (double*)malloc(sizeof(double) * (size_t)S * (size_t)H) : NULL;
    if (need_rows && (!Qa || !Ka || !Va || (need_attn && (!Oa || !la)))) {
        free(Qa); free(Ka); free(Va); free(Oa); free(la);
        return LHO_ERR_MEM;
    }
    /* scores, selection (O2-O4) and gather (O5), one head at a time */
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int h = 0; h < H; ++h) {
        int32_t* st = sel_start + (int64_t)h * S;
        int8_t* lv = sel_level + (int64_t)h * S;
        if (near_ties) near_ties[h] = 0;
        if (!given_sel || score_levels) {
            if (head_scores_select(&c, h, score_levels, given_sel ? NULL : st, given_sel ? NULL : lv,
                                   (near_ties && !given_sel) ? &near_ties[h] : NULL)) {
                err |= 1;
                continue;
            }
        }
        if (!need_rows) continue;
        double* scratch = (double*)malloc(sizeof(double) * (size_t)d * (size_t)(L + 1));
        if (!scratch) {
            err |= 1;
            continue;
        }
        head_gather(&c, q, h, st, lv, Qa + (size_t)h * sd, scratch);
        head_gather(&c, k, h, st, lv, Ka + (size_t)h * sd, scratch);
        head_gather(&c, v, h, st, lv, Va + (size_t)h * sd, scratch);
        free(scratch);
    }
    /* attention (O6), one query row of one head at a time */
    if (!err && need_attn) {
#pragma omp parallel reduction(| : err)
        {
            double* logit = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
            if (!logit) err |= 1;
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < (int64_t)H * S; ++r) {
                if (!logit) continue;
                int64_t h = r / S, i = r % S;
                attn_fwd_row(i, d, Qa + h * sd, Ka + h * sd, Va + h * sd, Oa + h * sd, la + h * S, logit);
            }
            free(logit);
        }
    }
    /* outputs and the scatter (O7), one head at a time */
    if (!err && need_rows) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int h = 0; h < H; ++h) {
            const int32_t* st = sel_start + (int64_t)h * S;
            const int8_t* lv = sel_level + (int64_t)h * S;
            if (Qt) memcpy(Qt + (int64_t)h * S * d, Qa + (size_t)h * sd, sizeof(double) * sd);
            if (Kt) memcpy(Kt + (int64_t)h * S * d, Ka + (size_t)h * sd, sizeof(double) * sd);
            if (Vt) memcpy(Vt + (int64_t)h * S * d, Va + (size_t)h * sd, sizeof(double) * sd);
            if (Ot) memcpy(Ot + (int64_t)h * S * d, Oa + (size_t)h * sd, sizeof(double) * sd);
            if (lse) memcpy(lse + (int64_t)h * S, la + (size_t)h * S, sizeof(double) * (size_t)S);
            if (O) {
                /* every token of entry i receives row i; with overlapping entries
                   (R2') a token sums the rows it receives */
                const double* Oh = Oa + (size_t)h * sd;
                for (int64_t t = 0; t < N; ++t)
                    for (int e = 0; e < d; ++e) O[(t * H + h) * (int64_t)d + e] = 0.0;
                for (int64_t i = 0; i < S; ++i) {
                    int64_t len = ipow(p, lv[i]);
                    for (int64_t t = st[i]; t < st[i] + len; ++t)
                        for (int e = 0; e < d; ++e) O[(t * H + h) * (int64_t)d + e] += Oh[i * d + e];
                }
            }
        }
    }
    free(Qa); free(Ka); free(Va); free(Oa); free(la);
    return err ? LHO_ERR_MEM : LHO_OK;
}

/*
 * Backward pass (Fig. 1 gradient path: O -> scatter -> attention -> gather ->
 * pool).  The selection (sel_start, sel_level from lho_forward) is an input:
 * indices carry no gradient.  Output pointers may be NULL.
 *   dOt, dQt, dKt, dVt [H][S][d];  dq, dk, dv [N][H][d]
 *   cond [8][H][S][d]: absolute term sums of O~, dQ~, dK~, dV~, then their
 *   first-order sensitivities to the rounding of the logits (see
 *   head_attention_bwd); a tolerance aid, not part of the layer.
 */
int lho_backward(const void* q, const void* k, const void* v, const void* dout, int N, int H, int d,
                 int dtype, int p, int L, int K, int select_mode, const int32_t* sel_start, const int8_t* sel_level,
                 double* dOt, double* dQt, double* dKt, double* dVt, double* dq, double* dk, double* dv,
                 double* cond, int nthreads) {
    int rc = check_shape(N, H, d, dtype, p, L, K);
    if (rc) return rc;
    if (d > 512 || !sel_start || !sel_level || !dout) return LHO_ERR_ARG;
    if (select_mode < 0 || select_mode > 1) return LHO_ERR_ARG;
    ctx_t c = {q, k, v, dout, N, H, d, dtype, p, L, K, lho_subseq_len_sel(N, p, L, K, select_mode), 0,
               select_mode};
    int64_t S = c.S;
    size_t sd = (size_t)(S * d), hsd = sd * (size_t)H;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    /* every head's rows: Q, K, V, O, dO, dQ, dK, dV, and the query rows' statistics */
    double* buf = (double*)malloc(sizeof(double) * hsd * 8);
    double* rs = (double*)malloc(sizeof(double) * (size_t)(H * S * RS_N > 0 ? H * S * RS_N : 1));
    if (!buf || !rs) {
        free(buf); free(rs);
        return LHO_ERR_MEM;
    }
    double *Qa = buf, *Ka = buf + hsd, *Va = buf + 2 * hsd, *Oa = buf + 3 * hsd;
    double *dOa = buf + 4 * hsd, *dQa = buf + 5 * hsd, *dKa = buf + 6 * hsd, *dVa = buf + 7 * hsd;
    if (cond) memset(cond, 0, sizeof(double) * hsd * 8);
    /* gather (O5) and the adjoint of the scatter (O8): an entry's dO is the sum
       over its tokens; one head at a time */
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int h = 0; h < H; ++h) {
        const int32_t* st = sel_start + (int64_t)h * S;
        const int8_t* lv = sel_level + (int64_t)h * S;
        double* scratch = (double*)malloc(sizeof(double) * (size_t)d * (size_t)(L + 1));
        if (!scratch) {
            err |= 1;
            continue;
        }
        head_gather(&c, q, h, st, lv, Qa + (size_t)h * sd, scratch);
        head_gather(&c, k, h, st, lv, Ka + (size_t)h * sd, scratch);
        head_gather(&c, v, h, st, lv, Va + (size_t)h * sd, scratch);
        double* dOh = dOa + (size_t)h * sd;
        for (int64_t i = 0; i < S; ++i) {
            int64_t len = ipow(p, lv[i]);
            for (int e = 0; e < d; ++e) dOh[i * d + e] = 0.0;
            for (int64_t t = st[i]; t < st[i] + len; ++t) {
                int64_t base = (t * H + h) * (int64_t)d;
                for (int e = 0; e < d; ++e) dOh[i * d + e] += (double)load_f32(dout, dtype, base + e);
            }
        }
        free(scratch);
    }
    /* attention forward (O6) for O, then the gradient (O8): the query side and
       the key side; one head after the other, its rows in parallel */
    size_t ntri = (size_t)(tri(S) > 0 ? tri(S) : 1);
    double* Pt = (double*)malloc(sizeof(double) * ntri);
    double* dSt = (double*)malloc(sizeof(double) * ntri);
    double* wt[3] = {NULL, NULL, NULL};
    for (int z = 0; z < 3 && cond; ++z) {
        wt[z] = (double*)malloc(sizeof(double) * ntri);
        if (!wt[z]) err |= 1;
    }
    if (!Pt || !dSt) err |= 1;
    for (int64_t h = 0; h < H && !err; ++h) {
        double* cz[8];
        for (int z = 0; z < 8; ++z) cz[z] = cond ? cond + ((size_t)z * H + (size_t)h) * sd : NULL;
        const double *Qh = Qa + h * sd, *Kh = Ka + h * sd, *Vh = Va + h * sd, *dOh = dOa + h * sd;
        double* Oh = Oa + h * sd;
        double* rh = rs + h * S * RS_N;
#pragma omp parallel reduction(| : err)
        {
            double* tmp = (double*)malloc(sizeof(double) * 3 * (size_t)(S > 0 ? S : 1));
            if (!tmp) err |= 1;
#pragma omp for schedule(dynamic, 16)
            for (int64_t i = 0; i < S; ++i)
                if (tmp) attn_fwd_row(i, d, Qh, Kh, Vh, Oh, NULL, tmp);
#pragma omp for schedule(dynamic, 16)
            for (int64_t i = 0; i < S; ++i)
                if (tmp)
                    attn_bwd_query_row(i, d, Qh, Kh, Vh, Oh, dOh, dQa + h * sd, rh, Pt, dSt, tmp, tmp + S, tmp + 2 * S,
                                       cond ? cz : NULL, wt);
#pragma omp for schedule(dynamic, 16)
            for (int64_t j = 0; j < S; ++j)
                attn_bwd_key_row(j, S, d, Qh, dOh, Pt, dSt, dKa + h * sd, dVa + h * sd, cond ? cz : NULL,
                                 (const double* const*)wt);
            free(tmp);
        }
    }
    free(Pt);
    free(dSt);
    for (int z = 0; z < 3; ++z) free(wt[z]);
    /* outputs and the adjoint of the mean-pool: each of the p^l tokens gets
       1/p^l of it, summed over the entries that cover the token (one of them
       unless R2'); one head at a time */
    if (!err) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int h = 0; h < H; ++h) {
            const int32_t* st = sel_start + (int64_t)h * S;
            const int8_t* lv = sel_level + (int64_t)h * S;
            const double *dQh = dQa + (size_t)h * sd, *dKh = dKa + (size_t)h * sd, *dVh = dVa + (size_t)h * sd;
            if (dOt) memcpy(dOt + (int64_t)h * S * d, dOa + (size_t)h * sd, sizeof(double) * sd);
            if (dQt) memcpy(dQt + (int64_t)h * S * d, dQh, sizeof(double) * sd);
            if (dKt) memcpy(dKt + (int64_t)h * S * d, dKh, sizeof(double) * sd);
            if (dVt) memcpy(dVt + (int64_t)h * S * d, dVh, sizeof(double) * sd);
            for (int64_t t = 0; t < N; ++t) {
                int64_t base = (t * H + h) * (int64_t)d;
                for (int e = 0; e < d; ++e) {
                    if (dq) dq[base + e] = 0.0;
                    if (dk) dk[base + e] = 0.0;
                    if (dv) dv[base + e] = 0.0;
                }
            }
            for (int64_t i = 0; i < S; ++i) {
                int64_t len = ipow(p, lv[i]);
                for (int64_t t = st[i]; t < st[i] + len; ++t) {
                    int64_t base = (t * H + h) * (int64_t)d;
                    for (int e = 0; e < d; ++e) {
                        if (dq) dq[base + e] += dQh[i * d + e] / (double)len;
                        if (dk) dk[base + e] += dKh[i * d + e] / (double)len;
                        if (dv) dv[base + e] += dVh[i * d + e] / (double)len;
                    }
                }
            }
        }
    }
    free(buf);
    free(rs);
    return err ? LHO_ERR_MEM : LHO_OK;
}
