/*
 * txl_oracle.c -- plain scalar CPU reference for Transformer-XL's
 * segment-recurrent relative-position attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP library is
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper
 * with the HIP library, and the HIP library never calls it.
 *
 * Arithmetic is IEEE double throughout.  Inputs arrive as double arrays that
 * hold the exact values the device path sees (e.g. bf16-rounded values widened
 * to double).  There is no blocking, fusion or reordering beyond what the
 * definitions below state: every quantity is formed the way the pages write
 * it, one scalar at a time.
 *
 * Sources (web pages; cited by title and section / class):
 *   [SRC] "Transformer-XL模型 核心源码阅读笔记" (source-reading notes,
 *         blog.csdn.net/ACM_hades/article/details/104742528)
 *   [XL]  "Transformer-XL" (textbook notes, zty624.github.io, DL notebooks,
 *         ch4_transformer/xl)
 *   [TF]  "Transformer-XL: Attentive Language Models Beyond a Fixed-Length
 *         Context" (m.ruidan.com/infomation/detail/161861)
 *
 * Layouts (row-major, contiguous):
 *   q   [B][H][L][dh]        queries of the current segment
 *   k,v [B][H][K][dh]        keys/values of [memory; current], K = M + L
 *   r   [H][K][dh]           projected relative encodings; row c holds the
 *                            encoding of position value K-1-c ([SRC]
 *                            MemTransformerLM._forward builds pos_seq as
 *                            K-1, K-2, ..., 0)
 *   u,w [H][dh]              r_w_bias (u) and r_r_bias (called vb here)
 *   out [B][H][L][dh], lse [B][H][L]
 *
 * Parity status of every function is stated in the test suite; none of the
 * functions here is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TXO_OK 0
#define TXO_EINVAL (-1)
#define TXO_ENOMEM (-2)

/* ------------------------------------------------------------------------ */
/* Mask                                                                     */
/* ------------------------------------------------------------------------ */

/* [SRC] MemTransformerLM._forward (same_length=False branch): the decoder mask
 * is triu(ones(qlen, klen), diagonal = 1 + mlen), where 1 marks a position
 * that is filled with -inf.  This function writes the complement: vis=1 for
 * a visible (query i, key j) pair, vis=0 for a masked one.  Layout [L][K]. */
int txo_visible_mask(int L, int M, unsigned char *vis)
{
    if (L < 0 || M < 0 || (!vis && L > 0)) return TXO_EINVAL;
    int K = M + L;
    for (int i = 0; i < L; ++i)
        for (int j = 0; j < K; ++j) {
            /* triu(., diagonal=d) keeps entries with column - row >= d. */
            int masked = (j - i) >= 1 + M;
            vis[(size_t)i * K + j] = (unsigned char)!masked;
        }
    return TXO_OK;
}

/* [SRC] MemTransformerLM._forward, same_length=True branch: the mask is
 * triu(ones, 1 + mlen) + tril(ones, -mask_shift_len), with
 * mask_len = klen - mem_len and mask_shift_len = qlen - mask_len when
 * mask_len > 0, else qlen.  mem_len is the configured memory length, mlen the
 * number of memory rows actually present.  vis=1 marks a visible pair. */
int txo_visible_mask_same_length(int L, int M_cur, int mem_len, unsigned char *vis)
{
    if (L < 0 || M_cur < 0 || mem_len < 0 || (!vis && L > 0)) return TXO_EINVAL;
    int K = M_cur + L;
    int mask_len = K - mem_len;
    int shift = mask_len > 0 ? L - mask_len : L;
    for (int i = 0; i < L; ++i)
        for (int j = 0; j < K; ++j) {
            int upper = (j - i) >= 1 + M_cur;  /* triu(., 1 + mlen) */
            int lower = (j - i) <= -shift;     /* tril(., -shift)   */
            vis[(size_t)i * K + j] = (unsigned char)!(upper || lower);
        }
    return TXO_OK;
}

/* ------------------------------------------------------------------------ */
/* The literal relative shift                                               */
/* ------------------------------------------------------------------------ */

/* [SRC] RelMultiHeadAttn._rel_shift on one [L][K] score plane: prepend a zero
 * column (giving [L][K+1]), reinterpret the same memory as [K+1][L], drop the
 * first row of that view, and reinterpret the remaining L*K values as [L][K].
 * [XL] "Relative Shift Trick" describes the same pad -> reshape -> slice.
 * Written with an explicit padded buffer so each step is visible. */
int txo_rel_shift(int L, int K, const double *x, double *y)
{
    if (L < 0 || K < 0) return TXO_EINVAL;
    size_t n = (size_t)L * (size_t)(K + 1);
    double *padded = (double *)malloc((n ? n : 1) * sizeof(double));
    if (!padded) return TXO_ENOMEM;
    /* step 1: padded[i][0] = 0, padded[i][1 + j] = x[i][j]  (row-major [L][K+1]) */
    for (int i = 0; i < L; ++i) {
        padded[(size_t)i * (K + 1)] = 0.0;
        for (int j = 0; j < K; ++j)
            padded[(size_t)i * (K + 1) + 1 + j] = x[(size_t)i * K + j];
    }
    /* step 2: view as [K+1][L]; step 3: drop view-row 0, i.e. the first L flat
     * elements; step 4: view the remaining L*K flat elements as [L][K]. */
    for (size_t t = 0; t < (size_t)L * K; ++t)
        y[t] = padded[(size_t)L + t];
    free(padded);
    return TXO_OK;
}

/* ------------------------------------------------------------------------ */
/* Scores for one (batch, head)                                             */
/* ------------------------------------------------------------------------ */

/* Direct form of the score.  For query i and key j (key positions -M..L-1 as
 * j-M), [XL] "Relative Positional Encoding" writes the score as the sum of
 * four terms q.k + q.r_{i-j} + u.k + v.r_{i-j}; [SRC]
 * RelPartialLearnableMultiHeadAttn.forward groups them as
 *   AC = (q_i + u) . k_j            and   BD = (q_i + v) . r_{i-(j-M)}
 * and multiplies AC + BD by scale = 1/sqrt(d_head).  r_{delta} is the row of
 * r whose position value is delta, i.e. row c = K-1-delta = L-1-i+j.
 * Masked pairs (j - i > M, see txo_visible_mask) get -inf, as masked_fill
 * does in [SRC]. */
static void head_scores_direct(int L, int M, int dh, double scale,
                               const double *q, const double *k, const double *r,
                               const double *u, const double *vb, double *S)
{
    int K = M + L;
    for (int i = 0; i < L; ++i) {
        for (int j = 0; j < K; ++j) {
            if (j - i > M) { S[(size_t)i * K + j] = -INFINITY; continue; }
            int c = L - 1 - i + j;
            double ac = 0.0, bd = 0.0;
            for (int e = 0; e < dh; ++e) {
                double qe = q[(size_t)i * dh + e];
                ac += (qe + u[e]) * k[(size_t)j * dh + e];
                bd += (qe + vb[e]) * r[(size_t)c * dh + e];
            }
            S[(size_t)i * K + j] = (ac + bd) * scale;
        }
    }
}

/* Literal form, following [SRC] RelPartialLearnableMultiHeadAttn.forward step
 * by step: AC over every (i, j); BD_raw over every (i, r-row); BD =
 * _rel_shift(BD_raw); score = (AC + BD) * scale; masked_fill(-inf) with the
 * triu(1 + M) mask.  Used on small shapes to cross-check the direct form. */
static int head_scores_literal(int L, int M, int dh, double scale,
                               const double *q, const double *k, const double *r,
                               const double *u, const double *vb, double *S)
{
    int K = M + L;
    size_t n = (size_t)L * K;
    double *ac = (double *)malloc((n ? n : 1) * sizeof(double));
    double *bdraw = (double *)malloc((n ? n : 1) * sizeof(double));
    double *bd = (double *)malloc((n ? n : 1) * sizeof(double));
    unsigned char *vis = (unsigned char *)malloc(n ? n : 1);
    if (!ac || !bdraw || !bd || !vis) { free(ac); free(bdraw); free(bd); free(vis); return TXO_ENOMEM; }
    for (int i = 0; i < L; ++i)
        for (int j = 0; j < K; ++j) {
            double s = 0.0;
            for (int e = 0; e < dh; ++e) s += (q[(size_t)i * dh + e] + u[e]) * k[(size_t)j * dh + e];
            ac[(size_t)i * K + j] = s;
        }
    for (int i = 0; i < L; ++i)
        for (int c = 0; c < K; ++c) {
            double s = 0.0;
            for (int e = 0; e < dh; ++e) s += (q[(size_t)i * dh + e] + vb[e]) * r[(size_t)c * dh + e];
            bdraw[(size_t)i * K + c] = s;
        }
    int rc = txo_rel_shift(L, K, bdraw, bd);
    if (rc == TXO_OK) rc = txo_visible_mask(L, M, vis);
    if (rc == TXO_OK)
        for (size_t t = 0; t < n; ++t)
            S[t] = vis[t] ? (ac[t] + bd[t]) * scale : -INFINITY;
    free(ac); free(bdraw); free(bd); free(vis);
    return rc;
}

/* [SRC] forward: softmax over the key axis, then attn_vec = sum_j p_ij v_j.
 * Written as m = max_j s_ij, p_ij = exp(s_ij - m), l = sum_j p_ij,
 * out_i = sum_j (p_ij / l) v_j; lse_i = m + log(l). */
static void head_softmax_pv(int L, int K, int dh, const double *S, const double *v,
                            double *out, double *lse)
{
    for (int i = 0; i < L; ++i) {
        const double *s = S + (size_t)i * K;
        double m = -INFINITY;
        for (int j = 0; j < K; ++j) if (s[j] > m) m = s[j];
        double l = 0.0;
        for (int j = 0; j < K; ++j) l += (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
        for (int e = 0; e < dh; ++e) {
            double acc = 0.0;
            for (int j = 0; j < K; ++j) {
                if (s[j] == -INFINITY) continue;
                acc += (exp(s[j] - m) / l) * v[(size_t)j * dh + e];
            }
            out[(size_t)i * dh + e] = acc;
        }
        if (lse) lse[i] = m + log(l);
    }
}

/* Scores of a single head, [L][K]; literal != 0 selects the literal form. */
int txo_relattn_scores(int L, int M, int dh, double scale, int literal,
                       const double *q, const double *k, const double *r,
                       const double *u, const double *vb, double *S)
{
    if (L < 1 || M < 0 || dh < 1) return TXO_EINVAL;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)dh);
    if (literal) return head_scores_literal(L, M, dh, scale, q, k, r, u, vb, S);
    head_scores_direct(L, M, dh, scale, q, k, r, u, vb, S);
    return TXO_OK;
}

/* Relative attention forward for all (b, h).  Heads in [h_begin, h_end) of the
 * flattened (b, h) index are computed; pass 0 and B*H for all of them (a
 * caller may split the range across threads, as the heads are independent).
 * scale <= 0 selects 1/sqrt(dh).  lse may be NULL. */
int txo_relattn_fwd_range(int B, int H, int L, int M, int dh, double scale, int literal,
                          const double *q, const double *k, const double *v,
                          const double *r, const double *u, const double *vb,
                          double *out, double *lse, int bh_begin, int bh_end)
{
    if (B < 1 || H < 1 || L < 1 || M < 0 || dh < 1) return TXO_EINVAL;
    if (bh_begin < 0 || bh_end > B * H || bh_begin > bh_end) return TXO_EINVAL;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)dh);
    int K = M + L;
    double *S = (double *)malloc((size_t)L * K * sizeof(double));
    if (!S) return TXO_ENOMEM;
    int rc = TXO_OK;
    for (int bh = bh_begin; bh < bh_end && rc == TXO_OK; ++bh) {
        int h = bh % H;
        const double *qh = q + (size_t)bh * L * dh;
        const double *kh = k + (size_t)bh * K * dh;
        const double *vh = v + (size_t)bh * K * dh;
        const double *rh = r + (size_t)h * K * dh;
        if (literal) rc = head_scores_literal(L, M, dh, scale, qh, kh, rh, u + (size_t)h * dh, vb + (size_t)h * dh, S);
        else head_scores_direct(L, M, dh, scale, qh, kh, rh, u + (size_t)h * dh, vb + (size_t)h * dh, S);
        if (rc == TXO_OK)
            head_softmax_pv(L, K, dh, S, vh, out + (size_t)bh * L * dh, lse ? lse + (size_t)bh * L : NULL);
    }
    free(S);
    return rc;
}

int txo_relattn_fwd(int B, int H, int L, int M, int dh, double scale, int literal,
                    const double *q, const double *k, const double *v,
                    const double *r, const double *u, const double *vb,
                    double *out, double *lse)
{
    return txo_relattn_fwd_range(B, H, L, M, dh, scale, literal, q, k, v, r, u, vb, out, lse, 0, B * H);
}

/* ------------------------------------------------------------------------ */
/* Mask variants: same_length and per-row memory validity                   */
/* ------------------------------------------------------------------------ */

/* Visibility of one batch row.  same_len > 0 selects the same_length mask of
 * [SRC] MemTransformerLM._forward with mem_len = same_len (see
 * txo_visible_mask_same_length); otherwise the plain triu(1 + M) mask.
 * mvalid is the number of valid memory rows of this batch row: after a
 * document boundary only the newest rows of the memory belong to the row's
 * own stream ([XL] "Batched Streams": the reset is per row), so keys
 * j < M - mvalid are hidden as well.  mvalid = M hides nothing. */
static int head_visible(int L, int M, int same_len, int mvalid, unsigned char *vis)
{
    int K = M + L;
    int rc = same_len > 0 ? txo_visible_mask_same_length(L, M, same_len, vis) : txo_visible_mask(L, M, vis);
    if (rc != TXO_OK) return rc;
    for (int i = 0; i < L; ++i)
        for (int j = 0; j < M - mvalid; ++j) vis[(size_t)i * K + j] = 0;
    return TXO_OK;
}

/* Direct-form scores of one head with an explicit visibility mask. */
static void head_scores_vis(int L, int M, int dh, double scale, const double *q, const double *k,
                            const double *r, const double *u, const double *vb, const unsigned char *vis,
                            double *S)
{
    int K = M + L;
    for (int i = 0; i < L; ++i)
        for (int j = 0; j < K; ++j) {
            if (!vis[(size_t)i * K + j]) { S[(size_t)i * K + j] = -INFINITY; continue; }
            int c = L - 1 - i + j;
            double ac = 0.0, bd = 0.0;
            for (int e = 0; e < dh; ++e) {
                double qe = q[(size_t)i * dh + e];
                ac += (qe + u[e]) * k[(size_t)j * dh + e];
                bd += (qe + vb[e]) * r[(size_t)c * dh + e];
            }
            S[(size_t)i * K + j] = (ac + bd) * scale;
        }
}

/* txo_relattn_fwd_range with the mask variants above.  same_len: 0 = off.
 * mem_valid: [B] valid memory rows per batch row, each in [0, M]; NULL means
 * all M rows are valid. */
int txo_relattn_fwd_vis_range(int B, int H, int L, int M, int dh, double scale, int same_len,
                              const int *mem_valid, const double *q, const double *k, const double *v,
                              const double *r, const double *u, const double *vb, double *out, double *lse,
                              int bh_begin, int bh_end)
{
    if (B < 1 || H < 1 || L < 1 || M < 0 || dh < 1 || same_len < 0) return TXO_EINVAL;
    if (bh_begin < 0 || bh_end > B * H || bh_begin > bh_end) return TXO_EINVAL;
    if (mem_valid)
        for (int b = 0; b < B; ++b)
            if (mem_valid[b] < 0 || mem_valid[b] > M) return TXO_EINVAL;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)dh);
    int K = M + L;
    double *S = (double *)malloc((size_t)L * K * sizeof(double));
    unsigned char *vis = (unsigned char *)malloc((size_t)L * K);
    if (!S || !vis) { free(S); free(vis); return TXO_ENOMEM; }
    int rc = TXO_OK;
    for (int bh = bh_begin; bh < bh_end && rc == TXO_OK; ++bh) {
        int b = bh / H, h = bh % H;
        rc = head_visible(L, M, same_len, mem_valid ? mem_valid[b] : M, vis);
        if (rc != TXO_OK) break;
        head_scores_vis(L, M, dh, scale, q + (size_t)bh * L * dh, k + (size_t)bh * K * dh, r + (size_t)h * K * dh,
                        u + (size_t)h * dh, vb + (size_t)h * dh, vis, S);
        head_softmax_pv(L, K, dh, S, v + (size_t)bh * K * dh, out + (size_t)bh * L * dh,
                        lse ? lse + (size_t)bh * L : NULL);
    }
    free(S);
    free(vis);
    return rc;
}

/* One query row with the mask variants (sampled checks at full size). */
int txo_relattn_row_vis(int H, int L, int M, int dh, double scale, int same_len, int mvalid, int b, int h, int i,
                        const double *q, const double *k, const double *v, const double *r, const double *u,
                        const double *vb, double *row_out, double *row_lse)
{
    if (H < 1 || L < 1 || M < 0 || dh < 1 || i < 0 || i >= L || h < 0 || h >= H || b < 0) return TXO_EINVAL;
    if (same_len < 0 || mvalid < 0 || mvalid > M) return TXO_EINVAL;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)dh);
    int K = M + L;
    size_t bh = (size_t)b * H + h;
    unsigned char *vis = (unsigned char *)malloc((size_t)L * K);
    double *s = (double *)malloc((size_t)K * sizeof(double));
    if (!vis || !s) { free(vis); free(s); return TXO_ENOMEM; }
    int rc = head_visible(L, M, same_len, mvalid, vis);
    if (rc == TXO_OK) {
        /* the row's scores alone: the first query row of the slice is row i */
        const double *qi = q + (bh * L + i) * dh;
        const double *kh = k + bh * K * dh, *rh = r + (size_t)h * K * dh;
        const double *uh = u + (size_t)h * dh, *wh = vb + (size_t)h * dh;
        for (int j = 0; j < K; ++j) {
            if (!vis[(size_t)i * K + j]) { s[j] = -INFINITY; continue; }
            int c = L - 1 - i + j;
            double ac = 0.0, bd = 0.0;
            for (int e = 0; e < dh; ++e) {
                ac += (qi[e] + uh[e]) * kh[(size_t)j * dh + e];
                bd += (qi[e] + wh[e]) * rh[(size_t)c * dh + e];
            }
            s[j] = (ac + bd) * scale;
        }
        head_softmax_pv(1, K, dh, s, v + bh * K * dh, row_out, row_lse);
    }
    free(vis);
    free(s);
    return rc;
}

/* One output element, for sampled checks at full size: out[b][h][i][e] and
 * lse[b][h][i] for a single query row i (all e written to row_out[dh]). */
int txo_relattn_row(int H, int L, int M, int dh, double scale, int b, int h, int i,
                    const double *q, const double *k, const double *v,
                    const double *r, const double *u, const double *vb,
                    double *row_out, double *row_lse)
{
    if (H < 1 || L < 1 || M < 0 || dh < 1 || i < 0 || i >= L || h < 0 || h >= H || b < 0) return TXO_EINVAL;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)dh);
    int K = M + L;
    size_t bh = (size_t)b * H + h;
    const double *qi = q + (bh * L + i) * dh;
    const double *kh = k + bh * K * dh;
    const double *vh = v + bh * K * dh;
    const double *rh = r + (size_t)h * K * dh;
    const double *uh = u + (size_t)h * dh, *wh = vb + (size_t)h * dh;
    double *s = (double *)malloc((size_t)K * sizeof(double));
    if (!s) return TXO_ENOMEM;
    for (int j = 0; j < K; ++j) {
        if (j - i > M) { s[j] = -INFINITY; continue; }
        int c = L - 1 - i + j;
        double ac = 0.0, bd = 0.0;
        for (int e = 0; e < dh; ++e) {
            ac += (qi[e] + uh[e]) * kh[(size_t)j * dh + e];
            bd += (qi[e] + wh[e]) * rh[(size_t)c * dh + e];
        }
        s[j] = (ac + bd) * scale;
    }
    head_softmax_pv(1, K, dh, s, vh, row_out, row_lse);
    free(s);
    return TXO_OK;
}

/* ------------------------------------------------------------------------ */
/* Backward (gradients of the attention above)                              */
/* ------------------------------------------------------------------------ */

/* Gradients of one head's attention output with respect to every input, by
 * the chain rule on the definition used by the forward functions above (the
 * pages print no backward; they fix the forward, and [XL] "Why Stop Gradient"
 * fixes which paths carry a gradient at the layer level).  With
 *   s_ij = (ac_ij + bd_ij) * scale   on visible pairs,
 *   p_ij = exp(s_ij) / sum_k exp(s_ik),        out_i = sum_j p_ij v_j,
 * and an upstream gradient dout_i:
 *   dP_ij = dout_i . v_j
 *   dS_ij = p_ij (dP_ij - sum_k p_ik dP_ik)    (softmax Jacobian)
 *   g_ij  = dS_ij * scale                      (gradient of ac_ij and of bd_ij)
 *   dq_i  = sum_j g_ij (k_j + r_c),  c = L-1-i+j  (q_i enters both terms)
 *   du    = sum_{i,j} g_ij k_j,   dvb = sum_{i,j} g_ij r_c
 *   dk_j  = sum_i g_ij (q_i + u),  dv_j = sum_i p_ij dout_i
 *   dr_c  = sum over (i, j) with L-1-i+j = c of g_ij (q_i + vb).
 * Masked pairs carry p = 0 and so no gradient.  Keys of the memory get dk and
 * dv like any other key: stop-gradient detaches the memory states themselves,
 * but a layer still needs these rows for its projection weights.
 * Outputs of this head: dq [L][dh], dk, dv [K][dh] (written), dr [K][dh],
 * du, dvb [dh] (written: this head's contribution only; the caller sums the
 * batch rows of a head). */
static void head_backward(int L, int M, int dh, double scale, const double *q, const double *k,
                          const double *v, const double *r, const double *u, const double *vb,
                          const double *dout, const double *S, double *P, double *dS,
                          double *dq, double *dk, double *dv, double *dr, double *du, double *dvb)
{
    int K = M + L;
    for (int i = 0; i < L; ++i) {
        const double *s = S + (size_t)i * K;
        double m = -INFINITY;
        for (int j = 0; j < K; ++j) if (s[j] > m) m = s[j];
        double l = 0.0;
        for (int j = 0; j < K; ++j) l += (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
        for (int j = 0; j < K; ++j) P[(size_t)i * K + j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m) / l;
    }
    for (int i = 0; i < L; ++i) {
        double rowdot = 0.0;
        for (int j = 0; j < K; ++j) {
            double dp = 0.0;
            for (int e = 0; e < dh; ++e) dp += dout[(size_t)i * dh + e] * v[(size_t)j * dh + e];
            dS[(size_t)i * K + j] = dp;
            rowdot += P[(size_t)i * K + j] * dp;
        }
        for (int j = 0; j < K; ++j)
            dS[(size_t)i * K + j] = P[(size_t)i * K + j] * (dS[(size_t)i * K + j] - rowdot);
    }
    memset(dq, 0, (size_t)L * dh * sizeof(double));
    memset(dk, 0, (size_t)K * dh * sizeof(double));
    memset(dv, 0, (size_t)K * dh * sizeof(double));
    memset(dr, 0, (size_t)K * dh * sizeof(double));
    memset(du, 0, (size_t)dh * sizeof(double));
    memset(dvb, 0, (size_t)dh * sizeof(double));
    for (int i = 0; i < L; ++i)
        for (int j = 0; j < K; ++j) {
            double p = P[(size_t)i * K + j];
            if (p == 0.0) continue;
            double gij = dS[(size_t)i * K + j] * scale;
            int c = L - 1 - i + j;
            for (int e = 0; e < dh; ++e) {
                double qe = q[(size_t)i * dh + e];
                double ke = k[(size_t)j * dh + e], re = r[(size_t)c * dh + e];
                dq[(size_t)i * dh + e] += gij * (ke + re);
                du[e] += gij * ke;
                dvb[e] += gij * re;
                dk[(size_t)j * dh + e] += gij * (qe + u[e]);
                dr[(size_t)c * dh + e] += gij * (qe + vb[e]);
                dv[(size_t)j * dh + e] += p * dout[(size_t)i * dh + e];
            }
        }
}

/* Backward over the heads [bh_begin, bh_end) of the flattened (b, h) index,
 * with the same mask options as txo_relattn_fwd_vis_range (same_len 0 = off,
 * mem_valid NULL = all memory rows valid).  Layouts as the forward; dout
 * [B][H][L][dh].  dq [B][H][L][dh] and dk, dv [B][H][K][dh] are written for
 * the heads in range; dr_bh [B*H][K][dh] and du_bh, dvb_bh [B*H][dh] receive
 * each head's own contribution (dr, du and dvb of head h are the sums of
 * these over the batch rows b). */
int txo_relattn_bwd_range(int B, int H, int L, int M, int dh, double scale, int same_len,
                          const int *mem_valid, const double *q, const double *k, const double *v,
                          const double *r, const double *u, const double *vb, const double *dout,
                          double *dq, double *dk, double *dv, double *dr_bh, double *du_bh, double *dvb_bh,
                          int bh_begin, int bh_end)
{
    if (B < 1 || H < 1 || L < 1 || M < 0 || dh < 1 || same_len < 0) return TXO_EINVAL;
    if (bh_begin < 0 || bh_end > B * H || bh_begin > bh_end) return TXO_EINVAL;
    if (mem_valid)
        for (int b = 0; b < B; ++b)
            if (mem_valid[b] < 0 || mem_valid[b] > M) return TXO_EINVAL;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)dh);
    int K = M + L;
    size_t n = (size_t)L * K;
    double *S = (double *)malloc(n * sizeof(double));
    double *P = (double *)malloc(n * sizeof(double));
    double *dS = (double *)malloc(n * sizeof(double));
    unsigned char *vis = (unsigned char *)malloc(n);
    if (!S || !P || !dS || !vis) { free(S); free(P); free(dS); free(vis); return TXO_ENOMEM; }
    int rc = TXO_OK;
    for (int bh = bh_begin; bh < bh_end; ++bh) {
        int b = bh / H, h = bh % H;
        rc = head_visible(L, M, same_len, mem_valid ? mem_valid[b] : M, vis);
        if (rc != TXO_OK) break;
        const double *qh = q + (size_t)bh * L * dh, *kh = k + (size_t)bh * K * dh;
        const double *vh = v + (size_t)bh * K * dh, *rh = r + (size_t)h * K * dh;
        const double *uh = u + (size_t)h * dh, *wh = vb + (size_t)h * dh;
        head_scores_vis(L, M, dh, scale, qh, kh, rh, uh, wh, vis, S);
        head_backward(L, M, dh, scale, qh, kh, vh, rh, uh, wh, dout + (size_t)bh * L * dh, S, P, dS,
                      dq + (size_t)bh * L * dh, dk + (size_t)bh * K * dh, dv + (size_t)bh * K * dh,
                      dr_bh + (size_t)bh * K * dh, du_bh + (size_t)bh * dh, dvb_bh + (size_t)bh * dh);
    }
    free(S); free(P); free(dS); free(vis);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Memory update                                                            */
/* ------------------------------------------------------------------------ */

/* [SRC] MemTransformerLM._update_mems: with mlen memory rows present and qlen
 * new rows, end = mlen + max(0, qlen - ext_len), beg = max(0, end - mem_len),
 * and the new memory is cat([mems, hids], seq)[beg:end], detached.  [XL]
 * "Segment-Level Recurrence" calls the ext_len = 0 case Tail_M.  This copies
 * raw bytes (elem_bytes per element), so the result is bit-exact for any
 * dtype.  Layout per batch row: mem [M_cur][d] at mem + b*mem_bs elements,
 * h [L][d] at h + b*h_bs, new_mem [M_new][d] at new_mem + b*new_bs.
 * Returns M_new = end - beg (>= 0), or a negative error code. */
int txo_mem_update(const void *mem, int M_cur, const void *h, int L, void *new_mem,
                   int mem_len, int ext_len, int B, int d, int elem_bytes,
                   int64_t mem_bs, int64_t h_bs, int64_t new_bs)
{
    if (M_cur < 0 || L < 0 || mem_len < 0 || ext_len < 0 || B < 0 || d < 1 || elem_bytes < 1)
        return TXO_EINVAL;
    int end = M_cur + (L - ext_len > 0 ? L - ext_len : 0);
    int beg = end - mem_len > 0 ? end - mem_len : 0;
    int M_new = end - beg;
    size_t row = (size_t)d * elem_bytes;
    for (int b = 0; b < B; ++b) {
        const unsigned char *mb = (const unsigned char *)mem + (size_t)b * mem_bs * elem_bytes;
        const unsigned char *hb = (const unsigned char *)h + (size_t)b * h_bs * elem_bytes;
        unsigned char *nb = (unsigned char *)new_mem + (size_t)b * new_bs * elem_bytes;
        for (int t = beg; t < end; ++t) {
            /* row t of cat([mem; h]) */
            const unsigned char *src = (t < M_cur) ? mb + (size_t)t * row : hb + (size_t)(t - M_cur) * row;
            memcpy(nb + (size_t)(t - beg) * row, src, row);
        }
    }
    return M_new;
}

/* ------------------------------------------------------------------------ */
/* Layer pieces                                                             */
/* ------------------------------------------------------------------------ */

/* [SRC] PositionalEmbedding: inv_freq[t] = 1 / 10000^(2t / demb) for
 * t = 0 .. demb/2 - 1; for a position value p the embedding is
 * [sin(p * inv_freq) | cos(p * inv_freq)] (the sines in the first half).
 * [SRC] MemTransformerLM._forward: the positions are klen-1, ..., 0, and with
 * clamp_len > 0 each is clamped to at most clamp_len.  out is [K][demb]; row c
 * uses position value min(K-1-c, clamp_len). demb must be even. */
int txo_pos_emb(int K, int demb, int clamp_len, double *out)
{
    if (K < 0 || demb < 2 || (demb & 1)) return TXO_EINVAL;
    int half = demb / 2;
    for (int c = 0; c < K; ++c) {
        double p = (double)(K - 1 - c);
        if (clamp_len > 0 && p > clamp_len) p = clamp_len;
        for (int t = 0; t < half; ++t) {
            double inv_freq = 1.0 / pow(10000.0, (2.0 * t) / (double)demb);
            out[(size_t)c * demb + t] = sin(p * inv_freq);
            out[(size_t)c * demb + half + t] = cos(p * inv_freq);
        }
    }
    return TXO_OK;
}

/* nn.Linear: y[n][o] = sum_i x[n][i] * W[o][i] (+ bias[o]); W is [out][in]. */
static void linear(int N, int in, int outd, const double *x, const double *W,
                   const double *bias, double *y)
{
    for (int n = 0; n < N; ++n)
        for (int o = 0; o < outd; ++o) {
            double s = 0.0;
            for (int i = 0; i < in; ++i) s += x[(size_t)n * in + i] * W[(size_t)o * in + i];
            y[(size_t)n * outd + o] = bias ? s + bias[o] : s;
        }
}

/* nn.LayerNorm over the last axis: (x - mean) / sqrt(var + eps) * g + b, with
 * the biased variance. */
static void layer_norm(int N, int d, const double *x, const double *g, const double *b,
                       double eps, double *y)
{
    for (int n = 0; n < N; ++n) {
        const double *xr = x + (size_t)n * d;
        double mean = 0.0, var = 0.0;
        for (int i = 0; i < d; ++i) mean += xr[i];
        mean /= d;
        for (int i = 0; i < d; ++i) var += (xr[i] - mean) * (xr[i] - mean);
        var /= d;
        double inv = 1.0 / sqrt(var + eps);
        for (int i = 0; i < d; ++i) y[(size_t)n * d + i] = (xr[i] - mean) * inv * g[i] + b[i];
    }
}

int txo_linear(int N, int in, int outd, const double *x, const double *W, const double *bias, double *y)
{
    if (N < 0 || in < 1 || outd < 1) return TXO_EINVAL;
    linear(N, in, outd, x, W, bias, y);
    return TXO_OK;
}

int txo_layer_norm(int N, int d, const double *x, const double *g, const double *b, double eps, double *y)
{
    if (N < 0 || d < 1) return TXO_EINVAL;
    layer_norm(N, d, x, g, b, eps, y);
    return TXO_OK;
}

/* One RelPartialLearnableDecoderLayer forward with post-LayerNorm, following
 * [SRC] RelPartialLearnableMultiHeadAttn.forward and PositionwiseFF.forward
 * (pre_lnorm = False), dropout = identity:
 *   cat   = [mem; h]                                  (K = M_cur + L rows)
 *   heads = cat W_qkv^T; q = last L rows of chunk 0, k = chunk 1, v = chunk 2
 *   r_k   = pos_emb(K-1 .. 0) W_r^T
 *   attn  = relative attention (direct form above), heads merged
 *   x     = LN1(h + attn W_o^T)
 *   y     = LN2(x + W2 relu(W1 x + b1) + b2)
 * Per batch row b: h_in [L][d] at h_in + b*L*d, mem [M_cur][d] at
 * mem + b*M_cur*d (M_cur may be 0 and mem NULL), out [L][d].
 * W_qkv [3*H*dh][d], W_r [H*dh][d], W_o [d][H*dh], W1 [d_inner][d], b1
 * [d_inner], W2 [d][d_inner], b2 [d]; u, vb [H][dh]. */
/* The layer with the options of [SRC] MemTransformerLM: clamp_len > 0 clamps
 * the position values ([SRC] _forward: pos_seq.clamp_(max=clamp_len)),
 * same_len > 0 selects the same_length mask with mem_len = same_len, and
 * mem_valid ([B] or NULL) hides the oldest M_cur - mem_valid[b] memory rows of
 * batch row b (per-row memory reset, see head_visible). */
int txo_layer_fwd_ex(int B, int L, int M_cur, int d, int H, int dh, int d_inner,
                     int clamp_len, int same_len, const int *mem_valid,
                     const double *h_in, const double *mem,
                     const double *W_qkv, const double *W_r, const double *W_o,
                     const double *ln1_g, const double *ln1_b,
                     const double *W1, const double *b1, const double *W2, const double *b2,
                     const double *ln2_g, const double *ln2_b,
                     const double *u, const double *vb, double eps, double *out)
{
    if (B < 1 || L < 1 || M_cur < 0 || d < 2 || (d & 1) || H < 1 || dh < 1 || d_inner < 1) return TXO_EINVAL;
    if (M_cur > 0 && !mem) return TXO_EINVAL;
    if (clamp_len < 0 || same_len < 0) return TXO_EINVAL;
    if (mem_valid)
        for (int b = 0; b < B; ++b)
            if (mem_valid[b] < 0 || mem_valid[b] > M_cur) return TXO_EINVAL;
    int K = M_cur + L, HD = H * dh;
    double scale = 1.0 / sqrt((double)dh);
    double *cat = malloc((size_t)K * d * sizeof(double));
    double *heads = malloc((size_t)K * 3 * HD * sizeof(double));
    double *pe = malloc((size_t)K * d * sizeof(double));
    double *rk = malloc((size_t)K * HD * sizeof(double));
    double *qh = malloc((size_t)L * dh * sizeof(double));
    double *kh = malloc((size_t)K * dh * sizeof(double));
    double *vh = malloc((size_t)K * dh * sizeof(double));
    double *rh = malloc((size_t)K * dh * sizeof(double));
    double *S = malloc((size_t)L * K * sizeof(double));
    double *oh = malloc((size_t)L * dh * sizeof(double));
    double *vec = malloc((size_t)L * HD * sizeof(double));
    double *ao = malloc((size_t)L * d * sizeof(double));
    double *x = malloc((size_t)L * d * sizeof(double));
    double *f1 = malloc((size_t)L * d_inner * sizeof(double));
    double *f2 = malloc((size_t)L * d * sizeof(double));
    unsigned char *vis = malloc((size_t)L * K);
    int rc = TXO_OK;
    if (!cat || !heads || !pe || !rk || !qh || !kh || !vh || !rh || !S || !oh || !vec || !ao || !x || !f1 || !f2 ||
        !vis) {
        rc = TXO_ENOMEM;
        goto done;
    }
    txo_pos_emb(K, d, clamp_len, pe);
    linear(K, d, HD, pe, W_r, NULL, rk);                 /* r_head_k [K][H][dh] */
    for (int b = 0; b < B; ++b) {
        rc = head_visible(L, M_cur, same_len, mem_valid ? mem_valid[b] : M_cur, vis);
        if (rc != TXO_OK) goto done;
        const double *hb = h_in + (size_t)b * L * d;
        for (int t = 0; t < M_cur; ++t)
            for (int i = 0; i < d; ++i) cat[(size_t)t * d + i] = mem[((size_t)b * M_cur + t) * d + i];
        for (int t = 0; t < L; ++t)
            for (int i = 0; i < d; ++i) cat[(size_t)(M_cur + t) * d + i] = hb[(size_t)t * d + i];
        linear(K, d, 3 * HD, cat, W_qkv, NULL, heads);   /* w_heads [K][3*H*dh] */
        for (int n = 0; n < H; ++n) {
            for (int t = 0; t < L; ++t)
                for (int e = 0; e < dh; ++e)
                    qh[(size_t)t * dh + e] = heads[(size_t)(M_cur + t) * 3 * HD + n * dh + e];
            for (int t = 0; t < K; ++t)
                for (int e = 0; e < dh; ++e) {
                    kh[(size_t)t * dh + e] = heads[(size_t)t * 3 * HD + HD + n * dh + e];
                    vh[(size_t)t * dh + e] = heads[(size_t)t * 3 * HD + 2 * HD + n * dh + e];
                    rh[(size_t)t * dh + e] = rk[(size_t)t * HD + n * dh + e];
                }
            head_scores_vis(L, M_cur, dh, scale, qh, kh, rh, u + (size_t)n * dh, vb + (size_t)n * dh, vis, S);
            head_softmax_pv(L, K, dh, S, vh, oh, NULL);
            for (int t = 0; t < L; ++t)
                for (int e = 0; e < dh; ++e) vec[(size_t)t * HD + n * dh + e] = oh[(size_t)t * dh + e];
        }
        linear(L, HD, d, vec, W_o, NULL, ao);
        for (size_t t = 0; t < (size_t)L * d; ++t) ao[t] += hb[t];
        layer_norm(L, d, ao, ln1_g, ln1_b, eps, x);
        linear(L, d, d_inner, x, W1, b1, f1);
        for (size_t t = 0; t < (size_t)L * d_inner; ++t) f1[t] = f1[t] > 0.0 ? f1[t] : 0.0;
        linear(L, d_inner, d, f1, W2, b2, f2);
        for (size_t t = 0; t < (size_t)L * d; ++t) f2[t] += x[t];
        layer_norm(L, d, f2, ln2_g, ln2_b, eps, out + (size_t)b * L * d);
    }
done:
    free(cat); free(heads); free(pe); free(rk); free(qh); free(kh); free(vh); free(rh);
    free(S); free(oh); free(vec); free(ao); free(x); free(f1); free(f2); free(vis);
    return rc;
}

/* [SRC] RelPartialLearnableDecoderLayer with the default options. */
int txo_layer_fwd(int B, int L, int M_cur, int d, int H, int dh, int d_inner,
                  const double *h_in, const double *mem,
                  const double *W_qkv, const double *W_r, const double *W_o,
                  const double *ln1_g, const double *ln1_b,
                  const double *W1, const double *b1, const double *W2, const double *b2,
                  const double *ln2_g, const double *ln2_b,
                  const double *u, const double *vb, double eps, double *out)
{
    return txo_layer_fwd_ex(B, L, M_cur, d, H, dh, d_inner, 0, 0, NULL, h_in, mem, W_qkv, W_r, W_o, ln1_g, ln1_b,
                            W1, b1, W2, b2, ln2_g, ln2_b, u, vb, eps, out);
}
