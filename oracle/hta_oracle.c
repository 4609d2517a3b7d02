/*
 * hta_oracle.c -- CPU oracle for tree verification attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark load this code.  The GPU library never links, calls or includes it, and
 * this file includes nothing of the GPU library.
 *
 * What it computes (the plain definition, no blocking, no fusion, no reordering):
 *
 * LongSpec verifies a speculated draft tree in one target forward whose attention has two
 * parts (LongSpec README, Introduction, "Hybrid Attention Aggregation"; paper summary,
 * Summary, "Hybrid Tree Attention"; arXiv abstract): every tree token attends to the whole
 * prefix with no mask, and to the tree tokens under the tree mask; the two parts are then
 * aggregated.  Because the decoding is lossless (README title; summary, first paragraph),
 * the aggregate must equal one softmax attention over the union of the visible keys.
 * So, for batch b, query head h and tree node i:
 *
 *   g        = h / (Hq / Hkv)                       (consecutive query heads share a KV head)
 *   visible  = { prefix keys j < prefix_len[b] }    (prefix: no mask)
 *            U { tree key t : t is i or an ancestor of i }   (tree mask, self included)
 *   s_j      = scale * <q[b,i,h,:], k_j>            (fp64 on the exactly widened inputs)
 *   m        = max_j s_j ,  Z = sum_j exp(s_j - m)  (two passes over the visible keys)
 *   out      = sum_j exp(s_j - m) v_j / Z
 *   lse      = m + ln Z                             (natural log of the full sum)
 *
 * An empty visible set (only possible for a part-only query) gives out = 0, lse = -inf.
 * The ancestor relation is read off the parent pointers by walking them to the root.
 * Node order must be topological: parent[i] in [-1, i-1]; anything else is rejected.
 *
 * Single-threaded, scalar, compiled without fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HTA_ORACLE_OK 0
#define HTA_ORACLE_BAD_TREE 1
#define HTA_ORACLE_BAD_ARG 2
#define HTA_ORACLE_NOMEM 3

/* part selector for hta_oracle_rows */
#define HTA_PART_ALL 0
#define HTA_PART_PREFIX 1
#define HTA_PART_TREE 2

/* Widen one stored element to double.  bf16 is the top half of an IEEE binary32. */
static double widen(const void *base, size_t idx, int is_bf16)
{
    if (is_bf16) {
        uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[idx];
}

/* Validate the parent pointers of one sequence: topological order, -1 marks a root. */
static int tree_is_valid(const int32_t *parent, int T)
{
    for (int i = 0; i < T; ++i)
        if (parent[i] < -1 || parent[i] >= i)
            return 0;
    return 1;
}

int hta_oracle_check_tree(int B, int T, const int32_t *parent)
{
    for (int b = 0; b < B; ++b)
        if (!tree_is_valid(parent + (size_t)b * T, T))
            return HTA_ORACLE_BAD_TREE;
    return HTA_ORACLE_OK;
}

/*
 * Ancestor-or-self masks, packed: word w of node i holds bit (t % 64) for tree node
 * t = 64 w + (t % 64), set iff t is i or an ancestor of i.  masks is [B, T, ceil(T/64)].
 */
int hta_oracle_masks(int B, int T, const int32_t *parent, uint64_t *masks)
{
    if (B < 0 || T < 0)
        return HTA_ORACLE_BAD_ARG;
    const int W = (T + 63) / 64;
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * T;
        if (!tree_is_valid(par, T))
            return HTA_ORACLE_BAD_TREE;
        for (int i = 0; i < T; ++i) {
            uint64_t *m = masks + ((size_t)b * T + i) * W;
            for (int w = 0; w < W; ++w)
                m[w] = 0;
            for (int p = i; p != -1; p = par[p])
                m[p / 64] |= (uint64_t)1 << (p % 64);
        }
    }
    return HTA_ORACLE_OK;
}

/*
 * Softmax attention of one query over an explicit list of keys.
 * key_ptr[j]/val_ptr[j] locate key j's row (element offset into kbase[j]/vbase[j]).
 */
typedef struct {
    const void *base;
    size_t offset; /* element offset of the row */
} row_ref;

static void attend(int D, const double *qrow, double scale, int n, const row_ref *keys,
                   const row_ref *vals, int is_bf16, double *scores, double *out, double *lse)
{
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    if (n == 0) {
        *lse = -INFINITY;
        return;
    }
    /* pass 1: scores and their maximum */
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double s = 0.0;
        for (int d = 0; d < D; ++d)
            s += qrow[d] * widen(keys[j].base, keys[j].offset + (size_t)d, is_bf16);
        s *= scale;
        scores[j] = s;
        if (s > m)
            m = s;
    }
    /* pass 2: normaliser and weighted values */
    double Z = 0.0;
    for (int j = 0; j < n; ++j) {
        double p = exp(scores[j] - m);
        Z += p;
        for (int d = 0; d < D; ++d)
            out[d] += p * widen(vals[j].base, vals[j].offset + (size_t)d, is_bf16);
    }
    for (int d = 0; d < D; ++d)
        out[d] /= Z;
    *lse = m + log(Z);
}

/*
 * Attention for an explicit list of rows (b, h, i).  Layouts:
 *   q [B,T,Hq,D]; k_prefix, v_prefix [B,Hkv,Lmax,D]; k_tree, v_tree [B,Hkv,T,D];
 *   parent [B,T]; prefix_len [B].
 * Outputs: out_rows [nrows, D], lse_rows [nrows].
 * part: 0 = prefix and tree (the full verification attention), 1 = prefix keys only,
 *       2 = tree keys only (used to check the two halves separately).
 */
int hta_oracle_rows(int B, int T, int Hq, int Hkv, int D, int Lmax, int is_bf16,
                    const void *q, const void *k_prefix, const void *v_prefix,
                    const void *k_tree, const void *v_tree, const int32_t *parent,
                    const int32_t *prefix_len, double scale, int part, int nrows,
                    const int32_t *row_b, const int32_t *row_h, const int32_t *row_i,
                    double *out_rows, double *lse_rows)
{
    if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Lmax < 0 || Hq % Hkv != 0)
        return HTA_ORACLE_BAD_ARG;
    if (part < 0 || part > 2)
        return HTA_ORACLE_BAD_ARG;
    for (int b = 0; b < B; ++b) {
        if (prefix_len[b] < 0 || prefix_len[b] > Lmax)
            return HTA_ORACLE_BAD_ARG;
        if (!tree_is_valid(parent + (size_t)b * T, T))
            return HTA_ORACLE_BAD_TREE;
    }
    const int G = Hq / Hkv;
    const size_t cap = (size_t)Lmax + (size_t)T;
    row_ref *keys = (row_ref *)malloc(cap * sizeof(row_ref));
    row_ref *vals = (row_ref *)malloc(cap * sizeof(row_ref));
    double *scores = (double *)malloc(cap * sizeof(double));
    double *qrow = (double *)malloc((size_t)D * sizeof(double));
    unsigned char *in_tree = (unsigned char *)malloc((size_t)T);
    if (!keys || !vals || !scores || !qrow || !in_tree) {
        free(keys); free(vals); free(scores); free(qrow); free(in_tree);
        return HTA_ORACLE_NOMEM;
    }
    int rc = HTA_ORACLE_OK;
    for (int r = 0; r < nrows; ++r) {
        const int b = row_b[r], h = row_h[r], i = row_i[r];
        if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= T) {
            rc = HTA_ORACLE_BAD_ARG;
            break;
        }
        const int g = h / G;
        for (int d = 0; d < D; ++d)
            qrow[d] = widen(q, (((size_t)b * T + i) * Hq + h) * D + d, is_bf16);
        /* explicit visibility list: prefix columns first, then the tree columns */
        int n = 0;
        if (part != HTA_PART_TREE) {
            const size_t base = ((size_t)b * Hkv + g) * (size_t)Lmax * D;
            for (int j = 0; j < prefix_len[b]; ++j) {
                keys[n].base = k_prefix; keys[n].offset = base + (size_t)j * D;
                vals[n].base = v_prefix; vals[n].offset = base + (size_t)j * D;
                ++n;
            }
        }
        if (part != HTA_PART_PREFIX) {
            const int32_t *par = parent + (size_t)b * T;
            memset(in_tree, 0, (size_t)T);
            for (int p = i; p != -1; p = par[p])
                in_tree[p] = 1;
            const size_t base = ((size_t)b * Hkv + g) * (size_t)T * D;
            for (int t = 0; t < T; ++t) {
                if (!in_tree[t])
                    continue;
                keys[n].base = k_tree; keys[n].offset = base + (size_t)t * D;
                vals[n].base = v_tree; vals[n].offset = base + (size_t)t * D;
                ++n;
            }
        }
        attend(D, qrow, scale, n, keys, vals, is_bf16, scores, out_rows + (size_t)r * D,
               lse_rows + r);
    }
    free(keys); free(vals); free(scores); free(qrow); free(in_tree);
    return rc;
}

/*
 * Whole verification attention: out [B,T,Hq,D] and lse [B,Hq,T] for every row.
 */
int hta_oracle_verify(int B, int T, int Hq, int Hkv, int D, int Lmax, int is_bf16,
                      const void *q, const void *k_prefix, const void *v_prefix,
                      const void *k_tree, const void *v_tree, const int32_t *parent,
                      const int32_t *prefix_len, double scale, int part, double *out,
                      double *lse)
{
    if (B <= 0 || T <= 0 || Hq <= 0)
        return HTA_ORACLE_BAD_ARG;
    const int nrows = B * T * Hq;
    int32_t *rb = (int32_t *)malloc((size_t)nrows * sizeof(int32_t));
    int32_t *rh = (int32_t *)malloc((size_t)nrows * sizeof(int32_t));
    int32_t *ri = (int32_t *)malloc((size_t)nrows * sizeof(int32_t));
    double *lse_rows = (double *)malloc((size_t)nrows * sizeof(double));
    if (!rb || !rh || !ri || !lse_rows) {
        free(rb); free(rh); free(ri); free(lse_rows);
        return HTA_ORACLE_NOMEM;
    }
    /* rows enumerated in out's order [B,T,Hq] so out needs no reshuffle */
    int r = 0;
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < T; ++i)
            for (int h = 0; h < Hq; ++h, ++r) {
                rb[r] = b; ri[r] = i; rh[r] = h;
            }
    int rc = hta_oracle_rows(B, T, Hq, Hkv, D, Lmax, is_bf16, q, k_prefix, v_prefix, k_tree,
                             v_tree, parent, prefix_len, scale, part, nrows, rb, rh, ri, out,
                             lse_rows);
    if (rc == HTA_ORACLE_OK)
        for (r = 0; r < nrows; ++r)
            lse[((size_t)rb[r] * Hq + rh[r]) * T + ri[r]] = lse_rows[r];
    free(rb); free(rh); free(ri); free(lse_rows);
    return rc;
}

/*
 * General masked attention in fp64 (the definition the verification attention is a case of):
 * q [nq,D], k,v [nk,D], mask [nq,nk] (nonzero = visible).  out [nq,D], lse [nq].
 */
int hta_oracle_masked_attention(int nq, int nk, int D, const double *q, const double *k,
                                const double *v, const unsigned char *mask, double scale,
                                double *out, double *lse)
{
    if (nq < 0 || nk < 0 || D <= 0)
        return HTA_ORACLE_BAD_ARG;
    double *scores = (double *)malloc(((size_t)nk + 1) * sizeof(double));
    if (!scores)
        return HTA_ORACLE_NOMEM;
    for (int i = 0; i < nq; ++i) {
        double *o = out + (size_t)i * D;
        for (int d = 0; d < D; ++d)
            o[d] = 0.0;
        double m = -INFINITY;
        int n = 0;
        for (int j = 0; j < nk; ++j) {
            if (!mask[(size_t)i * nk + j])
                continue;
            double s = 0.0;
            for (int d = 0; d < D; ++d)
                s += q[(size_t)i * D + d] * k[(size_t)j * D + d];
            s *= scale;
            scores[j] = s;
            if (s > m)
                m = s;
            ++n;
        }
        if (n == 0) {
            lse[i] = -INFINITY;
            continue;
        }
        double Z = 0.0;
        for (int j = 0; j < nk; ++j) {
            if (!mask[(size_t)i * nk + j])
                continue;
            double p = exp(scores[j] - m);
            Z += p;
            for (int d = 0; d < D; ++d)
                o[d] += p * v[(size_t)j * D + d];
        }
        for (int d = 0; d < D; ++d)
            o[d] /= Z;
        lse[i] = m + log(Z);
    }
    free(scores);
    return HTA_ORACLE_OK;
}

/*
 * Aggregation of partial attentions over disjoint key sets (the exact log-sum-exp merge,
 * as in Flash-Decoding, the long-context baseline the paper summary compares against):
 *   M = max_s lse_s ;  w_s = exp(lse_s - M) ;  out = sum_s w_s o_s / sum_s w_s ;
 *   lse = M + ln sum_s w_s.
 * Parts with lse = -inf (no visible key) weigh 0; if all are empty, out = 0, lse = -inf.
 * o_parts [nparts, D], lse_parts [nparts].
 */
int hta_oracle_lse_merge(int nparts, int D, const double *lse_parts, const double *o_parts,
                         double *out, double *lse)
{
    if (nparts < 0 || D <= 0)
        return HTA_ORACLE_BAD_ARG;
    double M = -INFINITY;
    for (int s = 0; s < nparts; ++s)
        if (lse_parts[s] > M)
            M = lse_parts[s];
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    if (M == -INFINITY) {
        *lse = -INFINITY;
        return HTA_ORACLE_OK;
    }
    double W = 0.0;
    for (int s = 0; s < nparts; ++s) {
        if (lse_parts[s] == -INFINITY)
            continue;
        double w = exp(lse_parts[s] - M);
        W += w;
        for (int d = 0; d < D; ++d)
            out[d] += w * o_parts[(size_t)s * D + d];
    }
    for (int d = 0; d < D; ++d)
        out[d] /= W;
    *lse = M + log(W);
    return HTA_ORACLE_OK;
}

/*
 * Attention mass per prefix chunk for an explicit list of rows (b, h, i).  With p_j the
 * softmax weights of the row's full verification attention (over its visible prefix and
 * tree keys, as above),
 *   mass[r, s]       = sum of p_j over the prefix keys j in [s*chunk, (s+1)*chunk), s < nchunks
 *   mass[r, nchunks] = sum of p_j over the row's visible tree keys
 * so every row sums to 1.  This is each split-K chunk's share of the row's attention
 * (LongSpec README, Introduction: the prefix part is computed chunk-parallel and aggregated
 * through the partial log-sum-exps).  nchunks * chunk must cover Lmax.
 */
int hta_oracle_chunk_mass(int B, int T, int Hq, int Hkv, int D, int Lmax, int is_bf16,
                          const void *q, const void *k_prefix, const void *k_tree,
                          const int32_t *parent, const int32_t *prefix_len, double scale,
                          int chunk, int nchunks, int nrows, const int32_t *row_b,
                          const int32_t *row_h, const int32_t *row_i, double *mass)
{
    if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Lmax < 0 || Hq % Hkv != 0 ||
        chunk <= 0 || nchunks < 0 || (long long)nchunks * chunk < Lmax)
        return HTA_ORACLE_BAD_ARG;
    for (int b = 0; b < B; ++b) {
        if (prefix_len[b] < 0 || prefix_len[b] > Lmax)
            return HTA_ORACLE_BAD_ARG;
        if (!tree_is_valid(parent + (size_t)b * T, T))
            return HTA_ORACLE_BAD_TREE;
    }
    const int G = Hq / Hkv;
    double *scores = (double *)malloc(((size_t)Lmax + (size_t)T) * sizeof(double));
    unsigned char *in_tree = (unsigned char *)malloc((size_t)T);
    if (!scores || !in_tree) {
        free(scores); free(in_tree);
        return HTA_ORACLE_NOMEM;
    }
    int rc = HTA_ORACLE_OK;
    for (int r = 0; r < nrows; ++r) {
        const int b = row_b[r], h = row_h[r], i = row_i[r];
        if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= T) {
            rc = HTA_ORACLE_BAD_ARG;
            break;
        }
        const int g = h / G, L = prefix_len[b];
        const size_t qoff = (((size_t)b * T + i) * Hq + h) * D;
        const size_t pbase = ((size_t)b * Hkv + g) * (size_t)Lmax * D;
        const size_t tbase = ((size_t)b * Hkv + g) * (size_t)T * D;
        const int32_t *par = parent + (size_t)b * T;
        memset(in_tree, 0, (size_t)T);
        for (int p = i; p != -1; p = par[p])
            in_tree[p] = 1;
        /* scores of the visible keys: prefix keys 0..L-1, then tree keys t (in_tree[t]) */
        double m = -INFINITY;
        for (int j = 0; j < L + T; ++j) {
            if (j >= L && !in_tree[j - L])
                continue;
            double s = 0.0;
            for (int d = 0; d < D; ++d) {
                const double kd = j < L ? widen(k_prefix, pbase + (size_t)j * D + d, is_bf16)
                                        : widen(k_tree, tbase + (size_t)(j - L) * D + d, is_bf16);
                s += widen(q, qoff + d, is_bf16) * kd;
            }
            scores[j] = s * scale;
            if (scores[j] > m)
                m = scores[j];
        }
        double Z = 0.0;
        for (int j = 0; j < L + T; ++j)
            if (j < L || in_tree[j - L])
                Z += exp(scores[j] - m);
        double *row = mass + (size_t)r * (nchunks + 1);
        for (int s = 0; s <= nchunks; ++s)
            row[s] = 0.0;
        for (int j = 0; j < L + T; ++j) {
            if (j >= L && !in_tree[j - L])
                continue;
            const int bin = j < L ? j / chunk : nchunks;
            row[bin] += exp(scores[j] - m) / Z;
        }
    }
    free(scores); free(in_tree);
    return rc;
}
