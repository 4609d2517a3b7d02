/*
 * step_oracle.c -- CPU oracle for the steps around the verification attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark load this code.  The GPU library never links, calls or includes it, and
 * this file includes nothing of the GPU library.
 *
 * One greedy verification step of tree speculative decoding (LongSpec README, Evaluation:
 * both inference commands decode at temperature 0 with a draft tree of level widths
 * 4,16,16,16,16) has, around the attention:
 *
 *  before: rotary position encoding of the tree's queries and keys.  A draft node sits at
 *          position prefix_len + depth, its depth counted from 0 at the nodes that hang off
 *          the prefix.  The rotation is RoFormer's (Su et al., "RoFormer: Enhanced
 *          transformer with rotary position embedding", cited by the LongSpec paper):
 *          pair j of a head vector (frequency theta^(-2j/D)) is turned by the angle
 *          position * theta^(-2j/D).  Pairs are (j, j + D/2) ("half" layout, the one of
 *          the Llama and Qwen checkpoints the README evaluates) or (2j, 2j+1)
 *          ("interleaved", RoFormer's own notation).
 *  after:  greedy acceptance: the target's argmax token after each node is compared with
 *          the drafted tokens, starting from the target's token for the position right
 *          after the prefix; the accepted path is followed while a child of the last
 *          accepted node carries exactly the target's token.  Temperature 0 makes the
 *          emitted tokens those plain greedy decoding would emit (the lossless property
 *          of the README title).
 *
 * Single-threaded, scalar, fp64, compiled without fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define STEP_ORACLE_OK 0
#define STEP_ORACLE_BAD_TREE 1
#define STEP_ORACLE_BAD_ARG 2

static double widen_elem(const void *base, size_t idx, int is_bf16)
{
    if (is_bf16) {
        uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[idx];
}

/*
 * Depth of every node: the number of steps from it to a node whose parent is -1.
 * Rejects a parent pointer outside [-1, i-1] (nodes are in topological order).
 */
int step_oracle_depths(int B, int T, const int32_t *parent, int32_t *depth)
{
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * T;
        for (int i = 0; i < T; ++i)
            if (par[i] < -1 || par[i] >= i)
                return STEP_ORACLE_BAD_TREE;
        for (int i = 0; i < T; ++i) {
            int d = 0;
            for (int p = par[i]; p != -1; p = par[p])
                ++d;
            depth[(size_t)b * T + i] = d;
        }
    }
    return STEP_ORACLE_OK;
}

/*
 * Rotary encoding of the tree rows of one tensor, exact in fp64:
 *   layout 0: x is [B, T, H, D] (the queries), layout 1: x is [B, H, T, D] (the tree keys).
 * Node i of sequence b is at position prefix_len[b] + depth(i).  For pair j with elements
 * (a, c): angle = position * theta^(-2j/D), and
 *   out[a] = x[a] cos(angle) - x[c] sin(angle),   out[c] = x[c] cos(angle) + x[a] sin(angle)
 * (the vector (x[a], x[c]) read as the complex number x[a] + i x[c], times e^{i angle}).
 * out has x's shape, fp64.  positions (may be NULL) receives [B, T] int32.
 */
int step_oracle_rope(int B, int T, int H, int D, int layout, int is_bf16, const void *x,
                     const int32_t *parent, const int32_t *prefix_len, double theta,
                     int interleaved, double *out, int32_t *positions)
{
    if (B < 1 || T < 1 || H < 1 || D < 2 || D % 2 != 0 || (layout != 0 && layout != 1) ||
        !(theta > 0.0))
        return STEP_ORACLE_BAD_ARG;
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * T;
        for (int i = 0; i < T; ++i)
            if (par[i] < -1 || par[i] >= i)
                return STEP_ORACLE_BAD_TREE;
    }
    const int half = D / 2;
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * T;
        for (int i = 0; i < T; ++i) {
            int depth = 0;
            for (int p = par[i]; p != -1; p = par[p])
                ++depth;
            const int64_t pos = (int64_t)prefix_len[b] + depth;
            if (positions)
                positions[(size_t)b * T + i] = (int32_t)pos;
            for (int h = 0; h < H; ++h) {
                const size_t row = layout == 0 ? (((size_t)b * T + i) * H + h) * D
                                               : (((size_t)b * H + h) * T + i) * D;
                for (int j = 0; j < half; ++j) {
                    const int a = interleaved ? 2 * j : j;
                    const int c = interleaved ? 2 * j + 1 : j + half;
                    const double freq = pow(theta, -2.0 * (double)j / (double)D);
                    const double angle = (double)pos * freq;
                    const double cs = cos(angle), sn = sin(angle);
                    const double xa = widen_elem(x, row + a, is_bf16);
                    const double xc = widen_elem(x, row + c, is_bf16);
                    out[row + a] = xa * cs - xc * sn;
                    out[row + c] = xc * cs + xa * sn;
                }
            }
        }
    }
    return STEP_ORACLE_OK;
}

/*
 * Round fp64 values to bf16 bit patterns, to nearest, ties to even, in one rounding:
 * the double's significand is cut to bf16's 8 bits.  Results beyond bf16's range become
 * infinities; NaN stays NaN.  (Results below 2^-126 in magnitude are not produced by the
 * tests' inputs; they would be rounded a second time by the float conversion.)
 */
void step_oracle_round_bf16(size_t n, const double *x, uint16_t *out)
{
    for (size_t k = 0; k < n; ++k) {
        uint64_t u;
        memcpy(&u, &x[k], sizeof u);
        if (isnan(x[k])) {
            out[k] = 0x7FC0;
            continue;
        }
        /* keep the sign, the exponent and the top 7 stored significand bits */
        const uint64_t drop = 52 - 7;
        const uint64_t half_ulp = (1ull << (drop - 1)) - 1 + ((u >> drop) & 1);
        u = (u + half_ulp) & ~((1ull << drop) - 1);
        double r;
        memcpy(&r, &u, sizeof r);
        const float f = (float)r; /* exact unless out of float range (then +-inf) */
        uint32_t fb;
        memcpy(&fb, &f, sizeof fb);
        out[k] = (uint16_t)(fb >> 16);
    }
}

/*
 * Index of the largest element of each row of logits [rows, V] (the target's greedy token).
 * Ties go to the smallest index; +0 and -0 compare equal; a NaN counts as larger than every
 * number, so the first NaN of a row is its argmax.
 */
int step_oracle_argmax(int rows, int V, int is_bf16, const void *logits, int32_t *idx)
{
    if (rows < 0 || V < 1)
        return STEP_ORACLE_BAD_ARG;
    for (int r = 0; r < rows; ++r) {
        const size_t base = (size_t)r * V;
        int best = 0;
        double bv = widen_elem(logits, base, is_bf16);
        for (int j = 1; j < V && !isnan(bv); ++j) {
            const double v = widen_elem(logits, base + j, is_bf16);
            if (isnan(v) || v > bv) {
                best = j;
                bv = v;
            }
        }
        idx[r] = best;
    }
    return STEP_ORACLE_OK;
}

/*
 * Greedy acceptance along each draft tree.
 *   tokens[b, i]      drafted token of node i
 *   target_next[b, i] the target's greedy token for the position after node i
 *   root_token[b]     the target's greedy token for the position after the prefix
 * Walk from the prefix: the token expected next is root_token[b]; among the nodes whose
 * parent is the last accepted node (-1 at the start) and whose token equals the expected
 * one, accept the one with the smallest index, and expect target_next of it next.  Stop
 * when no such child exists.  Outputs: accept_len[b] (nodes accepted), accepted[b, k] (the
 * k-th accepted node, -1 past accept_len), bonus[b] (the token expected after the last
 * accepted node: the target's own token that the step emits in addition).
 */
int step_oracle_accept(int B, int T, const int32_t *parent, const int32_t *tokens,
                       const int32_t *root_token, const int32_t *target_next,
                       int32_t *accept_len, int32_t *accepted, int32_t *bonus)
{
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * T;
        for (int i = 0; i < T; ++i)
            if (par[i] < -1 || par[i] >= i)
                return STEP_ORACLE_BAD_TREE;
    }
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * T;
        const int32_t *tok = tokens + (size_t)b * T;
        const int32_t *nxt = target_next + (size_t)b * T;
        int32_t *acc = accepted + (size_t)b * T;
        for (int k = 0; k < T; ++k)
            acc[k] = -1;
        int last = -1, n = 0;
        int32_t expect = root_token[b];
        while (n < T) { /* a path has at most T nodes */
            int chosen = -1;
            for (int i = 0; i < T; ++i)
                if (par[i] == last && tok[i] == expect) {
                    chosen = i;
                    break;
                }
            if (chosen < 0)
                break;
            acc[n++] = chosen;
            last = chosen;
            expect = nxt[chosen];
        }
        accept_len[b] = n;
        bonus[b] = expect;
    }
    return STEP_ORACLE_OK;
}
