/*
 * hta.h -- C ABI of the MI355X (gfx950) tree verification attention library (libhta.so).
 *
 * What the library computes.  LongSpec verifies a speculated draft tree with one target
 * forward pass whose attention is split in two (LongSpec README, Introduction, "Hybrid
 * Attention Aggregation"; paper summary, Summary, "Hybrid Tree Attention"; arXiv abstract):
 * the tree tokens attend to the whole prefix KV cache with no mask, and to each other under
 * the tree mask; the two partial results are aggregated.  The decoding is lossless (README
 * title; summary, first paragraph), so the aggregate here is exact: for batch b, query head
 * h, tree node i, with g = h / (Hq / Hkv),
 *
 *     visible(i) = { prefix keys j < prefix_len[b] }  U  { tree node i and its ancestors }
 *     out[b,i,h,:] = softmax_j( scale * q[b,i,h,:] . k_j ) @ v_j        over j in visible(i)
 *     lse[b,h,i]   = ln sum_j exp( scale * q[b,i,h,:] . k_j )
 *
 * computed as partial attentions over key chunks (split-K over the prefix, one partial for
 * the tree) merged through their log-sum-exp statistics.
 *
 * Layouts (all row-major, contiguous, caller-owned device memory):
 *     q            [B, T, Hq, D]        in_dtype
 *     k_prefix     [B, Hkv, Lmax, D]    in_dtype   rows >= prefix_len[b] are never read
 *     v_prefix     [B, Hkv, Lmax, D]    in_dtype   (they may hold anything, NaN included)
 *     k_tree       [B, Hkv, T, D]       in_dtype   (q and k arrive already position-encoded)
 *     v_tree       [B, Hkv, T, D]       in_dtype
 *     parent_idx   [B, T]   int32       parent of node i, -1 for a child of the prefix;
 *                                       nodes must be in topological order: parent < i
 *     prefix_len   [B]      int32       0 <= prefix_len[b] <= Lmax (0 allowed)
 *     out          [B, T, Hq, D]        float32
 *     lse          [B, Hq, T]           float32, natural log
 *     masks        [B, T, ceil(T/64)]   uint64: bit (t % 64) of word t / 64 of node i is set
 *                                       iff tree node t is i or an ancestor of i
 *
 * Ownership and threading.  The library allocates nothing and frees nothing.  Every call
 * takes a caller-allocated device workspace of at least hta_workspace_size() bytes and a
 * HIP stream (passed as void*, a hipStream_t; NULL = the default stream).  Calls are
 * asynchronous: a return of HTA_OK means the work was enqueued on the stream.  The library
 * keeps no mutable global state (plans are a pure function of the descriptor), so calls on
 * different streams with different workspaces may run concurrently; calls that share a
 * workspace must be ordered by the caller.
 *
 * Errors.  Every argument check happens on the host before anything is enqueued; on an
 * error the call returns a non-zero hta_status and enqueues nothing.  Errors only visible on
 * the device (a parent pointer outside [-1, i-1], a prefix_len outside [0, Lmax]) make the
 * affected sequence's out and lse rows NaN and are recorded in the workspace; read them
 * with hta_get_device_status().
 *
 * Limits: head_dim in {64, 128}; 1 <= tree_size <= 256; num_q_heads % num_kv_heads == 0;
 * num_q_heads / num_kv_heads <= 16; batch <= 65535; batch * tree_size * num_q_heads < 2^31
 * - 1024; num_kv_heads times the query-row blocks (ceil(tree_size * group / 272), at most 16)
 * <= 65535; every tensor pointer 16-byte aligned, the workspace
 * 256-byte aligned.  in_dtype HTA_BF16 runs the matrix-core kernels (bf16 products, fp32
 * accumulation, probabilities entering the PV product as fp16 and normalised by the sum of
 * those same rounded values, so a prefix part's log-sum-exp is within 2^-11 of the exact
 * one); HTA_F32 runs exact fp32 vector-ALU kernels meant for small validation shapes (same
 * plan, workspace and layouts).  Range of bf16 values: the PV products of the prefix pass
 * (and of hta_tree_partials) take V as fp16, so a prefix V value with |v| > 65504 -- legal in
 * bf16 -- is not supported: it makes its chunk's partial non-finite, and the merge then
 * writes every affected output row (out and lse) as NaN and records HTA_ERR_NONFINITE in the
 * workspace status (read with hta_get_device_status).  V values below 2^-14 in magnitude
 * enter as fp16 subnormals (absolute error at most 2^-25).  Any non-finite input (NaN/inf in
 * q, k or v, padding past prefix_len excluded) is reported the same way.  The tree keys of
 * hta_verify are exempt: its tree part runs in fp32.
 */
#ifndef HTA_H
#define HTA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HTA_OK = 0,
    HTA_ERR_NULL = 1,        /* a required pointer is NULL */
    HTA_ERR_SHAPE = 2,       /* a size is out of the supported range or inconsistent */
    HTA_ERR_DTYPE = 3,       /* unsupported in_dtype */
    HTA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    HTA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than hta_workspace_size() */
    HTA_ERR_TREE = 6,        /* (device) a parent pointer outside [-1, i-1] */
    HTA_ERR_PREFIX_LEN = 7,  /* (device) prefix_len[b] outside [0, max_prefix_len] */
    HTA_ERR_HIP = 8,         /* a HIP runtime call failed */
    HTA_ERR_CACHE_FULL = 9,  /* (device) prefix_len[b] + accepted nodes > max_prefix_len */
    HTA_ERR_NONFINITE = 10,  /* (device) an output row came out non-finite and was NaN-filled */
    HTA_ERR_SCRATCH = 11,    /* hta_verify_noalloc: the plan needs more than its static scratch */
    /* not a status: makes every int32_t value a valid hta_status, so hta_status_str() may be
     * handed any code (unknown ones read "HTA_ERR_UNKNOWN") */
    HTA_STATUS_MAX_ENUM = 0x7FFFFFFF
} hta_status;

typedef enum { HTA_BF16 = 0, HTA_F32 = 1 } hta_dtype;

/* Problem descriptor.  chunk = 0 lets the library pick the split-K chunk length. */
typedef struct {
    int32_t batch;          /* B */
    int32_t num_q_heads;    /* Hq */
    int32_t num_kv_heads;   /* Hkv; query head h reads KV head h / (Hq / Hkv) */
    int32_t head_dim;       /* D, 64 or 128 */
    int32_t tree_size;      /* T, draft tree nodes per sequence */
    int32_t max_prefix_len; /* Lmax, the prefix KV cache capacity (row stride of k/v_prefix) */
    int32_t in_dtype;       /* hta_dtype of q, k_*, v_* */
    float scale;            /* softmax scale; 0 means 1/sqrt(head_dim) */
    int32_t chunk;          /* prefix keys per split-K partial (multiple of 64); 0 = auto */
} hta_desc;

/* How a descriptor is executed; filled by hta_plan().  Sizes in bytes, offsets into the
 * workspace.  Partial results of split s (s < num_splits: prefix keys
 * [s*chunk, min((s+1)*chunk, prefix_len[b])); s == num_splits: the tree keys) live at
 *   lse_part[n], o_scale[n]                                                  (float)
 *   o_part row n                                                             (2*D bytes)
 * with n = ((b*Hkv + g)*(num_splits+1) + s)*rows_padded + r, where row r =
 * i*(Hq/Hkv) + (h % (Hq/Hkv)) packs the query heads sharing KV head g.  o_part holds the
 * normalised partial output, lse_part its natural-log normaliser (-inf for an empty chunk).
 * Splits at or past ceil(prefix_len[b]/chunk) are not written.
 * An o_part row stores D little-endian int16 values q_d (q_0 first); value d of the row is
 * q_d * o_scale[n].  The writer takes m >= max_d |x_d| (the row's largest magnitude, or a
 * bound on it no larger than the largest |v| the row attends to) and sets o_scale = m / 32767
 * and q_d = x_d * 32767 / m rounded to the nearest integer (ties to even), so |q_d| <= 32767
 * and a value's error is at most 2^-16 m (plus fp32 rounding); o_scale is 0 for an all-zero
 * row and NaN for a row holding a non-finite value. */
typedef struct {
    int32_t chunk;          /* prefix keys per split */
    int32_t num_splits;     /* ceil(max_prefix_len / chunk), at least 1 */
    int32_t rows;           /* T * Hq / Hkv: query rows per (b, kv head) */
    int32_t rows_padded;    /* rows rounded up to a multiple of 16 */
    size_t status_offset;   /* int32 [B]: device status per sequence */
    size_t masks_offset;    /* uint64 [B, T, ceil(T/64)] */
    size_t lse_part_offset;
    size_t o_part_offset;
    size_t o_scale_offset;  /* float, one per o_part row */
    size_t workspace_bytes; /* total, == hta_workspace_size() */
} hta_plan_info;

/* Fill *info for a descriptor.  Returns HTA_ERR_SHAPE/HTA_ERR_DTYPE/HTA_ERR_NULL on a bad
 * descriptor. */
hta_status hta_plan(const hta_desc *desc, hta_plan_info *info);

/* Workspace bytes needed by every entry point for this descriptor (0 if it is invalid). */
size_t hta_workspace_size(const hta_desc *desc);

/*
 * The whole verification attention step -> out, lse: the split-K prefix partials, then the
 * exact LSE aggregation with the tree part (README, Introduction; summary, Summary; arXiv
 * abstract).  Two launches: the prefix pass, and a merge that computes each row's tree
 * attention over its node's parent chain itself (validating the trees and recording the
 * device status) instead of reading a tree partial; the ancestor masks are not materialised
 * here (hta_ancestor_masks builds them).  The workspace partial buffers are overwritten:
 * the prefix slots with the prefix partials, the tree slot's lse_part with the tree part's
 * log-sum-exp (its o_part row is left as it was).
 */
hta_status hta_verify(const hta_desc *desc, const void *q, const void *k_prefix,
                      const void *v_prefix, const void *k_tree, const void *v_tree,
                      const int32_t *parent_idx, const int32_t *prefix_len, float *out,
                      float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * hta_verify without a workspace argument and without any allocation, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same launches, results bit-identical to hta_verify.
 * The workspace is a static device array inside the library, HTA_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, held by every GPU the library runs on until the process ends; a
 * descriptor whose hta_workspace_size() exceeds it is refused with HTA_ERR_SCRATCH before
 * anything is enqueued.  Every call on one GPU shares that GPU's scratch: calls that overlap
 * on one GPU (different streams, threads) race and must be ordered by the caller.  status
 * (device int32 [B], may be NULL) receives the per-sequence device verdicts that
 * hta_get_device_status would report, as OR-ed flags (1: invalid tree, 2: prefix_len out of
 * range, 8: a non-finite row); with NULL they stay in the scratch, and the affected rows are
 * NaN either way.  The first call on a device looks up the scratch's address (no allocation).
 */
#define HTA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hta_status hta_verify_noalloc(const hta_desc *desc, const void *q, const void *k_prefix,
                              const void *v_prefix, const void *k_tree, const void *v_tree,
                              const int32_t *parent_idx, const int32_t *prefix_len, float *out,
                              float *lse, int32_t *status, void *stream);

/*
 * Ancestor-or-self masks of every draft tree (the tree mask of README, Introduction),
 * built on the device from the parent pointers by pointer jumping, into masks (device,
 * uint64 [B, T, ceil(T/64)]).  An invalid tree is recorded in the workspace status and its
 * masks are written as all-ones.
 */
hta_status hta_ancestor_masks(const hta_desc *desc, const int32_t *parent_idx, uint64_t *masks,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Prefix part only, left as split-K partials in the workspace (layout in hta_plan_info):
 * the unmasked attention of every tree query over its sequence's prefix keys (summary,
 * Summary: the prefix pass).  The tree partial slot is not touched.
 */
hta_status hta_prefix_partials(const hta_desc *desc, const void *q, const void *k_prefix,
                               const void *v_prefix, const int32_t *prefix_len, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * Tree part only, left as the partial of slot s = num_splits in the workspace, plus the
 * ancestor masks in the workspace: tree queries over tree keys under the ancestor-or-self
 * mask (summary, Summary: the tree pass).  Also records device status.
 */
hta_status hta_tree_partials(const hta_desc *desc, const void *q, const void *k_tree,
                             const void *v_tree, const int32_t *parent_idx,
                             const int32_t *prefix_len, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * Aggregation only: merge the prefix partials s < ceil(prefix_len[b]/chunk) and the tree
 * partial found in the workspace into out, lse through their log-sum-exp statistics
 * (README, Introduction: the aggregation; exact because the decoding is lossless).
 * include_tree = 0 merges the prefix partials alone (prefix-only attention; an empty
 * prefix then gives out = 0, lse = -inf).
 */
hta_status hta_merge(const hta_desc *desc, const int32_t *prefix_len, int32_t include_tree,
                     float *out, float *lse, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * Each prefix chunk's share of every query row's attention, and the tree's: the split-K
 * partial log-sum-exps of the last hta_verify call on this workspace (or of
 * hta_prefix_partials + hta_tree_partials) against the rows' final lse from that call
 * (README, Introduction: the prefix is attended chunk by chunk and aggregated through
 * these statistics):
 *     mass[b, h, i, s] = exp(lse_part[b, g, s, r] - lse[b, h, i])     s <= num_splits
 * with g, r the row's KV head and packed row (hta_plan_info), column s < num_splits the
 * prefix keys [s*chunk, (s+1)*chunk) (0 for chunks past prefix_len[b]) and column
 * num_splits the tree; every row sums to 1 up to rounding.  mass is float
 * [B, Hq, T, num_splits + 1] (device).  chunk_scores (device float [B, num_splits + 1], may
 * be NULL) receives each column's mean over the sequence's Hq * T rows, summed in a fixed
 * order (bitwise reproducible): the attention each prefix chunk received, e.g. to choose
 * the context a drafter keeps.  The chunk length is the plan's (set desc->chunk to choose
 * the granularity; it must be the one the partials were computed with).  Rows of a
 * sequence that hta_verify rejected are NaN.  batch <= 65535.
 */
hta_status hta_chunk_mass(const hta_desc *desc, const int32_t *prefix_len, const float *lse,
                          float *mass, float *chunk_scores, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * ---- The drafter's attention (paper summary, Summary: a one-block drafter with
 *      sliding-window self-attention, window 512, and cross-attention into the target
 *      model's KV cache) ----
 *
 * Cross-attention: the drafter's queries attend to one layer of the target's KV cache with
 * no mask: desc->tree_size = Tq query tokens per sequence, desc->max_prefix_len = the cache
 * capacity; q [B, Tq, Hq, D], k_cache / v_cache [B, Hkv, Lmax, D] (the prefix layout),
 * cache_len [B] (keys j < cache_len[b] are seen) -> out [B, Tq, Hq, D] float, lse [B, Hq, Tq].
 * Two launches: the split-K prefix pass and the merge of its partials (no tree part).  A
 * sequence with cache_len 0 gets out 0, lse -inf; a cache_len outside [0, Lmax] gives NaN
 * (not recorded in the status); a non-finite output row is NaN-filled and recorded as
 * HTA_ERR_NONFINITE in the workspace status, which this call clears first.
 */
hta_status hta_cross_attention(const hta_desc *desc, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *cache_len, float *out,
                               float *lse, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * The drafter's sliding-window self-attention while it drafts a tree is hta_verify with its
 * window cache as the prefix: the cache is a ring of `window` slots holding the K/V of the
 * last `window` committed positions (position p in slot p % window; keys carry their
 * positions through the rotary encoding, and attention over a set of keys does not depend
 * on their order), desc->max_prefix_len = window, prefix_len[b] = min(committed, window);
 * the draft tree's own nodes are seen under the tree mask as in verification.
 *
 * hta_window_commit appends the accepted path's drafter K/V rows (node accepted[b, k] of
 * k_tree / v_tree [B, Hkv, T, D], k < accept_len[b]) to the ring [B, Hkv, window, D] at slots
 * (win_pos[b] + k) % window, and advances win_pos[b] by accept_len[b] (in place).  Only the
 * last `window` rows of a longer path are written.  accept_len outside [0, T] or a negative
 * win_pos is a device error (HTA_ERR_PREFIX_LEN in the status, nothing written).  Only the
 * status words of the workspace are written (any buffer of 4 * batch bytes rounded up to 256).
 */
hta_status hta_window_commit(const hta_desc *desc, int32_t window, void *k_win, void *v_win,
                             const void *k_tree, const void *v_tree, const int32_t *accepted,
                             const int32_t *accept_len, int32_t *win_pos, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * ---- Verification without the hybrid split: the method's "before" ----
 *
 * The paper summary (Summary; Key points, "Hybrid Tree Attention") says a tree mask keeps
 * verification off the optimized long-context attention kernels and that the hybrid split
 * cut the target's attention latency to about a quarter.  These two calls are that "before"
 * on this hardware: an explicit mask over all L + T keys of every node, and one masked
 * attention pass over them (parallel over query tiles and KV heads, every workgroup
 * streaming the whole key range of its KV head; no split over keys, no merge).  Same
 * result as hta_verify (up to rounding) when the mask is the one hta_dense_mask builds.
 *
 * Mask layout (word-major): uint64 [B, W, T_pad] with W = ceil(Lmax/64) + ceil(T/64) words
 * per node and T_pad = T rounded up to even; word w of node i of sequence b is element
 * (b, w, i).  Bit j % 64 of word j / 64 is prefix key j; bit t % 64 of word
 * ceil(Lmax/64) + t / 64 is tree key t.  (Word-major, so the words one key tile needs for
 * consecutive nodes are contiguous.)
 */

/* Bytes of the explicit mask, 8 * B * W * T_pad (0 for an invalid descriptor). */
size_t hta_dense_mask_bytes(const hta_desc *desc);

/*
 * Build the explicit mask of every node: prefix keys j < prefix_len[b] and the node's
 * ancestors-or-self in the tree.  An invalid tree or prefix_len leaves that sequence's mask
 * all zero (its rows then see nothing: out 0, lse -inf) and is recorded in the workspace
 * status (any buffer of at least 4 * batch bytes rounded up to 256).  The padding column of
 * an odd T is written as zero.
 */
hta_status hta_dense_mask(const hta_desc *desc, const int32_t *parent_idx,
                          const int32_t *prefix_len, uint64_t *mask, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Single-pass masked attention over all L + T keys: key j < prefix_len[b] of the prefix or
 * tree key t is visible to node i iff its mask bit is set.  out, lse as for hta_verify (a
 * row that sees no key gets out 0, lse -inf; a prefix_len outside [0, Lmax] gives NaN).
 * bf16 inputs only.  No workspace.
 */
hta_status hta_verify_dense(const hta_desc *desc, const void *q, const void *k_prefix,
                            const void *v_prefix, const void *k_tree, const void *v_tree,
                            const uint64_t *mask, const int32_t *prefix_len, float *out,
                            float *lse, void *stream);

/*
 * ---- The steps on either side of the attention in one greedy verification step ----
 *
 * Speculative decoding at temperature 0 (LongSpec README, Evaluation: both inference
 * commands pass --temperature 0 and --tree_shape 4 16 16 16 16) verifies a draft tree as
 * follows: the tree's queries and keys are position-encoded at the tree positions, the
 * attention above runs, the target's greedy token after every node is read off its logits,
 * the longest drafted path that agrees with those tokens is accepted, and the accepted
 * path's keys and values join the prefix cache.  The emitted tokens are exactly those plain
 * greedy decoding emits (the lossless property, README title).
 */

/*
 * Rotary position encoding of the draft tree, in place (RoFormer, cited by the LongSpec
 * paper).  Node i of sequence b sits at position prefix_len[b] + depth(i), depth 0 for a
 * node whose parent is -1.  Pair j of every head vector of q [B,T,Hq,D] and k_tree
 * [B,Hkv,T,D] (in_dtype) is turned by the angle position * rope_theta^(-2j/D):
 *     (x_a, x_c) -> (x_a cos - x_c sin, x_c cos + x_a sin)
 * with pairs (a, c) = (j, j + D/2) when interleaved == 0 (the Llama / Qwen layout) and
 * (2j, 2j + 1) when interleaved != 0.  Angles and products are evaluated in fp64 and each
 * result is rounded once to in_dtype (nearest even), so positions far beyond 2^16 keep
 * their accuracy.  positions (device int32 [B, T], may be NULL) receives the positions.
 * Device errors (an invalid tree, prefix_len outside [0, Lmax]) are recorded in the
 * workspace status (read with hta_get_device_status) and make that sequence's q and k_tree
 * rows NaN and its positions -1.  Only the status words at the start of the workspace are
 * written: any buffer of at least 4 * batch bytes rounded up to 256 serves (a workspace of
 * hta_verify does).  rope_theta must be positive and finite.
 */
hta_status hta_rope_tree(const hta_desc *desc, double rope_theta, int32_t interleaved, void *q,
                         void *k_tree, const int32_t *parent_idx, const int32_t *prefix_len,
                         int32_t *positions, void *workspace, size_t workspace_bytes,
                         void *stream);

/* Workspace bytes for hta_accept_commit with this vocabulary size (0 if invalid); at least
 * hta_workspace_size(desc), so one buffer of this size serves every entry point. */
size_t hta_accept_workspace_size(const hta_desc *desc, int32_t vocab);

/*
 * Greedy acceptance and KV commit (temperature 0; README, Evaluation).
 *   logits      [B, T, vocab]  logits_dtype (HTA_BF16 or HTA_F32): the target's scores for
 *                              the token after every tree node
 *   tokens      [B, T]  int32  the drafted token of every node
 *   root_token  [B]     int32  the target's greedy token for the position after the prefix
 * Outputs (device int32):
 *   target_next [B, T]  index of the largest logit of each row; ties go to the smallest
 *                       index, +0 equals -0, and a NaN counts as larger than any number
 *   accept_len  [B]     accepted nodes n: the walk starts from the prefix expecting
 *                       root_token[b]; while some child of the last accepted node (a root,
 *                       at the start) carries the expected token, the one with the smallest
 *                       index is accepted and target_next of it becomes the expected token
 *   accepted    [B, T]  the accepted nodes in path order, -1 past n
 *   bonus_token [B]     the expected token after the last accepted node (the target's own
 *                       token, emitted in addition to the n accepted ones)
 * KV commit, in place: row k < n of the path (node accepted[b,k]) of k_tree / v_tree is
 * copied to row prefix_len[b] + k of k_prefix / v_prefix for every KV head (in_dtype), and
 * prefix_len[b] grows by n.  The bonus token has no key or value yet and is not committed.
 * Device errors, recorded in the workspace status: an invalid tree (n = 0, accepted all -1,
 * bonus -1, nothing committed), prefix_len outside [0, Lmax] or a path that does not fit
 * (HTA_ERR_CACHE_FULL): the acceptance outputs are written, the cache and prefix_len are
 * left unchanged.  Any vocab >= 1 (rows whose byte length is a multiple of 16 and a
 * 16-byte aligned logits pointer take the vector path).  The workspace must hold
 * hta_accept_workspace_size(desc, vocab) bytes.
 */
hta_status hta_accept_commit(const hta_desc *desc, int32_t vocab, int32_t logits_dtype,
                             const void *logits, const int32_t *tokens,
                             const int32_t *root_token, const int32_t *parent_idx,
                             int32_t *prefix_len, void *k_prefix, void *v_prefix,
                             const void *k_tree, const void *v_tree, int32_t *target_next,
                             int32_t *accept_len, int32_t *accepted, int32_t *bonus_token,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Synchronise the stream, read the device status the last hta_verify / hta_tree_partials /
 * hta_ancestor_masks / hta_rope_tree / hta_accept_commit / hta_cross_attention call left in
 * the workspace (hta_merge adds non-finite rows to it), and return HTA_OK, HTA_ERR_TREE,
 * HTA_ERR_PREFIX_LEN, HTA_ERR_CACHE_FULL or HTA_ERR_NONFINITE (reported in that order of
 * precedence).  *bad_sequence (if not NULL) receives the first offending batch index, or -1.
 */
hta_status hta_get_device_status(const hta_desc *desc, const void *workspace, void *stream,
                                 int32_t *bad_sequence);

/* Measurement helper, not part of the verification path: the matrix-core rate this GPU
 * sustains, for reporting the prefix pass against a peak measured on the machine (the pages
 * give no hardware; the data-sheet peak assumes clocks a part may not hold under matrix load).
 * Enqueues on `stream` one launch of `blocks` workgroups of 8 waves; every wave runs `iters`
 * rounds of eight independent v_mfma_f32_16x16x32_bf16 products on register operands (no
 * memory traffic), then writes one float per lane to `out` (device, blocks * 512 floats,
 * 16-byte aligned; the values are meaningless).  *flops (host) receives the launch's
 * matrix-core flops (16384 per product); divide by the launch's duration, timed by the caller
 * on the same stream.  1 <= blocks <= 2^20, 1 <= iters <= 2^24, else HTA_ERR_SHAPE;
 * HTA_ERR_NULL / HTA_ERR_ALIGN / HTA_ERR_HIP as for the other calls. */
hta_status hta_mfma_peak_probe(int32_t blocks, int32_t iters, float *out, void *stream,
                               double *flops);

/* Static, human-readable name of a status code (never NULL). */
const char *hta_status_str(hta_status status);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t hta_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HTA_H */
