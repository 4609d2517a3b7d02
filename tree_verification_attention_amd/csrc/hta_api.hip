// hta_api.hip -- the C ABI of libhta.so (declared in include/hta.h): argument checking,
// planning (split-K chunk, workspace carve-up) and the kernel launch sequence.
//
// Nothing here allocates device memory: the caller hands in the workspace.  All checks run
// on the host before the first launch, so a rejected call enqueues nothing.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/hta.h"
#include "hta_internal.h"

using hta::Geometry;
using hta::Workspace;

namespace {

// The split-K chunk is sized so one (sequence, KV head, row block) pass over the prefix
// spreads across the chip's compute units.  A fixed count keeps plans (and workspace
// sizes) independent of which device is current; MI355X has 256 CUs.
constexpr int64_t kPlanCUs = 256;
constexpr int kMinChunk = 256;
constexpr int kMaxChunk = 8192;
constexpr int kMaxTree = 256;
constexpr int kMaxGroup = 16;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

hta_status make_plan(const hta_desc* d, Geometry* g, hta_plan_info* info) {
  if (!d) return HTA_ERR_NULL;
  if (d->in_dtype != HTA_BF16 && d->in_dtype != HTA_F32) return HTA_ERR_DTYPE;
  if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->tree_size < 1 ||
      d->tree_size > kMaxTree || d->max_prefix_len < 0 ||
      (d->head_dim != 64 && d->head_dim != 128) || d->num_q_heads % d->num_kv_heads != 0 ||
      d->num_q_heads / d->num_kv_heads > kMaxGroup || !(d->scale >= 0.f) || isinf(d->scale) ||
      d->chunk < 0 || d->chunk % 64 != 0)
    return HTA_ERR_SHAPE;
  Geometry G;
  G.B = d->batch;
  G.T = d->tree_size;
  G.Hq = d->num_q_heads;
  G.Hkv = d->num_kv_heads;
  G.D = d->head_dim;
  G.Lmax = d->max_prefix_len;
  G.G = G.Hq / G.Hkv;
  G.R = G.T * G.G;
  G.R_pad = (G.R + 15) / 16 * 16;
  G.NT = G.R_pad / 16;
  G.W = (G.T + 63) / 64;
  G.scale = d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)G.D);
  G.f32 = d->in_dtype == HTA_F32 ? 1 : 0;
  int tpb, nb;
  hta::prefix_row_blocking(G, &tpb, &nb);
  const int64_t row_blocks = nb;
  // Launch limits, checked before anything is enqueued: the batch and the KV heads times row
  // blocks are grid dimensions (at most 65535 each), and the merge numbers its B*T*Hq output
  // rows with 32-bit integers.
  if (G.B > 65535 || G.Hkv * row_blocks > 65535 ||
      (int64_t)G.B * G.T * G.Hq > (int64_t)INT32_MAX - 1024)
    return HTA_ERR_SHAPE;
  int64_t chunk = d->chunk;
  if (chunk == 0) {
    // As many splits as keep every CU busy without a second partial wave of workgroups:
    // S = CUs / (B * Hkv * row blocks), at least one.  Batches may be ragged (prefix_len
    // varies); four workgroups per CU then balance the load.
    const int64_t waves = G.B > 1 ? 4 : 1;
    const int64_t units = (int64_t)G.B * G.Hkv * row_blocks;
    const int64_t splits = units >= kPlanCUs * waves ? 1 : (kPlanCUs * waves) / units;
    chunk = (G.Lmax + splits - 1) / splits;
    chunk = (chunk + 63) / 64 * 64;
    if (chunk < kMinChunk) chunk = kMinChunk;
    if (chunk > kMaxChunk) chunk = kMaxChunk;
  }
  G.chunk = (int32_t)chunk;
  int64_t S = (G.Lmax + chunk - 1) / chunk;
  if (S < 1) S = 1;
  if (S > (1 << 20)) return HTA_ERR_SHAPE;
  G.S = (int32_t)S;

  hta_plan_info p;
  memset(&p, 0, sizeof p);
  p.chunk = G.chunk;
  p.num_splits = G.S;
  p.rows = G.R;
  p.rows_padded = G.R_pad;
  size_t off = 0;
  p.status_offset = off;
  off = round_up(off + sizeof(int32_t) * (size_t)G.B, 256);
  p.masks_offset = off;
  off = round_up(off + sizeof(uint64_t) * (size_t)G.B * G.T * G.W, 256);
  const size_t parts = (size_t)G.B * G.Hkv * (size_t)(G.S + 1) * G.R_pad;
  p.lse_part_offset = off;
  off = round_up(off + sizeof(float) * parts, 256);
  p.o_scale_offset = off;
  off = round_up(off + sizeof(float) * parts, 256);
  p.o_part_offset = off;
  off = round_up(off + 2 * parts * G.D, 256);  // 16-bit values
  p.workspace_bytes = off;
  if (g) *g = G;
  if (info) *info = p;
  return HTA_OK;
}

Workspace carve(void* base, const hta_plan_info& p) {
  char* c = (char*)base;
  Workspace w;
  w.status = (int32_t*)(c + p.status_offset);
  w.masks = (uint64_t*)(c + p.masks_offset);
  w.lse_part = (float*)(c + p.lse_part_offset);
  w.o_scale = (float*)(c + p.o_scale_offset);
  w.o_part = (uint32_t*)(c + p.o_part_offset);
  w.status_reset = nullptr;
  return w;
}

hta_status check_ws(const hta_plan_info& p, const void* ws, size_t bytes) {
  if (!ws || bytes < p.workspace_bytes) return HTA_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255u) != 0) return HTA_ERR_ALIGN;
  return HTA_OK;
}

hta_status check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (!p) return HTA_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return HTA_ERR_ALIGN;
  return HTA_OK;
}

hta_status hip_status(hipError_t e) { return e == hipSuccess ? HTA_OK : HTA_ERR_HIP; }

// The prefix pass for the descriptor's input dtype: bf16 on the matrix cores, fp32 on the
// vector ALUs.
hipError_t launch_prefix(const Geometry& G, const void* q, const void* k_prefix,
                         const void* v_prefix, const int32_t* prefix_len, const Workspace& ws,
                         hipStream_t s) {
  return G.f32 ? hta::launch_prefix_attn_f32(G, q, k_prefix, v_prefix, prefix_len, ws, s)
               : hta::launch_prefix_attn_splitk(G, q, k_prefix, v_prefix, prefix_len, ws, s);
}

// ---- the allocation-free entry point's scratch
//
// hta_verify_noalloc serves callers that cannot allocate (code under HIP graph capture,
// tight serving loops): its workspace is this file-scope device array instead of a buffer
// the caller hands in.  Each GPU the library runs on holds its own copy until the process
// ends.  In host code `scratch` names a host-side stand-in, not device memory, so its
// device address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is ever passed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (looked up on the first call on that device).
hta_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HTA_ERR_HIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    // (two threads racing here both find the same address)
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HTA_ERR_HIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return HTA_OK;
}

#define HTA_TRY(expr)                  \
  do {                                 \
    hta_status _s = (expr);            \
    if (_s != HTA_OK) return _s;       \
  } while (0)

}  // namespace

extern "C" {

hta_status hta_plan(const hta_desc* desc, hta_plan_info* info) {
  if (!info) return HTA_ERR_NULL;
  return make_plan(desc, nullptr, info);
}

size_t hta_workspace_size(const hta_desc* desc) {
  hta_plan_info p;
  if (make_plan(desc, nullptr, &p) != HTA_OK) return 0;
  return p.workspace_bytes;
}

hta_status hta_verify(const hta_desc* desc, const void* q, const void* k_prefix,
                      const void* v_prefix, const void* k_tree, const void* v_tree,
                      const int32_t* parent_idx, const int32_t* prefix_len, float* out,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  Geometry G;
  hta_plan_info p;
  HTA_TRY(make_plan(desc, &G, &p));
  HTA_TRY(check_ptrs({q, k_tree, v_tree, parent_idx, prefix_len, out, lse}));
  if (G.Lmax > 0) HTA_TRY(check_ptrs({k_prefix, v_prefix}));  // an empty cache is never read
  HTA_TRY(check_ws(p, workspace, workspace_bytes));
  Workspace ws = carve(workspace, p);
  ws.status_reset = ws.status;  // the merge ORs this call's verdicts into cleared words
  hipStream_t s = (hipStream_t)stream;
  // two launches: the split-K prefix pass, then the merge with the tree part fused in
  HTA_TRY(hip_status(launch_prefix(G, q, k_prefix, v_prefix, prefix_len, ws, s)));
  return hip_status(hta::launch_tree_merge(G, q, k_tree, v_tree, parent_idx, prefix_len, out,
                                           lse, ws, s));
}

hta_status hta_verify_noalloc(const hta_desc* desc, const void* q, const void* k_prefix,
                              const void* v_prefix, const void* k_tree, const void* v_tree,
                              const int32_t* parent_idx, const int32_t* prefix_len, float* out,
                              float* lse, int32_t* status, void* stream) {
  Geometry G;
  hta_plan_info p;
  HTA_TRY(make_plan(desc, &G, &p));
  if (p.workspace_bytes > kScratchBytes) return HTA_ERR_SCRATCH;
  HTA_TRY(check_ptrs({q, k_tree, v_tree, parent_idx, prefix_len, out, lse}));
  if (G.Lmax > 0) HTA_TRY(check_ptrs({k_prefix, v_prefix}));
  if (status && !aligned16(status)) return HTA_ERR_ALIGN;
  void* base = nullptr;
  HTA_TRY(scratch_for_current_device(&base));
  Workspace ws = carve(base, p);
  if (status) ws.status = status;  // the caller reads the verdicts from its own buffer
  ws.status_reset = ws.status;     // cleared by the prefix pass, OR-ed by the merge
  hipStream_t s = (hipStream_t)stream;
  // the same two launches as hta_verify, on the static scratch
  HTA_TRY(hip_status(launch_prefix(G, q, k_prefix, v_prefix, prefix_len, ws, s)));
  return hip_status(hta::launch_tree_merge(G, q, k_tree, v_tree, parent_idx, prefix_len, out,
                                           lse, ws, s));
}

hta_status hta_ancestor_masks(const hta_desc* desc, const int32_t* parent_idx, uint64_t* masks,
                              void* workspace, size_t workspace_bytes, void* stream) {
  Geometry G;
  hta_plan_info p;
  HTA_TRY(make_plan(desc, &G, &p));
  if (!parent_idx || !masks) return HTA_ERR_NULL;
  if (!aligned16(parent_idx) || !aligned16(masks)) return HTA_ERR_ALIGN;
  HTA_TRY(check_ws(p, workspace, workspace_bytes));
  const Workspace ws = carve(workspace, p);
  // masks-only mode: no attention, prefix_len not read (status records tree validity only)
  return hip_status(hta::launch_tree_attn_masked(G, nullptr, nullptr, nullptr, parent_idx,
                                                 nullptr, ws, masks, false,
                                                 (hipStream_t)stream));
}

hta_status hta_prefix_partials(const hta_desc* desc, const void* q, const void* k_prefix,
                               const void* v_prefix, const int32_t* prefix_len, void* workspace,
                               size_t workspace_bytes, void* stream) {
  Geometry G;
  hta_plan_info p;
  HTA_TRY(make_plan(desc, &G, &p));
  HTA_TRY(check_ptrs({q, prefix_len}));
  if (G.Lmax > 0) HTA_TRY(check_ptrs({k_prefix, v_prefix}));
  HTA_TRY(check_ws(p, workspace, workspace_bytes));
  const Workspace ws = carve(workspace, p);
  return hip_status(launch_prefix(G, q, k_prefix, v_prefix, prefix_len, ws, (hipStream_t)stream));
}

hta_status hta_tree_partials(const hta_desc* desc, const void* q, const void* k_tree,
                             const void* v_tree, const int32_t* parent_idx,
                             const int32_t* prefix_len, void* workspace, size_t workspace_bytes,
                             void* stream) {
  Geometry G;
  hta_plan_info p;
  HTA_TRY(make_plan(desc, &G, &p));
  HTA_TRY(check_ptrs({q, k_tree, v_tree, parent_idx, prefix_len}));
  HTA_TRY(check_ws(p, workspace, workspace_bytes));
  const Workspace ws = carve(workspace, p);
  hipStream_t s = (hipStream_t)stream;
  if (G.f32) {  // masks and status, then the tree partial from the parent chains
    HTA_TRY(hip_status(hta::launch_tree_attn_masked(G, nullptr, nullptr, nullptr, parent_idx,
                                                    prefix_len, ws, ws.masks, false, s)));
    return hip_status(
        hta::launch_tree_chain(G, q, k_tree, v_tree, parent_idx, prefix_len, ws, s));
  }
  return hip_status(hta::launch_tree_attn_masked(G, q, k_tree, v_tree, parent_idx, prefix_len, ws,
                                                 ws.masks, true, s));
}

hta_status hta_merge(const hta_desc* desc, const int32_t* prefix_len, int32_t include_tree,
                     float* out, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream) {
  Geometry G;
  hta_plan_info p;
  HTA_TRY(make_plan(desc, &G, &p));
  HTA_TRY(check_ptrs({prefix_len, out, lse}));
  HTA_TRY(check_ws(p, workspace, workspace_bytes));
  const Workspace ws = carve(workspace, p);
  return hip_status(hta::launch_lse_merge(G, prefix_len, include_tree != 0, out, lse, ws,
                                          (hipStream_t)stream));
}

hta_status hta_rope_tree(const hta_desc* desc, double rope_theta, int32_t interleaved, void* q,
                         void* k_tree, const int32_t* parent_idx, const int32_t* prefix_len,
                         int32_t* positions, void* workspace, size_t workspace_bytes,
                         void* stream) {
  Geometry G;
  hta_plan_info p;
  HTA_TRY(make_plan(desc, &G, &p));
  if (!(rope_theta > 0.0) || isinf(rope_theta)) return HTA_ERR_SHAPE;
  HTA_TRY(check_ptrs({q, k_tree, parent_idx, prefix_len}));
  if (positions && !aligned16(positions)) return HTA_ERR_ALIGN;
  // only the status words are written: any buffer past them will do
  if (!workspace || workspace_bytes < p.masks_offset) return HTA_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return HTA_ERR_ALIGN;
  const Workspace ws = carve(workspace, p);
  return hip_status(hta::launch_rope_tree(G, rope_theta, interleaved != 0, q, k_tree, parent_idx,
                                          prefix_len, positions, ws.status,
                                          (hipStream_t)stream));
}

hta_status hta_chunk_mass(const hta_desc* desc, const int32_t* prefix_len, const float* lse,
                          float* mass, float* chunk_scores, void* workspace,
                          size_t workspace_bytes, void* stream) {
  Geometry G;
  hta_plan_info p;
  HTA_TRY(make_plan(desc, &G, &p));
  HTA_TRY(check_ptrs({prefix_len, lse, mass}));
  if (chunk_scores && !aligned16(chunk_scores)) return HTA_ERR_ALIGN;
  if ((size_t)G.B > 65535) return HTA_ERR_SHAPE;
  HTA_TRY(check_ws(p, workspace, workspace_bytes));
  const Workspace ws = carve(workspace, p);
  return hip_status(hta::launch_chunk_mass(G, prefix_len, lse, mass, chunk_scores, ws,
                                           (hipStream_t)stream));
}

hta_status hta_cross_attention(const hta_desc* desc, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* cache_len, float* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               void* stream) {
  Geometry G;
  hta_plan_info p;
  HTA_TRY(make_plan(desc, &G, &p));
  HTA_TRY(check_ptrs({q, cache_len, out, lse}));
  if (G.Lmax > 0) HTA_TRY(check_ptrs({k_cache, v_cache}));
  HTA_TRY(check_ws(p, workspace, workspace_bytes));
  Workspace ws = carve(workspace, p);
  ws.status_reset = ws.status;  // the merge ORs non-finite rows into cleared words
  hipStream_t s = (hipStream_t)stream;
  // the prefix pass, then the merge of the prefix partials alone (no tree part)
  HTA_TRY(hip_status(launch_prefix(G, q, k_cache, v_cache, cache_len, ws, s)));
  return hip_status(hta::launch_lse_merge(G, cache_len, false, out, lse, ws, s));
}

hta_status hta_window_commit(const hta_desc* desc, int32_t window, void* k_win, void* v_win,
                             const void* k_tree, const void* v_tree, const int32_t* accepted,
                             const int32_t* accept_len, int32_t* win_pos, void* workspace,
                             size_t workspace_bytes, void* stream) {
  Geometry G;
  hta_plan_info p;
  HTA_TRY(make_plan(desc, &G, &p));
  if (window < 1) return HTA_ERR_SHAPE;
  HTA_TRY(check_ptrs({k_win, v_win, k_tree, v_tree, accepted, accept_len, win_pos}));
  if (!workspace || workspace_bytes < p.masks_offset) return HTA_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return HTA_ERR_ALIGN;
  const Workspace ws = carve(workspace, p);
  return hip_status(hta::launch_window_commit(G, window, k_win, v_win, k_tree, v_tree, accepted,
                                              accept_len, win_pos, ws.status,
                                              (hipStream_t)stream));
}

size_t hta_dense_mask_bytes(const hta_desc* desc) {
  Geometry G;
  if (make_plan(desc, &G, nullptr) != HTA_OK) return 0;
  int32_t wp, wm, t_pad;
  hta::dense_mask_words(G, &wp, &wm, &t_pad);
  return sizeof(uint64_t) * (size_t)G.B * wm * t_pad;
}

hta_status hta_dense_mask(const hta_desc* desc, const int32_t* parent_idx,
                          const int32_t* prefix_len, uint64_t* mask, void* workspace,
                          size_t workspace_bytes, void* stream) {
  Geometry G;
  hta_plan_info p;
  HTA_TRY(make_plan(desc, &G, &p));
  HTA_TRY(check_ptrs({parent_idx, prefix_len, mask}));
  if ((size_t)G.B > 65535) return HTA_ERR_SHAPE;
  if (!workspace || workspace_bytes < p.masks_offset) return HTA_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return HTA_ERR_ALIGN;
  const Workspace ws = carve(workspace, p);
  return hip_status(hta::launch_dense_mask(G, parent_idx, prefix_len, mask, ws.status,
                                           (hipStream_t)stream));
}

hta_status hta_verify_dense(const hta_desc* desc, const void* q, const void* k_prefix,
                            const void* v_prefix, const void* k_tree, const void* v_tree,
                            const uint64_t* mask, const int32_t* prefix_len, float* out,
                            float* lse, void* stream) {
  Geometry G;
  HTA_TRY(make_plan(desc, &G, nullptr));
  if (G.f32) return HTA_ERR_DTYPE;
  HTA_TRY(check_ptrs({q, k_tree, v_tree, mask, prefix_len, out, lse}));
  if (G.Lmax > 0) HTA_TRY(check_ptrs({k_prefix, v_prefix}));
  if ((size_t)G.B > 65535 || (size_t)G.Hkv > 65535) return HTA_ERR_SHAPE;
  return hip_status(hta::launch_dense_masked(G, q, k_prefix, v_prefix, k_tree, v_tree, mask,
                                             prefix_len, out, lse, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// The accept workspace: the verify workspace, then the argmax span keys.
hta_status accept_plan(const hta_desc* desc, int32_t vocab, int32_t logits_dtype, Geometry* g,
                       hta_plan_info* p, size_t* keys_offset, size_t* total) {
  HTA_TRY(make_plan(desc, g, p));
  if (logits_dtype != HTA_BF16 && logits_dtype != HTA_F32) return HTA_ERR_DTYPE;
  if (vocab < 1) return HTA_ERR_SHAPE;
  int32_t span, nsplit;
  hta::argmax_plan(vocab, logits_dtype == HTA_F32, &span, &nsplit);
  *keys_offset = p->workspace_bytes;
  *total = round_up(*keys_offset + sizeof(uint64_t) * (size_t)g->B * g->T * nsplit, 256);
  return HTA_OK;
}

}  // namespace

extern "C" {

size_t hta_accept_workspace_size(const hta_desc* desc, int32_t vocab) {
  // sized for either logits dtype (fp32 logits take more, shorter spans per row)
  Geometry G;
  hta_plan_info p;
  size_t off, total;
  if (accept_plan(desc, vocab, HTA_BF16, &G, &p, &off, &total) != HTA_OK) return 0;
  size_t off32, total32;
  if (accept_plan(desc, vocab, HTA_F32, &G, &p, &off32, &total32) != HTA_OK) return 0;
  return total > total32 ? total : total32;
}

hta_status hta_accept_commit(const hta_desc* desc, int32_t vocab, int32_t logits_dtype,
                             const void* logits, const int32_t* tokens,
                             const int32_t* root_token, const int32_t* parent_idx,
                             int32_t* prefix_len, void* k_prefix, void* v_prefix,
                             const void* k_tree, const void* v_tree, int32_t* target_next,
                             int32_t* accept_len, int32_t* accepted, int32_t* bonus_token,
                             void* workspace, size_t workspace_bytes, void* stream) {
  Geometry G;
  hta_plan_info p;
  size_t keys_offset, total;
  HTA_TRY(accept_plan(desc, vocab, logits_dtype, &G, &p, &keys_offset, &total));
  if (!logits) return HTA_ERR_NULL;
  HTA_TRY(check_ptrs({tokens, root_token, parent_idx, prefix_len, k_tree, v_tree, target_next,
                      accept_len, accepted, bonus_token}));
  if (G.Lmax > 0) HTA_TRY(check_ptrs({k_prefix, v_prefix}));
  if (!workspace || workspace_bytes < total) return HTA_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return HTA_ERR_ALIGN;
  const Workspace ws = carve(workspace, p);
  uint64_t* keys = (uint64_t*)((char*)workspace + keys_offset);
  return hip_status(hta::launch_accept_commit(
      G, vocab, logits_dtype == HTA_F32, logits, tokens, root_token, parent_idx, prefix_len,
      k_prefix, v_prefix, k_tree, v_tree, target_next, accept_len, accepted, bonus_token,
      ws.status, keys, (hipStream_t)stream));
}

hta_status hta_get_device_status(const hta_desc* desc, const void* workspace, void* stream,
                                 int32_t* bad_sequence) {
  Geometry G;
  hta_plan_info p;
  HTA_TRY(make_plan(desc, &G, &p));
  if (bad_sequence) *bad_sequence = -1;
  if (!workspace) return HTA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  int32_t host_status[1024];
  hta_status first_tree = HTA_OK, first_len = HTA_OK, first_full = HTA_OK;
  hta_status first_nonfinite = HTA_OK;
  int32_t bad_tree = -1, bad_len = -1, bad_full = -1, bad_nonfinite = -1;
  for (int b0 = 0; b0 < G.B; b0 += 1024) {
    const int n = G.B - b0 < 1024 ? G.B - b0 : 1024;
    const char* src = (const char*)workspace + p.status_offset + sizeof(int32_t) * (size_t)b0;
    if (hipMemcpyAsync(host_status, src, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return HTA_ERR_HIP;
    for (int k = 0; k < n; ++k) {
      if ((host_status[k] & hta::kStatusTree) && first_tree == HTA_OK) {
        first_tree = HTA_ERR_TREE;
        bad_tree = b0 + k;
      }
      if ((host_status[k] & hta::kStatusPrefixLen) && first_len == HTA_OK) {
        first_len = HTA_ERR_PREFIX_LEN;
        bad_len = b0 + k;
      }
      if ((host_status[k] & hta::kStatusCacheFull) && first_full == HTA_OK) {
        first_full = HTA_ERR_CACHE_FULL;
        bad_full = b0 + k;
      }
      if ((host_status[k] & hta::kStatusNonFinite) && first_nonfinite == HTA_OK) {
        first_nonfinite = HTA_ERR_NONFINITE;
        bad_nonfinite = b0 + k;
      }
    }
  }
  if (first_tree != HTA_OK) {
    if (bad_sequence) *bad_sequence = bad_tree;
    return first_tree;
  }
  if (first_len != HTA_OK) {
    if (bad_sequence) *bad_sequence = bad_len;
    return first_len;
  }
  if (first_full != HTA_OK) {
    if (bad_sequence) *bad_sequence = bad_full;
    return first_full;
  }
  if (first_nonfinite != HTA_OK) {
    if (bad_sequence) *bad_sequence = bad_nonfinite;
    return first_nonfinite;
  }
  return HTA_OK;
}

const char* hta_status_str(hta_status status) {
  switch (status) {
    case HTA_OK: return "HTA_OK";
    case HTA_ERR_NULL: return "HTA_ERR_NULL: a required pointer is NULL";
    case HTA_ERR_SHAPE: return "HTA_ERR_SHAPE: unsupported or inconsistent sizes";
    case HTA_ERR_DTYPE: return "HTA_ERR_DTYPE: unsupported input dtype";
    case HTA_ERR_ALIGN: return "HTA_ERR_ALIGN: pointer not 16-byte aligned (workspace: 256)";
    case HTA_ERR_WORKSPACE: return "HTA_ERR_WORKSPACE: workspace missing or too small";
    case HTA_ERR_TREE: return "HTA_ERR_TREE: a parent pointer lies outside [-1, i-1]";
    case HTA_ERR_PREFIX_LEN: return "HTA_ERR_PREFIX_LEN: prefix_len outside [0, max_prefix_len]";
    case HTA_ERR_HIP: return "HTA_ERR_HIP: a HIP runtime call failed";
    case HTA_ERR_CACHE_FULL:
      return "HTA_ERR_CACHE_FULL: the accepted path does not fit the prefix cache";
    case HTA_ERR_SCRATCH:
      return "HTA_ERR_SCRATCH: hta_verify_noalloc needs more scratch than its static 64 MiB "
             "(hta_workspace_size() of the descriptor is larger); use hta_verify";
    case HTA_ERR_NONFINITE:
      return "HTA_ERR_NONFINITE: an output row came out non-finite (an input outside the "
             "supported range, e.g. |v| > 65504 with bf16 inputs); the row was written as NaN";
    case HTA_STATUS_MAX_ENUM: break;
  }
  return "HTA_ERR_UNKNOWN";
}

int32_t hta_version(void) { return 200; }

}  // extern "C"
