// hta_internal.h -- shared declarations of the gfx950 kernels and their host launchers.
//
// Everything here is private to libhta.so; the public C ABI is include/hta.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hta {

// Operand types of the CDNA4 bf16 matrix-core instructions.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Device status codes, one int32 per sequence in the workspace.
constexpr int32_t kStatusTree = 1;       // a parent pointer outside [-1, i-1]
constexpr int32_t kStatusPrefixLen = 2;  // prefix_len[b] outside [0, Lmax]
constexpr int32_t kStatusCacheFull = 4;  // the accepted path does not fit the prefix cache
constexpr int32_t kStatusNonFinite = 8;  // an output row came out non-finite (e.g. a bf16 V
                                         // value outside the fp16 range of the PV product)

// Geometry shared by every kernel of one call (a plain struct passed by value).
struct Geometry {
  int32_t B, T, Hq, Hkv, D, Lmax;
  int32_t G;            // Hq / Hkv: query heads per KV head
  int32_t R;            // T * G query rows per (b, kv head)
  int32_t R_pad;        // R rounded up to 16
  int32_t NT;           // R_pad / 16 row tiles
  int32_t W;            // ceil(T / 64) mask words per node
  int32_t chunk;        // prefix keys per split
  int32_t S;            // number of prefix splits (the tree partial is slot S)
  float scale;          // softmax scale
  int32_t f32;          // 1: q, k_*, v_* are fp32 (else bf16)
};

struct Workspace {
  int32_t* status;      // [B]
  uint64_t* masks;      // [B, T, W]
  float* lse_part;      // [B, Hkv, S+1, R_pad]
  float* o_scale;       // [B, Hkv, S+1, R_pad]: the factor of each o_part row
  uint32_t* o_part;     // [B, Hkv, S+1, R_pad, D] 16-bit fixed point: D / 2 dwords a row
  // When set (== status), the prefix pass clears the status words first: a call whose later
  // launch records bits with atomic ORs starts from zero.  nullptr leaves them alone.
  int32_t* status_reset;
};

// Split-K partial output rows travel through memory as 16-bit fixed point with one fp32
// factor per row: value d of a row is q_d * f, where f = m / 32767 for the row's largest
// magnitude m (or a bound on it, at most the largest |v| the row attends to) and q_d is
// x_d / f rounded to the nearest integer (ties to even), |q_d| <= 32767.  A value's error is
// at most f / 2 = 2^-16 m (plus fp32 rounding): since a partial row is a convex combination
// of V rows, the merged output's error from this storage is at most 2^-16 max |v|.  The
// partial traffic -- written by the prefix pass, read by the merge -- is half of fp32.  An
// all-zero row has f = 0; a row holding a non-finite value gets f = NaN, so the merge's
// result is non-finite.  Two values per dword: value 2j in the low half of word j.
struct RowCode {
  float f;    // the stored factor
  float enc;  // 1 / f (0 for an all-zero row)
};
// amax: max |x| over the row (or the bound m); sum: the sum of the row's values (non-finite
// iff one of them is)
__device__ __forceinline__ RowCode row_code(float amax, float sum) {
  RowCode c;
  const bool finite = __builtin_isfinite(sum);
  c.f = finite ? amax * (1.f / 32767.f) : __builtin_nanf("");
  c.enc = (finite && amax > 0.f) ? 32767.f / amax : 0.f;
  return c;
}
__device__ __forceinline__ uint32_t pack16(float x0, float x1, float enc) {
  const int q0 = (int)__builtin_rintf(x0 * enc), q1 = (int)__builtin_rintf(x1 * enc);
  return ((uint32_t)q0 & 0xFFFFu) | ((uint32_t)q1 << 16);
}
// four values (one f32x4) -> two dwords
__device__ __forceinline__ uint2 pack16x4(f32x4 v, float enc) {
  return make_uint2(pack16(v[0], v[1], enc), pack16(v[2], v[3], enc));
}
__device__ __forceinline__ float lo16(uint32_t w) { return (float)(int)(short)(w & 0xFFFFu); }
__device__ __forceinline__ float hi16(uint32_t w) { return (float)((int)w >> 16); }

// Host launchers (each enqueues exactly one kernel on the stream).
hipError_t launch_prefix_attn_splitk(const Geometry& g, const void* q, const void* k_prefix,
                                     const void* v_prefix, const int32_t* prefix_len,
                                     const Workspace& ws, hipStream_t stream);
hipError_t launch_tree_attn_masked(const Geometry& g, const void* q, const void* k_tree,
                                   const void* v_tree, const int32_t* parent_idx,
                                   const int32_t* prefix_len, const Workspace& ws,
                                   uint64_t* masks_out, bool attention, hipStream_t stream);
hipError_t launch_lse_merge(const Geometry& g, const int32_t* prefix_len, bool include_tree,
                            float* out, float* lse, const Workspace& ws, hipStream_t stream);
// The merge with the tree part computed in the same kernel (validates the trees and writes
// the device status): the second half of the whole step after the prefix pass.
hipError_t launch_tree_merge(const Geometry& g, const void* q, const void* k_tree,
                             const void* v_tree, const int32_t* parent_idx,
                             const int32_t* prefix_len, float* out, float* lse,
                             const Workspace& ws, hipStream_t stream);

// The tree partial (slot S) computed from the parent chains, row by row (any input dtype);
// status and masks are left to tree_attn_masked.
hipError_t launch_tree_chain(const Geometry& g, const void* q, const void* k_tree,
                             const void* v_tree, const int32_t* parent_idx,
                             const int32_t* prefix_len, const Workspace& ws, hipStream_t stream);
// The prefix pass for fp32 inputs (VALU, exact fp32 arithmetic; for small validation shapes).
hipError_t launch_prefix_attn_f32(const Geometry& g, const void* q, const void* k_prefix,
                                  const void* v_prefix, const int32_t* prefix_len,
                                  const Workspace& ws, hipStream_t stream);

// Rotary encoding of the tree's q and k_tree rows in place at positions prefix_len + depth.
hipError_t launch_rope_tree(const Geometry& g, double theta, bool interleaved, void* q,
                            void* k_tree, const int32_t* parent_idx, const int32_t* prefix_len,
                            int32_t* positions, int32_t* status, hipStream_t stream);
// Span of logits each argmax workgroup scans, and the number of spans per row.
void argmax_plan(int32_t vocab, bool f32, int32_t* span, int32_t* nsplit);
// The target's greedy tokens (span keys in keys[B*T, nsplit]), greedy acceptance, KV commit:
// two launches.
hipError_t launch_accept_commit(const Geometry& g, int32_t vocab, bool logits_f32,
                                const void* logits, const int32_t* tokens,
                                const int32_t* root_token, const int32_t* parent_idx,
                                int32_t* prefix_len, void* k_prefix, void* v_prefix,
                                const void* k_tree, const void* v_tree, int32_t* target_next,
                                int32_t* accept_len, int32_t* accepted, int32_t* bonus,
                                int32_t* status, uint64_t* keys, hipStream_t stream);

// The drafter's window ring: the accepted path's rows appended at slots (pos + k) % window.
hipError_t launch_window_commit(const Geometry& g, int32_t window, void* k_win, void* v_win,
                                const void* k_tree, const void* v_tree, const int32_t* accepted,
                                const int32_t* accept_len, int32_t* win_pos, int32_t* status,
                                hipStream_t stream);

// Each chunk's (and the tree's) share of every query row's attention from the partial
// log-sum-exps in the workspace and the rows' final log-sum-exps; optional per-sequence means.
hipError_t launch_chunk_mass(const Geometry& g, const int32_t* prefix_len, const float* lse,
                             float* mass, float* scores, const Workspace& ws,
                             hipStream_t stream);

// The single-pass masked attention over all L + T keys (the method's "before"): explicit
// mask uint64 [B, Wm, T_pad] (word-major) with Wp prefix words then ceil(T / 64) tree words
// per node, T_pad = T rounded up to even.
void dense_mask_words(const Geometry& g, int32_t* wp, int32_t* wm, int32_t* t_pad);
hipError_t launch_dense_mask(const Geometry& g, const int32_t* parent_idx,
                             const int32_t* prefix_len, uint64_t* mask, int32_t* status,
                             hipStream_t stream);
hipError_t launch_dense_masked(const Geometry& g, const void* q, const void* k_prefix,
                               const void* v_prefix, const void* k_tree, const void* v_tree,
                               const uint64_t* mask, const int32_t* prefix_len, float* out,
                               float* lse, hipStream_t stream);

// How the prefix pass blocks the query rows of one KV head: tiles_per_block row tiles per
// workgroup, blocks workgroups per (sequence, KV head, chunk).
void prefix_row_blocking(const Geometry& g, int* tiles_per_block, int* blocks);

}  // namespace hta
