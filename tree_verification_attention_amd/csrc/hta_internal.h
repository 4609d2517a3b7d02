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
  uint32_t* o_part;     // [B, Hkv, S+1, R_pad, D] packed 24-bit values: 3 D / 4 dwords a row
  // When set (== status), the prefix pass clears the status words first: a call whose later
  // launch records bits with atomic ORs starts from zero.  nullptr leaves them alone.
  int32_t* status_reset;
};

// Split-K partial outputs travel through memory as packed 24-bit floats: the top 24 bits of
// the fp32 value (sign, 8-bit exponent, 15 mantissa bits), rounded to nearest even, four
// values in three dwords.  The relative error is at most 2^-16 (normalised partials are
// bounded by max |v|), and the partial traffic -- written by the prefix pass, read by the
// merge -- is three quarters of fp32.
struct Packed24 {
  uint32_t w[3];
};
__device__ __forceinline__ uint32_t round24(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7Fu + ((u >> 8) & 1u)) & 0xFFFFFF00u;
}
__device__ __forceinline__ Packed24 pack24(f32x4 v) {
  const uint32_t r0 = round24(v[0]), r1 = round24(v[1]), r2 = round24(v[2]), r3 = round24(v[3]);
  Packed24 p;
  p.w[0] = (r0 >> 8) | (r1 << 16);
  p.w[1] = (r1 >> 16) | (r2 << 8);
  p.w[2] = (r2 >> 24) | r3;
  return p;
}
__device__ __forceinline__ f32x4 unpack24(Packed24 p) {
  f32x4 v;
  v[0] = __uint_as_float(p.w[0] << 8);
  v[1] = __uint_as_float(((p.w[0] >> 16) | (p.w[1] << 16)) & 0xFFFFFF00u);
  v[2] = __uint_as_float(((p.w[1] >> 8) | (p.w[2] << 24)) & 0xFFFFFF00u);
  v[3] = __uint_as_float(p.w[2] & 0xFFFFFF00u);
  return v;
}
// Store / load group g (values 4 g .. 4 g + 3) of a packed row.
__device__ __forceinline__ void store24(uint32_t* row, int g, f32x4 v) {
  const Packed24 p = pack24(v);
  uint32_t* d = row + 3 * g;
  d[0] = p.w[0];
  d[1] = p.w[1];
  d[2] = p.w[2];
}
__device__ __forceinline__ f32x4 load24(const uint32_t* row, int g) {
  const uint32_t* s = row + 3 * g;
  Packed24 p;
  p.w[0] = s[0];
  p.w[1] = s[1];
  p.w[2] = s[2];
  return unpack24(p);
}

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
