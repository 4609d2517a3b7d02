// tree_step.hip -- the steps on either side of the verification attention in one greedy
// tree-speculation step (temperature 0 and the 4,16,16,16,16 draft tree of the LongSpec
// README, Evaluation):
//
//   rope_tree       rotary encoding (RoFormer) of the tree's queries and keys, in place, at
//                   positions prefix_len + depth.  One workgroup per (node, sequence):
//                   the sequence's parent pointers are validated and walked in LDS, the
//                   node's cos/sin table is built in fp64 (exact angles for positions far
//                   past 2^16), then every head vector of the node is turned in fp64 and
//                   rounded once.  Launch-bound: 1.4 MB moved for the Llama-3-8B tree.
//   tree_argmax     the target's greedy token after every node: each workgroup scans one
//                   16 KB span of one logits row with 16-byte loads (four in flight per
//                   lane) and leaves one 64-bit key (ordered value, inverted index) per span.
//                   Bound by HBM: the logits are read once.
//   accept_commit   one workgroup per sequence: reduces the span keys to target_next,
//                   marks for every node whether its token is the one expected after its
//                   parent, finds each node's first matching child with LDS atomics, walks
//                   the accepted path, writes the acceptance outputs, then copies the path's
//                   tree keys and values into the prefix cache and advances prefix_len.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hta_internal.h"

namespace hta {
namespace {

constexpr int kThreads = 256;

// ----------------------------------------------------------------------------- rotary

// Nearest-even rounding of a double to bf16 in one step: the significand is cut to bf16's
// eight bits directly (no intermediate float rounding); the result is then exactly a float.
__device__ __forceinline__ uint16_t bf16_from_double(double x) {
  if (x != x) return 0x7FC0;
  unsigned long long u = (unsigned long long)__double_as_longlong(x);
  constexpr int kDrop = 45;  // 52 stored significand bits of a double, 7 of a bf16
  u += ((1ull << (kDrop - 1)) - 1) + ((u >> kDrop) & 1ull);
  u &= ~((1ull << kDrop) - 1);
  const float f = (float)__longlong_as_double((long long)u);  // exact (or +-inf)
  return (uint16_t)(__float_as_uint(f) >> 16);
}

template <typename E>
__device__ __forceinline__ double widen(E x);
template <>
__device__ __forceinline__ double widen<uint16_t>(uint16_t x) {
  return (double)__uint_as_float((uint32_t)x << 16);
}
template <>
__device__ __forceinline__ double widen<float>(float x) {
  return (double)x;
}

template <typename E>
__device__ __forceinline__ E narrow(double x);
template <>
__device__ __forceinline__ uint16_t narrow<uint16_t>(double x) {
  return bf16_from_double(x);
}
template <>
__device__ __forceinline__ float narrow<float>(double x) {
  return (float)x;  // round to nearest even
}

template <typename E>
__device__ __forceinline__ E nan_of();
template <>
__device__ __forceinline__ uint16_t nan_of<uint16_t>() {
  return 0x7FC0;
}
template <>
__device__ __forceinline__ float nan_of<float>() {
  return __uint_as_float(0x7FC00000u);
}

// Four rotation pairs of one head vector: elements a[0..3] pair with c[0..3] (frequency
// indices j0..j0+3).  Half layout: a = row + j0, c = row + j0 + D/2 (two 4-element runs);
// interleaved: the 8-element run row + 2 j0 holds a0 c0 a1 c1 ...  x[0..3] are the a's and
// x[4..7] the c's in both layouts.
template <typename E, bool kInterleaved>
struct Quad {
  E* pa;
  E* pc;
  __device__ __forceinline__ Quad(E* row, int j0, int half)
      : pa(kInterleaved ? row + 2 * j0 : row + j0),
        pc(kInterleaved ? row + 2 * j0 + 1 : row + j0 + half) {}
  __device__ __forceinline__ void load(E (&x)[8]) const {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = kInterleaved ? pa[2 * k] : pa[k];
      x[4 + k] = kInterleaved ? pc[2 * k] : pc[k];
    }
  }
  __device__ __forceinline__ void store(const E (&y)[8]) const {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      (kInterleaved ? pa[2 * k] : pa[k]) = y[k];
      (kInterleaved ? pc[2 * k] : pc[k]) = y[4 + k];
    }
  }
};

struct RopeArgs {
  void* q;
  void* k_tree;
  const int32_t* parent;
  const int32_t* prefix_len;
  int32_t* positions;
  int32_t* status;
  double theta;
  int32_t B, T, Hq, Hkv, D, Lmax;
};

// grid (T, B, ceil(units / kThreads)): a unit is four rotation pairs of one head vector of
// the node (q heads first, then k_tree heads); each lane loads its unit before anything else.
template <typename E, bool kInterleaved>
__global__ __launch_bounds__(kThreads) void rope_tree(RopeArgs a) {
  __shared__ int32_t par[256];
  __shared__ double cs[64], sn[64];
  const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int T = a.T, D = a.D, half = D / 2;
  const int units_per_head = half / 4;
  const int nq = a.Hq * units_per_head, nk = a.Hkv * units_per_head;
  const int u = blockIdx.z * kThreads + tid;
  const bool active = u < nq + nk;
  E* row;
  int unit;
  if (u < nq) {
    row = (E*)a.q + (((size_t)b * T + i) * a.Hq + u / units_per_head) * D;
    unit = u % units_per_head;
  } else {
    const int v = active ? u - nq : 0;
    row = (E*)a.k_tree + (((size_t)b * a.Hkv + v / units_per_head) * T + i) * D;
    unit = v % units_per_head;
  }
  const Quad<E, kInterleaved> quad(row, 4 * unit, half);
  E x[8];
  if (active) quad.load(x);
  int bad = 0;
  if (tid < T) {
    const int p = a.parent[(size_t)b * T + tid];
    par[tid] = p;
    bad = p < -1 || p >= tid;
  }
  const int L = a.prefix_len[b];
  // the pair's frequency does not depend on the position: computed while the loads fly
  const double freq = tid < half ? pow(a.theta, -2.0 * (double)tid / (double)D) : 0.0;
  const bool bad_len = L < 0 || L > a.Lmax;
  const bool bad_tree = __syncthreads_or(bad) != 0;
  const bool fail = bad_tree || bad_len;
  int depth = 0;
  if (!bad_tree)  // parents strictly decrease along a valid chain: the walk ends
    for (int p = par[i]; p >= 0; p = par[p]) ++depth;
  const long long pos = (long long)L + depth;
  if (tid == 0 && blockIdx.z == 0) {
    if (i == 0) a.status[b] = (bad_tree ? kStatusTree : 0) | (bad_len ? kStatusPrefixLen : 0);
    if (a.positions) a.positions[(size_t)b * T + i] = fail ? -1 : (int32_t)pos;
  }
  if (tid < half) {
    double s, c;
    sincos((double)pos * freq, &s, &c);
    cs[tid] = c;
    sn[tid] = s;
  }
  __syncthreads();
  if (!active) return;
  const int j0 = 4 * unit;
  E y[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double xa = widen<E>(x[k]), xc = widen<E>(x[4 + k]);
    const double c = cs[j0 + k], s = sn[j0 + k];
    y[k] = fail ? nan_of<E>() : narrow<E>(xa * c - xc * s);
    y[4 + k] = fail ? nan_of<E>() : narrow<E>(xc * c + xa * s);
  }
  quad.store(y);
}

// ----------------------------------------------------------------------------- argmax

// Order-preserving 32-bit key of a float: larger value, larger key; +0 and -0 share one
// key and every NaN gets the largest key.
__device__ __forceinline__ uint32_t order_key(float v) {
  if (v != v) return 0xFFFFFFFFu;
  if (v == 0.f) return 0x80000000u;
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// 64-bit key: the value's key above the inverted index, so a larger key means a larger
// value or, between equal values, a smaller index.
__device__ __forceinline__ uint64_t pack_key(float v, uint32_t idx) {
  return ((uint64_t)order_key(v) << 32) | (uint64_t)(~idx);
}

// The running best of one lane, elements visited in increasing index order: replace on a
// strictly larger value, or on the first NaN.
struct Best {
  float v;
  uint32_t i;
  bool any;
};
__device__ __forceinline__ void consider(Best& bst, float v, uint32_t idx) {
  const bool take = !bst.any || v > bst.v || (v != v && bst.v == bst.v);
  bst.v = take ? v : bst.v;
  bst.i = take ? idx : bst.i;
  bst.any = true;
}

struct ArgmaxArgs {
  const void* logits;
  uint64_t* keys;  // [rows, nsplit]
  int32_t V, span, nsplit;
};

template <typename E, int kVec>
__device__ __forceinline__ void load_vec(const E* p, float (&v)[kVec]);

template <>
__device__ __forceinline__ void load_vec<uint16_t, 8>(const uint16_t* p, float (&v)[8]) {
  const uint4 w = *(const uint4*)p;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = __uint_as_float(ws[k] << 16);
    v[2 * k + 1] = __uint_as_float(ws[k] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void load_vec<float, 4>(const float* p, float (&v)[4]) {
  const float4 w = *(const float4*)p;
  v[0] = w.x;
  v[1] = w.y;
  v[2] = w.z;
  v[3] = w.w;
}
template <>
__device__ __forceinline__ void load_vec<uint16_t, 1>(const uint16_t* p, float (&v)[1]) {
  v[0] = __uint_as_float((uint32_t)*p << 16);
}
template <>
__device__ __forceinline__ void load_vec<float, 1>(const float* p, float (&v)[1]) {
  v[0] = *p;
}

// The workgroup maximum of one 64-bit key per lane, written by lane 0 of wave 0.
__device__ __forceinline__ void store_block_max_key(uint64_t key, uint64_t* dst) {
  __shared__ uint64_t wave_key[kThreads / 64];
  const int tid = threadIdx.x;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(key, off);
    key = o > key ? o : key;
  }
  if ((tid & 63) == 0) wave_key[tid >> 6] = key;
  __syncthreads();
  if (tid == 0) {
    uint64_t k = wave_key[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) k = wave_key[w] > k ? wave_key[w] : k;
    *dst = k;
  }
}

__device__ __forceinline__ float maximum(float x, float y) {
  return __builtin_elementwise_maximum(x, y);  // NaN-propagating; -0 < +0
}

// Wave-wide reduction through DPP: row shifts by 1, 2, 4, 8 leave each 16-lane row's result
// in its lane 15; row broadcasts 15 and 31 fold the rows into lane 63, read back as a scalar.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, uint32_t identity, Op op) {
  const int id = (int)identity;
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x111, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x112, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x114, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x118, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xA, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ float wave_maximum(float v) {
  return __uint_as_float(wave_reduce(__float_as_uint(v), 0xFF800000u, [](uint32_t x, uint32_t y) {
    return __float_as_uint(maximum(__uint_as_float(x), __uint_as_float(y)));
  }));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce(v, 0xFFFFFFFFu, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
}

// One workgroup: one span [s0, s1) of one row.  Lane l holds the kVec-element vectors
// s0 + (k * kThreads + l) * kVec, k < kInFlight, all loaded before any is used (the host
// sizes the span to exactly one such sweep: kThreads * kInFlight * kVec elements).
// Pass 1 takes the NaN-propagating maximum of the lane's values (three per instruction)
// and of the workgroup.  If it is a number M, only lanes whose own maximum equals M look
// for their first element equal to M (+0 equals -0 there), and the smallest such index
// wins; a NaN anywhere sends the workgroup through the exact element-by-element scan.
template <typename E, int kVec>
__global__ __launch_bounds__(kThreads) void tree_argmax(ArgmaxArgs a) {
  constexpr int kInFlight = 4;
  constexpr int kPer = kInFlight * kVec;
  const int row = blockIdx.x, split = blockIdx.y, tid = threadIdx.x;
  const int s0 = split * a.span;
  const int s1 = min(s0 + a.span, a.V);
  const E* base = (const E*)a.logits + (size_t)row * a.V;
  uint64_t* dst = a.keys + (size_t)row * a.nsplit + split;
  auto elem = [&](int j) { return s0 + ((j / kVec) * kThreads + tid) * kVec + j % kVec; };
  float v[kPer];
  if (s1 - s0 == kThreads * kPer) {
#pragma unroll
    for (int k = 0; k < kInFlight; ++k)
      load_vec<E, kVec>(base + s0 + (k * kThreads + tid) * kVec, *(float(*)[kVec])&v[k * kVec]);
  } else {  // the row's last span: vectors past its end read as -inf
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      const int e = s0 + (k * kThreads + tid) * kVec;
      if (e < s1) {
        load_vec<E, kVec>(base + e, *(float(*)[kVec])&v[k * kVec]);
      } else {
#pragma unroll
        for (int m = 0; m < kVec; ++m) v[k * kVec + m] = -__builtin_inff();
      }
    }
  }
  float lane_max = v[0];
#pragma unroll
  for (int j = 1; j < kPer; ++j) lane_max = maximum(lane_max, v[j]);
  const float m = wave_maximum(lane_max);
  __shared__ float wave_max[kThreads / 64];
  if ((tid & 63) == 0) wave_max[tid >> 6] = m;
  __syncthreads();
  float M = wave_max[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) M = maximum(M, wave_max[w]);
  if (M != M) {  // a NaN in the span (uniform branch): exact scan in index order
    Best bst{0.f, 0u, false};
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (elem(j) < s1) consider(bst, v[j], (uint32_t)elem(j));
    store_block_max_key(bst.any ? pack_key(bst.v, bst.i) : 0ull, dst);
    return;
  }
  uint32_t idx = 0xFFFFFFFFu;
  if (lane_max == M) {
#pragma unroll
    for (int j = kPer - 1; j >= 0; --j) idx = (v[j] == M && elem(j) < s1) ? (uint32_t)elem(j) : idx;
  }
  // only a wave holding the maximum has a candidate (wave-uniform test)
  if (__ballot(idx != 0xFFFFFFFFu) != 0) idx = wave_min_u32(idx);
  __shared__ uint32_t wave_idx[kThreads / 64];
  if ((tid & 63) == 0) wave_idx[tid >> 6] = idx;
  __syncthreads();
  if (tid == 0) {
    uint32_t i = wave_idx[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) i = min(i, wave_idx[w]);
    *dst = pack_key(M, i);
  }
}

// Rows whose byte length is not a multiple of 16 (or an unaligned logits pointer): one
// element per lane per step, element-by-element scan.
template <typename E>
__global__ __launch_bounds__(kThreads) void tree_argmax_scalar(ArgmaxArgs a) {
  const int row = blockIdx.x, split = blockIdx.y, tid = threadIdx.x;
  const int s0 = split * a.span;
  const int s1 = min(s0 + a.span, a.V);
  const E* base = (const E*)a.logits + (size_t)row * a.V;
  Best bst{0.f, 0u, false};
  for (int e = s0 + tid; e < s1; e += kThreads) {
    float v[1];
    load_vec<E, 1>(base + e, v);
    consider(bst, v[0], (uint32_t)e);
  }
  store_block_max_key(bst.any ? pack_key(bst.v, bst.i) : 0ull,
                      a.keys + (size_t)row * a.nsplit + split);
}

// ----------------------------------------------------------------------------- acceptance

struct AcceptArgs {
  const uint64_t* keys;
  const int32_t* tokens;
  const int32_t* root_token;
  const int32_t* parent;
  int32_t* prefix_len;
  void* k_prefix;
  void* v_prefix;
  const void* k_tree;
  const void* v_tree;
  int32_t* target_next;
  int32_t* accept_len;
  int32_t* accepted;
  int32_t* bonus;
  int32_t* status;
  int32_t T, Hkv, Lmax, nsplit;
  int32_t row_bytes;  // D * element size, a multiple of 16
};

__global__ __launch_bounds__(kThreads) void accept_commit(AcceptArgs a) {
  constexpr int kBatch = 4;  // independent global loads in flight per lane
  __shared__ int32_t par[256], nxt[256], path[256];
  __shared__ int32_t first[257];  // first[p + 1]: smallest matching child of node p (-1: roots)
  __shared__ unsigned long long best[256];
  __shared__ int32_t s_n, s_commit;
  const int b = blockIdx.x, tid = threadIdx.x, T = a.T;
  const size_t bt = (size_t)b * T;
  // every independent load first: parents, tokens, the sequence's scalars, the span keys
  int bad = 0;
  int32_t token = 0;
  if (tid < T) {
    const int p = a.parent[bt + tid];
    token = a.tokens[bt + tid];
    par[tid] = p;
    bad = p < -1 || p >= tid;
    best[tid] = 0;
  }
  const int32_t root = a.root_token[b];
  const int L = a.prefix_len[b];
  const int nkeys = T * a.nsplit;
  const uint64_t* keys = a.keys + bt * a.nsplit;
  uint64_t kv[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int k = tid + j * kThreads;
    kv[j] = k < nkeys ? keys[k] : 0ull;
  }
  for (int t = tid; t <= T; t += kThreads) first[t] = 0x7FFFFFFF;
  const bool bad_len = L < 0 || L > a.Lmax;
  const bool bad_tree = __syncthreads_or(bad) != 0;
  // the target's greedy token of every node: the largest span key of its row
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int k = tid + j * kThreads;
    if (k < nkeys) atomicMax(&best[k / a.nsplit], (unsigned long long)kv[j]);
  }
  for (int k0 = kBatch * kThreads; k0 < nkeys; k0 += kBatch * kThreads) {  // long trees
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int k = k0 + tid + j * kThreads;
      kv[j] = k < nkeys ? keys[k] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int k = k0 + tid + j * kThreads;
      if (k < nkeys) atomicMax(&best[k / a.nsplit], (unsigned long long)kv[j]);
    }
  }
  __syncthreads();
  if (tid < T) {
    const int32_t idx = (int32_t)(~(uint32_t)best[tid]);
    nxt[tid] = idx;
    a.target_next[bt + tid] = idx;
  }
  __syncthreads();
  if (!bad_tree && tid < T) {
    const int p = par[tid];
    const int32_t expect = p < 0 ? root : nxt[p];
    if (token == expect) atomicMin(&first[p + 1], tid);
  }
  __syncthreads();
  if (tid == 0) {
    int n = 0, bonus = -1;
    if (!bad_tree) {
      int last = -1;
      // a valid tree's children have larger indices than their parents: at most T steps
      while (n < T) {
        const int c = first[last + 1];
        if (c == 0x7FFFFFFF) break;
        path[n++] = c;
        last = c;
      }
      bonus = n ? nxt[last] : root;
    }
    const bool full = !bad_tree && !bad_len && L + n > a.Lmax;
    a.accept_len[b] = n;
    a.bonus[b] = bonus;
    a.status[b] = (bad_tree ? kStatusTree : 0) | (bad_len ? kStatusPrefixLen : 0) |
                  (full ? kStatusCacheFull : 0);
    s_n = n;
    s_commit = !bad_tree && !bad_len && !full && n > 0;
  }
  __syncthreads();
  const int n = s_n;
  for (int t = tid; t < T; t += kThreads) a.accepted[bt + t] = t < n ? path[t] : -1;
  if (!s_commit) return;
  // copy n rows per KV head of K and of V, 16 bytes per lane, kBatch loads in flight
  const int units = a.row_bytes / 16;
  const int per_tensor = n * a.Hkv * units;
  for (int u0 = 0; u0 < 2 * per_tensor; u0 += kBatch * kThreads) {
    uint4 val[kBatch];
    uint4* dst[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int u = u0 + j * kThreads + tid;
      dst[j] = nullptr;
      if (u < 2 * per_tensor) {
        const int is_v = u >= per_tensor;
        const int v = u - is_v * per_tensor;
        const int c = v % units, r = v / units;
        const int k = r % n, g = r / n;
        const char* src = (const char*)(is_v ? a.v_tree : a.k_tree) +
                          (((size_t)b * a.Hkv + g) * T + path[k]) * a.row_bytes;
        dst[j] = (uint4*)((char*)(is_v ? a.v_prefix : a.k_prefix) +
                          (((size_t)b * a.Hkv + g) * a.Lmax + L + k) * a.row_bytes) + c;
        val[j] = ((const uint4*)src)[c];
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (dst[j]) *dst[j] = val[j];
  }
  // every lane read prefix_len[b] before the first barrier: safe to advance it now
  if (tid == 0) a.prefix_len[b] = L + n;
}

// ----------------------------------------------------------------------------- drafter window

struct WindowArgs {
  void* k_win;  // [B, Hkv, W, D] ring: position p lives in slot p % W
  void* v_win;
  const void* k_tree;  // [B, Hkv, T, D]
  const void* v_tree;
  const int32_t* accepted;    // [B, T]
  const int32_t* accept_len;  // [B]
  int32_t* win_pos;           // [B] committed positions so far (in/out)
  int32_t* status;
  int32_t T, Hkv, W;
  int32_t row_bytes;
};

// One workgroup per sequence: the accepted path's rows go to ring slots (pos + k) % W; when
// the path is longer than the ring only its last W rows are written (no two lanes write one
// slot); pos advances by the path length.
__global__ __launch_bounds__(kThreads) void window_commit(WindowArgs a) {
  constexpr int kBatch = 4;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int n = a.accept_len[b];
  const int pos = a.win_pos[b];
  const bool bad = n < 0 || n > a.T || pos < 0;
  if (tid == 0) a.status[b] = bad ? kStatusPrefixLen : 0;
  if (bad) return;
  const int k0 = n > a.W ? n - a.W : 0;  // rows the ring keeps
  const int rows = n - k0;
  const int units = a.row_bytes / 16;
  const int per_tensor = rows * a.Hkv * units;
  for (int u0 = 0; u0 < 2 * per_tensor; u0 += kBatch * kThreads) {
    uint4 val[kBatch];
    uint4* dst[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int u = u0 + j * kThreads + tid;
      dst[j] = nullptr;
      if (u < 2 * per_tensor) {
        const int is_v = u >= per_tensor;
        const int v = u - is_v * per_tensor;
        const int c = v % units, r = v / units;
        const int k = k0 + r % rows, g = r / rows;
        const int node = a.accepted[(size_t)b * a.T + k];
        const int slot = (int)(((long long)pos + k) % a.W);
        const char* src = (const char*)(is_v ? a.v_tree : a.k_tree) +
                          (((size_t)b * a.Hkv + g) * a.T + node) * a.row_bytes;
        dst[j] = (uint4*)((char*)(is_v ? a.v_win : a.k_win) +
                          (((size_t)b * a.Hkv + g) * a.W + slot) * a.row_bytes) + c;
        val[j] = ((const uint4*)src)[c];
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (dst[j]) *dst[j] = val[j];
  }
  __syncthreads();  // every lane has read win_pos[b]
  if (tid == 0) a.win_pos[b] = pos + n;
}

}  // namespace

// ----------------------------------------------------------------------------- launchers

hipError_t launch_window_commit(const Geometry& g, int32_t window, void* k_win, void* v_win,
                                const void* k_tree, const void* v_tree, const int32_t* accepted,
                                const int32_t* accept_len, int32_t* win_pos, int32_t* status,
                                hipStream_t stream) {
  WindowArgs a;
  a.k_win = k_win;
  a.v_win = v_win;
  a.k_tree = k_tree;
  a.v_tree = v_tree;
  a.accepted = accepted;
  a.accept_len = accept_len;
  a.win_pos = win_pos;
  a.status = status;
  a.T = g.T;
  a.Hkv = g.Hkv;
  a.W = window;
  a.row_bytes = g.D * (g.f32 ? 4 : 2);
  hipLaunchKernelGGL(window_commit, dim3(g.B), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_rope_tree(const Geometry& g, double theta, bool interleaved, void* q,
                            void* k_tree, const int32_t* parent_idx, const int32_t* prefix_len,
                            int32_t* positions, int32_t* status, hipStream_t stream) {
  RopeArgs a;
  a.q = q;
  a.k_tree = k_tree;
  a.parent = parent_idx;
  a.prefix_len = prefix_len;
  a.positions = positions;
  a.status = status;
  a.theta = theta;
  a.B = g.B;
  a.T = g.T;
  a.Hq = g.Hq;
  a.Hkv = g.Hkv;
  a.D = g.D;
  a.Lmax = g.Lmax;
  const int units = (g.Hq + g.Hkv) * (g.D / 8);
  const dim3 grid(g.T, g.B, (units + kThreads - 1) / kThreads);
  if (g.f32) {
    if (interleaved)
      hipLaunchKernelGGL((rope_tree<float, true>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((rope_tree<float, false>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (interleaved)
      hipLaunchKernelGGL((rope_tree<uint16_t, true>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((rope_tree<uint16_t, false>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

void argmax_plan(int32_t vocab, bool f32, int32_t* span, int32_t* nsplit) {
  // 16 KB of logits per workgroup: 4 vectors of 16 bytes in flight per lane, one sweep
  // (tree_argmax relies on span == kThreads * 4 * elements per vector)
  const int32_t s = f32 ? 4096 : 8192;
  *span = s;
  *nsplit = (vocab + s - 1) / s;
}

hipError_t launch_accept_commit(const Geometry& g, int32_t vocab, bool logits_f32,
                                const void* logits, const int32_t* tokens,
                                const int32_t* root_token, const int32_t* parent_idx,
                                int32_t* prefix_len, void* k_prefix, void* v_prefix,
                                const void* k_tree, const void* v_tree, int32_t* target_next,
                                int32_t* accept_len, int32_t* accepted, int32_t* bonus,
                                int32_t* status, uint64_t* keys, hipStream_t stream) {
  ArgmaxArgs m;
  m.logits = logits;
  m.keys = keys;
  m.V = vocab;
  argmax_plan(vocab, logits_f32, &m.span, &m.nsplit);
  const size_t esz = logits_f32 ? 4 : 2;
  const bool vec = ((uintptr_t)logits & 15u) == 0 && ((size_t)vocab * esz) % 16 == 0;
  const dim3 grid(g.B * g.T, m.nsplit);
  if (logits_f32) {
    if (vec)
      hipLaunchKernelGGL((tree_argmax<float, 4>), grid, dim3(kThreads), 0, stream, m);
    else
      hipLaunchKernelGGL((tree_argmax_scalar<float>), grid, dim3(kThreads), 0, stream, m);
  } else {
    if (vec)
      hipLaunchKernelGGL((tree_argmax<uint16_t, 8>), grid, dim3(kThreads), 0, stream, m);
    else
      hipLaunchKernelGGL((tree_argmax_scalar<uint16_t>), grid, dim3(kThreads), 0, stream, m);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AcceptArgs a;
  a.keys = keys;
  a.tokens = tokens;
  a.root_token = root_token;
  a.parent = parent_idx;
  a.prefix_len = prefix_len;
  a.k_prefix = k_prefix;
  a.v_prefix = v_prefix;
  a.k_tree = k_tree;
  a.v_tree = v_tree;
  a.target_next = target_next;
  a.accept_len = accept_len;
  a.accepted = accepted;
  a.bonus = bonus;
  a.status = status;
  a.T = g.T;
  a.Hkv = g.Hkv;
  a.Lmax = g.Lmax;
  a.nsplit = m.nsplit;
  a.row_bytes = g.D * (g.f32 ? 4 : 2);
  hipLaunchKernelGGL(accept_commit, dim3(g.B), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hta
