// tree_attn_masked.hip -- the tree pass of tree verification attention on gfx950.
//
// Tree tokens attend to each other under the tree mask (LongSpec paper summary, Summary,
// "Hybrid Tree Attention": the separate kernel for the speculated tree; README,
// Introduction: standard attention for the tree-mask part).  Node i sees node t iff t is i
// or one of i's ancestors.
//
// Ancestor masks.  Each workgroup loads its sequence's parent pointers into LDS, checks
// them (parent[i] in [-1, i-1], combined across the workgroup with a barrier-OR), and
// builds every node's packed ancestor-or-self mask by pointer jumping: node i keeps a
// jump pointer a_i (initially its parent) and a mask M_i (initially bit i); each round
// sets M_i |= M_{a_i} and a_i = a_{a_i}, doubling the covered path length, until every
// jump pointer reaches the root.  ceil(log2(depth + 1)) rounds; bit-exact.
//
// Attention.  One wave per query row: the lanes that own a visible key compute its score,
// the wave reduces max and sum, and the lanes then own output dimensions and accumulate
// the visible values.  All fp32 on exactly widened bf16 inputs.  The result is the tree
// partial (slot S of the partial buffers), merged with the prefix partials by lse_merge.
#include "hta_internal.h"

namespace hta {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxT = 256;
constexpr int kMaxW = kMaxT / 64;
constexpr int kRowsPerWave = 2;

struct TreeArgs {
  const unsigned short* q;        // bf16 [B, T, Hq, D]
  const unsigned short* k_tree;   // [B, Hkv, T, D]
  const unsigned short* v_tree;
  const int32_t* parent_idx;      // [B, T]
  const int32_t* prefix_len;      // [B]
  int32_t* status;                // [B]
  uint64_t* masks_out;            // [B, T, W] or null
  float* lse_part;
  float* o_part;
  Geometry g;
  int32_t attention;              // 0: masks and status only
};

__device__ inline float bf16_to_f32(unsigned short h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Grid: x = row block of kRowsPerWave*4 rows, y = kv head, z = sequence.
template <int D>
__global__ __launch_bounds__(kThreads) void tree_attn_masked(TreeArgs a) {
  __shared__ uint64_t s_mask[kMaxT][kMaxW];
  __shared__ int32_t s_jump[kMaxT];
  __shared__ float s_p[kThreads / 64][kMaxT];
  const Geometry& G = a.g;
  const int b = blockIdx.z, kv = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = G.T, W = G.W;

  // ---- load and validate parent pointers; seed the pointer-jumping state
  int bad = 0;
  for (int i = tid; i < T; i += kThreads) {
    const int p = a.parent_idx[(size_t)b * T + i];
    const bool ok = p >= -1 && p < i;
    bad |= ok ? 0 : 1;
    s_jump[i] = ok ? p : -1;
    for (int w = 0; w < W; ++w) s_mask[i][w] = (w == (i >> 6)) ? (1ull << (i & 63)) : 0ull;
  }
  const int tree_bad = __syncthreads_or(bad);
  const int Lb = a.prefix_len ? a.prefix_len[b] : 0;
  const bool len_bad = Lb < 0 || Lb > G.Lmax;

  // ---- pointer jumping: M_i |= M_{a_i}; a_i = a_{a_i} until all a_i == -1.
  // T <= kThreads, so thread i owns node i.  Jump pointers only ever decrease, so the loop
  // ends after at most ceil(log2(T)) + 1 rounds even for a rejected tree.
  for (;;) {
    int j = -1, nj = -1;
    uint64_t nm[kMaxW];
    if (tid < T) {
      j = s_jump[tid];
      if (j >= 0) {
        nj = s_jump[j];
        for (int w = 0; w < W; ++w) nm[w] = s_mask[tid][w] | s_mask[j][w];
      }
    }
    if (!__syncthreads_or(j >= 0)) break;
    if (j >= 0) {
      for (int w = 0; w < W; ++w) s_mask[tid][w] = nm[w];
      s_jump[tid] = nj;
    }
    __syncthreads();
  }

  if (blockIdx.x == 0 && kv == 0) {
    if (tid == 0) a.status[b] = (tree_bad ? kStatusTree : 0) | (len_bad ? kStatusPrefixLen : 0);
    if (a.masks_out)
      for (int i = tid; i < T; i += kThreads)
        for (int w = 0; w < W; ++w)
          a.masks_out[((size_t)b * T + i) * W + w] = tree_bad ? ~0ull : s_mask[i][w];
  }
  if (!a.attention) return;

  // ---- masked attention, one wave per row
  const size_t slot = ((size_t)b * G.Hkv + kv) * (G.S + 1) + G.S;
  const unsigned short* Kt = a.k_tree + ((size_t)b * G.Hkv + kv) * (size_t)T * D;
  const unsigned short* Vt = a.v_tree + ((size_t)b * G.Hkv + kv) * (size_t)T * D;
  constexpr int DPL = D / 64;  // output dims per lane
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int row = (blockIdx.x * (kThreads / 64) + wave) * kRowsPerWave + rr;
    if (row >= G.R) break;
    const int node = row / G.G;
    const int head = kv * G.G + row % G.G;
    const unsigned short* qp = a.q + (((size_t)b * T + node) * G.Hq + head) * D;
    float* op = a.o_part + (slot * G.R_pad + row) * D;
    if (tree_bad) {
      for (int d = lane; d < D; d += 64) op[d] = NAN;
      if (lane == 0) a.lse_part[slot * G.R_pad + row] = NAN;
      continue;
    }
    // scores of the visible keys (lane t%64 owns key t)
    float mx = -INFINITY;
    for (int t0 = 0; t0 < T; t0 += 64) {
      const int t = t0 + lane;
      float s = -INFINITY;
      if (t < T && ((s_mask[node][t >> 6] >> (t & 63)) & 1ull)) {
        const uint4* kp = (const uint4*)(Kt + (size_t)t * D);
        const uint4* q4 = (const uint4*)qp;
        float dot = 0.f;
#pragma unroll 4
        for (int c = 0; c < D / 8; ++c) {
          const uint4 kk = kp[c], qq = q4[c];
          const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w};
          const uint32_t qw[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dot += bf16_to_f32(qw[e] & 0xffff) * bf16_to_f32(kw[e] & 0xffff);
            dot += bf16_to_f32(qw[e] >> 16) * bf16_to_f32(kw[e] >> 16);
          }
        }
        s = dot * G.scale;
      }
      if (t < T) s_p[wave][t] = s;
      mx = fmaxf(mx, s);
    }
    mx = wave_max(mx);  // finite: node itself is always visible
    float z = 0.f;
    for (int t = lane; t < T; t += 64) {
      const float s = s_p[wave][t];
      const float p = (s == -INFINITY) ? 0.f : __expf(s - mx);
      s_p[wave][t] = p;
      z += p;
    }
    z = wave_sum(z);
    __builtin_amdgcn_wave_barrier();
    float o[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = 0.f;
    for (int w = 0; w < W; ++w) {
      uint64_t bits = s_mask[node][w];
      while (bits) {
        const int t = w * 64 + __builtin_ctzll(bits);
        bits &= bits - 1;
        const float p = s_p[wave][t];
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] += p * bf16_to_f32(Vt[(size_t)t * D + lane + 64 * e]);
      }
    }
    const float inv = 1.f / z;
#pragma unroll
    for (int e = 0; e < DPL; ++e) op[lane + 64 * e] = o[e] * inv;
    if (lane == 0) a.lse_part[slot * G.R_pad + row] = mx + __logf(z);
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

hipError_t launch_tree_attn_masked(const Geometry& g, const void* q, const void* k_tree,
                                   const void* v_tree, const int32_t* parent_idx,
                                   const int32_t* prefix_len, const Workspace& ws,
                                   uint64_t* masks_out, bool attention, hipStream_t stream) {
  TreeArgs a;
  a.q = (const unsigned short*)q;
  a.k_tree = (const unsigned short*)k_tree;
  a.v_tree = (const unsigned short*)v_tree;
  a.parent_idx = parent_idx;
  a.prefix_len = prefix_len;
  a.status = ws.status;
  a.masks_out = masks_out;
  a.lse_part = ws.lse_part;
  a.o_part = ws.o_part;
  a.g = g;
  a.attention = attention ? 1 : 0;
  const int rows_per_block = kRowsPerWave * (kThreads / 64);
  const int xblocks = attention ? (g.R + rows_per_block - 1) / rows_per_block : 1;
  dim3 grid(xblocks, attention ? g.Hkv : 1, g.B);
  if (g.D == 128)
    hipLaunchKernelGGL(tree_attn_masked<128>, grid, dim3(kThreads), 0, stream, a);
  else if (g.D == 64)
    hipLaunchKernelGGL(tree_attn_masked<64>, grid, dim3(kThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hta
