// lse_merge.hip -- the aggregation step of tree verification attention on gfx950.
//
// The prefix pass and the tree pass each produce a normalised partial attention and its
// log-sum-exp over a disjoint set of keys; LongSpec aggregates them into the attention over
// the union (README, Introduction, "Hybrid Attention Aggregation"; arXiv abstract).  Since
// the decoding is lossless the aggregation must be exact, which the log-sum-exp merge is:
//     M = max_s lse_s,   w_s = exp(lse_s - M),
//     out = sum_s w_s o_s / sum_s w_s,   lse = M + ln sum_s w_s.
// Here the parts are the split-K chunks of the prefix (only the ceil(prefix_len/chunk)
// non-empty ones are read) and the tree partial.
//
// One wave per output row (b, i, h): lane s reads lse of part s, the wave reduces the
// maximum and the weight sum, then the lanes own output dimensions (D/64 each) and stream
// the partial rows with coalesced loads.  Output rows are contiguous in out [B, T, Hq, D],
// so consecutive waves write consecutive 512-byte rows.
#include "hta_internal.h"

namespace hta {

namespace {

constexpr int kThreads = 256;

struct MergeArgs {
  const int32_t* prefix_len;
  const int32_t* status;   // [B] or null
  const float* lse_part;
  const float* o_part;
  float* out;
  float* lse;
  Geometry g;
  int32_t include_tree;
};

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

template <int D>
__global__ __launch_bounds__(kThreads) void lse_merge(MergeArgs a) {
  constexpr int DPL = D / 64;
  const Geometry& G = a.g;
  const int lane = threadIdx.x & 63;
  const long row_id = (long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const long nrows = (long)G.B * G.T * G.Hq;
  if (row_id >= nrows) return;
  const int h = (int)(row_id % G.Hq);
  const int i = (int)((row_id / G.Hq) % G.T);
  const int b = (int)(row_id / ((long)G.Hq * G.T));
  const int kv = h / G.G;
  const int r = i * G.G + (h % G.G);
  float* outp = a.out + row_id * D;
  float* lsep = a.lse + ((size_t)b * G.Hq + h) * G.T + i;

  const int Lb = a.prefix_len[b];
  const bool bad = Lb < 0 || Lb > G.Lmax || (a.status && a.status[b] != 0);
  if (bad) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) outp[lane + 64 * e] = NAN;
    if (lane == 0) *lsep = NAN;
    return;
  }
  const int nsplit = (Lb + G.chunk - 1) / G.chunk;
  const size_t slot0 = ((size_t)b * G.Hkv + kv) * (G.S + 1);
  // parts: prefix splits 0..nsplit-1, then (optionally) the tree partial at slot S
  const int nparts = nsplit + (a.include_tree ? 1 : 0);
  auto part_slot = [&](int p) { return slot0 + (p < nsplit ? p : G.S); };

  float M = -INFINITY;
  for (int p = lane; p < nparts; p += 64) M = fmaxf(M, a.lse_part[part_slot(p) * G.R_pad + r]);
  M = wave_max(M);
  if (M == -INFINITY) {  // no visible key at all (prefix-only merge of an empty prefix)
#pragma unroll
    for (int e = 0; e < DPL; ++e) outp[lane + 64 * e] = 0.f;
    if (lane == 0) *lsep = -INFINITY;
    return;
  }
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  for (int p0 = 0; p0 < nparts; p0 += 64) {
    const int p = p0 + lane;
    float w = 0.f;
    if (p < nparts) {
      const float l = a.lse_part[part_slot(p) * G.R_pad + r];
      w = __builtin_amdgcn_exp2f((l - M) * kLog2e);
    }
    wsum += w;
    const int cnt = min(64, nparts - p0);
    for (int k = 0; k < cnt; ++k) {
      const float wk = __shfl(w, k);
      const float* op = a.o_part + (part_slot(p0 + k) * G.R_pad + r) * D;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += wk * op[lane + 64 * e];
    }
  }
  wsum = wave_sum(wsum);
  const float inv = 1.f / wsum;
#pragma unroll
  for (int e = 0; e < DPL; ++e) outp[lane + 64 * e] = acc[e] * inv;
  if (lane == 0) *lsep = M + __logf(wsum);
}

}  // namespace

hipError_t launch_lse_merge(const Geometry& g, const int32_t* prefix_len, bool include_tree,
                            float* out, float* lse, const Workspace& ws, hipStream_t stream) {
  MergeArgs a;
  a.prefix_len = prefix_len;
  a.status = include_tree ? ws.status : nullptr;
  a.lse_part = ws.lse_part;
  a.o_part = ws.o_part;
  a.out = out;
  a.lse = lse;
  a.g = g;
  a.include_tree = include_tree ? 1 : 0;
  const long nrows = (long)g.B * g.T * g.Hq;
  const int rows_per_block = kThreads / 64;
  dim3 grid((unsigned)((nrows + rows_per_block - 1) / rows_per_block));
  if (g.D == 128)
    hipLaunchKernelGGL(lse_merge<128>, grid, dim3(kThreads), 0, stream, a);
  else if (g.D == 64)
    hipLaunchKernelGGL(lse_merge<64>, grid, dim3(kThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hta
