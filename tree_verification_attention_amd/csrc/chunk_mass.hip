// chunk_mass.hip -- each split-K chunk's share of every query row's attention.
//
// The split-K prefix pass leaves, per query row, the log-sum-exp of every prefix chunk, and
// the whole step leaves the row's log-sum-exp over everything it sees (LongSpec README,
// Introduction: the prefix part is computed chunk by chunk and aggregated through these
// statistics).  The share of the row's attention that falls on chunk s is therefore
//     mass[s] = exp(lse_part[s] - lse),
// the tree's share likewise from the tree slot, and a row's shares sum to 1.  Per sequence,
// the mean over its query rows ranks the prefix chunks by the attention they received
// (target-guided context retrieval).
//
// Grid (slot s, sequence b), 256 threads: one workgroup per column of the [rows, S+1] mass
// matrix of one sequence.  A lane takes rows tid, tid + 256, ... (four loads in flight);
// lse_part reads are contiguous across lanes, lse reads are gathers of 8 KB per sequence.
// The column sum is reduced in a fixed order, so results are bitwise reproducible.
// Latency-bound (Llama-3-8B tree, 32 splits: 300 KB read, 290 KB written).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hta_internal.h"

namespace hta {
namespace {

constexpr int kThreads = 256;

struct MassArgs {
  Geometry g;
  const float* lse_part;     // [B, Hkv, S+1, R_pad]
  const float* lse;          // [B, Hq, T]
  const int32_t* prefix_len; // [B]
  float* mass;               // [B, Hq, T, S+1]
  float* scores;             // [B, S+1] or null
};

__global__ __launch_bounds__(kThreads) void chunk_mass(MassArgs a) {
  constexpr int kBatch = 4;
  const Geometry& G = a.g;
  const int s = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = a.prefix_len[b];
  const int Lc = L < 0 ? 0 : (L > G.Lmax ? G.Lmax : L);
  const int nsplit = (Lc + G.chunk - 1) / G.chunk;  // non-empty prefix chunks
  const bool empty = s < G.S && s >= nsplit;       // a chunk past the prefix: no keys
  const int rows = G.Hkv * G.R;
  const float kLog2e_ = kLog2e;
  float local = 0.f;
  for (int r0 = 0; r0 < rows; r0 += kBatch * kThreads) {
    float lp[kBatch], lt[kBatch];
    size_t dst[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int row = r0 + j * kThreads + tid;
      const int rr = row < rows ? row : rows - 1;  // clamped: loaded, never used
      const int g = rr / G.R, r = rr % G.R;
      const int h = g * G.G + r % G.G, i = r / G.G;
      lp[j] = empty ? 0.f : a.lse_part[(((size_t)b * G.Hkv + g) * (G.S + 1) + s) * G.R_pad + r];
      lt[j] = a.lse[((size_t)b * G.Hq + h) * G.T + i];
      dst[j] = (((size_t)b * G.Hq + h) * G.T + i) * (G.S + 1) + s;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int row = r0 + j * kThreads + tid;
      if (row < rows) {
        const float m = empty ? 0.f : __builtin_amdgcn_exp2f((lp[j] - lt[j]) * kLog2e_);
        a.mass[dst[j]] = m;
        local += m;
      }
    }
  }
  if (!a.scores) return;
  __shared__ float part[kThreads];
  part[tid] = local;
  __syncthreads();
#pragma unroll
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  if (tid == 0) a.scores[(size_t)b * (G.S + 1) + s] = part[0] / (float)(G.Hq * G.T);
}

}  // namespace

hipError_t launch_chunk_mass(const Geometry& g, const int32_t* prefix_len, const float* lse,
                             float* mass, float* scores, const Workspace& ws,
                             hipStream_t stream) {
  MassArgs a;
  a.g = g;
  a.lse_part = ws.lse_part;
  a.lse = lse;
  a.prefix_len = prefix_len;
  a.mass = mass;
  a.scores = scores;
  hipLaunchKernelGGL(chunk_mass, dim3(g.S + 1, g.B), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hta
