// prefix_attn_f32.hip -- the prefix pass for fp32 inputs.
//
// Same computation as prefix_attn_splitk (every tree query attends to the whole prefix with
// no mask, split into chunks, partial output and log-sum-exp per chunk; LongSpec paper
// summary, Summary, "Hybrid Tree Attention"), for q, K, V held in fp32.  This form exists
// for small validation shapes given in fp32; it uses plain fp32 vector arithmetic (no
// rounding of any operand), not the bf16/fp16 matrix cores.
//
// Grid (chunk s, KV head, sequence b); four waves, each taking query rows w, w+4, ... of
// the KV head's T*G rows.  Per row the wave walks the chunk 64 keys at a time: lane j scores
// key j (the query row read from LDS as a broadcast), the wave keeps a running maximum and
// sum (exp2 with scale*log2(e) folded in), and the lanes then own output dimensions
// (d = lane + 64 e) and accumulate the probability-weighted values, each key's probability
// taken from its lane by a shuffle.
#include "hta_internal.h"

namespace hta {

namespace {

constexpr int kWaves = 4;

struct PrefixF32Args {
  const float* q;           // [B, T, Hq, D]
  const float* k_prefix;    // [B, Hkv, Lmax, D]
  const float* v_prefix;
  const int32_t* prefix_len;
  int32_t* status_reset;  // [B] or nullptr: cleared by the first workgroup of b
  float* lse_part;
  float* o_scale;    // the factor of each o_part row
  uint32_t* o_part;  // 16-bit rows (pack16)
  Geometry g;
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
__global__ __launch_bounds__(64 * kWaves) void prefix_attn_f32(PrefixF32Args a) {
  constexpr int DPL = D / 64;  // output dimensions per lane
  __shared__ float s_q[kWaves][D];
  const Geometry& G = a.g;
  const int s = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (a.status_reset && s == 0 && kv == 0 && threadIdx.x == 0) a.status_reset[b] = 0;
  int Lb = a.prefix_len[b];
  Lb = Lb < 0 ? 0 : (Lb > G.Lmax ? G.Lmax : Lb);  // out-of-range lengths are flagged elsewhere
  const int kbeg = s * G.chunk;
  if (kbeg >= Lb) return;  // empty chunk: the merge never reads this slot
  const int kend = min(kbeg + G.chunk, Lb);
  const float c = G.scale * kLog2e;
  const size_t kv_base = ((size_t)b * G.Hkv + kv) * (size_t)G.Lmax * D;
  const float* Kg = a.k_prefix + kv_base;
  const float* Vg = a.v_prefix + kv_base;
  const size_t slot = ((size_t)b * G.Hkv + kv) * (G.S + 1) + s;

  for (int r = wave; r < G.R; r += kWaves) {
    const int node = r / G.G, head = kv * G.G + r % G.G;
    const float* qp = a.q + (((size_t)b * G.T + node) * G.Hq + head) * D;
    for (int d = lane; d < D; d += 64) s_q[wave][d] = qp[d];
    __builtin_amdgcn_wave_barrier();
    float m = -INFINITY, l = 0.f, acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
    for (int k0 = kbeg; k0 < kend; k0 += 64) {
      const int key = k0 + lane;
      float x = -INFINITY;
      if (key < kend) {
        const float4* kp = (const float4*)(Kg + (size_t)key * D);
        float dot = 0.f;
#pragma unroll 8
        for (int d4 = 0; d4 < D / 4; ++d4) {
          const float4 kk = kp[d4];
          dot += s_q[wave][4 * d4] * kk.x + s_q[wave][4 * d4 + 1] * kk.y +
                 s_q[wave][4 * d4 + 2] * kk.z + s_q[wave][4 * d4 + 3] * kk.w;
        }
        x = dot * c;
      }
      const float m_new = fmaxf(m, wave_max(x));  // finite: key k0 exists
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      const float p = key < kend ? __builtin_amdgcn_exp2f(x - m_new) : 0.f;
      m = m_new;
      l = l * alpha + wave_sum(p);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] *= alpha;
      const int n = min(64, kend - k0);
      for (int j = 0; j < n; ++j) {
        const float pj = __shfl(p, j);
        const float* vp = Vg + (size_t)(k0 + j) * D + lane;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] += pj * vp[64 * e];
      }
    }
    const float inv = 1.f / l;
    // lane owns dims lane + 64 e: the row's factor from a wave reduction, then every
    // second lane packs its pair of values
    float amax = 0.f, sum = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      acc[e] *= inv;
      amax = fmaxf(amax, __builtin_fabsf(acc[e]));
      sum += acc[e];
    }
    const RowCode rc = row_code(wave_max(amax), wave_sum(sum));
    uint32_t* orow = a.o_part + (slot * G.R_pad + r) * (D / 2);
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const float x1 = __shfl_down(acc[e], 1);
      if ((lane & 1) == 0) orow[(lane + 64 * e) / 2] = pack16(acc[e], x1, rc.enc);
    }
    if (lane == 0) {
      a.lse_part[slot * G.R_pad + r] = (m + __log2f(l)) * kLn2;
      a.o_scale[slot * G.R_pad + r] = rc.f;
    }
    __builtin_amdgcn_wave_barrier();  // s_q is rewritten for the next row
  }
}

}  // namespace

hipError_t launch_prefix_attn_f32(const Geometry& g, const void* q, const void* k_prefix,
                                  const void* v_prefix, const int32_t* prefix_len,
                                  const Workspace& ws, hipStream_t stream) {
  PrefixF32Args a;
  a.q = (const float*)q;
  a.k_prefix = (const float*)k_prefix;
  a.v_prefix = (const float*)v_prefix;
  a.prefix_len = prefix_len;
  a.status_reset = ws.status_reset;
  a.lse_part = ws.lse_part;
  a.o_scale = ws.o_scale;
  a.o_part = ws.o_part;
  a.g = g;
  dim3 grid(g.S, g.Hkv, g.B);
  if (g.D == 128)
    hipLaunchKernelGGL(prefix_attn_f32<128>, grid, dim3(64 * kWaves), 0, stream, a);
  else if (g.D == 64)
    hipLaunchKernelGGL(prefix_attn_f32<64>, grid, dim3(64 * kWaves), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hta
