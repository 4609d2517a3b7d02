// prefix_attn_splitk.hip -- the prefix pass of tree verification attention on gfx950.
//
// Every tree query attends to its sequence's whole prefix KV cache with no mask (LongSpec
// paper summary, Summary, "Hybrid Tree Attention": the long-context pass over the prefix;
// README, Introduction: fast prefix computation).  The prefix is split into chunks of
// `chunk` keys (split-K, as in Flash-Decoding, the baseline of the summary's Key points);
// each workgroup produces, for one (sequence b, KV head g, chunk s), the normalised partial
// output and log-sum-exp of every query row that reads KV head g.  lse_merge combines them.
//
// MI355X mapping
//  * GQA packing: the T*G query rows that share KV head g (row r = node*G + head-in-group)
//    are processed together, so each K/V byte is read from HBM once per chunk and feeds
//    4*T*G flops -- near the bf16 ridge for the LongSpec tree (T = 68, G = 4).
//  * Matrix cores: v_mfma_f32_16x16x32_bf16.  Scores are formed transposed, S^T = K Q^T
//    (A = 16 keys x 32 dims from LDS, B = 16 query rows held in registers), and the output
//    transposed too, O^T += V^T P^T.  With both products transposed, the lane that holds
//    score column "row" of S^T is exactly the lane that holds B-operand column "row" of
//    P^T and output column "row" of O^T, so the online softmax needs no data movement
//    between the two products and its rescale factors are lane-local.  The V^T operand is
//    read with ds_read_b64_tr_b16 (a transposing LDS read) from V kept row-major in LDS.
//  * Memory: 64-key K and V tiles are fetched with coalesced 16-byte loads into registers
//    while the previous tile is being consumed from LDS (double buffer), then stored to
//    padded LDS rows (stride D+8 for K, D+16 for V) so the MFMA operand reads and the
//    transposing reads are free of bank conflicts.
//  * Online softmax in fp32 with exp2 (scale * log2(e) folded into one multiply).  The
//    probabilities enter the PV product as fp16 (nearest-even; 11 significant bits against
//    bf16's 8, so a peaky softmax stays well inside the output tolerance), V is widened
//    from bf16 to fp16 on the way out of LDS (exact for |v| in [2^-14, 65504]), and the
//    normaliser sums the unrounded fp32 probabilities.  v_mfma_f32_16x16x32_f16 runs at
//    the bf16 rate.
#include "hta_internal.h"

namespace hta {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kKeyTile = 64;

template <int D>
struct PrefixLds {
  static constexpr int KS = D + 8;   // K row stride (bf16 elements)
  static constexpr int VS = D + 16;  // V row stride (bf16 elements)
  static constexpr int kStage = kKeyTile * (KS + VS);
  static constexpr int kElems = 2 * kStage;
};

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline i16x4 tr_read_b64(const unsigned short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// bf16 -> fp16 is exact for |v| in [2^-14, 65504]; smaller magnitudes round to fp16's
// subnormal grid (absolute error below 2^-25).
__device__ inline _Float16 bf16_bits_to_f16(short h) {
  return (_Float16)__builtin_bit_cast(float, (uint32_t)(unsigned short)h << 16);
}

__device__ inline float wave_max_across_groups(float x) {
  // lanes l, l^16, l^32, l^48 hold the same query row
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ inline float wave_sum_across_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

struct PrefixArgs {
  const unsigned short* q;         // bf16 bits [B, T, Hq, D]
  const unsigned short* k_prefix;  // [B, Hkv, Lmax, D]
  const unsigned short* v_prefix;
  const int32_t* prefix_len;       // [B]
  float* lse_part;
  float* o_part;
  Geometry g;
  int32_t row_blocks;              // query-row blocks per (b, kv head)
  float c;                         // scale * log2(e)
};

// One workgroup = 4 waves; wave w owns row tiles rb*4*MT + 4*k + w, k < MT.
template <int D, int MT>
__global__ __launch_bounds__(kThreads, 1) void prefix_attn_splitk(PrefixArgs a) {
  using L = PrefixLds<D>;
  constexpr int KS = L::KS, VS = L::VS;
  constexpr int DS = D / 32;        // 32-wide d steps of the score product
  constexpr int DB = D / 16;        // 16-wide d blocks of the output
  constexpr int CHUNKS = D / 8;     // 16-byte chunks per K/V row
  constexpr int LOADS = kKeyTile * CHUNKS / kThreads;  // 16-byte loads per thread per tile
  __shared__ __attribute__((aligned(16))) unsigned short lds[L::kElems];

  const Geometry& G = a.g;
  const int s = blockIdx.x;
  const int kv = blockIdx.y / a.row_blocks;
  const int rb = blockIdx.y % a.row_blocks;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int grp = lane >> 4;

  int Lb = a.prefix_len[b];
  Lb = Lb < 0 ? 0 : (Lb > G.Lmax ? G.Lmax : Lb);  // out-of-range lengths are flagged elsewhere
  const int kbeg = s * G.chunk;
  if (kbeg >= Lb) return;  // empty chunk: the merge never reads this slot
  const int kend = min(kbeg + G.chunk, Lb);
  const int ntiles = (kend - kbeg + kKeyTile - 1) / kKeyTile;

  const size_t kv_base = ((size_t)b * G.Hkv + kv) * (size_t)G.Lmax * D;
  const unsigned short* Kg = a.k_prefix + kv_base;
  const unsigned short* Vg = a.v_prefix + kv_base;

  // ---- query operand (B of S^T = K Q^T): lane holds Q[row = l16][d = 32*ds + 8*grp .. +7]
  bf16x8 qop[MT][DS];
  bool tile_ok[MT];
#pragma unroll
  for (int k = 0; k < MT; ++k) {
    const int tile = rb * kWaves * MT + kWaves * k + wave;
    tile_ok[k] = tile < G.NT;
    const int row = tile * 16 + l16;
    const bool row_ok = tile_ok[k] && row < G.R;
    const int node = row_ok ? row / G.G : 0;
    const int head = kv * G.G + (row_ok ? row % G.G : 0);
    const unsigned short* qp = a.q + (((size_t)b * G.T + node) * G.Hq + head) * D + 8 * grp;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      uint4 v = row_ok ? *(const uint4*)(qp + 32 * ds) : make_uint4(0, 0, 0, 0);
      qop[k][ds] = as_bf16x8(v);
    }
  }

  f32x4 acc[MT][DB];
  float m_run[MT], l_run[MT];
#pragma unroll
  for (int k = 0; k < MT; ++k) {
    m_run[k] = -INFINITY;
    l_run[k] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[k][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- global -> register staging of one 64-key K/V tile
  uint4 kreg[LOADS], vreg[LOADS];
  auto fetch = [&](int t) {
    const int key0 = kbeg + t * kKeyTile;
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int idx = it * kThreads + tid;
      const int key = idx / CHUNKS, ch = idx % CHUNKS;
      const int gk = key0 + key;
      if (gk < kend) {
        kreg[it] = *(const uint4*)(Kg + (size_t)gk * D + ch * 8);
        vreg[it] = *(const uint4*)(Vg + (size_t)gk * D + ch * 8);
      } else {
        kreg[it] = make_uint4(0, 0, 0, 0);
        vreg[it] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto stash = [&](int stage) {
    unsigned short* Ks = lds + stage * L::kStage;
    unsigned short* Vs = Ks + kKeyTile * KS;
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int idx = it * kThreads + tid;
      const int key = idx / CHUNKS, ch = idx % CHUNKS;
      *(uint4*)(Ks + key * KS + ch * 8) = kreg[it];
      *(uint4*)(Vs + key * VS + ch * 8) = vreg[it];
    }
  };

  fetch(0);
  stash(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    if (t + 1 < ntiles) fetch(t + 1);
    const unsigned short* Ks = lds + stage * L::kStage;
    const unsigned short* Vs = Ks + kKeyTile * KS;
    const int key0 = kbeg + t * kKeyTile;

    // ---- scores S^T[key][row] for the 64 keys of this tile, 4 blocks of 16 keys
    f32x4 sc[MT][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 kop[DS];
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        kop[ds] = *(const bf16x8*)(Ks + (kb * 16 + l16) * KS + 32 * ds + 8 * grp);
#pragma unroll
      for (int k = 0; k < MT; ++k) {
        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
        if (tile_ok[k]) {
#pragma unroll
          for (int ds = 0; ds < DS; ++ds)
            s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ds], qop[k][ds], s4, 0, 0, 0);
        }
        sc[k][kb] = s4;
      }
    }

    // ---- online softmax (this lane: row l16, keys kb*16 + 4*grp + r)
    const bool partial = key0 + kKeyTile > kend;
    f16x8 pop[MT][2];
#pragma unroll
    for (int k = 0; k < MT; ++k) {
      if (partial) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (key0 + kb * 16 + 4 * grp + r >= kend) sc[k][kb][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[k][kb][r]);
      mx = wave_max_across_groups(mx) * a.c;
      const float m_new = fmaxf(m_run[k], mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run[k] - m_new);
      m_run[k] = m_new;
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(sc[k][kb][r] * a.c - m_new);
          sc[k][kb][r] = p;
          lsum += p;
        }
      l_run[k] = l_run[k] * alpha + lsum;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[k][db] *= alpha;
      // P^T operand: k-index 8*grp + e  <->  key 32*ks + 16*(e/4) + 4*grp + e%4
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) pop[k][ks][e] = (_Float16)sc[k][2 * ks + e / 4][e % 4];
    }

    // ---- O^T[d][row] += V^T[d][key] P^T[key][row]
    {
      const int vr = lane & 15;      // lane within its 16-lane block
      const int vrow = 4 * grp + (vr >> 2);
      const int vcol = 4 * (vr & 3);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const unsigned short* p0 = Vs + (32 * ks + vrow) * VS + 16 * db + vcol;
          const i16x4 lo = tr_read_b64(p0);
          const i16x4 hi = tr_read_b64(p0 + 16 * VS);
          f16x8 vop;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vop[e] = bf16_bits_to_f16(lo[e]);
            vop[4 + e] = bf16_bits_to_f16(hi[e]);
          }
#pragma unroll
          for (int k = 0; k < MT; ++k)
            if (tile_ok[k])
              acc[k][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop[k][ks], acc[k][db],
                                                                  0, 0, 0);
        }
      }
    }

    if (t + 1 < ntiles) stash(stage ^ 1);
    __syncthreads();
  }

  // ---- normalise and write the partial of this chunk
  const size_t slot = ((size_t)b * G.Hkv + kv) * (G.S + 1) + s;
#pragma unroll
  for (int k = 0; k < MT; ++k) {
    if (!tile_ok[k]) continue;
    const int tile = rb * kWaves * MT + kWaves * k + wave;
    const int row = tile * 16 + l16;
    const float lt = wave_sum_across_groups(l_run[k]);
    const float inv = 1.f / lt;
    float* op = a.o_part + (slot * G.R_pad + row) * D + 4 * grp;
#pragma unroll
    for (int db = 0; db < DB; ++db) *(f32x4*)(op + 16 * db) = acc[k][db] * inv;
    if (grp == 0) a.lse_part[slot * G.R_pad + row] = (m_run[k] + __log2f(lt)) * kLn2;
  }
}

template <int D, int MT>
hipError_t launch_mt(const PrefixArgs& a, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((prefix_attn_splitk<D, MT>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefixArgs& a, int mt, dim3 grid, hipStream_t stream) {
  switch (mt) {
    case 1: return launch_mt<D, 1>(a, grid, stream);
    case 2: return launch_mt<D, 2>(a, grid, stream);
    case 3: return launch_mt<D, 3>(a, grid, stream);
    case 4: return launch_mt<D, 4>(a, grid, stream);
    case 5: return launch_mt<D, 5>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int prefix_tiles_per_wave(const Geometry& g) {
  // Register budget: at most 4 row tiles per wave for D = 128, 5 for D = 64; more rows are
  // split into row blocks of at most 4 * max tiles each, balanced across blocks.
  const int max_mt = g.D == 128 ? 4 : 5;
  const int blocks = (g.NT + 4 * max_mt - 1) / (4 * max_mt);
  const int tiles_per_block = (g.NT + blocks - 1) / blocks;
  return (tiles_per_block + 3) / 4;
}

hipError_t launch_prefix_attn_splitk(const Geometry& g, const void* q, const void* k_prefix,
                                     const void* v_prefix, const int32_t* prefix_len,
                                     const Workspace& ws, int cu_count, hipStream_t stream) {
  (void)cu_count;
  PrefixArgs a;
  a.q = (const unsigned short*)q;
  a.k_prefix = (const unsigned short*)k_prefix;
  a.v_prefix = (const unsigned short*)v_prefix;
  a.prefix_len = prefix_len;
  a.lse_part = ws.lse_part;
  a.o_part = ws.o_part;
  a.g = g;
  const int mt = prefix_tiles_per_wave(g);
  a.row_blocks = (g.NT + 4 * mt - 1) / (4 * mt);
  a.c = g.scale * kLog2e;
  dim3 grid(g.S, g.Hkv * a.row_blocks, g.B);
  if (g.D == 128) return launch_d<128>(a, mt, grid, stream);
  if (g.D == 64) return launch_d<64>(a, mt, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace hta
