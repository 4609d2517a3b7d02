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
// Attention on the matrix cores, one wave per 16-row tile (rows r = node*G + head-in-group
// of one KV head, as in the prefix pass).  The workgroup streams the sequence's tree K and V
// rows of its KV head into LDS with direct loads issued first thing, and loads its query
// operands, so their latency overlaps the mask construction.  Scores are formed transposed,
// S^T = K Q^T (v_mfma_f32_16x16x32_bf16), masked with the lane's node mask, and turned into
// probabilities against a per-row running maximum over 64-key tiles (at most four tiles:
// T <= 256).  The output is O^T += V^T P^T (v_mfma_f32_16x16x32_f16) with V^T operands read
// by transposing reads (ds_read_b64_tr_b16) and widened from bf16 to fp16 in registers;
// probabilities (at most 1) enter as fp16, the normaliser sums them unrounded in fp32.  The
// result is the tree partial (slot S of the partial buffers), merged with the prefix
// partials by lse_merge.
#include "hta_internal.h"
#include "lds_tiles.h"

namespace hta {

namespace {

constexpr int kWaves = 4;  // one 16-row tile per wave
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxT = 256;
constexpr int kMaxW = kMaxT / 64;

typedef __attribute__((ext_vector_type(4))) short i16x4;

struct TreeArgs {
  const unsigned short* q;        // bf16 [B, T, Hq, D]
  const unsigned short* k_tree;   // [B, Hkv, T, D]
  const unsigned short* v_tree;
  const int32_t* parent_idx;      // [B, T]
  const int32_t* prefix_len;      // [B]
  int32_t* status;                // [B]
  uint64_t* masks_out;            // [B, T, W] or null
  float* lse_part;
  float* o_scale;                 // the factor of each o_part row
  uint32_t* o_part;               // 16-bit rows (pack16x4)
  Geometry g;
  int32_t attention;              // 0: masks and status only
};

__device__ inline _Float16 bf16_bits_to_f16(short h) {
  return (_Float16)__builtin_bit_cast(float, (uint32_t)(unsigned short)h << 16);
}

// lanes l, l^16, l^32, l^48 hold the same query row
__device__ inline float group_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float group_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Grid: x = group of kWaves row tiles, y = kv head, z = sequence.
template <int D>
__global__ __launch_bounds__(kThreads) void tree_attn_masked(TreeArgs a) {
  constexpr int DS = D / 32;          // 32-wide d steps of the score product
  constexpr int DB = D / 16;          // 16-wide d blocks of the output
  __shared__ uint64_t s_mask[kMaxT][kMaxW];
  __shared__ int32_t s_jump[kMaxT];
  // K and V tiles of the sequence's tree keys: dynamic LDS of 2 * ceil(T / 64) tiles
  extern __shared__ __attribute__((aligned(1024))) unsigned char s_kv[];
  const Geometry& G = a.g;
  const int b = blockIdx.z, kv = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, grp = lane >> 4;
  const int T = G.T, W = G.W;
  constexpr int kTileBytes = kKeyTile * D * 2;
  const int ntile = (T + kKeyTile - 1) / kKeyTile;
  unsigned char* s_k = s_kv;
  unsigned char* s_vv = s_kv + ntile * kTileBytes;
  const unsigned short* Kt = a.k_tree + ((size_t)b * G.Hkv + kv) * (size_t)T * D;
  const unsigned short* Vt = a.v_tree + ((size_t)b * G.Hkv + kv) * (size_t)T * D;
  const int rt = blockIdx.x * kWaves + wave;  // this wave's row tile
  const int row = rt * 16 + l16;
  const bool row_ok = rt < G.NT && row < G.R;
  const int node = row_ok ? row / G.G : 0;
  const int head = kv * G.G + (row_ok ? row % G.G : 0);
  // parent pointers first: their latency then overlaps the issue of everything else
  const int par = tid < T ? a.parent_idx[(size_t)b * T + tid] : -1;
  bf16x8 qop[DS];
  if (a.attention) {
    // issue every global read of the attention up front: K/V tiles straight into LDS,
    // this wave's query operands (B of S^T: Q[row = l16][d = 32 ds + 8 grp ..]) into
    // registers; padding rows read zeros
    for (int t = 0; t < ntile; ++t)
      dma_kv_tile<D, kWaves, true>(Kt, Vt, t * kKeyTile, T, s_k + t * kTileBytes,
                                   s_vv + t * kTileBytes, wave, lane);
    // V rows of the blocks left out (past T, up to the end of the last tile) must hold
    // finite values: they meet probability 0 in the PV product.  K rows there stay
    // undefined; their scores are masked before use.
    constexpr int kRowsPerBlock = 1024 / (2 * D);
    const int zrow = (T + kRowsPerBlock - 1) / kRowsPerBlock * kRowsPerBlock;
    for (int u = zrow * (2 * D / 16) + tid; u < ntile * kKeyTile * (2 * D / 16); u += kThreads)
      *(uint4*)(s_vv + 16 * u) = make_uint4(0, 0, 0, 0);
    const unsigned short* qp = a.q + (((size_t)b * T + node) * G.Hq + head) * D + 8 * grp;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const uint4 v = row_ok ? *(const uint4*)(qp + 32 * ds) : make_uint4(0, 0, 0, 0);
      qop[ds] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- load and validate parent pointers; seed the pointer-jumping state
  int bad = 0;
  if (tid < T) {  // T <= kThreads: thread i owns node i
    const int i = tid;
    const bool ok = par >= -1 && par < i;
    bad = ok ? 0 : 1;
    s_jump[i] = ok ? par : -1;
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

  // the tiles have landed (this wave's loads) and are visible (barrier)
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  __syncthreads();

  if (rt >= G.NT) return;
  const size_t slot = ((size_t)b * G.Hkv + kv) * (G.S + 1) + G.S;
  uint32_t* orow = a.o_part + (slot * G.R_pad + row) * (D / 2);
  if (tree_bad) {  // a NaN factor makes the whole row NaN
    if (row_ok && grp == 0) {
      a.lse_part[slot * G.R_pad + row] = NAN;
      a.o_scale[slot * G.R_pad + row] = NAN;
    }
    return;
  }

  const float c = G.scale * kLog2e;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero4;
  float m_run = -INFINITY, l_run = 0.f;
  // V^T operand lanes: d = 16 db + l16, keys 32 h + 16 (e / 4) + 4 grp + e % 4
  const int vrow = 4 * grp + (l16 >> 2);
  const int vch = (l16 & 3) >> 1, vhalf = 8 * (l16 & 1);

  for (int tile = 0; tile < ntile; ++tile) {
    // ---- scores of keys 64 tile + 16 kb + 4 grp + i (keys past T re-read key T-1, masked)
    const unsigned char* Ks = s_k + tile * kTileBytes;
    f32x4 sc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int kr = kb * 16 + l16;
      sc[kb] = zero4;
      if (tile * kKeyTile + kb * 16 >= T) continue;  // no key of this block exists
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const bf16x8 kop =
            *(const bf16x8*)(Ks + kr * (2 * D) + 16 * ((4 * ds + grp) ^ swz_k<D>(kr)));
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[ds], sc[kb], 0, 0, 0);
      }
    }
    // ---- ancestor-or-self mask of this lane's node (key t visible iff bit t is set)
    const uint64_t mw = s_mask[node][tile];
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = kb * 16 + 4 * grp + i;
        const float x = ((mw >> k) & 1ull) ? sc[kb][i] * c : -INFINITY;
        sc[kb][i] = x;
        tmax = fmaxf(tmax, x);
      }
    const float m_new = fmaxf(m_run, group_max(tmax));
    // a row may see no key of this tile (and none before): keep its state at zero
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] *= alpha;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (tile * kKeyTile + 32 * h >= T) break;  // no key of this half exists
      // P^T operand of the 32-key half h: element e <-> key 32 h + 16 (e / 4) + 4 grp + e % 4
      f16x8 pop;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(sc[2 * h + e / 4][e % 4] - m_use);
        l_run += p;
        pop[e] = (_Float16)p;
      }
      const unsigned char* Vs = s_vv + tile * kTileBytes;
      const int r0 = 32 * h + vrow, r1 = r0 + 16;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int ch = 2 * db + vch;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(
            Vs + r0 * (2 * D) + 16 * (ch ^ swz_v<D>(r0)) + vhalf));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(
            Vs + r1 * (2 * D) + 16 * (ch ^ swz_v<D>(r1)) + vhalf));
        f16x8 vop;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vop[e] = bf16_bits_to_f16(lo[e]);
          vop[4 + e] = bf16_bits_to_f16(hi[e]);
        }
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop, acc[db], 0, 0, 0);
      }
    }
  }

  // ---- normalise and write the tree partial (every real row sees at least itself)
  // (16-bit values with the row's factor, from its largest magnitude over the 4 lanes
  // holding it; dims 16 db + 4 grp .. + 3 are dwords 8 db + 2 grp, + 1 of the row)
  const float lt = group_sum(l_run);
  float amax = 0.f, sum = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      amax = fmaxf(amax, __builtin_fabsf(acc[db][e]));
      sum += acc[db][e];
    }
  amax = group_max(amax);
  sum = group_sum(sum);
  if (!row_ok) return;
  const float inv = 1.f / lt;
  const RowCode rc = row_code(amax * inv, sum * inv);
#pragma unroll
  for (int db = 0; db < DB; ++db) *(uint2*)(orow + 8 * db + 2 * grp) = pack16x4(acc[db], rc.enc * inv);
  if (grp == 0) {
    a.lse_part[slot * G.R_pad + row] = (m_run + __log2f(lt)) * kLn2;
    a.o_scale[slot * G.R_pad + row] = rc.f;
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
  a.o_scale = ws.o_scale;
  a.o_part = ws.o_part;
  a.g = g;
  a.attention = attention ? 1 : 0;
  const int xblocks = attention ? (g.NT + kWaves - 1) / kWaves : 1;
  dim3 grid(xblocks, attention ? g.Hkv : 1, g.B);
  // K and V staging: ceil(T / 64) tiles each (none when only the masks are built)
  const size_t shmem = attention ? (size_t)2 * ((g.T + 63) / 64) * 64 * 2 * g.D : 0;
  if (shmem > 65536) {  // above the default dynamic-LDS limit (T > 128 at D = 128)
    const hipError_t e = g.D == 128
        ? hipFuncSetAttribute((const void*)tree_attn_masked<128>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem)
        : hipFuncSetAttribute((const void*)tree_attn_masked<64>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  if (g.D == 128)
    hipLaunchKernelGGL(tree_attn_masked<128>, grid, dim3(kThreads), shmem, stream, a);
  else if (g.D == 64)
    hipLaunchKernelGGL(tree_attn_masked<64>, grid, dim3(kThreads), shmem, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hta
