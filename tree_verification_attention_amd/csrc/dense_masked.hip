// dense_masked.hip -- tree verification without the hybrid split: one masked attention
// over all L + T keys in a single pass, reading an explicit mask.
//
// The LongSpec paper summary (Summary; Key points, "Hybrid Tree Attention") explains why the
// split is needed: a tree mask keeps verification off the optimized long-context attention
// kernels, and the hybrid split cut the target's attention latency to about a quarter.  This
// file is that "before" on MI355X, built the way an optimized kernel that accepts an
// arbitrary mask works (FlashAttention-2 style): parallel over query tiles and KV heads,
// every workgroup streaming the whole key range of its KV head once, with no split over keys
// and no merge.  Timing it against hta_verify gives the method's before/after ratio on this
// hardware.
//
// dense_mask     builds the explicit mask of each node: bit j of the prefix words is set iff
//                j < prefix_len[b]; bit t of the tree words iff t is the node or one of its
//                ancestors.  Word-major layout [B, W, T_pad] (T_pad = T rounded up to even),
//                so one key tile's words of consecutive nodes are contiguous.  One workgroup
//                per (node, sequence).
// dense_masked   grid (group of 4 row tiles, KV head, sequence), 4 waves, one 16-row tile
//                each (rows r = node * G + head-in-group, as everywhere here).  Key tiles of
//                64 (the prefix's, then the tree's) stream into a 4-stage LDS ring with
//                direct loads (K and V, plus each wave's 16 bytes per lane of the mask words of
//                its nodes for that tile, from the word-major mask); scores S^T = K Q^T and O^T += V^T P^T on the matrix cores, online
//                softmax in fp32, probabilities as fp16 (as in the tree kernel).
#include "hta_internal.h"
#include "lds_tiles.h"

namespace hta {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 4;
constexpr int kMaskWords = 128;  // per wave and stage: 16 bytes per lane

typedef __attribute__((ext_vector_type(4))) short i16x4;

struct DenseArgs {
  const unsigned short* q;         // bf16 [B, T, Hq, D]
  const unsigned short* k_prefix;  // [B, Hkv, Lmax, D]
  const unsigned short* v_prefix;
  const unsigned short* k_tree;    // [B, Hkv, T, D]
  const unsigned short* v_tree;
  const uint64_t* mask;            // [B, Wm, T_pad] words (word-major)
  const int32_t* prefix_len;
  float* out;                      // [B, T, Hq, D]
  float* lse;                      // [B, Hq, T]
  Geometry g;
  int32_t Wp, Wm, T_pad;           // prefix words, all words per node; node stride padded
};

__device__ inline _Float16 bf16_to_f16(short h) {
  return (_Float16)__builtin_bit_cast(float, (uint32_t)(unsigned short)h << 16);
}
__device__ inline float group_max(float x) {  // lanes l, l^16, l^32, l^48 share a row
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

// Wait until at most N of this wave's vector-memory operations (the direct loads of later
// tiles) are outstanding and its LDS accesses have completed, then barrier.  A plain
// __syncthreads() would also drain the later tiles' loads (its fence waits for all of them).
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// Barrier once this wave's LDS reads have completed (a stage may then be refilled).
__device__ __forceinline__ void lds_done_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Eight transposing LDS reads (ds_read_b64_tr_b16) and the wait for them, in one block:
// the compiler would otherwise drain every outstanding direct load in front of such a read.
__device__ __forceinline__ void tr_read8(i16x4 (&r)[8], const uint32_t (&addr)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]),
        "v"(addr[6]), "v"(addr[7])
      : "memory");
}

__device__ __forceinline__ void tr_read4(i16x4 (&r)[4], const uint32_t (&addr)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3])
      : "memory");
}

template <int D>
__global__ __launch_bounds__(kThreads) void dense_masked(DenseArgs a) {
  constexpr int DS = D / 32, DB = D / 16;
  constexpr int kTileBytes = kKeyTile * D * 2;
  constexpr int kLoadsPerTile = 2 * kTileBytes / (1024 * kWaves) + 1;  // K, V blocks + mask
  // one LDS buffer: per stage the K tile, the V tile and each wave's mask words
  constexpr int kMaskBytes = kWaves * kMaskWords * 8;
  constexpr int kStageBytes = 2 * kTileBytes + kMaskBytes;
  // after the ring: one fp16 V^T tile in PV operand order, built by the four waves together
  // (unit u = 2 db + h holds lane l's 16-byte operand at (u * 64 + l) * 16)
  constexpr int kUnits = 2 * DB, kUnitsPerWave = kUnits / kWaves;
  __shared__ __attribute__((aligned(1024))) unsigned char s_lds[kStages * kStageBytes + kTileBytes];
  unsigned char* const s_vt = s_lds + kStages * kStageBytes;
  auto k_tile = [&](int st) { return s_lds + st * kStageBytes; };
  auto v_tile = [&](int st) { return s_lds + st * kStageBytes + kTileBytes; };
  auto mask_words = [&](int st, int w) {
    return (uint64_t*)(s_lds + st * kStageBytes + 2 * kTileBytes) + w * kMaskWords;
  };
  const Geometry& G = a.g;
  const int b = blockIdx.z, kv = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, grp = lane >> 4;
  const int T = G.T;
  const int rt = blockIdx.x * kWaves + wave;
  const int row = rt * 16 + l16;
  const bool row_ok = rt < G.NT && row < G.R;
  // the wave's first node (clamped for waves of padding rows); padding rows stand in as it
  // (their query is zero and nothing is stored)
  const int nw = min((rt * 16) / G.G, G.T - 1);
  const int node = row_ok ? row / G.G : nw;
  const int head = kv * G.G + (row_ok ? row % G.G : 0);
  const int L = a.prefix_len[b];
  const bool len_bad = L < 0 || L > G.Lmax;
  const int Lc = len_bad ? 0 : L;
  const int ntp = (Lc + kKeyTile - 1) / kKeyTile, ntt = (T + kKeyTile - 1) / kKeyTile;
  const int ntiles = ntp + ntt;
  const size_t kvoff = (size_t)b * G.Hkv + kv;
  const unsigned short* Kp = a.k_prefix + kvoff * (size_t)G.Lmax * D;
  const unsigned short* Vp = a.v_prefix + kvoff * (size_t)G.Lmax * D;
  const unsigned short* Kt = a.k_tree + kvoff * (size_t)T * D;
  const unsigned short* Vt = a.v_tree + kvoff * (size_t)T * D;
  // mask words of the wave's nodes for one tile: lane l fetches the 16 bytes holding nodes
  // na + 2 l and na + 2 l + 1 (na = nw rounded down to even; rows are 16-byte aligned)
  const int na = nw & ~1;
  const uint32_t moff = 8u * (uint32_t)min(na + 2 * lane, a.T_pad - 2);
  const uint64_t* mseq = a.mask + (size_t)b * a.Wm * a.T_pad;

  auto issue = [&](int t) {
    const int st = t % kStages;
    if (t < ntp)
      dma_kv_tile<D, kWaves, false>(Kp, Vp, t * kKeyTile, Lc, k_tile(st), v_tile(st), wave, lane);
    else
      dma_kv_tile<D, kWaves, false>(Kt, Vt, (t - ntp) * kKeyTile, T, k_tile(st), v_tile(st),
                                    wave, lane);
    const int word = t < ntp ? t : a.Wp + (t - ntp);
    lds_dma16(opaque_uniform(mseq + (size_t)word * a.T_pad) + moff, mask_words(st, wave));
  };

  // query operands (B of S^T: Q[row][d = 32 ds + 8 grp ..]); padding rows read zeros
  bf16x8 qop[DS];
  {
    const unsigned short* qp = a.q + (((size_t)b * T + node) * G.Hq + head) * D + 8 * grp;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const uint4 v = row_ok ? *(const uint4*)(qp + 32 * ds) : make_uint4(0, 0, 0, 0);
      qop[ds] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the query loads, before any direct load
  for (int t = 0; t < kStages - 1 && t < ntiles; ++t) issue(t);

  const float c = G.scale * kLog2e;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero4;
  float m_run = -INFINITY, l_run = 0.f;
  const int vrow = 4 * grp + (l16 >> 2);
  const int vch = (l16 & 3) >> 1, vhalf = 8 * (l16 & 1);
  const int mslot = node - na;  // < 2 + 16 / G <= 18

  // scores of tile t (raw S^T, before scaling and masking) into sc
  auto scores = [&](int t, f32x4 (&sc)[4]) {
    const unsigned char* Ks = k_tile(t % kStages);
    bf16x8 kop[4][DS];  // all K operand reads first, then the products (one wait)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int kr = kb * 16 + l16;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        kop[kb][ds] = *(const bf16x8*)(Ks + kr * (2 * D) + 16 * ((4 * ds + grp) ^ swz_k<D>(kr)));
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sc[kb] = zero4;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kb][ds], qop[ds], sc[kb], 0, 0, 0);
    }
  };
  // wait until tile t has landed: the tiles issued after it (at most two) may stay in flight
  auto wait_tile = [&](int t, int last_issued) {
    const int after = min(last_issued, ntiles - 1) - t;
    if (after >= 2) wait_and_barrier<2 * kLoadsPerTile>();
    else if (after == 1) wait_and_barrier<kLoadsPerTile>();
    else wait_and_barrier<0>();
  };

  // this wave's quarter of V^T(t): tr reads of the V tile, widened bf16 -> fp16
  auto build_vt = [&](int t) {
    const unsigned char* Vs = v_tile(t % kStages);
    const uint32_t vbase =  // the tile's LDS byte address
        (uint32_t)(size_t)(const __attribute__((address_space(3))) unsigned char*)Vs;
    uint32_t addr[2 * kUnitsPerWave];
#pragma unroll
    for (int j = 0; j < kUnitsPerWave; ++j) {
      const int u = wave * kUnitsPerWave + j, db = u >> 1, h = u & 1;
      const int r0 = 32 * h + vrow, r1 = r0 + 16;
      const int ch = 2 * db + vch;
      addr[2 * j] = vbase + r0 * (2 * D) + 16 * (ch ^ swz_v<D>(r0)) + vhalf;
      addr[2 * j + 1] = vbase + r1 * (2 * D) + 16 * (ch ^ swz_v<D>(r1)) + vhalf;
    }
    i16x4 rd[2 * kUnitsPerWave];
    if constexpr (kUnitsPerWave == 4) tr_read8(rd, addr);
    else tr_read4(rd, addr);
#pragma unroll
    for (int j = 0; j < kUnitsPerWave; ++j) {
      f16x8 vop;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vop[e] = bf16_to_f16(rd[2 * j][e]);
        vop[4 + e] = bf16_to_f16(rd[2 * j + 1][e]);
      }
      const int u = wave * kUnitsPerWave + j;
      *(f16x8*)(s_vt + (u * 64 + lane) * 16) = vop;
    }
  };

  // Software-pipelined by one tile: the scores of tile t+1 enter the matrix core before the
  // softmax and PV product of tile t, so a wave's matrix work and its VALU and LDS work
  // overlap (one wave per SIMD: nothing else would hide them).
  f32x4 sc[4];
  wait_tile(0, kStages - 2);
  scores(0, sc);
  for (int t = 0; t < ntiles; ++t) {
    f32x4 sn[4];
    if (t + 1 < ntiles) {
      // tile t+3 goes to the stage of tile t-1 (its K was read two iterations ago, its V
      // last iteration, before that iteration's closing barrier)
      if (t + kStages - 1 < ntiles) issue(t + kStages - 1);
      wait_tile(t + 1, t + kStages - 1);
      scores(t + 1, sn);
    }
    const int st = t % kStages;
    const bool tree = t >= ntp;
    const int kend = tree ? T - (t - ntp) * kKeyTile : Lc - t * kKeyTile;  // valid keys here
    build_vt(t);
    lds_done_barrier();  // V^T(t) complete (the last reads of the previous one are done)
    // the node's visible keys of this tile (keys past the valid range cleared once), then
    // the lane's four-key nibble of each 16-key block
    uint64_t mw = mask_words(st, wave)[mslot];
    if (kend < 64) mw &= (1ull << kend) - 1;
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint32_t nib = (uint32_t)(mw >> (16 * kb + 4 * grp)) & 0xFu;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = (nib >> i) & 1u ? sc[kb][i] * c : -INFINITY;
        sc[kb][i] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    const float m_new = fmaxf(m_run, group_max(tmax));
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    // rescale only when some row's maximum rose (after the first tiles, rarely)
    if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    m_run = m_new;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f16x8 pop;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(sc[2 * h + e / 4][e % 4] - m_use);
        l_run += p;
        pop[e] = (_Float16)p;
      }
      f16x8 vop[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) vop[db] = *(const f16x8*)(s_vt + ((2 * db + h) * 64 + lane) * 16);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[db], pop, acc[db], 0, 0, 0);
    }
    lds_done_barrier();  // every wave is done with K(t+1) and V(t) before stages are refilled
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sc[kb] = sn[kb];
  }

  const float lt = group_sum(l_run);
  if (!row_ok) return;
  float* outp = a.out + (((size_t)b * T + node) * G.Hq + head) * D + 4 * grp;
  float* lsep = a.lse + ((size_t)b * G.Hq + head) * T + node;
  if (len_bad) {
#pragma unroll
    for (int db = 0; db < DB; ++db) *(f32x4*)(outp + 16 * db) = f32x4{NAN, NAN, NAN, NAN};
    if (grp == 0) *lsep = NAN;
    return;
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;  // a row that sees nothing: out 0, lse -inf
#pragma unroll
  for (int db = 0; db < DB; ++db) *(f32x4*)(outp + 16 * db) = acc[db] * inv;
  if (grp == 0) *lsep = lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
}

// ----------------------------------------------------------------------------- the mask

struct MaskArgs {
  const int32_t* parent;
  const int32_t* prefix_len;
  uint64_t* mask;  // [B, Wm, T_pad]
  int32_t* status;
  int32_t T, Lmax, Wp, Wm, T_pad;
};

__global__ __launch_bounds__(256) void dense_mask(MaskArgs a) {
  __shared__ int32_t par[256];
  __shared__ unsigned char anc[256];
  const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, T = a.T;
  int bad = 0;
  if (tid < T) {
    const int p = a.parent[(size_t)b * T + tid];
    par[tid] = p;
    bad = p < -1 || p >= tid;
    anc[tid] = 0;
  }
  const int L = a.prefix_len[b];
  const bool len_bad = L < 0 || L > a.Lmax;
  const bool tree_bad = __syncthreads_or(bad) != 0;
  if (tid == 0 && !tree_bad)  // a valid chain strictly decreases: the walk ends
    for (int p = i; p >= 0; p = par[p]) anc[p] = 1;
  if (tid == 0 && i == 0 && a.status)
    a.status[b] = (tree_bad ? kStatusTree : 0) | (len_bad ? kStatusPrefixLen : 0);
  __syncthreads();
  // node i's words are column i of the sequence's [Wm, T_pad] block; the last node also
  // clears the padding column
  uint64_t* col = a.mask + (size_t)b * a.Wm * a.T_pad + i;
  const bool pad = i == T - 1 && a.T_pad > T;
  for (int w = tid; w < a.Wm; w += 256) {
    uint64_t v = 0;
    if (!tree_bad && !len_bad) {
      if (w < a.Wp) {
        const int lo = 64 * w, n = L - lo;  // prefix keys lo .. lo+63 below L
        v = n >= 64 ? ~0ull : (n <= 0 ? 0ull : ((1ull << n) - 1));
      } else {
        const int t0 = 64 * (w - a.Wp);
        for (int k = 0; k < 64 && t0 + k < T; ++k) v |= (uint64_t)anc[t0 + k] << k;
      }
    }
    col[(size_t)w * a.T_pad] = v;
    if (pad) col[(size_t)w * a.T_pad + 1] = 0;
  }
}

}  // namespace

void dense_mask_words(const Geometry& g, int32_t* wp, int32_t* wm, int32_t* t_pad) {
  *wp = (g.Lmax + 63) / 64;
  *wm = *wp + (g.T + 63) / 64;
  *t_pad = g.T + (g.T & 1);
}

hipError_t launch_dense_mask(const Geometry& g, const int32_t* parent_idx,
                             const int32_t* prefix_len, uint64_t* mask, int32_t* status,
                             hipStream_t stream) {
  MaskArgs a;
  a.parent = parent_idx;
  a.prefix_len = prefix_len;
  a.mask = mask;
  a.status = status;
  a.T = g.T;
  a.Lmax = g.Lmax;
  dense_mask_words(g, &a.Wp, &a.Wm, &a.T_pad);
  hipLaunchKernelGGL(dense_mask, dim3(g.T, g.B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dense_masked(const Geometry& g, const void* q, const void* k_prefix,
                               const void* v_prefix, const void* k_tree, const void* v_tree,
                               const uint64_t* mask, const int32_t* prefix_len, float* out,
                               float* lse, hipStream_t stream) {
  DenseArgs a;
  a.q = (const unsigned short*)q;
  a.k_prefix = (const unsigned short*)k_prefix;
  a.v_prefix = (const unsigned short*)v_prefix;
  a.k_tree = (const unsigned short*)k_tree;
  a.v_tree = (const unsigned short*)v_tree;
  a.mask = mask;
  a.prefix_len = prefix_len;
  a.out = out;
  a.lse = lse;
  a.g = g;
  dense_mask_words(g, &a.Wp, &a.Wm, &a.T_pad);
  dim3 grid((g.NT + kWaves - 1) / kWaves, g.Hkv, g.B);
  if (g.D == 128)
    hipLaunchKernelGGL(dense_masked<128>, grid, dim3(kThreads), 0, stream, a);
  else if (g.D == 64)
    hipLaunchKernelGGL(dense_masked<64>, grid, dim3(kThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hta
