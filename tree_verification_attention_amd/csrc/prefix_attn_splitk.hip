// prefix_attn_splitk.hip -- the prefix pass of tree verification attention on gfx950.
//
// Every tree query attends to its sequence's whole prefix KV cache with no mask (LongSpec
// paper summary, Summary, "Hybrid Tree Attention": the long-context pass over the prefix;
// README, Introduction: fast prefix computation).  The prefix is split into chunks of
// `chunk` keys (split-K, as in Flash-Decoding, the baseline of the summary's Key points);
// each workgroup produces, for one (sequence b, KV head g, chunk s, row block), the
// normalised partial output and log-sum-exp of the query rows that read KV head g.
// lse_merge combines the chunks.
//
// MI355X mapping
//  * GQA packing: the T*G query rows sharing KV head g (row r = node*G + head-in-group) are
//    processed together, so each K/V byte leaves HBM once per chunk and feeds 4*T*G flops.
//  * Matrix cores: scores are formed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16;
//    A = 16 keys x 32 dims from LDS, B = 16 query rows kept in registers), and the output
//    transposed too, O^T += V^T P^T (v_mfma_f32_16x16x32_f16).  With both products
//    transposed, the lane holding score column "row" of S^T is the lane holding operand
//    column "row" of P^T and output column "row" of O^T: the softmax needs no data movement
//    between the products and its rescale factors are lane-local.  V^T operands come from
//    V kept row-major in LDS through the transposing read ds_read_b64_tr_b16.
//  * Load balance: the row tiles of a block are dealt to the four waves (one per SIMD);
//    when their count is not a multiple of four, the leftover tiles are split over the
//    waves by key sub-blocks instead, and the waves' partial results for them are merged
//    through LDS at the end, so every SIMD does the same matrix work.
//  * Memory: K and V tiles of 64 keys stream HBM -> LDS with direct LDS loads
//    (global_load_lds_dwordx4, no register staging) through a 4-stage ring, three tiles in
//    flight while one is consumed; rows are stored unpadded with an XOR swizzle of their
//    16-byte chunks so the operand reads and the transposing reads are conflict-free.  Keys
//    past the chunk end re-read the last valid key (never the padding) and are masked.
//  * Softmax in fp32 with exp2 (scale*log2(e) folded into one FMA).  The running maximum is
//    only raised when some score exceeds it by more than 2^8 (a wave-wide ballot), so the
//    accumulator rescale and the cross-lane maximum leave the common path; the result is
//    exact either way, since numerator and normaliser share the reference.  Probabilities
//    enter the PV product as fp16 (nearest-even, 11 significant bits), V is widened from
//    bf16 to fp16 in registers (exact for |v| in [2^-14, 65504]), and the normaliser sums
//    the unrounded fp32 probabilities.
#include "hta_internal.h"

namespace hta {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kKeyTile = 64;
constexpr int kStages = 4;
constexpr float kRescaleSlack = 8.f;  // log2 units: probabilities stay below 2^8

template <int D>
struct Layout {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                          // 16-byte chunks per row
  static constexpr int kTileBytes = kKeyTile * kRowBytes;        // one K or V tile
  static constexpr int kStageBytes = 2 * kTileBytes;
  static constexpr int kDmaPerWave = kTileBytes / (kWaves * 1024);  // per tensor per tile
};

// XOR swizzles of the 16-byte chunk index within a row: K rows are read 16 at a time at
// one chunk column (D = 128: chunk ^ row%16 spreads the 16 rows over all 64 banks), V rows
// 4 at a time over two chunk columns by the transposing read (chunk ^ 2*(row%8) keeps the
// 4 rows x 2 chunks of one 16-lane block on distinct banks).
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? 2 * (row & 7) : 2 * (row & 3);
}

// One 16-byte-per-lane direct load from global memory into LDS: lane l's 16 bytes land at
// lds + 16 l (global_load_lds_dwordx4).  The builtin only exists for the device; the host
// pass parses this body without generating it.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
#endif
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ i16x4 tr_read_b64(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

__device__ __forceinline__ _Float16 bf16_bits_to_f16(short h) {
  return (_Float16)__builtin_bit_cast(float, (uint32_t)(unsigned short)h << 16);
}

// lanes l, l^16, l^32, l^48 hold the same query row (four key groups)
__device__ __forceinline__ float group_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Wait until at most N of this wave's vector-memory operations are outstanding (the LDS
// direct loads of later tiles), then barrier.  The LDS reads issued before are drained
// too, so a stage may be refilled right after the barrier.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
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
  int32_t tiles_per_block;         // row tiles per block (MT * 4 + leftover)
  int32_t leftover;                // tiles_per_block - 4 * MT, 0..3
  float c;                         // scale * log2(e)
};

template <int D, int MT, int NL>
__global__ __launch_bounds__(kThreads, 1) void prefix_attn_splitk(PrefixArgs a) {
  using Y = Layout<D>;
  constexpr int DS = D / 32;  // 32-wide d steps of the score product
  constexpr int DB = D / 16;  // 16-wide d blocks of the output
  constexpr int DPW = Y::kDmaPerWave;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kStages * Y::kStageBytes];

  const Geometry& G = a.g;
  const int s = blockIdx.x;
  const int kv = blockIdx.y / a.row_blocks;
  const int rb = blockIdx.y % a.row_blocks;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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

  // ---- stream K/V tiles into the LDS ring
  auto issue = [&](int t) {
    unsigned char* st = lds + (t % kStages) * Y::kStageBytes;
    const int key0 = kbeg + t * kKeyTile;
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      const int blk = j * kWaves + wave;  // 1 KB block of the tile written by this wave
      const int u = 64 * blk + lane;      // 16-byte chunk position within the tile
      const int r = u / Y::kChunks, p = u % Y::kChunks;
      const size_t gk = (size_t)min(key0 + r, kend - 1);
      lds_dma16(Kg + gk * D + 8 * (p ^ swz_k<D>(r)), st + 1024 * blk);
      lds_dma16(Vg + gk * D + 8 * (p ^ swz_v<D>(r)), st + Y::kTileBytes + 1024 * blk);
    }
  };

  // ---- row tiles of this wave; query operand (B of S^T): Q[row = l16][d = 32 ds + 8 grp ..]
  const int t0 = rb * a.tiles_per_block;
  const int t_end = min(t0 + a.tiles_per_block, G.NT);
  auto load_q = [&](int tile, bf16x8* dst) {
    const int row = tile * 16 + l16;
    const bool ok = tile < t_end && row < G.R;
    const int node = ok ? row / G.G : 0;
    const int head = kv * G.G + (ok ? row % G.G : 0);
    const unsigned short* qp = a.q + (((size_t)b * G.T + node) * G.Hq + head) * D + 8 * grp;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      dst[ds] = as_bf16x8(ok ? *(const uint4*)(qp + 32 * ds) : make_uint4(0, 0, 0, 0));
  };
  constexpr int MTA = MT > 0 ? MT : 1;
  bf16x8 qop[MTA][DS];
#pragma unroll
  for (int k = 0; k < MT; ++k) load_q(t0 + kWaves * k + wave, qop[k]);
  // The query operands live in AGPRs for the whole kernel (MFMA reads its B operand from
  // AGPRs), leaving the VGPR file to scores, probabilities and operand staging.
#pragma unroll
  for (int k = 0; k < MT; ++k)
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) asm volatile("" : "+a"(qop[k][ds]));

  // Leftover tile (NL = 1 or 2 of them): shared by 4/NL waves; each computes its scores in
  // full but only LDB of the DB output d-blocks, starting at ldb0.
  constexpr int LDB = NL > 0 ? DB * NL / kWaves : 1;
  const int ltile = t0 + kWaves * MT + (NL == 2 ? (wave >> 1) : 0);
  const int ldb0 = NL > 0 ? (wave % (kWaves / (NL > 0 ? NL : 1))) * LDB : 0;
  bf16x8 qopl[DS];
  if (NL > 0) {
    load_q(ltile, qopl);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) asm volatile("" : "+a"(qopl[ds]));
  }

  const int npre = min(kStages - 1, ntiles);
  for (int t = 0; t < npre; ++t) issue(t);

  f32x4 acc[MTA][DB];
  f32x4 accl[LDB];
  float m_run[MTA], l_run[MTA], m_l = -INFINITY, l_l = 0.f;
#pragma unroll
  for (int k = 0; k < MT; ++k) {
    m_run[k] = -INFINITY;
    l_run[k] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[k][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int j = 0; j < LDB; ++j) accl[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int vr = lane & 15;  // lane within its 16-lane block, for the transposing reads
  const int vrow = 4 * grp + (vr >> 2);
  const int vch = (vr & 3) >> 1, vhalf = 8 * (vr & 1);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int t = 0; t < ntiles; ++t) {
    const int after = min(kStages - 2, ntiles - 1 - t);  // tiles issued after t
    if (after >= 2) wait_and_barrier<4 * DPW>();
    else if (after == 1) wait_and_barrier<2 * DPW>();
    else wait_and_barrier<0>();
    if (t + kStages - 1 < ntiles) issue(t + kStages - 1);  // refills the stage of tile t-1

    const unsigned char* Ks = lds + (t % kStages) * Y::kStageBytes;
    const unsigned char* Vs = Ks + Y::kTileBytes;
    const int key0 = kbeg + t * kKeyTile;
    const bool partial = key0 + kKeyTile > kend;

    // Two halves of 32 keys: half h covers key blocks 2h, 2h+1 (scores) and feeds the PV
    // product's k-step h.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // ---- scores S^T[key][row]: this lane holds row l16, keys 32 h + 16 j + 4 grp + r
      f32x4 sc[MTA][2];
      f32x4 scl[2];
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int row = 32 * h + 16 * j + l16;
          const bf16x8 kop = *(const bf16x8*)(Ks + row * Y::kRowBytes +
                                              16 * ((4 * ds + grp) ^ swz_k<D>(row)));
#pragma unroll
          for (int k = 0; k < MT; ++k)
            sc[k][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[k][ds],
                                                               ds ? sc[k][j] : zero4, 0, 0, 0);
          if (NL > 0)
            scl[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qopl[ds], ds ? scl[j] : zero4,
                                                             0, 0, 0);
        }
      }

      // ---- keys past the chunk end (last tile only)
      if (partial) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (key0 + 32 * h + 16 * j + 4 * grp + r >= kend) {
#pragma unroll
              for (int k = 0; k < MT; ++k) sc[k][j][r] = -INFINITY;
              if (NL > 0) scl[j][r] = -INFINITY;
            }
      }

      // ---- online softmax with a lazily raised reference maximum
      float lmax[MTA], lmaxl = -INFINITY;
      bool need = false;
#pragma unroll
      for (int k = 0; k < MT; ++k) {
        const float m0 = fmaxf(fmaxf(sc[k][0][0], sc[k][0][1]), fmaxf(sc[k][0][2], sc[k][0][3]));
        const float m1 = fmaxf(fmaxf(sc[k][1][0], sc[k][1][1]), fmaxf(sc[k][1][2], sc[k][1][3]));
        lmax[k] = fmaxf(m0, m1) * a.c;
        need |= lmax[k] > m_run[k] + kRescaleSlack;
      }
      if (NL > 0) {
        const float m0 = fmaxf(fmaxf(scl[0][0], scl[0][1]), fmaxf(scl[0][2], scl[0][3]));
        const float m1 = fmaxf(fmaxf(scl[1][0], scl[1][1]), fmaxf(scl[1][2], scl[1][3]));
        lmaxl = fmaxf(m0, m1) * a.c;
        need |= lmaxl > m_l + kRescaleSlack;
      }
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
        for (int k = 0; k < MT; ++k) {
          const float m_new = fmaxf(m_run[k], group_max(lmax[k]));
          const float alpha = __builtin_amdgcn_exp2f(m_run[k] - m_new);
          m_run[k] = m_new;
          l_run[k] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[k][db] *= alpha;
        }
        if (NL > 0) {
          const float m_new = fmaxf(m_l, group_max(lmaxl));
          const float alpha = __builtin_amdgcn_exp2f(m_l - m_new);
          m_l = m_new;
          l_l *= alpha;
#pragma unroll
          for (int j = 0; j < LDB; ++j) accl[j] *= alpha;
        }
      }

      // P^T operand of k-step h: element e <-> key 32 h + 16 (e / 4) + 4 grp + (e % 4)
      f16x8 pop[MTA];
      f16x8 popl;
#pragma unroll
      for (int k = 0; k < MT; ++k) {
        float ls = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[k][e / 4][e % 4], a.c, -m_run[k]));
          ls += p;
          pop[k][e] = (_Float16)p;
        }
        l_run[k] += ls;
      }
      if (NL > 0) {
        float ls = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(scl[e / 4][e % 4], a.c, -m_l));
          ls += p;
          popl[e] = (_Float16)p;
        }
        l_l += ls;
      }

      // ---- O^T[d][row] += V^T[d][key] P^T[key][row]  (keys 32 h .. 32 h + 31)
      auto v_operand = [&](int db) {
        const int r0 = 32 * h + vrow, r1 = r0 + 16;
        const int c = 2 * db + vch;
        const i16x4 lo = tr_read_b64(Vs + r0 * Y::kRowBytes + 16 * (c ^ swz_v<D>(r0)) + vhalf);
        const i16x4 hi = tr_read_b64(Vs + r1 * Y::kRowBytes + 16 * (c ^ swz_v<D>(r1)) + vhalf);
        f16x8 vop;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vop[e] = bf16_bits_to_f16(lo[e]);
          vop[4 + e] = bf16_bits_to_f16(hi[e]);
        }
        return vop;
      };
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f16x8 vop = v_operand(db);
#pragma unroll
        for (int k = 0; k < MT; ++k)
          acc[k][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop[k], acc[k][db], 0, 0, 0);
      }
      if (NL > 0) {
#pragma unroll
        for (int j = 0; j < LDB; ++j)
          accl[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v_operand(ldb0 + j), popl, accl[j], 0,
                                                           0, 0);
      }
    }
  }

  // ---- normalise and write this chunk's partial
  const size_t slot = ((size_t)b * G.Hkv + kv) * (G.S + 1) + s;
#pragma unroll
  for (int k = 0; k < MT; ++k) {
    const int tile = t0 + kWaves * k + wave;
    const float lt = group_sum(l_run[k]);
    if (tile >= t_end) continue;
    const int row = tile * 16 + l16;
    const float inv = 1.f / lt;
    float* op = a.o_part + (slot * G.R_pad + row) * D + 4 * grp;
#pragma unroll
    for (int db = 0; db < DB; ++db) *(f32x4*)(op + 16 * db) = acc[k][db] * inv;
    if (grp == 0) a.lse_part[slot * G.R_pad + row] = (m_run[k] + __log2f(lt)) * kLn2;
  }
  if (NL > 0) {
    const float lt = group_sum(l_l);
    if (ltile < t_end) {
      const int row = ltile * 16 + l16;
      const float inv = 1.f / lt;
      float* op = a.o_part + (slot * G.R_pad + row) * D + 4 * grp;
#pragma unroll
      for (int j = 0; j < LDB; ++j) *(f32x4*)(op + 16 * (ldb0 + j)) = accl[j] * inv;
      if (grp == 0 && ldb0 == 0) a.lse_part[slot * G.R_pad + row] = (m_l + __log2f(lt)) * kLn2;
    }
  }
}

template <int D, int MT, int NL>
hipError_t launch_cfg(const PrefixArgs& a, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((prefix_attn_splitk<D, MT, NL>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, int MT>
hipError_t launch_mt(const PrefixArgs& a, dim3 grid, hipStream_t stream) {
  switch (a.leftover) {
    case 0: return launch_cfg<D, MT, 0>(a, grid, stream);
    case 1: return launch_cfg<D, MT, 1>(a, grid, stream);
    case 2: return launch_cfg<D, MT, 2>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_d(const PrefixArgs& a, int mt, dim3 grid, hipStream_t stream) {
  switch (mt) {
    case 0: return launch_mt<D, 0>(a, grid, stream);
    case 1: return launch_mt<D, 1>(a, grid, stream);
    case 2: return launch_mt<D, 2>(a, grid, stream);
    case 3: return launch_mt<D, 3>(a, grid, stream);
    case 4: return launch_mt<D, 4>(a, grid, stream);
    case 5: return launch_mt<D, 5>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Row blocking: a workgroup covers up to 18 row tiles (288 query rows): 4 full tiles per
// wave plus up to two shared leftover tiles.  A remainder of three tiles becomes one more
// full slot per wave (the fourth wave's slot is empty).  More rows are split into equal
// row blocks.
void prefix_row_blocking(const Geometry& g, int* mt, int* tiles_per_block, int* blocks) {
  const int max_tiles = 4 * 4 + 2;
  const int nb = (g.NT + max_tiles - 1) / max_tiles;
  const int tpb = (g.NT + nb - 1) / nb;
  *blocks = (g.NT + tpb - 1) / tpb;
  *tiles_per_block = tpb;
  *mt = tpb % 4 == 3 ? tpb / 4 + 1 : tpb / 4;
}

hipError_t launch_prefix_attn_splitk(const Geometry& g, const void* q, const void* k_prefix,
                                     const void* v_prefix, const int32_t* prefix_len,
                                     const Workspace& ws, hipStream_t stream) {
  PrefixArgs a;
  a.q = (const unsigned short*)q;
  a.k_prefix = (const unsigned short*)k_prefix;
  a.v_prefix = (const unsigned short*)v_prefix;
  a.prefix_len = prefix_len;
  a.lse_part = ws.lse_part;
  a.o_part = ws.o_part;
  a.g = g;
  int mt, tpb, nb;
  prefix_row_blocking(g, &mt, &tpb, &nb);
  a.row_blocks = nb;
  a.tiles_per_block = tpb;
  a.leftover = tpb % 4 == 3 ? 0 : tpb - 4 * mt;
  a.c = g.scale * kLog2e;
  dim3 grid(g.S, g.Hkv * nb, g.B);
  if (g.D == 128) return launch_d<128>(a, mt, grid, stream);
  if (g.D == 64) return launch_d<64>(a, mt, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace hta
