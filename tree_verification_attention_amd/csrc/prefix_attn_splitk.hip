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
//    processed by one workgroup, so each K/V byte leaves HBM once per chunk and feeds
//    4*T*G flops.
//  * Matrix cores: scores are formed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16;
//    A = 16 keys x 32 dims from LDS, B = 16 query rows kept in registers), and the output
//    transposed too, O^T += V^T P^T (v_mfma_f32_16x16x32_f16).  With both products
//    transposed, the lane holding score column "row" of S^T is the lane holding operand
//    column "row" of P^T and output column "row" of O^T: the softmax needs no data movement
//    between the products and its rescale factors are lane-local.
//  * Two waves per SIMD (8 per workgroup), in two groups (waves 0-3 and 4-7, one of each
//    per SIMD).  A wave's own VALU work overlaps its matrix-core work poorly, but the VALU
//    work of one wave overlaps the MFMAs of the other, so the two groups alternate between
//    matrix-core phases and softmax phases half a phase pair apart (see run_chunk).  Each
//    first-group wave holds MT row tiles, each second-group wave MTB <= MT (fewer when the
//    block's tiles do not fill both groups: the matrix core of a SIMD is shared by its two
//    waves, so padding tiles would cost real products).  Leftover tiles go to the first
//    group, split by keys: each of its waves covers some 16-key blocks of every tile for
//    all D output dims, and the waves' partials are combined at the end.  The first group
//    also issues the tile loads; the second builds V^T.
//  * Memory: K and V tiles of 64 keys stream HBM -> LDS with direct LDS loads
//    (global_load_lds_dwordx4, no register staging), two to three tiles in flight while
//    one is consumed.  Rows land unpadded with an XOR swizzle of their 16-byte chunks so
//    operand reads are bank-conflict-free.  Keys past the chunk end re-read the last valid
//    key (never the padding) and are masked.
//  * V^T operand: once per tile the second group turns the landed bf16 V tile into an fp16
//    V^T tile (transposing reads ds_read_b64_tr_b16, widening in registers, one 16-byte
//    store per lane) laid out in the exact key order of the P^T operand, so the PV product
//    reads plain conflict-free 16-byte operands.  This runs one tile ahead of the compute.
//  * Softmax in fp32 with exp2 (scale*log2(e) folded into one FMA) against a per-row
//    reference: the maximum of the chunk's first 32 keys, raised only when a probability
//    of a 32-key half would exceed 2^15 (a wave-wide ballot), so the accumulator
//    rescale leaves the common path; the result is exact either way, since numerator and
//    normaliser share the reference.  Probabilities enter the PV product as fp16
//    (nearest-even, 11 significant bits, at most 2^15), V is widened from bf16 to fp16
//    (exact for |v| in [2^-14, 65504]), and the normaliser adds those same rounded
//    probabilities in fp32 on the matrix core (the PV product with a block of ones in place
//    of V^T, one more product per row tile and 32 keys, off the VALU): numerator and
//    normaliser weight every key alike, so a key that dominates its row comes out exact.
#include "hta_internal.h"
#include "lds_tiles.h"

#include <type_traits>

namespace hta {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kKStages = 4;  // K ring: tile t (scores), t+1 (landed), t+2, t+3 (in flight)
constexpr int kVStages = 3;  // V ring: tile t+1 (being transposed), t+2, t+3 (in flight)
constexpr int kVtStages = 3;  // V^T: tiles t-1 (PV of its last half), t, t+1 (being made)
// instruction classes of the scheduling hints (__builtin_amdgcn_sched_group_barrier masks)
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr float kRaiseLog2 = 15.f;  // probabilities stay at most 2^15 (fp16 max 65504)

template <int D>
struct Layout {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                             // 16-byte chunks per row
  static constexpr int kTileBytes = kKeyTile * kRowBytes;           // one K, V or V^T tile
  // the first wave group (4 waves) issues the tile loads
  static constexpr int kDmaPerWave = kTileBytes / (4 * 1024);  // per tensor per tile
  static constexpr int kKRing = 0;
  static constexpr int kVRing = kKStages * kTileBytes;
  static constexpr int kVt = kVRing + kVStages * kTileBytes;
  static constexpr int kBytes = kVt + kVtStages * kTileBytes;
};

// V^T rows (one per d, 64 keys fp16 = 8 chunks) are read 16 at a time at one chunk column:
// chunk ^ (row/2)%8 (rows 2m and 2m+1 sit in opposite bank halves).
__device__ __forceinline__ int swz_vt(int d) { return (d >> 1) & 7; }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ i16x4 tr_read_b64(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// The A operand of the row-sum product: a 16 x 32 block of ones, so O^T = ones P^T holds in
// every one of its 16 rows the sum over the 32 keys of each query row's fp16 probabilities.
__device__ __forceinline__ f16x8 ones_f16x8() {
  f16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (_Float16)1.f;
  return v;
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
// direct loads of later tiles), then barrier.  The LDS accesses issued before are drained
// too, so a buffer may be refilled right after the barrier.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// The split-K partials leave through agent-scope stores (sc1): the merge reads them in the
// next launch, possibly on other XCDs, whose L2s are not coherent with this one, so the
// stores write through this XCD's L2 instead of waiting in it for the end-of-launch
// write-back.  Raw buffer stores on a per-workgroup resource (dword 3 below: untyped dword
// access on CDNA3/CDNA4); bytes past num_records are dropped, never written.
constexpr int kBufWord3 = 0x00020000;
constexpr int kAgentScope = 16;  // the sc1 cache-policy bit
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
__device__ __forceinline__ void store_agent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, byte_off, 0, kAgentScope);
}
__device__ __forceinline__ void store_agent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, r, byte_off, 0, kAgentScope);
}

struct PrefixArgs {
  const unsigned short* q;         // bf16 bits [B, T, Hq, D]
  const unsigned short* k_prefix;  // [B, Hkv, Lmax, D]
  const unsigned short* v_prefix;
  const int32_t* prefix_len;       // [B]
  int32_t* status_reset;           // [B] or nullptr: cleared by the first workgroup of b
  float* lse_part;
  float* o_scale;                  // the factor of each o_part row
  uint32_t* o_part;                // 16-bit rows (pack16x4)
  Geometry g;
  int32_t row_blocks;              // query-row blocks per (b, kv head)
  int32_t tiles_per_block;         // row tiles per block
  float c;                         // scale * log2(e)
};

// What one call of the pass lambdas does: leftover keys (value) and the row tiles the
// calling wave owns (rows).
template <bool WL, int ROWS>
struct PassTag {
  static constexpr bool value = WL;
  static constexpr int rows = ROWS;
};

// MT full row tiles per first-group wave, MTB (0, 1 or MT) per second-group wave; NL
// leftover tiles (0..2) per block, split over the first wave group by keys.  Block tiles
// t0 .. t0 + 4 MT - 1 belong to the first group, the next 4 MTB to the second, then the
// leftover tiles.  MTB < MT keeps padding rows off the SIMDs (with MTB = 0 the second group
// only builds V^T).
template <int D, int MT, int NL, int MTB>
__global__ __launch_bounds__(kThreads, 1) void prefix_attn_splitk(PrefixArgs a) {
  using Y = Layout<D>;
  constexpr int DS = D / 32;  // 32-wide d steps of the score product
  constexpr int DB = D / 16;  // 16-wide d blocks of the output
  constexpr int DPW = Y::kDmaPerWave;
  constexpr int P = 2 * DPW;  // direct loads per first-group wave per tile (K and V)
  constexpr int MTA = MT > 0 ? MT : 1;
  static_assert(MTB == 0 || MTB == 1 || MTB == MT, "second-group tiles: 0, 1 or MT");
  constexpr bool LEFT = NL > 0;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[Y::kBytes];

  const Geometry& G = a.g;
  // Workgroups are dealt to the 8 XCDs round-robin in launch order.  When the grid divides
  // evenly, launch index L runs unit (L % 8) * (N / 8) + L / 8, so the consecutive units of one
  // (sequence, KV head) -- all its splits -- share an XCD and its L2 (their queries are read
  // once per XCD).  The mapping is a permutation of the units; otherwise it is the identity.
  int u = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  {
    const int n = gridDim.x * gridDim.y * gridDim.z;
    if (n % 8 == 0) u = (u % 8) * (n / 8) + u / 8;
  }
  // (wave-uniform; readfirstlane keeps them, and the K/V addresses derived from them, in
  // scalar registers, so each direct load is a scalar base plus one lane offset)
  const int s = __builtin_amdgcn_readfirstlane(u % gridDim.x);
  const int kv = __builtin_amdgcn_readfirstlane((u / gridDim.x) % gridDim.y / a.row_blocks);
  const int rb = __builtin_amdgcn_readfirstlane((u / gridDim.x) % gridDim.y % a.row_blocks);
  const int b = __builtin_amdgcn_readfirstlane(u / (gridDim.x * gridDim.y));
  const int lane = threadIdx.x & 63;
  // wave-uniform by construction; readfirstlane lets the compiler see it (scalar branches)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wg = wave >> 2;  // wave group (one wave of each group per SIMD)
  const int ww = wave & 3;   // wave within its group
  const int l16 = lane & 15;
  const int grp = lane >> 4;

  const int kbeg = s * G.chunk;
  // set once the prefix length is known
  int kend = kbeg + 2 * kKeyTile, ntiles = 0;

  const size_t kv_base = ((size_t)b * G.Hkv + kv) * (size_t)G.Lmax * D;
  const unsigned short* Kg = a.k_prefix + kv_base;
  const unsigned short* Vg = a.v_prefix + kv_base;

  // ---- query operands (B of S^T): Q[row = l16][d = 32 ds + 8 grp ..], kept in registers
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
  auto full_tile = [&](int k) { return t0 + wg * (kWaves / 2) * MT + 4 * k + ww; };
  bf16x8 qop[MTA][DS];

  // Leftover tiles (first wave group only), split by keys.  NL = 1: one tile; wave ww takes
  // the 16-key block ww of every 64-key tile (half ww/2, block ww%2).  NL = 2: tile ww/2;
  // wave ww takes the 32-key half ww%2.  Each wave keeps its own running softmax over its
  // keys and accumulates all D output dimensions; the waves' partials are combined through
  // LDS at the end.  The leftover products reuse the K and V^T operands the wave already
  // reads for its own rows, and the leftover scores are never computed twice.
  constexpr int LKB = NL == 2 ? 2 : 1;  // 16-key blocks per tile per wave
  const bool has_left = LEFT && wg == 0;
  const int ltile = t0 + 4 * (MT + MTB) + (NL == 2 ? (ww >> 1) : 0);
  const int lh = NL == 2 ? (ww & 1) : (ww >> 1);  // the wave's leftover half
  const int ljj = NL == 2 ? 0 : (ww & 1);         // its first 16-key block in that half
  bf16x8 qopl[DS];

  // ---- stream K/V tiles into the LDS rings
  auto issue = [&](int t) {
    // (each K/V byte is read once per pass: non-temporal loads)
    dma_kv_tile<D, 4, false, kLoadStream>(Kg, Vg, kbeg + t * kKeyTile, kend,
                      lds + Y::kKRing + (t % kKStages) * Y::kTileBytes,
                      lds + Y::kVRing + (t % kVStages) * Y::kTileBytes, ww, lane);
  };

  // ---- before the prefix length is known: the query operands of this wave's row tiles, and
  // (first group) tiles 0 and 1 of the chunk as whole tiles, when they lie inside the
  // cache's allocation.  They are checked against the length once it arrives.
  if (wg == 0) {
#pragma unroll
    for (int k = 0; k < MT; ++k) load_q(full_tile(k), qop[k]);
    if constexpr (LEFT) load_q(ltile, qopl);
  } else {
#pragma unroll
    for (int k = 0; k < MTB; ++k) load_q(full_tile(k), qop[k]);
  }
  const bool early = G.chunk >= 2 * kKeyTile && kbeg + 2 * kKeyTile <= G.Lmax;
  if (early && wg == 0) {
    issue(0);
    issue(1);
  }
  // The prefix length is read only now, by a scalar load (b is wave-uniform), so neither
  // its round trip nor the wait for it delays the loads above, which do not depend on it
  // (the compiler barrier keeps them in front).
  asm volatile("" ::: "memory");
  // (the status reset goes behind the loads: the wave that stores it would otherwise wait for
  // the store before issuing them)
  if (a.status_reset && s == 0 && kv == 0 && rb == 0 && threadIdx.x == 0) a.status_reset[b] = 0;
  const int Lraw = *(const __attribute__((address_space(4))) int32_t*)(a.prefix_len + b);
  int Lb = Lraw < 0 ? 0 : (Lraw > G.Lmax ? G.Lmax : Lraw);  // bad lengths are flagged elsewhere
  if (kbeg >= Lb) {  // empty chunk: the merge never reads this slot
    // (no direct load may land in LDS after the workgroup ends)
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
    return;
  }
  kend = min(kbeg + G.chunk, Lb);
  ntiles = (kend - kbeg + kKeyTile - 1) / kKeyTile;
  if (early && wg == 0 && kend < kbeg + 2 * kKeyTile) {
    // the early tiles reach past the prefix end (whose rows are never read): once they have
    // landed, load them again with the rows past the end replaced
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
    for (int t = 0; t < 2 && t < ntiles; ++t) issue(t);
  }

  // ---- V (bf16, keys x d) -> V^T (fp16, d x keys in P^T operand order).  Lane (grp, l16)
  // of (d block db, 32-key half ks) produces d = 16 db + l16, keys 32 ks + 16 (e/4) +
  // 4 grp + e%4 for e = 0..7: one 16-byte chunk, position 4 ks + grp of row d.
  const int vr = lane & 15;
  const int vrow = 4 * grp + (vr >> 2);
  const int vch = (vr & 3) >> 1, vhalf = 8 * (vr & 1);
  // Byte offset of tile t's slot in a ring, as one wave-uniform value: the compiler would
  // otherwise split the modulo into parts it adds to every lane address separately.
  auto ring_slot = [&](int base, int t, int stages) -> uint32_t {
    return __builtin_amdgcn_readfirstlane(base + (t % stages) * Y::kTileBytes);
  };
  // Lane offsets (loop-invariant).  Every swizzle below depends on the lane only, so the
  // ring slot is the one per-tile term and the remaining terms are immediate offsets.
  constexpr int kUnits = 2 * DB / 4;  // (d block, half) units per second-group wave
  static_assert(kUnits % 2 == 0, "units are read in pairs");
  uint32_t tr_src[kUnits];  // row r0 = 32 ks + vrow of unit i (row r0 + 16 is +16 rows)
#pragma unroll
  for (int i = 0; i < kUnits; ++i) {
    const int pr = ww + 4 * i;
    const int db = pr >> 1, ks = pr & 1;
    const int r0 = 32 * ks + vrow;
    tr_src[i] = r0 * Y::kRowBytes + 16 * ((2 * db + vch) ^ swz_v<D>(r0)) + vhalf;
  }
  // V^T row d = 16 db + l16: the chunk swizzle depends on l16 only
  const uint32_t tr_dst = l16 * (kKeyTile * 2) + 16 * ((4 * (ww & 1) + grp) ^ swz_vt(l16));
  // K operand rows 32 h + 16 j + l16 at chunk 4 ds + grp: the K swizzle has period 16 rows,
  // so it depends on l16 only
  uint32_t k_lane[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds)
    k_lane[ds] = l16 * Y::kRowBytes + 16 * ((4 * ds + grp) ^ swz_k<D>(l16));
  // V^T operand rows d = 16 db + l16 at chunk 4 h + grp (swizzle of l16 only)
  const uint32_t vt_lane[2] = {(uint32_t)(l16 * (kKeyTile * 2) + 16 * ((0 + grp) ^ swz_vt(l16))),
                               (uint32_t)(l16 * (kKeyTile * 2) + 16 * ((4 + grp) ^ swz_vt(l16)))};
  auto transpose_v = [&](int t) {
    const unsigned char* vs = lds + ring_slot(Y::kVRing, t, kVStages);
    unsigned char* vt = lds + ring_slot(Y::kVt, t, kVtStages);
#pragma unroll
    for (int i = 0; i < kUnits; i += 2) {
      // (the compiler drains this wave's direct loads before a transposing read; the second
      // group issues none, so that wait is free here)
      i16x4 r[4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        r[2 * u] = tr_read_b64(vs + tr_src[i + u]);
        r[2 * u + 1] = tr_read_b64(vs + tr_src[i + u] + 16 * Y::kRowBytes);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int db = (ww + 4 * (i + u)) >> 1;
        f16x8 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[e] = bf16_bits_to_f16(r[2 * u][e]);
          h[4 + e] = bf16_bits_to_f16(r[2 * u + 1][e]);
        }
        *(f16x8*)(vt + tr_dst + db * 16 * (kKeyTile * 2)) = h;
      }
    }
  };

  // barrier once at most `n` tiles of this wave's direct loads are still outstanding
  // (only first-group waves have direct loads in flight; the others just meet the barrier)
  auto wait_tiles_and_barrier = [&](int n) {
    if (wg != 0) wait_and_barrier<0>();
    else if (n >= 2) wait_and_barrier<2 * P>();
    else if (n == 1) wait_and_barrier<P>();
    else wait_and_barrier<0>();
  };

  f32x4 acc[MTA][DB];
  f32x4 accl[LEFT ? DB : 1];
  // running row sums (normalisers), accumulated by the row-sum product: every element of
  // lsum[k] holds the sum for this lane's query row
  f32x4 lsum[MTA];
  f32x4 lsuml = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < MT; ++k) {
    lsum[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[k][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int j = 0; j < (LEFT ? DB : 1); ++j) accl[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // P^T operands of the half in flight: made by the softmax step, consumed by the PV step
  f16x8 pop[MTA];
  f16x8 popl;   // leftover P^T: NL = 2 (32 keys)
  f16x4 popl4;  // leftover P^T: NL = 1 (16 keys)
  // Softmax reference per row (log2 units): starts at the maximum of the chunk's first 32
  // keys and is only raised when a probability of a half would exceed 2^15 (an exponent
  // above kRaiseLog2), so p = 2^(s c - m_ref) <= 2^15 always fits fp16 and the accumulator
  // rescale is rare (a lower bound raises the reference, and rescales, several times per
  // chunk on peaky keys).
  float m_ref[MTA], m_refl = 0.f;

  // ---- scores S^T[key][row] of keys 32 h .. 32 h + 31 of tile t: this lane holds row l16,
  // keys 32 h + 16 j + 4 grp + r in sc[.][j][r]; keys past the chunk end get -inf
  auto scores = [&](auto tag, int t, int h, f32x4 (&sc)[MTA][2], f32x4 (&scl)[2]) {
    constexpr bool WL = decltype(tag)::value;
    constexpr int MTE = decltype(tag)::rows;  // row tiles this wave computes
    __builtin_amdgcn_sched_barrier(0);
    const unsigned char* Ks = lds + ring_slot(Y::kKRing, t, kKStages);
    const int key0 = kbeg + t * kKeyTile;
    // all K operands of the half are read up front, so the products start as soon as the
    // first ones land and the rest of the reads overlap them
    bf16x8 kop[DS][2];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        kop[ds][j] = *(const bf16x8*)(Ks + k_lane[ds] + (32 * h + 16 * j) * Y::kRowBytes);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int k = 0; k < MTE; ++k)
          sc[k][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ds][j], qop[k][ds],
                                                             ds ? sc[k][j] : zero4, 0, 0, 0);
      }
    }
    // instruction order: operand reads run two d-steps ahead of the products
    if constexpr (MTE > 0) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * MTE, 0);
        if (ds + 2 < DS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // leftover scores of this wave's key blocks (the half's K operands are in registers):
    // scl[i] holds keys 32 h + 16 (ljj + i) + 4 grp + r
    if constexpr (WL) {
      if (h == lh) {
        if (NL == 2 || ljj == 0) {  // wave-uniform: no register array indexed at run time
#pragma unroll
          for (int i = 0; i < LKB; ++i) {
            scl[i] = zero4;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
              scl[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ds][i], qopl[ds], scl[i], 0, 0, 0);
          }
        } else {
          scl[0] = zero4;
#pragma unroll
          for (int ds = 0; ds < DS; ++ds)
            scl[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ds][1], qopl[ds], scl[0], 0, 0, 0);
        }
      }
    }
    if (key0 + 32 * h + 32 > kend) {  // keys past the chunk end (last tile only)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key0 + 32 * h + 16 * j + 4 * grp + r >= kend) {
#pragma unroll
            for (int k = 0; k < MTE; ++k) sc[k][j][r] = -INFINITY;
          }
      if constexpr (WL) {
        if (h == lh) {
#pragma unroll
          for (int i = 0; i < LKB; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (key0 + 32 * h + 16 * (ljj + i) + 4 * grp + r >= kend) scl[i][r] = -INFINITY;
        }
      }
    }
  };

  // ---- reference of the pass: maximum of the chunk's first 32 keys, taken from the scores
  // of tile 0's first half (tile 0 always holds a valid key); for the leftover rows, the
  // maximum over this wave's first key block(s), in half lh of tile 0
  auto set_reference = [&](auto tag, const f32x4 (&sc)[MTA][2]) {
    constexpr int MTE = decltype(tag)::rows;
#pragma unroll
    for (int k = 0; k < MTE; ++k) {
      const float m0 = fmaxf(fmaxf(sc[k][0][0], sc[k][0][1]), fmaxf(sc[k][0][2], sc[k][0][3]));
      const float m1 = fmaxf(fmaxf(sc[k][1][0], sc[k][1][1]), fmaxf(sc[k][1][2], sc[k][1][3]));
      m_ref[k] = group_max(fmaxf(m0, m1) * a.c);
    }
  };
  auto set_reference_left = [&](const f32x4 (&scl)[2]) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < LKB; ++i)
      m = fmaxf(m, fmaxf(fmaxf(scl[i][0], scl[i][1]), fmaxf(scl[i][2], scl[i][3])));
    m = group_max(m * a.c);
    // a block wholly past the chunk end leaves no valid key: any finite reference will do
    m_refl = m == -INFINITY ? 0.f : m;
  };

  // ---- softmax of the scores of half h (from scores()): probabilities, P^T operands
  auto softmax = [&](auto tag, int h, f32x4 (&sc)[MTA][2], f32x4 (&scl)[2]) {
    constexpr bool WL = decltype(tag)::value;
    constexpr int MTE = decltype(tag)::rows;
    // ---- probabilities against the running reference (fp32), rounded to the fp16 P^T
    // operands; the row-sum product in pv() adds exactly those rounded values (in fp32), so
    // numerator and normaliser weight every key alike.
    float p[MTA][8], pl[8], xm[MTA], xml = -INFINITY;
    auto make_ops = [&](int k) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pop[k][e] = (_Float16)p[k][e];
    };
    auto make_left = [&]() {
      if constexpr (LKB == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) popl[e] = (_Float16)pl[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) popl4[e] = (_Float16)pl[e];
      }
    };
    // (the exponents' maximum decides the rare reference raise, off the path of the sums)
    auto max8 = [](const float (&v)[8]) {  // four v_max3/v_max instructions
      const float a = fmaxf(fmaxf(v[0], v[1]), v[2]);
      const float b = fmaxf(fmaxf(v[3], v[4]), v[5]);
      return fmaxf(b, fmaxf(fmaxf(v[6], v[7]), a));
    };
#pragma unroll
    for (int k = 0; k < MTE; ++k) {
#pragma unroll
      for (int e = 0; e < 8; ++e) p[k][e] = __builtin_fmaf(sc[k][e / 4][e % 4], a.c, -m_ref[k]);
      xm[k] = max8(p[k]);
#pragma unroll
      for (int e = 0; e < 8; ++e) p[k][e] = __builtin_amdgcn_exp2f(p[k][e]);
      make_ops(k);
    }
    const bool lhere = WL && h == lh;  // this step carries the wave's leftover keys
    if constexpr (WL) {
      if (lhere) {
#pragma unroll
        for (int e = 0; e < 4 * LKB; ++e) pl[e] = __builtin_fmaf(scl[e / 4][e % 4], a.c, -m_refl);
        if constexpr (LKB == 2) xml = max8(pl);
        else xml = fmaxf(fmaxf(pl[0], pl[1]), fmaxf(pl[2], pl[3]));
#pragma unroll
        for (int e = 0; e < 4 * LKB; ++e) pl[e] = __builtin_amdgcn_exp2f(pl[e]);
        make_left();
      }
    }
    // ---- raise the reference of rows with a probability above 2^15 (rare: the
    // reference starts at the maximum of the chunk's first 32 keys); wave-uniform branch
    bool need = false;
#pragma unroll
    for (int k = 0; k < MTE; ++k) need |= xm[k] > kRaiseLog2;
    if constexpr (WL) need |= lhere && xml > kRaiseLog2;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
      // an empty volatile asm keeps this block a real (rarely taken) branch: without it the
      // compiler executes the rescale unconditionally, which doubles the VALU work per step
      asm volatile("" ::: "memory");
#pragma unroll
      for (int k = 0; k < MTE; ++k) {
        // the row's largest exponent of the half: the new reference is at least the row's
        // largest score so far, so every probability drops to at most 1
        const float mx = group_max(xm[k]);
        const float shift = mx > kRaiseLog2 ? mx : 0.f;
        const float alpha = __builtin_amdgcn_exp2f(-shift);
        m_ref[k] += shift;
        lsum[k] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) p[k][e] *= alpha;
        make_ops(k);
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[k][db] *= alpha;
      }
      if constexpr (WL) {
        if (lhere) {
          const float mx = group_max(xml);
          const float shift = mx > kRaiseLog2 ? mx : 0.f;
          const float alpha = __builtin_amdgcn_exp2f(-shift);
          m_refl += shift;
          lsuml *= alpha;
#pragma unroll
          for (int e = 0; e < 4 * LKB; ++e) pl[e] *= alpha;
          make_left();
#pragma unroll
          for (int j = 0; j < DB; ++j) accl[j] *= alpha;
        }
      }
    }
    // (P^T operand of k-step h: element e <-> key 32 h + 16 (e / 4) + 4 grp + (e % 4))
  };

  // ---- PV(t, h): O^T[d][row] += V^T[d][key] P^T[key][row] for keys 32 h .. 32 h + 31 of tile t
  auto pv = [&](auto tag, int t, int h) {
    constexpr bool WL = decltype(tag)::value;
    constexpr int MTE = decltype(tag)::rows;
    __builtin_amdgcn_sched_barrier(0);
    const unsigned char* Vt = lds + ring_slot(Y::kVt, t, kVtStages) + vt_lane[h];
    f16x8 vop[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) vop[db] = *(const f16x8*)(Vt + db * 16 * (kKeyTile * 2));
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int k = 0; k < MTE; ++k)
        acc[k][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[db], pop[k], acc[k][db], 0, 0, 0);
    // the row sums of the same P^T operands (one product per row tile, no LDS operand)
#pragma unroll
    for (int k = 0; k < MTE; ++k)
      lsum[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones_f16x8(), pop[k], lsum[k], 0, 0, 0);
    // instruction order: operand reads run four d-blocks ahead of the products
    if constexpr (MTE > 0) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, MTE, 1);
        if (db + 4 < DB) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 1);
      }
    }
    if constexpr (WL) {
      // leftover rows: this wave's key block(s) of the half, all D dims, from the same V^T
      // operands (a 16-key block is one 8-byte half of each operand: the K = 16 product)
      if (h == lh) {
        if constexpr (LKB == 2) {
#pragma unroll
          for (int db = 0; db < DB; ++db)
            accl[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[db], popl, accl[db], 0, 0, 0);
          lsuml = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones_f16x8(), popl, lsuml, 0, 0, 0);
        } else {
          // the K = 32 product over the whole half with P zero outside this wave's 16-key
          // block (block ljj: the first or second 8-byte half of the operand).  The K = 16
          // product would need a branch on ljj, and the compiler never updates that product's
          // accumulators in place: it copied all of them back where the branches join.
          const uint2 pb = __builtin_bit_cast(uint2, popl4);
          const uint4 pz = ljj == 0 ? make_uint4(pb.x, pb.y, 0u, 0u) : make_uint4(0u, 0u, pb.x, pb.y);
          const f16x8 p8 = __builtin_bit_cast(f16x8, pz);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            accl[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[db], p8, accl[db], 0, 0, 0);
          lsuml = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones_f16x8(), p8, lsuml, 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- pass over the chunk.  Tiles stream through the LDS rings: tile t+3 is issued while
  // tile t is consumed and V of tile t+1 is transposed.  Per 32-key half a wave forms the
  // scores (matrix core), the softmax (VALU) and the PV product (matrix core); merged with
  // its neighbours this is an alternation of matrix-core phases (PV of one half + scores of
  // the next) and VALU phases (softmax).  The second wave group runs half a phase pair
  // behind the first -- it carries the scores of a tile's last half across the barrier and
  // starts each tile with their softmax -- so on every SIMD one wave's softmax overlaps the
  // other wave's products:
  //   first group:   [PV(t-1,1) S(t,0)] [softmax(t,0)] [PV(t,0) S(t,1)] [softmax(t,1)]
  //   second group:  [softmax(t-1,1)]   [PV(t-1,1) S(t,0)] [softmax(t,0)] [PV(t,0) S(t,1)]
  // Only the first group carries leftover rows; the second also transposes V in its first
  // VALU phase.  With two row tiles per first-group wave (the compute-heavy shapes) the
  // first group issues tile t+3 after its first softmax of tile t rather than right after
  // the barrier: its first matrix phase then starts at once, and the loads still run 1.5
  // tiles ahead of their use (Llama 32k prefix pass -0.6 µs, 262k -2%).  Lighter shapes are
  // bound by the K/V stream and keep the full two tiles of lead (issuing later cost them
  // 2-3%).
  constexpr bool kLateIssue = MT >= 2;  // where the first group issues the next tile loads
  auto run_chunk = [&](auto group) {
    constexpr bool LAG = decltype(group)::value;  // second wave group
    constexpr PassTag<!LAG && LEFT, LAG ? MTB : MT> tag{};
    // Prologue: the query operands, tiles 0 and 1 (the first iteration needs both), then
    // tile 2.  The queries and, where the chunk allows, tiles 0 and 1 were issued before the
    // prefix length arrived, queries first: every split of the head reads them at the same
    // moment, and issued behind the tile loads they returned only after the whole first-tile
    // burst (~1 µs later than the tiles on Llama 32k).  The compiler does not count direct
    // loads, so it would wait for every one of them (vmcnt(0)) before the first use of the
    // query registers; an explicit full wait placed before tile 2 is issued lets tile 2
    // stream while tile 0 is consumed.  The softmax reference comes from the first scores of
    // the loop (no separate pass over tile 0).
    if constexpr (!LAG)
      if (!early)
        for (int t = 0; t < 2 && t < ntiles; ++t) issue(t);
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
    if constexpr (!LAG)
      if (ntiles > 2) issue(2);
    wait_tiles_and_barrier(min(2, ntiles - 1));
    if constexpr (LAG) transpose_v(0);
    f32x4 sc[MTA][2];  // scores of the half in flight (the second group carries them on)
    f32x4 scl[2];
    for (int t = 0; t < ntiles; ++t) {
      // tile t+1 landed (for the transpose), V^T of tile t complete, tile t-1 done
      wait_tiles_and_barrier(min(t + 2, ntiles - 1) - (t + 1));
      if constexpr (LAG) {
        if (t > 0) softmax(tag, 1, sc, scl);
        if (t + 1 < ntiles) transpose_v(t + 1);
      } else if constexpr (!kLateIssue) {
        if (t + 3 < ntiles) issue(t + 3);  // refills the K stage of t-1 and the V stage of t
      }
      if (t > 0) pv(tag, t - 1, 1);
      scores(tag, t, 0, sc, scl);
      if (t == 0) {
        set_reference(tag, sc);
        if constexpr (decltype(tag)::value)
          if (lh == 0) set_reference_left(scl);
      }
      softmax(tag, 0, sc, scl);
      if constexpr (!LAG && kLateIssue) {
        // refills the K stage of t-1 and the V stage of t (free since the barrier)
        if (t + 3 < ntiles) issue(t + 3);
      }
      pv(tag, t, 0);
      scores(tag, t, 1, sc, scl);
      if constexpr (decltype(tag)::value)
        if (t == 0 && lh == 1) set_reference_left(scl);
      if constexpr (!LAG) softmax(tag, 1, sc, scl);
    }
    if constexpr (LAG) softmax(tag, 1, sc, scl);
    pv(tag, ntiles - 1, 1);
  };

  // the two groups run separate copies of the loop (same barrier sequence), so each copy
  // is register-allocated on its own
  if (wg == 0) run_chunk(std::false_type{});
  else run_chunk(std::true_type{});

  // ---- normalise and write this chunk's partial (16-bit rows with one factor per row)
  const size_t slot = ((size_t)b * G.Hkv + kv) * (G.S + 1) + s;
  constexpr int kRowBytes = 2 * D;  // an encoded partial row
  const __amdgpu_buffer_rsrc_t part_rows = __builtin_amdgcn_make_buffer_rsrc(
      a.o_part + slot * G.R_pad * (D / 2), 0, G.R_pad * kRowBytes, kBufWord3);
  float* lse_rows = a.lse_part + slot * G.R_pad;
  float* scale_rows = a.o_scale + slot * G.R_pad;
  // A row's factor is its largest magnitude over the 4 lanes that hold it (row_code).  A lane
  // holds 4 consecutive dims of one row per d block, so direct stores would write 8-byte
  // pieces of 16 rows per instruction: each wave stages its encoded rows in LDS (the V and
  // V^T rings are free once every wave is past its loop) and writes them back whole, four
  // consecutive rows (1 KB) per store instruction at D = 128.
  __syncthreads();
  {
    constexpr int kC = kRowBytes / 16;      // 16-byte chunks per encoded row
    constexpr int kRowsPerInst = 64 / kC;   // rows per store instruction
    static_assert(Y::kVRing + kWaves * 16 * kRowBytes <= Y::kBytes, "staging fits the V rings");
    unsigned char* stage = lds + Y::kVRing + wave * (16 * kRowBytes);
#pragma unroll
    for (int k = 0; k < MT; ++k) {
      const int tile = full_tile(k);
      const float lt = lsum[k][0];  // (the product summed over all keys of the row)
      if (tile >= t_end || (wg != 0 && k >= MTB)) continue;  // (no rows of this wave)
      const float inv = 1.f / lt;
      float amax = 0.f, sum = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          amax = fmaxf(amax, __builtin_fabsf(acc[k][db][e]));
          sum += acc[k][db][e];
        }
      const RowCode rc = row_code(group_max(amax) * inv, group_sum(sum) * inv);
      const float enc = rc.enc * inv;
      // dims 16 db + 4 grp .. + 3: half (grp & 1) of chunk 2 db + grp / 2, which sits at
      // chunk position c ^ r in row r (conflict-free both ways)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *(uint2*)(stage + l16 * kRowBytes + 16 * ((2 * db + (grp >> 1)) ^ (l16 & (kC - 1))) +
                  8 * (grp & 1)) = pack16x4(acc[k][db], enc);
      // (the same wave reads the staging back: its LDS accesses complete in order)
#pragma unroll
      for (int j = 0; j < 16 / kRowsPerInst; ++j) {
        const int rr = j * kRowsPerInst + lane / kC, c = lane % kC;
        const uint4 v = *(const uint4*)(stage + rr * kRowBytes + 16 * (c ^ (rr & (kC - 1))));
        store_agent(part_rows, (tile * 16 + rr) * kRowBytes + 16 * c, v);
      }
      if (grp == 0) {
        lse_rows[tile * 16 + l16] = (m_ref[k] + __log2f(lt)) * kLn2;
        scale_rows[tile * 16 + l16] = rc.f;
      }
    }
  }
  if constexpr (LEFT) {
    // Leftover rows: combine the partials of the waves that share a leftover tile (each
    // covered some of its keys) through LDS, as in the merge: M = max m_w, weights 2^(m_w-M).
    // Every wave is past its loop (barrier above), so the K ring is free.  The row's factor
    // comes from the same combination of the waves' largest magnitudes, a bound on the
    // combined row's (no larger than the largest |v| the row attends to), so the sharers
    // need no second exchange.
    constexpr int kStride = 4 * DB + 4;  // floats per (wave, lane): acc, m, l, max |acc|, sum
    static_assert(kWaves / 2 * 64 * kStride * 4 <= kKStages * Y::kTileBytes,
                  "the leftover exchange fits the K ring");
    float* xl = (float*)(lds + Y::kKRing);
    if (has_left) {
      const float lsumw = lsuml[0];
      float amax = 0.f, sum = 0.f;
#pragma unroll
      for (int j = 0; j < DB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          amax = fmaxf(amax, __builtin_fabsf(accl[j][e]));
          sum += accl[j][e];
        }
      amax = group_max(amax);
      sum = group_sum(sum);
      float* mine = xl + (ww * 64 + lane) * kStride;
#pragma unroll
      for (int j = 0; j < DB; ++j) *(f32x4*)(mine + 4 * j) = accl[j];
      *(f32x4*)(mine + 4 * DB) = f32x4{m_refl, lsumw, amax, sum};
    }
    __syncthreads();
    if (has_left && ltile < t_end) {
      // sharers: NL = 1 -> waves 0..3; NL = 2 -> waves 2 (ww/2) and 2 (ww/2) + 1.  This wave
      // writes d-blocks [o0, o0 + DB * NL / 4) of the combined row.
      constexpr int kShare = NL == 2 ? 2 : 4;
      constexpr int kOwn = DB / kShare;
      const int w0 = NL == 2 ? (ww & ~1) : 0;
      const int o0 = (ww - w0) * kOwn;
      f32x4 st[kShare];  // (m, l, max |acc|, sum) of each sharer
      float M = -INFINITY;
#pragma unroll
      for (int i = 0; i < kShare; ++i) {
        st[i] = *(const f32x4*)(xl + ((w0 + i) * 64 + lane) * kStride + 4 * DB);
        M = fmaxf(M, st[i][0]);
      }
      float den = 0.f, bound = 0.f, sum = 0.f, wgt[kShare];
#pragma unroll
      for (int i = 0; i < kShare; ++i) {
        wgt[i] = __builtin_amdgcn_exp2f(st[i][0] - M);
        den += wgt[i] * st[i][1];
        bound += wgt[i] * st[i][2];
        sum += wgt[i] * st[i][3];
      }
      const float inv = 1.f / den;
      const RowCode rc = row_code(bound * inv, sum * inv);
      const float enc = rc.enc * inv;
      const int row = ltile * 16 + l16;
#pragma unroll
      for (int j = 0; j < kOwn; ++j) {
        f32x4 o = zero4;
#pragma unroll
        for (int i = 0; i < kShare; ++i)
          o += wgt[i] * *(const f32x4*)(xl + ((w0 + i) * 64 + lane) * kStride + 4 * (o0 + j));
        store_agent(part_rows, row * kRowBytes + 2 * (16 * (o0 + j) + 4 * grp), pack16x4(o, enc));
      }
      if (grp == 0 && o0 == 0) {
        lse_rows[row] = (M + __log2f(den)) * kLn2;
        scale_rows[row] = rc.f;
      }
    }
  }
}

template <int D, int MT, int NL, int MTB>
hipError_t launch_cfg(const PrefixArgs& a, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((prefix_attn_splitk<D, MT, NL, MTB>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// Row-tile shape of a block: MT tiles per first-group wave, MTB per second-group wave, NL
// leftover tiles split by keys over the first group.
struct RowShape {
  int mt, nl, mtb;
};

// The shapes the kernel is built for.  The register budget of two waves per SIMD (256 VGPRs,
// no scratch) admits (MT, NL) in {(0..1, 0..2), (2, 0..1)} for the first group.  An idle
// second group (MTB = 0) is kept to blocks of at most 4 tiles: with 5 or 6 tiles as one
// tile per first-group wave plus leftover keys, the prefix pass alone timed the same as one
// tile per wave of both groups, but whole steps on ragged batches (80 rows per KV head)
// measured slower.
constexpr RowShape kShapes[] = {
    {0, 1, 0}, {0, 2, 0}, {1, 0, 0}, {1, 0, 1}, {1, 1, 1},
    {1, 2, 1}, {2, 0, 1}, {2, 1, 1}, {2, 0, 2}, {2, 1, 2},
};

template <int D>
hipError_t launch_d(const PrefixArgs& a, RowShape r, dim3 grid, hipStream_t stream) {
#define HTA_SHAPE(M, L, MB) \
  if (r.mt == M && r.nl == L && r.mtb == MB) return launch_cfg<D, M, L, MB>(a, grid, stream);
  HTA_SHAPE(0, 1, 0) HTA_SHAPE(0, 2, 0) HTA_SHAPE(1, 0, 0) HTA_SHAPE(1, 0, 1) HTA_SHAPE(1, 1, 1)
  HTA_SHAPE(1, 2, 1) HTA_SHAPE(2, 0, 1) HTA_SHAPE(2, 1, 1) HTA_SHAPE(2, 0, 2) HTA_SHAPE(2, 1, 2)
#undef HTA_SHAPE
  return hipErrorInvalidValue;
}

// Four times the matrix-core load of a shape on each SIMD (one wave of each group), in row
// tiles per key tile (a leftover tile is spread over the four first-group waves); equal to
// the number of row tiles the shape holds.
constexpr int simd_load4(RowShape r) { return 4 * (r.mt + r.mtb) + r.nl; }

// The shape for `tiles` row tiles: the one that holds them all (4 (MT + MTB) + NL >= tiles)
// with the least matrix-core work per SIMD.  Up to 17 tiles (272 query rows) fit one
// workgroup; more rows are split into row blocks.
RowShape split_rows(int tiles) {
  RowShape best{2, 1, 2};
  for (const RowShape& r : kShapes) {
    if (4 * (r.mt + r.mtb) + r.nl < tiles) continue;
    if (simd_load4(r) < simd_load4(best)) best = r;
  }
  return best;
}

}  // namespace

void prefix_row_blocking(const Geometry& g, int* tiles_per_block, int* blocks) {
  // The fewest blocks: each extra block streams the chunk's K and V once more, and a block
  // with fewer tiles saves less than that (the per-tile staging and V^T work stays).
  const int max_tiles = 8 * 2 + 1;
  const int nb = (g.NT + max_tiles - 1) / max_tiles;
  const int tpb = (g.NT + nb - 1) / nb;
  *blocks = (g.NT + tpb - 1) / tpb;
  *tiles_per_block = tpb;
}

hipError_t launch_prefix_attn_splitk(const Geometry& g, const void* q, const void* k_prefix,
                                     const void* v_prefix, const int32_t* prefix_len,
                                     const Workspace& ws, hipStream_t stream) {
  PrefixArgs a;
  a.q = (const unsigned short*)q;
  a.k_prefix = (const unsigned short*)k_prefix;
  a.v_prefix = (const unsigned short*)v_prefix;
  a.prefix_len = prefix_len;
  a.status_reset = ws.status_reset;
  a.lse_part = ws.lse_part;
  a.o_scale = ws.o_scale;
  a.o_part = ws.o_part;
  a.g = g;
  int tpb, nb;
  prefix_row_blocking(g, &tpb, &nb);
  const RowShape shape = split_rows(tpb);
  a.row_blocks = nb;
  a.tiles_per_block = tpb;
  a.c = g.scale * kLog2e;
  dim3 grid(g.S, g.Hkv * nb, g.B);
  if (g.D == 128) return launch_d<128>(a, shape, grid, stream);
  if (g.D == 64) return launch_d<64>(a, shape, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace hta
