// lse_merge.hip -- the aggregation step of tree verification attention on gfx950.
//
// The prefix pass and the tree pass each produce a partial attention and its log-sum-exp
// over a disjoint set of keys; LongSpec aggregates them into the attention over the union
// (README, Introduction, "Hybrid Attention Aggregation"; arXiv abstract).  Since the
// decoding is lossless the aggregation must be exact, which the log-sum-exp merge is (in
// log2 units, L_s = lse_s * log2(e)):
//     M = max_s L_s,   w_s = 2^(L_s - M),
//     out = sum_s w_s o_s / sum_s w_s,   lse = (M + log2 sum_s w_s) * ln(2).
// Here the parts are the split-K chunks of the prefix (only the ceil(prefix_len/chunk)
// non-empty ones are read) and the tree part.
//
// One wave per output row (b, i, h), in four part groups of 16 lanes: group g handles prefix
// splits g, g+4, g+8, ... and each of its lanes owns D/16 consecutive output dimensions
// (8- or 16-byte loads of the 16-bit partial values), so a group reads whole partial rows;
// the row's factor (o_scale) and log-sum-exp come with them.  Every load of the
// first 4 KB splits (their log-sum-exps and partial rows; KB per lane, 1, 2, 4 or 9 by the
// split count, so few splits hold few registers and more waves stay resident), the tree
// part and the sequence's prefix length is issued before any is used, so the merge costs
// one memory round trip: the slots of splits past the prefix end are read speculatively
// and never used (they contribute through a select, never a multiply by zero, so stale
// contents are harmless).
// The four group sums are added across lanes l, l^16, l^32, l^48 and the first group writes
// the row.
//
// Two forms.  The plain merge reads the tree partial (slot S) written by tree_attn_masked.
// The fused merge, used by the whole step, computes the tree part itself: a query row sees
// exactly its node's ancestors and itself, at most depth + 1 keys, so the wave walks the
// parent chain (the sequence's parent pointers staged in LDS and validated as they load)
// and takes the visible keys four at a time, one per part group: each group forms its key's
// score with a 16-lane reduction over D, and the groups keep a running maximum, weight sum
// and weighted value sum in fp32.  This replaces a launch and the partial round trip
// through HBM with a few dozen dot products per row.  The fused merge also records the
// sequence's device status.
//
// Both forms check every output row they write: a row that comes out non-finite (an input
// outside what the prefix pass supports, such as a bf16 V value beyond the fp16 range of its
// PV product, or a non-finite input) is written as NaN and recorded in the sequence's status
// (kStatusNonFinite), so such a result is never silently wrong.
#include "hta_internal.h"

#include <type_traits>

namespace hta {

namespace {

constexpr int kThreads = 256;

constexpr int kMaxT = 256;

struct MergeArgs {
  const int32_t* prefix_len;
  const int32_t* status;   // [B]: read by the plain merge (the tree pass status)
  int32_t* status_or;      // [B]: non-finite rows (both forms) and, fused, the tree verdict
                           // are OR-ed in (the call cleared the words first, or the tree pass
                           // wrote them)
  float* lse_part;               // read by the merges, written by the tree-only form
  float* o_scale;                // the factor of each o_part row (likewise)
  uint32_t* o_part;              // 16-bit rows (pack16 / lo16, hi16)
  float* out;
  float* lse;
  // fused merge only
  const void* q;                 // in_dtype [B, T, Hq, D]
  const void* k_tree;            // [B, Hkv, T, D]
  const void* v_tree;
  const int32_t* parent_idx;     // [B, T]
  Geometry g;
  int32_t include_tree;
};

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// sum over the four part groups (lanes l, l^16, l^32, l^48)
__device__ inline float group_sum4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ inline float to_f32(unsigned short h) {  // bf16 bits, widened exactly
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}
__device__ inline float to_f32(float x) { return x; }

// What one launch does: the plain merge (tree partial read from slot S), the merge with the
// tree part fused in, or the tree part alone written as the tree partial (slot S).
enum Mode { kPlain = 0, kFused = 1, kTreeOnly = 2 };

// sum and maximum over the 16 lanes of a part group
__device__ inline float lane16_sum(float x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ inline float lane16_max(float x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// One lane's share of a partial row: NW dwords of 16-bit values (two per dword), loaded
// whole (16 bytes at D = 128, 8 at D = 64).
template <int NW>
struct Share16 {
  uint32_t w[NW];
};

// maximum over the four part groups (lanes l, l^16, l^32, l^48)
__device__ inline float group_max4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// TIN: element type of q, k_tree, v_tree (unsigned short = bf16 bits, or float)
template <int D, int MODE, typename TIN, int KB>
__global__ __launch_bounds__(kThreads) void lse_merge(MergeArgs a) {
  constexpr bool FUSED = MODE != kPlain;   // computes the tree part
  constexpr bool PREFIX = MODE != kTreeOnly;
  constexpr int DPL = D / 16;   // output dimensions per lane of a part group
  constexpr int NW = DPL / 2;   // dwords of 16-bit values per part and lane
  using Sh = Share16<NW>;
  constexpr int kBatch = KB;    // splits per lane per pass: 4 KB per pass
  __shared__ int32_t s_par[kThreads / 64][kMaxT];  // fused: parent pointers, one slice per wave
  const Geometry& G = a.g;
  // (one field of each 64-byte line of the arguments: all three lines come in the first batch
  // of scalar loads, where the compiler would otherwise fetch them in dependent rounds around
  // the row test below)
  asm volatile("" ::"s"(a.prefix_len), "s"(a.q), "s"(a.g.R_pad));
  const int lane = threadIdx.x & 63;
  // wave-uniform, and the row index 32-bit (the launch checks B T Hq < 2^31): the index
  // arithmetic is a few scalar instructions instead of 64-bit divisions on every lane in
  // front of the first load
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pg = lane >> 4, dl = lane & 15;
  const int row_id = (int)blockIdx.x * (kThreads / 64) + wave;
  if (row_id >= G.B * G.T * G.Hq) return;
  const int h = row_id % G.Hq;
  const int i = (row_id / G.Hq) % G.T;
  const int b = row_id / (G.Hq * G.T);
  const int kv = h / G.G;
  const int r = i * G.G + (h % G.G);
  const int T = G.T;
  float* outp = a.out + (size_t)row_id * D + DPL * dl;
  float* lsep = a.lse + ((size_t)b * G.Hq + h) * T + i;
  const size_t base = ((size_t)b * G.Hkv + kv) * (G.S + 1);
  const float* lrow = a.lse_part + base * G.R_pad + r;                 // slot s at s * R_pad
  const float* frow = a.o_scale + base * G.R_pad + r;                  // (likewise)
  // partial row of slot 0 (slot s at s * ostride); this lane's dwords NW dl ..
  const uint32_t* orow = a.o_part + (base * G.R_pad + r) * (D / 2);
  const size_t ostride = (size_t)G.R_pad * (D / 2);
  auto load_share = [&](int slot_s) {
    const uint32_t* src = orow + (size_t)slot_s * ostride + NW * dl;
    Sh v;
    if constexpr (NW == 4) {
      const uint4 x = *(const uint4*)src;
      v.w[0] = x.x, v.w[1] = x.y, v.w[2] = x.z, v.w[3] = x.w;
    } else {
      const uint2 x = *(const uint2*)src;
      v.w[0] = x.x, v.w[1] = x.y;
    }
    return v;
  };
  const bool tree_slot = MODE == kPlain && a.include_tree;  // the plain merge's tree partial

  // ---- issue the loads
  const int Lb = a.prefix_len[b];
  const int st = FUSED ? 0 : a.status[b];  // (read only where the tree slot is used)
  // Loads are unconditional (indices clamped into range, the value replaced where it is
  // used): a load under a lane-dependent branch makes the compiler wait for it inside the
  // branch, which would serialise the loads instead of having them all in flight.
  const float lse_raw = PREFIX ? lrow[(size_t)min(lane, G.S - 1) * G.R_pad] : 0.f;
  const float lse_lane = (PREFIX && lane < G.S) ? lse_raw : -INFINITY;
  Sh vt = {};  // the plain merge's tree partial (slot S, always allocated) and its factor
  const float lse_tree_raw = FUSED ? 0.f : lrow[(size_t)G.S * G.R_pad];
  const float f_tree = FUSED ? 0.f : frow[(size_t)G.S * G.R_pad];
  if constexpr (!FUSED) vt = load_share(G.S);
  const float lse_tree = tree_slot ? lse_tree_raw : -INFINITY;
  int par[kMaxT / 64];
  float qv[DPL];
  if constexpr (FUSED) {
#pragma unroll
    for (int k = 0; k < kMaxT / 64; ++k) {
      const int j = lane + 64 * k;
      const int pj = a.parent_idx[(size_t)b * T + min(j, T - 1)];
      par[k] = j < T ? pj : -1;
    }
    const TIN* qp = (const TIN*)a.q + (size_t)row_id * D + DPL * dl;
#pragma unroll
    for (int e = 0; e < DPL; ++e) qv[e] = to_f32(qp[e]);
  }
  float lk[kBatch], fk[kBatch];
  Sh v[kBatch];
  auto load_parts = [&](int k0, int k1) {
#pragma unroll
    for (int k = k0; k < k1; ++k) {
      // slot pg + 4k, clamped: lanes past the last split re-read it and never use it
      const int p = min(pg + 4 * k, G.S - 1);
      lk[k] = -INFINITY;
      fk[k] = 0.f;
      v[k] = Sh{};
      if (PREFIX && 4 * k < G.S) {  // wave-uniform
        lk[k] = lrow[(size_t)p * G.R_pad];
        fk[k] = frow[(size_t)p * G.R_pad];
        v[k] = load_share(p);
      }
    }
  };
  // A wave's loads complete in order.  The fused merge issues the first partials, then the
  // tree rows its row needs (found from the parent pointers, which were issued first), then
  // the remaining partials: the tree part is computed while those are still arriving.
  constexpr int kEarly = FUSED ? (kBatch < 4 ? kBatch : 4) : kBatch;
  load_parts(0, kEarly);

  // ---- validate
  // (only the tree pass's verdicts reject a sequence here: rows of this launch OR the
  // non-finite flag into the same words while it runs)
  bool bad = Lb < 0 || Lb > G.Lmax || (tree_slot && (st & (kStatusTree | kStatusPrefixLen)) != 0);
  bool tree_bad = false;  // the chain walk needs only this verdict, not the prefix length
  if constexpr (FUSED) {
    // parent pointers: parent[j] in [-1, j-1] for every node (the tree is topologically
    // ordered); the verdict is wave-uniform
    int bad_lane = 0;
#pragma unroll
    for (int k = 0; k < kMaxT / 64; ++k) {
      const int j = lane + 64 * k;
      if (j < T) {
        bad_lane |= (par[k] < -1 || par[k] >= j) ? 1 : 0;
        s_par[wave][j] = par[k];
      }
    }
    tree_bad = __builtin_amdgcn_ballot_w64(bad_lane != 0) != 0;
    bad = MODE == kFused ? (bad || tree_bad) : tree_bad;
  }
  // (a rejected sequence is only acted on at the end: an early exit here would let the
  // compiler wait for the verdict's loads before issuing the partial loads)

  // ---- fused: the tree part over the visible keys i, parent(i), ... (log2 units)
  float mt = -INFINITY, lt = 0.f;  // running maximum, this group's weight sum
  float at[DPL];                   // this group's weighted value sum
#pragma unroll
  for (int e = 0; e < DPL; ++e) at[e] = 0.f;
  const float c = G.scale * kLog2e;
  const TIN* Kt = (const TIN*)a.k_tree + ((size_t)b * G.Hkv + kv) * (size_t)T * D + DPL * dl;
  const TIN* Vt = (const TIN*)a.v_tree + ((size_t)b * G.Hkv + kv) * (size_t)T * D + DPL * dl;
  // one batch of keys, one per part group (key < 0: none): score, then online softmax
  auto batch = [&](int my, const float (&kv8)[DPL], const float (&vv)[DPL]) {
    float sc = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) sc += qv[e] * kv8[e];
    sc = lane16_sum(sc) * c;
    if (my < 0) sc = -INFINITY;
    // finite: the first batch holds the row's own node; later ones start at a valid key
    const float m_new = fmaxf(mt, group_max4(sc));
    const float alpha = __builtin_amdgcn_exp2f(mt - m_new);
    const float p = __builtin_amdgcn_exp2f(sc - m_new);
    mt = m_new;
    lt = lt * alpha + p;
#pragma unroll
    for (int e = 0; e < DPL; ++e) at[e] = at[e] * alpha + p * vv[e];
  };
  // (no key: node 0 is read and its score masked, so its p is 0)
  auto load_key = [&](int my, float (&kv8)[DPL], float (&vv)[DPL]) {
    const TIN* kp = Kt + (size_t)max(my, 0) * D;
    const TIN* vp = Vt + (size_t)max(my, 0) * D;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      kv8[e] = to_f32(kp[e]);
      vv[e] = to_f32(vp[e]);
    }
  };
  // the first eight keys of the chain (enough for trees up to depth 7) are found first and
  // their K/V rows loaded together
  int t = tree_bad ? -1 : i;  // next ancestor (wave-uniform); a chain ends at a root (-1)
  int my0 = -1, my1 = -1;
  float k0[DPL], v0[DPL], k1[DPL], v1[DPL];
  if constexpr (FUSED) {
    __builtin_amdgcn_wave_barrier();  // s_par written by this wave is read below
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (pg == (g & 3)) {
        if (g < 4) my0 = t;
        else my1 = t;
      }
      if (t >= 0) t = __builtin_amdgcn_readfirstlane(s_par[wave][t]);
    }
    load_key(my0, k0, v0);
    load_key(my1, k1, v1);
  }
  load_parts(kEarly, kBatch);
  if (MODE == kFused && i == 0 && h == 0 && lane == 0) {  // the sequence's device status
    const bool len_bad = Lb < 0 || Lb > G.Lmax;
    const int32_t bits = (tree_bad ? kStatusTree : 0) | (len_bad ? kStatusPrefixLen : 0);
    if (bits) atomicOr(a.status_or + b, bits);
  }
  if constexpr (FUSED) {
    if (!tree_bad) batch(my0, k0, v0);
    if (__builtin_amdgcn_ballot_w64(my1 >= 0) != 0) batch(my1, k1, v1);  // wave-uniform
    while (t >= 0) {  // deeper chains, four keys at a time
      int my = -1;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (pg == g) my = t;
        if (t >= 0) t = __builtin_amdgcn_readfirstlane(s_par[wave][t]);
      }
      float kk[DPL], vv[DPL];
      load_key(my, kk, vv);
      batch(my, kk, vv);
    }
  }

  if constexpr (MODE == kTreeOnly) {  // normalise and write the tree partial (slot S)
    // (16-bit values with the row's factor from a 16-lane reduction; the tree partial of a
    // rejected tree has a NaN factor and log-sum-exp)
    const float ltot = group_sum4(lt);
    const float inv = 1.f / ltot;
    float o[DPL], amax = 0.f, sum = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      o[e] = group_sum4(at[e]) * inv;
      amax = fmaxf(amax, __builtin_fabsf(o[e]));
      sum += o[e];
    }
    const RowCode rc = row_code(lane16_max(amax), lane16_sum(sum));
    const size_t n = (base + G.S) * G.R_pad + r;
    uint32_t* trow = a.o_part + n * (D / 2) + NW * dl;
    if (pg == 0)
#pragma unroll
      for (int j = 0; j < NW; ++j) trow[j] = pack16(o[2 * j], o[2 * j + 1], rc.enc);
    if (lane == 0) {
      a.lse_part[n] = bad ? NAN : (mt + __log2f(ltot)) * kLn2;
      a.o_scale[n] = bad ? NAN : rc.f;
    }
    return;
  }
  if (bad) {  // a rejected sequence: NaN
    if (pg == 0)
#pragma unroll
      for (int e = 0; e < DPL; ++e) outp[e] = NAN;
    if (lane == 0) *lsep = NAN;
    return;
  }

  // ---- weights against the largest log-sum-exp.  The maximum Mn is taken on the stored
  // (natural-log) values and each weight is 2^((l - Mn) log2(e)): nothing is computed from a
  // partial before the maximum, so the compiler has no reason to wait for one early.
  const int nsplit = (Lb + G.chunk - 1) / G.chunk;  // non-empty prefix splits (Lb valid here)
  float Mn = fmaxf(lane < nsplit ? lse_lane : -INFINITY, lse_tree);
  for (int p = 64 + lane; p < nsplit; p += 64) Mn = fmaxf(Mn, lrow[(size_t)p * G.R_pad]);
  Mn = wave_max(Mn);
  float ltot = 0.f;
  if constexpr (FUSED) {
    ltot = group_sum4(lt);                         // the tree's weight sum relative to mt
    const float lse_tree_nat = (mt + __log2f(ltot)) * kLn2;  // the tree part's log-sum-exp
    Mn = fmaxf(Mn, lse_tree_nat);
    // kept in the tree slot of lse_part (its o_part row is not written): with the prefix
    // slots it gives every chunk's share of the row's attention
    if (lane == 0) a.lse_part[(base + G.S) * G.R_pad + r] = lse_tree_nat;
  }
  const float M = Mn * kLog2e;  // the same maximum in log2 units
  if (Mn == -INFINITY) {  // no visible key at all (prefix-only merge of an empty prefix)
    if (pg == 0)
#pragma unroll
      for (int e = 0; e < DPL; ++e) outp[e] = 0.f;
    if (lane == 0) *lsep = -INFINITY;
    return;
  }
  float acc[DPL];
  float wl = 0.f;  // this group's weight sum
  {
    // the tree partial enters only when it is part of the merge: a select, not a weight of
    // 0 (the slot is not written otherwise and may hold anything, NaN included)
    const bool use_tree = tree_slot && pg == 0;
    const float wt = use_tree ? __builtin_amdgcn_exp2f((lse_tree - Mn) * kLog2e) : 0.f;
    wl += wt;
    const float wf = wt * f_tree;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      acc[2 * j] = use_tree ? wf * lo16(vt.w[j]) : 0.f;
      acc[2 * j + 1] = use_tree ? wf * hi16(vt.w[j]) : 0.f;
    }
  }
  // (a part's weight times its row factor scales the 16-bit values directly)
  auto add_part = [&](float l, float f, const Sh& pv) {
    const float w = __builtin_amdgcn_exp2f((l - Mn) * kLog2e);
    wl += w;
    const float wf = w * f;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      acc[2 * j] += wf * lo16(pv.w[j]);
      acc[2 * j + 1] += wf * hi16(pv.w[j]);
    }
  };
#pragma unroll
  for (int k = 0; k < kBatch; ++k)
    if (pg + 4 * k < nsplit) add_part(lk[k], fk[k], v[k]);
  // splits beyond the first 4 KB (long prefixes with many splits)
  for (int p0 = 4 * kBatch + pg; p0 < nsplit; p0 += 4 * kBatch) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int p = p0 + 4 * k;
      if (p < nsplit) {
        lk[k] = lrow[(size_t)p * G.R_pad];
        fk[k] = frow[(size_t)p * G.R_pad];
        v[k] = load_share(p);
      }
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (p0 + 4 * k < nsplit) add_part(lk[k], fk[k], v[k]);
  }
  float wsum = group_sum4(wl);
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = group_sum4(acc[e]);
  if constexpr (FUSED) {
    const float wt = __builtin_amdgcn_exp2f(mt - M);
    wsum += wt * ltot;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] += wt * group_sum4(at[e]);
  }
  const float inv = 1.f / wsum;
  const float lse_row = Mn + __log2f(wsum) * kLn2;
  bool finite = __builtin_isfinite(lse_row);
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    acc[e] *= inv;
    finite = finite && __builtin_isfinite(acc[e]);
  }
  // a non-finite value anywhere in the row: the whole row is NaN and the status records it
  const bool row_bad = __builtin_amdgcn_ballot_w64(!finite) != 0;
  if (pg == 0) {
#pragma unroll
    for (int j = 0; j < DPL / 4; ++j)
      ((float4*)outp)[j] = row_bad ? make_float4(NAN, NAN, NAN, NAN)
                                   : make_float4(acc[4 * j], acc[4 * j + 1], acc[4 * j + 2],
                                                 acc[4 * j + 3]);
  }
  if (lane == 0) {
    *lsep = row_bad ? NAN : lse_row;
    if (row_bad) atomicOr(a.status_or + b, kStatusNonFinite);
  }
}

template <int MODE, typename TIN>
hipError_t launch_merge(const MergeArgs& a, const Geometry& g, hipStream_t stream) {
  const long nrows = (long)g.B * g.T * g.Hq;
  if (nrows > 0x7fffffffL - kThreads) return hipErrorInvalidValue;  // (32-bit row indices)
  const int rows_per_block = kThreads / 64;
  dim3 grid((unsigned)((nrows + rows_per_block - 1) / rows_per_block));
  // partial loads held per lane: enough for the split count (fewer registers, more waves
  // resident when there are few splits)
  auto go = [&](auto kb) {
    constexpr int KB = decltype(kb)::value;
    if (g.D == 128)
      hipLaunchKernelGGL((lse_merge<128, MODE, TIN, KB>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((lse_merge<64, MODE, TIN, KB>), grid, dim3(kThreads), 0, stream, a);
  };
  if (g.D != 128 && g.D != 64) return hipErrorInvalidValue;
  if (MODE == kTreeOnly || g.S <= 4) go(std::integral_constant<int, 1>{});
  else if (g.S <= 8) go(std::integral_constant<int, 2>{});
  else if (g.S <= 16) go(std::integral_constant<int, 4>{});
  else go(std::integral_constant<int, 9>{});
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_tree_mode(const Geometry& g, const void* q, const void* k_tree,
                            const void* v_tree, const int32_t* parent_idx,
                            const int32_t* prefix_len, float* out, float* lse,
                            const Workspace& ws, hipStream_t stream) {
  MergeArgs a = {};
  a.prefix_len = prefix_len;
  a.lse_part = ws.lse_part;
  a.o_scale = ws.o_scale;
  a.o_part = ws.o_part;
  a.out = out;
  a.lse = lse;
  a.q = q;
  a.k_tree = k_tree;
  a.v_tree = v_tree;
  a.parent_idx = parent_idx;
  a.status_or = ws.status;
  a.g = g;
  a.include_tree = 1;
  return g.f32 ? launch_merge<MODE, float>(a, g, stream)
               : launch_merge<MODE, unsigned short>(a, g, stream);
}

}  // namespace

hipError_t launch_lse_merge(const Geometry& g, const int32_t* prefix_len, bool include_tree,
                            float* out, float* lse, const Workspace& ws, hipStream_t stream) {
  MergeArgs a = {};
  a.prefix_len = prefix_len;
  a.status = ws.status;  // read always, used only with the tree partial
  a.status_or = ws.status;
  a.lse_part = ws.lse_part;
  a.o_scale = ws.o_scale;
  a.o_part = ws.o_part;
  a.out = out;
  a.lse = lse;
  a.g = g;
  a.include_tree = include_tree ? 1 : 0;
  return launch_merge<kPlain, unsigned short>(a, g, stream);
}

hipError_t launch_tree_merge(const Geometry& g, const void* q, const void* k_tree,
                             const void* v_tree, const int32_t* parent_idx,
                             const int32_t* prefix_len, float* out, float* lse,
                             const Workspace& ws, hipStream_t stream) {
  return launch_tree_mode<kFused>(g, q, k_tree, v_tree, parent_idx, prefix_len, out, lse, ws,
                                  stream);
}

hipError_t launch_tree_chain(const Geometry& g, const void* q, const void* k_tree,
                             const void* v_tree, const int32_t* parent_idx,
                             const int32_t* prefix_len, const Workspace& ws,
                             hipStream_t stream) {
  return launch_tree_mode<kTreeOnly>(g, q, k_tree, v_tree, parent_idx, prefix_len, nullptr,
                                     nullptr, ws, stream);
}

}  // namespace hta
