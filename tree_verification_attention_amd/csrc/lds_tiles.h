// lds_tiles.h -- K/V tiles of 64 keys in LDS, shared by the prefix and tree kernels.
//
// Tiles stream HBM -> LDS with direct LDS loads (global_load_lds_dwordx4: lane l's 16 bytes
// land at base + 16 l, so a wave instruction fills one contiguous 1 KB block).  Rows land
// unpadded; the 16-byte chunks of each row are XOR-swizzled so the operand reads hit
// distinct banks:
//  K rows (D bf16) are read 16 at a time at one chunk column: D = 128 uses chunk ^ row%16,
//    which spreads the 16 rows over all 64 banks (D = 64: chunk ^ (row/2)%8).
//  V rows (D bf16) are read 4 at a time over two chunk columns by the transposing read
//    ds_read_b64_tr_b16: chunk ^ 2*(row%8) keeps the 4 rows x 2 chunks of one 16-lane block
//    on distinct banks (D = 64: chunk ^ 2*(row%4)).
#pragma once

#include "hta_internal.h"

namespace hta {

constexpr int kKeyTile = 64;

template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? 2 * (row & 7) : 2 * (row & 3);
}

// Cache-policy bits of a direct load: kLoadStream marks data read once (non-temporal).
constexpr int kLoadDefault = 0;
constexpr int kLoadStream = 2;

// One 16-byte-per-lane direct load from global memory into LDS.  The builtin only exists for
// the device; the host pass parses this body without generating it.
template <int POLICY = kLoadDefault>
__device__ __forceinline__ void lds_dma16(const void* src, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, POLICY);
#endif
}

// A wave-uniform pointer made opaque to the optimiser, so that adding a per-lane 32-bit offset
// to it stays "scalar base + vector offset" (the direct load's saddr form) instead of being
// reassociated into a per-lane 64-bit address.
__device__ __forceinline__ const unsigned char* opaque_uniform(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const unsigned char*)(((uint64_t)hi << 32) | lo);
}

// Direct loads of rows key0 .. key0+63 of a [rows, D] bf16 matrix into one K-swizzled and
// one V-swizzled LDS tile, split over `nwaves` waves (wave index w).  Rows at or past `kend`
// re-read row kend-1 (callers mask those keys).  Each wave issues 64 * D * 2 / (1024 * nwaves)
// loads per tensor.
// With SKIP_PAST_END, 1 KB blocks that lie wholly at or past `kend` are not loaded at all
// (their LDS contents stay undefined).  POLICY: the loads' cache-policy bits.
template <int D, int NWAVES, bool SKIP_PAST_END = false, int POLICY = kLoadDefault>
__device__ __forceinline__ void dma_kv_tile(const unsigned short* Kg, const unsigned short* Vg,
                                            int key0, int kend, unsigned char* ks,
                                            unsigned char* vs, int w, int lane) {
  constexpr int kChunks = D / 8;                // 16-byte chunks per row
  constexpr int kTileBytes = kKeyTile * D * 2;
  constexpr int kPerWave = kTileBytes / (1024 * NWAVES);
  constexpr int kBlkRows = 1024 / (2 * D);      // rows per 1 KB block
  static_assert(kPerWave * 1024 * NWAVES == kTileBytes, "tile splits into 1 KB blocks");
  static_assert((NWAVES * kBlkRows) % 16 == 0, "a wave's blocks share one swizzle phase");
  // The rows of this wave's blocks are NWAVES * kBlkRows apart, a multiple of both swizzle
  // periods, so every block uses the same swizzled chunk: lane offsets are 32-bit values on
  // a wave-uniform row base (scalar base + vector offset, no per-lane 64-bit addresses).
  const int r0 = w * kBlkRows + lane / kChunks, p = lane % kChunks;
  const uint32_t kx = 16u * (uint32_t)(p ^ swz_k<D>(r0));
  const uint32_t vx = 16u * (uint32_t)(p ^ swz_v<D>(r0));
  if (key0 + kKeyTile <= kend) {  // whole tile valid
    const uint32_t ko = 2u * D * r0 + kx, vo = 2u * D * r0 + vx;
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const size_t row0 = (size_t)key0 + j * NWAVES * kBlkRows;
      const int blk = j * NWAVES + w;
      lds_dma16<POLICY>(opaque_uniform(Kg + row0 * D) + ko, ks + 1024 * blk);
      lds_dma16<POLICY>(opaque_uniform(Vg + row0 * D) + vo, vs + 1024 * blk);
    }
    return;
  }
  const unsigned char* kb = opaque_uniform(Kg + (size_t)key0 * D);
  const unsigned char* vb = opaque_uniform(Vg + (size_t)key0 * D);
  const int last = kend - 1 - key0;  // >= 0: the tile holds at least one valid row
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int blk = j * NWAVES + w;  // 1 KB block of the tile written by this wave
    if (SKIP_PAST_END && blk * kBlkRows > last) continue;
    const uint32_t rr = (uint32_t)min(r0 + j * NWAVES * kBlkRows, last);
    lds_dma16<POLICY>(kb + (2u * D * rr + kx), ks + 1024 * blk);
    lds_dma16<POLICY>(vb + (2u * D * rr + vx), vs + 1024 * blk);
  }
}

}  // namespace hta
