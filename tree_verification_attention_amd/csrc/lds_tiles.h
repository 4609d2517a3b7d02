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

// One 16-byte-per-lane direct load from global memory into LDS.  The builtin only exists for
// the device; the host pass parses this body without generating it.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
#endif
}

// Direct loads of rows key0 .. key0+63 of a [rows, D] bf16 matrix into one K-swizzled and
// one V-swizzled LDS tile, split over `nwaves` waves (wave index w).  Rows at or past `kend`
// re-read row kend-1 (callers mask those keys).  Each wave issues 64 * D * 2 / (1024 * nwaves)
// loads per tensor.
// With SKIP_PAST_END, 1 KB blocks that lie wholly at or past `kend` are not loaded at all
// (their LDS contents stay undefined).
template <int D, int NWAVES, bool SKIP_PAST_END = false>
__device__ __forceinline__ void dma_kv_tile(const unsigned short* Kg, const unsigned short* Vg,
                                            int key0, int kend, unsigned char* ks,
                                            unsigned char* vs, int w, int lane) {
  constexpr int kChunks = D / 8;                // 16-byte chunks per row
  constexpr int kTileBytes = kKeyTile * D * 2;
  constexpr int kPerWave = kTileBytes / (1024 * NWAVES);
  static_assert(kPerWave * 1024 * NWAVES == kTileBytes, "tile splits into 1 KB blocks");
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int blk = j * NWAVES + w;   // 1 KB block of the tile written by this wave
    if (SKIP_PAST_END && key0 + blk * (1024 / (2 * D)) >= kend) continue;
    const int u = 64 * blk + lane;    // 16-byte chunk position within the tile
    const int r = u / kChunks, p = u % kChunks;
    const size_t gk = (size_t)min(key0 + r, kend - 1);
    lds_dma16(Kg + gk * D + 8 * (p ^ swz_k<D>(r)), ks + 1024 * blk);
    lds_dma16(Vg + gk * D + 8 * (p ^ swz_v<D>(r)), vs + 1024 * blk);
  }
}

}  // namespace hta
