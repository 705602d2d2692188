// Token tiles of the large-M GEMMs: global -> LDS copies and the swizzled
// LDS layout their MFMA fragment reads use.
//
// A 16-row block of a token tile occupies 4 KB of LDS per 128-k chunk: four
// 1 KB groups of 16 rows x 4 pieces of 16 bytes (k = 8 per piece). Row rr of
// a group keeps its 4 pieces in 64 bytes with piece p at position
// p ^ swz(rr), which makes every 16-byte MFMA B-fragment read (16 rows, one
// piece each) hit distinct banks whether the LDS serves 8 or 16 lanes of a
// 16-byte read per cycle (measured: 0 bank conflicts, ~256 B/clk/CU; the
// unswizzled layout runs at a third of that).
#pragma once

#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_layout.h"

namespace moe {

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ int swz(int rr) { return ((rr >> 1) ^ (rr >> 2)) & 3; }

// B-fragment read offset (16-byte slots) of MFMA step 0 of a chunk: row
// (lane & 15) of row block 0, piece 4*(lane >> 4); step g reads slot
// rd0 ^ g (the swizzle sits in the low two bits), row block nt 256 on.
__device__ __forceinline__ int frag_rd0(int lane) {
  return (lane >> 4) * 64 + (lane & 15) * 4 + swz(lane & 15);
}

// Byte offset of this lane's 16-byte piece within a row's 64-byte group:
// a lane writes row 16*q + (lane >> 2) of a row block, position (lane & 3),
// which holds piece (lane & 3) ^ swz(lane >> 2).
__device__ __forceinline__ int dma_piece(int lane) { return ((lane & 3) ^ swz(lane >> 2)) * 16; }

// One wave's share of a token tile for chunk kc: row blocks 2*wave and
// 2*wave + 1 (32 rows), all four piece groups (8 x 1 KB), straight from
// global memory to LDS. src0/src1: the lane's row pointers (plus its piece
// offset) at chunk 0.
__device__ __forceinline__ void dma_tile(u32x4_t* lds_buf, const char* src0, const char* src1,
                                         int kc, int wave) {
#pragma unroll
  for (int ql = 0; ql < 2; ++ql) {
    const char* src = (ql ? src1 : src0) + (size_t)kc * (kKC * 2);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t* dst = lds_buf + ((2 * wave + ql) * 4 + s) * 64;
      __builtin_amdgcn_global_load_lds(src + s * 64, (lds_void_t*)dst, 16, 0, 0);
    }
  }
}

}  // namespace moe
