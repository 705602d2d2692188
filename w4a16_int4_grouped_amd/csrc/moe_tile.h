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

// ---- Half-chunk stages (the K loops that stream the token tile through a
// ring of LDS stages). A stage holds 64 k of a 16*NB-row token tile: for
// each 16-row block nt and lane quarter q, the 16 rows' pieces of MFMA
// steps 2h and 2h + 1 of chunk half h (8 k each), at slot
// ((nt*4 + q)*16 + r)*2 + (j ^ (r >> 3 & 1)). A quarter's 16 fragment reads
// (16 rows, 32 B apart) then fall on distinct banks. Lane l of a 16x16x32
// MFMA reads block nt's step-j fragment at slot nt*128 + (stage_rd(l) ^ j).
__device__ __forceinline__ int stage_rd(int lane) {
  return (lane >> 4) * 32 + (lane & 15) * 2 + ((lane >> 3) & 1);
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left free)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// A bare s_barrier, with no memory operation moved across it (unlike
// __syncthreads, it waits for no outstanding load by itself).
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// This wave's share of stage s (chunk s/2, half s%2) of the token tile, copied
// straight from global memory to LDS: its 32 rows (16-row blocks 2*wave,
// 2*wave + 1), four 16-byte pieces per lane. Lane l copies rows
// stage_row(wave, 0, l) and stage_row(wave, 1, l); its piece i goes to stage
// slot (4*wave + i)*64 + l: block 2*wave + i/2, quarter q = (2i + l/32) % 4,
// row r = (l/2) % 16, position l % 2 holding step j = (l % 2) ^ (r / 8 % 2).
__device__ __forceinline__ int stage_row(int wave, int i, int lane) {
  return 32 * wave + 16 * i + ((lane >> 1) & 15);
}

// The lane's copy sources: one base for the workgroup (the token matrix)
// and the lane's two 32-bit byte offsets from it, its rows (at k = 0)
// advanced to the piece it copies, quarter l/32 of step j (pieces 1 and 3,
// quarter + 2, lie 128 bytes further on). Each copy is then the base in
// SGPRs plus one 32-bit VGPR offset, so a lane holds 2 VGPRs for its copies
// (with 64-bit row pointers, the K loop over 128 token rows spills): the
// token matrix must span less than 4 GiB.
struct StageSrc {
  const char* base;
  uint32_t off[2];
};

__device__ __forceinline__ StageSrc stage_src(const void* base, uint32_t row0_bytes, uint32_t row1_bytes,
                                              int lane) {
  const int r = (lane >> 1) & 15;
  const int j = (lane & 1) ^ ((r >> 3) & 1);
  const uint32_t off = (uint32_t)((lane >> 5) * 64 + j * 16);
  return StageSrc{static_cast<const char*>(base), {row0_bytes + off, row1_bytes + off}};
}

__device__ __forceinline__ void dma_stage(u32x4_t* stage, const StageSrc& src, int s, int wave) {
  const uint32_t soff = (uint32_t)((s >> 1) * (kKC * 2) + (s & 1) * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const char* g = src.base + (size_t)(src.off[i >> 1] + soff + (uint32_t)(i & 1) * 128u);
    __builtin_amdgcn_global_load_lds(g, (lds_void_t*)(stage + (4 * wave + i) * 64), 16, 0, 0);
  }
}

}  // namespace moe
