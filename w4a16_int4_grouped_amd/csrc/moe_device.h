// Device helpers for the gfx950 kernels: vector types, BF16 packing, the
// uint4 -> BF16 dequantisation of one packed word, the BF16 MFMA and the
// XCD-aware block remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two BF16 (round to nearest even) in one dword, low half
// first: v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Dequantise one packed word: eight uint4 values, low nibble first along K,
// with zero point 8 and scale s (Chord page, "H200 and Blackwell indexed
// decode": subtract-then-scale fused into the nibble extraction, keeping the
// unfused BF16 rounding order).
//
// fma(q, s, -8s) = q*s - 8*s is computed exactly before its single rounding,
// and the exact value (q - 8)*s has at most 4 + 8 significant bits, so the
// FP32 result is exactly (q - 8)*s (for |s| < 2^125, which keeps -8s finite);
// v_cvt_pk_bf16_f32 then rounds it once to BF16. The result is bit-identical
// to bf16_rne((q - 8) * s).
//
// The nibbles are split into two byte-aligned words so that
// v_cvt_f32_ubyte{0..3} reads each value directly; the empty asm hides the
// masks from the optimiser, which would otherwise re-extract every nibble
// with its own bit-field instruction.
// Result dword m holds k = 2m (low half) and k = 2m+1 (high half).
__device__ __forceinline__ u32x4_t dq8(uint32_t w, float s, float neg8s) {
  uint32_t lo = w & 0x0F0F0F0Fu;
  uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  asm("" : "+v"(lo));
  asm("" : "+v"(hi));
  u32x4_t r;
  r[0] = pack_bf16x2(fmaf((float)(lo & 0xFFu), s, neg8s), fmaf((float)(hi & 0xFFu), s, neg8s));
  r[1] = pack_bf16x2(fmaf((float)((lo >> 8) & 0xFFu), s, neg8s),
                     fmaf((float)((hi >> 8) & 0xFFu), s, neg8s));
  r[2] = pack_bf16x2(fmaf((float)((lo >> 16) & 0xFFu), s, neg8s),
                     fmaf((float)((hi >> 16) & 0xFFu), s, neg8s));
  r[3] = pack_bf16x2(fmaf((float)(lo >> 24), s, neg8s), fmaf((float)(hi >> 24), s, neg8s));
  return r;
}

// D += A . B on one 16x16x32 BF16 MFMA tile (FP32 accumulate). Lane l feeds
// row l%16 of A and column l%16 of B with eight consecutive k values
// (k-slot 8*(l/16) .. +7); D element (row 4*(l/16) + i, column l%16) is
// component i of lane l.
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on
// XCD b % 8). Remap so each XCD receives one contiguous range of logical
// work items: consecutive items (the tiles of one expert) then share that
// XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int nx = 8;
  const int xcd = b % nx, idx = b / nx;
  const int per = total / nx, rem = total % nx;
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + idx;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// SiLU(g) * u in FP32.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

}  // namespace moe
