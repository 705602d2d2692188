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

// v_cvt_off_f32_i4 on byte n of v (SDWA operand select): bits [3:0] of that
// byte, read as a signed 4-bit integer i, become the float i / 16 (exact).
#define MOE_CVT_OFF_BYTE(SEL)                                                         \
  __device__ __forceinline__ float cvt_off_##SEL(uint32_t v) {                        \
    float r;                                                                          \
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:" #SEL \
        : "=v"(r)                                                                     \
        : "v"(v));                                                                    \
    return r;                                                                         \
  }
MOE_CVT_OFF_BYTE(BYTE_0)
MOE_CVT_OFF_BYTE(BYTE_1)
MOE_CVT_OFF_BYTE(BYTE_2)
MOE_CVT_OFF_BYTE(BYTE_3)
#undef MOE_CVT_OFF_BYTE

// Dequantise one prepared word: eight uint4 values q, low nibble first along
// K, stored as q ^ 8 (which, read as a signed 4-bit integer, is q - 8), with
// the group scale given as s16 = 16 * s (Chord page, "H200 and Blackwell
// indexed decode": subtract-then-scale fused into the nibble extraction,
// keeping the unfused BF16 rounding order).
//
// v_cvt_off_f32_i4 gives (q - 8) / 16 exactly, the product with 16 * s is
// exactly (q - 8) * s (at most 4 + 8 significant bits, signed zeros
// included), and v_cvt_pk_bf16_f32 rounds it once to BF16: bit-identical to
// bf16_rne((q - 8) * s). The low nibble of each byte is read in place; the
// high nibbles after one 4-bit shift of the word.
// Result dword m holds k = 2m (low half) and k = 2m+1 (high half).
__device__ __forceinline__ u32x4_t dq8(uint32_t w, float s16) {
  const uint32_t h = w >> 4;
  u32x4_t r;
  r[0] = pack_bf16x2(cvt_off_BYTE_0(w) * s16, cvt_off_BYTE_0(h) * s16);
  r[1] = pack_bf16x2(cvt_off_BYTE_1(w) * s16, cvt_off_BYTE_1(h) * s16);
  r[2] = pack_bf16x2(cvt_off_BYTE_2(w) * s16, cvt_off_BYTE_2(h) * s16);
  r[3] = pack_bf16x2(cvt_off_BYTE_3(w) * s16, cvt_off_BYTE_3(h) * s16);
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
