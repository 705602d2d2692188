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

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// (v & mask) | magic in one VOP3 instruction (the compiler would emit an AND
// and an OR). The mask lives in an SGPR, the magic constant in a VGPR (one
// scalar operand per VOP3 instruction on gfx9).
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(mask), "v"(magic));
  return r;
}

// Per-group constants of dq8: the scale s, -1032 s and -72 s (all exact for
// |s| < 2^117, subnormal s included).
struct GroupScale {
  float s, c0, c1;
};

__device__ __forceinline__ GroupScale group_scale(float s) {
  return GroupScale{s, s * -1032.0f, s * -72.0f};
}

// Dequantise one packed word: eight uint4 values q, low nibble first along
// K, with the group scale s (Chord page, "H200 and Blackwell indexed
// decode": subtract-then-scale fused into the nibble extraction, keeping the
// unfused BF16 rounding order).
//
// Nibbles 0 and 4 masked into the mantissas of an FP16 pair with exponent
// bits 0x6400 (1024.0, unit step 1) read as 1024 + q; nibbles 1 and 5,
// masked in place one nibble higher under exponent bits 0x5400 (64.0, step
// 1/16), read as 64 + q; nibbles 2, 6 and 3, 7 likewise after one 8-bit
// shift. v_fma_mix_f32 widens one FP16 half and computes
//   (1024 + q) s - 1032 s   or   (64 + q) s - 72 s,
// exactly (q - 8) s before its single rounding, and (q - 8) s has at most
// 4 + 8 significant bits, so the FP32 result is exact; v_cvt_pk_bf16_f32
// then rounds it once to BF16: bf16_rne((q - 8) s) for every nonzero
// product. An exactly zero product comes out as +0 whatever the signs
// (x - x = +0); no MFMA result can tell +0 from -0 here, since the
// accumulators start at +0 and +0 + -0 = +0. 17 VALU instructions per 8
// weights. Result dword m holds k = 2m (low half) and k = 2m+1 (high half).
__device__ __forceinline__ u32x4_t dq8(uint32_t w, const GroupScale& g, uint32_t magic_lo,
                                      uint32_t magic_hi) {
  const uint32_t w8 = w >> 8;
  const f16x2_t r0 = __builtin_bit_cast(f16x2_t, and_or(w, 0x000F000Fu, magic_lo));    // q0, q4
  const f16x2_t r1 = __builtin_bit_cast(f16x2_t, and_or(w, 0x00F000F0u, magic_hi));    // q1, q5
  const f16x2_t r2 = __builtin_bit_cast(f16x2_t, and_or(w8, 0x000F000Fu, magic_lo));   // q2, q6
  const f16x2_t r3 = __builtin_bit_cast(f16x2_t, and_or(w8, 0x00F000F0u, magic_hi));   // q3, q7
  // all eight products first, then the packs: a pack reading the product
  // written just before it would wait a cycle (a hazard no-op)
  const float f0 = __builtin_fmaf((float)r0[0], g.s, g.c0), f1 = __builtin_fmaf((float)r1[0], g.s, g.c1);
  const float f2 = __builtin_fmaf((float)r2[0], g.s, g.c0), f3 = __builtin_fmaf((float)r3[0], g.s, g.c1);
  const float f4 = __builtin_fmaf((float)r0[1], g.s, g.c0), f5 = __builtin_fmaf((float)r1[1], g.s, g.c1);
  const float f6 = __builtin_fmaf((float)r2[1], g.s, g.c0), f7 = __builtin_fmaf((float)r3[1], g.s, g.c1);
  u32x4_t r;
  r[0] = pack_bf16x2(f0, f1);
  r[1] = pack_bf16x2(f2, f3);
  r[2] = pack_bf16x2(f4, f5);
  r[3] = pack_bf16x2(f6, f7);
  return r;
}

constexpr uint32_t kF16MagicLo = 0x64006400u;   // two FP16 1024.0
constexpr uint32_t kF16MagicHi = 0x54005400u;   // two FP16 64.0

// dq8 with the sign of zero products set as in (q - 8) * s (sign of q - 8
// times sign of s, +0 for q = 8 with s > 0): bit-identical to
// bf16_rne((q - 8) * s) everywhere. Used where the dequantised weights
// themselves are the result.
__device__ __forceinline__ u32x4_t dq8_exact(uint32_t w, const GroupScale& g) {
  u32x4_t r = dq8(w, g, kF16MagicLo, kF16MagicHi);
  const uint32_t s_neg = (__float_as_uint(g.s) >> 31) & 1u;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t q = (w >> (4 * (2 * m + h))) & 0xFu;
      const uint32_t bits = (r[m] >> (16 * h)) & 0xFFFFu;
      if ((bits & 0x7FFFu) == 0u) {
        const uint32_t neg = (q < 8u ? 1u : 0u) ^ s_neg;
        r[m] = (r[m] & ~(0xFFFFu << (16 * h))) | ((neg << 15) << (16 * h));
      }
    }
  }
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

// xcd_remap over only the first `active` logical items of a grid of at
// least that many workgroups: each XCD gets its share of the active items
// as one contiguous range, and -1 for a workgroup beyond its XCD's share.
// With a grid sized from an upper bound (routing capacity) and the active
// count read on the device, the empty tail no longer lands on whole XCDs.
__device__ __forceinline__ int xcd_remap_active(int b, int active) {
  const int nx = 8;
  const int xcd = b % nx, idx = b / nx;
  const int per = active / nx, rem = active % nx;
  if (idx >= per + (xcd < rem ? 1 : 0)) return -1;
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + idx;
}

// Blocks dealt round-robin to the XCDs in units of G consecutive blocks:
// unit u (blocks uG .. uG + G - 1) runs on XCD u % 8, an XCD takes its units
// in order and each block's `wpb` workgroups in a row. Returns the item
// block * wpb + quad, or -1 past the last of `nblocks`. The grid needs
// 8 * ceil(ceil(nblocks / G) / 8) * G * wpb workgroups. Runs of blocks of
// similar cost (one expert's) then spread over all XCDs instead of filling
// one XCD's range, while a unit's blocks share an XCD.
__device__ __forceinline__ int xcd_deal_blocks(int b, int nblocks, int wpb, int G) {
  const int x = b & 7, idx = b >> 3;
  const int span = G * wpb;
  const int ul = idx / span, rem = idx - ul * span;
  const int j = rem / wpb, q = rem - j * wpb;
  const int blk = (ul * 8 + x) * G + j;
  return blk < nblocks ? blk * wpb + q : -1;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// The n-th expert (in expert order) with rows in counts[0, E), or -1: one
// ballot per 64 experts, the same answer in every lane of the wave.
__device__ __forceinline__ int nth_active(const int32_t* counts, int E, int n) {
  const int lane = threadIdx.x & 63;
  for (int base = 0; base < E; base += 64) {
    const bool has = base + lane < E && counts[base + lane] > 0;
    const uint64_t m = __ballot(has);
    const int k = __popcll(m);
    if (n < k) {
      const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
      const uint64_t hit = __ballot(has && __popcll(m & below) == n);
      return base + __builtin_ctzll(hit);
    }
    n -= k;
  }
  return -1;
}

// Output column of a BF16 store epilogue for lane `lane` of MFMA tile mt of
// row group rg (4 columns from the returned one), or -1 past the output.
// A W13 store (gate_up_I = I) undoes the prepared gate/up interleave: tiles
// 0, 2 of a row group are gate columns rg*32 + (0, 16), tiles 1, 3 the same
// up columns, I further on.
__device__ __forceinline__ int store_col(int N, int gate_up_I, int rg, int mt, int lane) {
  if (gate_up_I) {
    const int c = rg * 32 + (mt >> 1) * 16 + (lane >> 4) * 4;
    return c < gate_up_I ? c + (mt & 1) * gate_up_I : -1;
  }
  const int n = rg * 64 + mt * 16 + (lane >> 4) * 4;
  return n < N ? n : -1;
}

// SiLU(g) * u in FP32.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Weighted rows w*y of the second GEMM, kept for the combine as 16-bit
// words with one power-of-two scale per 8 adjacent positions, the scale's
// exponent carried in the words' top bits. For a group of 8 values v with
// max|v| * (1 + 2^-13) < 2^e (e from frexp, clamped to >= -100), value i is
// n_i = round_to_nearest_even(v_i * 2^(14 - e)), |n_i| < 16383, stored as a
// 15-bit two's complement integer in bits 0..14 with bit 15 = b_i, where
// b_0 .. b_7 are the bits of the byte e + 128 (dword j of the group holds
// values 2j and 2j + 1 and exponent bits j and j + 4). Read
// back, n_i * 2^(e - 14) is within 2^-15 * 2^e <= 2^-14 * max|v| of v_i. The
// layer's output is a BF16 sum of a token's top-k rows, rounded at 2^-9 of
// its magnitude, so the error stays four orders of magnitude below the
// output's own rounding. A row costs 2 bytes a feature, written in whole
// 128-byte lines: a separate exponent plane, written in 8-byte pieces from
// different workgroups, measured 40 us of partial-line writes on the TP8
// shard's down projection.
//
// Within each 64-feature block (one row group of 4 MFMA tiles), feature
// n = 16*mt + 4*q + i sits at position 16*q + 4*mt + i: the 16 values a lane
// q holds for a token row (4 per tile mt) are adjacent, so a lane writes them
// with full 16-byte stores and the 4 lanes of a row fill 128 contiguous bytes
// (with plain [n] order each lane would write pieces 32 bytes apart).

constexpr float kRoundMagic = 12582912.0f;   // 1.5 * 2^23: x + magic has ulp 1
constexpr float kExpGuard = 1.0f + 0x1p-13f;  // keeps |n| below 16383

// Stores G groups of 4 values w * v[g] (tiles mt0 .. mt0 + G - 1 of lane q)
// at row position idx = row * ld + block + 16*q + 4*mt0 (G = 4: mt0 = 0; G = 2:
// mt0 even), idx a multiple of 8: G / 2 scale groups of 8.
template <int G>
__device__ __forceinline__ void store_y16(uint16_t* __restrict__ yq, size_t idx, float w,
                                          const f32x4_t (&v)[G]) {
  static_assert(G == 2 || G == 4, "2 or 4 groups");
  uint32_t d[2 * G];
#pragma unroll
  for (int k = 0; k < G / 2; ++k) {
    float amax = 0.f;
#pragma unroll
    for (int g = 2 * k; g < 2 * k + 2; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(v[g][i]));
    // fl(fl(amax * |w|) * guard) < 2^e implies |v * w| * 2^(14 - e) < 16383
    const int e = max(__builtin_amdgcn_frexp_expf(amax * fabsf(w) * kExpGuard), -100);
    const float sc = __builtin_amdgcn_ldexpf(w, 14 - e);   // exact: a power-of-two multiple of w
    const uint32_t eb = (uint32_t)(e + 128);
    const uint32_t sp = (eb << 12) | (eb << 24);            // bit j at 15, bit j + 4 at 31, after << (3 - j)
#pragma unroll
    for (int g = 2 * k; g < 2 * k + 2; ++g) {
      uint32_t x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = __float_as_uint(__builtin_fmaf(v[g][i], sc, kRoundMagic));
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * (g - 2 * k) + jj;   // dword of the group
        // low halves of the two values (the rounded integers, two's complement:
        // bits 14 and 15 both hold the sign), bit 15 of each replaced
        const uint32_t pair = __builtin_amdgcn_perm(x[2 * jj + 1], x[2 * jj], 0x05040100u);
        const uint32_t bits = sp << (3 - j);
        d[2 * g + jj] = (bits & 0x80008000u) | (pair & 0x7FFF7FFFu);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < G / 2; ++k)
    *reinterpret_cast<u32x4_t*>(yq + idx + 8 * k) = u32x4_t{d[4 * k], d[4 * k + 1], d[4 * k + 2], d[4 * k + 3]};
}

// A group of store_y16 that adds nothing: integers 0 and exponent byte 128.
constexpr u32x4_t kY16Zero = {0u, 0u, 0u, 0x80000000u};

// acc += the 8 values of a group (dwords d[0..3] as stored by store_y16).
__device__ __forceinline__ void add_y16(f32x4_t (&acc)[2], const u32x4_t& d) {
  const uint32_t t = ((d[0] & 0x80008000u) >> 15) | ((d[1] & 0x80008000u) >> 14) |
                     ((d[2] & 0x80008000u) >> 13) | ((d[3] & 0x80008000u) >> 12);
  const uint32_t eb = (t & 0xFu) | ((t >> 12) & 0xF0u);
  const float sc = __uint_as_float((eb - 128u + 127u - 14u) << 23);   // 2^(e - 14)
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float lo = (float)((int32_t)(d[m] << 17) >> 17);
    const float hi = (float)((int32_t)(d[m] << 1) >> 17);
    acc[m >> 1][2 * (m & 1)] = __builtin_fmaf(lo, sc, acc[m >> 1][2 * (m & 1)]);
    acc[m >> 1][2 * (m & 1) + 1] = __builtin_fmaf(hi, sc, acc[m >> 1][2 * (m & 1) + 1]);
  }
}

}  // namespace moe
