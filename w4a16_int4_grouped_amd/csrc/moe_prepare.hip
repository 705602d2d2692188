// Load-time weight repack, the inspection dequantiser, and the small
// elementwise kernels around the combine.
//
// Repack: canonical int32 [E][N][K/8] words and BF16 [E][N][K/32] scales ->
// the prepared, MFMA-fragment-major layout of moe_layout.h (Chord page,
// "Indexed kernels": layouts are fixed at load, before packing; "Grouped SM90
// kernels": the forward path reads pre-permuted INT4 bytes and re-tiled
// scales). Each lane's 16 bytes of a prepared tile are four consecutive
// canonical words of one row, so the repack is a 16-byte gather; no nibble
// moves inside a word and words and scales keep their canonical values.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void repack_words(const uint32_t* __restrict__ canon,
                                                    u32x4_t* __restrict__ prep, int N, int K,
                                                    int RG, int Kc, int interleave_I,
                                                    size_t total) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  size_t t = idx >> 6;
  const int mt = (int)(t & 3);
  t >>= 2;
  const int kc = (int)(t % Kc);
  t /= Kc;
  const int rg = (int)(t % RG);
  const size_t e = t / RG;
  const int row = canon_row(rg * kMT + mt, lane & 15, interleave_I);
  const int kword = kc * 16 + (lane >> 4) * 4;
  u32x4_t v = {0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};   // padding: q = 8
  if (row < N && kword * 8 < K)
    v = *reinterpret_cast<const u32x4_t*>(canon + (e * N + row) * (size_t)(K / 8) + kword);
  prep[idx] = v;
}

__global__ __launch_bounds__(256) void repack_scales(const uint16_t* __restrict__ canon,
                                                     uint16_t* __restrict__ prep, int N, int K,
                                                     int RG, int Kc, int interleave_I,
                                                     size_t total, int32_t* __restrict__ bad) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int mt = (int)(idx & 3);
  const int lane = (int)((idx >> 2) & 63);
  size_t t = idx >> 8;
  const int kc = (int)(t % Kc);
  t /= Kc;
  const int rg = (int)(t % RG);
  const size_t e = t / RG;
  const int row = canon_row(rg * kMT + mt, lane & 15, interleave_I);
  const int grp = kc * 4 + (lane >> 4);
  uint16_t s = 0;
  if (row < N && grp < K / 32) {
    s = canon[(e * N + row) * (size_t)(K / 32) + grp];
    // NaN, infinity or |s| >= 2^117 (where -1032 s would overflow) are rejected
    if ((s & 0x7FFF) >= 0x7A00) atomicOr(bad, 1);
  }
  prep[idx] = s;
}

// One thread per prepared lane-fragment (4 words = 32 weights of one row).
__global__ __launch_bounds__(256) void dequant_expert(const u32x4_t* __restrict__ wq,
                                                      const uint16_t* __restrict__ wsc,
                                                      uint16_t* __restrict__ out, int e, int N,
                                                      int K, int RG, int Kc, int interleave_I) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= RG * Kc * kMT * 64) return;
  const int lane = idx & 63;
  int t = idx >> 6;
  const int mt = t & 3;
  t >>= 2;
  const int kc = t % Kc;
  const int rg = t / Kc;
  const size_t tile = ((size_t)e * RG + rg) * Kc + kc;
  const u32x4_t A = wq[(tile * kMT + mt) * 64 + lane];
  const GroupScale gs = group_scale(__uint_as_float((uint32_t)wsc[(tile * 64 + lane) * kMT + mt] << 16));
  const int row = canon_row(rg * kMT + mt, lane & 15, interleave_I);
  if (row >= N) return;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int k0 = kc * kKC + (lane >> 4) * 32 + g * 8;
    if (k0 < K)
      *reinterpret_cast<u32x4_t*>(out + (size_t)row * K + k0) = dq8_exact(A[g], gs);
  }
}

__global__ __launch_bounds__(256) void zero_u32x4(u32x4_t* __restrict__ p, size_t n4) {
  const u32x4_t z = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256)
    p[i] = z;
}

__global__ __launch_bounds__(256) void zero_tail(uint32_t* __restrict__ p, size_t from, size_t n) {
  const size_t i = from + (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

inline unsigned grid_for(size_t n, size_t per_block, unsigned cap) {
  size_t g = (n + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (unsigned)(g > cap ? cap : g);
}

hipError_t zero_words(uint32_t* p, size_t n, hipStream_t s) {
  const size_t n4 = n / 4;
  if (n4) hipLaunchKernelGGL(zero_u32x4, dim3(grid_for(n4, 256, 8192)), dim3(256), 0, s,
                             reinterpret_cast<u32x4_t*>(p), n4);
  if (n4 * 4 < n) hipLaunchKernelGGL(zero_tail, dim3(1), dim3(256), 0, s, p, n4 * 4, n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_repack(const MatLayout& m, const int32_t* words, const uint16_t* scales,
                         char* prepared, int32_t* bad_scale_flag, hipStream_t s) {
  const size_t nw = (size_t)m.E * m.RG * m.Kc * kMT * 64;
  hipLaunchKernelGGL(repack_words, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(words),
                     reinterpret_cast<u32x4_t*>(prepared + m.off_words), m.N, m.K, m.RG, m.Kc,
                     m.interleave_I, nw);
  const size_t ns = (size_t)m.E * m.RG * m.Kc * 64 * kMT;
  hipLaunchKernelGGL(repack_scales, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, s, scales,
                     reinterpret_cast<uint16_t*>(prepared + m.off_scales), m.N, m.K, m.RG, m.Kc,
                     m.interleave_I, ns, bad_scale_flag);
  return hipGetLastError();
}

hipError_t launch_dequant_expert(const MatLayout& m, const char* prepared, int expert,
                                 uint16_t* out, hipStream_t s) {
  const int n = m.RG * m.Kc * kMT * 64;
  hipLaunchKernelGGL(dequant_expert, dim3((n + 255) / 256), dim3(256), 0, s,
                     reinterpret_cast<const u32x4_t*>(prepared + m.off_words),
                     reinterpret_cast<const uint16_t*>(prepared + m.off_scales), out, expert, m.N,
                     m.K, m.RG, m.Kc, m.interleave_I);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int32_t* p, size_t n, hipStream_t s) {
  return zero_words(reinterpret_cast<uint32_t*>(p), n, s);
}

}  // namespace moe
