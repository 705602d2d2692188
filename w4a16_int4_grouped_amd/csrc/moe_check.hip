// Data checks behind MOE_W4A16_VALIDATE=1. The layer kernels never fault on
// bad index data: they drop ids outside the expert range, clamp masked_m,
// take one expert per 128-row contiguous block and skip rows of any other.
// These kernels count such entries so that the host can report them (it
// reads the counts back and synchronises; the layer itself never does).
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ void add_wave_count(int v, int32_t* bad) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0 && v) atomicAdd(bad, v);
}

// *bad += #{i < n : v[i] outside [lo, hi)}
__global__ __launch_bounds__(256) void count_outside(const int32_t* __restrict__ v, int64_t n, int lo,
                                                     int hi, int32_t* __restrict__ bad) {
  int c = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int x = v[i];
    c += x < lo || x >= hi;
  }
  add_wave_count(c, bad);
}

// *bad += 128-row blocks of m_indices whose non-negative entries are not all
// equal (one wave per block, two rows per lane).
__global__ __launch_bounds__(64) void count_mixed_blocks(const int32_t* __restrict__ m,
                                                         int32_t* __restrict__ bad) {
  const int32_t* blk = m + (size_t)blockIdx.x * 128;
  const int a = blk[threadIdx.x], b = blk[threadIdx.x + 64];
  int lo = INT32_MAX, hi = -1;
  if (a >= 0) { lo = a; hi = a; }
  if (b >= 0) { lo = min(lo, b); hi = max(hi, b); }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, __shfl_xor(lo, o, 64));
    hi = max(hi, __shfl_xor(hi, o, 64));
  }
  if (threadIdx.x == 0 && hi >= 0 && lo != hi) atomicAdd(bad, 1);
}

// Pairing of m_indices and row_src: a pad row (m < 0) has row_src -1, a
// row's source lies in [0, n_flat), and no flat row is the source of two
// rows. seen[n_flat] must be zero on entry.
__global__ __launch_bounds__(256) void count_row_src(const int32_t* __restrict__ m,
                                                     const int32_t* __restrict__ src, int M_pad,
                                                     int n_flat, int32_t* __restrict__ seen,
                                                     int32_t* __restrict__ bad) {
  int c = 0;
  for (int p = blockIdx.x * 256 + threadIdx.x; p < M_pad; p += gridDim.x * 256) {
    const int e = m[p], f = src[p];
    if (e < 0)
      c += f != -1;
    else if (f < 0 || f >= n_flat)
      c += 1;
    else
      c += atomicAdd(&seen[f], 1) > 0;
  }
  add_wave_count(c, bad);
}

int grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (int)(b < 2048 ? (b > 0 ? b : 1) : 2048);
}

}  // namespace

hipError_t launch_count_outside(const int32_t* v, int64_t n, int lo, int hi, int32_t* bad, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(count_outside, dim3(grid_for(n)), dim3(256), 0, s, v, n, lo, hi, bad);
  return hipGetLastError();
}

hipError_t launch_count_mixed_blocks(const int32_t* m_indices, int M_pad, int32_t* bad, hipStream_t s) {
  if (M_pad <= 0) return hipSuccess;
  if (M_pad % 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(count_mixed_blocks, dim3(M_pad / 128), dim3(64), 0, s, m_indices, bad);
  return hipGetLastError();
}

hipError_t launch_count_row_src(const int32_t* m_indices, const int32_t* row_src, int M_pad, int n_flat,
                                int32_t* seen, int32_t* bad, hipStream_t s) {
  if (M_pad <= 0) return hipSuccess;
  hipError_t e = launch_zero_i32(seen, (size_t)n_flat, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(count_row_src, dim3(grid_for(M_pad)), dim3(256), 0, s, m_indices, row_src, M_pad,
                     n_flat, seen, bad);
  return hipGetLastError();
}

}  // namespace moe
