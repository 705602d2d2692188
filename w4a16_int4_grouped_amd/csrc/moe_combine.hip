// Top-k-weighted combine: out[t] = sum_j w[t, j] * y(t, j) (reading of the
// layer's combine: the routing weight applies after the second GEMM).
//
// The second GEMM stores each routed row already weighted, w * y, at its flat
// index f = t*topk + j, as 16-bit integers with a power-of-two scale per 8
// positions (store_y16). This kernel adds a token's top-k rows in FP32 in
// ascending j and rounds once to BF16. No atomics: the accumulator of an
// atomic scatter-add is shared by workgroups on all XCDs, so every add would
// be performed past the per-XCD L2 at a fraction of the streaming rate.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

// y where v, else +0 in every lane, by a mask rather than a select, so that
// the load feeding it is not moved under a branch.
__device__ __forceinline__ f32x4_t keep_if(f32x4_t y, bool v) {
  const uint32_t m = v ? ~0u : 0u;
  f32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __uint_as_float(__float_as_uint(y[i]) & m);
  return r;
}

// One thread per (token, 8 adjacent positions of a row: one scale group, two
// groups of 4 features in the W2 epilogue's lane-contiguous order, store_y16),
// read with one 16-byte load per row. A row f is summed when
// valid[f] >= 0 (the slot of f in the indexed layout's routing; 0 for the
// contiguous layout's rows). With a routing header that does not describe
// (E, block, T*topk) nothing was computed and the result is zero, as for the
// GEMMs. A token's rows are loaded kRowBatch at a time before any is added, so
// a thread keeps up to 8 rows' loads in flight instead of one. Rows still add
// in ascending j; a skipped row (another GPU's expert) costs no read and adds
// nothing (its integers are 0, and adding 0 * scale = +0 to a sum that starts
// at +0 and never becomes -0 is exact).
constexpr int kRowBatch = 8;

__global__ __launch_bounds__(256) void combine_rows(const uint16_t* __restrict__ yq,
                                                    const int32_t* __restrict__ valid,
                                                    const int32_t* __restrict__ hdr, int E, int block,
                                                    int T, int topk, int H, int ld,
                                                    uint16_t* __restrict__ out) {
  const int t = blockIdx.y;
  const int p0 = 8 * (blockIdx.x * 256 + threadIdx.x);   // positions p0 .. p0 + 7 of the row
  // position 16q + 4mt + i of a 64-feature block holds feature 16mt + 4q + i
  const int blk = p0 & ~63, q = (p0 >> 4) & 3, mt0 = (p0 >> 2) & 3;   // mt0 is 0 or 2
  if (t >= T || blk >= H) return;
  const bool ok = !hdr || (hdr[HDR_MAGIC] == kRoutingMagic && hdr[HDR_BLOCK] == block &&
                           hdr[HDR_E] == E && hdr[HDR_T] * hdr[HDR_TOPK] == T * topk);
  f32x4_t acc[2] = {};
  if (ok) {
    const int f0 = t * topk;
    for (int j0 = 0; j0 < topk; j0 += kRowBatch) {
      // the batch's flags first (scalar loads, one wait), then its rows
      bool use[kRowBatch];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) use[u] = j0 + u < topk && valid[f0 + j0 + u] >= 0;
      u32x4_t d[kRowBatch];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        d[u] = kY16Zero;   // integers 0: adds +0
        if (use[u]) {
          const size_t idx = (size_t)(f0 + j0 + u) * ld + p0;
          d[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(yq + idx));
        }
      }
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) add_y16(acc, d[u]);
    }
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int n = blk + (mt0 + g) * 16 + q * 4;
    if (n < H) {
      u32x2_t r;
      r[0] = pack_bf16x2(acc[g][0], acc[g][1]);
      r[1] = pack_bf16x2(acc[g][2], acc[g][3]);
      *reinterpret_cast<u32x2_t*>(out + (size_t)t * H + n) = r;
    }
  }
}

// Split-K reduction of W13 fused with its SwiGLU: one thread per (routing
// slot, 4 consecutive output columns). Output column c is gate row
// rg*64 + 2*pp*16 + r and up row rg*64 + (2*pp + 1)*16 + r of the prepared
// (interleaved) order, rg = c / 32, pp = (c / 16) % 2, r = c % 16; four
// consecutive columns are four consecutive prepared rows. Partials add in
// split order, so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void splitk_swiglu(const float* __restrict__ part, int S, int64_t F,
                                                     int I, const int32_t* __restrict__ sorted_ids,
                                                     int cap, int sentinel, uint16_t* __restrict__ a,
                                                     int64_t a_ld) {
  const int I4 = I / 4;
  const int64_t n = (int64_t)cap * I4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int slot = (int)(i / I4);
    const int c = (int)(i - (int64_t)slot * I4) * 4;
    const int f = sorted_ids[slot];
    if (f < 0 || f >= sentinel) continue;
    const int rg = c >> 5, pp = (c >> 4) & 1, r = c & 15;
    const int gr = rg * 64 + 2 * pp * 16 + r, ur = gr + 16;
    f32x4_t g = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < S; ++ks) {
      const float* row = part + ((size_t)ks * F + f) * (2 * I);
      g += *reinterpret_cast<const f32x4_t*>(row + gr);
      u += *reinterpret_cast<const f32x4_t*>(row + ur);
    }
    u32x2_t v;
    v[0] = pack_bf16x2(swiglu(g[0], u[0]), swiglu(g[1], u[1]));
    v[1] = pack_bf16x2(swiglu(g[2], u[2]), swiglu(g[3], u[3]));
    *reinterpret_cast<u32x2_t*>(a + (size_t)slot * a_ld + c) = v;
  }
}

// Split-K reduction of W2 fused with the combine: one thread per (token, 4
// features); out[t] = bf16(sum over j ascending of w[t,j] * y(t,j)) with
// y = the split partials added in split order, rows with slot_of < 0 left
// out, as combine_rows does for the unsplit rows.
__global__ __launch_bounds__(256) void splitk_combine(const float* __restrict__ part, int S,
                                                      const int32_t* __restrict__ slot_of,
                                                      const int32_t* __restrict__ hdr, int E, int block,
                                                      const float* __restrict__ topk_w, int T, int topk,
                                                      int H4, u32x2_t* __restrict__ out) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (t >= T || c >= H4) return;
  const bool ok = hdr[HDR_MAGIC] == kRoutingMagic && hdr[HDR_BLOCK] == block && hdr[HDR_E] == E &&
                  hdr[HDR_T] * hdr[HDR_TOPK] == T * topk;
  const int64_t F = (int64_t)T * topk;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (ok) {
    const int64_t f0 = (int64_t)t * topk;
    for (int j = 0; j < topk; ++j) {
      // loads without a branch (split calls are grid-starved: latency, not
      // bandwidth, decides), an invalid row's reads repeating the token's
      // first row and adding bitwise zeros
      const bool v = slot_of[f0 + j] >= 0;
      const int64_t f = f0 + (v ? j : 0);
      f32x4_t y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int ks = 0; ks < S; ++ks)
        y += __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(part) + ((size_t)ks * F + f) * H4 + c);
      acc += topk_w[f] * keep_if(y, v);
    }
  }
  u32x2_t r;
  r[0] = pack_bf16x2(acc[0], acc[1]);
  r[1] = pack_bf16x2(acc[2], acc[3]);
  out[(size_t)t * H4 + c] = r;
}

// Standalone SwiGLU of the unfused step sequence: one thread per (row, 8
// columns); gate and up are the row's BF16 halves [0, I) and [I, 2I), each
// widened exactly to FP32, and the product is rounded once to BF16 (the
// same arithmetic as the fused W13 epilogue, from BF16 instead of FP32
// inputs).
__global__ __launch_bounds__(256) void swiglu_rows(const u32x4_t* __restrict__ h, int64_t rows,
                                                   int I8, u32x4_t* __restrict__ a) {
  const int64_t n = rows * I8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / I8;
    const int c = (int)(i - r * I8);
    const u32x4_t g = __builtin_nontemporal_load(h + r * 2 * I8 + c);
    const u32x4_t u = __builtin_nontemporal_load(h + r * 2 * I8 + I8 + c);
    u32x4_t o;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = pack_bf16x2(swiglu(bf16_lo(g[k]), bf16_lo(u[k])), swiglu(bf16_hi(g[k]), bf16_hi(u[k])));
    a[i] = o;
  }
}

__global__ __launch_bounds__(256) void fill_i32(int32_t* __restrict__ p, int n, int v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// One workgroup per 128-row contiguous block: the block's expert is the
// largest valid m_index in it (as the GEMMs take it); rows of that expert
// mark their row_src as written.
__global__ __launch_bounds__(128) void contiguous_valid(const int32_t* __restrict__ m_indices,
                                                        const int32_t* __restrict__ row_src, int E,
                                                        int n_flat, int32_t* __restrict__ valid) {
  __shared__ int32_t best;
  const int p = blockIdx.x * 128 + threadIdx.x;
  if (threadIdx.x == 0) best = -1;
  __syncthreads();
  const int m = m_indices[p];
  if (m >= 0 && m < E) atomicMax(&best, m);
  __syncthreads();
  const int f = row_src[p];
  if (m == best && best >= 0 && f >= 0 && f < n_flat) valid[f] = 0;
}

}  // namespace

hipError_t launch_swiglu(const uint16_t* h, int64_t rows, int I, uint16_t* a, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (I <= 0 || I % 8) return hipErrorInvalidValue;
  const int64_t n = rows * (I / 8);
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(swiglu_rows, dim3((unsigned)(blocks < 16384 ? blocks : 16384)), dim3(256), 0, s,
                     reinterpret_cast<const u32x4_t*>(h), rows, I / 8, reinterpret_cast<u32x4_t*>(a));
  return hipGetLastError();
}

hipError_t launch_splitk_swiglu(const float* part, int S, int64_t F, int I, const int32_t* sorted_ids,
                                int cap, int sentinel, uint16_t* a, int64_t a_ld, hipStream_t s) {
  if (cap <= 0) return hipSuccess;
  if (I % 32 || S < 1) return hipErrorInvalidValue;
  const int64_t n = (int64_t)cap * (I / 4);
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(splitk_swiglu, dim3((unsigned)(blocks < 16384 ? blocks : 16384)), dim3(256), 0, s,
                     part, S, F, I, sorted_ids, cap, sentinel, a, a_ld);
  return hipGetLastError();
}

hipError_t launch_splitk_combine(const float* part, int S, const int32_t* slot_of, const int32_t* hdr,
                                 int E, int block, const float* topk_w, int T, int topk, int H,
                                 uint16_t* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (H % 4 || S < 1 || !hdr) return hipErrorInvalidValue;
  const int H4 = H / 4;
  hipLaunchKernelGGL(splitk_combine, dim3((H4 + 255) / 256, T), dim3(256), 0, s, part, S, slot_of, hdr, E,
                     block, topk_w, T, topk, H4, reinterpret_cast<u32x2_t*>(out));
  return hipGetLastError();
}

hipError_t launch_combine_rows(const uint16_t* yq, int ld, const int32_t* valid,
                               const int32_t* hdr, int E, int block, int T, int topk, int H, uint16_t* out,
                               hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (ld % 64 || ld < H || H % 4) return hipErrorInvalidValue;   // rows in 64-feature blocks (store_y16)
  const int pieces = (H + 63) / 64 * 8;   // 8-position pieces of a token's row blocks
  hipLaunchKernelGGL(combine_rows, dim3((pieces + 255) / 256, T), dim3(256), 0, s, yq, valid, hdr, E,
                     block, T, topk, H, ld, out);
  return hipGetLastError();
}

hipError_t launch_contiguous_valid(const int32_t* m_indices, const int32_t* row_src, int M_pad,
                                   int E, int n_flat, int32_t* valid, hipStream_t s) {
  if (n_flat > 0)
    hipLaunchKernelGGL(fill_i32, dim3((n_flat + 255) / 256), dim3(256), 0, s, valid, n_flat, -1);
  if (M_pad > 0)
    hipLaunchKernelGGL(contiguous_valid, dim3(M_pad / 128), dim3(128), 0, s, m_indices, row_src, E,
                       n_flat, valid);
  return hipGetLastError();
}

}  // namespace moe
