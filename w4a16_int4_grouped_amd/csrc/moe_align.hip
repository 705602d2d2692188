// Token -> expert alignment for the indexed layout, and the row gather that
// produces the contiguous layout (Chord page, "Grouped SM90 kernels", Fig. 3:
// the indexed layout keeps activations unpadded and carries the padding as
// sentinels in the routing indices).
//
// The result must be bit-exact and deterministic, so rows are never placed
// by atomic order. Three passes over fixed chunks of kAlignChunk flat rows:
//   1. count:   per-chunk expert histograms (LDS atomics; counts only);
//   2. scan:    per expert, an exclusive prefix over chunks; padded counts
//               ceil(c/B)*B; an exclusive scan over experts -> offsets;
//               sentinel fill of pad slots; the block -> expert map;
//   3. scatter: one wave per chunk walks its rows in order, 64 at a time;
//               a row's slot is offsets[e] + (rows of e in earlier chunks) +
//               (rows of e earlier in this chunk), i.e. a stable order by
//               flat index t*topk + j.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kCountThreads = 256;
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kCountThreads) void align_count(const int32_t* __restrict__ ids,
                                                             int n, int E,
                                                             int32_t* __restrict__ chunk_hist) {
  extern __shared__ int32_t hist[];
  for (int i = threadIdx.x; i < E; i += kCountThreads) hist[i] = 0;
  __syncthreads();
  const int base = blockIdx.x * kAlignChunk;
  for (int j = threadIdx.x; j < kAlignChunk; j += kCountThreads) {
    const int f = base + j;
    if (f < n) {
      const int e = ids[f];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += kCountThreads)
    chunk_hist[(size_t)blockIdx.x * E + i] = hist[i];
}

__global__ __launch_bounds__(kScanThreads) void align_scan(int32_t* __restrict__ routing, int E,
                                                           int B, int T, int topk, int nchunks,
                                                           int cap, int nblocks,
                                                           int64_t off_counts, int64_t off_offsets,
                                                           int64_t off_sorted, int64_t off_be,
                                                           int64_t off_scratch) {
  extern __shared__ int32_t padded[];   // [E + 1]
  int32_t* counts = routing + off_counts;
  int32_t* offsets = routing + off_offsets;
  int32_t* sorted_ids = routing + off_sorted;
  int32_t* block_expert = routing + off_be;
  int32_t* chunk_hist = routing + off_scratch;
  const int sentinel = T * topk;

  // per expert: exclusive prefix over chunks (in place) and the total
  for (int e = threadIdx.x; e < E; e += kScanThreads) {
    int run = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int h = chunk_hist[(size_t)c * E + e];
      chunk_hist[(size_t)c * E + e] = run;
      run += h;
    }
    counts[e] = run;
    padded[e] = (run + B - 1) / B * B;
  }
  __syncthreads();

  // exclusive scan of padded counts over experts: wave 0, each lane owns a
  // contiguous run of experts
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (E + 63) / 64;
    const int lo = min(lane * per, E), hi = min(lo + per, E);
    int sum = 0;
    for (int e = lo; e < hi; ++e) sum += padded[e];
    int incl = sum;
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    int run = incl - sum;
    for (int e = lo; e < hi; ++e) {
      const int p = padded[e];
      offsets[e] = run;
      padded[e] = run;       // reuse as the start offset
      run += p;
    }
    if (lane == 63) {
      offsets[E] = run;
      padded[E] = run;
      routing[HDR_TOTAL] = run;
    }
  }
  __syncthreads();
  const int total = padded[E];

  // sentinel in every pad slot, block -> expert map
  for (int e = threadIdx.x; e < E; e += kScanThreads) {
    const int start = padded[e], end = padded[e + 1];
    for (int p = start + counts[e]; p < end; ++p) sorted_ids[p] = sentinel;
    for (int b = start / B; b < end / B; ++b) block_expert[b] = e;
  }
  for (int p = total + threadIdx.x; p < cap; p += kScanThreads) sorted_ids[p] = sentinel;
  for (int b = total / B + threadIdx.x; b < nblocks; b += kScanThreads) block_expert[b] = -1;
  if (threadIdx.x == 0) {
    routing[HDR_MAGIC] = kRoutingMagic;
    routing[HDR_BLOCK] = B;
    routing[HDR_E] = E;
    routing[HDR_T] = T;
    routing[HDR_TOPK] = topk;
    routing[HDR_CAP] = cap;
    routing[HDR_NBLOCKS] = nblocks;
    routing[HDR_NCHUNKS] = nchunks;
  }
}

__global__ __launch_bounds__(64) void align_scatter(const int32_t* __restrict__ ids, int n, int E,
                                                    int32_t* __restrict__ routing,
                                                    int64_t off_offsets, int64_t off_sorted,
                                                    int64_t off_scratch) {
  extern __shared__ int32_t next[];   // [E]: next free slot of each expert in this chunk
  const int lane = threadIdx.x;
  const int chunk = blockIdx.x;
  const int32_t* offsets = routing + off_offsets;
  const int32_t* prefix = routing + off_scratch + (size_t)chunk * E;
  int32_t* sorted_ids = routing + off_sorted;
  for (int e = lane; e < E; e += 64) next[e] = offsets[e] + prefix[e];
  __syncthreads();
  const int base = chunk * kAlignChunk;
  for (int sb = 0; sb < kAlignChunk; sb += 64) {
    const int f = base + sb + lane;
    int e = -1;
    if (f < n) {
      e = ids[f];
      if (e < 0 || e >= E) e = -1;
    }
    // lanes of this 64-row step routed to the same expert
    uint64_t peers = 0;
    for (int j = 0; j < 64; ++j) {
      const int ej = __shfl(e, j, 64);
      peers |= (uint64_t)(ej == e) << j;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & below);
    const int cnt = __popcll(peers);
    int slot = 0;
    if (e >= 0) slot = next[e] + rank;
    __syncthreads();
    if (e >= 0) {
      sorted_ids[slot] = f;
      if (rank == cnt - 1) next[e] = slot + 1;   // one writer per expert
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void permute_rows(const uint16_t* __restrict__ x, int topk, int H,
                                                    int B, int sentinel,
                                                    const int32_t* __restrict__ sorted_ids,
                                                    const int32_t* __restrict__ block_expert,
                                                    uint16_t* __restrict__ a_out,
                                                    int32_t* __restrict__ m_indices,
                                                    int32_t* __restrict__ row_src) {
  const int p = blockIdx.x;
  const int f = sorted_ids[p];
  const bool valid = f >= 0 && f < sentinel;
  if (a_out) {
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(a_out + (size_t)p * H);
    if (valid) {   // uniform over the workgroup
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (size_t)(f / topk) * H);
      for (int c = threadIdx.x; c < H / 8; c += 256) dst[c] = src[c];
    } else {
      const u32x4_t z = {0u, 0u, 0u, 0u};
      for (int c = threadIdx.x; c < H / 8; c += 256) dst[c] = z;
    }
  }
  if (threadIdx.x == 0) {
    if (m_indices) m_indices[p] = valid ? block_expert[p / B] : -1;
    if (row_src) row_src[p] = valid ? f : -1;
  }
}

}  // namespace

hipError_t launch_align(const int32_t* topk_ids, int T, int topk, int E, const RoutingLayout& L,
                        int32_t* routing, hipStream_t s) {
  const int n = T * topk;
  const size_t lds_e = (size_t)E * sizeof(int32_t);
  if (L.nchunks > 0) {
    hipLaunchKernelGGL(align_count, dim3(L.nchunks), dim3(kCountThreads), lds_e, s, topk_ids, n, E,
                       routing + L.off_scratch);
  }
  hipLaunchKernelGGL(align_scan, dim3(1), dim3(kScanThreads), lds_e + sizeof(int32_t), s, routing,
                     E, L.block, T, topk, L.nchunks, L.cap, L.nblocks, L.off_counts, L.off_offsets,
                     L.off_sorted, L.off_block_expert, L.off_scratch);
  if (L.nchunks > 0) {
    hipLaunchKernelGGL(align_scatter, dim3(L.nchunks), dim3(64), lds_e, s, topk_ids, n, E, routing,
                       L.off_offsets, L.off_sorted, L.off_scratch);
  }
  return hipGetLastError();
}

hipError_t launch_permute(const uint16_t* x, int T, int topk, int H, const RoutingLayout& L,
                          const int32_t* routing, uint16_t* a_out, int32_t* m_indices,
                          int32_t* row_src, hipStream_t s) {
  if (L.cap == 0) return hipSuccess;
  hipLaunchKernelGGL(permute_rows, dim3(L.cap), dim3(256), 0, s, x, topk, H, L.block, T * topk,
                     routing + L.off_sorted, routing + L.off_block_expert, a_out, m_indices,
                     row_src);
  return hipGetLastError();
}

}  // namespace moe
