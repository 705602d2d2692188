// Token -> expert alignment for the indexed layout, and the row gather that
// produces the contiguous layout (Chord page, "Grouped SM90 kernels", Fig. 3:
// the indexed layout keeps activations unpadded and carries the padding as
// sentinels in the routing indices).
//
// The result must be bit-exact and deterministic, so rows are never placed
// by atomic order. Rows are placed in rounds of consecutive flat indices,
// one 64-row slice per wave; a row's slot is
//   (next free slot of its expert before the round)
//   + (rows of that expert in earlier waves of the round)
//   + (rows of that expert in earlier lanes of its wave),
// which is the stable order by flat index t*topk + j.
//
// Two paths:
//   small (decode-sized routings, up to 4096 rows): one workgroup of 16
//     waves counts, scans, fills the padding and places every row in a
//     single launch;
//   large: per-chunk counts (the chunk workgroups also write the sentinel
//     into every slot), a one-workgroup scan over experts (which also turns
//     the chunk counts into per-chunk prefixes), then one 4-wave workgroup
//     per chunk places that chunk's rows.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kCountThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kScanLoads = 32;   // chunk counts an expert's thread loads at once in the scan
// One-workgroup path limits. Above 4096 rows the multi-workgroup path is
// faster (the one-workgroup path places 1024 rows per round, about 1.7 us
// each).
constexpr int kSmallMaxRows = 4096;
constexpr int kSmallMaxExperts = 512;

// Lanes of this wave routed to the same expert as this lane (e < 0: none).
// Matches the key e + 1 bit by bit: one ballot per key bit (nbits covers
// 0 .. E), so the cost does not grow with the number of distinct experts in
// the wave.
__device__ __forceinline__ uint64_t match_peers(int e, int nbits) {
  const int key = e + 1;
  uint64_t m = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return e >= 0 ? m : 0ull;
}

// Key bits for experts 0 .. E-1 plus "none".
__device__ __forceinline__ int key_bits(int E) { return 32 - __builtin_clz((unsigned)E); }

// The local expert of flat row f: its id, or with an expert map (one GPU's
// share of Eg global experts) map[id]; -1 when the row has no expert here.
__device__ __forceinline__ int local_expert(const int32_t* __restrict__ ids, int f,
                                            const int32_t* __restrict__ map, int Eg, int E) {
  int e = ids[f];
  if (map) e = (e >= 0 && e < Eg) ? map[e] : -1;
  return (e >= 0 && e < E) ? e : -1;
}

// Places flat rows [lo, hi) stably. next[e] (LDS) holds expert e's next free
// slot and is advanced; cnt (LDS, NWAVES x E) must be zero on entry and is
// zero on exit. Called by all NWAVES*64 threads of the workgroup.
template <int NWAVES>
__device__ void place_rows(const int32_t* __restrict__ ids, const int32_t* __restrict__ map, int Eg,
                           int lo, int hi, int E, int32_t* next, int32_t* cnt,
                           int32_t* __restrict__ sorted_ids, int32_t* __restrict__ slot_of) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  for (int r0 = lo; r0 < hi; r0 += NWAVES * 64) {
    const int f = r0 + (int)threadIdx.x;
    const int e = f < hi ? local_expert(ids, f, map, Eg, E) : -1;
    const uint64_t peers = match_peers(e, key_bits(E));
    const int rank = __popcll(peers & below);
    const bool leader = e >= 0 && rank == 0;
    if (leader) cnt[w * E + e] = __popcll(peers);
    __syncthreads();
    if (e >= 0) {
      int pos = next[e] + rank;
      for (int w2 = 0; w2 < w; ++w2) pos += cnt[w2 * E + e];
      sorted_ids[pos] = f;
      slot_of[f] = pos;
    } else if (f < hi) {
      slot_of[f] = -1;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&next[e], __popcll(peers));
      cnt[w * E + e] = 0;
    }
    __syncthreads();
  }
}

// Exclusive scan of padded[0..E) into padded[] itself and offsets[], with
// padded[E] = offsets[E] = total (wave 0 only; each lane owns a run).
__device__ void scan_experts(int32_t* padded, int32_t* offsets, int E) {
  if (threadIdx.x >= 64) return;
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
    const int pe = padded[e];
    offsets[e] = run;
    padded[e] = run;
    run += pe;
  }
  if (lane == 63) {
    offsets[E] = run;
    padded[E] = run;
  }
}

// Sentinels, the block -> expert map and the header. Every slot of
// sorted_ids gets the sentinel (coalesced, all threads; skipped when a
// many-workgroup kernel before this one wrote them); placement, which runs
// after a barrier or in a later kernel, overwrites the slots that hold rows.
// start[0..E] holds the scanned offsets. (The placement also writes
// slot_of[f], the slot of flat row f or -1 for a dropped row, which the
// combine reads.)
__device__ void fill_padding(int32_t* routing, const int32_t* start, int E, int B, int T, int topk,
                             int cap, int nblocks, int nchunks, int32_t* sorted_ids,
                             int32_t* block_expert, bool fill_sentinels) {
  const int sentinel = T * topk;
  const int total = start[E];
  if (fill_sentinels)
    for (int q = threadIdx.x; q < cap; q += blockDim.x) sorted_ids[q] = sentinel;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int s0 = start[e], s1 = start[e + 1];
    for (int b = s0 / B; b < s1 / B; ++b) block_expert[b] = e;
  }
  for (int b = total / B + threadIdx.x; b < nblocks; b += blockDim.x) block_expert[b] = -1;
  if (threadIdx.x == 0) {
    routing[HDR_MAGIC] = kRoutingMagic;
    routing[HDR_BLOCK] = B;
    routing[HDR_E] = E;
    routing[HDR_T] = T;
    routing[HDR_TOPK] = topk;
    routing[HDR_CAP] = cap;
    routing[HDR_NBLOCKS] = nblocks;
    routing[HDR_TOTAL] = total;
    routing[HDR_NCHUNKS] = nchunks;
  }
}

// ---- small path: everything in one workgroup ------------------------------
// Thread t owns flat rows t, t + 1024, ... (at most kSmallRounds of them),
// loaded once into registers for both the count and the placement.
constexpr int kSmallRounds = kSmallMaxRows / 1024;

__global__ __launch_bounds__(1024) void align_small(const int32_t* __restrict__ ids,
                                                    const int32_t* __restrict__ map, int Eg, int E, int B,
                                                    int T, int topk, int cap, int nblocks,
                                                    int32_t* __restrict__ routing,
                                                    int64_t off_counts, int64_t off_offsets,
                                                    int64_t off_sorted, int64_t off_be,
                                                    int64_t off_slot_of) {
  extern __shared__ int32_t smem[];
  int32_t* hist = smem;                  // [E + 1]: counts, then next free slot
  int32_t* start = smem + (E + 1);       // [E + 1]: padded counts, then offsets
  int32_t* cnt = smem + 2 * (E + 1);     // [16][E]
  int32_t* counts = routing + off_counts;
  int32_t* sorted_ids = routing + off_sorted;
  const int n = T * topk;
  const int rounds = (n + 1023) / 1024;
  int my_e[kSmallRounds];
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r) {
    const int f = r * 1024 + (int)threadIdx.x;
    my_e[r] = (r < rounds && f < n) ? local_expert(ids, f, map, Eg, E) : -1;
  }
  for (int i = threadIdx.x; i < 2 * (E + 1) + 16 * E; i += 1024) smem[i] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r)
    if (my_e[r] >= 0) atomicAdd(&hist[my_e[r]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 1024) start[e] = (hist[e] + B - 1) / B * B;
  __syncthreads();
  scan_experts(start, routing + off_offsets, E);
  __syncthreads();
  fill_padding(routing, start, E, B, T, topk, cap, nblocks, 0, sorted_ids, routing + off_be, true);
  for (int e = threadIdx.x; e < E; e += 1024) {
    counts[e] = hist[e];
    hist[e] = start[e];   // next free slot
  }
  __syncthreads();   // sentinels stored before any row overwrites its slot

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r) {
    if (r >= rounds) break;   // uniform
    const int e = my_e[r];
    const uint64_t peers = match_peers(e, key_bits(E));
    const int rank = __popcll(peers & below);
    const bool leader = e >= 0 && rank == 0;
    if (leader) cnt[w * E + e] = __popcll(peers);
    __syncthreads();
    const int f = r * 1024 + (int)threadIdx.x;
    if (e >= 0) {
      int pos = hist[e] + rank;
      for (int w2 = 0; w2 < w; ++w2) pos += cnt[w2 * E + e];
      sorted_ids[pos] = f;
      routing[off_slot_of + f] = pos;
    } else if (f < n) {
      routing[off_slot_of + f] = -1;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&hist[e], __popcll(peers));
      cnt[w * E + e] = 0;
    }
    __syncthreads();
  }
}

// ---- large path ------------------------------------------------------------
// Per-chunk expert counts. The chunk workgroups also write the sentinel
// into every slot of sorted_ids (cap of them), so that the one-workgroup
// scan after them does not have to.
__global__ __launch_bounds__(kCountThreads) void align_count(const int32_t* __restrict__ ids,
                                                             const int32_t* __restrict__ map, int Eg,
                                                             int n, int E,
                                                             int32_t* __restrict__ chunk_hist,
                                                             int32_t* __restrict__ sorted_ids, int cap) {
  extern __shared__ int32_t hist[];
  for (int q = blockIdx.x * kCountThreads + threadIdx.x; q < cap; q += gridDim.x * kCountThreads)
    sorted_ids[q] = n;   // the sentinel T * topk
  for (int i = threadIdx.x; i < E; i += kCountThreads) hist[i] = 0;
  __syncthreads();
  const int base = blockIdx.x * kAlignChunk;
  for (int j = threadIdx.x; j < kAlignChunk; j += kCountThreads) {
    const int f = base + j;
    if (f < n) {
      const int e = local_expert(ids, f, map, Eg, E);
      if (e >= 0) atomicAdd(&hist[e], 1);
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
  int32_t* chunk_hist = routing + off_scratch;
  // per expert: exclusive prefix over chunks (in place) and the total
  for (int e = threadIdx.x; e < E; e += kScanThreads) {
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += kScanLoads) {   // kScanLoads independent loads in flight
      int h[kScanLoads];
#pragma unroll
      for (int i = 0; i < kScanLoads; ++i)
        h[i] = c0 + i < nchunks ? chunk_hist[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanLoads; ++i) {
        if (c0 + i < nchunks) chunk_hist[(size_t)(c0 + i) * E + e] = run;
        run += h[i];
      }
    }
    counts[e] = run;
    padded[e] = (run + B - 1) / B * B;
  }
  __syncthreads();
  scan_experts(padded, routing + off_offsets, E);
  __syncthreads();
  fill_padding(routing, padded, E, B, T, topk, cap, nblocks, nchunks, routing + off_sorted,
               routing + off_be, nchunks == 0);   // align_count wrote them when it ran
}

template <int NWAVES>
__global__ __launch_bounds__(NWAVES * 64) void align_scatter(const int32_t* __restrict__ ids,
                                                            const int32_t* __restrict__ map, int Eg,
                                                            int n, int E, int32_t* __restrict__ routing,
                                                            int64_t off_offsets, int64_t off_sorted,
                                                            int64_t off_slot_of, int64_t off_scratch) {
  extern __shared__ int32_t smem[];
  int32_t* next = smem;          // [E]
  int32_t* cnt = smem + E;       // [NWAVES][E]
  const int chunk = blockIdx.x;
  const int32_t* offsets = routing + off_offsets;
  const int32_t* prefix = routing + off_scratch + (size_t)chunk * E;
  for (int e = threadIdx.x; e < E; e += NWAVES * 64) next[e] = offsets[e] + prefix[e];
  for (int i = threadIdx.x; i < NWAVES * E; i += NWAVES * 64) cnt[i] = 0;
  __syncthreads();
  const int lo = chunk * kAlignChunk;
  place_rows<NWAVES>(ids, map, Eg, lo, min(n, lo + kAlignChunk), E, next, cnt, routing + off_sorted,
                     routing + off_slot_of);
}

// The row gather, one launch with two kinds of workgroups, dealt
// alternately (token, slot, token, ...) so that both kinds run together
// from start to end.
//  - Token workgroups: one wave per token reads the token's row once and
//    writes it to the slot of each of its routed rows (slot_of), so each x
//    row crosses HBM once.
//  - Slot workgroups: 64 slots each. Wave 0 writes m_indices and row_src of
//    the 64; the padding slots among them below the routing's padded total
//    get a zero row in a_out, wave w zeroing padding rows w, w + 4, ... so
//    that a slot workgroup's rows are spread over its four waves.
// Slots at or past the padded total are outside the contiguous layout:
// a_out is not written there. a_out rows are written with nontemporal
// stores (nothing here reads them back). Every slot read from the routing
// is checked against the capacity before it is written to.
constexpr int kPermutePieces = 4;   // 1 KB pieces of a row a wave holds at once

__global__ __launch_bounds__(256) void permute_rows(const uint16_t* __restrict__ x, int T, int topk, int H,
                                                    int B, int sentinel, int cap, int ntok_wg,
                                                    int nslot_wg, const int32_t* __restrict__ hdr,
                                                    const int32_t* __restrict__ sorted_ids,
                                                    const int32_t* __restrict__ slot_of,
                                                    const int32_t* __restrict__ block_expert,
                                                    uint16_t* __restrict__ a_out,
                                                    int32_t* __restrict__ m_indices,
                                                    int32_t* __restrict__ row_src) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H8 = H / 8;   // 16-byte pieces of a row
  // workgroup i: while both kinds last, even i the token workgroup i/2 and
  // odd i the slot workgroup i/2; then the rest of the larger kind
  const int i = (int)blockIdx.x, both = min(ntok_wg, nslot_wg);
  bool token_wg;
  int idx;
  if (i < 2 * both) {
    token_wg = !(i & 1);
    idx = i >> 1;
  } else {
    token_wg = ntok_wg > nslot_wg;
    idx = i - both;
  }
  if (token_wg) {
    const int t = idx * 4 + wave;
    if (t >= T) return;
    int my_slot = -1;   // lane j < topk: the slot of row (t, j), -1 if dropped
    if (lane < topk) {
      const int q = slot_of[(size_t)t * topk + lane];
      my_slot = (q >= 0 && q < cap) ? q : -1;
    }
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (size_t)t * H);
    for (int c0 = 0; c0 < H8; c0 += 64 * kPermutePieces) {
      u32x4_t v[kPermutePieces];
#pragma unroll
      for (int u = 0; u < kPermutePieces; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < H8) v[u] = src[c];
      }
      for (int j = 0; j < topk; ++j) {
        const int q = __builtin_amdgcn_readlane(my_slot, j);
        if (q < 0) continue;
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(a_out + (size_t)q * H);
#pragma unroll
        for (int u = 0; u < kPermutePieces; ++u) {
          const int c = c0 + u * 64 + lane;
          if (c < H8) __builtin_nontemporal_store(v[u], dst + c);
        }
      }
    }
    return;
  }
  const int base = idx * 64;   // this workgroup's first slot
  const int p = base + lane;
  bool pad = false;
  if (p < cap) {
    const int f = sorted_ids[p];
    const bool valid = f >= 0 && f < sentinel;
    if (wave == 0) {
      if (m_indices) m_indices[p] = valid ? block_expert[p / B] : -1;
      if (row_src) row_src[p] = valid ? f : -1;
    }
    pad = !valid;
  }
  if (!a_out) return;   // uniform: a kernel argument
  const int total = min(max(hdr[HDR_TOTAL], 0), cap);
  uint64_t pads = __ballot(pad && p < total);
  const u32x4_t z = {0u, 0u, 0u, 0u};
  for (int k = 0; pads; ++k) {
    const int l = __builtin_ctzll(pads);
    pads &= pads - 1;
    if ((k & 3) != wave) continue;
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(a_out + (size_t)(base + l) * H);
    for (int c = lane; c < H8; c += 64) __builtin_nontemporal_store(z, dst + c);
  }
}

}  // namespace

hipError_t launch_align(const int32_t* topk_ids, int T, int topk, int E, const RoutingLayout& L,
                        int32_t* routing, hipStream_t s, const int32_t* map, int Eg) {
  const int n = T * topk;
  if (n <= kSmallMaxRows && E <= kSmallMaxExperts) {
    const size_t lds = (size_t)(2 * (E + 1) + 16 * E) * sizeof(int32_t);
    hipLaunchKernelGGL(align_small, dim3(1), dim3(1024), lds, s, topk_ids, map, Eg, E, L.block, T, topk,
                       L.cap,
                       L.nblocks, routing, L.off_counts, L.off_offsets, L.off_sorted,
                       L.off_block_expert, L.off_slot_of);
    return hipGetLastError();
  }
  const size_t lds_e = (size_t)E * sizeof(int32_t);
  if (L.nchunks > 0) {
    hipLaunchKernelGGL(align_count, dim3(L.nchunks), dim3(kCountThreads), lds_e, s, topk_ids, map, Eg,
                       n, E, routing + L.off_scratch, routing + L.off_sorted, L.cap);
  }
  hipLaunchKernelGGL(align_scan, dim3(1), dim3(kScanThreads), lds_e + sizeof(int32_t), s, routing,
                     E, L.block, T, topk, L.nchunks, L.cap, L.nblocks, L.off_counts, L.off_offsets,
                     L.off_sorted, L.off_block_expert, L.off_scratch);
  if (L.nchunks > 0) {
    if (E <= 2048)   // 4 waves per chunk: 5 E ints of LDS
      hipLaunchKernelGGL(align_scatter<4>, dim3(L.nchunks), dim3(256), 5 * lds_e, s, topk_ids, map, Eg,
                         n, E,
                         routing, L.off_offsets, L.off_sorted, L.off_slot_of, L.off_scratch);
    else
      hipLaunchKernelGGL(align_scatter<1>, dim3(L.nchunks), dim3(64), 2 * lds_e, s, topk_ids, map, Eg,
                         n, E,
                         routing, L.off_offsets, L.off_sorted, L.off_slot_of, L.off_scratch);
  }
  return hipGetLastError();
}

hipError_t launch_permute(const uint16_t* x, int T, int topk, int H, const RoutingLayout& L,
                          const int32_t* routing, uint16_t* a_out, int32_t* m_indices,
                          int32_t* row_src, hipStream_t s) {
  if (L.cap == 0) return hipSuccess;
  const int ntok_wg = a_out ? (T + 3) / 4 : 0;
  const int nslot_wg = (L.cap + 63) / 64;
  hipLaunchKernelGGL(permute_rows, dim3(ntok_wg + nslot_wg), dim3(256), 0, s, x, T, topk, H, L.block,
                     T * topk, L.cap, ntok_wg, nslot_wg, routing + L.off_header, routing + L.off_sorted,
                     routing + L.off_slot_of, routing + L.off_block_expert, a_out, m_indices, row_src);
  return hipGetLastError();
}

}  // namespace moe
