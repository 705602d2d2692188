// Kernel launchers (host side). Each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_layout.h"

namespace moe {

// How the rows of one work item are found.
enum RowSet : int {
  SET_INDEXED = 0,   // expert e: slots offsets[e] .. + counts[e]
  SET_MASKED = 1,    // expert e: slots e*max_m .. + clamp(masked_m[e])
  SET_BLOCKS = 2,    // block b of block_rows slots; expert from m_indices
  SET_ROUTED = 3,    // block b of the indexed routing (block 128); expert block_expert[b]
};

// What the GEMM does with its FP32 tile.
enum Epilogue : int {
  EPI_SWIGLU = 0,    // W13: a[slot][c] = bf16(silu(gate) * up)
  EPI_COMBINE = 1,   // W2: yrows[f][n] = w[f] * y   (f from sorted_ids / row_src)
  EPI_STORE = 2,     // out[slot][n] = bf16(y); W13 with gate_up_I: gate columns [0, I), up [I, 2I)
  EPI_PARTIAL = 3,   // split K: part[ks][f][n] = this split's FP32 sum (n in prepared row order)
};

struct GemmParams {
  // prepared weights of one matrix
  const void* wq;        // u32x4 [E][RG][Kc][4][64]
  const void* wsc;       // u16 [E][RG][Kc][64][4]
  int E, RG, Kc, K, N;   // N: true rows (output features)
  int wg_per_set;        // workgroups per row set: ceil(RG / 4), or ceil(ceil(RG / 4) / qpw)
  int qpw;               // large-M K-resident form (K <= 256): row-group quads per workgroup; 0 off
  // small-M on routing blocks: 0 one workgroup per (expert, quad); 1 persistent
  // workgroups, static job ranges; 2 persistent workgroups on the job queue
  int dispatch;
  int passes;            // persistent forms: token passes of 16*NT rows per routing block
  int32_t* queue;        // dispatch 2: job counter, zero at launch
  int nsets;             // row sets (experts or blocks)
  int total_wg;
  int xcd_deal;          // large-M K loop on blocks: units of xcd_deal blocks dealt round-robin to the XCDs (0: off)
  // row sets
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* sorted_ids;
  const int32_t* routing_hdr;
  const int32_t* block_expert;
  int sentinel, topk, block;  // indexed
  const int32_t* masked_m;
  int max_m;                  // masked
  const int32_t* m_indices;
  int block_rows;             // blocks (contiguous)
  const int32_t* row_src;     // blocks with combine
  // B operand rows
  const uint16_t* src;
  int64_t src_ld;             // elements per row
  int gather;                 // 1: row = sorted_ids[slot] / topk
  // epilogue targets
  uint16_t* a_out;
  int64_t a_ld;               // SWIGLU
  uint16_t* yq;               // COMBINE: weighted rows [F][ld], one per flat index f, as 16-bit
  const float* topk_w;        //   integers with a scale per 8 positions (store_y16)
  int64_t yrows_ld;           //   ld: features per row (a multiple of 64)
  uint16_t* out;
  int64_t out_ld;             // STORE
  int gate_up_I;              // STORE of W13 (gate_up_I = I): un-interleave gate | up columns
  // split K (small-M, indexed): ksplit workgroups per (set, quad), each over an
  // equal share of the K chunks, writing FP32 partial sums part[ks][f][0, N)
  int ksplit;
  float* part;
  int64_t part_rows;          // F = T * topk rows per split
};

// Rows of the B operand matrix a GEMM may read, for each row set kind.
inline int64_t src_rows(const GemmParams& p, int set) {
  if (set == SET_ROUTED)
    return p.gather ? (int64_t)p.sentinel / (p.topk > 0 ? p.topk : 1) : (int64_t)p.nsets * p.block;
  if (set == SET_MASKED) return (int64_t)p.E * p.max_m;
  return (int64_t)p.nsets * p.block_rows;
}

// The half-chunk ring K loop (256-row tiles) addresses token rows by 32-bit
// byte offsets: the B operand matrix must span less than 4 GiB.
inline bool src_fits_u32(const GemmParams& p, int set) {
  const int64_t rows = src_rows(p, set);
  return rows <= 0 || (rows - 1) * p.src_ld * 2 + (int64_t)p.K * 2 <= (int64_t)0xFFFFFFFF;
}

// dispatch 1 or 2: routing blocks (SET_ROUTED, block 16*nt) only; total_wg
// workgroups, enough that a static range spans at most 64 blocks.
hipError_t launch_gemm_small_m(const GemmParams& p, int set, int epi, int nt, hipStream_t s);
// K must be a multiple of 128; qpw > 0 (K-resident form) needs K <= 256 and
// a routing or contiguous row set.
hipError_t launch_gemm_large_m(const GemmParams& p, int set, int epi, hipStream_t s);

// a[r][c] = bf16(silu(h[r][c]) * h[r][I + c]) for r < rows, c < I (I a
// multiple of 8; h rows of 2I, a rows of I, BF16).
hipError_t launch_swiglu(const uint16_t* h, int64_t rows, int I, uint16_t* a, hipStream_t s);
// Split-K reductions (partials in split order, s ascending):
//   W13: a[slot][c] = bf16(silu(sum_s g) * sum_s u) for valid routing slots,
//        g and u at the prepared gate / up rows of column c of part [S][F][2I];
//   W2:  out[t] = bf16(sum_j w[t,j] * sum_s part[s][t*topk + j]) over rows with
//        slot_of >= 0 (zeros when hdr does not describe (E, block, T*topk)).
hipError_t launch_splitk_swiglu(const float* part, int S, int64_t F, int I, const int32_t* sorted_ids,
                                int cap, int sentinel, uint16_t* a, int64_t a_ld, hipStream_t s);
hipError_t launch_splitk_combine(const float* part, int S, const int32_t* slot_of, const int32_t* hdr,
                                 int E, int block, const float* topk_w, int T, int topk, int H,
                                 uint16_t* out, hipStream_t s);

// map (NULL: ids are local): device int32 [Eg], global id -> local expert
// of this handle or -1; rows whose id maps outside [0, E) are dropped.
hipError_t launch_align(const int32_t* topk_ids, int T, int topk, int E, const RoutingLayout& L,
                        int32_t* routing, hipStream_t s, const int32_t* map = nullptr, int Eg = 0);
hipError_t launch_permute(const uint16_t* x, int T, int topk, int H, const RoutingLayout& L,
                          const int32_t* routing, uint16_t* a_out, int32_t* m_indices,
                          int32_t* row_src, hipStream_t s);
hipError_t launch_repack(const MatLayout& m, const int32_t* words, const uint16_t* scales,
                         char* prepared, int32_t* bad_scale_flag, hipStream_t s);
hipError_t launch_dequant_expert(const MatLayout& m, const char* prepared, int expert,
                                 uint16_t* out, hipStream_t s);
hipError_t launch_zero_i32(int32_t* p, size_t n, hipStream_t s);
// Large-M K loop over 256-row tiles (pairs of 128-row routing or contiguous
// blocks of one expert); p.total_wg = ceil(nsets / 2) * wg_per_set.
hipError_t launch_gemm_wide(const GemmParams& p, int set, int epi, hipStream_t s);
// Data checks (MOE_W4A16_VALIDATE=1); each adds its count to *bad.
// Entries of v[0, n) outside [lo, hi):
hipError_t launch_count_outside(const int32_t* v, int64_t n, int lo, int hi, int32_t* bad, hipStream_t s);
// 128-row blocks of m_indices holding two different experts:
hipError_t launch_count_mixed_blocks(const int32_t* m_indices, int M_pad, int32_t* bad, hipStream_t s);
// Rows whose row_src breaks the pairing with m_indices (pad <-> -1, a row's
// source in [0, n_flat), each source used once); seen: n_flat ints of scratch.
hipError_t launch_count_row_src(const int32_t* m_indices, const int32_t* row_src, int M_pad, int n_flat,
                                int32_t* seen, int32_t* bad, hipStream_t s);
// out[t] = bf16(sum over j ascending of yrows[t*topk + j]) for rows with
// valid[t*topk + j] >= 0; tokens with no such row get 0. hdr (may be NULL):
// routing header that must describe (E, block, T*topk), else out = 0.
// yq: the weighted rows (store_y16), ld features per row (a multiple of 64,
// >= H).
hipError_t launch_combine_rows(const uint16_t* yq, int ld, const int32_t* valid,
                               const int32_t* hdr, int E, int block, int T, int topk, int H, uint16_t* out,
                               hipStream_t s);
// valid[f] = 0 for every f = row_src[p] of a non-padding contiguous row (the
// block's expert, as the GEMMs take it), -1 for every other f < T*topk.
hipError_t launch_contiguous_valid(const int32_t* m_indices, const int32_t* row_src, int M_pad,
                                   int E, int n_flat, int32_t* valid, hipStream_t s);

}  // namespace moe
