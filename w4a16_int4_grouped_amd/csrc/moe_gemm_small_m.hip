// Grouped W4A16 GEMM, small-M schedule (few rows per expert).
//
// At a few routed rows per expert a GEMM is a weight stream, so the
// dequantised weights take the wide MFMA operand: they are the 16-row A side
// of v_mfma_f32_16x16x32_bf16 and the tokens are the 16-column B side, padded
// to 16 (Chord page, "H200 and Blackwell indexed decode": the decode
// configuration swaps the MMA operands so dequantised weights fill MMA-M).
//
// Work item: one row set (an expert, or a 128-row block of the contiguous
// layout) x 256 weight rows. Each of the 4 waves owns one row group of 64
// weight rows (4 MFMA tiles) over the whole K, and the workgroup loops over
// the set's rows 16*NT at a time, so an expert's weights are streamed once
// whenever its rows fit in 16*NT. The grid is fixed from host-known sizes and
// each workgroup reads its row count on the device (a semi-static token-tile
// schedule, the variant the Chord page measured faster than a fully dynamic
// one in "H200 and Blackwell indexed decode").
//
// Per K chunk of 128:
//   * each wave streams 4 KB of its packed weights (one coalesced 1 KB load
//     per tile) and 512 B of scales, two chunks ahead of the math, in three
//     rotating register buffers (about 9 KB in flight per wave, enough to
//     keep HBM busy at four waves per SIMD);
//   * the workgroup loads the token tile (16*NT rows x 128 k of BF16) once,
//     one chunk ahead, through registers into one of three LDS buffers
//     (rows padded to 272 B so the fragment reads hit 64 distinct banks):
//     with four tiles only the tiles that hold rows, with one tile in the
//     first GEMM only the rows the expert holds;
//   * every lane's 32 k values of a tile share one scale group, so each
//     (lane, tile, chunk) needs one scale.
// Loads past the last chunk go to a valid dummy address, so every load in
// the loop is unconditional and each wait covers exactly the buffer in use.
//
// Epilogues: SwiGLU into the BF16 intermediate (W13, gate/up tiles
// interleaved so both halves of a column sit in the same lane and register),
// the routing-weighted row w*y stored at its flat index for the combine
// kernel as 16-bit integers with a scale per 8 features (store_y16; W2,
// indexed / contiguous with row_src), or a BF16 store (W2, masked /
// contiguous without row_src).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kBRow = 136;   // LDS token row: 128 BF16 + 8 pad (272 B)

struct AFrag {
  u32x4_t A[kMT];
  u32x2_t S;
};

template <int NT>
struct TileLds {
  uint16_t b[3][NT][16][kBRow];
};

// wq / ws: the wave's chunk base (wave-uniform, kept in SGPRs); lane: the
// per-lane element offset.
__device__ __forceinline__ void load_a(AFrag& f, const u32x4_t* __restrict__ wq,
                                       const u32x2_t* __restrict__ ws, int lane) {
  // weights and scales are streamed once: nontemporal loads keep them from
  // displacing activation rows in L2
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) f.A[mt] = __builtin_nontemporal_load(wq + mt * 64 + lane);
  f.S = __builtin_nontemporal_load(ws + lane);
}

template <int NA, int NT>
__device__ __forceinline__ void load_b(u32x4_t (&st)[NT], const uint16_t* const (&lrow)[NT], int kc,
                                       int kmax, bool whole) {
  // this thread's 16-byte piece of each token row of the first NA tiles (a
  // pass's tiles past its rows are neither loaded nor stored); k past K reads zero (the
  // substitute address is the row's first element, always valid). whole
  // (uniform): K is whole chunks and kc (always below the chunk count) is one
  // of them, so every piece is read as is, with no per-lane select (5 VALU
  // instructions per chunk fewer in the VALU-bound decode loop).
  if (whole) {
#pragma unroll
    for (int nt = 0; nt < NA; ++nt) st[nt] = *reinterpret_cast<const u32x4_t*>(lrow[nt] + kc * kKC);
    return;
  }
  const int lpiece = (threadIdx.x & 15) * 8;
#pragma unroll
  for (int nt = 0; nt < NA; ++nt) {
    const bool ok = kc * kKC < kmax;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lrow[nt] + (ok ? kc * kKC : -lpiece));
    const u32x4_t z = {0u, 0u, 0u, 0u};
    st[nt] = ok ? v : z;
  }
}

// load_b for the rows a set holds only: a lane whose token row lies past
// them keeps its registers (zero from the pass start) and sends no request.
// Those rows' MFMA columns are never stored. Used by the one-tile kernels
// of the first GEMM, whose rows are gathered (decode: ~9 of 16 rows hold
// tokens; W13 1066-1074 -> 1055-1062 us). The second GEMM's rows are
// consecutive, so its padding rows cost little (W2 measured 3 us slower
// with it), and in the four-tile kernels the per-tile lane branches cost
// more than the loads they save (masked W13 1346 -> 1428 us).
template <int NT>
__device__ __forceinline__ void load_b_rows(u32x4_t (&st)[NT], const uint16_t* const (&lrow)[NT],
                                            const bool (&rv)[NT], int kc, int kmax, bool whole) {
  if (whole) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      if (rv[nt]) st[nt] = *reinterpret_cast<const u32x4_t*>(lrow[nt] + kc * kKC);
    return;
  }
  const int lpiece = (threadIdx.x & 15) * 8;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (!rv[nt]) continue;
    const bool ok = kc * kKC < kmax;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lrow[nt] + (ok ? kc * kKC : -lpiece));
    const u32x4_t z = {0u, 0u, 0u, 0u};
    st[nt] = ok ? v : z;
  }
}

template <int NA, int NT>
__device__ __forceinline__ void store_b(TileLds<NT>& lds, int buf, const u32x4_t (&st)[NT]) {
  const int r = threadIdx.x >> 4, piece = threadIdx.x & 15;
#pragma unroll
  for (int nt = 0; nt < NA; ++nt)
    *reinterpret_cast<u32x4_t*>(&lds.b[buf][nt][r][piece * 8]) = st[nt];
}

// One K chunk over the first NA of the NT token tiles (a pass whose rows
// fill fewer tiles computes only those). NA = 1 (decode, 4 waves/SIMD at
// <= 128 registers): weight tile outer, the single token fragment re-read
// from LDS per step. NA >= 2: step outer; the step's NA token fragments stay
// in registers across the 4 weight tiles (one LDS read per token tile and
// step instead of four), and each tile's MFMAs carry the next tile's
// dequantisation and, on the last tile, the next step's LDS reads (issue
// order set by sched_group_barrier).
template <int NA, int NT>
__device__ __forceinline__ void mma_chunk(const AFrag& f, const TileLds<NT>& lds, int buf,
                                          f32x4_t (&acc)[kMT][NT], uint32_t mlo,
                                          uint32_t mhi) {
  static_assert(NA >= 1 && NA <= NT, "active token tiles");
  const int lane = threadIdx.x & 63;
  const uint16_t* brow = &lds.b[buf][0][lane & 15][(lane >> 4) * 32];
  const float sc[4] = {bf16_lo(f.S[0]), bf16_hi(f.S[0]), bf16_lo(f.S[1]), bf16_hi(f.S[1])};
  if constexpr (NA == 1) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const GroupScale gs = group_scale(sc[mt]);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4_t bf = *reinterpret_cast<const u32x4_t*>(brow + g * 8);
        const u32x4_t a = dq8(f.A[mt][g], gs, mlo, mhi);
        acc[mt][0] = mfma16(a, bf, acc[mt][0]);
      }
    }
  } else {
    constexpr int kValu = (17 + NA - 1) / NA;
    GroupScale gs[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) gs[mt] = group_scale(sc[mt]);
    u32x4_t bf[NA];
#pragma unroll
    for (int nt = 0; nt < NA; ++nt) bf[nt] = *reinterpret_cast<const u32x4_t*>(brow + nt * (16 * kBRow));
    u32x4_t a = dq8(f.A[0][0], gs[0], mlo, mhi);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const bool last = (mt == kMT - 1);
        const int ng = last ? g + 1 : g, nmt = last ? 0 : mt + 1;
        u32x4_t an = a;
        if (ng < 4) an = dq8(f.A[nmt][ng], gs[nmt], mlo, mhi);
#pragma unroll
        for (int nt = 0; nt < NA; ++nt) {
          acc[mt][nt] = mfma16(a, bf[nt], acc[mt][nt]);
          if (last && g < 3)
            bf[nt] = *reinterpret_cast<const u32x4_t*>(brow + nt * (16 * kBRow) + (g + 1) * 8);
        }
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
          if (last && g < 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
          __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);                // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
        a = an;
      }
    }
  }
}

// Occupancy target per token-tile count: 4 workgroups (4 waves per SIMD) fit
// NT = 1 in 128 registers without spilling; wider tiles need more registers.
template <int NT>
constexpr int kSmallMBlocksPerCU = NT == 1 ? 4 : (NT == 2 ? 3 : 2);

template <int NT, int SET, int EPI>
__global__ __launch_bounds__(256, kSmallMBlocksPerCU<NT>) void gemm_small_m(const GemmParams p) {
  // rows of x gathered through the routing (W13 of the indexed layout)
  const bool gather = (SET == SET_INDEXED || SET == SET_ROUTED) && p.gather;
  __shared__ TileLds<NT> lds;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int logical_k = xcd_remap(blockIdx.x, p.total_wg);
  // split K: ksplit consecutive workgroups share one (set, quad)
  const int S = p.ksplit > 1 ? p.ksplit : 1;
  const int ks = logical_k % S, logical = logical_k / S;
  const int set = logical / p.wg_per_set;
  const int rg_raw = (logical - set * p.wg_per_set) * 4 + wave;
  const bool active = rg_raw < p.RG;          // waves past the last row group still load tiles
  const int rg = active ? rg_raw : p.RG - 1;

  // ---- the row set (uniform over the workgroup)
  int e, slot0, count;
  if constexpr (SET == SET_INDEXED) {
    const int32_t* hdr = p.routing_hdr;
    if (hdr[HDR_MAGIC] != kRoutingMagic || hdr[HDR_BLOCK] != p.block || hdr[HDR_E] != p.E ||
        hdr[HDR_T] * hdr[HDR_TOPK] != p.sentinel)
      return;   // routing made for other shapes: compute nothing
    // a grid of fewer sets than experts (fewer routed rows than experts)
    // takes the experts that hold rows, in expert order
    e = p.nsets < p.E ? nth_active(p.counts, p.E, set) : set;
    if (e < 0) return;
    slot0 = p.offsets[e];
    count = p.counts[e];
  } else if constexpr (SET == SET_ROUTED) {
    // one routing block of p.block slots; the grid covers a host bound on the
    // blocks, the header's total says which hold rows
    const int32_t* hdr = p.routing_hdr;
    if (hdr[HDR_MAGIC] != kRoutingMagic || hdr[HDR_BLOCK] != p.block || hdr[HDR_E] != p.E ||
        hdr[HDR_T] * hdr[HDR_TOPK] != p.sentinel)
      return;
    if (set >= min(max(hdr[HDR_TOTAL], 0) / p.block, p.nsets)) return;
    e = p.block_expert[set];
    if (e >= p.E) return;
    slot0 = set * p.block;
    count = p.block;   // pad slots hold the sentinel: read row 0, never written
  } else if constexpr (SET == SET_MASKED) {
    e = set;
    slot0 = e * p.max_m;
    count = min(max(p.masked_m[e], 0), p.max_m);
  } else {
    slot0 = set * p.block_rows;
    count = p.block_rows;
    int m = -1;
    for (int r = lane; r < p.block_rows; r += 64) {
      const int v = p.m_indices[slot0 + r];
      if (v >= 0 && v < p.E) m = max(m, v);
    }
    e = wave_max(m);
  }
  if (count <= 0 || e < 0) return;

  // this workgroup's chunks c0 .. c0 + Kc of the row group's p.Kc
  const int c0 = (int)((int64_t)p.Kc * ks / S);
  const int Kc = (int)((int64_t)p.Kc * (ks + 1) / S) - c0;
  const size_t tile0 = ((size_t)e * p.RG + rg) * p.Kc + c0;
  const size_t cstride = 1;   // tiles between consecutive chunks of a row group
  const u32x4_t* __restrict__ wq = reinterpret_cast<const u32x4_t*>(p.wq) + tile0 * (kMT * 64);
  const u32x2_t* __restrict__ ws = reinterpret_cast<const u32x2_t*>(p.wsc) + tile0 * 64;
  // dummy source for prefetches past the last chunk (valid, quickly cached)
  const u32x4_t* __restrict__ wq_dummy = reinterpret_cast<const u32x4_t*>(p.wq);
  const u32x2_t* __restrict__ ws_dummy = reinterpret_cast<const u32x2_t*>(p.wsc);
  const uint32_t mlo = kF16MagicLo, mhi = kF16MagicHi;
  const int lr = threadIdx.x >> 4;             // token row this thread loads into LDS
  const int lpiece = (threadIdx.x & 15) * 8;   // its k offset within a chunk
  const int kmax = p.K - c0 * kKC - lpiece;    // local chunk kc is readable if kc*128 < kmax
  const bool whole = p.K % kKC == 0;           // then every chunk kc < Kc is

  for (int tb = 0; tb < count; tb += 16 * NT) {
    const uint16_t* lrow[NT];
    bool rv[NT];   // the lane's token row holds a row of the set (one-tile first GEMM)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = min(tb + nt * 16 + lr, count - 1);   // pad columns repeat a valid row
      const int slot = slot0 + r;
      int row = slot;
      rv[nt] = tb + nt * 16 + lr < count;
      if (gather) {
        const int f = p.sorted_ids[slot];
        row = (f >= 0 && f < p.sentinel) ? f / p.topk : 0;   // pad slots read row 0
        rv[nt] = rv[nt] && f >= 0 && f < p.sentinel;
      }
      lrow[nt] = p.src + (size_t)row * p.src_ld + c0 * kKC + lpiece;
    }
    f32x4_t acc[kMT][NT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // three weight buffers and the token staging registers; k_loop first
    // loads weights of chunks 0 and 1 and the token tile of chunk 0
    AFrag fr0, fr1, fr2;
    u32x4_t st[NT];
    constexpr bool kRowsOnly = NT == 1 && EPI == EPI_SWIGLU;
    if constexpr (kRowsOnly) st[0] = u32x4_t{0u, 0u, 0u, 0u};
    // one chunk's token rows: all rows of the first NA tiles, or (one-tile
    // first GEMM) only the rows the set holds
    auto load_tokens = [&](auto na, int kc) __attribute__((always_inline)) {
      if constexpr (kRowsOnly) load_b_rows<NT>(st, lrow, rv, kc, kmax, whole);
      else load_b<decltype(na)::value, NT>(st, lrow, kc, kmax, whole);
    };
    // token tiles that hold rows: the NT = 4 kernels load, store and compute
    // only those (NT = 1 and 2 keep one body, all tiles; measured on the
    // masked workload, loading only those tiles took W13 from 1383-1397 to
    // 1354-1359 us)
    const int nta = min(NT, (count - tb + 15) >> 4);   // uniform: count is the set's
    auto with_live = [&](auto f) __attribute__((always_inline)) {
      if constexpr (NT == 1 || NT == 2 || SET == SET_BLOCKS) {
        f(std::integral_constant<int, NT>{});
      } else {
        static_assert(NT == 4, "token tiles per pass: 1, 2 or 4");
        if (nta == 1) f(std::integral_constant<int, 1>{});
        else if (nta == 2) f(std::integral_constant<int, 2>{});
        else if (nta == 3) f(std::integral_constant<int, 3>{});
        else f(std::integral_constant<int, 4>{});
      }
    };

    // step J computes chunk c from register buffer J and LDS buffer J, and
    // prefetches chunk c+2 into register buffer (J+2)%3 and the token tile of
    // chunk c+1 into LDS buffer (J+1)%3. The loads, the LDS stores and the
    // MFMAs cover the pass's first NA token tiles, those that hold rows.
    auto k_loop = [&](auto na) __attribute__((always_inline)) {
      constexpr int NA = decltype(na)::value;
      load_tokens(na, 0);
      load_a(fr0, wq, ws, lane);
      load_a(fr1, Kc > 1 ? wq + cstride * (kMT * 64) : wq_dummy, Kc > 1 ? ws + cstride * 64 : ws_dummy,
             lane);
      __syncthreads();   // the previous pass's readers are done with the LDS tiles
      store_b<NA, NT>(lds, 0, st);
      __syncthreads();
#define MOE_SMALL_M_STEP(J, CUR, NXT2)                                                           \
  {                                                                                              \
    const int c = kc + J;                                                                        \
    load_tokens(na, min(c + 1, Kc - 1));                                                         \
    const bool more = c + 2 < Kc;                                                                \
    load_a(NXT2, more ? wq + (size_t)(c + 2) * cstride * (kMT * 64) : wq_dummy,                  \
           more ? ws + (size_t)(c + 2) * cstride * 64 : ws_dummy, lane);                         \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    if (c < Kc) mma_chunk<NA, NT>(CUR, lds, J, acc, mlo, mhi);                                   \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    store_b<NA, NT>(lds, (J + 1) % 3, st);                                                       \
    __syncthreads();                                                                             \
  }
      // whole rotations, then the one or two chunks left (no step past the
      // last chunk pays for loads and a barrier)
      const int Kc3 = Kc - Kc % 3;
      int kc = 0;
      for (; kc < Kc3; kc += 3) {
        MOE_SMALL_M_STEP(0, fr0, fr2)
        MOE_SMALL_M_STEP(1, fr1, fr0)
        MOE_SMALL_M_STEP(2, fr2, fr1)
      }
      if (kc < Kc) {
        MOE_SMALL_M_STEP(0, fr0, fr2)
        if (kc + 1 < Kc) MOE_SMALL_M_STEP(1, fr1, fr0)
      }
#undef MOE_SMALL_M_STEP
    };
    // NT = 2 keeps one body: a second one does not fit its 168 registers
    // (3 workgroups per CU) without spilling; nor do four in the contiguous
    // blocks' BF16 store variant, whose rows are 128-row blocks anyway
    with_live(k_loop);
    if (!active) continue;

    // ---- epilogue
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = tb + nt * 16 + (lane & 15);
      if (r >= count) continue;
      const int slot = slot0 + r;
      if constexpr (SET == SET_ROUTED) {
        const int f = p.sorted_ids[slot];
        if (f < 0 || f >= p.sentinel) continue;   // pad slot
      }
      if constexpr (EPI == EPI_SWIGLU) {
        uint16_t* dst = p.a_out + (size_t)slot * p.a_ld + rg * 32 + (lane >> 4) * 4;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const f32x4_t g = acc[2 * pp][nt], u = acc[2 * pp + 1][nt];
          u32x2_t v;
          v[0] = pack_bf16x2(swiglu(g[0], u[0]), swiglu(g[1], u[1]));
          v[1] = pack_bf16x2(swiglu(g[2], u[2]), swiglu(g[3], u[3]));
          *reinterpret_cast<u32x2_t*>(dst + pp * 16) = v;
        }
      } else if constexpr (EPI == EPI_COMBINE) {
        int f;
        if constexpr (SET == SET_INDEXED || SET == SET_ROUTED) {
          f = p.sorted_ids[slot];
        } else {
          f = (p.m_indices[slot] == e) ? p.row_src[slot] : -1;
        }
        if (f < 0 || f >= p.sentinel) continue;
        const float w = p.topk_w[f];
        if (rg * kRowsRG < p.N) {   // the row group's 64 features, lane-contiguous (store_y16)
          f32x4_t v[kMT];
#pragma unroll
          for (int mt = 0; mt < kMT; ++mt) v[mt] = acc[mt][nt];
          store_y16<kMT>(p.yq, (size_t)f * p.yrows_ld + rg * kRowsRG + (lane >> 4) * 16, w, v);
        }
      } else if constexpr (EPI == EPI_PARTIAL) {
        const int f = p.sorted_ids[slot];
        if (f < 0 || f >= p.sentinel) continue;
        float* dst = p.part + ((size_t)ks * p.part_rows + f) * p.N;
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          const int n = rg * kRowsRG + mt * 16 + (lane >> 4) * 4;
          if (n < p.N) *reinterpret_cast<f32x4_t*>(dst + n) = acc[mt][nt];
        }
      } else {
        uint16_t* dst = p.out + (size_t)slot * p.out_ld;
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          const int n = store_col(p.N, p.gate_up_I, rg, mt, lane);
          if (n >= 0) {
            u32x2_t v;
            v[0] = pack_bf16x2(acc[mt][nt][0], acc[mt][nt][1]);
            v[1] = pack_bf16x2(acc[mt][nt][2], acc[mt][nt][3]);
            *reinterpret_cast<u32x2_t*>(dst + n) = v;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent forms (routing blocks of one weight pass), for the dispatch
// ablation of the Chord page ("H200 and Blackwell indexed decode"), which
// measured its semi-static token-tile schedule (the grid above) against a
// fully dynamic one.
//
// A job is one weight pass: (routing block, token pass, quad of row groups),
// numbered block-major. One workgroup per resident slot walks a sequence of
// jobs as one stream of K chunks: weights two chunks ahead and the token
// tile one chunk ahead keep flowing across job boundaries. DYN = false: each
// workgroup takes an equal contiguous range of the jobs (a static split,
// ranges on one XCD each). DYN = true: workgroups take jobs one at a time
// from an atomic counter (a fully dynamic work queue), two jobs ahead of the
// one being computed.
// ---------------------------------------------------------------------------

// Jobs of a set: ceil(rows / (16*NT)) token passes x quads.
struct JobSpace {
  int P, Q;        // passes per set, quads per set
  int s0;          // first set of this workgroup's range
  int info;        // lane i: ROUTED: expert of set s0+i (-1 none); MASKED: rows of expert s0+i
  int64_t j1;      // end of this workgroup's range
};

// One job's uniform data (SGPRs) and, for the current and next job, the
// lane's token row pointers.
struct Job {
  int64_t j;       // job index; j >= j1: none
  int e, slot0, count, tb, rg;
  bool active;
  const u32x4_t* wq;   // chunk 0 of this wave's row group
  const u32x2_t* ws;
};

template <int SET>
__device__ __forceinline__ bool job_valid(const JobSpace& js, int64_t j, int rows_per_pass) {
  const int s = (int)(j / ((int64_t)js.P * js.Q));
  const int v = __builtin_amdgcn_readlane(js.info, s - js.s0);
  if constexpr (SET == SET_ROUTED) {
    return v >= 0;
  } else {
    const int pass = (int)((j - (int64_t)s * js.P * js.Q) / js.Q);
    return pass * rows_per_pass < v;
  }
}

template <int SET>
__device__ __forceinline__ int64_t next_job(const JobSpace& js, int64_t j, int rows_per_pass) {
  do {
    ++j;
  } while (j < js.j1 && !job_valid<SET>(js, j, rows_per_pass));
  return j;
}

// A job from its index and its set's info value (the expert of a routing
// block; the rows of a masked expert).
template <int SET>
__device__ __forceinline__ Job make_job_e(const GemmParams& p, const JobSpace& js, int64_t j, int v,
                                          int wave, int rows_per_pass) {
  Job b;
  b.j = j;
  if (j >= js.j1) {   // none: valid dummy addresses
    b.e = 0; b.slot0 = 0; b.count = 1; b.tb = 0; b.rg = 0; b.active = false;
    b.wq = reinterpret_cast<const u32x4_t*>(p.wq);
    b.ws = reinterpret_cast<const u32x2_t*>(p.wsc);
    return b;
  }
  const int s = (int)(j / ((int64_t)js.P * js.Q));
  const int rem = (int)(j - (int64_t)s * js.P * js.Q);
  const int pass = rem / js.Q, quad = rem - pass * js.Q;
  if constexpr (SET == SET_ROUTED) {
    b.e = v;
    b.slot0 = s * p.block;
    b.count = p.block;
  } else {
    b.e = s;
    b.slot0 = s * p.max_m;
    b.count = v;
  }
  b.tb = pass * rows_per_pass;
  const int rg_raw = quad * 4 + wave;
  b.active = rg_raw < p.RG;
  b.rg = b.active ? rg_raw : p.RG - 1;
  const size_t tile0 = ((size_t)b.e * p.RG + b.rg) * p.Kc;
  b.wq = reinterpret_cast<const u32x4_t*>(p.wq) + tile0 * (kMT * 64);
  b.ws = reinterpret_cast<const u32x2_t*>(p.wsc) + tile0 * 64;
  return b;
}

template <int SET>
__device__ __forceinline__ Job make_job(const GemmParams& p, const JobSpace& js, int64_t j, int wave,
                                        int rows_per_pass) {
  const int v = j < js.j1 ? __builtin_amdgcn_readlane(js.info, (int)(j / ((int64_t)js.P * js.Q)) - js.s0)
                          : 0;
  return make_job_e<SET>(p, js, j, v, wave, rows_per_pass);
}

// The thread's token rows of a job (row 16*nt + thread/16 of its pass, pad
// rows repeating the last row of the set): the slot, or with GATHER the flat
// index stored there (a load whose value is first used a job later, in
// row_ptr).
template <int NT, bool GATHER>
__device__ __forceinline__ void job_row_ids(const GemmParams& p, const Job& b, int (&id)[NT]) {
  const int lr = threadIdx.x >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int slot = b.slot0 + min(b.tb + nt * 16 + lr, b.count - 1);
    id[nt] = GATHER ? p.sorted_ids[slot] : slot;
  }
}

template <int NT, bool GATHER>
__device__ __forceinline__ void row_ptrs(const GemmParams& p, const int (&id)[NT],
                                         const uint16_t* (&lrow)[NT]) {
  const int lpiece = (threadIdx.x & 15) * 8;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int row = id[nt];
    if constexpr (GATHER) row = (row >= 0 && row < p.sentinel) ? row / p.topk : 0;   // pad: row 0
    lrow[nt] = p.src + (size_t)row * p.src_ld + lpiece;
  }
}

// Keeps a loaded value untouched until this point: the compiler may not
// hoist its uses (and so the wait for the load) above it.
__device__ __forceinline__ int pin(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Routing data of the lane's output rows (row 16*nt + lane%16 of the pass),
// loaded when a job starts and first read by its epilogue: the slot's flat
// index (routing blocks), or the row itself (masked; -1 past masked_m).
template <int NT, int SET>
__device__ __forceinline__ void job_epi_ids(const GemmParams& p, const Job& b, int lane, int (&f)[NT]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = b.tb + nt * 16 + (lane & 15);
    if constexpr (SET == SET_ROUTED) {
      f[nt] = p.sorted_ids[b.slot0 + min(r, b.count - 1)];   // r < count = block
    } else {
      f[nt] = r < b.count ? r : -1;
    }
  }
}

// Epilogue of one job from its prefetched routing data: pad slots and rows
// past the set are skipped; SwiGLU and BF16 stores go to the row's slot,
// weighted 16-bit rows (store_y16) to its flat index.
template <int NT, int SET, int EPI>
__device__ __forceinline__ void job_epilogue(const GemmParams& p, const f32x4_t (&acc)[kMT][NT],
                                             const Job& b, const int (&fid)[NT], int lane) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int f = pin(fid[nt]);
    if (SET == SET_ROUTED ? (f < 0 || f >= p.sentinel) : f < 0) continue;
    const int slot = b.slot0 + b.tb + nt * 16 + (lane & 15);
    if constexpr (EPI == EPI_SWIGLU) {
      uint16_t* dst = p.a_out + (size_t)slot * p.a_ld + b.rg * 32 + (lane >> 4) * 4;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const f32x4_t g = acc[2 * pp][nt], u = acc[2 * pp + 1][nt];
        u32x2_t v;
        v[0] = pack_bf16x2(swiglu(g[0], u[0]), swiglu(g[1], u[1]));
        v[1] = pack_bf16x2(swiglu(g[2], u[2]), swiglu(g[3], u[3]));
        *reinterpret_cast<u32x2_t*>(dst + pp * 16) = v;
      }
    } else if constexpr (EPI == EPI_COMBINE) {
      const float w = p.topk_w[f];
      if (b.rg * kRowsRG < p.N) {   // the row group's 64 features, lane-contiguous (store_y16)
        f32x4_t v[kMT];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) v[mt] = acc[mt][nt];
        store_y16<kMT>(p.yq, (size_t)f * p.yrows_ld + b.rg * kRowsRG + (lane >> 4) * 16, w, v);
      }
    } else {
      uint16_t* dst = p.out + (size_t)slot * p.out_ld;
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const int n = store_col(p.N, p.gate_up_I, b.rg, mt, lane);
        if (n >= 0) {
          u32x2_t v;
          v[0] = pack_bf16x2(acc[mt][nt][0], acc[mt][nt][1]);
          v[1] = pack_bf16x2(acc[mt][nt][2], acc[mt][nt][3]);
          *reinterpret_cast<u32x2_t*>(dst + n) = v;
        }
      }
    }
  }
}

template <int NT, int SET, int EPI, bool DYN>
__global__ __launch_bounds__(256, kSmallMBlocksPerCU<NT>) void gemm_small_m_jobs(const GemmParams p) {
  static_assert(!DYN || SET == SET_ROUTED, "the job queue serves routing blocks");
  constexpr bool kGather = (SET == SET_ROUTED && EPI == EPI_SWIGLU);
  constexpr int kRows = 16 * NT;
  __shared__ TileLds<NT> lds;
  __shared__ int qslot[4][2];   // DYN: jobs taken from the queue (index, expert)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // ---- this workgroup's job range
  int nsets = p.nsets;
  if constexpr (SET == SET_ROUTED) {
    const int32_t* hdr = p.routing_hdr;
    if (hdr[HDR_MAGIC] != kRoutingMagic || hdr[HDR_BLOCK] != p.block || hdr[HDR_E] != p.E ||
        hdr[HDR_T] * hdr[HDR_TOPK] != p.sentinel)
      return;   // routing made for other shapes: compute nothing
    nsets = min(max(hdr[HDR_TOTAL], 0) / p.block, p.nsets);
  }
  JobSpace js;
  js.P = p.passes;
  js.Q = p.wg_per_set;
  const int64_t per_set = (int64_t)js.P * js.Q;
  const int64_t njobs = (int64_t)nsets * per_set;
  Job cur, nxt, nx2;
  int tk = 0;   // DYN: transitions so far (selects the queue slot)
  if constexpr (DYN) {
    // one thread takes jobs from the queue: index and the block's expert
    auto take = [&](int slot) {
      const int t = atomicAdd(p.queue, 1);
      qslot[slot][0] = t;
      qslot[slot][1] = t < njobs ? p.block_expert[t / per_set] : 0;
    };
    if (threadIdx.x == 0) {
      take(0);
      take(1);
      take(2);
      take(3);
    }
    __syncthreads();
    js.s0 = 0;
    js.j1 = njobs;
    cur = make_job_e<SET>(p, js, qslot[0][0], qslot[0][1], wave, kRows);
    nxt = make_job_e<SET>(p, js, qslot[1][0], qslot[1][1], wave, kRows);
    nx2 = make_job_e<SET>(p, js, qslot[2][0], qslot[2][1], wave, kRows);
    if (cur.j >= js.j1) return;
  } else {
    const int G = gridDim.x;
    const int logical = xcd_remap(blockIdx.x, G);
    const int64_t j0 = njobs * logical / G;
    js.j1 = njobs * (logical + 1) / G;
    if (j0 >= js.j1) return;
    js.s0 = (int)(j0 / per_set);
    if ((js.j1 - 1) / per_set - js.s0 >= 64) return;   // grid too small for the set table
    {
      const int s = js.s0 + lane;   // the range spans at most 64 sets (host-sized grid)
      int v = -1;
      if ((int64_t)s * per_set < js.j1) {
        if constexpr (SET == SET_ROUTED) {
          const int e = p.block_expert[s];
          v = (e >= 0 && e < p.E) ? e : -1;
        } else {
          v = min(max(p.masked_m[s], 0), p.max_m);
        }
      }
      js.info = v;
    }
    int64_t j = j0;
    if (!job_valid<SET>(js, j, kRows)) j = next_job<SET>(js, j, kRows);
    if (j >= js.j1) return;
    cur = make_job<SET>(p, js, j, wave, kRows);
    nxt = make_job<SET>(p, js, next_job<SET>(js, cur.j, kRows), wave, kRows);
    nx2 = make_job<SET>(p, js, next_job<SET>(js, nxt.j, kRows), wave, kRows);
  }
  const uint16_t* lrow_cur[NT];
  int id_nxt[NT];
  {
    int id_cur[NT];
    job_row_ids<NT, kGather>(p, cur, id_cur);
    row_ptrs<NT, kGather>(p, id_cur, lrow_cur);
  }
  job_row_ids<NT, kGather>(p, nxt, id_nxt);
  int ef[NT];
  job_epi_ids<NT, SET>(p, cur, lane, ef);

  const int Kc = p.Kc;
  const uint32_t mlo = kF16MagicLo, mhi = kF16MagicHi;
  const int kmax = p.K - (threadIdx.x & 15) * 8;   // chunk kc is readable if kc*128 < kmax
  const bool whole = p.K % kKC == 0;               // then every chunk kc < Kc is
  constexpr int kCh = kMT * 64;                    // u32x4 per chunk of one row group

  f32x4_t acc[kMT][NT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // prologue: weights of the first two chunks of the stream, token tile of
  // the first
  AFrag fr0, fr1, fr2;
  u32x4_t st[NT];
  load_b<NT, NT>(st, lrow_cur, 0, kmax, whole);
  load_a(fr0, cur.wq, cur.ws, lane);
  if (Kc > 1)
    load_a(fr1, cur.wq + kCh, cur.ws + 64, lane);
  else
    load_a(fr1, nxt.wq, nxt.ws, lane);
  __syncthreads();
  store_b<NT, NT>(lds, 0, st);
  __syncthreads();

  int c = 0;   // chunk of the current job computed by the next step
  bool live = true;
  // step J computes chunk c of the current job from register buffer J and LDS
  // buffer J, and prefetches the stream's next chunk of weights + 2 into
  // register buffer (J+2)%3 and its next token chunk into LDS buffer (J+1)%3.
  // A job's last chunk is followed by its epilogue and the shift to the next.
#define MOE_JOB_STEP(J, CUR, NXT2)                                                            \
  if (live) {                                                                                 \
    {                                                                                         \
      /* one load site each (selected addresses), so the waits stay where the */              \
      /* data is consumed: tokens at the LDS store, weights two steps later */                 \
      const bool tcur = c + 1 < Kc;                                                           \
      const uint16_t* tp[NT];                                                                 \
      if (tcur) {                                                                             \
        _Pragma("unroll") for (int nt = 0; nt < NT; ++nt) tp[nt] = lrow_cur[nt];              \
      } else {                                                                                \
        int idv[NT];                                                                          \
        _Pragma("unroll") for (int nt = 0; nt < NT; ++nt) idv[nt] = pin(id_nxt[nt]);          \
        row_ptrs<NT, kGather>(p, idv, tp);                                                    \
      }                                                                                       \
      load_b<NT, NT>(st, tp, tcur ? c + 1 : 0, kmax, whole);                                  \
      const int w2 = c + 2;                                                                   \
      const bool wcur = w2 < Kc, wnxt = !wcur && w2 - Kc < Kc;                                \
      const int wc = wcur ? w2 : (wnxt ? w2 - Kc : 0);                                        \
      const u32x4_t* wqb = wcur ? cur.wq : (wnxt ? nxt.wq : nx2.wq);                          \
      const u32x2_t* wsb = wcur ? cur.ws : (wnxt ? nxt.ws : nx2.ws);                          \
      load_a(NXT2, wqb + (size_t)wc * kCh, wsb + (size_t)wc * 64, lane);                      \
    }                                                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    mma_chunk<NT, NT>(CUR, lds, J, acc, mlo, mhi);                                            \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    if (++c == Kc) {                                                                          \
      if (cur.active) job_epilogue<NT, SET, EPI>(p, acc, cur, ef, lane);                      \
      _Pragma("unroll") for (int mt = 0; mt < kMT; ++mt)                                      \
        _Pragma("unroll") for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f}; \
      c = 0;                                                                                  \
      cur = nxt;                                                                              \
      nxt = nx2;                                                                              \
      row_ptrs<NT, kGather>(p, id_nxt, lrow_cur);                                             \
      job_row_ids<NT, kGather>(p, nxt, id_nxt);                                               \
      job_epi_ids<NT, SET>(p, cur, lane, ef);                                                 \
      if constexpr (DYN) {                                                                    \
        /* the job taken at the previous transition; take the next one */                     \
        const int sl = 3 - (tk & 1);                                                          \
        nx2 = make_job_e<SET>(p, js, qslot[sl][0], qslot[sl][1], wave, kRows);                \
        if (threadIdx.x == 0) {                                                               \
          const int t = atomicAdd(p.queue, 1);                                                \
          qslot[5 - sl][0] = t;                                                               \
          qslot[5 - sl][1] = t < njobs ? p.block_expert[t / per_set] : 0;                     \
        }                                                                                     \
        ++tk;                                                                                 \
      } else {                                                                                \
        nx2 = make_job<SET>(p, js, next_job<SET>(js, nx2.j, kRows), wave, kRows);             \
      }                                                                                       \
      live = cur.j < js.j1;                                                                   \
    }                                                                                         \
    store_b<NT, NT>(lds, (J + 1) % 3, st);                                                    \
    __syncthreads();                                                                          \
  }
  while (live) {
    MOE_JOB_STEP(0, fr0, fr2)
    MOE_JOB_STEP(1, fr1, fr0)
    MOE_JOB_STEP(2, fr2, fr1)
  }
#undef MOE_JOB_STEP
}


template <int NT>
hipError_t launch_nt(const GemmParams& p, int set, int epi, hipStream_t s) {
  const dim3 grid(p.total_wg), block(256);
  if (p.dispatch) {   // persistent forms: routing blocks of one weight pass
    if (set != SET_ROUTED || (epi != EPI_SWIGLU && epi != EPI_COMBINE)) return hipErrorInvalidValue;
    if (p.dispatch == 2 && !p.queue) return hipErrorInvalidValue;
#define MOE_JOBS_CASE(EPI_, DYN_)                                                  \
    if (epi == EPI_ && (p.dispatch == 2) == DYN_) {                                \
      hipLaunchKernelGGL((gemm_small_m_jobs<NT, SET_ROUTED, EPI_, DYN_>), grid, block, 0, s, p); \
      return hipGetLastError();                                                    \
    }
    MOE_JOBS_CASE(EPI_SWIGLU, false)
    MOE_JOBS_CASE(EPI_SWIGLU, true)
    MOE_JOBS_CASE(EPI_COMBINE, false)
    MOE_JOBS_CASE(EPI_COMBINE, true)
#undef MOE_JOBS_CASE
    return hipErrorInvalidValue;
  }
#define MOE_GEMM_CASE(SET_, EPI_)                                                  \
  if (set == SET_ && epi == EPI_) {                                                \
    hipLaunchKernelGGL((gemm_small_m<NT, SET_, EPI_>), grid, block, 0, s, p);     \
    return hipGetLastError();                                                      \
  }
  MOE_GEMM_CASE(SET_INDEXED, EPI_SWIGLU)
  MOE_GEMM_CASE(SET_INDEXED, EPI_COMBINE)
  MOE_GEMM_CASE(SET_INDEXED, EPI_STORE)
  MOE_GEMM_CASE(SET_INDEXED, EPI_PARTIAL)
  MOE_GEMM_CASE(SET_ROUTED, EPI_SWIGLU)
  MOE_GEMM_CASE(SET_ROUTED, EPI_COMBINE)
  MOE_GEMM_CASE(SET_ROUTED, EPI_PARTIAL)
  MOE_GEMM_CASE(SET_MASKED, EPI_SWIGLU)
  MOE_GEMM_CASE(SET_MASKED, EPI_STORE)
  MOE_GEMM_CASE(SET_BLOCKS, EPI_SWIGLU)
  MOE_GEMM_CASE(SET_BLOCKS, EPI_COMBINE)
  MOE_GEMM_CASE(SET_BLOCKS, EPI_STORE)
#undef MOE_GEMM_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_small_m(const GemmParams& p, int set, int epi, int nt, hipStream_t s) {
  if (p.total_wg <= 0) return hipSuccess;
  switch (nt) {
    case 1: return launch_nt<1>(p, set, epi, s);
    case 2: return launch_nt<2>(p, set, epi, s);
    case 4: return launch_nt<4>(p, set, epi, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
